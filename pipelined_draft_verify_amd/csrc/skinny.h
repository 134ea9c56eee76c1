// Skinny matrix-core GEMV for the draft module's products in the cycle
// (gfx950 v_mfma_f32_16x16x32_bf16): q/k/v, o-projection, gate/up and down
// over the M <= 16*MT trailing rows of one cycle ([PL] 3.3: the draft module
// runs every pipeline step on a handful of rows, so its products are
// weight-streaming GEMVs with a short row dimension).
//
//   Y[m][n] = s_m * sum_k W[n][k] Xg[m][k]
//
// Xg = gamma (.) X is handed over by the producer of X already split into
// bf16 hi + lo parts (Xg = hi + lo + O(2^-17 |Xg|)); both parts go through the
// matrix core, so the product is close to an fp32 GEMV while the weights
// stream once.  s_m is the RMSNorm scale 1/rms(X[m]) (1 without a norm),
// taken from per-row partial sums of squares the producer wrote, and applied
// to the finished sum (the norm's scale is a per-row constant, so it factors
// out of the sum).
//
// Work decomposition: one workgroup per 16-row weight tile; its NW waves
// split K into NW equal ranges, each wave streaming its range with up to P
// k-steps of loads in flight; the NW partial 16x16 tiles are summed through
// LDS in wave order, and the epilogue runs in the same kernel -- no partial
// tiles leave the workgroup and no reduction launch follows.  The weights
// were re-tiled at init (k_tile_weights) into the operand order: for tile T,
// range w, k-step s and lane l, the 8 weights of row row(T, l % 16) at
// k = w Kw + 32 s + 8 (l / 16) .. +7, so each wave load is one contiguous
// 1 KB that goes to the matrix core as loaded.  The activations are read per
// lane (row l % 16, the same 8 k) from the L2-resident split buffers.
#pragma once

#include "common.h"
#include "mfma.h"

namespace spd {

constexpr int kSkinnyCols = 16;  // columns per partial sum of squares written by the RESID epilogue

struct SkinnyArgs {
  const uint16_t* Wt;     // weights in tile order (k_tile_weights with the same N, K, NW)
  int N, K;               // weight rows, inputs
  const uint16_t* xh;     // split input rows [row][K]: hi and lo parts of gamma (.) x
  const uint16_t* xl;
  const float* ssq;       // per-row partial sums of squares of x [row][ssq_parts] (norm), or nullptr
  int ssq_parts;
  // epilogue
  float* out;             // QKV: q rows [row][ldo]; RESID: X rows [row][ldo], updated in place
  int ldo;
  float* ssq_out;         // RESID: [row][N / kSkinnyCols] partial sums of squares of the new X
  uint16_t* yh;           // RESID: split of ygamma (.) new X [row][N]; SWIGLU: split of the activation [row][N/2]
  uint16_t* yl;
  const float* ygamma;    // RESID: gain of the next consumer's norm, or nullptr (split of X itself)
  int layer;
  void* kc;
  void* vc;
  const float* rcos;
  const float* rsin;
  float* anchors;         // RESID: row-indexed anchor taps [row][m][d], or nullptr
  int anchor_idx;
  const Ctrl* ctrl;
  Geo g;
};

// K ranges (waves) of a product: enough waves to cover the CUs a few times
// over, each range a whole number of 32-wide k-steps.
__host__ __forceinline__ int skinny_ways(int N, int K) {
  const int tiles = N / 16;
  if (tiles < 512 && K % (32 * 16) == 0) return 16;
  if (tiles < 1024 || K % (32 * 4)) return 8;
  return 4;
}

// Re-tiling of a row-major [N][K] bf16 matrix into the operand order above.
// One thread per 16-byte chunk.
template <int EPI>
__global__ __launch_bounds__(kWG) void k_tile_weights(const uint16_t* __restrict__ W, uint16_t* __restrict__ Wt,
                                                      int N, int K, int NW, Geo g) {
  const int nks = K / NW / 32;
  const size_t total = (size_t)N * K / 8;
  for (size_t i = (size_t)blockIdx.x * kWG + threadIdx.x; i < total; i += (size_t)gridDim.x * kWG) {
    const int lane = (int)(i % kWave);
    size_t rest = i / kWave;
    const int s = (int)(rest % nks);
    rest /= nks;
    const int w = (int)(rest % NW);
    const int T = (int)(rest / NW);
    const int row = mfma_tile_row<EPI>(g, N, T, lane & 15);
    const int k = w * (K / NW) + 32 * s + 8 * (lane >> 4);
    reinterpret_cast<u32x4*>(Wt)[i] = *reinterpret_cast<const u32x4*>(W + (size_t)row * K + k);
  }
}

// Split of v into bf16 hi + lo at element i of a split buffer.
__device__ __forceinline__ void store_split(uint16_t* hb, uint16_t* lb, size_t i, float v) {
  uint16_t hi, lo;
  split_bf16(v, hi, lo);
  hb[i] = hi;
  lb[i] = lo;
}

template <int EPI, int MT, int NW>
__global__ __launch_bounds__(NW * kWave) void k_skinny(const SkinnyArgs A) {
  constexpr int R = 16 * MT;           // activation rows of the pass
  constexpr int P = MT == 1 ? 8 : 4;   // k-steps in flight per wave
  constexpr int SP = NW * kWave / R;   // threads per row for the norm's partial sums
  constexpr int NT = NW * kWave;
  __shared__ float red[NW][R][17];
  __shared__ float srs[R];
  const Geo& g = A.g;
  const int T = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, kq = lane >> 4;
  const int Kw = A.K / NW, nks = Kw / 32;

  // The first weight loads go out before the control block is read; the
  // activation rows (only the cycle's rows: the others are not in the cache)
  // follow once the row count is known -- they come from L2 and still arrive
  // before the weights.
  const u32x4* wp = reinterpret_cast<const u32x4*>(A.Wt) + (size_t)(T * NW + wave) * nks * kWave + lane;
  const int k0 = wave * Kw + 8 * kq;
  const u32x4* hp[MT];
  const u32x4* lp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    hp[mt] = reinterpret_cast<const u32x4*>(A.xh + (size_t)(16 * mt + r) * A.K + k0);
    lp[mt] = reinterpret_cast<const u32x4*>(A.xl + (size_t)(16 * mt + r) * A.K + k0);
  }
  u32x4 wb[P], hb[MT][P], lb[MT][P];
  bool live[MT];
  auto issue_w = [&](int s, int i) { wb[i] = __builtin_nontemporal_load(wp + (size_t)s * kWave); };
  auto issue_x = [&](int s, int i) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (live[mt]) {
        hb[mt][i] = hp[mt][4 * s];
        lb[mt][i] = lp[mt][4 * s];
      } else {
        hb[mt][i] = u32x4{0u, 0u, 0u, 0u};
        lb[mt][i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
#pragma unroll
  for (int i = 0; i < P; ++i)
    if (i < nks) issue_w(i, i);

  const Ctrl* C = A.ctrl;
  if (!C->active) return;
  const bool tree = g.W > 1;
  const int M = min(R, tree ? tree_of(C)->nrows : C->a + C->pending);
  if (M <= 0) return;
  const int pos0 = C->C;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) live[mt] = 16 * mt + r < M;
#pragma unroll
  for (int i = 0; i < P; ++i)
    if (i < nks) issue_x(i, i);

  // operands of the epilogue, requested while the weights stream: the
  // residual and next gain (RESID), the RoPE factors (QKV)
  constexpr int NE = (EPI == EPI_RESID || EPI == EPI_STORE) ? (R * 16 + NT - 1) / NT : (R * 8 + NT - 1) / NT;
  float pre0[NE], pre1[NE];
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    const int e = threadIdx.x + j * NT;
    pre0[j] = 0.f;
    pre1[j] = 1.f;
    if (EPI == EPI_RESID || EPI == EPI_STORE) {
      if (e < M * 16) {
        const int m = e >> 4, n = T * 16 + (e & 15);
        pre0[j] = A.out[(size_t)m * A.ldo + n];
        if (A.ygamma) pre1[j] = A.ygamma[n];
      }
    } else if (EPI == EPI_QKV) {
      if (e < M * 8) {
        const int m = e >> 3, u = T * 8 + (e & 7);
        const int half = g.hd >> 1;
        const int h = u / half, i = u - h * half;
        const int pos = tree ? tree_of(C)->row_pos[m] : pos0 + m;
        if (h < g.Hq + g.Hkv) {
          pre0[j] = A.rcos[(size_t)pos * half + i];
          pre1[j] = A.rsin[(size_t)pos * half + i];
        }
      }
    }
  }

  // RMSNorm scale of every row from the producer's partial sums
  if (A.ssq) {
    const int m = threadIdx.x / SP, j = threadIdx.x % SP;
    float sq = 0.f;
    if (m < M)
      for (int i = j; i < A.ssq_parts; i += SP) sq += A.ssq[(size_t)m * A.ssq_parts + i];
#pragma unroll
    for (int o = SP / 2; o > 0; o >>= 1) sq += __shfl_xor(sq, o, SP);
    if (m < M && j == 0) srs[m] = rstd_of(sq, A.K, g.eps);
  }

  f32x4m d[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) d[mt] = f32x4m{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nks; s0 += P) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const int s = s0 + i;
      if (s < nks) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, wb[i]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, hb[mt][i]), d[mt], 0, 0, 0);
          d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, lb[mt][i]), d[mt], 0, 0, 0);
        }
        if (s + P < nks) {
          issue_w(s + P, i);
          issue_x(s + P, i);
        }
      }
    }
  }
  // D lane layout: lane (r, kq) holds tile rows 4kq..4kq+3 of activation row 16mt + r
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][16 * mt + r][4 * kq + i] = d[mt][i];
  __syncthreads();

  auto total = [&](int m, int c) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[w][m][c];
    return A.ssq ? v * srs[m] : v;
  };
  if (EPI == EPI_QKV || EPI == EPI_SWIGLU) {
    // units u = 8 T + cu pair tile rows cu and cu + 8 (RoPE partners / gate and up)
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int e = threadIdx.x + j * NT;
      if (e >= M * 8) break;
      const int m = e >> 3, cu = e & 7;
      float a = total(m, cu), b = total(m, cu + 8);
      const int u = T * 8 + cu;
      if (EPI == EPI_QKV) {
        const int half = g.hd >> 1;
        const int h = u / half, i = u - h * half;
        const int pos = tree ? tree_of(C)->row_pos[m] : pos0 + m;
        if (h < g.Hq + g.Hkv) rope_pair(a, b, pre0[j], pre1[j]);
        if (h < g.Hq) {
          float* q = A.out + (size_t)m * A.ldo + (size_t)h * g.hd;
          q[i] = a;
          q[i + half] = b;
        } else {
          // a draft tree's row writes its key/values to every lane of its descendants
          const int lanes = tree ? tree_of(C)->row_lanes[m] : 1;
          const bool isk = h < g.Hq + g.Hkv;
          uint16_t* cache = reinterpret_cast<uint16_t*>(isk ? A.kc : A.vc);
          const int kvh = isk ? h - g.Hq : h - g.Hq - g.Hkv;
          const size_t i0 = isk ? k_index(g, A.layer, kvh, pos, i) : v_index(g, A.layer, kvh, pos, i);
          const size_t i1 = isk ? k_index(g, A.layer, kvh, pos, i + half) : v_index(g, A.layer, kvh, pos, i + half);
          for (int ln = 0; ln < kMaxW; ++ln) {
            if (!((lanes >> ln) & 1)) continue;
            cache[ln * g.lane_pkv + i0] = f32_to_bf16_rne(a);
            cache[ln * g.lane_pkv + i1] = f32_to_bf16_rne(b);
          }
        }
      } else {
        store_split(A.yh, A.yl, (size_t)m * (A.N >> 1) + u, silu_mul(a, b));
      }
    }
  } else {
    // residual: X[m][n] += y; the 16 columns of a row are 16 consecutive lanes
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      const int e = threadIdx.x + j * NT;
      if (e >= M * 16) break;
      const int m = e >> 4, c = e & 15;
      const int n = T * 16 + c;
      float* o = A.out + (size_t)m * A.ldo;
      const float hn = pre0[j] + total(m, c);
      if (A.anchors && A.anchor_idx >= 0) A.anchors[((size_t)m * g.m + A.anchor_idx) * g.d + n] = hn;
      o[n] = hn;
      float sq = hn * hn;
#pragma unroll
      for (int s = 8; s > 0; s >>= 1) sq += __shfl_xor(sq, s, 16);
      if (c == 0) A.ssq_out[(size_t)m * (A.N / kSkinnyCols) + T] = sq;
      if (A.yh) store_split(A.yh, A.yl, (size_t)m * A.N + n, A.ygamma ? pre1[j] * hn : hn);
    }
  }
}

}  // namespace spd
