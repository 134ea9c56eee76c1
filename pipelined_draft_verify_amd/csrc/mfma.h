// Row-batched skinny GEMM on the matrix cores (gfx950 v_mfma_f32_16x16x32_bf16)
// for the draft module's trailing rows, its anchor-fusion FC and prefill
// chunks of bf16 models.
//
// Y[m][n] = sum_k W[n][k] X'[m][k] for M <= 16*MT activation rows, where
// X' = X (or gamma * X / rms(X) with a fused RMSNorm).  The fp32 activations
// are split into bf16 hi + lo parts (x = hi + lo + O(2^-17 |x|)) and both
// products are accumulated in fp32, so the result is close to an fp32 GEMV
// while the weights stream through the matrix cores once.
//
// Work decomposition: a workgroup of four waves owns a 64-row group of W
// (one 16-row MFMA tile per wave) and one of S consecutive K ranges; it walks
// its range in chunks of KC = 256 (128 for two activation tiles, which keeps
// the workgroup's LDS near 50 KB so that two or more fit on a CU beside the
// stage kernels).  Per chunk:
//  * each wave loads its 16 weight rows with row-contiguous 16-byte loads
//    (the next chunk's loads are in flight while this one is multiplied) and
//    re-lays them through LDS into the MFMA operand layout (lane l holds row
//    l%16, k = 8*(l/16)..+7 of each 32-wide k-step);
//  * the workgroup stages the activation chunk once into LDS as bf16 hi/lo,
//    shared by the four waves.
// With S = 1 the workgroup applies the epilogue itself; with S > 1 it writes
// fp32 partial tiles and k_mfma_reduce sums them in split order and applies
// the epilogue (a kernel boundary instead of a device-wide fence).
//
// Fused RMSNorm: rms(X[m]) comes from per-row partial sums of squares that the
// producer of X wrote (one per 64-column group, summed here in group order),
// or, without them, from a direct pass over the row.  RESID/STORE epilogues
// write those partial sums for the next consumer.
#pragma once

#include "common.h"
#include "gemv.h"

namespace spd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4m __attribute__((ext_vector_type(4)));

constexpr int kMKC = 256;          // K per chunk
constexpr int kMGroup = 64;        // weight rows per workgroup
constexpr int kMMaxSplit = 64;     // K ranges per product
constexpr int kSsqCols = 64;       // columns per partial sum of squares

__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - bf16_bits_to_f32(hi));
}

struct MfmaArgs {
  // products (FC patterns: one per blockIdx.z; otherwise one)
  const uint16_t* W[SPD_MAX_ANCHORS];
  int K[SPD_MAX_ANCHORS];
  int S[SPD_MAX_ANCHORS];       // K ranges (K % (S * kMKC) == 0)
  int poff[SPD_MAX_ANCHORS];    // first partial slab of the product
  int N;                        // weight rows (multiple of kMGroup)
  // activation rows (fp32)
  int rmode;                    // RM_CONTIG, RM_FC or RM_ATTN
  const float* x;               // RM_CONTIG: row m at x + (row_base + m) * ldx
  int ldx;
  const float* slot_anchors;    // RM_FC: row i reads anchors 0..f of the slot of position pos0 + i
  const float* apacc;           // RM_ATTN: row i is the attention output of row i, merged from its
  const float* apml;            //   split partials [row][Hq][nsplit][hd] and (max, sum) [row][Hq][nsplit][2]
  const float* gamma;           // fused RMSNorm gain [K], or nullptr (no norm)
  const float* ssq;             // per-row partial sums of squares of the input [row][ssq_parts], or nullptr
  int ssq_parts;
  int M_arg, pos0_arg, from_ctrl, row_base;
  // epilogue
  float* out;                   // QKV: q rows; SWIGLU: activation rows; RESID/STORE: X rows
  int ldo;
  float* ssq_out;               // RESID/STORE: [row][N / kSsqCols] partial sums of squares of the result
  uint16_t* yh;                 // RESID/STORE: split (bf16 hi + lo) of ygamma (.) result [row][N], or nullptr
  uint16_t* yl;
  const float* ygamma;          //   gain of the next consumer's norm (nullptr: the result itself)
  int layer;
  void* kc;
  void* vc;
  const float* rcos;
  const float* rsin;
  int* kv_len;                  // QKV: length word of `layer` to check and advance, or nullptr
  float* anchors;               // RESID: row-indexed anchor taps [row][m][d], or nullptr
  int anchor_idx;
  float* part;                  // S > 1: partial tiles [slab][16*MT][N]
  Ctrl* ctrl;
  Geo g;
};

// Weight row of tile row r (0..15) of tile `tile`: RoPE partner pairs
// (i, i + hd/2) and gate/up pairs (u, F + u) sit in tile rows r and r + 8.
template <int EPI>
__device__ __forceinline__ int mfma_tile_row(const Geo& g, int N, int tile, int r) {
  if (EPI == EPI_QKV) {
    const int half = g.hd >> 1;
    const int u = tile * 8 + (r & 7);
    const int h = u / half, i = u - h * half;
    return h * g.hd + i + (r >= 8 ? half : 0);
  } else if (EPI == EPI_SWIGLU) {
    const int u = tile * 8 + (r & 7);
    return u + (r >= 8 ? (N >> 1) : 0);
  }
  return tile * 16 + r;
}

// Rows of this launch: count, first position and (FC) the trailing row of
// each activation row.  Thread 0 fills the shared values.
__device__ __forceinline__ void mfma_select_rows(const MfmaArgs& A, int prob, int cap, int* s_M, int* s_pos0,
                                                 int* rsrc) {
  if (threadIdx.x == 0) {
    const Ctrl* C = A.ctrl;
    const Geo& g = A.g;
    const bool tree = A.from_ctrl && g.W > 1;
    const int Mtot = tree ? tree_of(C)->nrows : A.from_ctrl ? (C->a + C->pending) : A.M_arg;
    const int pos0 = A.from_ctrl ? C->C : A.pos0_arg;
    int M;
    if (A.rmode == RM_FC) {
      M = 0;
      for (int i = 0; i < Mtot; ++i) {
        const int dep = tree ? tree_of(C)->row_depth[i] : pdm_row_depth(g, C, i, pos0 + i);
        if (g.fpat[dep] == prob && M < cap) rsrc[M++] = i;
      }
    } else {
      M = min(cap, Mtot - A.row_base);
      for (int i = 0; i < M; ++i) rsrc[i] = A.row_base + i;
    }
    *s_M = M;
    *s_pos0 = pos0;
  }
}

__device__ __forceinline__ const float* mfma_in_row(const MfmaArgs& A, int orow, int pos0) {
  if (A.rmode == RM_FC) {
    const int slot = (A.g.W > 1) ? tree_of(A.ctrl)->row_slot[orow] : (pos0 + orow) % A.g.nslots;
    return A.slot_anchors + (size_t)slot * A.g.m * A.g.d;
  }
  return A.x + (size_t)orow * A.ldx;
}

// Position of activation row orow (a draft tree's rows carry their own).
__device__ __forceinline__ int mfma_row_pos(const MfmaArgs& A, int orow, int pos0) {
  return (A.from_ctrl && A.g.W > 1) ? tree_of(A.ctrl)->row_pos[orow] : pos0 + orow;
}

// Epilogue of activation row m of one row group, run by one wave: lane c
// holds the finished product v of tile-ordered column c (c = 16 * tile +
// tile row) of the group.  QKV/SWIGLU pair columns (c, c + 8) of a tile into
// unit lanes 0..31.
template <int EPI>
__device__ __forceinline__ void mfma_epilogue_row(const MfmaArgs& A, int rg, int m, int pos0, const int* rsrc,
                                                  float v) {
  const Geo& g = A.g;
  const int lane = threadIdx.x & (kWave - 1);
  const int orow = rsrc[m];
  if (EPI == EPI_QKV || EPI == EPI_SWIGLU) {
    const int t = (lane >> 3) & 3, r = lane & 7;
    float a = __shfl(v, t * 16 + r, kWave);
    float b = __shfl(v, t * 16 + r + 8, kWave);
    if (lane >= 32) return;
    const int u = (rg * 4 + t) * 8 + r;
    if (EPI == EPI_QKV) {
      const int half = g.hd >> 1;
      const int h = u / half, i = u - h * half;
      const int pos = mfma_row_pos(A, orow, pos0);
      if (h < g.Hq + g.Hkv) rope_pair(a, b, A.rcos[(size_t)pos * half + i], A.rsin[(size_t)pos * half + i]);
      if (h < g.Hq) {
        float* q = A.out + (size_t)orow * A.ldo + (size_t)h * g.hd;
        q[i] = a;
        q[i + half] = b;
      } else {
        // a draft tree's row writes its key/values to every lane of its descendants
        const int lanes = (A.from_ctrl && g.W > 1) ? tree_of(A.ctrl)->row_lanes[orow] : 1;
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
      A.out[(size_t)orow * A.ldo + u] = silu_mul(a, b);
    }
  } else {
    const int n = rg * kMGroup + lane;
    float* o = A.out + (size_t)orow * A.ldo;
    float hn;
    if (EPI == EPI_RESID) {
      hn = o[n] + v;
      if (A.anchors && A.anchor_idx >= 0) A.anchors[((size_t)orow * g.m + A.anchor_idx) * g.d + n] = hn;
    } else {
      hn = v;
    }
    o[n] = hn;
    if (A.yh) {
      uint16_t hi, lo;
      split_bf16(A.ygamma ? A.ygamma[n] * hn : hn, hi, lo);
      A.yh[(size_t)orow * A.N + n] = hi;
      A.yl[(size_t)orow * A.N + n] = lo;
    }
    if (A.ssq_out) {
      const float sq = wave_sum(hn * hn);
      if (lane == 0) A.ssq_out[(size_t)orow * (A.N / kSsqCols) + rg] = sq;
    }
  }
}

// The QKV epilogue checks and advances the layer's KV length once per launch.
__device__ __forceinline__ void mfma_kv_len(const MfmaArgs& A, int M, int pos0, const int* rsrc) {
  int* len = A.kv_len + A.layer;
  if (*len != pos0 + rsrc[0]) atomicOr(&A.ctrl->flags, SPD_FLAG_KVLEN);
  *len = pos0 + rsrc[M - 1] + 1;
}

template <int EPI, int MT, int KC = kMKC>
__global__ __launch_bounds__(kWG) void k_mfma_gemv(const MfmaArgs A) {
  constexpr int R = 16 * MT;    // activation rows per pass
  constexpr int KP = KC + 8;    // LDS row pitch (elements): breaks bank aliasing of the 16 rows
  static_assert(kMKC % KC == 0 && KC % 128 == 0, "chunks divide the split unit");
  __shared__ __align__(16) uint16_t bh[2][R][KP];
  __shared__ __align__(16) uint16_t bl[2][R][KP];
  __shared__ __align__(16) uint16_t wl[kWG / kWave][16][KP];
  static_assert(sizeof(bh) >= sizeof(float) * R * (kMGroup + 1), "the epilogue tile reuses bh");
  __shared__ float srstd[R];
  __shared__ int rsrc[R];
  __shared__ int s_M, s_pos0;
  const Ctrl* C = A.ctrl;
  if (A.from_ctrl && !C->active) return;
  const int prob = blockIdx.z;
  const int S = A.S[prob];
  const int rg = blockIdx.x, sp = blockIdx.y;
  if (sp >= S) return;
  const int K = A.K[prob];
  const int KR = K / S;
  const int kb = sp * KR;
  const int nch = KR / KC;
  const Geo& g = A.g;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, kq = lane >> 4;

  // weight loads of the first chunk go out before anything else
  constexpr int LPR = KC / 8;        // lanes per weight row (8 bf16 each)
  constexpr int RPI = kWave / LPR;   // weight rows per load instruction
  constexpr int NI = 16 / RPI;       // load instructions per chunk
  const int tile = rg * 4 + wave;
  const int lr = lane / LPR, lk = (lane % LPR) * 8;  // instruction i: tile rows RPI i + lr, k = lk..lk+7
  const uint16_t* W = A.W[prob];
  const uint16_t* wrow[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
    wrow[i] = W + (size_t)mfma_tile_row<EPI>(g, A.N, tile, RPI * i + lr) * K + kb + lk;
  u32x4 wr[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) wr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[i]));

  mfma_select_rows(A, prob, R, &s_M, &s_pos0, rsrc);
  __syncthreads();
  const int M = s_M, pos0 = s_pos0;
  if (M <= 0) return;

  // RMSNorm scale of each row: 16 lanes per row sum the producer's partial
  // sums of squares (all rows at once), or, without them, a pass over the row
  if (A.gamma) {
    if (A.ssq) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = (threadIdx.x >> 4) + 16 * mt, sl = threadIdx.x & 15;
        float sq = 0.f;
        if (m < M) {
          const float* p = A.ssq + (size_t)rsrc[m] * A.ssq_parts;
          for (int i = sl; i < A.ssq_parts; i += 16) sq += p[i];
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) sq += __shfl_xor(sq, o, 16);
        if (m < M && sl == 0) srstd[m] = 1.0f / sqrtf(sq / (float)K + g.eps);
      }
    } else {
      for (int m = wave; m < M; m += kWG / kWave) {
        const float* x = mfma_in_row(A, rsrc[m], pos0);
        float sq = 0.f;
        for (int i = lane; i < K; i += kWave) sq = fmaf(x[i], x[i], sq);
        sq = wave_sum(sq);
        if (lane == 0) srstd[m] = 1.0f / sqrtf(sq / (float)K + g.eps);
      }
    }
  }
  __syncthreads();

  // activation staging: thread t covers row t/TPR (+RPP per pass), 16 consecutive k
  constexpr int TPR = KC / 16;               // threads per activation row
  constexpr int RPP = kWG / TPR;             // rows per staging pass
  constexpr int NP = (R + RPP - 1) / RPP;    // staging passes
  const int br = threadIdx.x / TPR, bk = (threadIdx.x % TPR) * 16;
  f32x4 xr[NP][4];
  auto load_x = [&](int c) {
#pragma unroll
    for (int mt = 0; mt < NP; ++mt) {
      const int m = br + RPP * mt;
      const int k = kb + c * KC + bk;
      if (m < M && A.rmode == RM_ATTN) {
        // merge the row's attention splits for the 16 dims k..k+15 (one head):
        // the same arithmetic, in split order, as the split-merge kernel
        const Geo& g = A.g;
        const int orow = rsrc[m];
        const int ns = mfma_row_pos(A, orow, pos0) / kSplit + 1;
        const int head = k / g.hd, d0 = k - head * g.hd;
        const size_t base = ((size_t)orow * g.Hq + head) * g.nsplit;
        float M = -INFINITY;
        for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, A.apml[(base + sp) * 2]);
        float num[16], den = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) num[e] = 0.f;
        for (int sp = 0; sp < ns; ++sp) {
          const float w = expf(A.apml[(base + sp) * 2] - M);
          den = fmaf(w, A.apml[(base + sp) * 2 + 1], den);
          const float* pa = A.apacc + (base + sp) * g.hd + d0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(pa + 4 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e) num[4 * j + e] = fmaf(w, a[e], num[4 * j + e]);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xr[mt][j] = f32x4{num[4 * j] / den, num[4 * j + 1] / den, num[4 * j + 2] / den, num[4 * j + 3] / den};
      } else if (m < M) {
        const float* x = mfma_in_row(A, rsrc[m], pos0) + k;
#pragma unroll
        for (int j = 0; j < 4; ++j) xr[mt][j] = *reinterpret_cast<const f32x4*>(x + 4 * j);
        if (A.gamma) {
          const float s = srstd[m];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 gm = *reinterpret_cast<const f32x4*>(A.gamma + k + 4 * j);
            xr[mt][j] = xr[mt][j] * s * gm;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) xr[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int mt = 0; mt < NP; ++mt) {
      const int m = br + RPP * mt;
      if (m >= R) continue;
      uint16_t h[16], l[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) split_bf16(xr[mt][j][e], h[4 * j + e], l[4 * j + e]);
      u32x4 hv[2], lv[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        hv[q] = u32x4{h[8 * q] | ((uint32_t)h[8 * q + 1] << 16), h[8 * q + 2] | ((uint32_t)h[8 * q + 3] << 16),
                      h[8 * q + 4] | ((uint32_t)h[8 * q + 5] << 16), h[8 * q + 6] | ((uint32_t)h[8 * q + 7] << 16)};
        lv[q] = u32x4{l[8 * q] | ((uint32_t)l[8 * q + 1] << 16), l[8 * q + 2] | ((uint32_t)l[8 * q + 3] << 16),
                      l[8 * q + 4] | ((uint32_t)l[8 * q + 5] << 16), l[8 * q + 6] | ((uint32_t)l[8 * q + 7] << 16)};
        *reinterpret_cast<u32x4*>(&bh[buf][m][bk + 8 * q]) = hv[q];
        *reinterpret_cast<u32x4*>(&bl[buf][m][bk + 8 * q]) = lv[q];
      }
    }
  };
  load_x(0);
  store_x(0);

  f32x4m d[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) d[mt] = f32x4m{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
#pragma unroll
    for (int i = 0; i < NI; ++i) *reinterpret_cast<u32x4*>(&wl[wave][RPI * i + lr][lk]) = wr[i];
    if (c + 1 < nch) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        wr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[i] + (c + 1) * KC));
      load_x(c + 1);
    }
    __syncthreads();  // weights of chunk c and activations buffer `buf` are in LDS
#pragma unroll
    for (int s = 0; s < KC / 32; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&wl[wave][r][32 * s + 8 * kq]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 h = *reinterpret_cast<const bf16x8*>(&bh[buf][16 * mt + r][32 * s + 8 * kq]);
        const bf16x8 l = *reinterpret_cast<const bf16x8*>(&bl[buf][16 * mt + r][32 * s + 8 * kq]);
        d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, h, d[mt], 0, 0, 0);
        d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, l, d[mt], 0, 0, 0);
      }
    }
    if (c + 1 < nch) store_x(buf ^ 1);
    __syncthreads();  // LDS reads of this chunk are done
  }

  // D lane layout: lane (r, kq) holds tile rows 4kq..4kq+3 of activation row 16mt + r
  if (S == 1) {
    float (*dt)[kMGroup + 1] = reinterpret_cast<float (*)[kMGroup + 1]>(&bh[0][0][0]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dt[16 * mt + r][wave * 16 + 4 * kq + i] = d[mt][i];
    __syncthreads();
    if (EPI == EPI_QKV && A.kv_len && rg == 0 && threadIdx.x == 0) mfma_kv_len(A, M, pos0, rsrc);
    for (int m = wave; m < M; m += kWG / kWave) mfma_epilogue_row<EPI>(A, rg, m, pos0, rsrc, dt[m][lane]);
  } else {
    float* P = A.part + (size_t)(A.poff[prob] + sp) * R * A.N;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = 16 * mt + r;
      if (m < M)
#pragma unroll
        for (int i = 0; i < 4; ++i) P[(size_t)m * A.N + rg * kMGroup + wave * 16 + 4 * kq + i] = d[mt][i];
    }
  }
}

// Sum of the S partial tiles (in split order) and the epilogue, for products
// whose K was split over workgroups.  One wave per (row group, activation
// row): grid (N / 64, 16 * MT, products), 64 threads.
template <int EPI, int MT>
__global__ __launch_bounds__(kWave) void k_mfma_reduce(const MfmaArgs A) {
  constexpr int R = 16 * MT;
  __shared__ int rsrc[R];
  __shared__ int s_M, s_pos0;
  const Ctrl* C = A.ctrl;
  if (A.from_ctrl && !C->active) return;
  const int prob = blockIdx.z;
  const int S = A.S[prob];
  if (S <= 1) return;
  const int rg = blockIdx.x, m = blockIdx.y;
  mfma_select_rows(A, prob, R, &s_M, &s_pos0, rsrc);
  __syncthreads();
  const int M = s_M, pos0 = s_pos0;
  if (m >= M) return;
  const int lane = threadIdx.x;
  const size_t slab = (size_t)R * A.N;
  const float* p = A.part + (size_t)A.poff[prob] * slab + (size_t)m * A.N + rg * kMGroup + lane;
  float v = 0.f;
  constexpr int B = 8;  // partials in flight per lane
  for (int s0 = 0; s0 < S; s0 += B) {
    float t[B];
#pragma unroll
    for (int u = 0; u < B; ++u) t[u] = (s0 + u < S) ? p[(size_t)(s0 + u) * slab] : 0.f;
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (s0 + u < S) v += t[u];
  }
  if (EPI == EPI_QKV && A.kv_len && rg == 0 && m == 0 && lane == 0) mfma_kv_len(A, M, pos0, rsrc);
  mfma_epilogue_row<EPI>(A, rg, m, pos0, rsrc, v);
}

}  // namespace spd
