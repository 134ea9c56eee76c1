// Row-batched GEMV on the matrix cores (gfx950 v_mfma_f32_16x16x32_bf16),
// used by the draft module's trailing rows and by prefill chunks of bf16
// models.
//
// D[16 weight rows][16 activation rows] = W_tile (16 x K, bf16) x X^T, with
// the fp32 activations split into bf16 hi + lo parts (x = hi + lo + O(2^-17 x))
// and both products accumulated in fp32, so the result is close to an fp32
// GEMV while the weights stream through the matrix cores once.  Operand
// layout (16x16x32): lane l holds row l%16 and k = 8*(l/16) .. +7 of A and,
// likewise, column l%16 of B; D lane l holds rows 4*(l/16) .. +3 of column
// l%16.  A workgroup owns one 16-row weight tile; its four waves split K into
// quarters and their partial tiles are summed in a fixed order.
#pragma once

#include "common.h"
#include "gemv.h"

namespace spd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4m __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - bf16_bits_to_f32(hi));
}

// Activation rows [M][K] fp32 -> bf16 hi/lo [M][K], optionally RMS-normalised.
__global__ __launch_bounds__(kWG) void k_split_rows(const float* X, int ldx, int M_arg, int from_ctrl, int K,
                                                    const float* gamma, float eps, uint16_t* xh, uint16_t* xl,
                                                    const Ctrl* C) {
  __shared__ float red[kWG / kWave];
  const int m = blockIdx.x;
  int M = M_arg;
  if (from_ctrl) {
    if (!C->active) return;
    M = C->a + C->pending;
  }
  if (m >= M) return;
  const float* x = X + (size_t)m * ldx;
  const float rstd = gamma ? row_rstd(x, K, eps, red) : 1.0f;
  for (int k = threadIdx.x; k < K; k += kWG) {
    const float u = gamma ? x[k] * rstd * gamma[k] : x[k];
    uint16_t hi, lo;
    split_bf16(u, hi, lo);
    xh[(size_t)m * K + k] = hi;
    xl[(size_t)m * K + k] = lo;
  }
}

struct MfmaGemv {
  const uint16_t* W;  // [N][K]
  int N, K;
  const uint16_t* xh;  // [rows][K]
  const uint16_t* xl;
  int M_arg, pos0_arg, from_ctrl;
  float* out;  // QKV: q rows [row][ldo]; RESID/STORE: rows [row][ldo]
  int ldo;
  uint16_t* oh;  // SWIGLU: activation hi/lo [row][N/2]
  uint16_t* ol;
  int layer;
  void* kc;
  void* vc;
  const float* rcos;
  const float* rsin;
  int* kv_len;
  float* anchors;
  int anchor_idx;
  Ctrl* ctrl;
  Geo g;
};

// Weight row feeding tile row r (0..15) of tile `tile`: RoPE partner pairs
// (i, i + hd/2) and gate/up pairs (u, F + u) put the two rows of a pair in
// tile rows r and r + 8.
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

template <int EPI, int MT>
__global__ __launch_bounds__(kWG) void k_gemv_mfma(const MfmaGemv A) {
  __shared__ float red[kWG / kWave][MT][16][17];
  const Ctrl* C = A.ctrl;
  if (A.from_ctrl && !C->active) return;
  const int M = A.from_ctrl ? C->a + C->pending : A.M_arg;
  const int pos0 = A.from_ctrl ? C->C : A.pos0_arg;
  const Geo& g = A.g;
  const int tile = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, kq = lane >> 4;
  const int wrow = mfma_tile_row<EPI>(g, A.N, tile, r);
  const uint16_t* wp = A.W + (size_t)wrow * A.K + kq * 8;
  const uint16_t* hp[MT];
  const uint16_t* lp[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    hp[mt] = A.xh + (size_t)(mt * 16 + r) * A.K + kq * 8;
    lp[mt] = A.xl + (size_t)(mt * 16 + r) * A.K + kq * 8;
  }
  const int ksteps = A.K / 32;
  const int sb = ksteps * wave / (kWG / kWave), se = ksteps * (wave + 1) / (kWG / kWave);
  f32x4m d[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) d[mt] = f32x4m{0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;
  for (int s = sb; s < se; s += U) {
    bf16x8 a[U], bh[U][MT], bl[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u < se) {
        const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wp + (size_t)(s + u) * 32));
        a[u] = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          bh[u][mt] = *reinterpret_cast<const bf16x8*>(hp[mt] + (size_t)(s + u) * 32);
          bl[u][mt] = *reinterpret_cast<const bf16x8*>(lp[mt] + (size_t)(s + u) * 32);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s + u < se) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bh[u][mt], d[mt], 0, 0, 0);
          d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], bl[u][mt], d[mt], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) red[wave][mt][kq * 4 + rr][r] = d[mt][rr];
  __syncthreads();

  if (EPI == EPI_QKV && A.kv_len && tile == 0 && threadIdx.x == 0) {
    int* len = A.kv_len + A.layer;
    if (*len != pos0) atomicOr(&A.ctrl->flags, SPD_FLAG_KVLEN);
    *len = pos0 + M;
  }
  const int i = threadIdx.x >> 4, j = threadIdx.x & 15;
  auto D = [&](int mt, int ii) {
    float v = red[0][mt][ii][j];
#pragma unroll
    for (int w = 1; w < kWG / kWave; ++w) v += red[w][mt][ii][j];
    return v;
  };
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + j;
    if (m >= M) continue;
    if (EPI == EPI_QKV || EPI == EPI_SWIGLU) {
      if (i >= 8) continue;
      float a = D(mt, i), b = D(mt, i + 8);
      const int u = tile * 8 + i;
      if (EPI == EPI_QKV) {
        const int half = g.hd >> 1;
        const int h = u / half, ii = u - h * half;
        const int pos = pos0 + m;
        if (h < g.Hq + g.Hkv) rope_pair(a, b, A.rcos[(size_t)pos * half + ii], A.rsin[(size_t)pos * half + ii]);
        if (h < g.Hq) {
          float* q = A.out + (size_t)m * A.ldo + (size_t)h * g.hd;
          q[ii] = a;
          q[ii + half] = b;
        } else if (h < g.Hq + g.Hkv) {
          uint16_t* kc = reinterpret_cast<uint16_t*>(A.kc);
          const int kvh = h - g.Hq;
          kc[k_index(g, A.layer, kvh, pos, ii)] = f32_to_bf16_rne(a);
          kc[k_index(g, A.layer, kvh, pos, ii + half)] = f32_to_bf16_rne(b);
        } else {
          uint16_t* vc = reinterpret_cast<uint16_t*>(A.vc);
          const int kvh = h - g.Hq - g.Hkv;
          vc[v_index(g, A.layer, kvh, pos, ii)] = f32_to_bf16_rne(a);
          vc[v_index(g, A.layer, kvh, pos, ii + half)] = f32_to_bf16_rne(b);
        }
      } else {
        const float act = silu_mul(a, b);
        uint16_t hi, lo;
        split_bf16(act, hi, lo);
        const size_t F = (size_t)(A.N >> 1);
        A.oh[(size_t)m * F + u] = hi;
        A.ol[(size_t)m * F + u] = lo;
      }
    } else {
      const float v = D(mt, i);
      const int n = tile * 16 + i;
      float* o = A.out + (size_t)m * A.ldo;
      if (EPI == EPI_RESID) {
        const float hn = o[n] + v;
        o[n] = hn;
        if (A.anchors && A.anchor_idx >= 0) A.anchors[((size_t)m * g.m + A.anchor_idx) * g.d + n] = hn;
      } else {
        o[n] = v;
      }
    }
  }
}

}  // namespace spd
