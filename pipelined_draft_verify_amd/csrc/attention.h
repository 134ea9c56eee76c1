// Split-KV grouped-query decode attention (gfx950).
//
// The context of a query row is cut into splits of kSplit = 256 positions.  A
// workgroup owns one KV head, one split and the queries that read that KV
// head (the Hq/Hkv query heads of one token, or of a block of consecutive
// rows of the draft module / a prefill chunk / the autoregressive decoder),
// so every key and value of the split is loaded once for all of them.  It
// writes the split's partial result -- the running max m, the sum l of
// exp(score - m) and the unnormalised weighted value sum -- and k_attn_merge
// combines the splits of each (row, head) in split order.
//
//  * k_attn_mfma (bf16 caches): scores and weighted values on the matrix
//    cores.  Each wave takes 64 positions of the split for the scores
//    (S = K Q^T, 16x16x32 MFMAs with the queries split into bf16 hi + lo),
//    the softmax weights P go through LDS (bf16 hi + lo), and each wave then
//    forms the weighted value sum of its own head-dim tiles over all 256
//    positions (O^T = V^T P^T), so no cross-wave sum of partial outputs is
//    needed.
//  * k_attn_valu (fp32 caches): thread j owns position j for the scores; the
//    weighted values are summed per position group and reduced across lanes.
//
// Cache layouts (per layer and KV head): keys [hd/8][ctx][8] -- consecutive
// positions are consecutive 16-byte chunks; values [ctx/8][hd][8] -- eight
// consecutive positions of one head dim are one 16-byte chunk.  Both give
// the matrix-core operands straight from 16-byte loads.
//
// A query's arithmetic never depends on which other queries share the
// workgroup (matrix-core results are per column; softmax statistics are per
// query), so the stage path and the row path give identical bits.
#pragma once

#include "common.h"

namespace spd {

enum PMode { PM_STAGE = 0, PM_ROWS = 1 };
constexpr int kAttnQ = 8;       // query vectors per workgroup (VALU kernel)
constexpr int kAttnMQ = 64;     // query vectors per workgroup (matrix-core kernel)
constexpr int kMaxSplit = 128;  // splits of kSplit positions per context (max_ctx <= 32768)

struct Attn {
  int pmode;
  int layer[SPD_MAX_STAGES];  // stage: layer of group g; rows: layer[0]
  int stage[SPD_MAX_STAGES];  // stage: pipeline stage of group g (increasing)
  const void* kc;
  const void* vc;
  const float* q;  // [prow][Hq*hd]
  float* pacc;     // [prow][Hq][nsplit][hd]
  float* pml;      // [prow][Hq][nsplit][2]
  float* o;        // merged output [prow][Hq*hd]
  uint16_t* oh;    // or, if set, its split into bf16 hi + lo parts [prow][Hq*hd]
  uint16_t* ol;
  int from_ctrl, pos0_arg, nrows_arg;
  int QB;          // rows per workgroup (rows mode)
  int qblocks;     // row blocks (rows mode)
  long long lane_stride;  // draft tree: elements between the caches' KV lanes
  const Ctrl* ctrl;
  Geo g;
};

// The problem of workgroup (z, row block qb): positions pos0 + r0 .. of its
// rows (r0 = qb * QB), the row count, the layer, the KV lane offset and the
// scratch row of its first query row.  A draft tree's stage groups hold one
// node each (z = group * W + rank); its draft-module rows take one row per
// workgroup (QB = 1), each at its own position and KV lane.
__device__ __forceinline__ bool attn_problem(const Attn& A, int z, int qb, int& pos0, int& nrows, int& layer,
                                             long long& kvoff, int& prow0) {
  const Ctrl* C = A.ctrl;
  const Geo& g = A.g;
  kvoff = 0;
  if (A.pmode == PM_STAGE) {
    const int grp = z / g.W, r = z - grp * g.W;
    if (!C->active || A.stage[grp] >= C->a) return false;
    if (layer_is_linear(g, A.layer[grp])) return false;  // the linear-attention kernel's group
    pos0 = C->t - A.stage[grp];
    if (g.W > 1) {
      const Tree* T = tree_of(C);
      const int ps = pos0 % g.nslots;
      if (r >= T->cnt[ps]) return false;
      kvoff = T->lane[ps * g.W + T->rk[ps][r]] * A.lane_stride;
    }
    nrows = 1;
    layer = A.layer[grp];
    prow0 = z;
    return qb == 0;
  }
  if (A.from_ctrl) {
    if (!C->active) return false;
    if (g.W > 1) {
      const Tree* T = tree_of(C);
      if (qb >= T->nrows) return false;
      pos0 = T->row_pos[qb] - qb;
      nrows = T->nrows;
      kvoff = T->row_lane[qb] * A.lane_stride;
    } else {
      pos0 = C->C;
      nrows = C->a + C->pending;
    }
  } else {
    pos0 = A.pos0_arg;
    nrows = A.nrows_arg;
  }
  layer = A.layer[0];
  prow0 = qb * A.QB;
  return true;
}

// Position of attention output row prow (merges).
__device__ __forceinline__ bool attn_row_pos(const Attn& A, int prow, int& pos) {
  const Ctrl* C = A.ctrl;
  const Geo& g = A.g;
  if (A.pmode == PM_STAGE) {
    const int grp = prow / g.W, r = prow - grp * g.W;
    if (!C->active || A.stage[grp] >= C->a) return false;
    if (layer_is_linear(g, A.layer[grp])) return false;  // written by the linear-attention kernel
    pos = C->t - A.stage[grp];
    if (g.W > 1 && r >= tree_of(C)->cnt[pos % g.nslots]) return false;
    return true;
  }
  if (A.from_ctrl) {
    if (!C->active) return false;
    if (g.W > 1) {
      const Tree* T = tree_of(C);
      if (prow >= T->nrows) return false;
      pos = T->row_pos[prow];
      return true;
    }
    if (prow >= C->a + C->pending) return false;
    pos = C->C + prow;
    return true;
  }
  if (prow >= A.nrows_arg) return false;
  pos = A.pos0_arg + prow;
  return true;
}

// 8 consecutive KV elements held in one (bf16) or two (fp32) 16-byte vectors.
template <typename KT>
__device__ __forceinline__ void unpack8(const u32x4* r, float* o);
template <>
__device__ __forceinline__ void unpack8<uint16_t>(const u32x4* r, float* o) {
  const u32x4 v = r[0];
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xFFFF0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xFFFF0000u);
  o[4] = __uint_as_float(v.z << 16);
  o[5] = __uint_as_float(v.z & 0xFFFF0000u);
  o[6] = __uint_as_float(v.w << 16);
  o[7] = __uint_as_float(v.w & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void unpack8<float>(const u32x4* r, float* o) {
  o[0] = __uint_as_float(r[0].x); o[1] = __uint_as_float(r[0].y);
  o[2] = __uint_as_float(r[0].z); o[3] = __uint_as_float(r[0].w);
  o[4] = __uint_as_float(r[1].x); o[5] = __uint_as_float(r[1].y);
  o[6] = __uint_as_float(r[1].z); o[7] = __uint_as_float(r[1].w);
}

// Index of the split partials of (row, head, split).
__device__ __forceinline__ size_t attn_part(const Geo& g, int prow, int head, int sp) {
  return ((size_t)prow * g.Hq + head) * g.nsplit + sp;
}

// ---------------------------------------------------------------------------
// VALU path (fp32 caches)
// ---------------------------------------------------------------------------
template <typename KT, int HD>
__global__ __launch_bounds__(kWG) void k_attn_valu(const Attn A) {
  __shared__ __align__(16) float qs[kAttnQ][HD];
  __shared__ float ps[kAttnQ][kSplit];
  __shared__ float rmax[kWG / kWave][kAttnQ];
  __shared__ float rsum[kWG / kWave][kAttnQ];
  __shared__ float racc[kWG / kWave][kAttnQ][HD];
  int pos0, nrows, layer, prow0;
  long long kvoff;
  if (!attn_problem(A, blockIdx.z, blockIdx.y / A.g.Hkv, pos0, nrows, layer, kvoff, prow0)) return;
  constexpr int NC = HD / 8;        // 8-element chunks per row
  constexpr int DL = HD / 8;        // lanes per value row
  constexpr int PG = kWave / DL;    // positions per wave instruction
  constexpr int NPG = PG * (kWG / kWave);
  constexpr int NI = kSplit / NPG;  // value rows per thread
  constexpr int VPC = sizeof(KT) * 8 / 16;  // 16-byte vectors per 8-element chunk
  const Geo& g = A.g;
  const int G = g.Hq / g.Hkv;
  const int kvh = blockIdx.y % g.Hkv;
  const int qb = blockIdx.y / g.Hkv;
  const int QB = (A.pmode == PM_STAGE) ? 1 : A.QB;
  const int r0 = qb * QB;
  if (r0 >= nrows) return;
  const int nr = min(QB, nrows - r0);
  const int nq = nr * G;
  const int s0 = blockIdx.x * kSplit;
  const int maxpos = pos0 + r0 + nr - 1;
  if (s0 > maxpos) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int dl = lane % DL, pg = lane / DL;
  const int gp = wave * PG + pg;
  const KT* K = reinterpret_cast<const KT*>(A.kc) + kvoff;
  const KT* Vc = reinterpret_cast<const KT*>(A.vc) + kvoff;

  for (int idx = threadIdx.x; idx < nq * HD; idx += kWG) {
    const int qi = idx / HD, dim = idx - qi * HD;
    const int r = qi / G, head = kvh * G + (qi - r * G);
    qs[qi][dim] = A.q[(size_t)(prow0 + r) * g.Hq * HD + (size_t)head * HD + dim];
  }
  const int pos = s0 + threadIdx.x;
  const bool have_key = pos <= maxpos;
  u32x4 rk[NC * VPC];
  if (have_key) {
    const size_t kbase = k_index(g, layer, kvh, pos, 0);
    const size_t cstride = (size_t)g.ctx_cap * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int h = 0; h < VPC; ++h)
        rk[c * VPC + h] = *reinterpret_cast<const u32x4*>(K + kbase + c * cstride + h * 4);
  }
  __syncthreads();

  // ---- scores: thread j owns position s0 + j (per query: dims in order) ----
  float s[kAttnQ];
#pragma unroll
  for (int qi = 0; qi < kAttnQ; ++qi) s[qi] = 0.f;
  if (have_key) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float kf[8];
      unpack8<KT>(&rk[c * VPC], kf);
#pragma unroll
      for (int qi = 0; qi < kAttnQ; ++qi) {
        if (qi < nq) {
          float acc = s[qi];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf(qs[qi][c * 8 + e], kf[e], acc);
          s[qi] = acc;
        }
      }
    }
  }
  const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
  for (int qi = 0; qi < kAttnQ; ++qi) {
    const int lim = pos0 + r0 + qi / G;
    s[qi] = (qi < nq && pos <= lim) ? s[qi] * scale : -INFINITY;
  }
#pragma unroll
  for (int qi = 0; qi < kAttnQ; ++qi) {
    if (qi < nq) {
      const float mx = wave_max(s[qi]);
      if (lane == 0) rmax[wave][qi] = mx;
    }
  }
  __syncthreads();
  float mq[kAttnQ];
#pragma unroll
  for (int qi = 0; qi < kAttnQ; ++qi) {
    float mx = -INFINITY;
    if (qi < nq)
      for (int w = 0; w < kWG / kWave; ++w) mx = fmaxf(mx, rmax[w][qi]);
    mq[qi] = mx;
    const float p = (s[qi] == -INFINITY) ? 0.f : expf(s[qi] - mx);
    if (qi < nq) ps[qi][threadIdx.x] = p;
    s[qi] = p;
  }
#pragma unroll
  for (int qi = 0; qi < kAttnQ; ++qi) {
    if (qi < nq) {
      const float sm = wave_sum(s[qi]);
      if (lane == 0) rsum[wave][qi] = sm;
    }
  }
  __syncthreads();

  // ---- weighted values: lanes (dl, pg) hold dims dl*8.. of rows gp + i*NPG ----
  float acc[kAttnQ][8];
#pragma unroll
  for (int qi = 0; qi < kAttnQ; ++qi)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[qi][e] = 0.f;
  for (int i = 0; i < NI; ++i) {
    const int jj = gp + i * NPG;
    float vf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      vf[e] = (s0 + jj <= maxpos) ? from_store(Vc[v_index(g, layer, kvh, s0 + jj, dl * 8 + e)]) : 0.f;
#pragma unroll
    for (int qi = 0; qi < kAttnQ; ++qi) {
      if (qi < nq) {
        const float p = ps[qi][jj];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[qi][e] = fmaf(p, vf[e], acc[qi][e]);
      }
    }
  }
  // reduce the position groups of a wave (lanes with equal dl), then waves
#pragma unroll
  for (int qi = 0; qi < kAttnQ; ++qi) {
    if (qi < nq) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[qi][e];
#pragma unroll
        for (int o = DL; o < kWave; o <<= 1) v += __shfl_xor(v, o, 64);
        if (pg == 0) racc[wave][qi][dl * 8 + e] = v;
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nq * HD; idx += kWG) {
    const int qi = idx / HD, dim = idx - qi * HD;
    float sum = racc[0][qi][dim];
    for (int w = 1; w < kWG / kWave; ++w) sum += racc[w][qi][dim];
    const int r = qi / G, head = kvh * G + (qi - r * G);
    const size_t base = attn_part(g, prow0 + r, head, blockIdx.x);
    A.pacc[base * HD + dim] = sum;
    if (dim == 0) {
      float l = rsum[0][qi];
      for (int w = 1; w < kWG / kWave; ++w) l += rsum[w][qi];
      A.pml[base * 2 + 0] = mq[qi];
      A.pml[base * 2 + 1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core path (bf16 caches)
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8a __attribute__((ext_vector_type(8)));
typedef float f32x4a __attribute__((ext_vector_type(4)));

// Dynamic LDS of k_attn_mfma for QT query tiles of 16.
__host__ __device__ constexpr size_t attn_mfma_lds(int HD, int QT) {
  return (size_t)QT * 16 * (HD + 8) * 2 * sizeof(uint16_t)        // queries, bf16 hi/lo
         + (size_t)QT * 16 * (kSplit + 8) * 2 * sizeof(uint16_t)  // softmax weights, bf16 hi/lo
         + (size_t)2 * (kWG / kWave) * QT * 16 * sizeof(float);  // per-wave max / sum
}

__device__ __forceinline__ uint32_t pack_bf16x2(uint16_t lo_half, uint16_t hi_half) {
  return (uint32_t)lo_half | ((uint32_t)hi_half << 16);
}

template <int HD, int QT>
__global__ __launch_bounds__(kWG) void k_attn_mfma(const Attn A) {
  constexpr int NKS = HD / 32;                  // 32-dim k-steps of a score
  constexpr int DTW = HD / 16 / (kWG / kWave);  // head-dim tiles per wave in the weighted sum
  constexpr int QP = HD + 8;                    // LDS row pitch of the queries (elements)
  constexpr int PP = kSplit + 8;                // LDS row pitch of the weights (elements)
  constexpr int NQ = QT * 16;
  extern __shared__ __align__(16) unsigned char attn_smem[];
  uint16_t* qh = reinterpret_cast<uint16_t*>(attn_smem);
  uint16_t* ql = qh + NQ * QP;
  uint16_t* ph = ql + NQ * QP;
  uint16_t* pl = ph + NQ * PP;
  float* wmax = reinterpret_cast<float*>(pl + NQ * PP);  // [wave][NQ]
  float* wsum = wmax + (kWG / kWave) * NQ;
  int pos0, nrows, layer, prow0;
  long long kvoff;
  if (!attn_problem(A, blockIdx.z, blockIdx.y / A.g.Hkv, pos0, nrows, layer, kvoff, prow0)) return;
  const Geo& g = A.g;
  const int G = g.Hq / g.Hkv;
  const int kvh = blockIdx.y % g.Hkv;
  const int qb = blockIdx.y / g.Hkv;
  const int QB = (A.pmode == PM_STAGE) ? 1 : A.QB;
  const int r0 = qb * QB;
  if (r0 >= nrows) return;
  const int nr = min(QB, nrows - r0);
  const int nq = nr * G;  // <= NQ
  const int s0 = blockIdx.x * kSplit;
  const int maxpos = pos0 + r0 + nr - 1;
  if (s0 > maxpos) return;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int r = lane & 15, kq = lane >> 4;
  const uint16_t* K = reinterpret_cast<const uint16_t*>(A.kc) + kvoff;
  const uint16_t* Vc = reinterpret_cast<const uint16_t*>(A.vc) + kvoff;
  const int pw0 = s0 + 64 * wave;  // this wave's 64 score positions

  // ---- loads: keys of the wave's positions, values of its head-dim tiles ----
  u32x4 kf[4][NKS];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) {
    const int p = pw0 + 16 * pt + r;
#pragma unroll
    for (int s = 0; s < NKS; ++s)
      kf[pt][s] = (p <= maxpos) ? *reinterpret_cast<const u32x4*>(K + k_index(g, layer, kvh, p, 32 * s + 8 * kq))
                                : u32x4{0u, 0u, 0u, 0u};
  }
  u32x4 vf[DTW][kSplit / 32];
#pragma unroll
  for (int j = 0; j < DTW; ++j) {
    const int dim = 16 * (wave * DTW + j) + r;
#pragma unroll
    for (int ps = 0; ps < kSplit / 32; ++ps) {
      const int p = s0 + 32 * ps + 8 * kq;  // first of 8 consecutive positions
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (p <= maxpos) {
        v = *reinterpret_cast<const u32x4*>(Vc + v_index(g, layer, kvh, p, dim));
        // positions past the last valid one may hold anything: zero them
        const int nv = maxpos - p + 1;
        if (nv < 8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t keep_lo = (2 * e < nv) ? 0x0000FFFFu : 0u;
            const uint32_t keep_hi = (2 * e + 1 < nv) ? 0xFFFF0000u : 0u;
            v[e] &= (keep_lo | keep_hi);
          }
        }
      }
      vf[j][ps] = v;
    }
  }
  // ---- queries -> LDS as bf16 hi/lo ----
  for (int idx = threadIdx.x; idx < NQ * HD; idx += kWG) {
    const int q = idx / HD, dim = idx - q * HD;
    float v = 0.f;
    if (q < nq) {
      const int rr = q / G, head = kvh * G + (q - rr * G);
      v = A.q[(size_t)(prow0 + rr) * g.Hq * HD + (size_t)head * HD + dim];
    }
    const uint16_t hi = f32_to_bf16_rne(v);
    qh[q * QP + dim] = hi;
    ql[q * QP + dim] = f32_to_bf16_rne(v - bf16_bits_to_f32(hi));
  }
  __syncthreads();

  // ---- scores S[position][query] = K Q^T ----
  f32x4a sc[4][QT];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) sc[pt][qt] = f32x4a{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const bf16x8a bh = *reinterpret_cast<const bf16x8a*>(qh + (16 * qt + r) * QP + 32 * s + 8 * kq);
      const bf16x8a bl = *reinterpret_cast<const bf16x8a*>(ql + (16 * qt + r) * QP + 32 * s + 8 * kq);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const bf16x8a a = __builtin_bit_cast(bf16x8a, kf[pt][s]);
        sc[pt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, sc[pt][qt], 0, 0, 0);
        sc[pt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, sc[pt][qt], 0, 0, 0);
      }
    }
  }
  // lane (r, kq) holds positions pw0 + 16pt + 4kq + i of query 16qt + r
  const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = 16 * qt + r;
    const int lim = (q < nq) ? pos0 + r0 + q / G : -1;
    float mx = -INFINITY;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = pw0 + 16 * pt + 4 * kq + i;
        const float v = (p <= lim) ? sc[pt][qt][i] * scale : -INFINITY;
        sc[pt][qt][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    if (kq == 0) wmax[wave * NQ + q] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int q = 16 * qt + r;
    float M = wmax[q];
#pragma unroll
    for (int w = 1; w < kWG / kWave; ++w) M = fmaxf(M, wmax[w * NQ + q]);
    float sum = 0.f;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      uint16_t h4[4], l4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = sc[pt][qt][i];
        const float p = (v == -INFINITY) ? 0.f : expf(v - M);
        sum += p;
        h4[i] = f32_to_bf16_rne(p);
        l4[i] = f32_to_bf16_rne(p - bf16_bits_to_f32(h4[i]));
      }
      const int col = 64 * wave + 16 * pt + 4 * kq;
      *reinterpret_cast<uint2*>(ph + q * PP + col) = uint2{pack_bf16x2(h4[0], h4[1]), pack_bf16x2(h4[2], h4[3])};
      *reinterpret_cast<uint2*>(pl + q * PP + col) = uint2{pack_bf16x2(l4[0], l4[1]), pack_bf16x2(l4[2], l4[3])};
    }
    sum += __shfl_xor(sum, 16, kWave);
    sum += __shfl_xor(sum, 32, kWave);
    if (kq == 0) wsum[wave * NQ + q] = sum;
  }
  __syncthreads();

  // ---- weighted values O^T[dim][query] = V^T P^T over all 256 positions ----
#pragma unroll
  for (int j = 0; j < DTW; ++j) {
    const int dt = wave * DTW + j;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      f32x4a acc = f32x4a{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ps = 0; ps < kSplit / 32; ++ps) {
        const bf16x8a a = __builtin_bit_cast(bf16x8a, vf[j][ps]);
        const bf16x8a bh = *reinterpret_cast<const bf16x8a*>(ph + (16 * qt + r) * PP + 32 * ps + 8 * kq);
        const bf16x8a bl = *reinterpret_cast<const bf16x8a*>(pl + (16 * qt + r) * PP + 32 * ps + 8 * kq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc, 0, 0, 0);
      }
      // lane (r, kq) holds dims 16dt + 4kq .. +3 of query 16qt + r
      const int q = 16 * qt + r;
      if (q < nq) {
        const int rr = q / G, head = kvh * G + (q - rr * G);
        const size_t base = attn_part(g, prow0 + rr, head, blockIdx.x);
        *reinterpret_cast<f32x4a*>(A.pacc + base * HD + 16 * dt + 4 * kq) = acc;
      }
    }
  }
  // ---- split statistics ----
  if ((int)threadIdx.x < nq) {
    const int q = threadIdx.x;
    float M = wmax[q], l = wsum[q];
#pragma unroll
    for (int w = 1; w < kWG / kWave; ++w) {
      M = fmaxf(M, wmax[w * NQ + q]);
      l += wsum[w * NQ + q];
    }
    const int rr = q / G, head = kvh * G + (q - rr * G);
    const size_t base = attn_part(g, prow0 + rr, head, blockIdx.x);
    A.pml[base * 2 + 0] = M;
    A.pml[base * 2 + 1] = l;
  }
}

// ---------------------------------------------------------------------------
// Merge of the splits: o = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s, in
// split order.  Grid (rows, Hq), HD threads (one per head dim).
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(HD) void k_attn_merge(const Attn A) {
  const Geo& g = A.g;
  const int prow = blockIdx.x, head = blockIdx.y;
  int pos;
  if (!attn_row_pos(A, prow, pos)) return;
  const int ns = pos / kSplit + 1;
  const int dim = threadIdx.x;
  const size_t base = attn_part(g, prow, head, 0);
  constexpr int B = 8;  // splits fetched per batch
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += B) {
    float m[B];
#pragma unroll
    for (int u = 0; u < B; ++u) m[u] = (s0 + u < ns) ? A.pml[(base + s0 + u) * 2] : -INFINITY;
#pragma unroll
    for (int u = 0; u < B; ++u) M = fmaxf(M, m[u]);
  }
  float num = 0.f, den = 0.f;
  for (int s0 = 0; s0 < ns; s0 += B) {
    float m[B], l[B], a[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const bool ok = s0 + u < ns;
      m[u] = ok ? A.pml[(base + s0 + u) * 2] : 0.f;
      l[u] = ok ? A.pml[(base + s0 + u) * 2 + 1] : 0.f;
      a[u] = ok ? A.pacc[(base + s0 + u) * HD + dim] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (s0 + u < ns) {
        const float w = expf(m[u] - M);
        num = fmaf(w, a[u], num);
        den = fmaf(w, l[u], den);
      }
    }
  }
  const size_t oi = (size_t)prow * g.Hq * HD + (size_t)head * HD + dim;
  if (A.oh) {
    const float v = num / den;
    const uint16_t hi = f32_to_bf16_rne(v);
    A.oh[oi] = hi;
    A.ol[oi] = f32_to_bf16_rne(v - bf16_bits_to_f32(hi));
  } else {
    A.o[oi] = num / den;
  }
}

}  // namespace spd
