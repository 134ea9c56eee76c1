// Split-KV grouped-query decode attention (gfx950, fp32 arithmetic).
//
// A workgroup owns one KV head, one split of kSplit = 256 positions and up to
// kAttnQ query vectors that read that KV head (the Hq/Hkv query heads of one
// token, or of consecutive rows of the draft module / a prefill chunk), so
// each key and value of the split is loaded once for all of them.
//  * scores: thread j owns position j and issues all of its key's 16-byte
//    chunks at once (keys are stored [hd/8][ctx][8], so the chunk loads of a
//    wave are contiguous);
//  * weighted values: a position's value row [hd] is read by hd/8 lanes with
//    16-byte loads, 64*8/hd positions per wave instruction;
//  * the splits of a (row block, KV head) are merged by the workgroup that
//    finishes last (a per-block arrival counter that it resets), in split
//    order, so no separate combine launch is needed.
// A query's arithmetic never depends on which other queries share the
// workgroup, so the stage path and the row path give identical bits.
#pragma once

#include "common.h"

namespace spd {

enum PMode { PM_STAGE = 0, PM_ROWS = 1 };
constexpr int kAttnQ = 8;  // query vectors per workgroup

struct Attn {
  int pmode;
  int layer[SPD_MAX_STAGES];  // stage: layer of group g; rows: layer[0]
  const void* kc;
  const void* vc;
  const float* q;  // [prow][Hq*hd]
  float* pacc;     // [prow][Hq][nsplit][hd]
  float* pml;      // [prow][Hq][nsplit][2]
  float* o;        // output [prow][Hq*hd] (fp32), or
  uint16_t* oh;    // ... its bf16 hi/lo split for the matrix-core GEMV (when set)
  uint16_t* ol;
  int* counters;   // [problem][qblock][Hkv] arrival counters, zero between launches
  int from_ctrl, pos0_arg, nrows_arg;
  int QB;          // rows per workgroup (rows mode)
  int qblocks;     // row blocks (rows mode)
  const Ctrl* ctrl;
  Geo g;
};

__device__ __forceinline__ bool attn_problem(const Attn& A, int z, int& pos0, int& nrows, int& layer) {
  const Ctrl* C = A.ctrl;
  if (A.pmode == PM_STAGE) {
    if (!C->active || z >= C->a) return false;
    pos0 = C->t - z;
    nrows = 1;
    layer = A.layer[z];
  } else {
    if (A.from_ctrl) {
      if (!C->active) return false;
      pos0 = C->C;
      nrows = C->a + C->pending;
    } else {
      pos0 = A.pos0_arg;
      nrows = A.nrows_arg;
    }
    layer = A.layer[0];
  }
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

template <typename KT, int HD>
__device__ __forceinline__ void attn_body(const Attn& A, int pos0, int nrows, int layer) {
  __shared__ float qs[kAttnQ][HD];
  __shared__ float ps[kAttnQ][kSplit];
  __shared__ float rmax[kWG / kWave][kAttnQ];
  __shared__ float rsum[kWG / kWave][kAttnQ];
  __shared__ float racc[kWG / kWave][kAttnQ][HD];
  __shared__ int last;
  constexpr int NC = HD / 8;        // 8-element chunks per row
  constexpr int DL = HD / 8;        // lanes per value row
  constexpr int PG = kWave / DL;    // positions per wave instruction
  constexpr int NPG = PG * (kWG / kWave);
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
  const int prow0 = (A.pmode == PM_STAGE) ? blockIdx.z : r0;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;

  for (int idx = threadIdx.x; idx < nq * HD; idx += kWG) {
    const int qi = idx / HD, dim = idx - qi * HD;
    const int r = qi / G, head = kvh * G + (qi - r * G);
    qs[qi][dim] = A.q[(size_t)(prow0 + r) * g.Hq * HD + (size_t)head * HD + dim];
  }
  __syncthreads();

  // ---- scores ----
  const int pos = s0 + threadIdx.x;
  const KT* K = reinterpret_cast<const KT*>(A.kc);
  float s[kAttnQ];
#pragma unroll
  for (int qi = 0; qi < kAttnQ; ++qi) s[qi] = 0.f;
  if (pos <= maxpos) {
    // up to 16 x 16-byte vectors of the key in flight per batch
    constexpr int VPC = sizeof(KT) * 8 / 16;           // vectors per 8-element chunk
    constexpr int CB = (NC * VPC <= 16) ? NC : 16 / VPC;  // chunks per batch
    const size_t kbase = k_index(g, layer, kvh, pos, 0);
    const size_t cstride = (size_t)g.ctx_cap * 8;
#pragma unroll
    for (int cb = 0; cb < NC; cb += CB) {
      u32x4 raw[CB * VPC];
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int h = 0; h < VPC; ++h)
          raw[c * VPC + h] = *reinterpret_cast<const u32x4*>(K + kbase + (cb + c) * cstride + h * 4);
#pragma unroll
      for (int qi = 0; qi < kAttnQ; ++qi) {
        if (qi < nq) {
          float acc = s[qi];
#pragma unroll
          for (int c = 0; c < CB; ++c) {
            float kf[8];
            unpack8<KT>(&raw[c * VPC], kf);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(qs[qi][(cb + c) * 8 + e], kf[e], acc);
          }
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

  // ---- weighted values ----
  const KT* Vc = reinterpret_cast<const KT*>(A.vc);
  const int dl = lane % DL, pg = lane / DL;
  const int gp = wave * PG + pg;
  float acc[kAttnQ][8];
#pragma unroll
  for (int qi = 0; qi < kAttnQ; ++qi)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[qi][e] = 0.f;
  constexpr int NI = kSplit / NPG;  // positions per thread
  constexpr int VPC = sizeof(KT) * 8 / 16;
  constexpr int IB = 4;             // positions per batch of loads
#pragma unroll
  for (int ib = 0; ib < NI; ib += IB) {
    u32x4 raw[IB * VPC];
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const int jj = gp + (ib + i) * NPG;
#pragma unroll
      for (int h = 0; h < VPC; ++h) {
        if (s0 + jj <= maxpos)
          raw[i * VPC + h] = *reinterpret_cast<const u32x4*>(Vc + v_index(g, layer, kvh, s0 + jj, dl * 8) + h * 4);
        else
          raw[i * VPC + h] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      const int jj = gp + (ib + i) * NPG;
      float vf[8];
      unpack8<KT>(&raw[i * VPC], vf);
#pragma unroll
      for (int qi = 0; qi < kAttnQ; ++qi) {
        if (qi < nq) {
          const float p = ps[qi][jj];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[qi][e] = fmaf(p, vf[e], acc[qi][e]);
        }
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
    const size_t base = (((size_t)(prow0 + r) * g.Hq + head) * g.nsplit + blockIdx.x);
    A.pacc[base * HD + dim] = sum;
    if (dim == 0) {
      float l = rsum[0][qi];
      for (int w = 1; w < kWG / kWave; ++w) l += rsum[w][qi];
      A.pml[base * 2 + 0] = mq[qi];
      A.pml[base * 2 + 1] = l;
    }
  }

  // ---- merge the splits: the last workgroup of this (row block, KV head) ----
  const int nsp = maxpos / kSplit + 1;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    int* cnt = A.counters + ((size_t)blockIdx.z * gridDim.y + blockIdx.y);
    const int prev = atomicAdd(cnt, 1);
    last = (prev == nsp - 1);
    if (last) *cnt = 0;  // ready for the next launch
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  for (int idx = threadIdx.x; idx < nq * HD; idx += kWG) {
    const int qi = idx / HD, dim = idx - qi * HD;
    const int r = qi / G, head = kvh * G + (qi - r * G);
    const int ns = (pos0 + r0 + r) / kSplit + 1;  // splits covering this row
    const size_t base = ((size_t)(prow0 + r) * g.Hq + head) * g.nsplit;
    const volatile float* pml = A.pml;
    const volatile float* pacc = A.pacc;
    float M = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, pml[(base + sp) * 2]);
    float num = 0.f, den = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
      const float w = expf(pml[(base + sp) * 2] - M);
      num = fmaf(w, pacc[(base + sp) * HD + dim], num);
      den = fmaf(w, pml[(base + sp) * 2 + 1], den);
    }
    const float ov = num / den;
    const size_t oi = (size_t)(prow0 + r) * g.Hq * HD + (size_t)head * HD + dim;
    if (A.oh) {
      A.oh[oi] = f32_to_bf16_rne(ov);
      A.ol[oi] = f32_to_bf16_rne(ov - bf16_bits_to_f32(A.oh[oi]));
    } else {
      A.o[oi] = ov;
    }
  }
}

template <typename KT, int HD>
__global__ __launch_bounds__(kWG) void k_attn(const Attn A) {
  int pos0, nrows, layer;
  if (!attn_problem(A, blockIdx.z, pos0, nrows, layer)) return;
  attn_body<KT, HD>(A, pos0, nrows, layer);
}

}  // namespace spd
