// Split-KV grouped-query decode attention (gfx950, fp32 arithmetic).
//
// A workgroup owns one KV head, one split of kSplit = 256 positions and up to
// kMaxQ query vectors that read that KV head (the Hq/Hkv query heads of one
// token, or of several consecutive rows of the draft module / a prefill
// chunk), so every key and value of the split is loaded once for all of
// them.  Keys are stored [hd/8][ctx][8]: in the score phase thread j owns
// position j and its 16-byte chunk loads are contiguous across the wave.
// Values are stored [ctx][hd]: in the weighted sum a wave walks positions
// with each lane owning hd/64 dimensions.  Each query's arithmetic does not
// depend on which other queries share the workgroup.  Partial results
// (max, sum, unnormalised output) per split are merged by k_attn_combine.
#pragma once

#include "common.h"

namespace spd {

enum PMode { PM_STAGE = 0, PM_ROWS = 1 };

struct Attn {
  int pmode;
  int layer[SPD_MAX_STAGES];  // stage: layer of group g; rows: layer[0]
  const void* kc;
  const void* vc;
  const float* q;  // [prow][Hq*hd]
  float* pacc;     // [prow][Hq][nsplit][hd]
  float* pml;      // [prow][Hq][nsplit][2]
  float* o;        // combine output [prow][Hq*hd]
  int from_ctrl, pos0_arg, nrows_arg;
  int QB;          // rows per workgroup (rows mode)
  const Ctrl* ctrl;
  Geo g;
};

// Problem geometry shared by both kernels.
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

template <typename KT>
__global__ __launch_bounds__(kWG) void k_attn(const Attn A) {
  __shared__ float qs[kMaxQ][128];
  __shared__ float sc[kMaxQ][kSplit];
  __shared__ float pv[kWG / kWave][kMaxQ][128];
  __shared__ float rmax[kWG / kWave][kMaxQ];
  __shared__ float rsum[kWG / kWave][kMaxQ];
  const Geo& g = A.g;
  int pos0, nrows, layer;
  if (!attn_problem(A, blockIdx.z, pos0, nrows, layer)) return;
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
  const int hd = g.hd;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;

  for (int idx = threadIdx.x; idx < nq * hd; idx += kWG) {
    const int qi = idx / hd, dim = idx - qi * hd;
    const int r = qi / G, head = kvh * G + (qi - r * G);
    qs[qi][dim] = A.q[(size_t)(prow0 + r) * g.Hq * hd + (size_t)head * hd + dim];
  }
  __syncthreads();

  // scores: thread j owns position s0 + j
  const int pos = s0 + threadIdx.x;
  const KT* K = reinterpret_cast<const KT*>(A.kc);
  float s[kMaxQ];
#pragma unroll
  for (int qi = 0; qi < kMaxQ; ++qi) s[qi] = 0.f;
  if (pos <= maxpos) {
    for (int c = 0; c < hd / 8; ++c) {
      const KT* kp = K + k_index(g, layer, kvh, pos, c * 8);
      float k8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) k8[e] = from_store(kp[e]);
#pragma unroll
      for (int qi = 0; qi < kMaxQ; ++qi) {
        if (qi < nq) {
#pragma unroll
          for (int e = 0; e < 8; ++e) s[qi] = fmaf(qs[qi][c * 8 + e], k8[e], s[qi]);
        }
      }
    }
  }
  const float scale = 1.0f / sqrtf((float)hd);
#pragma unroll
  for (int qi = 0; qi < kMaxQ; ++qi) {
    const int lim = pos0 + r0 + qi / G;
    s[qi] = (qi < nq && pos <= lim) ? s[qi] * scale : -INFINITY;
  }
  // per-query max and sum over the split (fixed order: butterfly, then waves 0..3)
#pragma unroll
  for (int qi = 0; qi < kMaxQ; ++qi) {
    if (qi < nq) {
      const float mx = wave_max(s[qi]);
      if (lane == 0) rmax[wave][qi] = mx;
    }
  }
  __syncthreads();
  float mq[kMaxQ];
#pragma unroll
  for (int qi = 0; qi < kMaxQ; ++qi) {
    float mx = -INFINITY;
    if (qi < nq)
      for (int w = 0; w < kWG / kWave; ++w) mx = fmaxf(mx, rmax[w][qi]);
    mq[qi] = mx;
    const float p = (s[qi] == -INFINITY) ? 0.f : expf(s[qi] - mx);
    if (qi < nq) sc[qi][threadIdx.x] = p;
    s[qi] = p;
  }
#pragma unroll
  for (int qi = 0; qi < kMaxQ; ++qi) {
    if (qi < nq) {
      const float sm = wave_sum(s[qi]);
      if (lane == 0) rsum[wave][qi] = sm;
    }
  }
  __syncthreads();

  // weighted values: wave w walks positions [64w, 64w+64), lane owns DPT dims
  const KT* Vc = reinterpret_cast<const KT*>(A.vc);
  const int DPT = hd / kWave;  // 1 or 2
  float acc[kMaxQ][2];
#pragma unroll
  for (int qi = 0; qi < kMaxQ; ++qi) acc[qi][0] = acc[qi][1] = 0.f;
  const int jbeg = wave * kWave;
  const int jend = min(jbeg + kWave, maxpos - s0 + 1);
  for (int jj = jbeg; jj < jend; ++jj) {
    const KT* vp = Vc + v_index(g, layer, kvh, s0 + jj, lane * DPT);
    float v0 = from_store(vp[0]);
    float v1 = (DPT == 2) ? from_store(vp[1]) : 0.f;
#pragma unroll
    for (int qi = 0; qi < kMaxQ; ++qi) {
      if (qi < nq) {
        const float p = sc[qi][jj];
        acc[qi][0] = fmaf(p, v0, acc[qi][0]);
        if (DPT == 2) acc[qi][1] = fmaf(p, v1, acc[qi][1]);
      }
    }
  }
#pragma unroll
  for (int qi = 0; qi < kMaxQ; ++qi) {
    if (qi < nq) {
      pv[wave][qi][lane * DPT] = acc[qi][0];
      if (DPT == 2) pv[wave][qi][lane * DPT + 1] = acc[qi][1];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nq * hd; idx += kWG) {
    const int qi = idx / hd, dim = idx - qi * hd;
    float sum = pv[0][qi][dim];
    for (int w = 1; w < kWG / kWave; ++w) sum += pv[w][qi][dim];
    const int r = qi / G, head = kvh * G + (qi - r * G);
    const size_t base = (((size_t)(prow0 + r) * g.Hq + head) * g.nsplit + blockIdx.x);
    A.pacc[base * hd + dim] = sum;
    if (dim == 0) {
      float l = rsum[0][qi];
      for (int w = 1; w < kWG / kWave; ++w) l += rsum[w][qi];
      A.pml[base * 2 + 0] = mq[qi];
      A.pml[base * 2 + 1] = l;
    }
  }
}

// o[prow][h*hd + dim] = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s over the
// splits covering the row's positions, in split order.
__global__ __launch_bounds__(128) void k_attn_combine(const Attn A) {
  const Geo& g = A.g;
  int pos0, nrows, layer;
  const int z = (A.pmode == PM_STAGE) ? blockIdx.y : 0;
  if (!attn_problem(A, z, pos0, nrows, layer)) return;
  const int r = (A.pmode == PM_STAGE) ? 0 : blockIdx.y;
  if (r >= nrows) return;
  const int prow = (A.pmode == PM_STAGE) ? blockIdx.y : r;
  const int h = blockIdx.x;
  const int dim = threadIdx.x;
  if (dim >= g.hd) return;
  const int ns = (pos0 + r) / kSplit + 1;
  const size_t base = ((size_t)prow * g.Hq + h) * g.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, A.pml[(base + s) * 2]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = expf(A.pml[(base + s) * 2] - M);
    num = fmaf(w, A.pacc[(base + s) * g.hd + dim], num);
    den = fmaf(w, A.pml[(base + s) * 2 + 1], den);
  }
  A.o[(size_t)prow * g.Hq * g.hd + (size_t)h * g.hd + dim] = num / den;
}

}  // namespace spd
