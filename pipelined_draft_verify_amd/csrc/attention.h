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
constexpr int kAttnQ = 8;      // query vectors per workgroup
constexpr int kMaxSplit = 128;  // splits of kSplit positions per context (max_ctx <= 32768)

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

// Relaxed agent-scope load: a value another workgroup published before the
// arrival counter said so (the merge reads the other splits' partials).
__device__ __forceinline__ float load_published(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename KT, int HD>
__device__ __forceinline__ void attn_body(const Attn& A, int pos0, int nrows, int layer) {
  __shared__ __align__(16) float qs[kAttnQ][HD];
  __shared__ float ps[kAttnQ][kSplit];
  __shared__ float rmax[kWG / kWave][kAttnQ];
  __shared__ float rsum[kWG / kWave][kAttnQ];
  __shared__ float racc[kWG / kWave][kAttnQ][HD];
  __shared__ float sml[kAttnQ][kMaxSplit][2];
  __shared__ int last;
  constexpr int NC = HD / 8;        // 8-element chunks per row
  constexpr int DL = HD / 8;        // lanes per value row
  constexpr int PG = kWave / DL;    // positions per wave instruction
  constexpr int NPG = PG * (kWG / kWave);
  constexpr int NI = kSplit / NPG;  // value rows per thread
  constexpr int VPC = sizeof(KT) * 8 / 16;  // 16-byte vectors per 8-element chunk
  // bf16: every key and value vector of the split is requested before any
  // arithmetic (one memory round trip); fp32: values after the scores
  constexpr bool kPrefetchV = sizeof(KT) == 2;
  constexpr int NVR = kPrefetchV ? NI * VPC : 1;
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
  const int dl = lane % DL, pg = lane / DL;
  const int gp = wave * PG + pg;
  const KT* K = reinterpret_cast<const KT*>(A.kc);
  const KT* Vc = reinterpret_cast<const KT*>(A.vc);

  // ---- loads: queries first (needed first), then keys, then values ----
  constexpr int QPT = (kAttnQ * HD + kWG - 1) / kWG;
  float qv[QPT];
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int idx = threadIdx.x + u * kWG;
    qv[u] = 0.f;
    if (idx < nq * HD) {
      const int qi = idx / HD, dim = idx - qi * HD;
      const int r = qi / G, head = kvh * G + (qi - r * G);
      qv[u] = A.q[(size_t)(prow0 + r) * g.Hq * HD + (size_t)head * HD + dim];
    }
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
  u32x4 rv[NVR];
  if (kPrefetchV) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int jj = gp + i * NPG;
#pragma unroll
      for (int h = 0; h < VPC; ++h) {
        if (s0 + jj <= maxpos)
          rv[i * VPC + h] = *reinterpret_cast<const u32x4*>(Vc + v_index(g, layer, kvh, s0 + jj, dl * 8) + h * 4);
        else
          rv[i * VPC + h] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
#pragma unroll
  for (int u = 0; u < QPT; ++u) {
    const int idx = threadIdx.x + u * kWG;
    if (idx < kAttnQ * HD) qs[idx / HD][idx % HD] = qv[u];
  }
  __syncthreads();

  // ---- scores: thread j owns position s0 + j ----
  // chunk-major: the queries' independent FMA chains interleave and each
  // query chunk is one broadcast 16-byte LDS read; per query the order is
  // still dims 0..HD-1
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
          const f32x4 qa = *reinterpret_cast<const f32x4*>(&qs[qi][c * 8]);
          const f32x4 qb = *reinterpret_cast<const f32x4*>(&qs[qi][c * 8 + 4]);
          float acc = s[qi];
          acc = fmaf(qa.x, kf[0], acc);
          acc = fmaf(qa.y, kf[1], acc);
          acc = fmaf(qa.z, kf[2], acc);
          acc = fmaf(qa.w, kf[3], acc);
          acc = fmaf(qb.x, kf[4], acc);
          acc = fmaf(qb.y, kf[5], acc);
          acc = fmaf(qb.z, kf[6], acc);
          acc = fmaf(qb.w, kf[7], acc);
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
  constexpr int IB = kPrefetchV ? NI : 4;  // value rows per batch of loads
#pragma unroll
  for (int ib = 0; ib < NI; ib += IB) {
    u32x4 raw[IB * VPC];
#pragma unroll
    for (int i = 0; i < IB; ++i) {
#pragma unroll
      for (int h = 0; h < VPC; ++h) {
        if (kPrefetchV) {
          raw[i * VPC + h] = rv[(ib + i) * VPC + h];
        } else {
          const int jj = gp + (ib + i) * NPG;
          if (s0 + jj <= maxpos)
            raw[i * VPC + h] = *reinterpret_cast<const u32x4*>(Vc + v_index(g, layer, kvh, s0 + jj, dl * 8) + h * 4);
          else
            raw[i * VPC + h] = u32x4{0u, 0u, 0u, 0u};
        }
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
  // every split's (max, sum) of every query, fetched in parallel
  for (int idx = threadIdx.x; idx < nq * nsp; idx += kWG) {
    const int qi = idx / nsp, sp = idx - qi * nsp;
    const int r = qi / G, head = kvh * G + (qi - r * G);
    const size_t b = ((size_t)(prow0 + r) * g.Hq + head) * g.nsplit + sp;
    sml[qi][sp][0] = load_published(A.pml + b * 2);
    sml[qi][sp][1] = load_published(A.pml + b * 2 + 1);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < nq * HD; idx += kWG) {
    const int qi = idx / HD, dim = idx - qi * HD;
    const int r = qi / G, head = kvh * G + (qi - r * G);
    const int ns = (pos0 + r0 + r) / kSplit + 1;  // splits covering this row
    const size_t base = ((size_t)(prow0 + r) * g.Hq + head) * g.nsplit;
    float M = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, sml[qi][sp][0]);
    float num = 0.f, den = 0.f;
    constexpr int MB = 8;  // partial rows fetched per batch
    for (int sb = 0; sb < ns; sb += MB) {
      float pv[MB];
#pragma unroll
      for (int u = 0; u < MB; ++u) pv[u] = (sb + u < ns) ? load_published(A.pacc + (base + sb + u) * HD + dim) : 0.f;
#pragma unroll
      for (int u = 0; u < MB; ++u) {
        if (sb + u < ns) {
          const float w = expf(sml[qi][sb + u][0] - M);
          num = fmaf(w, pv[u], num);
          den = fmaf(w, sml[qi][sb + u][1], den);
        }
      }
    }
    const float ov = num / den;
    const size_t oi = (size_t)(prow0 + r) * g.Hq * HD + (size_t)head * HD + dim;
    if (A.oh) {
      const uint16_t hi = f32_to_bf16_rne(ov);
      A.oh[oi] = hi;
      A.ol[oi] = f32_to_bf16_rne(ov - bf16_bits_to_f32(hi));
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
