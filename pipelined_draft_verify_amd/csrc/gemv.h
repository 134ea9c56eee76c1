// Matrix-vector kernels of the SPD cycle (gfx950, VALU, fp32 accumulation).
//
// y = W x for weight matrices W [N][K] (bf16 or fp32, row-major) streamed once
// per launch with 16-byte non-temporal loads.  One wavefront owns four output
// rows; its 64 lanes split K in 16-byte chunks (lane l reads elements
// l*VEC .. l*VEC+VEC-1 of every 64*VEC block, in ascending order) and the four
// partial sums are reduced with a butterfly.  Both kernels below use exactly
// this per-row arithmetic, so a row computed by either gives the same bits.
//
//  * k_gemv_stage: the stage-grouped decode GEMV.  Group g is pipeline stage
//    stage[g] (g itself under the uniform split; a non-uniform split leaves
//    out the stages that have no layer in a sub-step); its in-flight token's
//    input vector is normalised once per workgroup into LDS.  The grid is
//    persistent: the tiles of all ACTIVE groups (stage < a, known only on the
//    device) are spread over every workgroup, so warm-up cycles with few
//    tokens in flight still use the whole chip.
//  * k_gemv_rows: up to kRowsMR activation rows share one weight stream
//    (draft-module rows, prefill chunks, autoregressive decode); the input
//    rows are staged through LDS in K chunks.
#pragma once

#include "common.h"

namespace spd {

constexpr int kStageMinWG = 256;  // workgroups of a stage step at the lowest occupancy

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_ARGMAX = 3, EPI_STORE = 4 };
enum GMode { GM_STAGE = 0, GM_EXIT = 1, GM_FIXED = 2, GM_PDMLAST = 3 };
enum RMode { RM_CONTIG = 0, RM_FC = 1, RM_ATTN = 2 };

__host__ __device__ constexpr bool epi_pairs(int epi) { return epi == EPI_QKV || epi == EPI_SWIGLU; }

// Rows of output unit u: QKV pairs (i, i+hd/2) of one head (rotate-half RoPE
// partners); SwiGLU pairs (gate i, up i); otherwise one row.
template <int EPI>
__device__ __forceinline__ void unit_rows(const Geo& g, int N, int u, int& r0, int& r1) {
  if (EPI == EPI_QKV) {
    const int half = g.hd >> 1;
    const int h = u / half, i = u - h * half;
    r0 = h * g.hd + i;
    r1 = r0 + half;
  } else if (EPI == EPI_SWIGLU) {
    r0 = u;
    r1 = u + (N >> 1);
  } else {
    r0 = u;
    r1 = -1;
  }
}

// a[i] for a lane-dependent i without dynamic register indexing
__device__ __forceinline__ float sel4(const float (&a)[4], int i) {
  return i == 0 ? a[0] : (i == 1 ? a[1] : (i == 2 ? a[2] : a[3]));
}

__device__ __forceinline__ float silu_mul(float gte, float up) { return gte / (1.0f + expf(-gte)) * up; }

// RoPE rotation of the pair (a, b) = (x_i, x_{i+hd/2}) at table entry (pos, i).
__device__ __forceinline__ void rope_pair(float& a, float& b, float c, float s) {
  const float a2 = a * c - b * s;
  const float b2 = b * c + a * s;
  a = a2;
  b = b2;
}

// ---------------------------------------------------------------------------
// Stage-grouped GEMV
// ---------------------------------------------------------------------------
struct StageGemv {
  const void* W[SPD_MAX_STAGES];
  const float* gamma[SPD_MAX_STAGES];  // RMSNorm gain of the input (nullptr: no norm)
  int layer[SPD_MAX_STAGES];           // layer of group g (KV epilogue)
  int stage[SPD_MAX_STAGES];           // pipeline stage of group g (increasing; GM_STAGE)
  int anchor_idx[SPD_MAX_STAGES];      // anchor to tap after this layer, or -1
  int N, K, units, n_groups, gmode;
  const float* x;
  long long x_stride;
  int x_by_slot;  // input row = x + (slot or group row) * x_stride
  float* out;
  long long out_stride;
  int out_by_slot;
  void* kc;
  void* vc;
  const float* rcos;
  const float* rsin;
  int* kv_len;
  float* anchors;
  ArgPair* parts;
  Ctrl* ctrl;
  Geo g;
};

// XG: the input row is read straight from global memory (cache-resident)
// instead of being staged in LDS -- for un-normalised long inputs (the down
// projection), so that the kernel holds no LDS and the draft stream's kernels
// can share its CUs.  The arithmetic is the same either way.
// One k-step of four weight rows against NR input rows (nr of them live):
// the weights are converted once, then fp32 FMAs in element order into
// acc[m][r] -- per input row exactly the single-row chain.
template <typename WT, int NR>
__device__ __forceinline__ void gemv_step(const typename WVec<WT>::Raw* rw, const float* const* xr, int k0, int nr,
                                          float (&acc)[NR][4]) {
  constexpr int VEC = WVec<WT>::N;
  float w[4][VEC];
#pragma unroll
  for (int r = 0; r < 4; ++r) WVec<WT>::cvt(rw[r], w[r]);
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    if (NR == 1 || m < nr) {
      float xv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) xv[e] = xr[m][k0 + e];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[m][r] = fmaf(w[r][e], xv[e], acc[m][r]);
    }
  }
}

// xs[i] = x[i] * rstd * gm[i] (no gain: xs[i] = x[i]) for i < K, by kWG
// threads.  Rows of up to kWG * kXRegs elements are read once, row and gain
// loads all in flight together; the sum of squares runs in row_rstd's order
// and the scale is the same expression, so the staged values are the same
// bits as on the two-pass path used for longer rows.
constexpr int kXRegs = 16;
__device__ __forceinline__ void stage_input(const float* __restrict__ x, const float* __restrict__ gm, int K,
                                            float eps, float* red, float* xs) {
  if (K <= kWG * kXRegs) {
    float xr[kXRegs], gr[kXRegs];
#pragma unroll
    for (int j = 0; j < kXRegs; ++j) {
      const int i = threadIdx.x + j * kWG;
      xr[j] = i < K ? x[i] : 0.f;
      gr[j] = (gm != nullptr && i < K) ? gm[i] : 0.f;
    }
    if (gm) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < kXRegs; ++j)
        if (threadIdx.x + j * kWG < K) s = fmaf(xr[j], xr[j], s);
      const float rstd = rstd_of(block_sum(s, red), K, eps);
#pragma unroll
      for (int j = 0; j < kXRegs; ++j) {
        const int i = threadIdx.x + j * kWG;
        if (i < K) xs[i] = xr[j] * rstd * gr[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kXRegs; ++j) {
        const int i = threadIdx.x + j * kWG;
        if (i < K) xs[i] = xr[j];
      }
    }
  } else if (gm) {
    const float rstd = row_rstd(x, K, eps, red);
    for (int i = threadIdx.x; i < K; i += kWG) xs[i] = x[i] * rstd * gm[i];
  } else {
    for (int i = threadIdx.x; i < K; i += kWG) xs[i] = x[i];
  }
}

// Rows of group `grp` (position pos): the live count and the node slot of
// each (a single chain: one row, slot pos mod nslots; a draft tree: the live
// nodes at that position in rank order).
template <int NR>
__device__ __forceinline__ int stage_rows(const Geo& g, const Ctrl* C, int pos, int* slot) {
  const int ps = pos % g.nslots;
  if (NR == 1 || g.W == 1) {
    slot[0] = (g.W == 1) ? ps : ps * g.W + tree_of(C)->rk[ps][0];
    return 1;
  }
  const Tree* T = tree_of(C);
  const int nr = min(NR, (int)T->cnt[ps]);
#pragma unroll
  for (int r = 0; r < NR; ++r) slot[r] = ps * g.W + T->rk[ps][r < nr ? r : 0];
  return nr;
}

// NR: input rows per group (the nodes of a draft tree's stage; 1 for a chain
// and the verification head; the leaves for the tree's draft head).
template <typename WT, int EPI, bool XG = false, int NR = 1>
__global__ __launch_bounds__(kWG) void k_gemv_stage(const StageGemv A) {
  extern __shared__ float xs_lds[];  // [NR][K] (unless XG)
  __shared__ float red[kWG / kWave];
  __shared__ ArgPair wbest[NR][kWG / kWave];
  constexpr int VEC = WVec<WT>::N;
  constexpr int UPW = epi_pairs(EPI) ? 2 : 4;  // units per wave
  constexpr int UPT = UPW * (kWG / kWave);     // units per tile
  const Ctrl* __restrict__ C = A.ctrl;
  const Geo& g = A.g;
  const Tree* T = tree_of(C);

  int n_act, pos_base;
  if (A.gmode == GM_STAGE) {
    if (!C->active) return;
    // the groups whose stage holds a token: a prefix, stages being increasing
    n_act = 0;
    for (int k = 0; k < A.n_groups; ++k) n_act += A.stage[k] < C->a ? 1 : 0;
    pos_base = C->t;
  } else if (A.gmode == GM_EXIT) {
    if (!C->active || C->a != g.n) return;
    n_act = 1;
    pos_base = C->t - (g.n - 1);
  } else if (A.gmode == GM_PDMLAST) {
    if (!C->active) return;
    n_act = 1;
    pos_base = 0;
  } else {
    n_act = 1;
    pos_base = 0;
  }
  const int tpg = (A.units + UPT - 1) / UPT;
  const long long Tt = (long long)n_act * tpg;
  // stage steps with few tokens in flight use a proportional share of the
  // grid (at least one workgroup per CU): the step takes about as long, and
  // the draft stream's latency-bound kernels find free CUs.  A draft tree's
  // stage groups hold several rows (NR > 1): their GEMV is bound by its FMA
  // issue rate, not by HBM, and takes the whole grid.
  int nwg = gridDim.x;
  if (A.gmode == GM_STAGE && NR == 1)
    nwg = max(min((int)gridDim.x, kStageMinWG), (int)((long long)gridDim.x * n_act / A.n_groups));
  if ((int)blockIdx.x >= nwg) return;
  const long long t0 = Tt * blockIdx.x / nwg;
  const long long t1 = Tt * (blockIdx.x + 1) / nwg;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  float bv[NR];
  int bi[NR];
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    bv[m] = -INFINITY;
    bi[m] = 0x7FFFFFFF;
  }

  int cur = -1, pos = 0, nr = 1;
  int slot[NR];
  const float* xr[NR];
#pragma unroll
  for (int m = 0; m < NR; ++m) {
    slot[m] = 0;
    xr[m] = xs_lds;
  }
  for (long long tile = t0; tile < t1; ++tile) {
    const int grp = (int)(tile / tpg);
    const int ut = (int)(tile - (long long)grp * tpg);
    // four rows of this wave
    int rows[4];
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
      const int u = ut * UPT + wave * UPW + j;
      int r0, r1;
      unit_rows<EPI>(g, A.N, u < A.units ? u : 0, r0, r1);
      if (epi_pairs(EPI)) {
        rows[2 * j] = r0;
        rows[2 * j + 1] = r1;
      } else {
        rows[j] = r0;
      }
    }
    const WT* W = reinterpret_cast<const WT*>(A.W[grp]);
    const WT* p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = W + (size_t)rows[r] * A.K;
    // two k-steps per trip: the eight 16-byte weight loads are all issued
    // before the first is used; the odd last step (if any) likewise.  The
    // first trip's loads go out before a new group's input rows are staged,
    // so the staging overlaps their latency.
    constexpr int kStep = kWave * VEC;
    int k0 = lane * VEC;
    const bool pair0 = k0 + kStep < A.K;
    typename WVec<WT>::Raw ra[4], rb[4];
    if (k0 < A.K) {
#pragma unroll
      for (int r = 0; r < 4; ++r) ra[r] = WVec<WT>::ld(p[r] + k0);
    }
    if (pair0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) rb[r] = WVec<WT>::ld(p[r] + k0 + kStep);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (grp != cur) {
      cur = grp;
      pos = pos_base - A.stage[grp];
      const float* xin[NR];
      if (A.gmode == GM_STAGE) {
        nr = stage_rows<NR>(g, C, pos, slot);
#pragma unroll
        for (int m = 0; m < NR; ++m) xin[m] = A.x + (A.x_by_slot ? slot[m] : grp * NR + m) * A.x_stride;
      } else if (A.gmode == GM_EXIT) {
        nr = 1;
        slot[0] = (g.W == 1) ? pos % g.nslots : T->exit_slot;
        xin[0] = A.x + slot[0] * A.x_stride;
      } else if (A.gmode == GM_PDMLAST) {
        // the newest draft-module rows: a chain's last row, or a tree's leaves
        const int nrow = (g.W == 1) ? C->a + C->pending : T->nrows;
        nr = (g.W == 1) ? 1 : min(NR, (int)T->nleaves);
#pragma unroll
        for (int m = 0; m < NR; ++m) xin[m] = A.x + (size_t)(nrow - nr + (m < nr ? m : 0)) * A.x_stride;
      } else {
        nr = 1;
#pragma unroll
        for (int m = 0; m < NR; ++m) xin[m] = A.x;
      }
      if (XG) {
#pragma unroll
        for (int m = 0; m < NR; ++m) xr[m] = xin[m];
      } else {
        __syncthreads();
#pragma unroll
        for (int m = 0; m < NR; ++m)
          if (m < nr) stage_input(xin[m], A.gamma[grp], A.K, g.eps, red, xs_lds + (size_t)m * A.K);
#pragma unroll
        for (int m = 0; m < NR; ++m) xr[m] = xs_lds + (size_t)m * A.K;
        __syncthreads();
      }
      if (EPI == EPI_QKV && ut == 0 && threadIdx.x == 0 && A.kv_len && g.W == 1) {
        int* len = A.kv_len + A.layer[grp];
        if (*len != pos) atomicOr(&A.ctrl->flags, SPD_FLAG_KVLEN);
        *len = pos + 1;
      }
    }
    float acc[NR][4];
#pragma unroll
    for (int m = 0; m < NR; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][r] = 0.f;
    if (pair0) {
      gemv_step<WT, NR>(ra, xr, k0, nr, acc);
      gemv_step<WT, NR>(rb, xr, k0 + kStep, nr, acc);
      k0 += 2 * kStep;
      for (; k0 + kStep < A.K; k0 += 2 * kStep) {
#pragma unroll
        for (int r = 0; r < 4; ++r) ra[r] = WVec<WT>::ld(p[r] + k0);
#pragma unroll
        for (int r = 0; r < 4; ++r) rb[r] = WVec<WT>::ld(p[r] + k0 + kStep);
        __builtin_amdgcn_sched_barrier(0);
        gemv_step<WT, NR>(ra, xr, k0, nr, acc);
        gemv_step<WT, NR>(rb, xr, k0 + kStep, nr, acc);
      }
      if (k0 < A.K) {
#pragma unroll
        for (int r = 0; r < 4; ++r) ra[r] = WVec<WT>::ld(p[r] + k0);
        __builtin_amdgcn_sched_barrier(0);
        gemv_step<WT, NR>(ra, xr, k0, nr, acc);
      }
    } else if (k0 < A.K) {
      gemv_step<WT, NR>(ra, xr, k0, nr, acc);
    }

#pragma unroll
    for (int m = 0; m < NR; ++m) {
      if (NR > 1 && m >= nr) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[m][r] = wave_sum(acc[m][r]);

      // epilogue: lane j handles unit j of the wave
      if (lane < UPW) {
        const int j = lane;
        const int u = ut * UPT + wave * UPW + j;
        if (u < A.units) {
          if (EPI == EPI_QKV) {
            float a = sel4(acc[m], 2 * j), b = sel4(acc[m], 2 * j + 1);
            const int half = g.hd >> 1;
            const int h = u / half, i = u - h * half;
            if (h < g.Hq + g.Hkv) rope_pair(a, b, A.rcos[(size_t)pos * half + i], A.rsin[(size_t)pos * half + i]);
            if (h < g.Hq) {
              float* q = A.out + (size_t)(grp * NR + m) * A.out_stride + (size_t)h * g.hd;
              q[i] = a;
              q[i + half] = b;
            } else {
              // the node's key/values go to every KV lane of its descendants
              const int lanes = (g.W == 1) ? 1 : T->lanes[slot[m]];
              const bool isk = h < g.Hq + g.Hkv;
              auto* cache = reinterpret_cast<WT*>(isk ? A.kc : A.vc);
              const int kvh = isk ? h - g.Hq : h - g.Hq - g.Hkv, ly = A.layer[grp];
              const size_t i0 = isk ? k_index(g, ly, kvh, pos, i) : v_index(g, ly, kvh, pos, i);
              const size_t i1 = isk ? k_index(g, ly, kvh, pos, i + half) : v_index(g, ly, kvh, pos, i + half);
              for (int ln = 0; ln < kMaxW; ++ln) {
                if (!((lanes >> ln) & 1)) continue;
                cache[ln * g.lane_kv + i0] = to_store<WT>(a);
                cache[ln * g.lane_kv + i1] = to_store<WT>(b);
              }
            }
          } else if (EPI == EPI_SWIGLU) {
            A.out[(size_t)(grp * NR + m) * A.out_stride + u] = silu_mul(sel4(acc[m], 2 * j), sel4(acc[m], 2 * j + 1));
          } else if (EPI == EPI_RESID) {
            const int sl = slot[m];
            float* o = A.out + (A.out_by_slot ? sl : grp * NR + m) * A.out_stride;
            const float hn = o[u] + sel4(acc[m], j);
            o[u] = hn;
            const int ai = A.anchor_idx[grp];
            if (ai >= 0) A.anchors[((size_t)sl * g.m + ai) * g.d + u] = hn;
          } else if (EPI == EPI_ARGMAX) {
            const float y = sel4(acc[m], j);
            A.out[(size_t)m * A.N + u] = y;
            if (better(y, u, bv[m], bi[m])) {
              bv[m] = y;
              bi[m] = u;
            }
          } else {
            A.out[(size_t)(grp * NR + m) * A.out_stride + u] = sel4(acc[m], j);
          }
        }
      }
    }
  }
  if (EPI == EPI_ARGMAX) {
    // lanes 0..3 of each wave hold candidates; reduce in a fixed order
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      wave_argmax(bv[m], bi[m]);
      if (lane == 0) wbest[m][wave] = ArgPair{bv[m], bi[m]};
    }
    __syncthreads();
    if (threadIdx.x < NR) {
      const int m = threadIdx.x;
      ArgPair b = wbest[m][0];
      for (int w = 1; w < kWG / kWave; ++w)
        if (better(wbest[m][w].v, wbest[m][w].i, b.v, b.i)) b = wbest[m][w];
      A.parts[(size_t)m * gridDim.x + blockIdx.x] = b;
    }
  }
}

// ---------------------------------------------------------------------------
// Row-batched GEMV (M <= kRowsMR rows per weight stream)
// ---------------------------------------------------------------------------
struct RowsGemv {
  const void* W[SPD_MAX_ANCHORS];
  int Kg[SPD_MAX_ANCHORS];  // K per group (FC patterns differ)
  const float* gamma;       // RMSNorm gain of the input rows (nullptr: none)
  int N, units, n_groups, rmode;
  const float* x;
  int ldx;
  int M_arg, pos0_arg, from_ctrl;  // rows/positions from the args or (draft module) from the control block
  int row_base;                    // first row of this pass (rows >= kRowsMR run in two passes)
  float* out;
  int ldo;
  int layer;        // KV layer (QKV epilogue)
  void* kc;
  void* vc;
  const float* rcos;
  const float* rsin;
  int* kv_len;      // length word of `layer` to check/advance, or nullptr
  float* anchors;   // RESID: row-indexed anchor taps [row][m][d], or nullptr
  int anchor_idx;
  const float* slot_anchors;  // FC: anchor store [slot][m][d]
  Ctrl* ctrl;
  Geo g;
};

constexpr int kRowsKC = 512;  // K elements of each input row staged per pass (one 64-lane block of bf16)

template <typename WT, int EPI>
__global__ __launch_bounds__(kWG) void k_gemv_rows(const RowsGemv A) {
  __shared__ float xs[kRowsMR][kRowsKC];
  __shared__ float red[kWG / kWave];
  __shared__ float rstd[kRowsMR];
  __shared__ int rsrc[kRowsMR];  // FC: output row of input row r
  __shared__ int rcount;
  constexpr int VEC = WVec<WT>::N;
  constexpr int UPW = epi_pairs(EPI) ? 2 : 4;
  constexpr int UPT = UPW * (kWG / kWave);
  const Geo& g = A.g;
  const Ctrl* __restrict__ C = A.ctrl;
  if (A.from_ctrl && !C->active) return;
  const int grp = blockIdx.y;
  const int ut = blockIdx.x;
  const int K = A.Kg[grp];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;

  // rows of this pass (a draft tree's rows come from its row table)
  const bool tree = A.from_ctrl && g.W > 1;
  const Tree* TR = tree_of(C);
  int Mtot = tree ? TR->nrows : A.from_ctrl ? (C->a + C->pending) : A.M_arg;
  const int pos0 = A.from_ctrl ? C->C : A.pos0_arg;
  int M = Mtot - A.row_base;
  if (M > kRowsMR) M = kRowsMR;
  if (A.rmode == RM_FC) {
    // rows whose depth uses pattern `grp`: trailing row i is at position C+i,
    // depth n for the committed-next row, else t - position
    if (threadIdx.x == 0) {
      // pass `row_base / kRowsMR` takes the matching rows row_base .. row_base + kRowsMR - 1
      int cnt = 0, seen = 0;
      for (int i = 0; i < Mtot; ++i) {
        const int dep = tree ? TR->row_depth[i] : pdm_row_depth(g, C, i, pos0 + i);
        if (g.fpat[dep] == grp) {
          if (seen >= A.row_base && cnt < kRowsMR) rsrc[cnt++] = i;
          ++seen;
        }
      }
      rcount = cnt;
    }
    __syncthreads();
    M = rcount;
  }
  if (M <= 0) return;
  if (A.kv_len && EPI == EPI_QKV && ut == 0 && threadIdx.x == 0 && A.row_base == 0) {
    int* len = A.kv_len + A.layer;
    if (*len != pos0) atomicOr(&A.ctrl->flags, SPD_FLAG_KVLEN);
    *len = pos0 + Mtot;
  }
  auto in_row = [&](int r) -> const float* {
    if (A.rmode == RM_FC) {
      const int i = rsrc[r];
      const int slot = tree ? TR->row_slot[i] : (pos0 + i) % g.nslots;
      return A.slot_anchors + (size_t)slot * g.m * g.d;
    }
    return A.x + (size_t)(A.row_base + r) * A.ldx;
  };
  if (A.gamma) {
    for (int r = 0; r < M; ++r) {
      const float s = row_rstd(in_row(r), K, g.eps, red);
      if (threadIdx.x == 0) rstd[r] = s;
    }
  }
  __syncthreads();

  int rows[4];
  bool ok[4];
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int u = ut * UPT + wave * UPW + j;
    int r0, r1;
    unit_rows<EPI>(g, A.N, u < A.units ? u : 0, r0, r1);
    if (epi_pairs(EPI)) {
      rows[2 * j] = r0;
      rows[2 * j + 1] = r1;
      ok[2 * j] = ok[2 * j + 1] = u < A.units;
    } else {
      rows[j] = r0;
      ok[j] = u < A.units;
    }
  }
  const WT* W = reinterpret_cast<const WT*>(A.W[grp]);
  const WT* p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = W + (size_t)rows[r] * K;
  float acc[4][kRowsMR];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int m = 0; m < kRowsMR; ++m) acc[r][m] = 0.f;

  for (int kc = 0; kc < K; kc += kRowsKC) {
    const int kn = min(kRowsKC, K - kc);
    __syncthreads();
    for (int r = 0; r < M; ++r) {
      const float* x = in_row(r) + kc;
      if (A.gamma) {
        const float s = rstd[r];
        for (int i = threadIdx.x; i < kn; i += kWG) xs[r][i] = x[i] * s * A.gamma[kc + i];
      } else {
        for (int i = threadIdx.x; i < kn; i += kWG) xs[r][i] = x[i];
      }
    }
    __syncthreads();
    for (int k0 = lane * VEC; k0 < kn; k0 += kWave * VEC) {
      float wv[4][VEC];
#pragma unroll
      for (int r = 0; r < 4; ++r) WVec<WT>::load(p[r] + kc + k0, wv[r]);
#pragma unroll
      for (int m = 0; m < kRowsMR; ++m) {
        if (m < M) {
          float xv[VEC];
#pragma unroll
          for (int e = 0; e < VEC; ++e) xv[e] = xs[m][k0 + e];
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[r][m] = fmaf(wv[r][e], xv[e], acc[r][m]);
        }
      }
    }
  }
  const int half = g.hd >> 1;
#pragma unroll
  for (int m = 0; m < kRowsMR; ++m) {
    if (m >= M) continue;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = wave_sum(acc[r][m]);
    if (lane < UPW) {
      const int j = lane;
      const int u = ut * UPT + wave * UPW + j;
      if (u < A.units) {
        const int orow = (A.rmode == RM_FC) ? rsrc[m] : (A.row_base + m);
        const int pos = tree ? TR->row_pos[orow] : pos0 + orow;
        if (EPI == EPI_QKV) {
          float a = sel4(v, 2 * j), b = sel4(v, 2 * j + 1);
          const int h = u / half, i = u - h * half;
          if (h < g.Hq + g.Hkv) rope_pair(a, b, A.rcos[(size_t)pos * half + i], A.rsin[(size_t)pos * half + i]);
          if (h < g.Hq) {
            float* q = A.out + (size_t)orow * A.ldo + (size_t)h * g.hd;
            q[i] = a;
            q[i + half] = b;
          } else {
            // a draft tree's row writes its key/values to every lane of its descendants
            const int lanes = tree ? TR->row_lanes[orow] : 1;
            const bool isk = h < g.Hq + g.Hkv;
            auto* cache = reinterpret_cast<WT*>(isk ? A.kc : A.vc);
            const int kvh = isk ? h - g.Hq : h - g.Hq - g.Hkv;
            const size_t i0 = isk ? k_index(g, A.layer, kvh, pos, i) : v_index(g, A.layer, kvh, pos, i);
            const size_t i1 = isk ? k_index(g, A.layer, kvh, pos, i + half) : v_index(g, A.layer, kvh, pos, i + half);
            for (int ln = 0; ln < kMaxW; ++ln) {
              if (!((lanes >> ln) & 1)) continue;
              cache[ln * g.lane_pkv + i0] = to_store<WT>(a);
              cache[ln * g.lane_pkv + i1] = to_store<WT>(b);
            }
          }
        } else if (EPI == EPI_SWIGLU) {
          A.out[(size_t)orow * A.ldo + u] = silu_mul(sel4(v, 2 * j), sel4(v, 2 * j + 1));
        } else if (EPI == EPI_RESID) {
          float* o = A.out + (size_t)orow * A.ldo;
          const float hn = o[u] + sel4(v, j);
          o[u] = hn;
          if (A.anchors && A.anchor_idx >= 0) A.anchors[((size_t)orow * g.m + A.anchor_idx) * g.d + u] = hn;
        } else {
          A.out[(size_t)orow * A.ldo + u] = sel4(v, j);
        }
      }
    }
  }
}

}  // namespace spd
