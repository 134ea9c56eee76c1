// Linear-attention layers of a hybrid target (gfx950).
//
// [RB] limitations and [TW] §11: the 4B/9B targets interleave one standard
// and three faster linear-attention layers per block of four.  The pages do
// not define the linear layer; reading taken (the same in the oracle): the
// textbook kernelised causal attention with feature map phi = elu + 1 over
// the layer's usual q/k/v (after RoPE, k and v as stored in the KV cache):
// per kv head a state S = sum_i phi(k_i) v_i^T [hd x hd] and z = sum_i
// phi(k_i) [hd], and for each query head o = phi(q)^T S / phi(q)^T z.
//
// The state after each position lives in a ring of nslots slots per layer,
// indexed by position: a token at position p reads slot p-1 and writes slot
// p, so a rejection that truncates to length j+1 finds the state after j in
// its slot (in-flight positions never reach j + nslots) and rollback costs
// nothing.  One kernel serves the stage step (one token per active group,
// each of its own layer) and the row paths (prefill chunks and the
// autoregressive decoder: consecutive positions of one layer, the state
// carried in registers); the per-position arithmetic is the same in both, so
// the autoregressive reference reproduces the pipeline's bits.
#pragma once

#include "common.h"

namespace spd {

enum LMode { LM_STAGE = 0, LM_ROWS = 1 };

// Ring slot of (layer, slot, kv head): S [hd][hd] row-major (row i = key
// feature, column j = value dimension), then z [hd]; all fp32.
__device__ __host__ __forceinline__ size_t lin_state_index(const Geo& g, int layer, int slot, int kvh) {
  return (((size_t)layer * g.nslots + slot) * g.Hkv + kvh) * (size_t)(g.hd * g.hd + g.hd);
}

__device__ __forceinline__ float elu_plus_one(float x) { return x > 0.f ? x + 1.f : expf(x); }

struct LinAttn {
  int mode;                   // LM_STAGE or LM_ROWS
  int layer[SPD_MAX_STAGES];  // stage: layer of each group; rows: layer[0]
  int stage[SPD_MAX_STAGES];  // stage: pipeline stage of each group (increasing)
  const void* kc;
  const void* vc;
  const float* q;             // [row][Hq * hd], after RoPE
  int ldq;
  float* o;                   // [row][Hq * hd]
  int ldo;
  float* state;               // ring [L][nslots][Hkv][hd * hd + hd]
  int pos0, nrows;            // rows: positions pos0 .. pos0 + nrows - 1
  int keep_from;              // rows: states kept for positions >= keep_from (and the last row)
  const Ctrl* ctrl;
  Geo g;
};

// Grid (Hkv, groups) for LM_STAGE, (Hkv, 1) for LM_ROWS; kWG threads.
template <typename KT, int HD>
__global__ __launch_bounds__(kWG) void k_linattn(const LinAttn A) {
  constexpr int R = kWG / HD;   // threads per value column
  constexpr int RI = HD / R;    // key-feature rows per thread
  __shared__ float phik[HD], vv[HD], zs[HD];
  __shared__ float phiq[kAttnQ][HD];
  __shared__ float part[R][kAttnQ][HD];
  __shared__ float den[kAttnQ];
  const Geo& g = A.g;
  const int kvh = blockIdx.x;
  const int G = g.Hq / g.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  const int j = tid % HD, pr = tid / HD, i0 = pr * RI;
  int layer, pos, row, nitems;
  if (A.mode == LM_STAGE) {
    const Ctrl* C = A.ctrl;
    if (!C->active) return;
    const int grp = blockIdx.y;
    if (A.stage[grp] >= C->a) return;
    layer = A.layer[grp];
    if (!layer_is_linear(g, layer)) return;
    pos = C->t - A.stage[grp];
    row = grp;
    nitems = 1;
  } else {
    layer = A.layer[0];
    pos = A.pos0;
    row = 0;
    nitems = A.nrows;
  }
  const KT* kc = reinterpret_cast<const KT*>(A.kc);
  const KT* vc = reinterpret_cast<const KT*>(A.vc);
  // state after position pos - 1 (zero before the first position)
  float S[RI];
  float z = 0.f;
  if (pos > 0) {
    const float* sp = A.state + lin_state_index(g, layer, (pos - 1) % g.nslots, kvh);
#pragma unroll
    for (int r = 0; r < RI; ++r) S[r] = sp[(size_t)(i0 + r) * HD + j];
    if (tid < HD) z = sp[HD * HD + tid];
  } else {
#pragma unroll
    for (int r = 0; r < RI; ++r) S[r] = 0.f;
  }
  for (int it = 0; it < nitems; ++it, ++pos, ++row) {
    __syncthreads();  // the previous position's shared values are consumed
    if (tid < HD) {
      phik[tid] = elu_plus_one(from_store(kc[k_index(g, layer, kvh, pos, tid)]));
      vv[tid] = from_store(vc[v_index(g, layer, kvh, pos, tid)]);
    }
    for (int x = tid; x < G * HD; x += kWG) {
      const int hq = x / HD, c = x - hq * HD;
      phiq[hq][c] = elu_plus_one(A.q[(size_t)row * A.ldq + (size_t)(kvh * G + hq) * HD + c]);
    }
    __syncthreads();
    // S += phi(k) v^T, z += phi(k)
    const float vj = vv[j];
#pragma unroll
    for (int r = 0; r < RI; ++r) S[r] = fmaf(phik[i0 + r], vj, S[r]);
    if (tid < HD) {
      z = z + phik[tid];
      zs[tid] = z;
    }
    // numerators: this thread's rows of column j, per query head, in row order
    for (int hq = 0; hq < G; ++hq) {
      float acc = 0.f;
#pragma unroll
      for (int r = 0; r < RI; ++r) acc = fmaf(phiq[hq][i0 + r], S[r], acc);
      part[pr][hq][j] = acc;
    }
    __syncthreads();
    // denominators phi(q) . z: one wave per query head
    for (int hq = wave; hq < G; hq += kWG / kWave) {
      float s = 0.f;
      for (int c = lane; c < HD; c += kWave) s = fmaf(phiq[hq][c], zs[c], s);
      s = wave_sum(s);
      if (lane == 0) den[hq] = s;
    }
    __syncthreads();
    for (int x = tid; x < G * HD; x += kWG) {
      const int hq = x / HD, c = x - hq * HD;
      float num = part[0][hq][c];
#pragma unroll
      for (int p = 1; p < R; ++p) num += part[p][hq][c];
      A.o[(size_t)row * A.ldo + (size_t)(kvh * G + hq) * HD + c] = num / den[hq];
    }
    // the state after this position goes to its ring slot when it can be read
    // again: always in the stage step; in a row pass for the last row (the
    // next pass starts from it) and for positions a rollback may return to
    if (A.mode == LM_STAGE || it == nitems - 1 || pos >= A.keep_from) {
      float* sn = A.state + lin_state_index(g, layer, pos % g.nslots, kvh);
#pragma unroll
      for (int r = 0; r < RI; ++r) sn[(size_t)(i0 + r) * HD + j] = S[r];
      if (tid < HD) sn[HD * HD + tid] = z;
    }
  }
}

}  // namespace spd
