// Internal declarations shared by the libspd HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spd.h"

namespace spd {

constexpr int kWG = 256;          // threads per workgroup for the streaming kernels
constexpr int kWave = 64;         // CDNA wavefront
constexpr int kSplit = 256;       // attention positions per split (one per thread)
constexpr int kMaxQ = 16;         // query vectors per attention workgroup
constexpr int kRowsMR = 16;       // activation rows per pass of the row-batched GEMV
constexpr int kGemvRowsPerWave = 4;
constexpr int kGemvRowsPerWG = kGemvRowsPerWave * (kWG / kWave);  // 16

// Device control block.  Written by the entry kernel (cycle state), the
// verification kernel (r_*, reseed, seed_*, pend_next, emitted, done) and the
// draft finalisation kernel (r_draft, r_raw, C); every field has one writer
// per cycle, and each cycle's readers run after that writer.
struct Ctrl {
  int32_t t;          // newest in-flight position (this cycle's seed)
  int32_t a;          // occupancy after entry
  int32_t pending;    // this cycle commits the full-depth row at position C
  int32_t C;          // PDM committed length
  int32_t emitted;    // tokens emitted (incl. the prefill token)
  int32_t done;       // emitted == max_new
  int32_t active;     // this cycle does work
  int32_t cycle;      // cycles executed
  int32_t reseed;     // next entry starts an empty pipeline at (seed_tok, seed_pos)
  int32_t seed_tok;
  int32_t seed_pos;
  int32_t pend_next;  // the next cycle has a row to commit
  int32_t r_exit;     // last cycle: exit position or -1
  int32_t r_accept;
  int32_t r_y;
  int32_t r_draft;    // last cycle: draft for t+1
  int32_t r_raw;      // last cycle: PDM argmax / draw
  uint32_t flags;     // accumulated SPD_FLAG_*
  int32_t ar_pos;     // position of the token the AR decoder processes next
  int32_t launches;   // cycles enqueued (executed or idle): selects the record slot
  int32_t rec_slot;   // record slot of the current cycle
  int32_t pad[11];
};

struct ArgPair {
  float v;
  int32_t i;
};

// ---- draft trees ([RB] prerequisites "draft tree"; [PL] appendix B) --------
// The tokens in flight form a tree: at most W nodes per in-flight position,
// one at the oldest.  Node slot = (position mod nslots) * W + phys; the ranks
// of the live nodes at a position map to phys indices through rk.  Every
// node's target key/values go to the KV lanes of its descendant leaves (one
// full cache copy per lane), so each node attends to committed prefix +
// ancestors + itself in its own lane with the single-chain arithmetic.
constexpr int kMaxW = 4;
constexpr int kMaxTreeSlots = (SPD_MAX_STAGES + 1) * kMaxW;
constexpr int kMaxTreeRows = 32;
constexpr int kMaxCand = kMaxW * kMaxW + 1;

struct Tree {
  int32_t cnt[SPD_MAX_STAGES + 1];         // live nodes per position slot
  int32_t rk[SPD_MAX_STAGES + 1][kMaxW];   // phys index of rank r at a position slot
  int32_t tok[kMaxTreeSlots];
  int32_t parent[kMaxTreeSlots];           // node slot of the parent, -1: none
  int32_t lanes[kMaxTreeSlots];            // KV lanes (bitmask) its key/values go to
  int32_t lane[kMaxTreeSlots];             // the lane its attention reads
  double logq[kMaxTreeSlots];              // log Q of its token under its parent's draft
  // candidates of the last draft step, ranked (leaf node slot, token, log Q)
  int32_t ncand;
  int32_t cand_leaf[kMaxCand];
  int32_t cand_tok[kMaxCand];
  double cand_lq[kMaxCand];
  // lane copies the entry asked for: positions copy_lo..copy_hi of every layer
  int32_t ncopy, copy_lo, copy_hi;
  int32_t copy_src[kMaxW], copy_dst[kMaxW];
  // draft-module rows of the cycle: the committed-next row, then the nodes
  int32_t nrows, nleaves;
  int32_t row_slot[kMaxTreeRows], row_pos[kMaxTreeRows], row_depth[kMaxTreeRows];
  int32_t row_lanes[kMaxTreeRows], row_lane[kMaxTreeRows];
  int32_t exit_slot;   // slot of the oldest node (exits when the pipeline is full)
  int32_t pend_slot;   // slot of the exited node whose draft row is committed this cycle
  int32_t last_exit;   // slot of the node that exited last (-1: none)
};

// A token id from an argmax/draw, forced into [0, V); flags non-finite input.
__device__ __forceinline__ int valid_token(int y, int V, uint32_t* flags) {
  if (y < 0 || y >= V) {
    atomicOr(flags, SPD_FLAG_BADTOKEN);
    return 0;
  }
  return y;
}

__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 16 bytes of weights as floats: 8 bf16 or 4 fp32 elements.
template <typename WT>
struct WVec;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <>
struct WVec<uint16_t> {
  static constexpr int N = 8;
  typedef u32x4 Raw;
  __device__ __forceinline__ static Raw ld(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ static void cvt(const Raw& v, float* out) {
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xFFFF0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xFFFF0000u);
    out[4] = __uint_as_float(v.z << 16);
    out[5] = __uint_as_float(v.z & 0xFFFF0000u);
    out[6] = __uint_as_float(v.w << 16);
    out[7] = __uint_as_float(v.w & 0xFFFF0000u);
  }
  __device__ __forceinline__ static void load(const uint16_t* p, float* out) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    out[0] = __uint_as_float(v.x << 16);
    out[1] = __uint_as_float(v.x & 0xFFFF0000u);
    out[2] = __uint_as_float(v.y << 16);
    out[3] = __uint_as_float(v.y & 0xFFFF0000u);
    out[4] = __uint_as_float(v.z << 16);
    out[5] = __uint_as_float(v.z & 0xFFFF0000u);
    out[6] = __uint_as_float(v.w << 16);
    out[7] = __uint_as_float(v.w & 0xFFFF0000u);
  }
};
template <>
struct WVec<float> {
  static constexpr int N = 4;
  typedef f32x4 Raw;
  __device__ __forceinline__ static Raw ld(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  }
  __device__ __forceinline__ static void cvt(const Raw& v, float* out) {
    out[0] = v.x;
    out[1] = v.y;
    out[2] = v.z;
    out[3] = v.w;
  }
  __device__ __forceinline__ static void load(const float* p, float* out) {
    f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    out[0] = v.x;
    out[1] = v.y;
    out[2] = v.z;
    out[3] = v.w;
  }
};

// Storage of KV-cache elements.
template <typename KT>
__device__ __forceinline__ KT to_store(float v);
template <>
__device__ __forceinline__ float to_store<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t to_store<uint16_t>(float v) { return f32_to_bf16_rne(v); }
__device__ __forceinline__ float from_store(float v) { return v; }
__device__ __forceinline__ float from_store(uint16_t v) { return bf16_bits_to_f32(v); }

// Butterfly sum over the 64 lanes; every lane ends with the identical value.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float v2 = __shfl_xor(v, o, 64);
    int i2 = __shfl_xor(i, o, 64);
    if (better(v2, i2, v, i)) {
      v = v2;
      i = i2;
    }
  }
}

// Block sum over kWG threads in a fixed order (waves 0,1,2,3); all threads
// get the same value.  `red` is kWG/kWave floats of shared memory.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x % kWave) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int i = 1; i < kWG / kWave; ++i) s += red[i];
  return s;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x % kWave) == 0) red[w] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int i = 1; i < kWG / kWave; ++i) s = fmaxf(s, red[i]);
  return s;
}

// Sum of squares of x[0..K) by kWG threads, fixed order; returns
// 1/sqrt(mean + eps).  Every kernel that normalises a row uses this, so the
// same row gets the same scale everywhere.
__device__ __forceinline__ float rstd_of(float sumsq, int K, float eps) {
  return 1.0f / sqrtf(sumsq / (float)K + eps);
}
__device__ __forceinline__ float row_rstd(const float* __restrict__ x, int K, float eps, float* red) {
  float s = 0.f;
  for (int i = threadIdx.x; i < K; i += kWG) s = fmaf(x[i], x[i], s);
  return rstd_of(block_sum(s, red), K, eps);
}

// Geometry of the engine, passed by value to kernels.
struct Geo {
  int L, d, Hq, Hkv, hd, F, V, n, Ls, m;
  int per;       // layers of the longest stage (sub-steps of a stage step)
  int nslots;    // n + 1: position-indexed ring of in-flight slots
  int ctx_cap;   // KV capacity (positions), multiple of kSplit
  int nsplit;    // ctx_cap / kSplit
  int qkv_rows;  // (Hq + 2 Hkv) hd
  int max_new;
  int max_ctx;   // positions must stay below this (uniform-table rows, KV capacity)
  int post;      // draft module on post-step features (SPD_SCHED_POST)
  int topk;      // sample mode: top-k truncation of P and Q (0: none)
  int attn_period;  // hybrid target: softmax attention iff layer % P == P - 1, else linear (0: all softmax)
  float eps;
  int W;            // draft-tree width (1: a single chain of drafts)
  long long lane_kv;   // elements between target KV lanes (tree mode)
  long long lane_pkv;  // elements between draft-module KV lanes (tree mode)
  int anchor_of_layer[SPD_MAX_LAYERS + 1];  // anchor index of boundary b, or -1
  int fpat[SPD_MAX_STAGES + 1];             // f(k) for k = 0..n
  int sstart[SPD_MAX_STAGES + 1];           // first layer of stage k; sstart[n] = L
};

// Hybrid target ([RB] limitations, [TW] §11: one standard and three linear
// attention layers per block of four): layer l is a linear-attention layer
// unless attn_period is 0 or l is the last layer of its block.
__device__ __host__ __forceinline__ bool layer_is_linear(const Geo& g, int layer) {
  return g.attn_period > 0 && (layer % g.attn_period) != g.attn_period - 1;
}

// The tree state sits right after the control block.
__device__ __host__ __forceinline__ Tree* tree_of(Ctrl* C) {
  return reinterpret_cast<Tree*>(reinterpret_cast<char*>(C) + sizeof(Ctrl));
}
__device__ __host__ __forceinline__ const Tree* tree_of(const Ctrl* C) {
  return reinterpret_cast<const Tree*>(reinterpret_cast<const char*>(C) + sizeof(Ctrl));
}
// Node slot of rank r at position p.
__device__ __forceinline__ int tree_slot(const Geo& g, const Tree* T, int p, int r) {
  const int ps = p % g.nslots;
  return ps * g.W + T->rk[ps][r];
}

// Depth (stages completed) of the feature of draft-module row i, position p.
// Pre-step ([PL] §3.3): the just-verified row (pending) at depth n, in-flight
// tokens at t - p (the newest at 0).  Post-step: every row one stage deeper,
// t - p + 1, the exiting token then being at depth n.
__device__ __forceinline__ int pdm_row_depth(const Geo& g, const Ctrl* C, int i, int p) {
  if (g.post) return C->t - p + 1;
  return (C->pending && i == 0) ? g.n : (C->t - p);
}

// KV-cache addressing.  K is stored [layer][kvh][hd/8][ctx][8]: eight
// consecutive head dims of one position are a 16-byte chunk and consecutive
// positions are consecutive chunks.  V is stored [layer][kvh][ctx/8][hd][8]:
// eight consecutive positions of one head dim are a 16-byte chunk.  These are
// the operand layouts of the attention kernels' 16-byte loads.
__device__ __forceinline__ size_t k_index(const Geo& g, int layer, int kvh, int pos, int dim) {
  return ((((size_t)layer * g.Hkv + kvh) * (g.hd / 8) + (dim >> 3)) * g.ctx_cap + pos) * 8 + (dim & 7);
}
__device__ __forceinline__ size_t v_index(const Geo& g, int layer, int kvh, int pos, int dim) {
  return ((((size_t)layer * g.Hkv + kvh) * (g.ctx_cap / 8) + (pos >> 3)) * g.hd + dim) * 8 + (pos & 7);
}

}  // namespace spd
