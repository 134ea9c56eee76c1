// Control kernels of the SPD cycle: entry (fork), verification + rollback,
// draft finalisation, and the small helpers of prefill / autoregressive decode.
#pragma once

#include "common.h"

namespace spd {

constexpr int kCtlThreads = 1024;

// Strided loops over global memory in the control kernels issue kBatch loads
// before the first is used: a loop body with one load and its use waits out
// one memory round trip per iteration.  Each thread still handles its
// elements in the same order.
constexpr int kBatch = 8;

// ---- block-wide helpers for 1024-thread kernels ----------------------------
__device__ __forceinline__ ArgPair block_argmax_parts(const ArgPair* parts, int nparts, ArgPair* sh) {
  float v = -INFINITY;
  int i = 0x7FFFFFFF;
  for (int k = threadIdx.x; k < nparts; k += kCtlThreads) {
    const ArgPair p = parts[k];
    if (better(p.v, p.i, v, i)) {
      v = p.v;
      i = p.i;
    }
  }
  wave_argmax(v, i);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = ArgPair{v, i};
  __syncthreads();
  ArgPair b = sh[0];
  for (int k = 1; k < kCtlThreads / kWave; ++k)
    if (better(sh[k].v, sh[k].i, b.v, b.i)) b = sh[k];
  __syncthreads();
  return b;
}

// ---- sampling: softmax weights and inverse-CDF draws ------------------------
// The vocabulary is cut into blocks of kCdfBlock consecutive ids, lane l of a
// wave owning ids 4l..4l+3 of a block (one 16-byte load per lane).  A lane's
// four weights are summed in id order in fp64, and an inclusive scan over the
// 64 lanes gives the running sums inside the block; its last lane is the block
// sum.  Blocks group into superblocks of 64 blocks, scanned the same way, and
// one wave scans the superblock sums.  The cumulative weight of an id is the
// sum of its superblock, block, lane and in-lane prefixes (all fp64), and a
// draw takes the smallest id whose cumulative weight exceeds u * total.  Every
// pass is coalesced, and the only serial steps are the three 64-wide scans of
// the search, done by one wave.
constexpr int kCdfPer = 4;
constexpr int kCdfBlock = kWave * kCdfPer;                  // 256 ids
constexpr int kCdfMaxBlocks = SPD_MAX_VOCAB / kCdfBlock;    // 4096
constexpr int kCdfMaxSuper = kCdfMaxBlocks / kWave;         // 64
constexpr int kCdfUnroll = 4;                               // blocks in flight per wave
constexpr int kCtlWaves = kCtlThreads / kWave;
static_assert(kCdfMaxSuper <= kWave, "one wave scans the superblock sums");

struct CdfShared {
  double bs[kCdfMaxBlocks];  // block sums
  double ss[kCdfMaxSuper];   // superblock sums
  double sinc[kCdfMaxSuper]; // inclusive scan of ss
  double total;
  int pick;
};

// Inclusive prefix sum over the 64 lanes of a wave (fp64, log-step).
__device__ __forceinline__ double wave_scan_d(double v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ double lane_sum4(const double x[4]) { return ((x[0] + x[1]) + x[2]) + x[3]; }

// Four consecutive floats p[v0..v0+3], zero at ids >= V.
__device__ __forceinline__ void load4(const float* p, int v0, int V, bool vec, float out[4]) {
  if (vec && v0 + 4 <= V) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(p + v0);
    out[0] = t.x;
    out[1] = t.y;
    out[2] = t.z;
    out[3] = t.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = (v0 + k < V) ? p[v0 + k] : 0.f;
  }
}
__device__ __forceinline__ bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Block sums of the weights given by w4(v0, x[4]) (the fp64 weights of ids
// v0..v0+3, zero beyond V) into bs: this wave takes blocks wave,
// wave + nwaves, ... with kCdfUnroll of them in flight.
template <typename W4>
__device__ __forceinline__ void cdf_block_pass(W4 w4, int V, double* bs, int wave, int nwaves) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nb = (V + kCdfBlock - 1) / kCdfBlock;
  for (int b0 = wave; b0 < nb; b0 += nwaves * kCdfUnroll) {
    double x[kCdfUnroll][4];
#pragma unroll
    for (int u = 0; u < kCdfUnroll; ++u) {
      const int b = b0 + u * nwaves;
      if (b < nb) {
        w4(b * kCdfBlock + lane * kCdfPer, x[u]);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[u][k] = 0.0;
      }
    }
#pragma unroll
    for (int u = 0; u < kCdfUnroll; ++u) {
      const int b = b0 + u * nwaves;
      const double s = wave_scan_d(lane_sum4(x[u]));
      if (lane == kWave - 1 && b < nb) bs[b] = s;
    }
  }
}

// From the block sums in S.bs: superblock sums, their inclusive scan and the
// total.  Ends with a barrier; S.total is then valid in every thread.
__device__ __forceinline__ void cdf_super_sums(int V, CdfShared& S) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nb = (V + kCdfBlock - 1) / kCdfBlock;
  const int nsb = (nb + kWave - 1) / kWave;
  for (int sb = wave; sb < nsb; sb += kCtlWaves) {
    const int b = sb * kWave + lane;
    const double s = wave_scan_d(b < nb ? S.bs[b] : 0.0);
    if (lane == kWave - 1) S.ss[sb] = s;
  }
  __syncthreads();
  if (wave == 0) {
    const double s = wave_scan_d(lane < nsb ? S.ss[lane] : 0.0);
    if (lane < nsb) S.sinc[lane] = s;
    if (lane == nsb - 1) S.total = s;
  }
  __syncthreads();
}

// The whole pass in one workgroup: block sums into S.bs, then the superblock
// sums and the total.  Ends with a barrier; S.total is then valid in every
// thread.
template <typename W4>
__device__ __forceinline__ void cdf_sums(W4 w4, int V, CdfShared& S) {
  cdf_block_pass(w4, V, S.bs, threadIdx.x / kWave, kCtlWaves);
  __syncthreads();
  cdf_super_sums(V, S);
}

// Highest set lane of a nonzero ballot.
__device__ __forceinline__ int last_lane(unsigned long long m) { return 63 - __clzll(m); }
__device__ __forceinline__ int first_lane(unsigned long long m) { return __ffsll(m) - 1; }

// Last id of block b with a positive weight (wave-uniform), or -1.
template <typename W4>
__device__ __forceinline__ int cdf_last_in_block(W4 w4, int b) {
  const int lane = threadIdx.x & (kWave - 1);
  double x[4];
  w4(b * kCdfBlock + lane * kCdfPer, x);
  int k_last = -1;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (x[k] > 0.0) k_last = k;
  const unsigned long long m = __ballot(k_last >= 0);
  if (m == 0) return -1;
  const int l = last_lane(m);
  return b * kCdfBlock + l * kCdfPer + __shfl(k_last, l, kWave);
}

// Last id with a positive weight (wave-uniform), or -1.
template <typename W4>
__device__ __forceinline__ int cdf_last_positive(W4 w4, int nb, const CdfShared& S) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nsb = (nb + kWave - 1) / kWave;
  unsigned long long m = __ballot(lane < nsb && S.ss[lane] > 0.0);
  if (m == 0) return -1;
  const int sb = last_lane(m);
  const int b = sb * kWave + lane;
  m = __ballot(b < nb && S.bs[b] > 0.0);
  if (m == 0) return -1;
  return cdf_last_in_block(w4, sb * kWave + last_lane(m));
}

// Smallest id whose cumulative weight exceeds thr, else the last id with a
// positive weight (thr at or beyond the total), else -1.  Called after
// cdf_sums with the same weights; run by wave 0, whose lanes all return it.
template <typename W4>
__device__ __forceinline__ int cdf_search_wave(W4 w4, int V, double thr, const CdfShared& S) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nb = (V + kCdfBlock - 1) / kCdfBlock;
  const int nsb = (nb + kWave - 1) / kWave;
  // superblock
  double inc = lane < nsb ? S.sinc[lane] : 0.0;
  unsigned long long m = __ballot(lane < nsb && inc > thr);
  if (m == 0) return cdf_last_positive(w4, nb, S);
  const int sb = first_lane(m);
  double base = sb > 0 ? S.sinc[sb - 1] : 0.0;
  // block within the superblock
  const int b = sb * kWave + lane;
  inc = wave_scan_d(b < nb ? S.bs[b] : 0.0);
  double exc = __shfl_up(inc, 1, kWave);
  if (lane == 0) exc = 0.0;
  m = __ballot(b < nb && base + inc > thr);
  int blk;
  if (m == 0) {  // rounding between the two levels: the last block with weight
    m = __ballot(b < nb && S.bs[b] > 0.0);
    if (m == 0) return cdf_last_positive(w4, nb, S);
    return cdf_last_in_block(w4, sb * kWave + last_lane(m));
  }
  const int bi = first_lane(m);
  blk = sb * kWave + bi;
  base = base + __shfl(exc, bi, kWave);
  // lane within the block
  double x[4];
  w4(blk * kCdfBlock + lane * kCdfPer, x);
  inc = wave_scan_d(lane_sum4(x));
  exc = __shfl_up(inc, 1, kWave);
  if (lane == 0) exc = 0.0;
  m = __ballot(base + inc > thr);
  if (m == 0) {
    const int r = cdf_last_in_block(w4, blk);
    return r >= 0 ? r : cdf_last_positive(w4, nb, S);
  }
  const int l = first_lane(m);
  // id within the lane
  double c = base + exc;
  int found = -1, k_last = -1;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    c += x[k];
    if (found < 0 && c > thr) found = k;
    if (x[k] > 0.0) k_last = k;
  }
  if (found < 0) found = k_last;  // rounding inside the lane
  found = __shfl(found, l, kWave);
  if (found < 0) {
    const int r = cdf_last_in_block(w4, blk);
    return r >= 0 ? r : cdf_last_positive(w4, nb, S);
  }
  return blk * kCdfBlock + l * kCdfPer + found;
}

// The draw by the whole workgroup: wave 0 searches, all threads get the id.
template <typename W4>
__device__ __forceinline__ int cdf_draw(W4 w4, int V, double u, CdfShared& S) {
  if (threadIdx.x < kWave) {
    const int r = cdf_search_wave(w4, V, u * S.total, S);
    if (threadIdx.x == 0) S.pick = r;
  }
  __syncthreads();
  const int r = S.pick;
  __syncthreads();
  return r;
}

// Softmax weights w_v = exp(l_v / T - max_v l_v / T) stored to `w` (fp32);
// their block sums go to S and the fp64 total Z = sum_v w_v is returned.
// `lmax` is max_v l_v.
// The softmax weights of ids v0..v0+3 (stored to w, returned in x as fp64).
struct SoftmaxWeights4 {
  const float* logits;
  float* w;
  int V;
  float T, mt;
  bool vec;
  __device__ void operator()(int v0, double x[4]) const {
    float l[4];
    load4(logits, v0, V, vec, l);
    float e[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lt = (T == 1.0f) ? l[k] : l[k] / T;
      e[k] = (v0 + k < V) ? expf(lt - mt) : 0.f;
      x[k] = (double)e[k];
    }
    if (vec && v0 + 4 <= V) {
      *reinterpret_cast<f32x4*>(w + v0) = f32x4{e[0], e[1], e[2], e[3]};
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (v0 + k < V) w[v0 + k] = e[k];
    }
  }
};
__device__ __forceinline__ SoftmaxWeights4 softmax4(const float* logits, float* w, int V, float T, float lmax) {
  return SoftmaxWeights4{logits, w, V, T, (T == 1.0f) ? lmax : lmax / T, aligned16(logits) && aligned16(w)};
}

__device__ __forceinline__ double softmax_weights(const float* logits, float* w, int V, float T, float lmax,
                                                  CdfShared& S) {
  cdf_sums(softmax4(logits, w, V, T, lmax), V, S);
  return S.total;
}

// Softmax weights and their block sums over many workgroups (the dense
// sampling path of the cycle): wave w of workgroup b takes block 4b + w.
// The max logit comes from the head's per-workgroup argmax parts; the
// weights go to `w` or, with `qring`, to the ring slot of position t + 1.
// The finalisation and verification kernels then start from the block sums.
struct SoftmaxArgs {
  const ArgPair* parts;
  int nparts;
  const float* logits;
  float* w;
  float* qring;
  double* bs;
  int exit_only;  // only when a token exits this cycle
  float temp;
  const Ctrl* ctrl;
  Geo g;
};

__global__ __launch_bounds__(kWG) void k_softmax_blocks(const SoftmaxArgs A) {
  __shared__ float red[kWG / kWave];
  const Ctrl* C = A.ctrl;
  const Geo& g = A.g;
  if (!C->active) return;
  if (A.exit_only && C->a != g.n) return;
  float v = -INFINITY;
  for (int k = threadIdx.x; k < A.nparts; k += kWG) v = fmaxf(v, A.parts[k].v);
  const float lmax = block_max(v, red);
  float* w = A.qring ? A.qring + (size_t)((C->t + 1) % g.nslots) * g.V : A.w;
  const int nwaves = kWG / kWave;
  cdf_block_pass(softmax4(A.logits, w, g.V, A.temp, lmax), g.V, A.bs,
                 blockIdx.x * nwaves + (int)(threadIdx.x / kWave), gridDim.x * nwaves);
}

// Reads the stored fp32 weights back as the fp64 weights of a draw.
struct StoredWeights {
  const float* w;
  int V;
  bool vec;
  __device__ void operator()(int v0, double x[4]) const {
    float f[4];
    load4(w, v0, V, vec, f);
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (double)f[k];
  }
};

// ---- top-k sampling ---------------------------------------------------------
// Only the k largest logits keep their weight (equal logits rank by the lower
// id).  An element's rank key is 64 bits: an order-preserving image of its
// logit above the complement of its id, so a larger key is a higher logit or,
// on a tie, a lower id; 0 is "no element".  Each wave keeps the 64 best keys
// it has seen as one sorted register per lane and streams its share of the
// vocabulary: an element enters only if it beats the wave's current k-th key
// (after the first blocks almost none does); a few entrants are shifted in
// one at a time, many are sorted and merged.  Wave 0 then merges the 16 wave
// lists; the k kept (id, logit) pairs end up in wave 0's lanes in ascending id
// order, so weights, running sums and the draw are register work.
constexpr int kTopK = SPD_MAX_TOPK;
static_assert(kTopK == kWave, "one kept entry per lane of a wave");

// Draft distribution Q of one slot under top-k: the kept ids in ascending
// order, their fp32 weights and the count (its fp64 sum is kept in qz).
struct SparseQ {
  int32_t ids[kTopK];
  float w[kTopK];
  int32_t cnt;
  int32_t pad[3];
};

struct TopkShared {
  unsigned long long lists[kCtlWaves][kWave];
};

// Order-preserving unsigned image of a float; -0 ranks with +0, NaN lowest.
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;
  if (f == 0.f) f = 0.f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ unsigned long long rank_key(float l, int id) {
  return ((unsigned long long)order_key(l) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ int rank_key_id(unsigned long long k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }
__device__ __forceinline__ unsigned long long umin64(unsigned long long a, unsigned long long b) { return a < b ? a : b; }

// Bitonic sort of one value per lane, descending over the 64 lanes.
__device__ __forceinline__ unsigned long long wave_sort_desc(unsigned long long v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const unsigned long long o = __shfl_xor(v, stride, kWave);
      const bool desc = (lane & size) == 0;
      const bool lower = (lane & stride) == 0;
      v = (lower == desc) ? umax64(v, o) : umin64(v, o);
    }
  return v;
}

// The 64 largest of two descending lane-sorted lists, descending.
__device__ __forceinline__ unsigned long long wave_merge_desc(unsigned long long a, unsigned long long b) {
  const int lane = threadIdx.x & (kWave - 1);
  unsigned long long v = umax64(a, __shfl(b, kWave - 1 - lane, kWave));  // bitonic
#pragma unroll
  for (int stride = kWave / 2; stride > 0; stride >>= 1) {
    const unsigned long long o = __shfl_xor(v, stride, kWave);
    v = ((lane & stride) == 0) ? umax64(v, o) : umin64(v, o);
  }
  return v;
}

// Key x into the descending list (the smallest entry drops out).
__device__ __forceinline__ unsigned long long wave_insert_desc(unsigned long long lst, unsigned long long x) {
  const int lane = threadIdx.x & (kWave - 1);
  const int pos = __popcll(__ballot(lst > x));
  const unsigned long long up = __shfl_up(lst, 1, kWave);
  return lane < pos ? lst : (lane == pos ? x : up);
}

// One round of offers to a wave's list: each lane's key that beats the
// list's k-th key enters (a few are shifted in one at a time, more than 8 are
// sorted and merged).
__device__ __forceinline__ void wave_topk_offer(unsigned long long& lst, unsigned long long& thr,
                                                unsigned long long key, int k) {
  const unsigned long long cand = key > thr ? key : 0ull;
  unsigned long long m = __ballot(cand != 0ull);
  if (m == 0ull) return;
  if (__popcll(m) > 8) {
    lst = wave_merge_desc(lst, wave_sort_desc(cand));
  } else {
    while (m) {
      const int src = first_lane(m);
      m &= m - 1;
      lst = wave_insert_desc(lst, __shfl(cand, src, kWave));
    }
  }
  thr = __shfl(lst, k - 1, kWave);
}

// Wave w of nwaves streams blocks b_lo + w, b_lo + w + nwaves, ... (below
// b_hi) of kCdfBlock ids (lane l: ids 4l..4l+3) and keeps the best 64 keys it
// sees (at least the best k).
__device__ __forceinline__ unsigned long long wave_topk_pass(const float* logits, int V, int k, int b_lo, int b_hi,
                                                             int w, int nwaves) {
  const int lane = threadIdx.x & (kWave - 1);
  const bool vec = aligned16(logits);
  unsigned long long lst = 0ull;
  unsigned long long thr = 0ull;  // the list's k-th key
  for (int b0 = b_lo + w; b0 < b_hi; b0 += nwaves * kCdfUnroll) {
    float l[kCdfUnroll][4];
#pragma unroll
    for (int u = 0; u < kCdfUnroll; ++u) {
      const int b = b0 + u * nwaves;
      if (b < b_hi) {
        load4(logits, b * kCdfBlock + lane * kCdfPer, V, vec, l[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) l[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kCdfUnroll; ++u) {
      const int b = b0 + u * nwaves;
      if (b >= b_hi) break;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int id = b * kCdfBlock + lane * kCdfPer + e;
        wave_topk_offer(lst, thr, id < V ? rank_key(l[u][e], id) : 0ull, k);
      }
    }
  }
  return lst;
}

// The same over candidate keys cand[0, n) (0: no element), kCdfBlock keys
// per wave step (lane l: keys 4l..4l+3 of the step).
__device__ __forceinline__ unsigned long long wave_topk_keys(const unsigned long long* cand, int n, int k, int w,
                                                             int nwaves) {
  const int lane = threadIdx.x & (kWave - 1);
  unsigned long long lst = 0ull;
  unsigned long long thr = 0ull;
  for (int i0 = w * kCdfBlock; i0 < n; i0 += nwaves * kCdfBlock) {
    unsigned long long c[kCdfPer];
#pragma unroll
    for (int e = 0; e < kCdfPer; ++e) {
      const int i = i0 + lane * kCdfPer + e;
      c[e] = i < n ? cand[i] : 0ull;
    }
#pragma unroll
    for (int e = 0; e < kCdfPer; ++e) wave_topk_offer(lst, thr, c[e], k);
  }
  return lst;
}

// Candidate pass over many workgroups: workgroup b keeps the best 64 keys of
// blocks [b * kTopkBlocksPerWG, (b + 1) * kTopkBlocksPerWG) in cand[b][0..63]
// (descending, 0 for missing entries).  The k best of all candidates are the
// k best of the vocabulary, because every workgroup keeps at least its k
// best: the final selection over the candidates gives the same set as a pass
// over the logits.
constexpr int kTopkBlocksPerWG = 16;  // 4096 ids per workgroup

struct TopkArgs {
  const float* logits;
  unsigned long long* cand;  // [gridDim.x][kWave]
  int exit_only;             // only when a token exits this cycle
  const Ctrl* ctrl;
  Geo g;
};

__global__ __launch_bounds__(kWG) void k_topk_blocks(const TopkArgs A) {
  __shared__ unsigned long long lists[kWG / kWave][kWave];
  const Ctrl* C = A.ctrl;
  const Geo& g = A.g;
  if (!C->active) return;
  if (A.exit_only && C->a != g.n) return;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nb = (g.V + kCdfBlock - 1) / kCdfBlock;
  const int b_lo = blockIdx.x * kTopkBlocksPerWG;
  const int b_hi = min(nb, b_lo + kTopkBlocksPerWG);
  lists[wave][lane] = wave_topk_pass(A.logits, g.V, g.topk, b_lo, b_hi, wave, kWG / kWave);
  __syncthreads();
  if (wave == 0) {
    unsigned long long all = lists[0][lane];
#pragma unroll
    for (int w = 1; w < kWG / kWave; ++w) all = wave_merge_desc(all, lists[w][lane]);
    A.cand[(size_t)blockIdx.x * kWave + lane] = all;
  }
}

// Wave 0 merges the kCtlWaves lists `lst` (one per wave, called by every
// thread); lane i < k of wave 0 ends with the i-th kept id in ascending id
// order and its logit (lanes >= k, and every other thread: id -1).
__device__ __forceinline__ void topk_merge(unsigned long long lst, int k, TopkShared& S, int& id, float& val) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  S.lists[wave][lane] = lst;
  __syncthreads();
  id = -1;
  val = 0.f;
  if (wave == 0) {
    unsigned long long all = S.lists[0][lane];
    for (int w = 1; w < kCtlWaves; ++w) all = wave_merge_desc(all, S.lists[w][lane]);
    // the k best, re-sorted by ascending id (descending complement), logit carried along
    const bool kept = lane < k && all != 0ull;
    const uint32_t cid = kept ? (uint32_t)all : 0u;  // 0xFFFFFFFF - id
    const unsigned long long byid = kept ? (((unsigned long long)cid << 32) | (all >> 32)) : 0ull;
    const unsigned long long s = wave_sort_desc(byid);
    if (s != 0ull) {
      id = (int)(0xFFFFFFFFu - (uint32_t)(s >> 32));
      val = order_value((uint32_t)s);
    }
  }
  __syncthreads();
}

// Top-k of logits[0, V) by the kCtlWaves waves of the workgroup (results as
// topk_merge).  `k` <= min(64, V).
__device__ __forceinline__ void topk_select(const float* logits, int V, int k, TopkShared& S, int& id,
                                            float& val) {
  const int nb = (V + kCdfBlock - 1) / kCdfBlock;
  topk_merge(wave_topk_pass(logits, V, k, 0, nb, threadIdx.x / kWave, kCtlWaves), k, S, id, val);
}

// The same selection from k_topk_blocks' candidate keys cand[0, n).
__device__ __forceinline__ void topk_select_keys(const unsigned long long* cand, int n, int k, TopkShared& S,
                                                 int& id, float& val) {
  topk_merge(wave_topk_keys(cand, n, k, threadIdx.x / kWave, kCtlWaves), k, S, id, val);
}

// In wave 0 after topk_select: fp32 weight exp(l/T - lmax/T) of the lane's
// kept id (0 for empty lanes), as in the dense softmax.
__device__ __forceinline__ float topk_weight(int id, float val, float T, float lmax) {
  if (id < 0) return 0.f;
  const float mt = (T == 1.0f) ? lmax : lmax / T;
  const float lt = (T == 1.0f) ? val : val / T;
  return expf(lt - mt);
}

// In wave 0: the smallest kept id whose running sum (ascending ids, fp64)
// exceeds u * total, else the last id with positive weight, else -1; also
// returns the total.  x = the lane's weight (0 for empty lanes).
__device__ __forceinline__ int topk_draw(int id, double x, double u, double* total) {
  const double inc = wave_scan_d(x);
  const double tot = __shfl(inc, kWave - 1, kWave);
  if (total) *total = tot;
  const double thr = u * tot;
  unsigned long long m = __ballot(id >= 0 && inc > thr);
  if (m) return __shfl(id, first_lane(m), kWave);
  m = __ballot(id >= 0 && x > 0.0);
  if (m) return __shfl(id, last_lane(m), kWave);
  return -1;
}

// ---- tables -----------------------------------------------------------------
// cos/sin of pos * base^(-2i/hd), computed in fp64 and rounded to fp32.
__global__ void k_rope_table(float* cosv, float* sinv, int ctx, int hd, double base) {
  const int half = hd / 2;
  const size_t n = (size_t)ctx * half;
  for (size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x; idx < n; idx += (size_t)gridDim.x * blockDim.x) {
    const int pos = (int)(idx / half), i = (int)(idx % half);
    const double theta = pow(base, -2.0 * (double)i / (double)hd);
    const double ang = (double)pos * theta;
    cosv[idx] = (float)cos(ang);
    sinv[idx] = (float)sin(ang);
  }
}

// ---- cycle entry (A0/A1): resolve the seed, fork state, embed ---------------
template <typename WT>
__global__ __launch_bounds__(kWG) void k_entry(Ctrl* C, const Geo g, int32_t* tokens, const WT* embed,
                                               float* hslots, float* anchors, spd_cycle_rec* ring,
                                               int log_cap) {
  __shared__ int s_tok, s_pos, s_ok;
  if (threadIdx.x == 0) {
    // every enqueued cycle takes the next record slot, idle or not, so the
    // host knows where the records of its calls are
    const int cyc = C->launches;
    C->launches = cyc + 1;
    C->rec_slot = cyc % log_cap;
    spd_cycle_rec* r = ring + C->rec_slot;
    r->cycle = cyc;
    r->pdm_argmax = r->draft = r->exit_pos = r->target_token = -1;
    r->accepted = -1;
    r->accepted_rank = -1;
    r->nodes = 0;
    r->n_new = 0;
    for (int k = 0; k < SPD_MAX_WIDTH; ++k) r->new_parent[k] = r->new_token[k] = -1;
    s_ok = 0;
    if (C->done) {
      C->active = 0;
      r->t = -1;
      r->occupancy = 0;
      r->pending_row = 0;
      r->pdm_len = C->C;
      r->emitted = C->emitted;
      r->flags = SPD_FLAG_IDLE;
    } else {
      int tok, pos, a;
      r->new_parent[0] = C->reseed ? -1 : 0;
      if (C->reseed) {
        tok = C->seed_tok;
        pos = C->seed_pos;
        a = 1;
        C->reseed = 0;
      } else {
        tok = C->r_draft;
        pos = C->t + 1;
        a = C->a - (C->r_exit >= 0 ? 1 : 0) + 1;
      }
      uint32_t fl = 0;
      if (a < 1 || a > g.n) fl |= SPD_FLAG_OCCUPANCY;
      if (pos + 1 >= g.max_ctx) fl |= SPD_FLAG_CTX;
      C->pending = C->pend_next;
      C->t = pos;
      C->a = a;
      C->cycle += 1;
      C->flags |= fl;
      r->t = pos;
      r->occupancy = a;
      r->pending_row = C->pending;
      r->flags = fl;
      r->nodes = a;
      r->n_new = 1;
      r->new_token[0] = tok;
      if (fl) {
        C->active = 0;
        C->done = 1;
      } else {
        C->active = 1;
        tokens[pos] = tok;
        s_tok = tok;
        s_pos = pos;
        s_ok = 1;
      }
    }
  }
  __syncthreads();
  // the record's per-layer lengths beyond L stay zero (the verification
  // kernel fills the first L), so records never carry stale ring contents
  {
    spd_cycle_rec* r = ring + C->rec_slot;
    for (int l = threadIdx.x; l < SPD_MAX_LAYERS; l += kWG) r->kv_len[l] = 0;
  }
  if (!s_ok) return;
  const int slot = s_pos % g.nslots;
  const WT* e = embed + (size_t)s_tok * g.d;
  for (int i0 = threadIdx.x; i0 < g.d; i0 += kBatch * kWG) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = (i0 + u * kWG < g.d) ? from_store(e[i0 + u * kWG]) : 0.f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * kWG;
      if (i >= g.d) break;
      hslots[(size_t)slot * g.d + i] = v[u];
      anchors[((size_t)slot * g.m + 0) * g.d + i] = v[u];
    }
  }
}

struct VerifyArgs {
  const ArgPair* parts;
  int nparts;
  const double* bs;     // dense sampling: block sums of P from k_softmax_blocks (weights already in pw)
  const unsigned long long* tk;  // top-k: k_topk_blocks' candidate keys of P (ntk of them), or null
  int ntk;
  const float* logits;  // [V] target logits of the exiting token
  float* pw;            // [V] scratch: target softmax weights (sample mode)
  const int32_t* dring; // drafts by position mod nslots
  const float* qring;   // [nslots][V] draft softmax weights (sample mode)
  const double* qz;     // [nslots] their sums
  const float* uni;     // [ctx][SPD_U_COUNT]
  int mode;
  float temp;
  int32_t* tokens;
  int32_t* kv_len;
  spd_cycle_rec* ring;
  Ctrl* ctrl;
  Geo g;
};

// ---- verification (A5) + accept / three-step rollback (A6) -----------------
__global__ __launch_bounds__(kCtlThreads) void k_verify(const VerifyArgs A) {
  __shared__ ArgPair sh_ap[kCtlThreads / kWave];
  __shared__ CdfShared S;
  __shared__ TopkShared TS;
  __shared__ int s_y, s_acc;
  Ctrl* C = A.ctrl;
  const Geo& g = A.g;
  if (!C->active) return;
  spd_cycle_rec* rec = A.ring + C->rec_slot;
  const bool exit = (C->a == g.n);
  if (!exit) {
    __syncthreads();
    if (threadIdx.x == 0) {
      C->r_exit = -1;
      C->r_accept = -1;
      C->pend_next = 0;
      rec->emitted = C->emitted;
      rec->flags |= C->flags;
    }
    for (int l = threadIdx.x; l < g.L; l += kCtlThreads) rec->kv_len[l] = A.kv_len[l];
    return;
  }
  const int j = C->t - (g.n - 1);
  const int nslot = (j + 1) % g.nslots;
  const int xd = A.dring[nslot];
  const ArgPair best = block_argmax_parts(A.parts, A.nparts, sh_ap);
  if (A.mode == SPD_MODE_GREEDY) {
    if (threadIdx.x == 0) {
      s_y = best.i;
      s_acc = (xd == best.i);
    }
  } else if (g.topk > 0) {
    // P and Q truncated to their top k: P from this exit's logits, Q as drafted
    int pid;
    float pl;
    if (A.tk)
      topk_select_keys(A.tk, A.ntk, g.topk, TS, pid, pl);
    else
      topk_select(A.logits, g.V, g.topk, TS, pid, pl);
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      const float pwf = topk_weight(pid, pl, A.temp, best.v);
      const double pZ = __shfl(wave_scan_d((double)pwf), kWave - 1, kWave);
      const SparseQ* Qs = reinterpret_cast<const SparseQ*>(A.qring) + nslot;
      const int qn = Qs->cnt;
      const int qid = lane < qn ? Qs->ids[lane] : -1;
      const float qwf = lane < qn ? Qs->w[lane] : 0.f;
      const double qZ = A.qz[nslot];
      const unsigned long long mp = __ballot(pid >= 0 && pid == xd);
      const unsigned long long mq = __ballot(qid >= 0 && qid == xd);
      const double Px = mp ? (double)__shfl(pwf, first_lane(mp), kWave) / pZ : 0.0;
      const double Qx = mq ? (double)__shfl(qwf, first_lane(mq), kWave) / qZ : 0.0;
      const double u_acc = A.uni[(size_t)(j + 1) * SPD_U_COUNT + SPD_U_ACCEPT];
      const bool acc = u_acc * Qx < Px;
      int y = xd;
      if (!acc) {
        // max(0, P - Q) on P's kept ids, scaled by pZ * qZ > 0
        float qv = 0.f;
        for (int jj = 0; jj < qn; ++jj) {
          const int oid = __shfl(qid, jj, kWave);
          const float ow = __shfl(qwf, jj, kWave);
          if (oid == pid) qv = ow;
        }
        const double r = pid >= 0 ? fma((double)pwf, qZ, -((double)qv * pZ)) : 0.0;
        const double u_res = A.uni[(size_t)(j + 1) * SPD_U_COUNT + SPD_U_RESAMPLE];
        y = topk_draw(pid, r > 0.0 ? r : 0.0, u_res, nullptr);
      }
      if (lane == 0) {
        s_y = y;
        s_acc = acc ? 1 : 0;
      }
    }
  } else {
    // P = softmax(logits / T); accept iff u * Q(x) < P(x); else redraw from max(0, P - Q)
    double pZ;
    if (A.bs) {
      const int nb = (g.V + kCdfBlock - 1) / kCdfBlock;
      for (int b = threadIdx.x; b < nb; b += kCtlThreads) S.bs[b] = A.bs[b];
      __syncthreads();
      cdf_super_sums(g.V, S);
      pZ = S.total;
    } else {
      pZ = softmax_weights(A.logits, A.pw, g.V, A.temp, best.v, S);
    }
    const float* qw = A.qring + (size_t)nslot * g.V;
    const double qZ = A.qz[nslot];
    const double u_acc = A.uni[(size_t)(j + 1) * SPD_U_COUNT + SPD_U_ACCEPT];
    const double Px = (double)A.pw[xd] / pZ;
    const double Qx = (double)qw[xd] / qZ;
    const bool acc = u_acc * Qx < Px;
    int y = xd;
    if (!acc) {
      // max(0, P - Q) scaled by pZ * qZ > 0, which leaves the draw unchanged
      const double u_res = A.uni[(size_t)(j + 1) * SPD_U_COUNT + SPD_U_RESAMPLE];
      const float* pw = A.pw;
      const int V = g.V;
      const bool vec = aligned16(pw) && aligned16(qw);
      auto r4 = [&](int v0, double x[4]) {
        float p[4], q[4];
        load4(pw, v0, V, vec, p);
        load4(qw, v0, V, vec, q);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const double r = fma((double)p[k], qZ, -((double)q[k] * pZ));
          x[k] = r > 0.0 ? r : 0.0;
        }
      };
      cdf_sums(r4, V, S);
      y = cdf_draw(r4, V, u_res, S);
    }
    if (threadIdx.x == 0) {
      s_y = y;
      s_acc = acc ? 1 : 0;
    }
  }
  __syncthreads();
  const int y = valid_token(s_y, g.V, &C->flags);
  const int acc = s_acc && (y == xd);
  if (!acc)
    for (int l = threadIdx.x; l < g.L; l += kCtlThreads) A.kv_len[l] = j + 1;  // (i) truncate every layer
  if (threadIdx.x == 0) {
    A.tokens[j + 1] = y;
    C->emitted += 1;
    C->done = (C->emitted >= g.max_new);
    C->r_exit = j;
    C->r_y = y;
    C->r_accept = acc;
    // pre-step: the exiting row's draft-module key/values are committed by
    // the next cycle's draft step; post-step: by this cycle's
    C->pend_next = g.post ? 0 : 1;
    if (!acc) {  // (ii) flush in-flight state and (iii) reseed stage 0
      C->reseed = 1;
      C->seed_tok = y;
      C->seed_pos = j + 1;
    }
    rec->exit_pos = j;
    rec->target_token = y;
    rec->accepted = acc;
    rec->accepted_rank = acc ? 0 : -1;
    rec->emitted = C->emitted;
    rec->flags |= C->flags;
  }
  __syncthreads();
  for (int l = threadIdx.x; l < g.L; l += kCtlThreads) rec->kv_len[l] = A.kv_len[l];
}

struct FinalizeArgs {
  const ArgPair* parts;
  int nparts;
  const double* bs;     // dense sampling: block sums from k_softmax_blocks (weights already in qring)
  const unsigned long long* tk;  // top-k: k_topk_blocks' candidate keys of Q (ntk of them), or null
  int ntk;
  const float* logits;  // [V] PDM logits of the newest row
  int32_t* dring;
  float* qring;
  double* qz;
  const float* uni;
  int mode;
  float temp;
  int policy;
  float p_accept;
  const int32_t* ref;
  int ref_len;
  spd_cycle_rec* ring;
  Ctrl* ctrl;
  Geo g;
};

// ---- draft finalisation (A9): prediction, draft policy, commit -------------
__global__ __launch_bounds__(kCtlThreads) void k_pdm_finalize(const FinalizeArgs A) {
  __shared__ ArgPair sh_ap[kCtlThreads / kWave];
  __shared__ CdfShared S;
  __shared__ TopkShared TS;
  Ctrl* C = A.ctrl;
  const Geo& g = A.g;
  if (!C->active) return;
  const int q = C->t + 1;
  const int slot = q % g.nslots;
  const ArgPair best = block_argmax_parts(A.parts, A.nparts, sh_ap);
  int raw;
  if (A.mode == SPD_MODE_GREEDY) {
    raw = best.i;
  } else if (g.topk > 0) {
    // Q truncated to its top k: stored as (id, weight) pairs for the verification
    int id;
    float val;
    if (A.tk)
      topk_select_keys(A.tk, A.ntk, g.topk, TS, id, val);
    else
      topk_select(A.logits, g.V, g.topk, TS, id, val);
    raw = -1;
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      const float wf = topk_weight(id, val, A.temp, best.v);
      SparseQ* Qs = reinterpret_cast<SparseQ*>(A.qring) + slot;
      Qs->ids[lane] = id;
      Qs->w[lane] = wf;
      if (lane == 0) Qs->cnt = g.topk;
      double Z;
      const double u = A.uni[(size_t)q * SPD_U_COUNT + SPD_U_DRAFT];
      raw = topk_draw(id, (double)wf, u, &Z);
      if (lane == 0) A.qz[slot] = Z;
    }
  } else {
    float* qw = A.qring + (size_t)slot * g.V;
    double Z;
    if (A.bs) {  // weights and block sums from k_softmax_blocks
      const int nb = (g.V + kCdfBlock - 1) / kCdfBlock;
      for (int b = threadIdx.x; b < nb; b += kCtlThreads) S.bs[b] = A.bs[b];
      __syncthreads();
      cdf_super_sums(g.V, S);
      Z = S.total;
    } else {
      Z = softmax_weights(A.logits, qw, g.V, A.temp, best.v, S);
    }
    const double u = A.uni[(size_t)q * SPD_U_COUNT + SPD_U_DRAFT];
    raw = cdf_draw(StoredWeights{qw, g.V, aligned16(qw)}, g.V, u, S);
    if (threadIdx.x == 0) A.qz[slot] = Z;
  }
  if (threadIdx.x == 0) {
    raw = valid_token(raw, g.V, &C->flags);
    int d = raw;
    if (A.policy == SPD_DRAFT_FORCED && q < A.ref_len) {
      const int r = A.ref[q];
      const bool hit = A.uni[(size_t)q * SPD_U_COUNT + SPD_U_FORCE] < A.p_accept;
      d = hit ? r : (raw != r ? raw : (r + 1) % g.V);
      d = valid_token(d, g.V, &C->flags);
    }
    A.dring[slot] = d;
    C->r_draft = d;
    C->r_raw = raw;
    // the just-verified row's key/values stay cached
    C->C += g.post ? (C->a == g.n ? 1 : 0) : C->pending;
    spd_cycle_rec* rec = A.ring + C->rec_slot;
    rec->pdm_argmax = raw;
    rec->draft = d;
    rec->pdm_len = C->C;
  }
}

// ---- prefill / autoregressive helpers --------------------------------------
// X[r] = embed[tokens[pos0 + r]] for r < M; optional anchor-0 taps [r][m][d]
// and per-row partial sums of squares over 64-column groups [r][d/64] (the
// fused-norm input of the matrix-core path).
template <typename WT>
__global__ __launch_bounds__(kWG) void k_embed_rows(const int32_t* tokens, int pos0, const WT* embed, int d,
                                                    float* X, float* taps, int m, float* ssq) {
  const int r = blockIdx.x;
  const int tok = tokens[pos0 + r];
  const WT* e = embed + (size_t)tok * d;
  for (int i = threadIdx.x; i < d; i += kWG) {
    const float v = from_store(e[i]);
    X[(size_t)r * d + i] = v;
    if (taps) taps[((size_t)r * m + 0) * d + i] = v;
  }
  if (ssq) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    for (int cg = wave; cg < d / kWave; cg += kWG / kWave) {
      const float v = from_store(e[cg * kWave + lane]);
      const float sq = wave_sum(v * v);
      if (lane == 0) ssq[(size_t)r * (d / kWave) + cg] = sq;
    }
  }
}

// tokens[pos] = argmax (greedy) or a draw from softmax(logits/T) with
// u[pos][SPD_U_TARGET]; optionally also the control block's seed token.
__global__ __launch_bounds__(kCtlThreads) void k_pick_token(const ArgPair* parts, int nparts, const float* logits,
                                                            float* pw, int V, int mode, float temp, int topk,
                                                            const float* uni, int32_t* tokens, int pos, Ctrl* C,
                                                            uint32_t* flags) {
  __shared__ ArgPair sh_ap[kCtlThreads / kWave];
  __shared__ CdfShared S;
  __shared__ TopkShared TS;
  const ArgPair best = block_argmax_parts(parts, nparts, sh_ap);
  int y = best.i;
  if (mode == SPD_MODE_SAMPLE && topk > 0) {
    int id;
    float val;
    topk_select(logits, V, topk, TS, id, val);
    if (threadIdx.x < kWave) {
      const double u = uni[(size_t)pos * SPD_U_COUNT + SPD_U_TARGET];
      y = topk_draw(id, (double)topk_weight(id, val, temp, best.v), u, nullptr);
    }
  } else if (mode == SPD_MODE_SAMPLE) {
    softmax_weights(logits, pw, V, temp, best.v, S);
    const double u = uni[(size_t)pos * SPD_U_COUNT + SPD_U_TARGET];
    y = cdf_draw(StoredWeights{pw, V, aligned16(pw)}, V, u, S);
  }
  if (threadIdx.x == 0) {
    y = valid_token(y, V, flags);
    tokens[pos] = y;
    if (C) C->seed_tok = y;
  }
}

}  // namespace spd
