// Control kernels of the SPD cycle: entry (fork), verification + rollback,
// draft finalisation, and the small helpers of prefill / autoregressive decode.
#pragma once

#include "common.h"

namespace spd {

constexpr int kCtlThreads = 1024;

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
// v0..v0+3, zero beyond V) into S.bs, then the superblock sums and the total.
// Ends with a barrier; S.total is then valid in every thread.
template <typename W4>
__device__ __forceinline__ void cdf_sums(W4 w4, int V, CdfShared& S) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int nb = (V + kCdfBlock - 1) / kCdfBlock;
  const int nsb = (nb + kWave - 1) / kWave;
  for (int b0 = wave; b0 < nb; b0 += kCtlWaves * kCdfUnroll) {
    double x[kCdfUnroll][4];
#pragma unroll
    for (int u = 0; u < kCdfUnroll; ++u) {
      const int b = b0 + u * kCtlWaves;
      if (b < nb) {
        w4(b * kCdfBlock + lane * kCdfPer, x[u]);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[u][k] = 0.0;
      }
    }
#pragma unroll
    for (int u = 0; u < kCdfUnroll; ++u) {
      const int b = b0 + u * kCtlWaves;
      const double s = wave_scan_d(lane_sum4(x[u]));
      if (lane == kWave - 1 && b < nb) S.bs[b] = s;
    }
  }
  __syncthreads();
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
__device__ __forceinline__ double softmax_weights(const float* logits, float* w, int V, float T, float lmax,
                                                  CdfShared& S) {
  const float mt = (T == 1.0f) ? lmax : lmax / T;
  const bool vec = aligned16(logits) && aligned16(w);
  cdf_sums(
      [&](int v0, double x[4]) {
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
      },
      V, S);
  return S.total;
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
  for (int i = threadIdx.x; i < g.d; i += kWG) {
    const float v = from_store(e[i]);
    hslots[(size_t)slot * g.d + i] = v;
    anchors[((size_t)slot * g.m + 0) * g.d + i] = v;
  }
}

struct VerifyArgs {
  const ArgPair* parts;
  int nparts;
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
  } else {
    // P = softmax(logits / T); accept iff u * Q(x) < P(x); else redraw from max(0, P - Q)
    const double pZ = softmax_weights(A.logits, A.pw, g.V, A.temp, best.v, S);
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
    rec->emitted = C->emitted;
    rec->flags |= C->flags;
  }
  __syncthreads();
  for (int l = threadIdx.x; l < g.L; l += kCtlThreads) rec->kv_len[l] = A.kv_len[l];
}

struct FinalizeArgs {
  const ArgPair* parts;
  int nparts;
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
  Ctrl* C = A.ctrl;
  const Geo& g = A.g;
  if (!C->active) return;
  const int q = C->t + 1;
  const int slot = q % g.nslots;
  const ArgPair best = block_argmax_parts(A.parts, A.nparts, sh_ap);
  int raw;
  if (A.mode == SPD_MODE_GREEDY) {
    raw = best.i;
  } else {
    float* qw = A.qring + (size_t)slot * g.V;
    const double Z = softmax_weights(A.logits, qw, g.V, A.temp, best.v, S);
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
                                                            float* pw, int V, int mode, float temp, const float* uni,
                                                            int32_t* tokens, int pos, Ctrl* C, uint32_t* flags) {
  __shared__ ArgPair sh_ap[kCtlThreads / kWave];
  __shared__ CdfShared S;
  const ArgPair best = block_argmax_parts(parts, nparts, sh_ap);
  int y = best.i;
  if (mode == SPD_MODE_SAMPLE) {
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
