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

// Each thread owns the contiguous index range [lo, hi) of V.
__device__ __forceinline__ void chunk_of(int V, int& lo, int& hi) {
  const int ch = (V + kCtlThreads - 1) / kCtlThreads;
  lo = min(V, threadIdx.x * ch);
  hi = min(V, lo + ch);
}

// fp64 sum of per-thread values in thread order.
__device__ __forceinline__ double block_sum_ordered(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  __shared__ double tot;
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int k = 0; k < kCtlThreads; ++k) s += sh[k];
    tot = s;
  }
  __syncthreads();
  const double r = tot;
  __syncthreads();
  return r;
}

// Softmax weights w_v = exp(l_v / T - max) written to `w` (fp32), returns
// Z = sum_v w_v accumulated in fp64 (per-thread chunks in id order, then
// thread order).  `lmax` is max_v l_v.
__device__ __forceinline__ double softmax_weights(const float* logits, float* w, int V, float T, float lmax,
                                                  double* sh) {
  int lo, hi;
  chunk_of(V, lo, hi);
  const float mt = (T == 1.0f) ? lmax : lmax / T;
  double s = 0.0;
  for (int v = lo; v < hi; ++v) {
    const float l = (T == 1.0f) ? logits[v] : logits[v] / T;
    const float e = expf(l - mt);
    w[v] = e;
    s += (double)e;
  }
  return block_sum_ordered(s, sh);
}

// Inverse CDF: smallest id i with (ascending cumulative weight) > u * total,
// where weight(v) is given by `wf(v)` (fp64).  Falls back to the last id with
// positive weight.  All threads return the same id.
template <typename WF>
__device__ __forceinline__ int inverse_cdf(WF wf, int V, double u, double* sh) {
  __shared__ int pick;
  __shared__ int last_pos;
  int lo, hi;
  chunk_of(V, lo, hi);
  double s = 0.0;
  int lastnz = -1;
  for (int v = lo; v < hi; ++v) {
    const double x = wf(v);
    s += x;
    if (x > 0.0) lastnz = v;
  }
  sh[threadIdx.x] = s;
  if (threadIdx.x == 0) {
    pick = -1;
    last_pos = -1;
  }
  __syncthreads();
  if (lastnz >= 0) atomicMax(&last_pos, lastnz);
  __shared__ double thr_s;
  __shared__ int owner;
  __shared__ double pre_s;
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int k = 0; k < kCtlThreads; ++k) tot += sh[k];
    const double thr = u * tot;
    double pre = 0.0;
    int own = -1;
    for (int k = 0; k < kCtlThreads; ++k) {
      if (pre + sh[k] > thr) {
        own = k;
        break;
      }
      pre += sh[k];
    }
    thr_s = thr;
    owner = own;
    pre_s = pre;
  }
  __syncthreads();
  if ((int)threadIdx.x == owner) {
    double c = pre_s;
    int found = -1;
    for (int v = lo; v < hi; ++v) {
      c += wf(v);
      if (c > thr_s) {
        found = v;
        break;
      }
    }
    pick = found;
  }
  __syncthreads();
  const int r = (pick >= 0) ? pick : last_pos;
  __syncthreads();
  return r;
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
  __shared__ double sh_d[kCtlThreads];
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
    const double pZ = softmax_weights(A.logits, A.pw, g.V, A.temp, best.v, sh_d);
    __syncthreads();
    const float* qw = A.qring + (size_t)nslot * g.V;
    const double qZ = A.qz[nslot];
    const double u_acc = A.uni[(size_t)(j + 1) * SPD_U_COUNT + SPD_U_ACCEPT];
    const double Px = (double)A.pw[xd] / pZ;
    const double Qx = (double)qw[xd] / qZ;
    const bool acc = u_acc * Qx < Px;
    int y = xd;
    if (!acc) {
      const double u_res = A.uni[(size_t)(j + 1) * SPD_U_COUNT + SPD_U_RESAMPLE];
      const float* pw = A.pw;
      y = inverse_cdf(
          [&](int v) {
            const double r = (double)pw[v] / pZ - (double)qw[v] / qZ;
            return r > 0.0 ? r : 0.0;
          },
          g.V, u_res, sh_d);
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
    C->pend_next = 1;
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
  __shared__ double sh_d[kCtlThreads];
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
    const double Z = softmax_weights(A.logits, qw, g.V, A.temp, best.v, sh_d);
    __syncthreads();
    const double u = A.uni[(size_t)q * SPD_U_COUNT + SPD_U_DRAFT];
    raw = inverse_cdf([&](int v) { return (double)qw[v]; }, g.V, u, sh_d);
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
    C->C += C->pending;  // the just-verified row's key/values stay cached
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
  __shared__ double sh_d[kCtlThreads];
  const ArgPair best = block_argmax_parts(parts, nparts, sh_ap);
  int y = best.i;
  if (mode == SPD_MODE_SAMPLE) {
    softmax_weights(logits, pw, V, temp, best.v, sh_d);
    __syncthreads();
    const double u = uni[(size_t)pos * SPD_U_COUNT + SPD_U_TARGET];
    y = inverse_cdf([&](int v) { return (double)pw[v]; }, V, u, sh_d);
  }
  if (threadIdx.x == 0) {
    y = valid_token(y, V, flags);
    tokens[pos] = y;
    if (C) C->seed_tok = y;
  }
}

}  // namespace spd
