// Draft trees in the SPD cycle: control kernels (gfx950).
//
// [RB] prerequisites ("draft tree": the draft module proposes several branch
// candidates, keeping the top-W branches by cumulative probability) and [PL]
// appendix B (each SPD draft step widened into a width-4 tree).  Reading:
// the tokens in flight form a tree with at most W nodes per position and one
// at the oldest; each cycle the draft module scores the pairs (leaf, token)
// among every leaf's W most likely tokens by cum(leaf) + log Q_leaf(token)
// (cum: log Q summed over the leaf's path above the oldest position), the
// next cycle enters the best W whose leaf survived verification, the exiting
// node keeps its child that matches the target's argmax and prunes the rest,
// and the three-step rollback runs only when no child matches.
//
// Per-branch KV ([PL] §4 and [RB] limitations name branched KV caches as
// what a wall-clock tree needs): the target and draft caches hold W lanes
// (full copies).  A node's key/values go to the lanes of all its descendant
// leaves and it reads any one of them, so it attends to committed prefix +
// ancestors + itself with the arithmetic of the single chain.  A leaf that
// inherits its parent's lane needs nothing; a second child gets a free lane
// and a copy of the parent's in-flight window; an exiting node's key/values
// are broadcast to every lane (everything up to the last exit is common).
#pragma once

#include "common.h"
#include "control.h"

namespace spd {

// ---- entry (A0/A1 for a tree) --------------------------------------------
// The tree block staged in LDS for a kernel's serial bookkeeping: one
// thread's chains of dependent reads (parent walks, rank tables) then pay LDS
// latency instead of L2 latency.  Copied word by word by the workgroup.
static_assert(sizeof(Tree) % 4 == 0, "the tree block is copied in 4-byte words");
__device__ __forceinline__ void tree_copy(Tree* dst, const Tree* src) {
  constexpr int NW = (int)(sizeof(Tree) / 4);
  const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
  uint32_t* d = reinterpret_cast<uint32_t*>(dst);
  const int nt = blockDim.x;
  for (int i0 = threadIdx.x; i0 < NW; i0 += kBatch * nt) {
    uint32_t v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = s[min(i0 + u * nt, NW - 1)];  // unconditional: all in flight
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (i0 + u * nt < NW) d[i0 + u * nt] = v[u];
  }
}

template <typename WT>
__global__ __launch_bounds__(kWG) void k_tree_entry(Ctrl* C, const Geo g, int32_t* tokens, const WT* embed,
                                                    float* hslots, float* anchors, spd_cycle_rec* ring,
                                                    int log_cap) {
  __shared__ int s_n, s_slot[kMaxW], s_tok[kMaxW];
  // the entry is the only kernel on the tree block while it runs (the previous
  // cycle's streams are joined): it works on an LDS copy and writes it back
  __shared__ Tree sT;
  Tree* TG = tree_of(C);
  tree_copy(&sT, TG);
  __syncthreads();
  Tree* T = &sT;
  const int W = g.W, ns = g.nslots;
  if (threadIdx.x == 0) {
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
    s_n = 0;
    T->ncopy = 0;
    if (C->done) {
      C->active = 0;
      r->t = -1;
      r->occupancy = 0;
      r->pending_row = 0;
      r->pdm_len = C->C;
      r->emitted = C->emitted;
      r->flags = SPD_FLAG_IDLE;
    } else {
      int pos, a, n_new = 0;
      int par[kMaxW], tk[kMaxW], prank[kMaxW];
      double lq[kMaxW];
      const bool reseed = C->reseed != 0;
      if (reseed) {
        pos = C->seed_pos;
        a = 1;
        n_new = 1;
        par[0] = -1;
        tk[0] = C->seed_tok;
        lq[0] = 0.0;
        prank[0] = -1;
        C->reseed = 0;
        for (int ps = 0; ps < ns; ++ps) T->cnt[ps] = 0;
      } else {
        pos = C->t + 1;
        a = C->a - (C->r_exit >= 0 ? 1 : 0) + 1;
        // the first W candidates whose leaf survived this cycle's verification
        const int lps = C->t % ns, nl = T->cnt[lps];
        for (int c = 0; c < T->ncand && n_new < W; ++c) {
          const int leaf = T->cand_leaf[c];
          int lr = -1;
          for (int q = 0; q < nl; ++q)
            if (lps * W + T->rk[lps][q] == leaf) lr = q;
          if (lr < 0) continue;
          par[n_new] = leaf;
          tk[n_new] = T->cand_tok[c];
          lq[n_new] = T->cand_lq[c];
          prank[n_new] = lr;
          ++n_new;
        }
      }
      uint32_t fl = 0;
      if (a < 1 || a > g.n) fl |= SPD_FLAG_OCCUPANCY;
      if (pos + 1 >= g.max_ctx) fl |= SPD_FLAG_CTX;
      if (n_new < 1) fl |= SPD_FLAG_NODRAFT;
      C->flags |= fl;
      r->t = pos;
      r->occupancy = a;
      r->flags = fl;
      if (fl) {
        C->active = 0;
        C->done = 1;
        r->pending_row = 0;
      } else {
        const int oldest = pos - a + 1;
        const int pps = pos % ns;
        T->cnt[pps] = n_new;
        for (int k = 0; k < n_new; ++k) {
          T->rk[pps][k] = k;
          const int sl = pps * W + k;
          T->tok[sl] = tk[k];
          T->parent[sl] = par[k];
          T->logq[sl] = lq[k];
        }
        // branches that got no child are dead: keep the new nodes' ancestors
        int live[SPD_MAX_STAGES + 1];
        for (int ps = 0; ps < ns; ++ps) live[ps] = 0;
        for (int k = 0; k < n_new; ++k) {
          int x = par[k];
          for (int p = pos - 1; p >= oldest && x >= 0; --p) {
            live[p % ns] |= 1 << (x % W);
            if (p > oldest) x = T->parent[x];
          }
        }
        for (int p = oldest; p < pos; ++p) {
          const int ps = p % ns;
          int c2 = 0;
          for (int q = 0; q < T->cnt[ps]; ++q) {
            const int ph = T->rk[ps][q];
            if ((live[ps] >> ph) & 1) T->rk[ps][c2++] = ph;
          }
          T->cnt[ps] = c2;
        }
        // lanes: the first child of a leaf inherits its lane, the others take
        // free lanes and a copy of the parent's in-flight window
        int nlane[kMaxW];
        int taken = 0;
        if (reseed) {
          nlane[0] = 0;
          taken = 1;
        } else {
          for (int k = 0; k < n_new; ++k) {
            bool first = true;
            for (int k2 = 0; k2 < k; ++k2)
              if (par[k2] == par[k]) first = false;
            const int pl = T->lane[par[k]];
            if (first && !((taken >> pl) & 1)) {
              nlane[k] = pl;
              taken |= 1 << pl;
            } else {
              nlane[k] = -1;
            }
          }
          for (int k = 0; k < n_new; ++k) {
            if (nlane[k] >= 0) continue;
            int fr = 0;
            while ((taken >> fr) & 1) ++fr;
            nlane[k] = fr;
            taken |= 1 << fr;
            T->copy_src[T->ncopy] = T->lane[par[k]];
            T->copy_dst[T->ncopy] = fr;
            T->ncopy += 1;
          }
          T->copy_lo = oldest;
          T->copy_hi = pos - 1;
        }
        // lane masks: every live node writes to the lanes of its descendant leaves
        for (int p = oldest; p < pos; ++p) {
          const int ps = p % ns;
          for (int q = 0; q < T->cnt[ps]; ++q) T->lanes[ps * W + T->rk[ps][q]] = 0;
        }
        for (int k = 0; k < n_new; ++k) {
          const int sl = pps * W + k;
          T->lanes[sl] = 1 << nlane[k];
          T->lane[sl] = nlane[k];
          int x = par[k];
          for (int p = pos - 1; p >= oldest && x >= 0; --p) {
            T->lanes[x] |= 1 << nlane[k];
            if (p > oldest) x = T->parent[x];
          }
        }
        int nodes = n_new;
        for (int p = oldest; p < pos; ++p) {
          const int ps = p % ns;
          nodes += T->cnt[ps];
          for (int q = 0; q < T->cnt[ps]; ++q) {
            const int sl = ps * W + T->rk[ps][q];
            T->lane[sl] = __ffs(T->lanes[sl]) - 1;
          }
        }
        T->exit_slot = (oldest % ns) * W + T->rk[oldest % ns][0];
        // draft-module rows: the committed-next row (every lane), then the
        // nodes by position and rank
        int nr = 0;
        if (C->pend_next) {
          T->row_slot[nr] = T->last_exit;
          T->row_pos[nr] = C->C;
          T->row_depth[nr] = g.n;
          T->row_lanes[nr] = (1 << W) - 1;
          T->row_lane[nr] = 0;
          ++nr;
        }
        for (int p = oldest; p <= pos; ++p) {
          const int ps = p % ns;
          for (int q = 0; q < T->cnt[ps]; ++q) {
            if (nr >= kMaxTreeRows) break;  // cannot happen: 2 + (n - 1) W <= kMaxTreeRows
            const int sl = ps * W + T->rk[ps][q];
            T->row_slot[nr] = sl;
            T->row_pos[nr] = p;
            T->row_depth[nr] = pos - p;
            T->row_lanes[nr] = T->lanes[sl];
            T->row_lane[nr] = T->lane[sl];
            ++nr;
          }
        }
        T->nrows = nr;
        T->nleaves = n_new;
        T->pend_slot = C->pend_next ? T->last_exit : -1;
        C->pending = C->pend_next;
        C->t = pos;
        C->a = a;
        C->cycle += 1;
        C->active = 1;
        tokens[pos] = tk[0];
        r->pending_row = C->pending;
        r->nodes = nodes;
        r->n_new = n_new;
        for (int k = 0; k < n_new; ++k) {
          r->new_parent[k] = prank[k];
          r->new_token[k] = tk[k];
          s_slot[k] = pps * W + k;
          s_tok[k] = tk[k];
        }
        s_n = n_new;
      }
    }
  }
  __syncthreads();
  tree_copy(TG, &sT);
  {
    spd_cycle_rec* r = ring + C->rec_slot;
    for (int l = threadIdx.x; l < SPD_MAX_LAYERS; l += kWG) r->kv_len[l] = 0;
  }
  // the new nodes' embeddings (node k = index / d), kBatch loads in flight
  const int tot = s_n * g.d;
  for (int j0 = threadIdx.x; j0 < tot; j0 += kBatch * kWG) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int jj = min(j0 + u * kWG, tot - 1);
      const int k = jj / g.d, i = jj - k * g.d;
      v[u] = from_store(embed[(size_t)s_tok[k] * g.d + i]);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int jj = j0 + u * kWG;
      if (jj >= tot) break;
      const int k = jj / g.d, i = jj - k * g.d;
      hslots[(size_t)s_slot[k] * g.d + i] = v[u];
      anchors[((size_t)s_slot[k] * g.m + 0) * g.d + i] = v[u];
    }
  }
}

// ---- lane copies asked for by the entry: grid (layers, W) ----------------
template <typename WT>
__global__ __launch_bounds__(kWG) void k_tree_lane_copy(const Ctrl* C, const Geo g, WT* kc, WT* vc) {
  const Tree* T = tree_of(C);
  if (!C->active || (int)blockIdx.y >= T->ncopy) return;
  const int layer = blockIdx.x;
  const long long src = T->copy_src[blockIdx.y] * g.lane_kv, dst = T->copy_dst[blockIdx.y] * g.lane_kv;
  const int lo = T->copy_lo, np = T->copy_hi - T->copy_lo + 1;
  if (np <= 0) return;
  const int n = g.Hkv * g.hd * np;
  for (int i0 = threadIdx.x; i0 < n; i0 += kBatch * kWG) {
    size_t ik[kBatch], iv[kBatch];
    WT kx[kBatch], vx[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int idx = min(i0 + u * kWG, n - 1);
      const int p = lo + idx % np, rest = idx / np;
      const int dim = rest % g.hd, kvh = rest / g.hd;
      ik[u] = k_index(g, layer, kvh, p, dim);
      iv[u] = v_index(g, layer, kvh, p, dim);
      kx[u] = kc[src + ik[u]];
      vx[u] = vc[src + iv[u]];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (i0 + u * kWG >= n) break;
      kc[dst + ik[u]] = kx[u];
      vc[dst + iv[u]] = vx[u];
    }
  }
}

// ---- verification of the exiting node's children + rollback (A5/A6) ------
struct TreeVerifyArgs {
  const ArgPair* parts;
  int nparts;
  int32_t* tokens;
  int32_t* kv_len;
  void* kc;
  void* vc;
  int kv_bytes;  // bytes per KV element
  spd_cycle_rec* ring;
  Ctrl* ctrl;
  Geo g;
};

// Key/values of position j in KV lane src copied to every other lane, all
// layers; kBatch elements per thread in flight.
template <typename KT>
__device__ __forceinline__ void kv_broadcast(const Geo& g, KT* kc, KT* vc, int src, int j) {
  const int n = g.L * g.Hkv * g.hd;
  for (int i0 = threadIdx.x; i0 < n; i0 += kBatch * kCtlThreads) {
    size_t ik[kBatch], iv[kBatch];
    KT kx[kBatch], vx[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int idx = min(i0 + u * kCtlThreads, n - 1);
      const int dim = idx % g.hd, rest = idx / g.hd;
      const int kvh = rest % g.Hkv, layer = rest / g.Hkv;
      ik[u] = k_index(g, layer, kvh, j, dim);
      iv[u] = v_index(g, layer, kvh, j, dim);
      kx[u] = kc[src * g.lane_kv + ik[u]];
      vx[u] = vc[src * g.lane_kv + iv[u]];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (i0 + u * kCtlThreads >= n) break;
      for (int ln = 0; ln < g.W; ++ln) {
        if (ln == src) continue;
        kc[ln * g.lane_kv + ik[u]] = kx[u];
        vc[ln * g.lane_kv + iv[u]] = vx[u];
      }
    }
  }
}

__global__ __launch_bounds__(kCtlThreads) void k_tree_verify(const TreeVerifyArgs A) {
  __shared__ ArgPair sh_ap[kCtlThreads / kWave];
  Ctrl* C = A.ctrl;
  Tree* T = tree_of(C);
  const Geo& g = A.g;
  const int W = g.W, ns = g.nslots;
  if (!C->active) return;
  spd_cycle_rec* rec = A.ring + C->rec_slot;
  if (C->a != g.n) {
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
  // the draft stream's finalisation may write the candidate fields meanwhile:
  // work on an LDS copy and write back only the counts, the rank tables and
  // the last exit
  __shared__ Tree sT;
  Tree* TG = T;
  tree_copy(&sT, TG);
  __syncthreads();
  T = &sT;
  const int j = C->t - (g.n - 1);
  const int ex = T->exit_slot;
  const ArgPair best = block_argmax_parts(A.parts, A.nparts, sh_ap);
  // the exiting node's key/values join every lane (its position is verified)
  if (A.kv_bytes == 2)
    kv_broadcast(g, reinterpret_cast<uint16_t*>(A.kc), reinterpret_cast<uint16_t*>(A.vc), T->lane[ex], j);
  else
    kv_broadcast(g, reinterpret_cast<float*>(A.kc), reinterpret_cast<float*>(A.vc), T->lane[ex], j);
  for (int l = threadIdx.x; l < g.L; l += kCtlThreads) A.kv_len[l] = j + 1;  // committed (and (i) on reject)
  if (threadIdx.x == 0) {
    const int y = valid_token(best.i, g.V, &C->flags);
    const int ps1 = (j + 1) % ns;
    int acc_rank = -1;
    for (int q = 0; q < T->cnt[ps1]; ++q)
      if (T->tok[ps1 * W + T->rk[ps1][q]] == y) {
        acc_rank = q;
        break;
      }
    if (acc_rank >= 0) {
      // only the kept child's subtree stays
      const int keep = ps1 * W + T->rk[ps1][acc_rank];
      for (int p = j + 1; p <= C->t; ++p) {
        const int ps = p % ns;
        int c2 = 0;
        for (int q = 0; q < T->cnt[ps]; ++q) {
          const int sl = ps * W + T->rk[ps][q];
          int x = sl;
          for (int pp = p; pp > j + 1; --pp) x = T->parent[x];
          if (x == keep) T->rk[ps][c2++] = T->rk[ps][q];
        }
        T->cnt[ps] = c2;
      }
    } else {
      // (ii) flush the tree and (iii) re-seed stage 0
      for (int ps = 0; ps < ns; ++ps) T->cnt[ps] = 0;
      TG->ncand = 0;
      C->reseed = 1;
      C->seed_tok = y;
      C->seed_pos = j + 1;
    }
    const int acc = acc_rank >= 0 ? 1 : 0;
    A.tokens[j + 1] = y;
    C->emitted += 1;
    C->done = (C->emitted >= g.max_new);
    C->r_exit = j;
    C->r_y = y;
    C->r_accept = acc;
    C->pend_next = 1;
    T->last_exit = ex;
    rec->exit_pos = j;
    rec->target_token = y;
    rec->accepted = acc;
    rec->accepted_rank = acc_rank;
    rec->emitted = C->emitted;
    rec->flags |= C->flags;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < ns; i += kCtlThreads) {
    TG->cnt[i] = sT.cnt[i];
#pragma unroll
    for (int k = 0; k < kMaxW; ++k) TG->rk[i][k] = sT.rk[i][k];
  }
  if (threadIdx.x == 0) TG->last_exit = sT.last_exit;
  for (int l = threadIdx.x; l < g.L; l += kCtlThreads) rec->kv_len[l] = A.kv_len[l];
}

// ---- draft step of a tree: per leaf, the softmax normaliser and the W most
// likely tokens; then candidates, ranking and the forced policy -----------
constexpr int kTreeScanIds = 16;  // ids per thread of k_tree_scan
constexpr int kTreeScanBlk = kWG * kTreeScanIds;

__host__ __device__ constexpr int tree_scan_blocks(int V) { return (V + kTreeScanBlk - 1) / kTreeScanBlk; }

struct TreeScanArgs {
  const float* logits;    // [W][V] draft logits of the leaves
  const ArgPair* parts;   // [W][nparts] per-workgroup argmax of each leaf's logits
  int nparts;
  double* zpart;          // [W][nblk] partial sums of exp(l - max)
  ArgPair* tpart;         // [W][nblk][W] partial top-W (value, id)
  const Ctrl* ctrl;
  Geo g;
};

// Largest value among n per-workgroup partials, by the 64 lanes of one wave
// (every lane returns it).
__device__ __forceinline__ float parts_max_wave(const ArgPair* p, int n) {
  float m = -INFINITY;
  for (int k0 = threadIdx.x & (kWave - 1); k0 < n; k0 += kBatch * kWave) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = (k0 + u * kWave < n) ? p[k0 + u * kWave].v : -INFINITY;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) m = fmaxf(m, v[u]);
  }
  return wave_max(m);
}

// grid (blocks, W): block b of leaf m takes ids [b * kTreeScanBlk, ...)
__global__ __launch_bounds__(kWG) void k_tree_scan(const TreeScanArgs A) {
  __shared__ double sz[kWG / kWave];
  __shared__ ArgPair sh[kWG / kWave];
  __shared__ float s_max;
  const Ctrl* C = A.ctrl;
  const Geo& g = A.g;
  const int m = blockIdx.y, W = g.W;
  if (!C->active || m >= tree_of(C)->nleaves) return;
  const float* l = A.logits + (size_t)m * g.V;
  if (threadIdx.x < kWave) {
    const float mx = parts_max_wave(A.parts + (size_t)m * A.nparts, A.nparts);
    if (threadIdx.x == 0) s_max = mx;
  }
  __syncthreads();
  const double M = s_max;
  // each thread: its ids' exp sum (fp64) and its own best W (value desc, id asc)
  float tv[kMaxW];
  int ti[kMaxW];
  for (int k = 0; k < kMaxW; ++k) {
    tv[k] = -INFINITY;
    ti[k] = 0x7FFFFFFF;
  }
  double z = 0.0;
  const int base = blockIdx.x * kTreeScanBlk;
  float xs[kTreeScanIds];
#pragma unroll
  for (int e = 0; e < kTreeScanIds; ++e) {
    const int v = base + e * kWG + threadIdx.x;
    xs[e] = v < g.V ? l[v] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < kTreeScanIds; ++e) {
    const int v = base + e * kWG + threadIdx.x;
    if (v >= g.V) break;
    const float x = xs[e];
    z += exp((double)x - M);
    if (better(x, v, tv[W - 1], ti[W - 1])) {
      int k = W - 1;
      while (k > 0 && better(x, v, tv[k - 1], ti[k - 1])) {
        tv[k] = tv[k - 1];
        ti[k] = ti[k - 1];
        --k;
      }
      tv[k] = x;
      ti[k] = v;
    }
  }
  // block sums in a fixed order
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  double zw = wave_sum_d(z);
  if (lane == 0) sz[wave] = zw;
  // block top-W: W rounds of a block argmax over each thread's next candidate
  int head = 0;
  for (int k = 0; k < W; ++k) {
    float v = head < W ? tv[head] : -INFINITY;
    int i = head < W ? ti[head] : 0x7FFFFFFF;
    float bv = v;
    int bi = i;
    wave_argmax(bv, bi);
    __syncthreads();
    if (lane == 0) sh[wave] = ArgPair{bv, bi};
    __syncthreads();
    ArgPair b = sh[0];
    for (int w = 1; w < kWG / kWave; ++w)
      if (better(sh[w].v, sh[w].i, b.v, b.i)) b = sh[w];
    if (head < W && i == b.i && v == b.v) ++head;  // ids are unique: only the owner advances
    if (threadIdx.x == 0) A.tpart[((size_t)m * gridDim.x + blockIdx.x) * W + k] = b;
  }
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int w = 0; w < kWG / kWave; ++w) s += sz[w];
    A.zpart[(size_t)m * gridDim.x + blockIdx.x] = s;
  }
}

struct TreeFinalizeArgs {
  const float* logits;    // [W][V]
  const ArgPair* parts;   // [W][nparts]
  int nparts;
  const double* zpart;
  const ArgPair* tpart;
  int nblk;
  const float* uni;
  int policy;             // SPD_DRAFT_NATURAL / SPD_DRAFT_FORCED (tree policy)
  float p_first, p_tree;
  const int32_t* ref;
  int ref_len;
  spd_cycle_rec* ring;
  Ctrl* ctrl;
  Geo g;
};

__global__ __launch_bounds__(kWG) void k_tree_finalize(const TreeFinalizeArgs A) {
  static_assert(kWG / kWave >= kMaxW, "one wave per leaf");
  Ctrl* C = A.ctrl;
  Tree* TG = tree_of(C);
  const Geo& g = A.g;
  const int W = g.W, ns = g.nslots;
  if (!C->active) return;
  // reads from an LDS copy (the stage stream's verification may update the
  // counts and rank tables meanwhile; nothing read here changes); the
  // candidates are written to the tree block itself
  __shared__ Tree sT;
  // the forced policy's reference tokens at positions oldest .. t + 1, and the
  // draft logit of the token at t + 1 under each leaf
  __shared__ int s_ref[SPD_MAX_STAGES + 2];
  __shared__ float s_lref[kMaxW];
  tree_copy(&sT, TG);
  const int t = C->t, oldest = t - C->a + 1;
  const bool forced = A.policy == SPD_DRAFT_FORCED && t + 1 < A.ref_len;
  if (forced && (int)threadIdx.x <= t + 1 - oldest) {
    const int r = A.ref[oldest + threadIdx.x];
    s_ref[threadIdx.x] = r;
    if (oldest + (int)threadIdx.x == t + 1) {
      float lr[kMaxW];
#pragma unroll
      for (int m = 0; m < kMaxW; ++m) lr[m] = m < W ? A.logits[(size_t)m * g.V + r] : 0.f;
#pragma unroll
      for (int m = 0; m < kMaxW; ++m) s_lref[m] = lr[m];
    }
  }
  __syncthreads();
  const Tree* T = &sT;
  const int nl = T->nleaves;
  // per leaf, by one wave (leaf m on wave m): the max logit (over the head's
  // per-workgroup partials), the normaliser (the scan blocks' sums;
  // lane-strided, then a fixed butterfly) and the best W tokens (each lane's
  // best W of its share of the blocks' lists, then W rounds of a wave argmax)
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  __shared__ double s_lM[kMaxW], s_lZ[kMaxW];
  __shared__ float s_bv[kMaxW][kMaxW];
  __shared__ int s_bi[kMaxW][kMaxW];
  // the serial part's working lists, indexed at run time: in LDS rather than
  // in per-lane scratch memory
  __shared__ int cl[kMaxCand], ct[kMaxCand], crank[kMaxCand];
  __shared__ double cs[kMaxCand], clq[kMaxCand];
  __shared__ double lM[kMaxW], lZ[kMaxW], cum[kMaxW];
  __shared__ int lslot[kMaxW];
  __shared__ double lqs[SPD_MAX_STAGES + 1];
  __shared__ int match[SPD_MAX_STAGES + 1];
  for (int m = wave; m < nl; m += kWG / kWave) {
    const float mx = parts_max_wave(A.parts + (size_t)m * A.nparts, A.nparts);
    double z = 0.0;
    for (int b0 = lane; b0 < A.nblk; b0 += kBatch * kWave) {
      double zb[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int b = b0 + u * kWave;
        zb[u] = b < A.nblk ? A.zpart[(size_t)m * A.nblk + b] : 0.0;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (b0 + u * kWave < A.nblk) z += zb[u];
    }
    z = wave_sum_d(z);
    float tv[kMaxW];
    int ti[kMaxW];
    for (int k = 0; k < kMaxW; ++k) {
      tv[k] = -INFINITY;
      ti[k] = 0x7FFFFFFF;
    }
    const int ne = A.nblk * W;
    for (int e0 = lane; e0 < ne; e0 += kBatch * kWave) {
      ArgPair cb[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int e = e0 + u * kWave;
        cb[u] = e < ne ? A.tpart[(size_t)m * ne + e] : ArgPair{-INFINITY, 0x7FFFFFFF};
      }
      for (int u = 0; u < kBatch; ++u) {
        if (e0 + u * kWave >= ne) break;
        const ArgPair c = cb[u];
        if (!better(c.v, c.i, tv[W - 1], ti[W - 1])) continue;
        int q = W - 1;
        while (q > 0 && better(c.v, c.i, tv[q - 1], ti[q - 1])) {
          tv[q] = tv[q - 1];
          ti[q] = ti[q - 1];
          --q;
        }
        tv[q] = c.v;
        ti[q] = c.i;
      }
    }
    int head = 0;
    for (int k = 0; k < W; ++k) {
      const float v = head < W ? tv[head] : -INFINITY;
      const int i = head < W ? ti[head] : 0x7FFFFFFF;
      float bv = v;
      int bi = i;
      wave_argmax(bv, bi);
      if (lane == 0) {
        s_bv[m][k] = bv;
        s_bi[m][k] = bi;
      }
      if (head < W && i == bi && v == bv) ++head;  // ids are unique: only the owner advances
    }
    if (lane == 0) {
      s_lM[m] = mx;
      s_lZ[m] = log(z);
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  // candidates, ranking and the forced policy: one thread
  int nc = 0, top0 = -1;
  for (int m = 0; m < nl; ++m) {
    lM[m] = s_lM[m];
    lZ[m] = s_lZ[m];
    const int sl = T->row_slot[T->nrows - nl + m];
    lslot[m] = sl;
    // cum: log Q over the path above the oldest position, in position order
    int np = 0, x = sl;
    for (int p = t; p > oldest; --p) {
      lqs[np++] = T->logq[x];
      x = T->parent[x];
    }
    double s = 0.0;
    for (int k = np - 1; k >= 0; --k) s += lqs[k];
    cum[m] = s;
    if (m == 0) top0 = s_bi[0][0];
    for (int k = 0; k < W; ++k) {
      const double lq = (double)s_bv[m][k] - lM[m] - lZ[m];
      cl[nc] = sl;
      ct[nc] = s_bi[m][k];
      crank[nc] = m;
      clq[nc] = lq;
      cs[nc] = cum[m] + lq;
      ++nc;
    }
  }
  // rank: score desc, then leaf rank, then token id (insertion sort, <= 16)
  for (int i = 1; i < nc; ++i) {
    int k = i;
    while (k > 0 && (cs[k] > cs[k - 1] || (cs[k] == cs[k - 1] && (crank[k] < crank[k - 1] ||
                                                                   (crank[k] == crank[k - 1] && ct[k] < ct[k - 1]))))) {
      int ti;
      double td;
      ti = cl[k]; cl[k] = cl[k - 1]; cl[k - 1] = ti;
      ti = ct[k]; ct[k] = ct[k - 1]; ct[k - 1] = ti;
      ti = crank[k]; crank[k] = crank[k - 1]; crank[k - 1] = ti;
      td = cs[k]; cs[k] = cs[k - 1]; cs[k - 1] = td;
      td = clq[k]; clq[k] = clq[k - 1]; clq[k - 1] = td;
      --k;
    }
  }
  // forced policy (harness device): the pair (forced leaf, ref[q])
  const int q = t + 1;
  if (forced) {
    // the leaf whose path matches the reference for the longest prefix from
    // the oldest position (ties: the lower rank)
    int star = 0, best = -1;
    for (int m = 0; m < nl; ++m) {
      int x = lslot[m], np = 0;
      for (int p = t; p >= oldest; --p) {
        match[np++] = T->tok[x] == s_ref[p - oldest];
        if (p > oldest) x = T->parent[x];
      }
      int k = 0;
      while (k < np && match[np - 1 - k]) ++k;
      if (k > best) {
        best = k;
        star = m;
      }
    }
    const int R = s_ref[q - oldest];
    const float u = A.uni[(size_t)q * SPD_U_COUNT + SPD_U_FORCE];
    const float* ls = A.logits + (size_t)star * g.V;
    int at = -1;
    for (int i = 0; i < nc; ++i)
      if (crank[i] == star && ct[i] == R) at = i;
    if (u < A.p_first || (u < A.p_tree && W >= 2)) {
      if (at >= 0) {
        for (int i = at; i + 1 < nc; ++i) {
          cl[i] = cl[i + 1]; ct[i] = ct[i + 1]; crank[i] = crank[i + 1]; cs[i] = cs[i + 1]; clq[i] = clq[i + 1];
        }
        --nc;
      }
      const int ins = (u < A.p_first) ? 0 : min(W - 1, nc);
      for (int i = nc; i > ins; --i) {
        cl[i] = cl[i - 1]; ct[i] = ct[i - 1]; crank[i] = crank[i - 1]; cs[i] = cs[i - 1]; clq[i] = clq[i - 1];
      }
      const double lq = (double)s_lref[star] - lM[star] - lZ[star];
      cl[ins] = lslot[star];
      ct[ins] = R;
      crank[ins] = star;
      clq[ins] = lq;
      cs[ins] = cum[star] + lq;
      ++nc;
    } else {
      // a miss: the forced leaf's true token is replaced by the next id that
      // is not already one of its candidates, and its branch stays alive
      auto next_free = [&]() {
        int x = (R + 1) % g.V;
        for (;;) {
          bool used = false;
          for (int i = 0; i < nc; ++i)
            if (crank[i] == star && ct[i] == x) used = true;
          if (!used) return x;
          x = (x + 1) % g.V;
        }
      };
      if (at >= 0) {
        const int x = next_free();
        const double lq = (double)ls[x] - lM[star] - lZ[star];
        ct[at] = x;
        clq[at] = lq;
        cs[at] = cum[star] + lq;
      }
      bool alive = false;
      for (int i = 0; i < nc && i < W; ++i)
        if (crank[i] == star) alive = true;
      if (!alive) {
        const int x = next_free();
        const int ins = min(W - 1, nc);
        for (int i = nc; i > ins; --i) {
          cl[i] = cl[i - 1]; ct[i] = ct[i - 1]; crank[i] = crank[i - 1]; cs[i] = cs[i - 1]; clq[i] = clq[i - 1];
        }
        const double lq = (double)ls[x] - lM[star] - lZ[star];
        cl[ins] = lslot[star];
        ct[ins] = x;
        crank[ins] = star;
        clq[ins] = lq;
        cs[ins] = cum[star] + lq;
        ++nc;
      }
    }
  }
  TG->ncand = nc;
  for (int i = 0; i < nc; ++i) {
    TG->cand_leaf[i] = cl[i];
    TG->cand_tok[i] = ct[i];
    TG->cand_lq[i] = clq[i];
  }
  C->r_draft = ct[0];
  C->r_raw = top0;
  C->C += C->pending;  // the just-verified row's key/values stay cached
  spd_cycle_rec* rec = A.ring + C->rec_slot;
  rec->pdm_argmax = top0;
  rec->draft = ct[0];
  rec->pdm_len = C->C;
  (void)ns;
}

}  // namespace spd
