// libspd: host orchestration and the C ABI declared in spd.h.
//
// Per cycle the host enqueues, without waiting:
//   stage stream:  wait(previous draft done) -> entry -> record(E_entry)
//                  -> L/n x [qkv+RoPE+KV append, split-KV attention, combine,
//                            o-proj + residual, norm + gate/up + SwiGLU,
//                            down + residual + anchor taps]
//                  -> verification head -> verify / rollback
//   draft stream:  wait(E_entry) -> anchor gather + FC -> Ls x [the same layer
//                  over the trailing rows] -> draft head -> finalise -> record(E_pdm)
// The draft module reads only pre-step state, so the two streams overlap; the
// next cycle's entry joins them.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "attention.h"
#include "common.h"
#include "control.h"
#include "gemv.h"
#include "linattn.h"
#include "mfma.h"
#include "skinny.h"
#include "tree.h"

using namespace spd;

namespace {

constexpr int kPersistPerCU = 3;
constexpr int kCUs = 256;
constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct Layout {
  size_t ctrl, kv_len, tokens, dring, qring, qz, kc, vc, pkc, pvc, rcos, rsin, hslots, anchors;
  size_t s_q, s_pacc, s_pml, s_o, s_act;
  size_t Xt, Xp, r_q, r_pacc, r_pml, r_o, r_act, taps;
  size_t logits, plogits, pw, parts, pparts, ring;
  size_t ssq_t, ssq_p, mpart;
  size_t wtile;                   // draft-module layer weights in matrix-core tile order (bf16)
  size_t xs_h, xs_l, as_h, as_l, os_h, os_l;  // split (bf16 hi + lo) inputs of the draft module's products
  size_t lin_state, lin_ckpt;
  size_t zpart, tpart;
  size_t bsq, bsp;
  size_t tkq, tkp;
  size_t state_total;    // persistent state: KV caches, control block, rings, tables, in-flight slots
  size_t scratch_total;  // per-cycle scratch (offsets of the scratch fields are relative to its base)
  size_t total;          // one workspace holding both: state, then scratch
  int ctx_cap, nsplit, mr, log_cap, nparts_max;
};

bool has_split(const spd_config* c) {
  for (int k = 0; k < SPD_MAX_STAGES; ++k)
    if (c->stage_layers[k] != 0) return true;
  return false;
}

bool valid_config(const spd_config* c) {
  if (!c) return false;
  if (c->n_layers < 1 || c->n_layers > SPD_MAX_LAYERS) return false;
  if (c->n_stages < 1 || c->n_stages > SPD_MAX_STAGES) return false;
  if (c->pdm_layers < 1 || c->pdm_layers > SPD_MAX_PDM_LAYERS) return false;
  if (has_split(c)) {
    // non-uniform split: n_stages entries >= 1 summing to n_layers, zeros after
    int sum = 0, longest = 0;
    for (int k = 0; k < SPD_MAX_STAGES; ++k) {
      const int v = c->stage_layers[k];
      if (k >= c->n_stages) {
        if (v != 0) return false;
      } else {
        if (v < 1) return false;
        sum += v;
        longest = std::max(longest, v);
      }
    }
    if (sum != c->n_layers || c->pdm_layers > longest) return false;
  } else if (c->n_layers % c->n_stages || c->pdm_layers > c->n_layers / c->n_stages) {
    return false;
  }
  if (c->n_anchors < 1 || c->n_anchors > SPD_MAX_ANCHORS || c->anchors[0] != 0) return false;
  for (int i = 1; i < c->n_anchors; ++i)
    if (c->anchors[i] <= c->anchors[i - 1]) return false;
  if (c->anchors[c->n_anchors - 1] > c->n_layers) return false;
  if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads) return false;
  if (c->head_dim != 64 && c->head_dim != 128) return false;
  const int G = c->n_heads / c->n_kv_heads;
  if (G > kAttnQ) return false;
  if (c->d_model % 256 || c->d_ffn % 256 || (c->n_heads * c->head_dim) % 256) return false;
  if (c->d_model * c->n_anchors > 64 * 1024) return false;
  if (c->d_ffn > 12288 || c->d_model > 12288 || c->n_heads * c->head_dim > 12288) return false;
  if (c->vocab < 2 || c->vocab > SPD_MAX_VOCAB) return false;
  if (c->dtype != SPD_DTYPE_F32 && c->dtype != SPD_DTYPE_BF16) return false;
  if (c->mode != SPD_MODE_GREEDY && c->mode != SPD_MODE_SAMPLE) return false;
  if (c->mode == SPD_MODE_SAMPLE && !(c->temperature > 0.f)) return false;
  if (c->max_new < 1 || c->max_ctx < c->n_stages + 2) return false;
  if (align_up((size_t)c->max_ctx, kSplit) / kSplit > (size_t)kMaxSplit) return false;
  if (!(c->rms_eps >= 0.f) || !(c->rope_base > 1.f)) return false;
  if (c->schedule != SPD_SCHED_PRE && c->schedule != SPD_SCHED_POST) return false;
  // one stage: the exiting token verifies the draft made in its own cycle,
  // which the post-step schedule would make only after that verification
  if (c->schedule == SPD_SCHED_POST && c->n_stages < 2) return false;
  if (c->top_k < 0 || c->top_k > SPD_MAX_TOPK || c->top_k > c->vocab) return false;
  if (c->attn_period < 0 || c->attn_period > c->n_layers) return false;
  // draft trees: greedy, pre-step, n >= 2, softmax attention, uniform stages,
  // and the draft module's rows (2 + (n - 1) W) within two row tiles
  if (c->draft_width < 0 || c->draft_width > SPD_MAX_WIDTH) return false;
  if (c->draft_width >= 2) {
    if (c->mode != SPD_MODE_GREEDY || c->schedule != SPD_SCHED_PRE || c->n_stages < 2 || c->attn_period != 0 ||
        has_split(c))
      return false;
    if (2 + (c->n_stages - 1) * c->draft_width > kMaxTreeRows) return false;
  }
  return true;
}

int width_of(const spd_config* c) { return c->draft_width >= 2 ? c->draft_width : 1; }

// Workgroups of k_topk_blocks over a vocabulary of V ids, and the candidate
// keys they leave (64 each).
int topk_groups(int V) {
  const int nb = (V + kCdfBlock - 1) / kCdfBlock;
  return (nb + kTopkBlocksPerWG - 1) / kTopkBlocksPerWG;
}
int topk_candidates(int V) { return topk_groups(V) * kWave; }

// K ranges of one matrix-core product (N weight rows, K inputs): one when
// the 64-row groups alone cover the CUs (the epilogue then stays in the
// GEMV), else the divisor of K / kMKC closest to ~640 workgroups in total.
int mfma_splits(int N, int K) {
  const int groups = N / kMGroup;
  if (groups >= kCUs) return 1;  // the epilogue stays fused: no reduce launch
  const int chunks = K / kMKC;
  const int target = (640 + groups - 1) / groups;
  int best = 1;
  for (int s = 1; s <= std::min(chunks, kMMaxSplit); ++s) {
    if (chunks % s) continue;
    if (std::abs(s - target) < std::abs(best - target)) best = s;
  }
  return best;
}

// Partial-tile floats a product set needs (0 when no K is split).
size_t mfma_part_floats(int N, const int* Ks, int nprob, int rows) {
  size_t slabs = 0;
  for (int p = 0; p < nprob; ++p) {
    const int S = mfma_splits(N, Ks[p]);
    if (S > 1) slabs += S;
  }
  return slabs * rows * (size_t)N;
}

Layout make_layout(const spd_config* c) {
  Layout L{};
  const size_t es = c->dtype == SPD_DTYPE_BF16 ? 2 : 4;
  const int n = c->n_stages, d = c->d_model, Hq = c->n_heads, Hkv = c->n_kv_heads, hd = c->head_dim;
  const int F = c->d_ffn, V = c->vocab, m = c->n_anchors;
  const int Wd = width_of(c);  // draft-tree width: KV lanes, nodes per position
  L.ctx_cap = (int)align_up((size_t)c->max_ctx, kSplit);
  L.nsplit = L.ctx_cap / kSplit;
  const int prow_max = Wd > 1 ? 2 + (n - 1) * Wd : n + 1;  // draft-module rows
  L.mr = std::max(kRowsMR, (int)align_up((size_t)prow_max, kRowsMR));
  L.log_cap = std::max(4096, n * c->max_new + 64);
  L.nparts_max = kCUs * kPersistPerCU;
  const int nslots = n + 1;
  size_t off = 0, soff = 0;
  auto take = [&](size_t bytes) {  // persistent state
    size_t o = off;
    off = align_up(off + bytes, kAlign);
    return o;
  };
  auto scr = [&](size_t bytes) {  // scratch: rewritten before it is read within a cycle or a call
    size_t o = soff;
    soff = align_up(soff + bytes, kAlign);
    return o;
  };
  L.ctrl = take(sizeof(Ctrl) + sizeof(Tree));
  L.kv_len = take(sizeof(int32_t) * SPD_MAX_LAYERS);
  L.tokens = take(sizeof(int32_t) * L.ctx_cap);
  L.dring = take(sizeof(int32_t) * nslots);
  const bool smp = c->mode == SPD_MODE_SAMPLE;
  // draft distributions Q by slot: dense [V] weights, or the top-k (id, weight) pairs
  L.qring = take(!smp ? 0 : c->top_k ? sizeof(SparseQ) * nslots : sizeof(float) * nslots * (size_t)V);
  L.qz = take(sizeof(double) * nslots);
  const size_t kvl = (size_t)Hkv * hd * L.ctx_cap * es;
  L.kc = take(kvl * c->n_layers * Wd);
  L.vc = take(kvl * c->n_layers * Wd);
  L.pkc = take(kvl * c->pdm_layers * Wd);
  L.pvc = take(kvl * c->pdm_layers * Wd);
  L.rcos = take(sizeof(float) * (size_t)L.ctx_cap * (hd / 2));
  L.rsin = take(sizeof(float) * (size_t)L.ctx_cap * (hd / 2));
  L.hslots = take(sizeof(float) * (size_t)nslots * Wd * d);
  L.anchors = take(sizeof(float) * (size_t)nslots * Wd * m * d);
  const size_t qd = (size_t)Hq * hd;
  const int srows = n * Wd;  // stage-step rows: W nodes per stage group
  L.s_q = scr(sizeof(float) * srows * qd);
  L.s_pacc = scr(sizeof(float) * srows * (size_t)Hq * L.nsplit * hd);
  L.s_pml = scr(sizeof(float) * srows * (size_t)Hq * L.nsplit * 2);
  L.s_o = scr(sizeof(float) * srows * qd);
  L.s_act = scr(sizeof(float) * srows * (size_t)F);
  L.Xt = scr(sizeof(float) * L.mr * (size_t)d);
  L.Xp = scr(sizeof(float) * L.mr * (size_t)d);
  L.r_q = scr(sizeof(float) * L.mr * qd);
  L.r_pacc = scr(sizeof(float) * L.mr * (size_t)Hq * L.nsplit * hd);
  L.r_pml = scr(sizeof(float) * L.mr * (size_t)Hq * L.nsplit * 2);
  L.r_o = scr(sizeof(float) * L.mr * qd);
  L.r_act = scr(sizeof(float) * L.mr * (size_t)F);
  L.taps = scr(sizeof(float) * kRowsMR * (size_t)m * d);
  L.logits = scr(sizeof(float) * (size_t)V);
  L.plogits = scr(sizeof(float) * (size_t)V * Wd);
  L.pw = scr(sizeof(float) * (size_t)V);
  L.parts = scr(sizeof(ArgPair) * L.nparts_max);
  L.pparts = scr(sizeof(ArgPair) * L.nparts_max * Wd);
  const int nblk = Wd > 1 ? tree_scan_blocks(V) : 0;
  L.zpart = scr(sizeof(double) * Wd * nblk);
  L.tpart = scr(sizeof(ArgPair) * Wd * nblk * Wd);
  L.ring = take(sizeof(spd_cycle_rec) * (size_t)L.log_cap);
  // matrix-core path (bf16): per-row partial sums of squares of the prefill
  // rows and the draft-module rows, and the split-K partial tiles
  L.ssq_t = scr(sizeof(float) * L.mr * (size_t)(d / kSsqCols));
  L.ssq_p = scr(sizeof(float) * L.mr * (size_t)(d / kSkinnyCols));  // 64- or 16-column parts
  size_t pf = 0;
  if (c->dtype == SPD_DTYPE_BF16) {
    const int rows = L.mr;  // 16 * MT of the largest pass
    const int qk[1] = {(int)qd}, dd[1] = {d}, ff[1] = {F};
    pf = std::max(pf, mfma_part_floats((Hq + 2 * Hkv) * hd, dd, 1, rows));
    pf = std::max(pf, mfma_part_floats(d, qk, 1, rows));
    pf = std::max(pf, mfma_part_floats(2 * F, dd, 1, rows));
    pf = std::max(pf, mfma_part_floats(d, ff, 1, rows));
    int fk[SPD_MAX_ANCHORS];
    for (int f = 0; f < m; ++f) fk[f] = (f + 1) * d;
    pf = std::max(pf, mfma_part_floats(d, fk, m, rows));
    const int full[1] = {m * d};
    pf = std::max(pf, mfma_part_floats(d, full, 1, rows));
  }
  L.mpart = scr(sizeof(float) * std::max<size_t>(pf, 1));
  // draft module in the cycle (bf16): its layer weights re-tiled once at init,
  // and the split inputs its skinny products read
  const bool bf = c->dtype == SPD_DTYPE_BF16;
  const size_t qkv_rows = (size_t)(Hq + 2 * Hkv) * hd;
  L.wtile = take(bf ? (size_t)c->pdm_layers * (qkv_rows * d + d * qd + 2 * (size_t)F * d + (size_t)d * F) * 2 : 0);
  L.xs_h = scr(bf ? sizeof(uint16_t) * L.mr * (size_t)d : 0);
  L.xs_l = scr(bf ? sizeof(uint16_t) * L.mr * (size_t)d : 0);
  L.as_h = scr(bf ? sizeof(uint16_t) * L.mr * (size_t)F : 0);
  L.as_l = scr(bf ? sizeof(uint16_t) * L.mr * (size_t)F : 0);
  L.os_h = scr(bf ? sizeof(uint16_t) * L.mr * qd : 0);
  L.os_l = scr(bf ? sizeof(uint16_t) * L.mr * qd : 0);
  // hybrid target: linear-attention state ring [L][nslots][Hkv][hd*hd + hd]
  // and its copy at the end of prefill [L][Hkv][hd*hd + hd]
  const size_t lin_one = (size_t)Hkv * ((size_t)hd * hd + hd);
  L.lin_state = take(c->attn_period > 0 ? sizeof(float) * (size_t)c->n_layers * nslots * lin_one : 0);
  L.lin_ckpt = take(c->attn_period > 0 ? sizeof(float) * (size_t)c->n_layers * lin_one : 0);
  // dense sampling: block sums of Q (draft) and P (target) from k_softmax_blocks
  const size_t nbs = smp && !c->top_k ? (size_t)(V + kCdfBlock - 1) / kCdfBlock : 0;
  L.bsq = scr(sizeof(double) * nbs);
  L.bsp = scr(sizeof(double) * nbs);
  // top-k sampling: candidate keys of Q and P from k_topk_blocks
  const size_t ntk = smp && c->top_k ? (size_t)topk_candidates(V) : 0;
  L.tkq = scr(sizeof(unsigned long long) * ntk);
  L.tkp = scr(sizeof(unsigned long long) * ntk);
  L.state_total = off;
  L.scratch_total = std::max<size_t>(soff, kAlign);
  L.total = L.state_total + L.scratch_total;
  return L;
}

}  // namespace

struct spd_handle {
  spd_config cfg;
  spd_weights w;
  Geo g;
  Layout lay;
  hipStream_t ss, ps;
  hipEvent_t ev_entry = nullptr, ev_pdm = nullptr;
  char* ws;
  Ctrl* ctrl;
  int32_t *kv_len, *tokens, *dring;
  float* qring;
  double* qz;
  void *kc, *vc, *pkc, *pvc;
  float *rcos, *rsin, *hslots, *anchors;
  float *s_q, *s_pacc, *s_pml, *s_o, *s_act;
  float *Xt, *Xp, *r_q, *r_pacc, *r_pml, *r_o, *r_act, *taps;
  float *logits, *plogits, *pw;
  ArgPair *parts, *pparts;
  spd_cycle_rec* ring;
  float *ssq_t, *ssq_p, *mpart;
  uint16_t* wtile = nullptr;  // draft-module layer weights in tile order: per layer q/k/v, o, gate/up, down
  uint16_t *xs_h = nullptr, *xs_l = nullptr, *as_h = nullptr, *as_l = nullptr, *os_h = nullptr, *os_l = nullptr;
  float *lin_state = nullptr, *lin_ckpt = nullptr;
  double *bsq = nullptr, *bsp = nullptr;  // dense sampling block sums (Q, P)
  double* zpart = nullptr;                 // draft tree: per-leaf softmax partial sums
  ArgPair* tpart = nullptr;                // draft tree: per-leaf partial top-W
  float p_first = 0.f, p_tree = 0.f;       // draft tree forced policy
  unsigned long long *tkq = nullptr, *tkp = nullptr;  // top-k candidate keys (Q, P)
  int ckpt_len = 0;     // prefill length whose linear-attention states lin_ckpt holds
  int lin_newest = -1;  // newest position whose linear-attention state a row pass wrote
  int lin_keep_from = 0;
  int policy = SPD_DRAFT_NATURAL;
  float p_accept = 0.f;
  const int32_t* ref = nullptr;
  int ref_len = 0;
  const float* uni = nullptr;
  int uni_len = 0;
  int prefilled = 0, P = 0, needs_rollback = 0, ar_complete = 0;
  long long cyc = 0;
  int hip_err = 0;
  // timing
  int timing = 0;
  int launch_mode = 1;  // 0: every kernel launched from the host; 1: per-stream graphs
  int serialized = 0;   // the draft module runs on the stage stream before the stage step
  int graphs_valid = 0;
  hipGraphExec_t gx_stage = nullptr, gx_pdm = nullptr;
  std::vector<hipEvent_t> pool;
  size_t pool_next = 0;
  std::vector<hipEvent_t> cyc_ev;   // 3 per timed cycle: start, stage end, pdm end
  std::vector<hipEvent_t> gu_ev;    // 2 per timed gate/up launch
};

#define HIPCHK(h, x)                          \
  do {                                        \
    hipError_t _e = (x);                      \
    if (_e != hipSuccess) {                   \
      (h)->hip_err = (int)_e;                 \
      return SPD_EHIP;                        \
    }                                         \
  } while (0)

// Record a HIP error in the handle; the ABI result for it.
int hip_fail(spd_t* h, hipError_t e) {
  h->hip_err = (int)e;
  return SPD_EHIP;
}

// Most draft-module rows of one cycle: the committed-next row and the tokens
// in flight (a draft tree: one oldest node, W per later position).
int pdm_rows(const Geo& g) { return g.W > 1 ? 2 + (g.n - 1) * g.W : g.n + 1; }

namespace {

hipEvent_t pool_event(spd_t* h) {
  if (h->pool_next == h->pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    h->pool.push_back(e);
  }
  return h->pool[h->pool_next++];
}

// Persistent grid of the stage-grouped GEMV: three workgroups per CU (the
// measured optimum over 1..6 per CU for the 4B/9B shapes and occupancies),
// fewer if LDS does not allow it or there are fewer tiles.
int stage_grid(int units, int upt, int n_groups, int K) {
  const int tiles = n_groups * ((units + upt - 1) / upt);
  const int lds = K * (int)sizeof(float) + 512;
  const int occ = std::max(1, std::min(kPersistPerCU, 160 * 1024 / lds));
  return std::max(1, std::min(tiles, kCUs * occ));
}

template <typename WT, int EPI, int NR = 1>
void launch_stage(spd_t* h, const StageGemv& a, int n_groups_max, hipStream_t s, int* grid_out = nullptr) {
  constexpr int upt = (epi_pairs(EPI) ? 2 : 4) * (kWG / kWave);
  // un-normalised long inputs (the down projection) are read from the cache
  // rather than staged: no LDS, so the draft stream's kernels fit beside it
  const bool xg = EPI == EPI_RESID && a.K > h->g.d;
  const int grid = stage_grid(a.units, upt, n_groups_max, xg ? 0 : NR * a.K);
  if (grid_out) *grid_out = grid;
  if (xg)
    hipLaunchKernelGGL((k_gemv_stage<WT, EPI, true, NR>), dim3(grid), dim3(kWG), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemv_stage<WT, EPI, false, NR>), dim3(grid), dim3(kWG), NR * a.K * sizeof(float), s, a);
}

// The stage GEMVs of a draft tree take the W nodes of a stage as rows.
template <typename WT, int EPI>
void launch_stage_w(spd_t* h, const StageGemv& a, int n_groups_max, hipStream_t s, int* grid_out = nullptr) {
  switch (h->g.W) {
    case 1: launch_stage<WT, EPI, 1>(h, a, n_groups_max, s, grid_out); break;
    case 2: launch_stage<WT, EPI, 2>(h, a, n_groups_max, s, grid_out); break;
    case 3: launch_stage<WT, EPI, 3>(h, a, n_groups_max, s, grid_out); break;
    default: launch_stage<WT, EPI, 4>(h, a, n_groups_max, s, grid_out); break;
  }
}

template <typename WT, int EPI>
void launch_rows(spd_t* h, RowsGemv a, int max_rows, hipStream_t s) {
  constexpr int upt = (epi_pairs(EPI) ? 2 : 4) * (kWG / kWave);
  const int tiles = (a.units + upt - 1) / upt;
  for (int rb = 0; rb < max_rows; rb += kRowsMR) {
    a.row_base = rb;
    hipLaunchKernelGGL((k_gemv_rows<WT, EPI>), dim3(tiles, a.n_groups), dim3(kWG), 0, s, a);
  }
}

StageGemv stage_base(spd_t* h) {
  StageGemv a;
  memset(&a, 0, sizeof(a));
  for (int i = 0; i < SPD_MAX_STAGES; ++i) {
    a.anchor_idx[i] = -1;
    a.stage[i] = i;
  }
  a.ctrl = h->ctrl;
  a.g = h->g;
  a.rcos = h->rcos;
  a.rsin = h->rsin;
  return a;
}

RowsGemv rows_base(spd_t* h) {
  RowsGemv a;
  memset(&a, 0, sizeof(a));
  a.anchor_idx = -1;
  a.ctrl = h->ctrl;
  a.g = h->g;
  a.rcos = h->rcos;
  a.rsin = h->rsin;
  a.n_groups = 1;
  return a;
}

// Split attention + split merge.  Matrix cores for bf16 caches (query tiles
// of 16: QT = 1 for one token, up to 4 for blocks of rows), VALU for fp32.
template <typename WT, int HD>
void attention_launch(const Attn& t, dim3 grid, int QT, int merge_rows, hipStream_t s) {
  // merge_rows == 0: the consumer merges the splits itself
  if (sizeof(WT) == 2) {
    switch (QT) {
      case 1: hipLaunchKernelGGL((k_attn_mfma<HD, 1>), grid, dim3(kWG), attn_mfma_lds(HD, 1), s, t); break;
      case 2: hipLaunchKernelGGL((k_attn_mfma<HD, 2>), grid, dim3(kWG), attn_mfma_lds(HD, 2), s, t); break;
      case 3: hipLaunchKernelGGL((k_attn_mfma<HD, 3>), grid, dim3(kWG), attn_mfma_lds(HD, 3), s, t); break;
      default: hipLaunchKernelGGL((k_attn_mfma<HD, 4>), grid, dim3(kWG), attn_mfma_lds(HD, 4), s, t); break;
    }
  } else {
    hipLaunchKernelGGL((k_attn_valu<WT, HD>), grid, dim3(kWG), 0, s, t);
  }
  if (merge_rows > 0) hipLaunchKernelGGL((k_attn_merge<HD>), dim3(merge_rows, t.g.Hq), dim3(HD), 0, s, t);
}

template <typename WT>
void attention_any(const Attn& t, dim3 grid, int QT, int merge_rows, hipStream_t s) {
  if (t.g.hd == 128)
    attention_launch<WT, 128>(t, grid, QT, merge_rows, s);
  else
    attention_launch<WT, 64>(t, grid, QT, merge_rows, s);
}

// Dynamic LDS above the default limit for the matrix-core attention kernels.
hipError_t attn_lds_limits() {
  hipError_t e = hipSuccess;
#define SPD_ATTN_LDS(HD, QT)                                                                              \
  if (e == hipSuccess)                                                                                    \
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_mfma<HD, QT>),                         \
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)attn_mfma_lds(HD, QT));
  SPD_ATTN_LDS(128, 1) SPD_ATTN_LDS(128, 2) SPD_ATTN_LDS(128, 3) SPD_ATTN_LDS(128, 4)
  SPD_ATTN_LDS(64, 1) SPD_ATTN_LDS(64, 2) SPD_ATTN_LDS(64, 3) SPD_ATTN_LDS(64, 4)
#undef SPD_ATTN_LDS
  return e;
}

// Linear attention of a hybrid target's layer over consecutive rows (prefill
// chunk or autoregressive token), output fp32 rows r_o.
template <typename WT>
void rows_linattn(spd_t* h, int layer, int M, int pos0, hipStream_t s) {
  const Geo& g = h->g;
  LinAttn t;
  memset(&t, 0, sizeof(t));
  t.mode = LM_ROWS;
  t.layer[0] = layer;
  t.kc = h->kc;
  t.vc = h->vc;
  t.q = h->r_q;
  t.ldq = g.Hq * g.hd;
  t.o = h->r_o;
  t.ldo = g.Hq * g.hd;
  t.state = h->lin_state;
  t.pos0 = pos0;
  t.nrows = M;
  t.keep_from = h->lin_keep_from;
  t.ctrl = h->ctrl;
  t.g = g;
  if (g.hd == 128)
    hipLaunchKernelGGL((k_linattn<WT, 128>), dim3(g.Hkv, 1), dim3(kWG), 0, s, t);
  else
    hipLaunchKernelGGL((k_linattn<WT, 64>), dim3(g.Hkv, 1), dim3(kWG), 0, s, t);
  h->lin_newest = std::max(h->lin_newest, pos0 + M - 1);
}

// Attention over row-batched queries (prefill chunk, AR token or the draft
// module's trailing rows); output fp32 rows r_o.
template <typename WT>
void rows_attention(spd_t* h, void* kc, void* vc, int layer, int M, int pos0, int from_ctrl, int max_rows,
                    bool merge, hipStream_t s, uint16_t* oh = nullptr, uint16_t* ol = nullptr) {
  const Geo& g = h->g;
  const int G = g.Hq / g.Hkv;
  Attn t;
  memset(&t, 0, sizeof(t));
  t.pmode = PM_ROWS;
  t.layer[0] = layer;
  t.kc = kc;
  t.vc = vc;
  t.q = h->r_q;
  t.pacc = h->r_pacc;
  t.pml = h->r_pml;
  t.o = h->r_o;
  t.oh = oh;
  t.ol = ol;
  t.from_ctrl = from_ctrl;
  t.pos0_arg = pos0;
  t.nrows_arg = M;
  int QT = 1;
  if (from_ctrl && g.W > 1) {
    // a draft tree's rows: one per workgroup, each at its own position and lane
    t.QB = 1;
    QT = (G + 15) / 16;
    t.lane_stride = g.lane_pkv;
  } else if (sizeof(WT) == 2) {
    // one query tile per workgroup: more workgroups, each streaming its KV
    // split once more from the cache
    t.QB = std::max(1, std::min(16 / G, max_rows));
    QT = (t.QB * G + 15) / 16;
  } else {
    t.QB = std::max(1, kAttnQ / G);
  }
  t.qblocks = (max_rows + t.QB - 1) / t.QB;
  t.ctrl = h->ctrl;
  t.g = g;
  attention_any<WT>(t, dim3(g.nsplit, g.Hkv * t.qblocks, 1), QT, merge ? max_rows : 0, s);
}

// One decoder layer over row-batched activations X on the VALU row GEMV
// (fp32 models, and the autoregressive decoder, whose per-row arithmetic
// matches the stage kernels bit for bit).
template <typename WT>
void rows_layer(spd_t* h, const spd_layer_weights& lw, void* kc, void* vc, int layer, float* X, int M,
                int pos0, int from_ctrl, int* kv_len, float* taps, int anchor_idx, hipStream_t s,
                bool linear = false) {
  const Geo& g = h->g;
  const int max_rows = from_ctrl ? pdm_rows(g) : M;
  const int qd = g.Hq * g.hd;
  RowsGemv a = rows_base(h);
  a.from_ctrl = from_ctrl;
  a.M_arg = M;
  a.pos0_arg = pos0;
  // q/k/v + RoPE + cache append
  a.W[0] = lw.w_qkv;
  a.Kg[0] = g.d;
  a.gamma = (const float*)lw.attn_norm;
  a.N = g.qkv_rows;
  a.units = g.qkv_rows / 2;
  a.x = X;
  a.ldx = g.d;
  a.out = h->r_q;
  a.ldo = qd;
  a.layer = layer;
  a.kc = kc;
  a.vc = vc;
  a.kv_len = kv_len;
  launch_rows<WT, EPI_QKV>(h, a, max_rows, s);
  if (linear)
    rows_linattn<WT>(h, layer, M, pos0, s);
  else
    rows_attention<WT>(h, kc, vc, layer, M, pos0, from_ctrl, max_rows, true, s);
  // output projection + residual
  a = rows_base(h);
  a.from_ctrl = from_ctrl;
  a.M_arg = M;
  a.pos0_arg = pos0;
  a.W[0] = lw.w_o;
  a.Kg[0] = qd;
  a.N = g.d;
  a.units = g.d;
  a.x = h->r_o;
  a.ldx = qd;
  a.out = X;
  a.ldo = g.d;
  launch_rows<WT, EPI_RESID>(h, a, max_rows, s);
  // norm + gate/up + SwiGLU
  a.W[0] = lw.w_gu;
  a.Kg[0] = g.d;
  a.gamma = (const float*)lw.ffn_norm;
  a.N = 2 * g.F;
  a.units = g.F;
  a.x = X;
  a.ldx = g.d;
  a.out = h->r_act;
  a.ldo = g.F;
  launch_rows<WT, EPI_SWIGLU>(h, a, max_rows, s);
  // down + residual (+ anchor taps)
  a.W[0] = lw.w_down;
  a.Kg[0] = g.F;
  a.gamma = nullptr;
  a.N = g.d;
  a.units = g.d;
  a.x = h->r_act;
  a.ldx = g.F;
  a.out = X;
  a.ldo = g.d;
  a.anchors = taps;
  a.anchor_idx = anchor_idx;
  launch_rows<WT, EPI_RESID>(h, a, max_rows, s);
}

MfmaArgs mfma_base(spd_t* h) {
  MfmaArgs a;
  memset(&a, 0, sizeof(a));
  a.anchor_idx = -1;
  a.rmode = RM_CONTIG;
  a.ctrl = h->ctrl;
  a.g = h->g;
  a.rcos = h->rcos;
  a.rsin = h->rsin;
  a.part = h->mpart;
  return a;
}

// One matrix-core product set (nprob products of N rows): the GEMV, then the
// split-K reduction + epilogue if any product's K is split.
template <int EPI>
void launch_mfma(spd_t* h, MfmaArgs a, int nprob, int max_rows, hipStream_t s) {
  int smax = 1, off = 0;
  bool split = false;
  for (int p = 0; p < nprob; ++p) {
    a.S[p] = mfma_splits(a.N, a.K[p]);
    a.poff[p] = off;
    if (a.S[p] > 1) {
      off += a.S[p];
      split = true;
    }
    smax = std::max(smax, a.S[p]);
  }
  const dim3 grid(a.N / kMGroup, smax, nprob);
  if (max_rows <= 16) {
    hipLaunchKernelGGL((k_mfma_gemv<EPI, 1>), grid, dim3(kWG), 0, s, a);
    if (split)
      hipLaunchKernelGGL((k_mfma_reduce<EPI, 1>), dim3(a.N / kMGroup, 16, nprob), dim3(kWave), 0, s, a);
  } else {
    hipLaunchKernelGGL((k_mfma_gemv<EPI, 2, kMKC / 2>), grid, dim3(kWG), 0, s, a);
    if (split)
      hipLaunchKernelGGL((k_mfma_reduce<EPI, 2>), dim3(a.N / kMGroup, 32, nprob), dim3(kWave), 0, s, a);
  }
}

// The same layer on the matrix cores (bf16 weights): the draft module's
// trailing rows and prefill chunks.  X rows are updated in place; ssqX holds
// their per-row partial sums of squares (written by whoever wrote X).
void rows_layer_mfma(spd_t* h, const spd_layer_weights& lw, void* kc, void* vc, int layer, float* X, float* ssqX,
                     int M, int pos0, int from_ctrl, int* kv_len, float* taps, int anchor_idx, hipStream_t s,
                     bool linear = false) {
  const Geo& g = h->g;
  const int max_rows = from_ctrl ? pdm_rows(g) : M;
  const int qd = g.Hq * g.hd;
  MfmaArgs a = mfma_base(h);
  a.M_arg = M;
  a.pos0_arg = pos0;
  a.from_ctrl = from_ctrl;
  // norm + q/k/v + RoPE + cache append
  a.W[0] = (const uint16_t*)lw.w_qkv;
  a.K[0] = g.d;
  a.N = g.qkv_rows;
  a.x = X;
  a.ldx = g.d;
  a.gamma = (const float*)lw.attn_norm;
  a.ssq = ssqX;
  a.ssq_parts = g.d / kSsqCols;
  a.out = h->r_q;
  a.ldo = qd;
  a.layer = layer;
  a.kc = kc;
  a.vc = vc;
  a.kv_len = kv_len;
  launch_mfma<EPI_QKV>(h, a, 1, max_rows, s);
  // attention splits; the output projection merges them as it stages its
  // input (linear attention writes its rows whole)
  if (linear)
    rows_linattn<uint16_t>(h, layer, M, pos0, s);
  else
    rows_attention<uint16_t>(h, kc, vc, layer, M, pos0, from_ctrl, max_rows, false, s);
  // output projection + residual
  a.kv_len = nullptr;
  a.W[0] = (const uint16_t*)lw.w_o;
  a.K[0] = qd;
  a.N = g.d;
  if (linear) {
    a.rmode = RM_CONTIG;
    a.x = h->r_o;
    a.ldx = qd;
  } else {
    a.rmode = RM_ATTN;
    a.apacc = h->r_pacc;
    a.apml = h->r_pml;
  }
  a.gamma = nullptr;
  a.ssq = nullptr;
  a.out = X;
  a.ldo = g.d;
  a.ssq_out = ssqX;
  launch_mfma<EPI_RESID>(h, a, 1, max_rows, s);
  // norm + gate/up + SwiGLU
  a.rmode = RM_CONTIG;
  a.W[0] = (const uint16_t*)lw.w_gu;
  a.K[0] = g.d;
  a.N = 2 * g.F;
  a.x = X;
  a.ldx = g.d;
  a.gamma = (const float*)lw.ffn_norm;
  a.ssq = ssqX;
  a.out = h->r_act;
  a.ldo = g.F;
  a.ssq_out = nullptr;
  launch_mfma<EPI_SWIGLU>(h, a, 1, max_rows, s);
  // down + residual (+ anchor taps)
  a.W[0] = (const uint16_t*)lw.w_down;
  a.K[0] = g.F;
  a.N = g.d;
  a.x = h->r_act;
  a.ldx = g.F;
  a.gamma = nullptr;
  a.ssq = nullptr;
  a.out = X;
  a.ldo = g.d;
  a.ssq_out = ssqX;
  a.anchors = taps;
  a.anchor_idx = anchor_idx;
  launch_mfma<EPI_RESID>(h, a, 1, max_rows, s);
}

template <typename WT>
void layer_rows_any(spd_t* h, bool mfma, const spd_layer_weights& lw, void* kc, void* vc, int layer, float* X,
                    float* ssqX, int M, int pos0, int from_ctrl, int* kv_len, float* taps, int anchor_idx,
                    hipStream_t s, bool linear = false) {
  if (mfma && sizeof(WT) == 2)
    rows_layer_mfma(h, lw, kc, vc, layer, X, ssqX, M, pos0, from_ctrl, kv_len, taps, anchor_idx, s, linear);
  else
    rows_layer<WT>(h, lw, kc, vc, layer, X, M, pos0, from_ctrl, kv_len, taps, anchor_idx, s, linear);
}

// Head GEMV (final norm + LM head + per-workgroup argmax) on a fixed input row.
template <typename WT>
int head_fixed(spd_t* h, const float* x, const void* W, const void* gamma, float* logits, ArgPair* parts,
               hipStream_t s) {
  StageGemv a = stage_base(h);
  a.W[0] = W;
  a.gamma[0] = (const float*)gamma;
  a.N = h->g.V;
  a.K = h->g.d;
  a.units = h->g.V;
  a.n_groups = 1;
  a.gmode = GM_FIXED;
  a.x = x;
  a.out = logits;
  a.parts = parts;
  int grid = 0;
  launch_stage<WT, EPI_ARGMAX>(h, a, 1, s, &grid);
  return grid;
}

// ---- the draft module's products in the cycle on the skinny GEMV (bf16) ----
// Tile-order copy of draft layer l's matrix `which` (0 q/k/v, 1 o, 2 gate/up,
// 3 down) in the workspace, with its rows and inputs.
uint16_t* pdm_wtile(spd_t* h, int l, int which, int* N, int* K) {
  const Geo& g = h->g;
  const size_t qd = (size_t)g.Hq * g.hd;
  const size_t sz[4] = {(size_t)g.qkv_rows * g.d, (size_t)g.d * qd, 2 * (size_t)g.F * g.d, (size_t)g.d * g.F};
  const int Ns[4] = {g.qkv_rows, g.d, 2 * g.F, g.d};
  const int Ks[4] = {g.d, (int)qd, g.d, g.F};
  size_t off = (size_t)l * (sz[0] + sz[1] + sz[2] + sz[3]);
  for (int i = 0; i < which; ++i) off += sz[i];
  *N = Ns[which];
  *K = Ks[which];
  return h->wtile + off;
}

// Re-tile every draft layer's matrices once (at init; the caller's draft-layer
// buffers are not read by the cycle after this).
void tile_pdm_weights(spd_t* h, hipStream_t s) {
  const Geo& g = h->g;
  for (int l = 0; l < g.Ls; ++l) {
    const spd_layer_weights& lw = h->w.pdm[l];
    const void* src[4] = {lw.w_qkv, lw.w_o, lw.w_gu, lw.w_down};
    for (int i = 0; i < 4; ++i) {
      int N, K;
      uint16_t* dst = pdm_wtile(h, l, i, &N, &K);
      const int NW = skinny_ways(N, K);
      const uint16_t* w = (const uint16_t*)src[i];
      const dim3 grid(1024), blk(kWG);
      if (i == 0)
        hipLaunchKernelGGL(k_tile_weights<EPI_QKV>, grid, blk, 0, s, w, dst, N, K, NW, g);
      else if (i == 2)
        hipLaunchKernelGGL(k_tile_weights<EPI_SWIGLU>, grid, blk, 0, s, w, dst, N, K, NW, g);
      else
        hipLaunchKernelGGL(k_tile_weights<EPI_RESID>, grid, blk, 0, s, w, dst, N, K, NW, g);
    }
  }
}

template <int EPI, int MT>
void launch_skinny_mt(const SkinnyArgs& a, int NW, hipStream_t s) {
  const dim3 grid(a.N / 16);
  switch (NW) {
    case 16: hipLaunchKernelGGL((k_skinny<EPI, MT, 16>), grid, dim3(16 * kWave), 0, s, a); break;
    case 8: hipLaunchKernelGGL((k_skinny<EPI, MT, 8>), grid, dim3(8 * kWave), 0, s, a); break;
    default: hipLaunchKernelGGL((k_skinny<EPI, MT, 4>), grid, dim3(4 * kWave), 0, s, a); break;
  }
}

template <int EPI>
void launch_skinny(spd_t* h, const SkinnyArgs& a, hipStream_t s) {
  const int NW = skinny_ways(a.N, a.K);
  if (pdm_rows(h->g) <= 16)
    launch_skinny_mt<EPI, 1>(a, NW, s);
  else
    launch_skinny_mt<EPI, 2>(a, NW, s);
}

// One draft-module layer over the cycle's trailing rows (rows and positions
// from the control block).  X = Xp in place; on entry xs holds the split of
// attn_norm (.) X and ssq_p its partial sums of squares (ssq_parts per row).
void pdm_layer_skinny(spd_t* h, int l, int ssq_parts, hipStream_t s) {
  const Geo& g = h->g;
  const spd_layer_weights& lw = h->w.pdm[l];
  const int qd = g.Hq * g.hd;
  SkinnyArgs a;
  memset(&a, 0, sizeof(a));
  a.layer = l;
  a.kc = h->pkc;
  a.vc = h->pvc;
  a.rcos = h->rcos;
  a.rsin = h->rsin;
  a.anchor_idx = -1;
  a.ctrl = h->ctrl;
  a.g = g;
  // norm + q/k/v + RoPE + cache append
  a.Wt = pdm_wtile(h, l, 0, &a.N, &a.K);
  a.xh = h->xs_h;
  a.xl = h->xs_l;
  a.ssq = h->ssq_p;
  a.ssq_parts = ssq_parts;
  a.out = h->r_q;
  a.ldo = qd;
  launch_skinny<EPI_QKV>(h, a, s);
  // attention splits, merged into the split input of the o-projection
  rows_attention<uint16_t>(h, h->pkc, h->pvc, l, 0, 0, 1, pdm_rows(g), true, s, h->os_h, h->os_l);
  // o-projection + residual; hands over the split of ffn_norm (.) X
  a.Wt = pdm_wtile(h, l, 1, &a.N, &a.K);
  a.xh = h->os_h;
  a.xl = h->os_l;
  a.ssq = nullptr;
  a.out = h->Xp;
  a.ldo = g.d;
  a.ssq_out = h->ssq_p;
  a.yh = h->xs_h;
  a.yl = h->xs_l;
  a.ygamma = (const float*)lw.ffn_norm;
  launch_skinny<EPI_RESID>(h, a, s);
  // norm + gate/up + SwiGLU into the split input of the down projection
  a.Wt = pdm_wtile(h, l, 2, &a.N, &a.K);
  a.xh = h->xs_h;
  a.xl = h->xs_l;
  a.ssq = h->ssq_p;
  a.ssq_parts = g.d / kSkinnyCols;
  a.ssq_out = nullptr;
  a.yh = h->as_h;
  a.yl = h->as_l;
  a.ygamma = nullptr;
  launch_skinny<EPI_SWIGLU>(h, a, s);
  // down + residual; hands over the split of the next layer's attn_norm (.) X
  a.Wt = pdm_wtile(h, l, 3, &a.N, &a.K);
  a.xh = h->as_h;
  a.xl = h->as_l;
  a.ssq = nullptr;
  a.out = h->Xp;
  a.ldo = g.d;
  a.ssq_out = h->ssq_p;
  const bool next = l + 1 < g.Ls;
  a.yh = next ? h->xs_h : nullptr;
  a.yl = next ? h->xs_l : nullptr;
  a.ygamma = next ? (const float*)h->w.pdm[l + 1].attn_norm : nullptr;
  launch_skinny<EPI_RESID>(h, a, s);
}

// Draft-module chain of one cycle (draft stream): anchor gather + FC, Ls
// layers over the trailing rows, draft head, finalisation.
template <typename WT>
int pdm_chain(spd_t* h, hipStream_t ps) {
  const Geo& g = h->g;
  const spd_weights& w = h->w;
  // ---------------- draft module (pre-step) on the draft stream ----------------
  {
    // anchor gather + concat + FC: one product per fusion pattern f, over the
    // trailing rows whose depth uses it
    if (sizeof(WT) == 2) {
      MfmaArgs a = mfma_base(h);
      a.rmode = RM_FC;
      a.from_ctrl = 1;
      for (int f = 0; f < g.m; ++f) {
        a.W[f] = (const uint16_t*)w.fc[f];
        a.K[f] = (f + 1) * g.d;
      }
      a.N = g.d;
      a.slot_anchors = h->anchors;
      a.out = h->Xp;
      a.ldo = g.d;
      a.ssq_out = h->ssq_p;
      a.yh = h->xs_h;
      a.yl = h->xs_l;
      a.ygamma = (const float*)w.pdm[0].attn_norm;
      launch_mfma<EPI_STORE>(h, a, g.m, pdm_rows(g), ps);
    } else {
      RowsGemv a = rows_base(h);
      a.rmode = RM_FC;
      a.from_ctrl = 1;
      a.n_groups = g.m;
      for (int f = 0; f < g.m; ++f) {
        a.W[f] = w.fc[f];
        a.Kg[f] = (f + 1) * g.d;
      }
      a.N = g.d;
      a.units = g.d;
      a.out = h->Xp;
      a.ldo = g.d;
      a.slot_anchors = h->anchors;
      launch_rows<WT, EPI_STORE>(h, a, pdm_rows(g), ps);
    }
    for (int l = 0; l < g.Ls; ++l) {
      if (sizeof(WT) == 2)
        pdm_layer_skinny(h, l, l == 0 ? g.d / kSsqCols : g.d / kSkinnyCols, ps);
      else
        layer_rows_any<WT>(h, true, w.pdm[l], h->pkc, h->pvc, l, h->Xp, h->ssq_p, 0, 0, 1, nullptr, nullptr, -1, ps);
    }
    StageGemv hd = stage_base(h);
    hd.W[0] = w.pdm_lm_head;
    hd.gamma[0] = (const float*)w.pdm_final_norm;
    hd.N = g.V;
    hd.K = g.d;
    hd.units = g.V;
    hd.n_groups = 1;
    hd.gmode = GM_PDMLAST;
    hd.x = h->Xp;
    hd.x_stride = g.d;
    hd.out = h->plogits;
    hd.parts = h->pparts;
    int grid = 0;
    if (g.W > 1) {
      // a draft tree: the leaves' heads in one weight stream, then their
      // normalisers and best W tokens, the ranking and the forced policy
      launch_stage_w<WT, EPI_ARGMAX>(h, hd, 1, ps, &grid);
      TreeScanArgs sa;
      memset(&sa, 0, sizeof(sa));
      sa.logits = h->plogits;
      sa.parts = h->pparts;
      sa.nparts = grid;
      sa.zpart = h->zpart;
      sa.tpart = h->tpart;
      sa.ctrl = h->ctrl;
      sa.g = g;
      const int nblk = tree_scan_blocks(g.V);
      hipLaunchKernelGGL(k_tree_scan, dim3(nblk, g.W), dim3(kWG), 0, ps, sa);
      TreeFinalizeArgs fa;
      memset(&fa, 0, sizeof(fa));
      fa.logits = h->plogits;
      fa.parts = h->pparts;
      fa.nparts = grid;
      fa.zpart = h->zpart;
      fa.tpart = h->tpart;
      fa.nblk = nblk;
      fa.uni = h->uni;
      fa.policy = h->policy;
      fa.p_first = h->p_first;
      fa.p_tree = h->p_tree;
      fa.ref = h->ref;
      fa.ref_len = h->ref_len;
      fa.ring = h->ring;
      fa.ctrl = h->ctrl;
      fa.g = g;
      hipLaunchKernelGGL(k_tree_finalize, dim3(1), dim3(kWG), 0, ps, fa);
      return hipGetLastError() == hipSuccess ? SPD_OK : SPD_EHIP;
    }
    launch_stage<WT, EPI_ARGMAX>(h, hd, 1, ps, &grid);
    if (h->bsq) {
      SoftmaxArgs sm;
      memset(&sm, 0, sizeof(sm));
      sm.parts = h->pparts;
      sm.nparts = grid;
      sm.logits = h->plogits;
      sm.qring = h->qring;
      sm.bs = h->bsq;
      sm.temp = h->cfg.temperature;
      sm.ctrl = h->ctrl;
      sm.g = g;
      const int nb = (g.V + kCdfBlock - 1) / kCdfBlock;
      hipLaunchKernelGGL(k_softmax_blocks, dim3((nb + kWG / kWave - 1) / (kWG / kWave)), dim3(kWG), 0, ps, sm);
    }
    if (h->tkq) {
      TopkArgs tk;
      memset(&tk, 0, sizeof(tk));
      tk.logits = h->plogits;
      tk.cand = h->tkq;
      tk.ctrl = h->ctrl;
      tk.g = g;
      hipLaunchKernelGGL(k_topk_blocks, dim3(topk_groups(g.V)), dim3(kWG), 0, ps, tk);
    }
    FinalizeArgs f;
    memset(&f, 0, sizeof(f));
    f.parts = h->pparts;
    f.nparts = grid;
    f.bs = h->bsq;
    f.tk = h->tkq;
    f.ntk = h->tkq ? topk_candidates(g.V) : 0;
    f.logits = h->plogits;
    f.dring = h->dring;
    f.qring = h->qring;
    f.qz = h->qz;
    f.uni = h->uni;
    f.mode = h->cfg.mode;
    f.temp = h->cfg.temperature;
    f.policy = h->policy;
    f.p_accept = h->p_accept;
    f.ref = h->ref;
    f.ref_len = h->ref_len;
    f.ring = h->ring;
    f.ctrl = h->ctrl;
    f.g = g;
    hipLaunchKernelGGL(k_pdm_finalize, dim3(1), dim3(kCtlThreads), 0, ps, f);
  }
  return hipGetLastError() == hipSuccess ? SPD_OK : SPD_EHIP;
}

// Stage chain of one cycle (stage stream): L/n stage-grouped layer
// sub-steps, verification head, verify / rollback.  With timing_gu, every
// gate/up launch is bracketed by HIP events on this stream.
template <typename WT>
int stage_chain(spd_t* h, hipStream_t ss, bool timing_gu) {
  const Geo& g = h->g;
  const spd_weights& w = h->w;
  // ---------------- stage step on the stage stream ----------------
  const int qd = g.Hq * g.hd;
  for (int j = 0; j < g.per; ++j) {
    // groups of sub-step j: the stages that still have a layer, in stage
    // order (all n stages under the uniform split)
    int ng = 0, gstage[SPD_MAX_STAGES], glayer[SPD_MAX_STAGES];
    for (int k = 0; k < g.n; ++k)
      if (g.sstart[k] + j < g.sstart[k + 1]) {
        gstage[ng] = k;
        glayer[ng] = g.sstart[k] + j;
        ++ng;
      }
    StageGemv a = stage_base(h);
    a.n_groups = ng;
    a.gmode = GM_STAGE;
    for (int k = 0; k < ng; ++k) {
      a.layer[k] = glayer[k];
      a.stage[k] = gstage[k];
    }
    // q/k/v + RoPE + KV append
    for (int k = 0; k < ng; ++k) {
      a.W[k] = w.layers[a.layer[k]].w_qkv;
      a.gamma[k] = (const float*)w.layers[a.layer[k]].attn_norm;
    }
    a.N = g.qkv_rows;
    a.K = g.d;
    a.units = g.qkv_rows / 2;
    a.x = h->hslots;
    a.x_stride = g.d;
    a.x_by_slot = 1;
    a.out = h->s_q;
    a.out_stride = qd;
    a.kc = h->kc;
    a.vc = h->vc;
    a.kv_len = h->kv_len;
    launch_stage_w<WT, EPI_QKV>(h, a, ng, ss);
    // attention over each group's own layer cache
    Attn t;
    memset(&t, 0, sizeof(t));
    t.pmode = PM_STAGE;
    for (int k = 0; k < ng; ++k) {
      t.layer[k] = a.layer[k];
      t.stage[k] = a.stage[k];
    }
    t.kc = h->kc;
    t.vc = h->vc;
    t.q = h->s_q;
    t.pacc = h->s_pacc;
    t.pml = h->s_pml;
    t.o = h->s_o;
    t.lane_stride = g.lane_kv;
    t.ctrl = h->ctrl;
    t.g = g;
    // a hybrid target's sub-step may hold softmax and linear layers: each
    // kernel takes its own groups (the layer types are fixed per sub-step);
    // a draft tree's groups hold W nodes, one per workgroup
    bool any_soft = false, any_lin = false;
    for (int k = 0; k < ng; ++k) (layer_is_linear(g, a.layer[k]) ? any_lin : any_soft) = true;
    if (any_soft) attention_any<WT>(t, dim3(g.nsplit, g.Hkv, ng * g.W), 1, ng * g.W, ss);
    if (any_lin) {
      LinAttn la;
      memset(&la, 0, sizeof(la));
      la.mode = LM_STAGE;
      for (int k = 0; k < ng; ++k) {
        la.layer[k] = a.layer[k];
        la.stage[k] = a.stage[k];
      }
      la.kc = h->kc;
      la.vc = h->vc;
      la.q = h->s_q;
      la.ldq = qd;
      la.o = h->s_o;
      la.ldo = qd;
      la.state = h->lin_state;
      la.ctrl = h->ctrl;
      la.g = g;
      if (g.hd == 128)
        hipLaunchKernelGGL((k_linattn<WT, 128>), dim3(g.Hkv, ng), dim3(kWG), 0, ss, la);
      else
        hipLaunchKernelGGL((k_linattn<WT, 64>), dim3(g.Hkv, ng), dim3(kWG), 0, ss, la);
    }
    // output projection + residual
    StageGemv o = stage_base(h);
    o.n_groups = ng;
    o.gmode = GM_STAGE;
    for (int k = 0; k < ng; ++k) {
      o.stage[k] = a.stage[k];
      o.layer[k] = a.layer[k];
      o.W[k] = w.layers[a.layer[k]].w_o;
    }
    o.N = g.d;
    o.K = qd;
    o.units = g.d;
    o.x = h->s_o;
    o.x_stride = qd;
    o.out = h->hslots;
    o.out_stride = g.d;
    o.out_by_slot = 1;
    launch_stage_w<WT, EPI_RESID>(h, o, ng, ss);
    // norm + gate/up + SwiGLU
    StageGemv u = stage_base(h);
    u.n_groups = ng;
    u.gmode = GM_STAGE;
    for (int k = 0; k < ng; ++k) {
      u.stage[k] = a.stage[k];
      u.layer[k] = a.layer[k];
      u.W[k] = w.layers[a.layer[k]].w_gu;
      u.gamma[k] = (const float*)w.layers[a.layer[k]].ffn_norm;
    }
    u.N = 2 * g.F;
    u.K = g.d;
    u.units = g.F;
    u.x = h->hslots;
    u.x_stride = g.d;
    u.x_by_slot = 1;
    u.out = h->s_act;
    u.out_stride = g.F;
    hipEvent_t g0 = nullptr, g1 = nullptr;
    if (timing_gu) {
      g0 = pool_event(h);
      g1 = pool_event(h);
      HIPCHK(h, hipEventRecord(g0, ss));
    }
    launch_stage_w<WT, EPI_SWIGLU>(h, u, ng, ss);
    if (g1) {
      HIPCHK(h, hipEventRecord(g1, ss));
      h->gu_ev.push_back(g0);
      h->gu_ev.push_back(g1);
    }
    // down + residual + anchor taps
    StageGemv dn = stage_base(h);
    dn.n_groups = ng;
    dn.gmode = GM_STAGE;
    for (int k = 0; k < ng; ++k) {
      dn.stage[k] = a.stage[k];
      dn.layer[k] = a.layer[k];
      dn.W[k] = w.layers[a.layer[k]].w_down;
      dn.anchor_idx[k] = g.anchor_of_layer[a.layer[k] + 1];
    }
    dn.N = g.d;
    dn.K = g.F;
    dn.units = g.d;
    dn.x = h->s_act;
    dn.x_stride = g.F;
    dn.out = h->hslots;
    dn.out_stride = g.d;
    dn.out_by_slot = 1;
    dn.anchors = h->anchors;
    launch_stage_w<WT, EPI_RESID>(h, dn, ng, ss);
  }
  // verification head on the exiting token, then verify / rollback
  StageGemv hd = stage_base(h);
  hd.W[0] = w.lm_head;
  hd.gamma[0] = (const float*)w.final_norm;
  hd.N = g.V;
  hd.K = g.d;
  hd.units = g.V;
  hd.n_groups = 1;
  hd.gmode = GM_EXIT;
  hd.x = h->hslots;
  hd.x_stride = g.d;
  hd.x_by_slot = 1;
  hd.out = h->logits;
  hd.parts = h->parts;
  int grid = 0;
  launch_stage<WT, EPI_ARGMAX>(h, hd, 1, ss, &grid);
  if (g.W > 1) {
    TreeVerifyArgs tv;
    memset(&tv, 0, sizeof(tv));
    tv.parts = h->parts;
    tv.nparts = grid;
    tv.tokens = h->tokens;
    tv.kv_len = h->kv_len;
    tv.kc = h->kc;
    tv.vc = h->vc;
    tv.kv_bytes = (int)sizeof(WT);
    tv.ring = h->ring;
    tv.ctrl = h->ctrl;
    tv.g = g;
    hipLaunchKernelGGL(k_tree_verify, dim3(1), dim3(kCtlThreads), 0, ss, tv);
    return hipGetLastError() == hipSuccess ? SPD_OK : SPD_EHIP;
  }
  if (h->bsp) {
    SoftmaxArgs sm;
    memset(&sm, 0, sizeof(sm));
    sm.parts = h->parts;
    sm.nparts = grid;
    sm.logits = h->logits;
    sm.w = h->pw;
    sm.bs = h->bsp;
    sm.exit_only = 1;
    sm.temp = h->cfg.temperature;
    sm.ctrl = h->ctrl;
    sm.g = g;
    const int nb = (g.V + kCdfBlock - 1) / kCdfBlock;
    hipLaunchKernelGGL(k_softmax_blocks, dim3((nb + kWG / kWave - 1) / (kWG / kWave)), dim3(kWG), 0, ss, sm);
  }
  if (h->tkp) {
    TopkArgs tk;
    memset(&tk, 0, sizeof(tk));
    tk.logits = h->logits;
    tk.cand = h->tkp;
    tk.exit_only = 1;
    tk.ctrl = h->ctrl;
    tk.g = g;
    hipLaunchKernelGGL(k_topk_blocks, dim3(topk_groups(g.V)), dim3(kWG), 0, ss, tk);
  }
  VerifyArgs v;
  memset(&v, 0, sizeof(v));
  v.parts = h->parts;
  v.nparts = grid;
  v.bs = h->bsp;
  v.tk = h->tkp;
  v.ntk = h->tkp ? topk_candidates(g.V) : 0;
  v.logits = h->logits;
  v.pw = h->pw;
  v.dring = h->dring;
  v.qring = h->qring;
  v.qz = h->qz;
  v.uni = h->uni;
  v.mode = h->cfg.mode;
  v.temp = h->cfg.temperature;
  v.tokens = h->tokens;
  v.kv_len = h->kv_len;
  v.ring = h->ring;
  v.ctrl = h->ctrl;
  v.g = g;
  hipLaunchKernelGGL(k_verify, dim3(1), dim3(kCtlThreads), 0, ss, v);
  return hipGetLastError() == hipSuccess ? SPD_OK : SPD_EHIP;
}

// Capture each stream's chain once as a HIP graph (the chains read every
// per-cycle value from device memory, so one graph serves every cycle).
template <typename WT>
int capture_graphs(spd_t* h) {
  if (h->graphs_valid) return SPD_OK;
  // cycles already enqueued may still be running the old executables
  HIPCHK(h, hipStreamSynchronize(h->ss));
  HIPCHK(h, hipStreamSynchronize(h->ps));
  if (h->gx_stage) (void)hipGraphExecDestroy(h->gx_stage);
  if (h->gx_pdm) (void)hipGraphExecDestroy(h->gx_pdm);
  h->gx_stage = h->gx_pdm = nullptr;
  hipGraph_t gs = nullptr, gp = nullptr;
  // the captured graphs are released on every path; the executable graphs
  // stay with the handle (spd_destroy or the next capture releases them)
  auto done = [&](int r) {
    if (gp) (void)hipGraphDestroy(gp);
    if (gs) (void)hipGraphDestroy(gs);
    return r;
  };
  hipError_t e;
  if ((e = hipStreamBeginCapture(h->ps, hipStreamCaptureModeThreadLocal)) != hipSuccess) return done(hip_fail(h, e));
  int r = pdm_chain<WT>(h, h->ps);
  if ((e = hipStreamEndCapture(h->ps, &gp)) != hipSuccess) return done(hip_fail(h, e));
  if (r) return done(r);
  if ((e = hipStreamBeginCapture(h->ss, hipStreamCaptureModeThreadLocal)) != hipSuccess) return done(hip_fail(h, e));
  r = stage_chain<WT>(h, h->ss, false);
  if ((e = hipStreamEndCapture(h->ss, &gs)) != hipSuccess) return done(hip_fail(h, e));
  if (r) return done(r);
  if ((e = hipGraphInstantiate(&h->gx_pdm, gp, nullptr, nullptr, 0)) != hipSuccess) return done(hip_fail(h, e));
  if ((e = hipGraphInstantiate(&h->gx_stage, gs, nullptr, nullptr, 0)) != hipSuccess) return done(hip_fail(h, e));
  h->graphs_valid = 1;
  return done(SPD_OK);
}

template <typename WT>
int enqueue_cycle(spd_t* h) {
  const Geo& g = h->g;
  hipStream_t ss = h->ss, ps = h->ps;
  const bool graph = h->launch_mode == 1;
  // serialized: the draft module is enqueued on the stage stream ahead of the
  // stage step (it reads only pre-step state, so the result is unchanged).
  // Post-step schedule: it reads the stage step's output and the verification result, so
  // it follows them on the stage stream.
  // One stage (n = 1): the token entering a cycle also exits in it and
  // verifies the draft made in the same cycle, so the draft chain goes
  // first on the stage stream as well.
  const bool post = g.post != 0;
  if (h->serialized || post || g.n == 1) ps = ss;
  hipEvent_t e_start = nullptr, e_stage = nullptr, e_pdm_t = nullptr;
  if (h->timing) {
    e_start = pool_event(h);
    e_stage = pool_event(h);
    e_pdm_t = pool_event(h);
    if (!e_start || !e_stage || !e_pdm_t) return SPD_EHIP;
  }
  // join: the previous cycle's draft is done
  HIPCHK(h, hipStreamWaitEvent(ss, h->ev_pdm, 0));
  if (e_start) HIPCHK(h, hipEventRecord(e_start, ss));
  if (g.W > 1) {
    hipLaunchKernelGGL((k_tree_entry<WT>), dim3(1), dim3(kWG), 0, ss, h->ctrl, g, h->tokens, (const WT*)h->w.embed,
                       h->hslots, h->anchors, h->ring, h->lay.log_cap);
    hipLaunchKernelGGL((k_tree_lane_copy<WT>), dim3(g.L, g.W), dim3(kWG), 0, ss, (const Ctrl*)h->ctrl, g, (WT*)h->kc,
                       (WT*)h->vc);
  } else {
    hipLaunchKernelGGL((k_entry<WT>), dim3(1), dim3(kWG), 0, ss, h->ctrl, g, h->tokens, (const WT*)h->w.embed,
                       h->hslots, h->anchors, h->ring, h->lay.log_cap);
  }
  // fork
  if (ps != ss) {
    HIPCHK(h, hipEventRecord(h->ev_entry, ss));
    HIPCHK(h, hipStreamWaitEvent(ps, h->ev_entry, 0));
  }
  auto draft = [&]() -> int {
    int r = graph ? (hipGraphLaunch(h->gx_pdm, ps) == hipSuccess ? SPD_OK : SPD_EHIP) : pdm_chain<WT>(h, ps);
    if (r) return r;
    if (e_pdm_t) HIPCHK(h, hipEventRecord(e_pdm_t, ps));
    HIPCHK(h, hipEventRecord(h->ev_pdm, ps));
    return SPD_OK;
  };
  auto stage = [&]() -> int {
    return graph ? (hipGraphLaunch(h->gx_stage, ss) == hipSuccess ? SPD_OK : SPD_EHIP)
                 : stage_chain<WT>(h, ss, h->timing != 0);
  };
  int r;
  if (post) {
    if ((r = stage())) return r;
    if (e_stage) HIPCHK(h, hipEventRecord(e_stage, ss));
    if ((r = draft())) return r;
  } else {
    if ((r = draft())) return r;
    if ((r = stage())) return r;
    if (e_stage) HIPCHK(h, hipEventRecord(e_stage, ss));
  }
  if (e_stage) {
    h->cyc_ev.push_back(e_start);
    h->cyc_ev.push_back(e_stage);
    h->cyc_ev.push_back(e_pdm_t);
  }
  HIPCHK(h, hipGetLastError());
  h->cyc += 1;
  return SPD_OK;
}

template <typename WT>
int do_prefill(spd_t* h, int P) {
  const Geo& g = h->g;
  const spd_weights& w = h->w;
  hipStream_t s = h->ss;
  h->lin_keep_from = P - g.nslots;
  for (int s0 = 0; s0 < P; s0 += kRowsMR) {
    const int M = std::min(kRowsMR, P - s0);
    hipLaunchKernelGGL((k_embed_rows<WT>), dim3(M), dim3(kWG), 0, s, h->tokens, s0, (const WT*)w.embed, g.d, h->Xt,
                       h->taps, g.m, h->ssq_t);
    for (int l = 0; l < g.L; ++l)
      layer_rows_any<WT>(h, true, w.layers[l], h->kc, h->vc, l, h->Xt, h->ssq_t, M, s0, 0, h->kv_len, h->taps,
                         g.anchor_of_layer[l + 1], s, layer_is_linear(g, l));
    // draft module prefill on the full-depth features of the chunk
    if (sizeof(WT) == 2) {
      MfmaArgs a = mfma_base(h);
      a.M_arg = M;
      a.pos0_arg = s0;
      a.W[0] = (const uint16_t*)w.fc[g.m - 1];
      a.K[0] = g.m * g.d;
      a.N = g.d;
      a.x = h->taps;
      a.ldx = g.m * g.d;
      a.out = h->Xp;
      a.ldo = g.d;
      a.ssq_out = h->ssq_p;
      launch_mfma<EPI_STORE>(h, a, 1, M, s);
    } else {
      RowsGemv a = rows_base(h);
      a.M_arg = M;
      a.pos0_arg = s0;
      a.W[0] = w.fc[g.m - 1];
      a.Kg[0] = g.m * g.d;
      a.N = g.d;
      a.units = g.d;
      a.x = h->taps;
      a.ldx = g.m * g.d;
      a.out = h->Xp;
      a.ldo = g.d;
      launch_rows<WT, EPI_STORE>(h, a, M, s);
    }
    for (int l = 0; l < g.Ls; ++l)
      layer_rows_any<WT>(h, true, w.pdm[l], h->pkc, h->pvc, l, h->Xp, h->ssq_p, M, s0, 0, nullptr, nullptr, -1, s);
    if (s0 + M == P) {
      const int grid = head_fixed<WT>(h, h->Xt + (size_t)(M - 1) * g.d, w.lm_head, w.final_norm, h->logits,
                                      h->parts, s);
      hipLaunchKernelGGL(k_pick_token, dim3(1), dim3(kCtlThreads), 0, s, h->parts, grid, h->logits, h->pw, g.V,
                         h->cfg.mode, h->cfg.temperature, g.topk, h->uni, h->tokens, P, h->ctrl,
                         &h->ctrl->flags);
    }
  }
  // linear-attention states after the prompt: a rollback to this length
  // (after an autoregressive run past the ring) restores them from here
  if (g.attn_period > 0) {
    const size_t one = (size_t)g.Hkv * ((size_t)g.hd * g.hd + g.hd);
    for (int l = 0; l < g.L; ++l)
      if (layer_is_linear(g, l))
        HIPCHK(h, hipMemcpyAsync(h->lin_ckpt + (size_t)l * one,
                                 h->lin_state + lin_state_index(g, l, (P - 1) % g.nslots, 0), one * sizeof(float),
                                 hipMemcpyDeviceToDevice, s));
    h->ckpt_len = P;
  }
  HIPCHK(h, hipGetLastError());
  return SPD_OK;
}

template <typename WT>
int do_ar(spd_t* h, int s0, int n) {
  const Geo& g = h->g;
  const spd_weights& w = h->w;
  hipStream_t s = h->ss;
  for (int i = 0; i < n; ++i) {
    const int pos = s0 + i;
    hipLaunchKernelGGL((k_embed_rows<WT>), dim3(1), dim3(kWG), 0, s, h->tokens, pos, (const WT*)w.embed, g.d,
                       h->Xt, (float*)nullptr, g.m, (float*)nullptr);
    h->lin_keep_from = pos;
    for (int l = 0; l < g.L; ++l)
      rows_layer<WT>(h, w.layers[l], h->kc, h->vc, l, h->Xt, 1, pos, 0, h->kv_len, nullptr, -1, s,
                     layer_is_linear(g, l));
    const int grid = head_fixed<WT>(h, h->Xt, w.lm_head, w.final_norm, h->logits, h->parts, s);
    hipLaunchKernelGGL(k_pick_token, dim3(1), dim3(kCtlThreads), 0, s, h->parts, grid, h->logits, h->pw, g.V,
                       SPD_MODE_GREEDY, 1.0f, 0, h->uni, h->tokens, pos + 1, (Ctrl*)nullptr, &h->ctrl->flags);
  }
  HIPCHK(h, hipGetLastError());
  return SPD_OK;
}

int read_ctrl(spd_t* h, Ctrl* c) {
  HIPCHK(h, hipStreamSynchronize(h->ss));
  HIPCHK(h, hipStreamSynchronize(h->ps));
  HIPCHK(h, hipMemcpy(c, h->ctrl, sizeof(Ctrl), hipMemcpyDeviceToHost));
  return SPD_OK;
}

int write_ctrl(spd_t* h, const Ctrl* c) {
  HIPCHK(h, hipMemcpy(h->ctrl, c, sizeof(Ctrl), hipMemcpyHostToDevice));
  return SPD_OK;
}

// Every KV lane of a draft tree takes lane 0's contents: after prefill, a
// host rollback or an autoregressive run, the positions before the seed are
// common to every branch (and lane 0, which those passes write, holds them).
int sync_lanes(spd_t* h) {
  const Geo& g = h->g;
  if (g.W <= 1) return SPD_OK;
  const size_t es = h->cfg.dtype == SPD_DTYPE_BF16 ? 2 : 4;
  for (int ln = 1; ln < g.W; ++ln) {
    HIPCHK(h, hipMemcpyAsync((char*)h->kc + ln * g.lane_kv * es, h->kc, g.lane_kv * es, hipMemcpyDeviceToDevice,
                             h->ss));
    HIPCHK(h, hipMemcpyAsync((char*)h->vc + ln * g.lane_kv * es, h->vc, g.lane_kv * es, hipMemcpyDeviceToDevice,
                             h->ss));
    HIPCHK(h, hipMemcpyAsync((char*)h->pkc + ln * g.lane_pkv * es, h->pkc, g.lane_pkv * es,
                             hipMemcpyDeviceToDevice, h->ss));
    HIPCHK(h, hipMemcpyAsync((char*)h->pvc + ln * g.lane_pkv * es, h->pvc, g.lane_pkv * es,
                             hipMemcpyDeviceToDevice, h->ss));
  }
  HIPCHK(h, hipStreamSynchronize(h->ss));
  return SPD_OK;
}

// An empty draft tree (nothing in flight, no candidates, no exited node).
int reset_tree(spd_t* h) {
  Tree t0;
  memset(&t0, 0, sizeof(t0));
  t0.last_exit = -1;
  t0.pend_slot = -1;
  HIPCHK(h, hipMemcpy(tree_of(h->ctrl), &t0, sizeof(t0), hipMemcpyHostToDevice));
  return SPD_OK;
}

int set_kv_len(spd_t* h, int len) {
  std::vector<int32_t> v(SPD_MAX_LAYERS, len);
  HIPCHK(h, hipMemcpy(h->kv_len, v.data(), sizeof(int32_t) * SPD_MAX_LAYERS, hipMemcpyHostToDevice));
  return SPD_OK;
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

int spd_workspace_bytes(const spd_config* cfg, size_t* bytes) {
  if (!valid_config(cfg) || !bytes) return SPD_EINVAL;
  *bytes = make_layout(cfg).total;
  return SPD_OK;
}

}  // extern "C"

namespace {

// Validation shared by the init entry points (configuration, weights, streams).
bool valid_init_args(const spd_config* cfg, const spd_weights* w, void* stage_stream, void* pdm_stream) {
  if (!valid_config(cfg) || !w) return false;
  if (stage_stream == pdm_stream) return false;
  if (!w->embed || !w->final_norm || !w->lm_head || !w->pdm_final_norm || !w->pdm_lm_head) return false;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const spd_layer_weights& x = w->layers[l];
    if (!x.attn_norm || !x.w_qkv || !x.w_o || !x.ffn_norm || !x.w_gu || !x.w_down) return false;
  }
  for (int l = 0; l < cfg->pdm_layers; ++l) {
    const spd_layer_weights& x = w->pdm[l];
    if (!x.attn_norm || !x.w_qkv || !x.w_o || !x.ffn_norm || !x.w_gu || !x.w_down) return false;
  }
  for (int f = 0; f < cfg->n_anchors; ++f)
    if (!w->fc[f]) return false;
  return true;
}

// The handle over persistent state at `ws` (L.state_total bytes) and scratch
// at `sc` (L.scratch_total bytes).  Allocates no device memory.
int init_handle(const spd_config* cfg, const spd_weights* w, char* ws, char* sc, const Layout& L,
                void* stage_stream, void* pdm_stream, spd_t** out) {
  spd_t* h = new (std::nothrow) spd_handle();
  if (!h) return SPD_EINVAL;
  h->cfg = *cfg;
  h->w = *w;
  h->lay = L;
  h->ss = (hipStream_t)stage_stream;
  h->ps = (hipStream_t)pdm_stream;
  Geo& g = h->g;
  memset(&g, 0, sizeof(g));
  g.L = cfg->n_layers;
  g.d = cfg->d_model;
  g.Hq = cfg->n_heads;
  g.Hkv = cfg->n_kv_heads;
  g.hd = cfg->head_dim;
  g.F = cfg->d_ffn;
  g.V = cfg->vocab;
  g.n = cfg->n_stages;
  g.Ls = cfg->pdm_layers;
  g.m = cfg->n_anchors;
  // stage k runs layers sstart[k] .. sstart[k+1]-1; per = the longest stage
  // (the number of sub-steps of a stage step)
  g.per = 0;
  for (int k = 0, acc = 0; k < g.n; ++k) {
    const int sz = has_split(cfg) ? cfg->stage_layers[k] : g.L / g.n;
    g.sstart[k] = acc;
    acc += sz;
    g.per = std::max(g.per, sz);
  }
  g.sstart[g.n] = g.L;
  g.nslots = g.n + 1;
  g.ctx_cap = L.ctx_cap;
  g.nsplit = L.nsplit;
  g.qkv_rows = (g.Hq + 2 * g.Hkv) * g.hd;
  g.max_new = cfg->max_new;
  g.max_ctx = cfg->max_ctx;
  g.post = cfg->schedule == SPD_SCHED_POST ? 1 : 0;
  g.topk = cfg->mode == SPD_MODE_SAMPLE ? cfg->top_k : 0;
  g.attn_period = cfg->attn_period;
  g.eps = cfg->rms_eps;
  g.W = width_of(cfg);
  g.lane_kv = (long long)g.Hkv * g.hd * L.ctx_cap * g.L;
  g.lane_pkv = (long long)g.Hkv * g.hd * L.ctx_cap * g.Ls;
  for (int b = 0; b <= SPD_MAX_LAYERS; ++b) g.anchor_of_layer[b] = -1;
  for (int i = 0; i < g.m; ++i) g.anchor_of_layer[cfg->anchors[i]] = i;
  g.anchor_of_layer[0] = -1;  // anchor 0 (embedding) is written at entry
  // f(k) = max{i : b_i <= lmax(k)}, lmax(k) = layers of the first k stages
  // (min(L, k L/n) under the uniform split)
  for (int k = 0; k <= g.n; ++k) {
    const int lmax = g.sstart[k];
    int f = 0;
    for (int i = 0; i < g.m; ++i)
      if (cfg->anchors[i] <= lmax) f = i;
    g.fpat[k] = f;
  }
  h->ws = ws;
  h->ctrl = (Ctrl*)(ws + L.ctrl);
  h->kv_len = (int32_t*)(ws + L.kv_len);
  h->tokens = (int32_t*)(ws + L.tokens);
  h->dring = (int32_t*)(ws + L.dring);
  h->qring = (float*)(ws + L.qring);
  h->qz = (double*)(ws + L.qz);
  h->kc = ws + L.kc;
  h->vc = ws + L.vc;
  h->pkc = ws + L.pkc;
  h->pvc = ws + L.pvc;
  h->rcos = (float*)(ws + L.rcos);
  h->rsin = (float*)(ws + L.rsin);
  h->hslots = (float*)(ws + L.hslots);
  h->anchors = (float*)(ws + L.anchors);
  h->s_q = (float*)(sc + L.s_q);
  h->s_pacc = (float*)(sc + L.s_pacc);
  h->s_pml = (float*)(sc + L.s_pml);
  h->s_o = (float*)(sc + L.s_o);
  h->s_act = (float*)(sc + L.s_act);
  h->Xt = (float*)(sc + L.Xt);
  h->Xp = (float*)(sc + L.Xp);
  h->r_q = (float*)(sc + L.r_q);
  h->r_pacc = (float*)(sc + L.r_pacc);
  h->r_pml = (float*)(sc + L.r_pml);
  h->r_o = (float*)(sc + L.r_o);
  h->r_act = (float*)(sc + L.r_act);
  h->taps = (float*)(sc + L.taps);
  h->logits = (float*)(sc + L.logits);
  h->plogits = (float*)(sc + L.plogits);
  h->pw = (float*)(sc + L.pw);
  h->parts = (ArgPair*)(sc + L.parts);
  h->pparts = (ArgPair*)(sc + L.pparts);
  h->ring = (spd_cycle_rec*)(ws + L.ring);
  h->ssq_t = (float*)(sc + L.ssq_t);
  h->ssq_p = (float*)(sc + L.ssq_p);
  h->mpart = (float*)(sc + L.mpart);
  if (cfg->dtype == SPD_DTYPE_BF16) {
    h->wtile = (uint16_t*)(ws + L.wtile);
    h->xs_h = (uint16_t*)(sc + L.xs_h);
    h->xs_l = (uint16_t*)(sc + L.xs_l);
    h->as_h = (uint16_t*)(sc + L.as_h);
    h->as_l = (uint16_t*)(sc + L.as_l);
    h->os_h = (uint16_t*)(sc + L.os_h);
    h->os_l = (uint16_t*)(sc + L.os_l);
  }
  if (cfg->mode == SPD_MODE_SAMPLE && !cfg->top_k) {
    h->bsq = (double*)(sc + L.bsq);
    h->bsp = (double*)(sc + L.bsp);
  }
  if (cfg->mode == SPD_MODE_SAMPLE && cfg->top_k) {
    h->tkq = (unsigned long long*)(sc + L.tkq);
    h->tkp = (unsigned long long*)(sc + L.tkp);
  }
  if (g.W > 1) {
    h->zpart = (double*)(sc + L.zpart);
    h->tpart = (ArgPair*)(sc + L.tpart);
  }
  if (cfg->attn_period > 0) {
    h->lin_state = (float*)(ws + L.lin_state);
    h->lin_ckpt = (float*)(ws + L.lin_ckpt);
  }

  auto fail = [&](hipError_t e) {
    h->hip_err = (int)e;
    if (h->ev_entry) (void)hipEventDestroy(h->ev_entry);
    if (h->ev_pdm) (void)hipEventDestroy(h->ev_pdm);
    delete h;
    return SPD_EHIP;
  };
  hipError_t e;
  if ((e = hipEventCreateWithFlags(&h->ev_entry, hipEventDisableTiming)) != hipSuccess) return fail(e);
  if ((e = hipEventCreateWithFlags(&h->ev_pdm, hipEventDisableTiming)) != hipSuccess) return fail(e);
  // zero the control block and small state; RoPE table
  Ctrl c0;
  memset(&c0, 0, sizeof(c0));
  c0.r_exit = -1;
  c0.done = 1;
  if ((e = hipMemcpy(h->ctrl, &c0, sizeof(c0), hipMemcpyHostToDevice)) != hipSuccess) return fail(e);
  {
    Tree t0;
    memset(&t0, 0, sizeof(t0));
    t0.last_exit = -1;
    t0.pend_slot = -1;
    if ((e = hipMemcpy(tree_of(h->ctrl), &t0, sizeof(t0), hipMemcpyHostToDevice)) != hipSuccess) return fail(e);
  }
  std::vector<int32_t> zl(SPD_MAX_LAYERS, 0);
  if ((e = hipMemcpy(h->kv_len, zl.data(), sizeof(int32_t) * SPD_MAX_LAYERS, hipMemcpyHostToDevice)) != hipSuccess)
    return fail(e);
  // scratch (it may hold another handle's values) and the linear-attention
  // state are cleared once, so that nothing reads uninitialised memory
  if ((e = hipMemsetAsync(sc, 0, L.scratch_total, h->ss)) != hipSuccess) return fail(e);
  if (L.lin_ckpt > L.lin_state &&
      (e = hipMemsetAsync(ws + L.lin_state, 0, L.state_total - L.lin_state, h->ss)) != hipSuccess)
    return fail(e);
  if ((e = attn_lds_limits()) != hipSuccess) return fail(e);
  hipLaunchKernelGGL(k_rope_table, dim3(512), dim3(256), 0, h->ss, h->rcos, h->rsin, L.ctx_cap, g.hd,
                     (double)cfg->rope_base);
  if (h->wtile) tile_pdm_weights(h, h->ss);
  if ((e = hipGetLastError()) != hipSuccess) return fail(e);
  if ((e = hipEventRecord(h->ev_pdm, h->ps)) != hipSuccess) return fail(e);
  if ((e = hipStreamSynchronize(h->ss)) != hipSuccess) return fail(e);
  *out = h;
  return SPD_OK;
}

// The static scratch array of the allocation-free init: one per GPU the
// library runs on, for the life of the process.  Host code never passes its
// name to a kernel or a copy: it uses the device address looked up once per
// device (scratch_ptr).
constexpr size_t kStaticScratchBytes = (size_t)SPD_STATIC_SCRATCH_MB << 20;
__device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's static scratch, looked up with that
// device current on its first use.
hipError_t scratch_ptr(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = (char*)p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int spd_init(const spd_config* cfg, const spd_weights* w, void* workspace, size_t ws_bytes, void* stage_stream,
             void* pdm_stream, spd_t** out) {
  if (!out) return SPD_EINVAL;
  *out = nullptr;
  if (!workspace || !valid_init_args(cfg, w, stage_stream, pdm_stream)) return SPD_EINVAL;
  if (((uintptr_t)workspace) % kAlign) return SPD_EINVAL;
  const Layout L = make_layout(cfg);
  if (ws_bytes < L.total) return SPD_EINVAL;
  char* ws = (char*)workspace;
  return init_handle(cfg, w, ws, ws + L.state_total, L, stage_stream, pdm_stream, out);
}

int spd_init_static_scratch(const spd_config* cfg, const spd_weights* w, void* state, size_t* state_bytes,
                            void* stage_stream, void* pdm_stream, spd_t** out) {
  if (out) *out = nullptr;
  if (!state_bytes || !valid_config(cfg)) return SPD_EINVAL;
  const Layout L = make_layout(cfg);
  if (L.scratch_total > kStaticScratchBytes) return SPD_ESCRATCH;
  if (!state) {  // size query
    *state_bytes = L.state_total;
    return SPD_OK;
  }
  if (!out || !valid_init_args(cfg, w, stage_stream, pdm_stream)) return SPD_EINVAL;
  if (((uintptr_t)state) % kAlign || *state_bytes < L.state_total) return SPD_EINVAL;
  char* sc = nullptr;
  const hipError_t e = scratch_ptr(&sc);
  if (e != hipSuccess) return SPD_EHIP;
  return init_handle(cfg, w, (char*)state, sc, L, stage_stream, pdm_stream, out);
}

int spd_set_draft_policy(spd_t* h, int32_t policy, float p_accept, const int32_t* ref_tokens_dev, int32_t ref_len) {
  if (!h) return SPD_EINVAL;
  h->graphs_valid = 0;
  if (policy == SPD_DRAFT_NATURAL) {
    h->policy = policy;
    return SPD_OK;
  }
  // a draft tree's forced policy is spd_set_tree_policy
  if (policy != SPD_DRAFT_FORCED || h->cfg.mode != SPD_MODE_GREEDY || h->g.W > 1) return SPD_EINVAL;
  if (!ref_tokens_dev || ref_len < 0 || !(p_accept >= 0.f && p_accept <= 1.f) || !h->uni) return SPD_EINVAL;
  h->policy = policy;
  h->p_accept = p_accept;
  h->ref = ref_tokens_dev;
  h->ref_len = ref_len;
  return SPD_OK;
}

int spd_set_tree_policy(spd_t* h, float p_first, float p_tree, const int32_t* ref_tokens_dev, int32_t ref_len) {
  if (!h || h->g.W < 2 || !ref_tokens_dev || ref_len < 0 || !h->uni) return SPD_EINVAL;
  if (!(p_first >= 0.f && p_first <= p_tree && p_tree <= 1.f)) return SPD_EINVAL;
  h->graphs_valid = 0;
  h->policy = SPD_DRAFT_FORCED;
  h->p_first = p_first;
  h->p_tree = p_tree;
  h->ref = ref_tokens_dev;
  h->ref_len = ref_len;
  return SPD_OK;
}

int spd_set_launch_mode(spd_t* h, int32_t mode) {
  if (!h) return SPD_EINVAL;
  const int base = mode & ~SPD_LAUNCH_SERIALIZED;
  if (base != SPD_LAUNCH_EAGER && base != SPD_LAUNCH_GRAPH) return SPD_EINVAL;
  HIPCHK(h, hipStreamSynchronize(h->ss));
  HIPCHK(h, hipStreamSynchronize(h->ps));
  h->launch_mode = base;
  h->serialized = (mode & SPD_LAUNCH_SERIALIZED) ? 1 : 0;
  return SPD_OK;
}

int spd_set_uniforms(spd_t* h, const float* uniforms_dev, int32_t n_positions) {
  if (!h || !uniforms_dev || n_positions < h->cfg.max_ctx) return SPD_EINVAL;
  h->uni = uniforms_dev;
  h->uni_len = n_positions;
  h->graphs_valid = 0;
  return SPD_OK;
}

int spd_prefill(spd_t* h, const int32_t* prompt_host, int32_t len, int32_t* first_token) {
  if (!h || !prompt_host || len < 1) return SPD_EINVAL;
  for (int i = 0; i < len; ++i)
    if (prompt_host[i] < 0 || prompt_host[i] >= h->g.V) return SPD_EINVAL;
  if ((long long)len + h->cfg.max_new + h->cfg.n_stages > h->cfg.max_ctx) return SPD_ECTX;
  if (h->cfg.mode == SPD_MODE_SAMPLE && !h->uni) return SPD_ESTATE;
  HIPCHK(h, hipStreamSynchronize(h->ss));
  HIPCHK(h, hipStreamSynchronize(h->ps));
  HIPCHK(h, hipMemcpy(h->tokens, prompt_host, sizeof(int32_t) * len, hipMemcpyHostToDevice));
  int r = set_kv_len(h, 0);
  if (r) return r;
  Ctrl c;
  memset(&c, 0, sizeof(c));
  c.t = len - 1;
  c.a = 0;
  c.C = len;
  c.emitted = 1;
  c.done = (1 >= h->cfg.max_new);
  c.active = 0;
  c.reseed = 1;
  c.seed_pos = len;
  c.pend_next = 0;
  c.r_exit = -1;
  c.r_accept = -1;
  c.launches = (int32_t)(h->cyc % 0x40000000);
  if ((r = write_ctrl(h, &c))) return r;
  if ((r = reset_tree(h))) return r;
  r = h->cfg.dtype == SPD_DTYPE_BF16 ? do_prefill<uint16_t>(h, len) : do_prefill<float>(h, len);
  if (r) return r;
  HIPCHK(h, hipStreamSynchronize(h->ss));
  if ((r = sync_lanes(h))) return r;
  int32_t first = 0;
  HIPCHK(h, hipMemcpy(&first, h->tokens + len, sizeof(int32_t), hipMemcpyDeviceToHost));
  Ctrl cc;
  if ((r = read_ctrl(h, &cc))) return r;
  if (cc.flags) return SPD_EDEVICE;
  if (first_token) *first_token = first;
  h->prefilled = 1;
  h->P = len;
  h->needs_rollback = 0;
  return SPD_OK;
}

int spd_cycle(spd_t* h, int32_t n_cycles, spd_cycle_rec* log_host) {
  if (!h || n_cycles < 0) return SPD_EINVAL;
  if (!h->prefilled || h->needs_rollback) return SPD_ESTATE;
  if ((h->policy == SPD_DRAFT_FORCED || h->cfg.mode == SPD_MODE_SAMPLE) && !h->uni) return SPD_ESTATE;
  if (log_host && n_cycles > h->lay.log_cap) return SPD_EINVAL;
  const long long c0 = h->cyc;
  if (h->launch_mode == 1 && n_cycles > 0) {
    const int r = h->cfg.dtype == SPD_DTYPE_BF16 ? capture_graphs<uint16_t>(h) : capture_graphs<float>(h);
    if (r) return r;
  }
  for (int i = 0; i < n_cycles; ++i) {
    const int r = h->cfg.dtype == SPD_DTYPE_BF16 ? enqueue_cycle<uint16_t>(h) : enqueue_cycle<float>(h);
    if (r) return r;
  }
  if (log_host && n_cycles > 0) {
    HIPCHK(h, hipStreamWaitEvent(h->ss, h->ev_pdm, 0));
    const int cap = h->lay.log_cap;
    long long done = 0;
    while (done < n_cycles) {
      const int slot = (int)((c0 + done) % cap);
      const long long cnt = std::min<long long>(n_cycles - done, cap - slot);
      HIPCHK(h, hipMemcpyAsync(log_host + done, h->ring + slot, sizeof(spd_cycle_rec) * cnt,
                               hipMemcpyDeviceToHost, h->ss));
      done += cnt;
    }
  }
  return SPD_OK;
}

int spd_rollback(spd_t* h, int32_t keep_len, int32_t reseed_token) {
  if (!h) return SPD_EINVAL;
  if (!h->prefilled) return SPD_ESTATE;
  if (reseed_token < 0 || reseed_token >= h->g.V) return SPD_EINVAL;
  Ctrl c;
  int r = read_ctrl(h, &c);
  if (r) return r;
  // leading positions whose KV is complete in every layer: up to the last
  // verified exit (cycles), or everything the AR decoder processed
  const int complete = h->needs_rollback ? h->ar_complete : h->P + c.emitted - 1;
  if (keep_len < 1 || keep_len > complete || keep_len + 1 >= h->g.ctx_cap) return SPD_ESTATE;
  int C = std::min(c.C, keep_len);
  int pend = 0;
  if (C == keep_len - 1) {
    // the last verified position may stay uncommitted: its anchors are intact
    if (!(c.C == keep_len - 1 && c.pend_next == 1 && !h->needs_rollback)) return SPD_ESTATE;
    pend = 1;
  } else if (C != keep_len) {
    return SPD_ESTATE;
  }
  // hybrid target: the linear-attention state after keep_len - 1 must still
  // be in its ring slot, or be the one kept at the end of prefill
  const bool restore = h->g.attn_period > 0 && keep_len == h->ckpt_len;
  if (h->g.attn_period > 0 && !restore) {
    const int newest = std::max(h->lin_newest, c.t);
    if (keep_len - 1 > newest || newest - (keep_len - 1) >= h->g.nslots) return SPD_ESTATE;
  }
  if (keep_len < h->P) h->P = keep_len;
  if (restore) {
    const Geo& g = h->g;
    const size_t one = (size_t)g.Hkv * ((size_t)g.hd * g.hd + g.hd);
    for (int l = 0; l < g.L; ++l)
      if (layer_is_linear(g, l))
        HIPCHK(h, hipMemcpy(h->lin_state + lin_state_index(g, l, (keep_len - 1) % g.nslots, 0),
                            h->lin_ckpt + (size_t)l * one, one * sizeof(float), hipMemcpyDeviceToDevice));
  }
  if (h->g.attn_period > 0) h->lin_newest = keep_len - 1;
  Ctrl n;
  memset(&n, 0, sizeof(n));
  n.t = keep_len - 1;
  n.C = C;
  n.emitted = keep_len - h->P + 1;
  n.done = n.emitted >= h->cfg.max_new;
  n.cycle = c.cycle;
  n.reseed = 1;
  n.seed_tok = reseed_token;
  n.seed_pos = keep_len;
  n.pend_next = pend;
  n.r_exit = -1;
  n.r_accept = -1;
  n.flags = c.flags;
  n.launches = c.launches;
  if ((r = set_kv_len(h, keep_len))) return r;
  HIPCHK(h, hipMemcpy(h->tokens + keep_len, &reseed_token, sizeof(int32_t), hipMemcpyHostToDevice));
  if ((r = write_ctrl(h, &n))) return r;
  if ((r = reset_tree(h))) return r;
  if ((r = sync_lanes(h))) return r;
  h->needs_rollback = 0;
  return SPD_OK;
}

int spd_generate_ar(spd_t* h, int32_t n_tokens, int32_t* tokens_host) {
  if (!h || n_tokens < 0) return SPD_EINVAL;
  if (!h->prefilled || h->needs_rollback) return SPD_ESTATE;
  Ctrl c;
  int r = read_ctrl(h, &c);
  if (r) return r;
  if (!c.reseed) return SPD_ESTATE;  // needs an empty pipeline (after prefill, rollback or a rejection)
  const int s0 = c.seed_pos;
  if (s0 + n_tokens + 1 >= h->g.ctx_cap) return SPD_ECTX;
  r = h->cfg.dtype == SPD_DTYPE_BF16 ? do_ar<uint16_t>(h, s0, n_tokens) : do_ar<float>(h, s0, n_tokens);
  if (r) return r;
  HIPCHK(h, hipStreamSynchronize(h->ss));
  if (tokens_host && n_tokens)
    HIPCHK(h, hipMemcpy(tokens_host, h->tokens + s0 + 1, sizeof(int32_t) * n_tokens, hipMemcpyDeviceToHost));
  if ((r = read_ctrl(h, &c))) return r;
  h->needs_rollback = 1;
  h->ar_complete = s0 + n_tokens;
  if (c.flags) return SPD_EDEVICE;
  return SPD_OK;
}

int spd_sync(spd_t* h, spd_status* st) {
  if (!h) return SPD_EINVAL;
  Ctrl c;
  const int r = read_ctrl(h, &c);
  if (r) return r;
  if (st) {
    st->cycles = c.cycle;
    st->emitted = c.emitted;
    st->done = c.done;
    st->t = c.t;
    st->occupancy = c.a;
    st->pdm_len = c.C;
    st->flags = c.flags;
    st->hip_error = h->hip_err;
  }
  return c.flags ? SPD_EDEVICE : SPD_OK;
}

int spd_read_tokens(spd_t* h, int32_t first, int32_t count, int32_t* out_host) {
  if (!h || !out_host || first < 0 || count < 0 || (long long)first + count > h->g.ctx_cap) return SPD_EINVAL;
  HIPCHK(h, hipStreamSynchronize(h->ss));
  HIPCHK(h, hipStreamSynchronize(h->ps));
  if (count) HIPCHK(h, hipMemcpy(out_host, h->tokens + first, sizeof(int32_t) * count, hipMemcpyDeviceToHost));
  return SPD_OK;
}

int spd_debug_read(spd_t* h, int32_t what, int32_t index, void* out_host, size_t bytes) {
  if (!h || !out_host) return SPD_EINVAL;
  HIPCHK(h, hipStreamSynchronize(h->ss));
  HIPCHK(h, hipStreamSynchronize(h->ps));
  const Geo& g = h->g;
  const size_t es = h->cfg.dtype == SPD_DTYPE_BF16 ? 2 : 4;
  if (what == SPD_DBG_ANCHORS || what == SPD_DBG_HIDDEN) {
    if (index < 0) return SPD_EINVAL;
    const int slot = index % g.nslots;
    const size_t n = (what == SPD_DBG_ANCHORS) ? (size_t)g.m * g.d : (size_t)g.d;
    if (bytes != n * sizeof(float)) return SPD_EINVAL;
    const float* src = (what == SPD_DBG_ANCHORS) ? h->anchors + (size_t)slot * g.m * g.d : h->hslots + (size_t)slot * g.d;
    HIPCHK(h, hipMemcpy(out_host, src, bytes, hipMemcpyDeviceToHost));
    return SPD_OK;
  }
  if (what == SPD_DBG_LOGITS || what == SPD_DBG_PDM_LOGITS) {
    if (bytes != sizeof(float) * g.V) return SPD_EINVAL;
    HIPCHK(h, hipMemcpy(out_host, what == SPD_DBG_LOGITS ? h->logits : h->plogits, bytes, hipMemcpyDeviceToHost));
    return SPD_OK;
  }
  if (what == SPD_DBG_KV_K || what == SPD_DBG_KV_V) {
    if (index < 0 || index >= g.L) return SPD_EINVAL;
    const int mc = h->cfg.max_ctx;
    if (bytes != (size_t)mc * g.Hkv * g.hd * es) return SPD_EINVAL;
    const size_t blk = (size_t)g.Hkv * g.hd * g.ctx_cap * es;
    std::vector<char> tmp(blk);
    const char* base = (const char*)(what == SPD_DBG_KV_K ? h->kc : h->vc) + blk * index;
    HIPCHK(h, hipMemcpy(tmp.data(), base, blk, hipMemcpyDeviceToHost));
    char* out = (char*)out_host;
    for (int p = 0; p < mc; ++p)
      for (int kvh = 0; kvh < g.Hkv; ++kvh)
        for (int dim = 0; dim < g.hd; ++dim) {
          size_t src;
          if (what == SPD_DBG_KV_K)
            src = (((size_t)kvh * (g.hd / 8) + dim / 8) * g.ctx_cap + p) * 8 + dim % 8;
          else
            src = (((size_t)kvh * (g.ctx_cap / 8) + p / 8) * g.hd + dim) * 8 + p % 8;
          memcpy(out + (((size_t)p * g.Hkv + kvh) * g.hd + dim) * es, tmp.data() + src * es, es);
        }
    return SPD_OK;
  }
  return SPD_EINVAL;
}

int spd_timing_enable(spd_t* h, int32_t enable) {
  if (!h) return SPD_EINVAL;
  HIPCHK(h, hipStreamSynchronize(h->ss));
  HIPCHK(h, hipStreamSynchronize(h->ps));
  h->timing = enable ? 1 : 0;
  h->cyc_ev.clear();
  h->gu_ev.clear();
  h->pool_next = 0;
  return SPD_OK;
}

int spd_timing_read(spd_t* h, int32_t cap, float* cycle_ms, double* gu_ms, int32_t* gu_launches) {
  if (!h) return SPD_EINVAL;
  HIPCHK(h, hipStreamSynchronize(h->ss));
  HIPCHK(h, hipStreamSynchronize(h->ps));
  const int ncyc = (int)(h->cyc_ev.size() / 3);
  for (int i = 0; i < ncyc && cycle_ms && i < cap; ++i) {
    float a = 0.f, b = 0.f;
    HIPCHK(h, hipEventElapsedTime(&a, h->cyc_ev[3 * i], h->cyc_ev[3 * i + 1]));
    HIPCHK(h, hipEventElapsedTime(&b, h->cyc_ev[3 * i], h->cyc_ev[3 * i + 2]));
    cycle_ms[3 * i + 0] = a;
    cycle_ms[3 * i + 1] = b;
    cycle_ms[3 * i + 2] = std::max(a, b);
  }
  double tot = 0.0;
  const int ngu = (int)(h->gu_ev.size() / 2);
  for (int i = 0; i < ngu; ++i) {
    float ms = 0.f;
    HIPCHK(h, hipEventElapsedTime(&ms, h->gu_ev[2 * i], h->gu_ev[2 * i + 1]));
    tot += ms;
  }
  if (gu_ms) *gu_ms = tot;
  if (gu_launches) *gu_launches = ngu;
  // recorded events are consumed: the pool is reused by later cycles
  h->cyc_ev.clear();
  h->gu_ev.clear();
  h->pool_next = 0;
  return ncyc;
}

int spd_destroy(spd_t* h) {
  if (!h) return SPD_EINVAL;
  (void)hipStreamSynchronize(h->ss);
  (void)hipStreamSynchronize(h->ps);
  (void)hipEventDestroy(h->ev_entry);
  (void)hipEventDestroy(h->ev_pdm);
  for (hipEvent_t e : h->pool) (void)hipEventDestroy(e);
  if (h->gx_stage) (void)hipGraphExecDestroy(h->gx_stage);
  if (h->gx_pdm) (void)hipGraphExecDestroy(h->gx_pdm);
  delete h;
  return SPD_OK;
}

const char* spd_strerror(int code) {
  switch (code) {
    case SPD_OK: return "ok";
    case SPD_EINVAL: return "invalid argument or configuration";
    case SPD_ESTATE: return "call not valid in the engine's current state";
    case SPD_ECTX: return "sequence would exceed max_ctx";
    case SPD_EHIP: return "HIP runtime error";
    case SPD_EDEVICE: return "device-side invariant check failed";
    case SPD_ESCRATCH: return "the configuration needs more scratch than the static scratch array holds";
    default: return "unknown error";
  }
}

}  // extern "C"
