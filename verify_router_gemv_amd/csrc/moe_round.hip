// MoE decode/verify round for MI355X (gfx950): the handle, launch plans and the C ABI.
// The kernels are in moe_kernels.h; this file only validates, allocates, launches and captures.
//
// A round is replayed either eagerly (four launches per layer, ingress pointers passed by value)
// or as one captured hipGraph per (T, k) whose kernels read the ingress pointers and the weight
// table from fixed device buffers, so new per-request pointers never force a recapture
// ("How AlphaInfer makes local decoding fast", section 2: per-request data is ingress written
// into fixed buffers and the graph is never rebuilt). Rounds of more than MOE_ROUND_MAX_ROWS rows
// (prefill) run the kernels of moe_prefill.h eagerly, nine per layer.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <vector>

#include "moe_internal.h"
#include "moe_floor.h"
#include "moe_kernels.h"
#include "moe_prefill.h"

using namespace moe;

// ------------------------------------------------------------------------------------------
// Host side: the handle and the C ABI
// ------------------------------------------------------------------------------------------

namespace {

struct Launch {
  KernelFn fn;
  dim3 grid;
  int threads;
  int shmem;
  int layer;
  int kind;  // 0 logits, 1 selection, 2 gate/up, 3 down, 4 combine
};

constexpr int kKernelsPerLayer = 5;  // kinds of kernel per layer: logits, select, gate/up, down, combine
constexpr int kLaunchesPerLayer = 9;  // most launches of one layer (a prefill round)

struct GraphEntry {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  std::vector<hipGraphNode_t> nodes;  // kernel nodes in stream order
  std::vector<int> node_launch;       // index of each node's launch in `launches`
  std::vector<struct Launch> launches;
  unsigned weights_version = 0;       // the handle's weights the nodes' parameters carry
};

constexpr int kStagingSlots = 16;
constexpr int kProfileEvents = 512;  // event budget of the profiling ring (two per kernel)

}  // namespace

struct moe_round {
  moe_round_config cfg{};
  hipStream_t stream = nullptr;
  int device = 0;
  int Ucap = 0, Pcap = 0, Icap = 0;
  int Gh = 0, NBh = 0, Gi = 0, NBi = 0;
  // device scratch
  Ingress* d_ing = nullptr;            // graph-mode ingress
  float* xall = nullptr;               // layer outputs before the last (xslots slots of xstride floats)
  int xslots = 2;
  int xstride = 0;
  double* logits = nullptr;
  int32_t* n_unique = nullptr;
  int32_t* uniq = nullptr;
  int32_t* offs = nullptr;
  int32_t* pairs = nullptr;
  float* pair_w = nullptr;
  int32_t* rec = nullptr;
  float* hbuf = nullptr;
  float* ybuf = nullptr;               // exact mode: [Pcap][H]
  int32_t* slot_of = nullptr;          // [L][Pcap]
  int32_t* tsel = nullptr;             // [Pcap] wide rounds: top-k ids by (row, rank)
  float* tp = nullptr;                 // [Pcap] and their routing weights
  uint32_t* xq = nullptr;
  float2* xss = nullptr;
  // host state
  Ingress h_ing{};                     // last ingress of a run
  bool dev_ing_valid = false;          // d_ing holds h_ing
  std::vector<moe_layer_weights> h_wtab;
  const moe_layer_weights* wts = nullptr;  // the current weights [L] (h_wtab's data, or the caller's)
  unsigned weights_version = 1;        // bumped when a run names new weights (graph nodes follow it)
  unsigned char* staging = nullptr;    // pinned ring for graph-mode ingress uploads
  size_t slot_bytes = 0;
  hipEvent_t slot_ev[kStagingSlots] = {};
  bool slot_used[kStagingSlots] = {};
  int next_slot = 0;
  std::map<int, GraphEntry> graphs;
  // profiling: a ring of runs, each with a start/stop event per kernel (dispatch timestamps)
  bool profiling = false;
  int prof_runs = 0;                   // ring capacity in runs
  std::vector<hipEvent_t> prof_ev;     // [prof_runs][n kernels][2]
  std::vector<int> prof_nk;            // kernels recorded in each ring slot (0 = free)
  std::vector<int> prof_kind;          // [prof_runs][kernels] accumulator index (layer * 4 + kind)
  int prof_next = 0;
  std::vector<double> prof_ms;         // accumulated milliseconds [L][4]
  int32_t prof_count = 0;              // runs accumulated since the last read
  int last_T = 0, last_k = 0;
  int32_t last_hip = 0;
  int mfma_rows = 0;                   // gate/up (wide rounds): matrix-core tile from this many rows per item (0: never)
  int rows_per_item = 0;               // 0: by round width
  int fused_max_rows = kFusedMaxRows;  // selection folded into gate/up up to this many rows
  // prefill scratch (max_rows > MOE_ROUND_MAX_ROWS): rows Tp, pair slots pfP, work items pfI
  int Tp = 0, pfP = 0, pfI = 0;
  float* pf_xbuf[2] = {nullptr, nullptr};
  uint32_t* pf_xq = nullptr;
  float* pf_xstep = nullptr;
  unsigned long long* pf_mask = nullptr;
  int32_t* pf_wpre = nullptr;
  int32_t* pf_sel = nullptr;
  float* pf_selp = nullptr;
  int32_t* pf_uniq = nullptr;
  int32_t* pf_offs = nullptr;
  int32_t* pf_eoff = nullptr;
  int32_t* pf_pairs = nullptr;
  float* pf_pair_w = nullptr;
  int32_t* pf_slot_of = nullptr;
  int4* pf_items = nullptr;
  int32_t* pf_n_items = nullptr;
  float* pf_hbuf = nullptr;
  uint32_t* pf_hq = nullptr;
  float* pf_hstep = nullptr;
  float* pf_ybuf = nullptr;
  uint32_t* floor_sink = nullptr;      // [kFloorMaxBlocks] measurement kernels' sink
  // expert table mode and tail skip (caller-owned device arrays, bound with moe_round_bind_experts)
  const moe_expert_ref* etab = nullptr;  // [L][E]
  const uint32_t* resident = nullptr;    // [L][ceil(E/32)]
  int32_t* n_skipped = nullptr;          // [L] experts the tail skip left out
};

static moe_status hip_fail(moe_round* h, hipError_t e) {
  if (h) h->last_hip = static_cast<int32_t>(e);
  return e == hipErrorOutOfMemory ? MOE_ERR_OOM : MOE_ERR_HIP;
}

#define MOE_HIP(h, call)                              \
  do {                                                \
    hipError_t _e = (call);                           \
    if (_e != hipSuccess) return hip_fail((h), _e);   \
  } while (0)

// Rows of SwiGLU digits the down kernel stages in LDS at a time (per row: I/32 blocks of kXqWords
// digit words and a (step, sum) pair).
static int xstage_rows(int K) {
  const int r = kXStageBytes / (static_cast<int>(sizeof(uint32_t)) * (K / 32) * (kXqWords + 2));
  return r < 1 ? 1 : (r > kXStageMax ? kXStageMax : r);
}

// Rows of one expert handled by one work item: verify rounds split an expert shared by many rows
// over several blocks (each re-reads the expert's tile, which the caches serve: the measured
// gate/up traffic stays at the unique experts' bytes) so no
// block carries many rows, down to one row per item up to kOneRowItemsMaxRows rows (timed faster
// there than two-row items, whose blocks do twice the fold work each; from 12 rows the two-row
// items are faster); wide rounds keep larger items (2 rows up to kWideTwoRowMaxRows rows, then 4:
// timed faster at T = 32 and slower at T = 64 than the other size, and equal at T = 16).
constexpr int kOneRowItemsMaxRows = 10;
constexpr int kWideTwoRowMaxRows = 32;  // wide rounds up to this many rows: 2-row items, then 4
constexpr int kPairItemMaxRows = 4;  // items the row-pair form takes in wide rounds (see make_plan)
static int rows_per_item(const moe_round* h, int T) {
  if (h->rows_per_item > 0) return h->rows_per_item;
  if (T >= kWideRows) return T <= kWideTwoRowMaxRows ? 2 : 4;
  return T <= kOneRowItemsMaxRows ? 1 : 2;
}

// Upper bound of the work items of a round: sum over experts of ceil(rows / rg).
static int items_bound(int pairs, int E, int rg) {
  const int nu = pairs < E ? pairs : E;
  const int b = (pairs + nu * (rg - 1)) / rg;
  return b < pairs ? b : pairs;
}

static Args base_args(const moe_round* h, int T, int k) {
  Args a{};
  a.xall = h->xall;
  a.xslots = h->xslots;
  a.xstride = h->xstride;
  a.logits = h->logits;
  a.n_unique = h->n_unique;
  a.uniq = h->uniq;
  a.offs = h->offs;
  a.pairs = h->pairs;
  a.pair_w = h->pair_w;
  a.rec = h->rec;
  a.hbuf = h->hbuf;
  a.ybuf = h->ybuf;
  a.slot_of = h->slot_of;
  a.tsel = h->tsel;
  a.tp = h->tp;
  a.exact = h->cfg.exact;
  a.xq = h->xq;
  a.xss = h->xss;
  a.H = h->cfg.hidden;
  a.I = h->cfg.inter;
  a.E = h->cfg.n_experts;
  a.L = h->cfg.n_layers;
  a.T = T;
  a.k = k;
  a.residual = h->cfg.residual;
  a.Ucap = h->Ucap;
  a.Icap = h->Icap;
  a.rg = rows_per_item(h, T);
  a.Pcap = h->Pcap;
  a.xstage_h = gateup_stage_rows(h->cfg.hidden);
  a.mfma_rows = h->cfg.exact ? 0 : h->mfma_rows;  // the tile's sums differ in order from the GEMV
  a.xstage_i = xstage_rows(h->cfg.inter);
  a.prefetch = h->cfg.prefetch;
  a.skip_j = h->cfg.tail_skip_rank > 0 ? h->cfg.tail_skip_rank - 1 : (1 << 30);
  a.n_skipped = h->n_skipped;
  return a;
}

// Launches of a round. Rounds of up to kFusedMaxRows rows run three kernels per layer: the gate/up
// kernel computes the selection itself. Larger rounds run a separate selection kernel (and, from
// kSplitTopkRows rows, a many-block top-k before it); exact mode adds the combine.
struct RoundPlan {
  KernelFn lg = nullptr, sel = nullptr, gu = nullptr, dn = nullptr, topk = nullptr;
  dim3 grid_lg, grid_gu, grid_dn, grid_topk, grid_comb;
  int shm_gu = 0, shm_dn = 0;
  int thr_gu = kThreads;  // gate/up block size (fused many-row forms: groups of kThreads)
  bool fused = false, split_topk = false, exact = false;
};
constexpr int kMaxLaunchesPerLayer = 6;  // logits, top-k, select, gate/up, down, combine

static bool make_plan(const moe_round* h, int T, int k, RoundPlan* p) {
  const int E = h->cfg.n_experts, H = h->cfg.hidden, I = h->cfg.inter;
  const int umax = items_bound(T * k, E, rows_per_item(h, T));
  const bool wide = T >= kWideRows;
  p->fused = T <= h->fused_max_rows;
  p->split_topk = T >= kSplitTopkRows;
  p->exact = h->cfg.exact != 0;
  p->lg = pick_logits(H, T);
  p->sel = pick_select(E, p->split_topk);
  p->topk = pick_topk_rows(E);
  int rows_gu = 0, rows_dn = 0;
  // Wide rounds take the row-pair form, which loads each pair's input digits from L2, for items of
  // up to kPairItemMaxRows rows (timed faster than staging the rows in LDS at T = 16, 32 and 64); the
  // staged form serves larger items and the matrix-core tile.
  const bool staged = wide && (rows_per_item(h, T) > kPairItemMaxRows || (h->mfma_rows > 0 && !h->cfg.exact));
  const int gu_mode = staged ? kGuStaged : (T == 1 ? kGuOneRow : (rows_per_item(h, T) == 1 ? kGuRowItems : kGuPairs));
  const int fmt = h->cfg.weight_format;
  // the down tile: wide rounds with the matrix-core tiles enabled, I = 512 (G = 16 x 1 block)
  const bool down_tile = wide && h->mfma_rows > 0 && !h->cfg.exact && h->Gi == 16 && h->NBi == 1 &&
                         fmt == MOE_WEIGHT_Q4B32;
  if (!p->lg || !pick_gemv(h->Gh, h->NBh, gu_mode, true, p->fused ? fused_select_keys(E) : 0, fmt, &p->gu, &rows_gu) ||
      !pick_gemv(h->Gi, h->NBi, down_tile ? 1 : 0, false, h->cfg.exact, fmt, &p->dn, &rows_dn))
    return false;
  // Rounds whose down grid is small (at most kDownHalfMaxBlocks full-height blocks, up to three per
  // CU) take half-height down blocks: twice the blocks, each with half the rows of H, so more of
  // the expert tiles' loads are in flight at once. Rounds of one-row items whose full-height grid
  // is more than the CUs hold at once (kDownDoubleMinBlocks) take double-height blocks: each
  // block's record read and SwiGLU staging then serve twice the rows of H.
  const int blocks_dn = umax * ((H + rows_dn - 1) / rows_dn);
  const int dn_mode = down_tile ? 1
                      : blocks_dn <= kDownHalfMaxBlocks ? 2
                      : (blocks_dn > kDownDoubleMinBlocks && rows_per_item(h, T) == 1) ? 3 : 0;
  if (dn_mode >= 2 && !pick_gemv(h->Gi, h->NBi, dn_mode, false, h->cfg.exact, fmt, &p->dn, &rows_dn)) return false;
  p->grid_lg = logits_grid(E, H, T);
  const int units_gu = umax * ((I + rows_gu - 1) / rows_gu);
  const int groups = gateup_groups(gu_mode, p->fused ? fused_select_keys(E) : 0);
  p->thr_gu = kThreads * groups;
  p->grid_gu = dim3(p->fused && units_gu > kFusedBlocks / groups ? kFusedBlocks / groups : units_gu);
  p->grid_dn = dim3(umax * ((H + rows_dn - 1) / rows_dn));
  p->grid_topk = dim3((T + kWaves - 1) / kWaves);
  p->grid_comb = dim3(T, (H + 4 * kThreads - 1) / (4 * kThreads));
  int gu_words = gateup_stage_words(H);
  if (h->Gh == 64 && h->NBh == 1) gu_words += kMfmaExtraWords;  // matrix-core tile: (s, m) tables, partial sums
  p->shm_gu = staged ? static_cast<int>(sizeof(uint32_t)) * gu_words : 0;
  p->shm_dn = static_cast<int>(sizeof(uint32_t)) * xstage_rows(I) * (I / 32) * (kXqWords + 2);
  if (down_tile) p->shm_dn += static_cast<int>(sizeof(uint32_t)) * kDownTileExtraWords;  // its (s, m) tables
  return true;
}

// The launches of layer l, in stream order, into out[0 .. kMaxLaunchesPerLayer - 1]; returns their number.
static int layer_launches(const RoundPlan& p, int l, Launch* out) {
  int n = 0;
  out[n++] = {p.lg, p.grid_lg, kThreads, 0, l, 0};
  if (!p.fused && p.split_topk) out[n++] = {p.topk, p.grid_topk, kThreads, 0, l, 1};
  if (!p.fused) out[n++] = {p.sel, dim3(1), kSelectThreads, 0, l, 1};
  out[n++] = {p.gu, p.grid_gu, p.thr_gu, p.shm_gu, l, 2};
  out[n++] = {p.dn, p.grid_dn, kThreads, p.shm_dn, l, 3};
  if (p.exact) out[n++] = {combine_kernel, p.grid_comb, kThreads, 0, l, 4};
  return n;
}

// The parameters of a launch of layer `layer`: the round's arguments with that layer's weights
// and the next layer's router (for the down kernel's early touch of it).
static Args layer_args(const moe_round* h, Args a, int layer) {
  a.w = h->wts[layer];
  a.router_next = layer + 1 < h->cfg.n_layers ? h->wts[layer + 1].router_w : nullptr;
  const size_t E = h->cfg.n_experts;
  a.etab = h->etab ? h->etab + layer * E : nullptr;
  a.resident = h->resident ? h->resident + layer * ((E + 31) / 32) : nullptr;
  return a;
}

// Graph mode: one graph per (T, k) whose kernels read the per-run pointers from the fixed ingress
// buffer; each node carries its layer's weight pointers as parameters, rewritten in place in the
// instantiated graph when a run names new weights (no recapture).
static moe_status build_graph(moe_round* h, int T, int k, GraphEntry* ge) {
  RoundPlan p;
  if (!make_plan(h, T, k, &p)) return MOE_ERR_UNSUPPORTED;
  Args base = base_args(h, T, k);
  base.ing = h->d_ing;
  hipGraph_t g = nullptr;
  MOE_HIP(h, hipGraphCreate(&g, 0));
  hipGraphNode_t prev = nullptr;
  for (int l = 0; l < h->cfg.n_layers; ++l) {
    Launch ls[kMaxLaunchesPerLayer];
    const int n = layer_launches(p, l, ls);
    Args a = layer_args(h, base, l);
    for (int i = 0; i < n; ++i) {
      const Launch& L = ls[i];
      int layer = L.layer;
      void* params[] = {&a, &layer};
      hipKernelNodeParams kp{};
      kp.func = reinterpret_cast<void*>(L.fn);
      kp.gridDim = L.grid;
      kp.blockDim = dim3(L.threads);
      kp.sharedMemBytes = L.shmem;
      kp.kernelParams = params;
      kp.extra = nullptr;
      hipGraphNode_t node = nullptr;
      hipError_t e = hipGraphAddKernelNode(&node, g, prev ? &prev : nullptr, prev ? 1 : 0, &kp);
      if (e != hipSuccess) {
        (void)hipGraphDestroy(g);
        return hip_fail(h, e);
      }
      prev = node;
      ge->nodes.push_back(node);
      ge->node_launch.push_back(static_cast<int>(ge->launches.size()));
      ge->launches.push_back(L);
    }
  }
  hipGraphExec_t x = nullptr;
  hipError_t e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_fail(h, e);
  }
  ge->graph = g;
  ge->exec = x;
  ge->weights_version = h->weights_version;
  return MOE_OK;
}

// New weights for a captured graph: every node's parameters rewritten in the instantiated graph.
static moe_status update_graph_weights(moe_round* h, GraphEntry* ge, int T, int k) {
  Args base = base_args(h, T, k);
  base.ing = h->d_ing;
  for (size_t i = 0; i < ge->nodes.size(); ++i) {
    const Launch& L = ge->launches[ge->node_launch[i]];
    Args a = layer_args(h, base, L.layer);
    int layer = L.layer;
    void* params[] = {&a, &layer};
    hipKernelNodeParams kp{};
    kp.func = reinterpret_cast<void*>(L.fn);
    kp.gridDim = L.grid;
    kp.blockDim = dim3(L.threads);
    kp.sharedMemBytes = L.shmem;
    kp.kernelParams = params;
    kp.extra = nullptr;
    MOE_HIP(h, hipGraphExecKernelNodeSetParams(ge->exec, ge->nodes[i], &kp));
  }
  ge->weights_version = h->weights_version;
  return MOE_OK;
}

// Eager: every launch carries the ingress pointers and its layer's weights by value. No host
// allocation: the plan is a fixed struct and the launches are expanded one layer at a time.
static moe_status launch_eager(moe_round* h, int T, int k, hipEvent_t* evs, int* kinds = nullptr,
                               int* n_launched = nullptr) {
  RoundPlan p;
  if (!make_plan(h, T, k, &p)) return MOE_ERR_UNSUPPORTED;
  Args a = base_args(h, T, k);
  a.in = h->h_ing;
  int i = 0;
  for (int l = 0; l < h->cfg.n_layers; ++l) {
    Launch ls[kMaxLaunchesPerLayer];
    const int n = layer_launches(p, l, ls);
    a = layer_args(h, a, l);
    for (int j = 0; j < n; ++j, ++i) {
      const Launch& L = ls[j];
      if (kinds) kinds[i] = L.layer * kKernelsPerLayer + L.kind;
      int layer = L.layer;
      void* params[] = {&a, &layer};
      if (evs)  // events stamped with the dispatch's own start and end times
        MOE_HIP(h, hipExtLaunchKernel(reinterpret_cast<const void*>(L.fn), L.grid, dim3(L.threads), params,
                                      L.shmem, h->stream, evs[2 * i], evs[2 * i + 1], 0));
      else
        MOE_HIP(h, hipLaunchKernel(reinterpret_cast<const void*>(L.fn), L.grid, dim3(L.threads), params,
                                   L.shmem, h->stream));
    }
  }
  if (n_launched) *n_launched = i;
  return MOE_OK;
}

// Work items of a prefill round bound: sum over experts of ceil(rows / 64).
static int pf_items_bound(int pairs, int E) {
  const int b = E + (pairs + pf::kTile - 1) / pf::kTile;
  return b < pairs ? b : pairs;
}

typedef void (*PfKernelFn)(pf::PfArgs, int);

// Prefill rounds of up to this many rows split the router GEMM's reduction over four waves. At
// 512 rows the one-wave-per-tile grid fills half the SIMDs and the split halves the kernel's time
// (68 -> 32 us); at 4096 rows the split is slightly slower (159 vs 148 us).
constexpr int kPfSplitKRows = 2048;

// The down kernel that copies rows once, for the round's weight format and I / 128 steps (1..4).
static PfKernelFn pf_pick_down32(bool s256, int nstep) {
  switch (nstep) {
    case 1: return s256 ? pf::pf_down32_kernel<kFmtQ4S256, 1> : pf::pf_down32_kernel<kFmtQ4B32, 1>;
    case 2: return s256 ? pf::pf_down32_kernel<kFmtQ4S256, 2> : pf::pf_down32_kernel<kFmtQ4B32, 2>;
    case 3: return s256 ? pf::pf_down32_kernel<kFmtQ4S256, 3> : pf::pf_down32_kernel<kFmtQ4B32, 3>;
    default: return s256 ? pf::pf_down32_kernel<kFmtQ4S256, 4> : pf::pf_down32_kernel<kFmtQ4B32, 4>;
  }
}

static PfKernelFn pf_pick_topk(int E) {
  if (E <= 64) return pf::pf_topk_kernel<1>;
  if (E <= 128) return pf::pf_topk_kernel<2>;
  if (E <= 256) return pf::pf_topk_kernel<4>;
  return pf::pf_topk_kernel<8>;
}

// A prefill round (T > MOE_ROUND_MAX_ROWS), eagerly: per layer the fp16 pairs of the layer input,
// router logits, top-k, the counting sort (offsets, then the scatter), gate/up, the SwiGLU rows'
// fp16 pairs, down and the combine.
// evs: with profiling, a start/stop pair per launch; kinds: their accumulator (layer, kind).
static moe_status launch_prefill(moe_round* h, int T, int k, hipEvent_t* evs, int* kinds, int* n_launched) {
  const int E = h->cfg.n_experts, H = h->cfg.hidden, I = h->cfg.inter, L = h->cfg.n_layers;
  pf::PfArgs a{};
  a.in = h->h_ing;
  a.xbuf0 = h->pf_xbuf[0];
  a.xbuf1 = h->pf_xbuf[1];
  a.logits = h->logits;
  a.xq = h->pf_xq;
  a.xstep = h->pf_xstep;
  a.mask = h->pf_mask;
  a.wpre = h->pf_wpre;
  a.sel = h->pf_sel;
  a.selp = h->pf_selp;
  a.n_unique = h->n_unique;
  a.uniq = h->pf_uniq;
  a.offs = h->pf_offs;
  a.eoff = h->pf_eoff;
  a.pairs = h->pf_pairs;
  a.pair_w = h->pf_pair_w;
  a.slot_of = h->pf_slot_of;
  a.items = h->pf_items;
  a.n_items = h->pf_n_items;
  a.hbuf = h->pf_hbuf;
  a.hq = h->pf_hq;
  a.hstep = h->pf_hstep;
  a.ybuf = h->pf_ybuf;
  a.H = H;
  a.I = I;
  a.E = E;
  a.L = L;
  a.T = T;
  a.k = k;
  a.residual = h->cfg.residual;
  a.Pcap = h->pfP;
  a.Icap = h->pfI;
  a.W = (T + 63) / 64;
  const int np = T * k;
  const int ib = pf_items_bound(np, E);
  const int gu_units = ((ib * (I / pf::kTile) + 7) / 8) * 8;
  // Down: rows copied once per (item half, 256 rows of H) where they fit (I <= 512), else per step.
  const bool dn32 = I <= pf::kDown32MaxI;
  const int dn_units = ((ib * (dn32 ? 2 * (H / pf::kDown32Rows) : H / pf::kDownRows) + 7) / 8) * 8;
  const int dn_lds = dn32 ? pf::down32_lds(I) : pf::kGemmLds;
  const PfKernelFn topk = pf_pick_topk(E);
  const bool s256 = h->cfg.weight_format == MOE_WEIGHT_Q4S256;
  const PfKernelFn gateup = s256 ? pf::pf_gateup_kernel<kFmtQ4S256, pf::kGateupTiles>
                                 : pf::pf_gateup_kernel<kFmtQ4B32, pf::kGateupTiles>;
  const PfKernelFn down = dn32 ? pf_pick_down32(s256, I / (32 * pf::kStepBlocks))
                                : s256 ? pf::pf_down_kernel<kFmtQ4S256> : pf::pf_down_kernel<kFmtQ4B32>;
  int i = 0;
  auto launch = [&](const void* fn, dim3 grid, int threads, int shmem, void** params, int layer, int kind) {
    if (kinds) kinds[i] = layer * kKernelsPerLayer + kind;
    hipError_t e = evs ? hipExtLaunchKernel(fn, grid, dim3(threads), params, shmem, h->stream, evs[2 * i],
                                            evs[2 * i + 1], 0)
                       : hipLaunchKernel(fn, grid, dim3(threads), params, shmem, h->stream);
    ++i;
    return e;
  };
  for (int l = 0; l < L; ++l) {
    a.w = h->wts[l];
    int layer = l;
    void* gp[] = {&a, &layer};
    const float* xin = l == 0 ? h->h_ing.hidden : h->pf_xbuf[(l - 1) & 1];
    int kH = H, nT = T, zw = E * a.W, kI = I, nP = np, zero0 = 0;
    unsigned long long* no_mask = nullptr;
    void* qx[] = {&xin, &kH, &nT, &a.xq, &a.xstep, &a.mask, &zw};
    void* qh[] = {&a.hbuf, &kI, &nP, &a.hq, &a.hstep, &no_mask, &zero0};
    hipError_t e;
    if ((e = launch(reinterpret_cast<const void*>(pf::quant_rows_kernel), dim3((T + kWaves - 1) / kWaves), kThreads, 0,
                    qx, l, 0)) != hipSuccess ||
        (e = (T <= kPfSplitKRows
                  ? launch(reinterpret_cast<const void*>(pf::pf_logits_splitk_kernel), dim3((E + 15) / 16, (T + 15) / 16),
                           kThreads, 0, gp, l, 0)
                  : launch(reinterpret_cast<const void*>(pf::pf_logits_kernel), dim3((E + 31) / 32, (T + 31) / 32),
                           kThreads, 0, gp, l, 0))) != hipSuccess ||
        (e = launch(reinterpret_cast<const void*>(topk), dim3((T + kWaves - 1) / kWaves), kThreads, 0, gp, l, 1)) !=
            hipSuccess ||
        (e = launch(reinterpret_cast<const void*>(pf::pf_scan_kernel), dim3(1), pf::kScanThreads, 0, gp, l, 1)) !=
            hipSuccess ||
        (e = launch(reinterpret_cast<const void*>(pf::pf_scatter_kernel), dim3((np + kThreads - 1) / kThreads),
                    kThreads, 0, gp, l, 1)) != hipSuccess ||
        (e = launch(reinterpret_cast<const void*>(gateup), dim3(gu_units), pf::kGateupThreads,
                    pf::kGemmLds, gp, l, 2)) != hipSuccess ||
        (e = launch(reinterpret_cast<const void*>(pf::quant_rows_kernel), dim3((np + kWaves - 1) / kWaves), kThreads,
                    0, qh, l, 3)) != hipSuccess ||
        (e = launch(reinterpret_cast<const void*>(down), dim3(dn_units), pf::kGemmThreads, dn_lds, gp, l, 3)) !=
            hipSuccess ||
        (e = launch(reinterpret_cast<const void*>(pf::pf_combine_kernel), dim3(T, (H + 4 * kThreads - 1) / (4 * kThreads)),
                    kThreads, 0, gp, l, 4)) != hipSuccess)
      return hip_fail(h, e);
  }
  if (n_launched) *n_launched = i;
  return MOE_OK;
}

// Graph mode: upload changed ingress pointers through a pinned slot.
static moe_status sync_device_ingress(moe_round* h) {
  if (h->dev_ing_valid) return MOE_OK;
  const int s = h->next_slot;
  h->next_slot = (s + 1) % kStagingSlots;
  if (h->slot_used[s]) MOE_HIP(h, hipEventSynchronize(h->slot_ev[s]));
  unsigned char* slot = h->staging + static_cast<size_t>(s) * h->slot_bytes;
  std::memcpy(slot, &h->h_ing, sizeof(Ingress));
  MOE_HIP(h, hipMemcpyAsync(h->d_ing, slot, sizeof(Ingress), hipMemcpyHostToDevice, h->stream));
  h->dev_ing_valid = true;
  MOE_HIP(h, hipEventRecord(h->slot_ev[s], h->stream));
  h->slot_used[s] = true;
  return MOE_OK;
}

// Fold one ring slot's kernel durations into the accumulators (waits for its last kernel).
static moe_status harvest(moe_round* h, int slot) {
  const int nk = h->prof_nk[slot];
  if (nk == 0) return MOE_OK;
  hipEvent_t* ev = h->prof_ev.data() + static_cast<size_t>(slot) * 2 * kLaunchesPerLayer * h->cfg.n_layers;
  h->prof_nk[slot] = 0;
  MOE_HIP(h, hipEventSynchronize(ev[2 * nk - 1]));
  const int* kind = h->prof_kind.data() + static_cast<size_t>(slot) * kLaunchesPerLayer * h->cfg.n_layers;
  for (int i = 0; i < nk; ++i) {
    float ms = 0.f;
    MOE_HIP(h, hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]));
    h->prof_ms[kind[i]] += ms;
  }
  ++h->prof_count;
  return MOE_OK;
}

static void free_profile(moe_round* h) {
  for (auto& ev : h->prof_ev)
    if (ev) (void)hipEventDestroy(ev);
  h->prof_ev.clear();
  h->prof_nk.clear();
  h->prof_kind.clear();
  h->prof_runs = 0;
}

static void free_handle(moe_round* h) {
  if (!h) return;
  if (h->stream) (void)hipStreamSynchronize(h->stream);
  free_profile(h);
  for (auto& kv : h->graphs) {
    if (kv.second.exec) (void)hipGraphExecDestroy(kv.second.exec);
    if (kv.second.graph) (void)hipGraphDestroy(kv.second.graph);
  }
  for (int i = 0; i < kStagingSlots; ++i)
    if (h->slot_ev[i]) (void)hipEventDestroy(h->slot_ev[i]);
  if (h->staging) (void)hipHostFree(h->staging);
  void* ptrs[] = {h->d_ing, h->xall, h->logits, h->n_unique, h->uniq, h->offs,
                  h->pairs, h->pair_w, h->rec, h->hbuf, h->ybuf, h->slot_of, h->tsel, h->tp, h->xq, h->xss,
                  h->pf_xbuf[0], h->pf_xbuf[1], h->pf_xq, h->pf_xstep, h->pf_mask, h->pf_wpre,
                  h->pf_sel, h->pf_selp, h->pf_uniq, h->pf_offs, h->pf_eoff, h->pf_pairs, h->pf_pair_w, h->pf_slot_of,
                  h->pf_items, h->pf_n_items, h->pf_hbuf, h->pf_hq, h->pf_hstep, h->pf_ybuf, h->floor_sink,
                  h->n_skipped};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
  delete h;
}

extern "C" moe_status moe_round_init(const moe_round_config* cfg, const moe_layer_weights* layers,
                                     void* stream, moe_round** out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  *out = nullptr;
  moe_status st = validate_config(cfg);
  if (st != MOE_OK) return st;
  st = validate_layers(cfg, layers);
  if (st != MOE_OK) return st;

  moe_round* h = new moe_round();
  h->cfg = *cfg;
  h->stream = static_cast<hipStream_t>(stream);
  split_blocks(cfg->hidden, &h->Gh, &h->NBh);
  split_blocks(cfg->inter, &h->Gi, &h->NBi);
  // decode/verify scratch for rounds of up to MOE_ROUND_MAX_ROWS rows; prefill scratch beyond
  const int T = cfg->max_rows < MOE_ROUND_MAX_ROWS ? cfg->max_rows : MOE_ROUND_MAX_ROWS;
  const int E = cfg->n_experts, K = cfg->top_k_max, L = cfg->n_layers;
  const int H = cfg->hidden, I = cfg->inter;
  h->Pcap = T * K;
  h->Ucap = (T * K < E) ? T * K : E;
  h->Icap = T * K;  // work items never outnumber (row, rank) pairs
  h->h_wtab.assign(layers, layers + L);
  h->wts = h->h_wtab.data();
  if (cfg->fused_max_rows != 0) h->fused_max_rows = cfg->fused_max_rows < 0 ? 0 : cfg->fused_max_rows;
  h->rows_per_item = cfg->rows_per_item;
  if (cfg->mfma_min_rows != 0) h->mfma_rows = cfg->mfma_min_rows < 0 ? 0 : cfg->mfma_min_rows;

  auto fail = [&](hipError_t e) {
    moe_status s = hip_fail(h, e);
    free_handle(h);
    return s;
  };
  hipError_t e;
  if ((e = hipGetDevice(&h->device)) != hipSuccess) return fail(e);
#define MOE_ALLOC(ptr, bytes) \
  if ((e = hipMalloc(reinterpret_cast<void**>(&(ptr)), (bytes))) != hipSuccess) return fail(e);
  MOE_ALLOC(h->d_ing, sizeof(Ingress));
  h->xslots = (cfg->record_layers && L > 2) ? L - 1 : 2;
  h->xstride = T * H;
  MOE_ALLOC(h->xall, sizeof(float) * h->xslots * T * H);
  MOE_ALLOC(h->logits, sizeof(double) * cfg->max_rows * E);
  MOE_ALLOC(h->n_unique, sizeof(int32_t) * L);
  MOE_ALLOC(h->n_skipped, sizeof(int32_t) * L);
  MOE_ALLOC(h->uniq, sizeof(int32_t) * L * h->Ucap);
  MOE_ALLOC(h->offs, sizeof(int32_t) * L * (h->Ucap + 1));
  MOE_ALLOC(h->pairs, sizeof(int32_t) * L * h->Pcap);
  MOE_ALLOC(h->pair_w, sizeof(float) * L * h->Pcap);
  MOE_ALLOC(h->rec, sizeof(int32_t) * L * h->Icap * kRecWords);
  MOE_ALLOC(h->hbuf, sizeof(float) * h->Pcap * I);
  MOE_ALLOC(h->slot_of, sizeof(int32_t) * L * h->Pcap);
  MOE_ALLOC(h->tsel, sizeof(int32_t) * h->Pcap);
  MOE_ALLOC(h->tp, sizeof(float) * h->Pcap);
  if (cfg->exact) MOE_ALLOC(h->ybuf, sizeof(float) * h->Pcap * H);
  MOE_ALLOC(h->xq, sizeof(uint32_t) * T * (H / 32) * kXqWords);
  MOE_ALLOC(h->xss, sizeof(float2) * T * (H / 32));
  MOE_ALLOC(h->floor_sink, sizeof(uint32_t) * kFloorMaxBlocks);
  if (cfg->max_rows > MOE_ROUND_MAX_ROWS) {
    const size_t Tp = cfg->max_rows, P = Tp * K, W = (Tp + 63) / 64;
    h->Tp = static_cast<int>(Tp);
    h->pfP = static_cast<int>(P);
    h->pfI = pf_items_bound(static_cast<int>(P), E);
    if (L > 1) {
      MOE_ALLOC(h->pf_xbuf[0], sizeof(float) * Tp * H);
      MOE_ALLOC(h->pf_xbuf[1], sizeof(float) * Tp * H);
    }
    MOE_ALLOC(h->pf_xq, sizeof(uint32_t) * Tp * pf::pf_row_words(H));
    MOE_ALLOC(h->pf_xstep, sizeof(float) * Tp);
    MOE_ALLOC(h->pf_mask, sizeof(unsigned long long) * E * W);
    MOE_ALLOC(h->pf_wpre, sizeof(int32_t) * E * W);
    MOE_ALLOC(h->pf_sel, sizeof(int32_t) * P);
    MOE_ALLOC(h->pf_selp, sizeof(float) * P);
    MOE_ALLOC(h->pf_uniq, sizeof(int32_t) * L * E);
    MOE_ALLOC(h->pf_offs, sizeof(int32_t) * L * (E + 1));
    MOE_ALLOC(h->pf_eoff, sizeof(int32_t) * E);
    MOE_ALLOC(h->pf_pairs, sizeof(int32_t) * L * P);
    MOE_ALLOC(h->pf_pair_w, sizeof(float) * P);
    MOE_ALLOC(h->pf_slot_of, sizeof(int32_t) * P);
    MOE_ALLOC(h->pf_items, sizeof(int4) * h->pfI);
    MOE_ALLOC(h->pf_n_items, sizeof(int32_t));
    MOE_ALLOC(h->pf_hbuf, sizeof(float) * P * I);
    MOE_ALLOC(h->pf_hq, sizeof(uint32_t) * P * pf::pf_row_words(I));
    MOE_ALLOC(h->pf_hstep, sizeof(float) * P);
    MOE_ALLOC(h->pf_ybuf, sizeof(float) * P * H);
  }
#undef MOE_ALLOC
  h->slot_bytes = 256;
  if ((e = hipHostMalloc(reinterpret_cast<void**>(&h->staging), h->slot_bytes * kStagingSlots, 0)) !=
      hipSuccess)
    return fail(e);
  for (int i = 0; i < kStagingSlots; ++i)
    if ((e = hipEventCreateWithFlags(&h->slot_ev[i], hipEventDisableTiming)) != hipSuccess) return fail(e);
  if ((e = hipMemsetAsync(h->n_unique, 0, sizeof(int32_t) * L, h->stream)) != hipSuccess) return fail(e);
  if ((e = hipMemsetAsync(h->n_skipped, 0, sizeof(int32_t) * L, h->stream)) != hipSuccess) return fail(e);
  if ((e = hipMemsetAsync(h->rec, 0, sizeof(int32_t) * L * h->Icap * kRecWords, h->stream)) != hipSuccess)
    return fail(e);
  if ((e = hipStreamSynchronize(h->stream)) != hipSuccess) return fail(e);
  *out = h;
  return MOE_OK;
}

static moe_status prepare_run(moe_round* h, const float* hidden, int32_t T, int32_t k,
                              const moe_layer_weights* layers, float* out, int32_t* ids, float* rw) {
  if (!h) return MOE_ERR_INVALID_ARG;
  moe_status st = validate_run(&h->cfg, hidden, T, k, out, ids, rw);
  if (st != MOE_OK) return st;
  if (T > 0 && ((h->cfg.expert_table && !h->etab) || (h->cfg.tail_skip_rank > 0 && !h->resident)))
    return MOE_ERR_STATE;  // the table or the residency bits are not bound yet
  if (layers) {
    st = validate_layers(&h->cfg, layers);
    if (st != MOE_OK) return st;
    if (std::memcmp(layers, h->h_wtab.data(), sizeof(moe_layer_weights) * h->cfg.n_layers) != 0) {
      std::memcpy(h->h_wtab.data(), layers, sizeof(moe_layer_weights) * h->cfg.n_layers);
      ++h->weights_version;
    }
  }
  const Ingress ing{hidden, out, ids, rw};
  if (std::memcmp(&ing, &h->h_ing, sizeof(Ingress)) != 0) {
    h->h_ing = ing;
    h->dev_ing_valid = false;
  }
  return MOE_OK;
}

extern "C" moe_status moe_round_bind_experts(moe_round* h, const moe_expert_ref* table,
                                             const uint32_t* resident) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if ((table != nullptr) != (h->cfg.expert_table != 0)) return MOE_ERR_INVALID_ARG;
  if ((resident != nullptr) != (h->cfg.tail_skip_rank > 0)) return MOE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(table) & 15u) || (reinterpret_cast<uintptr_t>(resident) & 3u))
    return MOE_ERR_INVALID_ARG;
  if (table != h->etab || resident != h->resident) {
    h->etab = table;
    h->resident = resident;
    ++h->weights_version;  // captured graphs' nodes carry the per-layer pointers
  }
  return MOE_OK;
}

extern "C" moe_status moe_round_host_tier_pointer(const void* host_ptr, void** device_ptr) {
  if (!host_ptr || !device_ptr) return MOE_ERR_INVALID_ARG;
  *device_ptr = nullptr;
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, host_ptr) != hipSuccess) {
    (void)hipGetLastError();  // not memory the runtime knows: clear the sticky error
    return MOE_ERR_INVALID_ARG;
  }
  if (attr.type != hipMemoryTypeHost) return MOE_ERR_INVALID_ARG;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void*>(host_ptr), 0) != hipSuccess || !d) {
    (void)hipGetLastError();
    return MOE_ERR_INVALID_ARG;
  }
  *device_ptr = d;
  return MOE_OK;
}

extern "C" moe_status moe_round_run(moe_round* h, const float* hidden, int32_t T, int32_t k,
                                    const moe_layer_weights* layers, float* out, int32_t* expert_ids,
                                    float* route_w) {
  moe_status st = prepare_run(h, hidden, T, k, layers, out, expert_ids, route_w);
  if (st != MOE_OK) return st;
  if (T == 0) {  // empty round: nothing to enqueue; introspection has no round to report
    h->last_T = 0;
    return MOE_OK;
  }
  if (h->profiling) {
    const int slot = h->prof_next;
    h->prof_next = (slot + 1) % h->prof_runs;
    st = harvest(h, slot);  // a slot is reused only after its previous run has been read
    if (st != MOE_OK) return st;
    hipEvent_t* ev = h->prof_ev.data() + static_cast<size_t>(slot) * 2 * kLaunchesPerLayer * h->cfg.n_layers;
    int* kinds = h->prof_kind.data() + static_cast<size_t>(slot) * kLaunchesPerLayer * h->cfg.n_layers;
    int nl = 0;
    st = T > MOE_ROUND_MAX_ROWS ? launch_prefill(h, T, k, ev, kinds, &nl) : launch_eager(h, T, k, ev, kinds, &nl);
    if (st != MOE_OK) return st;
    h->prof_nk[slot] = nl;
  } else if (T > MOE_ROUND_MAX_ROWS) {
    st = launch_prefill(h, T, k, nullptr, nullptr, nullptr);
    if (st != MOE_OK) return st;
  } else if (h->cfg.use_graph) {
    st = sync_device_ingress(h);
    if (st != MOE_OK) return st;
    const int key = T * 64 + k;
    auto it = h->graphs.find(key);
    if (it == h->graphs.end()) {
      GraphEntry ge;
      st = build_graph(h, T, k, &ge);
      if (st != MOE_OK) return st;
      it = h->graphs.emplace(key, std::move(ge)).first;
    } else if (it->second.weights_version != h->weights_version) {
      st = update_graph_weights(h, &it->second, T, k);
      if (st != MOE_OK) return st;
    }
    MOE_HIP(h, hipGraphLaunch(it->second.exec, h->stream));
  } else {
    st = launch_eager(h, T, k, nullptr);
    if (st != MOE_OK) return st;
  }
  h->last_T = T;
  h->last_k = k;
  return MOE_OK;
}

extern "C" moe_status moe_round_profile(moe_round* h, int32_t enable) {
  if (!h || (enable != 0 && enable != 1)) return MOE_ERR_INVALID_ARG;
  if (enable == h->profiling) return MOE_OK;
  if (enable) {
    const int per_run = 2 * kLaunchesPerLayer * h->cfg.n_layers;
    const int runs = kProfileEvents / per_run > 2 ? kProfileEvents / per_run : 2;
    h->prof_ev.assign(static_cast<size_t>(runs) * per_run, nullptr);
    h->prof_nk.assign(runs, 0);
    h->prof_kind.assign(static_cast<size_t>(runs) * kLaunchesPerLayer * h->cfg.n_layers, 0);
    h->prof_runs = runs;
    h->prof_next = 0;
    for (auto& ev : h->prof_ev) {
      hipError_t e = hipEventCreate(&ev);
      if (e != hipSuccess) {
        free_profile(h);
        return hip_fail(h, e);
      }
    }
    h->prof_ms.assign(kKernelsPerLayer * h->cfg.n_layers, 0.0);
    h->prof_count = 0;
    h->profiling = true;
    return MOE_OK;
  }
  // Disabling keeps the accumulated sums for a later read but drops the ring.
  for (int s2 = 0; s2 < h->prof_runs; ++s2) {
    moe_status st = harvest(h, (h->prof_next + s2) % h->prof_runs);
    if (st != MOE_OK) return st;
  }
  MOE_HIP(h, hipStreamSynchronize(h->stream));
  free_profile(h);
  h->profiling = false;
  return MOE_OK;
}

extern "C" moe_status moe_round_profile_read(moe_round* h, double* kernel_ms, int32_t* n_runs) {
  if (!h || !kernel_ms || !n_runs) return MOE_ERR_INVALID_ARG;
  if (h->prof_ms.empty()) return MOE_ERR_STATE;
  for (int s2 = 0; s2 < h->prof_runs; ++s2) {  // oldest first
    moe_status st = harvest(h, (h->prof_next + s2) % h->prof_runs);
    if (st != MOE_OK) return st;
  }
  for (size_t i = 0; i < h->prof_ms.size(); ++i) {
    kernel_ms[i] = h->prof_ms[i];
    h->prof_ms[i] = 0.0;
  }
  *n_runs = h->prof_count;
  h->prof_count = 0;
  return MOE_OK;
}

extern "C" moe_status moe_round_worklist(moe_round* h, int32_t layer, int32_t* n_unique, int32_t* uniq,
                                         int32_t* offs, int32_t* pairs) {
  if (!h || !n_unique) return MOE_ERR_INVALID_ARG;
  if (layer < 0 || layer >= h->cfg.n_layers) return MOE_ERR_INVALID_ARG;
  if (h->last_T == 0) return MOE_ERR_STATE;
  MOE_HIP(h, hipStreamSynchronize(h->stream));
  int32_t nu = 0;
  MOE_HIP(h, hipMemcpy(&nu, h->n_unique + layer, sizeof(int32_t), hipMemcpyDeviceToHost));
  *n_unique = nu;
  // prefill rounds: their own lists (capacity E per layer), pairs packed as t | j << 16
  const bool pf = h->last_T > MOE_ROUND_MAX_ROWS;
  const int ucap = pf ? h->cfg.n_experts : h->Ucap;
  const int32_t* d_uniq = pf ? h->pf_uniq : h->uniq;
  const int32_t* d_offs = pf ? h->pf_offs : h->offs;
  const int32_t* d_pairs = pf ? h->pf_pairs + static_cast<size_t>(layer) * h->pfP
                              : h->pairs + static_cast<size_t>(layer) * h->Pcap;
  if (nu < 0 || nu > ucap) return MOE_ERR_STATE;
  if (uniq && nu)
    MOE_HIP(h, hipMemcpy(uniq, d_uniq + static_cast<size_t>(layer) * ucap, sizeof(int32_t) * nu, hipMemcpyDeviceToHost));
  if (offs)
    MOE_HIP(h, hipMemcpy(offs, d_offs + static_cast<size_t>(layer) * (ucap + 1), sizeof(int32_t) * (nu + 1),
                         hipMemcpyDeviceToHost));
  if (pairs) {
    const int np = h->last_T * h->last_k;
    int kept = np;  // the tail skip may leave pairs out: the worklist holds offs[n_unique] of them
    if (!pf)
      MOE_HIP(h, hipMemcpy(&kept, d_offs + static_cast<size_t>(layer) * (ucap + 1) + nu, sizeof(int32_t),
                           hipMemcpyDeviceToHost));
    if (kept < 0 || kept > np) return MOE_ERR_STATE;
    std::vector<int32_t> packed(np);
    if (kept) MOE_HIP(h, hipMemcpy(packed.data(), d_pairs, sizeof(int32_t) * kept, hipMemcpyDeviceToHost));
    for (int i = 0; i < np; ++i) {
      pairs[2 * i] = i >= kept ? -1 : pf ? (packed[i] & 0xFFFF) : (packed[i] & 0xFF);
      pairs[2 * i + 1] = i >= kept ? -1 : pf ? (packed[i] >> 16) : ((packed[i] >> 8) & 0xFF);
    }
  }
  return MOE_OK;
}

extern "C" moe_status moe_round_layer_input(moe_round* h, int32_t layer, float* host_rows) {
  if (!h || !host_rows) return MOE_ERR_INVALID_ARG;
  if (layer < 0 || layer >= h->cfg.n_layers) return MOE_ERR_INVALID_ARG;
  if (h->last_T == 0 || h->last_T > MOE_ROUND_MAX_ROWS) return MOE_ERR_STATE;
  if (layer > 0 && h->xslots < h->cfg.n_layers - 1) return MOE_ERR_STATE;  // not recorded
  MOE_HIP(h, hipStreamSynchronize(h->stream));
  const size_t n = static_cast<size_t>(h->last_T) * h->cfg.hidden;
  const float* src = layer == 0 ? h->h_ing.hidden : h->xall + static_cast<size_t>(layer - 1) * h->xstride;
  if (layer == 0 && h->h_ing.hidden == h->h_ing.out) return MOE_ERR_STATE;  // overwritten by the round
  MOE_HIP(h, hipMemcpy(host_rows, src, sizeof(float) * n, hipMemcpyDeviceToHost));
  return MOE_OK;
}

extern "C" moe_status moe_round_swiglu_rows(moe_round* h, float* host_rows) {
  if (!h || !host_rows) return MOE_ERR_INVALID_ARG;
  if (h->last_T == 0) return MOE_ERR_STATE;
  MOE_HIP(h, hipStreamSynchronize(h->stream));
  const size_t n = static_cast<size_t>(h->last_T) * h->last_k * h->cfg.inter;
  const float* src = h->last_T > MOE_ROUND_MAX_ROWS ? h->pf_hbuf : h->hbuf;
  MOE_HIP(h, hipMemcpy(host_rows, src, sizeof(float) * n, hipMemcpyDeviceToHost));
  return MOE_OK;
}

extern "C" moe_status moe_round_last_unique(moe_round* h, int32_t* n_unique_per_layer) {
  if (!h || !n_unique_per_layer) return MOE_ERR_INVALID_ARG;
  if (h->last_T == 0) return MOE_ERR_STATE;
  MOE_HIP(h, hipStreamSynchronize(h->stream));
  MOE_HIP(h, hipMemcpy(n_unique_per_layer, h->n_unique, sizeof(int32_t) * h->cfg.n_layers, hipMemcpyDeviceToHost));
  return MOE_OK;
}

// Bytes of one expert's gate, up and down codes and scales (or super-block records) in the layout.
static int64_t expert_bytes(const moe_round_config& c) {
  const int64_t w = static_cast<int64_t>(c.hidden) * c.inter;
  const int64_t per = c.weight_format == MOE_WEIGHT_Q4S256 ? (128 + 16) : (16 + 4);  // per 256 / per 32
  const int64_t blk = c.weight_format == MOE_WEIGHT_Q4S256 ? 256 : 32;
  return 3 * w / blk * per;
}

extern "C" moe_status moe_round_last_stats(moe_round* h, moe_round_stats* stats, int32_t* n_unique,
                                           int64_t* layer_metric_bytes) {
  if (!h || !stats) return MOE_ERR_INVALID_ARG;
  if (h->last_T == 0) return MOE_ERR_STATE;
  const int L = h->cfg.n_layers;
  std::vector<int32_t> nu(L), ns(L, 0);
  MOE_HIP(h, hipStreamSynchronize(h->stream));
  MOE_HIP(h, hipMemcpy(nu.data(), h->n_unique, sizeof(int32_t) * L, hipMemcpyDeviceToHost));
  if (h->cfg.tail_skip_rank > 0 && h->last_T <= MOE_ROUND_MAX_ROWS)
    MOE_HIP(h, hipMemcpy(ns.data(), h->n_skipped, sizeof(int32_t) * L, hipMemcpyDeviceToHost));
  int32_t skipped = 0;
  for (int l = 0; l < L; ++l) skipped += ns[l];
  const int64_t eb = expert_bytes(h->cfg);
  const int64_t act = 2LL * h->last_T * h->cfg.hidden * static_cast<int64_t>(sizeof(float));
  int64_t total = 0;
  for (int l = 0; l < L; ++l) {
    const int64_t mb = nu[l] * eb + act;
    if (n_unique) n_unique[l] = nu[l];
    if (layer_metric_bytes) layer_metric_bytes[l] = mb;
    total += mb;
  }
  stats->n_layers = L;
  stats->rows = h->last_T;
  stats->top_k = h->last_k;
  stats->skipped = skipped;
  stats->expert_bytes = eb;
  stats->metric_bytes = total;
  return MOE_OK;
}

static moe_status launch_floor(moe_round* h, FloorArgs fa, int units_max, int grid_cap = 16384) {
  int grid = units_max < grid_cap ? units_max : grid_cap;
  if (grid < 1) grid = 1;
  fa.magic = 0x9E3779B9u;
  fa.sink = h->floor_sink;
  fa.chunks_per_expert = 0;
  for (int i = 0; i < fa.nr; ++i)
    fa.chunks_per_expert += static_cast<int>((fa.r[i].bytes + kFloorChunk - 1) / kFloorChunk);
  void* params[] = {&fa};
  MOE_HIP(h, hipLaunchKernel(reinterpret_cast<const void*>(floor_read_kernel), dim3(grid), dim3(kThreads), params, 0,
                             h->stream));
  return MOE_OK;
}

extern "C" moe_status moe_round_floor(moe_round* h) {
  if (!h) return MOE_ERR_INVALID_ARG;
  if (h->last_T == 0) return MOE_ERR_STATE;
  if (h->cfg.expert_table) return MOE_ERR_UNSUPPORTED;  // no common base address per layer
  const moe_round_config& c = h->cfg;
  const int64_t H = c.hidden, I = c.inter, E = c.n_experts;
  const bool pf = h->last_T > MOE_ROUND_MAX_ROWS;
  const int ucap = pf ? c.n_experts : h->Ucap;
  const int32_t* uniq = pf ? h->pf_uniq : h->uniq;
  const bool s256 = c.weight_format == MOE_WEIGHT_Q4S256;
  const int64_t smh = (s256 ? H / 64 : H / 32) * 4, smi = (s256 ? I / 64 : I / 32) * 4;  // bytes per row
  for (int l = 0; l < c.n_layers; ++l) {
    const moe_layer_weights& w = h->wts[l];
    FloorArgs r{};
    r.nr = 1;
    r.r[0] = {reinterpret_cast<const uint8_t*>(w.router_w), 0, E * H * 4};
    moe_status st = launch_floor(h, r, static_cast<int>((E * H * 4 + kFloorChunk - 1) / kFloorChunk));
    if (st != MOE_OK) return st;
    FloorArgs g{};
    g.nr = 4;
    g.r[0] = {w.gate_q, I * H / 2, I * H / 2};
    g.r[1] = {reinterpret_cast<const uint8_t*>(w.gate_sm), I * smh, I * smh};
    g.r[2] = {w.up_q, I * H / 2, I * H / 2};
    g.r[3] = {reinterpret_cast<const uint8_t*>(w.up_sm), I * smh, I * smh};
    g.uniq = uniq + static_cast<size_t>(l) * ucap;
    g.n_unique = h->n_unique + l;
    g.ucap = ucap;
    g.emax = c.n_experts - 1;
    const int cg = static_cast<int>(2 * ((I * H / 2 + kFloorChunk - 1) / kFloorChunk + (I * smh + kFloorChunk - 1) / kFloorChunk));
    st = launch_floor(h, g, ucap * cg);
    if (st != MOE_OK) return st;
    FloorArgs d{};
    d.nr = 2;
    d.r[0] = {w.down_q, H * I / 2, H * I / 2};
    d.r[1] = {reinterpret_cast<const uint8_t*>(w.down_sm), H * smi, H * smi};
    d.uniq = g.uniq;
    d.n_unique = g.n_unique;
    d.ucap = ucap;
    d.emax = c.n_experts - 1;
    const int cd = static_cast<int>((H * I / 2 + kFloorChunk - 1) / kFloorChunk + (H * smi + kFloorChunk - 1) / kFloorChunk);
    st = launch_floor(h, d, ucap * cd);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

extern "C" moe_status moe_round_stream_read(moe_round* h, const void* buf, int64_t bytes) {
  if (!h || !buf || bytes < 16 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15u)) return MOE_ERR_INVALID_ARG;
  FloorArgs f{};
  f.nr = 1;
  f.r[0] = {static_cast<const uint8_t*>(buf), 0, bytes};
  const int64_t chunks = (bytes + kFloorChunk - 1) / kFloorChunk;
  return launch_floor(h, f, static_cast<int>(chunks < (1 << 20) ? chunks : (1 << 20)), 1 << 20);
}

// One wave per block: an optional fixed sleep (so that all blocks end together), then an optional
// store of the block index. Bounded, no wait on any other block.
static __global__ void __launch_bounds__(64) empty_kernel(int sleep_units, int32_t* __restrict__ flags) {
  for (int i = 0; i < sleep_units; ++i) __builtin_amdgcn_s_sleep(32);
  if (flags && threadIdx.x == 0) flags[blockIdx.x] = static_cast<int32_t>(blockIdx.x);
}

extern "C" moe_status moe_round_empty_launches(moe_round* h, int32_t blocks, int32_t launches,
                                               int32_t sleep_units, int32_t* flags) {
  if (!h || blocks < 1 || blocks > 65536 || launches < 1 || launches > 1024) return MOE_ERR_INVALID_ARG;
  if (sleep_units < 0 || sleep_units > 64) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(flags) & 3u) return MOE_ERR_INVALID_ARG;
  int su = sleep_units;
  void* params[] = {&su, &flags};
  for (int i = 0; i < launches; ++i)
    MOE_HIP(h, hipLaunchKernel(reinterpret_cast<const void*>(empty_kernel), dim3(blocks), dim3(64), params, 0,
                               h->stream));
  return MOE_OK;
}

// ------------------------------------------------------------------------------------------
// The no-allocation entry point: a decode/verify round whose scratch lives in a fixed device array
// ------------------------------------------------------------------------------------------

// Scratch of moe_round_run_noalloc: one array per device, alive until the process ends. Host code
// never uses this name as an address (on the host it is only a stand-in for the symbol); the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kNoAllocScratchBytes = MOE_ROUND_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static std::atomic<unsigned char*> g_scratch_ptr[kMaxDevices];

static moe_status noalloc_scratch(int dev, unsigned char** out, int32_t* hip_err) {
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  unsigned char* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {  // first call on this device (the device is current): look the symbol up once
    void* addr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !addr) {
      *hip_err = static_cast<int32_t>(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return MOE_ERR_HIP;
    }
    p = static_cast<unsigned char*>(addr);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return MOE_OK;
}

// Carve the round's scratch out of `base` (or, with base null, only count it): returns the bytes.
static size_t noalloc_layout(moe_round* h, int T, unsigned char* base) {
  const moe_round_config& c = h->cfg;
  const size_t L = c.n_layers, H = c.hidden, I = c.inter, E = c.n_experts;
  size_t off = 0;
  auto take = [&](size_t bytes) -> unsigned char* {
    off = (off + 255) & ~size_t(255);
    unsigned char* q = base ? base + off : nullptr;
    off += bytes;
    return q;
  };
  const size_t P = h->Pcap, U = h->Ucap, It = h->Icap;
  h->xslots = (c.record_layers && L > 2) ? static_cast<int>(L) - 1 : 2;
  h->xstride = static_cast<int>(T * H);
  h->xall = reinterpret_cast<float*>(L > 1 ? take(sizeof(float) * h->xslots * T * H) : nullptr);
  h->logits = reinterpret_cast<double*>(take(sizeof(double) * T * E));
  h->n_unique = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * L));
  h->uniq = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * L * U));
  h->offs = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * L * (U + 1)));
  h->pairs = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * L * P));
  h->pair_w = reinterpret_cast<float*>(take(sizeof(float) * L * P));
  h->rec = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * L * It * kRecWords));
  h->hbuf = reinterpret_cast<float*>(take(sizeof(float) * P * I));
  h->slot_of = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * L * P));
  h->tsel = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * P));
  h->tp = reinterpret_cast<float*>(take(sizeof(float) * P));
  h->ybuf = reinterpret_cast<float*>(c.exact ? take(sizeof(float) * P * H) : nullptr);
  h->xq = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * T * (H / 32) * kXqWords));
  h->xss = reinterpret_cast<float2*>(take(sizeof(float2) * T * (H / 32)));
  return off;
}

extern "C" moe_status moe_round_run_noalloc(const moe_round_config* cfg, const moe_layer_weights* layers,
                                            const float* hidden, int32_t T, int32_t k, float* out,
                                            int32_t* expert_ids, float* route_w, void* stream,
                                            int32_t* hip_error) {
  if (hip_error) *hip_error = 0;
  moe_status st = validate_config(cfg);
  if (st != MOE_OK) return st;
  st = validate_layers(cfg, layers);
  if (st != MOE_OK) return st;
  st = validate_run(cfg, hidden, T, k, out, expert_ids, route_w);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (T > MOE_ROUND_MAX_ROWS) return MOE_ERR_UNSUPPORTED;  // prefill rounds need handle scratch
  if (cfg->expert_table || cfg->tail_skip_rank) return MOE_ERR_UNSUPPORTED;  // no handle to bind a table to
  // A handle on the stack over the fixed array: nothing here allocates, on the host or the device.
  moe_round h;
  h.cfg = *cfg;
  h.stream = static_cast<hipStream_t>(stream);
  split_blocks(cfg->hidden, &h.Gh, &h.NBh);
  split_blocks(cfg->inter, &h.Gi, &h.NBi);
  h.Pcap = T * k;
  h.Ucap = (T * k < cfg->n_experts) ? T * k : cfg->n_experts;
  h.Icap = T * k;
  if (cfg->fused_max_rows != 0) h.fused_max_rows = cfg->fused_max_rows < 0 ? 0 : cfg->fused_max_rows;
  h.rows_per_item = cfg->rows_per_item;
  if (cfg->mfma_min_rows != 0) h.mfma_rows = cfg->mfma_min_rows < 0 ? 0 : cfg->mfma_min_rows;
  if (noalloc_layout(&h, T, nullptr) > kNoAllocScratchBytes) return MOE_ERR_UNSUPPORTED;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    if (hip_error) *hip_error = static_cast<int32_t>(e);
    return MOE_ERR_HIP;
  }
  unsigned char* base = nullptr;
  int32_t herr = 0;
  st = noalloc_scratch(dev, &base, &herr);
  if (st != MOE_OK) {
    if (hip_error) *hip_error = herr;
    return st;
  }
  noalloc_layout(&h, T, base);
  h.h_ing = Ingress{hidden, out, expert_ids, route_w};
  h.wts = layers;
  st = launch_eager(&h, T, k, nullptr);
  if (hip_error) *hip_error = h.last_hip;
  return st;
}

extern "C" int32_t moe_round_last_hip_error(const moe_round* h) { return h ? h->last_hip : 0; }

extern "C" void moe_round_destroy(moe_round* h) { free_handle(h); }
