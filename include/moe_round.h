/*
 * moe_round.h — C ABI of the MI355X (gfx950) MoE decode/verify round.
 *
 * One call evaluates the mixture-of-experts feed-forward of one decode or
 * speculative-verify round over T token rows (1 <= T <= 64) and L stacked
 * MoE layers, or of a prefill round of more rows (see max_rows: the infero
 * README, "Beyond plain text decode", routes prefill through a counting sort
 * and a GEMM per expert).  Per layer, on the GPU:
 *   router GEMV (fp32 weights and activations, fp64 accumulation) -> top-k
 *   per row -> softmax over the k selected logits -> union of the rows'
 *   experts as a deterministic worklist -> fused dequant-GEMV of the unique
 *   experts' 4-bit gate/up weights with SwiGLU -> dequant-GEMV of their
 *   down weights with the routing-weighted scatter-add back into each row.
 *
 * The pages this follows:
 *   - "How AlphaInfer makes local decoding fast", section 2 (One captured
 *     graph per decode round): a round is one forward pass over 1-8 rows,
 *     recorded once as a graph and replayed; per-request data, including
 *     which expert lives where, is ingress written into fixed buffers, and
 *     the graph is never rebuilt.  Section 3.1: each extra verified row
 *     routes to experts the other rows did not need, so it adds weight bytes.
 *   - infero README, "Beyond plain text decode" (MoE bullet): top-k routing
 *     at decode, counting sort of (row, expert) pairs into per-expert work.
 *   - infero README, "Layout" figure: expert = silu(W_g x) * (W_u x) -> W_d.
 *   - infero README, "Design notes": block-encoded weights are consumed in
 *     place, never dequantised into memory; activations stay fp32.
 *   - infero README, "Status" (tensor parallelism): unsupported requests are
 *     refused outright rather than mishandled.
 *
 * Weight format (one matrix W[rows][K], K = reduction length, K % 32 == 0):
 *   codes    uint8  [rows][K/2]  byte j holds element 2j in bits 0-3 and
 *                                element 2j+1 in bits 4-7; 16-byte aligned
 *   scalemin uint32 [rows][K/32] bits 0-15: fp16 scale s, bits 16-31: fp16
 *                                minimum m; weight = s*q + m, q in 0..15
 *                                (MOE_WEIGHT_Q4B32, the default)
 *   or, with weight_format MOE_WEIGHT_Q4S256 (K % 256 == 0), the same codes and
 *   superblk uint32 [rows][K/256][4], one 16-byte record per 256 weights:
 *                                word 0 bits 0-15 fp16 d, bits 16-31 fp16
 *                                dmin; words 1-3 a little-endian 96-bit
 *                                string, bits 12j..12j+11 = sub-block j's
 *                                6-bit scale sc_j (low) and 6-bit minimum m_j
 *                                (high); a weight of the 32-weight sub-block
 *                                j is d*sc_j*q - dmin*m_j (4.5 bits per
 *                                weight: the 256-element super-block with a
 *                                packed twelve-byte scale/minimum field of
 *                                the infero README, "Supported weight
 *                                encodings" and "AWQ, FP8, and NVFP4
 *                                checkpoints")
 *   gate, up: [E][I][H] (K = H); down: [E][H][I] (K = I).
 *   router: fp32 [E][H], optional fp32 bias [E].
 *
 * Memory: every pointer argument except `cfg`, `layers` and the host
 * outputs of the introspection calls is DEVICE memory on the current HIP
 * device.  Weights are caller-owned and borrowed: they must stay valid until
 * the handle is destroyed or a later run names other weights.  The handle
 * owns only its scratch.
 *
 * Errors: every call returns a moe_status; nothing aborts, prints or
 * throws.  A rejected call leaves the handle unchanged.  After MOE_ERR_HIP
 * the failing hipError_t is kept and returned by moe_round_last_hip_error.
 *
 * Threading: a handle is not re-entrant; use one handle per stream.
 */
#ifndef MOE_ROUND_H
#define MOE_ROUND_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ROUND_ABI_VERSION 3

#if defined(__GNUC__) || defined(__clang__)
#define MOE_ROUND_API __attribute__((visibility("default")))
#else
#define MOE_ROUND_API
#endif

/* Supported set (outside it, init refuses with MOE_ERR_UNSUPPORTED): H a multiple of 256 up to
 * 8192; I a multiple of 32 up to 8192 (a multiple of 256 with MOE_WEIGHT_Q4S256, of 128 when
 * max_rows exceeds 64); E up to 512; k up to min(E, 16); T up to 64 (decode/verify) or 16384
 * (prefill).  A reduction length K (H for gate/up, I for down) is split over G lanes per weight row
 * and NB 32-weight blocks per lane (G in 4..64, NB in 1..4); when K/32 has no exact split the
 * spare block slots are masked, so e.g. I = 64 (an 8-way tensor-parallel shard of I = 512) runs. */
#define MOE_ROUND_MAX_ROWS 64      /* T_max of decode/verify rounds                     */
#define MOE_ROUND_MAX_PREFILL_ROWS 16384 /* T_max with the prefill path (see max_rows) */
#define MOE_ROUND_MAX_EXPERTS 512  /* E     */
#define MOE_ROUND_MAX_TOPK 16      /* k     */

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG -1  /* null/misaligned pointer, bad size, overlap   */
#define MOE_ERR_UNSUPPORTED -2  /* a shape outside the supported set            */
#define MOE_ERR_HIP -3          /* a HIP runtime call failed                    */
#define MOE_ERR_OOM -4          /* scratch allocation failed                    */
#define MOE_ERR_STATE -5        /* call out of order (e.g. worklist before run) */

typedef struct moe_round_config {
  int32_t abi_version; /* must equal MOE_ROUND_ABI_VERSION                        */
  int32_t hidden;      /* H: multiple of 256, at most 8192                       */
  int32_t inter;       /* I: multiple of 32, at most 8192                        */
  int32_t n_experts;   /* E: 1..512                                               */
  int32_t top_k_max;   /* largest k a run may ask for: 1..min(E, 16)              */
  int32_t n_layers;    /* L >= 1                                                  */
  int32_t max_rows;    /* T_max: 1..MOE_ROUND_MAX_PREFILL_ROWS. Rounds of up to 64 rows
                          are decode/verify rounds; rounds of more rows take the prefill
                          path: per layer, a counting sort of the (row, rank) pairs into
                          work items of up to 64 pairs of one expert, then gate/up and
                          down as fp16 matrix-core GEMMs over each item (each activation
                          row scaled by a power of two and split into two fp16 values,
                          22 significant bits; block scales folded in fp32), and a
                          combine in rank order (so a row's output never
                          depends on the other rows). Prefill rounds launch eagerly
                          (use_graph applies to rounds of up to 64 rows), ignore the
                          launch-shape fields and `exact` (their combine is always the
                          fixed-order one) and read either weight format. Their scratch
                          grows with max_rows * top_k_max * (4 H + 16 I) bytes.        */
  int32_t residual;    /* 0: out = MoE(x), needs L == 1; 1: x_{l+1} = x_l + MoE_l */
  int32_t use_graph;   /* 1: replay one captured hipGraph per (T, k); 0: eager    */
  /* Launch-shape choices (0 = the default for each; none changes results beyond fp32 rounding
   * order):                                                                               */
  int32_t fused_max_rows; /* rounds of up to this many rows fold the selection into the
                             gate/up kernel; default 15, -1 = never, at most 15            */
  int32_t rows_per_item;  /* rows of one expert per GEMV work item; default 1 for rounds of
                             up to 10 rows, 2 up to 32 rows, 4 from 33 rows; 1..64         */
  int32_t mfma_min_rows;  /* rounds of 16+ rows: work items with at least this many rows
                             use the int8 matrix-core tiles of gate/up (H = 2048) and down
                             (I = 512); default -1 = never (the integer-dot GEMVs measured
                             faster at the rows per expert wide verify rounds produce),
                             1..64 = from that many rows                                    */
  int32_t exact;          /* 1: fixed-order combine. The down stage stores each (row, rank)
                             product W_d h and a combine kernel adds them to the residual in
                             rank order: results are bitwise reproducible, and a row's output
                             does not depend on the other rows of the round or on T. (The
                             matrix-core tile is not used.) 0: fp32 atomics (faster).       */
  int32_t weight_format;  /* layout of the expert weights' scales and minima (the codes are the
                             same in both; see moe_layer_weights):
                             MOE_WEIGHT_Q4B32 (0): one word per 32-weight block, 0.625 B/weight;
                             MOE_WEIGHT_Q4S256 (1): one 16-byte record per 256-weight
                             super-block, 0.5625 B/weight; needs I a multiple of 256 (H always
                             is), else init returns MOE_ERR_UNSUPPORTED. The matrix-core tile
                             is used with MOE_WEIGHT_Q4B32 only.                            */
  int32_t prefetch;       /* 1: overlap independent reads across the layer's kernels: each gate/up
                             block touches the down rows the down block with the same index will
                             read, and each down block the next layer's router row of the logits
                             block with its index (no extra HBM bytes, results unchanged); 0
                             (default): off (measured slower: the touches queue behind the
                             weight loads in each CU's load path)                          */
  int32_t record_layers;  /* 1: keep every layer's input of decode/verify rounds (L - 1 buffers of
                             max_rows x H floats instead of two reused ones), readable with
                             moe_round_layer_input, for checking each layer on its own input
                             ("How AlphaInfer makes local decoding fast", section 4: a
                             teacher-forced comparator); 0 (default): no                    */
  int32_t expert_table;   /* 1: every expert's weights are read through a per-(layer, expert) table
                             of pointers (moe_expert_ref, bound with moe_round_bind_experts), so
                             each expert may sit at any address: in device memory or in pinned
                             host memory (hipHostMalloc) that the kernels read in place over the
                             host link.  The layers' expert pointers must then be NULL (only the
                             router is taken from them).  Costs one dependent load of the
                             expert's table entry per kernel that reads its weights.  Rounds of
                             up to 64 rows only (init refuses it with max_rows > 64).
                             "How AlphaInfer makes local decoding fast", "Fused-infer: three
                             memory tiers as one expert store" (decode reads each routed expert
                             through a table; residency is per-request data).  0 (default): the
                             layers' contiguous [E][..] arrays                                */
  int32_t tail_skip_rank; /* r > 0: a round skips each missed expert (its residency bit clear, see
                             moe_round_bind_experts) that every row selecting it ranks at r or
                             below (rank = 1-based position in the row's descending top-k); its
                             (row, rank) pairs add nothing and the other pairs keep their routing
                             weights (no renormalisation).  An approximation: results differ from
                             the plain round by the skipped terms.  Avalon README, results section
                             (rank 7 or lower, on by default there).  0 (default): off.  At most
                             MOE_ROUND_MAX_TOPK + 1; rounds of up to 64 rows only           */
} moe_round_config;

#define MOE_WEIGHT_Q4B32 0
#define MOE_WEIGHT_Q4S256 1

/* One layer's weights (device pointers, caller-owned). router_bias may be NULL. */
typedef struct moe_layer_weights {
  const float* router_w;     /* [E][H]                 */
  const float* router_bias;  /* [E] or NULL            */
  const uint8_t* gate_q;     /* [E][I][H/2]            */
  const uint32_t* gate_sm;   /* [E][I][H/32]  (Q4S256: [E][I][H/256][4]) */
  const uint8_t* up_q;       /* [E][I][H/2]            */
  const uint32_t* up_sm;     /* [E][I][H/32]  (Q4S256: [E][I][H/256][4]) */
  const uint8_t* down_q;     /* [E][H][I/2]            */
  const uint32_t* down_sm;   /* [E][H][I/32]  (Q4S256: [E][H][I/256][4]) */
} moe_layer_weights;

/* One expert's weights for the table mode (expert_table = 1): device-readable pointers to its own
 * matrices, gate and up [I][H] (K = H), down [H][I] (K = I), in the layout above; codes 16-byte
 * aligned, scales 4-byte (Q4S256: 16-byte).  48 bytes; the table is an array [L][E] of these. */
typedef struct moe_expert_ref {
  const uint8_t* gate_q;
  const uint32_t* gate_sm;
  const uint8_t* up_q;
  const uint32_t* up_sm;
  const uint8_t* down_q;
  const uint32_t* down_sm;
} moe_expert_ref;

typedef struct moe_round moe_round; /* opaque handle */

/* Pure host check of a configuration; touches no GPU. MOE_OK if init would accept its shape.
 * Refusing unsupported shapes instead of mishandling them: infero README, "Status" (the
 * tensor-parallel item). */
MOE_ROUND_API moe_status moe_round_validate_config(const moe_round_config* cfg);

/*
 * Create a handle: validates cfg and layers[0..L-1] (host array of structs holding device
 * pointers), allocates scratch on the current device and binds the handle to `stream`
 * (a hipStream_t; NULL = the null stream).  Graphs are captured lazily, once per (T, k).
 * Passage: "How AlphaInfer makes local decoding fast", section 2 (one captured graph per decode
 * round; its buffers are fixed once, and per-request data is written into them).
 * Errors: MOE_ERR_INVALID_ARG (null or misaligned pointer, bad field), MOE_ERR_UNSUPPORTED (shape
 * outside the supported set), MOE_ERR_OOM / MOE_ERR_HIP (allocation); *out is NULL on failure.
 */
MOE_ROUND_API moe_status moe_round_init(const moe_round_config* cfg, const moe_layer_weights* layers,
                          void* stream, moe_round** out);

/*
 * Run one round, asynchronously on the handle's stream.
 * Passages: infero README, "Beyond plain text decode" (MoE: a router picks the top-k experts per
 * row at decode and a counting sort groups the (row, expert) pairs per expert), "Layout" (the
 * expert is silu(W_g x) * (W_u x) -> W_d), "Design notes" (block weights read in place);
 * "How AlphaInfer makes local decoding fast", section 2 (per-request data, including which
 * weights to read, is ingress into fixed buffers: new pointers never rebuild a graph) and
 * section 3.1 (a verify round's rows share the experts they have in common).
 *   hidden      device fp32 [T][H] input rows; may be `out` itself (then overwritten), but must
 *               not partly overlap it
 *   T, k        0 <= T <= max_rows, 1 <= k <= top_k_max; T = 0 is an empty round: nothing is
 *               enqueued, hidden/out/expert_ids/route_w may be NULL, MOE_OK is returned and the
 *               introspection calls report MOE_ERR_STATE until the next round with rows
 *   layers      host array [L] of new weight pointers, or NULL to keep the current ones
 *               (new pointers are ingress: written into the handle's fixed table, no recapture)
 *   out         device fp32 [T][H] result: MoE(x) (residual = 0) or x_L (residual = 1)
 *   expert_ids  device int32 [L][T][k] selected experts per row, descending logit, or NULL
 *   route_w     device fp32 [L][T][k] routing weights (softmax of the selected logits), or NULL
 * Pointers must be 16-byte aligned (expert_ids, route_w: 4-byte).  Returns after enqueueing; no
 * host synchronisation.  A rejected call (MOE_ERR_INVALID_ARG) enqueues nothing and leaves the
 * handle's weights unchanged.
 */
MOE_ROUND_API moe_status moe_round_run(moe_round* h, const float* hidden, int32_t T, int32_t k,
                         const moe_layer_weights* layers, float* out, int32_t* expert_ids,
                         float* route_w);

/*
 * Bind the expert table and the residency bits that later runs read (on the GPU, when each round
 * executes: the caller may rewrite their contents between rounds, in stream order, without any call
 * here and without a graph rebuild; binding other arrays updates captured graphs in place).
 * Passages: "How AlphaInfer makes local decoding fast", "Fused-infer: three memory tiers as one
 * expert store" (each routed expert is read through a device-resolved table; a non-resident expert
 * is not copied to the GPU first) and section 2 (per-request data is ingress into fixed buffers);
 * Avalon README, results section (the tail skip applies to missed experts only).
 *   table     device moe_expert_ref [L][E], 16-byte aligned: required when cfg.expert_table = 1,
 *             must be NULL otherwise.  Every entry a round may select must name valid memory the
 *             GPU can read (device memory, or pinned host memory mapped for the device); entries
 *             of experts the tail skip leaves out are not read.
 *   resident  device uint32 [L][ceil(E/32)]: bit e % 32 of word e / 32 of layer l is 1 when expert
 *             e of layer l is resident (in device memory), 0 when it is missed.  Required when
 *             cfg.tail_skip_rank > 0, must be NULL otherwise.
 * Both are caller-owned and borrowed until the handle is destroyed or other arrays are bound.
 * Errors: MOE_ERR_INVALID_ARG (null handle, misaligned pointer, a pointer the configuration does
 * not take or a required one missing).  Runs of a handle that needs them before they are bound
 * return MOE_ERR_STATE.
 */
MOE_ROUND_API moe_status moe_round_bind_experts(moe_round* h, const moe_expert_ref* table,
                                                const uint32_t* resident);

/*
 * The device address of pinned host memory for an expert table entry (the host tier read in place):
 * `host_ptr` must lie in memory allocated with hipHostMalloc (mapped for the device); *device_ptr
 * receives the address kernels use for it.  Passage: "How AlphaInfer makes local decoding fast",
 * "Fused-infer: three memory tiers as one expert store" (experts stay where they sit in RAM instead
 * of being copied to the GPU first).  Errors: MOE_ERR_INVALID_ARG (NULL argument, or memory that is
 * not pinned host memory known to the runtime; *device_ptr is then NULL).
 */
MOE_ROUND_API moe_status moe_round_host_tier_pointer(const void* host_ptr, void** device_ptr);

/*
 * Introspection of the last run (synchronises the stream; host outputs).
 * Passage: infero README, "Beyond plain text decode" (the counting sort of (row, expert) pairs into
 * per-expert work); the worklist is that sort's result.
 *   n_unique     number of distinct experts layer `layer` touched
 *   uniq         [n_unique] those experts, ascending                   (may be NULL)
 *   offs         [n_unique + 1] exclusive prefix sum of rows per expert (may be NULL)
 *   pairs        [T*k][2] (row t, rank j) grouped by expert, t ascending (may be NULL); with the
 *                tail skip the first offs[n_unique] entries are the kept pairs and the rest -1
 * Buffers must hold at least min(T*k, E) (uniq), that + 1 (offs) and 2*T*k (pairs) entries.
 * Experts the tail skip left out are not in the worklist.
 * This and the calls below return MOE_ERR_STATE when there is no last run to report: none
 * since init, or the last one was an empty round (T = 0).
 */
MOE_ROUND_API moe_status moe_round_worklist(moe_round* h, int32_t layer, int32_t* n_unique, int32_t* uniq,
                              int32_t* offs, int32_t* pairs);

/*
 * The gate/up stage's output of the last run's last layer, silu(W_g x_t) * (W_u x_t), one fp32 row of
 * length I per (row, rank) pair in worklist order (pair slot p = the p-th entry of `pairs` above),
 * into host float [T*k][I] (synchronises the stream).  Passage: infero README, "Layout" (the
 * expert's SwiGLU) and "Design notes" (intermediates are kept comparable with a CPU reference).
 */
MOE_ROUND_API moe_status moe_round_swiglu_rows(moe_round* h, float* host_rows);

/*
 * The input rows of layer `layer` in the last decode/verify run, into host float [T][H] (synchronises
 * the stream): layer 0's is the caller's `hidden`; later layers' need record_layers = 1.  Passage:
 * "How AlphaInfer makes local decoding fast", section 4 (a teacher-forced comparator checks each
 * layer on the input the engine actually fed it).  Errors: MOE_ERR_INVALID_ARG (bad handle, layer
 * or buffer), MOE_ERR_STATE (no last decode/verify run; the layer's input was not kept; or, for
 * layer 0, `hidden` was `out` and has been overwritten).
 */
MOE_ROUND_API moe_status moe_round_layer_input(moe_round* h, int32_t layer, float* host_rows);

/* n_unique of every layer of the last run into host int32 [L] (synchronises the stream).
 * Passage: "How AlphaInfer makes local decoding fast", section 3.1 (an extra verified row costs
 * the experts only it routes to). */
MOE_ROUND_API moe_status moe_round_last_unique(moe_round* h, int32_t* n_unique_per_layer);

/* What the last run moved (host outputs; synchronises the stream). */
typedef struct moe_round_stats {
  int32_t n_layers;       /* L                                                          */
  int32_t rows;           /* T of the last run                                          */
  int32_t top_k;          /* k of the last run                                          */
  int32_t skipped;        /* experts the tail skip left out, summed over layers (0 off)  */
  int64_t expert_bytes;   /* bytes of one expert's gate, up and down codes and scales    */
  int64_t metric_bytes;   /* sum over layers of n_unique * expert_bytes + 2 * T * H * 4
                             (n_unique counts the experts read: skipped ones excluded)   */
} moe_round_stats;

/*
 * Per-layer statistics of the last run: the unique experts each layer read (n_unique, host int32
 * [L] or NULL) and each layer's metric bytes (host int64 [L] or NULL): the unique experts' weight
 * bytes (codes and scales) plus the T input and T output rows.  Passages: "How AlphaInfer makes
 * local decoding fast", section 3.1 (the price of a verified row is the bytes of the experts only it
 * needs); infero README, "CPU offload" (a decode step's rate read as bytes moved per second).
 * Errors: MOE_ERR_INVALID_ARG (h or stats NULL), MOE_ERR_STATE (no last run).
 */
MOE_ROUND_API moe_status moe_round_last_stats(moe_round* h, moe_round_stats* stats, int32_t* n_unique,
                                int64_t* layer_metric_bytes);

/*
 * The byte floor of the last run, enqueued on the handle's stream (asynchronous): per layer three
 * launches that only read, at the last run's addresses, the router matrix, the gate and up codes and
 * scales of the layer's unique experts, and their down codes and scales, and do no arithmetic beyond
 * folding the loaded words together.  Timing it beside the round splits the round's time into what
 * moving its bytes with that many launches costs and what the rest (routing, arithmetic) adds.
 * Passage: infero README, "Where the time goes" (a decode-floor program that replays exactly the
 * matrix-vector reads of a step, as the floor a step cannot beat).  Reads the worklist the last run
 * left in device memory, so the weights it names must still be valid.
 * Errors: MOE_ERR_INVALID_ARG (h NULL), MOE_ERR_STATE (no last run), MOE_ERR_UNSUPPORTED (a handle
 * with expert_table = 1: its experts have no common base address), MOE_ERR_HIP (launch).
 */
MOE_ROUND_API moe_status moe_round_floor(moe_round* h);

/*
 * A control measurement: one launch of the byte floor's read kernel over `bytes` contiguous bytes at
 * device address `buf` (16-byte aligned, bytes a positive multiple of 16), on the handle's stream.
 * Passage: "How AlphaInfer makes local decoding fast", section 7, rule 2 (always run a same-session
 * control arm).  Errors: MOE_ERR_INVALID_ARG (bad pointer or size), MOE_ERR_HIP (launch).
 */
MOE_ROUND_API moe_status moe_round_stream_read(moe_round* h, const void* buf, int64_t bytes);

/*
 * A control measurement of launch costs: `launches` kernels of `blocks` minimal blocks (one wave of
 * 64 threads each) back to back on the handle's stream (asynchronous). Each wave first sleeps
 * `sleep_units` times about 2048 shader clocks (0 = not at all), so that the blocks of one kernel
 * end together; then, when `flags` is not NULL, its first lane stores the block index to
 * flags[block] (a device buffer of at least `blocks` int32, written, never read). Timed beside the
 * round it shows what a kernel boundary costs by itself and how that grows with the blocks of the
 * kernel before it, with and without stores. Passage: "How AlphaInfer makes local decoding fast",
 * section 7, rule 2 (a same-session control arm).
 * Errors: MOE_ERR_INVALID_ARG (h NULL, blocks outside 1..65536, launches outside 1..1024,
 * sleep_units outside 0..64, flags not 4-byte aligned), MOE_ERR_HIP (launch).
 */
MOE_ROUND_API moe_status moe_round_empty_launches(moe_round* h, int32_t blocks, int32_t launches,
                                                  int32_t sleep_units, int32_t* flags);

/*
 * Kernel timing, for measurement ("How AlphaInfer makes local decoding fast", section 7: time
 * uninstrumented, decompose before crediting; the per-kernel times here come from events the runtime
 * stamps with each dispatch's own start and end).  moe_round_profile(h, 1) makes every following run launch its
 * kernels eagerly (also on a graph handle: graph nodes carry no events) with a start/stop event
 * pair per kernel that the runtime stamps with the dispatch's own start and end times, so each
 * duration is the kernel's execution alone, without the launch gap before it.  The events form a
 * ring per handle; a slot is read back (waiting for its run) before it is reused, so profiling
 * costs no host synchronisation until the ring wraps.  moe_round_profile(h, 0) reads back what is
 * outstanding and returns to normal launches; the sums are kept for a later read.
 * Returns MOE_ERR_INVALID_ARG for enable outside {0, 1}; MOE_ERR_HIP if events cannot be created.
 */
MOE_ROUND_API moe_status moe_round_profile(moe_round* h, int32_t enable);

/*
 * Sum of the per-kernel durations (milliseconds) of the runs profiled since profiling was
 * enabled or last read, into host double [L][5] (router logits, selection + worklist, gate/up,
 * down, combine; a kind a round does not launch stays 0), and their number of runs into *n_runs;
 * then resets both.  Synchronises on the
 * outstanding events.  MOE_ERR_STATE if profiling was never enabled on this handle.
 */
MOE_ROUND_API moe_status moe_round_profile_read(moe_round* h, double* kernel_ms, int32_t* n_runs);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): one decode/verify round exactly like moe_round_run on a handle made from
 * cfg and layers, eager, with no handle and no allocation.  Its scratch is a fixed device array of
 * MOE_ROUND_NOALLOC_SCRATCH_BYTES per device, held until the process ends; the library looks up its
 * device address on the first call on each device (that device must be current).
 *   cfg, layers  as for moe_round_init (use_graph is ignored: the launches are eager; expert_table
 *                and tail_skip_rank must be 0: there is no handle to bind a table to)
 *   hidden .. route_w, T, k   as for moe_round_run (T <= min(max_rows, 64): no prefill rounds)
 *   stream       the hipStream_t to enqueue on (NULL = the null stream)
 *   hip_error    if not NULL, the hipError_t (as int) behind a MOE_ERR_HIP, else 0
 * Returns MOE_ERR_UNSUPPORTED when the round's scratch (about T*k*(I + H*exact)*4 bytes plus the
 * per-layer worklists) exceeds MOE_ROUND_NOALLOC_SCRATCH_BYTES; every other error as moe_round_run.
 * No scratch word needs to start at zero: every word a kernel reads is written earlier in the same
 * call.  Calls on one device share the array: calls that overlap in time on one device (on
 * different streams, or from different host threads) race and give wrong results; serialise them.
 */
#define MOE_ROUND_NOALLOC_SCRATCH_BYTES (16u << 20)
MOE_ROUND_API moe_status moe_round_run_noalloc(const moe_round_config* cfg, const moe_layer_weights* layers,
                                 const float* hidden, int32_t T, int32_t k, float* out,
                                 int32_t* expert_ids, float* route_w, void* stream, int32_t* hip_error);

/* The hipError_t (as int) of the last MOE_ERR_HIP on this handle, 0 if none. */
MOE_ROUND_API int32_t moe_round_last_hip_error(const moe_round* h);

/* A static, human-readable description of a status code. */
MOE_ROUND_API const char* moe_round_strerror(moe_status s);

/* Free the handle's scratch and graphs. NULL is a no-op. Synchronises the handle's stream. */
MOE_ROUND_API void moe_round_destroy(moe_round* h);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUND_H */
