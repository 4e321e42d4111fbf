/*
 * mk.h -- C ABI of the persistent tile-instruction decode megakernel for MI355X (gfx950).
 *
 * The library lowers a decode workload into tile instructions, queues them per worker and
 * runs them either inside one persistent kernel (one worker block per compute unit) or as
 * one standalone kernel per op inside a hipGraph.  This follows the MegaRTP page
 * ("Kernel-Mega-PDL", section 4): a host-built instruction tensor, event counters with
 * thresholds, and an operand pointer table that keeps addresses out of the instructions,
 * so that new tensor addresses only rebind the table.
 *
 * Conventions
 *   - Every entry point returns mk_status; nothing throws across the ABI.  On failure
 *     mk_last_error() returns a thread-local message.
 *   - Device pointers are plain addresses of caller-owned device memory (allocated by the
 *     caller, e.g. through PyTorch).  Host pointers are marked host_.  The library owns the
 *     plan and everything it allocates (device queue, counters, pointer tables, RoPE table,
 *     captured graphs); mk_plan_destroy frees them.
 *   - Work is enqueued on the caller's HIP stream (hipStream_t passed as void*); the graph
 *     baseline forks internal streams from it with events and joins back.
 *   - Layouts are row-major.  Weight matrices are [N, K] with K contiguous, stacked on a
 *     leading layer axis for multi-layer workloads.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MK_OK = 0,
  MK_ERR_INVALID = -1,     /* bad argument, shape or alignment: nothing was launched */
  MK_ERR_UNSUPPORTED = -2, /* valid but not built in this library (e.g. workload variant) */
  MK_ERR_HIP = -3,         /* a HIP runtime call failed */
  MK_ERR_NOMEM = -4,       /* library-side allocation failed */
  MK_ERR_TIMEOUT = -5      /* device watchdog: a counter wait did not complete */
} mk_status;

typedef enum {
  MK_QWEN3_LAYER = 0,   /* one Qwen3-shaped decode layer, returns (y, r2) */
  MK_QWEN3_STEP = 1,    /* num_layers chained layers + final RMSNorm + lm_head + greedy argmax */
  MK_INDEXER_FRONT = 2  /* A0 -> {B0, C0, B1} -> D1 -> E1 indexer front (MegaRTP page, section 4),
                           optionally with the main-MLA query half D0 -> D2 (mk_config.mla_heads) and
                           the per-token top-k of the scores (mk_config.topk) */
} mk_workload;

enum {
  MK_FLAG_NO_PREFETCH = 1u << 0, /* megakernel: no weight prefetch across instructions (ablation) */
  MK_FLAG_NOOP_ONLY = 1u << 1,   /* megakernel: run the queue with every op body skipped: the waits,
                                    stagings and output stores remain, weights are not read */
  MK_FLAG_TRACE = 1u << 2,       /* megakernel: record per-instruction timestamps */
  MK_FLAG_DEBUG_GATHER = 1u << 3, /* both modes: record the physical cache slot of every K / V row and indexer
                                    key the run gathers through the block table (mk_read_gather) */
  MK_FLAG_DEBUG_SHORT_WATCHDOG = 1u << 4 /* megakernel: a wait that is not met at its first check expires
                                    (10 ns instead of 2 s), to exercise the watchdog and abort path */
};

/* mk_config.tile_params entries.  Rows per task of the single-token (M = 1) projections: QKV a power
 * of two <= head_dim; O and down a divisor of hidden, <= 128; gate/up an even divisor of inter; each
 * within one 64 KiB LDS lease with the norm gain.  lm_head (decode step): rows per task, >= 1 (task j
 * takes the rows j, j + n, ... of n tasks).  Attention split: tokens per split-KV task, a power of two
 * in 4 .. 128 (both op families).  The multi-row projections' 64-row tiles and the indexer front's
 * tiles are fixed: their row entries and every entry of an indexer plan must be 0. */
#define MK_TILE_PARAMS 8
enum { MK_TP_ROWS_QKV = 0, MK_TP_ROWS_O = 1, MK_TP_ROWS_GATEUP = 2, MK_TP_ROWS_DOWN = 3, MK_TP_ROWS_LMHEAD = 4,
       MK_TP_SPLIT_TOKENS = 5 /* 6, 7: reserved, 0 */ };

/* Plain data, caller-owned, copied by mk_build_queue. */
typedef struct {
  int32_t workload;            /* mk_workload */
  int32_t weight_fp8, act_fp8; /* FP8 e4m3 weights with 128x128 fp32 block scales / FP8 activations */
  int32_t hidden, inter, n_q_heads, n_kv_heads, head_dim, num_layers, vocab;
  int32_t n_requests, tokens_per_request; /* M = n_requests * tokens_per_request rows */
  int32_t page_size, max_pages_per_req, num_phys_pages;
  int32_t idx_q_rank, idx_heads, idx_head_dim;
  float rms_eps, rope_theta;
  int32_t num_workers; /* 0 => one worker per compute unit of the current device */
  uint32_t flags;      /* MK_FLAG_* */
  int32_t topk;        /* MK_INDEXER_FRONT: positions each token selects after the score (0: none,
                          else 1 .. 8192 keys per row); 0 for the other workloads */
  int32_t mla_heads;   /* MK_INDEXER_FRONT: heads of the main-MLA query half (D0 Main-Q -> D2 Q-BMM,
                          128 no-RoPE dims and a 512-wide latent per head); 0: the indexer half only */
  int32_t rotary_dim;  /* dims of a head the RoPE rotates: 0 or the head dim (head_dim, idx_head_dim):
                          the whole head; any other value is refused with MK_ERR_UNSUPPORTED */
  int32_t tile_params[MK_TILE_PARAMS]; /* tile sizes of the plan, MK_TP_* above; 0 lets the planner
                          choose (its rules: the queue specification of the design notes); a value
                          the op bodies cannot run is refused with MK_ERR_UNSUPPORTED */
} mk_config;

/* Device addresses in a fixed order per workload (MK_T_* below); n = number used. */
#define MK_MAX_TENSORS 32
typedef struct {
  uint64_t ptr[MK_MAX_TENSORS];
  int32_t n;
} mk_tensors;

/* Tensor order for MK_QWEN3_LAYER / MK_QWEN3_STEP (L = num_layers, M rows, d = head_dim):
 *   W_QKV   [L, (Hq+2Hkv)d, H] bf16      W_O     [L, H, Hq d] bf16
 *   W_GU    [L, 2I, H] bf16 (rows [0,I) gate, [I,2I) up)     W_DOWN [L, H, I] bf16
 *   G_ATTN, G_MLP [L, H] bf16;  G_Q, G_K [L, d] bf16  (RMSNorm gains)
 *   K_CACHE, V_CACHE [L, pages, P, Hkv, d] bf16 (updated in place at slot ctx-1 of each request)
 *   BLOCK_TABLE [R, max_pages_per_req] int32;  CONTEXT_LENS [R] int32 (include the new token)
 *   X [M, H] bf16;  R_IN [M, H] fp32 (residual stream)
 *   Y_OUT [M, H] bf16;  R2_OUT [M, H] fp32       (layer workload outputs; for the step: last layer)
 *   WORKSPACE  mk_plan_workspace_bytes() bytes, 256-byte aligned, contents need not be preserved
 *   step only: G_FINAL [H] bf16; W_LM [V, H] bf16; LOGITS_OUT [M, V] fp32; TOKEN_OUT [M] int32
 *     (layer workloads leave these four entries 0)
 *   FP8 weights (weight_fp8 = act_fp8 = 1) only: W_QKV, W_O, W_GU, W_DOWN hold e4m3 codes (OCP
 *     E4M3FN, one byte per weight, same [N, K] layout) and S_QKV, S_O, S_GU, S_DOWN their fp32
 *     scales per 128 x 128 block, [L, ceil(N/128), ceil(K/128)] row-major: weight = code * scale */
enum {
  MK_T_W_QKV = 0, MK_T_W_O, MK_T_W_GU, MK_T_W_DOWN,
  MK_T_G_ATTN, MK_T_G_MLP, MK_T_G_Q, MK_T_G_K,
  MK_T_K_CACHE, MK_T_V_CACHE, MK_T_BLOCK_TABLE, MK_T_CONTEXT_LENS,
  MK_T_X, MK_T_R_IN, MK_T_Y_OUT, MK_T_R2_OUT, MK_T_WORKSPACE,
  MK_T_G_FINAL, MK_T_W_LM, MK_T_LOGITS_OUT, MK_T_TOKEN_OUT,
  MK_T_S_QKV, MK_T_S_O, MK_T_S_GU, MK_T_S_DOWN,
  MK_T_COUNT_QWEN3
};

/* Tensor order for MK_INDEXER_FRONT (M = n_requests x tokens_per_request rows, request r's rows
 * r T .. r T + T - 1 are its T new tokens at positions ctx_r - T .. ctx_r - 1; qr = idx_q_rank,
 * nh = idx_heads, hd = idx_head_dim = 128; e4m3 = OCP E4M3FN code bytes, scales fp32 per 128 x 128
 * block [ceil(N/128), ceil(K/128)]):
 *   W_QA [qr, H] e4m3 + S_QA;  W_W [nh, H] e4m3 + S_W;  W_K [hd, H] e4m3 + S_K;
 *   W_QI [nh hd, qr] e4m3 + S_QI          (rows h hd .. h hd + hd - 1 are head h)
 *   G_NORM [H] bf16;  G_QA [qr] bf16    (RMSNorm gains)
 *   KEY_CACHE [pages, P, hd] e4m3;  KEY_SCALE [pages, P] fp32  (written in place at the new positions)
 *   BLOCK_TABLE [R, max_pages_per_req] int32;  CONTEXT_LENS [R] int32 (include the new tokens)
 *   X [M, H] bf16;  R_IN [M, H] fp32
 *   SCORE_OUT [M, S] fp32 with S = the largest context length: row m gets the scores of keys
 *     t < ctx_r (-inf for t > its position); entries t >= ctx_r are not written
 *   WORKSPACE  mk_plan_workspace_bytes() bytes, 256-byte aligned
 *   main-MLA half, only when mk_config.mla_heads = nm > 0 (else the entries may be 0 or absent):
 *     W_QB [nm 128, qr] e4m3 + S_QB (D0 Main-Q: rows h 128 .. h 128 + 127 are head h's no-RoPE query
 *     from the normalised q_a); W_UK [nm 512, 128] bf16 (D2 Q-BMM: rows h 512 .. h 512 + 511 are head
 *     h's [512, 128] up-projection of keys, absorbed into the query); QLAT_OUT [M, nm, 512] bf16:
 *     q_lat[m][h] = W_UK[h] q_nope[m][h], q_nope[m][h] = bf16(W_QB[h] q_a(m)) (MegaRTP page, section 4:
 *     the D0 -> D2 edge of the attention-pre graph)
 *   TOPK_OUT [M, topk] int32, only when mk_config.topk > 0 (else the entry may be 0 or absent): row m
 *     gets the positions of the topk largest scores among its keys t <= its position (MegaRTP page:
 *     the Top-2048 that follows the paged indexer score), ties to the smaller position, listed in
 *     ascending order; -1 fills the row past the number of keys when a token has fewer than topk */
enum {
  MK_TI_W_QA = 0, MK_TI_S_QA, MK_TI_W_W, MK_TI_S_W, MK_TI_W_K, MK_TI_S_K, MK_TI_W_QI, MK_TI_S_QI,
  MK_TI_G_NORM, MK_TI_G_QA, MK_TI_KEY_CACHE, MK_TI_KEY_SCALE, MK_TI_BLOCK_TABLE, MK_TI_CONTEXT_LENS,
  MK_TI_X, MK_TI_R_IN, MK_TI_SCORE_OUT, MK_TI_WORKSPACE, MK_TI_TOPK_OUT,
  MK_TI_W_QB, MK_TI_S_QB, MK_TI_W_UK, MK_TI_QLAT_OUT,
  MK_TI_COUNT
};

typedef struct mk_plan mk_plan; /* opaque, library-owned */

/* Lower a workload into tile tasks, events and per-worker queues, and upload the queue,
 * zeroed counters and tables to the current device (MegaRTP page, section 4: the host lowering
 * OpGraph -> tile expansion -> TaskGraph -> KernelPlan).  host_context_lens: n_requests
 * entries (context length per request including the new token).  The plan fixes tile
 * counts and thresholds, so a new plan is needed only when shapes, context lengths or the
 * worker count change; the same section rebuilds its plan only when the row count or the KV
 * lengths change, and rebinds tensors through the pointer table otherwise.
 * Without a HIP device the plan is built on the host only (num_workers must then be > 0):
 * its queue, events and info can be read, and the run entry points return MK_ERR_INVALID.
 * Errors: MK_ERR_INVALID for inconsistent shapes; MK_ERR_UNSUPPORTED for variants not built. */
mk_status mk_build_queue(const mk_config* cfg, const int32_t* host_context_lens, mk_plan** out);

/* Host view of the queue (MegaRTP page, section 4: the KernelPlan's instruction tensor, tasks dealt
 * round-robin onto W worker queues padded with NoOp): uint32 [W, L, 32], 32 words per instruction:
 *   w0 opcode, w1 wait count, w2 signal count, w3 operand row, w4 spec id, w5 task id,
 *   w6..w13 four (event id, threshold) waits, w14..w19 two (event id, increment,
 *   publication id) signals, w20..w31 payload (layer, tile coordinates, arrival group id,
 *   arrival group size, rank in group).  Padding slots are NoOp (32 zero words).
 * The pointer stays valid until mk_plan_destroy. */
mk_status mk_plan_queue(const mk_plan* plan, const uint32_t** host_instr, int32_t* W, int32_t* L);

/* Event thresholds (MegaRTP page, section 4: the TaskGraph's counter events, a consumer waiting for
 * counter >= threshold): uint32 [num_events]; each equals the increments its producers issue per run. */
mk_status mk_plan_events(const mk_plan* plan, const uint32_t** host_thresholds, int32_t* num_events);

/* Plan facts (MegaRTP page, section 4: tasks, and one operand-table row per op instance): n_tasks,
 * n_ops (rows of the operand pointer table, 16 addresses each), n_arrivals (arrival groups). */
mk_status mk_plan_info(const mk_plan* plan, int32_t* n_tasks, int32_t* n_ops, int32_t* n_arrivals);

/* Bytes of scratch the caller passes as MK_T_WORKSPACE / MK_TI_WORKSPACE: the intermediates the
 * MegaRTP page's operand table points at (section 4), owned by the caller. */
mk_status mk_plan_workspace_bytes(const mk_plan* plan, size_t* bytes);

/* Byte offset and size of a named intermediate inside the workspace, for inspection.  In
 * single-token plans the vectors written inside a run are tagged records of 8 bytes
 * {uint32 payload, uint32 tag}, the tag being salt + epoch * 1024 + layer + 1 of the run and layer
 * that wrote them (salt: a per-plan multiple of 1024; epoch: runs of this plan before): "qkv" fp32
 * [M, N_qkv], "o" bf16 pairs [M, Hq d / 2], "m" bf16 pairs [M, I / 2], "r2" fp32 [M, H]
 * (residual after attention), "r1" fp32 [M, H] (r2 + y, the next layer's residual input).
 * "part" holds the split-KV partials as plain fp32 (kernel prologue/epilogue page, section 4: per
 * split its normalised output and log-sum-exp), "lm_part" the lm_head tasks' maxima (one slot per task).  Multi-row
 * plans keep "qkv" as records and everything else plain (projection inputs in the matrix-core
 * operand order, fp32 partial sums per tile and K chunk).  Errors: MK_ERR_INVALID for an unknown name. */
mk_status mk_plan_workspace_region(const mk_plan* plan, const char* name, size_t* offset, size_t* bytes);

/* Run the plan once as ONE persistent kernel launch on `hip_stream` (asynchronous): one worker
 * block per compute unit walks its queue (MegaRTP page, section 4: the persistent kernel reading
 * its instruction tensor, waiting on events before a tile's first read and signalling after its
 * last write).  Single-token plans realise the waits on the data: producers store tagged records (see
 * mk_plan_workspace_region), and a consumer stages the records it needs until all carry the
 * run's tag -- the event reaches its threshold when every producer tile's records are current.
 * The split-KV combine and the argmax use arrival counters.  Multi-row plans and the indexer
 * front wait on the queue's event counters, as the page does, with device-scope data accesses.
 * Polls are bounded by a watchdog (see mk_sync).  Not capturable into a graph (the run epoch is a
 * launch argument).  Runs on one plan must be issued on one stream.  Errors: MK_ERR_INVALID for a
 * missing or misaligned tensor, a host-only plan or a launch failure (nothing is launched); device
 * errors are reported by mk_sync. */
mk_status mk_run_layer(mk_plan* plan, const mk_tensors* tensors, void* hip_stream);

/* For callers that cannot allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc: the same run as mk_run_layer (same kernels, same results
 * bit for bit) with its scratch in a statically allocated device array instead of the caller's
 * workspace.  The MK_T_WORKSPACE / MK_TI_WORKSPACE entry of `tensors` is ignored (it may be 0); every
 * other tensor is the caller's, as for mk_run_layer.
 * The array is MK_SCRATCH_MAX_BYTES per GPU, allocated with the library's code object on each GPU
 * the library runs on and held until the process ends; it holds the plan's workspace
 * (mk_plan_workspace_bytes, rounded up to 256) followed by its operand pointer table (16 x 8 bytes per
 * op).  A plan that needs more returns MK_ERR_INVALID and launches nothing.  The call allocates
 * nothing: its address is looked up once per device at plan set-up (mk_build_queue), the table is
 * written into the array by a small kernel on `hip_stream`, and the workspace is cleared (an
 * asynchronous memset on `hip_stream`) whenever another plan used the array last.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other streams,
 * other threads) race and must not be issued; calls in one stream order are safe.  Asynchronous. */
#define MK_SCRATCH_MAX_BYTES (40u << 20)
mk_status mk_run_layer_noalloc(mk_plan* plan, const mk_tensors* tensors, void* hip_stream);

/* The graph baseline the megakernel is measured against (MegaRTP page, sections 5 and 6: the same
 * ops as standalone kernels composed in a graph, independent branches on streams of their own):
 * the same op bodies as
 * one kernel per op (an op's tasks dealt over min(tasks, workers) blocks of the eight-wave worker,
 * no waits, signals or tag checks: stream order orders the ops) inside a hipGraph captured on first
 * use per tensor set; multistream = 0: one stream in topological order; 1: an op with no edge to
 * the op before it goes on a second stream (at most two streams), joined by events.  Same results
 * as mk_run_layer bit for bit.  Asynchronous.  Errors as mk_run_layer. */
mk_status mk_run_graph_baseline(mk_plan* plan, const mk_tensors* tensors, int32_t multistream, void* hip_stream);

/* Wait for the plan's last run on its stream and report the device error record (the watchdog
 * bounds the MegaRTP page's section-4 wait for counter >= threshold, which has no bound of its own):
 * MK_ERR_TIMEOUT if a worker's watchdog expired; MK_ERR_INVALID if a block-table entry was outside
 * [0, num_phys_pages) (it was read as page 0, so no access left the cache pool, and the run's outputs
 * are not valid).  On either error the other workers abandon their waits, and the plan's counters
 * are reset so that the next run starts clean. */
mk_status mk_sync(mk_plan* plan, void* hip_stream);

/* Copy the trace of the last MK_FLAG_TRACE megakernel run into host memory (MegaRTP page,
 * sections 4 and 5: per-task timestamps from which its timeline and empty-framework time are
 * read; synchronous): uint32 [W, L, 16]
 * per instruction: low 32 bits of the 100 MHz realtime clock when the controller saw it, when
 * its waits were met, when its activations were staged, after the compute start / end
 * barriers, when its outputs were acknowledged, when its arrival resolved (0 if none), when it
 * was done; word 8 counts the staging rounds repeated because an input was not yet current; word 9:
 * when the compute waves issued the instruction's lease (kernels with loader waves: shader cycles
 * between the two compute barriers); words 10..15 hold per-family details. */
mk_status mk_read_trace(const mk_plan* plan, uint32_t* host_out, size_t n_words);

/* Copy the gather record of the last run of an MK_FLAG_DEBUG_GATHER plan into host memory (synchronous).
 * Each entry is the physical cache slot page * P + offset a run fetched for one token through the
 * block table (the page walk of the MegaRTP page's E1 operand row: block_table and context_lens),
 * or -1 where nothing was fetched (every run first sets all entries to -1):
 *   MK_QWEN3_LAYER / MK_QWEN3_STEP: int32 [layers][n_requests][n_kv_heads][2 (K, V)][max_pages_per_req * P];
 *     the tokens t < ctx_r - 1 of request r (the new token's row comes from the run itself)
 *   MK_INDEXER_FRONT: int32 [n_requests][max_pages_per_req * P]; the keys t < ctx_r - T written before the run
 * n_words: capacity of host_out in int32 entries (extra entries are left untouched).
 * Errors: MK_ERR_INVALID when the plan was built without the flag. */
mk_status mk_read_gather(const mk_plan* plan, int32_t* host_out, size_t n_words);

/* Plumbing, defined by no page: the calling thread's message for its last failed call (never
 * NULL), and freeing a plan with everything it allocated (NULL is ignored; the plan's runs must
 * have completed). */
const char* mk_last_error(void);
void mk_plan_destroy(mk_plan* plan);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
