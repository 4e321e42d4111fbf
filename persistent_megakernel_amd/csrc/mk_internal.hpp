// Internal host-side definitions shared by the planner, the launch code and the C ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/mk.h"

namespace mk {

enum Opcode : uint32_t {
  OP_NOOP = 0,
  OP_QKV = 1,     // fused add + RMSNorm prologue, QKV projection rows
  OP_ATTN = 2,    // QK-norm + RoPE + cache write + split-KV attention partial; last arrival combines
  OP_OPROJ = 3,   // O projection rows + residual add
  OP_GATEUP = 4,  // RMSNorm prologue, gate and up rows, SiLU-mul epilogue
  OP_DOWN = 5,    // down projection rows
  OP_LMHEAD = 6,  // final add + RMSNorm prologue, a worker's lm_head rows streamed, their max; last arrival takes the argmax
  // multi-row (M = 16) plans
  OP_NORM = 7,    // one row: (add +) RMSNorm (+ FP8 quantisation) into the projection input layout
  OP_GEMM = 8,    // one (64-row tile, K chunk) of a projection: MFMA partial sums
  OP_FIN = 9,     // one row tile: add the K chunks in order, then the projection's epilogue
  OP_QUANT = 10,  // one row of o or m: per-token FP8 quantisation into the projection input layout
  OP_COMB = 11,   // one (request, kv head): combine the split-KV partials into o
  // indexer front
  OP_KCACHE = 12, // the new tokens' keys: RoPE, per-token e4m3, key-cache write
  OP_SCORE = 13,  // one (request, key split): paged indexer score
  OP_TOPK = 14    // one token row: the positions of its top-k scores
};
enum ProjKind : uint32_t { K_QKV = 0, K_O = 1, K_GU = 2, K_DOWN = 3, K_QA = 4, K_W = 5, K_KI = 6, K_QI = 7,
                           K_QB = 8,    // main-MLA query (D0): e4m3, K = q rank, finalized per head
                           K_UK = 9 };  // main-MLA query BMM (D2): bf16, K = 128 (one head), one chunk
constexpr int kMlaNope = 128, kMlaLatent = 512;  // per main-MLA head: D0 output, D2 output
constexpr int kScoreTok = 128;  // keys per indexer-score task
constexpr int kMaxRows = 256;  // multi-row plans: at most 16 groups of 16 rows
constexpr int kM16Rows = 64;  // weight rows of a multi-row projection tile (gate/up: 32 + 32)
constexpr int kMaxChunks = 24;  // K chunks a multi-row finalize task adds

constexpr uint32_t kNone = 0xFFFFFFFFu;
constexpr int kWords = 32;
constexpr int kLeaseBytes = 65536;  // largest LDS lease of one instruction

// instruction word positions
enum Word : int {
  W_OPCODE = 0, W_NWAIT = 1, W_NSIG = 2, W_ROW = 3, W_SPEC = 4, W_TASK = 5,
  W_WAIT0 = 6,    // (event, threshold) x 4
  W_SIG0 = 14,    // (event, increment, publication id) x 2
  W_LAYER = 20,
  W_P1 = 21,      // n0 | request
  W_P2 = 22,      // rows | kv head
  W_P3 = 23,      // k0 | split
  W_P4 = 24,      // k length | token start
  W_P5 = 25,      // token end (exclusive)
  W_ARR_ID = 26,  // arrival group
  W_ARR_N = 27,   // arrival group size (0: no arrival group)
  W_ARR_RANK = 28, // rank of this task in its group
  W_NSPLIT = 29,  // multi-row attention: splits of the (request, kv head)
  W_GROUP = 29,   // multi-row finalize: the 16-row group of M it finalizes
  W_CHAIN = 30,   // multi-row attention: bit 0 continues the worker's previous task's chain, bit 1 ends it
  W_PSLOT = 31    // multi-row attention: the chain's partial slot in its (request, kv head)
};

// operand pointer table: 16 slots per op row
constexpr int kTableSlots = 16;
// Workspace vectors written inside a run (qkv, o, m, r2, r1) hold tagged 8-byte records
// {payload, tag}; X / RIN are the caller's first-layer inputs, R2OUT / Y the caller's last-layer
// outputs (0 on other layers).
enum QkvSlot { QKV_W = 0, QKV_GAMMA, QKV_X, QKV_RIN, QKV_OUT, QKV_R1 };
enum AttnSlot { ATT_QKV = 0, ATT_GQ, ATT_GK, ATT_KC, ATT_VC, ATT_BT, ATT_PART, ATT_O, ATT_ROPE,
                ATT_QB };  // multi-row: the bf16 q heads after QK-norm and RoPE, [M][Hq][d] (read by the tests)
enum OSlot { O_W = 0, O_IN, O_X, O_RIN, O_R2, O_R1, O_R2OUT };
enum GuSlot { GU_W = 0, GU_GAMMA, GU_R2, GU_M };
enum DownSlot { DN_W = 0, DN_M, DN_Y, DN_R2, DN_R1 };
enum LmSlot { LM_W = 0, LM_GAMMA, LM_R1, LM_LOGITS, LM_PART, LM_TOKEN };
// Multi-row plans keep their intermediates plain (no record tags: event counters order them).
// Projection inputs are stored in the matrix-core operand order, 1 KiB per K step: bf16 steps of
// 32, lane l = row + 16 * ((k % 32) / 8) holding 8 consecutive k; e4m3 steps of 64, lane
// l = row + 16 * ((k % 64) / 16) holding 16 consecutive k.  Rows >= M stay 0.
// NORM: x (0 for the post-attention norm), residual in, gain, r1 out (first norm only), h out, scale out
enum NormSlot { NM_X = 0, NM_R, NM_GAIN, NM_R1, NM_H, NM_S };
// GEMM tile: weights, operand-order input, fp32 partial sums [tile][chunk][4 x 64 lanes x 4], weight scales
enum GemmSlot { GM_W = 0, GM_ACT, GM_PART, GM_SW };
// FIN: partial sums, per-token input scales (FP8), output, r1 (O projection), caller's output (last layer)
enum FinSlot { FN_PART = 0, FN_SA, FN_OUT, FN_R1, FN_OUT2 };
// QUANT: fp32 rows in, e4m3 operand-order rows out, per-token scales out
enum QuantSlot { QT_IN = 0, QT_OUT, QT_S };
// KCACHE: key rows (fp32 [M][d]), RoPE table, key cache codes, key scales, block table, row positions
enum KcSlot { KC_K = 0, KC_ROPE, KC_CACHE, KC_SCALE, KC_BT, KC_POS };
// SCORE: q (bf16, score operand order), head weights (fp32 [M][heads]), key cache, key scales,
// block table, scores out (fp32 [M][max context]), row positions
enum ScSlot { SC_Q = 0, SC_W, SC_CACHE, SC_SCALE, SC_BT, SC_OUT, SC_POS };
// TOPK: scores (fp32 [M][max context]), row positions, selected positions out (int32 [M][topk])
enum TkSlot { TK_SCORE = 0, TK_POS, TK_OUT };
constexpr int kTopkMaxKeys = 8192;  // keys a top-k row holds in registers (16 per lane of 512)

struct TileParams {
  int r_qkv = 0, r_o = 0, r_gu = 0, r_down = 0, r_lm = 0, s_tok = 0, spec = 0;
  int kc = 0;  // multi-row plans: K chunk of a projection tile (kM16Rows x kc weights fill a lease)
  int kc_q = 0;  // indexer front: K chunk of the q projection (K = q rank)
};

struct OpInfo {      // one row of the operand table = one op instance
  uint32_t opcode;
  uint32_t sub;      // GEMM / FIN: projection kind; NORM / QUANT: which (0: first, 1: second)
  int layer;
  int first_task, n_tasks;
  std::vector<int> deps;  // op rows this op waits on (graph edges)
};

struct WorkspaceRegion {
  std::string name;
  size_t offset, bytes;
};

struct HostPlan {
  mk_config cfg{};
  std::vector<int32_t> ctx;
  int W = 0, L = 0, T = 0;
  TileParams tp;
  std::vector<uint32_t> queue;       // [W, L, 32]
  std::vector<uint32_t> tasks;       // [T, 32] in task order (graph baseline)
  std::vector<uint32_t> thresholds;  // [E]
  int n_arrivals = 0;
  std::vector<OpInfo> ops;           // indexed by operand row
  int max_splits = 0;                // largest number of KV splits of any (request, kv head)
  std::vector<WorkspaceRegion> regions;
  size_t workspace_bytes = 0;
};

// planner.cpp
mk_status plan_build(const mk_config& cfg, const int32_t* ctx, int W, HostPlan& out, std::string& err);

}  // namespace mk
