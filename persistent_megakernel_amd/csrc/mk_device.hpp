// Kernel-side constants and the launch argument block shared by the device code and the
// host launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.hpp"

namespace mk {

struct Shapes {
  int H, I, Hq, Hkv, g, n_qkv, P, maxp, max_splits, V;
  float eps, inv_sqrt_d;
  int M, kc, fp8, layers;  // multi-row plans: rows, K chunk of a projection tile, W8A8, layers
  int qr, nh, T, smax;     // indexer front: q rank, heads, tokens per request, score row stride
  int npages;              // physical pages of the cache pool: every block-table entry must be below it
  int topk;                // indexer front: positions each token row selects (0: no top-k)
  int mla;                 // indexer front: heads of the main-MLA query half (0: none)
  int rg;                  // multi-row plans: 16-row groups of M (operand order, partial sums, finalizes)
};

struct KArgs {
  const uint32_t* instrs;  // megakernel: queue [W, L, 32]; graph: task list [T, 32]
  int L;                   // megakernel: queue length per worker; graph: tasks of the op
  int first_task;          // graph: task id of block 0
  const uint64_t* table;   // operand pointer table [n_ops, 16]
  uint32_t* events;        // [E][kNSub sub-counters, kSubStride words apart]
  uint32_t* arrivals;      // [A], kSubStride words apart, self re-arming
  uint32_t* err;           // device error record: flag, worker, task, event, value, target
  uint32_t* trace;         // [W, L, kTraceWords] or null
  int32_t* gather;         // MK_FLAG_DEBUG_GATHER: the physical cache slot of every gathered K / V row or key, or null
  uint32_t tag0;           // megakernel: this run's record tag base (plan salt + runs so far * 1024)
  uint32_t run;            // megakernel: runs since the event counters were zeroed (targets (run + 1) * threshold)
  uint32_t flags;          // MK_FLAG_* | kModeGraph
  Shapes sh;
};

constexpr uint32_t kModeGraph = 1u << 16;
constexpr int kTraceWords = 16;  // per instruction: visible, ready, prologue, A, B, stored, arrived, done, poll, ...
constexpr int kNSub = 16;                  // sub-counters per event (spreads the atomics)
constexpr int kSubStride = 32;             // words between sub-counters (128 bytes)
constexpr int kEvStride = kNSub * kSubStride;
constexpr uint32_t kErrWatchdog = 1u, kErrBlockTable = 2u;  // error record word 0
constexpr unsigned long long kWatchdogTicks = 200000000ull;  // 2 s of the 100 MHz clock

namespace dev {
constexpr int kThreads = 512;  // 8 waves: controller + 7 loader/compute waves
constexpr int kNCW = 7;
constexpr int kNW = 8;     // waves of a projection tile: the seven compute waves and the controller
constexpr int kNPages = 8;     // LDS ring of 8 x 16 KiB pages
#ifndef MK_LOOKAHEAD_PAGES
#define MK_LOOKAHEAD_PAGES 8
#endif
constexpr int kLookPages = MK_LOOKAHEAD_PAGES;  // prefetch at most this many pages from the current lease
constexpr int kRingOff = 0;
constexpr int kActOff = kNPages * 16384;   // activation staging
constexpr int kActBytes = 27648;
constexpr int kActStageBytes = kActBytes;  // largest staged block (a 1 KiB multiple)
constexpr int kOutOff = kActOff + kActBytes;  // compute results
constexpr int kOutBytes = 4096;
constexpr int kMaxKQ = 12;     // projection K <= 12 * 512: quad sums per row  // g*128 + g floats of an attention partial: GQA group <= 7
constexpr int kCtrlOff = kOutOff + kOutBytes;  // abort flag + per-wave lease tables
constexpr int kCtrlBytes = 1024;
constexpr int kLeaseTabOff = 64;   // in the control area: [7 waves][32] lease tables
constexpr int kInvOff = 8;         // in the control area: the fused norm's rsqrt(mean square + eps)
// multi-row kernel: kLoaders more waves that only stream leases and never take a barrier; the
// other eight synchronise through an LDS arrival counter instead of s_barrier
constexpr int kLoaders = 3;
constexpr int kThreadsM = kThreads + 64 * kLoaders;
constexpr int kBarOff = 24;        // in the control area: arrivals at the eight waves' barrier
constexpr int kRetiredOff = 28;    // in the control area: instructions the eight waves have finished
constexpr int kDoneOff = 32;       // in the control area: [kLoaders] instructions whose lease share landed
constexpr int kFetchedOff = 48;    // in the control area: instructions loader 0 has copied into the instruction ring
static_assert(kLeaseTabOff + 7 * 32 * 4 <= kCtrlBytes, "control area");
static_assert(kDoneOff + 4 * kLoaders <= kFetchedOff && kFetchedOff + 4 <= kLeaseTabOff && kLoaders <= 7, "control area");
constexpr int kLdsBytes = kCtrlOff + kCtrlBytes;  // all 160 KiB: one block per CU
// attention sub-areas of the activation staging area
constexpr int kMaxG = 5;       // GQA group (q heads per kv head) of the M = 1 attention body
constexpr int kActQ = 0;       // bf16 [g][128] rotated q heads
constexpr int kActK = 2048;    // bf16 [128] new key
constexpr int kActV = 2304;    // bf16 [128] new value
constexpr int kActMerge = 2560;  // fp32 [8 waves][g][128] per-wave partial P V, then (m_w, l_w)
constexpr int kAttGq = 2560;     // q and k norm gains (bf16 [128] each) and the request's RoPE row
constexpr int kAttGk = 2816;     // (fp32 (cos, sin) [64]): read in the first phase, before the merge
constexpr int kAttRope = 3072;   // area they share is written
constexpr int kAttQraw = 4096;   // tagged records of the raw q heads (g KiB), k and v (1 KiB each);
constexpr int kAttKraw = kAttQraw + kMaxG * 1024;  // consumed before the merge area is written
constexpr int kAttVraw = kAttKraw + 1024;
constexpr int kActR1 = kActBytes - 1024;    // O projection / down: residual rows of the tile as records (<= 128)
// multi-row ops in the activation staging area: a projection tile's input chunk (16 rows x one K
// chunk in operand order, 16 KiB), the eight waves' 16 x 16 fp32 results, reduction scratch
constexpr int kActA = 0;
constexpr int kActABytes = 16384;
constexpr int kActD = kActA + kActABytes;   // [8 waves][64 lanes][4] fp32
constexpr int kActRed = kActD + 8192;       // [2][8] fp32 per-wave partial reductions
static_assert(kActRed + 64 <= kActBytes, "multi-row staging overflows the activation area");
// multi-row kernel with loader waves: the next sixteen instructions (128 B each), copied by loader 0
// as it walks the queue, at the end of the activation area (no multi-row layer op uses it)
constexpr int kActInstr = kActBytes - 2048;
static_assert(kActRed + 64 <= kActInstr && kActMerge + 8 * kMaxG * 130 * 4 <= kActInstr, "instruction ring overlaps staging");
// single-token kernel: the next eight instructions, copied by compute wave 0 as it prefetches, at the
// end of the output area (attention output <= 4 x 129 floats, combine weights 64 x kMaxG + kMaxG x 3
// floats, projection sums <= 128 floats), each slot with its instruction index + 1 in the control area
constexpr int kOutInstr = kOutBytes - 1024;
constexpr int kITagOff = 960;
static_assert(4 * 129 * 4 <= kOutInstr && (64 * kMaxG + 3 * kMaxG) * 4 <= kOutInstr, "instruction ring overlaps outputs");
static_assert(kLeaseTabOff + 7 * 32 * 4 <= kITagOff && kITagOff + 8 * 4 <= kCtrlBytes, "control area");
static_assert(kActMerge + 8 * kMaxG * 130 * 4 <= kActBytes, "attention merge area overflows the staging area");
static_assert(kAttRope + 512 <= kAttQraw, "attention gains overlap the raw q staging");
static_assert(kLdsBytes == 163840, "LDS budget");
static_assert(kLdsBytes <= 163840, "LDS budget");
}  // namespace dev

// No-allocation runs: one statically allocated device array per GPU holds the workspace and the
// operand pointer table of the run (mk_run_layer_noalloc).  The table is written on the device from a
// relocation list the plan builds once: entry = (tensor index, byte offset), or an absolute library
// address when the index is kRelocAbs.
constexpr size_t kScratchBytes = (size_t)40 << 20;
constexpr uint32_t kRelocAbs = 0xFFFFFFFFu;
struct TableReloc {
  uint64_t off;  // byte offset from tensor `idx`, or the absolute address (or 0) when idx == kRelocAbs
  uint32_t idx;
  uint32_t pad;
};
struct TensorPtrs {
  uint64_t ptr[MK_MAX_TENSORS];
};
hipError_t scratch_init(int device);  // once per device, with that device current: the array's address
void* scratch_base(int device);       // null until scratch_init succeeded on that device
hipError_t launch_fill_table(const TableReloc* reloc, int n, const TensorPtrs& t, uint64_t* out, hipStream_t stream);

// spec: the plan's op family (0 single-token bodies, 1 multi-row bodies), one kernel instance each
// loaders: the multi-row kernel with its loader waves (kThreadsM threads) rather than the eight
// waves prefetching for themselves (kThreads)
hipError_t launch_worker(const KArgs& a, int grid, hipStream_t stream, int spec, bool loaders);
hipError_t worker_occupancy(int* blocks_per_cu, int spec);

}  // namespace mk
