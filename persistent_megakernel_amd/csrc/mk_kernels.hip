// Device side of the decode-layer megakernel for MI355X (gfx950, CDNA4, wave64).
//
// One worker block per compute unit runs its instruction queue (MegaRTP page, section 4:
// resident worker blocks, a host-built queue, dependencies as global event counters).  The
// same worker body also runs one instruction per block as the standalone kernels of the
// graph baseline.
//
// Block = 8 waves.  Wave 0 is the controller: it reads instructions, polls the event
// counters of the current instruction, stages the instruction's activations into LDS
// (fused add + RMSNorm, QK-norm + RoPE), and after the compute writes the outputs, waits for
// their completion and signals the counters (fused epilogues: residual add, SiLU-mul, split-KV
// combine, argmax).  Waves 1..7 are loader/compute waves: they lease LDS pages of a 128 KiB
// ring to the upcoming instructions in queue order and issue direct-to-LDS 16-byte loads of
// each instruction's weights (or KV rows) as soon as pages are free -- before its counter wait
// -- so weight streaming overlaps the dependency waits (the page's weight prefetch ahead of the
// activation wait, and its logical-to-physical page leasing).  Because the vector-memory
// counter is per wave, the polling wave never issues prefetch loads and the prefetching waves
// never poll, so each side's waits see only its own loads.
//
// Cross-CU visibility and waits.  MI355X has one L2 per XCD and plain cached lines are not
// coherent across XCDs.  Every value produced inside a run is stored at device scope (sc1) as an
// 8-byte record {payload, tag}, the tag naming the plan, the run and the producing layer; an
// aligned 8-byte store is seen whole or not at all.  An event of the queue is thereby
// carried by the data itself: a consumer's wait is the staging of the records it needs into LDS,
// repeated for the 1 KiB blocks whose tags are not current yet -- one memory round trip once the
// data is there, no acknowledgement wait on the producer side and no separate counter.  Only
// the split-KV combine and the argmax keep an arrival counter (the last arriver reduces).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "mk_device.hpp"

namespace mk {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));  // 16x16x32 bf16 matrix-core operand
typedef short i16x4 __attribute__((ext_vector_type(4)));    // 16x16x16 bf16 matrix-core operand
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const char lds_cchar;

#define DEV __device__ __forceinline__

// ---------------------------------------------------------------------------------------
// small helpers
DEV uint32_t lane() { return __lane_id(); }
// a value every lane of the wave holds (e.g. read back from a per-wave LDS table), made uniform
DEV uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
DEV unsigned long long rtc() { return __builtin_amdgcn_s_memrealtime(); }

DEV float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
// bf16 pair view of a 32-bit word.  (A bit_cast of an ext-vector element is taken from
// element 0 by this compiler, so the word is copied out first.)
// two fp32 to packed bf16 (round to nearest even; one v_cvt_pk_bf16_f32 on gfx950)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
DEV uint32_t pack_bf2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  const bf16x2 h = __builtin_convertvector(v, bf16x2);
  uint32_t u;
  __builtin_memcpy(&u, &h, 4);
  return u;
}
DEV bf16x2 as_bf2(uint32_t v) {
  bf16x2 r;
  __builtin_memcpy(&r, &v, 4);
  return r;
}
DEV float dot8(u32x4 w, u32x4 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w.x), as_bf2(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w.y), as_bf2(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w.z), as_bf2(x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w.w), as_bf2(x.w), acc, false);
  return acc;
}

// Wave reductions without the LDS pipe: DPP within rows of 16 lanes (quad xor 1, quad xor 2,
// half-row mirror, row mirror leave every lane of a row holding the row total), then
// row_bcast:15 / row_bcast:31 accumulate the four rows into lane 63.
template <int CTRL>
DEV float dppf(float v) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false)); }
template <int CTRL>
DEV int dppi(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false); }
template <int CTRL, int ROWS>
DEV float dpp_rows(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWS, 0xF, false));
}
DEV float row16_sum(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  v += dppf<0x140>(v);
  return v;
}
DEV float wave_sum(float v) {
  v = row16_sum(v);
  v += dpp_rows<0x142, 0xA>(0.f, v);
  v += dpp_rows<0x143, 0xC>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
DEV float wave_max(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));
  v = fmaxf(v, dpp_rows<0x142, 0xA>(v, v));
  v = fmaxf(v, dpp_rows<0x143, 0xC>(v, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// the same lane position summed over the four 16-lane rows (gfx950 cross-row lane swaps)
DEV float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float p = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
DEV float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float p = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// inclusive prefix sum over the lanes (row_shr steps inside rows of 16, then the row totals
// broadcast forward), and over lanes 0 .. 15 only
DEV uint32_t row16_incl_scan(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
  return (uint32_t)x;
}
DEV uint32_t wave_incl_scan(uint32_t v) {
  int x = (int)row16_incl_scan(v);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return (uint32_t)x;
}
DEV uint32_t wave_min_u32(uint32_t v) {
  int x = (int)v;
  x = min((uint32_t)x, (uint32_t)dppi<0xB1>(x));
  x = min((uint32_t)x, (uint32_t)dppi<0x4E>(x));
  x = min((uint32_t)x, (uint32_t)dppi<0x141>(x));
  x = min((uint32_t)x, (uint32_t)dppi<0x140>(x));
  x = min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x142, 0xA, 0xF, false));
  x = min((uint32_t)x, (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}
DEV uint32_t wave_max_u32(uint32_t v) { return ~wave_min_u32(~v); }
DEV uint32_t wave_or_u32(uint32_t v) {
  int x = (int)v;
  x |= dppi<0xB1>(x);
  x |= dppi<0x4E>(x);
  x |= dppi<0x141>(x);
  x |= dppi<0x140>(x);
  x |= __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x |= __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}
DEV uint32_t wave_sum_u32(uint32_t v) {
  int x = (int)v;
  x += dppi<0xB1>(x);
  x += dppi<0x4E>(x);
  x += dppi<0x141>(x);
  x += dppi<0x140>(x);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return (uint32_t)__builtin_amdgcn_readlane(x, 63);
}

// Loads of data that no one writes during a run (queue, pointer table, block table) go through
// the constant address space: uniform addresses become scalar loads (scalar cache, lgkm
// counter), which leaves the vector-memory counter to the prefetch accounting.
template <typename T>
DEV T c_ld(const void* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}
DEV uint32_t s_ld32(const void* p) { return c_ld<uint32_t>(p); }
DEV uint64_t s_ld64(const void* p) { return c_ld<uint64_t>(p); }
DEV u32x8 s_ld256(const void* p) { return c_ld<u32x8>(p); }

struct Instr {
  uint32_t w[32];
};
DEV void fetch(const uint32_t* p, Instr& in) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u32x8 v = s_ld256(p + 8 * k);
#pragma unroll
    for (int j = 0; j < 8; ++j) in.w[8 * k + j] = v[j];
  }
}

// the instruction ring of the multi-row kernel with loader waves: slot i mod 16 of the activation
// area's last 2 KiB (loader 0 writes it on its first look at instruction i; the controller reads it
// once loader 0 has published i, instead of a scalar fetch from the queue in memory)
DEV void put_instr(char* smem, int j, const Instr& in) {
  if (__lane_id() == 0) {
    u32x4* d = (u32x4*)(smem + dev::kActOff + dev::kActInstr + (j & 15) * 128);
#pragma unroll
    for (int k = 0; k < 8; ++k) d[k] = u32x4{in.w[4 * k], in.w[4 * k + 1], in.w[4 * k + 2], in.w[4 * k + 3]};
  }
}
DEV void get_instr(const char* smem, int i, Instr& in) {
  asm volatile("" ::: "memory");  // not before the read of the published count (LDS serves a wave in order)
  const u32x4* s = (const u32x4*)(smem + dev::kActOff + dev::kActInstr + (i & 15) * 128);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const u32x4 v = s[k];
#pragma unroll
    for (int q = 0; q < 4; ++q) in.w[4 * k + q] = __builtin_amdgcn_readfirstlane(v[q]);
  }
}

// the instruction ring of the kernels without loader waves: slot i mod 8, tagged with i + 1, of the
// output area's last KiB (single-token) or of the activation area's ring (multi-row); compute wave 0
// writes the instructions it prefetches at most seven ahead of its own (so never the slot of one the
// controller has yet to read)
template <int S>
DEV char* ring8_slot(const char* smem, int j) {
  return (char*)smem + (S == 0 ? dev::kOutOff + dev::kOutInstr : dev::kActOff + dev::kActInstr) + (j & 7) * 128;
}
template <int S>
DEV void put_instr8(char* smem, int j, const Instr& in) {
  if (__lane_id() == 0) {
    u32x4* d = (u32x4*)ring8_slot<S>(smem, j);
#pragma unroll
    for (int k = 0; k < 8; ++k) d[k] = u32x4{in.w[4 * k], in.w[4 * k + 1], in.w[4 * k + 2], in.w[4 * k + 3]};
    *(volatile uint32_t*)(smem + dev::kCtrlOff + dev::kITagOff + (j & 7) * 4) = (uint32_t)j + 1u;
  }
}
// the operand-table row of instruction i if compute wave 0 has copied it into the ring, else kNone
template <int S>
DEV uint32_t ring8_row(const char* smem, int i) {
  if (__builtin_amdgcn_readfirstlane(*(const volatile uint32_t*)(smem + dev::kCtrlOff + dev::kITagOff + (i & 7) * 4)) !=
      (uint32_t)i + 1u)
    return 0xFFFFFFFFu;
  asm volatile("" ::: "memory");
  return __builtin_amdgcn_readfirstlane(*(const uint32_t*)(ring8_slot<S>(smem, i) + 4 * W_ROW));
}
template <int S>
DEV bool get_instr8(const char* smem, int i, Instr& in) {
  if (__builtin_amdgcn_readfirstlane(*(const volatile uint32_t*)(smem + dev::kCtrlOff + dev::kITagOff + (i & 7) * 4)) !=
      (uint32_t)i + 1u)
    return false;
  asm volatile("" ::: "memory");  // the words after their tag (LDS serves a wave in order)
  const u32x4* s = (const u32x4*)ring8_slot<S>(smem, i);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const u32x4 v = s[k];
#pragma unroll
    for (int q = 0; q < 4; ++q) in.w[4 * k + q] = __builtin_amdgcn_readfirstlane(v[q]);
  }
  return true;
}

// Device-scope (sc1) loads and stores through buffer resources; aux bit 4 = sc1 on gfx950.
DEV __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000);
}
constexpr int SC1 = 16;
DEV u32x4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SC1); }
DEV uint32_t ld32(__amdgpu_buffer_rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, SC1); }
DEV void st32(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) { __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, SC1); }
DEV void st16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, off, 0, SC1);
}

// tagged records (8 bytes each): one {payload, tag} per store, or two adjacent ones in 16 bytes.
// A megakernel run tags with tag0 + layer + 1 (tag0 = plan salt + runs * 1024: never 0 in the low
// ten bits); the graph baseline, whose order comes from the stream, writes tag 0, which no
// megakernel run waits for.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
DEV uint32_t ll_tag(const KArgs& a, uint32_t layer) { return (a.flags & kModeGraph) ? 0u : a.tag0 + layer + 1u; }
DEV void ll_put(__amdgpu_buffer_rsrc_t r, uint32_t idx, uint32_t payload, uint32_t tag) {
  const u32x2 v = {payload, tag};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, idx * 8u, 0, SC1);
}
DEV void ll_put2(__amdgpu_buffer_rsrc_t r, uint32_t idx, uint32_t p0, uint32_t p1, uint32_t tag) {
  const u32x4 v = {p0, tag, p1, tag};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, idx * 8u, 0, SC1);
}
// the payload of record k of a vector staged into LDS
DEV float ll_f32(const char* base, int k) { return *(const float*)(base + 8 * k); }

DEV void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// the kernels' dynamic LDS (the same base as each kernel's own `smem`)
extern __shared__ __attribute__((aligned(1024))) char mk_lds[];

// Barrier of the eight waves that run the op bodies.  The multi-row kernel also has loader waves
// that never take a barrier, so there the eight meet on an LDS arrival counter: the arrivals of
// one barrier are 8k .. 8k + 7, and a wave waits for the count to reach 8(k + 1).  A wait that
// outlasts the watchdog marks the block aborted (control word 2) and lets the wave go.
DEV void group_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  uint32_t* cnt = (uint32_t*)(mk_lds + kCtrlOff + kBarOff);
  uint32_t old = 0;
  if (__lane_id() == 0) old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const uint32_t target = (__builtin_amdgcn_readfirstlane(old) & ~7u) + 8u;
  for (uint32_t it = 1;; ++it) {
    const uint32_t now = __builtin_amdgcn_readfirstlane(__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if ((int32_t)(now - target) >= 0) break;
    __builtin_amdgcn_s_sleep(1);
    if ((it & 0xFFFFFu) == 0u) {  // about every 0.1 s: give up once the block has aborted or after ~2 s
      volatile uint32_t* ctrl = (volatile uint32_t*)(mk_lds + kCtrlOff);
      if (*ctrl != 0u) break;
      if (it >= 0x1400000u) {
        if (__lane_id() == 0) *ctrl = 2u;
        break;
      }
    }
  }
  asm volatile("" ::: "memory");
}
DEV void lds_barrier() {
  if (blockDim.x > (uint32_t)kThreads) group_barrier();
  else asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// the wave's own LDS writes done, and no LDS access moved across this point (a wave-private
// exchange between lanes: LDS serves one wave's accesses in order once they are issued)
DEV void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// wait until at most n vector-memory operations of this wave are outstanding
DEV void wait_vm_le(uint32_t n) {
  switch (n > 63u ? 63u : n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
    case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
    case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
    case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
    case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
    case 15: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    case 16: asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); break;
    case 17: asm volatile("s_waitcnt vmcnt(17)" ::: "memory"); break;
    case 18: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
    case 19: asm volatile("s_waitcnt vmcnt(19)" ::: "memory"); break;
    case 20: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
    case 21: asm volatile("s_waitcnt vmcnt(21)" ::: "memory"); break;
    case 22: asm volatile("s_waitcnt vmcnt(22)" ::: "memory"); break;
    case 23: asm volatile("s_waitcnt vmcnt(23)" ::: "memory"); break;
    case 24: asm volatile("s_waitcnt vmcnt(24)" ::: "memory"); break;
    case 25: asm volatile("s_waitcnt vmcnt(25)" ::: "memory"); break;
    case 26: asm volatile("s_waitcnt vmcnt(26)" ::: "memory"); break;
    case 27: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    case 28: asm volatile("s_waitcnt vmcnt(28)" ::: "memory"); break;
    case 29: asm volatile("s_waitcnt vmcnt(29)" ::: "memory"); break;
    case 30: asm volatile("s_waitcnt vmcnt(30)" ::: "memory"); break;
    case 31: asm volatile("s_waitcnt vmcnt(31)" ::: "memory"); break;
    case 32: asm volatile("s_waitcnt vmcnt(32)" ::: "memory"); break;
    case 33: asm volatile("s_waitcnt vmcnt(33)" ::: "memory"); break;
    case 34: asm volatile("s_waitcnt vmcnt(34)" ::: "memory"); break;
    case 35: asm volatile("s_waitcnt vmcnt(35)" ::: "memory"); break;
    case 36: asm volatile("s_waitcnt vmcnt(36)" ::: "memory"); break;
    case 37: asm volatile("s_waitcnt vmcnt(37)" ::: "memory"); break;
    case 38: asm volatile("s_waitcnt vmcnt(38)" ::: "memory"); break;
    case 39: asm volatile("s_waitcnt vmcnt(39)" ::: "memory"); break;
    case 40: asm volatile("s_waitcnt vmcnt(40)" ::: "memory"); break;
    case 41: asm volatile("s_waitcnt vmcnt(41)" ::: "memory"); break;
    case 42: asm volatile("s_waitcnt vmcnt(42)" ::: "memory"); break;
    case 43: asm volatile("s_waitcnt vmcnt(43)" ::: "memory"); break;
    case 44: asm volatile("s_waitcnt vmcnt(44)" ::: "memory"); break;
    case 45: asm volatile("s_waitcnt vmcnt(45)" ::: "memory"); break;
    case 46: asm volatile("s_waitcnt vmcnt(46)" ::: "memory"); break;
    case 47: asm volatile("s_waitcnt vmcnt(47)" ::: "memory"); break;
    case 48: asm volatile("s_waitcnt vmcnt(48)" ::: "memory"); break;
    case 49: asm volatile("s_waitcnt vmcnt(49)" ::: "memory"); break;
    case 50: asm volatile("s_waitcnt vmcnt(50)" ::: "memory"); break;
    case 51: asm volatile("s_waitcnt vmcnt(51)" ::: "memory"); break;
    case 52: asm volatile("s_waitcnt vmcnt(52)" ::: "memory"); break;
    case 53: asm volatile("s_waitcnt vmcnt(53)" ::: "memory"); break;
    case 54: asm volatile("s_waitcnt vmcnt(54)" ::: "memory"); break;
    case 55: asm volatile("s_waitcnt vmcnt(55)" ::: "memory"); break;
    case 56: asm volatile("s_waitcnt vmcnt(56)" ::: "memory"); break;
    case 57: asm volatile("s_waitcnt vmcnt(57)" ::: "memory"); break;
    case 58: asm volatile("s_waitcnt vmcnt(58)" ::: "memory"); break;
    case 59: asm volatile("s_waitcnt vmcnt(59)" ::: "memory"); break;
    case 60: asm volatile("s_waitcnt vmcnt(60)" ::: "memory"); break;
    case 61: asm volatile("s_waitcnt vmcnt(61)" ::: "memory"); break;
    case 62: asm volatile("s_waitcnt vmcnt(62)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(63)" ::: "memory"); break;
  }
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane.  Written
// as inline assembly so that the compiler does not track these loads: it cannot tell which
// LDS pages they write and would otherwise wait for every outstanding prefetch before any
// LDS read.  The per-wave issue counts and wait_vm_le() order them instead.
// M0 (the LDS base of the transfer, read at issue) is saved and restored around it.
DEV void lds_dma16(const void* src, uint32_t lds_base) {
  lds_base = uni(lds_base);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds_base), "v"(src)
               : "memory");
}

DEV uint32_t ring_off(uint32_t lease, uint32_t off) {
  return (((lease + (off >> 14)) & (kNPages - 1)) << 14) | (off & 16383u);
}

// ---------------------------------------------------------------------------------------
// prefetch descriptors: what an instruction streams into its LDS lease, in 1 KiB blocks
// An instruction's lease holds up to five spans, each starting on a 1 KiB block:
//   QKV, LM_HEAD: weight rows | norm gain       GATE_UP: gate rows | up rows | norm gain
//   O_PROJ, DOWN: weight rows                   ATTN: K rows | V rows
//   multi-row GEMM: 64 weight rows x one K chunk in matrix-core operand order   NORM: norm gain
// Attention K / V spans are gathered token by token through the block table.
constexpr int kMaxSpans = 5;
enum PfMode : uint32_t { PF_SPANS = 0, PF_ATTN = 1, PF_W_BF16 = 2, PF_W_FP8 = 3, PF_KEYS = 4 };
// weight fragments (multi-row family only): tile row tr < split is weight row base0 + tr, else
// base1 + tr; rowb bytes per weight row; k0b byte offset of the K chunk in a row.  The single-token
// family carries none of it, which keeps its descriptor small enough to stay in registers.
template <int S>
struct PfFrag {};
template <>
struct PfFrag<1> {
  uint32_t rowb, k0b, base0, base1, split, bpn;  // bpn: lease blocks per 16-row block of the tile
};
// Every span is a whole number of 1 KiB blocks (the launcher checks the shapes for it), so a
// block's 64 lanes always load 1 KiB of the span; no per-span length is kept (selecting one by span
// index would put the descriptor in private memory).
template <int S>
struct Pf : PfFrag<S> {
  const char* src[kMaxSpans];
  uint32_t blk[kMaxSpans + 1];  // first block of each span; blk[n] = total blocks
  int n;
  uint32_t total;  // blocks of all spans (kept apart from blk so that no access indexes blk by n)
  uint32_t mode;
  const int32_t* bt;  // attention: block-table row of the request
  int t0, nk, hk;
  uint64_t gout;  // MK_FLAG_DEBUG_GATHER: address of the gathered rows' physical slots (token t0 first), or 0
};
// one word of the gather record (MK_FLAG_DEBUG_GATHER only): a plain vector store issued as assembly, so
// that the compiler's lowering of the surrounding LDS-pointer arithmetic is left as it is without the flag
// (read by the host after the run; nothing in the kernel reads it back)
DEV void gather_put(uint64_t addr, uint32_t v) {
  asm volatile("global_store_dword %0, %1, off" ::"v"(addr), "v"(v) : "memory");
}
DEV uint32_t blocks_of(uint32_t bytes) { return (bytes + 1023u) >> 10; }

// span k of the descriptor (k is a compile-time constant at every call: no indexed registers)
template <int K, int S>
DEV void pf_set(Pf<S>& pf, const void* src, uint32_t bytes) {
  pf.src[K] = (const char*)src;
  pf.blk[K + 1] = pf.blk[K] + blocks_of(bytes);
  pf.n = K + 1;
  pf.total = pf.blk[K + 1];
}

// A block-table entry of request r, checked against the page pool: an entry outside [0, pages) is
// written to the error record (mk_sync reports it) and read as page 0, so that no cache access leaves
// the pool whatever the table holds.  `entry` is the table row of request r plus the logical page.
DEV uint32_t bt_check(const KArgs& a, uint32_t v, uint32_t r) {
  if (v < (uint32_t)a.sh.npages) return v;
  uint32_t z = 0;
  if (__hip_atomic_compare_exchange_strong(a.err, &z, kErrBlockTable, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(a.err + 3, r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.err + 4, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return 0u;
}
DEV uint32_t bt_page(const KArgs& a, const int32_t* entry, uint32_t r) { return bt_check(a, (uint32_t)s_ld32(entry), r); }

// K of a projection kind
DEV uint32_t proj_k(const Shapes& sh, uint32_t kind) {
  switch (kind) {
    case K_O: return (uint32_t)sh.Hq * 128u;
    case K_DOWN: return (uint32_t)sh.I;
    case K_QI: return (uint32_t)sh.qr;
    case K_QB: return (uint32_t)sh.qr;
    case K_UK: return (uint32_t)kMlaNope;
    default: return (uint32_t)sh.H;
  }
}
// row length of a NORM instruction: the hidden size, or the q rank for the indexer's q_a norm
DEV uint32_t norm_len(const Shapes& sh, const Instr& in) { return in.w[W_LAYER + 1] == 2 ? (uint32_t)sh.qr : (uint32_t)sh.H; }
// a NORM adding the caller's x to its r_in (the first norm, waiting on nothing: both are inputs of
// the launch) gets them through its lease, after the gain: r at 2H bytes, x at 6H bytes
DEV bool norm_inputs_in_lease(const Instr& in, const uint64_t* row) {
  return in.w[W_NWAIT] == 0u && in.w[W_LAYER + 1] == 0u && s_ld64(row + NM_X) != 0u;
}

// splits of an attention instruction's (request, kv head).  S is the op family of the kernel
// instance: 0 the single-token bodies, 1 the multi-row ones (the plan's spec id, fixed per plan).
template <int S>
DEV int attn_splits(const Instr& in) { return (int)in.w[S == 1 ? W_NSPLIT : W_ARR_N]; }

template <int S>
DEV void pf_desc(const KArgs& a, const Instr& in, Pf<S>& pf) {
  const uint32_t op = in.w[W_OPCODE];
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const Shapes& sh = a.sh;
  pf.blk[0] = 0;
  pf.n = 0;
  pf.total = 0;
  pf.gout = 0;
  pf.mode = op == OP_ATTN ? PF_ATTN : PF_SPANS;
  if constexpr (S == 1) if (op == OP_GEMM) {
    // 64 KiB: block b = 16 nb + q holds 64 bytes of each of the tile rows [16 nb, 16 nb + 16) (K
    // step q: 32 bf16 or 64 e4m3 weights), lane l taking row 16 nb + l % 16, bytes 16 (l / 16) ...
    const uint32_t kind = in.w[W_LAYER + 1], n0 = in.w[W_LAYER + 3], k0 = in.w[W_LAYER + 5], kc = in.w[W_LAYER + 6];
    const uint32_t K = proj_k(sh, kind);
    const bool f8 = sh.fp8 && kind != K_UK;  // the main-MLA query BMM has bf16 weights in an e4m3 plan
    const uint32_t el = f8 ? 1u : 2u;
    pf.mode = f8 ? PF_W_FP8 : PF_W_BF16;
    pf.rowb = K * el;
    pf.k0b = k0 * el;
    pf.base0 = n0;
    pf.split = kind == K_GU ? 32u : 64u;  // gate/up: 32 gate rows, then the 32 matching up rows
    pf.base1 = kind == K_GU ? (uint32_t)sh.I + n0 - 32u : n0;
    pf.bpn = kc * el / 64u;
    pf_set<0>(pf, (const void*)s_ld64(row + GM_W), 64u * kc * el);
    return;
  }
  if (S == 1 && op == OP_NORM) {
    const uint32_t H = norm_len(sh, in);
    pf_set<0>(pf, (const void*)s_ld64(row + NM_GAIN), 2u * H);
    if (norm_inputs_in_lease(in, row)) {  // the layer's own inputs: stream them in with the gain
      const uint32_t m = in.w[W_LAYER + 2];
      pf_set<1>(pf, (const float*)s_ld64(row + NM_R) + (size_t)m * H, 4u * H);
      pf_set<2>(pf, (const uint16_t*)s_ld64(row + NM_X) + (size_t)m * H, 2u * H);
    }
    return;
  }
  if (S == 1 && op == OP_SCORE) {
    // the split's keys from before this step, 8 tokens (1 KiB) per block, and their scales (32 bytes
    // per key block) in one block after them; the step's own keys are staged after the wait
    const uint32_t r = in.w[W_LAYER + 1], t0 = in.w[W_LAYER + 3], t1 = in.w[W_LAYER + 4];
    const uint32_t T = (uint32_t)sh.T;
    const uint32_t ctx = (uint32_t)c_ld<int32_t>((const int32_t*)s_ld64(row + SC_POS) + r * T + T - 1u) + 1u;
    const uint32_t lim = min(t1, ctx - T), nko = lim > t0 ? lim - t0 : 0u;
    pf.mode = PF_KEYS;
    pf.bt = (const int32_t*)s_ld64(row + SC_BT) + (size_t)r * sh.maxp;
    if (a.gather) pf.gout = (uint64_t)(uintptr_t)(a.gather + (size_t)r * (uint32_t)(sh.maxp * sh.P) + t0);  // [request][token]
    pf.t0 = (int)t0;
    pf.nk = (int)nko;
    pf_set<0>(pf, (const void*)s_ld64(row + SC_CACHE), nko * 128u);
    pf_set<1>(pf, (const void*)s_ld64(row + SC_SCALE), nko ? 1024u : 0u);
    return;
  }
  if (S == 1 && (op == OP_FIN || op == OP_QUANT || op == OP_KCACHE || op == OP_TOPK))
    return;  // nothing to prefetch: inputs are produced in the run
  if (pf.mode == PF_ATTN) {
    const int r = in.w[W_P1], hk = in.w[W_P2], s = in.w[W_P3];
    const int t0 = in.w[W_P4], t1 = in.w[W_P5];
    const bool last = s == attn_splits<S>(in) - 1;
    pf.bt = (const int32_t*)s_ld64(row + ATT_BT) + (size_t)r * sh.maxp;
    if (a.gather)  // [layer][request][kv head][K, V][token]
      pf.gout = (uint64_t)(uintptr_t)(a.gather + ((((size_t)in.w[W_LAYER] * (uint32_t)(sh.M / sh.T) + (uint32_t)r) *
                                                       (uint32_t)sh.Hkv + (uint32_t)hk) * 2u) * (uint32_t)(sh.maxp * sh.P) + t0);
    pf.t0 = t0;
    pf.hk = hk;
    pf.nk = (last ? t1 - 1 : t1) - t0;
    pf_set<0>(pf, (const void*)s_ld64(row + ATT_KC), (uint32_t)pf.nk * 256u);
    pf_set<1>(pf, (const void*)s_ld64(row + ATT_VC), (uint32_t)pf.nk * 256u);
    (void)r;
    return;
  }
  if (S == 1 && op == OP_COMB) return;
  if (op == OP_LMHEAD) {  // the rows stream from HBM inside the body; the lease holds the norm gain
    pf_set<0>(pf, (const void*)s_ld64(row + LM_GAMMA), 2u * (uint32_t)sh.H);
    return;
  }
  const char* w = (const char*)s_ld64(row + 0);
  const uint32_t n0 = in.w[W_P1], nr = in.w[W_P2], K = in.w[W_P4];
  const uint32_t rowb = K * 2u;
  pf_set<0>(pf, w + (size_t)n0 * rowb, nr * rowb);
  if (op == OP_GATEUP) {
    pf_set<1>(pf, w + (size_t)(sh.I + n0) * rowb, nr * rowb);
    pf_set<2>(pf, (const void*)s_ld64(row + GU_GAMMA), 2u * (uint32_t)sh.H);
  } else if (op == OP_QKV) {
    pf_set<1>(pf, (const void*)s_ld64(row + QKV_GAMMA), 2u * (uint32_t)sh.H);
  }
}

// issue this wave's share of an instruction's prefetch into its lease: a contiguous run of blocks
// (about a seventh of them), span by span, with the per-block address work kept incremental (a
// block-table entry is read once per page, a weight row address once per 16-row block) so that a
// wave issues its loads back to back
template <int S>
DEV void pf_issue(const KArgs& a, const Pf<S>& pf, uint32_t lease, int cw, uint32_t& issued, char* smem, int nw = kNCW) {
  const uint32_t ln = lane();
  const uint32_t per = (pf.total + (uint32_t)nw - 1u) / (uint32_t)nw;
  const uint32_t lo = min((uint32_t)cw * per, pf.total), hi = min(lo + per, pf.total);
  const uint32_t ring = (uint32_t)(uintptr_t)(lds_void*)(smem + kRingOff);
#pragma unroll
  for (int k = 0; k < kMaxSpans; ++k) {
    if (k >= pf.n) break;
    const uint32_t b0 = max(lo, pf.blk[k]), b1 = min(hi, pf.blk[k + 1]);
    if (b0 >= b1) continue;
    const char* base = pf.src[k];
    if constexpr (S == 1) {
      if (pf.mode == PF_W_BF16 || pf.mode == PF_W_FP8) {
        // block b = 16-row block nb, K step q: lane l takes row 16 nb + l % 16, bytes 16 (l / 16) of the step
        uint32_t nb = b0 / pf.bpn, q = b0 - nb * pf.bpn;
        const char* rowp = nullptr;
        uint32_t rnb = 0xFFFFFFFFu;
        for (uint32_t b = b0; b < b1; ++b) {
          if (nb != rnb) {
            const uint32_t tr = nb * 16u + (ln & 15u);
            const uint32_t grow = tr < pf.split ? pf.base0 + tr : pf.base1 + tr;
            rowp = base + (size_t)grow * pf.rowb + pf.k0b + (ln >> 4) * 16u;
            rnb = nb;
          }
          lds_dma16(rowp + q * 64u, ring + ring_off(lease, b * 1024u));
          ++issued;
          if (++q == pf.bpn) {
            q = 0;
            ++nb;
          }
        }
        continue;
      }
      if (pf.mode == PF_KEYS) {
        if (k == 1) break;  // the scale block is filled alongside the key blocks
        // 8 tokens of one page (8 divides the page size and t0): 1 KiB contiguous in the cache
        const uint32_t P = (uint32_t)a.sh.P;
        uint32_t pidx = 0xFFFFFFFFu, page = 0;
        for (uint32_t b = b0; b < b1; ++b) {
          const uint32_t tok = (uint32_t)pf.t0 + 8u * b;
          if (tok / P != pidx) {
            pidx = tok / P;
            page = bt_page(a, pf.bt + pidx, kNone);
          }
          const uint32_t slot = page * P + tok % P;
          // chunk c of key u sits at position c ^ (u mod 8) of the key's 128 bytes, so that the score's
          // reads of one chunk of 16 consecutive keys spread over the LDS banks
          const uint32_t off = 8u * b + (ln >> 3) < (uint32_t)pf.nk ? (ln >> 3) * 128u + (((ln & 7u) ^ (ln >> 3)) << 4)
                                                                      : 0u;  // past the split: reload the block start
          const uint32_t sdst = ring + ring_off(lease, pf.blk[1] * 1024u + b * 32u);
          if (ln < 2u)  // the 8 tokens' scales (32 bytes) into the scale block: one more load of the wave
            lds_dma16(pf.src[1] + (size_t)slot * 4u + ln * 16u, sdst);
          lds_dma16(base + (size_t)slot * 128u + off, ring + ring_off(lease, b * 1024u));
          issued += 2u;
          if (pf.gout != 0u && (ln & 7u) == 0u && 8u * b + (ln >> 3) < (uint32_t)pf.nk)
            gather_put(pf.gout + 4u * (8u * b + (ln >> 3)), slot + (ln >> 3));
        }
        continue;
      }
    }
    if (pf.mode == PF_ATTN && k < 2) {
      // block bb of the K (or V) span: the split's rows 4 bb .. 4 bb + 3 (one page: 4 divides the page
      // size and t0), chunk c of row u at position c ^ (u mod 16); lane ln takes row 4 bb + ln / 16,
      // chunk ln mod 16.  Addresses advance row by row inside a page; the block table is read once
      // per page.
      const uint32_t P = (uint32_t)a.sh.P, rowb = (uint32_t)a.sh.Hkv * 256u;  // bytes between a head's tokens
      const uint32_t r16 = ln >> 4, c16 = ln & 15u;
      uint32_t bb = b0 - pf.blk[k];
      const uint32_t tok = (uint32_t)pf.t0 + 4u * bb;
      uint32_t pidx = tok / P, pos = tok - pidx * P;
      uint32_t pg = bt_page(a, pf.bt + pidx, kNone);  // physical page of block-table entry pidx
      auto page_base = [&](uint32_t page) {  // the span's head in physical page `page`
        return base + ((size_t)page * P * (uint32_t)a.sh.Hkv + (uint32_t)pf.hk) * 256u;
      };
      const char* pb = page_base(pg);
      const uint64_t go = pf.gout ? pf.gout + 4u * (k ? (uint32_t)(a.sh.maxp * a.sh.P) : 0u) : 0u;  // K or V slots
      for (uint32_t b = b0; b < b1; ++b, ++bb) {
        const uint32_t u = 4u * bb + r16;
        const uint32_t rp = u < (uint32_t)pf.nk ? pos + r16 : pos;  // beyond the tile: reload the block's first row
        lds_dma16(pb + rp * rowb + ((c16 ^ (u & 15u)) << 4), ring + ring_off(lease, b * 1024u));
        ++issued;
        // the slot this lane fetched, recorded by all 16 lanes of its row (one word); a row past the split's
        // tokens (the last block of the last split) re-fetches the block's first row and records that
        if (go != 0u) gather_put(go + 4u * u, pg * P + rp);
        pos += 4u;
        if (pos == P && b + 1u < b1) {  // the next block starts the next page
          pos = 0;
          pg = bt_page(a, pf.bt + ++pidx, kNone);
          pb = page_base(pg);
        }
      }
      continue;
    }
    for (uint32_t b = b0; b < b1; ++b) {
      lds_dma16(base + (b - pf.blk[k]) * 1024u + ln * 16u, ring + ring_off(lease, b * 1024u));
      ++issued;
    }
  }
}

// total blocks of a descriptor
template <int S>
DEV uint32_t pf_blocks(const Pf<S>& pf) {
  return pf.total;
}

// ---------------------------------------------------------------------------------------
// controller prologues (activation staging into LDS)
//
// Activations are staged with device-scope direct-to-LDS loads: one short loop issues every
// 1 KiB block, then a single wait -- one memory round trip, no registers, little code.

DEV void lds_dma16_sc1(const void* src, uint32_t lds_base) {
  lds_base = uni(lds_base);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off sc1\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "s"(lds_base), "v"(src)
               : "memory");
}
// copy `bytes` (16-byte aligned source) into LDS at `dst`; the destination region must extend to
// the next 1 KiB boundary (lanes past the end reload the block's first 16 bytes there)
DEV void stage(const void* src, uint32_t bytes, char* dst) {
  const uint32_t ln = lane();
  for (uint32_t b = 0; b < bytes; b += 1024u) {
    uint32_t off = b + ln * 16u;
    if (off >= bytes) off = b;
    lds_dma16_sc1((const char*)src + off, (uint32_t)(uintptr_t)(lds_void*)(dst + b));
  }
}
DEV uint32_t kb_round(uint32_t bytes) { return (bytes + 1023u) & ~1023u; }

// A run of tagged records to stage: `bytes` (8 per record) from global `src` into the activation
// area at `dst` (1 KiB aligned, room for whole 1 KiB blocks); current when every tag is `tag`.
struct LlRegion {
  const char* src;
  uint32_t bytes, dst, tag;
};

// how long a wait may take: 2 s of the 100 MHz clock, or one tick under MK_FLAG_DEBUG_SHORT_WATCHDOG
DEV unsigned long long watchdog_ticks(const KArgs& a) {
  return (a.flags & MK_FLAG_DEBUG_SHORT_WATCHDOG) ? 1ull : kWatchdogTicks;
}

DEV void record_timeout(const KArgs& a, const Instr& in, uint32_t what, uint32_t value) {
  if (lane() != 0) return;
  uint32_t z = 0;
  if (__hip_atomic_compare_exchange_strong(a.err, &z, 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(a.err + 1, blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.err + 2, in.w[W_TASK], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.err + 3, what, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.err + 4, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The 1 KiB blocks of a staged run of records (bit b: block b) holding a record whose tag is not
// `tag`: every lane checks its two records of every block (four blocks' reads in flight at a
// time), then one wave-wide OR of the per-lane masks.  Kept out of line: its registers stay out of
// the allocation of the kernel's hot loops.
__device__ __attribute__((noinline)) uint32_t stale_blocks(const char* base, uint32_t bytes, uint32_t tag) {
  const uint32_t ln = lane(), nb = blocks_of(bytes);
  uint32_t stale = 0u;
  for (uint32_t b0 = 0; b0 < nb; b0 += 4u) {
    u32x4 v[4];
    uint32_t off[4], b[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      b[q] = min(b0 + (uint32_t)q, nb - 1u);  // past the last block: check it again
      off[q] = b[q] * 1024u + ln * 16u;
      if (off[q] >= bytes) off[q] = b[q] * 1024u;  // lanes past the end look at the block's first records
      v[q] = *(const u32x4*)(base + off[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // nonzero when a tag differs; the second record counts only when it lies inside the run
      const uint32_t inside = (uint32_t)((int32_t)(off[q] + 8u - bytes) >> 31);
      stale |= min((v[q].y ^ tag) | ((v[q].w ^ tag) & inside), 1u) << b[q];
    }
  }
  return wave_or_u32(stale);
}

// The wait of an instruction: stage every block of its regions in one round trip; with `verify`
// (the megakernel), stage again the blocks holding a record whose tag is not current, until all
// are.  False when the watchdog expired or another worker aborted.
// One trace word of instruction i (MK_FLAG_TRACE runs): stored when it is taken, so that no stamp
// stays live in registers across the instruction's body.
DEV void tput(const KArgs& a, uint32_t i, int w, unsigned long long v) {
  if (a.trace && lane() == 0) a.trace[((size_t)blockIdx.x * a.L + i) * kTraceWords + w] = (uint32_t)v;
}
struct StageStamps {  // trace: the instruction whose staging is stamped (words 12, 13: issued, landed)
  uint32_t i;
};

DEV bool ll_stage(const KArgs& a, const Instr& in, const LlRegion* rg, int nrg, char* act, bool verify, uint32_t& polls,
                  StageStamps& ss) {
  const uint32_t ln = lane();
  uint32_t pend[3] = {0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < nrg) pend[j] = (1u << blocks_of(rg[j].bytes)) - 1u;  // at most 27 blocks
  const unsigned long long t0 = rtc();
  if (a.flags & MK_FLAG_TRACE) tput(a, ss.i, 12, t0);
  for (uint32_t it = 1;; ++it) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      for (uint32_t m = j < nrg ? pend[j] : 0u; m; m &= m - 1u) {
        const uint32_t b = (uint32_t)__builtin_ctz(m);
        uint32_t off = b * 1024u + ln * 16u;
        if (off >= rg[j].bytes) off = b * 1024u;
        lds_dma16_sc1(rg[j].src + off, (uint32_t)(uintptr_t)(lds_void*)(act + rg[j].dst + b * 1024u));
      }
    }
    wait_vm0();
    if ((a.flags & MK_FLAG_TRACE) && it == 1) tput(a, ss.i, 13, rtc());
    if (!verify) return true;
    bool done = true;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (j >= nrg || pend[j] == 0u) continue;
      pend[j] &= uni(stale_blocks(act + rg[j].dst, rg[j].bytes, rg[j].tag));
      if (pend[j]) done = false;
    }
    if (done) return true;
    ++polls;
    if ((it & 15u) == 0 && __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
    if (rtc() - t0 > watchdog_ticks(a)) {
      record_timeout(a, in, rg[0].tag, polls);
      return false;
    }
  }
}

// Fused add + RMSNorm.  The residual r sits at act + kb_round(2H): fp32 as the caller gave it
// (PLAIN: the first layer, with its x at act[0, 2H)) or as tagged records (later layers, no x).
// The controller takes the sum of squares once staged; all eight waves then write
// h = bf16((r + x) * rsqrt(mean((r + x)^2) + eps) * gain) over act[0, 2H).
template <bool PLAIN>
DEV void norm_chunk(const char* act, uint32_t R0, int c, float v[8]) {
  if (PLAIN) {
    const u32x4 ra = *(const u32x4*)(act + R0 + c * 32), rb = *(const u32x4*)(act + R0 + c * 32 + 16);
    const u32x4 xv = *(const u32x4*)(act + c * 16);
    v[0] = __uint_as_float(ra.x) + bf2f(xv.x & 0xffffu);
    v[1] = __uint_as_float(ra.y) + bf2f(xv.x >> 16);
    v[2] = __uint_as_float(ra.z) + bf2f(xv.y & 0xffffu);
    v[3] = __uint_as_float(ra.w) + bf2f(xv.y >> 16);
    v[4] = __uint_as_float(rb.x) + bf2f(xv.z & 0xffffu);
    v[5] = __uint_as_float(rb.y) + bf2f(xv.z >> 16);
    v[6] = __uint_as_float(rb.z) + bf2f(xv.w & 0xffffu);
    v[7] = __uint_as_float(rb.w) + bf2f(xv.w >> 16);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 rr = *(const u32x4*)(act + R0 + c * 64 + q * 16);
      v[2 * q] = __uint_as_float(rr.x);
      v[2 * q + 1] = __uint_as_float(rr.z);
    }
  }
}

template <bool PLAIN>
DEV void norm_ss(char* act, int H, float eps, char* smem) {
  const uint32_t R0 = kb_round(2u * H);
  const int ln = (int)lane(), nk8 = H / 8;
  float ss = 0.f;
#pragma unroll 2
  for (int c = ln; c < nk8; c += 64) {
    float v[8];
    norm_chunk<PLAIN>(act, R0, c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) ss += v[q] * v[q];
  }
  const float inv = rsqrtf(wave_sum(ss) / (float)H + eps);
  if (ln == 0) *(float*)(smem + kCtrlOff + kInvOff) = inv;
}

template <bool PLAIN>
DEV void norm_h(const char* smem, uint32_t lease, uint32_t goff, int H, int wv) {
  char* act = (char*)smem + kActOff;
  const uint32_t R0 = kb_round(2u * H);
  const float inv = *(const float*)(smem + kCtrlOff + kInvOff);
  const int nk8 = H / 8;
  for (int c = wv * 64 + (int)lane(); c < nk8; c += kNW * 64) {
    float v[8];
    norm_chunk<PLAIN>(act, R0, c, v);
    const u32x4 gv = *(const u32x4*)(smem + kRingOff + ring_off(lease, goff + (uint32_t)c * 16u));
    const uint32_t gs[4] = {gv.x, gv.y, gv.z, gv.w};
    u32x4 o;
    o.x = pack_bf2(v[0] * inv * bf2f(gs[0] & 0xffffu), v[1] * inv * bf2f(gs[0] >> 16));
    o.y = pack_bf2(v[2] * inv * bf2f(gs[1] & 0xffffu), v[3] * inv * bf2f(gs[1] >> 16));
    o.z = pack_bf2(v[4] * inv * bf2f(gs[2] & 0xffffu), v[5] * inv * bf2f(gs[2] >> 16));
    o.w = pack_bf2(v[6] * inv * bf2f(gs[3] & 0xffffu), v[7] * inv * bf2f(gs[3] >> 16));
    *(u32x4*)(act + c * 16) = o;
  }
}

// QKV, GATE_UP, LM_HEAD (its first tile): stage the norm input and take its sum of squares.
// First-layer QKV reads the caller's x and r_in; otherwise the tagged residual: r1 of the layer
// before (QKV, LM_HEAD) or r2 of this layer (GATE_UP).
DEV bool norm_prologue(const KArgs& a, const Instr& in, const uint64_t* row, char* act, char* smem, bool verify,
                       bool noop, uint32_t& polls, StageStamps& ss) {
  const uint32_t op = in.w[W_OPCODE], layer = in.w[W_LAYER];
  const int H = a.sh.H;
  const uint32_t R0 = kb_round(2u * H);
  if (op == OP_QKV && layer == 0) {
    stage((const void*)s_ld64(row + QKV_X), 2u * H, act);
    stage((const void*)s_ld64(row + QKV_RIN), 4u * H, act + R0);
    wait_vm0();
    if (!noop) norm_ss<true>(act, H, a.sh.eps, smem);
    return true;
  }
  const int slot = op == OP_QKV ? QKV_R1 : (op == OP_GATEUP ? GU_R2 : LM_R1);
  const LlRegion rg{(const char*)s_ld64(row + slot), 8u * H, R0, ll_tag(a, op == OP_GATEUP ? layer : layer - 1u)};
  if (!ll_stage(a, in, &rg, 1, act, verify, polls, ss)) return false;
  if (!noop) norm_ss<false>(act, H, a.sh.eps, smem);
  return true;
}

// O projection: the tagged o (bf16 pairs) at act[0, ...), and r1 of the tile's rows as records at
// act + kActR1 (tagged records of the layer before; the first layer adds the caller's r_in + x)
DEV bool oproj_prologue(const KArgs& a, const Instr& in, const uint64_t* row, char* act, bool verify, uint32_t& polls,
                        StageStamps& ss) {
  const uint32_t layer = in.w[W_LAYER];
  const int n0 = in.w[W_P1], nr = in.w[W_P2];
  const uint32_t n = (uint32_t)a.sh.Hq * 128u;
  LlRegion rg[2];
  rg[0] = LlRegion{(const char*)s_ld64(row + O_IN), 4u * n, 0u, ll_tag(a, layer)};
  int nrg = 1;
  if (layer > 0) rg[nrg++] = LlRegion{(const char*)s_ld64(row + O_R1) + (size_t)n0 * 8, 8u * nr, (uint32_t)kActR1,
                                      ll_tag(a, layer - 1u)};
  if (!ll_stage(a, in, rg, nrg, act, verify, polls, ss)) return false;
  if (layer == 0) {
    __amdgpu_buffer_rsrc_t rx = rsrc((const void*)s_ld64(row + O_X));
    __amdgpu_buffer_rsrc_t rr = rsrc((const void*)s_ld64(row + O_RIN));
    float xr[2], rv[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int jj = (int)lane() + 64 * q;
      if (jj < nr) {
        xr[q] = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rx, (uint32_t)(n0 + jj) * 2u, 0, SC1));
        rv[q] = __uint_as_float(ld32(rr, (uint32_t)(n0 + jj) * 4u));
      }
    }
    wait_vm0();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int jj = (int)lane() + 64 * q;
      if (jj < nr) *(float*)(act + kActR1 + 8 * jj) = rv[q] + xr[q];
    }
  }
  return true;
}

// down projection: the tagged m (bf16 pairs) at act[0, ...) and r2 of the tile's rows at act + kActR1
DEV bool down_prologue(const KArgs& a, const Instr& in, const uint64_t* row, char* act, bool verify, uint32_t& polls,
                       StageStamps& ss) {
  const uint32_t tag = ll_tag(a, in.w[W_LAYER]);
  const int n0 = in.w[W_P1], nr = in.w[W_P2];
  const LlRegion rg[2] = {{(const char*)s_ld64(row + DN_M), 4u * (uint32_t)a.sh.I, 0u, tag},
                          {(const char*)s_ld64(row + DN_R2) + (size_t)n0 * 8, 8u * nr, (uint32_t)kActR1, tag}};
  return ll_stage(a, in, rg, 2, act, verify, polls, ss);
}

// at most 1 KiB (a multiple of 16 bytes) into LDS at dst: only the lanes that carry data write
DEV void stage_small(const void* src, uint32_t bytes, char* dst) {
  const uint32_t ln = lane();
  if (ln * 16u < bytes) lds_dma16_sc1((const char*)src + ln * 16u, (uint32_t)(uintptr_t)(lds_void*)dst);
}

// attention: the q / k norm gains and the request's RoPE row, then the tagged raw (fp32) q heads of
// the group and its k / v heads (one round trip: the record staging waits for all of it)
DEV bool attn_stage(const KArgs& a, const Instr& in, char* act, bool verify, uint32_t& polls, StageStamps& ss) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const int r = in.w[W_P1], hk = in.w[W_P2];
  stage_small((const void*)s_ld64(row + ATT_GQ), 256u, act + kAttGq);
  stage_small((const void*)s_ld64(row + ATT_GK), 256u, act + kAttGk);
  stage_small((const float*)s_ld64(row + ATT_ROPE) + (size_t)r * 128, 512u, act + kAttRope);
  const char* qkv = (const char*)s_ld64(row + ATT_QKV) + (size_t)r * sh.n_qkv * 8;
  const uint32_t tag = ll_tag(a, in.w[W_LAYER]);
  const LlRegion rg[3] = {{qkv + (size_t)hk * sh.g * 128 * 8, (uint32_t)sh.g * 1024u, (uint32_t)kAttQraw, tag},
                          {qkv + (size_t)(sh.Hq + hk) * 128 * 8, 1024u, (uint32_t)kAttKraw, tag},
                          {qkv + (size_t)(sh.Hq + sh.Hkv + hk) * 128 * 8, 1024u, (uint32_t)kAttVraw, tag}};
  return ll_stage(a, in, rg, 3, act, verify, polls, ss);
}

// ---------------------------------------------------------------------------------------
// compute bodies (waves 1..7; cw = 0..6)

// Projection tile on all eight waves: part[Q] = sum over quad Q of h[k] * W[r][k], for the tile's
// R rows of K elements cut into quads of 512 (Q = r * KQ + kq, KQ = K / 512); rows [0, nr0) sit
// at r * rowb in the lease, rows [nr0, R) at off1 + (r - nr0) * rowb; h (bf16) is at the start of
// the activation area.  Wave w takes quads w, w + 8, ...; inside a quad, 16-lane row rho takes
// the 128 elements [kq * 512 + 128 rho, + 128), lane `sub` eight of them.  Four quads at a time
// are summed over the 16 lanes of each row by a transposing butterfly (about four instructions
// per quad), then over the four rows by cross-row lane swaps.  Every address is wave-uniform
// but for a per-lane constant.  The epilogue adds a row's KQ quad sums in order.
DEV float butterfly4(float a0, float a1, float a2, float a3, int sub) {
  const bool lo8 = sub < 8, lo4 = (sub & 4) == 0;
  // partner 15 - sub (row mirror): lanes < 8 keep blocks 0, 1 and hand over 2, 3
  float k0 = lo8 ? a0 : a2, k1 = lo8 ? a1 : a3;
  const float s0 = lo8 ? a2 : a0, s1 = lo8 ? a3 : a1;
  k0 += dppf<0x140>(s0);
  k1 += dppf<0x140>(s1);
  // partner 7 - sub within the half row: lanes with bit 2 clear keep k0
  float k = lo4 ? k0 : k1;
  const float t = lo4 ? k1 : k0;
  k += dppf<0x141>(t);
  // the quad's four lanes hold the same block: finish over the quad
  k += dppf<0x4E>(k);
  k += dppf<0xB1>(k);
  return k;  // lanes 4i .. 4i + 3 of the row hold block i
}

template <bool LLX>  // x as tagged records (bf16 pairs) rather than plain bf16
DEV void gemv(const char* smem, uint32_t lease, int R, int nr0, uint32_t off1, int K, int wv, float* part) {
  const int ln = (int)lane(), sub = ln & 15;
  const uint32_t KQ = (uint32_t)K >> 9, NQ = (uint32_t)R * KQ;
  const uint32_t rowb = (uint32_t)K * 2u;
  const uint32_t magic = (65536u + KQ - 1u) / KQ;  // Q / KQ == (Q * magic) >> 16 for Q < 2^16 / KQ
  const uint32_t up = off1 - (uint32_t)nr0 * rowb;  // rows past nr0 start at off1
  const char* act = smem + kActOff;
  const uint32_t lbase = (lease << 14) + (uint32_t)(ln >> 4) * 256u + (uint32_t)sub * 16u;
  const uint32_t xlane = (uint32_t)ln * 16u;  // row rho, lane sub: rho * 256 + sub * 16
  for (uint32_t q0 = (uint32_t)wv; q0 < NQ; q0 += 4u * kNW) {
    u32x4 w[4], x[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t Q = min(q0 + (uint32_t)m * kNW, NQ - 1u);  // wave-uniform: scalar arithmetic
      const uint32_t r = (Q * magic) >> 16, kq = Q - r * KQ;
      const uint32_t wo = r * rowb + (r >= (uint32_t)nr0 ? up : 0u) + kq * 1024u;
      w[m] = *(const u32x4*)(smem + kRingOff + ((lbase + wo) & (uint32_t)(kNPages * 16384 - 1)));
      if (LLX) {
        const char* xp = act + 2u * (kq * 1024u + xlane);
        const u32x4 ra = *(const u32x4*)xp, rb = *(const u32x4*)(xp + 16);
        x[m] = u32x4{ra.x, ra.z, rb.x, rb.z};
      } else {
        x[m] = *(const u32x4*)(act + kq * 1024u + xlane);
      }
    }
    const float v = rows_sum(butterfly4(dot8(w[0], x[0], 0.f), dot8(w[1], x[1], 0.f), dot8(w[2], x[2], 0.f),
                                        dot8(w[3], x[3], 0.f), sub));
    const uint32_t Q = q0 + (uint32_t)(sub >> 2) * kNW;  // lanes 4i hold quad q0 + 8 i
    if (ln < 16 && (sub & 3) == 0 && Q < NQ) part[Q] = v;
  }
}

// a row of a projection tile: its KQ quad sums in order.  The loads are unconditional (the output
// area extends past the last row's sums) so that they go out together; entries past KQ add 0.
DEV float row_sum(const float* part, int r, int KQ) {
  const float* p = part + r * KQ;
  float v[kMaxKQ];
#pragma unroll
  for (int k = 0; k < kMaxKQ; ++k) v[k] = p[k];
  float s = v[0];
#pragma unroll
  for (int k = 1; k < kMaxKQ; ++k) s += k < KQ ? v[k] : 0.f;
  return s;
}

// lm_head rows n0 + st j (j < nr) of one instruction on one wave (all eight take part), streamed from
// HBM into registers rather than through an LDS lease: one instruction per worker covers its whole
// share of the vocabulary, so the per-instruction costs (staging, barriers, epilogue) are paid once
// and the loads of four steps stay in flight while a step is summed.  h (bf16, K = 512 KQ) sits at
// the start of the activation area; lane l holds its elements 512 kq + 8 l .. + 8 in registers for
// the whole run.  A step is P = 4 / KQ consecutive rows (KQ = 3: one row and an empty fourth block),
// i.e. four quads laid out as in the leased tile (lane l reads bytes 16 l .. + 16 of each quad),
// summed by the same butterfly and cross-row swaps, and a row's quad sums are added in quad order:
// the same arithmetic as the tiled GEMV.  The plan interleaves the workers' rows (stride = number of
// tasks), so that at any time all compute units stream one narrow window of the matrix; the weights
// are read once, with non-temporal loads.  Wave wv takes steps wv, wv + 8, ...; loads past a
// wave's last step repeat the instruction's last step (cache hits, in bounds).  Logits go straight
// to memory; the wave's (max, first index) lands in the output area for the epilogue.
DEV void argmax_merge(float& best, int& bi);
// Out of line: its load buffers stay out of the register allocation of the kernel's other bodies
// (inlined, it raised the single-token kernel's spilled scalar registers from 163 to 200).
typedef __attribute__((address_space(3))) float lds_float;
template <int KQ>
__device__ __attribute__((noinline)) void lm_rows(const char* wm, float* logits, int n0, int nr, int stride,
                                                  lds_cchar* act, lds_float* out, int wv) {
  constexpr int P = KQ == 3 ? 1 : 4 / KQ;
  // the pointers arrive in vector registers: made wave-uniform (scalar) and typed as global memory, so
  // that the loads are global loads whose counter the compiler tracks one by one (generic-pointer
  // loads would wait for every load in flight before the first use)
  typedef const __attribute__((address_space(1))) char gchar;
  const uint64_t wa = (uint64_t)(uintptr_t)wm, la = (uint64_t)(uintptr_t)logits;
  gchar* wg = (gchar*)(uintptr_t)(((uint64_t)uni((uint32_t)(wa >> 32)) << 32) | uni((uint32_t)wa));
  __amdgpu_buffer_rsrc_t rl = rsrc((const void*)(uintptr_t)(((uint64_t)uni((uint32_t)(la >> 32)) << 32) | uni((uint32_t)la)));
  n0 = (int)uni((uint32_t)n0);
  nr = (int)uni((uint32_t)nr);
  stride = (int)uni((uint32_t)stride);
  wv = (int)uni((uint32_t)wv);
  const int ln = (int)lane(), sub = ln & 15;
  u32x4 xr[KQ];
#pragma unroll
  for (int kq = 0; kq < KQ; ++kq) xr[kq] = *(const __attribute__((address_space(3))) u32x4*)(act + kq * 1024 + ln * 16);
  const int nst = (nr + P - 1) / P;
  const int my = nst > wv ? (nst - wv + kNW - 1) / kNW : 0;
  const size_t rowb = (size_t)KQ * 1024u;
  auto load = [&](u32x4 (&w)[4], int i) {
    const int t = min(wv + kNW * i, nst - 1);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = min(t * P + (KQ == 3 ? 0 : m / KQ), nr - 1);
      const int kq = KQ == 3 ? min(m, 2) : m % KQ;
      w[m] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(
          wg + (size_t)(n0 + r * stride) * rowb + (size_t)kq * 1024u + (size_t)ln * 16u));
    }
  };
  float best = -INFINITY;
  int bi = 0x7fffffff;
  auto consume = [&](const u32x4 (&w)[4], int i) {
    if (i >= my) return;
    const int t = wv + kNW * i;
    float d[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      d[m] = (KQ == 3 && m == 3) ? 0.f : dot8(w[m], xr[KQ == 3 ? m : m % KQ], 0.f);
    const float v = rows_sum(butterfly4(d[0], d[1], d[2], d[3], sub));  // lanes 4m .. 4m + 3: block m
    const int blk = KQ == 3 ? 16 : 4 * KQ;  // lanes of one row's blocks
    float sv = v;
#pragma unroll
    for (int k = 1; k < (KQ == 3 ? 3 : KQ); ++k) sv += __shfl(v, (ln & ~(blk - 1)) + 4 * k);
    const int p = ln / blk, r = t * P + p;
    if (ln < 16 && (ln & (blk - 1)) == 0 && p < P && r < nr) {
      st32(rl, (uint32_t)(n0 + r * stride) * 4u, __float_as_uint(sv));
      if (sv > best) {
        best = sv;
        bi = n0 + r * stride;
      }
    }
  };
  u32x4 b0[4], b1[4], b2[4], b3[4];
  load(b0, 0);
  load(b1, 1);
  load(b2, 2);
  load(b3, 3);
  for (int i = 0; i < my; i += 4) {
    consume(b0, i);
    load(b0, i + 4);
    consume(b1, i + 1);
    load(b1, i + 5);
    consume(b2, i + 2);
    load(b2, i + 6);
    consume(b3, i + 3);
    load(b3, i + 7);
  }
  argmax_merge(best, bi);
  if (ln == 0) {
    out[2 * wv] = best;
    out[2 * wv + 1] = __int_as_float(bi);
  }
}

// the projection body of one instruction on one wave (wv 0..6 compute waves, 7 the controller):
// the second half of a fused norm (then a barrier), then the tile's quad sums into the output area
DEV void proj_body(const KArgs& a, const Instr& in, const char* smem, uint32_t lease, bool fused_norm, int wv) {
  const uint32_t op = in.w[W_OPCODE];
  const int nr = in.w[W_P2], K = in.w[W_P4];
  const uint32_t wblk = blocks_of((uint32_t)nr * K * 2u);
  float* out = (float*)(smem + kOutOff);
  if (fused_norm) {
    const uint32_t goff = op == OP_LMHEAD ? 0u : (op == OP_GATEUP ? 2u : 1u) * wblk * 1024u;
    if (op == OP_QKV && in.w[W_LAYER] == 0)
      norm_h<true>(smem, lease, goff, K, wv);
    else
      norm_h<false>(smem, lease, goff, K, wv);
    lds_barrier();
  }
  if (op == OP_LMHEAD) {
    const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
    const char* wm = (const char*)s_ld64(row + LM_W);
    float* lg = (float*)s_ld64(row + LM_LOGITS);
    const int n0 = in.w[W_P1], st = in.w[W_P3];  // rows n0, n0 + st, ...
    lds_cchar* act = (lds_cchar*)(smem + kActOff);
    lds_float* lo = (lds_float*)(smem + kOutOff);
    switch (K >> 9) {
      case 1: lm_rows<1>(wm, lg, n0, nr, st, act, lo, wv); break;
      case 2: lm_rows<2>(wm, lg, n0, nr, st, act, lo, wv); break;
      case 3: lm_rows<3>(wm, lg, n0, nr, st, act, lo, wv); break;
      default: lm_rows<4>(wm, lg, n0, nr, st, act, lo, wv); break;
    }
  } else if (op == OP_OPROJ || op == OP_DOWN)
    gemv<true>(smem, lease, nr, nr, 0u, K, wv, out);
  else
    gemv<false>(smem, lease, op == OP_GATEUP ? 2 * nr : nr, nr, wblk * 1024u, K, wv, out);
}

// QK-norm (RMSNorm over the 128 dims of a head, gain gn) then rotate-half RoPE of one raw fp32
// head vector (staged tagged records), by one wave: lane i holds the rotation pair (i, i + 64);
// bf16 result into dst
DEV void qk_norm_rope(const char* raw, const char* gn, const char* rope, float eps, char* dst) {
  const int i = (int)lane();
  const float x0 = ll_f32(raw, i), x1 = ll_f32(raw, i + 64);
  const float inv = rsqrtf(wave_sum(x0 * x0 + x1 * x1) / 128.f + eps);
  const float g0 = bf2f(*(const uint16_t*)(gn + i * 2)), g1 = bf2f(*(const uint16_t*)(gn + (i + 64) * 2));
  const float c = *(const float*)(rope + i * 8), sn = *(const float*)(rope + i * 8 + 4);
  const float n0 = x0 * inv * g0, n1 = x1 * inv * g1;
  const uint32_t o = pack_bf2(n0 * c - n1 * sn, n1 * c + n0 * sn);
  ((uint16_t*)dst)[i] = (uint16_t)(o & 0xffffu);
  ((uint16_t*)dst)[i + 64] = (uint16_t)(o >> 16);
}

// An attention lease holds the split's K rows, then its V rows (256 bytes each).  Chunk c (16 bytes,
// dims 8c .. 8c + 7) of lease row u sits at position c ^ (u mod 16) of the row: the 16 rows that one
// matrix-core operand load reads at the same chunk then fall in 16 different bank groups.
DEV uint32_t att_pos(uint32_t u, uint32_t c) { return u * 256u + ((c ^ (u & 15u)) << 4); }

// reductions over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48), every lane getting the result
DEV float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
DEV float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// split-KV attention partial for one (request, kv head, split) over its G (<= 16) query heads, on all
// eight waves (wv 0..6 the compute waves, 7 the controller: two per SIMD), with two block barriers:
//   0. QK-norm + RoPE once per head (wave j < G: q head j, wave G: the new key, wave G + 1: the new
//      value, bf16) into LDS;
//   1. wave wv takes a contiguous block of at most 16 of the split's tokens and works on the matrix
//      cores: S^T = K Q^T (16x16x32 bf16; token rows by key rows, head columns), the wave's maximum
//      m_w and sum l_w per head over its tokens, P = exp(S - m_w) -- whose result layout is already
//      the A operand of the next product -- and O_w = P V (16x16x16 bf16 on P's three bf16 parts);
//   2. the eight waves' (m_w, l_w, O_w) merge with weights exp(m_w - max m_w).
// Output: the split's normalised O [G][128] and its lse [G] in the output area.
// Multi-row plans deal a worker consecutive splits of one (request, kv head), a chain: step 0 runs
// on its first split only (q, k and v stay in LDS), each later split's (m_w, l_w, O_w) is folded
// into the wave's running state in its own merge slots (both rescaled to the larger maximum), and
// step 2 runs on its last split only, so the chain leaves one partial.
template <int G, int S>
DEV void attn_body(const KArgs& a, const Instr& in, const char* smem, char* act, uint32_t lease, int wv) {
  static_assert(G <= 16, "one matrix-core column per query head");
  const Shapes& sh = a.sh;
  const int s = in.w[W_P3], t0 = in.w[W_P4], t1 = in.w[W_P5];
  const bool last = s == attn_splits<S>(in) - 1;
  const int ntok = t1 - t0;               // 1 .. 128
  const int nk = last ? ntok - 1 : ntok;  // tokens read from the cache; the last split adds the new one
  const uint32_t nbk = blocks_of((uint32_t)nk * 256u);
  const uint32_t voff = nbk * 1024u;      // lease: K | V
  const char* ring = smem + kRingOff;
  const int ln = (int)lane();
  // multi-row plans: a chain of splits on this worker folds into each wave's running state; its
  // first split prepares q, k and v, its last merges the waves (single-token: chains of one)
  const uint32_t chain = S == 1 ? in.w[W_CHAIN] : 2u;
  const bool cont = (chain & 1u) != 0u, end = (chain & 2u) != 0u;
  if (!cont) {
    if (wv < G) {
      qk_norm_rope(act + kAttQraw + wv * 1024, act + kAttGq, act + kAttRope, sh.eps, act + kActQ + wv * 256);
      if (S == 1) {  // the q head as materialised in bf16, for the record (this lane wrote dims ln, ln + 64)
        const uint16_t* qh = (const uint16_t*)(act + kActQ + wv * 256);
        const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
        __amdgpu_buffer_rsrc_t rq = rsrc((const void*)s_ld64(row + ATT_QB));
        const uint32_t h = in.w[W_LAYER + 1] * (uint32_t)sh.Hq + in.w[W_LAYER + 2] * (uint32_t)G + (uint32_t)wv;
        st16(rq, (h * 128u + (uint32_t)ln) * 2u, qh[ln]);
        st16(rq, (h * 128u + (uint32_t)ln + 64u) * 2u, qh[ln + 64]);
      }
    } else if (wv == G) {
      qk_norm_rope(act + kAttKraw, act + kAttGk, act + kAttRope, sh.eps, act + kActK);
    } else if (wv == G + 1) {
      const char* vr = act + kAttVraw;  // tagged records
      ((uint32_t*)(act + kActV))[ln] = pack_bf2(ll_f32(vr, 2 * ln), ll_f32(vr, 2 * ln + 1));
    }
    lds_barrier();
  }
  const int sub = ln & 15, grp = ln >> 4;
  const int per = (ntok + kNW - 1) / kNW;  // <= 16 tokens per wave
  const int tw0 = min(wv * per, ntok), tw1 = min(tw0 + per, ntok);
  // scores: A row sub = key row tw0 + sub (a row past the block loads a valid row; masked below),
  // lane group grp holding dims 32 k + 8 grp .. + 8 at step k; B column sub = q head sub (zero past
  // G).  Result: S[token tw0 + 4 grp + e][head sub] in element e.
  f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
  {
    const int ua = min(tw0 + sub, ntok - 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t c = 4u * k + (uint32_t)grp;
      const bf16x8 kv = *(const bf16x8*)(ua < nk ? ring + ring_off(lease, att_pos((uint32_t)ua, c)) : act + kActK + c * 16u);
      bf16x8 qv = *(const bf16x8*)(act + kActQ + (sub < G ? sub : 0) * 256 + c * 16u);
      if (sub >= G) qv = bf16x8{};
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv, sacc, 0, 0, 0);
    }
  }
  const float scale = sh.inv_sqrt_d;
  float p[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = tw0 + 4 * grp + e < tw1 ? sacc[e] * scale : -INFINITY;
    mloc = fmaxf(mloc, p[e]);
  }
  const float mw = rows4_max(mloc);  // -inf for a wave without tokens
  float lloc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = p[e] == -INFINITY ? 0.f : __expf(p[e] - mw);
    lloc += p[e];
  }
  const float lw = rows4_sum(lloc);
  // P V: A = P (lane: head sub, tokens 4 grp + e -- the layout the scores came in) as the sum of three
  // bf16 parts, P = hi + lo + lo2 (each the nearest bf16 to what the parts before it leave, every
  // remainder exact in fp32), so the product keeps about 24 bits of P, as an fp32 evaluation would
  // (two parts carry 16 bits, and a sum of V rows of both signs cancels).  B fragment c holds
  // V[token 4 grp + e][dim 8 sub + c], taken from one 16-byte load per token (chunk sub of the row)
  i16x4 pa, pl, pl2;
  {
    const u32x2 hw = {pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3])};
    const float r[4] = {p[0] - bf2f(hw[0] & 0xffffu), p[1] - bf2f(hw[0] >> 16), p[2] - bf2f(hw[1] & 0xffffu),
                        p[3] - bf2f(hw[1] >> 16)};
    const u32x2 lw2 = {pack_bf2(r[0], r[1]), pack_bf2(r[2], r[3])};
    const u32x2 lw3 = {pack_bf2(r[0] - bf2f(lw2[0] & 0xffffu), r[1] - bf2f(lw2[0] >> 16)),
                       pack_bf2(r[2] - bf2f(lw2[1] & 0xffffu), r[3] - bf2f(lw2[1] >> 16))};
    __builtin_memcpy(&pa, &hw, 8);
    __builtin_memcpy(&pl, &lw2, 8);
    __builtin_memcpy(&pl2, &lw3, 8);
  }
  u32x4 vv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int u = min(tw0 + 4 * grp + e, ntok - 1);  // past the block: a valid row, weight 0
    vv[e] = *(const u32x4*)(u < nk ? ring + ring_off(lease, voff + att_pos((uint32_t)u, (uint32_t)sub)) : act + kActV + sub * 16);
  }
  f32x4 o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    u32x2 bw;
    if (c & 1) {
      bw[0] = (vv[0][w] >> 16) | (vv[1][w] & 0xffff0000u);
      bw[1] = (vv[2][w] >> 16) | (vv[3][w] & 0xffff0000u);
    } else {
      bw[0] = (vv[0][w] & 0xffffu) | (vv[1][w] << 16);
      bw[1] = (vv[2][w] & 0xffffu) | (vv[3][w] << 16);
    }
    i16x4 b;
    __builtin_memcpy(&b, &bw, 8);
    o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl2, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, b, o[c], 0, 0, 0);
    o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, b, o[c], 0, 0, 0);
  }
  // O_w[head 4 grp + i][dim 8 sub + c] is element i of o[c]
  float* mrg = (float*)(act + kActMerge);  // [wave][G][128] partial P V, then [wave][G] (m_w, l_w)
  float* ml = mrg + kNW * G * 128;
  float m_w = mw, l_w = lw;
  float fo[4] = {0.f, 0.f, 0.f, 0.f}, fc[4] = {1.f, 1.f, 1.f, 1.f};  // weights of the state and of this split
  if (S == 1 && cont) {
    // the wave's state so far (this wave's own slots, from the chain's previous split): rescale
    // both parts to the larger maximum; lane sub of row 0 holds head sub's weights
    const f32x2 so = *(const f32x2*)(ml + (wv * G + (sub < G ? sub : 0)) * 2);
    m_w = fmaxf(so.x, mw);
    const float ao = so.x == -INFINITY ? 0.f : __expf(so.x - m_w);
    const float ac = mw == -INFINITY ? 0.f : __expf(mw - m_w);
    l_w = ao * so.y + ac * lw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fo[i] = __shfl(ao, 4 * grp + i);
      fc[i] = __shfl(ac, 4 * grp + i);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * grp + i;
    if (h < G) {
      float* po = mrg + (wv * G + h) * 128 + 8 * sub;
      f32x4 o0 = f32x4{o[0][i], o[1][i], o[2][i], o[3][i]} * fc[i];
      f32x4 o1 = f32x4{o[4][i], o[5][i], o[6][i], o[7][i]} * fc[i];
      if (S == 1 && cont) {
        o0 += *(const f32x4*)po * fo[i];
        o1 += *(const f32x4*)(po + 4) * fo[i];
      }
      *(f32x4*)po = o0;
      *(f32x4*)(po + 4) = o1;
    }
  }
  if (grp == 0 && sub < G) *(f32x2*)(ml + (wv * G + sub) * 2) = f32x2{m_w, l_w};
  if (!end) return;  // the chain goes on: the state stays in this wave's slots
  lds_barrier();
  // merge the eight waves: weights exp(m_w - M) with M the largest m_w; lane o = j * 128 + d
  float* out = (float*)(smem + kOutOff);
  for (int o2 = wv * 64 + ln; o2 < G * 128; o2 += kNW * 64) {
    const int j = o2 >> 7, d = o2 & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, ml[(w * G + j) * 2]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float mv = ml[(w * G + j) * 2];
      const float e = mv == -INFINITY ? 0.f : __expf(mv - M);
      O += e * mrg[(w * G + j) * 128 + d];
      L += e * ml[(w * G + j) * 2 + 1];
    }
    out[o2] = O / L;
    if (d == 0) out[G * 128 + j] = M + __logf(L);
  }
}

template <int S>
DEV void attn_compute(const KArgs& a, const Instr& in, const char* smem, char* act, uint32_t lease, int cw) {
  switch (a.sh.g) {
    case 1: attn_body<1, S>(a, in, smem, act, lease, cw); break;
    case 2: attn_body<2, S>(a, in, smem, act, lease, cw); break;
    default: attn_body<4, S>(a, in, smem, act, lease, cw); break;  // GQA groups 1, 2 and 4 are built
  }
}

// ---------------------------------------------------------------------------------------
// multi-row (M <= 16 tokens) ops
//
// The multi-row plans order their work with the queue's event counters: a producer stores its
// results at device scope, waits for the stores to complete, then adds its increment to the
// event (one of kNSub sub-counters, spreading the atomics); a consumer sums the sub-counters
// until they reach (runs + 1) x threshold, so counters never need clearing between runs.
// Intermediates are plain (untagged) values; projection inputs sit in HBM already in the
// matrix-core operand order, so a tile's input chunk is one contiguous copy.


DEV void signal_all(const KArgs& a, const Instr& in) {
  if (a.flags & kModeGraph) return;
  if (lane() == 0) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if ((uint32_t)k >= in.w[W_NSIG]) break;
      uint32_t* ctr = a.events + (size_t)in.w[W_SIG0 + 3 * k] * kEvStride + (blockIdx.x % kNSub) * kSubStride;
      __hip_atomic_fetch_add(ctr, in.w[W_SIG0 + 3 * k + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

struct WaitCache {  // the last (event, threshold) wait found satisfied in this run
  uint32_t e, thr;
};

// A multi-row instruction's signals, held by the controller from its compute-end barrier until
// its stores have completed: the completion wait is taken together with the next instruction's
// staging, or on its own before any wait that has to poll and at the end of the queue.
struct SigPend {
  uint32_t n, e0, i0, e1, i1;
};
DEV SigPend sig_of(const Instr& in) {
  return SigPend{in.w[W_NSIG], in.w[W_SIG0], in.w[W_SIG0 + 1], in.w[W_SIG0 + 3], in.w[W_SIG0 + 4]};
}
DEV void signal_pend(const KArgs& a, const SigPend& sp) {
  if (a.flags & kModeGraph) return;
  if (lane() == 0) {
    const size_t sub = (blockIdx.x % kNSub) * kSubStride;
    if (sp.n > 0u) __hip_atomic_fetch_add(a.events + (size_t)sp.e0 * kEvStride + sub, sp.i0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (sp.n > 1u) __hip_atomic_fetch_add(a.events + (size_t)sp.e1 * kEvStride + sub, sp.i1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
// every wait of the instruction is the one last found satisfied (no polling needed)
DEV bool waits_cached(const Instr& in, const WaitCache& wc) {
  bool all = true;
#pragma unroll
  for (int k = 0; k < 4; ++k)  // constant indices: the instruction words stay in registers
    if ((uint32_t)k < in.w[W_NWAIT] && (in.w[W_WAIT0 + 2 * k] != wc.e || in.w[W_WAIT0 + 2 * k + 1] != wc.thr)) all = false;
  return all;
}

// false when the watchdog expired or another worker aborted
DEV bool wait_events(const KArgs& a, const Instr& in, uint32_t& polls, WaitCache& wc) {
  const uint32_t ln = lane();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if ((uint32_t)k >= in.w[W_NWAIT]) break;
    const uint32_t e = in.w[W_WAIT0 + 2 * k], thr = in.w[W_WAIT0 + 2 * k + 1];
    if (e == wc.e && thr == wc.thr) continue;  // counters only grow within a run
    const uint32_t target = (a.run + 1u) * thr;
    const uint32_t* base = a.events + (size_t)e * kEvStride;
    const unsigned long long t0 = rtc();
    for (uint32_t it = 1;; ++it) {
      uint32_t v = 0;
      if (ln < (uint32_t)kNSub) v = __hip_atomic_load(base + ln * kSubStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t sum = wave_sum_u32(v);
      if ((int32_t)(sum - target) >= 0) break;
      ++polls;
      if ((it & 31u) == 0 && __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return false;
      if (rtc() - t0 > watchdog_ticks(a)) {
        record_timeout(a, in, e, sum);
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    wc.e = e;
    wc.thr = thr;
  }
  asm volatile("" ::: "memory");
  return true;
}

// byte offset of element (m, k) of an operand-order matrix with K columns: rows in groups of 16,
// one group after the other; inside a group 1 KiB per K step (32 bf16 or 64 e4m3), lane
// l = (m mod 16) + 16 g holding the step's 16-byte group g of row m
DEV uint32_t opnd_bf16(uint32_t m, uint32_t k, uint32_t K) {
  return (m >> 4) * K * 32u + (k >> 5) * 1024u + ((m & 15u) + 16u * ((k & 31u) >> 3)) * 16u + (k & 7u) * 2u;
}
DEV uint32_t opnd_fp8(uint32_t m, uint32_t k, uint32_t K) {
  return (m >> 4) * K * 16u + (k >> 6) * 1024u + ((m & 15u) + 16u * ((k & 63u) >> 4)) * 16u + (k & 15u);
}
// eight e4m3 codes (bytes of w0, w1) as bf16: every e4m3 value is a bf16 value, so this is exact
DEV bf16x8 e4m3x8_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
DEV void st64(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) { __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, SC1); }
DEV void st128(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, SC1); }
DEV uint32_t bf16_bits(float v) { return pack_bf2(v, 0.f) & 0xffffu; }
// e4m3 codes of four values, saturated to +-448 first (OCP E4M3FN, round to nearest even)
DEV uint32_t e4m3x4(float v0, float v1, float v2, float v3) {
  const auto c = [](float v) { return fminf(fmaxf(v, -448.f), 448.f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c(v0), c(v1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c(v2), c(v3), w, true);
  return (uint32_t)w;
}

// Projection tile on the eight waves: Y[16 tokens][64 tile rows] over one K chunk.  The weights
// sit in the lease in B-operand order (block 16 nb + q), the input chunk in the activation area in
// A-operand order.  Wave w takes row block nb = w & 3 and half w >> 2 of the chunk's K steps;
// its 16 x 16 fp32 result goes to the activation area for the controller to add and store.
// W8A8: the e4m3 operands are widened to bf16 (exactly) for the bf16 matrix-core product, whose
// fp32 sums keep full precision -- the e4m3 products of gfx950's fp8 instructions are summed at
// lower internal precision, which the chain of per-token quantisations downstream amplifies.
// Each 128-wide K block's sum is scaled by its weight block scale as it is added.
// NQ, a compile-time bound so that the unrolled loop keeps its LDS reads ahead of the matrix-core
// chain (a run-time bound cost the bf16 16-row layer 12 %): bf16, the K steps per half of the chunk
// (8: chunk 512; 2: the main-MLA query BMM's 128); e4m3, the 128-wide scale blocks per half (4:
// chunk 1024; 3: 768), or 0 for a bound read from the instruction
template <bool FP8, int NQ>
DEV void gemm_tile(const KArgs& a, const Instr& in, char* smem, uint32_t lease, int wv) {
  const uint32_t ln = lane(), nb = (uint32_t)wv & 3u, kh = (uint32_t)wv >> 2;
  const char* act = smem + kActOff + kActA;
  const char* ring = smem + kRingOff;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const uint32_t kc = in.w[W_LAYER + 6];
  if (!FP8) {  // K chunk of 2 NQ steps of 32
    constexpr uint32_t bpn = 2u * NQ;  // steps per 16-row block
#pragma unroll
    for (uint32_t i = 0; i < (uint32_t)NQ; ++i) {
      const uint32_t q = kh * NQ + i;
      const bf16x8 av = *(const bf16x8*)(act + q * 1024u + ln * 16u);
      const bf16x8 bv = *(const bf16x8*)(ring + ring_off(lease, (nb * bpn + q) * 1024u + ln * 16u));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    }
  } else {
    const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
    const uint32_t kind = in.w[W_LAYER + 1], n0 = in.w[W_LAYER + 3], k0 = in.w[W_LAYER + 5];
    const uint32_t K = proj_k(a.sh, kind), nkb = K >> 7;
    const uint32_t tr0 = nb * 16u;
    const uint32_t grow = kind == K_GU && tr0 >= 32u ? (uint32_t)a.sh.I + n0 + tr0 - 32u : n0 + tr0;
    const float* sw = (const float*)s_ld64(row + GM_SW) + (size_t)(grow >> 7) * nkb + (k0 >> 7);
    const uint32_t nkh = NQ ? (uint32_t)NQ : kc >> 8;  // 128-wide scale blocks per half of the chunk
#pragma unroll
    for (uint32_t kb = 0; kb < (NQ ? (uint32_t)NQ : 4u); ++kb) {  // the wave's scale blocks, two 64-k steps each
      if (!NQ && kb >= nkh) break;
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (uint32_t h = 0; h < 2; ++h) {
        const uint32_t q = kh * 2u * nkh + kb * 2u + h;
        const u32x4 av = *(const u32x4*)(act + q * 1024u + ln * 16u);
        const u32x4 bv = *(const u32x4*)(ring + ring_off(lease, (nb * (kc >> 6) + q) * 1024u + ln * 16u));
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(av.x, av.y), e4m3x8_bf16(bv.x, bv.y), t, 0, 0, 0);
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(av.z, av.w), e4m3x8_bf16(bv.z, bv.w), t, 0, 0, 0);
      }
      acc += c_ld<float>(sw + kh * nkh + kb) * t;
    }
  }
  *(f32x4*)(smem + kActOff + kActD + ((uint32_t)wv * 64u + ln) * 16u) = acc;
}

// Plans of more than 16 rows: the same tile for every 16-row group of M, the weights read once from
// the lease.  Wave w takes row block nb = w & 3 and the row groups w >> 2, w >> 2 + 2, ...; it reads
// each group's input chunk straight from the workspace (operand order, device-scope loads: the
// chunk would not fit the activation area for all groups), sums the whole K chunk and stores the
// group's 16 x 16 partial sums itself, [tile][chunk][group][row block][lane][4].
// NST: the chunk's 1 KiB steps (16: bf16 chunk 512, e4m3 chunk 1024)
template <bool FP8, int NST>
DEV void gemm_tile_groups(const KArgs& a, const Instr& in, const char* smem, uint32_t lease, int wv) {
  const uint32_t ln = lane(), nb = (uint32_t)wv & 3u;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t kind = in.w[W_LAYER + 1], j = in.w[W_LAYER + 2], n0 = in.w[W_LAYER + 3], k0 = in.w[W_LAYER + 5];
  const uint32_t kc = in.w[W_LAYER + 6], K = proj_k(a.sh, kind), G = (uint32_t)a.sh.rg;
  constexpr uint32_t nst = NST;
  static_assert(NST == 16, "two halves of 8 steps");
  const uint32_t gstride = FP8 ? K * 16u : K * 32u;
  const char* ring = smem + kRingOff;
  __amdgpu_buffer_rsrc_t ra = rsrc((const char*)s_ld64(row + GM_ACT) + (FP8 ? k0 >> 6 : k0 >> 5) * 1024u);
  __amdgpu_buffer_rsrc_t rp = rsrc((float*)s_ld64(row + GM_PART) + ((size_t)j * (K / kc) + k0 / kc) * G * 1024);
  const float* sw = nullptr;
  if (FP8) {
    const uint32_t tr0 = nb * 16u;
    const uint32_t grow = kind == K_GU && tr0 >= 32u ? (uint32_t)a.sh.I + n0 + tr0 - 32u : n0 + tr0;
    sw = (const float*)s_ld64(row + GM_SW) + (size_t)(grow >> 7) * (K >> 7) + (k0 >> 7);
  }
  for (uint32_t gi = (uint32_t)wv >> 2; gi < G; gi += 2u) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (uint32_t hh = 0; hh < 2; ++hh) {  // the chunk in two halves of 8 steps: 32 registers of input each
      u32x4 av[8];
#pragma unroll
      for (uint32_t i = 0; i < 8; ++i) av[i] = ld128(ra, gi * gstride + (hh * 8u + i) * 1024u + ln * 16u);
      if (!FP8) {
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i) {
          const bf16x8 bv = *(const bf16x8*)(ring + ring_off(lease, (nb * nst + hh * 8u + i) * 1024u + ln * 16u));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16((bf16x8)av[i], bv, acc, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (uint32_t kb = 0; kb < 4; ++kb) {  // 128-wide scale blocks, two 64-k steps each
          f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t i = 2u * kb + h;
            const u32x4 bv = *(const u32x4*)(ring + ring_off(lease, (nb * nst + hh * 8u + i) * 1024u + ln * 16u));
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(av[i].x, av[i].y), e4m3x8_bf16(bv.x, bv.y), t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_bf16(av[i].z, av[i].w), e4m3x8_bf16(bv.z, bv.w), t, 0, 0, 0);
          }
          acc += c_ld<float>(sw + hh * 4u + kb) * t;
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // the next half's loads after this half's products: bounded registers
    }
    st128(rp, gi * 4096u + (nb * 64u + ln) * 16u,
          u32x4{__float_as_uint(acc.x), __float_as_uint(acc.y), __float_as_uint(acc.z), __float_as_uint(acc.w)});
  }
  wait_vm0();  // the signals follow barrier B
}

// controller: add the two K halves of each row block and store the tile's partial sums
// [chunk][row block][lane][4] (element (m, c) of the 16 x 64 tile at lane c % 16 + 16 (m / 4) of
// block c / 16, position m % 4), then signal
template <bool LD, bool RG>
DEV void gemm_epilogue(const KArgs& a, const Instr& in, const char* smem) {
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t kind = in.w[W_LAYER + 1], j = in.w[W_LAYER + 2], k0 = in.w[W_LAYER + 5];
  const uint32_t kc = in.w[W_LAYER + 6], nk = proj_k(a.sh, kind) / kc;
  const char* D = smem + kActOff + kActD;
  const uint32_t ln = lane();
  if (!LD && kind == K_UK) {  // the main-MLA query BMM is one chunk: its tile is final, bf16 q_lat [M][heads][512]
    const uint32_t n0 = in.w[W_LAYER + 3], h = n0 / (uint32_t)kMlaLatent, c0 = n0 % (uint32_t)kMlaLatent;
    __amdgpu_buffer_rsrc_t ro = rsrc((const void*)s_ld64(row + GM_PART));
#pragma unroll
    for (uint32_t nb = 0; nb < 4; ++nb) {
      const f32x4 v = *(const f32x4*)(D + (nb * 64u + ln) * 16u) + *(const f32x4*)(D + ((nb + 4u) * 64u + ln) * 16u);
      const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (uint32_t q = 0; q < 4; ++q) {
        const uint32_t m = 4u * (ln >> 4) + q, c = c0 + nb * 16u + (ln & 15u);
        if (m < (uint32_t)a.sh.M)
          st16(ro, ((m * (uint32_t)a.sh.mla + h) * (uint32_t)kMlaLatent + c) * 2u, bf16_bits(e[q]));
      }
    }
    return;
  }
  if (RG) return;  // the waves stored every group's partial sums
  float* part = (float*)s_ld64(row + GM_PART) + ((size_t)j * nk + k0 / kc) * 1024;
  __amdgpu_buffer_rsrc_t rp = rsrc(part);
#pragma unroll
  for (uint32_t nb = 0; nb < 4; ++nb) {
    const f32x4 v = *(const f32x4*)(D + (nb * 64u + ln) * 16u) + *(const f32x4*)(D + ((nb + 4u) * 64u + ln) * 16u);
    st128(rp, (nb * 64u + ln) * 16u, u32x4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)});
  }
}

// float index of tile element (m, c) in one chunk's partial sums
DEV uint32_t part_idx(uint32_t m, uint32_t c) { return ((c >> 4) * 64u + (c & 15u) + 16u * (m >> 2)) * 4u + (m & 3u); }

// Finalize of one projection tile on the eight waves: add its K chunks in order (thread t: the
// two tile elements (m, c) and (m + 8, c) with m = t / 64, c = t % 64; gate/up: the gate and up
// sums of (m, c), m = t / 32, c = t % 32), then the projection's epilogue:
//   QKV: fp32 q | k | v as tagged records (the attention staging reads records)
//   O: r2 = r1 + bf16(a)                    GATE_UP: m = silu(g) u (bf16 operand order, or fp32 rows)
//   DOWN: y = bf16(.)                        W8A8: sums times the token's input scale first
template <int NK, bool RG>
DEV void fin_tile(const KArgs& a, const Instr& in, int wv) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t kind = in.w[W_LAYER + 1], j = in.w[W_LAYER + 2], n0 = in.w[W_LAYER + 3], nk = in.w[W_LAYER + 5];
  const uint32_t gi = RG ? in.w[W_GROUP] : 0u, G = RG ? (uint32_t)sh.rg : 1u;  // the 16-row group it finalizes
  const uint32_t t = (uint32_t)wv * 64u + lane();
  const bool gu = kind == K_GU;
  const uint32_t l0 = gu ? t >> 5 : t >> 6, c = gu ? t & 31u : t & 63u;
  const uint32_t l1 = gu ? l0 : l0 + 8u, c1 = gu ? c + 32u : c;
  const uint32_t m0 = 16u * gi + l0, m1 = 16u * gi + l1;
  __amdgpu_buffer_rsrc_t rp = rsrc((const float*)s_ld64(row + FN_PART) + ((size_t)j * nk * G + gi) * 1024);
  const uint32_t i0 = part_idx(l0, c), i1 = part_idx(l1, c1);
  float v0[NK], v1[NK];
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const uint32_t kk = min((uint32_t)k, nk - 1u);
    v0[k] = __uint_as_float(ld32(rp, (kk * G * 1024u + i0) * 4u));
    v1[k] = __uint_as_float(ld32(rp, (kk * G * 1024u + i1) * 4u));
  }
  const uint64_t out = s_ld64(row + FN_OUT), out2 = s_ld64(row + FN_OUT2);
  const uint32_t H = (uint32_t)sh.H, M = (uint32_t)sh.M;
  float r1v[2] = {0.f, 0.f};
  if (kind == K_O) {
    __amdgpu_buffer_rsrc_t rr = rsrc((const void*)s_ld64(row + FN_R1));
    if (m0 < M) r1v[0] = __uint_as_float(ld32(rr, (m0 * H + n0 + c) * 4u));
    if (m1 < M) r1v[1] = __uint_as_float(ld32(rr, (m1 * H + n0 + c) * 4u));
  }
  float sa[2] = {1.f, 1.f};
  if (sh.fp8) {
    const float* sp = (const float*)s_ld64(row + FN_SA);
    sa[0] = __uint_as_float(ld32(rsrc(sp), m0 * 4u));
    sa[1] = __uint_as_float(ld32(rsrc(sp), m1 * 4u));
  }
  wait_vm0();
  float s0 = v0[0], s1 = v1[0];
#pragma unroll
  for (int k = 1; k < NK; ++k) {
    if ((uint32_t)k < nk) {
      s0 += v0[k];
      s1 += v1[k];
    }
  }
  s0 *= sa[0];
  s1 *= sa[1];
  __amdgpu_buffer_rsrc_t ro = rsrc((const void*)out);
  if (kind == K_GU) {
    if (m0 < M) {
      const float mv = s0 / (1.f + __expf(-s0)) * s1;
      if (sh.fp8)
        st32(ro, (m0 * (uint32_t)sh.I + n0 + c) * 4u, __float_as_uint(mv));
      else
        st16(ro, opnd_bf16(m0, n0 + c, (uint32_t)sh.I), bf16_bits(mv));
    }
  } else if (kind >= K_QA) {  // indexer q_a, head weights, key: fp32 rows
    const uint32_t w = kind == K_QA ? (uint32_t)sh.qr : kind == K_W ? (uint32_t)sh.nh : 128u;
    if (m0 < M) st32(ro, (m0 * w + n0 + c) * 4u, __float_as_uint(s0));
    if (m1 < M) st32(ro, (m1 * w + n0 + c) * 4u, __float_as_uint(s1));
  } else {
    const uint32_t ms[2] = {m0, m1};
    const float vs[2] = {s0, s1};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t m = ms[q];
      if (m >= M) continue;
      if (kind == K_QKV) {
        ll_put(ro, m * (uint32_t)sh.n_qkv + n0 + c, __float_as_uint(vs[q]), ll_tag(a, in.w[W_LAYER]));
      } else if (kind == K_O) {
        const float r2 = r1v[q] + bf2f(bf16_bits(vs[q]));
        st32(ro, (m * H + n0 + c) * 4u, __float_as_uint(r2));
        if (out2) st32(rsrc((const void*)out2), (m * H + n0 + c) * 4u, __float_as_uint(r2));
      } else {  // down
        const uint32_t y = bf16_bits(vs[q]);
        st16(ro, (m * H + n0 + c) * 2u, y);
        if (out2) st16(rsrc((const void*)out2), (m * H + n0 + c) * 2u, y);
      }
    }
  }
  wait_vm0();
}

// Add (+ residual) + RMSNorm of one row on the eight waves, thread t taking elements
// [8 t, 8 t + 8) and [8 (t + 512), ...): r1 = r + x written out (first norm), h = r1 / rms * gain
// into the operand order, bf16 or (W8A8) per-token e4m3 with scale amax / 448.
template <bool FP8>
DEV void norm_row(const KArgs& a, const Instr& in, char* smem, uint32_t lease, int wv) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t m = in.w[W_LAYER + 2], H = norm_len(sh, in), t = (uint32_t)wv * 64u + lane();
  const uint64_t xp = s_ld64(row + NM_X), r1p = s_ld64(row + NM_R1);
  __amdgpu_buffer_rsrc_t rr = rsrc((const float*)s_ld64(row + NM_R) + (size_t)m * H);
  __amdgpu_buffer_rsrc_t rx = rsrc((const uint16_t*)xp + (size_t)m * H);
  float v[2][8];
  u32x4 ra[2], rb[2], xv[2];
  const bool in_lease = norm_inputs_in_lease(in, row);
  const char* ring = smem + kRingOff;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t e = min(t + 512u * i, H / 8u - 1u) * 8u;
    if (in_lease) {
      ra[i] = *(const u32x4*)(ring + ring_off(lease, 2u * H + e * 4u));
      rb[i] = *(const u32x4*)(ring + ring_off(lease, 2u * H + e * 4u + 16u));
      xv[i] = *(const u32x4*)(ring + ring_off(lease, 6u * H + e * 2u));
    } else {
      ra[i] = ld128(rr, e * 4u);
      rb[i] = ld128(rr, e * 4u + 16u);
      xv[i] = xp ? ld128(rx, e * 2u) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  wait_vm0();
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t r[8] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w, rb[i].x, rb[i].y, rb[i].z, rb[i].w};
    const uint32_t x[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
#pragma unroll
    for (int q = 0; q < 8; ++q) v[i][q] = __uint_as_float(r[q]) + bf2f((q & 1) ? x[q >> 1] >> 16 : x[q >> 1] & 0xffffu);
    if (t + 512u * i < H / 8u) {
#pragma unroll
      for (int q = 0; q < 8; ++q) ss += v[i][q] * v[i][q];
    }
  }
  float* red = (float*)(smem + kActOff + kActRed);
  const float ws = wave_sum(ss);
  if (lane() == 0) red[wv] = ws;
  lds_barrier();
  float tot = red[0];
#pragma unroll
  for (int w = 1; w < kNW; ++w) tot += red[w];
  const float inv = rsqrtf(tot / (float)H + sh.eps);
  float h[2][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t e = min(t + 512u * i, H / 8u - 1u) * 8u;
    const u32x4 gv = *(const u32x4*)(smem + kRingOff + ring_off(lease, e * 2u));
    const uint32_t g[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      h[i][q] = v[i][q] * inv * bf2f((q & 1) ? g[q >> 1] >> 16 : g[q >> 1] & 0xffffu);
      if (t + 512u * i < H / 8u) amax = fmaxf(amax, fabsf(h[i][q]));
    }
  }
  float s = 1.f;
  if (FP8) {
    const float wm = wave_max(amax);
    if (lane() == 0) red[8 + wv] = wm;
    lds_barrier();
    float am = red[8];
#pragma unroll
    for (int w = 1; w < kNW; ++w) am = fmaxf(am, red[8 + w]);
    s = am > 0.f ? am / 448.f : 1.f;
  }
  __amdgpu_buffer_rsrc_t rh = rsrc((const void*)s_ld64(row + NM_H));
  __amdgpu_buffer_rsrc_t r1o = rsrc((float*)r1p + (size_t)m * H);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (t + 512u * i >= H / 8u) continue;
    const uint32_t e = (t + 512u * i) * 8u;
    if (r1p) {
      st128(r1o, e * 4u, u32x4{__float_as_uint(v[i][0]), __float_as_uint(v[i][1]), __float_as_uint(v[i][2]), __float_as_uint(v[i][3])});
      st128(r1o, e * 4u + 16u, u32x4{__float_as_uint(v[i][4]), __float_as_uint(v[i][5]), __float_as_uint(v[i][6]), __float_as_uint(v[i][7])});
    }
    if (FP8) {
      st64(rh, opnd_fp8(m, e, H), u32x2{e4m3x4(h[i][0] / s, h[i][1] / s, h[i][2] / s, h[i][3] / s),
                                     e4m3x4(h[i][4] / s, h[i][5] / s, h[i][6] / s, h[i][7] / s)});
    } else {
      st128(rh, opnd_bf16(m, e, H), u32x4{pack_bf2(h[i][0], h[i][1]), pack_bf2(h[i][2], h[i][3]), pack_bf2(h[i][4], h[i][5]),
                                       pack_bf2(h[i][6], h[i][7])});
    }
  }
  if (FP8 && t == 0) st32(rsrc((const void*)s_ld64(row + NM_S)), m * 4u, __float_as_uint(s));
  wait_vm0();
}

// per-token e4m3 quantisation of one fp32 row (attention output o, or m) into the operand order,
// on the eight waves: thread t takes the 4-element groups t, t + 512, ...
constexpr int kQuantIt = 6;  // rows up to 6 x 512 x 4 = 12288 elements
DEV void quant_row(const KArgs& a, const Instr& in, char* smem, int wv) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t which = in.w[W_LAYER + 1], m = in.w[W_LAYER + 2], t = (uint32_t)wv * 64u + lane();
  const uint32_t K = which == 0 ? (uint32_t)sh.Hq * 128u : (uint32_t)sh.I, ng = K / 4u;
  __amdgpu_buffer_rsrc_t ri = rsrc((const float*)s_ld64(row + QT_IN) + (size_t)m * K);
  u32x4 v[kQuantIt];
#pragma unroll
  for (int i = 0; i < kQuantIt; ++i) v[i] = ld128(ri, min(t + 512u * i, ng - 1u) * 16u);
  wait_vm0();
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kQuantIt; ++i)
    if (t + 512u * i < ng)
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(__uint_as_float(v[i].x)), fabsf(__uint_as_float(v[i].y))),
                               fmaxf(fabsf(__uint_as_float(v[i].z)), fabsf(__uint_as_float(v[i].w)))));
  float* red = (float*)(smem + kActOff + kActRed);
  const float wm = wave_max(amax);
  if (lane() == 0) red[8 + wv] = wm;
  lds_barrier();
  float am = red[8];
#pragma unroll
  for (int w = 1; w < kNW; ++w) am = fmaxf(am, red[8 + w]);
  const float s = am > 0.f ? am / 448.f : 1.f;
  __amdgpu_buffer_rsrc_t ro = rsrc((const void*)s_ld64(row + QT_OUT));
#pragma unroll
  for (int i = 0; i < kQuantIt; ++i) {
    const uint32_t gi = t + 512u * i;
    if (gi < ng)
      st32(ro, opnd_fp8(m, gi * 4u, K), e4m3x4(__uint_as_float(v[i].x) / s, __uint_as_float(v[i].y) / s,
                                            __uint_as_float(v[i].z) / s, __uint_as_float(v[i].w) / s));
  }
  if (t == 0) st32(rsrc((const void*)s_ld64(row + QT_S)), m * 4u, __float_as_uint(s));
  wait_vm0();
}

// Combine of one (request, kv head) on the eight waves: thread t takes output element t of the
// group's g heads x 128 dims, o = sum_s exp(lse_s - L) O_s with L = log sum_s exp(lse_s), over the
// splits in order, 32 at a time with a running maximum (online rescaling)
DEV void comb_group(const KArgs& a, const Instr& in, int wv) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t r = in.w[W_LAYER + 1], hk = in.w[W_LAYER + 2], ns = in.w[W_LAYER + 3];
  const uint32_t g = (uint32_t)sh.g, t = (uint32_t)wv * 64u + lane();
  const uint32_t pstride = g * 128u + 8u;
  const uint32_t gbase = ((r * (uint32_t)sh.Hkv + hk) * (uint32_t)sh.max_splits) * pstride;
  __amdgpu_buffer_rsrc_t rp = rsrc((const float*)s_ld64(row + ATT_PART) + gbase);
  const uint32_t tt = min(t, g * 128u - 1u), j = tt >> 7;
  float M = -INFINITY, S = 0.f, acc = 0.f;
  for (uint32_t s0 = 0; s0 < ns; s0 += 32u) {
    float lv[32], ov[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t sp = min(s0 + (uint32_t)i, ns - 1u);
      lv[i] = __uint_as_float(ld32(rp, (sp * pstride + g * 128u + j) * 4u));
      ov[i] = __uint_as_float(ld32(rp, (sp * pstride + tt) * 4u));
    }
    wait_vm0();
    float mc = M;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (s0 + (uint32_t)i < ns) mc = fmaxf(mc, lv[i]);
    const float sc = M == -INFINITY ? 0.f : __expf(M - mc);
    S *= sc;
    acc *= sc;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (s0 + (uint32_t)i < ns) {
        const float e = __expf(lv[i] - mc);
        S += e;
        acc += e * ov[i];
      }
    }
    M = mc;
  }
  if (t < g * 128u) {
    const uint32_t k = hk * g * 128u + t;
    __amdgpu_buffer_rsrc_t ro = rsrc((const void*)s_ld64(row + ATT_O));
    const float v = acc / S;
    if (sh.fp8)
      st32(ro, (r * (uint32_t)sh.Hq * 128u + k) * 4u, __float_as_uint(v));
    else
      st16(ro, opnd_bf16(r, k, (uint32_t)sh.Hq * 128u), bf16_bits(v));
  }
  wait_vm0();
}

// ---------------------------------------------------------------------------------------
// indexer front

// byte offset of q element (token m, head h, dim d) in the score's A-operand order: per (token,
// 16-head block, dim step) 1 KiB, dim step f = 2 (d / 64) + (d % 16) / 8, lane (h % 16) + 16 ((d % 64) / 16)
// holding 8 consecutive dims -- the order in which a lane's 16 key bytes (dims 64 s + 16 g ..) feed
// two bf16 matrix-core steps
DEV uint32_t qi_off(uint32_t m, uint32_t h, uint32_t d, uint32_t nh) {
  return ((m * (nh >> 4) + (h >> 4)) * 4u + 2u * (d >> 6) + ((d >> 3) & 1u)) * 1024u +
         ((h & 15u) + 16u * ((d & 63u) >> 4)) * 16u + (d & 7u) * 2u;
}

// D1 finalize of one head on the eight waves: thread t takes the RoPE pairs (i, i + 64) of tokens
// m = t / 64 and m + 8, i = t % 64: q = (sum of the head's two tiles' chunks) x the token's q_a scale,
// rotated at the token's position, then bf16 into the score operand order
DEV void fin_qi(const KArgs& a, const Instr& in, int wv) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t h = in.w[W_LAYER + 2], nk = in.w[W_LAYER + 5];
  const uint32_t t = (uint32_t)wv * 64u + lane(), i = t & 63u, M = (uint32_t)sh.M;
  const uint32_t ms[2] = {t >> 6, (t >> 6) + 8u};
  __amdgpu_buffer_rsrc_t rp = rsrc((const float*)s_ld64(row + FN_PART) + (size_t)2u * h * nk * 1024);
  __amdgpu_buffer_rsrc_t rs = rsrc((const void*)s_ld64(row + FN_SA));
  __amdgpu_buffer_rsrc_t rr = rsrc((const void*)s_ld64(row + FN_R1));
  float x[2][2][4], sa[2], cs[2][2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t m = min(ms[q], M - 1u);
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t kk = min((uint32_t)k, nk - 1u);
        x[q][tl][k] = __uint_as_float(ld32(rp, (((uint32_t)tl * nk + kk) * 1024u + part_idx(m, i)) * 4u));
      }
    sa[q] = __uint_as_float(ld32(rs, m * 4u));
    cs[q][0] = __uint_as_float(ld32(rr, (m * 64u + i) * 8u));
    cs[q][1] = __uint_as_float(ld32(rr, (m * 64u + i) * 8u + 4u));
  }
  wait_vm0();
  __amdgpu_buffer_rsrc_t ro = rsrc((const void*)s_ld64(row + FN_OUT));
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (ms[q] >= M) continue;
    float v[2];
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      float acc = x[q][tl][0];
#pragma unroll
      for (uint32_t k = 1; k < 4; ++k)
        if (k < nk) acc += x[q][tl][k];
      v[tl] = acc * sa[q];
    }
    const float y0 = v[0] * cs[q][0] - v[1] * cs[q][1], y1 = v[1] * cs[q][0] + v[0] * cs[q][1];
    st16(ro, qi_off(ms[q], h, i, (uint32_t)sh.nh), bf16_bits(y0));
    st16(ro, qi_off(ms[q], h, i + 64u, (uint32_t)sh.nh), bf16_bits(y1));
  }
  wait_vm0();
}

// The step's keys on the eight waves (rows m = wave and wave + 8): RoPE at the row's position (lane i:
// the pair (i, i + 64)), per-token e4m3 with scale amax / 448, codes and scale into the key cache at
// (block_table[r][pos / P], pos % P)
// D0's finalize of one main-MLA head: its two 64-row tiles' K chunks added in order, times the
// per-token scale of the normalised q_a, rounded to bf16 into D2's A-operand order (16 rows,
// K = heads x 128); thread t takes columns t % 64 of both tiles for rows t / 64 and t / 64 + 8
DEV void fin_qb(const KArgs& a, const Instr& in, int wv) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t h = in.w[W_LAYER + 2], nk = in.w[W_LAYER + 5];
  const uint32_t t = (uint32_t)wv * 64u + lane(), i = t & 63u, M = (uint32_t)sh.M;
  const uint32_t ms[2] = {t >> 6, (t >> 6) + 8u};
  __amdgpu_buffer_rsrc_t rp = rsrc((const float*)s_ld64(row + FN_PART) + (size_t)2u * h * nk * 1024);
  __amdgpu_buffer_rsrc_t rs = rsrc((const void*)s_ld64(row + FN_SA));
  float x[2][2][4], sa[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t m = min(ms[q], M - 1u);
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t kk = min((uint32_t)k, nk - 1u);
        x[q][tl][k] = __uint_as_float(ld32(rp, (((uint32_t)tl * nk + kk) * 1024u + part_idx(m, i)) * 4u));
      }
    sa[q] = __uint_as_float(ld32(rs, m * 4u));
  }
  wait_vm0();
  __amdgpu_buffer_rsrc_t ro = rsrc((const void*)s_ld64(row + FN_OUT));
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (ms[q] >= M) continue;
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      float acc = x[q][tl][0];
#pragma unroll
      for (uint32_t k = 1; k < 4; ++k)
        if (k < nk) acc += x[q][tl][k];
      st16(ro, opnd_bf16(ms[q], h * (uint32_t)kMlaNope + (uint32_t)tl * 64u + i, (uint32_t)sh.mla * kMlaNope),
           bf16_bits(acc * sa[q]));
    }
  }
  wait_vm0();
}

DEV void kcache(const KArgs& a, const Instr& in, int wv) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t i = lane(), M = (uint32_t)sh.M, P = (uint32_t)sh.P;
  __amdgpu_buffer_rsrc_t rk = rsrc((const void*)s_ld64(row + KC_K));
  __amdgpu_buffer_rsrc_t rr = rsrc((const void*)s_ld64(row + KC_ROPE));
  __amdgpu_buffer_rsrc_t rc = rsrc((const void*)s_ld64(row + KC_CACHE));
  __amdgpu_buffer_rsrc_t rsc = rsrc((const void*)s_ld64(row + KC_SCALE));
  const int32_t* bt = (const int32_t*)s_ld64(row + KC_BT);
  const int32_t* pos = (const int32_t*)s_ld64(row + KC_POS);
  for (uint32_t m = (uint32_t)wv; m < M; m += kNW) {
    const float x0 = __uint_as_float(ld32(rk, (m * 128u + i) * 4u)), x1 = __uint_as_float(ld32(rk, (m * 128u + i + 64u) * 4u));
    const float c = __uint_as_float(ld32(rr, (m * 64u + i) * 8u)), sn = __uint_as_float(ld32(rr, (m * 64u + i) * 8u + 4u));
    wait_vm0();
    const float y0 = x0 * c - x1 * sn, y1 = x1 * c + x0 * sn;
    const float amax = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
    const float sc = amax > 0.f ? amax / 448.f : 1.f;
    const uint32_t p = (uint32_t)c_ld<int32_t>(pos + m), r = m / (uint32_t)sh.T;
    const uint32_t page = bt_check(a, (uint32_t)c_ld<int32_t>(bt + (size_t)r * sh.maxp + p / P), r);
    const uint32_t slot = page * P + p % P;
    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(e4m3x4(y0 / sc, 0.f, 0.f, 0.f) & 0xffu), rc, slot * 128u + i, 0, SC1);
    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)(e4m3x4(y1 / sc, 0.f, 0.f, 0.f) & 0xffu), rc, slot * 128u + i + 64u, 0, SC1);
    if (i == 0) st32(rsc, slot * 4u, __float_as_uint(sc));
  }
  wait_vm0();
}

// controller, score tasks overlapping the step's own keys: those T keys (written by the key-cache
// task this run) and their scales into the activation area (kScoreNewK, kScoreNewS)
constexpr int kScoreNewK = 0;     // [T][128] e4m3
constexpr int kScoreNewS = 1024;  // [T] fp32
DEV void score_stage(const KArgs& a, const Instr& in, char* act) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t r = in.w[W_LAYER + 1], t1 = in.w[W_LAYER + 4], T = (uint32_t)sh.T, P = (uint32_t)sh.P;
  const int32_t* pos = (const int32_t*)s_ld64(row + SC_POS);
  const uint32_t ctx = (uint32_t)c_ld<int32_t>(pos + r * T + T - 1u) + 1u;
  if (t1 <= ctx - T) return;  // no new key in this split
  const int32_t* bt = (const int32_t*)s_ld64(row + SC_BT) + (size_t)r * sh.maxp;
  const char* cache = (const char*)s_ld64(row + SC_CACHE);
  const float* scale = (const float*)s_ld64(row + SC_SCALE);
  // lane l: 16 bytes of new token l / 8 and the scale of new token l (per-lane block-table reads:
  // the new tokens may straddle a page boundary)
  const uint32_t ln = lane();
  const uint32_t tk = ctx - T + min(ln >> 3, T - 1u), ts = ctx - T + min(ln, T - 1u);
  const uint32_t sk_slot = bt_check(a, (uint32_t)bt[tk / P], r) * P + tk % P, ss_slot = bt_check(a, (uint32_t)bt[ts / P], r) * P + ts % P;
  const float sj = __uint_as_float(ld32(rsrc(scale), ss_slot * 4u));
  if (ln < 8u * T)  // chunks permuted as in the lease: chunk c of new key u at position c ^ (u mod 8)
    lds_dma16_sc1(cache + (size_t)sk_slot * 128u + (((ln & 7u) ^ (ln >> 3)) << 4), (uint32_t)(uintptr_t)(lds_void*)(act + kScoreNewK));
  wait_vm0();
  if (ln < T) *(float*)(act + kScoreNewS + ln * 4u) = sj;
}

// Indexer score of one (request, key split) on the eight waves, wave j taking token m = r T + j:
// its q (64 heads x 128, bf16) stays in registers as 16 A fragments; per 16 keys, two steps of dims
// per 64 widen the keys' e4m3 bytes to bf16 for the matrix core (exact products, fp32 sums), then
// score[t] = sum_h w[m][h] max(0, scale[t] (q_h . k_t)) -- the 4 rows of each 16-head block a lane
// holds are weighted and added, then the four 16-lane rows -- -inf past the token's position.
DEV void score_tile(const KArgs& a, const Instr& in, char* smem, uint32_t lease, int wv) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t r = in.w[W_LAYER + 1], t0 = in.w[W_LAYER + 3], t1 = in.w[W_LAYER + 4];
  const uint32_t T = (uint32_t)sh.T, nh = (uint32_t)sh.nh;
  if ((uint32_t)wv >= T) return;
  const int32_t* pos = (const int32_t*)s_ld64(row + SC_POS);
  const uint32_t m = r * T + (uint32_t)wv, pm = (uint32_t)c_ld<int32_t>(pos + m);
  const uint32_t ctx = (uint32_t)c_ld<int32_t>(pos + r * T + T - 1u) + 1u, new0 = ctx - T;
  const uint32_t lim = min(t1, new0), nko = lim > t0 ? lim - t0 : 0u;
  const uint32_t kb = (nko + 7u) >> 3;  // key blocks in the lease; the scale block follows
  const uint32_t ln = lane(), j16 = ln & 15u, g = ln >> 4;
  __amdgpu_buffer_rsrc_t rq = rsrc((const void*)s_ld64(row + SC_Q));
  __amdgpu_buffer_rsrc_t rw = rsrc((const void*)s_ld64(row + SC_W));
  u32x4 qa[4][4];
  f32x4 wv4[4];
#pragma unroll
  for (uint32_t hb = 0; hb < 4; ++hb) {
#pragma unroll
    for (uint32_t f = 0; f < 4; ++f) qa[hb][f] = ld128(rq, ((m * (nh >> 4) + hb) * 4u + f) * 1024u + ln * 16u);
    const u32x4 wq = ld128(rw, (m * nh + hb * 16u + 4u * g) * 4u);
    wv4[hb] = f32x4{__uint_as_float(wq.x), __uint_as_float(wq.y), __uint_as_float(wq.z), __uint_as_float(wq.w)};
  }
  wait_vm0();
  const char* ring = smem + kRingOff;
  const char* act = smem + kActOff;
  __amdgpu_buffer_rsrc_t ro = rsrc((const float*)s_ld64(row + SC_OUT) + (size_t)m * sh.smax);
  const uint32_t ntok = t1 - t0;
  for (uint32_t tb = 0; tb * 16u < ntok; ++tb) {
    const uint32_t tt = t0 + tb * 16u + j16;
    const uint32_t tc = min(tt, t1 - 1u);  // past the split: any of its keys, not stored
    const char* kp;
    float sk;
    uint32_t u;  // the key's index in its LDS area: chunk c sits at position c ^ (u mod 8)
    if (tc < new0) {
      u = tc - t0;
      kp = ring + ring_off(lease, u * 128u);
      sk = *(const float*)(ring + ring_off(lease, kb * 1024u + u * 4u));
    } else {
      u = tc - new0;
      kp = act + kScoreNewK + u * 128u;
      sk = *(const float*)(act + kScoreNewS + u * 4u);
    }
    f32x4 d[4];
#pragma unroll
    for (uint32_t hb = 0; hb < 4; ++hb) d[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (uint32_t s2 = 0; s2 < 2; ++s2) {
      const u32x4 kv = *(const u32x4*)(kp + (((g + 4u * s2) ^ (u & 7u)) << 4));
      const bf16x8 b0 = e4m3x8_bf16(kv.x, kv.y), b1 = e4m3x8_bf16(kv.z, kv.w);
#pragma unroll
      for (uint32_t hb = 0; hb < 4; ++hb) {
        bf16x8 a0, a1;
        __builtin_memcpy(&a0, &qa[hb][2u * s2], 16);
        __builtin_memcpy(&a1, &qa[hb][2u * s2 + 1u], 16);
        d[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, d[hb], 0, 0, 0);
        d[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, d[hb], 0, 0, 0);
      }
    }
    float p = 0.f;
#pragma unroll
    for (uint32_t hb = 0; hb < 4; ++hb) {
      p += wv4[hb].x * fmaxf(0.f, sk * d[hb].x) + wv4[hb].y * fmaxf(0.f, sk * d[hb].y);
      p += wv4[hb].z * fmaxf(0.f, sk * d[hb].z) + wv4[hb].w * fmaxf(0.f, sk * d[hb].w);
    }
    const float tot = rows_sum(p);
    if (g == 0 && tt < t1) st32(ro, tt * 4u, __float_as_uint(tt <= pm ? tot : -INFINITY));
  }
  wait_vm0();
}

// the multi-row op body of one instruction on one of the eight waves (ATTN aside)
// Top-k of one token row (the Top-2048 that follows the paged indexer score on the MegaRTP page;
// k is a plan parameter): the positions of the k largest scores among the keys t <= the token's
// position, ties to the smaller position, in ascending order, -1 past the number of keys.
// The eight waves hold the row in registers as order-preserving integer keys, lane g of the 512
// holding positions g, g + 512, ... (coalesced loads).  The bits all keys share (from a block-wide
// minimum and maximum) are fixed first; radix selection then fixes the k-th largest key 8 bits at a
// time from the highest differing bit: each wave counts the keys matching the bits fixed so far in
// its own 256-bin histogram (LDS atomics), and wave 0 sums the eight and walks the bins from the top.
// The selected positions are written in ascending order with wave ballots and two tables of
// per-(position block, wave) counts: first how many keys equal to the threshold come earlier (the
// first ones are taken), then where each selected position goes.
DEV uint32_t order_key(float f) {  // unsigned order of the keys = float order of the scores (-0 as +0)
  const uint32_t u = __float_as_uint(f) == 0x80000000u ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DEV float key_value(uint32_t kk) { return __uint_as_float((kk & 0x80000000u) ? (kk ^ 0x80000000u) : ~kk); }

// One selection pass of the top-k: every counted key (count(j)) adds 1 to bin(j) (0..255) of this
// wave's histogram; wave 0 sums the eight histograms and walks the bins from the top.  Returns the
// bin that holds the krem-th largest counted key, sets krem to that key's rank inside the bin and
// nbin to the bin's count.
template <int J, class Bin, class Count>
DEV uint32_t topk_pass(uint32_t* hist, uint32_t* ctl, int wv, uint32_t& krem, uint32_t& nbin, Bin bin, Count count) {
  const uint32_t ln = lane();
  uint32_t* mine = hist + wv * 256;
#pragma unroll
  for (int q = 0; q < 4; ++q) mine[q * 64 + (int)ln] = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (count(j)) __hip_atomic_fetch_add(mine + bin(j), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  lds_barrier();
  if (wv == 0) {  // lane l holds bins 255 - 4 l - q (q = 0..3): counts from the top
    u32x4 hv[kNW];  // the eight waves' counts of bins 252 - 4 l .. 255 - 4 l, read together
#pragma unroll
    for (int w = 0; w < kNW; ++w) hv[w] = *(const u32x4*)(hist + w * 256 + 252 - 4 * (int)ln);
    uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      c[0] += hv[w].w;
      c[1] += hv[w].z;
      c[2] += hv[w].y;
      c[3] += hv[w].x;
    }
    const uint32_t s4 = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_incl_scan(s4);
    const uint64_t hit = __builtin_amdgcn_ballot_w64(incl >= krem);  // the bins hold at least krem keys
    if (ln == (uint32_t)__builtin_ctzll(hit)) {
      uint32_t above = incl - s4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above + c[q] >= krem) {
          ctl[0] = 255u - 4u * ln - (uint32_t)q;
          ctl[1] = krem - above;
          ctl[2] = c[q];
          break;
        }
        above += c[q];
      }
    }
  }
  lds_barrier();
  krem = ctl[1];
  nbin = ctl[2];
  return ctl[0];
}

// block-wide minimum and maximum of the keys with count(j); `ctl`: 16 LDS words of its own, 16-byte aligned
template <int J, class Count>
DEV void topk_range(const uint32_t* key, uint32_t* ctl, int wv, Count count, uint32_t& lo, uint32_t& hi) {
  lo = 0xFFFFFFFFu;
  hi = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (count(j)) {
      lo = min(lo, key[j]);
      hi = max(hi, key[j]);
    }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if (lane() == 0u) {
    ctl[wv] = lo;
    ctl[8 + wv] = hi;
  }
  lds_barrier();
  const u32x4 l0 = *(const u32x4*)ctl, l1 = *(const u32x4*)(ctl + 4);  // four loads for the sixteen words
  const u32x4 h0 = *(const u32x4*)(ctl + 8), h1 = *(const u32x4*)(ctl + 12);
  lo = min(min(min(l0.x, l0.y), min(l0.z, l0.w)), min(min(l1.x, l1.y), min(l1.z, l1.w)));
  hi = max(max(max(h0.x, h0.y), max(h0.z, h0.w)), max(max(h1.x, h1.y), max(h1.z, h1.w)));
}
DEV uint32_t lanes_below(uint64_t b) {  // set bits of b in the lanes below this one
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}
// Block-wide ordering of flagged keys over (position block j, wave, lane): `bits` holds, per lane,
// a flag for each of its kTopkMaxKeys / 512 keys (bit j: position 512 j + 64 wave + lane).  Returns,
// in lane j, how many flagged keys come before position block j's part of this wave (all earlier
// blocks, then this block's earlier waves); `total`: all flagged keys.  `tab`: [J][8] LDS words.
DEV uint32_t pos_prefix(uint32_t bits, int wv, uint32_t* tab, uint32_t& total) {
  constexpr int J = kTopkMaxKeys / (kNW * 64);
  const uint32_t ln = lane();
  uint32_t mine = 0u;  // lane j: this wave's count in block j
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t c = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64((bits >> j) & 1u));
    mine = ln == (uint32_t)j ? c : mine;
  }
  if (ln < (uint32_t)J) tab[ln * kNW + wv] = mine;
  lds_barrier();
  uint32_t blk = 0u, earlier = 0u;  // lane j: block j's count over all waves, and over the waves before this one
  if (ln < (uint32_t)J) {
    const u32x4 a0 = *(const u32x4*)(tab + ln * kNW), a1 = *(const u32x4*)(tab + ln * kNW + 4);
    const uint32_t c[kNW] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      blk += c[w];
      earlier += w < wv ? c[w] : 0u;
    }
  }
  static_assert(J == 16, "the block prefix runs over one row of 16 lanes");
  const uint32_t incl = row16_incl_scan(blk);  // inclusive prefix over the J blocks (lanes 0 .. J-1)
  total = (uint32_t)__builtin_amdgcn_readlane((int)incl, J - 1);
  return incl - blk + earlier;
}
DEV void topk_row(const KArgs& a, const Instr& in, int wv) {
  constexpr int J = kTopkMaxKeys / (kNW * 64);  // keys per lane
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t m = in.w[W_LAYER + 1], k = (uint32_t)sh.topk, ln = lane();
  const uint32_t g = (uint32_t)wv * 64u + ln;
  const uint32_t nvalid = (uint32_t)c_ld<int32_t>((const int32_t*)s_ld64(row + TK_POS) + m) + 1u;
  __amdgpu_buffer_rsrc_t rs = rsrc((const float*)s_ld64(row + TK_SCORE) + (size_t)m * (uint32_t)sh.smax);
  uint32_t key[J];
#pragma unroll
  for (int j = 0; j < J; ++j)  // every load unconditional (past the row's keys: its last key again), so
    key[j] = ld32(rs, min((uint32_t)j * 512u + g, nvalid - 1u) * 4u);  // that they are in flight together
#pragma unroll
  for (int j = 0; j < J; ++j)
    key[j] = (uint32_t)j * 512u + g < nvalid ? order_key(__uint_as_float(key[j])) : 0u;  // 0: not a key of the row
  uint32_t* hist = (uint32_t*)(mk_lds + kActOff);  // [8 waves][256] bins
  uint32_t* ctl = hist + kNW * 256;                 // [2] bin, remainder; at 4 and 20 two min / max tables
  uint32_t* tab = ctl + 64;                         // [2][J][8 waves] counts per (position block, wave)
  uint32_t thr = 0u, krem = 0u;  // with k >= the keys, every key (all above 0) is taken
  uint32_t neq = 0u;             // keys equal to thr (when known without a count of its own)
  if (nvalid > k) {
    auto valid = [&](int j) { return (uint32_t)j * 512u + g < nvalid; };
    uint32_t lo, hi;
    topk_range<J>(key, ctl + 4, wv, valid, lo, hi);
    krem = k;
    thr = hi;  // all keys equal: the first k of them
    neq = nvalid;
    if (lo != hi) {
      // two passes of 256 bins linear in the score: first between the smallest and the largest key
      // (a bin is a non-decreasing function of the score, so the bins order the keys, and they spread
      // the keys whatever their exponents), then across the chosen bin's own interval; the chosen
      // sub-bin almost always holds keys of one value
      const float flo = key_value(lo), scale = 256.f / (key_value(hi) - flo);
      auto vbin = [&](int j) { return min(255u, (uint32_t)((key_value(key[j]) - flo) * scale)); };
      uint32_t nb;
      const uint32_t d0 = topk_pass<J>(hist, ctl, wv, krem, nb, vbin, valid);
      const float blo = flo + (float)d0 / scale, scale2 = fminf(256.f * scale, 3.0e38f);
      auto vbin2 = [&](int j) { return min(255u, (uint32_t)fmaxf(0.f, (key_value(key[j]) - blo) * scale2)); };
      auto in_d0 = [&](int j) { return valid(j) && vbin(j) == d0; };
      const uint32_t d1 = topk_pass<J>(hist, ctl, wv, krem, nb, vbin2, in_d0);
      auto in_d1 = [&](int j) { return in_d0(j) && vbin2(j) == d1; };
      uint32_t clo, chi;
      topk_range<J>(key, ctl + 20, wv, in_d1, clo, chi);
      thr = chi;
      neq = nb;
      if (clo != chi) {
        // then the order keys of the remaining ones, 8 bits at a time from the highest bit in which
        // they differ (keys in [clo, chi] are exactly the chosen sub-bin's)
        const int hb = 31 - __builtin_clz(clo ^ chi);
        uint32_t pmask = hb == 31 ? 0u : ~((2u << hb) - 1u), prefix = chi & pmask;
        for (int s = hb - 7;; s -= 8) {
          const uint32_t sft = (uint32_t)max(s, 0), dmask = (1u << (s > 0 ? 8 : 8 + s)) - 1u;
          const uint32_t d = topk_pass<J>(
              hist, ctl, wv, krem, nb, [&](int j) { return (key[j] >> sft) & dmask; },
              [&](int j) { return valid(j) && key[j] >= clo && key[j] <= chi && (key[j] & pmask) == prefix; });
          prefix |= d << sft;
          pmask |= dmask << sft;
          if (s <= 0) break;
        }
        thr = prefix;
        neq = nb;  // the last pass fixes every bit: its bin is the keys equal to thr
      }
    }
  }
  // ties: the krem first keys equal to thr in position order; then each selected key's output slot
  // (per-lane bit masks over the lane's J keys, so that no lane mask per key stays live)
  uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const bool v = (uint32_t)j * 512u + g < nvalid;
    gtm |= v && key[j] > thr ? 1u << j : 0u;
    eqm |= v && key[j] == thr ? 1u << j : 0u;
  }
  uint32_t selm = gtm | eqm;
  if (krem < neq) {  // only some of the equal keys: the krem first in position order
    uint32_t tot;
    const uint32_t eq_pos = pos_prefix(eqm, wv, tab, tot);
    selm = gtm;
#pragma unroll
    for (int j = 0; j < J; ++j)  // this lane's equal keys in position order: take those before the krem-th
      selm |= ((eqm >> j) & 1u) && __builtin_amdgcn_readlane(eq_pos, j) + lanes_below(__builtin_amdgcn_ballot_w64((eqm >> j) & 1u)) < krem
                  ? 1u << j : 0u;
  }
  uint32_t run;
  const uint32_t sel_pos = pos_prefix(selm, wv, tab + J * kNW, run);
  __amdgpu_buffer_rsrc_t ro = rsrc((const int32_t*)s_ld64(row + TK_OUT) + (size_t)m * k);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t o = __builtin_amdgcn_readlane(sel_pos, j) + lanes_below(__builtin_amdgcn_ballot_w64((selm >> j) & 1u));
    if ((selm >> j) & 1u) st32(ro, o * 4u, (uint32_t)j * 512u + g);
  }
  for (uint32_t i = run + g; i < k; i += (uint32_t)kNW * 64u) st32(ro, i * 4u, 0xFFFFFFFFu);
  wait_vm0();
}

// LD: the instance with loader waves (the Qwen3 layers), which never runs the indexer's ops (key
// cache, score, top-k, the D1 / D0 finalizes, the main-MLA BMM): their code stays out of that
// instance's register allocation (with them in, it spilled 492 scalar registers instead of 298).
// RG: plans of more than 16 rows (row-group GEMM tiles and finalizes).
template <bool LD, bool RG>
DEV void m16_body(const KArgs& a, const Instr& in, char* smem, uint32_t lease, int wv) {
  const uint32_t op = in.w[W_OPCODE];
  if (op == OP_GEMM) {
    if constexpr (RG) {  // plans of more than 16 rows: their own kernel instance
      // 16 steps of 1 KiB: bf16 chunks are always 512 wide, and the planner takes e4m3 plans beyond
      // 16 rows only with chunks of 1024
      if (a.sh.fp8) gemm_tile_groups<true, 16>(a, in, smem, lease, wv);
      else gemm_tile_groups<false, 16>(a, in, smem, lease, wv);
    } else if (a.sh.fp8 && in.w[W_LAYER + 1] != K_UK) {
      const uint32_t kc = in.w[W_LAYER + 6];  // the layers' e4m3 chunks are 1024; the indexer's 1024 or 768
      if (LD || kc == 1024u) gemm_tile<true, 4>(a, in, smem, lease, wv);
      else if (kc == 768u) gemm_tile<true, 3>(a, in, smem, lease, wv);
      else gemm_tile<true, 0>(a, in, smem, lease, wv);
    } else if (!LD && in.w[W_LAYER + 1] == K_UK) {  // the main-MLA query BMM (indexer front only)
      gemm_tile<false, kMlaNope / 64>(a, in, smem, lease, wv);
    } else {
      gemm_tile<false, 8>(a, in, smem, lease, wv);
    }
  } else if (op == OP_NORM) {
    if (a.sh.fp8) norm_row<true>(a, in, smem, lease, wv);
    else norm_row<false>(a, in, smem, lease, wv);
  } else if (op == OP_FIN) {
    const uint32_t nk = in.w[W_LAYER + 5];
    if (!LD && in.w[W_LAYER + 1] == K_QI) fin_qi(a, in, wv);
    else if (!LD && in.w[W_LAYER + 1] == K_QB) fin_qb(a, in, wv);
    else if (nk <= 4) fin_tile<4, RG>(a, in, wv);
    else if (nk <= 8) fin_tile<8, RG>(a, in, wv);
    else if (nk <= 12) fin_tile<12, RG>(a, in, wv);
    else fin_tile<kMaxChunks, RG>(a, in, wv);
  } else if (op == OP_QUANT) {
    quant_row(a, in, smem, wv);
  } else if (op == OP_COMB) {
    comb_group(a, in, wv);
  } else if (LD) {  // the indexer's ops below never run in the Qwen3 layers' loader instance
  } else if (op == OP_KCACHE) {
    kcache(a, in, wv);
  } else if (op == OP_SCORE) {
    score_tile(a, in, smem, lease, wv);
  } else if (op == OP_TOPK) {
    topk_row(a, in, wv);
  }
}

// controller: a projection tile's input chunk into the activation area (skipped when the previous
// instruction staged the same chunk and nothing has written the area since)
template <bool RG>
DEV void gemm_stage(const KArgs& a, const Instr& in, char* act, uint64_t& staged) {
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const uint32_t kind = in.w[W_LAYER + 1], kc = in.w[W_LAYER + 6];
  // the main-MLA query BMM reads its head's 128 columns of the D0 output (payload word 7), in bf16
  const uint32_t k0 = kind == K_UK ? in.w[W_LAYER + 7] : in.w[W_LAYER + 5];
  if (RG) return;  // more than 16 rows: the waves read their groups' chunks themselves
  const bool f8 = a.sh.fp8 && kind != K_UK;
  const uint32_t off = f8 ? (k0 >> 6) * 1024u : (k0 >> 5) * 1024u;
  const uint32_t bytes = f8 ? (kc >> 6) * 1024u : (kc >> 5) * 1024u;  // at most kActABytes
  const char* src = (const char*)s_ld64(row + GM_ACT) + off;
  if ((uint64_t)src == staged) return;
  stage(src, bytes, act + kActA);
  wait_vm0();
  staged = (uint64_t)src;
}

// ---------------------------------------------------------------------------------------
// controller epilogues

// record arrival in the instruction's group; true for the producer that completes the group,
// which also re-arms the counter for the next run
DEV bool arrive(const KArgs& a, const Instr& in) {
  uint32_t old = 0;
  uint32_t* ctr = a.arrivals + (size_t)in.w[W_ARR_ID] * kSubStride;
  if (lane() == 0) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __builtin_amdgcn_readfirstlane(old);
  const bool last = old == in.w[W_ARR_N] - 1;
  if (last && lane() == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// controller timestamps of one instruction (trace runs of the kernels without loader waves, whose
// loader 0 uses these words): 5, 6 when its stores were acknowledged and its arrival resolved, 10, 11
// when a split combine was staged and computed
struct Stamps {
  uint32_t i;
  bool on;
};

// four consecutive attention-output elements k .. k + 3 of row r: M = 1 plans as tagged records of
// bf16 pairs; multi-row plans in the O projection's operand order (bf16), or as fp32 rows for the
// per-token quantisation (W8A8)
template <int S>
DEV void o_store(const KArgs& a, const Instr& in, __amdgpu_buffer_rsrc_t ro, uint32_t r, uint32_t k, f32x4 v,
                 uint32_t tag) {
  const uint32_t w = (uint32_t)a.sh.Hq * 128u;
  if (S == 0)
    ll_put2(ro, (r * w + k) / 2u, pack_bf2(v.x, v.y), pack_bf2(v.z, v.w), tag);
  else if (!a.sh.fp8)
    st64(ro, opnd_bf16(r, k, w), u32x2{pack_bf2(v.x, v.y), pack_bf2(v.z, v.w)});
  else
    st128(ro, (r * w + k) * 4u, u32x4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)});
}

// Store the split's partial (and, for the split holding the new token, the cache rows).  M = 1
// plans: record arrival; the split completing its group combines it (true for that worker).
// Multi-row plans: the last split of a chain stores the chain's partial and signals the group's
// event; a combine task reduces the group's chains.
template <int S>
DEV bool attn_epilogue(const KArgs& a, const Instr& in, char* smem, const Stamps& st) {
  const Shapes& sh = a.sh;
  const int g = sh.g;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const int r = in.w[W_P1], hk = in.w[W_P2], s = in.w[W_P3];
  const int ns = attn_splits<S>(in);
  const uint32_t pstride = (uint32_t)g * 128u + 8u;  // floats per split: g*128 O, g lse, padding
  const uint32_t gbase = ((uint32_t)(r * sh.Hkv + hk) * (uint32_t)sh.max_splits) * pstride;
  float* part = (float*)s_ld64(row + ATT_PART);
  __amdgpu_buffer_rsrc_t rp = rsrc(part);
  const float* out = (const float*)(smem + kOutOff);
  // multi-row plans: the partial of a chain of splits, by its last split, in the chain's slot
  if (S == 0 || (in.w[W_CHAIN] & 2u) != 0u) {
    const uint32_t slot = S == 1 ? in.w[W_PSLOT] : (uint32_t)s;
    for (int e = (int)lane(); e < g * 129; e += 64)
      st32(rp, (gbase + slot * pstride + e) * 4u, __float_as_uint(out[e]));
  }
  if (s == ns - 1) {  // the split holding the new token writes its K / V row into the paged caches
    const int p = (int)in.w[W_P5] - 1;
    const int32_t* bt = (const int32_t*)s_ld64(row + ATT_BT) + (size_t)r * sh.maxp;
    const int page = (int)bt_page(a, bt + p / sh.P, (uint32_t)r);
    const size_t rowi = ((size_t)page * sh.P + (p % sh.P)) * sh.Hkv + hk;
    const uint32_t* kl = (const uint32_t*)(smem + kActOff + kActK);
    const uint32_t* vl = (const uint32_t*)(smem + kActOff + kActV);
    st32(rsrc((uint16_t*)s_ld64(row + ATT_KC) + rowi * 128), lane() * 4u, kl[lane()]);
    st32(rsrc((uint16_t*)s_ld64(row + ATT_VC) + rowi * 128), lane() * 4u, vl[lane()]);
  }
  if (S == 1) return false;  // multi-row plans: the controller completes the stores and signals later
  wait_vm0();
  if (st.on) tput(a, st.i, 5, rtc());
  const bool last = arrive(a, in);
  if (st.on) tput(a, st.i, 6, rtc());
  if (!last) return false;
  // combine the group's splits, o = sum_i exp(lse_i - lse) O_i with lse = log sum_i exp(lse_i)
  // o: tagged records of bf16 pairs, [request][Hq * 128 / 2]
  char* act = smem + kActOff;
  __amdgpu_buffer_rsrc_t ro = rsrc((const void*)s_ld64(row + ATT_O));
  const uint32_t kbase = (uint32_t)hk * g * 128u, otag = ll_tag(a, in.w[W_LAYER]);
  if ((uint32_t)ns * pstride * 4u <= (uint32_t)kActStageBytes && ns <= 64) {
    // every split at once: lane t < ns takes the weights of split t, then lanes over 4-dim units
    // accumulate the outputs in split order
    stage(part + gbase, (uint32_t)ns * pstride * 4u, act);
    wait_vm0();
    if (st.on) tput(a, st.i, 10, rtc());
    const float* pl = (const float*)act;
    float* wts = (float*)(smem + kOutOff);  // [64][kMaxG] normalised weights
    const int ln = (int)lane();
    for (int j = 0; j < g; ++j) {
      const float lv = ln < ns ? pl[ln * pstride + g * 128 + j] : -INFINITY;
      const float M = wave_max(lv);
      const float e = ln < ns ? __expf(lv - M) : 0.f;
      const float sum = wave_sum(e);
      if (ln < ns) wts[ln * kMaxG + j] = e / sum;
    }
    for (int u = 0; u * 256 < g * 128; ++u) {
      const int oi = u * 256 + 4 * ln;
      if (oi < g * 128) {
        const int j = oi >> 7;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int t = 0; t < ns; ++t) acc += wts[t * kMaxG + j] * *(const f32x4*)(pl + t * pstride + oi);
        o_store<S>(a, in, ro, (uint32_t)r, kbase + (uint32_t)oi, acc, otag);
      }
    }
    if (st.on) tput(a, st.i, 11, rtc());
    return true;
  }
  // many splits: online over chunks of splits staged into LDS: lanes over splits take the
  // statistics, lanes over 4-dim units accumulate the outputs
  float* wts = (float*)(smem + kOutOff);          // [64][kMaxG] weights of the chunk's splits
  float* hst = (float*)(smem + kOutOff) + 64 * kMaxG;  // [kMaxG][3]: running max, sum, chunk rescale
  const uint32_t chunk = min(64u, (uint32_t)kActStageBytes / (pstride * 4u));
  const int ln = (int)lane();
  float acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[u][q] = 0.f;
  if (ln < g) {
    hst[ln * 3] = -INFINITY;
    hst[ln * 3 + 1] = 0.f;
  }
  for (int t0 = 0; t0 < ns; t0 += (int)chunk) {
    const int nc = min((int)chunk, ns - t0);
    stage(part + gbase + (uint32_t)t0 * pstride, (uint32_t)nc * pstride * 4u, act);
    wait_vm0();
    if (st.on && t0 == 0) tput(a, st.i, 10, rtc());
    const float* pl = (const float*)act;
    for (int j = 0; j < g; ++j) {
      const float lv = ln < nc ? pl[ln * pstride + g * 128 + j] : -INFINITY;
      const float mo = hst[j * 3];
      const float mn = fmaxf(mo, wave_max(lv));
      const float w = ln < nc ? __expf(lv - mn) : 0.f;
      const float ws = wave_sum(w);
      const float sc = __expf(mo - mn);
      wts[ln * kMaxG + j] = w;
      if (ln == 0) {
        hst[j * 3] = mn;
        hst[j * 3 + 1] = hst[j * 3 + 1] * sc + ws;
        hst[j * 3 + 2] = sc;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int unit = ln + 64 * u;
      if (unit < g * 32) {
        const int j = unit >> 5, c4 = unit & 31;
        const float sc = hst[j * 3 + 2];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[u][q] *= sc;
#pragma unroll 8
        for (int t = 0; t < nc; ++t) {
          const float w = wts[t * kMaxG + j];
          const u32x4 ov = *(const u32x4*)(pl + t * pstride + j * 128 + c4 * 4);
          acc[u][0] += w * __uint_as_float(ov.x);
          acc[u][1] += w * __uint_as_float(ov.y);
          acc[u][2] += w * __uint_as_float(ov.z);
          acc[u][3] += w * __uint_as_float(ov.w);
        }
      }
    }
  }
  if (st.on) tput(a, st.i, 11, rtc());
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int unit = ln + 64 * u;
    if (unit < g * 32) {
      const int j = unit >> 5, c4 = unit & 31;
      const float inv = 1.f / hst[j * 3 + 1];
      const f32x4 v = {acc[u][0] * inv, acc[u][1] * inv, acc[u][2] * inv, acc[u][3] * inv};
      o_store<S>(a, in, ro, (uint32_t)r, kbase + (uint32_t)(j * 128 + c4 * 4), v, otag);
    }
  }
  return true;
}

// (max, smallest index) over the wave
DEV void argmax_merge(float& best, int& bi) {
  for (int sh = 32; sh >= 1; sh >>= 1) {
    const float ob = __shfl_xor(best, sh);
    const int oi = __shfl_xor(bi, sh);
    if (ob > best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
}

struct LmState {
  float best;
  int idx;
};

DEV void gemv_epilogue(const KArgs& a, const Instr& in, const char* smem, LmState& lm, const Stamps& st) {
  const uint32_t op = in.w[W_OPCODE];
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const int n0 = in.w[W_P1], nr = in.w[W_P2];
  const float* part = (const float*)(smem + kOutOff);  // block sums of the tile
  const int KB = (int)in.w[W_P4] >> 9;  // quads per row
  const int j = (int)lane();
  const uint32_t tag = ll_tag(a, in.w[W_LAYER]);
  if (op == OP_QKV) {  // qkv rows as tagged fp32 records
    __amdgpu_buffer_rsrc_t ro = rsrc((const void*)s_ld64(row + QKV_OUT));
    for (int jj = j; jj < nr; jj += 64) ll_put(ro, (uint32_t)(n0 + jj), __float_as_uint(row_sum(part, jj, KB)), tag);
  } else if (op == OP_OPROJ) {  // r2 = r1 + bf16(a) as tagged records (and the caller's r2 after the last layer)
    __amdgpu_buffer_rsrc_t r2 = rsrc((const void*)s_ld64(row + O_R2));
    const uint64_t out = s_ld64(row + O_R2OUT);
    const char* r1 = smem + kActOff + kActR1;
    for (int jj = j; jj < nr; jj += 64) {
      const float av = bf2f(pack_bf2(row_sum(part, jj, KB), 0.f) & 0xffffu);
      const float v = ll_f32(r1, jj) + av;
      ll_put(r2, (uint32_t)(n0 + jj), __float_as_uint(v), tag);
      if (out) st32(rsrc((const void*)out), (uint32_t)(n0 + jj) * 4u, __float_as_uint(v));
    }
  } else if (op == OP_GATEUP) {  // m = silu(gate) * up, bf16 pairs as tagged records (nr is even)
    __amdgpu_buffer_rsrc_t rm = rsrc((const void*)s_ld64(row + GU_M));
    for (int pp = j; pp < nr / 2; pp += 64) {
      const float g0 = row_sum(part, 2 * pp, KB), u0 = row_sum(part, nr + 2 * pp, KB);
      const float g1 = row_sum(part, 2 * pp + 1, KB), u1 = row_sum(part, nr + 2 * pp + 1, KB);
      ll_put(rm, (uint32_t)(n0 / 2 + pp), pack_bf2(g0 / (1.f + __expf(-g0)) * u0, g1 / (1.f + __expf(-g1)) * u1), tag);
    }
  } else if (op == OP_DOWN) {  // y = bf16(m W^T); r1 of the next layer = r2 + y as tagged records
    __amdgpu_buffer_rsrc_t r1 = rsrc((const void*)s_ld64(row + DN_R1));
    const uint64_t yout = s_ld64(row + DN_Y);
    const char* r2 = smem + kActOff + kActR1;
    for (int jj = j; jj < nr; jj += 64) {
      const uint32_t yb = pack_bf2(row_sum(part, jj, KB), 0.f) & 0xffffu;
      ll_put(r1, (uint32_t)(n0 + jj), __float_as_uint(ll_f32(r2, jj) + bf2f(yb)), tag);
      if (yout) st16(rsrc((const void*)yout), (uint32_t)(n0 + jj) * 2u, yb);
    }
  } else if (op == OP_LMHEAD) {
    // the body stored the logits; lane w < 8 takes wave w's (max, first index)
    __amdgpu_buffer_rsrc_t rp = rsrc((const void*)s_ld64(row + LM_PART));
    float best = j < kNW ? part[2 * j] : -INFINITY;
    int bi = j < kNW ? ((const int*)part)[2 * j + 1] : 0x7fffffff;
    argmax_merge(best, bi);
    if (best > lm.best || (best == lm.best && bi < lm.idx)) {
      lm.best = best;
      lm.idx = bi;
    }
    const uint32_t slot = in.w[W_ARR_RANK];
    if (slot == kNone) return;  // not this worker's last lm_head task
    if (j == 0) {
      st32(rp, slot * 8u, __float_as_uint(lm.best));
      st32(rp, slot * 8u + 4u, (uint32_t)lm.idx);
    }
    wait_vm0();
    if (st.on) tput(a, st.i, 5, rtc());
    const bool last = arrive(a, in);
    if (st.on) tput(a, st.i, 6, rtc());
    if (!last) return;
    const uint32_t n = in.w[W_ARR_N];
    best = -INFINITY;
    bi = 0x7fffffff;
    for (uint32_t t0 = 0; t0 < n; t0 += 512) {
      u32x4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t t = t0 + 128u * q + 2u * (uint32_t)j;
        if (t < n) v[q] = ld128(rp, t * 8u);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t t = t0 + 128u * q + 2u * (uint32_t)j;
        if (t < n) {
          const float v0 = __uint_as_float(v[q].x);
          if (v0 > best || (v0 == best && (int)v[q].y < bi)) { best = v0; bi = (int)v[q].y; }
          if (t + 1 < n) {
            const float v1 = __uint_as_float(v[q].z);
            if (v1 > best || (v1 == best && (int)v[q].w < bi)) { best = v1; bi = (int)v[q].w; }
          }
        }
      }
    }
    argmax_merge(best, bi);
    if (j == 0) st32(rsrc((const void*)s_ld64(row + LM_TOKEN)), 0, (uint32_t)bi);
    wait_vm0();
    return;
  }
  if (st.on) tput(a, st.i, 5, rtc());
}

// ---------------------------------------------------------------------------------------
// the two roles

// Multi-row kernel: loader wave k of kLoaders.  The loaders walk the queue ahead of the eight
// compute-group waves, lease ring pages to instructions in queue order (each loader keeps the same
// lease table; loader 0's is the one the compute group reads), stream their share of each lease
// (a contiguous run of its blocks), and publish in order how many instructions' shares have
// landed.  Pages of an instruction are reused once the compute group has retired it.  Loaders take
// no barrier, so a full memory pipeline stalls only them, never the op bodies.
template <int S>
DEV void loader(const KArgs& a, const uint32_t* base, int count, int stride, int k, char* smem) {
  volatile uint32_t* ctrl = (volatile uint32_t*)(smem + kCtrlOff);
  volatile uint32_t* done = (volatile uint32_t*)(smem + kCtrlOff + kDoneOff) + k;
  const volatile uint32_t* retired = (const volatile uint32_t*)(smem + kCtrlOff + kRetiredOff);
  uint32_t* lease_tab = (uint32_t*)(smem + kCtrlOff + kLeaseTabOff) + k * 32;  // [16] lease, [16] issued_end
  const bool noop_only = a.flags & MK_FLAG_NOOP_ONLY;
  const int lookahead = (a.flags & MK_FLAG_NO_PREFETCH) ? 0 : 15;  // lease slots are indexed mod 16
  uint32_t head = 0, issued = 0;
  int j = 0;  // next instruction to lease
  int d = 0;  // instructions whose share has landed
  int have = -1;  // the instruction whose prefetch descriptor pf / npg hold
  Pf<S> pf;
  uint32_t npg = 0;
  uint32_t idle = 0;
  while (d < count) {
    const int r = (int)uni(*retired);
    while (j < count && j <= r + lookahead) {
      const bool tr0 = (a.flags & MK_FLAG_TRACE) && a.trace && k == 0 && lane() == 0;
      if (have != j) {  // the descriptor is kept while the instruction waits for free pages
        if (tr0) a.trace[((size_t)blockIdx.x * a.L + j) * kTraceWords + 11] = (uint32_t)rtc();  // loader 0: first look
        Instr nx;
        fetch(base + (size_t)uni((uint32_t)j) * stride, nx);
        if (k == 0) {  // publish the words for the controller
          put_instr(smem, j, nx);
          if (lane() == 0) *(volatile uint32_t*)(smem + kCtrlOff + kFetchedOff) = (uint32_t)j + 1u;
        }
        npg = 0;
        if (nx.w[W_OPCODE] != OP_NOOP && !noop_only) {
          pf_desc<S>(a, nx, pf);
          npg = (pf_blocks(pf) + 15u) >> 4;
        }
        have = j;
      }
      if (npg) {
        const uint32_t freed = j > r ? uni(lease_tab[r & 15]) : head;  // pages before instruction r are free
        if (head + npg - freed > (uint32_t)kNPages) break;
        if (tr0) a.trace[((size_t)blockIdx.x * a.L + j) * kTraceWords + 10] = (uint32_t)rtc();  // its pages are free
        pf_issue<S>(a, pf, head, k, issued, smem, kLoaders);
      }
      if ((a.flags & MK_FLAG_TRACE) && a.trace && k == 0 && lane() == 0)  // loader 0: lease issued
        a.trace[((size_t)blockIdx.x * a.L + j) * kTraceWords + 5] = (uint32_t)rtc();
      lease_tab[j & 15] = head;
      lease_tab[16 + (j & 15)] = issued;
      head += npg;
      ++j;
    }
    if (d < j) {  // the oldest leased instruction: wait for this loader's share, then publish it
      wait_vm_le(issued - uni(lease_tab[16 + (d & 15)]));
      if ((a.flags & MK_FLAG_TRACE) && a.trace && k == 0 && lane() == 0)  // loader 0: its share landed
        a.trace[((size_t)blockIdx.x * a.L + d) * kTraceWords + 6] = (uint32_t)rtc();
      ++d;
      if (lane() == 0) *done = (uint32_t)d;
      idle = 0;
      continue;
    }
    // nothing in flight and nothing that fits: wait for the compute group to retire an instruction
    __builtin_amdgcn_s_sleep(2);
    if ((++idle & 0xFFFFu) == 0u && (*ctrl != 0u || idle >= 0x800000u)) {
      if (lane() == 0 && *ctrl == 0u) *ctrl = 2u;
      break;
    }
  }
  wait_vm0();  // no LDS-bound load may be in flight when the block retires
}

// multi-row kernel, controller: wait until every loader has landed its share of instruction i
DEV bool wait_loaders(const char* smem, int i) {
  const volatile uint32_t* done = (const volatile uint32_t*)(smem + kCtrlOff + kDoneOff);
  const volatile uint32_t* ctrl = (const volatile uint32_t*)(smem + kCtrlOff);
  for (uint32_t it = 1;; ++it) {
    bool all = true;
#pragma unroll
    for (int k = 0; k < kLoaders; ++k) all = all && (int)uni(done[k]) > i;
    if (all) return true;
    __builtin_amdgcn_s_sleep(1);
    if ((it & 0xFFFFFu) == 0u && (*ctrl != 0u || it >= 0x1400000u)) return false;
  }
}

template <int S, bool LD, bool RG>
DEV void controller(const KArgs& a, const uint32_t* base, int count, int stride, char* smem) {
  uint32_t* ctrl = (uint32_t*)(smem + kCtrlOff);  // LDS; read and written only across barriers
  const bool noop_only = a.flags & MK_FLAG_NOOP_ONLY;
  const bool graph = a.flags & kModeGraph;
  uint32_t last_row = 0xFFFFFFFFu;
  LmState lm{-INFINITY, 0x7fffffff};
  WaitCache wc{0xFFFFFFFFu, 0u};
  uint64_t staged = 0;  // multi-row: the projection input chunk held in the activation area
  SigPend pend{0u, 0u, 0u, 0u, 0u};
  bool pending = false;  // multi-row: the previous instruction's signals wait for its stores
  for (int i = 0; i < count; ++i) {
    Instr in;
    if (LD) {
      if ((int)uni(*(volatile uint32_t*)(smem + kCtrlOff + kFetchedOff)) > i)
        get_instr(smem, i, in);  // loader 0 has copied it into the instruction ring
      else
        fetch(base + (size_t)i * stride, in);
    } else if (!get_instr8<S>(smem, i, in)) {  // compute wave 0 may have copied it
      fetch(base + (size_t)i * stride, in);
    }
    const uint32_t op = in.w[W_OPCODE];
    if (op == OP_NOOP) {
      if (S == 1 && lane() == 0) *(volatile uint32_t*)(smem + kCtrlOff + kRetiredOff) = (uint32_t)i + 1u;
      continue;
    }
    constexpr bool m16 = S == 1;
    const bool tracing = a.flags & MK_FLAG_TRACE;
    if (tracing) tput(a, (uint32_t)i, 0, rtc());
    const bool fused_norm = op == OP_QKV || op == OP_GATEUP || (op == OP_LMHEAD && last_row != in.w[W_ROW]);
    const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
    const uint64_t row_touch = s_ld64(row);  // the pointer row into the scalar cache before the epilogue reads it
    // single-token kernel: both cache lines of the next instruction's pointer row too, so that its
    // prologue's pointer loads hit the scalar cache
    uint64_t next_touch0 = 0, next_touch1 = 0;
    if (!LD && !m16) {
      const uint32_t nrow = ring8_row<S>(smem, i + 1);
      if (nrow != 0xFFFFFFFFu) {
        const uint64_t* nr = a.table + (size_t)nrow * kTableSlots;
        next_touch0 = s_ld64(nr);
        next_touch1 = s_ld64(nr + 8);
      }
    }
    char* act = smem + kActOff;
    // the instruction's wait: its tagged inputs staged into LDS (the graph baseline's stream order
    // already guarantees them, so it stages without checking tags)
    uint32_t poll = 0;
    bool ok = true;
    StageStamps sst{(uint32_t)i};
    if constexpr (m16) {
      // multi-row: wait for the event counters (the graph baseline's stream order guarantees them),
      // then stage what the op reads from LDS
      if (pending && !graph && !waits_cached(in, wc)) {  // a wait that may poll: no signal of ours held back
        wait_vm0();
        signal_pend(a, pend);
        pending = false;
      }
      ok = graph || wait_events(a, in, poll, wc);
      if (tracing) tput(a, (uint32_t)i, 14, rtc());  // multi-row: events met
      if (ok && op == OP_ATTN && (in.w[W_CHAIN] & 1u) == 0u) ok = attn_stage(a, in, act, false, poll, sst);  // a chain's first split
      if (ok && op == OP_GEMM) gemm_stage<RG>(a, in, act, staged);
      if (ok && op == OP_SCORE) score_stage(a, in, act);
      if (op != OP_GEMM) staged = 0;
      if (tracing) tput(a, (uint32_t)i, 15, rtc());  // multi-row: staging done
      if (LD && ok && !wait_loaders(smem, i)) {  // the loaders' shares of this lease
        record_timeout(a, in, 0xB0u, 0u);
        ok = false;
      }
      if (pending) {  // the staging and the loaders' wait above mostly covered our stores' round trip
        wait_vm0();
        signal_pend(a, pend);
        pending = false;
      }
    } else if (op == OP_ATTN)
      ok = attn_stage(a, in, act, !graph, poll, sst);
    else if (op == OP_OPROJ)
      ok = oproj_prologue(a, in, row, act, !graph, poll, sst);
    else if (op == OP_DOWN)
      ok = down_prologue(a, in, row, act, !graph, poll, sst);
    else if (fused_norm)
      ok = norm_prologue(a, in, row, act, smem, !graph, noop_only, poll, sst);
    last_row = in.w[W_ROW];
    if (tracing) {
      const unsigned long long t_ready = rtc();
      tput(a, (uint32_t)i, 1, t_ready);
      tput(a, (uint32_t)i, 2, t_ready);
    }
    const Stamps st{(uint32_t)i, tracing && !LD};
    if (!ok && lane() == 0) ctrl[0] = 1u;
    lds_barrier();  // A: activations staged, prefetch of this instruction landed
    if (tracing) tput(a, (uint32_t)i, 3, rtc());
    if (!ok) break;
    if (m16 && uni(ctrl[0]) != 0u) {  // a barrier or a loader of this block gave up (watchdog)
      record_timeout(a, in, 0xBAu, 0u);
      break;
    }
    if (!noop_only) {  // the controller is the eighth wave of every op body
      const uint32_t lease = uni(((const uint32_t*)(smem + kCtrlOff + kLeaseTabOff))[i & 15]);  // compute wave 0's table
      if (op == OP_ATTN)
        attn_compute<S>(a, in, smem, act, lease, kNW - 1);
      else if constexpr (m16)
        m16_body<LD, RG>(a, in, smem, lease, kNW - 1);
      else
        proj_body(a, in, smem, lease, fused_norm, kNW - 1);
    }
    lds_barrier();  // B: compute done, results in the output area
    if (m16 && lane() == 0) *(volatile uint32_t*)(smem + kCtrlOff + kRetiredOff) = (uint32_t)i + 1u;  // its pages are free
    if (tracing) tput(a, (uint32_t)i, 4, rtc());
    if constexpr (m16) {
      // stores only; norm / finalize / quantise / combine / key-cache / score bodies completed theirs
      // in every wave before B
      if (op == OP_ATTN)
        attn_epilogue<S>(a, in, smem, st);
      else if (op == OP_GEMM)
        gemm_epilogue<LD, RG>(a, in, smem);
      pend = sig_of(in);
      pending = true;
    } else if (op == OP_ATTN) {
      attn_epilogue<S>(a, in, smem, st);
    } else {
      gemv_epilogue(a, in, smem, lm, st);
    }
    asm volatile("" ::"s"(row_touch), "s"(next_touch0), "s"(next_touch1));
    if (tracing) {
      tput(a, (uint32_t)i, 7, rtc());
      tput(a, (uint32_t)i, 8, poll);
    }
  }
  if (pending) {  // the last instruction's signals
    wait_vm0();
    signal_pend(a, pend);
  }
}

template <int S, bool LD, bool RG>
DEV void compute(const KArgs& a, const uint32_t* base, int count, int stride, int cw, char* smem) {
  const uint32_t* ctrl = (const uint32_t*)(smem + kCtrlOff);  // LDS abort flag
  constexpr bool loaders = LD;  // loader waves stream the leases
  uint32_t* lease_tab = (uint32_t*)(smem + kCtrlOff + kLeaseTabOff) + cw * 32;  // [16] lease, [16] issued_end
  const bool noop_only = a.flags & MK_FLAG_NOOP_ONLY;
  const bool stamp = cw == 0 && (a.flags & MK_FLAG_TRACE) && a.trace;  // lease issue times into trace word 9
  const int lookahead = (a.flags & MK_FLAG_NO_PREFETCH) ? 0 : 15;
  uint32_t head = 0, issued = 0;
  uint32_t last_row = 0xFFFFFFFFu;  // as in the controller: the lm_head norm runs once per worker
  int pf_i = 0;
  for (int i = 0; i < count; ++i) {
    Instr in;
    fetch(base + (size_t)i * stride, in);
    const uint32_t op = in.w[W_OPCODE];
    if (op == OP_NOOP) {
      if (pf_i <= i) pf_i = i + 1;
      continue;
    }
    const bool fused_norm = op == OP_QKV || op == OP_GATEUP || (op == OP_LMHEAD && last_row != in.w[W_ROW]);
    if (!loaders && !noop_only) {
      // pages of every instruction before i are free now
      const uint32_t freed = (pf_i > i) ? uni(lease_tab[i & 15]) : head;
      if (pf_i < i) pf_i = i;
      // The multi-row kernel without loader waves (the indexer front, graph nodes) issues only this
      // instruction's own lease here and the leases ahead once a body is done (below): its bodies read
      // global memory themselves, and a worker's first instructions no longer wait behind the whole
      // lookahead (indexer front 50.8 -> 47.4 us against issuing ahead here).
      const int ahead = S == 1 ? 0 : lookahead;
      while (pf_i < count && pf_i <= i + ahead) {
        Instr nx;
        fetch(base + (size_t)uni((uint32_t)pf_i) * stride, nx);  // pf_i is wave-uniform: scalar loads
        if (cw == 0 && pf_i - i < 8) put_instr8<S>(smem, pf_i, nx);  // for the controller
        if (nx.w[W_OPCODE] == OP_NOOP) {
          lease_tab[pf_i & 15] = head;
          lease_tab[16 + (pf_i & 15)] = issued;
          ++pf_i;
          continue;
        }
        Pf<S> pf;
        pf_desc<S>(a, nx, pf);
        const uint32_t npg = (pf_blocks(pf) + 15u) >> 4;
        if (head + npg - freed > (uint32_t)kNPages) break;
        // bounded depth: loads in flight queue ahead of the controller's staging in this CU's
        // memory pipeline, so leases beyond kLookPages pages from instruction i's wait
        if (pf_i > i && head + npg - uni(lease_tab[i & 15]) > (uint32_t)kLookPages) break;
        pf_issue<S>(a, pf, head, cw, issued, smem);
        if (stamp && lane() == 0) a.trace[((size_t)blockIdx.x * a.L + pf_i) * kTraceWords + 9] = (uint32_t)rtc();
        lease_tab[pf_i & 15] = head;
        lease_tab[16 + (pf_i & 15)] = issued;
        head += npg;
        ++pf_i;
      }
      wait_vm_le(issued - uni(lease_tab[16 + (i & 15)]));
    }
    lds_barrier();  // A
    if (uni(ctrl[0])) break;
    if (!noop_only) {
      // with loaders: loader 0's lease table (the loaders landed this lease before barrier A)
      const uint32_t lease = loaders ? uni(((const uint32_t*)(smem + kCtrlOff + kLeaseTabOff))[i & 15]) : uni(lease_tab[i & 15]);
      char* act = smem + kActOff;
      if (op == OP_ATTN) {
        attn_compute<S>(a, in, smem, act, lease, cw);
      } else if constexpr (S == 1) {
        m16_body<LD, RG>(a, in, smem, lease, cw);
      } else {
        proj_body(a, in, smem, lease, fused_norm, cw);
      }
    }
    last_row = in.w[W_ROW];
    lds_barrier();  // B
    if (S == 1 && !loaders && !noop_only) {  // the leases ahead, once this body is done
      // instruction i's pages are free once every wave has passed B; the same bounds as above, with
      // instruction i + 1 as the one the block is at
      const uint32_t freed = pf_i > i + 1 ? uni(lease_tab[(i + 1) & 15]) : head;
      if (pf_i < i + 1) pf_i = i + 1;
      while (pf_i < count && pf_i <= i + lookahead) {
        Instr nx;
        fetch(base + (size_t)uni((uint32_t)pf_i) * stride, nx);
        if (cw == 0 && pf_i - i < 8) put_instr8<S>(smem, pf_i, nx);
        if (nx.w[W_OPCODE] == OP_NOOP) {
          lease_tab[pf_i & 15] = head;
          lease_tab[16 + (pf_i & 15)] = issued;
          ++pf_i;
          continue;
        }
        Pf<S> pf;
        pf_desc<S>(a, nx, pf);
        const uint32_t npg = (pf_blocks(pf) + 15u) >> 4;
        if (head + npg - freed > (uint32_t)kNPages) break;
        if (pf_i > i + 1 && head + npg - uni(lease_tab[(i + 1) & 15]) > (uint32_t)kLookPages) break;
        pf_issue<S>(a, pf, head, cw, issued, smem);
        if (stamp && lane() == 0) a.trace[((size_t)blockIdx.x * a.L + pf_i) * kTraceWords + 9] = (uint32_t)rtc();
        lease_tab[pf_i & 15] = head;
        lease_tab[16 + (pf_i & 15)] = issued;
        head += npg;
        ++pf_i;
      }
    }
  }
  wait_vm0();  // no LDS-bound load may be in flight when the block retires
}

}  // namespace dev

// one kernel per op family: the single-token plans' bodies (S = 0) and the multi-row plans' (S = 1)
// are compiled separately, so neither family's register allocation carries the other's code; the
// multi-row family comes with loader waves (LD) or with the eight waves prefetching for themselves
template <int S, bool LD, bool RG>
__global__ void __launch_bounds__(LD ? dev::kThreadsM : dev::kThreads, 1) mk_worker(KArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t* base;
  int count, stride;
  if (a.flags & kModeGraph) {  // one op: block b runs the op's tasks b, b + grid, ...
    base = a.instrs + (size_t)(a.first_task + blockIdx.x) * kWords;
    count = (a.L - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    stride = (int)gridDim.x * kWords;
  } else {
    base = a.instrs + (size_t)blockIdx.x * a.L * kWords;
    count = a.L;
    stride = kWords;
  }
  if (threadIdx.x < 16) ((uint32_t*)(smem + dev::kCtrlOff))[threadIdx.x] = 0u;  // abort flag .. loader counts
  if (threadIdx.x < 8) ((uint32_t*)(smem + dev::kCtrlOff + dev::kITagOff))[threadIdx.x] = 0u;  // instruction ring tags
  __syncthreads();
  if (LD && wave >= dev::kNW) dev::loader<S>(a, base, count, stride, wave - dev::kNW, smem);
  else if (wave == 0) dev::controller<S, LD, RG>(a, base, count, stride, smem);
  else dev::compute<S, LD, RG>(a, base, count, stride, wave - 1, smem);
}

hipError_t launch_worker(const KArgs& a, int grid, hipStream_t stream, int spec, bool loaders) {
  const bool groups = spec == 1 && a.sh.rg > 1;  // more than 16 rows: the row-group GEMM tiles
  if (groups && loaders)
    hipLaunchKernelGGL((mk_worker<1, true, true>), dim3(grid), dim3(dev::kThreadsM), dev::kLdsBytes, stream, a);
  else if (groups)
    hipLaunchKernelGGL((mk_worker<1, false, true>), dim3(grid), dim3(dev::kThreads), dev::kLdsBytes, stream, a);
  else if (spec == 1 && loaders)
    hipLaunchKernelGGL((mk_worker<1, true, false>), dim3(grid), dim3(dev::kThreadsM), dev::kLdsBytes, stream, a);
  else if (spec == 1)
    hipLaunchKernelGGL((mk_worker<1, false, false>), dim3(grid), dim3(dev::kThreads), dev::kLdsBytes, stream, a);
  else
    hipLaunchKernelGGL((mk_worker<0, false, false>), dim3(grid), dim3(dev::kThreads), dev::kLdsBytes, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// the no-allocation scratch: a file-scope device array, one copy per GPU, kept until the process ends.
// Host code never passes `scratch` itself (its host-side name is only a stand-in for the symbol): it
// looks the device address up once per device and hands that address to the kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;  // the caller makes the device current
  void* ptr = nullptr;
  e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch[device] = ptr;
  return hipSuccess;
}

void* scratch_base(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return g_scratch[device];
}

// the operand pointer table from the plan's relocation list and the run's tensor addresses
__global__ void __launch_bounds__(256) mk_fill_table(const TableReloc* reloc, int n, TensorPtrs t, uint64_t* out) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
    const TableReloc r = reloc[i];
    out[i] = r.idx == kRelocAbs ? r.off : t.ptr[r.idx] + r.off;
  }
}

hipError_t launch_fill_table(const TableReloc* reloc, int n, const TensorPtrs& t, uint64_t* out, hipStream_t stream) {
  const int grid = (n + 255) / 256 < 64 ? (n + 255) / 256 : 64;
  hipLaunchKernelGGL(mk_fill_table, dim3(grid > 0 ? grid : 1), dim3(256), 0, stream, reloc, n, t, out);
  return hipGetLastError();
}

hipError_t worker_occupancy(int* blocks_per_cu, int spec) {
  // the multi-row family's larger block (with loader waves) bounds both of its instances
  const void* f = spec == 1 ? (const void*)mk_worker<1, true, false> : (const void*)mk_worker<0, false, false>;
  hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, dev::kLdsBytes);
  if (e != hipSuccess) return e;
  if (spec == 1) {
    for (const void* g : {(const void*)mk_worker<1, false, false>, (const void*)mk_worker<1, true, true>,
                          (const void*)mk_worker<1, false, true>}) {
      e = hipFuncSetAttribute(g, hipFuncAttributeMaxDynamicSharedMemorySize, dev::kLdsBytes);
      if (e != hipSuccess) return e;
    }
  }
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f, spec == 1 ? dev::kThreadsM : dev::kThreads,
                                                      dev::kLdsBytes);
}

}  // namespace mk
