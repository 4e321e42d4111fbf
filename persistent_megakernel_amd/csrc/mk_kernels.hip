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
// Cross-CU visibility.  MI355X has one L2 per XCD and plain cached lines are not coherent
// across XCDs.  Every access to data produced inside a run (activations, partials, counters)
// is made at device scope (sc1), producers wait for their stores to complete before the
// relaxed device-scope counter add, and consumers issue their device-scope loads after the
// satisfying poll -- the release/acquire pairing of the counter protocol without whole-L2
// write-back / invalidate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_device.hpp"

namespace mk {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

#define DEV __device__ __forceinline__

// ---------------------------------------------------------------------------------------
// small helpers
DEV uint32_t lane() { return __lane_id(); }
DEV unsigned long long rtc() { return __builtin_amdgcn_s_memrealtime(); }

DEV float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
DEV uint32_t f2bf(float f) {  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// bf16 pair view of a 32-bit word.  (A bit_cast of an ext-vector element is taken from
// element 0 by this compiler, so the word is copied out first.)
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

// Wave reductions: DPP within rows of 16 lanes (quad xor 1, quad xor 2, half-row mirror,
// row mirror leave every lane of a row holding the row total), ds_swizzle xor 16 for pairs of
// rows, then the two 32-lane halves through readlane.
template <int CTRL>
DEV float dppf(float v) { return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false)); }
template <int CTRL>
DEV int dppi(int v) { return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false); }
DEV float row16_sum(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  v += dppf<0x140>(v);
  return v;
}
DEV float wave_sum(float v) {
  v = row16_sum(v);
  v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
}
DEV float wave_max(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
  return fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
               __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)));
}
DEV uint32_t wave_sum_u32(uint32_t v) {
  int x = (int)v;
  x += dppi<0xB1>(x);
  x += dppi<0x4E>(x);
  x += dppi<0x141>(x);
  x += dppi<0x140>(x);
  x += __builtin_amdgcn_ds_swizzle(x, 0x401F);
  return (uint32_t)(__builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 32));
}

// Scalar loads of data that no one writes during a run (queue, pointer table, block table):
// they go through the scalar cache and the lgkm counter, leaving the vector-memory counter
// to the prefetch accounting.
DEV uint32_t s_ld32(const void* p) {
  uint32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p));
  return v;
}
DEV uint64_t s_ld64(const void* p) {
  uint64_t v;
  asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p));
  return v;
}
DEV u32x8 s_ld256(const void* p) {
  u32x8 v;
  asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p));
  return v;
}

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

DEV void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

DEV uint32_t ring_off(uint32_t lease, uint32_t off) {
  return (((lease + (off >> 14)) & (kNPages - 1)) << 14) | (off & 16383u);
}

// ---------------------------------------------------------------------------------------
// prefetch descriptors: what an instruction streams into its LDS lease, in 1 KiB blocks
struct Pf {
  const char* s0;  // span 0 base (or K cache base)
  const char* s1;  // span 1 base (or V cache base)
  uint32_t len0, len1, nb0, nblk;
  const int32_t* bt;  // attention: block-table row of the request
  int t0, nk, hk;
  bool attn;
};
DEV uint32_t blocks_of(uint32_t bytes) { return (bytes + 1023u) >> 10; }

DEV void pf_desc(const KArgs& a, const Instr& in, Pf& pf) {
  const uint32_t op = in.w[W_OPCODE];
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const Shapes& sh = a.sh;
  pf.attn = false;
  pf.s1 = nullptr;
  pf.len1 = 0;
  if (op == OP_ATTN) {
    const int r = in.w[W_P1], hk = in.w[W_P2], s = in.w[W_P3];
    const int t0 = in.w[W_P4], t1 = in.w[W_P5];
    const bool last = s == (int)in.w[W_ARR_N] - 1;
    pf.attn = true;
    pf.s0 = (const char*)s_ld64(row + ATT_KC);
    pf.s1 = (const char*)s_ld64(row + ATT_VC);
    pf.bt = (const int32_t*)s_ld64(row + ATT_BT) + (size_t)r * sh.maxp;
    pf.t0 = t0;
    pf.hk = hk;
    pf.nk = (last ? t1 - 1 : t1) - t0;
    pf.len0 = (uint32_t)pf.nk * 256u;
    pf.nb0 = blocks_of(pf.len0);
    pf.nblk = 2 * pf.nb0;
    return;
  }
  const char* w = (const char*)s_ld64(row + 0);
  const uint32_t n0 = in.w[W_P1], nr = in.w[W_P2], K = in.w[W_P4];
  const uint32_t rowb = K * 2u;
  pf.s0 = w + (size_t)n0 * rowb;
  pf.len0 = nr * rowb;
  pf.nb0 = blocks_of(pf.len0);
  pf.nblk = pf.nb0;
  if (op == OP_GATEUP) {
    pf.s1 = w + (size_t)(sh.I + n0) * rowb;
    pf.len1 = pf.len0;
    pf.nblk = pf.nb0 + blocks_of(pf.len1);
  }
}

// issue this wave's share (blocks b = cw mod 7) of an instruction's prefetch into its lease
DEV void pf_issue(const KArgs& a, const Pf& pf, uint32_t lease, int cw, uint32_t& issued, char* smem) {
  const uint32_t ln = lane();
  for (uint32_t b = cw; b < pf.nblk; b += kNCW) {
    const char* src;
    if (pf.attn) {
      const bool isv = b >= pf.nb0;
      const uint32_t bb = isv ? b - pf.nb0 : b;
      uint32_t u = bb * 4u + (ln >> 4);
      if (u >= (uint32_t)pf.nk) u = 4u * bb;  // beyond the tile: reload the block's first row
      const int t = pf.t0 + (int)(4u * bb);
      const int page = (int)s_ld32(pf.bt + t / a.sh.P);
      const int tt = pf.t0 + (int)u;
      const size_t rowi = ((size_t)page * a.sh.P + (tt % a.sh.P)) * a.sh.Hkv + pf.hk;
      src = (isv ? pf.s1 : pf.s0) + rowi * 256u + (ln & 15u) * 16u;
    } else {
      const bool sp1 = b >= pf.nb0;
      const uint32_t bb = sp1 ? b - pf.nb0 : b;
      uint32_t off = bb * 1024u + ln * 16u;
      const uint32_t len = sp1 ? pf.len1 : pf.len0;
      if (off >= len) off = bb * 1024u;
      src = (sp1 ? pf.s1 : pf.s0) + off;
    }
    lds_void* dst = (lds_void*)(smem + kRingOff + ring_off(lease, b * 1024u));
    __builtin_amdgcn_global_load_lds((const void*)src, dst, 16, 0, 0);
    ++issued;
  }
}

// ---------------------------------------------------------------------------------------
// controller prologues (activation staging into LDS)

// act[e] = bf16(RMSNorm(r + x)[e] * gamma[e]) for the M = 1 row; x may be null.
DEV void norm_prologue(const uint16_t* x, const float* r, const uint16_t* gamma, int H, float eps, char* act) {
  constexpr int MAXC = 16;  // hidden <= 8192
  const uint32_t ln = lane();
  const int nch = (H + 511) / 512;
  __amdgpu_buffer_rsrc_t rx = rsrc(x), rr = rsrc(r), rg = rsrc(gamma);
  float v[MAXC][8];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int e = 512 * k + 8 * (int)ln;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[k][j] = 0.f;
    if (k < nch && e < H) {
      u32x4 ra = ld128(rr, e * 4), rb = ld128(rr, e * 4 + 16);
      float rv[8] = {__uint_as_float(ra.x), __uint_as_float(ra.y), __uint_as_float(ra.z), __uint_as_float(ra.w),
                     __uint_as_float(rb.x), __uint_as_float(rb.y), __uint_as_float(rb.z), __uint_as_float(rb.w)};
      if (x) {
        u32x4 xv = ld128(rx, e * 2);
        uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rv[2 * j] += bf2f(xs[j] & 0xffffu);
          rv[2 * j + 1] += bf2f(xs[j] >> 16);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[k][j] = rv[j];
        ss += rv[j] * rv[j];
      }
    }
  }
  ss = wave_sum(ss);
  const float inv = rsqrtf(ss / (float)H + eps);
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int e = 512 * k + 8 * (int)ln;
    if (k < nch && e < H) {
      u32x4 gv = __builtin_amdgcn_raw_buffer_load_b128(rg, e * 2, 0, 0);
      uint32_t gs[4] = {gv.x, gv.y, gv.z, gv.w};
      u32x4 o;
      uint32_t os[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float h0 = v[k][2 * j] * inv * bf2f(gs[j] & 0xffffu);
        const float h1 = v[k][2 * j + 1] * inv * bf2f(gs[j] >> 16);
        os[j] = f2bf(h0) | (f2bf(h1) << 16);
      }
      o.x = os[0]; o.y = os[1]; o.z = os[2]; o.w = os[3];
      *(u32x4*)(act + e * 2) = o;
    }
  }
}

// act[0 .. n) = bf16 vector copied from device memory (n <= 8192); all loads issue first
DEV void copy_prologue(const uint16_t* src, int n, char* act) {
  constexpr int MAXC = 16;
  __amdgpu_buffer_rsrc_t rs = rsrc(src);
  u32x4 v[MAXC];
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int e = 512 * k + 8 * (int)lane();
    if (e < n) v[k] = ld128(rs, e * 2);
  }
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int e = 512 * k + 8 * (int)lane();
    if (e < n) *(u32x4*)(act + e * 2) = v[k];
  }
}

// attention: QK-norm + RoPE of the group's q heads and k head, bf16 q / k / v into LDS; the
// last split also writes the new k / v row into the paged caches.
DEV void attn_prologue(const KArgs& a, const Instr& in, char* act) {
  const Shapes& sh = a.sh;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const int r = in.w[W_P1], hk = in.w[W_P2], s = in.w[W_P3], t1 = in.w[W_P5];
  const bool last = s == (int)in.w[W_ARR_N] - 1;
  const float* qkv = (const float*)s_ld64(row + ATT_QKV) + (size_t)r * sh.n_qkv;
  const uint16_t* gq = (const uint16_t*)s_ld64(row + ATT_GQ);
  const uint16_t* gk = (const uint16_t*)s_ld64(row + ATT_GK);
  const float* rope = (const float*)s_ld64(row + ATT_ROPE) + (size_t)r * 128;
  __amdgpu_buffer_rsrc_t rq = rsrc(qkv), rgq = rsrc(gq), rgk = rsrc(gk), rro = rsrc(rope);
  const uint32_t i = lane();  // dims i and i + 64
  const float c = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rro, i * 8, 0, 0));
  const float sn = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rro, i * 8 + 4, 0, 0));
  uint16_t* qs = (uint16_t*)(act + kActQ);
  // vectors j < g: the group's q heads; j == g: its k head; j == g + 1: its v head
  float x0v[10], x1v[10];
#pragma unroll
  for (int j = 0; j < 10; ++j) {
    if (j <= sh.g + 1) {
      const int col = j < sh.g ? (hk * sh.g + j) * 128 : (j == sh.g ? (sh.Hq + hk) * 128 : (sh.Hq + sh.Hkv + hk) * 128);
      x0v[j] = __uint_as_float(ld32(rq, (col + i) * 4));
      x1v[j] = __uint_as_float(ld32(rq, (col + i + 64) * 4));
    }
  }
#pragma unroll
  for (int j = 0; j < 9; ++j) {
    if (j > sh.g) break;
    const bool isk = j == sh.g;
    const float x0 = x0v[j], x1 = x1v[j];
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float inv = rsqrtf(ss / 128.f + sh.eps);
    __amdgpu_buffer_rsrc_t rg = isk ? rgk : rgq;
    const uint32_t g01 = __builtin_amdgcn_raw_buffer_load_b16(rg, i * 2, 0, 0);
    const uint32_t g23 = __builtin_amdgcn_raw_buffer_load_b16(rg, (i + 64) * 2, 0, 0);
    const float n0 = x0 * inv * bf2f(g01), n1 = x1 * inv * bf2f(g23);
    const float o0 = n0 * c - n1 * sn, o1 = n1 * c + n0 * sn;
    uint16_t* dst = isk ? (uint16_t*)(act + kActK) : qs + j * 128;
    dst[i] = (uint16_t)f2bf(o0);
    dst[i + 64] = (uint16_t)f2bf(o1);
  }
  {
    uint16_t* dv = (uint16_t*)(act + kActV);
    float v0 = 0.f, v1 = 0.f;
#pragma unroll
    for (int j = 0; j < 10; ++j)
      if (j == sh.g + 1) {
        v0 = x0v[j];
        v1 = x1v[j];
      }
    dv[i] = (uint16_t)f2bf(v0);
    dv[i + 64] = (uint16_t)f2bf(v1);
  }
  if (last) {
    const int p = t1 - 1;
    const int32_t* bt = (const int32_t*)s_ld64(row + ATT_BT) + (size_t)r * sh.maxp;
    const int page = (int)s_ld32(bt + p / sh.P);
    const size_t rowi = ((size_t)page * sh.P + (p % sh.P)) * sh.Hkv + hk;
    uint16_t* kc = (uint16_t*)s_ld64(row + ATT_KC) + rowi * 128;
    uint16_t* vc = (uint16_t*)s_ld64(row + ATT_VC) + rowi * 128;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the LDS writes above are done
    const uint16_t* kl = (const uint16_t*)(act + kActK);
    const uint16_t* vl = (const uint16_t*)(act + kActV);
    __amdgpu_buffer_rsrc_t rk = rsrc(kc), rv = rsrc(vc);
    st16(rk, i * 2, kl[i]);
    st16(rk, (i + 64) * 2, kl[i + 64]);
    st16(rv, i * 2, vl[i]);
    st16(rv, (i + 64) * 2, vl[i + 64]);
  }
}

// ---------------------------------------------------------------------------------------
// compute bodies (waves 1..7; cw = 0..6)

// out[j] = sum_k act[k] * W[row j][k]; rows [0, nr0) at j * rowb, rows [nr0, nrows) at off1.
DEV void gemv(const char* smem, uint32_t lease, int nrows, int nr0, uint32_t off1, int K, int cw, float* out) {
  const int ln = (int)lane();
  const uint32_t rowb = (uint32_t)K * 2u;
  const int nk8 = K / 8;
  const char* act = smem + kActOff;
  const char* ring = smem + kRingOff;
  for (int r0 = cw; r0 < nrows; r0 += kNCW * 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    uint32_t rb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r0 + kNCW * j;
      rb[j] = r < nr0 ? (uint32_t)r * rowb : off1 + (uint32_t)(r - nr0) * rowb;
    }
    for (int c = ln; c < nk8; c += 64) {
      const u32x4 x = *(const u32x4*)(act + c * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (r0 + kNCW * j < nrows) {
          const u32x4 wv = *(const u32x4*)(ring + ring_off(lease, rb[j] + (uint32_t)c * 16u));
          acc[j] = dot8(wv, x, acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = r0 + kNCW * j;
      if (r < nrows) {
        const float s = wave_sum(acc[j]);
        if (ln == 0) out[r] = s;
      }
    }
  }
}

// split-KV attention partial for one (request, kv head, split): g query heads.
// inner barriers: 3 (scores | softmax | PV partials | reduce)
DEV void attn_compute(const KArgs& a, const Instr& in, const char* smem, char* act, uint32_t lease, int cw) {
  const Shapes& sh = a.sh;
  const int g = sh.g;
  const int s = in.w[W_P3], t0 = in.w[W_P4], t1 = in.w[W_P5];
  const bool last = s == (int)in.w[W_ARR_N] - 1;
  const int ntok = t1 - t0;
  const int nk = last ? ntok - 1 : ntok;
  const uint32_t voff = blocks_of((uint32_t)nk * 256u) * 1024u;
  const char* ring = smem + kRingOff;
  const int ln = (int)lane();
  const int gl = cw * 64 + ln;  // 0..447
  float* sc = (float*)(act + kActS);      // [g][kSStride]
  float* st = (float*)(act + kActStat);   // [g][2]: max, sum
  float* red = (float*)(act + kActRed);   // [TG][g][128]
  const float scale = sh.inv_sqrt_d;
  // 1) scores: one (head, token) pair per 16-lane row
  {
    const int grp = gl >> 4, sub = ln & 15;
    for (int pidx = grp; pidx < g * ntok; pidx += kNCW * 4) {
      const int j = pidx / ntok, u = pidx % ntok;
      const u32x4 qv = *(const u32x4*)(act + kActQ + j * 256 + sub * 16);
      u32x4 kv;
      if (u < nk) kv = *(const u32x4*)(ring + ring_off(lease, (uint32_t)u * 256u + sub * 16u));
      else kv = *(const u32x4*)(act + kActK + sub * 16);
      float d = row16_sum(dot8(kv, qv, 0.f));
      if (sub == 0) sc[j * kSStride + u] = d * scale;
    }
  }
  lds_barrier();
  // 2) softmax statistics per head, p = exp(s - max) in place
  for (int j = cw; j < g; j += kNCW) {
    float m = -INFINITY;
    for (int u = ln; u < ntok; u += 64) m = fmaxf(m, sc[j * kSStride + u]);
    m = wave_max(m);
    float l = 0.f;
    for (int u = ln; u < ntok; u += 64) {
      const float e = __expf(sc[j * kSStride + u] - m);
      sc[j * kSStride + u] = e;
      l += e;
    }
    l = wave_sum(l);
    if (ln == 0) {
      st[2 * j] = m;
      st[2 * j + 1] = l;
    }
  }
  lds_barrier();
  // 3) PV partials: unit = (head, 8 dims); TG token groups
  {
    const int units = g * 16;
    const int TG = (kNCW * 64) / units;
    const int unit = gl % units, tg = gl / units;
    if (tg < TG) {
      const int j = unit >> 4, c8 = unit & 15;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int u = tg; u < ntok; u += TG) {
        const float p = sc[j * kSStride + u];
        u32x4 vv;
        if (u < nk) vv = *(const u32x4*)(ring + ring_off(lease, voff + (uint32_t)u * 256u + c8 * 16u));
        else vv = *(const u32x4*)(act + kActV + c8 * 16);
        const uint32_t vs[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += p * bf2f(vs[q] & 0xffffu);
          acc[2 * q + 1] += p * bf2f(vs[q] >> 16);
        }
      }
      float* dst = red + ((size_t)tg * g + j) * 128 + c8 * 8;
#pragma unroll
      for (int q = 0; q < 8; ++q) dst[q] = acc[q];
    }
  }
  lds_barrier();
  // 4) reduce token groups -> normalised O and lse into the output area
  {
    const int units = g * 16;
    const int TG = (kNCW * 64) / units;
    float* out = (float*)(smem + kOutOff);
    for (int o = gl; o < g * 128; o += kNCW * 64) {
      const int j = o >> 7;
      float acc = 0.f;
      for (int tg = 0; tg < TG; ++tg) acc += red[((size_t)tg * g + j) * 128 + (o & 127)];
      out[o] = acc / st[2 * j + 1];
    }
    if (gl < g) out[g * 128 + gl] = st[2 * gl] + __logf(st[2 * gl + 1]);
  }
}

// ---------------------------------------------------------------------------------------
// controller epilogues

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

DEV void attn_epilogue(const KArgs& a, const Instr& in, const char* smem) {
  const Shapes& sh = a.sh;
  const int g = sh.g;
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const int r = in.w[W_P1], hk = in.w[W_P2], s = in.w[W_P3];
  const int ns = in.w[W_ARR_N];
  const uint32_t pstride = (uint32_t)g * 129u;  // floats per split: g*128 O + g lse
  const uint32_t gbase = ((uint32_t)(r * sh.Hkv + hk) * (uint32_t)sh.max_splits) * pstride;
  float* part = (float*)s_ld64(row + ATT_PART);
  __amdgpu_buffer_rsrc_t rp = rsrc(part);
  const float* out = (const float*)(smem + kOutOff);
  for (int e = (int)lane(); e < (int)pstride; e += 64)
    st32(rp, (gbase + (uint32_t)s * pstride + e) * 4u, __float_as_uint(out[e]));
  wait_vm0();
  if (!arrive(a, in)) return;
  // combine the group's splits: o = sum_i exp(lse_i - lse) O_i, lse = log sum_i exp(lse_i)
  uint16_t* o = (uint16_t*)s_ld64(row + ATT_O) + (size_t)r * sh.Hq * 128;
  __amdgpu_buffer_rsrc_t ro = rsrc(o);
  const int ln = (int)lane();
  float* wts = (float*)(smem + kOutOff);  // [ns][g] combine weights (this split's output is stored)
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= g) break;
    float mx = -INFINITY;
    for (int t0 = 0; t0 < ns; t0 += 64) {
      const int t = t0 + ln;
      const float l = t < ns ? __uint_as_float(ld32(rp, (gbase + t * pstride + g * 128 + j) * 4u)) : -INFINITY;
      if (t < ns) wts[t * g + j] = l;
      mx = fmaxf(mx, l);
    }
    mx = wave_max(mx);
    float den = 0.f;
    for (int t0 = 0; t0 < ns; t0 += 64) {
      const int t = t0 + ln;
      if (t < ns) {
        const float w = __expf(wts[t * g + j] - mx);
        wts[t * g + j] = w;
        den += w;
      }
    }
    den = wave_sum(den);
    const float inv = 1.f / den;
    for (int t0 = 0; t0 < ns; t0 += 64) {
      const int t = t0 + ln;
      if (t < ns) wts[t * g + j] *= inv;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);
  for (int u = ln; u < g * 32; u += 64) {  // unit = (head j, 4 dims)
    const int j = u >> 5, c4 = u & 31;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0; t0 < ns; t0 += 16) {
      u32x4 v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (t0 + q < ns) v[q] = ld128(rp, (gbase + (t0 + q) * pstride + j * 128 + c4 * 4) * 4u);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (t0 + q < ns) {
          const float w = wts[(t0 + q) * g + j];
          acc[0] += w * __uint_as_float(v[q].x);
          acc[1] += w * __uint_as_float(v[q].y);
          acc[2] += w * __uint_as_float(v[q].z);
          acc[3] += w * __uint_as_float(v[q].w);
        }
      }
    }
    const uint32_t col = (uint32_t)(hk * g + j) * 128u + c4 * 4u;
    st32(ro, col * 2u, f2bf(acc[0]) | (f2bf(acc[1]) << 16));
    st32(ro, col * 2u + 4u, f2bf(acc[2]) | (f2bf(acc[3]) << 16));
  }
  wait_vm0();
  signal_all(a, in);
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

DEV void gemv_epilogue(const KArgs& a, const Instr& in, const char* smem, LmState& lm) {
  const uint32_t op = in.w[W_OPCODE];
  const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
  const int n0 = in.w[W_P1], nr = in.w[W_P2];
  const float* out = (const float*)(smem + kOutOff);
  const int j = (int)lane();
  if (op == OP_QKV) {
    __amdgpu_buffer_rsrc_t ro = rsrc((const void*)s_ld64(row + QKV_OUT));
    for (int jj = j; jj < nr; jj += 64) st32(ro, (uint32_t)(n0 + jj) * 4u, __float_as_uint(out[jj]));
  } else if (op == OP_OPROJ) {
    __amdgpu_buffer_rsrc_t rx = rsrc((const void*)s_ld64(row + O_X));
    __amdgpu_buffer_rsrc_t rr = rsrc((const void*)s_ld64(row + O_RIN));
    __amdgpu_buffer_rsrc_t r2 = rsrc((const void*)s_ld64(row + O_R2));
    for (int jj = j; jj < nr; jj += 64) {
      const uint32_t n = (uint32_t)(n0 + jj);
      const float av = bf2f(f2bf(out[jj]));
      const float xv = bf2f(__builtin_amdgcn_raw_buffer_load_b16(rx, n * 2u, 0, SC1));
      const float rin = __uint_as_float(ld32(rr, n * 4u));
      const float r1 = rin + xv;
      st32(r2, n * 4u, __float_as_uint(r1 + av));
    }
  } else if (op == OP_GATEUP) {
    __amdgpu_buffer_rsrc_t rm = rsrc((const void*)s_ld64(row + GU_M));
    for (int jj = j; jj < nr; jj += 64) {
      const float gv = out[jj], uv = out[nr + jj];
      st16(rm, (uint32_t)(n0 + jj) * 2u, f2bf(gv / (1.f + __expf(-gv)) * uv));
    }
  } else if (op == OP_DOWN) {
    __amdgpu_buffer_rsrc_t ry = rsrc((const void*)s_ld64(row + DN_Y));
    for (int jj = j; jj < nr; jj += 64) st16(ry, (uint32_t)(n0 + jj) * 2u, f2bf(out[jj]));
  } else if (op == OP_LMHEAD) {
    __amdgpu_buffer_rsrc_t rl = rsrc((const void*)s_ld64(row + LM_LOGITS));
    __amdgpu_buffer_rsrc_t rp = rsrc((const void*)s_ld64(row + LM_PART));
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int jj = j; jj < nr; jj += 64) {
      const float v = out[jj];
      st32(rl, (uint32_t)(n0 + jj) * 4u, __float_as_uint(v));
      if (v > best) {
        best = v;
        bi = n0 + jj;
      }
    }
    argmax_merge(best, bi);
    if (best > lm.best || (best == lm.best && bi < lm.idx)) {
      lm.best = best;
      lm.idx = bi;
    }
    const uint32_t slot = in.w[W_ARR_RANK];
    if (slot == kNone) return;  // not this worker's last lm_head tile
    if (j == 0) {
      st32(rp, slot * 8u, __float_as_uint(lm.best));
      st32(rp, slot * 8u + 4u, (uint32_t)lm.idx);
    }
    wait_vm0();
    if (!arrive(a, in)) return;
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
  wait_vm0();
  signal_all(a, in);
}

// ---------------------------------------------------------------------------------------
// the two roles

DEV int inner_barriers(uint32_t op) { return op == OP_ATTN ? 3 : 0; }

// returns false when the watchdog expired or another worker aborted
DEV bool wait_events(const KArgs& a, const Instr& in, uint32_t& poll_ticks) {
  const uint32_t ln = lane();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if ((uint32_t)k >= in.w[W_NWAIT]) break;
    const uint32_t e = in.w[W_WAIT0 + 2 * k], thr = in.w[W_WAIT0 + 2 * k + 1];
    const uint32_t target = (a.epoch + 1u) * thr;
    const uint32_t* base = a.events + (size_t)e * kEvStride;
    const unsigned long long t_start = rtc();
    uint32_t it = 0;
    while (true) {
      uint32_t v = 0;
      if (ln < (uint32_t)kNSub) v = __hip_atomic_load(base + ln * kSubStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t sum = wave_sum_u32(v);
      if ((int32_t)(sum - target) >= 0) break;
      const unsigned long long now = rtc();
      if ((++it & 31u) == 0) {
        const uint32_t abort_flag = __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (abort_flag) return false;
      }
      if (now - t_start > kWatchdogTicks) {
        if (ln == 0) {
          uint32_t z = 0;
          if (__hip_atomic_compare_exchange_strong(a.err, &z, 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            __hip_atomic_store(a.err + 1, blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.err + 2, in.w[W_TASK], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.err + 3, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.err + 4, sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.err + 5, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        return false;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    poll_ticks += (uint32_t)(rtc() - t_start);
  }
  asm volatile("" ::: "memory");
  return true;
}

DEV void controller(const KArgs& a, const uint32_t* base, int count, int stride, char* smem) {
  volatile uint32_t* ctrl = (volatile uint32_t*)(smem + kCtrlOff);
  const bool noop_only = a.flags & MK_FLAG_NOOP_ONLY;
  const bool graph = a.flags & kModeGraph;
  uint32_t last_row = 0xFFFFFFFFu;
  LmState lm{-INFINITY, 0x7fffffff};
  for (int i = 0; i < count; ++i) {
    Instr in;
    fetch(base + (size_t)i * stride, in);
    const uint32_t op = in.w[W_OPCODE];
    if (op == OP_NOOP) continue;
    const unsigned long long t_vis = rtc();
    uint32_t poll = 0;
    bool ok = graph ? true : wait_events(a, in, poll);
    const unsigned long long t_ready = rtc();
    if (ok && !noop_only) {
      const uint64_t* row = a.table + (size_t)in.w[W_ROW] * kTableSlots;
      char* act = smem + kActOff;
      switch (op) {
        case OP_QKV:
          norm_prologue((const uint16_t*)s_ld64(row + QKV_X), (const float*)s_ld64(row + QKV_RIN),
                        (const uint16_t*)s_ld64(row + QKV_GAMMA), a.sh.H, a.sh.eps, act);
          break;
        case OP_ATTN: attn_prologue(a, in, act); break;
        case OP_OPROJ: copy_prologue((const uint16_t*)s_ld64(row + O_IN), a.sh.Hq * 128, act); break;
        case OP_GATEUP:
          norm_prologue(nullptr, (const float*)s_ld64(row + GU_R2), (const uint16_t*)s_ld64(row + GU_GAMMA),
                        a.sh.H, a.sh.eps, act);
          break;
        case OP_DOWN: copy_prologue((const uint16_t*)s_ld64(row + DN_M), a.sh.I, act); break;
        case OP_LMHEAD:
          if (last_row != in.w[W_ROW])
            norm_prologue((const uint16_t*)s_ld64(row + LM_Y), (const float*)s_ld64(row + LM_R2),
                          (const uint16_t*)s_ld64(row + LM_GAMMA), a.sh.H, a.sh.eps, act);
          break;
        default: break;
      }
      last_row = in.w[W_ROW];
    }
    if (!ok && lane() == 0) ctrl[0] = 1u;
    lds_barrier();  // A: activations staged, prefetch of this instruction landed
    if (!ok) break;
    for (int b = 0; b < inner_barriers(op); ++b) lds_barrier();
    lds_barrier();  // B: compute done, results in the output area
    if (noop_only) {
      if (op == OP_ATTN || op == OP_LMHEAD) {
        if (arrive(a, in) && op == OP_ATTN) signal_all(a, in);
      } else {
        signal_all(a, in);
      }
    } else if (op == OP_ATTN) {
      attn_epilogue(a, in, smem);
    } else {
      gemv_epilogue(a, in, smem, lm);
    }
    if ((a.flags & MK_FLAG_TRACE) && a.trace && lane() == 0) {
      uint32_t* tr = a.trace + ((size_t)blockIdx.x * a.L + i) * 4;
      tr[0] = (uint32_t)t_vis;
      tr[1] = (uint32_t)t_ready;
      tr[2] = (uint32_t)rtc();
      tr[3] = poll;
    }
  }
}

DEV void compute(const KArgs& a, const uint32_t* base, int count, int stride, int cw, char* smem) {
  volatile uint32_t* ctrl = (volatile uint32_t*)(smem + kCtrlOff);
  uint32_t* lease_tab = (uint32_t*)(smem + kCtrlOff + 64) + cw * 32;  // [16] lease, [16] issued_end
  const bool noop_only = a.flags & MK_FLAG_NOOP_ONLY;
  const int lookahead = (a.flags & MK_FLAG_NO_PREFETCH) ? 0 : 15;
  uint32_t head = 0, issued = 0;
  int pf_i = 0;
  for (int i = 0; i < count; ++i) {
    Instr in;
    fetch(base + (size_t)i * stride, in);
    const uint32_t op = in.w[W_OPCODE];
    if (op == OP_NOOP) {
      if (pf_i <= i) pf_i = i + 1;
      continue;
    }
    if (!noop_only) {
      // pages of every instruction before i are free now
      const uint32_t freed = (pf_i > i) ? lease_tab[i & 15] : head;
      if (pf_i < i) pf_i = i;
      while (pf_i < count && pf_i <= i + lookahead) {
        Instr nx;
        fetch(base + (size_t)pf_i * stride, nx);
        if (nx.w[W_OPCODE] == OP_NOOP) {
          lease_tab[pf_i & 15] = head;
          lease_tab[16 + (pf_i & 15)] = issued;
          ++pf_i;
          continue;
        }
        Pf pf;
        pf_desc(a, nx, pf);
        const uint32_t npg = (pf.nblk + 15u) >> 4;
        if (head + npg - freed > (uint32_t)kNPages) break;
        pf_issue(a, pf, head, cw, issued, smem);
        lease_tab[pf_i & 15] = head;
        lease_tab[16 + (pf_i & 15)] = issued;
        head += npg;
        ++pf_i;
      }
      wait_vm_le(issued - lease_tab[16 + (i & 15)]);
    }
    lds_barrier();  // A
    if (ctrl[0]) break;
    if (!noop_only) {
      const uint32_t lease = lease_tab[i & 15];
      char* act = smem + kActOff;
      float* out = (float*)(smem + kOutOff);
      if (op == OP_ATTN) {
        attn_compute(a, in, smem, act, lease, cw);
      } else {
        const int nr = in.w[W_P2], K = in.w[W_P4];
        if (op == OP_GATEUP) gemv(smem, lease, 2 * nr, nr, blocks_of((uint32_t)nr * K * 2u) * 1024u, K, cw, out);
        else gemv(smem, lease, nr, nr, 0, K, cw, out);
      }
    } else {
      for (int b = 0; b < inner_barriers(op); ++b) lds_barrier();
    }
    lds_barrier();  // B
  }
  wait_vm0();  // no LDS-bound load may be in flight when the block retires
}

}  // namespace dev

__global__ void __launch_bounds__(dev::kThreads, 1) mk_worker(KArgs a) {
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
  if (threadIdx.x == 0) *(volatile uint32_t*)(smem + dev::kCtrlOff) = 0u;
  __syncthreads();
  if (wave == 0) dev::controller(a, base, count, stride, smem);
  else dev::compute(a, base, count, stride, wave - 1, smem);
}

hipError_t launch_worker(const KArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(mk_worker, dim3(grid), dim3(dev::kThreads), dev::kLdsBytes, stream, a);
  return hipGetLastError();
}

hipError_t worker_occupancy(int* blocks_per_cu) {
  hipError_t e = hipFuncSetAttribute((const void*)mk_worker, hipFuncAttributeMaxDynamicSharedMemorySize, dev::kLdsBytes);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, (const void*)mk_worker, dev::kThreads, dev::kLdsBytes);
}

}  // namespace mk
