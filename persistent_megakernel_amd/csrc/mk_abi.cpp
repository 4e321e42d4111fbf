// C ABI of the decode-layer megakernel: plan construction and upload, operand pointer
// tables (rebinding without replanning), the persistent launch, the hipGraph baseline, and
// error reporting.  The operand pointer table keeps tensor addresses out of the
// instructions, so a new set of tensors only needs a new table (MegaRTP page, section 4,
// OperandPtrTable).
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "mk_device.hpp"

namespace {
thread_local std::string g_err;

mk_status fail(mk_status s, const std::string& msg) {
  g_err = msg;
  return s;
}
#define HIP_TRY(x)                                                                         \
  do {                                                                                     \
    hipError_t _e = (x);                                                                   \
    if (_e != hipSuccess) return fail(MK_ERR_HIP, std::string(#x ": ") + hipGetErrorString(_e)); \
  } while (0)

struct GraphEntry {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};
}  // namespace

struct mk_plan {
  mk::HostPlan hp;
  mk::Shapes sh{};
  int device = 0;
  int cus = 0;
  uint32_t* d_queue = nullptr;
  uint32_t* d_tasks = nullptr;
  uint32_t* d_events = nullptr;
  uint32_t* d_arrivals = nullptr;
  uint32_t* d_err = nullptr;
  float* d_rope = nullptr;   // per row: (cos, sin) at the row's position, [M][head_dim / 2][2]
  int32_t* d_pos = nullptr;  // per row: position of the row's token
  uint32_t* d_trace = nullptr;
  int32_t* d_gather = nullptr;  // MK_FLAG_DEBUG_GATHER: physical slots of the gathered rows
  size_t gather_words = 0;
  mk::TableReloc* d_reloc = nullptr;  // the operand pointer table as (tensor, offset) pairs (no-allocation runs)
  int n_reloc = 0;
  uint64_t uid = 0;                   // identifies the plan to the per-device scratch
  mk::TensorPtrs noalloc_last{};      // tensor set whose table the scratch holds for this plan
  size_t events_bytes = 0, arrivals_bytes = 0;
  uint32_t epoch = 0;  // megakernel runs so far; never reset (record tags must not repeat)
  uint32_t cruns = 0;  // megakernel runs since the event counters were last zeroed
  uint32_t salt = 0;   // per-plan record tag base, a multiple of 1024
  bool occupancy_checked = false;
  bool host_only = false;  // planned without a device: queue inspection only
  std::map<std::vector<uint64_t>, uint64_t*> tables;
  std::map<std::vector<uint64_t>, GraphEntry> graphs;
  std::vector<hipStream_t> streams;
  std::vector<hipEvent_t> events;
};

namespace {

// per device: the plan whose workspace and table the no-allocation scratch holds (0: none)
std::atomic<uint64_t> g_scratch_owner[64];
std::atomic<uint64_t> g_plan_uid{0};

bool aligned16(uint64_t p) { return (p & 15u) == 0; }

int ws_index(const mk_config& c) { return c.workload == MK_INDEXER_FRONT ? (int)MK_TI_WORKSPACE : (int)MK_T_WORKSPACE; }

mk_status check_tensors(const mk_plan* p, const mk_tensors* t) {
  if (!t) return fail(MK_ERR_INVALID, "null tensors");
  const mk_config& c = p->hp.cfg;
  if (c.workload == MK_INDEXER_FRONT) {
    // the top-k output only with a top-k, the main-MLA tensors only with the main-MLA half
    const int need = c.mla_heads > 0 ? MK_TI_COUNT : c.topk > 0 ? MK_TI_TOPK_OUT + 1 : MK_TI_TOPK_OUT;
    if (t->n < need) return fail(MK_ERR_INVALID, "too few tensors for the indexer front");
    for (int i = 0; i < need; ++i) {
      if (i == MK_TI_TOPK_OUT && c.topk == 0) continue;
      if (t->ptr[i] == 0) return fail(MK_ERR_INVALID, "null tensor at index " + std::to_string(i));
      if (!aligned16(t->ptr[i])) return fail(MK_ERR_INVALID, "tensor " + std::to_string(i) + " is not 16-byte aligned");
    }
    if (t->ptr[MK_TI_WORKSPACE] & 255u) return fail(MK_ERR_INVALID, "workspace must be 256-byte aligned");
    return MK_OK;
  }
  const bool step = c.workload == MK_QWEN3_STEP, fp8 = c.weight_fp8 != 0;
  const int need = fp8 ? MK_T_COUNT_QWEN3 : step ? MK_T_TOKEN_OUT + 1 : MK_T_WORKSPACE + 1;
  if (t->n < need) return fail(MK_ERR_INVALID, "too few tensors for this workload");
  for (int i = 0; i < need; ++i) {
    const bool used = i <= MK_T_WORKSPACE || (step && i <= MK_T_TOKEN_OUT) || (fp8 && i >= MK_T_S_QKV);
    if (!used) continue;
    if (t->ptr[i] == 0) return fail(MK_ERR_INVALID, "null tensor at index " + std::to_string(i));
    if (!aligned16(t->ptr[i])) return fail(MK_ERR_INVALID, "tensor " + std::to_string(i) + " is not 16-byte aligned");
  }
  if (t->ptr[MK_T_WORKSPACE] & 255u) return fail(MK_ERR_INVALID, "workspace must be 256-byte aligned");
  return MK_OK;
}

size_t region_off(const mk::HostPlan& hp, const char* name) {
  for (auto& r : hp.regions)
    if (r.name == name) return r.offset;
  return 0;
}

// indexer front: one row of 16 slots per op instance
void fill_table_indexer(const mk_plan* p, const mk_tensors* t, std::vector<uint64_t>& tab) {
  using namespace mk;
  const mk::HostPlan& hp = p->hp;
  const uint64_t ws = t->ptr[MK_TI_WORKSPACE];
  auto rg = [&](const char* n) { return ws + region_off(hp, n); };
  const bool mla = hp.cfg.mla_heads > 0;
  const uint64_t wt[10] = {0, 0, 0, 0, t->ptr[MK_TI_W_QA], t->ptr[MK_TI_W_W], t->ptr[MK_TI_W_K], t->ptr[MK_TI_W_QI],
                           mla ? t->ptr[MK_TI_W_QB] : 0, mla ? t->ptr[MK_TI_W_UK] : 0};
  const uint64_t st[10] = {0, 0, 0, 0, t->ptr[MK_TI_S_QA], t->ptr[MK_TI_S_W], t->ptr[MK_TI_S_K], t->ptr[MK_TI_S_QI],
                           mla ? t->ptr[MK_TI_S_QB] : 0, 0};
  const char* gp[10] = {"", "", "", "", "gp_qa", "gp_w", "gp_k", "gp_qi", "gp_qb", ""};
  const char* out[10] = {"", "", "", "", "qa", "w", "k", "qi", "qn", ""};
  tab.assign(hp.ops.size() * kTableSlots, 0);
  for (size_t row = 0; row < hp.ops.size(); ++row) {
    uint64_t* s = &tab[row * kTableSlots];
    const uint32_t sub = hp.ops[row].sub;
    switch (hp.ops[row].opcode) {
      case OP_NORM:  // A0 (sub 0) or the q_a norm (sub 2)
        s[NM_X] = sub == 0 ? t->ptr[MK_TI_X] : 0;
        s[NM_R] = sub == 0 ? t->ptr[MK_TI_R_IN] : rg("qa");
        s[NM_GAIN] = sub == 0 ? t->ptr[MK_TI_G_NORM] : t->ptr[MK_TI_G_QA];
        s[NM_R1] = 0;
        s[NM_H] = rg(sub == 0 ? "hq" : "qaq");
        s[NM_S] = rg(sub == 0 ? "sh" : "sqa");
        break;
      case OP_GEMM:
        s[GM_W] = wt[sub];
        s[GM_ACT] = rg(sub == K_UK ? "qn" : sub == K_QI || sub == K_QB ? "qaq" : "hq");
        s[GM_PART] = sub == K_UK ? t->ptr[MK_TI_QLAT_OUT] : rg(gp[sub]);  // D2 writes its output directly
        s[GM_SW] = st[sub];
        break;
      case OP_FIN:
        s[FN_PART] = rg(gp[sub]);
        s[FN_SA] = rg(sub == K_QI || sub == K_QB ? "sqa" : "sh");
        s[FN_OUT] = rg(out[sub]);
        s[FN_R1] = (uint64_t)p->d_rope;  // D1's RoPE
        break;
      case OP_KCACHE:
        s[KC_K] = rg("k");
        s[KC_ROPE] = (uint64_t)p->d_rope;
        s[KC_CACHE] = t->ptr[MK_TI_KEY_CACHE];
        s[KC_SCALE] = t->ptr[MK_TI_KEY_SCALE];
        s[KC_BT] = t->ptr[MK_TI_BLOCK_TABLE];
        s[KC_POS] = (uint64_t)p->d_pos;
        break;
      case OP_SCORE:
        s[SC_Q] = rg("qi");
        s[SC_W] = rg("w");
        s[SC_CACHE] = t->ptr[MK_TI_KEY_CACHE];
        s[SC_SCALE] = t->ptr[MK_TI_KEY_SCALE];
        s[SC_BT] = t->ptr[MK_TI_BLOCK_TABLE];
        s[SC_OUT] = t->ptr[MK_TI_SCORE_OUT];
        s[SC_POS] = (uint64_t)p->d_pos;
        break;
      case OP_TOPK:
        s[TK_SCORE] = t->ptr[MK_TI_SCORE_OUT];
        s[TK_POS] = (uint64_t)p->d_pos;
        s[TK_OUT] = t->ptr[MK_TI_TOPK_OUT];
        break;
      default: break;
    }
  }
}

// one row of 16 slots per op instance, layer-offset addresses
void fill_table(const mk_plan* p, const mk_tensors* t, std::vector<uint64_t>& tab) {
  using namespace mk;
  const mk::HostPlan& hp = p->hp;
  if (hp.cfg.workload == MK_INDEXER_FRONT) {
    fill_table_indexer(p, t, tab);
    return;
  }
  const mk_config& c = hp.cfg;
  const uint64_t H = c.hidden, I = c.inter, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const uint64_t nqkv = (Hq + 2 * Hkv) * d;
  const uint64_t welem = c.weight_fp8 ? 1 : 2;
  const uint64_t cache_layer = (uint64_t)c.num_phys_pages * c.page_size * Hkv * d * 2;
  const uint64_t ws = t->ptr[MK_T_WORKSPACE];
  const int L = c.num_layers;
  const uint64_t qkv = ws + region_off(hp, "qkv"), ob = ws + region_off(hp, "o"), mb = ws + region_off(hp, "m");
  const uint64_t r2b = ws + region_off(hp, "r2"), r1b = ws + region_off(hp, "r1");
  auto rg = [&](const char* n) { return ws + region_off(hp, n); };
  const bool fp8 = c.act_fp8 != 0;
  // multi-row projections by kind: weights, their block scales, N, K, operand-order input,
  // partial sums, per-token input scales
  const uint64_t wt[4] = {t->ptr[MK_T_W_QKV], t->ptr[MK_T_W_O], t->ptr[MK_T_W_GU], t->ptr[MK_T_W_DOWN]};
  const uint64_t st[4] = {t->ptr[MK_T_S_QKV], t->ptr[MK_T_S_O], t->ptr[MK_T_S_GU], t->ptr[MK_T_S_DOWN]};
  const uint64_t pn[4] = {nqkv, H, 2 * I, H}, pk[4] = {H, Hq * d, H, I};
  const char* pin[4] = {"h1", fp8 ? "oq" : "o", "h2", fp8 ? "mq" : "m"};
  const char* pgp[4] = {"gp_qkv", "gp_o", "gp_gu", "gp_down"};
  const char* psa[4] = {"s1", "so", "s2", "sm"};
  tab.assign(hp.ops.size() * kTableSlots, 0);
  for (size_t row = 0; row < hp.ops.size(); ++row) {
    uint64_t* s = &tab[row * kTableSlots];
    const int l = hp.ops[row].layer;
    const uint32_t sub = hp.ops[row].sub;
    const bool spec1 = hp.tp.spec == 1;
    switch (hp.ops[row].opcode) {
      case OP_NORM:
        s[NM_X] = sub == 0 ? (l == 0 ? t->ptr[MK_T_X] : rg("y")) : 0;
        s[NM_R] = sub == 0 && l == 0 ? t->ptr[MK_T_R_IN] : rg("r2");
        s[NM_GAIN] = (sub == 0 ? t->ptr[MK_T_G_ATTN] : t->ptr[MK_T_G_MLP]) + l * H * 2;
        s[NM_R1] = sub == 0 ? r1b : 0;
        s[NM_H] = rg(sub == 0 ? "h1" : "h2");
        s[NM_S] = fp8 ? rg(sub == 0 ? "s1" : "s2") : 0;
        break;
      case OP_GEMM: {
        const uint64_t nb = (pn[sub] + 127) / 128, kb = (pk[sub] + 127) / 128;
        s[GM_W] = wt[sub] + l * pn[sub] * pk[sub] * welem;
        s[GM_ACT] = rg(pin[sub]);
        s[GM_PART] = rg(pgp[sub]);
        s[GM_SW] = fp8 ? st[sub] + l * nb * kb * 4 : 0;
        break;
      }
      case OP_FIN:
        s[FN_PART] = rg(pgp[sub]);
        s[FN_SA] = fp8 ? rg(psa[sub]) : 0;
        s[FN_OUT] = sub == K_QKV ? qkv : sub == K_O ? r2b : sub == K_GU ? mb : rg("y");
        s[FN_R1] = sub == K_O ? r1b : 0;
        s[FN_OUT2] = l == L - 1 ? (sub == K_O ? t->ptr[MK_T_R2_OUT] : sub == K_DOWN ? t->ptr[MK_T_Y_OUT] : 0) : 0;
        break;
      case OP_ATTN:
        s[ATT_QKV] = qkv;
        s[ATT_GQ] = t->ptr[MK_T_G_Q] + l * d * 2;
        s[ATT_GK] = t->ptr[MK_T_G_K] + l * d * 2;
        s[ATT_KC] = t->ptr[MK_T_K_CACHE] + l * cache_layer;
        s[ATT_VC] = t->ptr[MK_T_V_CACHE] + l * cache_layer;
        s[ATT_BT] = t->ptr[MK_T_BLOCK_TABLE];
        s[ATT_PART] = ws + region_off(hp, "part");
        s[ATT_O] = ob;
        s[ATT_ROPE] = (uint64_t)p->d_rope;
        s[ATT_QB] = ws + region_off(hp, "qb");
        break;
      case OP_COMB:
        s[ATT_PART] = ws + region_off(hp, "part");
        s[ATT_O] = ob;
        break;
      case OP_QUANT:
        s[QT_IN] = sub == 0 ? ob : mb;
        s[QT_OUT] = rg(sub == 0 ? "oq" : "mq");
        s[QT_S] = rg(sub == 0 ? "so" : "sm");
        break;
      default: break;
    }
    if (spec1) continue;
    switch (hp.ops[row].opcode) {
      case OP_QKV:
        s[QKV_W] = t->ptr[MK_T_W_QKV] + l * nqkv * H * welem;
        s[QKV_GAMMA] = t->ptr[MK_T_G_ATTN] + l * H * 2;
        s[QKV_X] = l == 0 ? t->ptr[MK_T_X] : 0;
        s[QKV_RIN] = l == 0 ? t->ptr[MK_T_R_IN] : 0;
        s[QKV_OUT] = qkv;
        s[QKV_R1] = l == 0 ? 0 : r1b;
        break;
      case OP_ATTN:
        s[ATT_QKV] = qkv;
        s[ATT_GQ] = t->ptr[MK_T_G_Q] + l * d * 2;
        s[ATT_GK] = t->ptr[MK_T_G_K] + l * d * 2;
        s[ATT_KC] = t->ptr[MK_T_K_CACHE] + l * cache_layer;
        s[ATT_VC] = t->ptr[MK_T_V_CACHE] + l * cache_layer;
        s[ATT_BT] = t->ptr[MK_T_BLOCK_TABLE];
        s[ATT_PART] = ws + region_off(hp, "part");
        s[ATT_O] = ob;
        s[ATT_ROPE] = (uint64_t)p->d_rope;
        break;
      case OP_OPROJ:
        s[O_W] = t->ptr[MK_T_W_O] + l * H * Hq * d * welem;
        s[O_IN] = ob;
        s[O_X] = l == 0 ? t->ptr[MK_T_X] : 0;
        s[O_RIN] = l == 0 ? t->ptr[MK_T_R_IN] : 0;
        s[O_R2] = r2b;
        s[O_R1] = l == 0 ? 0 : r1b;
        s[O_R2OUT] = l == L - 1 ? t->ptr[MK_T_R2_OUT] : 0;
        break;
      case OP_GATEUP:
        s[GU_W] = t->ptr[MK_T_W_GU] + l * 2 * I * H * welem;
        s[GU_GAMMA] = t->ptr[MK_T_G_MLP] + l * H * 2;
        s[GU_R2] = r2b;
        s[GU_M] = mb;
        break;
      case OP_DOWN:
        s[DN_W] = t->ptr[MK_T_W_DOWN] + l * H * I * welem;
        s[DN_M] = mb;
        s[DN_Y] = l == L - 1 ? t->ptr[MK_T_Y_OUT] : 0;
        s[DN_R2] = r2b;
        s[DN_R1] = r1b;
        break;
      case OP_LMHEAD:
        s[LM_W] = t->ptr[MK_T_W_LM];
        s[LM_GAMMA] = t->ptr[MK_T_G_FINAL];
        s[LM_R1] = r1b;
        s[LM_LOGITS] = t->ptr[MK_T_LOGITS_OUT];
        s[LM_PART] = ws + region_off(hp, "lm_part");
        s[LM_TOKEN] = t->ptr[MK_T_TOKEN_OUT];
        break;
      default: break;
    }
  }
}

mk_status get_table(mk_plan* p, const mk_tensors* t, uint64_t** out) {
  std::vector<uint64_t> key(t->ptr, t->ptr + t->n);
  auto it = p->tables.find(key);
  if (it != p->tables.end()) {
    *out = it->second;
    return MK_OK;
  }
  std::vector<uint64_t> tab;
  fill_table(p, t, tab);
  uint64_t* d = nullptr;
  HIP_TRY(hipMalloc(&d, tab.size() * sizeof(uint64_t)));
  HIP_TRY(hipMemcpy(d, tab.data(), tab.size() * sizeof(uint64_t), hipMemcpyHostToDevice));
  p->tables[key] = d;
  *out = d;
  return MK_OK;
}

// Multi-row plans run with loader waves, which keep HBM streaming while the op bodies compute,
// except the indexer front: its phases are a few tasks per worker, bound by dependency hops,
// where the loaders' LDS barrier costs more than the streaming gains.
static bool use_loaders(const mk_plan* p) { return p->hp.tp.spec == 1 && p->hp.cfg.workload != MK_INDEXER_FRONT; }

mk_status check_runnable(mk_plan* p) {
  if (p->host_only) return fail(MK_ERR_INVALID, "plan was built without a device");
  const mk::HostPlan& hp = p->hp;
  const mk_config& c = hp.cfg;
  const int g = c.workload == MK_INDEXER_FRONT ? 1 : c.n_q_heads / c.n_kv_heads;
  if (g != 1 && g != 2 && g != 4) return fail(MK_ERR_UNSUPPORTED, "GQA group must be 1, 2 or 4");
  if (c.weight_fp8 != c.act_fp8) return fail(MK_ERR_UNSUPPORTED, "FP8 weights come with FP8 activations (W8A8) only");
  if (hp.tp.spec == 0) {
    if (c.weight_fp8)
      return fail(MK_ERR_UNSUPPORTED, "the single-token (M = 1) op bodies are built for bf16 weights only");
    if (c.hidden > 2048 || c.inter > 6144 || c.n_q_heads * c.head_dim > 6144 || hp.tp.r_o > 128 ||
        hp.tp.r_down > 128 || hp.tp.r_gu % 2 || c.hidden % 512 || c.inter % 512 || (c.n_q_heads * c.head_dim) % 512)
      return fail(MK_ERR_UNSUPPORTED, "shape exceeds the M = 1 op bodies (hidden <= 2048; inter, q width <= 6144; "
                                      "hidden, inter and q width multiples of 512; even gate/up tiles)");
  } else if (c.workload == MK_INDEXER_FRONT) {
    if (c.idx_heads != 64) return fail(MK_ERR_UNSUPPORTED, "the indexer score body holds 64 heads");
  } else {
    const int K[3] = {c.hidden, c.n_q_heads * c.head_dim, c.inter};
    for (int k : K)
      if (k / hp.tp.kc > mk::kMaxChunks)
        return fail(MK_ERR_UNSUPPORTED, "multi-row projection with more K chunks than a finalize task adds");
    if (c.hidden > 8192 || c.inter > 12288 || c.n_q_heads * c.head_dim > 12288 || c.hidden % 512 || c.inter % 512)
      return fail(MK_ERR_UNSUPPORTED, "shape exceeds the multi-row op bodies (hidden <= 8192, inter and q width "
                                      "<= 12288, hidden and inter multiples of 512)");
  }
  if (!p->occupancy_checked) {
    int per_cu = 0;
    HIP_TRY(hipSetDevice(p->device));
    HIP_TRY(mk::worker_occupancy(&per_cu, hp.tp.spec));
    if (per_cu < 1) return fail(MK_ERR_UNSUPPORTED, "worker block does not fit on a compute unit");
    if (hp.W > p->cus * per_cu) return fail(MK_ERR_INVALID, "more workers than co-resident blocks: the persistent kernel could deadlock");
    p->occupancy_checked = true;
  }
  return MK_OK;
}

mk::KArgs base_args(const mk_plan* p, const uint64_t* table) {
  mk::KArgs a{};
  a.table = table;
  a.events = p->d_events;
  a.arrivals = p->d_arrivals;
  a.err = p->d_err;
  a.trace = p->d_trace;
  a.gather = p->d_gather;
  a.tag0 = p->salt + p->epoch * 1024u;
  a.run = p->cruns;
  a.flags = p->hp.cfg.flags;
  a.sh = p->sh;
  return a;
}

}  // namespace

extern "C" {

const char* mk_last_error(void) { return g_err.c_str(); }

mk_status mk_build_queue(const mk_config* cfg, const int32_t* host_context_lens, mk_plan** out) {
  if (!cfg || !host_context_lens || !out) return fail(MK_ERR_INVALID, "null argument");
  *out = nullptr;
  auto p = std::make_unique<mk_plan>();
  {  // record tag base of this plan: a plan count and the clock mixed (multiplicative hashing)
    static std::atomic<uint32_t> plans{0};
    const uint64_t ns = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
    uint32_t h = (plans.fetch_add(1) + 1u) * 0x9E3779B1u ^ (uint32_t)(ns ^ (ns >> 32)) * 0x85EBCA77u;
    p->salt = h & ~1023u;
  }
  // without a device (host-only planning, e.g. to inspect queues) the worker count must be given
  bool have_device = hipGetDevice(&p->device) == hipSuccess;
  if (have_device) {
    hipDeviceProp_t prop;
    have_device = hipGetDeviceProperties(&prop, p->device) == hipSuccess;
    if (have_device) p->cus = prop.multiProcessorCount;
  }
  if (!have_device) {
    (void)hipGetLastError();
    if (cfg->num_workers <= 0) return fail(MK_ERR_HIP, "no HIP device: give num_workers to plan on the host only");
  }
  const int W = cfg->num_workers > 0 ? cfg->num_workers : p->cus;
  std::string err;
  mk_status st = mk::plan_build(*cfg, host_context_lens, W, p->hp, err);
  if (st != MK_OK) return fail(st, err);
  p->host_only = !have_device;
  const mk::HostPlan& hp = p->hp;
  const mk_config& c = hp.cfg;
  if (p->host_only) {
    *out = p.release();
    return MK_OK;
  }
  p->sh = mk::Shapes{c.hidden, c.inter, c.n_q_heads, c.n_kv_heads, c.n_kv_heads ? c.n_q_heads / c.n_kv_heads : 1,
                     (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, c.page_size, c.max_pages_per_req,
                     hp.max_splits, c.vocab, c.rms_eps, 1.0f / std::sqrt((float)c.head_dim),
                     c.n_requests * c.tokens_per_request, hp.tp.kc, c.act_fp8 ? 1 : 0, c.num_layers,
                     c.idx_q_rank, c.idx_heads, c.tokens_per_request, 0};
  for (int r = 0; r < c.n_requests; ++r) p->sh.smax = std::max(p->sh.smax, (int)host_context_lens[r]);
  p->sh.npages = c.num_phys_pages;
  p->sh.topk = c.topk;
  p->sh.mla = c.mla_heads;
  p->sh.rg = (p->sh.M + 15) / 16;
  HIP_TRY(hipMalloc(&p->d_queue, hp.queue.size() * 4));
  HIP_TRY(hipMemcpy(p->d_queue, hp.queue.data(), hp.queue.size() * 4, hipMemcpyHostToDevice));
  HIP_TRY(hipMalloc(&p->d_tasks, hp.tasks.size() * 4));
  HIP_TRY(hipMemcpy(p->d_tasks, hp.tasks.data(), hp.tasks.size() * 4, hipMemcpyHostToDevice));
  p->events_bytes = std::max<size_t>(1, hp.thresholds.size()) * mk::kEvStride * 4;
  p->arrivals_bytes = std::max(1, hp.n_arrivals) * mk::kSubStride * 4;
  HIP_TRY(hipMalloc(&p->d_events, p->events_bytes));
  HIP_TRY(hipMemset(p->d_events, 0, p->events_bytes));
  HIP_TRY(hipMalloc(&p->d_arrivals, p->arrivals_bytes));
  HIP_TRY(hipMemset(p->d_arrivals, 0, p->arrivals_bytes));
  HIP_TRY(hipMalloc(&p->d_err, 64));
  HIP_TRY(hipMemset(p->d_err, 0, 64));
  // RoPE table: per row m (request r = m / T, its token m % T of T new ones), (cos, sin) of
  // pos * theta^(-2i/d) for i < d/2 with pos = ctx_r - T + m % T
  const int T = c.tokens_per_request, M = c.n_requests * T;
  const int hd = c.workload == MK_INDEXER_FRONT ? c.idx_head_dim : c.head_dim, half = hd / 2;
  std::vector<float> rope((size_t)M * half * 2);
  std::vector<int32_t> posv(M);
  for (int m = 0; m < M; ++m) {
    posv[m] = host_context_lens[m / T] - T + m % T;
    for (int i = 0; i < half; ++i) {
      const double ang = (double)posv[m] * std::pow((double)c.rope_theta, -2.0 * i / hd);
      rope[((size_t)m * half + i) * 2] = (float)std::cos(ang);
      rope[((size_t)m * half + i) * 2 + 1] = (float)std::sin(ang);
    }
  }
  HIP_TRY(hipMalloc(&p->d_rope, rope.size() * 4));
  HIP_TRY(hipMemcpy(p->d_rope, rope.data(), rope.size() * 4, hipMemcpyHostToDevice));
  HIP_TRY(hipMalloc(&p->d_pos, posv.size() * 4));
  HIP_TRY(hipMemcpy(p->d_pos, posv.data(), posv.size() * 4, hipMemcpyHostToDevice));
  if (c.flags & MK_FLAG_TRACE) {
    HIP_TRY(hipMalloc(&p->d_trace, (size_t)hp.W * hp.L * mk::kTraceWords * 4));
    HIP_TRY(hipMemset(p->d_trace, 0, (size_t)hp.W * hp.L * mk::kTraceWords * 4));
  }
  {  // no-allocation runs: the scratch address of this device, and the table as a relocation list (the
     // table of a tensor set whose entry i is (i + 1) << 48: every slot is 0, a library address below 2^48,
     // or tensor i plus an offset)
    HIP_TRY(mk::scratch_init(p->device));
    mk_tensors tag{};
    tag.n = MK_MAX_TENSORS;
    for (int i = 0; i < MK_MAX_TENSORS; ++i) tag.ptr[i] = (uint64_t)(i + 1) << 48;
    std::vector<uint64_t> tab;
    fill_table(p.get(), &tag, tab);
    std::vector<mk::TableReloc> rel(tab.size());
    for (size_t k = 0; k < tab.size(); ++k) {
      const uint64_t v = tab[k], hi = v >> 48;
      rel[k] = hi == 0 ? mk::TableReloc{v, mk::kRelocAbs, 0} : mk::TableReloc{v & ((1ull << 48) - 1), (uint32_t)(hi - 1), 0};
    }
    p->n_reloc = (int)rel.size();
    HIP_TRY(hipMalloc(&p->d_reloc, std::max<size_t>(1, rel.size()) * sizeof(mk::TableReloc)));
    if (!rel.empty()) HIP_TRY(hipMemcpy(p->d_reloc, rel.data(), rel.size() * sizeof(mk::TableReloc), hipMemcpyHostToDevice));
    p->uid = ++g_plan_uid;
  }
  if (c.flags & MK_FLAG_DEBUG_GATHER) {  // one slot per (layer, request, kv head, K|V, token) or (request, key)
    const size_t tokens = (size_t)c.max_pages_per_req * c.page_size;
    p->gather_words = c.workload == MK_INDEXER_FRONT ? (size_t)c.n_requests * tokens
                                                     : (size_t)c.num_layers * c.n_requests * c.n_kv_heads * 2 * tokens;
    HIP_TRY(hipMalloc(&p->d_gather, p->gather_words * 4));
    HIP_TRY(hipMemset(p->d_gather, 0xFF, p->gather_words * 4));
  }
  *out = p.release();
  return MK_OK;
}

mk_status mk_plan_queue(const mk_plan* p, const uint32_t** q, int32_t* W, int32_t* L) {
  if (!p || !q || !W || !L) return fail(MK_ERR_INVALID, "null argument");
  *q = p->hp.queue.data();
  *W = p->hp.W;
  *L = p->hp.L;
  return MK_OK;
}

mk_status mk_plan_events(const mk_plan* p, const uint32_t** thr, int32_t* n) {
  if (!p || !thr || !n) return fail(MK_ERR_INVALID, "null argument");
  *thr = p->hp.thresholds.data();
  *n = (int32_t)p->hp.thresholds.size();
  return MK_OK;
}

mk_status mk_plan_info(const mk_plan* p, int32_t* n_tasks, int32_t* n_ops, int32_t* n_arrivals) {
  if (!p) return fail(MK_ERR_INVALID, "null plan");
  if (n_tasks) *n_tasks = p->hp.T;
  if (n_ops) *n_ops = (int32_t)p->hp.ops.size();
  if (n_arrivals) *n_arrivals = p->hp.n_arrivals;
  return MK_OK;
}

mk_status mk_plan_workspace_bytes(const mk_plan* p, size_t* bytes) {
  if (!p || !bytes) return fail(MK_ERR_INVALID, "null argument");
  *bytes = p->hp.workspace_bytes;
  return MK_OK;
}

mk_status mk_plan_workspace_region(const mk_plan* p, const char* name, size_t* offset, size_t* bytes) {
  if (!p || !name || !offset || !bytes) return fail(MK_ERR_INVALID, "null argument");
  for (auto& r : p->hp.regions)
    if (r.name == name) {
      *offset = r.offset;
      *bytes = r.bytes;
      return MK_OK;
    }
  return fail(MK_ERR_INVALID, std::string("no workspace region ") + name);
}

mk_status mk_run_layer(mk_plan* p, const mk_tensors* t, void* stream) {
  if (!p) return fail(MK_ERR_INVALID, "null plan");
  mk_status st = check_tensors(p, t);
  if (st != MK_OK) return st;
  if ((st = check_runnable(p)) != MK_OK) return st;
  uint64_t* table = nullptr;
  const bool new_set = p->tables.find(std::vector<uint64_t>(t->ptr, t->ptr + t->n)) == p->tables.end();
  if ((st = get_table(p, t, &table)) != MK_OK) return st;
  if (new_set)  // a workspace first seen by this plan: no stale record may carry one of its tags
    HIP_TRY(hipMemsetAsync((void*)t->ptr[ws_index(p->hp.cfg)], 0, p->hp.workspace_bytes, (hipStream_t)stream));
  if (p->d_gather) HIP_TRY(hipMemsetAsync(p->d_gather, 0xFF, p->gather_words * 4, (hipStream_t)stream));
  mk::KArgs a = base_args(p, table);
  a.instrs = p->d_queue;
  a.L = p->hp.L;
  a.first_task = 0;
  HIP_TRY(mk::launch_worker(a, p->hp.W, (hipStream_t)stream, p->hp.tp.spec, use_loaders(p)));
  p->epoch++;
  p->cruns++;
  return MK_OK;
}

mk_status mk_run_layer_noalloc(mk_plan* p, const mk_tensors* t, void* stream) {
  if (!p || !t) return fail(MK_ERR_INVALID, "null argument");
  const size_t tab_off = (p->hp.workspace_bytes + 255) & ~(size_t)255;
  const size_t tab_bytes = p->hp.ops.size() * mk::kTableSlots * sizeof(uint64_t);
  if (tab_off + tab_bytes > mk::kScratchBytes)
    return fail(MK_ERR_INVALID, "workspace of " + std::to_string(p->hp.workspace_bytes) + " bytes and a pointer table of " +
                                    std::to_string(tab_bytes) + " bytes exceed the no-allocation scratch of " +
                                    std::to_string(mk::kScratchBytes) + " bytes");
  if (p->host_only) return fail(MK_ERR_INVALID, "plan was built without a device");
  char* base = (char*)mk::scratch_base(p->device);
  if (!base) return fail(MK_ERR_INVALID, "no-allocation scratch not set up on this device");
  mk::TensorPtrs tp{};
  const int n = std::min<int>(t->n, MK_MAX_TENSORS);
  for (int i = 0; i < n; ++i) tp.ptr[i] = t->ptr[i];
  const int wsi = ws_index(p->hp.cfg);
  tp.ptr[wsi] = (uint64_t)(uintptr_t)base;  // the workspace is the scratch, whatever the caller passed
  mk_tensors chk = *t;
  chk.ptr[wsi] = tp.ptr[wsi];
  mk_status st = check_tensors(p, &chk);
  if (st != MK_OK) return st;
  if ((st = check_runnable(p)) != MK_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  uint64_t* table = (uint64_t*)(base + tab_off);
  const bool owner = g_scratch_owner[p->device].load() == p->uid;
  if (!owner)  // another plan's (or no) contents: start from a zeroed workspace, as a new workspace does
    HIP_TRY(hipMemsetAsync(base, 0, p->hp.workspace_bytes, s));
  if (!owner || std::memcmp(&tp, &p->noalloc_last, sizeof(tp)) != 0) {
    HIP_TRY(mk::launch_fill_table(p->d_reloc, p->n_reloc, tp, table, s));
    p->noalloc_last = tp;
    g_scratch_owner[p->device].store(p->uid);
  }
  if (p->d_gather) HIP_TRY(hipMemsetAsync(p->d_gather, 0xFF, p->gather_words * 4, s));
  mk::KArgs a = base_args(p, table);
  a.instrs = p->d_queue;
  a.L = p->hp.L;
  a.first_task = 0;
  HIP_TRY(mk::launch_worker(a, p->hp.W, s, p->hp.tp.spec, use_loaders(p)));
  p->epoch++;
  p->cruns++;
  return MK_OK;
}

mk_status mk_run_graph_baseline(mk_plan* p, const mk_tensors* t, int32_t multistream, void* stream_) {
  if (!p) return fail(MK_ERR_INVALID, "null plan");
  mk_status st = check_tensors(p, t);
  if (st != MK_OK) return st;
  if ((st = check_runnable(p)) != MK_OK) return st;
  hipStream_t stream = (hipStream_t)stream_;
  std::vector<uint64_t> key(t->ptr, t->ptr + t->n);
  key.push_back(multistream ? 1 : 0);
  auto it = p->graphs.find(key);
  if (it == p->graphs.end()) {
    uint64_t* table = nullptr;
    if ((st = get_table(p, t, &table)) != MK_OK) return st;
    const auto& ops = p->hp.ops;
    // stream per op: an op continues the stream of its first dependency unless another
    // consumer already continued it (independent branches then fork onto new streams)
    // at most kMaxBranchStreams streams: a branch beyond them shares one round-robin (every edge between
    // streams is an event, so any assignment keeps the order the graph needs; more streams than the
    // graph's real branch width only add cross-queue waits)
    constexpr int kMaxBranchStreams = 2;
    std::vector<int> op_stream(ops.size(), 0);
    std::vector<bool> continued(ops.size(), false);
    int n_streams = 1, forks = 0;
    if (multistream) {
      for (size_t k = 0; k < ops.size(); ++k) {
        const auto& deps = ops[k].deps;
        if (!deps.empty() && !continued[deps[0]]) {
          op_stream[k] = op_stream[deps[0]];
          continued[deps[0]] = true;
        } else if (!deps.empty()) {
          op_stream[k] = 1 + (forks++ % (kMaxBranchStreams - 1));
          n_streams = std::max(n_streams, op_stream[k] + 1);
        }
      }
    }
    // capture on library streams (the caller's stream may be the legacy null stream, which
    // cannot be captured); the instantiated graph is then launched on the caller's stream
    while ((int)p->streams.size() < n_streams) {
      hipStream_t s;
      HIP_TRY(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
      p->streams.push_back(s);
    }
    while (p->events.size() < ops.size() + 1) {
      hipEvent_t e;
      HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
      p->events.push_back(e);
    }
    auto sget = [&](int i) { return p->streams[i]; };
    hipStream_t cap = p->streams[0];
    GraphEntry ge;
    HIP_TRY(hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal));
    hipEvent_t fork = p->events[ops.size()];
    HIP_TRY(hipEventRecord(fork, cap));
    std::vector<bool> started(n_streams, false);
    started[0] = true;
    for (size_t k = 0; k < ops.size(); ++k) {
      hipStream_t s = sget(op_stream[k]);
      if (!started[op_stream[k]]) {
        HIP_TRY(hipStreamWaitEvent(s, fork, 0));
        started[op_stream[k]] = true;
      }
      for (int dep : ops[k].deps)
        if (op_stream[dep] != op_stream[k]) HIP_TRY(hipStreamWaitEvent(s, p->events[dep], 0));
      mk::KArgs a = base_args(p, table);
      a.flags = (a.flags & ~(uint32_t)(MK_FLAG_TRACE)) | mk::kModeGraph;
      a.instrs = p->d_tasks;
      a.first_task = ops[k].first_task;
      a.L = ops[k].n_tasks;
      const int grid = std::min(ops[k].n_tasks, p->hp.W);
      // a node's blocks run one task each (more tasks than workers: a few each), so the loader waves,
      // which stream leases ahead across a worker's queue, have nothing to run ahead of
      HIP_TRY(mk::launch_worker(a, grid, s, p->hp.tp.spec, false));
      HIP_TRY(hipEventRecord(p->events[k], s));
    }
    for (int i = 1; i < n_streams; ++i) {  // join every forked stream back
      int last = -1;
      for (size_t k = 0; k < ops.size(); ++k)
        if (op_stream[k] == i) last = (int)k;
      if (last >= 0) HIP_TRY(hipStreamWaitEvent(cap, p->events[last], 0));
    }
    HIP_TRY(hipStreamEndCapture(cap, &ge.graph));
    HIP_TRY(hipGraphInstantiate(&ge.exec, ge.graph, nullptr, nullptr, 0));
    it = p->graphs.emplace(key, ge).first;
  }
  if (p->d_gather) HIP_TRY(hipMemsetAsync(p->d_gather, 0xFF, p->gather_words * 4, stream));  // outside the graph
  HIP_TRY(hipGraphLaunch(it->second.exec, stream));
  return MK_OK;
}

mk_status mk_sync(mk_plan* p, void* stream) {
  if (!p) return fail(MK_ERR_INVALID, "null plan");
  if (p->host_only) return fail(MK_ERR_INVALID, "plan was built without a device");
  HIP_TRY(hipStreamSynchronize((hipStream_t)stream));
  uint32_t e[8];
  HIP_TRY(hipMemcpy(e, p->d_err, sizeof(e), hipMemcpyDeviceToHost));
  if (e[0]) {
    p->cruns = 0;
    HIP_TRY(hipMemset(p->d_events, 0, p->events_bytes));
    HIP_TRY(hipMemset(p->d_arrivals, 0, p->arrivals_bytes));
    HIP_TRY(hipMemset(p->d_err, 0, 64));
    HIP_TRY(hipDeviceSynchronize());
    if (e[0] == mk::kErrBlockTable)
      return fail(MK_ERR_INVALID, "block table entry " + std::to_string((int32_t)e[4]) + " of request " + std::to_string(e[3]) +
                                      " is outside the pool of " + std::to_string(p->hp.cfg.num_phys_pages) +
                                      " pages (read as page 0; the run's outputs are not valid)");
    return fail(MK_ERR_TIMEOUT, "watchdog: worker " + std::to_string(e[1]) + " task " + std::to_string(e[2]) +
                                    " waited for tag " + std::to_string(e[3]) + " over " + std::to_string(e[4]) +
                                    " polls");
  }
  return MK_OK;
}

mk_status mk_read_trace(const mk_plan* p, uint32_t* out, size_t n_words) {
  if (!p || !out) return fail(MK_ERR_INVALID, "null argument");
  if (!p->d_trace) return fail(MK_ERR_INVALID, "plan was not built with MK_FLAG_TRACE");
  const size_t have = (size_t)p->hp.W * p->hp.L * mk::kTraceWords;
  HIP_TRY(hipMemcpy(out, p->d_trace, std::min(have, n_words) * 4, hipMemcpyDeviceToHost));
  return MK_OK;
}

mk_status mk_read_gather(const mk_plan* p, int32_t* out, size_t n_words) {
  if (!p || !out) return fail(MK_ERR_INVALID, "null argument");
  if (!p->d_gather) return fail(MK_ERR_INVALID, "plan was not built with MK_FLAG_DEBUG_GATHER");
  HIP_TRY(hipMemcpy(out, p->d_gather, std::min(p->gather_words, n_words) * 4, hipMemcpyDeviceToHost));
  return MK_OK;
}

void mk_plan_destroy(mk_plan* p) {
  if (!p) return;
  for (auto& kv : p->graphs) {
    if (kv.second.exec) (void)hipGraphExecDestroy(kv.second.exec);
    if (kv.second.graph) (void)hipGraphDestroy(kv.second.graph);
  }
  for (auto& kv : p->tables) (void)hipFree(kv.second);
  for (auto s : p->streams) (void)hipStreamDestroy(s);
  for (auto e : p->events) (void)hipEventDestroy(e);
  (void)hipFree(p->d_queue);
  (void)hipFree(p->d_tasks);
  (void)hipFree(p->d_events);
  (void)hipFree(p->d_arrivals);
  (void)hipFree(p->d_err);
  (void)hipFree(p->d_rope);
  (void)hipFree(p->d_pos);
  if (p->d_trace) (void)hipFree(p->d_trace);
  if (p->d_gather) (void)hipFree(p->d_gather);
  (void)hipFree(p->d_reloc);
  if (p->device >= 0 && p->device < 64) {  // the scratch no longer holds a live plan's table
    uint64_t mine = p->uid;
    g_scratch_owner[p->device].compare_exchange_strong(mine, 0);
  }
  delete p;
}

}  // extern "C"
