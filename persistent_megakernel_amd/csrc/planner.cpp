// Host planner: workload template -> tile tasks -> events -> round-robin worker queues.
//
// The lowering follows the MegaRTP page ("Kernel-Mega-PDL", section 4): each op expands
// into tile tasks; each (producer op, consumer op) pair becomes events whose threshold is
// the number of producer tasks writing the region the consumer reads; tasks are numbered in
// topological order and dealt round-robin onto fixed worker queues padded with NoOp, giving
// an instruction tensor [W, L, 32] of uint32.  Deadlock freedom needs only that every wait
// names events produced by smaller task ids and that all workers are co-resident (handbook
// megakernel section, exercise 3); the builder checks the first, the launcher the second.
#include <algorithm>
#include <cstring>

#include "mk_internal.hpp"

namespace mk {
namespace {

int pow2floor(int x) {
  int p = 1;
  while (p * 2 <= x) p *= 2;
  return p;
}
int pow2ceil(int x) {
  int p = 1;
  while (p < x) p *= 2;
  return p;
}
int largest_divisor_le(int n, int cap) {
  cap = std::max(1, std::min(n, cap));
  for (int r = cap; r > 0; --r)
    if (n % r == 0) return r;
  return 1;
}

struct Builder {
  std::vector<uint32_t> tasks;
  std::vector<uint32_t> thr;
  int n_arrivals = 0;
  std::vector<OpInfo> ops;

  int event(uint32_t threshold) {
    thr.push_back(threshold);
    return (int)thr.size() - 1;
  }
  int op_row(uint32_t opcode, int layer, std::vector<int> deps, uint32_t sub = 0) {
    ops.push_back(OpInfo{opcode, sub, layer, (int)(tasks.size() / kWords), 0, std::move(deps)});
    return (int)ops.size() - 1;
  }
  int task(uint32_t opcode, int row, int spec, std::initializer_list<std::pair<int, uint32_t>> waits,
           std::initializer_list<std::pair<int, uint32_t>> sigs, std::initializer_list<int64_t> payload) {
    int tid = (int)(tasks.size() / kWords);
    size_t base = tasks.size();
    tasks.resize(base + kWords, 0u);
    uint32_t* w = tasks.data() + base;
    w[W_OPCODE] = opcode;
    w[W_NWAIT] = (uint32_t)waits.size();
    w[W_NSIG] = (uint32_t)sigs.size();
    w[W_ROW] = (uint32_t)row;
    w[W_SPEC] = (uint32_t)spec;
    w[W_TASK] = (uint32_t)tid;
    int i = 0;
    for (auto& e : waits) {
      w[W_WAIT0 + 2 * i] = (uint32_t)e.first;
      w[W_WAIT0 + 2 * i + 1] = e.second;
      ++i;
    }
    i = 0;
    for (auto& s : sigs) {
      w[W_SIG0 + 3 * i] = (uint32_t)s.first;
      w[W_SIG0 + 3 * i + 1] = s.second;
      w[W_SIG0 + 3 * i + 2] = (uint32_t)tid;
      ++i;
    }
    i = 0;
    for (int64_t v : payload) w[W_LAYER + i++] = (uint32_t)(v & 0xFFFFFFFFll);
    if (ops[row].n_tasks == 0) ops[row].first_task = tid;
    ops[row].n_tasks++;
    return tid;
  }
};

// K chunk of an e4m3 projection tile: the largest multiple of 128 dividing K with kM16Rows rows
// within one lease
int kchunk(int K) {
  for (int kc = kLeaseBytes / kM16Rows; kc > 0; kc -= 128)
    if (K % kc == 0) return kc;
  return 0;
}

bool tile_params(const mk_config& c, int W, const int32_t* ctx, TileParams& p, std::string& err) {
  for (int k = 6; k < MK_TILE_PARAMS; ++k)
    if (c.tile_params[k] != 0) {
      err = "tile_params entries 6 and 7 are reserved and must be 0";
      return false;
    }
  if (c.workload == MK_INDEXER_FRONT) {
    for (int k = 0; k < MK_TILE_PARAMS; ++k)
      if (c.tile_params[k] != 0) {
        err = "the indexer front's tiles are fixed: its tile_params must be 0";
        return false;
      }
    p.spec = 1;
    p.kc = kchunk(c.hidden);
    p.kc_q = kchunk(c.idx_q_rank);
    p.s_tok = kScoreTok;
    if (!p.kc || !p.kc_q) {
      err = "indexer projections need K a multiple of 128";
      return false;
    }
    return true;
  }
  const int H = c.hidden, I = c.inter, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int R = c.n_requests;
  const int elem = c.weight_fp8 ? 1 : 2;
  const int n_qkv = (Hq + 2 * Hkv) * d;
  // rows of one tile: the lease (weights, plus the 1 KiB-rounded norm gain of the fused
  // add + RMSNorm ops) stays within kLeaseBytes
  const int gain = (2 * H + 1023) / 1024 * 1024;
  auto cap_rows = [&](int k, int nmat, int extra) { return std::max(1, (kLeaseBytes - extra) / (k * elem * nmat)); };
  p.r_qkv = pow2floor(std::min({d, std::max(1, n_qkv / W), cap_rows(H, 1, gain)}));
  p.r_o = largest_divisor_le(H, std::min(std::max(1, H / W), cap_rows(Hq * d, 1, 0)));
  p.r_gu = largest_divisor_le(I, std::min(std::max(1, I / W), cap_rows(H, 2, gain + 1024)));
  p.r_down = largest_divisor_le(H, std::min(std::max(1, H / W), cap_rows(I, 1, 0)));
  // lm_head: one task per worker, its rows streamed from HBM inside the body (no weight lease)
  p.r_lm = c.workload == MK_QWEN3_STEP ? (c.vocab + W - 1) / W : 0;
  int ctx_max = 0;
  for (int r = 0; r < R; ++r) ctx_max = std::max(ctx_max, (int)ctx[r]);
  // about W/2 attention tasks: fewer splits keep the combine short; the KV is prefetched anyway
  long long want = (2ll * R * ctx_max * Hkv + W - 1) / W;
  p.s_tok = std::max(4, std::min(kLeaseBytes / (4 * d), pow2ceil((int)std::max(1ll, want))));
  p.spec = (R * c.tokens_per_request == 1) ? 0 : 1;
  p.kc = p.spec == 1 ? kLeaseBytes / (kM16Rows * elem) : 0;
  // the caller's tile sizes, each checked against what the op bodies run
  const int32_t* t = c.tile_params;
  if (p.spec == 1 && (t[MK_TP_ROWS_QKV] || t[MK_TP_ROWS_O] || t[MK_TP_ROWS_GATEUP] || t[MK_TP_ROWS_DOWN] ||
                      t[MK_TP_ROWS_LMHEAD])) {
    err = "multi-row plans use fixed 64-row projection tiles: tile_params rows entries must be 0";
    return false;
  }
  auto bad = [&](const char* m) {
    err = m;
    return false;
  };
  if (const int v = t[MK_TP_ROWS_QKV]) {
    if (v < 1 || v > d || (v & (v - 1)) || v > cap_rows(H, 1, gain) || n_qkv % v)
      return bad("tile_params QKV rows: a power of two <= head_dim whose weights and gain fit one lease");
    p.r_qkv = v;
  }
  if (const int v = t[MK_TP_ROWS_O]) {
    if (v < 1 || H % v || v > 128 || v > cap_rows(Hq * d, 1, 0))
      return bad("tile_params O rows: a divisor of hidden, <= 128, whose weights fit one lease");
    p.r_o = v;
  }
  if (const int v = t[MK_TP_ROWS_GATEUP]) {
    if (v < 2 || v % 2 || I % v || v > cap_rows(H, 2, gain + 1024))
      return bad("tile_params gate/up rows: an even divisor of inter whose gate, up and gain fit one lease");
    p.r_gu = v;
  }
  if (const int v = t[MK_TP_ROWS_DOWN]) {
    if (v < 1 || H % v || v > 128 || v > cap_rows(I, 1, 0))
      return bad("tile_params down rows: a divisor of hidden, <= 128, whose weights fit one lease");
    p.r_down = v;
  }
  if (const int v = t[MK_TP_ROWS_LMHEAD]) {
    if (c.workload != MK_QWEN3_STEP || v < 1 || v > c.vocab)
      return bad("tile_params lm_head rows: 1 .. vocab, decode step only");
    p.r_lm = v;
  }
  if (const int v = t[MK_TP_SPLIT_TOKENS]) {
    if (v < 4 || v > kLeaseBytes / (4 * d) || (v & (v - 1)))
      return bad("tile_params split tokens: a power of two in 4 .. 128");
    p.s_tok = v;
  }
  return true;
}

// Multi-row (M = R x T <= 256) layer: row-task norms, projections as (64-row tile, K chunk) tasks
// writing partial sums for every 16-row group of M (the weights are read once), one finalize task
// per (row tile, row group) adding the chunks in K order and applying the epilogue; FP8 plans
// quantise o and m per row.  Row-level consumers wait for their own group's finalizes only.  The
// same rules as the oracle's builder.
void build_m16(const mk_config& c, const int32_t* ctx, const TileParams& p, int W, Builder& b, int& max_splits) {
  const int H = c.hidden, I = c.inter, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int g = Hq / Hkv, R = c.n_requests, T = c.tokens_per_request, M = R * T, G = (M + 15) / 16;
  const int spec = p.spec, kc = p.kc, st = p.s_tok, rt = kM16Rows;
  const int n_qkv = (Hq + 2 * Hkv) * d;
  const bool fp8 = c.act_fp8 != 0;
  auto proj = [&](uint32_t kind, int l, int N, int K, int rows, std::pair<int, uint32_t> wait, int dep_row,
                  auto fin_event) -> int {
    const int row_g = b.op_row(OP_GEMM, l, {dep_row}, kind);
    const int nt = N / rows, nk = K / kc;
    std::vector<int> parts(nt);
    for (int j = 0; j < nt; ++j) parts[j] = b.event((uint32_t)nk);
    for (int j = 0; j < nt; ++j)
      for (int ck = 0; ck < nk; ++ck)
        b.task(OP_GEMM, row_g, spec, {wait}, {{parts[j], 1u}}, {l, kind, j, j * rows, rows, ck * kc, kc});
    const int row_f = b.op_row(OP_FIN, l, {row_g}, kind);
    for (int j = 0; j < nt; ++j)
      for (int gi = 0; gi < G; ++gi)
        b.task(OP_FIN, row_f, spec, {{parts[j], (uint32_t)nk}}, {{fin_event(j, gi), 1u}},
               {l, kind, j, j * rows, rows, nk, kc, 0, 0, gi});  // gi at W_GROUP
    return row_f;
  };
  std::vector<int> prev;  // per row group: the previous layer's down finalizes
  int prev_row = -1;
  uint32_t prev_thr = 0;
  for (int l = 0; l < c.num_layers; ++l) {
    const int row_na = b.op_row(OP_NORM, l, prev_row >= 0 ? std::vector<int>{prev_row} : std::vector<int>{}, 0);
    const int ev_na = b.event((uint32_t)M);
    for (int m = 0; m < M; ++m) {
      if (prev.empty())
        b.task(OP_NORM, row_na, spec, {}, {{ev_na, 1u}}, {l, 0, m});
      else
        b.task(OP_NORM, row_na, spec, {{prev[m / 16], prev_thr}}, {{ev_na, 1u}}, {l, 0, m});
    }
    // QKV: a 64-row tile lies inside one head; its finalize of a row group counts for the head's
    // kv group and that row group
    const uint32_t tiles_per_group = (uint32_t)((g + 2) * d / rt);
    std::vector<int> ev_qkv((size_t)Hkv * G);
    for (int q = 0; q < Hkv * G; ++q) ev_qkv[q] = b.event(tiles_per_group);
    auto qkv_group = [&](int j) {
      const int n0 = j * rt;
      if (n0 < Hq * d) return (n0 / d) / g;
      if (n0 < (Hq + Hkv) * d) return (n0 - Hq * d) / d;
      return (n0 - (Hq + Hkv) * d) / d;
    };
    const int row_qf = proj(K_QKV, l, n_qkv, H, rt, {ev_na, (uint32_t)M}, row_na,
                            [&](int j, int gi) { return ev_qkv[qkv_group(j) * G + gi]; });
    // split-KV attention: the (request, kv head, split) tasks are laid out so that dealing them
    // round-robin hands each worker a run of consecutive splits of one (request, kv head) -- a
    // chain, folded into one running softmax state on chip and written as one partial.  The
    // splits, pair after pair, fill columns 0 .. C-1 of the op's rounds of C tasks (C = min(W,
    // tasks), a column being one worker's share, longer columns first); a chain is a column's
    // maximal run inside one pair.  One event per pair counts its chains; one combine task per
    // pair reduces their partials (dealt round-robin, not left to whichever chain ends last).
    const int row_attn = b.op_row(OP_ATTN, l, {row_qf});
    struct Split {
      int pair, s;
    };
    std::vector<Split> seq;
    std::vector<int> nsplit(R);
    for (int r = 0; r < R; ++r) {
      nsplit[r] = (ctx[r] + st - 1) / st;
      max_splits = std::max(max_splits, nsplit[r]);
      for (int hk = 0; hk < Hkv; ++hk)
        for (int s = 0; s < nsplit[r]; ++s) seq.push_back({r * Hkv + hk, s});
    }
    const int n = (int)seq.size(), C = std::min(W, n), rounds = (n + C - 1) / C, full = n - (rounds - 1) * C;
    std::vector<int> start(C), len(C), flags(n), slot(n), nchain((size_t)R * Hkv, 0);
    for (int j = 0, at = 0; j < C; ++j) {
      len[j] = j < full ? rounds : rounds - 1;
      start[j] = at;
      at += len[j];
      for (int k = 0; k < len[j]; ++k) {
        const int i = start[j] + k;
        const bool cont = k > 0 && seq[i - 1].pair == seq[i].pair;
        const bool end = k == len[j] - 1 || seq[i + 1].pair != seq[i].pair;
        if (!cont) nchain[seq[i].pair]++;
        flags[i] = (cont ? 1 : 0) | (end ? 2 : 0);
        slot[i] = nchain[seq[i].pair] - 1;
      }
    }
    std::vector<int> ev_att((size_t)R * Hkv);
    for (int q = 0; q < R * Hkv; ++q) ev_att[q] = b.event((uint32_t)nchain[q]);
    for (int k = 0; k < rounds; ++k)
      for (int j = 0; j < C && k < len[j]; ++j) {
        const int i = start[j] + k, r = seq[i].pair / Hkv, hk = seq[i].pair % Hkv, s = seq[i].s;
        const int t0 = s * st, t1 = std::min((int)ctx[r], (s + 1) * st);
        const std::pair<int, uint32_t> qkv_wait{ev_qkv[hk * G + r * T / 16], tiles_per_group};
        if (flags[i] & 2)
          b.task(OP_ATTN, row_attn, spec, {qkv_wait}, {{ev_att[seq[i].pair], 1u}},
                 {l, r, hk, s, t0, t1, 0, 0, 0, nsplit[r], flags[i], slot[i]});
        else
          b.task(OP_ATTN, row_attn, spec, {qkv_wait}, {}, {l, r, hk, s, t0, t1, 0, 0, 0, nsplit[r], flags[i], slot[i]});
      }
    const int row_comb = b.op_row(OP_COMB, l, {row_attn});
    const int ev_oready = b.event((uint32_t)(R * Hkv));
    for (int q = 0; q < R * Hkv; ++q)
      b.task(OP_COMB, row_comb, spec, {{ev_att[q], (uint32_t)nchain[q]}}, {{ev_oready, 1u}},
             {l, q / Hkv, q % Hkv, nchain[q]});
    std::pair<int, uint32_t> o_wait{ev_oready, (uint32_t)(R * Hkv)};
    int o_dep = row_comb;
    if (fp8) {
      const int row_qo = b.op_row(OP_QUANT, l, {row_comb}, 0);
      const int ev_oq = b.event((uint32_t)M);
      for (int m = 0; m < M; ++m) b.task(OP_QUANT, row_qo, spec, {o_wait}, {{ev_oq, 1u}}, {l, 0, m});
      o_wait = {ev_oq, (uint32_t)M};
      o_dep = row_qo;
    }
    std::vector<int> ev_o(G);
    for (int gi = 0; gi < G; ++gi) ev_o[gi] = b.event((uint32_t)(H / rt));
    const int row_of = proj(K_O, l, H, Hq * d, rt, o_wait, o_dep, [&](int, int gi) { return ev_o[gi]; });
    const int row_nb = b.op_row(OP_NORM, l, {row_of}, 1);
    const int ev_nb = b.event((uint32_t)M);
    for (int m = 0; m < M; ++m)
      b.task(OP_NORM, row_nb, spec, {{ev_o[m / 16], (uint32_t)(H / rt)}}, {{ev_nb, 1u}}, {l, 1, m});
    // gate/up: a tile holds rt/2 gate rows and the matching rt/2 up rows.  W8A8: the per-row
    // quantisation waits for its row group's finalizes; bf16: the down tiles read every group
    const uint32_t n_gu = (uint32_t)(I / (rt / 2));
    std::vector<int> ev_gu(fp8 ? G : 1);
    for (auto& e : ev_gu) e = b.event(fp8 ? n_gu : n_gu * (uint32_t)G);
    const int row_gf = proj(K_GU, l, I, H, rt / 2, {ev_nb, (uint32_t)M}, row_nb,
                            [&](int, int gi) { return ev_gu[fp8 ? gi : 0]; });
    std::pair<int, uint32_t> m_wait{ev_gu[0], n_gu * (uint32_t)G};
    int m_dep = row_gf;
    if (fp8) {
      const int row_qm = b.op_row(OP_QUANT, l, {row_gf}, 1);
      const int ev_mq = b.event((uint32_t)M);
      for (int m = 0; m < M; ++m) b.task(OP_QUANT, row_qm, spec, {{ev_gu[m / 16], n_gu}}, {{ev_mq, 1u}}, {l, 1, m});
      m_wait = {ev_mq, (uint32_t)M};
      m_dep = row_qm;
    }
    std::vector<int> ev_down(G);
    for (int gi = 0; gi < G; ++gi) ev_down[gi] = b.event((uint32_t)(H / rt));
    prev_row = proj(K_DOWN, l, H, I, rt, m_wait, m_dep, [&](int, int gi) { return ev_down[gi]; });
    prev = ev_down;
    prev_thr = (uint32_t)(H / rt);
  }
}

// Indexer front (MegaRTP page, section 4: A0 -> {B0, C0, B1}; {B0, C0} -> D1; {D1, B1} -> E1):
// row norms, e4m3 projection tiles with per-tile finalizes (per head for D1, so that RoPE pairs
// dimensions i and i + 64), the q_a norm rows, one key-cache task, per-(request, key split) score
// tasks.  The same rules as the oracle's builder.
void build_indexer(const mk_config& c, const int32_t* ctx, const TileParams& p, Builder& b) {
  const int H = c.hidden, qr = c.idx_q_rank, nh = c.idx_heads, hd = c.idx_head_dim;
  const int R = c.n_requests, M = R * c.tokens_per_request;
  const int spec = p.spec, rt = kM16Rows, st = p.s_tok, l = 0;
  auto tiles = [&](uint32_t kind, int N, int K, int kc, std::pair<int, uint32_t> wait, int dep, auto part_event) {
    const int row_g = b.op_row(OP_GEMM, l, {dep}, kind);
    for (int j = 0; j < N / rt; ++j)
      for (int ck = 0; ck < K / kc; ++ck)
        b.task(OP_GEMM, row_g, spec, {wait}, {{part_event(j), 1u}}, {l, kind, j, j * rt, rt, ck * kc, kc});
    return row_g;
  };
  auto fin = [&](uint32_t kind, int nt, int nk, int kc, const std::vector<int>& parts, int fin_event, int dep) {
    const int row_f = b.op_row(OP_FIN, l, {dep}, kind);
    for (int j = 0; j < nt; ++j)
      b.task(OP_FIN, row_f, spec, {{parts[j], (uint32_t)nk}}, {{fin_event, 1u}}, {l, kind, j, j * rt, rt, nk, kc});
    return row_f;
  };
  const int row_a0 = b.op_row(OP_NORM, l, {}, 0);
  const int ev_a0 = b.event((uint32_t)M);
  for (int m = 0; m < M; ++m) b.task(OP_NORM, row_a0, spec, {}, {{ev_a0, 1u}}, {l, 0, m});
  const int kc = p.kc, nk = H / kc;
  // B0
  const int nt = qr / rt;
  std::vector<int> parts(nt);
  for (int j = 0; j < nt; ++j) parts[j] = b.event((uint32_t)nk);
  const int row_b0 = tiles(K_QA, qr, H, kc, {ev_a0, (uint32_t)M}, row_a0, [&](int j) { return parts[j]; });
  const int ev_b0 = b.event((uint32_t)nt);
  const int row_b0f = fin(K_QA, nt, nk, kc, parts, ev_b0, row_b0);
  const int row_qn = b.op_row(OP_NORM, l, {row_b0f}, 2);
  const int ev_qn = b.event((uint32_t)M);
  for (int m = 0; m < M; ++m) b.task(OP_NORM, row_qn, spec, {{ev_b0, (uint32_t)nt}}, {{ev_qn, 1u}}, {l, 2, m});
  // C0
  const int nt_w = nh / rt;
  std::vector<int> parts_w(nt_w);
  for (int j = 0; j < nt_w; ++j) parts_w[j] = b.event((uint32_t)nk);
  const int row_c0 = tiles(K_W, nh, H, kc, {ev_a0, (uint32_t)M}, row_a0, [&](int j) { return parts_w[j]; });
  const int ev_w = b.event((uint32_t)nt_w);
  const int row_c0f = fin(K_W, nt_w, nk, kc, parts_w, ev_w, row_c0);
  // B1
  const int nt_k = hd / rt;
  std::vector<int> parts_k(nt_k);
  for (int j = 0; j < nt_k; ++j) parts_k[j] = b.event((uint32_t)nk);
  const int row_b1 = tiles(K_KI, hd, H, kc, {ev_a0, (uint32_t)M}, row_a0, [&](int j) { return parts_k[j]; });
  const int ev_k = b.event((uint32_t)nt_k);
  const int row_b1f = fin(K_KI, nt_k, nk, kc, parts_k, ev_k, row_b1);
  const int row_kc = b.op_row(OP_KCACHE, l, {row_b1f});
  const int ev_kc = b.event(1u);
  b.task(OP_KCACHE, row_kc, spec, {{ev_k, (uint32_t)nt_k}}, {{ev_kc, 1u}}, {l});
  // D1
  const int kcq = p.kc_q, nk_q = qr / kcq, per_head = hd / rt;
  std::vector<int> ev_head(nh);
  for (int h = 0; h < nh; ++h) ev_head[h] = b.event((uint32_t)(per_head * nk_q));
  const int row_d1 = tiles(K_QI, nh * hd, qr, kcq, {ev_qn, (uint32_t)M}, row_qn,
                           [&](int j) { return ev_head[j / per_head]; });
  const int row_d1f = b.op_row(OP_FIN, l, {row_d1}, K_QI);
  const int ev_qi = b.event((uint32_t)nh);
  for (int h = 0; h < nh; ++h)
    b.task(OP_FIN, row_d1f, spec, {{ev_head[h], (uint32_t)(per_head * nk_q)}}, {{ev_qi, 1u}},
           {l, K_QI, h, h * hd, hd, nk_q, kcq});
  // main-MLA query half, dealt after D1 and before E1 as in the page's tile list: D0 tiles of the
  // normalised q_a (as D1), a finalize per head, and D2's tiles of each head as soon as that head is
  // finalized (one event per head: the page's per-head tile_cover of D0 -> D2)
  if (c.mla_heads > 0) {
    const int nm = c.mla_heads, per_head_qb = kMlaNope / rt;
    std::vector<int> ev_qb(nm);
    for (int h = 0; h < nm; ++h) ev_qb[h] = b.event((uint32_t)(per_head_qb * nk_q));
    const int row_d0 = tiles(K_QB, nm * kMlaNope, qr, kcq, {ev_qn, (uint32_t)M}, row_qn,
                             [&](int j) { return ev_qb[j / per_head_qb]; });
    const int row_d0f = b.op_row(OP_FIN, l, {row_d0}, K_QB);
    std::vector<int> ev_qn_h(nm);
    for (int h = 0; h < nm; ++h) ev_qn_h[h] = b.event(1u);
    for (int h = 0; h < nm; ++h)
      b.task(OP_FIN, row_d0f, spec, {{ev_qb[h], (uint32_t)(per_head_qb * nk_q)}}, {{ev_qn_h[h], 1u}},
             {l, K_QB, h, h * kMlaNope, kMlaNope, nk_q, kcq});
    const int row_d2 = b.op_row(OP_GEMM, l, {row_d0f}, K_UK);
    for (int h = 0; h < nm; ++h)
      for (int j = 0; j < kMlaLatent / rt; ++j)
        b.task(OP_GEMM, row_d2, spec, {{ev_qn_h[h], 1u}}, {},
               {l, K_UK, h * (kMlaLatent / rt) + j, h * kMlaLatent + j * rt, rt, 0, kMlaNope, h * kMlaNope});
  }
  // E1; with a top-k, one event per request counts its score tasks
  const int row_e = b.op_row(OP_SCORE, l, {row_d1f, row_c0f, row_kc});
  const int T = c.tokens_per_request;
  std::vector<int> ev_e1;
  if (c.topk > 0)
    for (int r = 0; r < R; ++r) ev_e1.push_back(b.event((uint32_t)((ctx[r] + st - 1) / st)));
  for (int r = 0; r < R; ++r)
    for (int s2 = 0; s2 < (ctx[r] + st - 1) / st; ++s2) {
      const int t0 = s2 * st, t1 = std::min((int)ctx[r], (s2 + 1) * st);
      if (c.topk > 0)
        b.task(OP_SCORE, row_e, spec, {{ev_qi, (uint32_t)nh}, {ev_w, (uint32_t)nt_w}, {ev_kc, 1u}}, {{ev_e1[r], 1u}},
               {l, r, s2, t0, t1});
      else
        b.task(OP_SCORE, row_e, spec, {{ev_qi, (uint32_t)nh}, {ev_w, (uint32_t)nt_w}, {ev_kc, 1u}}, {}, {l, r, s2, t0, t1});
    }
  // top-k: one task per token row, after every score task of its request
  if (c.topk > 0) {
    const int row_tk = b.op_row(OP_TOPK, l, {row_e});
    for (int m = 0; m < M; ++m)
      b.task(OP_TOPK, row_tk, spec, {{ev_e1[m / T], (uint32_t)((ctx[m / T] + st - 1) / st)}}, {}, {l, m});
  }
}

// deal the tasks round-robin onto W queues padded with NoOp; move the builder's tables into the plan
mk_status pack_plan(Builder& b, int W, int max_splits, HostPlan& out, std::string& err) {
  out.T = (int)(b.tasks.size() / kWords);
  out.L = (out.T + W - 1) / W;
  out.queue.assign((size_t)W * out.L * kWords, 0u);
  for (int t = 0; t < out.T; ++t)
    std::memcpy(&out.queue[((size_t)(t % W) * out.L + t / W) * kWords], &b.tasks[(size_t)t * kWords],
                kWords * sizeof(uint32_t));
  out.tasks = std::move(b.tasks);
  out.thresholds = std::move(b.thr);
  out.n_arrivals = b.n_arrivals;
  out.ops = std::move(b.ops);
  out.max_splits = max_splits;

  // each op's tasks form one contiguous run of task ids (the graph baseline launches it)
  for (size_t r = 0; r < out.ops.size(); ++r) {
    const OpInfo& op = out.ops[r];
    for (int t = op.first_task; t < op.first_task + op.n_tasks; ++t)
      if (out.tasks[(size_t)t * kWords + W_ROW] != (uint32_t)r) {
        err = "planner invariant violated (op tasks not contiguous)";
        return MK_ERR_INVALID;
      }
  }

  return MK_OK;
}

mk_status check_events(const HostPlan& out, std::string& err) {
  // invariants: every wait names an event whose producers precede the waiter; thresholds equal
  // the increments issued per run
  std::vector<long long> produced(out.thresholds.size(), 0);
  std::vector<int> last_prod(out.thresholds.size(), -1);
  for (int t = 0; t < out.T; ++t) {
    const uint32_t* w = &out.tasks[(size_t)t * kWords];
    for (uint32_t k = 0; k < w[W_NWAIT]; ++k) {
      uint32_t e = w[W_WAIT0 + 2 * k];
      if (e >= out.thresholds.size() || w[W_WAIT0 + 2 * k + 1] != out.thresholds[e] || last_prod[e] >= t) {
        err = "planner invariant violated (wait)";
        return MK_ERR_INVALID;
      }
    }
    for (uint32_t k = 0; k < w[W_NSIG]; ++k) {
      uint32_t e = w[W_SIG0 + 3 * k];
      bool fires = w[W_ARR_N] == 0 || w[W_ARR_RANK] == w[W_ARR_N] - 1;
      if (fires) produced[e] += w[W_SIG0 + 3 * k + 1];
      last_prod[e] = t;
    }
  }
  for (size_t e = 0; e < produced.size(); ++e)
    if (produced[e] != (long long)out.thresholds[e]) {
      err = "planner invariant violated (threshold != increments)";
      return MK_ERR_INVALID;
    }
  return MK_OK;
}

mk_status plan_indexer(const mk_config& c, const int32_t* ctx, int W, HostPlan& out, std::string& err) {
  const int H = c.hidden, qr = c.idx_q_rank, nh = c.idx_heads, hd = c.idx_head_dim;
  const int R = c.n_requests, T = c.tokens_per_request, M = R * T, P = c.page_size;
  if (W < 1 || R < 1 || T < 1 || H < 1 || qr < 1 || nh < 1 || hd < 1) {
    err = "invalid shape";
    return MK_ERR_INVALID;
  }
  if (!c.weight_fp8 || !c.act_fp8) {
    err = "the indexer front is built for e4m3 weights and activations";
    return MK_ERR_UNSUPPORTED;
  }
  if (hd != 128 || nh % kM16Rows || qr % kM16Rows || H % 512 || qr % 512 || H > 8192 || qr > 8192 || T > 8 ||
      M > 16 || P % 8) {
    err = "unsupported indexer shape: head dim 128, heads a multiple of 64, hidden and q rank multiples of 512 "
          "(at most 8192), at most 8 tokens per request and 16 rows, page size a multiple of 8";
    return MK_ERR_UNSUPPORTED;
  }
  for (int r = 0; r < R; ++r)
    if (ctx[r] < T || ctx[r] > c.max_pages_per_req * P) {
      err = "context length out of range (at least the request's new tokens, at most its block table)";
      return MK_ERR_INVALID;
    }
  if (c.topk < 0 || c.mla_heads < 0) {
    err = "negative top-k or main-MLA head count";
    return MK_ERR_INVALID;
  }
  if (c.topk > 0)
    for (int r = 0; r < R; ++r)
      if (ctx[r] > kTopkMaxKeys) {
        err = "a top-k over more than 8192 keys per token is not built";
        return MK_ERR_UNSUPPORTED;
      }
  out = HostPlan{};
  out.cfg = c;
  out.ctx.assign(ctx, ctx + R);
  out.W = W;
  if (!tile_params(c, W, ctx, out.tp, err)) return MK_ERR_UNSUPPORTED;
  Builder b;
  build_indexer(c, ctx, out.tp, b);
  if (pack_plan(b, W, 0, out, err) != MK_OK) return MK_ERR_INVALID;
  size_t off = 0;
  auto region = [&](const char* name, size_t bytes) {
    out.regions.push_back({name, off, bytes});
    off += (bytes + 255) / 256 * 256;
  };
  const size_t kc = out.tp.kc, kcq = out.tp.kc_q;
  region("hq", (size_t)16 * H);          // A0 output, e4m3 operand order
  region("sh", 16 * 4);
  region("qa", (size_t)M * qr * 4);      // B0 output, fp32 rows
  region("qaq", (size_t)16 * qr);        // q_a norm output, e4m3 operand order
  region("sqa", 16 * 4);
  region("w", (size_t)M * nh * 4);       // C0 output, fp32 rows
  region("k", (size_t)M * hd * 4);       // B1 output, fp32 rows
  region("qi", (size_t)16 * nh * hd * 2);  // D1 output, bf16 in the score operand order
  region("gp_qa", (size_t)(qr / kM16Rows) * (H / kc) * 4096);
  region("gp_w", (size_t)(nh / kM16Rows) * (H / kc) * 4096);
  region("gp_k", (size_t)(hd / kM16Rows) * (H / kc) * 4096);
  region("gp_qi", (size_t)(nh * hd / kM16Rows) * (qr / kcq) * 4096);
  if (c.mla_heads > 0) {
    region("gp_qb", (size_t)(c.mla_heads * kMlaNope / kM16Rows) * (qr / kcq) * 4096);
    region("qn", (size_t)16 * c.mla_heads * kMlaNope * 2);  // D0 output, bf16 in D2's operand order
  }
  out.workspace_bytes = off;
  return check_events(out, err);
}

}  // namespace

mk_status plan_build(const mk_config& c, const int32_t* ctx, int W, HostPlan& out, std::string& err) {
  if (c.rotary_dim != 0 && c.rotary_dim != (c.workload == MK_INDEXER_FRONT ? c.idx_head_dim : c.head_dim)) {
    err = "partial rotary embeddings are not built: rotary_dim must be 0 or the head dim";
    return MK_ERR_UNSUPPORTED;
  }
  if (c.workload == MK_INDEXER_FRONT) return plan_indexer(c, ctx, W, out, err);
  if (c.topk != 0 || c.mla_heads != 0) {
    err = "top-k and the main-MLA half belong to the indexer front";
    return MK_ERR_INVALID;
  }
  if (c.workload != MK_QWEN3_LAYER && c.workload != MK_QWEN3_STEP) {
    err = "workload not built in this library";
    return MK_ERR_UNSUPPORTED;
  }
  const int H = c.hidden, I = c.inter, d = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int R = c.n_requests, P = c.page_size;
  if (W < 1 || H < 1 || I < 1 || d < 2 || Hq < 1 || Hkv < 1 || Hq % Hkv || c.num_layers < 1 || R < 1) {
    err = "invalid shape";
    return MK_ERR_INVALID;
  }
  if (c.tokens_per_request != 1) {
    err = "the decode-layer workloads take one new token per request";
    return MK_ERR_INVALID;
  }
  if (d != 128 || H % 8 || I % 8 || P < 4 || P % 4 || Hq / Hkv > 8) {
    err = "unsupported shape: head_dim must be 128, hidden/inter multiples of 8, page size a multiple of 4, GQA group <= 8";
    return MK_ERR_UNSUPPORTED;
  }
  if (c.workload == MK_QWEN3_STEP && c.vocab < 1) {
    err = "vocab must be positive";
    return MK_ERR_INVALID;
  }
  for (int r = 0; r < R; ++r) {
    if (ctx[r] < 1 || ctx[r] > c.max_pages_per_req * P) {
      err = "context length out of range of the block table";
      return MK_ERR_INVALID;
    }
  }
  out = HostPlan{};
  out.cfg = c;
  out.ctx.assign(ctx, ctx + R);
  out.W = W;
  TileParams& p = out.tp;
  if (!tile_params(c, W, ctx, p, err)) return MK_ERR_UNSUPPORTED;

  Builder b;
  const int g = Hq / Hkv;
  const int n_qkv = (Hq + 2 * Hkv) * d;
  const int rq = p.r_qkv, ro = p.r_o, rgu = p.r_gu, rd = p.r_down, st = p.s_tok;
  const int n_qkv_t = n_qkv / rq, n_o_t = H / ro, n_gu_t = I / rgu, n_d_t = H / rd;
  const uint32_t thr_grp = (uint32_t)((g + 2) * d / rq);
  int prev_down = -1, prev_down_row = -1;
  int max_splits = 0;
  if (p.spec == 1) {
    if (c.workload == MK_QWEN3_STEP) {
      err = "the full decode step is planned for one row (M = 1) only";
      return MK_ERR_UNSUPPORTED;
    }
    if ((Hq + 2 * Hkv) * d % kM16Rows || H % kM16Rows || I % (kM16Rows / 2) || H % p.kc || I % p.kc ||
        (Hq * d) % p.kc || R * c.tokens_per_request > kMaxRows) {
      err = "unsupported multi-row shape: projection sizes must be multiples of the 64-row tile and of the K chunk, "
            "and at most 256 rows";
      return MK_ERR_UNSUPPORTED;
    }
    build_m16(c, ctx, p, W, b, max_splits);
  }
  for (int l = 0; l < (p.spec == 0 ? c.num_layers : 0); ++l) {
    int row_qkv = b.op_row(OP_QKV, l, prev_down_row >= 0 ? std::vector<int>{prev_down_row} : std::vector<int>{});
    int row_attn = b.op_row(OP_ATTN, l, {row_qkv});
    int row_o = b.op_row(OP_OPROJ, l, {row_attn});
    int row_gu = b.op_row(OP_GATEUP, l, {row_o});
    int row_d = b.op_row(OP_DOWN, l, {row_gu});
    std::vector<int> ev_qkv(Hkv);
    for (int hk = 0; hk < Hkv; ++hk) ev_qkv[hk] = b.event(thr_grp);
    int ev_oready = b.event((uint32_t)(R * Hkv));
    int ev_o = b.event((uint32_t)n_o_t);
    int ev_gu = b.event((uint32_t)n_gu_t);
    int ev_down = b.event((uint32_t)n_d_t);
    for (int j = 0; j < n_qkv_t; ++j) {
      int n0 = j * rq, grp;
      if (n0 < Hq * d) grp = (n0 / d) / g;
      else if (n0 < (Hq + Hkv) * d) grp = (n0 - Hq * d) / d;
      else grp = (n0 - (Hq + Hkv) * d) / d;
      if (prev_down < 0)
        b.task(OP_QKV, row_qkv, p.spec, {}, {{ev_qkv[grp], 1u}}, {l, n0, rq, 0, H});
      else
        b.task(OP_QKV, row_qkv, p.spec, {{prev_down, (uint32_t)n_d_t}}, {{ev_qkv[grp], 1u}}, {l, n0, rq, 0, H});
    }
    int grp_id = 0;
    for (int r = 0; r < R; ++r) {
      int cx = ctx[r], ns = (cx + st - 1) / st;
      max_splits = std::max(max_splits, ns);
      for (int hk = 0; hk < Hkv; ++hk) {
        grp_id = b.n_arrivals++;
        for (int s = 0; s < ns; ++s) {
          int t0 = s * st, t1 = std::min(cx, (s + 1) * st);
          b.task(OP_ATTN, row_attn, p.spec, {{ev_qkv[hk], thr_grp}}, {{ev_oready, 1u}},
                 {l, r, hk, s, t0, t1, grp_id, ns, s});
        }
      }
    }
    for (int j = 0; j < n_o_t; ++j)
      b.task(OP_OPROJ, row_o, p.spec, {{ev_oready, (uint32_t)(R * Hkv)}}, {{ev_o, 1u}}, {l, j * ro, ro, 0, Hq * d});
    for (int j = 0; j < n_gu_t; ++j)
      b.task(OP_GATEUP, row_gu, p.spec, {{ev_o, (uint32_t)n_o_t}}, {{ev_gu, 1u}}, {l, j * rgu, rgu, 0, H});
    for (int j = 0; j < n_d_t; ++j)
      b.task(OP_DOWN, row_d, p.spec, {{ev_gu, (uint32_t)n_gu_t}}, {{ev_down, 1u}}, {l, j * rd, rd, 0, I});
    prev_down = ev_down;
    prev_down_row = row_d;
  }
  if (c.workload == MK_QWEN3_STEP) {
    int row_lm = b.op_row(OP_LMHEAD, c.num_layers, {prev_down_row});
    int rl = p.r_lm, n_lm = (c.vocab + rl - 1) / rl;
    int grp = b.n_arrivals++;
    // each worker keeps a running max over its lm_head tasks and publishes it with its last
    // one: the last min(W, n_lm) tasks publish, each into its own slot of the arrival group
    const int n_pub = std::min(W, n_lm);
    // task j takes rows j, j + n_lm, ... (the workers' rows interleaved)
    for (int j = 0; j < n_lm; ++j) {
      int64_t slot = j >= n_lm - n_pub ? (int64_t)(j - (n_lm - n_pub)) : (int64_t)kNone;
      b.task(OP_LMHEAD, row_lm, p.spec, {{prev_down, (uint32_t)n_d_t}}, {},
             {c.num_layers, j, (c.vocab - j + n_lm - 1) / n_lm, n_lm, H, 0, grp, n_pub, slot});
    }
  }
  if (pack_plan(b, W, max_splits, out, err) != MK_OK) return MK_ERR_INVALID;

  // workspace regions (256-byte aligned)
  size_t off = 0;
  const int M = R * c.tokens_per_request;
  auto region = [&](const char* name, size_t bytes) {
    out.regions.push_back({name, off, bytes});
    off += (bytes + 255) / 256 * 256;
  };
  if (p.spec == 1) {
    // multi-row: qkv as tagged records (the attention staging reads records), everything else
    // plain; projection inputs in the matrix-core operand order over 16 row slots
    const size_t el = c.act_fp8 ? 1 : 2;
    const size_t kc = (size_t)p.kc;
    const size_t G = (size_t)(M + 15) / 16, rows = 16 * G;  // 16-row groups of the operand order
    region("qkv", (size_t)M * n_qkv * 8);
    region("part", (size_t)R * Hkv * max_splits * (g * d + 8) * 4);
    region("qb", (size_t)M * Hq * d * 2);  // the attention's bf16 q heads, as materialised
    region("r1", (size_t)M * H * 4);
    region("r2", (size_t)M * H * 4);
    region("y", (size_t)M * H * 2);
    region("h1", rows * H * el);
    region("h2", rows * H * el);
    if (c.act_fp8) {  // attention output and m in fp32 rows, quantised per token into oq / mq
      region("o", (size_t)M * Hq * d * 4);
      region("m", (size_t)M * I * 4);
      region("oq", rows * Hq * d);
      region("mq", rows * I);
      for (const char* s : {"s1", "s2", "so", "sm"}) region(s, rows * 4);
    } else {
      region("o", rows * Hq * d * 2);
      region("m", rows * I * 2);
    }
    // fp32 partial sums of the projection tiles: [tile][K chunk][row group][16 x 64]
    region("gp_qkv", (size_t)(n_qkv / kM16Rows) * (H / kc) * G * 4096);
    region("gp_o", (size_t)(H / kM16Rows) * (Hq * d / kc) * G * 4096);
    region("gp_gu", (size_t)(I / (kM16Rows / 2)) * (H / kc) * G * 4096);
    region("gp_down", (size_t)(H / kM16Rows) * (I / kc) * G * 4096);
  } else {
    // vectors written inside a run are tagged 8-byte records: fp32 or a bf16 pair per record
    region("qkv", (size_t)M * n_qkv * 8);
    region("part", (size_t)R * Hkv * max_splits * (g * d + 8) * 4);  // per split: g*d O, g lse, padding (fp32)
    region("o", (size_t)M * Hq * d / 2 * 8);
    region("m", (size_t)M * I / 2 * 8);
    region("r2", (size_t)M * H * 8);
    region("r1", (size_t)M * H * 8);
  }
  if (c.workload == MK_QWEN3_STEP) region("lm_part", (size_t)((c.vocab + p.r_lm - 1) / p.r_lm) * 8);
  out.workspace_bytes = off;

  return check_events(out, err);
}

}  // namespace mk
