"""Host tile-instruction queue builder, re-implemented from the written queue rules.

Follows the lowering described on the MegaRTP page, section 4 ("OpGraph -> per-op
tile expansion -> TaskGraph -> KernelPlan -> instruction tensor + event counters +
operand pointer table"):

* each op expands into tile tasks (row tiles for norms, output-row tiles for the
  skinny projections, (request, kv head, KV split) tiles for attention);
* a (producer op, consumer op) pair turns into events: a counter plus a threshold
  equal to the number of producer tasks writing (or reducing into) the region the
  consumer reads ("whole", "tile_cover", "tile_reduce");
* tasks are numbered in topological order and dealt round-robin onto the worker
  queues, which are padded with NoOp to a common length [W, L, 32];
* each instruction is 32 uint32 words: opcode, wait count, signal count, operand
  row, spec id, task id, four (event, threshold) waits, two (event, increment,
  publication id) signals, then the tile payload.

Deadlock freedom (handbook, megakernel section and its exercise 3): every wait
names an event whose producers all have smaller task ids, and all workers are
co-resident, so the smallest unfinished task can always run.

Reductions whose result a consumer reads once (the split-KV combine, the global
argmax) use an arrival group instead of an extra wave of finalize tasks: each
producer records its arrival; the one that completes the group finalises and then
issues the instruction's signals.  The arrival group id, its size and the
producer's rank in it are part of the payload.
"""
from __future__ import annotations

from typing import Dict, List

import numpy as np

OP_NOOP, OP_QKV, OP_ATTN, OP_OPROJ, OP_GATEUP, OP_DOWN, OP_LMHEAD = 0, 1, 2, 3, 4, 5, 6
# multi-row (M = 16) plans: per-row norms, projection tiles over K chunks with explicit finalize
# tasks, per-row FP8 quantisation of the O and down inputs
OP_NORM, OP_GEMM, OP_FIN, OP_QUANT = 7, 8, 9, 10
OP_COMB = 11  # multi-row: combine the split-KV partials of one (request, kv head)
# indexer front
OP_KCACHE, OP_SCORE = 12, 13  # key RoPE + per-token e4m3 + cache write; paged indexer score
OP_TOPK = 14  # one token row: the positions of its top-k scores
K_QA, K_W, K_KI, K_QI = 4, 5, 6, 7  # projection kinds: q_a, head weights, indexer key, indexer q
K_QB, K_UK = 8, 9  # main-MLA query (D0, finalized per head) and query BMM (D2, one chunk)
MLA_NOPE, MLA_LATENT = 128, 512  # per main-MLA head: D0 output, D2 output
SCORE_TOK = 128  # keys per indexer-score task
K_QKV, K_O, K_GU, K_DOWN = 0, 1, 2, 3  # projection kinds
NONE = 0xFFFFFFFF
LEASE_BYTES = 65536  # largest LDS lease of one instruction
M16_ROWS = 64        # weight rows of one multi-row projection tile (gate/up: 32 gate + 32 up)


def _pow2floor(x: int) -> int:
    p = 1
    while p * 2 <= x:
        p *= 2
    return p


def _pow2ceil(x: int) -> int:
    p = 1
    while p < x:
        p *= 2
    return p


def _largest_divisor_le(n: int, cap: int) -> int:
    cap = max(1, min(n, cap))
    for r in range(cap, 0, -1):
        if n % r == 0:
            return r
    return 1


def kchunk(K: int) -> int:
    """K chunk of an e4m3 projection tile: the largest multiple of 128 that divides K and keeps
    M16_ROWS rows within one lease (1024)."""
    for kc in range(LEASE_BYTES // M16_ROWS, 0, -128):
        if K % kc == 0:
            return kc
    raise ValueError(K)


def tile_params(cfg, W: int, ctx_lens) -> Dict[str, int]:
    if cfg.workload == "indexer_front":
        return {"spec": 1, "kc": kchunk(cfg.hidden), "kc_q": kchunk(cfg.idx_q_rank), "s_tok": SCORE_TOK}
    H, I, d = cfg.hidden, cfg.inter, cfg.head_dim
    Hq, Hkv = cfg.n_q_heads, cfg.n_kv_heads
    R = cfg.n_requests
    elem = 1 if cfg.weight_fp8 else 2
    n_qkv = (Hq + 2 * Hkv) * d

    # rows of one tile: the LDS lease (weights, plus the 1 KiB-rounded norm gain of the fused
    # add + RMSNorm ops) stays within LEASE_BYTES
    gain = -(-2 * H // 1024) * 1024

    def cap_rows(k: int, nmat: int, extra: int) -> int:
        return max(1, (LEASE_BYTES - extra) // (k * elem * nmat))

    p = {}
    p["r_qkv"] = _pow2floor(min(d, max(1, n_qkv // W), cap_rows(H, 1, gain)))
    p["r_o"] = _largest_divisor_le(H, min(max(1, H // W), cap_rows(Hq * d, 1, 0)))
    p["r_gu"] = _largest_divisor_le(I, min(max(1, I // W), cap_rows(H, 2, gain + 1024)))
    p["r_down"] = _largest_divisor_le(H, min(max(1, H // W), cap_rows(I, 1, 0)))
    p["r_lm"] = -(-cfg.vocab // W) if cfg.workload == "qwen3_step" else 0  # one lm_head task per worker
    ctx_max = int(max(ctx_lens))
    want = -(-(2 * R * ctx_max * Hkv) // W)  # about W/2 attention tasks
    p["s_tok"] = max(4, min(LEASE_BYTES // (4 * d), _pow2ceil(max(1, want))))
    p["spec"] = 0 if cfg.m == 1 else 1
    # multi-row projection tiles: M16_ROWS weight rows x kc columns fill one lease
    p["kc"] = LEASE_BYTES // (M16_ROWS * elem) if p["spec"] == 1 else 0
    # tile sizes the caller fixed (mk_config.tile_params; 0 keeps the rule above).  The library
    # refuses values its op bodies cannot run; this builder only takes them over.
    tp = tuple(getattr(cfg, "tile_params", ()) or ()) + (0,) * 8
    for key, idx in (("r_qkv", 0), ("r_o", 1), ("r_gu", 2), ("r_down", 3), ("r_lm", 4), ("s_tok", 5)):
        if tp[idx]:
            p[key] = int(tp[idx])
    return p


class _Builder:
    def __init__(self):
        self.tasks: List[np.ndarray] = []
        self.thresholds: List[int] = []
        self.n_arrivals = 0
        self.n_ops = 0

    def event(self, threshold: int) -> int:
        self.thresholds.append(int(threshold))
        return len(self.thresholds) - 1

    def arrival_group(self) -> int:
        self.n_arrivals += 1
        return self.n_arrivals - 1

    def op_row(self) -> int:
        self.n_ops += 1
        return self.n_ops - 1

    def task(self, opcode, op_row, spec, waits, signals, payload) -> int:
        tid = len(self.tasks)
        w = np.zeros(32, dtype=np.uint32)
        w[0], w[1], w[2], w[3], w[4], w[5] = opcode, len(waits), len(signals), op_row, spec, tid
        assert len(waits) <= 4 and len(signals) <= 2 and len(payload) <= 12
        for i, (e, t) in enumerate(waits):
            w[6 + 2 * i], w[7 + 2 * i] = e, t
        for i, (e, inc) in enumerate(signals):
            w[14 + 3 * i], w[15 + 3 * i], w[16 + 3 * i] = e, inc, tid
        for i, v in enumerate(payload):
            w[20 + i] = np.uint32(v & 0xFFFFFFFF)
        self.tasks.append(w)
        return tid


def _qwen3(cfg, W: int, ctx_lens, b: _Builder, p) -> None:
    H, I, d = cfg.hidden, cfg.inter, cfg.head_dim
    Hq, Hkv = cfg.n_q_heads, cfg.n_kv_heads
    g = Hq // Hkv
    R = cfg.n_requests
    spec = p["spec"]
    n_qkv = (Hq + 2 * Hkv) * d
    rq, ro, rgu, rd, st = p["r_qkv"], p["r_o"], p["r_gu"], p["r_down"], p["s_tok"]
    n_qkv_t, n_o_t, n_gu_t, n_d_t = n_qkv // rq, H // ro, I // rgu, H // rd
    prev_down = None
    for l in range(cfg.num_layers):
        row_qkv, row_attn, row_o, row_gu, row_d = (b.op_row() for _ in range(5))
        ev_qkv = [b.event((g + 2) * d // rq) for _ in range(Hkv)]
        ev_oready = b.event(R * Hkv)
        ev_o = b.event(n_o_t)
        ev_gu = b.event(n_gu_t)
        ev_down = b.event(n_d_t)
        # QKV row tiles; a tile lies inside one head, whose kv group is its event
        for j in range(n_qkv_t):
            n0 = j * rq
            if n0 < Hq * d:
                grp = (n0 // d) // g
            elif n0 < (Hq + Hkv) * d:
                grp = (n0 - Hq * d) // d
            else:
                grp = (n0 - (Hq + Hkv) * d) // d
            waits = [] if prev_down is None else [(prev_down, n_d_t)]
            b.task(OP_QKV, row_qkv, spec, waits, [(ev_qkv[grp], 1)], [l, n0, rq, 0, H])
        # split-KV attention tiles: (request, kv head, split); arrival group per (request, kv head)
        for r in range(R):
            ctx = int(ctx_lens[r])
            ns = -(-ctx // st)
            for hk in range(Hkv):
                grp = b.arrival_group()
                for s in range(ns):
                    t0, t1 = s * st, min(ctx, (s + 1) * st)
                    b.task(OP_ATTN, row_attn, spec, [(ev_qkv[hk], (g + 2) * d // rq)], [(ev_oready, 1)],
                           [l, r, hk, s, t0, t1, grp, ns, s])
        for j in range(n_o_t):
            b.task(OP_OPROJ, row_o, spec, [(ev_oready, R * Hkv)], [(ev_o, 1)], [l, j * ro, ro, 0, Hq * d])
        for j in range(n_gu_t):
            b.task(OP_GATEUP, row_gu, spec, [(ev_o, n_o_t)], [(ev_gu, 1)], [l, j * rgu, rgu, 0, H])
        for j in range(n_d_t):
            b.task(OP_DOWN, row_d, spec, [(ev_gu, n_gu_t)], [(ev_down, 1)], [l, j * rd, rd, 0, I])
        prev_down = ev_down
    if cfg.workload == "qwen3_step":
        row_lm = b.op_row()
        rl = p["r_lm"]
        n_lm = -(-cfg.vocab // rl)
        grp = b.arrival_group()
        # a worker keeps a running max over its lm_head tasks and publishes it with its last
        # one: the last min(W, n_lm) tasks publish, each into its own slot of the group
        n_pub = min(W, n_lm)
        for j in range(n_lm):  # task j takes rows j, j + n_lm, ... (interleaved)
            slot = j - (n_lm - n_pub) if j >= n_lm - n_pub else NONE
            b.task(OP_LMHEAD, row_lm, spec, [(prev_down, n_d_t)], [],
                   [cfg.num_layers, j, -(-(cfg.vocab - j) // n_lm), n_lm, H, 0, grp, n_pub, slot])


def _qwen3_m16(cfg, W: int, ctx_lens, b: _Builder, p) -> None:
    """Multi-row (M = R x T rows, M <= 256) layer: row-task norms, projections as
    (output-row tile, K chunk) tasks writing partial sums for every 16-row group of M (one read
    of the weights), one finalize task per (row tile, row group) that adds the chunks in K order
    and applies the epilogue; FP8 plans quantise o and m per row.

    Waits (all "whole" unless stated): NORM_A of a row on the previous layer's down finalizes of
    its row group; QKV tiles on NORM_A; QKV finalize on its tile's chunks ("tile_reduce");
    attention on the QKV finalizes of its kv group and row group ("tile_cover"); a combine on its
    group's chain partials ("tile_reduce"); [QUANT_O on every combine]; O tiles on the combines
    [or QUANT_O]; NORM_B of a row on its row group's O finalizes; gate/up tiles on NORM_B;
    [QUANT_M of a row on its row group's gate/up finalizes]; down tiles on the gate/up finalizes
    [or QUANT_M]."""
    H, I, d = cfg.hidden, cfg.inter, cfg.head_dim
    Hq, Hkv = cfg.n_q_heads, cfg.n_kv_heads
    g = Hq // Hkv
    R, M, T = cfg.n_requests, cfg.m, cfg.tokens_per_request
    G = -(-M // 16)  # 16-row groups
    spec, kc, st = p["spec"], p["kc"], p["s_tok"]
    n_qkv = (Hq + 2 * Hkv) * d
    fp8 = bool(cfg.act_fp8)
    rt = M16_ROWS

    def proj(kind, l, N, K, rows, wait, fin_signal):
        row_g, row_f = b.op_row(), b.op_row()
        nt, nk = N // rows, K // kc
        parts = [b.event(nk) for _ in range(nt)]
        for j in range(nt):
            for c in range(nk):
                b.task(OP_GEMM, row_g, spec, [wait], [(parts[j], 1)], [l, kind, j, j * rows, rows, c * kc, kc])
        for j in range(nt):
            for gi in range(G):
                b.task(OP_FIN, row_f, spec, [(parts[j], nk)], [fin_signal(j, gi)],
                       [l, kind, j, j * rows, rows, nk, kc, 0, 0, gi])  # the group in word 29

    prev = None  # per row group: the previous layer's down finalizes
    for l in range(cfg.num_layers):
        row_na = b.op_row()
        ev_na = b.event(M)
        for m in range(M):
            b.task(OP_NORM, row_na, spec, [] if prev is None else [prev[m // 16]], [(ev_na, 1)], [l, 0, m])
        # QKV: a 64-row tile lies inside one head; its finalize of a row group counts for the
        # head's kv group and that row group
        tiles_per_group = (g + 2) * d // rt
        ev_qkv = [b.event(tiles_per_group) for _ in range(Hkv * G)]

        def qkv_group(j):
            n0 = j * rt
            if n0 < Hq * d:
                return (n0 // d) // g
            if n0 < (Hq + Hkv) * d:
                return (n0 - Hq * d) // d
            return (n0 - (Hq + Hkv) * d) // d

        proj(K_QKV, l, n_qkv, H, rt, (ev_na, M), lambda j, gi: (ev_qkv[qkv_group(j) * G + gi], 1))
        # split-KV attention: the (request, kv head, split) tasks are laid out so that dealing them
        # round-robin hands each worker a run of consecutive splits of one (request, kv head) -- a
        # chain, which the worker folds into one running softmax state and writes as one partial.
        # The splits, pair after pair, fill the columns 0 .. C-1 of the op's rounds of C tasks
        # (C = min(W, tasks); a column is one worker's share, longer columns first); a chain is a
        # column's maximal run inside one pair.  One event per pair counts its chains; one
        # combine task per pair reduces their partials.
        row_attn = b.op_row()
        nsplit = [-(-int(ctx_lens[r]) // st) for r in range(R)]
        seq = [(r, hk, s) for r in range(R) for hk in range(Hkv) for s in range(nsplit[r])]
        n = len(seq)
        C = min(W, n)
        rounds = -(-n // C)
        full = n - (rounds - 1) * C
        lens = [rounds if j < full else rounds - 1 for j in range(C)]
        starts = [sum(lens[:j]) for j in range(C)]
        nchain = [0] * (R * Hkv)
        chain = {}  # seq index -> (flags, slot): bit 0 continues the column's previous task, bit 1 ends a chain
        for j in range(C):
            for k in range(lens[j]):
                i = starts[j] + k
                pair = seq[i][0] * Hkv + seq[i][1]
                cont = k > 0 and seq[i - 1][:2] == seq[i][:2]
                end = k == lens[j] - 1 or seq[i + 1][:2] != seq[i][:2]
                if not cont:
                    nchain[pair] += 1
                chain[i] = (int(cont) | int(end) << 1, nchain[pair] - 1)
        ev_att = [b.event(nchain[pair]) for pair in range(R * Hkv)]
        for k in range(rounds):
            for j in range(C):
                if k >= lens[j]:
                    continue
                i = starts[j] + k
                r, hk, s = seq[i]
                flags, slot = chain[i]
                t0, t1 = s * st, min(int(ctx_lens[r]), (s + 1) * st)
                b.task(OP_ATTN, row_attn, spec, [(ev_qkv[hk * G + r * T // 16], tiles_per_group)],
                       [(ev_att[r * Hkv + hk], 1)] if flags & 2 else [],
                       [l, r, hk, s, t0, t1, 0, 0, 0, nsplit[r], flags, slot])
        row_comb = b.op_row()
        ev_oready = b.event(R * Hkv)
        for r in range(R):
            for hk in range(Hkv):
                b.task(OP_COMB, row_comb, spec, [(ev_att[r * Hkv + hk], nchain[r * Hkv + hk])], [(ev_oready, 1)],
                       [l, r, hk, nchain[r * Hkv + hk]])
        o_wait = (ev_oready, R * Hkv)
        if fp8:
            row_qo = b.op_row()
            ev_oq = b.event(M)
            for m in range(M):
                b.task(OP_QUANT, row_qo, spec, [o_wait], [(ev_oq, 1)], [l, 0, m])
            o_wait = (ev_oq, M)
        ev_o = [b.event(H // rt) for _ in range(G)]
        proj(K_O, l, H, Hq * d, rt, o_wait, lambda j, gi: (ev_o[gi], 1))
        row_nb = b.op_row()
        ev_nb = b.event(M)
        for m in range(M):
            b.task(OP_NORM, row_nb, spec, [(ev_o[m // 16], H // rt)], [(ev_nb, 1)], [l, 1, m])
        # gate/up: a tile holds rt/2 gate rows and the matching rt/2 up rows.  W8A8: the per-row
        # quantisation waits for its row group's finalizes; bf16: the down tiles read every group
        n_gu = I // (rt // 2)
        ev_gu = [b.event(n_gu) for _ in range(G)] if fp8 else [b.event(n_gu * G)]
        proj(K_GU, l, I, H, rt // 2, (ev_nb, M), lambda j, gi: (ev_gu[gi if fp8 else 0], 1))
        m_wait = (ev_gu[0], n_gu * G)
        if fp8:
            row_qm = b.op_row()
            ev_mq = b.event(M)
            for m in range(M):
                b.task(OP_QUANT, row_qm, spec, [(ev_gu[m // 16], n_gu)], [(ev_mq, 1)], [l, 1, m])
            m_wait = (ev_mq, M)
        ev_down = [b.event(H // rt) for _ in range(G)]
        proj(K_DOWN, l, H, I, rt, m_wait, lambda j, gi: (ev_down[gi], 1))
        prev = [(e, H // rt) for e in ev_down]


def _indexer(cfg, W: int, ctx_lens, b: _Builder, p) -> None:
    """Indexer front (MegaRTP page, section 4: A0 -> {B0, C0, B1}; {B0, C0} -> D1; {D1, B1} -> E1):
      A0: one NORM row task per token (add + RMSNorm + per-token e4m3)
      B0 / C0 / B1: e4m3 projection tiles of 64 weight rows x one K chunk, finalize per tile
        (B0 -> q_a rows, C0 -> head weights, B1 -> key rows); B0's rows then get a NORM row task
        each (RMSNorm of q_a + per-token e4m3); B1's finalizes feed one key-cache task (RoPE,
        per-token e4m3, cache write)
      D1: projection tiles of q_a; one finalize per head (its two 64-row tiles, so that RoPE pairs
        dimensions i and i + 64)
      E1: one score task per (request, SCORE_TOK keys)
      top-k (when cfg.topk > 0): one task per token row
      D0 / D2 (when cfg.mla_heads > 0): D0 projection tiles (as D1) with a finalize per head, then
        per head 8 tiles of 64 latent rows of D2 over that head's 128 columns
    Waits: B0 / C0 / B1 tiles on A0 ("tile_cover"); finalizes on their tiles' chunks
    ("tile_reduce"); the q_a norms on B0's finalizes; D1 tiles on the q_a norms; the key-cache
    task on B1's finalizes; E1 on D1's finalizes, C0's finalize and the key-cache task; a top-k
    task on every score task of its request ("whole" per request); D0 tiles on the q_a norms, a
    D0 finalize on its head's tiles, D2 tiles on their head's finalize ("tile_cover" per head)."""
    H, qr, nh, hd = cfg.hidden, cfg.idx_q_rank, cfg.idx_heads, cfg.idx_head_dim
    R, T = cfg.n_requests, cfg.tokens_per_request
    M = R * T
    spec, rt, st = p["spec"], M16_ROWS, p["s_tok"]
    l = 0

    def tiles(kind, N, K, kc, wait, part_event):
        row_g = b.op_row()
        nt, nk = N // rt, K // kc
        for j in range(nt):
            for c in range(nk):
                b.task(OP_GEMM, row_g, spec, [wait], [(part_event(j), 1)], [l, kind, j, j * rt, rt, c * kc, kc])
        return nt, nk

    def fin(kind, nt, nk, kc, parts, fin_event):
        row_f = b.op_row()
        for j in range(nt):
            b.task(OP_FIN, row_f, spec, [(parts[j], nk)], [(fin_event, 1)], [l, kind, j, j * rt, rt, nk, kc])

    row_a0 = b.op_row()
    ev_a0 = b.event(M)
    for m in range(M):
        b.task(OP_NORM, row_a0, spec, [], [(ev_a0, 1)], [l, 0, m])
    kc = p["kc"]
    # B0: q_a, then its per-token RMSNorm + quantisation
    nt, nk = qr // rt, H // kc
    parts = [b.event(nk) for _ in range(nt)]
    tiles(K_QA, qr, H, kc, (ev_a0, M), lambda j: parts[j])
    ev_b0 = b.event(nt)
    fin(K_QA, nt, nk, kc, parts, ev_b0)
    row_qn = b.op_row()
    ev_qn = b.event(M)
    for m in range(M):
        b.task(OP_NORM, row_qn, spec, [(ev_b0, nt)], [(ev_qn, 1)], [l, 2, m])
    # C0: head weights
    nt_w = nh // rt
    parts_w = [b.event(nk) for _ in range(nt_w)]
    tiles(K_W, nh, H, kc, (ev_a0, M), lambda j: parts_w[j])
    ev_w = b.event(nt_w)
    fin(K_W, nt_w, nk, kc, parts_w, ev_w)
    # B1: indexer key, then RoPE + quantisation + cache write
    nt_k = hd // rt
    parts_k = [b.event(nk) for _ in range(nt_k)]
    tiles(K_KI, hd, H, kc, (ev_a0, M), lambda j: parts_k[j])
    ev_k = b.event(nt_k)
    fin(K_KI, nt_k, nk, kc, parts_k, ev_k)
    row_kc = b.op_row()
    ev_kc = b.event(1)
    b.task(OP_KCACHE, row_kc, spec, [(ev_k, nt_k)], [(ev_kc, 1)], [l])
    # D1: indexer q per head (two tiles each)
    kcq = p["kc_q"]
    nk_q = qr // kcq
    per_head = hd // rt
    ev_head = [b.event(per_head * nk_q) for _ in range(nh)]
    tiles(K_QI, nh * hd, qr, kcq, (ev_qn, M), lambda j: ev_head[j // per_head])
    row_f = b.op_row()
    ev_qi = b.event(nh)
    for h in range(nh):
        b.task(OP_FIN, row_f, spec, [(ev_head[h], per_head * nk_q)], [(ev_qi, 1)],
               [l, K_QI, h, h * hd, hd, nk_q, kcq])
    # main-MLA query half, dealt after D1 and before E1 as in the page's tile list: D0 tiles over the
    # normalised q_a (as D1), one finalize per head, then D2's tiles of a head once that head is
    # finalized (an event per head: the page's per-head tile_cover of D0 -> D2)
    nm = getattr(cfg, "mla_heads", 0)
    if nm:
        per_head_qb = MLA_NOPE // rt
        ev_qb = [b.event(per_head_qb * nk_q) for _ in range(nm)]
        tiles(K_QB, nm * MLA_NOPE, qr, kcq, (ev_qn, M), lambda j: ev_qb[j // per_head_qb])
        row_d0f = b.op_row()
        ev_qn_h = [b.event(1) for _ in range(nm)]
        for h in range(nm):
            b.task(OP_FIN, row_d0f, spec, [(ev_qb[h], per_head_qb * nk_q)], [(ev_qn_h[h], 1)],
                   [l, K_QB, h, h * MLA_NOPE, MLA_NOPE, nk_q, kcq])
        row_d2 = b.op_row()
        for h in range(nm):
            for j in range(MLA_LATENT // rt):
                b.task(OP_GEMM, row_d2, spec, [(ev_qn_h[h], 1)], [],
                       [l, K_UK, h * (MLA_LATENT // rt) + j, h * MLA_LATENT + j * rt, rt, 0, MLA_NOPE, h * MLA_NOPE])
    # E1: scores; with a top-k, one event per request counts its score tasks
    row_e = b.op_row()
    nsc = [-(-int(ctx_lens[r]) // st) for r in range(R)]
    ev_e1 = [b.event(nsc[r]) for r in range(R)] if cfg.topk else []
    for r in range(R):
        ctx = int(ctx_lens[r])
        for s in range(nsc[r]):
            b.task(OP_SCORE, row_e, spec, [(ev_qi, nh), (ev_w, nt_w), (ev_kc, 1)], [(ev_e1[r], 1)] if cfg.topk else [],
                   [l, r, s, s * st, min(ctx, (s + 1) * st)])
    # top-k: one task per token row, after every score task of its request
    if cfg.topk:
        row_tk = b.op_row()
        for m in range(M):
            b.task(OP_TOPK, row_tk, spec, [(ev_e1[m // T], nsc[m // T])], [], [l, m])


def build_queue(cfg, W: int, ctx_lens=None) -> Dict[str, np.ndarray]:
    """Returns {'queue': uint32 [W, L, 32], 'thresholds': uint32 [E], 'n_tasks', 'n_ops',
    'n_arrivals', 'params'}."""
    if ctx_lens is None:
        ctx_lens = [cfg.context] * cfg.n_requests
    b = _Builder()
    p = tile_params(cfg, W, ctx_lens)
    if cfg.workload == "indexer_front":
        _indexer(cfg, W, ctx_lens, b, p)
    elif cfg.workload in ("qwen3_layer", "qwen3_step") and p["spec"] == 1:
        if cfg.workload == "qwen3_step":
            raise NotImplementedError("multi-row decode step")
        _qwen3_m16(cfg, W, ctx_lens, b, p)
    elif cfg.workload in ("qwen3_layer", "qwen3_step"):
        _qwen3(cfg, W, ctx_lens, b, p)
    else:
        raise NotImplementedError(cfg.workload)
    T = len(b.tasks)
    L = -(-T // W)
    q = np.zeros((W, L, 32), dtype=np.uint32)
    for tid, words in enumerate(b.tasks):
        q[tid % W, tid // W] = words
    return {"queue": q, "thresholds": np.array(b.thresholds, dtype=np.uint32), "n_tasks": T,
            "n_ops": b.n_ops, "n_arrivals": b.n_arrivals, "params": p}


def check_invariants(plan) -> None:
    """Every task appears once; waits name events whose producers all precede the waiter;
    each event's threshold equals the increments its producers issue per run."""
    q = plan["queue"]
    W, L, _ = q.shape
    thr = plan["thresholds"]
    produced = np.zeros(len(thr), dtype=np.int64)
    last_producer = np.full(len(thr), -1, dtype=np.int64)
    tasks = {}
    for w in range(W):
        for i in range(L):
            words = q[w, i]
            if words[0] == OP_NOOP:
                assert not words.any()
                continue
            tid = int(words[5])
            assert tid not in tasks and tid % W == w and tid // W == i
            tasks[tid] = words
    assert sorted(tasks) == list(range(plan["n_tasks"]))
    for tid in range(plan["n_tasks"]):
        words = tasks[tid]
        for k in range(int(words[1])):
            e, t = int(words[6 + 2 * k]), int(words[7 + 2 * k])
            assert t == thr[e] and last_producer[e] < tid
        for k in range(int(words[2])):
            e, inc = int(words[14 + 3 * k]), int(words[15 + 3 * k])
            arrival_total = int(words[27])
            # a finalised signal is issued once per arrival group, by its last producer
            if arrival_total:
                if int(words[28]) == arrival_total - 1:
                    produced[e] += inc
            else:
                produced[e] += inc
            last_producer[e] = tid
    assert np.array_equal(produced, thr.astype(np.int64)), "threshold != increments"
