"""Instruction tensor: an independent builder, a validator and a simulator.

The persistent-kernel idea this serves: one kernel occupies the whole GPU and
each block reads a host-built instruction tensor to decide its next work
(Kittens VM summary, "Method"); the blocks get "a schedule of every operation
in the forward pass" and synchronise on the device (Hyperkernel teardown,
"What a megakernel buys").  The pages fix no format, tiling or assignment, so
the tensor below is this project's own specification ("schedule spec v4",
also written out in the design notes); the GPU library's C++ builder must
produce the same bytes.

Spec v4 (all int32):

* a launch decodes B sequences together (batch B >= 1): every row-tiled
  instruction computes its rows for all B, attention and its reduction are
  per sequence.

* stage order per token: for each layer ``QKV, ATTN, [AREDUCE if n_chunks > 1],
  OPROJ, UPGATE|MOE_UPGATE, DOWN|MOE_DOWN``; then ``LMHEAD``.
* a row-tiled stage over R rows has ``n = min(n_wg, R)`` tiles; tile i covers
  rows ``[i*R//n, (i+1)*R//n)``.  R: QKV = qd + 2 kvd, OPROJ = DOWN =
  MOE_DOWN = d, UPGATE = F, MOE_UPGATE = top_k * F, LMHEAD = V.
* ATTN: with one chunk, one instruction per q head (a = q head, b = 0); with
  several, one per (kv head, chunk) serving the kv head's q heads together
  (a = kv head, b = chunk), and AREDUCE has hq (a = q head) merging them.
  Each of these is repeated for every sequence: instruction i of the stage
  serves sequence ``i // n`` (n = instructions per sequence) with the operands
  of instruction ``i % n`` above, and names the sequence in word 10.
* instruction i of a stage goes to block ``(offset + i) % n_wg``; a block's
  list is the concatenation of its instructions in stage order.  The offset
  is 0 except for OPROJ: its tiles skip the blocks that ran the stage just
  before it (ATTN, or AREDUCE when n_chunks > 1), whose O-projection would
  otherwise start late and hold up the whole stage -- when there are more
  blocks than that, OPROJ has ``min(d, n_wg - E)`` tiles at offset E, E being
  the preceding stage's instruction count.
* words: header[16] = {magic, version, n_wg, n_stages, max_instr, n_chunks, L,
  d, hq, hkv, hd, F, V, E, top_k, B}; counts[n_wg]; then
  ``[n_wg][max_instr][16]`` with instruction = {opcode, layer, stage, index,
  a, b, wait_stage, wait_count, wait_prev_token, signal_stage, sequence, 0...};
  ``a, b`` = row range (row-tiled stages), as above for ATTN and AREDUCE;
  ``wait_stage`` is the stage whose outputs the instruction reads (QKV of
  layer 0 reads the previous token's LMHEAD: wait_prev_token = 1); LMHEAD's
  layer field is L.  Unused slots are zero.

Parity pins: tests check the validator invariants (every row of every stage
produced exactly once, waits name the producing stage and its size, lists in
stage order) and the simulator (no deadlock and no overwrite of a value that
a pending instruction still needs, over random interleavings).
"""
from __future__ import annotations

import random
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

MAGIC = 0x314B444D
VERSION = 4
WORDS = 16

OP_QKV, OP_ATTN, OP_AREDUCE, OP_OPROJ, OP_UPGATE, OP_DOWN, OP_MOE_UPGATE, OP_MOE_DOWN, OP_LMHEAD = range(1, 10)
OP_NAMES = {OP_QKV: "QKV", OP_ATTN: "ATTN", OP_AREDUCE: "AREDUCE", OP_OPROJ: "OPROJ",
            OP_UPGATE: "UPGATE", OP_DOWN: "DOWN", OP_MOE_UPGATE: "MOE_UPGATE",
            OP_MOE_DOWN: "MOE_DOWN", OP_LMHEAD: "LMHEAD"}
# stages whose instructions are row tiles
TILED_OPS = (OP_QKV, OP_OPROJ, OP_UPGATE, OP_DOWN, OP_MOE_UPGATE, OP_MOE_DOWN, OP_LMHEAD)


def stages(cfg, n_chunks: int, batch: int = 1) -> List[Tuple[int, int, int]]:
    """(opcode, layer, rows-or-count) for every stage of one token, in order."""
    out = []
    qkv_rows = cfg.qd + 2 * cfg.kvd
    for l in range(cfg.n_layers):
        out.append((OP_QKV, l, qkv_rows))
        out.append((OP_ATTN, l, batch * (cfg.n_q_heads if n_chunks == 1 else cfg.n_kv_heads * n_chunks)))
        if n_chunks > 1:
            out.append((OP_AREDUCE, l, batch * cfg.n_q_heads))
        out.append((OP_OPROJ, l, cfg.d_model))
        if cfg.is_moe:
            out.append((OP_MOE_UPGATE, l, cfg.top_k * cfg.d_ff))
            out.append((OP_MOE_DOWN, l, cfg.d_model))
        else:
            out.append((OP_UPGATE, l, cfg.d_ff))
            out.append((OP_DOWN, l, cfg.d_model))
    out.append((OP_LMHEAD, cfg.n_layers, cfg.vocab))
    return out


def placement(st: List[Tuple[int, int, int]], s: int, n_wg: int) -> Tuple[int, int]:
    """(blocks available, first block) for stage s."""
    op = st[s][0]
    if op == OP_OPROJ:
        prev_count = st[s - 1][2]          # ATTN or AREDUCE instruction count
        if n_wg > prev_count:
            return n_wg - prev_count, prev_count
    return n_wg, 0


def stage_instructions(op: int, layer: int, size: int, n_wg: int, n_chunks: int,
                       batch: int = 1) -> List[Tuple[int, int, int]]:
    """The (a, b, sequence) operands of one stage's instructions, by index;
    ``n_wg`` is the number of blocks the stage may use."""
    if op in TILED_OPS:
        n = min(n_wg, size)
        return [(i * size // n, (i + 1) * size // n, 0) for i in range(n)]
    per = size // batch
    if op == OP_ATTN:
        if n_chunks == 1:
            return [(i % per, 0, i // per) for i in range(size)]
        return [((i % per) // n_chunks, (i % per) % n_chunks, i // per) for i in range(size)]
    if op == OP_AREDUCE:
        return [(i % per, 0, i // per) for i in range(size)]
    raise ValueError(op)


def build(cfg, n_wg: int, n_chunks: int, batch: int = 1) -> np.ndarray:
    """Instruction tensor (int32 words) for ``cfg`` on ``n_wg`` blocks,
    decoding ``batch`` sequences together."""
    if n_wg < 1 or n_chunks < 1 or batch < 1:
        raise ValueError("n_wg, n_chunks and batch must be >= 1")
    st = stages(cfg, n_chunks, batch)
    n_st = len(st)
    lists: List[List[List[int]]] = [[] for _ in range(n_wg)]
    places = [placement(st, s, n_wg) for s in range(n_st)]
    counts_per_stage = [len(stage_instructions(op, l, sz, places[s][0], n_chunks, batch))
                        for s, (op, l, sz) in enumerate(st)]
    for s, (op, l, sz) in enumerate(st):
        if s == 0:
            wait_stage, wait_prev = n_st - 1, 1
        else:
            wait_stage, wait_prev = s - 1, 0
        avail, first = places[s]
        for i, (a, b, seq) in enumerate(stage_instructions(op, l, sz, avail, n_chunks, batch)):
            words = [op, l, s, i, a, b, wait_stage, counts_per_stage[wait_stage], wait_prev, s, seq]
            words += [0] * (WORDS - len(words))
            lists[(first + i) % n_wg].append(words)
    max_instr = max(len(x) for x in lists)
    hdr = [MAGIC, VERSION, n_wg, n_st, max_instr, n_chunks, cfg.n_layers, cfg.d_model,
           cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_ff, cfg.vocab,
           cfg.n_experts, cfg.top_k, batch]
    body = np.zeros((n_wg, max_instr, WORDS), dtype=np.int32)
    for w, lst in enumerate(lists):
        if lst:
            body[w, :len(lst)] = np.asarray(lst, dtype=np.int32)
    counts = np.array([len(x) for x in lists], dtype=np.int32)
    return np.concatenate([np.asarray(hdr, dtype=np.int32), counts, body.reshape(-1)])


def parse(words: np.ndarray) -> Tuple[List[int], List[List[List[int]]]]:
    words = np.asarray(words, dtype=np.int32)
    hdr = [int(x) for x in words[:WORDS]]
    n_wg, max_instr = hdr[2], hdr[4]
    counts = [int(x) for x in words[WORDS:WORDS + n_wg]]
    body = words[WORDS + n_wg:].reshape(n_wg, max_instr, WORDS)
    lists = [[[int(v) for v in body[w, j]] for j in range(counts[w])] for w in range(n_wg)]
    return hdr, lists


def validate(words: np.ndarray, cfg) -> None:
    """Raise ValueError unless the tensor satisfies the spec's invariants."""
    hdr, lists = parse(words)
    if hdr[0] != MAGIC or hdr[1] != VERSION:
        raise ValueError("bad magic/version")
    n_wg, n_st, max_instr, n_chunks, batch = hdr[2], hdr[3], hdr[4], hdr[5], hdr[15]
    if batch < 1:
        raise ValueError("batch")
    st = stages(cfg, n_chunks, batch)
    if n_st != len(st):
        raise ValueError("stage count")
    seen: Dict[int, List[Tuple[int, int, int, int]]] = {s: [] for s in range(n_st)}
    for w, lst in enumerate(lists):
        prev = -1
        for ins in lst:
            op, l, s, i, a, b, ws, wc, wp, sig, seq = ins[:11]
            if any(ins[11:]):
                raise ValueError("reserved words")
            if not (0 <= s < n_st) or st[s][0] != op or st[s][1] != l:
                raise ValueError(f"wg {w}: stage/opcode mismatch {ins}")
            if s < prev:
                raise ValueError(f"wg {w}: list not in stage order")
            prev = s
            avail, first = placement(st, s, n_wg)
            if (first + i) % n_wg != w:
                raise ValueError(f"wg {w}: instruction {i} of stage {s} on the wrong block")
            if sig != s:
                raise ValueError("signal stage")
            want_ws = n_st - 1 if s == 0 else s - 1
            if ws != want_ws or wp != (1 if s == 0 else 0):
                raise ValueError("wait stage")
            seen[s].append((i, a, b, seq))
    for s, (op, l, sz) in enumerate(st):
        got = sorted(seen[s])
        want = stage_instructions(op, l, sz, placement(st, s, n_wg)[0], n_chunks, batch)
        if [x[0] for x in got] != list(range(len(want))):
            raise ValueError(f"stage {s}: instruction indices")
        if [(x[1], x[2], x[3]) for x in got] != want:
            raise ValueError(f"stage {s}: operands")
        if op in TILED_OPS:
            rows = np.zeros(sz, dtype=np.int64)
            for _, a, b, _ in got:
                rows[a:b] += 1
            if not np.all(rows == 1):
                raise ValueError(f"stage {s}: rows not covered exactly once")
    for s, (op, l, sz) in enumerate(st):
        n_prod = len(seen[n_st - 1 if s == 0 else s - 1])
        for w, lst in enumerate(lists):
            for ins in lst:
                if ins[2] == s and ins[7] != n_prod:
                    raise ValueError("wait count")


# ----------------------------------------------------------------------------
# simulator: what each instruction reads and writes, and a random interleaver
# ----------------------------------------------------------------------------

def chunk_range(T: int, n_chunks: int, c: int) -> Tuple[int, int]:
    """Positions [lo, hi) of split-KV chunk c when T positions are visible:
    chunk length = ceil(T / n_chunks) rounded up to a multiple of 16."""
    clen = ((T + n_chunks - 1) // n_chunks + 15) // 16 * 16
    return min(T, c * clen), min(T, (c + 1) * clen)


def _rw_sets(cfg, ins: Sequence[int], n_chunks: int, n_tiles: Dict[str, int], t: int,
             start_pos: Sequence[int], batch: int):
    """Element reads and writes of one instruction at token t.

    Buffers hold tagged values; a read of (buffer, element) expects the
    version written at ``(t, layer)`` named in the tuple.  Buffers: 'h'
    (residual entering a layer), 'qkv', 'part' (attention partials),
    'aout', 'hmid', 'act', 'route' (MoE), 'lm' (per-tile max/argmax), and
    'kv' (cache rows, element = (sequence, layer, kv_head, position); version =
    token that appended it, -1 for the context present before the run).
    Every element but the cache's carries its sequence first.
    """
    op, l, s, i, a, b = ins[:6]
    seq = ins[10]
    d, qd, kvd, hd, G = cfg.d_model, cfg.qd, cfg.kvd, cfg.head_dim, cfg.group
    reads: List[Tuple[str, object, Tuple[int, int]]] = []
    writes: List[Tuple[str, object, Tuple[int, int]]] = []
    seqs = range(batch)

    def token_reads():
        if t > 0:
            for q in seqs:
                for k in range(n_tiles["lm"]):
                    reads.append(("lm", (q, k), (t - 1, cfg.n_layers)))

    if op == OP_QKV:
        if l == 0:
            token_reads()
        else:
            reads.extend(("h", (q, r), (t, l)) for q in seqs for r in range(d))
        writes.extend(("qkv", (q, r), (t, l)) for q in seqs for r in range(a, b))
    elif op == OP_ATTN:
        p0 = start_pos[seq]
        pos = p0 + t
        if n_chunks == 1:
            qheads, kvh, c = [a], a // G, 0
            appends = a % G == 0
        else:
            qheads, kvh, c = list(range(a * G, (a + 1) * G)), a, b
            appends = True
        lo, hi = chunk_range(pos + 1, n_chunks, c)
        for j in range(lo, hi):
            if j < pos:
                reads.append(("kv", (seq, l, kvh, j), (j - p0 if j >= p0 else -1, 0)))
        if appends and lo <= pos < hi:
            writes.append(("kv", (seq, l, kvh, pos), (t, 0)))
        rows = [r for qh in qheads for r in range(qh * hd, (qh + 1) * hd)]
        rows += list(range(qd + kvh * hd, qd + (kvh + 1) * hd))
        rows += list(range(qd + kvd + kvh * hd, qd + kvd + (kvh + 1) * hd))
        reads.extend(("qkv", (seq, r), (t, l)) for r in rows)
        if n_chunks > 1:
            for j in qheads:
                writes.append(("part", (seq, j * n_chunks + c), (t, l)))
        else:
            writes.extend(("aout", (seq, r), (t, l)) for r in range(a * hd, (a + 1) * hd))
    elif op == OP_AREDUCE:
        j = a
        reads.extend(("part", (seq, j * n_chunks + c), (t, l)) for c in range(n_chunks))
        writes.extend(("aout", (seq, r), (t, l)) for r in range(j * hd, (j + 1) * hd))
    elif op == OP_OPROJ:
        reads.extend(("aout", (q, r), (t, l)) for q in seqs for r in range(qd))
        if l == 0:
            token_reads()
        else:
            reads.extend(("h", (q, r), (t, l)) for q in seqs for r in range(a, b))
        writes.extend(("hmid", (q, r), (t, l)) for q in seqs for r in range(a, b))
    elif op in (OP_UPGATE, OP_MOE_UPGATE):
        reads.extend(("hmid", (q, r), (t, l)) for q in seqs for r in range(d))
        writes.extend(("act", (q, r), (t, l)) for q in seqs for r in range(a, b))
        if op == OP_MOE_UPGATE and i == 0:
            writes.extend(("route", (q, 0), (t, l)) for q in seqs)
    elif op in (OP_DOWN, OP_MOE_DOWN):
        n_act = cfg.d_ff * (cfg.top_k if op == OP_MOE_DOWN else 1)
        reads.extend(("act", (q, r), (t, l)) for q in seqs for r in range(n_act))
        if op == OP_MOE_DOWN:
            reads.extend(("route", (q, 0), (t, l)) for q in seqs)
        reads.extend(("hmid", (q, r), (t, l)) for q in seqs for r in range(a, b))
        writes.extend(("h", (q, r), (t, l + 1)) for q in seqs for r in range(a, b))
    elif op == OP_LMHEAD:
        reads.extend(("h", (q, r), (t, l)) for q in seqs for r in range(d))
        writes.extend(("lm", (q, i), (t, l)) for q in seqs)
    return reads, writes


def simulate(cfg, words: np.ndarray, n_tokens: int = 2, seed: int = 0, start_pos=0) -> None:
    """Run every block's list under a random interleaving of tagged buffers.

    ``start_pos``: one position for every sequence, or one per sequence.  An
    instruction may run when every element it reads holds the version it
    expects.  Raises on deadlock (no block can run) and on a write that would
    replace a version some pending instruction still has to read.
    """
    hdr, lists = parse(words)
    n_wg, n_chunks, batch = hdr[2], hdr[5], hdr[15]
    starts = [int(start_pos)] * batch if np.isscalar(start_pos) else [int(x) for x in start_pos]
    if len(starts) != batch:
        raise ValueError("one start position per sequence")
    n_tiles = {"lm": min(n_wg, cfg.vocab)}
    rng = random.Random(seed)
    mem: Dict[Tuple[str, object], Tuple[int, int]] = {}
    for q in range(batch):
        for l in range(cfg.n_layers):
            for h in range(cfg.n_kv_heads):
                for j in range(starts[q]):
                    mem[("kv", (q, l, h, j))] = (-1, 0)
    # every (token, block, position) as a job in program order
    progs = [[(t, ins) for t in range(n_tokens) for ins in lst] for lst in lists]
    pc = [0] * n_wg
    # pending reads per (buffer, element, version): how many unfinished
    # instructions still need that version
    need: Dict[Tuple[str, int, Tuple[int, int]], int] = {}
    sets = []
    for w in range(n_wg):
        sw = []
        for t, ins in progs[w]:
            r, wr = _rw_sets(cfg, ins, n_chunks, n_tiles, t, starts, batch)
            sw.append((r, wr))
            for (buf, e, v) in r:
                need[(buf, e, v)] = need.get((buf, e, v), 0) + 1
        sets.append(sw)
    remaining = sum(len(p) for p in progs)
    while remaining:
        runnable = []
        for w in range(n_wg):
            if pc[w] < len(progs[w]):
                r, _ = sets[w][pc[w]]
                if all(mem.get((buf, e)) == v for (buf, e, v) in r):
                    runnable.append(w)
        if not runnable:
            stuck = [(w, progs[w][pc[w]][1][:6]) for w in range(n_wg) if pc[w] < len(progs[w])]
            raise RuntimeError(f"deadlock: {stuck[:4]}")
        w = rng.choice(runnable)
        r, wr = sets[w][pc[w]]
        for (buf, e, v) in r:
            need[(buf, e, v)] -= 1
        for (buf, e, v) in wr:
            old = mem.get((buf, e))
            if old is not None and need.get((buf, e, old), 0) > 0:
                raise RuntimeError(f"overwrite hazard: {buf}[{e}] {old} -> {v} by wg {w}")
            mem[(buf, e)] = v
        pc[w] += 1
        remaining -= 1
