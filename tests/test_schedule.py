"""Schedule spec v1: the oracle's builder against its invariants and the
simulator; the GPU library's C++ builder against the oracle's, byte for byte."""
import numpy as np
import pytest

import synth
from oracle import schedule as S


@pytest.mark.parametrize("name", ["tiny", "llama1b", "llama3b", "mixtral"])
@pytest.mark.parametrize("n_wg", [1, 3, 8, 64, 256, 304])
def test_oracle_schedule_valid(name, n_wg):
    cfg = synth.PRESETS[name]
    for n_chunks in (1, 4, 32):
        w = S.build(cfg, n_wg, n_chunks)
        assert w.dtype == np.int32
        S.validate(w, cfg)


@pytest.mark.parametrize("n_wg,n_chunks,start", [(1, 1, 0), (3, 2, 5), (8, 4, 40), (32, 1, 3), (5, 3, 17)])
def test_simulator_no_deadlock_no_hazard(n_wg, n_chunks, start):
    cfg = synth.PRESETS["tiny"]
    w = S.build(cfg, n_wg, n_chunks)
    for seed in range(3):
        S.simulate(cfg, w, n_tokens=3, seed=seed, start_pos=start)


@pytest.mark.parametrize("batch", [2, 3, 8])
def test_oracle_batched_schedule_valid(batch):
    for name in ("tiny", "llama1b"):
        cfg = synth.PRESETS[name]
        for n_wg in (1, 5, 64, 256):
            for n_chunks in (1, 4):
                w = S.build(cfg, n_wg, n_chunks, batch)
                S.validate(w, cfg)
                hdr, lists = S.parse(w)
                assert hdr[15] == batch
                seqs = {ins[10] for lst in lists for ins in lst if ins[0] in (S.OP_ATTN, S.OP_AREDUCE)}
                assert seqs == set(range(batch))
                assert all(ins[10] == 0 for lst in lists for ins in lst if ins[0] in S.TILED_OPS)


@pytest.mark.parametrize("n_wg,n_chunks,batch,starts", [(1, 1, 2, [0, 3]), (5, 2, 3, [7, 0, 20]),
                                                         (16, 4, 4, [40, 2, 9, 33]), (3, 1, 8, list(range(8)))])
def test_simulator_batched_no_deadlock_no_hazard(n_wg, n_chunks, batch, starts):
    cfg = synth.PRESETS["tiny"]
    w = S.build(cfg, n_wg, n_chunks, batch)
    for seed in range(2):
        S.simulate(cfg, w, n_tokens=2, seed=seed, start_pos=starts)


def test_simulator_moe():
    from tests.test_oracle_pins import MICRO_MOE
    w = S.build(MICRO_MOE, 4, 2)
    S.validate(w, MICRO_MOE)
    S.simulate(MICRO_MOE, w, n_tokens=3, seed=1, start_pos=2)


def test_validator_rejects_planted_errors():
    cfg = synth.PRESETS["tiny"]
    good = S.build(cfg, 8, 2)
    hdr, lists = S.parse(good)
    base = S.WORDS + 8
    # 1) a GEMV tile whose row range overlaps its neighbour
    bad = good.copy()
    bad[base + 5] += 1
    with pytest.raises(ValueError):
        S.validate(bad, cfg)
    # 2) a wrong wait count
    bad = good.copy()
    bad[base + 7] += 1
    with pytest.raises(ValueError):
        S.validate(bad, cfg)
    # 3) two instructions of one block swapped out of stage order
    bad = good.copy()
    a, b = base, base + S.WORDS
    tmp = bad[a:a + S.WORDS].copy()
    bad[a:a + S.WORDS] = bad[b:b + S.WORDS]
    bad[b:b + S.WORDS] = tmp
    with pytest.raises(ValueError):
        S.validate(bad, cfg)


def test_simulator_finds_planted_deadlock():
    """A block whose list runs a later stage before an earlier one it feeds
    cannot make progress: the simulator must report it, not loop."""
    cfg = synth.PRESETS["tiny"]
    w = S.build(cfg, 2, 1)
    hdr, lists = S.parse(w)
    n_wg, max_instr = hdr[2], hdr[4]
    body = w[S.WORDS + n_wg:].reshape(n_wg, max_instr, S.WORDS).copy()
    # swap block 0's first two instructions (QKV of layer 0 and ATTN of layer 0)
    body[0, [0, 1]] = body[0, [1, 0]]
    bad = np.concatenate([w[:S.WORDS + n_wg], body.reshape(-1)])
    with pytest.raises(RuntimeError, match="deadlock"):
        S.simulate(cfg, bad, n_tokens=1, seed=0, start_pos=0)


def test_chunk_ranges_cover_positions():
    for T in range(1, 300, 7):
        for n in (1, 2, 5, 32):
            got = []
            for c in range(n):
                lo, hi = S.chunk_range(T, n, c)
                got.extend(range(lo, hi))
            assert got == list(range(T))
