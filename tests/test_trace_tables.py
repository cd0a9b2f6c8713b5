"""bench.py's per-opcode tables from a hand-made device trace: two
workgroups, a QKV stage on both and an attention stage on one, one step, a
clock of 1 MHz (one tick per microsecond), so every figure can be worked out
by hand from the timestamps."""
import numpy as np

import bench
import synth

OP_QKV, OP_ATTN = 1, 2


def _schedule():
    n_wg, max_instr, n_st = 2, 2, 2
    words = np.zeros(16 + n_wg + n_wg * max_instr * 16, dtype=np.int32)
    words[2], words[3], words[4] = n_wg, n_st, max_instr
    words[16:16 + n_wg] = [2, 1]                       # instructions per workgroup
    body = words[16 + n_wg:].reshape(n_wg, max_instr, 16)
    body[0, 0, :3] = [OP_QKV, 0, 0]                    # opcode, layer, stage
    body[1, 0, :3] = [OP_QKV, 0, 0]
    body[0, 1, :3] = [OP_ATTN, 0, 1]
    return words


def _trace():
    t = np.zeros((2, 1, 2, 4), dtype=np.int64)         # [wg][step][instr][start, ready, published, -]
    t[0, 0, 0, :3] = [0, 2, 5]
    t[1, 0, 0, :3] = [1, 3, 7]
    t[0, 0, 1, :3] = [6, 8, 10]
    return t


def _row(lines, prefix):
    rows = [ln for ln in lines if ln.startswith(prefix)]
    assert rows, prefix
    return [c.strip() for c in rows[0].strip("|").split("|")]


def test_trace_tables_by_hand():
    cfg = synth.PRESETS["tiny"]
    lines = bench.trace_tables(_trace(), _schedule(), 1e6, cfg, 32)
    # per instruction: QKV waits 2 and 2, works 3 and 4; attention waits 2, works 2
    assert _row(lines, "| QKV | 2 x 1")[2:] == ["2.00", "2.00", "3.50", "3.00", "4.00"]
    assert _row(lines, "| ATTN | 1 x 1")[2:] == ["2.00", "2.00", "2.00", "2.00", "2.00"]
    # per token: QKV's share runs from the step's first start (0) to its last
    # publish (7): first consumer ready at 2, last at 3, so 2 + 1 + 4;
    # attention's from 7 to 10: ready at 8, so 1 + 0 + 2; total 10
    q = _row(lines, "| QKV | 7.0")
    assert q[1:6] == ["7.0", "70.0", "2.0", "1.0", "4.0"]
    a = _row(lines, "| ATTN | 3.0")
    assert a[1:6] == ["3.0", "30.0", "1.0", "0.0", "2.0"]
    mb = bench.stage_bytes(cfg, "QKV", 32) / 1e6
    assert q[6] == f"{mb:.1f}" and q[7] == f"{bench.stage_bytes(cfg, 'QKV', 32) / 7e-6 / 1e9:.0f}"
    assert _row(lines, "| total")[1] == "10.0"
    # the attention consumer starts 1 us before QKV's last publish and holds
    # its inputs 1 us after it
    assert _row(lines, "| ATTN | -1.00") == ["ATTN", "-1.00", "-1.00", "-1.00", "1.00", "1.00", "1.00", "1.00"]
    # stages of at most 8 consumers are not counted for the last-consumer line
    assert not any(ln.startswith("The last consumer") for ln in lines)
