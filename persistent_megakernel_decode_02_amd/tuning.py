"""Launch shape for a decode workload: workgroups and split-KV chunks."""
from __future__ import annotations

import math


def launch_config(cfg, start_pos: int, n_steps: int, n_cu: int = 256):
    """(n_wg, n_chunks): one workgroup per compute unit; K/V of a head split so
    that a chunk holds about 32 KiB of K and V at the run's longest context,
    at most n_wg / n_kv_heads chunks (every workgroup gets at most one) and 64."""
    n_wg = n_cu
    T = start_pos + n_steps
    per_head = T * cfg.head_dim * 2 * 2
    want = max(1, math.ceil(per_head / 32768))
    cap = max(1, min(64, n_wg // cfg.n_kv_heads))
    return n_wg, min(want, cap)
