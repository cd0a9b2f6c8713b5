"""Launch shape for a decode workload: workgroups and split-KV chunks."""
from __future__ import annotations


def chunks_for(head_bytes: int, n_wg: int, n_kv_heads: int) -> int:
    """Split-KV chunk count for ``head_bytes`` of K plus V per KV head.

    Measured on the Llama-1B shape (µs/token, 1 / 2 / 4 / 8 / 16 / 32 chunks):
    KV 128: 856 / 1086 / 951 / 958 / 963; KV 1024: 1303 / 1356 / 1089 / 1089 / 994;
    KV 4096: 1912 / 1579 / 1205 / 1193 / 1024; KV 16384: 8 -> 1390, 16 -> 1219,
    32 -> 1092.  A split costs one more dependency stage (the reduction), which
    only pays once a head's K/V no longer streams quickly through one workgroup.
    The same rule is coded in mkd_build_schedule for n_chunks == 0."""
    cap = max(1, min(64, n_wg // n_kv_heads))
    if head_bytes <= 128 * 1024:
        return 1
    if head_bytes <= 2 * 1024 * 1024:
        return min(16, cap)
    return cap


def launch_config(cfg, start_pos: int, n_steps: int, n_cu: int = 256):
    """(n_wg, n_chunks): one workgroup per compute unit; chunks from the run's
    longest context."""
    n_wg = n_cu
    T = start_pos + n_steps
    return n_wg, chunks_for(T * cfg.head_dim * 4, n_wg, cfg.n_kv_heads)
