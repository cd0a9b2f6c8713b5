"""Launch shape for a decode workload: workgroups and split-KV chunks."""
from __future__ import annotations


def chunks_for(head_bytes: int, n_wg: int, n_kv_heads: int) -> int:
    """Split-KV chunk count for ``head_bytes`` of K plus V per KV head.

    With one chunk the attention instructions are one per q head (schedule
    spec v4); with several, one per (kv head, chunk) plus a reduction stage.
    Measured on one MI355X (µs/token, 128 or 32 decode steps):
    1B KV 1024: 1 -> 724, 4 -> 1024, 8 -> 931, 16 -> 901, 32 -> 845;
    1B KV 4096: 1 -> 1182, 4 -> 1183, 8 -> 1023, 16 -> 915, 32 -> 868;
    3B KV 2048: 1 -> 2273, 8 -> 1968, 16 -> 1785, 32 -> 1699;
    1B KV 16384: 16 -> 1049, 32 -> 997, 64 -> 1223 (64 leaves some workgroups
    two attention instructions).
    So: one chunk up to 512 KiB per head, else as many chunks as give every
    workgroup at most one (kv head, chunk).  The same rule is coded in
    mkd_build_schedule for n_chunks == 0."""
    cap = max(1, min(64, n_wg // n_kv_heads))
    if head_bytes <= 512 * 1024:
        return 1
    return cap


def launch_config(cfg, start_pos: int, n_steps: int, n_cu: int = 256):
    """(n_wg, n_chunks): one workgroup per compute unit; chunks from the run's
    longest context."""
    n_wg = n_cu
    T = start_pos + n_steps
    return n_wg, chunks_for(T * cfg.head_dim * 4, n_wg, cfg.n_kv_heads)
