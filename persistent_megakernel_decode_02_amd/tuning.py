"""Launch shape for a decode workload: workgroups and split-KV chunks."""
from __future__ import annotations


def chunks_for(head_bytes: int, n_wg: int, n_kv_heads: int) -> int:
    """Split-KV chunk count for ``head_bytes`` of K plus V per KV head.

    With one chunk the attention instructions are one per q head (schedule
    spec v3); with several, one per (kv head, chunk) plus a reduction stage.
    Measured on the Llama-1B shape (µs/token):
    KV 128: 1 chunk 811; KV 1024: 1 -> 862, 4 -> 1138, 16 -> 978;
    KV 4096: 1 -> 1174, 2 -> 1427, 4 -> 1316, 8 -> 1225, 16 -> 988, 32 -> 993;
    KV 16384: 1 -> 1970, 4 -> 2155, 8 -> 1469, 16 -> 1176, 32 -> 1081.
    The same rule is coded in mkd_build_schedule for n_chunks == 0."""
    cap = max(1, min(64, n_wg // n_kv_heads))
    if head_bytes <= 512 * 1024:
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
