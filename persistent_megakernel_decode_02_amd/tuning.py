"""Launch shape for a decode workload: workgroups and split-KV chunks.

The chunk rule lives in the library (mkd_default_chunks); this module only
asks it.  Measured on one MI355X (µs/token, 128 or 32 decode steps):
1B KV 1024: 1 chunk -> 724, 4 -> 1024, 8 -> 931, 16 -> 901, 32 -> 845;
1B KV 4096: 1 -> 1182, 4 -> 1183, 8 -> 1023, 16 -> 915, 32 -> 868;
3B KV 2048: 1 -> 2273, 8 -> 1968, 16 -> 1785, 32 -> 1699;
1B KV 16384: 16 -> 1049, 32 -> 997, 64 -> 1223 (64 leaves some workgroups
two attention instructions).  Hence one chunk up to 512 KiB of K and V per
head, else as many chunks as give every workgroup at most one (kv head,
chunk).
"""
from __future__ import annotations

from . import capi


def launch_config(cfg, start_pos: int, n_steps: int, n_cu: int = 256):
    """(n_wg, n_chunks): one workgroup per compute unit; chunks from the run's
    longest context."""
    n_wg = n_cu
    return n_wg, capi.mkd_default_chunks(capi.make_config(cfg), n_wg, start_pos + n_steps)
