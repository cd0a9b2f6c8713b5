"""Algorithmic HBM bytes of batch-1 decode and the bandwidth floor.

A batch-1 step reads each weight it uses at least once per step, so its
algorithmic bytes over the peak bandwidth bound the step time from below (the
weight-read floor of the Hyperkernel teardown, "Where the numbers sit against
the hardware").  Counted per step at position
p (p + 1 visible positions):

* every weight the step reads: all dense matrices and norm gains, the full
  LM head (the embedding matrix when tied), one embedding row, and for MoE
  the router plus only the top-k experts' up/gate/down;
* K and V of positions 0..p in every layer (the stored bf16 rows);
* the appended K and V row of every layer (written once).

Not counted: activations, partial results, tags, and instruction fetch.
"""
from __future__ import annotations

from typing import Tuple

HBM_PEAK_BYTES_PER_S = 8.0e12     # MI355X HBM3E, published peak


def weight_bytes_per_step(cfg) -> int:
    d, F, V, L = cfg.d_model, cfg.d_ff, cfg.vocab, cfg.n_layers
    attn = cfg.qd * d + 2 * cfg.kvd * d + d * cfg.qd
    if cfg.is_moe:
        ffn = cfg.n_experts * d + cfg.top_k * 3 * F * d
    else:
        ffn = 3 * F * d
    per_layer = attn + ffn + 2 * d                    # + two norm gains
    total = L * per_layer + V * d + d + d             # LM head, embedding row, final norm
    return 2 * total


def kv_bytes_per_position(cfg) -> int:
    """bf16 K and V of one position over all layers."""
    return cfg.n_layers * 2 * cfg.kvd * 2


def step_bytes(cfg, pos: int) -> int:
    """Bytes of the step that consumes a token at position ``pos``."""
    kv = kv_bytes_per_position(cfg)
    return weight_bytes_per_step(cfg) + kv * (pos + 1) + kv


def run_bytes(cfg, start_pos: int, n_steps: int) -> int:
    """Bytes of a decode run of ``n_steps`` steps starting at ``start_pos``."""
    kv = kv_bytes_per_position(cfg)
    w = weight_bytes_per_step(cfg)
    # sum over p = start .. start+n-1 of (p + 2) * kv
    s = n_steps * (start_pos + 2) + n_steps * (n_steps - 1) // 2
    return n_steps * w + kv * s


def batch_run_bytes(cfg, start_positions, n_steps: int) -> int:
    """Bytes of one launch decoding several sequences together for ``n_steps``
    steps: each step reads every weight once for all of them (plus one
    embedding row per sequence), and each sequence reads and appends its own
    cache rows as in ``run_bytes``."""
    B = len(start_positions)
    w = weight_bytes_per_step(cfg) + (B - 1) * 2 * cfg.d_model
    kv = sum(run_bytes(cfg, s, n_steps) - n_steps * weight_bytes_per_step(cfg) for s in start_positions)
    return n_steps * w + kv


def floor_seconds(n_bytes: float, bandwidth: float = HBM_PEAK_BYTES_PER_S) -> float:
    return n_bytes / bandwidth


def roofline(cfg, start_pos: int, n_steps: int, seconds: float,
             bandwidth: float = HBM_PEAK_BYTES_PER_S) -> Tuple[float, float, float]:
    """(achieved bytes/s, floor seconds, fraction of roofline) of a timed run."""
    b = run_bytes(cfg, start_pos, n_steps)
    return b / seconds, b / bandwidth, (b / bandwidth) / seconds
