"""Seeded synthetic inputs and workload presets.

This module is shared by the CPU oracle (``oracle/``) and by the GPU path's
harness (tests, bench).  It holds no arithmetic of the decode method itself:
only model shapes, the fixed order of the weight tensors, and counter-based
generators for weights, KV-cache fill and token ids.

Generation is done with integer torch ops (exact on any device) followed by a
table lookup, so the same call gives bit-identical bf16 tensors on the CPU and
on the GPU.  The GPU harness generates its copy on the device (fast); the
oracle generates its copy on the host; neither copies the other's.

Value recipe (the pages only say "random-init weights from seed"; the shapes
follow the model families the epic-kernel README names in "3B model support"
and "Mixtral 8x7B MoE for batch-1 inference"):

* every matrix (embedding, projections, router, experts) ~ N(0, 0.02^2),
* RMSNorm gains = 1.0 (or 1 + N(0, gain_std^2) when a test asks for it),
* KV-cache fill ~ N(0, 1),
* tokens uniform over [0, vocab).

A normal variate is ``table[u16]`` where ``u16`` is 16 bits of a 32-bit
counter hash and ``table[k]`` is the bf16 rounding of the inverse normal CDF at
``(k + 0.5) / 65536`` scaled by the standard deviation (inverse-transform
sampling with 16-bit resolution).
"""
from __future__ import annotations

import dataclasses
import math
import statistics
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "ModelConfig", "Workload", "PRESETS", "WORKLOADS", "weight_specs",
    "gen_weights", "gen_kv_cache", "gen_tokens", "normal_table_bf16",
    "SEED_WEIGHTS", "SEED_TOKENS", "SEED_KV",
]

SEED_WEIGHTS = 0
SEED_TOKENS = 1
SEED_KV = 2

_M32 = 0xFFFFFFFF


@dataclasses.dataclass(frozen=True)
class ModelConfig:
    """Shape of a pre-norm Llama-style (or Mixtral-style MoE) decoder."""
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    n_experts: int = 0
    top_k: int = 0
    tied: bool = False
    rms_eps: float = 1e-5
    rope_theta: float = 10000.0

    @property
    def qd(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kvd(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode workload: a model, the KV lengths it starts from, and steps."""
    name: str
    model: ModelConfig
    kv_lengths: Tuple[int, ...]
    steps: int
    prompt_len: int = 0          # >0: the run starts with a prompt prefill


TINY = ModelConfig("tiny", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2,
                   head_dim=64, d_ff=768, vocab=1024, rope_theta=10000.0)
LLAMA_1B = ModelConfig("llama-3.2-1b-shaped", n_layers=16, d_model=2048,
                       n_q_heads=32, n_kv_heads=8, head_dim=64, d_ff=8192,
                       vocab=128256, tied=True, rope_theta=500000.0)
LLAMA_3B = ModelConfig("llama-3.2-3b-shaped", n_layers=28, d_model=3072,
                       n_q_heads=24, n_kv_heads=8, head_dim=128, d_ff=8192,
                       vocab=128256, tied=True, rope_theta=500000.0)
MIXTRAL = ModelConfig("mixtral-8x7b-shaped", n_layers=32, d_model=4096,
                      n_q_heads=32, n_kv_heads=8, head_dim=128, d_ff=14336,
                      vocab=32000, n_experts=8, top_k=2, rope_theta=1e6)

# a small top-2 MoE of the Mixtral kind, for parity runs of the MoE opcodes
TINY_MOE = ModelConfig("tiny-moe", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2,
                       head_dim=64, d_ff=512, vocab=1024, n_experts=8, top_k=2, rope_theta=1e6)

PRESETS: Dict[str, ModelConfig] = {
    "tiny": TINY, "llama1b": LLAMA_1B, "llama3b": LLAMA_3B, "mixtral": MIXTRAL,
    "tiny_moe": TINY_MOE,
}

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, (32,), 16, prompt_len=32),
    "llama1b": Workload("llama1b", LLAMA_1B, (128, 1024, 4096), 128),
    "llama3b": Workload("llama3b", LLAMA_3B, (128, 2048), 128),
    "llama1b_long": Workload("llama1b_long", LLAMA_1B, (16384, 32768), 64),
    "mixtral": Workload("mixtral", MIXTRAL, (1024,), 64),
}


def weight_specs(cfg: ModelConfig) -> List[Tuple[str, Tuple[int, ...]]]:
    """Names and shapes of the weight tensors, in the fixed pointer order.

    Matrices are row-major ``[out, in]``.  Order: ``embed, final_norm,
    [lm_head if untied]``, then per layer ``attn_norm, wq, wk, wv, wo,
    ffn_norm`` followed by ``w_gate, w_up, w_down`` (dense) or
    ``router, gate[0..E), up[0..E), down[0..E)`` (MoE).
    """
    d, F, V = cfg.d_model, cfg.d_ff, cfg.vocab
    specs: List[Tuple[str, Tuple[int, ...]]] = [("embed", (V, d)), ("final_norm", (d,))]
    if not cfg.tied:
        specs.append(("lm_head", (V, d)))
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        specs += [(p + "attn_norm", (d,)), (p + "wq", (cfg.qd, d)),
                  (p + "wk", (cfg.kvd, d)), (p + "wv", (cfg.kvd, d)),
                  (p + "wo", (d, cfg.qd)), (p + "ffn_norm", (d,))]
        if cfg.is_moe:
            specs.append((p + "router", (cfg.n_experts, d)))
            specs += [(p + f"gate.{e}", (F, d)) for e in range(cfg.n_experts)]
            specs += [(p + f"up.{e}", (F, d)) for e in range(cfg.n_experts)]
            specs += [(p + f"down.{e}", (d, F)) for e in range(cfg.n_experts)]
        else:
            specs += [(p + "w_gate", (F, d)), (p + "w_up", (F, d)), (p + "w_down", (d, F))]
    return specs


# ----------------------------------------------------------------------------
# counter-based generator
# ----------------------------------------------------------------------------

def _mix32(x: torch.Tensor) -> torch.Tensor:
    """32-bit integer finaliser on int64 tensors holding values in [0, 2^32).

    Every product stays below 2^59, so int64 arithmetic is exact on any device.
    """
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    return (x >> 16) ^ x


def _mix32_int(x: int) -> int:
    x &= _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    x = (((x >> 16) ^ x) * 0x45D9F3B) & _M32
    return (x >> 16) ^ x


def _stream_key(seed: int, stream: int) -> int:
    return _mix32_int(_mix32_int(seed + 0x3C6EF372) ^ ((stream * 0x27D4EB2F) & _M32))


def _f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


_TABLES: Dict[Tuple[float, float], torch.Tensor] = {}


def normal_table_bf16(std: float, mean: float = 0.0) -> torch.Tensor:
    """65536 bf16 values: mean + std * Phi^-1((k + 0.5) / 65536), k = 0..65535."""
    key = (float(std), float(mean))
    if key not in _TABLES:
        nd = statistics.NormalDist(0.0, 1.0)
        z = np.array([nd.inv_cdf((k + 0.5) / 65536.0) for k in range(65536)], dtype=np.float64)
        vals = (mean + std * z).astype(np.float32)
        bits = _f32_to_bf16_bits(vals).view(np.int16)
        _TABLES[key] = torch.from_numpy(bits.copy()).view(torch.bfloat16)
    return _TABLES[key]


def _gen_u16(key: int, start: int, n: int, device) -> torch.Tensor:
    """16-bit uniforms for element indices [start, start + n) of one stream."""
    idx = torch.arange(start, start + n, dtype=torch.int64, device=device)
    h = _mix32((idx >> 1) ^ key)
    return (h >> ((idx & 1) * 16)) & 0xFFFF


def gen_bf16(seed: int, stream: int, shape: Sequence[int], std: float, mean: float = 0.0,
             device="cpu", chunk: int = 1 << 24) -> torch.Tensor:
    """bf16 tensor of ``shape`` with entries ``mean + std * N(0,1)`` (table sampled)."""
    n = int(np.prod(shape)) if len(shape) else 1
    table = normal_table_bf16(std, mean).to(device)
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    key = _stream_key(seed, stream)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        out[s:s + m] = table[_gen_u16(key, s, m, device)]
    return out.view(*shape)


def gen_weights(cfg: ModelConfig, seed: int = SEED_WEIGHTS, device="cpu",
                gain_std: float = 0.0, std: float = 0.02,
                only: Optional[Sequence[int]] = None) -> List[Optional[torch.Tensor]]:
    """All weight tensors of ``cfg`` in pointer order (bf16).

    ``only``: generate just these indices (others are returned as ``None``);
    lets a check rebuild a few tensors of a model too large for host memory.
    """
    out: List[Optional[torch.Tensor]] = []
    for i, (name, shape) in enumerate(weight_specs(cfg)):
        if only is not None and i not in only:
            out.append(None)
            continue
        if len(shape) == 1:  # RMSNorm gain
            if gain_std > 0.0:
                out.append(gen_bf16(seed, i, shape, gain_std, 1.0, device))
            else:
                out.append(torch.ones(shape, dtype=torch.bfloat16, device=device))
        else:
            out.append(gen_bf16(seed, i, shape, std, 0.0, device))
    return out


def kv_cache_shape(cfg: ModelConfig, max_seq: int) -> Tuple[int, int, int, int, int]:
    """KV cache layout ``[L][2 (K, V)][n_kv_heads][max_seq][head_dim]`` (bf16)."""
    return (cfg.n_layers, 2, cfg.n_kv_heads, max_seq, cfg.head_dim)


def gen_kv_cache(cfg: ModelConfig, max_seq: int, filled: int, seed: int = SEED_KV,
                 device="cpu") -> torch.Tensor:
    """KV cache with positions [0, filled) ~ N(0,1) (bf16), the rest zero.

    The filled keys are taken as already rotated (they stand for a context
    the model has already seen).  Each (layer, K|V, head) row block is its own
    stream so that the fill does not depend on ``max_seq``.
    """
    shape = kv_cache_shape(cfg, max_seq)
    kv = torch.zeros(shape, dtype=torch.bfloat16, device=device)
    if filled > 0:
        L, two, H, _, hd = shape
        for l in range(L):
            for kvi in range(2):
                for h in range(H):
                    stream = (l * 2 + kvi) * H + h
                    kv[l, kvi, h, :filled] = gen_bf16(seed, stream, (filled, hd), 1.0, 0.0, device)
    return kv


def gen_tokens(n: int, vocab: int, seed: int = SEED_TOKENS, stream: int = 0) -> List[int]:
    """``n`` token ids uniform over [0, vocab)."""
    key = _stream_key(seed, stream)
    idx = torch.arange(n, dtype=torch.int64)
    h = _mix32(idx ^ key)
    return [int(v) for v in ((h * vocab) >> 32).tolist()]


def bytes_of(cfg: ModelConfig) -> int:
    """Bytes of all stored weights (bf16)."""
    return 2 * sum(int(np.prod(s)) for _, s in weight_specs(cfg))
