"""Plain decoder forward pass (numpy), one token at a time with a KV cache.

What is computed follows the model families the epic-kernel README builds
batch-1 megakernels for (its intro and "3B model support": Llama-3.2 1B/3B;
"Mixtral 8x7B MoE for batch-1 inference": router scoring, top-2 expert
selection, expert up/gate and down projections).  The pages never write the
layer equations, so this module takes the standard pre-norm Llama/Mixtral
decoder, with these readings (each listed in the design notes):

* RMSNorm ``x = h / sqrt(mean(h^2) + eps) * gamma``.
* RoPE in the "rotate-half" form: pairs ``(i, i + hd/2)``, frequency
  ``theta^(-2i/hd)``; angles and cos/sin in fp64, rounded to fp32.
* K and V are stored in the cache as bf16 (round-to-nearest-even of the fp32
  value after RoPE); attention reads the stored values, including the one
  just appended.
* Attention: softmax over ``q . K_j / sqrt(hd)`` for ``j <= pos``; q head
  ``j`` reads KV head ``j // (hq / hkv)``.
* FFN ``W_d (silu(W_g x) * (W_u x))``, ``silu(z) = z / (1 + e^-z)``.
* MoE: ``z = W_r x``; the two largest logits (lower index first on ties);
  gate weights = softmax over those two logits; output = weighted sum of the
  two experts' FFNs.
* Logits ``W_lm rmsnorm(h)`` (``W_lm = embed`` when tied); next token is
  the argmax, lowest index on ties.
* Activations are fp32 (or fp64 in the noise-floor mode); weights are the
  bf16 inputs converted exactly.

Parity pins: every function here is pinned by tests under ``tests/``
(closed forms, invariants, brute force on tiny inputs, prefill-vs-decode).
The whole-model logits at full sizes are "parity unpinned" beyond those
component pins: with random weights the pages print no worked example.
"""
from __future__ import annotations

import math
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# elementary pieces
# ----------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even), as fp32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32)


def rmsnorm(h: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """``h / sqrt(mean(h^2) + eps) * gamma`` over the last axis."""
    dt = h.dtype
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return (h / np.sqrt(ms + dt.type(eps))) * gamma


def rope_cos_sin(pos: int, head_dim: int, theta: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of ``pos * theta^(-2i/hd)``, i < hd/2: fp64 math, fp32 result."""
    half = head_dim // 2
    ang = [float(pos) * (float(theta) ** (-2.0 * i / head_dim)) for i in range(half)]
    c = np.array([math.cos(a) for a in ang], dtype=np.float64).astype(np.float32)
    s = np.array([math.sin(a) for a in ang], dtype=np.float64).astype(np.float32)
    return c, s


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate each row of ``x[..., hd]``: pair (i, i+hd/2) by the angle of i."""
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    c = cos.astype(x.dtype)
    s = sin.astype(x.dtype)
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Grouped-query attention of one position over cached keys/values.

    q: [hq, hd]; K, V: [hkv, T, hd] (the T visible positions).  Returns [hq, hd].
    """
    hq, hd = q.shape
    hkv = K.shape[0]
    G = hq // hkv
    out = np.empty_like(q)
    scale = q.dtype.type(1.0 / math.sqrt(hd))
    for j in range(hq):
        g = j // G
        s = (K[g] @ q[j]) * scale
        out[j] = softmax(s) @ V[g]
    return out


def silu(z: np.ndarray) -> np.ndarray:
    return z / (z.dtype.type(1.0) + np.exp(-z))


def top2_route(z: np.ndarray, k: int = 2) -> Tuple[List[int], np.ndarray]:
    """Indices of the k largest router logits (ties -> lower index first)
    and their softmax weights (softmax over the chosen logits only)."""
    order = sorted(range(len(z)), key=lambda e: (-float(z[e]), e))[:k]
    sel = np.array([z[e] for e in order], dtype=z.dtype)
    return order, softmax(sel)


def argmax_first(x: np.ndarray) -> int:
    """Index of the maximum, the lowest one on ties."""
    return int(np.argmax(x))


# ----------------------------------------------------------------------------
# model
# ----------------------------------------------------------------------------

class Weights:
    """Weight access by pointer-order index, converted to the oracle dtype.

    ``source(i)`` returns tensor ``i`` as anything ``np.asarray`` accepts after
    ``.float()`` (a bf16 torch tensor).  Converted tensors are kept when
    ``cache`` is true, or, when it is a function of the index, for the indices
    it accepts (models larger than host memory keep only some tensors).
    """

    def __init__(self, cfg, source: Callable[[int], object], dtype=np.float32, cache=True):
        import synth  # seeded inputs: names/shapes only
        self.cfg = cfg
        self.dtype = np.dtype(dtype)
        self.names = [n for n, _ in synth.weight_specs(cfg)]
        self.index = {n: i for i, n in enumerate(self.names)}
        self._source = source
        self._keep = cache if callable(cache) else (lambda i, c=bool(cache): c)
        self._cache = {}

    def __call__(self, name: str) -> np.ndarray:
        i = self.index[name]
        if i in self._cache:
            return self._cache[i]
        t = self._source(i)
        a = np.asarray(t.float().cpu().numpy(), dtype=self.dtype)
        if self._keep(i):
            self._cache[i] = a
        return a

    @classmethod
    def from_list(cls, cfg, tensors: Sequence[object], dtype=np.float32):
        return cls(cfg, lambda i: tensors[i], dtype)


class Oracle:
    """Decode with a KV cache held as float arrays of bf16 values.

    ``kv`` is ``[L][2][hkv][max_seq][hd]`` (numpy, oracle dtype) and is updated
    in place at each step's position.
    """

    def __init__(self, cfg, weights: Weights):
        self.cfg = cfg
        self.w = weights
        self.dt = weights.dtype

    def _ln(self, name):
        return self.w(name)

    # one decode step ----------------------------------------------------
    def step(self, token: int, pos: int, kv: np.ndarray, record: Optional[dict] = None) -> np.ndarray:
        cfg, w, dt = self.cfg, self.w, self.dt
        eps = cfg.rms_eps
        hd, hq, hkv = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
        h = w("embed")[token].astype(dt).copy()
        cos, sin = rope_cos_sin(pos, hd, cfg.rope_theta)
        for l in range(cfg.n_layers):
            p = f"layers.{l}."
            x = rmsnorm(h, w(p + "attn_norm"), eps)
            q = (w(p + "wq") @ x).reshape(hq, hd)
            k = (w(p + "wk") @ x).reshape(hkv, hd)
            v = (w(p + "wv") @ x).reshape(hkv, hd)
            if record is not None:
                record[f"{l}.q_raw"] = q.copy()
                record[f"{l}.k_raw"] = k.copy()
                record[f"{l}.v_raw"] = v.copy()
            q = apply_rope(q, cos, sin)
            k = apply_rope(k, cos, sin)
            kv[l, 0, :, pos, :] = bf16_round(k.astype(np.float32)).astype(dt)
            kv[l, 1, :, pos, :] = bf16_round(v.astype(np.float32)).astype(dt)
            o = attention(q, kv[l, 0, :, :pos + 1, :], kv[l, 1, :, :pos + 1, :])
            if record is not None:
                record[f"{l}.attn"] = o.copy()
            h = h + w(p + "wo") @ o.reshape(-1)
            if record is not None:
                record[f"{l}.h_mid"] = h.copy()
            x = rmsnorm(h, w(p + "ffn_norm"), eps)
            h = h + self._ffn(l, x, record)
            if record is not None:
                record[f"{l}.h_out"] = h.copy()
        x = rmsnorm(h, w("final_norm"), eps)
        W_lm = w("embed") if cfg.tied else w("lm_head")
        return W_lm @ x

    def _ffn(self, l: int, x: np.ndarray, record: Optional[dict]) -> np.ndarray:
        cfg, w = self.cfg, self.w
        p = f"layers.{l}."
        if not cfg.is_moe:
            a = silu(w(p + "w_gate") @ x) * (w(p + "w_up") @ x)
            if record is not None:
                record[f"{l}.act"] = a.copy()
            return w(p + "w_down") @ a
        z = w(p + "router") @ x
        experts, gates = top2_route(z, cfg.top_k)
        if record is not None:
            record[f"{l}.route"] = (list(experts), gates.copy())
        out = np.zeros_like(x)
        for e, g in zip(experts, gates):
            a = silu(w(p + f"gate.{e}") @ x) * (w(p + f"up.{e}") @ x)
            out = out + g * (w(p + f"down.{e}") @ a)
        return out

    # runs ---------------------------------------------------------------
    def decode(self, first_token: int, start_pos: int, n_steps: int, kv: np.ndarray,
               forced: Optional[Sequence[int]] = None) -> Tuple[List[int], np.ndarray]:
        """Greedy decode.  Step i consumes a token at position start_pos + i:
        ``first_token`` for i = 0, else ``forced[i]`` when given and >= 0, else
        the argmax of step i-1.  Returns (argmax of every step, logits[n, V])."""
        toks: List[int] = []
        logits = np.empty((n_steps, self.cfg.vocab), dtype=self.dt)
        tok = first_token
        for i in range(n_steps):
            if i > 0:
                tok = toks[-1]
                if forced is not None and forced[i] >= 0:
                    tok = int(forced[i])
            logits[i] = self.step(tok, start_pos + i, kv)
            toks.append(argmax_first(logits[i]))
        return toks, logits

    def prefill(self, tokens: Sequence[int], kv: np.ndarray) -> np.ndarray:
        """All positions 0..n-1 at once (causal), no incremental cache reads:
        an independent route to the same logits as ``decode`` with forcing."""
        cfg, w, dt = self.cfg, self.w, self.dt
        n = len(tokens)
        eps = cfg.rms_eps
        hd, hq, hkv, G = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.group
        H = w("embed")[np.asarray(tokens)].astype(dt)           # [n, d]
        cs = [rope_cos_sin(p, hd, cfg.rope_theta) for p in range(n)]
        C = np.stack([c for c, _ in cs])[:, None, :]             # [n, 1, hd/2]
        S = np.stack([s for _, s in cs])[:, None, :]
        mask = np.triu(np.full((n, n), -np.inf, dtype=dt), k=1)
        scale = dt.type(1.0 / math.sqrt(hd))
        for l in range(cfg.n_layers):
            p = f"layers.{l}."
            X = rmsnorm(H, w(p + "attn_norm"), eps)
            Q = (X @ w(p + "wq").T).reshape(n, hq, hd)
            K = (X @ w(p + "wk").T).reshape(n, hkv, hd)
            Vv = (X @ w(p + "wv").T).reshape(n, hkv, hd)
            Q = apply_rope(Q, C, S)
            K = bf16_round(apply_rope(K, C, S).astype(np.float32)).astype(dt)
            Vv = bf16_round(Vv.astype(np.float32)).astype(dt)
            kv[l, 0, :, :n, :] = K.transpose(1, 0, 2)
            kv[l, 1, :, :n, :] = Vv.transpose(1, 0, 2)
            O = np.empty((n, hq, hd), dtype=dt)
            for j in range(hq):
                g = j // G
                s = (Q[:, j, :] @ K[:, g, :].T) * scale + mask
                O[:, j, :] = softmax(s) @ Vv[:, g, :]
            H = H + O.reshape(n, -1) @ w(p + "wo").T
            X = rmsnorm(H, w(p + "ffn_norm"), eps)
            H = H + np.stack([self._ffn(l, X[i], None) for i in range(n)])
        X = rmsnorm(H, w("final_norm"), eps)
        W_lm = w("embed") if cfg.tied else w("lm_head")
        return X @ W_lm.T


def kv_to_oracle(kv_bf16, dtype=np.float32) -> np.ndarray:
    """Cache tensor (bf16 torch) -> oracle float array."""
    return np.asarray(kv_bf16.float().cpu().numpy(), dtype=dtype)
