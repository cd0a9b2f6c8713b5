"""Pins of the CPU oracle against closed forms, invariants, library routines and
brute force -- none of them re-derives the oracle's own vectorised code."""
import math
import random

import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from synth import ModelConfig


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_round_matches_torch_rne():
    """Library routine: torch's fp32 -> bf16 conversion rounds to nearest even."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0], dtype=np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(om.bf16_round(x), ref)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa is 1.0
    assert om.bf16_round(np.float32([1.0 + 2 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert om.bf16_round(np.float32([1.0 + 3 * 2 ** -8]))[0] == np.float32(1.0 + 2 ** -6)


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_unit_rms_closed_form():
    """gamma = 1: RMS(out) = sqrt(m / (m + eps)) with m = mean(h^2)."""
    rng = np.random.default_rng(1)
    for d, eps in [(256, 1e-5), (2048, 1e-5), (7, 0.5)]:
        h = rng.standard_normal(d) * 3.0
        out = om.rmsnorm(h, np.ones(d), eps)
        m = float(np.mean(h * h))
        assert math.isclose(math.sqrt(float(np.mean(out * out))), math.sqrt(m / (m + eps)), rel_tol=1e-12)


def test_rmsnorm_hand_example_and_gain():
    out = om.rmsnorm(np.array([3.0, 4.0]), np.array([1.0, 1.0]), 0.0)
    assert np.allclose(out, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    g = np.array([2.0, -0.5])
    assert np.allclose(om.rmsnorm(np.array([3.0, 4.0]), g, 0.0), out * g, atol=1e-15)


def test_rmsnorm_scale_invariance():
    rng = np.random.default_rng(2)
    h = rng.standard_normal(512)
    g = 1 + 0.1 * rng.standard_normal(512)
    a = om.rmsnorm(h, g, 1e-5)
    b = om.rmsnorm(1000.0 * h, g, 1e-5)
    assert np.allclose(a, b, rtol=1e-5, atol=0)


# ---------------------------------------------------------------- RoPE

def test_rope_position_zero_is_identity():
    c, s = om.rope_cos_sin(0, 64, 10000.0)
    assert np.all(c == 1.0) and np.all(s == 0.0)
    x = np.random.default_rng(3).standard_normal((4, 64)).astype(np.float32)
    assert np.array_equal(om.apply_rope(x, c, s), x)


def test_rope_pairs_half_split_and_angle():
    """Unit vector e_i goes to cos(a) e_i + sin(a) e_{i+hd/2}, a = p * theta^(-2i/hd)."""
    hd, theta, p = 64, 500000.0, 37
    c, s = om.rope_cos_sin(p, hd, theta)
    for i in (0, 1, 17, 31):
        e = np.zeros(hd, dtype=np.float32)
        e[i] = 1.0
        out = om.apply_rope(e, c, s)
        a = p * theta ** (-2.0 * i / hd)
        want = np.zeros(hd)
        want[i] = math.cos(a)
        want[i + hd // 2] = math.sin(a)
        assert np.allclose(out, want, atol=1e-7)


def test_rope_preserves_pair_norms():
    rng = np.random.default_rng(4)
    hd = 128
    x = rng.standard_normal((8, hd)).astype(np.float32)
    for p in (1, 100, 32767):
        c, s = om.rope_cos_sin(p, hd, 1e6)
        y = om.apply_rope(x, c, s)
        n0 = x[:, :hd // 2] ** 2 + x[:, hd // 2:] ** 2
        n1 = y[:, :hd // 2] ** 2 + y[:, hd // 2:] ** 2
        assert np.allclose(n0, n1, rtol=2e-6, atol=1e-6)


def test_rope_relative_position_identity():
    """<R_m q, R_n k> = <R_(m-n) q, k>: scores depend on the offset only."""
    rng = np.random.default_rng(5)
    hd = 64
    q = rng.standard_normal(hd).astype(np.float32)
    k = rng.standard_normal(hd).astype(np.float32)
    for m, n in [(10, 3), (1000, 999), (4096, 17)]:
        cm, sm = om.rope_cos_sin(m, hd, 10000.0)
        cn, sn = om.rope_cos_sin(n, hd, 10000.0)
        cd, sd = om.rope_cos_sin(m - n, hd, 10000.0)
        lhs = float(np.dot(om.apply_rope(q, cm, sm).astype(np.float64), om.apply_rope(k, cn, sn)))
        rhs = float(np.dot(om.apply_rope(q, cd, sd).astype(np.float64), k))
        assert abs(lhs - rhs) <= 1e-4 * (1 + abs(rhs))


# ---------------------------------------------------------------- attention

def _attn_brute(q, K, V):
    """fp64 loops: o_j = sum_t softmax_t(q_j.K_g(t)/sqrt(hd)) V_g(t), g = j // G."""
    hq, hd = len(q), len(q[0])
    hkv = len(K)
    G = hq // hkv
    out = []
    for j in range(hq):
        g = j // G
        T = len(K[g])
        s = [sum(q[j][i] * K[g][t][i] for i in range(hd)) / math.sqrt(hd) for t in range(T)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = sum(e)
        out.append([sum(e[t] / z * V[g][t][i] for t in range(T)) for i in range(hd)])
    return out


@pytest.mark.parametrize("hq,hkv,hd,T", [(4, 2, 8, 5), (3, 1, 4, 8), (6, 2, 8, 1), (4, 4, 2, 3)])
def test_attention_brute_force(hq, hkv, hd, T):
    rng = np.random.default_rng(hq * 100 + T)
    q = rng.standard_normal((hq, hd))
    K = rng.standard_normal((hkv, T, hd))
    V = rng.standard_normal((hkv, T, hd))
    ref = np.array(_attn_brute(q.tolist(), K.tolist(), V.tolist()))
    assert np.allclose(om.attention(q, K, V), ref, rtol=1e-12, atol=1e-12)


def test_attention_single_position_returns_value():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 8)).astype(np.float32)
    K = rng.standard_normal((2, 1, 8)).astype(np.float32)
    V = rng.standard_normal((2, 1, 8)).astype(np.float32)
    o = om.attention(q, K, V)
    # q heads 0,1 read kv head 0; 2,3 read kv head 1 (grouped, not interleaved)
    assert np.array_equal(o, V[[0, 0, 1, 1], 0, :])


def test_attention_equal_keys_average_values():
    rng = np.random.default_rng(7)
    K = np.repeat(rng.standard_normal((1, 1, 16)), 9, axis=1)
    V = rng.standard_normal((1, 9, 16))
    o = om.attention(rng.standard_normal((2, 16)), K, V)
    assert np.allclose(o, V[0].mean(axis=0), atol=1e-14)


def test_attention_scale_closed_form():
    """Two keys with scores x/sqrt(hd) and 0: weights are a logistic of x/sqrt(hd)."""
    hd, x = 16, 3.0
    q = np.zeros((1, hd)); q[0, 0] = 1.0
    K = np.zeros((1, 2, hd)); K[0, 0, 0] = x
    V = np.zeros((1, 2, hd)); V[0, 0, 1] = 1.0; V[0, 1, 2] = 1.0
    p0 = 1.0 / (1.0 + math.exp(-x / 4.0))
    o = om.attention(q, K, V)
    assert math.isclose(o[0, 1], p0, rel_tol=1e-14) and math.isclose(o[0, 2], 1 - p0, rel_tol=1e-14)


def test_split_kv_merge_equals_whole():
    """Log-sum-exp merge of any chunking of the positions gives the same output
    (the merge the GPU's split-KV reduction performs, checked on the oracle)."""
    rng = np.random.default_rng(8)
    hd = 8
    for T in range(1, 17):
        q = rng.standard_normal((1, hd))
        K = rng.standard_normal((1, T, hd))
        V = rng.standard_normal((1, T, hd))
        whole = om.attention(q, K, V)[0]
        for n_chunks in range(1, T + 1):
            bounds = np.linspace(0, T, n_chunks + 1).astype(int)
            ms, ls, os_ = [], [], []
            for c in range(n_chunks):
                lo, hi = bounds[c], bounds[c + 1]
                if lo == hi:
                    continue
                s = K[0, lo:hi] @ q[0] / math.sqrt(hd)
                m = s.max()
                e = np.exp(s - m)
                ms.append(m); ls.append(e.sum()); os_.append(e @ V[0, lo:hi])
            M = max(ms)
            l = sum(math.exp(m - M) * x for m, x in zip(ms, ls))
            o = sum(math.exp(m - M) * x for m, x in zip(ms, os_)) / l
            assert np.allclose(o, whole, atol=1e-12)


# ---------------------------------------------------------------- SiLU, GEMV

def test_silu_limits_and_reference():
    z = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 2.5])
    s = om.silu(z)
    assert s[0] == 0.0
    assert abs(s[3] - 30.0) < 1e-11 and abs(s[4]) < 1e-11
    for zi, si in zip(z, s):
        assert math.isclose(si, zi / (1 + math.exp(-zi)), rel_tol=1e-15, abs_tol=1e-300)


def test_gemv_fp32_within_summation_bound():
    """fp32 matvec of exact bf16 inputs vs an exact (fsum) dot: Higham's bound
    |err| <= gamma_n sum|w x|, gamma_n = n u / (1 - n u), u = 2^-24."""
    rng = np.random.default_rng(9)
    for n in (256, 2048, 8192):
        W = om.bf16_round(rng.standard_normal((16, n)).astype(np.float32) * 0.02)
        x = rng.standard_normal(n).astype(np.float32)
        y = W @ x
        u = 2.0 ** -24
        gam = n * u / (1 - n * u)
        for r in range(16):
            exact = math.fsum(float(a) * float(b) for a, b in zip(W[r], x))
            bound = gam * math.fsum(abs(float(a) * float(b)) for a, b in zip(W[r], x))
            assert abs(float(y[r]) - exact) <= bound


# ---------------------------------------------------------------- MoE routing, argmax

def test_top2_is_best_pair_exhaustive():
    rng = np.random.default_rng(10)
    for trial in range(200):
        z = rng.standard_normal(8).astype(np.float32)
        if trial % 5 == 0:
            z[rng.integers(8)] = z[rng.integers(8)]  # plant a tie
        (a, b), w = om.top2_route(z)
        best = max(((float(z[i]) + float(z[j]), -i, -j) for i in range(8) for j in range(8) if i != j))
        assert float(z[a]) + float(z[b]) == best[0]
        assert z[a] >= z[b]
        if z[a] == z[b]:
            assert a < b
        ea, eb = math.exp(float(z[a])), math.exp(float(z[b]))
        assert math.isclose(float(w[0]), ea / (ea + eb), rel_tol=1e-6)
        assert math.isclose(float(w[0] + w[1]), 1.0, rel_tol=1e-6)


def test_top2_tie_rule():
    z = np.array([0.5, 2.0, 1.0, 2.0, 1.0, 2.0, 0.0, 0.0], dtype=np.float32)
    (a, b), w = om.top2_route(z)
    assert (a, b) == (1, 3) and w[0] == w[1] == 0.5


def test_argmax_first_occurrence():
    x = np.array([1.0, 3.0, 2.0, 3.0, -1.0])
    assert om.argmax_first(x) == 1
    assert om.argmax_first(np.array([-5.0, -5.0])) == 0


# ---------------------------------------------------------------- brute-force micro models

MICRO_DENSE = ModelConfig("micro", n_layers=2, d_model=8, n_q_heads=4, n_kv_heads=2,
                          head_dim=4, d_ff=12, vocab=16, rope_theta=10000.0)
MICRO_MOE = ModelConfig("micro-moe", n_layers=2, d_model=8, n_q_heads=2, n_kv_heads=1,
                        head_dim=8, d_ff=6, vocab=10, n_experts=4, top_k=2, rope_theta=1e6)
MICRO_TIED = ModelConfig("micro-tied", n_layers=1, d_model=8, n_q_heads=2, n_kv_heads=2,
                         head_dim=4, d_ff=4, vocab=12, tied=True, rope_theta=500000.0)


def _brute_step(cfg, W, token, pos, cache):
    """One decode step written as explicit loops over indices (fp64, math).

    W maps names to nested lists with matrices stored [out][in]; cache maps
    (layer, 'k'|'v', kv_head) to a list of per-position vectors (bf16 values).
    """
    d, hd, hq, hkv = cfg.d_model, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads
    G = hq // hkv

    def mv(M, x):
        return [sum(M[r][c] * x[c] for c in range(len(x))) for r in range(len(M))]

    def norm(h, g):
        ms = sum(v * v for v in h) / len(h)
        return [h[i] / math.sqrt(ms + cfg.rms_eps) * g[i] for i in range(len(h))]

    def rot(x):
        out = list(x)
        for i in range(hd // 2):
            a = pos * cfg.rope_theta ** (-2.0 * i / hd)
            c, s = float(np.float32(math.cos(a))), float(np.float32(math.sin(a)))
            out[i] = x[i] * c - x[i + hd // 2] * s
            out[i + hd // 2] = x[i + hd // 2] * c + x[i] * s
        return out

    def bf(x):
        return [float(om.bf16_round(np.float32([v]))[0]) for v in x]

    def ffn(prefix, x):
        if not cfg.is_moe:
            g, u = mv(W[prefix + "w_gate"], x), mv(W[prefix + "w_up"], x)
            a = [g[i] / (1 + math.exp(-g[i])) * u[i] for i in range(len(g))]
            return mv(W[prefix + "w_down"], a)
        z = mv(W[prefix + "router"], x)
        best = None
        for i in range(len(z)):
            for j in range(len(z)):
                if i != j and (z[i] > z[j] or (z[i] == z[j] and i < j)):
                    key = (z[i] + z[j], -i, -j)
                    if best is None or key > best[0]:
                        best = (key, i, j)
        _, e1, e2 = best
        w1 = 1.0 / (1.0 + math.exp(z[e2] - z[e1]))
        out = [0.0] * d
        for e, wt in ((e1, w1), (e2, 1.0 - w1)):
            g, u = mv(W[prefix + f"gate.{e}"], x), mv(W[prefix + f"up.{e}"], x)
            a = [g[i] / (1 + math.exp(-g[i])) * u[i] for i in range(len(g))]
            dn = mv(W[prefix + f"down.{e}"], a)
            out = [out[i] + wt * dn[i] for i in range(d)]
        return out

    h = list(W["embed"][token])
    for l in range(cfg.n_layers):
        p = f"layers.{l}."
        x = norm(h, W[p + "attn_norm"])
        q, k, v = mv(W[p + "wq"], x), mv(W[p + "wk"], x), mv(W[p + "wv"], x)
        att = []
        for g in range(hkv):
            cache[(l, "k", g)].append(bf(rot(k[g * hd:(g + 1) * hd])))
            cache[(l, "v", g)].append(bf(v[g * hd:(g + 1) * hd]))
            assert len(cache[(l, "k", g)]) == pos + 1
        for j in range(hq):
            g = j // G
            qj = rot(q[j * hd:(j + 1) * hd])
            Ks, Vs = cache[(l, "k", g)], cache[(l, "v", g)]
            s = [sum(qj[i] * Ks[t][i] for i in range(hd)) / math.sqrt(hd) for t in range(pos + 1)]
            m = max(s)
            e = [math.exp(v_ - m) for v_ in s]
            z = sum(e)
            att += [sum(e[t] / z * Vs[t][i] for t in range(pos + 1)) for i in range(hd)]
        o = mv(W[p + "wo"], att)
        h = [h[i] + o[i] for i in range(d)]
        x = norm(h, W[p + "ffn_norm"])
        f = ffn(p, x)
        h = [h[i] + f[i] for i in range(d)]
    x = norm(h, W["final_norm"])
    return mv(W["embed"] if cfg.tied else W["lm_head"], x)


@pytest.mark.parametrize("cfg", [MICRO_DENSE, MICRO_MOE, MICRO_TIED], ids=lambda c: c.name)
def test_oracle_matches_brute_force_micro_model(cfg):
    ws = synth.gen_weights(cfg, seed=11, gain_std=0.3, std=0.3)
    names = [n for n, _ in synth.weight_specs(cfg)]
    W = {n: t.float().tolist() for n, t in zip(names, ws)}
    orc = om.Oracle(cfg, om.Weights.from_list(cfg, ws, dtype=np.float64))
    n_steps = 5
    kv = np.zeros((cfg.n_layers, 2, cfg.n_kv_heads, n_steps, cfg.head_dim))
    cache = {(l, kk, g): [] for l in range(cfg.n_layers) for kk in "kv" for g in range(cfg.n_kv_heads)}
    toks = synth.gen_tokens(n_steps, cfg.vocab, seed=3)
    for pos, tok in enumerate(toks):
        ref = _brute_step(cfg, W, tok, pos, cache)
        got = orc.step(tok, pos, kv)
        assert np.allclose(got, ref, rtol=1e-9, atol=1e-9), (pos, np.max(np.abs(got - ref)))


# ---------------------------------------------------------------- KV cache logic, noise floor

@pytest.mark.parametrize("cfg", [synth.PRESETS["tiny"], MICRO_MOE], ids=lambda c: c.name)
def test_incremental_decode_equals_prefill(cfg):
    ws = synth.gen_weights(cfg, seed=0, gain_std=0.1)
    n = 12
    toks = synth.gen_tokens(n, cfg.vocab)
    orc = om.Oracle(cfg, om.Weights.from_list(cfg, ws, dtype=np.float64))
    kv_a = np.zeros((cfg.n_layers, 2, cfg.n_kv_heads, n, cfg.head_dim))
    kv_b = np.zeros_like(kv_a)
    pre = orc.prefill(toks, kv_a)
    _, dec = orc.decode(toks[0], 0, n, kv_b, forced=toks)
    assert np.allclose(pre, dec, rtol=1e-9, atol=1e-9)
    assert np.array_equal(kv_a, kv_b)


@pytest.mark.parametrize("cfg,std,seed", [(synth.PRESETS["tiny"], 0.02, 2), (MICRO_MOE, 0.5, 2),
                                          (MICRO_TIED, 0.5, 8)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_greedy_decode_feeds_each_argmax_to_the_next_step(cfg, std, seed):
    """The free-running branch of Oracle.decode: step i consumes the argmax of
    step i-1.  A causal prefill over [first] + tokens[:-1] -- no incremental
    cache and no token feed of its own -- must give every step's logits, and
    each row's argmax must be the token decode returned for that step.  The
    run must visit several tokens, so that feeding the wrong step's token
    (an off-by-one) would change the logits."""
    ws = synth.gen_weights(cfg, seed=seed, gain_std=0.1, std=std)
    n = 12
    first = synth.gen_tokens(1, cfg.vocab, stream=4)[0]
    orc = om.Oracle(cfg, om.Weights.from_list(cfg, ws, dtype=np.float64))
    kv_a = np.zeros((cfg.n_layers, 2, cfg.n_kv_heads, n, cfg.head_dim))
    toks, logits = orc.decode(first, 0, n, kv_a)
    assert len(set(toks)) >= 4, f"degenerate greedy run {toks}"
    assert any(a != b for a, b in zip(toks, toks[1:]))
    kv_b = np.zeros_like(kv_a)
    pre = orc.prefill([first] + toks[:-1], kv_b)
    assert np.allclose(pre, logits, rtol=1e-9, atol=1e-9)
    assert [int(np.argmax(r)) for r in pre] == toks
    assert np.array_equal(kv_a, kv_b)


def test_fp32_oracle_within_noise_floor_of_fp64():
    cfg = synth.PRESETS["tiny"]
    ws = synth.gen_weights(cfg, seed=0)
    T0, n = 32, 8
    kv0 = synth.gen_kv_cache(cfg, T0 + n, T0)
    outs = []
    for dt in (np.float32, np.float64):
        orc = om.Oracle(cfg, om.Weights.from_list(cfg, ws, dtype=dt))
        kv = om.kv_to_oracle(kv0, dt)
        outs.append(orc.decode(5, T0, n, kv)[1].astype(np.float64))
    assert np.max(np.abs(outs[0] - outs[1])) < 1e-4


# ---------------------------------------------------------------- generator

def test_generator_is_deterministic_and_shaped():
    cfg = synth.PRESETS["tiny"]
    a = synth.gen_weights(cfg, seed=0)
    b = synth.gen_weights(cfg, seed=0)
    c = synth.gen_weights(cfg, seed=1)
    for x, y, (name, shape) in zip(a, b, synth.weight_specs(cfg)):
        assert tuple(x.shape) == shape and x.dtype == torch.bfloat16
        assert torch.equal(x, y)
    assert not torch.equal(a[0], c[0])
    big = synth.gen_bf16(0, 99, (1 << 20,), 0.02).float()
    assert abs(big.mean().item()) < 1e-4 and abs(big.std().item() - 0.02) < 2e-4
    toks = synth.gen_tokens(1000, 1024)
    assert min(toks) >= 0 and max(toks) < 1024 and len(set(toks)) > 500
