"""GPU parity: the HIP megakernel (through the C ABI) against the CPU oracle,
element by element on the same seeded inputs, on the small shapes and launch
shapes (the full-size workloads' whole decode runs are in test_gpu_runs.py)."""
import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from persistent_megakernel_decode_02_amd import capi
from persistent_megakernel_decode_02_amd.decoder import Decoder
from persistent_megakernel_decode_02_amd.tuning import launch_config
from tests.gpu_common import ATOL, RTOL, check_run, close_enough, oracle_run, require_gpu, say

pytestmark = pytest.mark.gpu


def _setup(cfg, max_seq, filled, gain_std=0.0):
    require_gpu()
    w_gpu = synth.gen_weights(cfg, device="cuda", gain_std=gain_std)
    kv_gpu = synth.gen_kv_cache(cfg, max_seq, filled, device="cuda")
    torch.cuda.synchronize()
    return w_gpu, kv_gpu


def test_generator_identical_on_gpu_and_cpu():
    require_gpu()
    cfg = synth.PRESETS["tiny"]
    a = synth.gen_weights(cfg, device="cuda", gain_std=0.1)
    b = synth.gen_weights(cfg, device="cpu", gain_std=0.1)
    for x, y in zip(a, b):
        assert torch.equal(x.cpu(), y)
    assert torch.equal(synth.gen_kv_cache(cfg, 40, 33, device="cuda").cpu(), synth.gen_kv_cache(cfg, 40, 33))


@pytest.mark.parametrize("n_wg,n_chunks", [(256, 1), (7, 3), (1, 1), (64, 4), (33, 2)])
def test_tiny_prompt_then_greedy(n_wg, n_chunks):
    """Tiny config: a 32-token prompt run through the megakernel with forced
    tokens (the prefill), then 16 greedy steps, in one launch; the oracle does
    a batched causal prefill and 16 decode steps."""
    cfg = synth.PRESETS["tiny"]
    P, N = 32, 16
    prompt = synth.gen_tokens(P, cfg.vocab)
    w_gpu, kv_gpu = _setup(cfg, P + N, 0, gain_std=0.1)
    say(f"tiny n_wg={n_wg} n_chunks={n_chunks}")
    dec = Decoder(cfg, w_gpu, kv_gpu, P + N, n_wg=n_wg, n_chunks=n_chunks)
    forced = prompt + [-1] * N
    toks, logits = dec.decode(prompt[0], 0, P + N, forced=forced)
    toks, logits = toks.cpu().numpy(), logits.cpu().numpy()
    kv_after = kv_gpu.cpu()
    dec.close()

    w_cpu = synth.gen_weights(cfg, device="cpu", gain_std=0.1)
    orc = om.Oracle(cfg, om.Weights.from_list(cfg, w_cpu))
    kv_o = np.zeros((cfg.n_layers, 2, cfg.n_kv_heads, P + N, cfg.head_dim), dtype=np.float32)
    pre = orc.prefill(prompt, kv_o)
    ok, mx, nbad = close_enough(logits[:P], pre)
    say(f"prefill logits max|err| {mx:.3e}")
    assert ok, f"prefill logits: {nbad} outside tolerance"
    # the prompt positions' argmax (tokens_out) must match the oracle's
    assert [int(x) for x in toks[:P]] == [int(np.argmax(r)) for r in pre]
    otoks, ologits = orc.decode(int(np.argmax(pre[-1])), P, N, kv_o)
    # GPU step P consumes argmax of step P-1 (= the prefill's last row)
    check_run("tiny decode", toks[P:], logits[P:], otoks, ologits)
    # the cache the kernel appended: every position, K and V, all layers
    kv_g = kv_after.float().numpy()
    ok, mx, nbad = close_enough(kv_g, kv_o)
    say(f"kv cache max|err| {mx:.3e}")
    assert ok, f"kv cache: {nbad} values outside tolerance"


def test_tiny_kv_context_and_determinism():
    """Tiny config from a random-filled cache (the long-context recipe at
    small size); two launches from the same state are bit-identical and the
    pre-filled positions are left untouched."""
    cfg = synth.PRESETS["tiny"]
    T0, N = 200, 9
    w_gpu, kv_gpu = _setup(cfg, T0 + N, T0, gain_std=0.1)
    kv0 = kv_gpu.clone()
    dec = Decoder(cfg, w_gpu, kv_gpu, T0 + N, n_wg=64, n_chunks=5)
    first = synth.gen_tokens(1, cfg.vocab, stream=7)[0]
    t1, l1 = dec.decode(first, T0, N)
    t2, l2 = dec.decode(first, T0, N)
    assert torch.equal(t1, t2) and torch.equal(l1, l2), "two identical launches differ"
    assert torch.equal(kv_gpu[:, :, :, :T0], kv0[:, :, :, :T0])
    w_cpu = synth.gen_weights(cfg, device="cpu", gain_std=0.1)
    otoks, ologits, kv_o = oracle_run(cfg, w_cpu, synth.gen_kv_cache(cfg, T0 + N, T0), first, T0, N)
    check_run("tiny ctx", t1.cpu().numpy(), l1.cpu().numpy(), otoks, ologits)
    ok, mx, _ = close_enough(kv_gpu.cpu().float().numpy(), kv_o)
    assert ok, f"kv cache max err {mx}"


@pytest.mark.parametrize("n_wg,n_chunks", [(256, 1), (33, 2)])
def test_tiny_moe_kv_context(n_wg, n_chunks):
    """MoE opcodes (router, top-2, both experts' down rows in one
    instruction) on a small top-2 MoE from a random-filled cache."""
    cfg = synth.PRESETS["tiny_moe"]
    T0, N = 40, 8
    w_gpu, kv_gpu = _setup(cfg, T0 + N, T0, gain_std=0.1)
    say(f"tiny-moe n_wg={n_wg} n_chunks={n_chunks}")
    dec = Decoder(cfg, w_gpu, kv_gpu, T0 + N, n_wg=n_wg, n_chunks=n_chunks)
    first = synth.gen_tokens(1, cfg.vocab, stream=3)[0]
    toks, logits = dec.decode(first, T0, N)
    toks, logits = toks.cpu().numpy(), logits.cpu().numpy()
    kv_new = kv_gpu[:, :, :, T0:T0 + N].float().cpu().numpy()
    dec.close()
    w_cpu = synth.gen_weights(cfg, device="cpu", gain_std=0.1)
    otoks, ologits, kv_o = oracle_run(cfg, w_cpu, synth.gen_kv_cache(cfg, T0 + N, T0), first, T0, N)
    check_run("tiny-moe", toks, logits, otoks, ologits)
    ok, mx, _ = close_enough(kv_new, kv_o[:, :, :, T0:T0 + N])
    assert ok, f"appended kv max err {mx}"


def _random_shapes(n, seed=11):
    """Seeded launch shapes: model, grid size (1 to 256 workgroups), chunk count
    and start position."""
    import random
    rng = random.Random(seed)
    return [(rng.choice(["tiny", "tiny_moe"]), rng.choice([1, 3, 6, 13, 40, 77, 128, 191, 250, 256]),
             rng.choice([1, 1, 2, 3, 6, 8]), rng.randrange(0, 180)) for _ in range(n)]


@pytest.mark.parametrize("name,n_wg,n_chunks,T0", _random_shapes(12))
def test_tiny_random_launch_shapes(name, n_wg, n_chunks, T0):
    """Batch-1 dense and MoE kernels over seeded grids of 1 to 256 workgroups and
    1 to 8 chunks from random-filled caches: ragged tiles, several instructions
    per workgroup, empty chunks at short contexts."""
    cfg = synth.PRESETS[name]
    N = 4
    w_gpu, kv_gpu = _setup(cfg, T0 + N, T0, gain_std=0.1)
    say(f"{name} n_wg={n_wg} n_chunks={n_chunks} T0={T0}")
    dec = Decoder(cfg, w_gpu, kv_gpu, T0 + N, n_wg=n_wg, n_chunks=n_chunks)
    first = synth.gen_tokens(1, cfg.vocab, stream=5)[0]
    toks, logits = dec.decode(first, T0, N)
    toks, logits = toks.cpu().numpy(), logits.cpu().numpy()
    kv_new = kv_gpu[:, :, :, T0:T0 + N].float().cpu().numpy()
    dec.close()
    w_cpu = synth.gen_weights(cfg, device="cpu", gain_std=0.1)
    otoks, ologits, kv_o = oracle_run(cfg, w_cpu, synth.gen_kv_cache(cfg, T0 + N, T0), first, T0, N)
    check_run(f"{name} n_wg={n_wg}", toks, logits, otoks, ologits)
    ok, mx, _ = close_enough(kv_new, kv_o[:, :, :, T0:T0 + N])
    assert ok, f"appended kv max err {mx}"


# Shapes the library accepts beyond the presets: one q head per kv head (G = 1,
# attention instructions per head with and without split-KV), and MoE models
# with 4 experts (router rows requested before the input wait, as for 8) and
# 16 experts (more experts than wavefronts: the router is scored row by row),
# and an expert width that is not a whole number of 512-element segments.
EXTRA_SHAPES = {
    "tiny_g1": synth.ModelConfig("tiny-g1", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=4,
                                 head_dim=64, d_ff=768, vocab=1024, rope_theta=10000.0),
    "tiny_moe_e4": synth.ModelConfig("tiny-moe-e4", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2,
                                     head_dim=64, d_ff=512, vocab=1024, n_experts=4, top_k=2, rope_theta=1e6),
    "tiny_moe_e16": synth.ModelConfig("tiny-moe-e16", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2,
                                      head_dim=128, d_ff=512, vocab=1024, n_experts=16, top_k=2, rope_theta=1e6),
    # an expert width that is not a multiple of 512: each expert's activations
    # are fetched on their own, zero-padded to whole segments
    "tiny_moe_f768": synth.ModelConfig("tiny-moe-f768", n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2,
                                       head_dim=64, d_ff=768, vocab=1024, n_experts=8, top_k=2, rope_theta=1e6),
    # an attention width of three 512-element segments (12 q heads of 128, three
    # per kv head): the O-projection takes the runtime-length streamer
    "tiny_moe_q3": synth.ModelConfig("tiny-moe-q3", n_layers=2, d_model=256, n_q_heads=12, n_kv_heads=4,
                                     head_dim=128, d_ff=512, vocab=1024, n_experts=8, top_k=2, rope_theta=1e6),
}


@pytest.mark.parametrize("name,n_wg,n_chunks", [("tiny_g1", 256, 1), ("tiny_g1", 40, 3), ("tiny_moe_e4", 256, 1),
                                                ("tiny_moe_e4", 33, 2), ("tiny_moe_e16", 256, 1),
                                                ("tiny_moe_e16", 64, 4), ("tiny_moe_f768", 256, 1),
                                                ("tiny_moe_f768", 33, 2), ("tiny_moe_q3", 256, 1)])
def test_accepted_shapes_beyond_the_presets(name, n_wg, n_chunks):
    cfg = EXTRA_SHAPES[name]
    T0, N = 50, 8
    w_gpu, kv_gpu = _setup(cfg, T0 + N, T0, gain_std=0.1)
    say(f"{name} n_wg={n_wg} n_chunks={n_chunks}")
    dec = Decoder(cfg, w_gpu, kv_gpu, T0 + N, n_wg=n_wg, n_chunks=n_chunks)
    first = synth.gen_tokens(1, cfg.vocab, stream=6)[0]
    toks, logits = dec.decode(first, T0, N)
    toks, logits = toks.cpu().numpy(), logits.cpu().numpy()
    kv_new = kv_gpu[:, :, :, T0:T0 + N].float().cpu().numpy()
    dec.close()
    w_cpu = synth.gen_weights(cfg, device="cpu", gain_std=0.1)
    otoks, ologits, kv_o = oracle_run(cfg, w_cpu, synth.gen_kv_cache(cfg, T0 + N, T0), first, T0, N)
    check_run(name, toks, logits, otoks, ologits)
    ok, mx, _ = close_enough(kv_new, kv_o[:, :, :, T0:T0 + N])
    assert ok, f"appended kv max err {mx}"


@pytest.mark.parametrize("name,n_wg", [("tiny_moe", 256), ("tiny_moe", 33), ("tiny_moe_e4", 64), ("tiny_moe_q3", 64)])
def test_moe_expert_prediction_never_changes_the_result(name, n_wg):
    """MoE models predict each layer's experts from the pre-attention residual
    and stage the predicted expert's first gate/up rows early; the routed
    expert is always the router's.  Launches with the prediction on and off
    (the default) must be bit-identical, and the prediction counts must
    cover every gate/up tile that lies in one expert's half."""
    cfg = synth.PRESETS.get(name) or EXTRA_SHAPES[name]
    T0, N = 40, 12
    w_gpu, kv_gpu = _setup(cfg, T0 + N, T0, gain_std=0.1)
    kv0 = kv_gpu.clone()
    first = synth.gen_tokens(1, cfg.vocab, stream=8)[0]
    dec = Decoder(cfg, w_gpu, kv_gpu, T0 + N, n_wg=n_wg, n_chunks=1, expert_prediction=True)
    t_on, l_on = dec.decode(first, T0, N)
    hits, preds = capi.mkd_spec_stats(dec.handle)
    dec.close()
    kv_on = kv_gpu.clone()
    kv_gpu.copy_(kv0)
    dec = Decoder(cfg, w_gpu, kv_gpu, T0 + N, n_wg=n_wg, n_chunks=1)   # off: the default
    t_off, l_off = dec.decode(first, T0, N)
    assert capi.mkd_spec_stats(dec.handle) == (0, 0)
    dec.close()
    say(f"{name} n_wg={n_wg}: {hits} of {preds} predictions named the routed expert")
    assert preds > 0
    assert torch.equal(t_on, t_off) and torch.equal(l_on, l_off), "prediction changed the result"
    assert torch.equal(kv_on, kv_gpu)
