"""GPU parity of batched decode: B sequences decoded together in one launch
(each weight row read once per step for all of them), each sequence checked
against its own oracle run from its own cache and start position."""
import numpy as np
import pytest
import torch

import synth
from persistent_megakernel_decode_02_amd import capi
from persistent_megakernel_decode_02_amd.decoder import Decoder
from tests.gpu_common import check_run, close_enough, oracle_run, require_gpu, say

pytestmark = pytest.mark.gpu

STARTS = [40, 13, 77, 1, 0, 120, 31, 64]


def _caches(cfg, max_seq, starts, device):
    """One random-filled cache per sequence (its own seed), filled up to its start."""
    return [synth.gen_kv_cache(cfg, max_seq, s, seed=synth.SEED_KV + 101 * b, device=device)
            for b, s in enumerate(starts)]


def _run_batched(cfg, starts, N, n_wg, n_chunks, gain_std, lds_limits=None):
    B = len(starts)
    max_seq = max(starts) + N
    w_gpu = synth.gen_weights(cfg, device="cuda", gain_std=gain_std)
    kv_gpu = torch.stack(_caches(cfg, max_seq, starts, "cuda")).contiguous()
    kv0 = kv_gpu.clone()
    firsts = synth.gen_tokens(B, cfg.vocab, stream=11)
    say(f"{cfg.name} B={B} starts={starts} steps={N} n_wg={n_wg} n_chunks={n_chunks}")
    dec = Decoder(cfg, w_gpu, kv_gpu, max_seq, n_wg=n_wg, n_chunks=n_chunks, batch=B, lds_limits=lds_limits)
    toks, logits = dec.decode_batch(firsts, starts, N)
    toks2, logits2 = dec.decode_batch(firsts, starts, N)
    assert torch.equal(toks, toks2) and torch.equal(logits, logits2), "two identical launches differ"
    dec.close()
    for b, s in enumerate(starts):
        # positions before each sequence's start are left untouched
        assert torch.equal(kv_gpu[b, :, :, :, :s], kv0[b, :, :, :, :s]), f"seq {b}: cache prefix changed"
    out = (toks.cpu().numpy(), logits.cpu().numpy(), kv_gpu.float().cpu().numpy(), firsts, max_seq)
    del w_gpu, kv_gpu, kv0
    torch.cuda.empty_cache()
    return out


def _check_against_oracle(cfg, starts, N, res, gain_std):
    toks, logits, kv_g, firsts, max_seq = res
    w_cpu = synth.gen_weights(cfg, device="cpu", gain_std=gain_std)
    for b, (s, kv_cpu) in enumerate(zip(starts, _caches(cfg, max_seq, starts, "cpu"))):
        otoks, ologits, kv_o = oracle_run(cfg, w_cpu, kv_cpu, firsts[b], s, N)
        check_run(f"{cfg.name} B={len(starts)} seq {b}", toks[b], logits[b], otoks, ologits)
        ok, mx, _ = close_enough(kv_g[b][:, :, :, s:s + N], kv_o[:, :, :, s:s + N])
        assert ok, f"seq {b}: appended kv max err {mx}"


@pytest.mark.parametrize("B,n_wg,n_chunks", [(2, 256, 1), (3, 33, 2), (4, 64, 4), (5, 7, 3),
                                             (8, 256, 1), (8, 40, 2)])
def test_tiny_batched_kv_context(B, n_wg, n_chunks):
    require_gpu()
    cfg = synth.PRESETS["tiny"]
    starts, N = STARTS[:B], 6
    res = _run_batched(cfg, starts, N, n_wg, n_chunks, 0.1)
    _check_against_oracle(cfg, starts, N, res, 0.1)


@pytest.mark.parametrize("B,n_wg,n_chunks", [(3, 33, 2), (8, 256, 1)])
def test_tiny_batched_down_projection_in_passes(B, n_wg, n_chunks):
    """The LDS input area capped to one 512-element segment of every sequence: the
    down projection (d_ff 768) then streams its rows in two passes over K,
    the second ragged, adding to the first pass's partial sums."""
    require_gpu()
    cfg = synth.PRESETS["tiny"]
    starts, N = STARTS[:B], 5
    res = _run_batched(cfg, starts, N, n_wg, n_chunks, 0.1, lds_limits=(64 * (8 * B + 4), -1))
    _check_against_oracle(cfg, starts, N, res, 0.1)


def _random_shapes(n, seed=7):
    """Seeded launch shapes: batch, grid size (1 to 256 workgroups), chunk count
    and per-sequence start positions."""
    import random
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        B = rng.choice([2, 3, 4, 5, 6, 7, 8])
        n_wg = rng.choice([1, 2, 5, 9, 17, 31, 48, 100, 128, 200, 255, 256])
        n_chunks = rng.choice([1, 1, 2, 3, 5, 8])
        out.append((B, n_wg, n_chunks, [rng.randrange(0, 150) for _ in range(B)]))
    return out


@pytest.mark.parametrize("B,n_wg,n_chunks,starts", _random_shapes(14))
def test_tiny_batched_random_launch_shapes(B, n_wg, n_chunks, starts):
    """Every batch size 2-8 over grids of 1 to 256 workgroups and 1 to 8 chunks:
    ragged tiles, several instructions per workgroup, partial staging."""
    require_gpu()
    cfg = synth.PRESETS["tiny"]
    res = _run_batched(cfg, starts, 3, n_wg, n_chunks, 0.1)
    _check_against_oracle(cfg, starts, 3, res, 0.1)


@pytest.mark.parametrize("B,n_wg", [(2, 7), (4, 256), (3, 33)])
def test_tiny_batched_staged_gate_up_bit_exact(B, n_wg):
    """Gate/up weight rows staged in LDS during the attention phase are consumed in
    the order the streamer would load them, so the results are bit-identical to a
    launch with no staging (staged units limited to 0). n_wg 7 stages 4 of a wavefront's 7
    steps (the rest streamed); n_wg 256 stages every step."""
    require_gpu()
    cfg = synth.PRESETS["tiny"]
    starts, N = STARTS[:B], 4
    staged = _run_batched(cfg, starts, N, n_wg, 1, 0.1)
    plain = _run_batched(cfg, starts, N, n_wg, 1, 0.1, lds_limits=(0, 0))
    assert np.array_equal(staged[0], plain[0]), "tokens differ with staging"
    assert np.array_equal(staged[1], plain[1]), "logits differ with staging"
    assert np.array_equal(staged[2], plain[2]), "caches differ with staging"


def test_llama1b_batched_full_size_b8():
    """Eight sequences on the 1B shape: the interleaved down-projection input
    (8192 x 8 floats) does not fit in LDS, so it streams in passes over K."""
    require_gpu()
    cfg = synth.PRESETS["llama1b"]
    starts, N = [128, 96, 131, 64, 1, 200, 128, 17], 2
    res = _run_batched(cfg, starts, N, 0, 0, 0.0)
    _check_against_oracle(cfg, starts, N, res, 0.0)


@pytest.mark.parametrize("starts", [[128, 96, 131, 64], [128, 300]])
def test_llama1b_batched_full_size(starts):
    """Four and two sequences at different cache lengths on the 1B shape (gate/up
    rows staged in LDS: 3 of each wavefront's 8 steps at B = 4, 4 at B = 2)."""
    require_gpu()
    cfg = synth.PRESETS["llama1b"]
    N = 3
    res = _run_batched(cfg, starts, N, 0, 0, 0.0)
    _check_against_oracle(cfg, starts, N, res, 0.0)


def test_batched_handle_rejects_single_sequence_call():
    require_gpu()
    cfg = synth.PRESETS["tiny"]
    w = synth.gen_weights(cfg, device="cuda")
    kv = torch.stack(_caches(cfg, 64, [8, 8], "cuda")).contiguous()
    dec = Decoder(cfg, w, kv, 64, batch=2)
    toks = torch.empty(4, dtype=torch.int32, device="cuda")
    with pytest.raises(capi.MkdError):
        capi.mkd_decode(dec.handle, 1, 8, 4, toks)
    # a start position past the cache is rejected before launch
    toks2 = torch.empty(2, 4, dtype=torch.int32, device="cuda")
    with pytest.raises(capi.MkdError):
        capi.mkd_decode_batch(dec.handle, [1, 2], [8, 62], 4, toks2)
    dec.close()
