"""Failure handling on the device, forced from the host.

The host's stop word (mkd_abort; Hyperkernel teardown, "Hardware fault
detection and replanning": a stop word in the kernel's control block) must end
a running launch at whichever wait each workgroup is in, report
MKD_E_ABORTED, and leave the model usable: the next launch from the same
position decodes the same tokens as before.  A stop asked for while nothing
runs must not leak into the next launch.  No test here makes the device fault
or hang: every device-side wait polls the stop word and its own watchdog
deadline.
"""
import pytest
import torch

import synth
from persistent_megakernel_decode_02_amd import capi
from persistent_megakernel_decode_02_amd.decoder import Decoder
from tests.gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu


def _tiny(max_seq, filled):
    cfg = synth.TINY
    w = synth.gen_weights(cfg, device="cuda")
    kv = synth.gen_kv_cache(cfg, max_seq, filled, device="cuda")
    return cfg, w, kv


def test_abort_ends_a_running_launch_and_the_model_still_decodes():
    require_gpu()
    T0, max_seq, long_n = 32, 4096, 4000
    cfg, w, kv = _tiny(max_seq, T0)
    dec = Decoder(cfg, w, kv, max_seq)
    first = int(synth.gen_tokens(1, cfg.vocab)[0])
    ref, _ = dec.decode(first, T0, 8, want_logits=False)
    ref = [int(x) for x in ref.cpu()]
    say(f"reference tokens {ref}")

    # 4000 steps take far longer than the few microseconds between the
    # enqueue and the stop request: the launch cannot finish first
    toks = torch.empty(long_n, dtype=torch.int32, device="cuda")
    dec.launch(first, T0, long_n, toks)
    capi.mkd_abort(dec.handle)
    st = capi.mkd_wait(dec.handle, 60000, raise_on_error=False)
    say(f"stopped launch: code {st.code} at workgroup {st.wg}, instruction {st.instr}, step {st.token}")
    assert st.code == capi.MKD_E_ABORTED
    assert 0 <= st.token < long_n

    again, _ = dec.decode(first, T0, 8, want_logits=False)
    again = [int(x) for x in again.cpu()]
    say(f"after the abort {again}")
    assert again == ref
    dec.close()


def test_abort_while_idle_does_not_stop_the_next_launch():
    """mkd_abort on a handle with nothing in flight has no effect: the next
    decode returns MKD_OK with the reference tokens (a leaking stop word
    would end it through its own bounded wait with MKD_E_ABORTED instead)."""
    require_gpu()
    T0, max_seq = 32, 256
    cfg, w, kv = _tiny(max_seq, T0)
    dec = Decoder(cfg, w, kv, max_seq)
    first = int(synth.gen_tokens(1, cfg.vocab)[0])
    ref, _ = dec.decode(first, T0, 100, want_logits=False)
    capi.mkd_abort(dec.handle)             # idle: after a completed, waited-for launch
    toks = torch.empty(100, dtype=torch.int32, device="cuda")
    dec.launch(first, T0, 100, toks)
    st = capi.mkd_wait(dec.handle, 60000, raise_on_error=False)
    say(f"launch after an idle abort: code {st.code}")
    assert st.code == capi.MKD_OK
    assert torch.equal(toks, ref)
    dec.close()


def test_second_launch_while_one_runs_is_rejected():
    """A handle runs one launch at a time: a decode enqueued before the running
    one was waited for is refused on the host (its buffer reset would clear
    the running launch's flags), and the running launch completes normally."""
    require_gpu()
    T0, max_seq, n = 32, 4096, 3000
    cfg, w, kv = _tiny(max_seq, T0)
    dec = Decoder(cfg, w, kv, max_seq)
    first = int(synth.gen_tokens(1, cfg.vocab)[0])
    toks = torch.empty(n, dtype=torch.int32, device="cuda")
    dec.launch(first, T0, n, toks)
    other = torch.empty(4, dtype=torch.int32, device="cuda")
    with pytest.raises(capi.MkdError) as e:
        dec.launch(first, T0, 4, other)
    assert e.value.code == capi.MKD_E_INVALID
    st = capi.mkd_wait(dec.handle, 60000, raise_on_error=False)
    assert st.code == capi.MKD_OK
    dec.close()


def test_watchdog_setting_is_validated():
    require_gpu()
    cfg, w, kv = _tiny(64, 32)
    dec = Decoder(cfg, w, kv, 64)
    with pytest.raises(capi.MkdError):
        capi.mkd_set_watchdog(dec.handle, 0)
    capi.mkd_set_watchdog(dec.handle, 5000)
    toks, _ = dec.decode(3, 32, 4, want_logits=False)
    assert toks.numel() == 4
    dec.close()


def test_expert_prediction_setting_is_validated():
    """mkd_set_expert_prediction takes 0 or 1; on a dense model it is accepted
    and changes nothing (no predictions are counted)."""
    require_gpu()
    cfg, w, kv = _tiny(64, 32)
    dec = Decoder(cfg, w, kv, 64)
    ref, _ = dec.decode(3, 32, 4, want_logits=False)
    for bad in (2, -1):
        with pytest.raises(capi.MkdError) as e:   # (the binding passes only 0 or 1)
            capi._check(capi.load().mkd_set_expert_prediction(dec.handle, bad))
        assert e.value.code == capi.MKD_E_INVALID
    capi.mkd_set_expert_prediction(dec.handle, True)
    toks, _ = dec.decode(3, 32, 4, want_logits=False)
    assert torch.equal(toks, ref)
    assert capi.mkd_spec_stats(dec.handle) == (0, 0)
    dec.close()


def test_workspace_too_small_for_a_schedule_is_rejected():
    """A schedule whose instruction tensor and activations do not fit in the
    handle's workspace is refused on the host with the size it needs."""
    require_gpu()
    cfg, w, kv = _tiny(64, 32)
    dec = Decoder(cfg, w, kv, 64, n_wg=8, n_chunks=1)
    with pytest.raises(capi.MkdError) as e:
        dec.rebuild(n_wg=256, n_chunks=8)  # a longer schedule and more split-KV partials
    assert e.value.code == capi.MKD_E_INVALID and "workspace" in str(e.value)
    dec.rebuild(n_wg=8, n_chunks=1)
    toks, _ = dec.decode(3, 32, 4, want_logits=False)
    assert toks.numel() == 4
    dec.close()


def test_read_probe_runs_and_reads_the_whole_buffer():
    """mkd_read_probe streams a device buffer; it writes its sink only if the
    XOR of everything read equals a value a buffer of ones cannot give, so the
    sink stays 0, and it runs at a plausible HBM rate."""
    require_gpu()
    buf = torch.ones(1 << 26, dtype=torch.int32, device="cuda")   # 256 MiB
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    capi.mkd_read_probe(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    capi.mkd_read_probe(buf, sink)
    e1.record()
    e1.synchronize()
    gbs = buf.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    say(f"read probe: {gbs:.0f} GB/s over 256 MiB")
    assert int(sink.item()) == 0
    assert 500 < gbs < 20000
