"""Failure handling on the device, forced from the host.

The host's stop word (mkd_abort) must end a running launch at whichever wait
each workgroup is in, report MKD_E_ABORTED, and leave the model usable: the
next launch from the same position decodes the same tokens as before.  No
test here makes the device fault or hang: every device-side wait polls the
stop word and its own watchdog deadline.
"""
import pytest
import torch

import synth
from persistent_megakernel_decode_02_amd import capi
from persistent_megakernel_decode_02_amd.decoder import Decoder
from tests.gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu


def test_abort_ends_a_running_launch_and_the_model_still_decodes():
    require_gpu()
    cfg = synth.TINY
    T0, max_seq, long_n = 32, 4096, 4000
    w = synth.gen_weights(cfg, device="cuda")
    kv = synth.gen_kv_cache(cfg, max_seq, T0, device="cuda")
    dec = Decoder(cfg, w, kv, max_seq)
    first = int(synth.gen_tokens(1, cfg.vocab)[0])
    ref, _ = dec.decode(first, T0, 8, want_logits=False)
    ref = [int(x) for x in ref.cpu()]
    say(f"reference tokens {ref}")

    toks = torch.empty(long_n, dtype=torch.int32, device="cuda")
    dec.launch(first, T0, long_n, toks)
    capi.mkd_abort(dec.handle)
    st = capi.mkd_wait(dec.handle, 60000, raise_on_error=False)
    say(f"stopped launch: code {st.code}")
    # a launch that somehow finished before the stop word was read is fine too
    assert st.code in (0, capi.MKD_E_ABORTED)

    again, _ = dec.decode(first, T0, 8, want_logits=False)
    again = [int(x) for x in again.cpu()]
    say(f"after the abort {again}")
    assert again == ref
    dec.close()


def test_watchdog_setting_is_validated():
    require_gpu()
    cfg = synth.TINY
    w = synth.gen_weights(cfg, device="cuda")
    kv = synth.gen_kv_cache(cfg, 64, 32, device="cuda")
    dec = Decoder(cfg, w, kv, 64)
    with pytest.raises(capi.MkdError):
        capi.mkd_set_watchdog(dec.handle, 0)
    capi.mkd_set_watchdog(dec.handle, 5000)
    toks, _ = dec.decode(3, 32, 4, want_logits=False)
    assert toks.numel() == 4
    dec.close()
