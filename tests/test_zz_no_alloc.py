"""The entry point for callers that cannot allocate device memory
(mkd_init_static: the workspace is the library's static per-device array):
through the C ABI, its decode must equal the caller-workspace entry point's
(mkd_init) bit for bit -- tokens, logits and the appended cache -- on two
handles in a row, the second with a smaller input, so the array's leftovers
from the first must not matter.  Its limits are checked on the host."""
import numpy as np
import pytest
import torch

import synth
from persistent_megakernel_decode_02_amd import capi
from persistent_megakernel_decode_02_amd.decoder import Decoder
from tests.gpu_common import require_gpu, say

pytestmark = pytest.mark.gpu


def _static_decode(cfg, w, kv, max_seq, n_wg, n_chunks, first, T0, N):
    ccfg = capi.make_config(cfg)
    ctrl = torch.zeros(capi.CONTROL_WORDS, dtype=torch.int32, pin_memory=True)
    h = capi.mkd_init_static(ccfg, w, kv, max_seq, ctrl, 0)
    try:
        capi.mkd_build_schedule(h, n_wg, n_chunks)
        toks = torch.empty(N, dtype=torch.int32, device="cuda")
        logits = torch.empty(N, cfg.vocab, dtype=torch.float32, device="cuda")
        capi.mkd_decode(h, first, T0, N, toks, logits)
        st = capi.mkd_wait(h, 60000, raise_on_error=False)
        assert st.code == capi.MKD_OK, st.code
        torch.cuda.synchronize()
    finally:
        capi.mkd_destroy(h)
    return toks, logits


def test_static_workspace_decode_equals_caller_workspace_decode():
    require_gpu()
    # the second call is smaller: shorter cache, fewer steps, fewer workgroups
    for name, T0, N, n_wg, n_chunks in (("tiny", 60, 24, 64, 3), ("tiny", 17, 6, 32, 2)):
        cfg = synth.PRESETS[name]
        max_seq = T0 + N
        w = synth.gen_weights(cfg, device="cuda", gain_std=0.1)
        kv_ref = synth.gen_kv_cache(cfg, max_seq, T0, device="cuda")
        kv_st = kv_ref.clone()
        first = synth.gen_tokens(1, cfg.vocab, stream=9)[0]
        say(f"{name} T0={T0} N={N} n_wg={n_wg} n_chunks={n_chunks}")
        dec = Decoder(cfg, w, kv_ref, max_seq, n_wg=n_wg, n_chunks=n_chunks)
        t_ref, l_ref = dec.decode(first, T0, N)
        dec.close()
        t_st, l_st = _static_decode(cfg, w, kv_st, max_seq, n_wg, n_chunks, first, T0, N)
        say(f"  tokens {t_st.tolist()}")
        assert torch.equal(t_st, t_ref), "tokens differ from the caller-workspace decode"
        assert torch.equal(l_st, l_ref), "logits differ from the caller-workspace decode"
        assert torch.equal(kv_st, kv_ref), "caches differ from the caller-workspace decode"


def test_static_workspace_limits():
    """Checked on the host: a max_seq whose RoPE table outgrows the static
    size, a schedule too large for it, and a second handle on the same device
    while one holds the array are refused with MKD_E_INVALID."""
    require_gpu()
    cfg = synth.PRESETS["tiny"]
    ccfg = capi.make_config(cfg)
    w = synth.gen_weights(cfg, device="cuda")
    kv = synth.gen_kv_cache(cfg, 64, 32, device="cuda")
    ctrl = torch.zeros(capi.CONTROL_WORDS, dtype=torch.int32, pin_memory=True)
    big = capi.STATIC_WORKSPACE_BYTES // (cfg.head_dim * 4) + 1   # RoPE rows alone exceed the array
    with pytest.raises(capi.MkdError) as e:
        capi.mkd_init_static(ccfg, w, kv, big, ctrl, 0)
    assert e.value.code == capi.MKD_E_INVALID and "static workspace" in str(e.value)
    h = capi.mkd_init_static(ccfg, w, kv, 64, ctrl, 0)
    try:
        with pytest.raises(capi.MkdError) as e:
            capi.mkd_init_static(ccfg, w, kv, 64, torch.zeros(16, dtype=torch.int32, pin_memory=True), 0)
        assert e.value.code == capi.MKD_E_INVALID
        capi.mkd_build_schedule(h, 8, 1)
        toks = torch.empty(4, dtype=torch.int32, device="cuda")
        capi.mkd_decode(h, 3, 32, 4, toks)
        assert capi.mkd_wait(h, 60000, raise_on_error=False).code == capi.MKD_OK
    finally:
        capi.mkd_destroy(h)
    # a cache length whose tables fit but leave too little for a 256-workgroup,
    # 8-chunk schedule (found from the host-side layout query)
    ms = big
    while capi.mkd_workspace_layout(ccfg, 256, 8, 1, ms)["schedule"] > capi.STATIC_WORKSPACE_BYTES:
        ms -= 64
    assert capi.mkd_workspace_bytes(ccfg, 256, 8, 1, ms) > capi.STATIC_WORKSPACE_BYTES
    kv_long = synth.gen_kv_cache(cfg, ms, 32, device="cuda")
    h = capi.mkd_init_static(ccfg, w, kv_long, ms, ctrl, 0)
    try:
        with pytest.raises(capi.MkdError) as e:
            capi.mkd_build_schedule(h, 256, 8)
        assert e.value.code == capi.MKD_E_INVALID and "static workspace" in str(e.value)
    finally:
        capi.mkd_destroy(h)
    # the array is free again
    h = capi.mkd_init_static(ccfg, w, kv, 64, ctrl, 0)
    capi.mkd_destroy(h)
