"""Shared pieces of the GPU parity tests (imported by tests/test_gpu_*.py)."""
import sys
import time

import numpy as np
import torch

import synth
from oracle import model as om

ATOL, RTOL = 2e-2, 1e-2   # |gpu - oracle| <= ATOL + RTOL * |oracle|


_capture = None   # pytest's capture manager, set by tests/conftest.py


def say(*a):
    """Progress line, printed past pytest's output capture so that a long
    test is seen to be alive."""
    msg = " ".join(str(x) for x in ("[gpu-test]",) + a)
    if _capture is not None:
        with _capture.global_and_fixture_disabled():
            print(msg, flush=True)
    else:
        print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU; torch.cuda.is_available() is False")
    from persistent_megakernel_decode_02_amd import capi
    capi.load()


def close_enough(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    bad = err > ATOL + RTOL * np.abs(want)
    return (not bad.any()), float(err.max()) if err.size else 0.0, int(bad.sum())


def oracle_run(cfg, w_cpu, kv_cpu, first, start, n, forced=None, dtype=np.float32):
    orc = om.Oracle(cfg, om.Weights.from_list(cfg, w_cpu, dtype=dtype))
    kv = om.kv_to_oracle(kv_cpu, dtype)
    t = time.time()
    toks, logits = orc.decode(first, start, n, kv, forced=forced)
    say(f"oracle {n} steps in {time.time() - t:.1f}s")
    return toks, logits, kv


def check_run(name, toks_gpu, logits_gpu, toks_orc, logits_orc):
    toks_gpu = [int(x) for x in toks_gpu]
    agree = 0
    while agree < len(toks_orc) and toks_gpu[agree] == toks_orc[agree]:
        agree += 1
    ok, mx, nbad = close_enough(logits_gpu[:agree + 1 if agree < len(toks_orc) else agree],
                                logits_orc[:agree + 1 if agree < len(toks_orc) else agree])
    say(f"{name}: greedy agreement {agree}/{len(toks_orc)}, logits max|err| {mx:.3e}, out-of-tol {nbad}")
    if agree < len(toks_orc):
        row = np.sort(logits_orc[agree])[::-1]
        say(f"  first mismatch at step {agree}: gpu {toks_gpu[agree]} oracle {toks_orc[agree]}, "
            f"oracle top-2 margin {row[0] - row[1]:.3e}")
    assert ok, f"{name}: {nbad} logits outside tolerance (max err {mx})"
    assert agree == len(toks_orc), f"{name}: greedy tokens diverge at step {agree}"
