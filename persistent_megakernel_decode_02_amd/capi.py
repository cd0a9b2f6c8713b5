"""ctypes binding of libmkd.so: the functions of include/mkd.h under the same
names, with argument marshalling only (torch tensors -> device pointers,
return codes -> exceptions).  Every step of the decode runs in the library's
HIP kernels; there is no fallback: if the library is missing, loading fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmkd.so")

MKD_OK = 0
MKD_E_INVALID = -1
MKD_E_HIP = -2
MKD_E_COOPERATIVE = -3
MKD_E_TIMEOUT = -4
MKD_E_WATCHDOG = -5
MKD_E_BOUNDS = -6
MKD_E_NONFINITE = -7
MKD_E_ABORTED = -8
MKD_E_UNSUPPORTED = -9
ERROR_NAMES = {0: "MKD_OK", -1: "MKD_E_INVALID", -2: "MKD_E_HIP", -3: "MKD_E_COOPERATIVE",
               -4: "MKD_E_TIMEOUT", -5: "MKD_E_WATCHDOG", -6: "MKD_E_BOUNDS",
               -7: "MKD_E_NONFINITE", -8: "MKD_E_ABORTED", -9: "MKD_E_UNSUPPORTED"}

# instruction opcodes of the schedule tensor (csrc/mkd_internal.h)
OPCODE_NAMES = {1: "QKV", 2: "ATTN", 3: "AREDUCE", 4: "OPROJ", 5: "UPGATE", 6: "DOWN",
                7: "MOE_UPGATE", 8: "MOE_DOWN", 9: "LMHEAD"}

# every function include/mkd.h declares
EXPORTS = ("mkd_version", "mkd_last_error", "mkd_config_check", "mkd_weight_count",
           "mkd_weight_shape", "mkd_kv_cache_bytes", "mkd_schedule_build",
           "mkd_schedule_build_batch", "mkd_schedule_validate", "mkd_default_chunks",
           "mkd_workspace_bytes", "mkd_workspace_layout", "mkd_init", "mkd_init_batch", "mkd_init_static",
           "mkd_device_info", "mkd_lds_plan", "mkd_build_schedule", "mkd_load_schedule", "mkd_decode",
           "mkd_decode_batch", "mkd_wait", "mkd_abort", "mkd_set_watchdog",
           "mkd_set_trace", "mkd_kernel_ms", "mkd_clock_hz", "mkd_read_probe", "mkd_set_expert_prediction", "mkd_spec_stats",
           "mkd_set_lds_limits",
           "mkd_set_launch_mode", "mkd_destroy")

# regions of a workspace, in mkd_workspace_layout's order
WORKSPACE_REGIONS = ("wtab", "rope", "status", "zero", "schedule", "activations", "flags", "total")
CONTROL_WORDS = 16   # int32 words of the pinned host control block
STATIC_WORKSPACE_BYTES = 16 << 20   # MKD_STATIC_WORKSPACE_BYTES


class mkd_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("tied", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("reserved0", ctypes.c_float),
                ("rope_theta", ctypes.c_double)]


class mkd_status(ctypes.Structure):
    _fields_ = [("code", ctypes.c_int32), ("wg", ctypes.c_int32),
                ("instr", ctypes.c_int32), ("token", ctypes.c_int32)]


class MkdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmkd.so (raises if it has not been built).  MKD_LIBRARY names
    another build of the library to load instead of the in-tree one."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("MKD_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m persistent_megakernel_decode_02_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(mkd_config)
    sig = {
        "mkd_version": ([], ctypes.c_int),
        "mkd_last_error": ([], ctypes.c_char_p),
        "mkd_config_check": ([cfgp], ctypes.c_int),
        "mkd_weight_count": ([cfgp, ctypes.POINTER(SZ)], ctypes.c_int),
        "mkd_weight_shape": ([cfgp, SZ, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
        "mkd_kv_cache_bytes": ([cfgp, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "mkd_schedule_build": ([cfgp, I32, I32, P, SZ, ctypes.POINTER(SZ)], ctypes.c_int),
        "mkd_schedule_build_batch": ([cfgp, I32, I32, I32, P, SZ, ctypes.POINTER(SZ)], ctypes.c_int),
        "mkd_schedule_validate": ([cfgp, P, SZ], ctypes.c_int),
        "mkd_default_chunks": ([cfgp, I32, I32, ctypes.POINTER(I32)], ctypes.c_int),
        "mkd_workspace_bytes": ([cfgp, I32, I32, I32, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "mkd_workspace_layout": ([cfgp, I32, I32, I32, I32, ctypes.POINTER(SZ)], ctypes.c_int),
        "mkd_init": ([cfgp, ctypes.POINTER(P), SZ, P, I32, P, SZ, P, I32, ctypes.POINTER(P)], ctypes.c_int),
        "mkd_init_batch": ([cfgp, ctypes.POINTER(P), SZ, P, I32, I32, P, SZ, P, I32, ctypes.POINTER(P)],
                           ctypes.c_int),
        "mkd_init_static": ([cfgp, ctypes.POINTER(P), SZ, P, I32, P, I32, ctypes.POINTER(P)], ctypes.c_int),
        "mkd_device_info": ([P, ctypes.POINTER(I32), ctypes.POINTER(I32)], ctypes.c_int),
        "mkd_lds_plan": ([cfgp, I32, I32, I32, I32, ctypes.POINTER(I32)], ctypes.c_int),
        "mkd_build_schedule": ([P, I32, I32, P, SZ, ctypes.POINTER(SZ)], ctypes.c_int),
        "mkd_load_schedule": ([P, P, SZ], ctypes.c_int),
        "mkd_decode": ([P, I32, I32, I32, P, P, P, P], ctypes.c_int),
        "mkd_decode_batch": ([P, P, P, I32, P, P, P], ctypes.c_int),
        "mkd_wait": ([P, I32, ctypes.POINTER(mkd_status)], ctypes.c_int),
        "mkd_abort": ([P], ctypes.c_int),
        "mkd_set_watchdog": ([P, I32], ctypes.c_int),
        "mkd_set_trace": ([P, P, SZ], ctypes.c_int),
        "mkd_kernel_ms": ([P, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
        "mkd_clock_hz": ([P, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        "mkd_set_expert_prediction": ([P, I32], ctypes.c_int),
        "mkd_spec_stats": ([P, ctypes.POINTER(I32), ctypes.POINTER(I32)], ctypes.c_int),
        "mkd_read_probe": ([P, SZ, P, P], ctypes.c_int),
        "mkd_set_lds_limits": ([P, I32, I32], ctypes.c_int),
        "mkd_set_launch_mode": ([P, I32], ctypes.c_int),
        "mkd_destroy": ([P], None),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc: int) -> int:
    if rc < 0:
        raise MkdError(rc, load().mkd_last_error().decode())
    return rc


def make_config(cfg) -> mkd_config:
    """mkd_config from a shape object with the synth.ModelConfig fields."""
    return mkd_config(cfg.n_layers, cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim,
                      cfg.d_ff, cfg.vocab, cfg.n_experts, cfg.top_k, int(cfg.tied),
                      float(cfg.rms_eps), 0.0, float(cfg.rope_theta))


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


# ---------------------------------------------------------------- same-name wrappers

def mkd_version() -> int:
    return load().mkd_version()


def mkd_last_error() -> str:
    return load().mkd_last_error().decode()


def mkd_config_check(cfg: mkd_config) -> None:
    _check(load().mkd_config_check(ctypes.byref(cfg)))


def mkd_weight_count(cfg: mkd_config) -> int:
    n = ctypes.c_size_t()
    _check(load().mkd_weight_count(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def mkd_weight_shape(cfg: mkd_config, index: int):
    r, c = ctypes.c_int64(), ctypes.c_int64()
    _check(load().mkd_weight_shape(ctypes.byref(cfg), index, ctypes.byref(r), ctypes.byref(c)))
    return r.value, c.value


def mkd_kv_cache_bytes(cfg: mkd_config, max_seq: int) -> int:
    n = ctypes.c_size_t()
    _check(load().mkd_kv_cache_bytes(ctypes.byref(cfg), max_seq, ctypes.byref(n)))
    return n.value


def mkd_schedule_build(cfg: mkd_config, n_wg: int, n_chunks: int) -> np.ndarray:
    lib = load()
    n = ctypes.c_size_t()
    _check(lib.mkd_schedule_build(ctypes.byref(cfg), n_wg, n_chunks, None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, dtype=np.int32)
    _check(lib.mkd_schedule_build(ctypes.byref(cfg), n_wg, n_chunks, out.ctypes.data, out.size,
                                  ctypes.byref(n)))
    return out


def mkd_schedule_build_batch(cfg: mkd_config, n_wg: int, n_chunks: int, batch: int) -> np.ndarray:
    lib = load()
    n = ctypes.c_size_t()
    _check(lib.mkd_schedule_build_batch(ctypes.byref(cfg), n_wg, n_chunks, batch, None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, dtype=np.int32)
    _check(lib.mkd_schedule_build_batch(ctypes.byref(cfg), n_wg, n_chunks, batch, out.ctypes.data, out.size,
                                        ctypes.byref(n)))
    return out


def mkd_schedule_validate(cfg: mkd_config, words: np.ndarray) -> None:
    w = np.ascontiguousarray(words, dtype=np.int32)
    _check(load().mkd_schedule_validate(ctypes.byref(cfg), w.ctypes.data, w.size))


def mkd_default_chunks(cfg: mkd_config, n_wg: int, n_positions: int) -> int:
    n = ctypes.c_int32()
    _check(load().mkd_default_chunks(ctypes.byref(cfg), n_wg, n_positions, ctypes.byref(n)))
    return n.value


def mkd_workspace_bytes(cfg: mkd_config, n_wg: int, n_chunks: int, batch: int, max_seq: int) -> int:
    n = ctypes.c_size_t()
    _check(load().mkd_workspace_bytes(ctypes.byref(cfg), n_wg, n_chunks, batch, max_seq, ctypes.byref(n)))
    return n.value


def mkd_workspace_layout(cfg: mkd_config, n_wg: int, n_chunks: int, batch: int, max_seq: int) -> dict:
    out = (ctypes.c_size_t * len(WORKSPACE_REGIONS))()
    _check(load().mkd_workspace_layout(ctypes.byref(cfg), n_wg, n_chunks, batch, max_seq, out))
    return dict(zip(WORKSPACE_REGIONS, list(out)))


def mkd_init(cfg: mkd_config, weights: Sequence, kv_cache, max_seq: int, workspace, control,
             device: int = 0) -> int:
    """Handle (an int) for device tensors ``weights`` (pointer order), ``kv_cache`` and
    ``workspace`` (uint8) and the pinned host tensor ``control`` (int32[16])."""
    return mkd_init_batch(cfg, weights, kv_cache, max_seq, 1, workspace, control, device)


def mkd_init_batch(cfg: mkd_config, weights: Sequence, kv_cache, max_seq: int, batch: int, workspace,
                   control, device: int = 0) -> int:
    """As mkd_init for ``batch`` sequences; ``kv_cache`` holds every sequence's cache."""
    arr = (ctypes.c_void_p * len(weights))(*[_ptr(w) for w in weights])
    h = ctypes.c_void_p()
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().mkd_init_batch(ctypes.byref(cfg), arr, len(weights), _ptr(kv_cache), max_seq, batch,
                                 _ptr(workspace), nbytes, _ptr(control), device, ctypes.byref(h)))
    return h.value


def mkd_init_static(cfg: mkd_config, weights: Sequence, kv_cache, max_seq: int, control, device: int = 0) -> int:
    """As mkd_init, with the library's static per-device workspace (no workspace argument)."""
    arr = (ctypes.c_void_p * len(weights))(*[_ptr(w) for w in weights])
    h = ctypes.c_void_p()
    _check(load().mkd_init_static(ctypes.byref(cfg), arr, len(weights), _ptr(kv_cache), max_seq, _ptr(control),
                                  device, ctypes.byref(h)))
    return h.value


def mkd_device_info(m: int):
    n_cu, mx = ctypes.c_int32(), ctypes.c_int32()
    _check(load().mkd_device_info(m, ctypes.byref(n_cu), ctypes.byref(mx)))
    return n_cu.value, mx.value


def mkd_lds_plan(cfg: mkd_config, batch: int, n_wg: int, n_chunks: int, lds_max: int) -> dict:
    out = (ctypes.c_int32 * 6)()
    _check(load().mkd_lds_plan(ctypes.byref(cfg), batch, n_wg, n_chunks, lds_max, out))
    keys = ("x_floats", "out_floats", "res_floats", "pre_units", "pre_off", "lds_bytes")
    return dict(zip(keys, list(out)))


def mkd_build_schedule(m: int, n_wg: int = 0, n_chunks: int = 0, want_words: bool = False):
    lib = load()
    n = ctypes.c_size_t()
    if not want_words:
        _check(lib.mkd_build_schedule(m, n_wg, n_chunks, None, 0, ctypes.byref(n)))
        return None
    _check(lib.mkd_build_schedule(m, n_wg, n_chunks, None, 0, ctypes.byref(n)))
    out = np.zeros(n.value, dtype=np.int32)
    _check(lib.mkd_build_schedule(m, n_wg, n_chunks, out.ctypes.data, out.size, ctypes.byref(n)))
    return out


def mkd_load_schedule(m: int, words: np.ndarray) -> None:
    w = np.ascontiguousarray(words, dtype=np.int32)
    _check(load().mkd_load_schedule(m, w.ctypes.data, w.size))


def mkd_decode(m: int, first_token: int, start_pos: int, n_steps: int, tokens_out, logits_out=None,
               forced=None, stream=None) -> None:
    """Enqueue one launch; tensors are device tensors (int32 / float32)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    _check(load().mkd_decode(m, first_token, start_pos, n_steps, _ptr(forced), _ptr(tokens_out),
                             _ptr(logits_out), stream))


def mkd_decode_batch(m: int, first_tokens: Sequence[int], start_pos: Sequence[int], n_steps: int,
                     tokens_out, logits_out=None, stream=None) -> None:
    """Enqueue one launch for every sequence of a batched handle (host lists in,
    device tensors out: tokens [B, n_steps] int32, logits [B, n_steps, V] float32)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    ft = (ctypes.c_int32 * len(first_tokens))(*[int(x) for x in first_tokens])
    sp = (ctypes.c_int32 * len(start_pos))(*[int(x) for x in start_pos])
    _check(load().mkd_decode_batch(m, ft, sp, n_steps, _ptr(tokens_out), _ptr(logits_out), stream))


def mkd_wait(m: int, timeout_ms: int = -1, raise_on_error: bool = True) -> mkd_status:
    st = mkd_status()
    rc = load().mkd_wait(m, timeout_ms, ctypes.byref(st))
    if rc < 0 and raise_on_error:
        raise MkdError(rc, mkd_last_error())
    if rc < 0 and st.code == 0:
        st.code = rc
    return st


def mkd_abort(m: int) -> None:
    _check(load().mkd_abort(m))


def mkd_set_watchdog(m: int, watchdog_ms: int) -> None:
    _check(load().mkd_set_watchdog(m, watchdog_ms))


def mkd_set_trace(m: int, trace=None) -> None:
    _check(load().mkd_set_trace(m, _ptr(trace), 0 if trace is None else trace.numel()))


def mkd_kernel_ms(m: int) -> float:
    ms = ctypes.c_float()
    _check(load().mkd_kernel_ms(m, ctypes.byref(ms)))
    return ms.value


def mkd_clock_hz(m: int) -> float:
    hz = ctypes.c_double()
    _check(load().mkd_clock_hz(m, ctypes.byref(hz)))
    return hz.value


def mkd_read_probe(buf, sink, stream=None) -> None:
    """Enqueue a plain streaming read of the device tensor ``buf`` (its whole
    byte size, a multiple of 16) on ``stream`` (default: torch's current
    stream); ``sink`` is a device int32/uint32 tensor of at least one element."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    nbytes = buf.numel() * buf.element_size()
    _check(load().mkd_read_probe(_ptr(buf), nbytes, _ptr(sink), stream))


def mkd_set_expert_prediction(m: int, on: bool) -> None:
    """Speculative expert prediction on or off for later launches (MoE models; off by default)."""
    _check(load().mkd_set_expert_prediction(m, 1 if on else 0))


def mkd_spec_stats(m: int):
    """(hits, predictions) of the last waited-for launch's expert predictions."""
    h, n = ctypes.c_int32(), ctypes.c_int32()
    _check(load().mkd_spec_stats(m, ctypes.byref(h), ctypes.byref(n)))
    return h.value, n.value


def mkd_set_lds_limits(m: int, max_input_floats: int = 0, max_staged_units: int = -1) -> None:
    _check(load().mkd_set_lds_limits(m, max_input_floats, max_staged_units))


def mkd_set_launch_mode(m: int, cooperative: bool) -> None:
    _check(load().mkd_set_launch_mode(m, 1 if cooperative else 0))


def mkd_destroy(m: int) -> None:
    if m:
        load().mkd_destroy(m)
