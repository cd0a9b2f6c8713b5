"""Keeps the torch tensors a libmkd handle borrows alive (weights, KV cache,
the device workspace and the pinned host control block), and turns calls into
the C ABI's (argument marshalling only; all compute runs in the library)."""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import capi


class Decoder:
    """One model on one GPU: weights (bf16 device tensors in pointer order),
    a bf16 KV cache tensor, the library's workspace (a uint8 device tensor
    sized by mkd_workspace_bytes for the launch shape), its pinned host
    control block, and the library handle with a loaded schedule.  With
    ``batch`` > 1 the cache tensor holds every sequence's cache, one after
    the other, and decoding goes through ``decode_batch``.  ``cooperative``
    False dispatches the same grid without the cooperative flag (profiling);
    ``lds_limits`` = (max input floats, max staged units) is passed to
    mkd_set_lds_limits before the schedule is built (tests);
    ``expert_prediction`` turns on mkd_set_expert_prediction (MoE models)."""

    def __init__(self, cfg, weights: Sequence[torch.Tensor], kv_cache: torch.Tensor, max_seq: int,
                 n_wg: int = 0, n_chunks: int = 0, device: Optional[int] = None, batch: int = 1,
                 cooperative: bool = True, lds_limits=None, expert_prediction: bool = False):
        self.cfg = cfg
        self.ccfg = capi.make_config(cfg)
        self.weights = list(weights)
        self.kv = kv_cache
        self.max_seq = max_seq
        self.batch = batch
        self.device = kv_cache.device.index if device is None else device
        for i, w in enumerate(self.weights):
            r, c = capi.mkd_weight_shape(self.ccfg, i)
            if w.dtype != torch.bfloat16 or not w.is_contiguous() or w.numel() != r * c:
                raise ValueError(f"weight {i}: expected contiguous bf16 with {r}x{c} elements")
        if kv_cache.dtype != torch.bfloat16 or not kv_cache.is_contiguous():
            raise ValueError("kv cache must be contiguous bf16")
        if kv_cache.numel() * 2 != batch * capi.mkd_kv_cache_bytes(self.ccfg, max_seq):
            raise ValueError("kv cache size does not match max_seq and batch")
        if n_wg == 0:
            n_wg = torch.cuda.get_device_properties(self.device).multi_processor_count
        if n_chunks == 0:
            n_chunks = capi.mkd_default_chunks(self.ccfg, n_wg, max_seq)
        nbytes = capi.mkd_workspace_bytes(self.ccfg, n_wg, n_chunks, batch, max_seq)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=kv_cache.device)
        self.control = torch.zeros(capi.CONTROL_WORDS, dtype=torch.int32, pin_memory=True)
        self.handle = capi.mkd_init_batch(self.ccfg, self.weights, kv_cache, max_seq, batch, self.workspace,
                                          self.control, self.device)
        if not cooperative:
            capi.mkd_set_launch_mode(self.handle, False)
        if lds_limits is not None:
            capi.mkd_set_lds_limits(self.handle, *lds_limits)
        if expert_prediction:
            capi.mkd_set_expert_prediction(self.handle, True)
        self.schedule = capi.mkd_build_schedule(self.handle, n_wg, n_chunks, want_words=True)

    @property
    def n_wg(self) -> int:
        return int(self.schedule[2])

    @property
    def n_chunks(self) -> int:
        return int(self.schedule[5])

    @property
    def max_instr(self) -> int:
        return int(self.schedule[4])

    def rebuild(self, n_wg: int = 0, n_chunks: int = 0) -> None:
        """Build and load another schedule; it must fit the workspace sized at
        construction (the library checks)."""
        self.schedule = capi.mkd_build_schedule(self.handle, n_wg, n_chunks, want_words=True)

    def launch(self, first_token: int, start_pos: int, n_steps: int, tokens_out: torch.Tensor,
               logits_out: Optional[torch.Tensor] = None, forced: Optional[torch.Tensor] = None,
               stream=None) -> None:
        """Enqueue one decode launch (asynchronous)."""
        capi.mkd_decode(self.handle, first_token, start_pos, n_steps, tokens_out, logits_out, forced,
                        stream)

    def decode(self, first_token: int, start_pos: int, n_steps: int, want_logits: bool = True,
               forced: Optional[Sequence[int]] = None, timeout_ms: int = 120000):
        """Run one launch and wait: (tokens [n] int32, logits [n, V] float32 or None)."""
        dev = self.kv.device
        toks = torch.empty(n_steps, dtype=torch.int32, device=dev)
        logits = torch.empty(n_steps, self.cfg.vocab, dtype=torch.float32, device=dev) if want_logits else None
        f = None
        if forced is not None:
            f = torch.tensor(list(forced), dtype=torch.int32, device=dev)
        self.launch(first_token, start_pos, n_steps, toks, logits, f)
        capi.mkd_wait(self.handle, timeout_ms)
        torch.cuda.synchronize(dev)
        return toks, logits

    def launch_batch(self, first_tokens: Sequence[int], start_pos: Sequence[int], n_steps: int,
                     tokens_out: torch.Tensor, logits_out: Optional[torch.Tensor] = None, stream=None) -> None:
        """Enqueue one decode launch for every sequence (asynchronous)."""
        if len(first_tokens) != self.batch or len(start_pos) != self.batch:
            raise ValueError(f"need {self.batch} first tokens and start positions")
        capi.mkd_decode_batch(self.handle, first_tokens, start_pos, n_steps, tokens_out, logits_out, stream)

    def decode_batch(self, first_tokens: Sequence[int], start_pos: Sequence[int], n_steps: int,
                     want_logits: bool = True, timeout_ms: int = 120000):
        """Run one batched launch and wait: (tokens [B, n] int32, logits [B, n, V] float32 or None)."""
        dev = self.kv.device
        B = self.batch
        toks = torch.empty(B, n_steps, dtype=torch.int32, device=dev)
        logits = (torch.empty(B, n_steps, self.cfg.vocab, dtype=torch.float32, device=dev)
                  if want_logits else None)
        self.launch_batch(first_tokens, start_pos, n_steps, toks, logits)
        capi.mkd_wait(self.handle, timeout_ms)
        torch.cuda.synchronize(dev)
        return toks, logits

    def close(self) -> None:
        if getattr(self, "handle", None):
            capi.mkd_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
