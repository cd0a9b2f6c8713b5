"""Batch-1 decode benchmark of the persistent megakernel on one MI355X.

A step is one decode launch of the workload: the Llama-3.2-1B-shaped model
from a 128-position KV cache, 128 greedy decode steps (all opcodes of the
path, every token), inputs already resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload llama1b --kv 128]

`value` is decode tokens/s; `roofline` prices the megakernel's algorithmic
bytes (weights each step reads + K/V of the visible positions + the appended
K/V) against the MI355X HBM peak, over the kernel's own duration from HIP
events on its stream; `cpu_baseline` is the CPU oracle on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "persistent_megakernel_decode_02_amd", "csrc", "mkd_kernel.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_digest() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel and workload, if it was taken on the current kernel source;
    else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload_key}_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("kernel_sha256_16") != kernel_digest():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, T0: int, n_sample: int, first: int):
    """The oracle as it stands, timed on this host: n_sample decode steps of
    the same model from the same cache."""
    import numpy as np
    import synth
    from oracle import model as om
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    log(f"cpu baseline: generating host weights ({cfg.name})")
    w = synth.gen_weights(cfg, device="cpu")
    orc = om.Oracle(cfg, om.Weights.from_list(cfg, w))
    kv = om.kv_to_oracle(synth.gen_kv_cache(cfg, T0 + n_sample, T0))
    orc.step(first, T0, kv)   # converts the weights once (not timed)
    kv = om.kv_to_oracle(synth.gen_kv_cache(cfg, T0 + n_sample, T0))
    t = time.perf_counter()
    orc.decode(first, T0, n_sample, kv)
    dt = time.perf_counter() - t
    return {"value": n_sample / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_sample} greedy decode steps of the same model from the same "
                      f"{T0}-position cache (numpy fp32, {dt:.1f}s)"}


def calib_copy(n_bytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.empty(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n_bytes, "calib_copy_bytes_written": n_bytes,
                      "reps": reps}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed decode launches")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama1b")
    ap.add_argument("--kv", type=int, default=None, help="starting KV length (default: the workload's first)")
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--batch", type=int, default=1,
                    help="sequences decoded together (all from the same KV length)")
    ap.add_argument("--n-wg", type=int, default=0)
    ap.add_argument("--n-chunks", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=640,
                    help="oracle decode steps timed on the host, 10-30 s (0 = skip)")
    ap.add_argument("--trace", action="store_true", help="per-opcode time breakdown (stderr)")
    ap.add_argument("--calib-copy", type=int, default=0, help="only run a plain copy of this many bytes")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        return 2
    if args.calib_copy:
        calib_copy(args.calib_copy, max(1, args.steps))
        return 0

    import numpy as np
    import torch
    import synth
    from persistent_megakernel_decode_02_amd import capi, roofline
    from persistent_megakernel_decode_02_amd.decoder import Decoder
    from persistent_megakernel_decode_02_amd.tuning import launch_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    wl = synth.WORKLOADS[args.workload]
    cfg = wl.model
    T0 = args.kv if args.kv is not None else wl.kv_lengths[0]
    N = args.decode_steps or wl.steps
    max_seq = T0 + N
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    n_wg, n_chunks = launch_config(cfg, T0, N, n_cu)
    n_wg = args.n_wg or n_wg
    n_chunks = args.n_chunks or n_chunks

    B = args.batch
    log(f"generating {cfg.name} weights and {B} {T0}-position KV cache(s) on the GPU")
    w = synth.gen_weights(cfg, device="cuda")
    if B == 1:
        kv = synth.gen_kv_cache(cfg, max_seq, T0, device="cuda")
    else:
        kv = torch.stack([synth.gen_kv_cache(cfg, max_seq, T0, seed=synth.SEED_KV + 101 * b, device="cuda")
                          for b in range(B)]).contiguous()
    torch.cuda.synchronize()
    dec = Decoder(cfg, w, kv, max_seq, n_wg=n_wg, n_chunks=n_chunks, batch=B)
    log(f"schedule: n_wg={dec.n_wg} n_chunks={dec.n_chunks} max_instr={dec.max_instr} batch={B}")
    firsts = synth.gen_tokens(B, cfg.vocab)
    first = firsts[0]
    toks = torch.empty(B, N, dtype=torch.int32, device="cuda")

    def one():
        if B == 1:
            dec.launch(first, T0, N, toks)
        else:
            dec.launch_batch(firsts, [T0] * B, N, toks)
        capi.mkd_wait(dec.handle, 600000)
        return capi.mkd_kernel_ms(dec.handle)

    for i in range(args.warmup):
        ms = one()
        log(f"warmup {i}: kernel {ms:.2f} ms")
    torch.cuda.synchronize()
    kms = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        kms.append(one())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i, ms in enumerate(kms):
        log(f"step {i}: kernel {ms:.3f} ms ({ms * 1e3 / N:.1f} us/token)")

    ms_per_step = wall * 1e3 / args.steps
    kernel_s = float(np.mean(kms)) / 1e3
    n_bytes = roofline.run_bytes(cfg, T0, N) if B == 1 else roofline.batch_run_bytes(cfg, [T0] * B, N)
    achieved = n_bytes / kernel_s
    peak = roofline.HBM_PEAK_BYTES_PER_S
    floor_us = roofline.floor_seconds(n_bytes) * 1e6 / N

    if args.trace:
        trace_breakdown(dec, one, N)

    cpu = None
    if args.cpu_sample > 0:
        cpu = cpu_baseline(cfg, T0, args.cpu_sample, first)
        log(f"cpu baseline: {cpu['value']:.3f} tokens/s on {cpu['cores']} threads")
    key = f"{args.workload}_kv{T0}_n{N}" + (f"_b{B}" if B > 1 else "")
    kernel = "mkd_megakernel_batch" if B > 1 else ("mkd_megakernel_moe" if cfg.is_moe else "mkd_megakernel")
    traffic = measured_traffic(kernel, key)
    out = {
        "metric": "batch-1 decode tokens/s" if B == 1 else f"batch-{B} decode tokens/s",
        "value": B * N * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} decoder, batch {B}, KV cache {T0} positions, {N} greedy "
                               f"decode steps per step (one launch)",
                   "weights": "bf16", "kv_cache": "bf16", "activations": "fp32",
                   "kv_start": T0, "decode_tokens_per_step": N, "n_wg": dec.n_wg,
                   "n_chunks": dec.n_chunks, "parallelism": "single GPU"},
        "us_per_token": kernel_s * 1e6 / N,   # per decode step (all sequences)
        "roofline_us_per_token": floor_us,
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": peak / 1e9, "unit": "GB/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": kernel,
                     "algorithmic_bytes_per_launch": n_bytes,
                     "kernel_ms_mean": kernel_s * 1e3},
        "cpu_baseline": cpu,
    }
    dec.close()
    print(json.dumps(out), flush=True)
    return 0


def trace_breakdown(dec, launch_and_wait, N):
    """Per-opcode time from the device trace (one extra traced launch)."""
    import numpy as np
    import torch
    from persistent_megakernel_decode_02_amd import capi
    words = dec.schedule
    n_wg, max_instr = int(words[2]), int(words[4])
    tr = torch.zeros(n_wg * N * max_instr * 4, dtype=torch.int64, device="cuda")
    capi.mkd_set_trace(dec.handle, tr)
    launch_and_wait()
    capi.mkd_set_trace(dec.handle, None)
    hz = capi.mkd_clock_hz(dec.handle)
    t = tr.cpu().numpy().reshape(n_wg, N, max_instr, 4)
    counts = words[16:16 + n_wg]
    body = words[16 + n_wg:].reshape(n_wg, max_instr, 16)
    per_op = {}
    for w in range(n_wg):
        for i in range(int(counts[w])):
            op = capi.OPCODE_NAMES.get(int(body[w, i, 0]), "?")
            wait = (t[w, :, i, 1] - t[w, :, i, 0]).astype(np.float64) / hz * 1e6
            work = (t[w, :, i, 2] - t[w, :, i, 1]).astype(np.float64) / hz * 1e6
            has3 = t[w, :, i, 3] > 0
            comp = np.where(has3, (t[w, :, i, 3] - t[w, :, i, 1]), 0).astype(np.float64) / hz * 1e6
            per_op.setdefault(op, []).append((wait.mean(), work.mean(), comp.mean()))
    log("per-opcode time per instruction (us; wait = start to inputs ready, work = ready to "
        "published, of which comp = ready to end of the row stream):")
    for op, v in sorted(per_op.items()):
        v = np.array(v)
        log(f"  {op:12s} n={len(v):5d} wait mean={v[:, 0].mean():8.2f} max={v[:, 0].max():8.2f}"
            f"   work mean={v[:, 1].mean():8.2f} max={v[:, 1].max():8.2f}   comp mean={v[:, 2].mean():8.2f}")
    # stage-to-stage latency: for each (step, stage), the last producer's
    # publish time vs the first and last consumer's inputs-ready time
    stage_of = body[..., 2]
    n_st = int(words[3])
    pub = np.full((N, n_st), -np.inf)
    pub_min = np.full((N, n_st), np.inf)
    rdy_min = np.full((N, n_st), np.inf)
    rdy_max = np.full((N, n_st), -np.inf)
    opname = {}
    for w in range(n_wg):
        for i in range(int(counts[w])):
            st = int(stage_of[w, i])
            opname[st] = capi.OPCODE_NAMES.get(int(body[w, i, 0]), "?")
            pub[:, st] = np.maximum(pub[:, st], t[w, :, i, 2])
            pub_min[:, st] = np.minimum(pub_min[:, st], t[w, :, i, 2])
            rdy_min[:, st] = np.minimum(rdy_min[:, st], t[w, :, i, 1])
            rdy_max[:, st] = np.maximum(rdy_max[:, st], t[w, :, i, 1])
    lat, spread_pub, spread_rdy = {}, {}, {}
    for st in range(1, n_st):
        k = f"{opname[st - 1]}->{opname[st]}"
        lat.setdefault(k, []).append(np.mean(rdy_min[:, st] - pub[:, st - 1]) / hz * 1e6)
        spread_pub.setdefault(k, []).append(np.mean(pub[:, st - 1] - pub_min[:, st - 1]) / hz * 1e6)
        spread_rdy.setdefault(k, []).append(np.mean(rdy_max[:, st] - rdy_min[:, st]) / hz * 1e6)
    log("stage transitions (us): last publish -> first ready | producer publish spread | consumer ready spread")
    for k in lat:
        log(f"  {k:18s} {np.mean(lat[k]):7.2f} | {np.mean(spread_pub[k]):7.2f} | {np.mean(spread_rdy[k]):7.2f}")
    # token time split: per-step makespan
    starts = t[..., 0].astype(np.float64)
    ends = t[..., 2].astype(np.float64)
    valid = ends > 0
    span = [(ends[:, s][valid[:, s]].max() - starts[:, s][valid[:, s]].min()) / hz * 1e6 for s in range(N)]
    log(f"  traced step makespan: mean {np.mean(span):.1f} us")


if __name__ == "__main__":
    sys.exit(main())
