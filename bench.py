"""Batch-1 decode benchmark of the persistent megakernel on one MI355X.

A step is one decode launch of the workload: by default the
Mixtral-8x7B-shaped top-2 MoE model (32 layers, d 4096, 8 experts of FFN
14336, 93 GB of bf16 weights) from a 1024-position KV cache, 64 greedy decode
steps (all opcodes of the path, every token), inputs already resident in HBM.
It is the largest of the workloads, and one GPU holds it.  Prints one JSON
line.

    python bench.py [--steps K] [--warmup W] [--workload mixtral|llama1b|llama3b|llama1b_long --kv T]

`value` is decode tokens/s; `roofline` prices the megakernel's algorithmic
bytes (weights each step reads + K/V of the visible positions + the appended
K/V) against the MI355X HBM peak, over the kernel's own duration from HIP
events on its stream; `cpu_baseline` is the CPU oracle on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
METRIC = "batch-1 decode tokens/s and % of HBM roofline (weight+KV bytes/token)"
# digest of the kernels' device sources: a profile taken on other sources is stale
from persistent_megakernel_decode_02_amd.profile_summary import kernel_digest  # noqa: E402


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


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


def cpu_baseline(cfg, T0: int, budget_s: float, first: int, w_gpu):
    """The oracle as it stands, timed on this host: whole greedy decode steps
    of the same model from the same cache, until budget_s is spent (at least
    two).  Dense models: the oracle's own host copy of the weights, converted
    once before timing.  The MoE model is too large for host memory as fp32:
    the oracle keeps everything but the experts on the host and reads the two
    routed experts of each layer back from the generated device tensors per
    use (bit-identical to the host generator's), and that read is timed as
    part of its step."""
    import numpy as np
    import synth
    from oracle import model as om
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    n_max = 4096
    if cfg.is_moe:
        names = [n for n, _ in synth.weight_specs(cfg)]
        keep = [not (".gate." in n or ".up." in n or ".down." in n) for n in names]
        wts = om.Weights(cfg, lambda i: w_gpu[i], cache=lambda i: keep[i])
        how = "routed experts read back from the device per use"
    else:
        log(f"cpu baseline: generating host weights ({cfg.name})")
        wts = om.Weights.from_list(cfg, synth.gen_weights(cfg, device="cpu"))
        how = "host weights"
    orc = om.Oracle(cfg, wts)
    kv = om.kv_to_oracle(synth.gen_kv_cache(cfg, T0 + n_max, T0))
    orc.step(first, T0, kv)   # converts the kept weights once (not timed)
    kv = om.kv_to_oracle(synth.gen_kv_cache(cfg, T0 + n_max, T0))
    t = time.perf_counter()
    n, tok = 0, first
    while n < n_max and (n < 2 or time.perf_counter() - t < budget_s):
        tk, _ = orc.decode(tok, T0 + n, 1, kv)
        tok = tk[0]
        n += 1
    dt = time.perf_counter() - t
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} greedy decode steps of the same model from the same {T0}-position cache "
                      f"(numpy fp32, {how}, {dt:.1f}s)"}


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
    ap.add_argument("--workload", default="mixtral")
    ap.add_argument("--kv", type=int, default=None, help="starting KV length (default: the workload's first)")
    ap.add_argument("--decode-steps", type=int, default=None)
    ap.add_argument("--batch", type=int, default=1,
                    help="sequences decoded together (all from the same KV length)")
    ap.add_argument("--n-wg", type=int, default=0)
    ap.add_argument("--n-chunks", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="host time budget of the oracle sample: whole decode steps until it is spent "
                         "(0 = skip)")
    ap.add_argument("--trace", action="store_true", help="per-opcode time breakdown (stderr)")
    ap.add_argument("--trace-out", default=None, help="also write the breakdown to this markdown file")
    ap.add_argument("--plain-launch", action="store_true",
                    help="dispatch the grid without the cooperative flag (for profilers)")
    ap.add_argument("--staged-units", type=int, default=-1,
                    help="cap on the weight units per wavefront staged ahead in LDS (-1: no cap; 0 turns "
                         "staging off)")
    ap.add_argument("--expert-prediction", action="store_true",
                    help="MoE: predict each layer's experts and stage their first rows (off by default: "
                         "measured slower on MI355X)")
    ap.add_argument("--calib-copy", type=int, default=0, help="only run a plain copy of this many bytes")
    ap.add_argument("--read-probe-gib", type=float, default=4.0,
                    help="size of the plain streaming read that measures the reachable HBM rate (0: skip)")
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
    tg = time.perf_counter()
    n_t = len(synth.weight_specs(cfg))
    w = []
    for i in range(n_t):
        w.append(synth.gen_weights(cfg, device="cuda", only=[i])[i])
        if i % 64 == 63:
            torch.cuda.synchronize()
            log(f"  {i + 1}/{n_t} tensors, {time.perf_counter() - tg:.1f}s")
    if B == 1:
        kv = synth.gen_kv_cache(cfg, max_seq, T0, device="cuda")
    else:
        kv = torch.stack([synth.gen_kv_cache(cfg, max_seq, T0, seed=synth.SEED_KV + 101 * b, device="cuda")
                          for b in range(B)]).contiguous()
    torch.cuda.synchronize()
    log(f"inputs generated in {time.perf_counter() - tg:.1f}s")
    dec = Decoder(cfg, w, kv, max_seq, n_wg=n_wg, n_chunks=n_chunks, batch=B, cooperative=not args.plain_launch,
                  lds_limits=None if args.staged_units < 0 else (0, args.staged_units),
                  expert_prediction=args.expert_prediction)
    dec.trace_pos = T0
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
        trace_breakdown(dec, one, N, args.trace_out, f"{args.workload} KV {T0}, {N} steps per launch")

    probe = read_probe(args.read_probe_gib) if args.read_probe_gib > 0 else None

    cpu = None
    if args.cpu_seconds > 0 and B == 1:
        cpu = cpu_baseline(cfg, T0, args.cpu_seconds, first, w)
        log(f"cpu baseline: {cpu['value']:.3f} tokens/s on {cpu['cores']} threads")
    spec = None
    if cfg.is_moe:
        hits, preds = capi.mkd_spec_stats(dec.handle)
        spec = {"on": bool(args.expert_prediction), "hits": hits, "predictions": preds,
                "hit_rate": hits / preds if preds else None}
        log(f"expert prediction {'on' if args.expert_prediction else 'off'}: {hits} of {preds} gate/up tiles "
            f"had their routed expert predicted")
    key = f"{args.workload}_kv{T0}_n{N}" + (f"_b{B}" if B > 1 else "")
    kernel = "mkd_megakernel_batch" if B > 1 else ("mkd_megakernel_moe" if cfg.is_moe else "mkd_megakernel")
    traffic = measured_traffic(kernel, key)
    out = {
        "metric": METRIC if B == 1 else f"batch-{B} decode tokens/s",
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
                   "launch": "cooperative" if not args.plain_launch else "plain",
                   "expert_prediction": spec,
                   "weights": "bf16", "kv_cache": "bf16", "activations": "fp32",
                   "kv_start": T0, "decode_tokens_per_step": N, "n_wg": dec.n_wg,
                   "n_chunks": dec.n_chunks, "parallelism": "single GPU"},
        "us_per_token": kernel_s * 1e6 / N,   # per decode step (all sequences)
        "roofline_us_per_token": floor_us,
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": peak / 1e9, "unit": "GB/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": kernel,
                     "algorithmic_bytes_per_launch": n_bytes,
                     "kernel_ms_mean": kernel_s * 1e3,
                     "read_probe_gbs": probe},
        "cpu_baseline": cpu,
    }
    dec.close()
    print(json.dumps(out), flush=True)
    return 0


def read_probe(gib: float):
    """GB/s of a plain streaming read of a device buffer (the library's
    mkd_read_probe; median of 5 timed launches after one untimed), measured
    on torch's current stream with its events: the HBM read rate this device
    reaches, beside which the decode kernels' fraction of the published peak
    is read."""
    import numpy as np
    import torch
    from persistent_megakernel_decode_02_amd import capi
    n = int(gib * (1 << 30)) // 16 * 16
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    capi.mkd_read_probe(buf, sink)
    ms = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        capi.mkd_read_probe(buf, sink)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    del buf
    torch.cuda.empty_cache()
    gbs = n / (float(np.median(ms)) * 1e-3) / 1e9
    log(f"read probe: {n / 2**30:.1f} GiB at {gbs:.0f} GB/s")
    return gbs


def stage_bytes(cfg, op: str, pos: int) -> int:
    """Algorithmic HBM bytes of one stage of one layer at position pos (the
    weights it reads, K/V of positions 0..pos for attention; the LM head's
    per token) -- the per-opcode split of roofline.step_bytes."""
    d, F, qd, kvd = cfg.d_model, cfg.d_ff, cfg.qd, cfg.kvd
    return {"QKV": 2 * (qd + 2 * kvd) * d + 2 * d, "ATTN": 2 * kvd * 2 * (pos + 2), "AREDUCE": 0,
            "OPROJ": 2 * d * qd, "UPGATE": 2 * 2 * F * d + 2 * d, "DOWN": 2 * d * F,
            "MOE_UPGATE": 2 * (cfg.n_experts * d + 2 * 2 * F * d) + 2 * d, "MOE_DOWN": 2 * 2 * d * F,
            "LMHEAD": 2 * cfg.vocab * d + 2 * d + 2 * d}.get(op, 0)


def trace_breakdown(dec, launch_and_wait, N, out_path=None, title=""):
    """Each opcode's cost from the device trace (one extra traced launch):
    per instruction, the wait for inputs and the work after them; per stage,
    its share of the token's critical path -- from the previous stage's last
    publish to its own last publish, split into the transition (to its first
    consumer ready), the spread of its consumers becoming ready, and its work
    -- and the algorithmic bytes it moves in that time."""
    import torch
    from persistent_megakernel_decode_02_amd import capi
    words = dec.schedule
    n_wg, max_instr = int(words[2]), int(words[4])
    tr = torch.zeros(n_wg * N * max_instr * 4, dtype=torch.int64, device="cuda")
    capi.mkd_set_trace(dec.handle, tr)
    launch_and_wait()
    capi.mkd_set_trace(dec.handle, None)
    hz = capi.mkd_clock_hz(dec.handle)
    lines = trace_tables(tr.cpu().numpy().reshape(n_wg, N, max_instr, 4), words, hz, dec.cfg, dec.trace_pos)
    for ln in lines:
        log(ln)
    if out_path:
        with open(out_path, "w") as f:
            f.write(f"# Per-opcode cost: {title}\n\n" + "\n".join(lines) + "\n")


def trace_tables(trace, words, hz, cfg, trace_pos):
    """The tables of trace_breakdown from a launch's device trace: trace is
    [workgroup][step][instruction][start, inputs ready, outputs published,
    spare] in clock ticks of hz, words the launch's schedule words."""
    import numpy as np
    from persistent_megakernel_decode_02_amd import capi
    n_wg, N, max_instr = trace.shape[0], trace.shape[1], int(words[4])
    us = 1e6 / hz
    t = np.asarray(trace).astype(np.float64)
    counts = words[16:16 + n_wg]
    body = words[16 + n_wg:].reshape(n_wg, max_instr, 16)
    n_st = int(words[3])
    per_op = {}
    pub = np.full((N, n_st), -np.inf)
    rdy_min = np.full((N, n_st), np.inf)
    rdy_max = np.full((N, n_st), -np.inf)
    opname, layer_of = {}, {}
    for w in range(n_wg):
        for i in range(int(counts[w])):
            op = capi.OPCODE_NAMES.get(int(body[w, i, 0]), "?")
            st = int(body[w, i, 2])
            opname[st], layer_of[st] = op, int(body[w, i, 1])
            wait = (t[w, :, i, 1] - t[w, :, i, 0]) * us
            work = (t[w, :, i, 2] - t[w, :, i, 1]) * us
            per_op.setdefault(op, []).append(np.stack([wait, work], axis=1))
            pub[:, st] = np.maximum(pub[:, st], t[w, :, i, 2])
            rdy_min[:, st] = np.minimum(rdy_min[:, st], t[w, :, i, 1])
            rdy_max[:, st] = np.maximum(rdy_max[:, st], t[w, :, i, 1])
    lines = []
    lines.append("Per instruction (us): wait = start to inputs ready; work = inputs ready to outputs published.")
    lines.append("")
    lines.append("| Opcode | Instructions | wait mean | wait max | work mean | work min | work max |")
    lines.append("|---|---|---|---|---|---|---|")
    for op, v in sorted(per_op.items()):
        v = np.concatenate(v)
        lines.append(f"| {op} | {len(v) // N} x {N} | {v[:, 0].mean():.2f} | {v[:, 0].max():.2f} | "
                     f"{v[:, 1].mean():.2f} | {v[:, 1].min():.2f} | {v[:, 1].max():.2f} |")
    # the critical path of each step, stage by stage
    acc = {}
    for k in range(N):
        prev = np.min(t[:, k, 0, 0][counts > 0]) if k == 0 else pub[k - 1, n_st - 1]
        for st in range(n_st):
            op = opname[st]
            p0 = prev if st == 0 else pub[k, st - 1]
            a = acc.setdefault(op, np.zeros(5))
            a[0] += (pub[k, st] - p0) * us                      # share of the critical path
            a[1] += max(0.0, rdy_min[k, st] - p0) * us          # transition
            a[2] += (rdy_max[k, st] - rdy_min[k, st]) * us      # consumer-ready spread
            a[3] += (pub[k, st] - rdy_max[k, st]) * us          # work after the last consumer was ready
            a[4] += stage_bytes(cfg, op, trace_pos + k)
    total = sum(a[0] for a in acc.values()) / N
    lines.append("")
    lines.append(f"Per token (us, mean over {N} steps): each stage's share of the critical path (previous stage's "
                 "last publish to its own last publish) = transition (to its first consumer ready) + ready spread "
                 "+ work; bytes are its algorithmic HBM bytes, GB/s = bytes / share.")
    lines.append("")
    lines.append("| Opcode | share us/token | % | transition | ready spread | work | MB/token | GB/s | % of 8 TB/s |")
    lines.append("|---|---|---|---|---|---|---|---|---|")
    for op, a in sorted(acc.items(), key=lambda kv: -kv[1][0]):
        a = a / N
        gbs = a[4] / (a[0] * 1e-6) / 1e9 if a[0] > 0 else 0.0
        lines.append(f"| {op} | {a[0]:.1f} | {100 * a[0] / total:.1f} | {a[1]:.1f} | {a[2]:.1f} | {a[3]:.1f} | "
                     f"{a[4] / 1e6:.1f} | {gbs:.0f} | {100 * gbs / 8000:.1f} |")
    lines.append(f"| total | {total:.1f} | 100 | | | | | | |")
    # when each stage's consumers start their instruction and hold their
    # inputs, relative to the producing stage's last publish
    rel = {}
    chain = [0, 0]
    members = {}
    for w in range(n_wg):
        for i in range(int(counts[w])):
            members.setdefault(int(body[w, i, 2]), []).append((w, i))
    for k in range(N):
        for st in range(1, n_st):
            m0, m1 = members[st - 1], members[st]
            pubs0 = np.array([t[w, k, i, 2] for w, i in m0])
            last = pubs0.max()
            starts = np.array([t[w, k, i, 0] for w, i in m1])
            rdys = np.array([t[w, k, i, 1] for w, i in m1])
            r = rel.setdefault(opname[st], [[], []])
            r[0].append((starts - last) * us)
            r[1].append((rdys - last) * us)
            if len(m1) > 8:
                chain[1] += 1
                chain[0] += m1[int(np.argmax(rdys))][0] == m0[int(np.argmax(pubs0))][0]
    lines.append("")
    lines.append("Consumers against the producing stage's last publish (us; negative: before it): when they start "
                 "the instruction, and when they hold its inputs.")
    lines.append("")
    lines.append("| Opcode | start p10 | start median | start p90 | ready p10 | ready median | ready p90 | ready max |")
    lines.append("|---|---|---|---|---|---|---|---|")
    for op, (a, b) in sorted(rel.items()):
        a, b = np.concatenate(a), np.concatenate(b)
        pa, pb = np.percentile(a, [10, 50, 90]), np.percentile(b, [10, 50, 90])
        lines.append(f"| {op} | {pa[0]:.2f} | {pa[1]:.2f} | {pa[2]:.2f} | {pb[0]:.2f} | {pb[1]:.2f} | {pb[2]:.2f} | "
                     f"{b.max():.2f} |")
    if chain[1]:
        lines.append("")
        lines.append(f"The last consumer to hold its inputs was the producing stage's last publisher in {chain[0]} of "
                     f"{chain[1]} stage instances.")
    return lines


if __name__ == "__main__":
    sys.exit(main())
