"""Benchmark of the MoE decode/verify round on one MI355X.

Workload: one MoE layer of the speculative-verify shape (H=2048, 256 experts, top-8, I=512, 4-bit
blocks of 32 with fp16 scale and minimum), rows correlated (shared base + 0.5 * noise) so the
experts of a round's rows partly overlap. One step = three rounds, at T = 1, 3 and 8 rows, so the
headline tok/s covers the three verify widths; per-width latency, unique experts and bytes are
reported beside it.

Cache honesty: every round uses the next of R weight replicas (identical bytes at distinct
addresses, over 16 GB in total) and the next of a pool of pre-generated activations, so a
round's expert bytes come from HBM, not from the 256 MB Infinity Cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--graph] [--no-cpu]
prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TS = (1, 3, 8)                 # the headline step's widths
TS_SWEEP = (1, 2, 3, 4, 5, 8)  # the verify sweep's widths, reported per width
CONTROL_BUF_BYTES = 2 << 30


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--replicas", type=int, default=32)
    p.add_argument("--graph", action="store_true", help="replay captured hipGraphs instead of eager launches")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="seconds per CPU-baseline setting")
    p.add_argument("--pmc-calibrate", action="store_true",
                   help="finish with a copy of 1 GiB (torch.neg) that calibrates the HBM byte counters")
    p.add_argument("--no-extra", action="store_true", help="skip the wide-round and deep-stack sections")
    p.add_argument("--launch", default="", help="launch-shape fields for the verify sweep, e.g. fused_max_rows=4,rows_per_item=2")
    p.add_argument("--no-profile", dest="profile", action="store_false",
                   help="skip the kernel-timing pass (no roofline)")
    p.add_argument("--prefill-only", type=int, default=0, metavar="T",
                   help="only the prefill section, at T rows (for profiling it); prints its JSON")
    p.add_argument("--only", default="", choices=("", "decode", "wide", "deep", "tier", "launch", "choices"),
                   help="only that extra section (for profiling it); prints its JSON")
    return p.parse_args()


def gateup_bytes(cfg, n_unique, T):
    """Algorithmic bytes of one gate/up launch: unique experts' gate+up codes and scale/min words,
    the T input rows, and the T*k SwiGLU output rows."""
    w = n_unique * 2 * cfg.I * cfg.H * (0.5 + 4.0 / 32.0)
    return w + T * cfg.H * 4 + T * cfg.k * cfg.I * 4


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gateup_kernel_verify_sweep_traffic.txt")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_gateup_T4096_traffic.txt")
PREFILL_TRAFFIC_T = 4096
CALIB_BYTES = 1 << 30


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this build "
              "(a round runs on one GPU; splitting experts across GPUs is not built)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from verify_router_gemv_amd import MoeRound
    from verify_router_gemv_amd.profsum import read_traffic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    cfg = synth.config("verify")
    base = synth.make_layer(cfg, seed=0, layer=0, device=dev)
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_rounds(base, torch, np, synth, MoeRound, (args.prefill_only,))}), flush=True)
        if args.pmc_calibrate:
            calibration_copy(torch, dev)
        return
    if args.only:
        run_one = {"decode": lambda: decode_rounds(torch, np, synth, MoeRound),
                   "wide": lambda: wide_rounds(cfg, base, torch, np, synth, MoeRound),
                   "deep": lambda: deep_stack(torch, np, synth, MoeRound),
                   "tier": lambda: tier_rounds(torch, np, synth, MoeRound),
                   "launch": lambda: launch_costs(torch, np, synth, MoeRound),
                   "choices": lambda: launch_choices(cfg, base, torch, np, MoeRound)}[args.only]
        print(json.dumps({args.only: run_one()}), flush=True)
        return
    reps = [base] + [base.clone() for _ in range(args.replicas - 1)]
    n_acts = 256
    acts = {T: torch.stack([synth.make_activations(cfg, T, seed=0, round_idx=r, device=dev)
                            for r in range(n_acts)]) for T in TS}
    outs = {T: torch.empty((T, cfg.H), device=dev) for T in TS}
    shape = {kv.split("=")[0]: int(kv.split("=")[1]) for kv in args.launch.split(",") if kv}
    handles = [MoeRound([reps[i]], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=max(TS), use_graph=args.graph, **shape)
               for i in range(args.replicas)]
    R = args.replicas
    nT = len(TS)

    # Unique experts of every (width, activation) pair, read back once before timing: the
    # timed loop then needs no bookkeeping to know each launch's algorithmic bytes.
    nu = {}
    for a in range(n_acts):
        for j, T in enumerate(TS):
            h = handles[(nT * a + j) % R]
            h.run(acts[T][a], cfg.k, outs[T])
            nu[(T, a)] = h.last_unique()[0]
    step_gu_bytes = [sum(gateup_bytes(cfg, nu[(T, a)], T) for T in TS) for a in range(n_acts)]

    sc = [0]

    def step():
        s = sc[0]
        a = s % n_acts
        for j, T in enumerate(TS):
            handles[(nT * s + j) % R].run(acts[T][a], cfg.k, outs[T])
        sc[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    tokens_per_step = sum(TS)
    value = tokens_per_step * args.steps / elapsed

    # Dominant kernel (gate/up): the same K steps again with every kernel launched with dispatch-
    # timestamp events (the runtime stamps them with the kernel's own start and end, as the
    # profiler does). Those launches cost the host more, so they are not part of the timed steps
    # above; the kernels run unchanged. achieved = algorithmic bytes of every gate/up launch of
    # the pass / the summed durations of those launches.
    roofline = None
    if args.profile:
        for h in handles:
            h.profile(True)
            h.profile_read()
        first = sc[0]
        for _ in range(args.steps):
            step()
        kms, runs = np.zeros(5), 0
        for h in handles:
            ms, n = h.profile_read()
            kms += np.array(ms[0])
            runs += n
            h.profile(False)
        assert runs == nT * args.steps, (runs, nT * args.steps)
        gu_bytes = sum(step_gu_bytes[s % n_acts] for s in range(first, first + args.steps))
        achieved = gu_bytes / (kms[2] * 1e-3) / 1e9
        roofline = {"kernel": "gateup_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": read_traffic(TRAFFIC_FILE), "launches": runs,
                    "avg_launch_us": round(kms[2] * 1e3 / runs, 3),
                    "avg_bytes_per_launch": int(gu_bytes / runs),
                    "kernel_share": {n: round(float(v / kms.sum()), 3)
                                     for n, v in zip(("logits", "select", "gateup", "down", "combine"), kms)},
                    "avg_kernel_us": {n: round(float(v) * 1e3 / runs, 3)
                                      for n, v in zip(("logits", "select", "gateup", "down", "combine"), kms)}}

    # Per-width round latency (eager, events on torch's current stream = the handles' stream,
    # one synchronised round at a time) and per-kernel durations; outside the timed region. All six
    # verify widths (the headline step covers 1, 3 and 8); the rounds of the widths the step does
    # not run use the same handles (max_rows 8).
    per_T = {}
    ctl_buf = torch.empty(CONTROL_BUF_BYTES // 4, device=dev)
    ctl_off = [0]
    # (a counter pass, --pmc-calibrate, runs only the T = 1, 3, 8 steps: its per-dispatch traffic then
    # averages the same mix of gate/up launches as the roofline above)
    for T in (() if args.pmc_calibrate else TS_SWEEP):
        if T not in acts:
            acts[T] = torch.stack([synth.make_activations(cfg, T, seed=0, round_idx=r, device=dev)
                                   for r in range(n_acts)])
            outs[T] = torch.empty((T, cfg.H), device=dev)
        lat, nus = [], []
        for r in range(64):
            h = handles[(sc[0] + r) % R]
            a = acts[T][r % n_acts]
            lat.append(event_us(torch, lambda: h.run(a, cfg.k, outs[T])))
            nus.append(h.last_unique()[0])
        for h in handles:
            h.profile(True)
            h.profile_read()
        for r in range(64):
            handles[(sc[0] + r) % R].run(acts[T][r % n_acts], cfg.k, outs[T])
        kms, runs = np.zeros(5), 0
        for h in handles:
            ms, n = h.profile_read()
            kms += np.array(ms[0])
            runs += n
            h.profile(False)
        sc[0] += 64
        n_u = float(np.mean(nus))
        mb = synth.inputs.metric_bytes(cfg, n_u, T)
        med = float(np.median(lat))
        # Byte floor: every handle runs a round at T, then (R - 1 rounds later, its bytes long out of
        # the 256 MB cache) replays only its weight reads, with the same launches per layer.
        flo = []
        for rep in range(2):
            for r in range(R):
                handles[r].run(acts[T][(rep * R + r) % n_acts], cfg.k, outs[T])
            for r in range(R):
                flo.append(event_us(torch, handles[r].floor))
        # Streaming control: the same number of bytes, one contiguous read, each from a new window of
        # a 2 GB buffer (no window is read again before the buffer has cycled).
        ctl = []
        nbytes = (int(mb) + 15) // 16 * 16
        for r in range(32):
            if ctl_off[0] + nbytes > CONTROL_BUF_BYTES:
                ctl_off[0] = 0
            view = ctl_buf[ctl_off[0] // 4:(ctl_off[0] + nbytes) // 4]
            ctl_off[0] += nbytes
            ctl.append(event_us(torch, lambda: handles[0].stream_read(view)))
        fmed, cmed = float(np.median(flo)), float(np.median(ctl))
        per_T[str(T)] = {
            "round_us_median": round(med, 2),
            "round_us_p10_p90": [round(float(np.percentile(lat, 10)), 2), round(float(np.percentile(lat, 90)), 2)],
            "tok_per_s": round(T / med * 1e6, 1),
            "n_unique": round(n_u, 2),
            "metric_bytes": int(mb),
            "metric_GBps": round(mb / med / 1e3, 1),
            "frac_of_peak": round(mb / med / 1e3 / HBM_PEAK_GBS, 4),
            "kernel_us": {n: round(float(v) * 1e3 / runs, 2) for n, v in
                          zip(("logits", "select", "gateup", "down", "combine"), kms)},
            "byte_floor": {"us_median": round(fmed, 2), "GBps": round(mb / fmed / 1e3, 1),
                           "round_frac_of_floor": round(fmed / med, 3),
                           "what": "the round's weight reads alone (router, unique experts' gate/up, down) "
                                   "at the same addresses, 3 launches per layer"},
            "stream_control": {"us_median": round(cmed, 2), "GBps": round(mb / cmed / 1e3, 1),
                               "what": "one contiguous read of the metric bytes, one launch, same session"},
        }
    del ctl_buf
    # extra verify-row cost between consecutive widths and against T = 1
    per_T["extra_row"] = {}
    for a_, b_ in ([] if args.pmc_calibrate else list(zip(TS_SWEEP[:-1], TS_SWEEP[1:])) + [(1, 8)]):
        pa, pb = per_T[str(a_)], per_T[str(b_)]
        per_T["extra_row"][f"{a_}->{b_}"] = {
            "us_per_row": round((pb["round_us_median"] - pa["round_us_median"]) / (b_ - a_), 2),
            "bytes_per_row": int((pb["metric_bytes"] - pa["metric_bytes"]) / (b_ - a_)),
            "unique_experts_per_row": round((pb["n_unique"] - pa["n_unique"]) / (b_ - a_), 2),
        }

    # Labelled extra: the same widths replayed as captured hipGraphs (one graph per (T, k) and handle;
    # each round names a new input buffer, so each replay first uploads the ingress pointers).
    graph_per_T = None
    if not args.no_extra and not args.graph and not args.pmc_calibrate:
        ghs = [MoeRound([reps[i]], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=max(TS_SWEEP), use_graph=True, **shape)
               for i in range(R)]
        graph_per_T = {"mode": "hipGraph replay, one graph per (T, k), ingress upload per round"}
        for T in TS_SWEEP:
            for r in range(R):
                ghs[r].run(acts[T][r % n_acts], cfg.k, outs[T])  # capture
            lat = [event_us(torch, lambda: ghs[r % R].run(acts[T][(r + 7) % n_acts], cfg.k, outs[T]))
                   for r in range(64)]
            med = float(np.median(lat))
            # the same graphs with the round's input always in the same buffer: no ingress upload
            fixed = [event_us(torch, lambda: ghs[r % R].run(acts[T][0], cfg.k, outs[T])) for r in range(64)]
            graph_per_T[str(T)] = {"round_us_median": round(med, 2), "tok_per_s": round(T / med * 1e6, 1),
                                   "fixed_buffers_round_us_median": round(float(np.median(fixed)), 2),
                                   "eager_round_us_median": per_T[str(T)]["round_us_median"]}
        for h in ghs:
            h.close()
        del ghs

    for h in handles:
        h.close()
    del handles, reps
    torch.cuda.empty_cache()

    decode = None if args.no_extra else decode_rounds(torch, np, synth, MoeRound)
    exact = None if args.no_extra else exact_rounds(cfg, base, acts, torch, np, MoeRound)
    wide = None if args.no_extra else wide_rounds(cfg, base, torch, np, synth, MoeRound)
    deep = None if args.no_extra else deep_stack(torch, np, synth, MoeRound)
    superblock = None if args.no_extra else superblock_rounds(acts, args.replicas, torch, np, synth, MoeRound)
    prefill = None if args.no_extra else prefill_rounds(base, torch, np, synth, MoeRound)
    tier = None if args.no_extra else tier_rounds(torch, np, synth, MoeRound)
    launch = None if args.no_extra else launch_costs(torch, np, synth, MoeRound)
    choices = None if args.no_extra else launch_choices(cfg, base, torch, np, MoeRound)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, base, acts, args.cpu_seconds)

    line = {
        "metric": "MoE-round tok/s at T=1/3/8 rows; achieved HBM GB/s vs peak",
        "value": round(value, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": "verify sweep: one MoE layer, H=2048, E=256, top-8, I=512, Q4 blocks of 32; "
                               "one step = rounds at T=1, 3, 8 (12 rows)",
                   "global_batch": tokens_per_step, "seq_len": 1, "parallelism": "none (1 GPU)",
                   "mode": "hipGraph" if args.graph else "eager", "weight_replicas": args.replicas,
                   "launch": shape or "default"},
        "per_T": per_T,
        "graph_per_T": graph_per_T,
        "decode": decode,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "exact_mode": exact,
        "wide_rounds": wide,
        "deep_stack": deep,
        "superblock_format": superblock,
        "prefill": prefill,
        "expert_tier": tier,
        "launch_costs": launch,
        "launch_choices": choices,
    }
    print(json.dumps(line), flush=True)
    if args.pmc_calibrate:
        calibration_copy(torch, dev)


def calibration_copy(torch, dev):
    """A copy of CALIB_BYTES in and out (torch.neg of fp32), whose byte counters scale the kernels'."""
    src = torch.randn(CALIB_BYTES // 4, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


INT8_DENSE_PEAK_OPS = 5.0e15
BF16_DENSE_PEAK_FLOPS = 2.5e15


def event_us(torch, fn):
    """Microseconds between events recorded on the current stream around fn(), synchronised."""
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) * 1e3


def timed_rounds(h, xs, k, out, n, torch):
    """Median / p10 / p90 microseconds of n synchronised rounds, and the last per-kernel profile."""
    import numpy as np
    lat = []
    for r in range(n):
        torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        h.run(xs[r % len(xs)], k, out)
        e.record()
        e.synchronize()
        lat.append(s.elapsed_time(e) * 1e3)
    return float(np.median(lat)), float(np.percentile(lat, 10)), float(np.percentile(lat, 90))


def decode_rounds(torch, np, synth, MoeRound, n_rounds=1000, replicas=8):
    """Batch-1 decode, one layer (H=2048, E=128 with a Zipf(1.1) router bias, top-8, I=768): 1000
    rounds with fresh seeded activations over 8 weight replicas (3 GB, beyond the 256 MB cache):
    latency, unique experts, metric bytes, per-kernel time and the byte floor."""
    cfg = synth.config("decode")
    base = synth.make_layer(cfg, seed=0, layer=0, device="cuda")
    reps = [base] + [base.clone() for _ in range(replicas - 1)]
    hs = [MoeRound([rp], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=1, use_graph=False) for rp in reps]
    xs = torch.stack([synth.make_activations(cfg, 1, seed=0, round_idx=r, device="cuda") for r in range(n_rounds)])
    out = torch.empty((1, cfg.H), device="cuda")
    for r in range(2 * replicas):
        hs[r % replicas].run(xs[r], cfg.k, out)
    lat, nus = [], []
    for r in range(n_rounds):
        h = hs[r % replicas]
        lat.append(event_us(torch, lambda: h.run(xs[r], cfg.k, out)))
        nus.append(h.last_unique()[0])
    for h in hs:
        h.profile(True)
        h.profile_read()
    for r in range(64):
        hs[r % replicas].run(xs[r], cfg.k, out)
    kms, runs = np.zeros(5), 0
    for h in hs:
        ms, n = h.profile_read()
        kms += np.array(ms[0])
        runs += n
        h.profile(False)
    flo = []
    for rep in range(4):
        for r in range(replicas):
            hs[r].run(xs[rep * replicas + r], cfg.k, out)
        for r in range(replicas):
            flo.append(event_us(torch, hs[r].floor))
    for h in hs:
        h.close()
    med, fmed = float(np.median(lat)), float(np.median(flo))
    nu = float(np.mean(nus))
    mb = synth.inputs.metric_bytes(cfg, nu, 1)
    del reps, hs, base
    torch.cuda.empty_cache()
    return {"workload": "one MoE layer, H=2048, E=128 (Zipf 1.1 bias), top-8, I=768, T=1; 1000 fresh rounds",
            "rounds": n_rounds, "round_us_median": round(med, 2),
            "round_us_p10_p90": [round(float(np.percentile(lat, 10)), 2), round(float(np.percentile(lat, 90)), 2)],
            "tok_per_s": round(1 / med * 1e6, 1), "n_unique": round(nu, 2), "metric_bytes": int(mb),
            "metric_GBps": round(mb / med / 1e3, 1), "frac_of_peak": round(mb / med / 1e3 / HBM_PEAK_GBS, 4),
            "kernel_us": {n: round(float(v) * 1e3 / runs, 2)
                          for n, v in zip(("logits", "select", "gateup", "down", "combine"), kms)},
            "byte_floor": {"us_median": round(fmed, 2), "GBps": round(mb / fmed / 1e3, 1),
                           "round_frac_of_floor": round(fmed / med, 3)}}


def exact_rounds(cfg, layer, acts, torch, np, MoeRound):
    """The verify sweep in exact mode (fixed-order combine, bitwise row-independent outputs):
    median round latency and per-kernel time per width, on 8 weight replicas."""
    reps = [layer] + [layer.clone() for _ in range(7)]
    hs = [MoeRound([rp], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=max(TS), use_graph=False, exact=True) for rp in reps]
    res = {}
    for T in TS:
        out = torch.empty((T, cfg.H), device="cuda")
        for r in range(8):
            hs[r % 8].run(acts[T][r], cfg.k, out)
        lat = [timed_rounds(hs[r % 8], [acts[T][r]], cfg.k, out, 1, torch)[0] for r in range(48)]
        for h in hs:
            h.profile(True)
            h.profile_read()
        for r in range(48):
            hs[r % 8].run(acts[T][r], cfg.k, out)
        kms, runs = np.zeros(5), 0
        for h in hs:
            ms, n = h.profile_read()
            kms += np.array(ms[0])
            runs += n
            h.profile(False)
        med = float(np.median(lat))
        res[str(T)] = {"round_us_median": round(med, 2), "tok_per_s": round(T / med * 1e6, 1),
                       "kernel_us": {n: round(float(v) * 1e3 / runs, 2)
                                     for n, v in zip(("logits", "select", "gateup", "down", "combine"), kms)}}
    for h in hs:
        h.close()
    del reps
    torch.cuda.empty_cache()
    return res


def wide_rounds(vcfg, layer, torch, np, synth, MoeRound):
    """Copy-heavy wide verify (T = 16, 32, 64 independent rows, same layer shape): round latency,
    per-kernel time, unique experts and bytes, with the default (the integer-dot GEMV for every work
    item), with work items of 2 and of 4 rows explicitly (the default takes 2 up to 32 rows, 4
    above) and with the int8 matrix-core tiles (gate/up and down) for 4-row items' 3+ rows; the round's
    useful expert flops (2 T k 3 H I) against the dense bf16 matrix peak, and the useful operations the
    tiles carried against the dense int8 peak."""
    cfg = synth.config("wide")
    reps = [layer] + [layer.clone() for _ in range(3)]  # 4 x 503 MB: beyond the 256 MB cache
    res = {}
    for T in cfg.T:
        xs = [synth.make_activations(cfg, T, seed=0, round_idx=r, device="cuda") for r in range(16)]
        out = torch.empty((T, cfg.H), device="cuda")
        row = {}
        for name, mfma, rpi in (("default", 0, 0), ("two_row_items", 0, 2), ("four_row_items", 0, 4),
                                ("mfma_tile", 3, 4)):
            hs = [MoeRound([rp], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=64, use_graph=False, mfma_min_rows=mfma,
                           rows_per_item=rpi) for rp in reps]
            for r in range(8):
                hs[r % 4].run(xs[r], cfg.k, out)
            lat = []
            for r in range(24):
                med = timed_rounds(hs[r % 4], [xs[r % 16]], cfg.k, out, 1, torch)[0]
                lat.append(med)
            nus, mfma_ops = [], 0.0
            for h in hs:
                h.profile(True)
                h.profile_read()
            for r in range(16):
                h = hs[r % 4]
                h.run(xs[r], cfg.k, out)
                uniq, offs, _ = h.worklist(0)
                nus.append(len(uniq))
                for npr in np.diff(offs):  # items of <= 4 rows; those with >= 3 rows take the tiles
                    for it in range(0, int(npr), 4):
                        rows = min(4, int(npr) - it)
                        if mfma > 0 and rows >= mfma:  # gate, up and down on the matrix cores
                            mfma_ops += 2.0 * 3 * cfg.I * cfg.H * rows
            kms, runs = np.zeros(5), 0
            for h in hs:
                ms, n = h.profile_read()
                kms += np.array(ms[0])
                runs += n
                h.profile(False)
                h.close()
            nu = float(np.mean(nus))
            mb = synth.inputs.metric_bytes(cfg, nu, T)
            med = float(np.median(lat))
            gu_s = kms[2] * 1e-3
            row[name] = {
                "round_us_median": round(med, 2), "n_unique": round(nu, 1), "metric_bytes": int(mb),
                "metric_GBps": round(mb / med / 1e3, 1), "tok_per_s": round(T / med * 1e6, 1),
                "kernel_us": {n: round(float(v) * 1e3 / runs, 2)
                              for n, v in zip(("logits", "select", "gateup", "down", "combine"), kms)},
            }
            useful = 2.0 * T * cfg.k * 3 * cfg.H * cfg.I   # the round's expert multiply-adds x 2
            row[name]["useful_TFLOPs_round"] = round(useful / med / 1e6, 2)
            row[name]["useful_frac_of_bf16_peak"] = round(useful / (med * 1e-6) / BF16_DENSE_PEAK_FLOPS, 5)
            tile_ops = mfma_ops / 16  # per round (16 rounds counted above)
            row[name]["mfma_tile_useful_ops_per_round"] = tile_ops
            row[name]["mfma_tile_frac_of_int8_peak"] = round(tile_ops / (med * 1e-6) / INT8_DENSE_PEAK_OPS, 6)
        res[str(T)] = row
    del reps
    torch.cuda.empty_cache()
    return res


# The prefill GEMMs run on fp16 matrix instructions, each activation split into two fp16 values:
# per model multiply-add the matrix cores execute two (4 flops), against MI355X's dense fp16 peak.
FP16_DENSE_PEAK_FLOPS = 2.5e15


def prefill_rounds(layer, torch, np, synth, MoeRound, widths=None):
    """Prefill rounds (T = 512, 4096 independent rows, the verify layer shape): rows per second,
    per-kernel time, and the gate/up GEMM's executed fp16 matrix rate (two planes over 64-pair
    tiles) against the dense fp16 peak, with its model rate beside it."""
    from verify_router_gemv_amd.profsum import read_traffic

    cfg = synth.config("prefill")
    widths = tuple(widths or cfg.T)
    h = MoeRound([layer], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=max(widths), use_graph=False)
    res = {}
    for T in widths:
        xs = [synth.make_activations(cfg, T, seed=0, round_idx=r, device="cuda") for r in range(4)]
        out = torch.empty((T, cfg.H), device="cuda")
        for r in range(2):
            h.run(xs[r], cfg.k, out)
        lat = [timed_rounds(h, [xs[r % 4]], cfg.k, out, 1, torch)[0] for r in range(10)]
        h.profile(True)
        h.profile_read()
        tiles = 0
        for r in range(4):
            h.run(xs[r], cfg.k, out)
            _, offs, _ = h.worklist(0)
            tiles += int(sum((int(n) + 63) // 64 for n in np.diff(offs)))
        ms, runs = h.profile_read()
        h.profile(False)
        kms = np.array(ms[0]) / runs
        med = float(np.median(lat))
        pairs = T * cfg.k
        gu_model = 2.0 * 2 * cfg.I * cfg.H * pairs          # model ops (multiply-add = 2)
        dn_model = 2.0 * cfg.I * cfg.H * pairs
        gu_exec = 2 * 2.0 * 2 * cfg.I * cfg.H * 64 * tiles / runs   # fp16 flops the matrix cores ran
        gu_s = kms[2] * 1e-3
        res[str(T)] = {
            "round_us_median": round(med, 1),
            "tok_per_s": round(T / med * 1e6, 1),
            "kernel_us": {n: round(float(v) * 1e3, 1) for n, v in
                          zip(("quant_x+logits", "topk+sort", "gateup", "quant_h+down", "combine"), kms)},
            "model_TOPs_round": round((gu_model + dn_model) / med / 1e6, 1),
            "gateup": {"bound": "mfma", "achieved": round(gu_exec / gu_s / 1e12, 1),
                       "peak": round(FP16_DENSE_PEAK_FLOPS / 1e12, 1),
                       "unit": "TFLOP/s (fp16, executed: 2 planes, 64-pair tiles)",
                       "frac": round(gu_exec / gu_s / FP16_DENSE_PEAK_FLOPS, 3),
                       "avg_launch_us": round(float(kms[2]) * 1e3, 1),
                       "model_TOPs": round(gu_model / gu_s / 1e12, 1),
                       "traffic": (read_traffic(PREFILL_TRAFFIC_FILE, "pf_gateup")
                                   if T == PREFILL_TRAFFIC_T else None)},
        }
        del xs
    h.close()
    torch.cuda.empty_cache()
    return {"workload": "one MoE layer, H=2048, E=256, top-8, I=512, Q4B32; independent rows",
            "fp16_dense_peak_TFLOPs": round(FP16_DENSE_PEAK_FLOPS / 1e12, 1), "rounds": res}


def deep_stack(torch, np, synth, MoeRound, fmt="q4b32", modes=("graph", "eager"), split=True):
    """48 MoE layers (E=512, top-10, I=512), T=3, residual, ~48 GB of expert weights resident (43.5 GB
    in the 4.5-bit layout): one round as one captured hipGraph, and eager, with per-layer unique
    experts and metric bytes; the per-kernel split of a layer (dispatch timestamps of eager rounds,
    averaged over layers and rounds) and the round's byte floor (its weight reads alone, 3 launches
    per layer, after a 1 GB read that pushes the round's bytes out of the cache)."""
    cfg = synth.config("deep").replace(fmt=fmt)
    t0 = time.perf_counter()
    layers = [synth.make_layer(cfg, seed=0, layer=l, device="cuda") for l in range(cfg.L)]
    gen_s = time.perf_counter() - t0
    T = cfg.T[0]
    xs = [synth.make_activations(cfg, T, seed=0, round_idx=r, device="cuda") for r in range(8)]
    out = torch.empty((T, cfg.H), device="cuda")
    res = {"layers": cfg.L, "T": T, "weights_GB": round(cfg.L * cfg.E * cfg.expert_bytes() / 1e9, 2),
           "generate_s": round(gen_s, 1)}
    flush = torch.empty(CONTROL_BUF_BYTES // 8, device="cuda")
    for mode in modes:
        h = MoeRound(layers, cfg.H, cfg.I, cfg.E, cfg.k, max_rows=T, residual=True, use_graph=(mode == "graph"))
        for r in range(3):
            h.run(xs[r], cfg.k, out)
        lat = [timed_rounds(h, [xs[r % 8]], cfg.k, out, 1, torch)[0] for r in range(12)]
        nus = h.last_unique()
        med = float(np.median(lat))
        mb = sum(synth.inputs.metric_bytes(cfg, nu, T) for nu in nus)
        res[mode] = {"round_us_median": round(med, 1), "per_layer_us": round(med / cfg.L, 2),
                     "n_unique_mean": round(float(np.mean(nus)), 2), "metric_bytes": int(mb),
                     "metric_GBps": round(mb / med / 1e3, 1), "frac_of_peak": round(mb / med / 1e3 / HBM_PEAK_GBS, 4),
                     "tok_per_s": round(T / med * 1e6, 1)}
        if split and mode == "graph":
            flo = []
            for r in range(6):
                h.run(xs[r], cfg.k, out)
                h.stream_read(flush)
                flo.append(event_us(torch, h.floor))
            fmed = float(np.median(flo))
            res[mode]["byte_floor"] = {"us_median": round(fmed, 1), "per_layer_us": round(fmed / cfg.L, 2),
                                       "GBps": round(mb / fmed / 1e3, 1), "round_frac_of_floor": round(fmed / med, 3)}
        if split and mode == "eager":
            h.profile(True)
            h.profile_read()
            for r in range(6):
                h.run(xs[r], cfg.k, out)
            ms, n = h.profile_read()
            h.profile(False)
            per = np.array(ms).sum(axis=0) / (n * cfg.L)
            res[mode]["per_layer_kernel_us"] = {nm: round(float(v) * 1e3, 2) for nm, v in
                                                zip(("logits", "select", "gateup", "down", "combine"), per)}
        h.close()
    del layers, flush
    torch.cuda.empty_cache()
    return res


def launch_choices(cfg, base, torch, np, MoeRound, replicas=8):
    """The measurements behind two launch-shape defaults, per verify width:
    - selection_placement: the selection folded into every gate/up block (fused_max_rows = 15)
      against its own one-block kernel (-1); the default folds it in up to the widest T where
      that is faster;
    - rows_per_item: work items of 1 against 2 rows of an expert; the default takes 1 up to the
      widest T where that is faster.
    Rounds of one width over `replicas` copies of the layer (each round reads its weights from
    HBM), 16 launched back to back between two events; median of 12 such chains, per round."""
    import synth
    reps = [base] + [base.clone() for _ in range(replicas - 1)]
    res = {"timing": "16 rounds back to back between events, median of 12, per round"}

    def compare(widths, variants):
        table = {}
        for T in widths:
            xs = [synth.make_activations(cfg, T, seed=0, round_idx=r, device="cuda") for r in range(16)]
            out = torch.empty((T, cfg.H), device="cuda")
            row = {}
            for name, shape in variants:
                hs = [MoeRound([rp], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=max(widths), use_graph=False, **shape)
                      for rp in reps]

                def chain():
                    for i in range(16):
                        hs[i % replicas].run(xs[i], cfg.k, out)
                chain()
                lat = [event_us(torch, chain) / 16 for _ in range(12)]
                row[name + "_round_us"] = round(float(np.median(lat)), 2)
                for h in hs:
                    h.close()
            table[str(T)] = row
        return table

    res["selection_placement"] = compare((1, 4, 8, 12, 15),
                                         (("fused", {"fused_max_rows": 15}), ("separate", {"fused_max_rows": -1})))
    res["rows_per_item"] = compare((3, 6, 8, 10, 12, 15),
                                   (("one_row", {"rows_per_item": 1}), ("two_rows", {"rows_per_item": 2})))
    del reps
    torch.cuda.empty_cache()
    return res


def launch_costs(torch, np, synth, MoeRound):
    """What launching costs on this GPU, for the design's launch budget: chains of N minimal kernels
    (the byte floor's read kernel over 16 bytes, one block) between two events, and one such kernel
    alone; then chains of 16 one-wave-per-block kernels of B blocks each (B = 1 .. 1024), empty, storing
    one word per block, or sleeping a fixed time first so that all blocks of a kernel end together:
    how the time per launch grows with the blocks of the kernel. Medians of 50 timings each."""
    cfg = synth.config("tiny")
    layer = synth.make_layer(cfg, seed=0, layer=0, device="cuda")
    h = MoeRound([layer], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=1, use_graph=False)
    buf = torch.zeros(4, device="cuda")
    flags = torch.zeros(1024, dtype=torch.int32, device="cuda")
    # Half a second of back-to-back launches first, so that the figures do not depend on whether
    # the GPU was idle (its clocks ramp up under load).
    t_end = time.perf_counter() + 0.5
    while time.perf_counter() < t_end:
        h.empty_launches(1024, 64, 4, flags)
        torch.cuda.synchronize()
    res = {"kernel": "one block reading 16 bytes", "timing": "torch events around the launches",
           "warmup": "0.5 s of launches before the first timing"}
    for n in (1, 3, 10, 50):
        def chain():
            for _ in range(n):
                h.stream_read(buf)
        chain()
        lat = [event_us(torch, chain) for _ in range(50)]
        med = float(np.median(lat))
        res[f"chain_{n}"] = {"us_median": round(med, 2), "us_per_launch": round(med / n, 2)}
    # Chains of 16 one-wave kernels of B blocks: empty; each block storing one word; each block
    # sleeping ~4 × 2048 clocks first (all blocks of a kernel end together) and then storing.
    variants = {"empty": (0, None), "store": (0, flags), "sleep_store": (4, flags), "sleep": (4, None)}
    for name, (su, fl) in variants.items():
        per_blocks = {}
        for b in (1, 64, 256, 512, 1024):
            h.empty_launches(b, 16, su, fl)
            lat = [event_us(torch, lambda: h.empty_launches(b, 16, su, fl)) for _ in range(50)]
            per_blocks[str(b)] = round(float(np.median(lat)) / 16, 2)
        res[f"{name}_kernels_us_per_launch_by_blocks"] = per_blocks
        res[f"{name}_ns_per_block"] = round((per_blocks["1024"] - per_blocks["1"]) / 1023 * 1e3, 1)
    h.close()
    return res


def tier_rounds(torch, np, synth, MoeRound, L=8, resident_frac=0.25, skip_rank=7):
    """Both residency patterns of tier_placement: the hottest experts resident (a cache filled by
    popularity) and a random quarter resident (a cold cache: most routed experts are missed)."""
    return {"hottest_resident": tier_placement(torch, np, synth, MoeRound, L, resident_frac, skip_rank, "hot"),
            "random_resident": tier_placement(torch, np, synth, MoeRound, L, resident_frac, skip_rank, "random")}


def tier_placement(torch, np, synth, MoeRound, L, resident_frac, skip_rank, placement):
    """Experts read through the pointer table (T=3 rounds of the 512-expert, top-10 stack's shape,
    8 layers): the contiguous arrays; the table with every expert in device memory (the cost of the
    indirection); a quarter of each layer's experts in device memory (placement "hot": the most
    popular under the router's Zipf bias; "random": a seeded random quarter) and the rest in pinned
    host memory read in place over the host link, without and with the tail skip at rank 7; and the
    tail skip over the same residency with every expert in device memory. Per mode: round latency,
    unique experts read, missed experts read from the host tier and the host-link rate they imply,
    experts skipped and their bytes."""
    from verify_router_gemv_amd import binding
    cfg = synth.config("deep").replace(L=L)
    T = cfg.T[0]
    layers = [synth.make_layer(cfg, seed=0, layer=l, device="cuda") for l in range(L)]
    rcfg = cfg if placement == "hot" else cfg.replace(zipf_s=None)  # no bias: a seeded random subset
    res = [synth.make_residency(rcfg, resident_frac, seed=0, layer=l) for l in range(L)]
    t0 = time.perf_counter()
    host = []  # per layer: the missed experts' matrices in pinned host memory
    for l in range(L):
        missed = torch.as_tensor(np.flatnonzero(~res[l]), device="cuda")
        hl = {}
        for f in binding.EXPERT_FIELDS:
            src = getattr(layers[l], f)
            hl[f] = torch.empty((len(missed),) + tuple(src.shape[1:]), dtype=src.dtype, pin_memory=True)
            hl[f].copy_(src[missed].cpu())
        host.append(hl)
    pin_s = time.perf_counter() - t0

    def entries(tiered):
        rows = []
        for l in range(L):
            slot = {int(e): i for i, e in enumerate(np.flatnonzero(~res[l]))}
            rows.append([{f: (host[l][f][slot[e]] if tiered and not res[l][e] else getattr(layers[l], f)[e])
                          for f in binding.EXPERT_FIELDS} for e in range(cfg.E)])
        return rows

    dev_table = binding.make_expert_table(entries(False), cfg.H, cfg.I)
    tier_table = binding.make_expert_table(entries(True), cfg.H, cfg.I)
    bits = binding.residency_bits(np.stack(res))
    routers = [{"router_w": l.router_w, "router_b": l.router_b} for l in layers]
    xs = [synth.make_activations(cfg, T, seed=0, round_idx=r, device="cuda") for r in range(8)]
    out = torch.empty((T, cfg.H), device="cuda")
    eb = cfg.expert_bytes()
    result = {"layers": L, "T": T, "E": cfg.E, "k": cfg.k, "resident_frac": resident_frac,
              "skip_rank": skip_rank, "host_tier_GB": round(sum(v.numel() * v.element_size()
                                                                for hl in host for v in hl.values()) / 1e9, 2),
              "pin_and_copy_s": round(pin_s, 1)}
    modes = {
        "contiguous": (dict(), layers, None, None),
        "table_device": (dict(expert_table=True), routers, dev_table, None),
        "table_host_tier": (dict(expert_table=True), routers, tier_table, None),
        "table_host_tier_skip": (dict(expert_table=True, tail_skip_rank=skip_rank), routers, tier_table, bits),
        "contiguous_skip": (dict(tail_skip_rank=skip_rank), layers, None, bits),
    }
    for name, (kw, lays, table, rbits) in modes.items():
        h = MoeRound(lays, cfg.H, cfg.I, cfg.E, cfg.k, max_rows=T, residual=True, use_graph=True, **kw)
        if table is not None or rbits is not None:
            h.bind_experts(table, rbits)
        for r in range(3):
            h.run(xs[r], cfg.k, out)
        lat, nus, missed_read, skipped = [], [], [], []
        for r in range(8):
            lat.append(timed_rounds(h, [xs[r]], cfg.k, out, 1, torch)[0])
            st, nu, _ = h.last_stats()
            nus.append(float(np.mean(nu)))
            skipped.append(st.skipped / L)
            m = 0
            for l in range(L):
                uniq = h.worklist(l)[0]
                m += sum(1 for e in uniq if not res[l][e])
            missed_read.append(m / L)
        med = float(np.median(lat))
        per_layer = med / L
        mr = float(np.mean(missed_read))
        tiered = name.startswith("table_host")
        result[name] = {"round_us_median": round(med, 1), "per_layer_us": round(per_layer, 2),
                        "n_unique_per_layer": round(float(np.mean(nus)), 2),
                        "missed_experts_read_per_layer": round(mr, 2),
                        "skipped_experts_per_layer": round(float(np.mean(skipped)), 2),
                        "skipped_bytes_per_layer": int(float(np.mean(skipped)) * eb),
                        "host_link_GBps": round(mr * eb / per_layer / 1e3, 1) if tiered else None,
                        "tok_per_s": round(T / med * 1e6, 1)}
        h.close()
    del host, layers, dev_table, tier_table
    torch.cuda.empty_cache()
    return result


def superblock_rounds(acts, replicas, torch, np, synth, MoeRound):
    """The verify sweep with the 4.5-bit super-block layout (Q4S256): per width, round latency, per-kernel
    time, unique experts and metric bytes, on as many weight replicas as the headline; then the
    48-layer stack in that layout as one hipGraph."""
    cfg = synth.config("verify").replace(fmt="q4s256")
    base = synth.make_layer(cfg, seed=0, layer=0, device="cuda")
    reps = [base] + [base.clone() for _ in range(replicas - 1)]
    hs = [MoeRound([rp], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=max(TS), use_graph=False) for rp in reps]
    R = len(hs)
    res = {"format": "q4s256: 4-bit codes, 256-weight super-blocks, 6-bit sub-block scale/min (0.5625 B/weight)",
           "expert_bytes": cfg.expert_bytes(), "verify": {}}
    for T in TS:
        out = torch.empty((T, cfg.H), device="cuda")
        for r in range(2 * R):
            hs[r % R].run(acts[T][r % len(acts[T])], cfg.k, out)
        lat, nus = [], []
        for r in range(64):
            h = hs[r % R]
            lat.append(timed_rounds(h, [acts[T][r % len(acts[T])]], cfg.k, out, 1, torch)[0])
            nus.append(h.last_unique()[0])
        for h in hs:
            h.profile(True)
            h.profile_read()
        for r in range(64):
            hs[r % R].run(acts[T][r % len(acts[T])], cfg.k, out)
        kms, runs = np.zeros(5), 0
        for h in hs:
            ms, n = h.profile_read()
            kms += np.array(ms[0])
            runs += n
            h.profile(False)
        med = float(np.median(lat))
        nu = float(np.mean(nus))
        mb = synth.inputs.metric_bytes(cfg, nu, T)
        res["verify"][str(T)] = {
            "round_us_median": round(med, 2), "tok_per_s": round(T / med * 1e6, 1), "n_unique": round(nu, 2),
            "metric_bytes": int(mb), "metric_GBps": round(mb / med / 1e3, 1),
            "kernel_us": {n: round(float(v) * 1e3 / runs, 2)
                          for n, v in zip(("logits", "select", "gateup", "down", "combine"), kms)}}
    for h in hs:
        h.close()
    del hs, reps, base
    torch.cuda.empty_cache()
    res["deep_stack"] = deep_stack(torch, np, synth, MoeRound, fmt="q4s256", modes=("graph",), split=False)
    return res


def host_description():
    """nproc, the CPU model and this process's affinity mask, as reported by the host."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = sorted(os.sched_getaffinity(0))
    except AttributeError:
        aff = []
    return {"nproc": os.cpu_count(), "cpu_model": model, "affinity": compress_ranges(aff),
            "usable_cpus": len(aff)}


def compress_ranges(ids):
    out, i = [], 0
    while i < len(ids):
        j = i
        while j + 1 < len(ids) and ids[j + 1] == ids[j] + 1:
            j += 1
        out.append(f"{ids[i]}-{ids[j]}" if j > i else f"{ids[i]}")
        i = j + 1
    return ",".join(out)


def cpu_baseline(cfg, layer, acts, seconds):
    """The fp64 oracle on the host cores over a bounded sample of the same rounds (T = 1, 3, 8
    cycling): once with the BLAS pool at its default size (all usable cores) and once with one
    thread."""
    import numpy as np

    import oracle
    view = {
        "router_w": layer.router_w.cpu().numpy(), "router_b": None,
        **{f: (getattr(layer, f).cpu().numpy().view(np.uint32) if f.endswith("_sm")
               else getattr(layer, f).cpu().numpy())
           for f in ("gate_q", "gate_sm", "up_q", "up_sm", "down_q", "down_sm")},
    }

    def sample(limit):
        done_rows, n_rounds, r = 0, 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < limit or n_rounds < 3:
            for T in TS:
                X = acts[T][r % acts[T].shape[0]].cpu().numpy()
                oracle.moe_round([view], X, cfg.k, residual=False)
                done_rows += T
                n_rounds += 1
            r += 1
        el = time.perf_counter() - t0
        return done_rows / el, n_rounds, el

    threads = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threadpool_limits = None
    rate, n_all, el_all = sample(seconds)
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            r1, n1, el1 = sample(seconds)
        one = {"value": round(r1, 2), "unit": "tok/s", "cores": 1,
               "sample": f"{n1} rounds in {el1:.1f}s"}
    return {"value": round(rate, 2), "unit": "tok/s", "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": f"{n_all} rounds (T=1,3,8 cycling) of the same workload in {el_all:.1f}s, fp64 numpy, "
                      f"weights copied to host; BLAS threads = the pool's default",
            "one_thread": one, "host": host_description()}


if __name__ == "__main__":
    main()
