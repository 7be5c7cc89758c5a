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
TS = (1, 3, 8)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--replicas", type=int, default=32)
    p.add_argument("--graph", action="store_true", help="replay captured hipGraphs instead of eager launches")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    return p.parse_args()


def gateup_bytes(cfg, n_unique, T):
    """Algorithmic bytes of one gate/up launch: unique experts' gate+up codes and scale/min words,
    the T input rows, and the T*k SwiGLU output rows."""
    w = n_unique * 2 * cfg.I * cfg.H * (0.5 + 4.0 / 32.0)
    return w + T * cfg.H * 4 + T * cfg.k * cfg.I * 4


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported by this build "
              "(the round would shard by splitting each expert's I rows across GPUs, see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from verify_router_gemv_amd import MoeRound

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    cfg = synth.config("verify")
    base = synth.make_layer(cfg, seed=0, layer=0, device=dev)
    reps = [base] + [base.clone() for _ in range(args.replicas - 1)]
    n_acts = 256
    acts = {T: torch.stack([synth.make_activations(cfg, T, seed=0, round_idx=r, device=dev)
                            for r in range(n_acts)]) for T in TS}
    outs = {T: torch.empty((T, cfg.H), device=dev) for T in TS}
    handles = [MoeRound([reps[i]], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=max(TS), use_graph=args.graph)
               for i in range(args.replicas)]
    R = args.replicas
    counter = [0]

    def step():
        for T in TS:
            i = counter[0]
            handles[i % R].run(acts[T][i % n_acts], cfg.k, outs[T])
            counter[0] += 1

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

    # Per-width latency and per-kernel durations (HIP events around each kernel, eager, on the
    # handles' stream), plus unique-expert counts; outside the timed region.
    per_T = {}
    gu_ms, gu_bytes = [], []
    for T in TS:
        lat, nus, kern = [], [], []
        for r in range(64):
            h = handles[(counter[0] + r) % R]
            a = acts[T][r % n_acts]
            torch.cuda.synchronize()
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            h.run(a, cfg.k, outs[T])
            e.record()
            e.synchronize()
            lat.append(s.elapsed_time(e) * 1e3)
            nus.append(h.last_unique()[0])
            kern.append(h.run_timed(a, cfg.k, outs[T])[0])
        kern = np.array(kern) * 1e3  # us, [round][kernel]
        nu = float(np.mean(nus))
        mb = synth.inputs.metric_bytes(cfg, nu, T)
        med = float(np.median(lat))
        per_T[str(T)] = {
            "round_us_median": round(med, 2),
            "tok_per_s": round(T / med * 1e6, 1),
            "n_unique": round(nu, 2),
            "metric_bytes": int(mb),
            "metric_GBps": round(mb / med / 1e3, 1),
            "kernel_us": {n: round(float(v), 2) for n, v in
                          zip(("logits", "select", "gateup", "down"), kern.mean(0))},
        }
        gu_ms.extend(kern[:, 2].tolist())
        gu_bytes.extend([gateup_bytes(cfg, n, T) for n in nus])
    # extra verify-row cost, T=1 -> 3 -> 8
    per_T["extra_row"] = {
        f"{a}->{b}": {
            "us_per_row": round((per_T[str(b)]["round_us_median"] - per_T[str(a)]["round_us_median"]) / (b - a), 2),
            "bytes_per_row": int((per_T[str(b)]["metric_bytes"] - per_T[str(a)]["metric_bytes"]) / (b - a)),
        } for a, b in ((1, 3), (3, 8))}

    achieved = float(np.mean(gu_bytes)) / (float(np.mean(gu_ms)) * 1e-6) / 1e9  # GB/s
    roofline = {"kernel": "gateup", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, reps[0], acts, args.cpu_seconds)

    for h in handles:
        h.close()

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
                   "mode": "hipGraph" if args.graph else "eager", "weight_replicas": args.replicas},
        "per_T": per_T,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def cpu_baseline(cfg, layer, acts, seconds):
    """The fp64 oracle on the host cores over a bounded sample of the same rounds."""
    import numpy as np

    import oracle
    view = {
        "router_w": layer.router_w.cpu().numpy(), "router_b": None,
        **{f: (getattr(layer, f).cpu().numpy().view(np.uint32) if f.endswith("_sm")
               else getattr(layer, f).cpu().numpy())
           for f in ("gate_q", "gate_sm", "up_q", "up_sm", "down_q", "down_sm")},
    }
    done_rows, t0, n_rounds = 0, time.perf_counter(), 0
    r = 0
    while time.perf_counter() - t0 < seconds or n_rounds < 3:
        for T in TS:
            X = acts[T][r % acts[T].shape[0]].cpu().numpy()
            oracle.moe_round([view], X, cfg.k, residual=False)
            done_rows += T
            n_rounds += 1
        r += 1
    el = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    return {"value": round(done_rows / el, 2), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_rounds} rounds ({r} steps of T=1,3,8) of the same workload in {el:.1f}s, "
                      f"fp64 numpy, weights copied to host"}


if __name__ == "__main__":
    main()
