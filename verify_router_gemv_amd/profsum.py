"""Short text summaries of rocprofv3 output for the round's kernels.

    python -m verify_router_gemv_amd.profsum stats  STATS_CSV OUT "COMMAND"
        per-kernel dispatch durations (calls, average, min, max) of the moe:: kernels from a
        `rocprofv3 --kernel-trace --stats` *_kernel_stats.csv
    python -m verify_router_gemv_amd.profsum traffic FETCH_DIR WRITE_DIR OUT "COMMAND" [KERNEL]
        gate/up HBM traffic per dispatch from a FETCH_SIZE pass and a WRITE_SIZE pass of
        `bench.py --pmc-calibrate`, each scaled by its own reading for the run's closing copy of
        CALIB_BYTES in and out (torch.neg of a 1 GiB fp32 tensor). KERNEL is "gateup" (the decode
        gate/up, default) or "pf_gateup" (the prefill gate/up GEMM).
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CALIB_BYTES = 1 << 30
KERNEL_SOURCES = [os.path.join(PKG, "csrc", f) for f in
                  ("moe_common.h", "moe_route.h", "moe_gemv.h", "moe_gateup.h", "moe_gemv_g64.hip")]
PREFILL_SOURCES = [os.path.join(PKG, "csrc", f) for f in
                   ("moe_common.h", "moe_route.h", "moe_gemv.h", "moe_prefill.h")]

# Traffic targets: the kernel-name prefix a dispatch must carry, the sources its code comes from,
# and the workload line of the summary.
TRAFFIC_KERNELS = {
    "gateup": ("moe::gateup_kernel<", KERNEL_SOURCES,
               "gate/up HBM traffic per dispatch, verify sweep (T = 1, 3, 8; 32 weight replicas)"),
    "pf_gateup": ("moe::pf::pf_gateup_kernel<", PREFILL_SOURCES,
                  "prefill gate/up GEMM HBM traffic per dispatch (T = 4096 rows, top-8, E = 256)"),
}


def kernel_source_hash(sources=None) -> str:
    """Hash of the sources a kernel is compiled from (a traffic figure is valid for these)."""
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(path: str, kernel: str = "gateup"):
    """traffic_bytes_per_launch of a traffic summary if it was taken on the current kernel sources."""
    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    except OSError:
        return None
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(TRAFFIC_KERNELS[kernel][1]):
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def stats(stats_csv: str, out_path: str, command: str) -> None:
    rows = []
    for r in csv.DictReader(open(stats_csv)):
        n = r["Name"]
        if "moe::" in n:  # the library's kernels (input generation and copies are left out)
            short = n.split("(")[0].replace("void moe::", "")
            rows.append((short, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    rows.sort(key=lambda x: -x[1] * x[2])
    sweep = [r for r in rows if r[0] in VERIFY_SWEEP_GATEUP]
    with open(out_path, "w") as fh:
        fh.write(f"# rocprofv3 kernel statistics\n# command: {command}\n")
        fh.write(f"{'kernel':36s} {'calls':>7s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s} {'pct':>6s}\n")
        for s in rows:
            fh.write(f"{s[0]:36s} {s[1]:7d} {s[2]:8.3f} {s[3]:8.3f} {s[4]:8.3f} {s[5]:6.2f}\n")
        if sweep:
            calls = sum(r[1] for r in sweep)
            mean = sum(r[1] * r[2] for r in sweep) / calls
            fh.write(f"# gate/up of the verify sweep (the forms T = 1, 3, 8 launch: {', '.join(VERIFY_SWEEP_GATEUP)};\n"
                     f"# exact-mode rounds launch the same ones): {calls} calls, call-weighted mean {mean:.3f} us\n")
    print(open(out_path).read())


# The gate/up instantiations the verify sweep launches (H = 2048: 64 lanes x 1 block, 4 rows per
# lane group; the one-row form with the folded selection at T = 1, one-row items with it at T = 3
# and 8; per-32 weight format). These forms also serve the bench's other widths up to 10 rows, so
# the mean covers those launches too.
VERIFY_SWEEP_GATEUP = ("gateup_kernel<64, 1, 4, 0, 4, 0>", "gateup_kernel<64, 1, 4, 3, 4, 0>")


def _per_dispatch(d: str, counter: str, prefix: str):
    acc = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") != counter:
                continue
            name = r["Kernel_Name"]
            key = "gateup" if prefix in name else ("copy" if "neg_kernel" in name else None)
            if key:
                disp = acc.setdefault(key, {})
                did = r["Dispatch_Id"]
                disp[did] = disp.get(did, 0.0) + float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}


def traffic(fetch_dir: str, write_dir: str, out_path: str, command: str, kernel: str = "gateup") -> None:
    prefix, sources, title = TRAFFIC_KERNELS[kernel]
    fetch, nf = _per_dispatch(fetch_dir, "FETCH_SIZE", prefix)
    write, nw = _per_dispatch(write_dir, "WRITE_SIZE", prefix)
    f_scale = CALIB_BYTES / (fetch["copy"] * 1024.0)
    w_scale = CALIB_BYTES / (write["copy"] * 1024.0)
    rd = fetch["gateup"] * 1024.0 * f_scale
    wr = write["gateup"] * 1024.0 * w_scale
    with open(out_path, "w") as fh:
        fh.write(f"# {title}\n"
                 f"# command: {command}\n"
                 "# FETCH_SIZE and WRITE_SIZE (KiB per dispatch) come from two rocprofv3 --pmc passes; each is\n"
                 f"# scaled by its own reading for the closing copy of {CALIB_BYTES} bytes in and out.\n"
                 f"kernel_source_sha256_16: {kernel_source_hash(sources)}\n"
                 f"gateup_dispatches: {nf['gateup']} / {nw['gateup']}\n"
                 f"fetch_kib_per_dispatch_raw: {fetch['gateup']:.1f}\n"
                 f"write_kib_per_dispatch_raw: {write['gateup']:.1f}\n"
                 f"copy_fetch_kib_raw: {fetch['copy']:.1f}\n"
                 f"copy_write_kib_raw: {write['copy']:.1f}\n"
                 f"fetch_scale: {f_scale:.4f}\n"
                 f"write_scale: {w_scale:.4f}\n"
                 f"read_bytes_per_launch: {rd:.0f}\n"
                 f"write_bytes_per_launch: {wr:.0f}\n"
                 f"traffic_bytes_per_launch: {rd + wr:.0f}\n")
    print(open(out_path).read())


if __name__ == "__main__":
    cmd, args = sys.argv[1], sys.argv[2:]
    {"stats": stats, "traffic": traffic}[cmd](*args)
