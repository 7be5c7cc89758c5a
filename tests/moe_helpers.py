"""Shared helpers for the GPU parity tests: oracle views of device-resident weights, tolerances."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import synth

REL_L2 = 1e-4          # relative L2 error bound on a round's output
MAX_ABS_FRAC = 1e-3    # max abs error bound, as a fraction of max |reference|


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


class LazyExperts:
    """Index by expert id -> that expert's host copy (copied from the device on first use)."""

    def __init__(self, t: torch.Tensor, as_u32: bool):
        self.t, self.as_u32, self.cache = t, as_u32, {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            a = self.t[e].detach().cpu().numpy()
            self.cache[e] = a.view(np.uint32) if self.as_u32 else a
        return self.cache[e]


def oracle_view(layer: synth.LayerInputs) -> dict:
    """The oracle's view of a layer whose weights live on the GPU (inputs from the generator)."""
    return {
        "router_w": layer.router_w.detach().cpu().numpy(),
        "router_b": None if layer.router_b is None else layer.router_b.detach().cpu().numpy(),
        "gate_q": LazyExperts(layer.gate_q, False), "gate_sm": LazyExperts(layer.gate_sm, True),
        "up_q": LazyExperts(layer.up_q, False), "up_sm": LazyExperts(layer.up_sm, True),
        "down_q": LazyExperts(layer.down_q, False), "down_sm": LazyExperts(layer.down_sm, True),
        "format": layer.fmt,
    }


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=16)
    return _POOL


class DequantCache(dict):
    """Expert id -> the oracle's dequantised (W_g, W_u, W_d) for one layer view, shared by many
    rounds; missing experts are dequantised in parallel threads (the oracle's own routine)."""

    def __init__(self, view):
        super().__init__()
        self.view = view

    def ensure(self, experts):
        missing = sorted(set(int(e) for e in experts) - set(self))
        v = self.view
        arrays = {e: [v[f][e] for f in ("gate_q", "gate_sm", "up_q", "up_sm", "down_q", "down_sm")] for e in missing}
        futs = {e: _pool().submit(oracle.expert_matrices, *arrays[e], fmt=v.get("format") or "q4b32")
                for e in missing}
        for e, f in futs.items():
            self[e] = f.result()
        return self


def oracle_layer_cached(view, cache: DequantCache, X: np.ndarray, k: int, residual: bool):
    """oracle.moe_layer with its experts taken from (and added to) a shared cache."""
    need = set()
    for t in range(X.shape[0]):
        need.update(oracle.select_topk(oracle.router_logits(view["router_w"], view["router_b"], X[t]), k).tolist())
    cache.ensure(need)
    return oracle.moe_layer(view, X, k, residual=residual, cache=cache)


def errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mabs = np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300)
    return float(rel), float(mabs)


def assert_close(got, ref, what=""):
    rel, mabs = errors(got, ref)
    print(f"[close] {what}: rel-L2 {rel:.3e}, max-abs/max|y| {mabs:.3e}")
    assert rel <= REL_L2 and mabs <= MAX_ABS_FRAC, f"{what}: rel-L2 {rel:.3e}, max-abs/max|y| {mabs:.3e}"
    return rel, mabs


class GpuRound:
    """A handle plus reusable device buffers for one shape."""

    def __init__(self, layers, cfg: synth.ShapeConfig, max_rows: int, use_graph=True, k_max=None, **shape):
        from verify_router_gemv_amd import MoeRound
        self.cfg = cfg
        self.layers = layers
        self.k_max = k_max or cfg.k
        self.h = MoeRound(layers, cfg.H, cfg.I, cfg.E, self.k_max, max_rows=max_rows,
                          residual=cfg.residual, use_graph=use_graph, **shape)

    def run(self, X: torch.Tensor, k=None, layers=None, timed=False):
        k = k or self.cfg.k
        T = X.shape[0]
        out = torch.empty_like(X)
        ids = torch.full((len(self.layers), T, k), -1, dtype=torch.int32, device=X.device)
        rw = torch.zeros((len(self.layers), T, k), dtype=torch.float32, device=X.device)
        if timed:
            ms = self.h.run_timed(X, k, out, ids, rw, layers=layers)
        else:
            self.h.run(X, k, out, ids, rw, layers=layers)
            ms = None
        torch.cuda.synchronize()
        return out.cpu().numpy(), ids.cpu().numpy(), rw.cpu().numpy(), ms

    def close(self):
        self.h.close()


def check_layer_round(g: GpuRound, views, X: torch.Tensor, k: int, what: str, worklist=True, caches=None):
    """Run one round on the GPU and check it against the oracle; returns (rel, mabs, n_unique).
    caches: one DequantCache per layer (optional), so repeated rounds dequantise each expert once."""
    out, ids, rw, _ = g.run(X, k)
    Xh = X.cpu().numpy()
    if caches is None:
        ref, rids, rp, gaps = oracle.moe_round(views, Xh, k, residual=g.cfg.residual)
    else:
        x, rids, rp = Xh.astype(np.float64), [], []
        for view, cache in zip(views, caches):
            x, i, p, _ = oracle_layer_cached(view, cache, x, k, g.cfg.residual)
            rids.append(i)
            rp.append(p)
        ref, rids, rp = x, np.stack(rids), np.stack(rp)
    L = len(views)
    for l in range(L):
        assert np.array_equal(ids[l], rids[l]), f"{what}: layer {l} ids differ\nGPU {ids[l]}\nref {rids[l]}"
        np.testing.assert_allclose(rw[l], rp[l], rtol=2e-6, atol=1e-7, err_msg=f"{what}: routing weights")
    if g.cfg.residual:
        rel, mabs = assert_close(out - Xh, ref - Xh, what + " (MoE part)")
    else:
        rel, mabs = assert_close(out, ref, what)
    nu = g.h.last_unique()
    if worklist:
        for l in range(L):
            uniq, offs, pairs = g.h.worklist(l)
            eu, eo, ep = oracle.build_worklist(rids[l])
            assert uniq == eu.tolist(), f"{what}: uniq"
            assert offs == eo.tolist(), f"{what}: offs"
            assert pairs == [tuple(p) for p in ep.tolist()], f"{what}: pairs"
            assert nu[l] == len(set(rids[l].ravel().tolist()))
    return rel, mabs, nu
