"""Prefill rounds (more than 64 rows) through the C ABI vs the fp64 oracle (needs an MI355X).

The path: counting sort of the (row, rank) pairs into 64-pair work items, gate/up and down as fp16
matrix-core GEMMs (each activation row scaled by a power of two and split into two fp16 values),
combine in rank order. Ids and the worklist must match bit-exactly, routing
weights to fp32 rounding, outputs within relative L2 1e-4 and max-abs 1e-3 * max|y|. At 4096 rows
the outputs are checked on sampled rows (the oracle evaluates each row on its own, so a row's
expected output does not depend on the rest of the round).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from moe_helpers import GpuRound, assert_close, check_layer_round, oracle_view, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def prefill_layer():
    cfg = synth.config("prefill")
    layer = synth.make_layer(cfg, seed=0, layer=0, device=DEV)
    return cfg, layer, oracle_view(layer)


def test_prefill_ragged_shape_all_rows():
    """H=768, I=384, E=40, k=5: T just above the decode limit, ragged T, and T = max_rows."""
    cfg = synth.ShapeConfig("ragged", H=768, E=40, k=5, I=384, T=(65, 100, 257), zipf_s=0.7)
    layer = synth.make_layer(cfg, seed=3, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=257)
    for T in cfg.T:
        say(f"case prefill ragged T={T}")
        X = synth.make_activations(cfg, T, seed=11, round_idx=T, device=DEV)
        rel, mabs, nu = check_layer_round(g, [view], X, cfg.k, f"prefill ragged T={T}")
        _, offs, _ = g.h.worklist(0)
        say(f"  n_unique={nu[0]} max pairs per expert={int(np.diff(offs).max())} rel-L2={rel:.2e}")
    g.close()


@pytest.mark.parametrize("fmt", ["q4b32", "q4s256"])
def test_prefill_wide_inter_all_rows(fmt):
    """A wider expert than the other prefill shapes: I = 768 (6 steps of down's reduction, 12 gate/up
    row tiles), H=512, E=24, k=4, T = 70 and 133 (ragged tiles), both weight formats."""
    cfg = synth.ShapeConfig("wide_inter", H=512, E=24, k=4, I=768, T=(70, 133), zipf_s=0.7).replace(fmt=fmt)
    layer = synth.make_layer(cfg, seed=5, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=133)
    for T in cfg.T:
        say(f"case prefill I=768 {fmt} T={T}")
        X = synth.make_activations(cfg, T, seed=13, round_idx=T, device=DEV)
        rel, mabs, nu = check_layer_round(g, [view], X, cfg.k, f"prefill I=768 {fmt} T={T}")
        say(f"  n_unique={nu[0]} rel-L2={rel:.2e}")
    g.close()


@pytest.mark.parametrize("k", [1, 8])
def test_prefill_verify_shape_all_rows(prefill_layer, k):
    """The prefill workload's layer at T = 65 and 200, every row against the oracle; k = 1 makes
    routing weights exactly 1."""
    cfg, layer, view = prefill_layer
    g = GpuRound([layer], cfg, max_rows=256)
    for T in (65, 200):
        say(f"case prefill verify-shape T={T} k={k}")
        X = synth.make_activations(cfg, T, seed=12, round_idx=T, device=DEV)
        rel, mabs, nu = check_layer_round(g, [view], X, k, f"prefill T={T} k={k}")
        say(f"  n_unique={nu[0]} rel-L2={rel:.2e}")
    g.close()


def test_prefill_row_scales_heavy_tails_and_zero_rows(prefill_layer):
    """The activation split at the edges of its row scaling: rows scaled by 2^u, u uniform in
    [-40, 40] (the per-row power-of-two step), heavy-tailed rows (four elements 10^4 times the
    rest), and all-zero rows. Ids and routing weights as always; each row's output is checked on
    its own scale (relative L2 and max-abs against that row of the oracle), and zero rows give
    exact zeros."""
    cfg, layer, view = prefill_layer
    T = 160
    g = GpuRound([layer], cfg, max_rows=T)
    say(f"case prefill row scales T={T}")
    rng = np.random.default_rng(31)
    X = synth.make_activations(cfg, T, seed=31, round_idx=T, device="cpu").numpy().astype(np.float32)
    X *= (2.0 ** rng.uniform(-40.0, 40.0, size=T)).astype(np.float32)[:, None]
    for t in range(10, 20):
        X[t, rng.choice(cfg.H, size=4, replace=False)] *= np.float32(1e4)
    zero_rows = [0, 77, T - 1]
    X[zero_rows] = 0.0
    out, ids, rw, _ = g.run(torch.from_numpy(X).to(DEV))
    with np.errstate(over="ignore"):  # silu(a) = a / (1 + e^-a) at a << 0: e^-a overflows, silu -> -0
        ref, rids, rp, _ = oracle.moe_round([view], X, cfg.k, residual=False)
    assert np.array_equal(ids[0], rids[0]), "ids differ"
    np.testing.assert_allclose(rw[0], rp[0], rtol=2e-6, atol=1e-7, err_msg="routing weights")
    worst = 0.0
    for t in range(T):
        if t in zero_rows:
            assert np.all(out[t] == 0.0), f"zero row {t} gave nonzero output"
            continue
        rel, _ = assert_close(out[t], ref[t], f"prefill scaled row {t}")
        worst = max(worst, rel)
    say(f"  worst row rel-L2={worst:.2e}")
    g.close()


def test_prefill_gateup_stage(prefill_layer):
    """The prefill gate/up stage alone: silu(W_g x) * (W_u x) per pair slot (read back through
    moe_round_swiglu_rows) against the oracle, at T = 200 (every pair slot of the round)."""
    cfg, layer, view = prefill_layer
    T = 200
    g = GpuRound([layer], cfg, max_rows=T)
    say(f"case prefill gate/up stage T={T}")
    X = synth.make_activations(cfg, T, seed=21, round_idx=T, device=DEV)
    out, ids, _, _ = g.run(X)
    h = g.h.swiglu_rows(T, cfg.k)
    uniq, offs, pairs = g.h.worklist(0)
    Xh = X.cpu().numpy().astype(np.float64)
    ref = np.zeros_like(h, dtype=np.float64)
    mats = {}
    for p, (t, j) in enumerate(pairs):
        e = int(ids[0, t, j])
        if e not in mats:
            mats[e] = oracle.expert_matrices(view["gate_q"][e], view["gate_sm"][e], view["up_q"][e],
                                             view["up_sm"][e], view["down_q"][e], view["down_sm"][e])
        Wg, Wu, _ = mats[e]
        ref[p] = oracle.silu(Wg @ Xh[t]) * (Wu @ Xh[t])
    rel, _ = assert_close(h, ref, f"prefill gate/up T={T}")
    say(f"  rel-L2={rel:.2e}")
    g.close()


def test_prefill_hot_experts_split_into_items():
    """Zipf-biased routing (E=128, k=8, I=768) at T=600: popular experts get several hundred rows,
    so their pairs span several 64-pair work items."""
    cfg = synth.config("decode").replace(T=(600,))
    layer = synth.make_layer(cfg, seed=0, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=600)
    say("case prefill zipf T=600")
    X = synth.make_activations(cfg, 600, seed=13, round_idx=600, device=DEV)
    rel, mabs, nu = check_layer_round(g, [view], X, cfg.k, "prefill zipf T=600")
    _, offs, _ = g.h.worklist(0)
    most = int(np.diff(offs).max())
    say(f"  n_unique={nu[0]} max pairs per expert={most} rel-L2={rel:.2e}")
    assert most > 2 * 64
    g.close()


def test_prefill_4096_rows_sampled(prefill_layer):
    """T = 4096: ids, routing weights and the worklist of every row bit-exact / to fp32 rounding;
    outputs of 48 sampled rows (first, last, and spread) within tolerance."""
    cfg, layer, view = prefill_layer
    T, k = 4096, cfg.k
    g = GpuRound([layer], cfg, max_rows=T)
    say(f"case prefill T={T}")
    X = synth.make_activations(cfg, T, seed=14, round_idx=T, device=DEV)
    out, ids, rw, _ = g.run(X, k)
    Xh = X.cpu().numpy()
    rids = np.zeros((T, k), dtype=np.int64)
    rp = np.zeros((T, k))
    for t in range(T):
        z = oracle.router_logits(view["router_w"], view["router_b"], Xh[t])
        rids[t] = oracle.select_topk(z, k)
        rp[t] = oracle.routing_weights(z, rids[t])
    assert np.array_equal(ids[0], rids)
    np.testing.assert_allclose(rw[0], rp, rtol=2e-6, atol=1e-7)
    uniq, offs, pairs = g.h.worklist(0)
    eu, eo, ep = oracle.build_worklist(rids)
    assert uniq == eu.tolist() and offs == eo.tolist()
    assert np.array_equal(np.asarray(pairs), ep)
    rng = np.random.default_rng(0)
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 46, replace=False)]))
    ref, _, _, _ = oracle.moe_layer(view, Xh[sample], k)
    rel, mabs = assert_close(out[sample], ref, f"prefill T={T} sampled rows")
    say(f"  n_unique={len(uniq)} max pairs per expert={int(np.diff(offs).max())} rel-L2={rel:.2e}")
    g.close()


def test_prefill_superblock_format():
    """Prefill rounds on the 4.5-bit super-block layout (Q4S256): the prefill layer at T = 65 and
    300, and a 3-layer residual stack (H=1024, I=256, E=64, k=4) at T = 100, every row against the
    oracle."""
    cfg = synth.config("prefill").replace(fmt="q4s256")
    layer = synth.make_layer(cfg, seed=2, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=300)
    for T in (65, 300):
        say(f"case prefill q4s256 T={T}")
        X = synth.make_activations(cfg, T, seed=19, round_idx=T, device=DEV)
        rel, mabs, nu = check_layer_round(g, [view], X, cfg.k, f"prefill q4s256 T={T}")
        say(f"  n_unique={nu[0]} rel-L2={rel:.2e}")
    g.close()
    scfg = synth.ShapeConfig("stack", H=1024, E=64, k=4, I=256, L=3, T=(100,), zipf_s=1.0, residual=True,
                             fmt="q4s256")
    layers = [synth.make_layer(scfg, seed=0, layer=l, device=DEV) for l in range(scfg.L)]
    g = GpuRound(layers, scfg, max_rows=100)
    say("case prefill q4s256 stack L=3 T=100")
    X = synth.make_activations(scfg, 100, seed=20, round_idx=100, device=DEV)
    rel, mabs, nu = check_layer_round(g, [oracle_view(l) for l in layers], X, scfg.k, "prefill q4s256 stack")
    say(f"  n_unique per layer={nu} rel-L2={rel:.2e}")
    g.close()


def test_prefill_largest_round():
    """The largest prefill round: T = MOE_ROUND_MAX_PREFILL_ROWS = 16384, k = 16, E = 512 (262144
    pairs: the counting sort's packed counters at their widest). Ids, routing weights and the
    worklist of every row bit-exact / to fp32 rounding; outputs of 12 sampled rows."""
    from verify_router_gemv_amd import binding
    T = binding.MAX_PREFILL_ROWS
    cfg = synth.ShapeConfig("prefill-max", H=2048, E=512, k=16, I=512, T=(T,), zipf_s=1.0)
    layer = synth.make_layer(cfg, seed=1, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=T)
    say(f"case prefill largest T={T} k={cfg.k} E={cfg.E}")
    X = synth.make_activations(cfg, T, seed=18, round_idx=T, device=DEV)
    out, ids, rw, _ = g.run(X, cfg.k)
    Xh = X.cpu().numpy()
    rids = np.zeros((T, cfg.k), dtype=np.int64)
    rp = np.zeros((T, cfg.k))
    for t in range(T):
        z = oracle.router_logits(view["router_w"], view["router_b"], Xh[t])
        rids[t] = oracle.select_topk(z, cfg.k)
        rp[t] = oracle.routing_weights(z, rids[t])
    assert np.array_equal(ids[0], rids)
    np.testing.assert_allclose(rw[0], rp, rtol=2e-6, atol=1e-7)
    uniq, offs, pairs = g.h.worklist(0)
    eu, eo, ep = oracle.build_worklist(rids)
    assert uniq == eu.tolist() and offs == eo.tolist()
    assert np.array_equal(np.asarray(pairs), ep)
    sample = np.array([0, 1, 777, 4095, 4096, 8191, 9000, 12345, 15000, 16000, T - 2, T - 1])
    ref, _, _, _ = oracle.moe_layer(view, Xh[sample], cfg.k)
    rel, mabs = assert_close(out[sample], ref, "prefill largest sampled rows")
    say(f"  n_unique={len(uniq)} max pairs per expert={int(np.diff(offs).max())} rel-L2={rel:.2e}")
    g.close()
    del layer, view
    torch.cuda.empty_cache()


def test_prefill_rows_do_not_depend_on_the_round(prefill_layer):
    """Every pair's products depend only on its own row and expert, and the combine adds the ranks
    in order: rows 0..99 of a 300-row round equal a 100-row round of those rows bitwise, and so do
    the reversed rows."""
    cfg, layer, _ = prefill_layer
    g = GpuRound([layer], cfg, max_rows=300)
    say("case prefill row invariance")
    X = synth.make_activations(cfg, 300, seed=15, round_idx=300, device=DEV)
    full = g.run(X)[0]
    part = g.run(X[:100].contiguous())[0]
    assert np.array_equal(full[:100], part)
    rev = g.run(X.flip(0).contiguous())[0]
    assert np.array_equal(rev[::-1], full)
    g.close()


def test_prefill_residual_stack():
    """Three layers with the residual between them (Zipf routing, E=64, k=4) at T=130, against the
    oracle's free-running stack; ids of every layer bit-exact."""
    cfg = synth.ShapeConfig("stack", H=1024, E=64, k=4, I=256, L=3, T=(130,), zipf_s=1.0, residual=True)
    layers = [synth.make_layer(cfg, seed=0, layer=l, device=DEV) for l in range(cfg.L)]
    views = [oracle_view(l) for l in layers]
    g = GpuRound(layers, cfg, max_rows=130)
    say("case prefill residual stack L=3 T=130")
    X = synth.make_activations(cfg, 130, seed=16, round_idx=130, device=DEV)
    rel, mabs, nu = check_layer_round(g, views, X, cfg.k, "prefill stack")
    say(f"  n_unique per layer={nu} rel-L2={rel:.2e}")
    g.close()


def test_prefill_profiling(prefill_layer):
    """Kernel timing of prefill rounds: the nine launches of a layer fold into the five kinds
    (input split + logits, top-k + sort, gate/up, SwiGLU split + down, combine), every kind timed, and
    the run count matches; the outputs equal an unprofiled run's bitwise."""
    cfg, layer, _ = prefill_layer
    g = GpuRound([layer], cfg, max_rows=300)
    say("case prefill profiling T=300")
    X = synth.make_activations(cfg, 300, seed=22, round_idx=300, device=DEV)
    plain = g.run(X)[0]
    g.h.profile(True)
    g.h.profile_read()
    outs = [g.run(X)[0] for _ in range(3)]
    ms, runs = g.h.profile_read()
    g.h.profile(False)
    assert runs == 3
    assert all(v > 0 for v in ms[0]), ms
    for o in outs:
        assert np.array_equal(o, plain)
    say(f"  ms per kind over 3 runs: {[round(v, 3) for v in ms[0]]}")
    g.close()


def test_prefill_then_verify_rounds_on_one_handle(prefill_layer):
    """One handle serves a prefill round, then verify rounds (graph replay), then prefill again."""
    cfg, layer, view = prefill_layer
    g = GpuRound([layer], cfg, max_rows=128)
    for T in (128, 3, 8, 70):
        say(f"case mixed handle T={T}")
        X = synth.make_activations(cfg, T, seed=17, round_idx=T, device=DEV)
        check_layer_round(g, [view], X, cfg.k, f"mixed T={T}")
    g.close()
