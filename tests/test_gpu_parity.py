"""HIP path vs the fp64 oracle, through the C ABI, on every workload shape (needs an MI355X).

Expert ids and the worklist must match bit-exactly; routing weights to fp32 rounding; the round's
output within relative L2 1e-4 and max-abs 1e-3 * max|y|.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from moe_helpers import DequantCache, GpuRound, assert_close, check_layer_round, errors, oracle_view, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.config("tiny")
    layer = synth.make_layer(cfg, seed=0, layer=0, device=DEV)
    return cfg, layer, oracle_view(layer)


def test_tiny_many_seeded_rounds(tiny):
    """The tiny layer on 1000 seeded rounds, every one checked."""
    cfg, layer, view = tiny
    say("case tiny: 1000 seeded rounds, T=1, k=2")
    g = GpuRound([layer], cfg, max_rows=1)
    cache = DequantCache(view)
    worst = 0.0
    for r in range(1000):
        X = synth.make_activations(cfg, 1, seed=0, round_idx=r, device=DEV)
        rel, _, _ = check_layer_round(g, [view], X, cfg.k, f"tiny round {r}", worklist=(r % 50 == 0),
                                      caches=[cache])
        worst = max(worst, rel)
    say(f"  1000 rounds checked, worst rel-L2 {worst:.2e}")
    g.close()


@pytest.mark.parametrize("k", [1, 3, 8])
def test_tiny_k_edges(tiny, k):
    cfg, layer, view = tiny
    say(f"case tiny k={k}")
    g = GpuRound([layer], cfg, max_rows=4, k_max=8)
    for T in (1, 4):
        X = synth.make_activations(cfg, T, seed=1, round_idx=k, device=DEV)
        check_layer_round(g, [view], X, k, f"tiny k={k} T={T}")
        if k == 1:
            _, _, rw, _ = g.run(X, k)
            assert np.all(rw == 1.0)
    g.close()


@pytest.fixture(scope="module")
def verify():
    cfg = synth.config("verify")
    layer = synth.make_layer(cfg, seed=0, layer=0, device=DEV)
    view = oracle_view(layer)
    return cfg, layer, view


@pytest.fixture(scope="module")
def verify_cache(verify):
    return DequantCache(verify[2])


@pytest.mark.parametrize("use_graph,rounds", [(False, 100), (True, 10)])
def test_verify_sweep(verify, verify_cache, use_graph, rounds):
    """The verify sweep T = 1, 2, 3, 4, 5, 8: 100 seeded rounds per width eagerly and 10 as graph
    replays, every one checked (ids and worklist bit-exact, weights, output)."""
    cfg, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=8, use_graph=use_graph)
    for T in cfg.T:
        worst, nus = 0.0, []
        for r in range(rounds):
            X = synth.make_activations(cfg, T, seed=0, round_idx=r, device=DEV)
            rel, mabs, nu = check_layer_round(g, [view], X, cfg.k, f"verify T={T} r={r}", caches=[verify_cache])
            worst = max(worst, rel)
            nus.append(nu[0])
        say(f"case verify T={T} graph={use_graph}: {rounds} rounds checked, mean n_unique {np.mean(nus):.2f},"
            f" worst rel-L2 {worst:.2e}")
    g.close()


def test_decode():
    """Batch-1 decode (E=128 with the Zipf router bias, I=768): 1000 fresh seeded rounds, all checked."""
    cfg = synth.config("decode")
    layer = synth.make_layer(cfg, seed=0, layer=0, device=DEV)
    view = oracle_view(layer)
    cache = DequantCache(view)
    g = GpuRound([layer], cfg, max_rows=1)
    worst, nus = 0.0, []
    for r in range(1000):
        X = synth.make_activations(cfg, 1, seed=0, round_idx=r, device=DEV)
        rel, mabs, nu = check_layer_round(g, [view], X, cfg.k, f"decode r={r}", worklist=(r % 20 == 0),
                                          caches=[cache])
        worst = max(worst, rel)
        nus.append(nu[0])
    say(f"case decode: 1000 rounds checked, distinct experts used {len(cache)}, worst rel-L2 {worst:.2e}")
    g.close()


def test_wide(verify, verify_cache):
    """Copy-heavy wide verify T = 16, 32, 64 (independent rows): 20 seeded rounds per width."""
    cfg = synth.config("wide")
    # the wide workload has the verify shape (H, E, k, I) with independent rows
    _, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=64)
    for T in cfg.T:
        worst, nus = 0.0, []
        for r in range(20):
            X = synth.make_activations(cfg, T, seed=0, round_idx=1000 * T + r, device=DEV)
            rel, mabs, nu = check_layer_round(g, [view], X, cfg.k, f"wide T={T} r={r}", caches=[verify_cache])
            worst = max(worst, rel)
            nus.append(nu[0])
        say(f"case wide T={T}: 20 rounds checked, mean n_unique {np.mean(nus):.1f}, worst rel-L2 {worst:.2e}")
    g.close()


@pytest.mark.parametrize("name,T", [("tiny", 1), ("verify", 1), ("verify", 3), ("verify", 8)])
def test_gateup_stage(name, T, tiny, verify):
    """The gate/up stage alone: silu(W_g x) * (W_u x) per (row, rank) pair against the oracle."""
    cfg, layer, view = tiny if name == "tiny" else verify
    say(f"case gate/up stage {name} T={T}")
    g = GpuRound([layer], cfg, max_rows=max(T, 1))
    X = synth.make_activations(cfg, T, seed=2, round_idx=T, device=DEV)
    out, ids, _, _ = g.run(X)
    h = g.h.swiglu_rows(T, cfg.k)
    uniq, offs, pairs = g.h.worklist(0)
    Xh = X.cpu().numpy().astype(np.float64)
    ref = np.zeros_like(h, dtype=np.float64)
    for p, (t, j) in enumerate(pairs):
        e = int(ids[0, t, j])
        Wg, Wu, _ = oracle.expert_matrices(view["gate_q"][e], view["gate_sm"][e], view["up_q"][e], view["up_sm"][e],
                                           view["down_q"][e], view["down_sm"][e])
        ref[p] = oracle.silu(Wg @ Xh[t]) * (Wu @ Xh[t])
    assert_close(h, ref, f"gate/up {name} T={T}")
    g.close()


@pytest.mark.parametrize("T,mfma_min_rows", [(3, 0), (16, -1), (16, 1), (40, 1), (64, 2)])
def test_down_stage(verify, T, mfma_min_rows):
    """The down stage alone, on the GPU's own SwiGLU rows: each output row equals sum_j p_j W_d h_(t,j)
    with h read back from the gate/up stage (so the check does not depend on gate/up's rounding).
    Covers the down GEMV and, in wide rounds with the matrix-core tiles on, the down tile (items of at
    least mfma_min_rows rows)."""
    cfg, layer, view = verify
    say(f"case down stage T={T} mfma_min_rows={mfma_min_rows}")
    wide = synth.config("wide")
    g = GpuRound([layer], cfg, max_rows=64, mfma_min_rows=mfma_min_rows)
    X = synth.make_activations(wide if T >= 16 else cfg, T, seed=12, round_idx=T, device=DEV)
    out, ids, rw, _ = g.run(X)
    h = g.h.swiglu_rows(T, cfg.k).astype(np.float64)
    _, _, pairs = g.h.worklist(0)
    cache = {}
    ref = np.zeros((T, cfg.H), dtype=np.float64)
    for p, (t, j) in enumerate(pairs):
        e = int(ids[0, t, j])
        if e not in cache:
            cache[e] = oracle.dequantize(view["down_q"][e], view["down_sm"][e])
        ref[t] += float(rw[0, t, j]) * (cache[e] @ h[p])
    assert_close(out, ref, f"down stage T={T} mfma {mfma_min_rows}")
    g.close()


def test_rows_are_independent(verify):
    """A row's output does not depend on the other rows of the round (within fp32 rounding)."""
    cfg, layer, _ = verify
    g = GpuRound([layer], cfg, max_rows=8)
    X = synth.make_activations(cfg, 5, seed=3, round_idx=0, device=DEV)
    say("case row independence T=5")
    out, ids, _, _ = g.run(X)
    for t in range(5):
        o1, i1, _, _ = g.run(X[t:t + 1].contiguous())
        assert np.array_equal(i1[0, 0], ids[0, t])
        rel, mabs = errors(o1[0], out[t])
        assert rel < 1e-6, rel
    g.close()


def test_weight_and_pointer_ingress(verify):
    """New weight pointers and new hidden/out buffers are picked up without a recapture."""
    cfg, layer, view = verify
    other = synth.make_layer(cfg, seed=7, layer=0, device=DEV)
    oview = oracle_view(other)
    g = GpuRound([layer], cfg, max_rows=8)
    X = synth.make_activations(cfg, 3, seed=0, round_idx=11, device=DEV)
    say("case ingress: weights A")
    check_layer_round(g, [view], X, cfg.k, "weights A")
    say("case ingress: weights B via run(layers=...)")
    out, ids, _, _ = g.run(X, layers=[other])
    ref, rids, _, _ = oracle.moe_round([oview], X.cpu().numpy(), cfg.k, residual=False)
    assert np.array_equal(ids[0], rids[0])
    assert_close(out, ref, "weights B")
    say("case ingress: weights B kept when layers=None, new buffers")
    X2 = X.clone()
    out2, ids2, _, _ = g.run(X2)
    assert np.array_equal(ids2, ids)
    assert_close(out2, ref, "weights B again")
    g.close()


def test_ragged_shape_paths():
    """Other lane splits (H=768: 8 lanes x 3 blocks; I=384: 4 lanes x 3 blocks), ragged T, bias."""
    cfg = synth.ShapeConfig("ragged", H=768, E=40, k=5, I=384, T=(1, 7, 13), zipf_s=0.7)
    layer = synth.make_layer(cfg, seed=5, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=16)
    for T in cfg.T:
        say(f"case ragged H=768 I=384 E=40 k=5 T={T}")
        X = synth.make_activations(cfg, T, seed=5, round_idx=T, device=DEV)
        check_layer_round(g, [view], X, cfg.k, f"ragged T={T}")
    g.close()


def test_folded_selection_widths_at_512_experts():
    """E = 512, top-10 (eight keys per lane): the selection folded into gate/up on its many-row
    forms (one-row items up to 10 rows, two-row items above, the block-wide union past 64 pairs,
    up to the fold's last width) and the selection kernel just past it, each against the oracle."""
    cfg = synth.config("deep").replace(L=1)
    layer = synth.make_layer(cfg, seed=12, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=16)
    for T in (5, 9, 12, 15, 16):
        say(f"case E=512 k=10 T={T}")
        X = synth.make_activations(cfg, T, seed=12, round_idx=T, device=DEV)
        check_layer_round(g, [view], X, cfg.k, f"E=512 T={T}")
    g.close()


@pytest.mark.parametrize("use_graph", [False, True])
def test_stack_with_prefetch(use_graph):
    """A 4-layer residual stack with the early touches on (down blocks touch the next layer's router
    rows): the same ids and outputs as the oracle, eager and as a graph."""
    cfg = synth.config("deep").replace(L=4, E=128)
    layers = [synth.make_layer(cfg, seed=9, layer=l, device=DEV) for l in range(cfg.L)]
    views = [oracle_view(l) for l in layers]
    g = GpuRound(layers, cfg, max_rows=8, use_graph=use_graph, prefetch=1)
    for T in (1, 3, 8):
        say(f"case stack prefetch graph={use_graph} T={T}")
        X = synth.make_activations(cfg, T, seed=19, round_idx=T, device=DEV)
        check_layer_round(g, views, X, cfg.k, f"stack prefetch T={T}")
    g.close()


def test_many_rows_share_experts(verify):
    """40 correlated rows: the hot experts get far more than 16 rows (several matrix-core passes)."""
    cfg, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=64)
    for T in (16, 40, 64):
        say(f"case shared experts T={T}")
        X = synth.make_activations(cfg, T, seed=4, round_idx=T, device=DEV)  # verify rows: base + 0.5 noise
        rel, mabs, nu = check_layer_round(g, [view], X, cfg.k, f"shared T={T}")
        _, offs, _ = g.h.worklist(0)
        say(f"  n_unique={nu[0]} max rows per expert={int(np.diff(offs).max())} rel-L2={rel:.2e}")
    g.close()


@pytest.mark.parametrize("k", [7, 8])
def test_tied_logits_go_to_the_lower_id(verify, k):
    """Router rows duplicated in pairs, so experts 2m and 2m+1 get bitwise equal logits. Every
    selection path (the one-row worklist, the selection folded into gate/up, the selection kernel,
    ragged T, a prefill round) orders a tied pair lower id first, and a pair cut at rank k keeps
    the lower id: the ids match the oracle's stable order, and the rule is also checked on the ids
    directly."""
    cfg, layer, _ = verify
    rw = layer.router_w.clone()
    rw[1::2] = rw[0::2]
    rb = None
    if layer.router_b is not None:
        rb = layer.router_b.clone()
        rb[1::2] = rb[0::2]
    tied = dataclasses.replace(layer, router_w=rw, router_b=rb)
    view = oracle_view(tied)
    g = GpuRound([tied], cfg, max_rows=130)
    for T in (1, 3, 8, 24, 37, 130):
        say(f"case tied logits k={k} T={T}")
        X = synth.make_activations(cfg, T, seed=8, round_idx=T, device=DEV)
        z = oracle.router_logits(view["router_w"], view["router_b"], X[0].cpu().numpy())
        assert np.array_equal(z[0::2], z[1::2])  # the oracle sees the ties too
        check_layer_round(g, [view], X, k, f"tied k={k} T={T}")
        _, ids, _, _ = g.run(X, k)
        for t in range(T):
            row = ids[0, t].tolist()
            for j, e in enumerate(row):
                if e % 2:
                    assert j > 0 and row[j - 1] == e - 1, f"row {t}: {row}"
                elif e + 1 not in row:
                    assert j == k - 1, f"row {t}: {row}"
    g.close()


@pytest.mark.parametrize("shape", [
    dict(fused_max_rows=-1, rows_per_item=1),   # separate selection kernel, one row per item
    dict(fused_max_rows=15, rows_per_item=8),   # selection in gate/up up to 15 rows, big items
    dict(rows_per_item=2),                      # two-row items at every verify width
    dict(prefetch=1),                           # gate/up touches the down rows of its index
])
def test_launch_shape_choices(verify, shape):
    """Other launch shapes give the same ids and worklists and outputs within tolerance."""
    cfg, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=16, **shape)
    for T in (1, 3, 8, 12, 15):
        say(f"case launch shape {shape} T={T}")
        X = synth.make_activations(cfg, T, seed=6, round_idx=T, device=DEV)
        check_layer_round(g, [view], X, cfg.k, f"shape {shape} T={T}")
    g.close()


@pytest.mark.parametrize("mfma_min_rows", [1, -1])
def test_wide_tile_choice(verify, mfma_min_rows):
    """Wide rounds with every work item on the matrix-core tile (1) or none (-1)."""
    cfg = synth.config("wide")
    _, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=64, mfma_min_rows=mfma_min_rows)
    for T in (16, 64):
        say(f"case wide T={T} mfma_min_rows={mfma_min_rows}")
        X = synth.make_activations(cfg, T, seed=7, round_idx=T, device=DEV)
        check_layer_round(g, [view], X, cfg.k, f"wide T={T} mfma {mfma_min_rows}")
    g.close()


def test_empty_round_is_a_no_op(verify):
    """T = 0: MOE_OK, nothing written, introspection reports no round; the next round is normal."""
    import ctypes
    from verify_router_gemv_amd.binding import MoeRoundError
    cfg, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=8)
    say("case empty round T=0")
    X0 = torch.empty((0, cfg.H), device=DEV)
    out0 = torch.empty((0, cfg.H), device=DEV)
    g.h.run(X0, cfg.k, out0)
    torch.cuda.synchronize()
    st = g.h.lib.moe_round_run(g.h.h, None, 0, cfg.k, None, None, None, None)
    assert st == 0
    with pytest.raises(MoeRoundError):
        g.h.last_unique()
    X = synth.make_activations(cfg, 3, seed=30, round_idx=0, device=DEV)
    check_layer_round(g, [view], X, cfg.k, "after an empty round")
    g.close()


def test_largest_supported_shape():
    """H = 8192, I = 2048, E = 512, k = 16, T = 64 (16 GB of expert weights): ids and the worklist of
    every row against the oracle's router, and the full output of sampled rows (rows are evaluated
    independently, so the oracle computes those rows alone)."""
    cfg = synth.ShapeConfig("max", H=8192, E=512, k=16, I=2048, T=(64,), zipf_s=1.0)
    say("case largest shape: generating 16 GB of weights")
    layer = synth.make_layer(cfg, seed=3, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=64, use_graph=False)
    X = synth.make_activations(cfg, 64, seed=31, round_idx=0, device=DEV)
    say("case largest shape: GPU round")
    out, ids, rw, _ = g.run(X)
    Xh = X.cpu().numpy()
    rids = np.stack([oracle.select_topk(oracle.router_logits(view["router_w"], view["router_b"], Xh[t]), cfg.k)
                     for t in range(64)])
    assert np.array_equal(ids[0], rids)
    uniq, offs, pairs = g.h.worklist(0)
    eu, eo, ep = oracle.build_worklist(rids)
    assert uniq == eu.tolist() and offs == eo.tolist() and pairs == [tuple(p) for p in ep.tolist()]
    for t in (0, 37, 63):
        say(f"case largest shape: oracle row {t}")
        ref, _, rp, _ = oracle.moe_layer(view, Xh[t:t + 1], cfg.k)
        np.testing.assert_allclose(rw[0, t], rp[0], rtol=2e-6, atol=1e-7)
        assert_close(out[t:t + 1], ref, f"largest shape row {t}")
    g.close()
    del layer, view
    torch.cuda.empty_cache()
