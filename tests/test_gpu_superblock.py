"""Parity of the 4.5-bit super-block weight layout (Q4S256) on the GPU (needs an MI355X).

The oracle dequantises the same bytes by its own reading of the layout (pinned by hand-worked
super-blocks and by bitwise agreement with the per-32 layout); these tests run every kernel form
the round picks over such weights: the folded selection (T <= 4), the selection kernel (T >= 5),
the staged gate/up of wide rounds, other lane splits, the fixed-order combine and a layer stack."""
import numpy as np
import pytest
import torch

import oracle
import synth
from moe_helpers import GpuRound, check_layer_round, oracle_view, say, assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def verify_s():
    cfg = synth.config("verify").replace(fmt="q4s256")
    layer = synth.make_layer(cfg, seed=0, layer=0, device=DEV)
    return cfg, layer, oracle_view(layer)


@pytest.mark.parametrize("use_graph", [False, True])
def test_superblock_verify_sweep(verify_s, use_graph):
    cfg, layer, view = verify_s
    g = GpuRound([layer], cfg, max_rows=8, use_graph=use_graph)
    for T in (1, 2, 3, 4, 5, 8):
        say(f"case q4s256 verify T={T} graph={use_graph}")
        X = synth.make_activations(cfg, T, seed=21, round_idx=T, device=DEV)
        check_layer_round(g, [view], X, cfg.k, f"q4s256 T={T}")
    g.close()


def test_superblock_decode():
    cfg = synth.config("decode").replace(fmt="q4s256")     # I = 768: three super-blocks per down row
    layer = synth.make_layer(cfg, seed=0, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=1)
    for r in range(4):
        say(f"case q4s256 decode round {r}")
        X = synth.make_activations(cfg, 1, seed=22, round_idx=r, device=DEV)
        check_layer_round(g, [view], X, cfg.k, f"q4s256 decode r={r}")
    g.close()


def test_superblock_wide(verify_s):
    cfg, layer, view = verify_s
    wcfg = synth.config("wide").replace(fmt="q4s256")
    g = GpuRound([layer], wcfg, max_rows=64)
    for T in (16, 40):
        say(f"case q4s256 wide T={T}")
        X = synth.make_activations(wcfg, T, seed=23, round_idx=T, device=DEV)
        check_layer_round(g, [view], X, cfg.k, f"q4s256 wide T={T}")
    g.close()


def test_superblock_exact_row_invariance(verify_s):
    cfg, layer, view = verify_s
    g = GpuRound([layer], cfg, max_rows=16, exact=True)
    T = 13
    say(f"case q4s256 exact T={T}")
    X = synth.make_activations(cfg, T, seed=24, round_idx=T, device=DEV)
    check_layer_round(g, [view], X, cfg.k, f"q4s256 exact T={T}")
    out = g.run(X)[0]
    for t in (0, 5, 12):
        alone = g.run(X[t:t + 1].contiguous())[0]
        assert np.array_equal(alone[0], out[t]), f"row {t}"
    g.close()


def test_superblock_other_lane_splits():
    """H = 768 (8 lanes x 3 blocks per gate/up row), I = 256 (8 lanes x 1 block per down row)."""
    cfg = synth.ShapeConfig("ragged_s", H=768, E=40, k=5, I=256, T=(1, 7, 13), zipf_s=0.7, fmt="q4s256")
    layer = synth.make_layer(cfg, seed=6, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=16)
    for T in cfg.T:
        say(f"case q4s256 H=768 I=256 E=40 k=5 T={T}")
        X = synth.make_activations(cfg, T, seed=6, round_idx=T, device=DEV)
        check_layer_round(g, [view], X, cfg.k, f"q4s256 ragged T={T}")
    g.close()


def test_superblock_stack():
    """Four layers of the 512-expert stack in the 4.5-bit layout, residual, T = 3."""
    cfg = synth.config("deep").replace(L=4, fmt="q4s256")
    layers = [synth.make_layer(cfg, seed=0, layer=l, device=DEV) for l in range(cfg.L)]
    views = [oracle_view(l) for l in layers]
    g = GpuRound(layers, cfg, max_rows=3)
    checked = 0
    for r in range(3):
        X = synth.make_activations(cfg, 3, seed=25, round_idx=r, device=DEV)
        say(f"case q4s256 stack round {r}")
        ref, rids, _, gaps = oracle.moe_round(views, X.cpu().numpy(), cfg.k, residual=True)
        if gaps.min() < 1e-5:
            say(f"  round {r}: oracle selection gap {gaps.min():.2e} < 1e-5, ill-conditioned; skipped")
            continue
        out, ids, _, _ = g.run(X)
        for l in range(cfg.L):
            assert np.array_equal(ids[l], rids[l]), f"layer {l}"
        Xh = X.cpu().numpy()
        assert_close(out - Xh, ref - Xh, f"q4s256 stack round {r}")
        checked += 1
    assert checked >= 1
    g.close()
