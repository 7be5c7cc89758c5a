"""One-hot activations through the gate/up stage on the GPU (needs an MI355X).

With input row t equal to the unit vector e_c, W x is column c of W, so each pair's SwiGLU row is
silu(W_g[:, c]) * W_u[:, c] of its expert: a direct pin of the weight layout the kernels read
(nibble order inside a byte, 32-weight block mapping, output-major rows, the scale and minimum of
the right block) against the oracle's dequantised columns. Every gate/up form is covered: one row
with the selection folded in, row pairs (folded and separate selection), staged wide rounds, and the
int8 matrix-core tile. The comparison is to 1e-5 of the row's largest value (the kernels round the
24-bit activation digits' products to fp32 and use a fast exponential); a layout slip moves whole
columns and misses by orders of magnitude, which the test also checks for the neighbouring column.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from moe_helpers import GpuRound, oracle_view, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
# both nibbles of a byte, block edges (31 | 32), the row ends and a spread of others
COLS = [0, 1, 2, 3, 14, 15, 16, 17, 30, 31, 32, 33, 62, 63, 64, 65, 1022, 1023, 1024, 1025, 2046, 2047,
        5, 100, 257, 511, 777, 1500, 1919, 2001, 40, 41]


@pytest.fixture(scope="module")
def verify():
    cfg = synth.config("verify")
    layer = synth.make_layer(cfg, seed=0, layer=0, device=DEV)
    return cfg, layer, oracle_view(layer)


def onehot(H, cols):
    X = torch.zeros((len(cols), H), dtype=torch.float32, device=DEV)
    for t, c in enumerate(cols):
        X[t, c] = 1.0
    return X


def check_onehot(g, view, cols, k, what):
    cfg = g.cfg
    X = onehot(cfg.H, cols)
    _, ids, _, _ = g.run(X, k)
    h = g.h.swiglu_rows(len(cols), k)
    _, _, pairs = g.h.worklist(0)
    worst, worst_other = 0.0, np.inf
    cache = {}
    for p, (t, j) in enumerate(pairs):
        e = int(ids[0, t, j])
        if e not in cache:
            cache[e] = oracle.expert_matrices(view["gate_q"][e], view["gate_sm"][e], view["up_q"][e],
                                              view["up_sm"][e], view["down_q"][e], view["down_sm"][e])
        Wg, Wu, _ = cache[e]
        c = cols[t]
        ref = oracle.silu(Wg[:, c]) * Wu[:, c]
        scale = np.max(np.abs(ref))
        err = np.max(np.abs(h[p] - ref)) / scale
        worst = max(worst, err)
        assert err <= 1e-5, f"{what}: pair {p} (row {t}, column {c}, expert {e}): error {err:.2e} of max"
        other = c ^ 1   # the other nibble of the same byte
        swapped = oracle.silu(Wg[:, other]) * Wu[:, other]
        worst_other = min(worst_other, np.max(np.abs(h[p] - swapped)) / scale)
    say(f"  {what}: {len(pairs)} pairs, worst error {worst:.1e} of max; neighbouring column misses by >= {worst_other:.1e}")
    assert worst_other > 1e-2


def test_onehot_one_row(verify):
    cfg, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=1)
    for c in COLS[:12]:
        check_onehot(g, view, [c], cfg.k, f"one row, column {c}")
    g.close()


@pytest.mark.parametrize("fused_max_rows", [0, -1])
def test_onehot_row_pairs(verify, fused_max_rows):
    cfg, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=8, fused_max_rows=fused_max_rows)
    for i in range(0, len(COLS), 4):
        check_onehot(g, view, COLS[i:i + 4], cfg.k, f"pairs (fused {fused_max_rows}), columns {COLS[i:i + 4]}")
    check_onehot(g, view, COLS[:8], cfg.k, "pairs, 8 rows")
    g.close()


@pytest.mark.parametrize("mfma_min_rows", [-1, 1])
def test_onehot_wide(verify, mfma_min_rows):
    """Wide rounds (staged digits), on the integer-dot GEMV (-1) and on the int8 matrix-core tile for
    every work item (1); each row of a work item sits in a different tile column."""
    cfg, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=64, mfma_min_rows=mfma_min_rows)
    check_onehot(g, view, COLS, cfg.k, f"wide T={len(COLS)}, mfma_min_rows {mfma_min_rows}")
    g.close()
