"""Pins for the fp64 oracle, each independent of the formula it checks.

Hand-written golden blocks pin the weight format; exact sums, brute force and
textbook routines pin the router and the selection; closed forms and
explicit loops pin the expert; the dense all-experts formulation pins the
combine; invariants pin the round and the worklist.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from conftest import read_golden


# ---------------------------------------------------------------------------
# helpers that build weights by hand (no oracle code)
# ---------------------------------------------------------------------------

def fp16_bits(v):
    return int(np.array(v, dtype=np.float16).view(np.uint16))


def const_matrix(rows, K, q, scale, minimum):
    """A [rows][K] matrix whose every weight is scale*q + minimum, in the packed layout."""
    byte = (q & 0xF) | ((q & 0xF) << 4)
    codes = np.full((rows, K // 2), byte, dtype=np.uint8)
    sm = np.full((rows, K // 32), fp16_bits(scale) | (fp16_bits(minimum) << 16), dtype=np.uint32)
    return codes, sm


def small_layer(E=6, H=64, I=32, seed=3, zipf=None):
    cfg = synth.ShapeConfig("t", H=H, E=E, k=2, I=I, zipf_s=zipf)
    return synth.make_layer(cfg, seed=seed, layer=0, device="cpu").numpy()


# ---------------------------------------------------------------------------
# weight format
# ---------------------------------------------------------------------------

def golden_blocks():
    blocks, cur = [], None
    for key, toks in read_golden("q4b32_blocks.txt"):
        if key == "block":
            cur = {"name": toks[0]}
            blocks.append(cur)
        elif key == "codes":
            cur["codes"] = np.array([int(t, 16) for t in toks], dtype=np.uint8)
        elif key == "scale_bits":
            cur["s"] = int(toks[0], 16)
        elif key == "min_bits":
            cur["m"] = int(toks[0], 16)
        elif key == "w":
            cur["w"] = np.array([float(t) for t in toks])
    return blocks


def test_golden_blocks_dequantise_exactly():
    blocks = golden_blocks()
    assert len(blocks) == 3
    for b in blocks:
        sm = np.array([b["s"] | (b["m"] << 16)], dtype=np.uint32)
        w = oracle.dequantize(b["codes"][None, :], sm[None, :])[0]
        assert w.shape == (32,)
        np.testing.assert_array_equal(w, b["w"], err_msg=b["name"])


def test_golden_block_codes_and_multi_block_rows():
    A, B, C = golden_blocks()
    np.testing.assert_array_equal(oracle.unpack_codes(A["codes"]), np.arange(32) % 16)
    # a row of three blocks: each block must use its own scale/min
    codes = np.concatenate([A["codes"], B["codes"], C["codes"]])[None, :]
    sm = np.array([[b["s"] | (b["m"] << 16) for b in (A, B, C)]], dtype=np.uint32)
    w = oracle.dequantize(codes, sm)[0]
    np.testing.assert_array_equal(w, np.concatenate([A["w"], B["w"], C["w"]]))


def test_quantise_then_dequantise_is_within_half_a_step():
    g = torch.Generator().manual_seed(11)
    W = torch.randn((6, 256), generator=g) * 0.02
    codes, sm = synth.quantize_q4b32(W)
    deq = oracle.dequantize(codes.numpy(), sm.numpy().view(np.uint32))
    Wd = W.double().numpy()
    blocks = Wd.reshape(6, 8, 32)
    mn = blocks.min(-1)
    s16 = ((blocks.max(-1) - mn) / 15).astype(np.float32).astype(np.float16).astype(np.float64)
    m16 = mn.astype(np.float32).astype(np.float16).astype(np.float64)
    bound = 0.5 * s16 + np.abs(m16 - mn) + 1e-9
    err = np.abs(deq - Wd).reshape(6, 8, 32)
    assert np.all(err <= bound[..., None])
    # rounding error of a uniform grid has rms ~ s/sqrt(12); a swapped or shifted nibble would not
    assert np.sqrt(np.mean(err ** 2)) < 0.4 * s16.mean()


# ---------------------------------------------------------------------------
# 4.5-bit super-block layout (Q4S256)
# ---------------------------------------------------------------------------

def golden_superblock_row():
    recs, w = [], {}
    for key, toks in read_golden("q4s256_superblocks.txt"):
        if key == "record":
            recs.append([int(t, 16) for t in toks])
        elif key == "w":
            w[int(toks[0])] = float(toks[1])
    codes = np.tile(np.array([0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE], dtype=np.uint8), 32)
    return codes[None, :], np.array(recs, dtype=np.uint32)[None, :, :], w


def test_golden_superblocks_dequantise_exactly():
    codes, rec, expect = golden_superblock_row()
    W = oracle.dequantize_q4s256(codes, rec)
    assert W.shape == (1, 512)
    for c, v in expect.items():
        assert W[0, c] == v, (c, W[0, c], v)


def _pow2_superblock_layer(seed, E=5, H=512, I=256):
    """A random Q4S256 layer whose d and dmin are powers of two, so every sub-block's d*sc and
    dmin*m are exact fp16 values; returns it with the equivalent Q4B32 layer (same codes, per-32
    fp16 scale d*sc and minimum -dmin*m, built here from the definition)."""
    rng = np.random.default_rng(seed)
    cfg = synth.ShapeConfig("t", H=H, E=E, k=2, I=I)
    base = synth.make_layer(cfg, seed=seed, layer=0, device="cpu").numpy()
    q4s = dict(base)
    q4b = dict(base)
    q4s["format"] = "q4s256"
    for name, K in (("gate", H), ("up", H), ("down", I)):
        rows = base[name + "_q"].shape[1]
        nsb = K // 256
        e_d = rng.integers(-14, -8, size=(E, rows, nsb))
        e_m = rng.integers(-15, -9, size=(E, rows, nsb))
        sc = rng.integers(0, 64, size=(E, rows, nsb, 8))
        mn = rng.integers(0, 64, size=(E, rows, nsb, 8))
        d = np.ldexp(1.0, e_d)
        dmin = np.ldexp(1.0, e_m)
        rec = np.zeros((E, rows, nsb, 4), dtype=np.uint32)
        rec[..., 0] = np.array(d, dtype=np.float16).view(np.uint16).astype(np.uint32) | (
            np.array(dmin, dtype=np.float16).view(np.uint16).astype(np.uint32) << 16)
        bits = [0] * 96
        for idx in np.ndindex(E, rows, nsb):
            string = 0
            for j in range(8):
                string |= (int(sc[idx + (j,)]) | (int(mn[idx + (j,)]) << 6)) << (12 * j)
            for wd in range(3):
                rec[idx + (wd + 1,)] = (string >> (32 * wd)) & 0xFFFFFFFF
        q4s[name + "_sm"] = rec
        s_blk = (d[..., None] * sc).reshape(E, rows, nsb * 8)
        m_blk = (-dmin[..., None] * mn).reshape(E, rows, nsb * 8)
        s16 = np.array(s_blk, dtype=np.float16)
        m16 = np.array(m_blk, dtype=np.float16)
        assert np.array_equal(s16.astype(np.float64), s_blk) and np.array_equal(m16.astype(np.float64), m_blk)
        q4b[name + "_sm"] = s16.view(np.uint16).astype(np.uint32) | (m16.view(np.uint16).astype(np.uint32) << 16)
    return q4s, q4b


def test_superblock_layer_equals_equivalent_block_layer():
    """The same weights in both layouts give bitwise the same round (the Q4B32 side is pinned by
    the golden blocks above); random scales and minima per sub-block pin the field order, the
    sub-block and super-block indexing and the sign of the minimum."""
    q4s, q4b = _pow2_superblock_layer(seed=5)
    rng = np.random.default_rng(6)
    X = rng.standard_normal((3, q4s["router_w"].shape[1]))
    a = oracle.moe_layer(q4s, X, 2)
    b = oracle.moe_layer(q4b, X, 2)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    for name in ("gate", "up", "down"):
        assert np.array_equal(oracle.dequantize_any(q4s[name + "_q"], q4s[name + "_sm"], "q4s256"),
                              oracle.dequantize(q4b[name + "_q"], q4b[name + "_sm"]))


def test_superblock_quantise_then_dequantise_is_within_a_step():
    g = torch.Generator().manual_seed(7)
    w = torch.randn((6, 512), generator=g) * 0.02
    codes, rec = synth.quantize_q4s256(w)
    W = oracle.dequantize_q4s256(codes.numpy(), rec.numpy())
    b = w.double().numpy().reshape(6, 2, 8, 32)
    step = (b.max(-1) - b.min(-1)) / 15.0           # the sub-block's own quantisation step
    err = np.abs(W.reshape(6, 2, 8, 32) - b).max(-1)
    assert np.all(err <= 1.5 * step + 1e-4), err.max()


# ---------------------------------------------------------------------------
# router and selection
# ---------------------------------------------------------------------------

def test_router_logits_equal_exactly_rounded_sums():
    rng = np.random.default_rng(5)
    Wr = rng.standard_normal((5, 96)).astype(np.float32) * 0.02
    x = rng.standard_normal(96).astype(np.float32)
    b = rng.standard_normal(5).astype(np.float32)
    z = oracle.router_logits(Wr, b, x)
    for e in range(5):
        terms = [float(Wr[e, h]) * float(x[h]) for h in range(96)]   # exact in fp64
        ref = math.fsum(terms + [float(b[e])])
        assert abs(z[e] - ref) <= 1e-14 * (sum(abs(t) for t in terms) + abs(float(b[e])))
    z0 = oracle.router_logits(Wr, None, x)
    for e in range(5):
        ref = math.fsum(float(Wr[e, h]) * float(x[h]) for h in range(96))
        assert abs(z0[e] - ref) <= 1e-14 * np.abs(Wr[e].astype(np.float64) * x).sum()


@pytest.mark.parametrize("k", range(1, 8))
def test_topk_matches_brute_force(k):
    rng = np.random.default_rng(k)
    for _ in range(20):
        z = rng.standard_normal(7)
        ids = oracle.select_topk(z, k)
        best = max(itertools.combinations(range(7), k), key=lambda c: sum(z[list(c)]))
        assert set(ids.tolist()) == set(best)
        assert all(z[ids[i]] > z[ids[i + 1]] for i in range(k - 1))


def test_topk_ties_go_to_lower_id():
    z = np.array([1.0, 2.0, 2.0, 0.0, 2.0])
    assert oracle.select_topk(z, 1).tolist() == [1]
    assert oracle.select_topk(z, 2).tolist() == [1, 2]
    assert oracle.select_topk(z, 3).tolist() == [1, 2, 4]
    assert oracle.select_topk(z, 4).tolist() == [1, 2, 4, 0]
    assert oracle.selection_gap(z, 2) == 0.0
    assert oracle.selection_gap(np.array([3.0, 1.0, 0.5, -2.0]), 2) == 0.5


def test_routing_weights_reduce_to_textbook_softmax():
    rng = np.random.default_rng(9)
    z = rng.standard_normal(6) * 3
    ids = oracle.select_topk(z, 6)
    p = oracle.routing_weights(z, ids)
    np.testing.assert_allclose(p, scipy.special.softmax(z)[ids], rtol=1e-14, atol=0)
    assert oracle.routing_weights(z, oracle.select_topk(z, 1)).tolist() == [1.0]
    i2 = oracle.select_topk(z, 2)
    p2 = oracle.routing_weights(z, i2)
    assert abs(p2[0] - scipy.special.expit(z[i2[0]] - z[i2[1]])) < 1e-15
    assert abs(p2.sum() - 1.0) < 1e-15


def test_silu_is_x_times_sigmoid():
    a = np.linspace(-30, 30, 241)
    np.testing.assert_allclose(oracle.silu(a), a * scipy.special.expit(a), rtol=1e-14, atol=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


# ---------------------------------------------------------------------------
# expert feed-forward
# ---------------------------------------------------------------------------

def test_closed_form_expert():
    H, I = 64, 32
    gq, gs = const_matrix(I, H, 1, 1.0, 0.0)     # gate: all ones
    uq, us = const_matrix(I, H, 0, 0.0, 1.0)     # up: all ones, through the minimum
    dq, ds = const_matrix(H, I, 1, 1.0, 0.0)     # down: all ones
    for x0, x1 in ((1.0, 0.0), (0.5, 0.25), (-2.0, 0.5)):
        x = np.zeros(H)
        x[0], x[1] = x0, x1
        S = x0 + x1
        y = oracle.expert_forward(gq, gs, uq, us, dq, ds, x)
        expect = I * (S / (1.0 + math.exp(-S))) * S
        np.testing.assert_allclose(y, np.full(H, expect), rtol=1e-15)
    dq2, ds2 = const_matrix(H, I, 1, 2.0, 0.0)   # down: all twos
    x = np.zeros(H)
    x[3] = 1.0
    np.testing.assert_array_equal(oracle.expert_forward(gq, gs, uq, us, dq2, ds2, x),
                                  2 * oracle.expert_forward(gq, gs, uq, us, dq, ds, x))


def test_single_expert_layer_equals_explicit_loops():
    L = small_layer(E=1, H=64, I=32, seed=21)
    x = np.random.default_rng(2).standard_normal(64).astype(np.float32)
    out, ids, p, _ = oracle.moe_layer(L, x[None, :], k=1)
    assert ids.tolist() == [[0]] and p.tolist() == [[1.0]]
    Wg = oracle.dequantize(L["gate_q"][0], L["gate_sm"][0])
    Wu = oracle.dequantize(L["up_q"][0], L["up_sm"][0])
    Wd = oracle.dequantize(L["down_q"][0], L["down_sm"][0])
    h = []
    for i in range(32):
        g = sum(Wg[i, c] * float(x[c]) for c in range(64))
        v = sum(Wu[i, c] * float(x[c]) for c in range(64))
        h.append(g / (1.0 + math.exp(-g)) * v)
    y = [sum(Wd[r, i] * h[i] for i in range(32)) for r in range(64)]
    np.testing.assert_allclose(out[0], y, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# combine, round structure
# ---------------------------------------------------------------------------

def test_sparse_combine_equals_dense_all_experts():
    E, H, I, T, k = 6, 64, 32, 3, 3
    L = small_layer(E=E, H=H, I=I, seed=4, zipf=1.0)
    X = np.random.default_rng(1).standard_normal((T, H)).astype(np.float32)
    out, ids, p, _ = oracle.moe_layer(L, X, k)
    # dense: evaluate every expert on every row, weight by a softmax restricted to the top-k mask
    Y = np.stack([[oracle.expert_forward(L["gate_q"][e], L["gate_sm"][e], L["up_q"][e], L["up_sm"][e],
                                         L["down_q"][e], L["down_sm"][e], X[t]) for e in range(E)]
                  for t in range(T)])                                   # [T, E, H]
    Z = X.astype(np.float64) @ L["router_w"].astype(np.float64).T + L["router_b"].astype(np.float64)
    for t in range(T):
        kth = np.sort(Z[t])[::-1][k - 1]
        mask = Z[t] >= kth
        assert mask.sum() == k
        gate = np.where(mask, scipy.special.softmax(np.where(mask, Z[t], -np.inf)), 0.0)
        np.testing.assert_allclose(out[t], gate @ Y[t], rtol=1e-12, atol=1e-14)
        assert set(ids[t].tolist()) == set(np.nonzero(mask)[0].tolist())


def test_round_equals_per_row_evaluations():
    L = small_layer(E=8, H=64, I=32, seed=6)
    X = np.random.default_rng(3).standard_normal((5, 64)).astype(np.float32)
    out, ids, p, _ = oracle.moe_layer(L, X, k=2)
    for t in range(5):
        o1, i1, p1, _ = oracle.moe_layer(L, X[t:t + 1], k=2)
        np.testing.assert_array_equal(o1[0], out[t])
        np.testing.assert_array_equal(i1[0], ids[t])
        np.testing.assert_array_equal(p1[0], p[t])


def test_doubling_down_scale_and_min_doubles_output():
    L = small_layer(E=5, H=64, I=32, seed=8)
    X = np.random.default_rng(4).standard_normal((2, 64)).astype(np.float32)
    out, *_ = oracle.moe_layer(L, X, k=2)
    L2 = dict(L)
    s, m = L["down_sm"] & 0xFFFF, L["down_sm"] >> 16
    s2 = (s.astype(np.uint16).view(np.float16) * np.float16(2)).view(np.uint16).astype(np.uint32)
    m2 = (m.astype(np.uint16).view(np.float16) * np.float16(2)).view(np.uint16).astype(np.uint32)
    L2["down_sm"] = (s2 | (m2 << 16)).astype(np.uint32)
    out2, *_ = oracle.moe_layer(L2, X, k=2)
    np.testing.assert_array_equal(out2, 2 * out)


def test_permuting_experts_permutes_ids_only():
    E = 7
    L = small_layer(E=E, H=64, I=32, seed=10, zipf=1.1)
    X = np.random.default_rng(5).standard_normal((3, 64)).astype(np.float32)
    out, ids, p, _ = oracle.moe_layer(L, X, k=3)
    perm = np.random.default_rng(0).permutation(E)          # new expert i is old expert perm[i]
    LP = {key: (v if v is None or isinstance(v, str) else v[perm]) for key, v in L.items()}
    outP, idsP, pP, _ = oracle.moe_layer(LP, X, k=3)
    np.testing.assert_array_equal(perm[idsP], ids)
    np.testing.assert_array_equal(pP, p)
    np.testing.assert_array_equal(outP, out)


def test_residual_stack_is_layer_composition():
    layers = [small_layer(E=6, H=64, I=32, seed=s) for s in (12, 13, 14)]
    X = np.random.default_rng(6).standard_normal((2, 64)).astype(np.float32)
    out, ids, p, gaps = oracle.moe_round(layers, X, k=2, residual=True)
    x = X.astype(np.float64)
    for li, L in enumerate(layers):
        y, i, _, _ = oracle.moe_layer(L, x, k=2)
        np.testing.assert_array_equal(i, ids[li])
        x = x + y
    np.testing.assert_array_equal(out, x)
    assert ids.shape == (3, 2, 2) and gaps.shape == (3, 2)
    with pytest.raises(ValueError):
        oracle.moe_round(layers, X, k=2, residual=False)


def test_router_bias_forces_selection():
    L = small_layer(E=6, H=64, I=32, seed=15)
    L["router_b"] = np.zeros(6, dtype=np.float32)
    L["router_b"][4] = 100.0
    X = np.random.default_rng(7).standard_normal((3, 64)).astype(np.float32)
    _, ids, p, _ = oracle.moe_layer(L, X, k=2)
    assert (ids[:, 0] == 4).all()
    assert (p[:, 0] > 0.999).all()


# ---------------------------------------------------------------------------
# worklist
# ---------------------------------------------------------------------------

def golden_worklists():
    cases, cur = [], None
    parse = lambda toks: [[int(v) for v in grp.split()] for grp in " ".join(toks).split("/")]
    for key, toks in read_golden("worklist_small.txt"):
        if key == "ids":
            cur = {"ids": np.array(parse(toks))}
            cases.append(cur)
        elif key in ("uniq", "offs"):
            cur[key] = [int(v) for v in toks]
        elif key == "pairs":
            cur["pairs"] = parse(toks)
    return cases


def test_worklist_golden():
    cases = golden_worklists()
    assert len(cases) == 2
    for c in cases:
        uniq, offs, pairs = oracle.build_worklist(c["ids"])
        assert uniq.tolist() == c["uniq"]
        assert offs.tolist() == c["offs"]
        assert pairs.tolist() == c["pairs"]


@pytest.mark.parametrize("T,k,E", [(1, 8, 128), (3, 10, 512), (8, 8, 256), (64, 8, 256), (5, 2, 8)])
def test_worklist_invariants(T, k, E):
    rng = np.random.default_rng(T * 1000 + k)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    uniq, offs, pairs = oracle.build_worklist(ids)
    union = sorted(set(ids.ravel().tolist()))
    assert uniq.tolist() == union                     # n_unique == |union of per-row sets|
    assert offs[0] == 0 and offs[-1] == T * k and np.all(np.diff(offs) >= 1)
    seen = sorted(map(tuple, pairs.tolist()))
    assert seen == [(t, j) for t in range(T) for j in range(k)]   # every pair exactly once
    for u, e in enumerate(uniq):
        seg = pairs[offs[u]:offs[u + 1]]
        assert all(ids[t, j] == e for t, j in seg)
        assert np.all(np.diff(seg[:, 0]) > 0)           # rows ascending within an expert


# ---------------------------------------------------------------------------
# tail skip (Avalon README, results section)
# ---------------------------------------------------------------------------

def golden_tail_skip():
    parse = lambda toks: [[int(v) for v in grp.split()] for grp in " ".join(toks).split("/") if grp.strip()]
    head, cases, cur = {}, [], None
    for key, toks in read_golden("tail_skip.txt"):
        if key == "ids":
            head["ids"] = np.array(parse(toks))
        elif key == "resident":
            head["resident"] = [int(v) for v in toks]
        elif key == "case":
            cur = {"rank": int(toks[0])}
            cases.append(cur)
        elif key in ("skipped", "uniq", "offs"):
            cur[key] = [int(v) for v in toks]
        elif key in ("dropped", "pairs"):
            cur[key] = parse(toks)
    return head, cases


def test_tail_skip_golden():
    head, cases = golden_tail_skip()
    ids = head["ids"]
    E = 16
    resident = np.zeros(E, dtype=bool)
    resident[head["resident"]] = True
    assert [c["rank"] for c in cases] == [7, 6, 1, 9]
    for c in cases:
        keep = oracle.tail_skip_keep(ids, resident, c["rank"])
        skipped = sorted(set(ids[~keep].tolist()))
        assert skipped == c["skipped"], c["rank"]
        # a skipped expert loses every pair, a kept one none
        assert not set(ids[keep].tolist()) & set(skipped)
        if "dropped" in c:
            assert sorted(map(list, np.argwhere(~keep).tolist())) == sorted(c["dropped"])
        if "uniq" in c:
            uniq, offs, pairs = oracle.build_worklist(ids, keep)
            assert uniq.tolist() == c["uniq"]
            assert offs.tolist() == c["offs"]
            assert pairs.tolist() == c["pairs"]


def test_tail_skip_off_cases_keep_everything():
    rng = np.random.default_rng(5)
    ids = np.stack([rng.choice(64, size=8, replace=False) for _ in range(4)])
    missed = np.zeros(64, dtype=bool)
    for rank in (0, -1, 9, 100):  # off, or past k
        assert oracle.tail_skip_keep(ids, missed, rank).all()
    assert oracle.tail_skip_keep(ids, None, 7).all()
    assert oracle.tail_skip_keep(ids, np.ones(64, dtype=bool), 1).all()  # nothing missed
    assert oracle.build_worklist(ids, np.ones(ids.shape, dtype=bool))[1][-1] == ids.size


def test_tail_skip_brute_force_over_subsets():
    """Per expert, straight from the rule's wording: skipped iff missed and no selecting row ranks
    it above skip_rank; checked on random rounds against the expert-by-expert evaluation."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        T, k, E = int(rng.integers(1, 6)), int(rng.integers(1, 9)), 12
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
        resident = rng.random(E) < 0.4
        r = int(rng.integers(1, k + 2))
        keep = oracle.tail_skip_keep(ids, resident, r)
        for e in range(E):
            rows = [(t, j) for t in range(T) for j in range(k) if ids[t, j] == e]
            if not rows:
                continue
            skipped = (not resident[e]) and all(j + 1 >= r for _, j in rows)
            assert all(keep[t, j] == (not skipped) for t, j in rows)


def test_tail_skip_layer_drops_exactly_the_skipped_terms():
    """out(skip) + sum over dropped pairs of p * expert(x) == out(no skip), routing weights and ids
    unchanged (no renormalisation)."""
    layer = small_layer(E=12, H=64, I=32, seed=7)
    X = np.random.default_rng(3).standard_normal((4, 64))
    k = 6
    resident = np.zeros(12, dtype=bool)
    resident[[0, 4, 8]] = True
    full, ids, p, _ = oracle.moe_layer(layer, X, k)
    for r in (1, 3, 5, 6):
        out, ids2, p2, _ = oracle.moe_layer(layer, X, k, resident=resident, skip_rank=r)
        assert np.array_equal(ids2, ids) and np.array_equal(p2, p)
        keep = oracle.tail_skip_keep(ids, resident, r)
        back = out.copy()
        for t, j in np.argwhere(~keep):
            e = int(ids[t, j])
            w = [layer[n][e] for n in ("gate_q", "gate_sm", "up_q", "up_sm", "down_q", "down_sm")]
            back[t] += p[t, j] * oracle.expert_forward(*w, X[t])
        np.testing.assert_allclose(back, full, rtol=1e-12, atol=1e-12)
    # skip_rank 1: only resident experts contribute, each row on its own ranks
    out1, _, _, _ = oracle.moe_layer(layer, X, k, resident=resident, skip_rank=1)
    for t in range(4):
        acc = np.zeros(64)
        for j in range(k):
            e = int(ids[t, j])
            if resident[e]:
                w = [layer[n][e] for n in ("gate_q", "gate_sm", "up_q", "up_sm", "down_q", "down_sm")]
                acc += p[t, j] * oracle.expert_forward(*w, X[t])
        np.testing.assert_allclose(out1[t], acc, rtol=1e-12, atol=1e-14)


def test_tail_skip_depends_on_the_round():
    """A missed expert at rank 7 of one row is skipped alone, and kept once another row of the
    same round ranks it higher."""
    resident = np.zeros(16, dtype=bool)
    a = np.array([[0, 1, 2, 3, 4, 5, 6, 7]])
    b = np.array([[6, 8, 9, 10, 11, 12, 13, 14]])
    assert not oracle.tail_skip_keep(a, resident, 7)[0, 6]
    both = oracle.tail_skip_keep(np.concatenate([a, b]), resident, 7)
    assert both[0, 6] and both[1, 0]


def test_residency_generator_keeps_the_hottest_experts():
    """With a Zipf router bias the resident experts are those with the largest bias."""
    cfg = synth.config("deep").replace(H=256, I=32)
    res = synth.make_residency(cfg, 0.25, seed=0, layer=2)
    assert res.sum() == cfg.E // 4
    b = synth.make_layer(cfg, seed=0, layer=2).router_b.numpy()
    assert b[res].min() >= b[~res].max()
    plain = synth.make_residency(synth.config("verify"), 0.5, seed=1)
    assert plain.sum() == 128
