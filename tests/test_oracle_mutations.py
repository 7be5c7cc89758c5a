"""Plant plausible mistakes in the oracle (CPU only) and check that some pin catches each one."""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as om
import test_oracle_pins as pins

BLOCK = 32


def _swap_nibbles(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = codes >> 4
    out[..., 1::2] = codes & 0x0F
    return out


def _dequant_no_min(codes, sm):
    q = om.unpack_codes(codes)
    s, m = om.unpack_scale_min(sm)
    blk = np.arange(q.shape[-1]) // BLOCK
    return s[..., blk] * q


def _dequant_wrong_block(codes, sm):
    q = om.unpack_codes(codes)
    s, m = om.unpack_scale_min(sm)
    blk = (np.arange(q.shape[-1]) % s.shape[-1])
    return s[..., blk] * q + m[..., blk]


def _swap_scale_min(sm):
    s, m = ORIG["unpack_scale_min"](sm)
    return m, s


def _q4s_min_added(codes, rec):
    q = om.unpack_codes(codes)
    d, dmin, sc, mn = om.unpack_superblocks(rec)
    qb = q.reshape(q.shape[:-1] + (q.shape[-1] // 256, 8, 32))
    return (d[..., None, None] * sc[..., None] * qb + dmin[..., None, None] * mn[..., None]).reshape(q.shape)


def _q4s_subblock_shifted(codes, rec):
    q = om.unpack_codes(codes)
    d, dmin, sc, mn = om.unpack_superblocks(rec)
    sc, mn = np.roll(sc, 1, axis=-1), np.roll(mn, 1, axis=-1)
    qb = q.reshape(q.shape[:-1] + (q.shape[-1] // 256, 8, 32))
    return (d[..., None, None] * sc[..., None] * qb - dmin[..., None, None] * mn[..., None]).reshape(q.shape)


def _q4s_fields_swapped(rec):
    d, dmin, sc, mn = ORIG["unpack_superblocks"](rec)
    return d, dmin, mn, sc


def _q4s_first_superblock_only(codes, rec):
    rec = np.asarray(rec).view(np.uint32)
    rec0 = np.broadcast_to(rec[..., :1, :], rec.shape).copy()
    return ORIG["dequantize_q4s256"](codes, rec0)


def _router_no_bias(router_w, router_b, x):
    return np.asarray(router_w, dtype=np.float64) @ np.asarray(x, dtype=np.float64)


def _router_fp32(router_w, router_b, x):
    z = (np.asarray(router_w, dtype=np.float32) @ np.asarray(x, dtype=np.float32)).astype(np.float64)
    if router_b is not None:
        z = z + np.asarray(router_b, dtype=np.float64)
    return z


def _topk_ties_high(z, k):
    return np.argsort(np.asarray(z, dtype=np.float64), kind="stable")[::-1][:k].astype(np.int64)


def _topk_ascending(z, k):
    return ORIG["select_topk"](z, k)[::-1].copy()


def _softmax_all(z, ids):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max())
    return e[ids] / e.sum()


def _silu_sign(a):
    a = np.asarray(a, dtype=np.float64)
    return a / (1.0 + np.exp(a))


def _ffn_silu_on_up(Wg, Wu, Wd, x):
    x = np.asarray(x, dtype=np.float64)
    return Wd @ ((Wg @ x) * om.silu(Wu @ x))


def _ffn_add(Wg, Wu, Wd, x):
    x = np.asarray(x, dtype=np.float64)
    return Wd @ (om.silu(Wg @ x) + Wu @ x)


def _ffn_transposed_down(Wg, Wu, Wd, x):
    x = np.asarray(x, dtype=np.float64)
    h = om.silu(Wg @ x) * (Wu @ x)
    return (Wd.reshape(Wd.shape[1], Wd.shape[0]) @ h) if Wd.shape[0] != Wd.shape[1] else Wd.T @ h


def _worklist_rows_descending(ids):
    uniq, offs, pairs = ORIG["build_worklist"](ids)
    for u in range(len(uniq)):
        pairs[offs[u]:offs[u + 1]] = pairs[offs[u]:offs[u + 1]][::-1]
    return uniq, offs, pairs


def _layer_unweighted(layer, X, k, residual=False):
    out, ids, p, gaps = ORIG["moe_layer"](layer, X, k, residual)
    X = np.asarray(X, dtype=np.float64)
    out2 = np.zeros_like(out)
    for t in range(X.shape[0]):
        for j in range(k):
            e = int(ids[t, j])
            out2[t] += om.expert_forward(layer["gate_q"][e], layer["gate_sm"][e], layer["up_q"][e],
                                         layer["up_sm"][e], layer["down_q"][e], layer["down_sm"][e], X[t])
        if residual:
            out2[t] += X[t]
    return out2, ids, p, gaps


def _round_no_residual(layers, X, k, residual):
    x = np.asarray(X, dtype=np.float64)
    outs = []
    for layer in layers:
        x, ids, p, gaps = ORIG["moe_layer"](layer, x, k, False)
        outs.append((ids, p, gaps))
    return (x, np.stack([o[0] for o in outs]), np.stack([o[1] for o in outs]),
            np.stack([o[2] for o in outs]))


def _skip_ignores_residency(ids, resident, skip_rank):
    return ORIG["tail_skip_keep"](ids, None if resident is None else np.zeros(len(resident), bool), skip_rank)


def _skip_rank_off_by_one(ids, resident, skip_rank):
    return ORIG["tail_skip_keep"](ids, resident, skip_rank + 1 if skip_rank > 0 else skip_rank)


def _skip_per_pair(ids, resident, skip_rank):
    ids = np.asarray(ids)
    keep = np.ones(ids.shape, dtype=bool)
    if skip_rank <= 0 or resident is None:
        return keep
    for (t, j), e in np.ndenumerate(ids):
        keep[t, j] = bool(resident[e]) or j + 1 < skip_rank
    return keep


def _layer_renormalised_after_skip(layer, X, k, residual=False, cache=None, resident=None, skip_rank=0):
    out, ids, p, gaps = ORIG["moe_layer"](layer, X, k, residual, cache, resident, skip_rank)
    keep = ORIG["tail_skip_keep"](ids, resident, skip_rank)
    if keep.all():
        return out, ids, p, gaps
    X = np.asarray(X, dtype=np.float64)
    out2 = X.copy() if residual else np.zeros_like(out)
    for t in range(X.shape[0]):
        tot = p[t][keep[t]].sum()
        for j in range(k):
            if keep[t, j]:
                e = int(ids[t, j])
                out2[t] += p[t, j] / tot * om.expert_forward(
                    layer["gate_q"][e], layer["gate_sm"][e], layer["up_q"][e], layer["up_sm"][e],
                    layer["down_q"][e], layer["down_sm"][e], X[t])
    return out2, ids, p, gaps


ORIG = {name: getattr(om, name) for name in
        ("unpack_codes", "unpack_scale_min", "dequantize", "unpack_superblocks", "dequantize_q4s256",
         "router_logits", "select_topk",
         "routing_weights", "silu", "swiglu_ffn", "expert_forward", "moe_layer", "moe_round",
         "build_worklist", "tail_skip_keep")}

MUTATIONS = {
    "swapped nibbles": ("unpack_codes", _swap_nibbles),
    "dropped minimum": ("dequantize", _dequant_no_min),
    "wrong block index": ("dequantize", _dequant_wrong_block),
    "scale/min swapped": ("unpack_scale_min", _swap_scale_min),
    "super-block minimum added": ("dequantize_q4s256", _q4s_min_added),
    "sub-block index shifted": ("dequantize_q4s256", _q4s_subblock_shifted),
    "super-block scale/min fields swapped": ("unpack_superblocks", _q4s_fields_swapped),
    "first super-block only": ("dequantize_q4s256", _q4s_first_superblock_only),
    "router bias dropped": ("router_logits", _router_no_bias),
    "router accumulates in fp32": ("router_logits", _router_fp32),
    "ties to higher id": ("select_topk", _topk_ties_high),
    "ascending order": ("select_topk", _topk_ascending),
    "softmax over all experts": ("routing_weights", _softmax_all),
    "silu sign": ("silu", _silu_sign),
    "silu on up": ("swiglu_ffn", _ffn_silu_on_up),
    "add instead of multiply": ("swiglu_ffn", _ffn_add),
    "down projection transposed": ("swiglu_ffn", _ffn_transposed_down),
    "unweighted combine": ("moe_layer", _layer_unweighted),
    "rows descending in worklist": ("build_worklist", _worklist_rows_descending),
    "residual dropped": ("moe_round", _round_no_residual),
    "tail skip ignores residency": ("tail_skip_keep", _skip_ignores_residency),
    "tail skip rank off by one": ("tail_skip_keep", _skip_rank_off_by_one),
    "tail skip decided per pair": ("tail_skip_keep", _skip_per_pair),
    "weights renormalised after the skip": ("moe_layer", _layer_renormalised_after_skip),
}


def _all_pins():
    calls = []
    for name in dir(pins):
        fn = getattr(pins, name)
        if not name.startswith("test_") or not callable(fn):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argnames, values = params[0].args[0], params[0].args[1]
            for v in list(values)[:3]:
                if isinstance(argnames, str) and "," in argnames:
                    kw = dict(zip([a.strip() for a in argnames.split(",")], v))
                else:
                    kw = {argnames: v}
                calls.append((name, fn, kw))
        else:
            calls.append((name, fn, {}))
    return calls


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_some_pin_catches(mutation, monkeypatch):
    target, fake = MUTATIONS[mutation]
    monkeypatch.setattr(om, target, fake)
    monkeypatch.setattr(oracle, target, fake)
    caught = []
    for name, fn, kw in _all_pins():
        try:
            fn(**kw)
        except (AssertionError, ValueError, IndexError, KeyError, TypeError):
            caught.append(name)
    assert caught, f"no pin caught the planted mistake: {mutation}"
