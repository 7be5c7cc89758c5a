"""fp64 reference of one MoE decode/verify round — TEST INFRASTRUCTURE ONLY.

Written from the pages, row by row, with no blocking, fusion or reordering:

  * infero README, "Beyond plain text decode" (MoE bullet): a router scores
    experts, a top-k kernel picks them at decode, and a counting sort groups
    (row, expert) pairs by expert for a per-expert GEMM.
  * infero README, "Layout" (decoder-block figure): the expert is the SwiGLU
    feed-forward silu(W_g x) * (W_u x) followed by W_d.
  * infero README, "Design notes": block-encoded weights are read in place;
    activations are fp32 so intermediates compare against a CPU reference.
  * infero README, "AWQ, FP8, and NVFP4 checkpoints": a 4-bit block format
    keeps a scale and a minimum every 32 weights; its K-quant unpacks a 6-bit
    scale and a 6-bit minimum from a packed twelve-byte field every 32
    weights, in 256-element super-blocks ("Supported weight encodings").
  * AlphaInfer page, section 2 ("One captured graph per decode round"): a
    round is one forward pass over 1-8 token rows; section 3.1: each extra
    verified row routes to experts the others did not need, so the set of
    experts a round touches is the union over its rows.

Readings where the pages are silent (each also listed in the design notes):
  * dequantisation is w = s*q + m (fp16 scale s, fp16 minimum m, q in 0..15);
  * in the 4.5-bit layout (Q4S256) a 256-weight super-block carries fp16 d and
    dmin and, per 32-weight sub-block j, a 6-bit scale sc_j and a 6-bit
    minimum m_j (12-bit field j at bit 12j of a 96-bit string); a weight is
    d*sc_j*q - dmin*m_j;
  * byte j of a 32-block holds element 2j (low nibble) and 2j+1 (high nibble);
  * selection is the k largest logits in descending order, ties to the lower
    expert id;
  * routing weights are the softmax of the k selected logits, nothing else;
  * SiLU is applied to the gate projection; no shared expert, no norm;
  * a multi-layer round adds each layer's MoE output to its input
    (residual), and a single-layer round returns the MoE output alone;
  * tail skip (Avalon README, results section): an expert is "missed" when it
    is not resident in GPU memory; ranks are the 1-based positions of the
    descending top-k; a missed expert is skipped for the whole round when
    every row that selected it ranks it at the skip rank or below (rank >=
    skip_rank), so its (row, rank) pairs add nothing; the other pairs keep
    their routing weights (no renormalisation: the page names none).

Parity pins (tests/test_oracle_pins.py): every function below is pinned by a
check independent of its own formula (hand-written golden blocks, closed
forms, brute force, textbook routines, invariants).  No function is "parity
unpinned".
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
SUPER = 256


# ---------------------------------------------------------------------------
# Weight format
# ---------------------------------------------------------------------------

def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """uint8 [..., K/2] -> float64 [..., K]: element 2j is byte j's low nibble, 2j+1 its high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = codes & 0x0F
    out[..., 1::2] = codes >> 4
    return out


def unpack_scale_min(sm: np.ndarray):
    """uint32 [..., K/32] -> (scale f64, minimum f64): low half fp16 scale, high half fp16 minimum."""
    sm = np.asarray(sm).view(np.uint32)
    s16 = (sm & 0xFFFF).astype(np.uint16).view(np.float16)
    m16 = (sm >> 16).astype(np.uint16).view(np.float16)
    return s16.astype(np.float64), m16.astype(np.float64)


def dequantize(codes: np.ndarray, sm: np.ndarray) -> np.ndarray:
    """W[r, c] = s[r, c//32] * q[r, c] + m[r, c//32], exact in fp64 (an 11-bit x 4-bit product plus an fp16)."""
    q = unpack_codes(codes)
    s, m = unpack_scale_min(sm)
    K = q.shape[-1]
    qb = q.reshape(q.shape[:-1] + (K // BLOCK, BLOCK))
    return (s[..., None] * qb + m[..., None]).reshape(q.shape)


def unpack_superblocks(rec: np.ndarray):
    """uint32 [..., K/256, 4] -> (d, dmin) f64 [..., K/256] and (sc, mn) f64 [..., K/256, 8].

    Word 0 holds fp16 d (low half) and fp16 dmin (high half); words 1..3 are a little-endian 96-bit
    string whose bits 12j..12j+11 are sub-block j's field: scale in bits 0-5, minimum in bits 6-11.
    """
    rec = np.asarray(rec).view(np.uint32)
    d = (rec[..., 0] & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    dmin = (rec[..., 0] >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    # the 96-bit string as three 32-bit pieces; field j starts at bit 12j
    words = [rec[..., 1].astype(np.uint64), rec[..., 2].astype(np.uint64), rec[..., 3].astype(np.uint64)]
    sc = np.empty(rec.shape[:-1] + (8,), dtype=np.float64)
    mn = np.empty(rec.shape[:-1] + (8,), dtype=np.float64)
    for j in range(8):
        start = 12 * j
        field = np.zeros(rec.shape[:-1], dtype=np.uint64)
        for bit in range(12):                      # gather the field bit by bit
            pos = start + bit
            b = (words[pos // 32] >> np.uint64(pos % 32)) & np.uint64(1)
            field |= b << np.uint64(bit)
        sc[..., j] = (field & np.uint64(63)).astype(np.float64)
        mn[..., j] = (field >> np.uint64(6)).astype(np.float64)
    return d, dmin, sc, mn


def dequantize_q4s256(codes: np.ndarray, rec: np.ndarray) -> np.ndarray:
    """W[r, c] = d*sc_j*q[r, c] - dmin*m_j with super-block c//256 and sub-block j = (c % 256)//32;
    exact in fp64 (an 11-bit x 6-bit x 4-bit product and an 11-bit x 6-bit one)."""
    q = unpack_codes(codes)
    d, dmin, sc, mn = unpack_superblocks(rec)
    K = q.shape[-1]
    qb = q.reshape(q.shape[:-1] + (K // SUPER, SUPER // BLOCK, BLOCK))
    w = d[..., None, None] * sc[..., None] * qb - dmin[..., None, None] * mn[..., None]
    return w.reshape(q.shape)


def dequantize_any(codes: np.ndarray, sm: np.ndarray, fmt: str = "q4b32") -> np.ndarray:
    """The matrix of either weight layout ("q4b32" or "q4s256")."""
    if fmt == "q4s256":
        return dequantize_q4s256(codes, sm)
    if fmt != "q4b32":
        raise ValueError(f"unknown weight format {fmt!r}")
    return dequantize(codes, sm)


# ---------------------------------------------------------------------------
# Router, selection, routing weights
# ---------------------------------------------------------------------------

def router_logits(router_w: np.ndarray, router_b, x: np.ndarray) -> np.ndarray:
    """z[e] = sum_h Wr[e, h] * x[h] (+ b[e]) in fp64; each fp32 x fp32 product is exact in fp64."""
    z = np.asarray(router_w, dtype=np.float64) @ np.asarray(x, dtype=np.float64)
    if router_b is not None:
        z = z + np.asarray(router_b, dtype=np.float64)
    return z


def select_topk(z: np.ndarray, k: int) -> np.ndarray:
    """The k largest logits' expert ids, descending; equal logits go to the lower id (stable sort)."""
    order = np.argsort(-np.asarray(z, dtype=np.float64), kind="stable")
    return order[:k].astype(np.int64)


def selection_gap(z: np.ndarray, k: int) -> float:
    """Smallest logit gap that decides the selection or its order (ranks 0..k, i.e. k+1 values)."""
    zs = np.sort(np.asarray(z, dtype=np.float64))[::-1]
    n = min(k + 1, zs.size)
    if n < 2:
        return float("inf")
    return float(np.min(zs[: n - 1] - zs[1:n]))


def routing_weights(z: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits only: p_j = exp(z_j - max) / sum_j' exp(z_j' - max)."""
    zs = np.asarray(z, dtype=np.float64)[ids]
    e = np.exp(zs - zs.max())
    return e / e.sum()


# ---------------------------------------------------------------------------
# Expert feed-forward
# ---------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a))."""
    a = np.asarray(a, dtype=np.float64)
    return a / (1.0 + np.exp(-a))


def expert_matrices(gate_q, gate_sm, up_q, up_sm, down_q, down_sm, fmt: str = "q4b32"):
    """Dequantise one expert: (W_g [I,H], W_u [I,H], W_d [H,I]) in fp64."""
    return (dequantize_any(gate_q, gate_sm, fmt), dequantize_any(up_q, up_sm, fmt),
            dequantize_any(down_q, down_sm, fmt))


def swiglu_ffn(Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = W_d (silu(W_g x) * (W_u x))."""
    x = np.asarray(x, dtype=np.float64)
    g = Wg @ x
    v = Wu @ x
    h = silu(g) * v
    return Wd @ h


def expert_forward(gate_q, gate_sm, up_q, up_sm, down_q, down_sm, x: np.ndarray, fmt: str = "q4b32") -> np.ndarray:
    """One expert on one row, from its packed weights."""
    return swiglu_ffn(*expert_matrices(gate_q, gate_sm, up_q, up_sm, down_q, down_sm, fmt), x)


def _expert_arrays(layer: dict, e: int):
    return (layer["gate_q"][e], layer["gate_sm"][e], layer["up_q"][e], layer["up_sm"][e],
            layer["down_q"][e], layer["down_sm"][e])


# ---------------------------------------------------------------------------
# One layer, one round
# ---------------------------------------------------------------------------

def tail_skip_keep(ids: np.ndarray, resident, skip_rank: int) -> np.ndarray:
    """Which (row, rank) pairs of one round survive the tail skip (Avalon README, results section).

    ids [T, k] are the rows' selections, rank j + 1 at column j; resident[e] says whether expert e
    is resident (missed when False).  A missed expert that every row selecting it ranks at
    skip_rank or below (1-based rank >= skip_rank) is skipped: keep[t, j] is False for each of its
    pairs.  skip_rank <= 0 or resident None: nothing is skipped.
    """
    ids = np.asarray(ids, dtype=np.int64)
    keep = np.ones(ids.shape, dtype=bool)
    if skip_rank <= 0 or resident is None:
        return keep
    T, k = ids.shape
    best = {}  # expert -> its smallest 1-based rank over the round's rows
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            best[e] = min(best.get(e, j + 1), j + 1)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if not bool(resident[e]) and best[e] >= skip_rank:
                keep[t, j] = False
    return keep


def moe_layer(layer: dict, X: np.ndarray, k: int, residual: bool = False, cache=None,
              resident=None, skip_rank: int = 0):
    """One MoE layer over rows X [T, H].

    Each row's selection and routing weights are its own; only the tail skip (resident, skip_rank:
    see tail_skip_keep) looks across the round's rows, to decide which experts are skipped.
    `layer` maps the weight names (router_w, router_b, gate_q, gate_sm, up_q, up_sm, down_q, down_sm)
    to arrays indexable by expert, and optionally "format" to the weight layout ("q4b32" when
    absent).  `cache`, if given, is a dict expert id -> that expert's dequantised matrices
    (expert_matrices) shared across calls on the same layer; missing entries are added.  It only
    saves repeated dequantisation.  Returns (out [T,H] f64, ids [T,k] int64, p [T,k] f64, gaps [T]).
    """
    fmt = layer.get("format") or "q4b32"
    X = np.asarray(X, dtype=np.float64)
    T, H = X.shape
    out = np.zeros((T, H), dtype=np.float64)
    ids = np.zeros((T, k), dtype=np.int64)
    p = np.zeros((T, k), dtype=np.float64)
    gaps = np.zeros(T, dtype=np.float64)
    if cache is None:
        cache = {}
    for t in range(T):
        z = router_logits(layer["router_w"], layer.get("router_b"), X[t])
        ids[t] = select_topk(z, k)
        p[t] = routing_weights(z, ids[t])
        gaps[t] = selection_gap(z, k)
    keep = tail_skip_keep(ids, resident, skip_rank)
    for t in range(T):
        acc = np.zeros(H, dtype=np.float64)
        for j in range(k):
            if not keep[t, j]:
                continue
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = expert_matrices(*_expert_arrays(layer, e), fmt=fmt)
            acc = acc + p[t, j] * swiglu_ffn(*cache[e], X[t])
        out[t] = X[t] + acc if residual else acc
    return out, ids, p, gaps


def moe_round(layers, X: np.ndarray, k: int, residual: bool, resident=None, skip_rank: int = 0):
    """A round over L layers: X^{l+1} = X^l + MoE_l(X^l) with residual, else a single MoE layer.

    resident: None, or per layer a boolean [E] (the tail skip's residency; see tail_skip_keep).
    Returns (out [T,H] f64, ids [L,T,k], p [L,T,k], gaps [L,T]).
    """
    layers = list(layers)
    if not residual and len(layers) != 1:
        raise ValueError("a round without residual has exactly one layer")
    x = np.asarray(X, dtype=np.float64)
    all_ids, all_p, all_gaps = [], [], []
    for l, layer in enumerate(layers):
        res = None if resident is None else resident[l]
        x, ids, p, gaps = moe_layer(layer, x, k, residual, resident=res, skip_rank=skip_rank)
        all_ids.append(ids)
        all_p.append(p)
        all_gaps.append(gaps)
    return x, np.stack(all_ids), np.stack(all_p), np.stack(all_gaps)


# ---------------------------------------------------------------------------
# Worklist: counting sort of (row, rank) pairs by expert
# ---------------------------------------------------------------------------

def build_worklist(ids: np.ndarray, keep=None):
    """Group the T*k (row t, rank j) pairs by expert.

    keep: None, or a boolean [T, k] (tail_skip_keep); pairs with keep False are left out, and an
    expert none of whose pairs is kept is not in the union.
    Returns (uniq, offs, pairs):
      uniq  : the union of the rows' selected experts (of kept pairs), ascending;
      offs  : exclusive prefix sum of how many kept pairs each unique expert has (len n_unique + 1);
      pairs : [n_kept, 2] (t, j), grouped by expert in uniq order, t ascending within an expert.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    if keep is None:
        keep = np.ones((T, k), dtype=bool)
    E = int(ids.max()) + 1 if ids.size else 0
    count = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for j in range(k):
            if keep[t, j]:
                count[ids[t, j]] += 1
    uniq = np.array([e for e in range(E) if count[e] > 0], dtype=np.int64)
    offs = np.zeros(len(uniq) + 1, dtype=np.int64)
    for u, e in enumerate(uniq):
        offs[u + 1] = offs[u] + count[e]
    pairs = np.zeros((int(offs[-1]), 2), dtype=np.int64)
    fill = offs[:-1].copy()
    pos = {int(e): u for u, e in enumerate(uniq)}
    for t in range(T):
        for j in range(k):
            if not keep[t, j]:
                continue
            u = pos[int(ids[t, j])]
            pairs[fill[u]] = (t, j)
            fill[u] += 1
    return uniq, offs, pairs
