"""Experts read through a per-(layer, expert) pointer table, some of them from pinned host memory
read in place, and the tail skip of missed experts (needs an MI355X).

The table and the residency bits are ingress: their contents are read by each round on the GPU.
The oracle applies the tail skip from its own reading of the rule (oracle.tail_skip_keep)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from moe_helpers import DequantCache, assert_close, oracle_view, say
from verify_router_gemv_amd import MoeRound, binding

pytestmark = pytest.mark.gpu

DEV = "cuda"
FIELDS = binding.EXPERT_FIELDS
SKIP = 7          # the rank the Avalon README's results section quotes
RESIDENT = 0.25   # share of experts resident in device memory (the rest: host tier)


class Tier:
    """One layer's experts placed by residency: resident ones stay in the layer's device tensors,
    missed ones are copied into pinned host tensors; table rows point at wherever each one sits."""

    def __init__(self, layer, resident):
        self.resident = np.asarray(resident, dtype=bool)
        missed = np.flatnonzero(~self.resident)
        self.host = {}
        for f in FIELDS:
            src = getattr(layer, f)
            h = torch.empty((len(missed),) + tuple(src.shape[1:]), dtype=src.dtype, pin_memory=True)
            if len(missed):
                h.copy_(src[torch.as_tensor(missed, device=src.device)].cpu())
            self.host[f] = h
        slot = {int(e): i for i, e in enumerate(missed)}
        self.entries = []
        for e in range(len(self.resident)):
            if self.resident[e]:
                self.entries.append({f: getattr(layer, f)[e] for f in FIELDS})
            else:
                self.entries.append({f: self.host[f][slot[e]] for f in FIELDS})


def make_table(tiers, cfg):
    return binding.make_expert_table([t.entries for t in tiers], cfg.H, cfg.I, cfg.fmt)


def router_only(layer):
    return {"router_w": layer.router_w, "router_b": layer.router_b}


@pytest.fixture(scope="module")
def verify():
    cfg = synth.config("verify")
    layer = synth.make_layer(cfg, seed=0, layer=0, device=DEV)
    view = oracle_view(layer)
    return cfg, layer, view, DequantCache(view)


def run(h, X, k, L=1):
    T = X.shape[0]
    out = torch.empty_like(X)
    ids = torch.full((L, T, k), -1, dtype=torch.int32, device=DEV)
    rw = torch.zeros((L, T, k), dtype=torch.float32, device=DEV)
    h.run(X, k, out, ids, rw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), rw.cpu().numpy()


def oracle_layer(view, cache, Xh, k, resident=None, rank=0):
    need = set()
    for t in range(Xh.shape[0]):
        need.update(oracle.select_topk(oracle.router_logits(view["router_w"], view["router_b"], Xh[t]), k).tolist())
    cache.ensure(need)
    return oracle.moe_layer(view, Xh, k, cache=cache, resident=resident, skip_rank=rank)


def check_round(h, view, cache, X, k, what, resident=None, rank=0):
    """ids bit-exact, worklist bit-exact (skipped experts and their pairs left out), skipped count,
    routing weights and output against the oracle. Returns the number of skipped experts."""
    out, ids, rw = run(h, X, k)
    Xh = X.cpu().numpy()
    ref, rids, rp, _ = oracle_layer(view, cache, Xh, k, resident, rank)
    assert np.array_equal(ids[0], rids), f"{what}: ids differ"
    np.testing.assert_allclose(rw[0], rp, rtol=2e-6, atol=1e-7, err_msg=f"{what}: routing weights")
    keep = oracle.tail_skip_keep(rids, resident, rank)
    uniq, offs, pairs = h.worklist(0)
    eu, eo, ep = oracle.build_worklist(rids, keep)
    assert uniq == eu.tolist(), f"{what}: uniq"
    assert offs == eo.tolist(), f"{what}: offs"
    assert pairs == [tuple(p) for p in ep.tolist()], f"{what}: pairs"
    skipped = len(set(rids[~keep].tolist()))
    st, nu, _ = h.last_stats()
    assert st.skipped == skipped and nu[0] == len(eu), f"{what}: stats"
    assert_close(out, ref, what)
    return skipped


ROUNDS = (1, 2, 3, 4, 5, 8, 16, 40)   # one-row, fused pairs, selection kernel, staged, split top-k


@pytest.mark.parametrize("exact", [False, True])
def test_table_of_device_experts_equals_the_contiguous_arrays(verify, exact):
    """Every expert resident, the table pointing into the layer's own tensors: the same kernels over
    the same bytes; exact mode is bitwise equal to the contiguous layout."""
    cfg, layer, view, cache = verify
    tier = Tier(layer, np.ones(cfg.E, dtype=bool))
    table = make_table([tier], cfg)
    ht = MoeRound([router_only(layer)], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=64, exact=exact, expert_table=True)
    ht.bind_experts(table)
    hc = MoeRound([layer], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=64, exact=exact)
    for T in ROUNDS:
        say(f"case table=contiguous exact={exact} T={T}")
        X = synth.make_activations(cfg, T, seed=21, round_idx=T, device=DEV)
        a, ia, _ = run(ht, X, cfg.k)
        b, ib, _ = run(hc, X, cfg.k)
        assert np.array_equal(ia, ib)
        if exact:
            assert np.array_equal(a, b), f"T={T}"
        else:
            assert_close(a, b.astype(np.float64), f"table vs contiguous T={T}")
        check_round(ht, view, cache, X, cfg.k, f"table T={T}")
    ht.close()
    hc.close()


@pytest.mark.parametrize("use_graph", [True, False])
def test_host_tier_read_in_place(verify, use_graph):
    """Three quarters of the experts in pinned host memory, read by the kernels over the host link."""
    cfg, layer, view, cache = verify
    res = synth.make_residency(cfg, RESIDENT, seed=0, layer=0)
    tier = Tier(layer, res)
    table = make_table([tier], cfg)
    h = MoeRound([router_only(layer)], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=64, use_graph=use_graph,
                 expert_table=True)
    h.bind_experts(table)
    for T in ROUNDS:
        say(f"case host tier graph={use_graph} T={T}")
        X = synth.make_activations(cfg, T, seed=22, round_idx=T, device=DEV)
        check_round(h, view, cache, X, cfg.k, f"host tier T={T}")
    h.close()


@pytest.mark.parametrize("mode", ["contiguous", "table", "table-exact", "table-eager", "table-mfma"])
def test_tail_skip_parity(verify, mode):
    """The tail skip at rank 7 over 25% resident experts: ids, worklist and skipped count bit-exact,
    output within tolerance of the oracle's skipped round."""
    cfg, layer, view, cache = verify
    res = synth.make_residency(cfg, RESIDENT, seed=0, layer=0)
    bits = binding.residency_bits(res[None, :])
    kw = dict(max_rows=64, tail_skip_rank=SKIP, exact=mode == "table-exact", use_graph=mode != "table-eager",
              mfma_min_rows=1 if mode == "table-mfma" else 0)
    if mode == "contiguous":
        h = MoeRound([layer], cfg.H, cfg.I, cfg.E, cfg.k, **kw)
        h.bind_experts(None, bits)
    else:
        tier = Tier(layer, res)
        table = make_table([tier], cfg)
        h = MoeRound([router_only(layer)], cfg.H, cfg.I, cfg.E, cfg.k, expert_table=True, **kw)
        h.bind_experts(table, bits)
    total = 0
    for T in ROUNDS:
        for r in range(3):
            say(f"case tail skip {mode} T={T} input {r}")
            X = synth.make_activations(cfg, T, seed=23 + r, round_idx=T, device=DEV)
            total += check_round(h, view, cache, X, cfg.k, f"skip {mode} T={T}", res, SKIP)
    say(f"  {mode}: {total} experts skipped over {3 * len(ROUNDS)} rounds")
    assert total > 0, "no round skipped anything: the test would not exercise the skip"
    h.close()


@pytest.mark.parametrize("rank", [1, 6, 9])
def test_tail_skip_other_ranks(verify, rank):
    """Rank 1 skips every missed expert (a row may keep nothing); 9 is past k and skips nothing."""
    cfg, layer, view, cache = verify
    res = synth.make_residency(cfg, RESIDENT, seed=0, layer=0)
    h = MoeRound([layer], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=64, tail_skip_rank=rank)
    h.bind_experts(None, binding.residency_bits(res[None, :]))
    for T in (1, 3, 8, 40):
        say(f"case tail skip rank {rank} T={T}")
        X = synth.make_activations(cfg, T, seed=24, round_idx=T, device=DEV)
        n = check_round(h, view, cache, X, cfg.k, f"skip rank {rank} T={T}", res, rank)
        if rank == 9:
            assert n == 0
    h.close()


def test_ingress_contents_and_rebinding(verify):
    """The table and residency contents are read by each round: rewriting them in place (no call to
    the library) or binding other arrays changes the next replay of the captured graph."""
    cfg, layer, view, cache = verify
    res = synth.make_residency(cfg, RESIDENT, seed=0, layer=0)
    tier = Tier(layer, res)
    table = make_table([tier], cfg)
    bits = binding.residency_bits(res[None, :])
    h = MoeRound([router_only(layer)], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=8, expert_table=True,
                 tail_skip_rank=SKIP)
    h.bind_experts(table, bits)
    X = synth.make_activations(cfg, 3, seed=25, round_idx=0, device=DEV)
    check_round(h, view, cache, X, cfg.k, "first binding", res, SKIP)
    # a permuted placement: expert e's entry now names expert perm[e]'s matrices
    perm = np.random.default_rng(3).permutation(cfg.E)
    pview = {**view, **{f: PermutedExperts(view[f], perm) for f in FIELDS}}
    pcache = DequantCache(pview)
    table2 = table[:, torch.as_tensor(perm, device=DEV)].contiguous()
    h.bind_experts(table2, bits)
    check_round(h, pview, pcache, X, cfg.k, "rebound table", res, SKIP)
    table.copy_(table2)                 # in place, then bind the first arrays again: same contents
    h.bind_experts(table, bits)
    check_round(h, pview, pcache, X, cfg.k, "rewritten table", res, SKIP)
    none = np.zeros(cfg.E, dtype=bool)  # every expert missed: rewrite the bits in place
    bits.copy_(binding.residency_bits(none[None, :]))
    check_round(h, pview, pcache, X, cfg.k, "rewritten residency", none, SKIP)
    h.close()


class PermutedExperts:
    def __init__(self, base, perm):
        self.base, self.perm = base, perm

    def __getitem__(self, e):
        return self.base[int(self.perm[int(e)])]


@pytest.mark.parametrize("use_graph", [True, False])
def test_stack_with_host_tier_and_tail_skip(use_graph):
    """Four layers of the 512-expert, top-10 stack (residual), the hottest quarter of each layer
    resident, the rest in pinned host memory, tail skip at rank 7: every layer's ids and the
    output against the oracle on an input clear of selection ties."""
    cfg = synth.config("deep").replace(L=4)
    layers = [synth.make_layer(cfg, seed=0, layer=l, device=DEV) for l in range(cfg.L)]
    res = [synth.make_residency(cfg, RESIDENT, seed=0, layer=l) for l in range(cfg.L)]
    tiers = [Tier(layers[l], res[l]) for l in range(cfg.L)]
    table = make_table(tiers, cfg)
    bits = binding.residency_bits(np.stack(res))
    h = MoeRound([router_only(l) for l in layers], cfg.H, cfg.I, cfg.E, cfg.k, max_rows=3, residual=True,
                 use_graph=use_graph, expert_table=True, tail_skip_rank=SKIP)
    h.bind_experts(table, bits)
    views = [oracle_view(l) for l in layers]
    checked = 0
    for r in range(8):
        X = synth.make_activations(cfg, 3, seed=26, round_idx=r, device=DEV)
        ref, rids, rp, gaps = oracle.moe_round(views, X.cpu().numpy(), cfg.k, True, resident=res, skip_rank=SKIP)
        if gaps.min() < 1e-5:
            say(f"  input {r}: selection gap {gaps.min():.2e}, next input")
            continue
        say(f"case stack host tier + skip graph={use_graph} input {r}")
        out, ids, rw = run(h, X, cfg.k, cfg.L)
        skipped = 0
        for l in range(cfg.L):
            assert np.array_equal(ids[l], rids[l]), f"layer {l}"
            skipped += len(set(rids[l][~oracle.tail_skip_keep(rids[l], res[l], SKIP)].tolist()))
        assert h.last_stats()[0].skipped == skipped
        Xh = X.cpu().numpy()
        assert_close(out - Xh, ref - Xh, f"stack input {r} (MoE part)")
        checked += 1
        if checked == 2:
            break
    assert checked >= 1, "no well-conditioned input among 8"
    h.close()
