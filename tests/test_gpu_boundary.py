"""The C ABI's boundary cases on the GPU: `hidden` passed as `out`, per-layer statistics, reduction
lengths without an exact lane split, and the measurement calls (needs an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from moe_helpers import GpuRound, assert_close, check_layer_round, oracle_view, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def verify():
    cfg = synth.config("verify")
    layer = synth.make_layer(cfg, seed=0, layer=0, device=DEV)
    return cfg, layer, oracle_view(layer)


def run_in_place(g, X, k):
    """One round with hidden == out: the input buffer is overwritten with the result."""
    L = len(g.layers)
    T = X.shape[0]
    buf = X.clone()
    ids = torch.full((L, T, k), -1, dtype=torch.int32, device=DEV)
    rw = torch.zeros((L, T, k), dtype=torch.float32, device=DEV)
    g.h.run(buf, k, buf, ids, rw)
    torch.cuda.synchronize()
    return buf.cpu().numpy(), ids.cpu().numpy(), rw.cpu().numpy()


@pytest.mark.parametrize("mode", ["eager", "graph", "exact"])
def test_hidden_may_be_out(verify, mode):
    """out = MoE(x) written over x itself, for every selection path (T = 1, 3, 8, 40)."""
    cfg, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=64, use_graph=(mode == "graph"), exact=(mode == "exact"))
    for T in (1, 3, 8, 40):
        say(f"case in place {mode} T={T}")
        X = synth.make_activations(cfg, T, seed=12, round_idx=T, device=DEV)
        got, ids, rw = run_in_place(g, X, cfg.k)
        ref, rids, rp, _ = oracle.moe_round([view], X.cpu().numpy(), cfg.k, residual=False)
        assert np.array_equal(ids, rids)
        np.testing.assert_allclose(rw, rp, rtol=2e-6, atol=1e-7)
        assert_close(got, ref, f"in place {mode} T={T}")
    g.close()


def test_hidden_may_be_out_in_a_stack_and_prefill():
    """A 3-layer residual stack (eager and graph) and a prefill round, in place."""
    cfg = synth.config("deep").replace(L=3, E=64)
    layers = [synth.make_layer(cfg, seed=2, layer=l, device=DEV) for l in range(cfg.L)]
    views = [oracle_view(l) for l in layers]
    for use_graph in (False, True):
        g = GpuRound(layers, cfg, max_rows=80, use_graph=use_graph)
        for T in (3, 80):
            say(f"case in place stack graph={use_graph} T={T}")
            X = synth.make_activations(cfg, T, seed=13, round_idx=T, device=DEV)
            got, ids, _ = run_in_place(g, X, cfg.k)
            ref, rids, _, _ = oracle.moe_round(views, X.cpu().numpy(), cfg.k, residual=True)
            assert np.array_equal(ids, rids)
            Xh = X.cpu().numpy()
            assert_close(got - Xh, ref - Xh, f"in place stack T={T}")
        g.close()


def test_partly_overlapping_buffers_are_refused(verify):
    from verify_router_gemv_amd.binding import MoeRoundError
    cfg, layer, _ = verify
    g = GpuRound([layer], cfg, max_rows=8)
    buf = torch.zeros((9, cfg.H), device=DEV)
    with pytest.raises(MoeRoundError):
        g.h.run(buf[0:8], cfg.k, buf[1:9])
    g.close()


def test_last_stats_match_the_metric_bytes(verify):
    """Per-layer unique experts and metric bytes of the last run: the oracle's union size and the
    generator's byte formula (codes + scales of each unique expert, plus the input and output rows)."""
    cfg, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=8)
    for T in (1, 3, 8):
        X = synth.make_activations(cfg, T, seed=14, round_idx=T, device=DEV)
        g.run(X)
        st, nu, mb = g.h.last_stats()
        _, rids, _, _ = oracle.moe_round([view], X.cpu().numpy(), cfg.k, residual=False)
        n_union = len(set(rids[0].ravel().tolist()))
        say(f"case last_stats T={T}: n_unique {nu[0]} metric bytes {mb[0]}")
        assert st.n_layers == 1 and st.rows == T and st.top_k == cfg.k
        assert st.expert_bytes == cfg.expert_bytes()
        assert nu == [n_union]
        assert mb == [synth.inputs.metric_bytes(cfg, n_union, T)]
        assert st.metric_bytes == mb[0]
    g.close()
    cfg4 = synth.config("deep").replace(L=4, E=64, fmt="q4s256")
    layers = [synth.make_layer(cfg4, seed=3, layer=l, device=DEV) for l in range(cfg4.L)]
    g = GpuRound(layers, cfg4, max_rows=3)
    X = synth.make_activations(cfg4, 3, seed=15, round_idx=0, device=DEV)
    g.run(X)
    st, nu, mb = g.h.last_stats()
    assert nu == g.h.last_unique()
    assert mb == [synth.inputs.metric_bytes(cfg4, n, 3) for n in nu]
    assert st.metric_bytes == sum(mb) and st.expert_bytes == cfg4.expert_bytes()
    g.close()


@pytest.mark.parametrize("H,I", [(2048, 64), (2048, 96), (1280, 640), (768, 32), (2304, 160)])
def test_reductions_without_an_exact_lane_split(H, I):
    """Padded lane splits (spare block slots masked) against the oracle, T = 1, 3, 8, 20."""
    cfg = synth.ShapeConfig("padded", H=H, E=24, k=4, I=I, T=(1, 3, 8, 20), zipf_s=0.5)
    layer = synth.make_layer(cfg, seed=6, layer=0, device=DEV)
    view = oracle_view(layer)
    g = GpuRound([layer], cfg, max_rows=32)
    for T in cfg.T:
        say(f"case padded split H={H} I={I} T={T}")
        X = synth.make_activations(cfg, T, seed=16, round_idx=T, device=DEV)
        check_layer_round(g, [view], X, cfg.k, f"padded H={H} I={I} T={T}")
    g.close()


def test_floor_and_stream_read_leave_results_alone(verify):
    """The measurement calls leave the round alone: its outputs are the same before and after them;
    the launch control's store variant writes exactly its blocks' indices."""
    cfg, layer, view = verify
    g = GpuRound([layer], cfg, max_rows=8)
    X = synth.make_activations(cfg, 3, seed=17, round_idx=0, device=DEV)
    out1, ids1, _, _ = g.run(X)
    say("case floor + stream read")
    g.h.floor()
    buf = torch.randn(1 << 20, device=DEV)
    g.h.stream_read(buf)
    say("case empty launches (plain, storing, sleeping)")
    flags = torch.full((300,), -1, dtype=torch.int32, device=DEV)
    g.h.empty_launches(64, 3)
    g.h.empty_launches(256, 2, 1, flags)
    torch.cuda.synchronize()
    assert flags[:256].cpu().tolist() == list(range(256))
    assert (flags[256:] == -1).all().item()
    out2, ids2, _, _ = g.run(X)
    assert np.array_equal(ids1, ids2)
    np.testing.assert_allclose(out1, out2, rtol=1e-5, atol=1e-6)
    g.close()
