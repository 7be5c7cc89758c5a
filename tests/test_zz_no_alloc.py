"""moe_round_run_noalloc (scratch in the library's fixed device array, nothing allocated) against
moe_round_run on a handle, through the C ABI, two calls in a row with the second one smaller
(needs an MI355X)."""
import numpy as np
import pytest
import torch

import synth
from moe_helpers import GpuRound, assert_close, say
from verify_router_gemv_amd.binding import run_noalloc

pytestmark = pytest.mark.gpu

DEV = "cuda"


def noalloc(layers, cfg, X, k, **kw):
    L, T = len(layers), X.shape[0]
    out = torch.full_like(X, float("nan"))
    ids = torch.full((L, T, k), -1, dtype=torch.int32, device=DEV)
    rw = torch.full((L, T, k), float("nan"), dtype=torch.float32, device=DEV)
    run_noalloc(layers, cfg.H, cfg.I, cfg.E, kw.pop("k_max", cfg.k), X, k, out, ids, rw,
                residual=cfg.residual, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), rw.cpu().numpy()


def compare(g, layers, cfg, Ts, what, exact=False, **kw):
    for T in Ts:   # consecutive calls, each smaller than the one before
        say(f"case no-alloc {what} T={T}")
        X = synth.make_activations(cfg, T, seed=40, round_idx=T, device=DEV)
        ref, rids, rrw, _ = g.run(X)
        got, ids, rw = noalloc(layers, cfg, X, cfg.k, max_rows=max(Ts), exact=exact, **kw)
        assert np.array_equal(ids, rids), f"{what} T={T}: ids"
        # layer 0 sees the same input bits on both paths: its routing weights agree bitwise; later
        # layers' inputs differ at fp32 rounding (atomic order of the combine), so to 2e-6
        assert np.array_equal(rw[0], rrw[0]), f"{what} T={T}: routing weights"
        np.testing.assert_allclose(rw, rrw, rtol=2e-6, atol=1e-7, err_msg=f"{what} T={T}: routing weights")
        if exact:
            assert np.array_equal(got, ref), f"{what} T={T}: exact-mode outputs differ"
        elif cfg.residual:
            Xh = X.cpu().numpy()
            assert_close(got - Xh, ref - Xh, f"no-alloc {what} T={T}")
        else:
            assert_close(got, ref, f"no-alloc {what} T={T}")


@pytest.fixture(scope="module")
def verify():
    cfg = synth.config("verify")
    return cfg, synth.make_layer(cfg, seed=0, layer=0, device=DEV)


def test_noalloc_matches_the_handle_verify(verify):
    cfg, layer = verify
    g = GpuRound([layer], cfg, max_rows=8, use_graph=False)
    compare(g, [layer], cfg, (8, 3), "verify")
    compare(g, [layer], cfg, (5, 1), "verify")
    g.close()


def test_noalloc_matches_the_handle_exact_and_wide(verify):
    cfg, layer = verify
    g = GpuRound([layer], cfg, max_rows=64, use_graph=False, exact=True)
    compare(g, [layer], cfg, (40, 3), "exact", exact=True)
    g.close()
    g = GpuRound([layer], cfg, max_rows=64, use_graph=False)
    compare(g, [layer], cfg, (64, 16), "wide")
    g.close()


def test_noalloc_matches_the_handle_stack():
    cfg = synth.config("deep").replace(L=4, E=64)
    layers = [synth.make_layer(cfg, seed=4, layer=l, device=DEV) for l in range(cfg.L)]
    g = GpuRound(layers, cfg, max_rows=3, use_graph=False)
    compare(g, layers, cfg, (3, 1), "stack")
    g.close()


def test_noalloc_refuses_an_oversized_round(verify):
    from verify_router_gemv_amd.binding import MoeRoundError
    cfg = synth.ShapeConfig("big", H=8192, E=64, k=16, I=2048)
    layer = synth.make_layer(cfg.replace(E=16), seed=0, layer=0, device=DEV)
    X = torch.zeros((64, cfg.H), device=DEV)
    out = torch.zeros_like(X)
    with pytest.raises(MoeRoundError) as ei:
        run_noalloc([layer], cfg.H, cfg.I, 16, 16, X, 16, out, exact=True)
    assert ei.value.status == -2
