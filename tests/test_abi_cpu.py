"""The C ABI library loads and exports every declared symbol; host-side validation (no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe_round.h")


@pytest.fixture(scope="module")
def lib():
    from verify_router_gemv_amd import binding, build
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return binding.load()


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MOE_ROUND_API\s+[\w\s\*]+?\b(moe_round_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared()
    assert "moe_round_init" in names and "moe_round_run" in names and "moe_round_destroy" in names
    assert len(names) == 19
    assert {"moe_round_last_stats", "moe_round_floor", "moe_round_stream_read"} <= set(names)


def test_library_exports_exactly_the_declared_symbols(lib):
    from verify_router_gemv_amd import binding
    for name in declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T moe_round_" in l)
    assert exported == declared()


def cfg(**kw):
    from verify_router_gemv_amd import binding
    base = dict(H=2048, I=512, E=256, top_k_max=8, n_layers=1, max_rows=8, residual=False, use_graph=True)
    base.update(kw)
    c = binding.make_config(base["H"], base["I"], base["E"], base["top_k_max"], base["n_layers"],
                            base["max_rows"], base["residual"], base["use_graph"])
    for k, v in kw.items():
        if k.startswith("raw_"):
            setattr(c, k[4:], v)
    return c


@pytest.mark.parametrize("kw", [
    dict(H=256, I=128, E=8, top_k_max=2, max_rows=1),
    dict(H=2048, I=768, E=128, top_k_max=8, max_rows=1),
    dict(H=2048, I=512, E=256, top_k_max=8, max_rows=8),
    dict(H=2048, I=512, E=512, top_k_max=10, n_layers=48, max_rows=3, residual=True),
    dict(H=2048, I=512, E=256, top_k_max=8, max_rows=64),
    dict(H=768, I=384, E=40, top_k_max=5, max_rows=16),
    dict(H=8192, I=2048, E=512, top_k_max=16, max_rows=64),
    dict(H=2048, I=512, E=256, top_k_max=8, max_rows=8, raw_fused_max_rows=-1, raw_rows_per_item=1,
         raw_mfma_min_rows=-1),
    dict(H=2048, I=512, E=256, top_k_max=8, max_rows=64, raw_fused_max_rows=15, raw_rows_per_item=64,
         raw_mfma_min_rows=16),
    dict(H=2048, I=512, E=256, top_k_max=8, max_rows=8, raw_weight_format=1),
    dict(H=2048, I=768, E=128, top_k_max=8, max_rows=1, raw_weight_format=1),
    dict(H=768, I=256, E=40, top_k_max=5, max_rows=16, raw_weight_format=1),
    dict(H=2048, I=512, E=256, top_k_max=8, max_rows=65),        # prefill rounds from 65 rows
    dict(H=2048, I=512, E=256, top_k_max=8, max_rows=4096),
    dict(H=768, I=384, E=40, top_k_max=5, max_rows=1000),
    dict(H=2048, I=512, E=512, top_k_max=10, n_layers=4, max_rows=16384, residual=True),
    dict(H=2048, I=512, E=256, top_k_max=8, max_rows=4096, raw_weight_format=1),  # prefill, 4.5-bit
    # reduction lengths with no exact lane split: the spare block slots are masked
    dict(H=1280, I=512, E=64, top_k_max=8, max_rows=8),      # H/32 = 40: 16 lanes x 3 blocks
    dict(H=2048, I=640, E=64, top_k_max=8, max_rows=8),      # I/32 = 20: 8 lanes x 3 blocks
    dict(H=2048, I=96, E=64, top_k_max=8, max_rows=8),       # I/32 = 3
    dict(H=2048, I=64, E=256, top_k_max=8, max_rows=8),      # I = 512 / 8: one tensor-parallel shard
    dict(H=2048, I=32, E=16, top_k_max=4, max_rows=8),
    dict(H=2048, I=160, E=16, top_k_max=4, max_rows=8),
    dict(H=2304, I=8160, E=8, top_k_max=2, max_rows=4),      # H/32 = 72, I/32 = 255
    dict(H=2048, I=8192, E=8, top_k_max=2, max_rows=4),
    # the expert table and the tail skip (decode/verify rounds)
    dict(H=2048, I=512, E=256, top_k_max=8, max_rows=8, raw_expert_table=1),
    dict(H=2048, I=512, E=256, top_k_max=8, max_rows=8, raw_tail_skip_rank=7),
    dict(H=2048, I=512, E=512, top_k_max=10, n_layers=48, max_rows=3, residual=True, raw_expert_table=1,
         raw_tail_skip_rank=7),
    dict(H=2048, I=512, E=256, top_k_max=16, max_rows=64, raw_tail_skip_rank=17),   # past k: never skips
])
def test_supported_configs_validate(lib, kw):
    from verify_router_gemv_amd import binding
    assert binding.validate_config(cfg(**kw)) == 0


@pytest.mark.parametrize("kw,expect", [
    (dict(raw_abi_version=1), -1),     # the configuration struct of ABI 1 lacks `prefetch`
    (dict(raw_abi_version=2), -1),     # ... of ABI 2 lacks `expert_table` and `tail_skip_rank`
    (dict(raw_abi_version=4), -1),
    (dict(raw_expert_table=2), -1),
    (dict(raw_tail_skip_rank=-1), -1),
    (dict(raw_tail_skip_rank=18), -1),
    (dict(max_rows=100, raw_expert_table=1), -2),   # prefill rounds read the contiguous arrays
    (dict(max_rows=100, raw_tail_skip_rank=7), -2),
    (dict(raw_prefetch=2), -1),
    (dict(raw_prefetch=-1), -1),
    (dict(raw_record_layers=2), -1),
    (dict(H=0), -1),
    (dict(I=-32), -1),
    (dict(E=0), -1),
    (dict(top_k_max=0), -1),
    (dict(max_rows=0), -1),
    (dict(n_layers=2, residual=False), -1),
    (dict(E=4, top_k_max=8), -1),
    (dict(raw_use_graph=2), -1),
    (dict(raw_residual=3), -1),
    (dict(raw_fused_max_rows=16), -1),
    (dict(raw_fused_max_rows=-2), -1),
    (dict(raw_rows_per_item=-1), -1),
    (dict(raw_rows_per_item=65), -1),
    (dict(raw_mfma_min_rows=-3), -1),
    (dict(raw_exact=2), -1),
    (dict(raw_weight_format=2), -1),
    (dict(raw_weight_format=-1), -1),
    (dict(I=384, raw_weight_format=1), -2),   # super-blocks need I a multiple of 256
    (dict(H=256, I=128, E=8, top_k_max=2, raw_weight_format=1), -2),
    (dict(max_rows=16385), -2),
    (dict(E=513, top_k_max=8), -2),
    (dict(top_k_max=17, E=256), -2),
    (dict(H=2080), -2),          # not a multiple of 256
    (dict(I=8224), -2),          # I/32 = 257: more than 256 blocks per row
    (dict(I=48), -2),            # not a multiple of 32
    (dict(I=96, max_rows=100), -2),   # prefill needs I a multiple of 128
    (dict(H=16384), -2),
])
def test_unsupported_or_invalid_configs_are_refused(lib, kw, expect):
    from verify_router_gemv_amd import binding
    assert binding.validate_config(cfg(**kw)) == expect


def test_null_and_bad_arguments_are_refused_before_any_gpu_call(lib):
    from verify_router_gemv_amd import binding
    h = ctypes.c_void_p()
    c = cfg()
    assert lib.moe_round_init(ctypes.byref(c), None, None, ctypes.byref(h)) == -1
    assert lib.moe_round_init(None, None, None, ctypes.byref(h)) == -1
    w = (binding.LayerWeights * 1)()
    assert lib.moe_round_init(ctypes.byref(c), w, None, ctypes.byref(h)) == -1     # null weight pointers
    w[0] = binding.LayerWeights(*([0x1000] * 8))
    w[0].gate_q = 0x1008                                                            # misaligned codes
    assert lib.moe_round_init(ctypes.byref(c), w, None, ctypes.byref(h)) == -1
    bad = cfg(max_rows=16385)
    assert lib.moe_round_init(ctypes.byref(bad), w, None, ctypes.byref(h)) == -2
    assert lib.moe_round_run(None, None, 1, 1, None, None, None, None) == -1
    assert lib.moe_round_worklist(None, 0, None, None, None, None) == -1
    assert lib.moe_round_last_unique(None, None) == -1
    assert lib.moe_round_last_hip_error(None) == 0
    assert lib.moe_round_profile(None, 1) == -1
    n = ctypes.c_int32()
    ms = (ctypes.c_double * 5)()
    assert lib.moe_round_profile_read(None, ms, ctypes.byref(n)) == -1
    lib.moe_round_destroy(None)


def test_noalloc_checks_happen_before_any_gpu_call(lib):
    """moe_round_run_noalloc refuses bad arguments and rounds whose scratch exceeds its fixed array
    on the host, and an empty round is a no-op, all without touching a GPU."""
    from verify_router_gemv_amd import binding
    w = (binding.LayerWeights * 1)(binding.LayerWeights(*([0x100000] * 8)))
    herr = ctypes.c_int32(7)
    big = cfg(H=8192, I=2048, E=16, top_k_max=16, max_rows=64)
    big.exact = 1                               # ybuf alone: 64 * 16 * 8192 * 4 B = 32 MiB
    assert lib.moe_round_run_noalloc(ctypes.byref(big), w, 0x200000, 64, 16, 0x4000000, None, None, None,
                                     ctypes.byref(herr)) == -2
    assert herr.value == 0
    ok = cfg()
    assert lib.moe_round_run_noalloc(ctypes.byref(ok), w, None, 0, 8, None, None, None, None, None) == 0
    assert lib.moe_round_run_noalloc(ctypes.byref(ok), w, 0x200000, 9, 8, 0x4000000, None, None, None, None) == -1
    assert lib.moe_round_run_noalloc(None, w, 0x200000, 1, 8, 0x4000000, None, None, None, None) == -1
    assert lib.moe_round_run_noalloc(ctypes.byref(ok), None, 0x200000, 1, 8, 0x4000000, None, None, None, None) == -1
    pf = cfg(max_rows=100)
    assert lib.moe_round_run_noalloc(ctypes.byref(pf), w, 0x200000, 100, 8, 0x4000000, None, None, None, None) == -2


def test_table_mode_checks_happen_before_any_gpu_call(lib):
    """Table mode takes only the routers from the layers; the no-allocation entry point refuses the
    table and the tail skip (nothing to bind them to); null arguments are refused."""
    from verify_router_gemv_amd import binding
    h = ctypes.c_void_p()
    c = cfg(raw_expert_table=1)
    full = (binding.LayerWeights * 1)(binding.LayerWeights(*([0x100000] * 8)))
    assert lib.moe_round_init(ctypes.byref(c), full, None, ctypes.byref(h)) == -1   # expert pointers set
    router_only = (binding.LayerWeights * 1)(binding.LayerWeights(0x100000, None, *([None] * 6)))
    assert lib.moe_round_run_noalloc(ctypes.byref(c), router_only, 0x200000, 1, 8, 0x4000000, None, None, None,
                                     None) == -2
    skip = cfg(raw_tail_skip_rank=7)
    assert lib.moe_round_run_noalloc(ctypes.byref(skip), full, 0x200000, 1, 8, 0x4000000, None, None, None,
                                     None) == -2
    assert lib.moe_round_run_noalloc(ctypes.byref(c), full, 0x200000, 1, 8, 0x4000000, None, None, None,
                                     None) == -1
    assert lib.moe_round_bind_experts(None, 0x100000, None) == -1
    dev = ctypes.c_void_p()
    assert lib.moe_round_host_tier_pointer(None, ctypes.byref(dev)) == -1
    assert lib.moe_round_host_tier_pointer(0x100000, None) == -1


def test_residency_words_pack_bit_e_of_word_e_over_32():
    from verify_router_gemv_amd import binding
    res = torch.zeros(2, 70, dtype=torch.bool)
    res[0, [0, 31, 32, 69]] = True
    res[1, 5] = True
    w = binding.residency_bits(res.numpy(), device="cpu").view(torch.uint32).to(torch.int64) & 0xFFFFFFFF
    assert w.shape == (2, 3)
    assert w[0].tolist() == [1 | (1 << 31), 1, 1 << 5]
    assert w[1].tolist() == [1 << 5, 0, 0]


def test_new_entry_points_refuse_null_handles(lib):
    assert lib.moe_round_last_stats(None, None, None, None) == -1
    assert lib.moe_round_floor(None) == -1
    assert lib.moe_round_layer_input(None, 0, None) == -1
    assert lib.moe_round_stream_read(None, None, 16) == -1
    assert lib.moe_round_empty_launches(None, 1, 1, 0, None) == -1


def test_rejected_layers_keep_the_old_weights_referenced(lib, monkeypatch):
    """A run with new layers that the binding or the library rejects leaves the handle's Python
    references to the previous weight tensors in place (the library keeps reading them)."""
    from verify_router_gemv_amd import binding
    E, H, I = 4, 256, 128
    h = binding.MoeRound.__new__(binding.MoeRound)
    h.lib, h.h, h.H, h.I, h.E, h.L, h.weight_format, h.expert_table = lib, None, H, I, E, 1, 0, False
    old = [object()]
    h._layers, h._wt = old, "old-array"
    host_layer = dict(router_w=torch.zeros(E, H), router_b=None,
                      gate_q=torch.zeros(E, I, H // 2, dtype=torch.uint8),
                      gate_sm=torch.zeros(E, I, H // 32, dtype=torch.int32),
                      up_q=torch.zeros(E, I, H // 2, dtype=torch.uint8),
                      up_sm=torch.zeros(E, I, H // 32, dtype=torch.int32),
                      down_q=torch.zeros(E, H, I // 2, dtype=torch.uint8),
                      down_sm=torch.zeros(E, H, I // 32, dtype=torch.int32))
    x = torch.zeros(1, H)
    with pytest.raises(ValueError):          # the binding refuses host tensors
        h.run(x, 1, x, layers=[host_layer])
    assert h._layers is old and h._wt == "old-array"
    # the library refuses the call (e.g. a misaligned pointer): nothing is committed either
    monkeypatch.setattr(binding.MoeRound, "_marshal_layers", lambda self, layers: "new-array")
    monkeypatch.setattr(binding.MoeRound, "_run_args", lambda self, *a: ())
    monkeypatch.setattr(binding.MoeRound, "_raise", lambda self, st, what: (_ for _ in ()).throw(RuntimeError(what)))

    class FakeLib:
        def moe_round_run(self, *a):
            return binding.ERR_INVALID_ARG
    h.lib = FakeLib()
    with pytest.raises(RuntimeError):
        h.run(x, 1, x, layers=[object()])
    assert h._layers is old and h._wt == "old-array"


def test_status_strings(lib):
    from verify_router_gemv_amd import binding
    assert binding.strerror(0) == "ok"
    assert "unsupported" in binding.strerror(-2) or "supported" in binding.strerror(-2)
    assert binding.strerror(-3) == "HIP runtime error"
    assert binding.strerror(99) == "unknown status"


def test_binding_refuses_host_tensors(lib):
    from verify_router_gemv_amd import binding
    E, H, I = 4, 256, 128
    layer = dict(router_w=torch.zeros(E, H), router_b=None,
                 gate_q=torch.zeros(E, I, H // 2, dtype=torch.uint8), gate_sm=torch.zeros(E, I, H // 32, dtype=torch.int32),
                 up_q=torch.zeros(E, I, H // 2, dtype=torch.uint8), up_sm=torch.zeros(E, I, H // 32, dtype=torch.int32),
                 down_q=torch.zeros(E, H, I // 2, dtype=torch.uint8), down_sm=torch.zeros(E, H, I // 32, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        binding.layer_struct(layer, H, I, E)
