"""Thin ctypes binding over libmoe_round.so (argument marshalling only).

Every step of the round runs in the HIP library; this module only checks tensor
dtypes/shapes/devices, passes raw device pointers and maps status codes to
exceptions.  PyTorch provides device memory and the stream.  If the library is
not built, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_round.so")

ABI_VERSION = 3
MAX_ROWS = 64
MAX_PREFILL_ROWS = 16384
MAX_EXPERTS = 512
MAX_TOPK = 16
KERNELS_PER_LAYER = 5
KERNEL_NAMES = ("logits", "select", "gateup", "down", "combine")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_OOM, ERR_STATE = 0, -1, -2, -3, -4, -5


class MoeRoundError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{what}: {strerror(status)} (status {status}"
        msg += f", hipError {hip_error})" if hip_error else ")"
        super().__init__(msg)


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "abi_version", "hidden", "inter", "n_experts", "top_k_max", "n_layers", "max_rows",
        "residual", "use_graph", "fused_max_rows", "rows_per_item", "mfma_min_rows", "exact",
        "weight_format", "prefetch", "record_layers", "expert_table", "tail_skip_rank")]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "router_w", "router_bias", "gate_q", "gate_sm", "up_q", "up_sm", "down_q", "down_sm")]


EXPERT_FIELDS = ("gate_q", "gate_sm", "up_q", "up_sm", "down_q", "down_sm")


class ExpertRef(ctypes.Structure):
    """moe_expert_ref: one expert's six device-readable pointers (48 bytes)."""
    _fields_ = [(n, ctypes.c_void_p) for n in EXPERT_FIELDS]


class Stats(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("rows", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("skipped", ctypes.c_int32), ("expert_bytes", ctypes.c_int64), ("metric_bytes", ctypes.c_int64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m verify_router_gemv_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, vp = ctypes.c_int32, ctypes.c_void_p
    P = ctypes.POINTER
    sig = {
        "moe_round_validate_config": (i32, [P(Config)]),
        "moe_round_init": (i32, [P(Config), P(LayerWeights), vp, P(vp)]),
        "moe_round_run": (i32, [vp, vp, i32, i32, P(LayerWeights), vp, vp, vp]),
        "moe_round_profile": (i32, [vp, i32]),
        "moe_round_profile_read": (i32, [vp, P(ctypes.c_double), P(i32)]),
        "moe_round_worklist": (i32, [vp, i32, P(i32), P(i32), P(i32), P(i32)]),
        "moe_round_last_unique": (i32, [vp, P(i32)]),
        "moe_round_swiglu_rows": (i32, [vp, P(ctypes.c_float)]),
        "moe_round_layer_input": (i32, [vp, i32, P(ctypes.c_float)]),
        "moe_round_last_stats": (i32, [vp, P(Stats), P(i32), P(ctypes.c_int64)]),
        "moe_round_floor": (i32, [vp]),
        "moe_round_stream_read": (i32, [vp, vp, ctypes.c_int64]),
        "moe_round_empty_launches": (i32, [vp, i32, i32, i32, vp]),
        "moe_round_run_noalloc": (i32, [P(Config), P(LayerWeights), vp, i32, i32, vp, vp, vp, vp, P(i32)]),
        "moe_round_bind_experts": (i32, [vp, vp, vp]),
        "moe_round_host_tier_pointer": (i32, [vp, P(vp)]),
        "moe_round_last_hip_error": (i32, [vp]),
        "moe_round_strerror": (ctypes.c_char_p, [i32]),
        "moe_round_destroy": (None, [vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strerror(status: int) -> str:
    try:
        return load().moe_round_strerror(status).decode()
    except ImportError:
        return f"status {status}"


WEIGHT_FORMATS = {"q4b32": 0, "q4s256": 1}   # MOE_WEIGHT_Q4B32, MOE_WEIGHT_Q4S256


def weight_format_code(fmt) -> int:
    """0 / 1, or the layout's name ("q4b32", "q4s256")."""
    if isinstance(fmt, str):
        return WEIGHT_FORMATS[fmt]
    return int(fmt)


def make_config(H, I, E, top_k_max, n_layers=1, max_rows=8, residual=False, use_graph=True,
                fused_max_rows=0, rows_per_item=0, mfma_min_rows=0, exact=False, weight_format=0,
                prefetch=0, record_layers=False, expert_table=False, tail_skip_rank=0) -> Config:
    """Launch-shape fields: 0 = default (see moe_round.h); -1 = never (fused_max_rows, mfma_min_rows).
    exact: fixed-order combine (bitwise reproducible, row outputs independent of the round).
    weight_format: 0 / "q4b32" (per-32 fp16 scale and minimum) or 1 / "q4s256" (super-blocks).
    prefetch: 1 = touch the next kernel's weight lines early, 0 = off (default).
    record_layers: keep every layer's input rows (read back with MoeRound.layer_input).
    expert_table: read the experts through a bound per-(layer, expert) pointer table (MoeRound.bind_experts).
    tail_skip_rank: r > 0 skips missed experts that every row selecting them ranks at r or below."""
    return Config(ABI_VERSION, H, I, E, top_k_max, n_layers, max_rows, int(bool(residual)), int(bool(use_graph)),
                  fused_max_rows, rows_per_item, mfma_min_rows, int(bool(exact)), weight_format_code(weight_format),
                  prefetch, int(bool(record_layers)), int(bool(expert_table)), int(tail_skip_rank))


def validate_config(cfg: Config) -> int:
    return load().moe_round_validate_config(ctypes.byref(cfg))


_FIELDS = ("router_w", "router_bias", "gate_q", "gate_sm", "up_q", "up_sm", "down_q", "down_sm")


def _get(layer, name):
    if isinstance(layer, dict):
        return layer.get(name if name != "router_bias" else "router_b", layer.get(name))
    return getattr(layer, "router_b" if name == "router_bias" else name)


def _check(t: torch.Tensor, name: str, dtypes, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def layer_format(layer):
    """The weight layout a layer object or dict declares ("fmt" / "format"), or None."""
    if isinstance(layer, dict):
        return layer.get("format")
    return getattr(layer, "fmt", None)


def layer_struct(layer, H: int, I: int, E: int, weight_format=0, router_only=False) -> LayerWeights:
    """Marshal one layer's weights (object or dict with the eight tensors) into the C struct.
    router_only: the expert table mode, where only the router comes from the layer (the expert
    pointers are left NULL)."""
    if weight_format_code(weight_format) == 1:
        sm_g, sm_d = (E, I, H // 256, 4), (E, H, I // 256, 4)
    else:
        sm_g, sm_d = (E, I, H // 32), (E, H, I // 32)
    spec = {
        "router_w": ((torch.float32,), (E, H)),
        "router_bias": ((torch.float32,), (E,)),
        "gate_q": ((torch.uint8,), (E, I, H // 2)),
        "gate_sm": ((torch.int32, torch.uint32), sm_g),
        "up_q": ((torch.uint8,), (E, I, H // 2)),
        "up_sm": ((torch.int32, torch.uint32), sm_g),
        "down_q": ((torch.uint8,), (E, H, I // 2)),
        "down_sm": ((torch.int32, torch.uint32), sm_d),
    }
    ptrs = {}
    for f in _FIELDS:
        if router_only and f in EXPERT_FIELDS:
            ptrs[f] = None
            continue
        t = _get(layer, f)
        if t is None and f == "router_bias":
            ptrs[f] = None
            continue
        _check(t, f, *spec[f])
        ptrs[f] = t.data_ptr()
    return LayerWeights(*[ptrs[f] for f in _FIELDS])


def host_tier_pointer(t: torch.Tensor) -> int:
    """The device address of pinned host memory (a tensor made with pin_memory=True), checked by the
    library: raises if the memory is not pinned and mapped for the GPU."""
    if t.device.type != "cpu" or not t.is_pinned():
        raise ValueError("a host-tier tensor must be pinned CPU memory")
    dev = ctypes.c_void_p()
    st = load().moe_round_host_tier_pointer(ctypes.c_void_p(t.data_ptr()), ctypes.byref(dev))
    if st != OK:
        raise MoeRoundError(st, "moe_round_host_tier_pointer")
    return int(dev.value)


def expert_slices(layer, e: int) -> dict:
    """Expert e's six matrices of a layer (views of its [E][..] tensors)."""
    return {f: _get(layer, f)[e] for f in EXPERT_FIELDS}


def make_expert_table(entries, H: int, I: int, weight_format=0, device="cuda") -> torch.Tensor:
    """The moe_expert_ref [L][E] table as a device int64 tensor [L, E, 6] from entries[l][e], a dict
    of the expert's six tensors (device tensors, or pinned host tensors read in place). Shapes and
    dtypes are checked; the caller keeps the tensors alive while the table is bound."""
    fmt = weight_format_code(weight_format)
    sm_g = (I, H // 256, 4) if fmt == 1 else (I, H // 32)
    sm_d = (H, I // 256, 4) if fmt == 1 else (H, I // 32)
    spec = {"gate_q": ((torch.uint8,), (I, H // 2)), "gate_sm": ((torch.int32, torch.uint32), sm_g),
            "up_q": ((torch.uint8,), (I, H // 2)), "up_sm": ((torch.int32, torch.uint32), sm_g),
            "down_q": ((torch.uint8,), (H, I // 2)), "down_sm": ((torch.int32, torch.uint32), sm_d)}
    rows = []
    for layer_entries in entries:
        lrow = []
        for ent in layer_entries:
            ptrs = []
            for f in EXPERT_FIELDS:
                t = ent[f]
                dtypes, shape = spec[f]
                if t.dtype not in dtypes or tuple(t.shape) != shape or not t.is_contiguous():
                    raise ValueError(f"{f}: {t.dtype} {tuple(t.shape)} (want {shape}, contiguous)")
                p = t.data_ptr() if t.device.type == "cuda" else host_tier_pointer(t)
                if p % 16:
                    raise ValueError(f"{f} must be 16-byte aligned")
                ptrs.append(p)
            lrow.append(ptrs)
        rows.append(lrow)
    return torch.tensor(rows, dtype=torch.int64).to(device)


def residency_bits(resident, device="cuda") -> torch.Tensor:
    """Per layer a boolean [E] (True = resident in device memory) packed as the library's residency
    words: int32 [L][ceil(E/32)], bit e % 32 of word e / 32."""
    import numpy as np
    res = np.asarray(resident, dtype=bool)
    L, E = res.shape
    words = np.zeros((L, (E + 31) // 32), dtype=np.uint32)
    for e in range(E):
        words[:, e // 32] |= res[:, e].astype(np.uint32) << np.uint32(e % 32)
    return torch.from_numpy(words.view(np.int32)).to(device)


def run_noalloc(layers: Sequence, H: int, I: int, E: int, top_k_max: int, hidden: torch.Tensor, k: int,
                out: torch.Tensor, ids: Optional[torch.Tensor] = None, route_w: Optional[torch.Tensor] = None,
                max_rows: Optional[int] = None, residual: bool = False, exact: bool = False, weight_format=None,
                fused_max_rows: int = 0, rows_per_item: int = 0, mfma_min_rows: int = 0, prefetch: int = 0,
                stream: Optional[torch.cuda.Stream] = None):
    """One decode/verify round through moe_round_run_noalloc: no handle, no allocation (the library's
    fixed per-device scratch array). Same arguments and results as MoeRound(...).run(...)."""
    lib = load()
    L = len(layers)
    T = hidden.shape[0]
    if weight_format is None:
        weight_format = layer_format(layers[0]) or "q4b32"
    fmt = weight_format_code(weight_format)
    cfg = make_config(H, I, E, top_k_max, L, max_rows or max(T, 1), residual, False, fused_max_rows,
                      rows_per_item, mfma_min_rows, exact, fmt, prefetch)
    wt = (LayerWeights * L)(*[layer_struct(l, H, I, E, fmt) for l in layers])
    _check(hidden, "hidden", (torch.float32,), (T, H))
    _check(out, "out", (torch.float32,), (T, H))
    if ids is not None:
        _check(ids, "expert_ids", (torch.int32,), (L, T, k))
    if route_w is not None:
        _check(route_w, "route_w", (torch.float32,), (L, T, k))
    st_ = stream if stream is not None else torch.cuda.current_stream()
    herr = ctypes.c_int32()
    st = lib.moe_round_run_noalloc(ctypes.byref(cfg), wt, ctypes.c_void_p(hidden.data_ptr()), T, k,
                                   ctypes.c_void_p(out.data_ptr()),
                                   ctypes.c_void_p(ids.data_ptr() if ids is not None else 0),
                                   ctypes.c_void_p(route_w.data_ptr() if route_w is not None else 0),
                                   ctypes.c_void_p(st_.cuda_stream), ctypes.byref(herr))
    if st != OK:
        raise MoeRoundError(st, "moe_round_run_noalloc", herr.value)


class MoeRound:
    """A handle over the C ABI: one MoE round evaluator bound to a stream."""

    def __init__(self, layers: Sequence, H: int, I: int, E: int, top_k_max: int, max_rows: int = 8,
                 residual: bool = False, use_graph: bool = True, stream: Optional[torch.cuda.Stream] = None,
                 fused_max_rows: int = 0, rows_per_item: int = 0, mfma_min_rows: int = 0, exact: bool = False,
                 weight_format=None, prefetch: int = 0, record_layers: bool = False, expert_table: bool = False,
                 tail_skip_rank: int = 0):
        """weight_format: None = what the layers declare (default "q4b32"), else 0/1 or its name.
        expert_table: the layers supply the routers only; bind the experts with bind_experts()."""
        self.lib = load()
        self.H, self.I, self.E, self.L = H, I, E, len(layers)
        self.top_k_max, self.max_rows = top_k_max, max_rows
        if weight_format is None:
            weight_format = layer_format(layers[0]) or "q4b32"
        self.weight_format = weight_format_code(weight_format)
        self.expert_table = bool(expert_table)
        self.cfg = make_config(H, I, E, top_k_max, self.L, max_rows, residual, use_graph,
                               fused_max_rows, rows_per_item, mfma_min_rows, exact, self.weight_format, prefetch,
                               record_layers, expert_table, tail_skip_rank)
        self.stream = stream if stream is not None else torch.cuda.current_stream()
        self._layers = list(layers)          # keep the weight tensors alive
        self._wt = (LayerWeights * self.L)(*[layer_struct(l, H, I, E, self.weight_format, self.expert_table)
                                             for l in layers])
        self._bound = (None, None)
        h = ctypes.c_void_p()
        st = self.lib.moe_round_init(ctypes.byref(self.cfg), self._wt, ctypes.c_void_p(self.stream.cuda_stream),
                                     ctypes.byref(h))
        if st != OK:
            raise MoeRoundError(st, "moe_round_init")
        self.h = h
        self._profiling = False

    def _raise(self, st, what):
        raise MoeRoundError(st, what, self.lib.moe_round_last_hip_error(self.h))

    def _marshal_layers(self, layers: Sequence):
        """The C array for `layers` (checked), without touching the handle's current weights."""
        if len(layers) != self.L:
            raise ValueError("layer count must not change")
        return (LayerWeights * self.L)(*[layer_struct(l, self.H, self.I, self.E, self.weight_format,
                                                      self.expert_table) for l in layers])

    def bind_experts(self, table: Optional[torch.Tensor] = None, resident: Optional[torch.Tensor] = None):
        """Bind the expert table (device int64 [L, E, 6], make_expert_table) and the residency words
        (device int32 [L, ceil(E/32)], residency_bits); their contents are read by each later round."""
        if table is not None:
            _check(table, "table", (torch.int64,), (self.L, self.E, 6))
        if resident is not None:
            _check(resident, "resident", (torch.int32, torch.uint32), (self.L, (self.E + 31) // 32))
        st = self.lib.moe_round_bind_experts(self.h, ctypes.c_void_p(table.data_ptr() if table is not None else 0),
                                             ctypes.c_void_p(resident.data_ptr() if resident is not None else 0))
        if st != OK:
            self._raise(st, "moe_round_bind_experts")
        self._bound = (table, resident)

    def _run_args(self, hidden, k, out, ids, route_w, wt):
        T = hidden.shape[0]
        _check(hidden, "hidden", (torch.float32,), (T, self.H))
        _check(out, "out", (torch.float32,), (T, self.H))
        if ids is not None:
            _check(ids, "expert_ids", (torch.int32,), (self.L, T, k))
        if route_w is not None:
            _check(route_w, "route_w", (torch.float32,), (self.L, T, k))
        return (self.h, ctypes.c_void_p(hidden.data_ptr()), T, k, wt, ctypes.c_void_p(out.data_ptr()),
                ctypes.c_void_p(ids.data_ptr() if ids is not None else 0),
                ctypes.c_void_p(route_w.data_ptr() if route_w is not None else 0))

    def run(self, hidden: torch.Tensor, k: int, out: torch.Tensor, ids: Optional[torch.Tensor] = None,
            route_w: Optional[torch.Tensor] = None, layers: Optional[Sequence] = None):
        """One round. `layers`: new weights for this and later rounds; the handle keeps referencing
        the old tensors until the library has accepted the new ones (a rejected call changes nothing)."""
        wt = self._marshal_layers(layers) if layers is not None else None
        st = self.lib.moe_round_run(*self._run_args(hidden, k, out, ids, route_w, wt))
        if st != OK:
            self._raise(st, "moe_round_run")
        if layers is not None:
            self._layers, self._wt = list(layers), wt

    def profile(self, enable: bool = True):
        """Start (or stop) per-kernel timing of the following runs (dispatch timestamps)."""
        st = self.lib.moe_round_profile(self.h, int(bool(enable)))
        if st != OK:
            self._raise(st, "moe_round_profile")
        self._profiling = bool(enable)

    def profile_read(self):
        """(sum of milliseconds [L][5] per kernel kind (KERNEL_NAMES); number of runs) since profiling
        started or was last read."""
        ms = (ctypes.c_double * (KERNELS_PER_LAYER * self.L))()
        n = ctypes.c_int32()
        st = self.lib.moe_round_profile_read(self.h, ms, ctypes.byref(n))
        if st != OK:
            self._raise(st, "moe_round_profile_read")
        return [[ms[KERNELS_PER_LAYER * l + i] for i in range(KERNELS_PER_LAYER)] for l in range(self.L)], n.value

    def run_timed(self, hidden, k, out, ids=None, route_w=None, layers=None):
        """One run with per-kernel timing; returns [L][5] milliseconds by KERNEL_NAMES (synchronises)."""
        was = self._profiling
        if not was:
            self.profile(True)
        self.profile_read()
        self.run(hidden, k, out, ids, route_w, layers)
        ms, _ = self.profile_read()
        if not was:
            self.profile(False)
        return ms

    def worklist(self, layer: int = 0):
        T_k = self.max_rows * self.top_k_max
        ucap = min(T_k, self.E)
        n = ctypes.c_int32()
        uniq = (ctypes.c_int32 * ucap)()
        offs = (ctypes.c_int32 * (ucap + 1))()
        pairs = (ctypes.c_int32 * (2 * T_k))()
        st = self.lib.moe_round_worklist(self.h, layer, ctypes.byref(n), uniq, offs, pairs)
        if st != OK:
            self._raise(st, "moe_round_worklist")
        nu = n.value
        return list(uniq[:nu]), list(offs[:nu + 1]), [tuple(pairs[2 * i:2 * i + 2]) for i in range(offs[nu])]

    def swiglu_rows(self, T: int, k: int):
        """The last run's last-layer gate/up output: [T*k][I] rows in worklist pair order."""
        import numpy as np
        buf = np.zeros((T * k, self.I), dtype=np.float32)
        st = self.lib.moe_round_swiglu_rows(self.h, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
        if st != OK:
            self._raise(st, "moe_round_swiglu_rows")
        return buf

    def layer_input(self, layer: int, T: int):
        """The last run's input rows of `layer` ([T][H] fp32 numpy; later layers need record_layers)."""
        import numpy as np
        buf = np.zeros((T, self.H), dtype=np.float32)
        st = self.lib.moe_round_layer_input(self.h, layer, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
        if st != OK:
            self._raise(st, "moe_round_layer_input")
        return buf

    def last_stats(self):
        """(Stats of the last run, per-layer n_unique list, per-layer metric bytes list)."""
        st_ = Stats()
        nu = (ctypes.c_int32 * self.L)()
        mb = (ctypes.c_int64 * self.L)()
        st = self.lib.moe_round_last_stats(self.h, ctypes.byref(st_), nu, mb)
        if st != OK:
            self._raise(st, "moe_round_last_stats")
        return st_, list(nu), list(mb)

    def floor(self):
        """Enqueue the byte floor of the last run (its weight reads alone, same launches per layer)."""
        st = self.lib.moe_round_floor(self.h)
        if st != OK:
            self._raise(st, "moe_round_floor")

    def stream_read(self, buf: torch.Tensor):
        """Enqueue one streaming read of the whole of `buf` (a device tensor; the control arm)."""
        if buf.device.type != "cuda" or not buf.is_contiguous():
            raise ValueError("stream_read needs a contiguous device tensor")
        st = self.lib.moe_round_stream_read(self.h, ctypes.c_void_p(buf.data_ptr()),
                                            buf.numel() * buf.element_size())
        if st != OK:
            self._raise(st, "moe_round_stream_read")

    def empty_launches(self, blocks: int, launches: int = 1, sleep_units: int = 0, flags=None):
        """Enqueue `launches` kernels of `blocks` one-wave blocks each (a launch-cost control): every
        wave sleeps `sleep_units` × ~2048 clocks, then stores its block index to `flags` (a device
        int32 tensor of at least `blocks` elements) when one is given."""
        fp = None
        if flags is not None:
            if (flags.device.type != "cuda" or flags.dtype != torch.int32 or not flags.is_contiguous()
                    or flags.numel() < blocks):
                raise ValueError("flags must be a contiguous device int32 tensor of at least `blocks` elements")
            fp = ctypes.c_void_p(flags.data_ptr())
        st = self.lib.moe_round_empty_launches(self.h, int(blocks), int(launches), int(sleep_units), fp)
        if st != OK:
            self._raise(st, "moe_round_empty_launches")

    def last_unique(self):
        arr = (ctypes.c_int32 * self.L)()
        st = self.lib.moe_round_last_unique(self.h, arr)
        if st != OK:
            self._raise(st, "moe_round_last_unique")
        return list(arr)

    def close(self):
        if getattr(self, "h", None):
            self.lib.moe_round_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
