"""Seeded synthetic workloads and the 4-bit block weight layout.

Every tensor here is drawn from a seeded generator and written in the layout
the library reads; nothing here evaluates the MoE round.

Weight layout ("Q4B32"), one matrix W[rows][K] with K the reduction length:
  * codes  uint8 [rows][K/2]: byte j of a row holds element 2j in its low
    nibble and element 2j+1 in its high nibble (so one 32-element block is
    16 consecutive bytes);
  * scale/min uint32 [rows][K/32]: the low half is the block's fp16 scale s,
    the high half its fp16 minimum m.  A weight is represented as s*q + m
    with q in 0..15.
A block with a scale and a minimum per 32 weights follows the K-quant
family described in the infero README ("AWQ, FP8, and NVFP4 checkpoints":
a 6-bit scale and a 6-bit minimum every 32 weights); here both are fp16.

Weight layout ("Q4S256", 4.5 bits per weight): the same codes, and per
256-weight super-block (eight 32-weight sub-blocks, K a multiple of 256) one
16-byte record, int32 [rows][K/256][4]:
  * word 0: fp16 super-scale d in the low half, fp16 super-minimum dmin in
    the high half;
  * words 1..3: a 96-bit little-endian string of eight 12-bit fields, field
    j at bits 12j..12j+11 holding the sub-block's 6-bit scale sc_j (bits
    0-5) and 6-bit minimum m_j (bits 6-11).
A weight of sub-block j is d*sc_j*q - dmin*m_j.  That is 128 B of codes and
16 B of scales per 256 weights, the super-block size and the packed
twelve-byte scale/minimum field the infero README describes for its 4-bit
K-quant ("Supported weight encodings"; "AWQ, FP8, and NVFP4 checkpoints").

Expert matrices are stored output-major: gate and up as [E][I][H] (reduce
over H), down as [E][H][I] (reduce over I).  The router is fp32 [E][H] with
an optional fp32 bias [E].

Workload shapes and distributions (all seeded):
  tiny    H=256  E=8   k=2  I=128 T=1, no bias
  decode  H=2048 E=128 k=8  I=768 T=1, Zipf(s=1.1) router bias
  verify  H=2048 E=256 k=8  I=512 T in {1,2,3,4,5,8}, rows = base + 0.5*noise
  deep    H=2048 E=512 k=10 I=512 T=3, 48 layers, Zipf(s=1.0), residual
  wide    H=2048 E=256 k=8  I=512 T in {16,32,64}, independent rows
  prefill H=2048 E=256 k=8  I=512 T in {512,4096}, independent rows (a prompt)
Router weights ~ N(0, 0.02) fp32; expert weights ~ N(0, 0.02) then
quantised; activations ~ N(0, 1).  The pages measure text benchmarks on
trained models; these synthetic inputs stand in for them with the shapes of
the 512-expert, top-10, 48-layer MoE the Avalon README describes (intro) and
the 1-8 row verify rounds of the AlphaInfer page (section 2).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

BLOCK = 32
SUPER = 256
FORMATS = ("q4b32", "q4s256")


@dataclasses.dataclass(frozen=True)
class ShapeConfig:
    name: str
    H: int
    E: int
    k: int
    I: int
    L: int = 1
    T: Sequence[int] = (1,)
    zipf_s: Optional[float] = None
    rows: str = "indep"          # "indep" | "correlated"
    residual: bool = False
    fmt: str = "q4b32"           # weight layout: "q4b32" | "q4s256"

    def expert_bytes(self) -> int:
        """Bytes of one expert's gate+up+down in the configured weight layout."""
        if self.fmt == "q4s256":
            return 3 * self.H * self.I * (SUPER // 2 + 16) // SUPER   # 128 B codes + 16 B per 256
        per_weight_num = BLOCK // 2 + 4     # 16 B codes + 4 B scale/min per 32
        return 3 * self.H * self.I * per_weight_num // BLOCK

    def replace(self, **kw) -> "ShapeConfig":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": ShapeConfig("tiny", H=256, E=8, k=2, I=128, T=(1,)),
    "decode": ShapeConfig("decode", H=2048, E=128, k=8, I=768, T=(1,), zipf_s=1.1),
    "verify": ShapeConfig("verify", H=2048, E=256, k=8, I=512, T=(1, 2, 3, 4, 5, 8),
                          rows="correlated"),
    "deep": ShapeConfig("deep", H=2048, E=512, k=10, I=512, L=48, T=(3,), zipf_s=1.0,
                        residual=True),
    "wide": ShapeConfig("wide", H=2048, E=256, k=8, I=512, T=(16, 32, 64)),
    "prefill": ShapeConfig("prefill", H=2048, E=256, k=8, I=512, T=(512, 4096)),
}


def config(name: str) -> ShapeConfig:
    return CONFIGS[name]


def derive_seed(*words: int) -> int:
    """A 63-bit generator seed from a tuple of small integers."""
    st = np.random.SeedSequence([int(w) for w in words]).generate_state(2, dtype=np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def _gen(device, *words) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(*words))
    return g


def quantize_q4b32(w: torch.Tensor):
    """Encode float weights [..., K] into (codes uint8 [..., K/2], sm int32 [..., K/32]).

    Per block: m = fp16(min), s = fp16((max - min) / 15), q = clip(round_half_even((w - m) / s), 0, 15),
    q = 0 where s == 0.  This only prepares input data; the codes are what the round consumes.
    """
    K = w.shape[-1]
    assert K % BLOCK == 0
    lead = w.shape[:-1]
    b = w.float().reshape(*lead, K // BLOCK, BLOCK)
    mn = b.amin(dim=-1)
    mx = b.amax(dim=-1)
    s16 = ((mx - mn) / 15.0).to(torch.float16)
    m16 = mn.to(torch.float16)
    s = s16.float().unsqueeze(-1)
    m = m16.float().unsqueeze(-1)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    q = torch.where(s > 0, torch.round((b - m) / safe), torch.zeros_like(b))
    q = q.clamp_(0, 15).to(torch.uint8).reshape(*lead, K // 2, 2)
    codes = q[..., 0] | (q[..., 1] << 4)
    sbits = s16.view(torch.int16).to(torch.int32) & 0xFFFF
    mbits = m16.view(torch.int16).to(torch.int32) << 16
    sm = sbits | mbits
    return codes.contiguous(), sm.contiguous()


def _wrap_int32(v: torch.Tensor) -> torch.Tensor:
    """int64 values in [0, 2^32) -> the int32 tensor with the same 32 bits."""
    v = v & 0xFFFFFFFF
    return torch.where(v >= (1 << 31), v - (1 << 32), v).to(torch.int32)


def quantize_q4s256(w: torch.Tensor):
    """Encode float weights [..., K] (K a multiple of 256) into (codes uint8 [..., K/2],
    records int32 [..., K/256, 4]) in the Q4S256 layout described above.

    Per super-block, for its sub-blocks j: range r_j = (max_j - min_j) / 15 and offset
    o_j = max(-min_j, 0); d = fp16(max_j r_j / 63), dmin = fp16(max_j o_j / 63);
    sc_j = clip(rint(r_j / d), 0, 63) and m_j = clip(rint(o_j / dmin), 0, 63) (0 where d or dmin is
    0); q = clip(rint((w + dmin*m_j) / (d*sc_j)), 0, 15) (0 where d*sc_j is 0).  Input data only.
    """
    K = w.shape[-1]
    assert K % SUPER == 0
    lead = w.shape[:-1]
    nsb = K // SUPER
    b = w.float().reshape(*lead, nsb, SUPER // BLOCK, BLOCK)
    mn = b.amin(dim=-1)
    mx = b.amax(dim=-1)
    rng = (mx - mn) / 15.0
    off = (-mn).clamp(min=0.0)
    d16 = (rng.amax(dim=-1) / 63.0).to(torch.float16)
    dmin16 = (off.amax(dim=-1) / 63.0).to(torch.float16)
    d = d16.float().unsqueeze(-1)
    dmin = dmin16.float().unsqueeze(-1)
    sc = torch.where(d > 0, torch.round(rng / torch.where(d > 0, d, torch.ones_like(d))), torch.zeros_like(rng))
    sc = sc.clamp_(0, 63)
    m6 = torch.where(dmin > 0, torch.round(off / torch.where(dmin > 0, dmin, torch.ones_like(dmin))),
                     torch.zeros_like(off))
    m6 = m6.clamp_(0, 63)
    a = (d * sc).unsqueeze(-1)      # exact: an fp16 times an integer below 64
    o = (dmin * m6).unsqueeze(-1)
    safe = torch.where(a > 0, a, torch.ones_like(a))
    q = torch.where(a > 0, torch.round((b + o) / safe), torch.zeros_like(b))
    q = q.clamp_(0, 15).to(torch.uint8).reshape(*lead, K // 2, 2)
    codes = q[..., 0] | (q[..., 1] << 4)
    f = sc.to(torch.int64) | (m6.to(torch.int64) << 6)           # [..., nsb, 8] 12-bit fields
    w1 = f[..., 0] | (f[..., 1] << 12) | ((f[..., 2] & 0xFF) << 24)
    w2 = (f[..., 2] >> 8) | (f[..., 3] << 4) | (f[..., 4] << 16) | ((f[..., 5] & 0xF) << 28)
    w3 = (f[..., 5] >> 4) | (f[..., 6] << 8) | (f[..., 7] << 20)
    w0 = (d16.view(torch.int16).to(torch.int64) & 0xFFFF) | ((dmin16.view(torch.int16).to(torch.int64) & 0xFFFF) << 16)
    rec = torch.stack([_wrap_int32(w0), _wrap_int32(w1), _wrap_int32(w2), _wrap_int32(w3)], dim=-1)
    return codes.contiguous(), rec.contiguous()


@dataclasses.dataclass
class LayerInputs:
    """One MoE layer's weights in the library layout (torch tensors, any device)."""
    router_w: torch.Tensor            # f32 [E, H]
    router_b: Optional[torch.Tensor]  # f32 [E] or None
    gate_q: torch.Tensor              # u8  [E, I, H/2]
    gate_sm: torch.Tensor             # i32 [E, I, H/32]
    up_q: torch.Tensor
    up_sm: torch.Tensor
    down_q: torch.Tensor              # u8  [E, H, I/2]
    down_sm: torch.Tensor             # i32 [E, H, I/32]  (q4s256: [E, H, I/256, 4])
    fmt: str = "q4b32"                # "q4b32": *_sm per 32-block; "q4s256": super-block records

    FIELDS = ("router_w", "router_b", "gate_q", "gate_sm", "up_q", "up_sm", "down_q", "down_sm")

    def map(self, fn) -> "LayerInputs":
        return LayerInputs(**{f: (None if getattr(self, f) is None else fn(getattr(self, f)))
                              for f in self.FIELDS}, fmt=self.fmt)

    def to(self, device) -> "LayerInputs":
        return self.map(lambda t: t.to(device))

    def clone(self) -> "LayerInputs":
        return self.map(lambda t: t.clone())

    def numpy(self) -> dict:
        """Host numpy copies (the oracle's view); scale/min words as uint32."""
        out = {}
        for f in self.FIELDS:
            t = getattr(self, f)
            if t is None:
                out[f] = None
                continue
            a = t.detach().cpu().numpy()
            if f.endswith("_sm"):
                a = a.view(np.uint32)
            out[f] = a
        out["format"] = self.fmt
        return out

    def expert_numpy(self, e: int) -> dict:
        """Host copies of one expert's six arrays (for checks that touch few experts)."""
        out = {}
        for f in ("gate_q", "gate_sm", "up_q", "up_sm", "down_q", "down_sm"):
            a = getattr(self, f)[e].detach().cpu().numpy()
            out[f] = a.view(np.uint32) if f.endswith("_sm") else a
        return out


_EXPERT_CHUNK = 16
_STREAM_ROUTER, _STREAM_BIAS, _STREAM_GATE, _STREAM_UP, _STREAM_DOWN, _STREAM_RESIDENT = range(6)


def _expert_matrix(cfg: ShapeConfig, seed: int, layer: int, stream: int, rows: int, K: int,
                   device) -> tuple:
    E = cfg.E
    codes = torch.empty((E, rows, K // 2), dtype=torch.uint8, device=device)
    if cfg.fmt == "q4s256":
        sm = torch.empty((E, rows, K // SUPER, 4), dtype=torch.int32, device=device)
        quantize = quantize_q4s256
    else:
        sm = torch.empty((E, rows, K // BLOCK), dtype=torch.int32, device=device)
        quantize = quantize_q4b32
    for e0 in range(0, E, _EXPERT_CHUNK):
        e1 = min(E, e0 + _EXPERT_CHUNK)
        w = torch.empty((e1 - e0, rows, K), dtype=torch.float32, device=device)
        for e in range(e0, e1):
            g = _gen(device, seed, 0, layer, stream, e)
            w[e - e0].normal_(0.0, 0.02, generator=g)
        c, s = quantize(w)
        codes[e0:e1] = c
        sm[e0:e1] = s
        del w
    return codes, sm


def make_layer(cfg: ShapeConfig, seed: int = 0, layer: int = 0, device="cpu") -> LayerInputs:
    """All weights of one layer, drawn on `device` (CPU and GPU draws differ; each is seeded)."""
    device = torch.device(device)
    H, E, I = cfg.H, cfg.E, cfg.I
    g = _gen(device, seed, 0, layer, _STREAM_ROUTER)
    router_w = torch.empty((E, H), dtype=torch.float32, device=device).normal_(0.0, 0.02, generator=g)
    router_b = None
    if cfg.zipf_s is not None:
        # Zipf popularity: a per-expert logit offset -s*ln(rank), rank a seeded permutation of 1..E.
        gp = _gen("cpu", seed, 0, layer, _STREAM_BIAS)
        rank = torch.randperm(E, generator=gp).to(torch.float64) + 1.0
        router_b = (-cfg.zipf_s * torch.log(rank)).to(torch.float32).to(device)
    gate_q, gate_sm = _expert_matrix(cfg, seed, layer, _STREAM_GATE, I, H, device)
    up_q, up_sm = _expert_matrix(cfg, seed, layer, _STREAM_UP, I, H, device)
    down_q, down_sm = _expert_matrix(cfg, seed, layer, _STREAM_DOWN, H, I, device)
    return LayerInputs(router_w, router_b, gate_q, gate_sm, up_q, up_sm, down_q, down_sm, fmt=cfg.fmt)


def make_activations(cfg: ShapeConfig, T: int, seed: int = 0, round_idx: int = 0,
                     device="cpu") -> torch.Tensor:
    """Round `round_idx`'s input rows X [T, H] fp32 ~ N(0,1) (correlated rows for the verify sweep)."""
    device = torch.device(device)
    g = _gen(device, seed, 1, round_idx, T)
    if cfg.rows == "correlated":
        base = torch.randn((1, cfg.H), generator=g, device=device, dtype=torch.float32)
        noise = torch.randn((T, cfg.H), generator=g, device=device, dtype=torch.float32)
        return (base + 0.5 * noise).contiguous()
    return torch.randn((T, cfg.H), generator=g, device=device, dtype=torch.float32)


def make_residency(cfg: ShapeConfig, frac: float, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Which experts of a layer sit in GPU memory (bool [E]): round(frac * E) of them.

    With a Zipf router bias they are the most popular experts (the bias's rank permutation, as a
    cache filled with the hottest experts of a ranking: Avalon README, hardware section); without
    one, a seeded random subset.  The rest are "missed" experts, kept in host memory.
    """
    E = cfg.E
    n = int(round(frac * E))
    if cfg.zipf_s is not None:
        gp = _gen("cpu", seed, 0, layer, _STREAM_BIAS)
        rank = torch.randperm(E, generator=gp).numpy() + 1   # the same draw as make_layer's bias
        return rank <= n
    g = _gen("cpu", seed, 0, layer, _STREAM_RESIDENT)
    res = np.zeros(E, dtype=bool)
    res[torch.randperm(E, generator=g)[:n].numpy()] = True
    return res


def metric_bytes(cfg: ShapeConfig, n_unique: int, T: int) -> int:
    """Bytes the round must move: unique experts' codes + scales/mins, plus T input and T output rows."""
    return n_unique * cfg.expert_bytes() + 2 * T * cfg.H * 4


def all_bytes(cfg: ShapeConfig, n_unique: int, T: int) -> int:
    """metric_bytes plus the router weights (and bias) and the gate/up -> down intermediate."""
    extra = cfg.E * cfg.H * 4 + (cfg.E * 4 if cfg.zipf_s is not None else 0)
    extra += 2 * T * cfg.k * cfg.I * 4
    return metric_bytes(cfg, n_unique, T) + extra


def human(cfg: ShapeConfig) -> str:
    return (f"{cfg.name}: H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} L={cfg.L} T={tuple(cfg.T)}"
            f" zipf={cfg.zipf_s} rows={cfg.rows}")


assert math.isclose(CONFIGS["verify"].expert_bytes(), 1_966_080)
assert math.isclose(CONFIGS["decode"].expert_bytes(), 2_949_120)
assert CONFIGS["verify"].replace(fmt="q4s256").expert_bytes() == 1_769_472
