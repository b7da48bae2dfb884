"""Seeded synthetic inputs for the EXL3 trellis-coded MoE layer.

This module draws random tensors and nothing else: it holds none of the
layer's arithmetic (no decode, routing, GEMM or rounding rule of the method).
Both the CPU oracle (tests, bench baseline) and the HIP path consume exactly
the bytes produced here.

Shapes follow the GLM-5.3-Flash MoE layer described on the kindlingai exlr8
page ("Loading": hidden 4096, expert intermediate 2048, 288 routed experts,
top-8, one shared expert) and the 7168-row prefill chunk of the MiaAI-Lab page
("Cold prefill (E3 grouped MoE)", MNBT 7168 and the isolated 7168-token layer
bench).  The pages measure real text through trained weights; neither exists
here, so these distributions stand in for them:

* activations x ~ N(0, 1), rounded to the activation dtype (fp16 or bf16);
* router weights fp16 ~ N(0, 0.02); optional per-expert fp32 bias ~ N(0, 1)
  that skews the expert loads;
* trellis codes: uniform random 16-bit words (every bit pattern is a valid
  trellis stream);
* side vectors suh/svh: fp16 ~ U(0.5, 1.5) / sqrt(H_ref) with H_ref = hidden
  (1/16 for the tiny layer, 1/64 for the real shapes);
* shared expert: fp16 ~ N(0, 1/4096).

Every tensor has its own PCG64 stream keyed by (seed, tensor tag, index), so
any single expert's codes can be regenerated without drawing the others.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

# activation / weight dtype tags (match the C ABI's enum values)
DT_F32, DT_F16, DT_BF16, DT_FP8 = 0, 1, 2, 3
CB_MCG, CB_MCG_E4M3 = 0, 1
PROJ_GATE, PROJ_UP, PROJ_DOWN = 0, 1, 2

# Multiplier of the multiplicative congruential hash.  The pages store it as a
# (1,) int32 tensor per expert tensor but never print a value; Knuth's
# golden-ratio constant is used for every synthetic tensor.
MCG_DEFAULT = 0x9E3779B1

_TAGS = {
    "x": 1, "router_w": 2, "router_bias": 3, "codes": 4, "suh": 5, "svh": 6,
    "shared": 7, "ktab": 8, "signs": 9,
}


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    seed: int
    tokens: int
    hidden: int
    inter: int
    n_experts: int
    top_k: int
    K: int
    codebook: int = CB_MCG
    act_dtype: int = DT_BF16
    router_bias: bool = False
    shared: bool = False
    mcg: int = MCG_DEFAULT
    # every (projection, expert) tensor at its own width, drawn from {3, 4}
    mixed_k: bool = False
    # the layer's two int8 sign vectors over the hidden size (rotated experts)
    hadamard: bool = False
    # a trellis-coded shared expert stored after the routed ones (index E)
    shared_trellis: bool = False
    # with router_bias: a bias that makes experts 0 .. hot_experts-1 win for
    # every token (shapes the row tiles for per-tile-class measurements)
    hot_experts: int = 0

    @property
    def side_scale(self) -> float:
        return 1.0 / math.sqrt(self.hidden)

    @property
    def n_trellis(self) -> int:
        """Trellis-coded experts stored: the routed ones (+ the shared one)."""
        return self.n_experts + (1 if self.shared_trellis else 0)

    def proj_shape(self, p: int):
        """(in, out) of projection p; gate/up are [H][I], down is [I][H]."""
        return (self.hidden, self.inter) if p != PROJ_DOWN else (self.inter, self.hidden)

    def words_per_expert(self, p: int, K: Optional[int] = None) -> int:
        i, o = self.proj_shape(p)
        return (i // 16) * (o // 16) * 16 * (self.K if K is None else K)

    def words_of(self, p: int, e: int, ktab=None) -> int:
        """Words of tensor (p, e) at its width (ktab[p][e] when given)."""
        return self.words_per_expert(p, None if ktab is None else int(ktab[p][e]))

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny correctness layer, a decode-sized step, the
# 7168-token prefill chunk, a 2048-token prefill at K=3 and K=4, and a
# 16384-token prefill with the E4M3-rounded codebook.
CONFIGS: List[LayerConfig] = [
    LayerConfig("tiny", 0, 64, 256, 128, 8, 2, 2, CB_MCG, DT_F16, False, False),
    LayerConfig("decode", 1, 8, 4096, 2048, 288, 8, 2, CB_MCG, DT_BF16, False, True),
    LayerConfig("prefill", 2, 7168, 4096, 2048, 288, 8, 2, CB_MCG, DT_BF16, True, True),
    LayerConfig("mixed_k3", 3, 2048, 4096, 2048, 288, 8, 3, CB_MCG, DT_BF16, True, True),
    LayerConfig("mixed_k4", 3, 2048, 4096, 2048, 288, 8, 4, CB_MCG, DT_BF16, True, True),
    LayerConfig("fp8", 4, 16384, 4096, 2048, 288, 8, 4, CB_MCG_E4M3, DT_BF16, True, True),
]
# Further workloads for the format variants: per-tensor widths K3/K4 at the
# 2048-token prefill (the K3/K4 split of a 3.5 bpw build), and the decode step
# and the 2048-token prefill with rotated experts and a trellis-coded shared
# expert (the exlr8 v2 layout, K4, E4M3-rounded codebook).
VARIANTS: List[LayerConfig] = [
    LayerConfig("mixed_k34", 3, 2048, 4096, 2048, 288, 8, 4, CB_MCG, DT_BF16, True, True, mixed_k=True),
    LayerConfig("exlr8_decode", 5, 8, 4096, 2048, 288, 8, 4, CB_MCG_E4M3, DT_BF16, False, False,
                hadamard=True, shared_trellis=True),
    LayerConfig("exlr8_prefill", 6, 2048, 4096, 2048, 288, 8, 4, CB_MCG_E4M3, DT_BF16, True, False,
                hadamard=True, shared_trellis=True),
]
# Routings that isolate one class of MFMA row tile, for per-class timing and
# counters: every tile full (4096 tokens on 8 experts, 16 tiles of 256 rows
# each), tiles of at most 32 rows (512 tokens over 288 experts, run with
# every expert on the MFMA kernels), and tiles of mostly 33-96 rows (2048
# tokens over 288 experts).
TILE_CLASSES: List[LayerConfig] = [
    LayerConfig("tiles_full", 7, 4096, 4096, 2048, 288, 8, 2, CB_MCG, DT_BF16, True, False, hot_experts=8),
    LayerConfig("tiles_small", 8, 512, 4096, 2048, 288, 8, 2, CB_MCG, DT_BF16, False, False),
    LayerConfig("tiles_mid", 9, 2048, 4096, 2048, 288, 8, 2, CB_MCG, DT_BF16, False, False),
]
# One tensor-parallel rank's share of the prefill layer: the intermediate
# dimension split in two (each rank holds half of every expert's channels).
TP_SHARES: List[LayerConfig] = [
    LayerConfig("prefill_tp2", 2, 7168, 4096, 1024, 288, 8, 2, CB_MCG, DT_BF16, True, True),
]
BY_NAME: Dict[str, LayerConfig] = {c.name: c for c in CONFIGS + VARIANTS + TILE_CLASSES + TP_SHARES}


def _rng(seed: int, tag: str, *idx: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAGS[tag], *idx])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    assert np.isfinite(a).all()
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u                      # no overflow: finite inputs stay below 0xFF800000
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def act_bits_to_f32(bits: np.ndarray, act_dtype: int) -> np.ndarray:
    if act_dtype == DT_BF16:
        return bf16_bits_to_f32(bits)
    if act_dtype == DT_F16:
        return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    raise ValueError(act_dtype)


def gen_x(cfg: LayerConfig, tokens: Optional[int] = None) -> np.ndarray:
    """Activations [T][H] as uint16 bit patterns of cfg.act_dtype."""
    T = cfg.tokens if tokens is None else tokens
    v = _rng(cfg.seed, "x").standard_normal((T, cfg.hidden), dtype=np.float32)
    if cfg.act_dtype == DT_BF16:
        return f32_to_bf16_bits(v)
    return v.astype(np.float16).view(np.uint16)


def gen_router_w(cfg: LayerConfig) -> np.ndarray:
    """Router weights [E][H] fp16 ~ N(0, 0.02)."""
    v = _rng(cfg.seed, "router_w").standard_normal((cfg.n_experts, cfg.hidden), dtype=np.float32)
    return (v * np.float32(0.02)).astype(np.float16)


def gen_router_bias(cfg: LayerConfig) -> Optional[np.ndarray]:
    if not cfg.router_bias:
        return None
    if cfg.hot_experts:
        b = np.zeros(cfg.n_experts, dtype=np.float32)
        b[:cfg.hot_experts] = 64.0    # router logits are about N(0, 1.3)
        return b
    return _rng(cfg.seed, "router_bias").standard_normal(cfg.n_experts).astype(np.float32)


def gen_ktab(cfg: LayerConfig) -> Optional[np.ndarray]:
    """Per-tensor widths [3][n_trellis] int32, each K3 or K4 with equal odds,
    or None for a layer at one width."""
    if not cfg.mixed_k:
        return None
    return _rng(cfg.seed, "ktab").integers(3, 5, size=(3, cfg.n_trellis)).astype(np.int32)


def gen_signs(cfg: LayerConfig) -> Optional[np.ndarray]:
    """The layer's two sign vectors [2][H] int8 (+1 or -1 with equal odds)."""
    if not cfg.hadamard:
        return None
    return (_rng(cfg.seed, "signs").integers(0, 2, size=(2, cfg.hidden)) * 2 - 1).astype(np.int8)


def gen_codes_expert(cfg: LayerConfig, p: int, e: int, K: Optional[int] = None) -> np.ndarray:
    """Uniform random 16-bit trellis words of expert e, projection p (flat),
    at width K (default: the layer's)."""
    K = cfg.K if K is None else K
    return _rng(cfg.seed, "codes", K, p, e).integers(
        0, 1 << 16, size=cfg.words_per_expert(p, K), dtype=np.uint16)


def gen_codes(cfg: LayerConfig, p: int, experts=None, ktab=None):
    """Codes of projection p: [n_trellis][words] for all experts (a list of
    per-expert arrays when the widths differ), or, with `experts` given, a dict
    {expert: words} holding only those experts."""
    kof = (lambda e: None) if ktab is None else (lambda e: int(ktab[p][e]))
    if experts is not None:
        return {int(e): gen_codes_expert(cfg, p, int(e), kof(int(e))) for e in experts}
    if ktab is not None:
        return [gen_codes_expert(cfg, p, e, kof(e)) for e in range(cfg.n_trellis)]
    n = cfg.words_per_expert(p)
    out = np.empty((cfg.n_trellis, n), dtype=np.uint16)
    for e in range(cfg.n_trellis):
        out[e] = gen_codes_expert(cfg, p, e)
    return out


def gen_side(cfg: LayerConfig, p: int):
    """(suh [n_trellis][in], svh [n_trellis][out]) fp16 ~ U(0.5, 1.5) * side_scale."""
    i, o = cfg.proj_shape(p)
    r = _rng(cfg.seed, "suh", p)
    suh = (r.uniform(0.5, 1.5, (cfg.n_trellis, i)) * cfg.side_scale).astype(np.float16)
    r = _rng(cfg.seed, "svh", p)
    svh = (r.uniform(0.5, 1.5, (cfg.n_trellis, o)) * cfg.side_scale).astype(np.float16)
    return suh, svh


def gen_shared(cfg: LayerConfig):
    """Shared expert weights in nn.Linear layout: gate/up [I][H], down [H][I]."""
    if not cfg.shared:
        return None
    H, I = cfg.hidden, cfg.inter
    out = []
    for p, shp in ((0, (I, H)), (1, (I, H)), (2, (H, I))):
        v = _rng(cfg.seed, "shared", p).standard_normal(shp, dtype=np.float32)
        out.append((v * np.float32(1.0 / 64.0)).astype(np.float16))
    return out


@dataclasses.dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray                      # [T][H] uint16 bits of act dtype
    router_w: np.ndarray               # [E][H] fp16
    router_bias: Optional[np.ndarray]  # [E] fp32 or None
    codes: list                        # 3 x ([n_trellis][words] uint16, per-expert list, or dict)
    suh: List[np.ndarray]              # 3 x [n_trellis][in] fp16
    svh: List[np.ndarray]              # 3 x [n_trellis][out] fp16
    shared: Optional[List[np.ndarray]]
    ktab: Optional[np.ndarray] = None  # [3][n_trellis] int32 per-tensor widths
    signs: Optional[np.ndarray] = None # [2][H] int8 sign vectors


def gen_layer(cfg: LayerConfig, tokens: Optional[int] = None, experts=None) -> LayerInputs:
    suh, svh = zip(*(gen_side(cfg, p) for p in range(3)))
    ktab = gen_ktab(cfg)
    if experts is not None and cfg.shared_trellis:
        experts = sorted(set(int(e) for e in experts) | {cfg.n_experts})
    return LayerInputs(
        cfg=cfg,
        x=gen_x(cfg, tokens),
        router_w=gen_router_w(cfg),
        router_bias=gen_router_bias(cfg),
        codes=[gen_codes(cfg, p, experts, ktab) for p in range(3)],
        suh=list(suh),
        svh=list(svh),
        shared=gen_shared(cfg),
        ktab=ktab,
        signs=gen_signs(cfg),
    )
