"""Seeded synthetic inputs for the sparse-MoE layer forward.

This module only *draws* inputs.  It holds none of the layer's arithmetic
(no gating, routing, GEMM, SwiGLU, combine or MX quantisation); the HIP path
and the CPU oracle both take what it returns and compute independently.

Layer shapes follow the models the pages describe:

* the Qwen3-MoE low-latency page (Atlas A3 / 950, section on MoE TP and
  fused routing) for the softmax-renormalised top-8 layer over 128 experts;
* the Hy3 295B MoE on Atlas A3 page, section 1.2 (key parameters: hidden
  4096, expert intermediate 1536, 192 experts, top-8, one shared expert) and
  section 1.3 (sigmoid router, learnable e_score_correction_bias, top-k
  weights scaled by 2.826).

Value distributions: x ~ N(0,1), router weight ~ N(0,0.02), expert weights
~ N(0,0.02), all drawn in fp32 with torch's CPU generator and rounded to
bf16 by torch's round-to-nearest-even cast.  Every tensor (and every expert
of a weight tensor) has its own seed, derived from (family seed, tensor tag,
expert index), so a single expert can be regenerated on its own.

W4A8 weights are drawn directly as MXFP4 element codes plus E8M0 block
scales from a fixed categorical distribution whose decoded values have the
magnitude of an N(0,0.02) matrix (block scale mostly 2^-7, element codes
spread over the E2M1 grid).  The codes *are* the weights; nothing here
quantises anything.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import torch

# tensor tags used in seed derivation
_TAG_X, _TAG_ROUTER, _TAG_BIAS, _TAG_W13, _TAG_W2, _TAG_SHARED = 1, 2, 3, 4, 5, 6
_TAG_MX_W13, _TAG_MX_W2, _TAG_MX_SHARED = 7, 8, 9
_TAG_NORM_X, _TAG_NORM_RES, _TAG_NORM_W = 10, 11, 12
_TAG_CMB_Y, _TAG_CMB_PERM, _TAG_CMB_W = 13, 14, 15


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                 # tokens
    H: int                 # hidden size
    E: int                 # routed experts
    k: int                 # experts per token
    I: int                 # expert intermediate size
    gate: str = "softmax"  # "softmax" (renormalised over the selected k) or "sigmoid"
    routed_scale: float = 1.0
    eps: float = 1e-20
    bias: str = "none"     # "none" | "normal0.1" (selection-only) | "zipf1.1" (added to logits)
    shared_I: int = 0      # 0: no shared expert
    fmt: str = "bf16"      # "bf16" | "w4a8" (MXFP4 weights, MXFP8 activations)
    family_seed: int = 0   # weights are shared by configs of one model family
    x_seed: int = 0
    mx_scales: str = "narrow"  # W4A8 block scales: "narrow" (mostly 2^-7) | "wide" (2^-27 .. 2^13)

    def with_(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def R(self) -> int:
        return self.T * self.k


# The five synthetic layers.  "tiny" is the small case the oracle finishes in
# seconds; "qwen3_decode" is the weight-streaming decode layer.
CONFIGS = {
    "tiny": LayerConfig("tiny", T=16, H=256, E=8, k=2, I=128,
                        family_seed=1001, x_seed=1),
    "qwen3_decode": LayerConfig("qwen3_decode", T=16, H=4096, E=128, k=8, I=1536,
                                family_seed=1002, x_seed=2),
    "qwen3_prefill": LayerConfig("qwen3_prefill", T=4096, H=4096, E=128, k=8, I=1536,
                                 family_seed=1002, x_seed=3),
    "hy3": LayerConfig("hy3", T=4096, H=4096, E=192, k=8, I=1536, gate="sigmoid",
                       routed_scale=2.826, eps=1e-20, bias="normal0.1", shared_I=1536,
                       family_seed=1004, x_seed=4),
    "qwen3_decode_w4a8": LayerConfig("qwen3_decode_w4a8", T=16, H=4096, E=128, k=8, I=1536,
                                     bias="zipf1.1", fmt="w4a8",
                                     family_seed=1005, x_seed=5),
    # the prefill shape with MXFP4 weights and MXFP8 activations (same weights
    # as the W4A8 decode layer, no router bias)
    "qwen3_prefill_w4a8": LayerConfig("qwen3_prefill_w4a8", T=4096, H=4096, E=128, k=8, I=1536,
                                      fmt="w4a8", family_seed=1005, x_seed=6),
}

# Mid-size token counts of the Qwen3-style layers (same weights as the
# decode layers), across the switch from the weight-streaming GEMMs to the
# LDS-tiled ones (bf16: above 3 rows per expert on average, T > 48 here;
# W4A8: above 8, T > 128).
for _T in (64, 128, 256, 320, 512, 1024):
    CONFIGS[f"qwen3_T{_T}"] = CONFIGS["qwen3_decode"].with_(name=f"qwen3_T{_T}", T=_T, x_seed=100 + _T)
for _T in (64, 128, 256, 512, 1024):
    CONFIGS[f"qwen3_w4a8_T{_T}"] = CONFIGS["qwen3_decode_w4a8"].with_(name=f"qwen3_w4a8_T{_T}", T=_T,
                                                                      x_seed=200 + _T)

# The Hy3-style layer at decode size (same weights): the few-token front end
# with sigmoid gating over 192 experts, and the shared expert on its own
# weight-streaming launches.
CONFIGS["hy3_decode"] = CONFIGS["hy3"].with_(name="hy3_decode", T=16, x_seed=300)


def _seed(*parts: int) -> int:
    ss = np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts])
    return int(ss.generate_state(1, np.uint64)[0] & 0x7FFFFFFFFFFFFFFF)


def _gen(*parts: int) -> torch.Generator:
    return torch.Generator().manual_seed(_seed(*parts))


def _normal(shape, std: float, *parts: int) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(*parts), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def draw_x(cfg: LayerConfig) -> torch.Tensor:
    """Token activations [T, H] bf16, N(0,1)."""
    return _normal((cfg.T, cfg.H), 1.0, cfg.x_seed, _TAG_X, cfg.T, cfg.H).to(torch.bfloat16)


def draw_router(cfg: LayerConfig) -> torch.Tensor:
    """Router weight [E, H] fp32, N(0,0.02) (the gate runs in fp32)."""
    return _normal((cfg.E, cfg.H), 0.02, cfg.family_seed, _TAG_ROUTER, cfg.E, cfg.H)


def draw_bias(cfg: LayerConfig) -> Optional[torch.Tensor]:
    """Router bias [E] fp32, or None.

    normal0.1: Hy3's e_score_correction_bias stand-in, N(0, 0.1).
    zipf1.1:   b_e = ln p_e with p_e proportional to (e+1)^-1.1, so expert 0
               is the most popular; a fixed table, no randomness.
    """
    if cfg.bias == "none":
        return None
    if cfg.bias == "normal0.1":
        return _normal((cfg.E,), 0.1, cfg.family_seed, _TAG_BIAS, cfg.E)
    if cfg.bias == "zipf1.1":
        r = np.arange(1, cfg.E + 1, dtype=np.float64)
        p = r ** -1.1
        p /= p.sum()
        return torch.from_numpy(np.log(p).astype(np.float32))
    raise ValueError(cfg.bias)


def draw_expert_bf16(cfg: LayerConfig, e: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Expert e's weights in [out, in] layout, bf16 N(0,0.02).

    w13 [2I, H]: rows [0, I) are gate_proj, rows [I, 2I) are up_proj.
    w2  [H, I]:  down_proj.
    """
    w13 = _normal((2 * cfg.I, cfg.H), 0.02, cfg.family_seed, _TAG_W13, e, cfg.I, cfg.H)
    w2 = _normal((cfg.H, cfg.I), 0.02, cfg.family_seed, _TAG_W2, e, cfg.I, cfg.H)
    return w13.to(torch.bfloat16), w2.to(torch.bfloat16)


def draw_shared_bf16(cfg: LayerConfig) -> Tuple[torch.Tensor, torch.Tensor]:
    """The always-on shared expert: w13 [2*shared_I, H], w2 [H, shared_I]."""
    assert cfg.shared_I > 0
    Is = cfg.shared_I
    w13 = _normal((2 * Is, cfg.H), 0.02, cfg.family_seed, _TAG_SHARED, 0, Is, cfg.H)
    w2 = _normal((cfg.H, Is), 0.02, cfg.family_seed, _TAG_SHARED, 1, Is, cfg.H)
    return w13.to(torch.bfloat16), w2.to(torch.bfloat16)


# Categorical distribution of E2M1 magnitude codes 0..7 (values 0, .5, 1,
# 1.5, 2, 3, 4, 6): roughly the histogram an N(0,1) block scaled by 2.56 lands
# on.  Sign is a fair coin.  Block scale codes: 2^-7 (code 120) for most
# blocks, 2^-8 / 2^-6 for a few.
_E2M1_MAG_P = (0.078, 0.077, 0.141, 0.125, 0.121, 0.221, 0.142, 0.095)
_E8M0_CODES = (119, 120, 121)
_E8M0_P = (0.02, 0.925, 0.055)
# "wide": every code from 100 to 140 equally likely (scales 2^-27 .. 2^13)
_E8M0_WIDE = tuple(range(100, 141))


def _categorical(p, n: int, g: torch.Generator) -> torch.Tensor:
    """n draws of indices 0..len(p)-1 with probabilities p (inverse CDF)."""
    cdf = torch.tensor(np.cumsum(p) / np.sum(p), dtype=torch.float64)
    u = torch.rand(n, generator=g, dtype=torch.float64)
    return torch.searchsorted(cdf, u, right=True).clamp_(max=len(p) - 1)


def _mx_block(rows: int, cols: int, *parts: int, wide: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """MXFP4 codes [rows, cols/2] (low nibble = even column) and E8M0 scales
    [rows, cols/32] for a rows x cols weight (cols = reduction dimension).
    wide: block scale codes uniform over 100..140 instead of mostly 120."""
    g = _gen(*parts)
    mag = _categorical(_E2M1_MAG_P, rows * cols, g).to(torch.uint8)
    sign = torch.randint(0, 2, (rows * cols,), generator=g, dtype=torch.uint8)
    nib = (mag | (sign << 3)).view(rows, cols)
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).contiguous()
    table = _E8M0_WIDE if wide else _E8M0_CODES
    sidx = _categorical((1.0,) * len(table) if wide else _E8M0_P, rows * (cols // 32), g)
    scales = torch.tensor(table, dtype=torch.uint8)[sidx].view(rows, cols // 32)
    return codes, scales.contiguous()


def draw_expert_mx(cfg: LayerConfig, e: int):
    """Expert e's W4A8 weights: (w13_codes [2I, H/2], w13_scales [2I, H/32],
    w2_codes [H, I/2], w2_scales [H, I/32]), all uint8."""
    wide = cfg.mx_scales == "wide"
    c13, s13 = _mx_block(2 * cfg.I, cfg.H, cfg.family_seed, _TAG_MX_W13, e, cfg.I, cfg.H, wide=wide)
    c2, s2 = _mx_block(cfg.H, cfg.I, cfg.family_seed, _TAG_MX_W2, e, cfg.I, cfg.H, wide=wide)
    return c13, s13, c2, s2


def draw_shared_mx(cfg: LayerConfig):
    """The shared expert in W4A8: (w13_codes [2*shared_I, H/2], w13_scales,
    w2_codes [H, shared_I/2], w2_scales), same distributions as the routed
    experts."""
    assert cfg.shared_I > 0
    Is = cfg.shared_I
    wide = cfg.mx_scales == "wide"
    c13, s13 = _mx_block(2 * Is, cfg.H, cfg.family_seed, _TAG_MX_SHARED, 0, Is, cfg.H, wide=wide)
    c2, s2 = _mx_block(cfg.H, Is, cfg.family_seed, _TAG_MX_SHARED, 1, Is, cfg.H, wide=wide)
    return c13, s13, c2, s2


def describe(cfg: LayerConfig) -> dict:
    d = dataclasses.asdict(cfg)
    d["R"] = cfg.R
    return d


def draw_layer(cfg: LayerConfig, progress=None) -> dict:
    """All inputs of one layer as CPU tensors (weights stacked over experts).

    bf16: w13 [E, 2I, H], w2 [E, H, I] (+ shared_w13, shared_w2).
    w4a8: w13 codes [E, 2I, H/2], w13_scales [E, 2I, H/32], w2 codes
    [E, H, I/2], w2_scales [E, H, I/32] (+ the shared expert's codes and
    scales)."""
    t = {"x": draw_x(cfg), "wr": draw_router(cfg), "bias": draw_bias(cfg)}
    E = cfg.E
    if cfg.fmt == "bf16":
        w13 = torch.empty((E, 2 * cfg.I, cfg.H), dtype=torch.bfloat16)
        w2 = torch.empty((E, cfg.H, cfg.I), dtype=torch.bfloat16)
        for e in range(E):
            w13[e], w2[e] = draw_expert_bf16(cfg, e)
            if progress is not None and (e % 32 == 31 or e == E - 1):
                progress(f"{cfg.name}: drew experts 0..{e}")
        t["w13"], t["w2"] = w13, w2
        if cfg.shared_I:
            t["shared_w13"], t["shared_w2"] = draw_shared_bf16(cfg)
    else:
        c13 = torch.empty((E, 2 * cfg.I, cfg.H // 2), dtype=torch.uint8)
        s13 = torch.empty((E, 2 * cfg.I, cfg.H // 32), dtype=torch.uint8)
        c2 = torch.empty((E, cfg.H, cfg.I // 2), dtype=torch.uint8)
        s2 = torch.empty((E, cfg.H, cfg.I // 32), dtype=torch.uint8)
        for e in range(E):
            c13[e], s13[e], c2[e], s2[e] = draw_expert_mx(cfg, e)
            if progress is not None and (e % 32 == 31 or e == E - 1):
                progress(f"{cfg.name}: drew experts 0..{e}")
        t["w13"], t["w13_scales"], t["w2"], t["w2_scales"] = c13, s13, c2, s2
        if cfg.shared_I:
            (t["shared_w13"], t["shared_w13_scales"], t["shared_w2"],
             t["shared_w2_scales"]) = draw_shared_mx(cfg)
    return t


def draw_norm_inputs(T: int, H: int, seed: int):
    """Inputs of the residual add + RMSNorm before the layer: hidden states
    x and residual [T, H] bf16 ~ N(0,1), and the norm weight [H] bf16 ~
    N(1, 0.1) (RMSNorm weights start at one)."""
    x = _normal((T, H), 1.0, seed, _TAG_NORM_X, T, H).to(torch.bfloat16)
    r = _normal((T, H), 1.0, seed, _TAG_NORM_RES, T, H).to(torch.bfloat16)
    w = (1.0 + _normal((H,), 0.1, seed, _TAG_NORM_W, H)).to(torch.bfloat16)
    return x, r, w


def draw_combine_inputs(T: int, k: int, H: int, seed: int):
    """Stand-ins for a layer's expert outputs at the combine: rows y
    [T*k, H] bf16 ~ N(0, 0.05) (the size of expert outputs at these
    shapes), pair positions [T*k] int32 = a random permutation of the rows,
    and top-k weights [T, k] fp32 ~ U(0, 2/k)."""
    R = T * k
    y = _normal((R, H), 0.05, seed, _TAG_CMB_Y, R, H).to(torch.bfloat16)
    pos = torch.randperm(R, generator=_gen(seed, _TAG_CMB_PERM, R)).to(torch.int32)
    w = torch.rand((T, k), generator=_gen(seed, _TAG_CMB_W, T, k)) * (2.0 / k)
    return y, pos, w
