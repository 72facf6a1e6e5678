"""Seeded synthetic inputs for the MoE-layer forward.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It only *draws* tensors; it holds none of the layer's arithmetic
(no routing, no activation, no quantisation of activations).  Every tensor has
its own seed derived from (base seed, tensor name[, expert]), so any expert's
weights can be regenerated on their own.

Shapes follow the model descriptions:
  * Step-3.5-Flash: 288 routed experts, top-8, expert and shared intermediate
    1280, router scaling 3.0, normalised expert weights (page "MAX 中
    Step-3.5-Flash 架构解析…", config table of Step3p5Config).  Its hidden size
    is not printed; 4096 follows exactly from the parameter counts of the
    Megatron-Bridge "Step-3.5-Flash" verification cards (total vs. per-EP8-rank
    parameters, 42 MoE layers, 3 matrices of hidden x 1280 per expert).
  * Step-5-Preview: hidden 4096, 352 routed experts, top-8, one shared expert,
    expert/shared intermediate 1536 (NeMo AutoModel page "Step-5-Preview",
    Model Architecture table); routed experts in FP8 E4M3 with 128x128 block
    scales (miles page "Step-5-Preview", section 1 Model Introduction).

Distributions: activations N(0,1) (a normed hidden state), every weight
N(0, 0.02), router bias U(-0.1, 0.1) in fp32, hot-expert skew for the decode
case, FP8 block scales U(0.5, 2) x block-absmax / 448.

Tensors are drawn with torch's own generator on the device they will live on;
a host copy for the oracle is made with ``.cpu()`` so both sides see identical
bits.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One MoE layer's configuration; field names follow Step3p5Config."""
    hidden_size: int
    num_experts: int
    top_k: int
    moe_intermediate_size: int
    share_expert_dim: int
    router_scaling_factor: float = 3.0
    norm_expert_weight: bool = True
    swiglu_limit: float = 0.0          # routed experts; 0 means no clipping
    swiglu_limit_shared: float = 0.0   # shared expert; 0 means no clipping
    expert_dtype: str = "bf16"         # "bf16" or "fp8" (E4M3FN, 128x128 block scales)
    out_dtype: str = "fp32"            # "fp32" or "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    cfg: MoEConfig
    hot_fraction: float = 0.0   # fraction of experts that receive a bias boost
    hot_bias: float = 0.0       # added to the hot experts' router bias
    x_scale: float = 1.0        # multiplies the activations (clip-stress cases)


def _mk(H, E, k, I, Is, limit, limit_sh, **kw):
    return MoEConfig(hidden_size=H, num_experts=E, top_k=k, moe_intermediate_size=I,
                     share_expert_dim=Is, swiglu_limit=limit, swiglu_limit_shared=limit_sh, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny layer the oracle finishes in CPU seconds
    "tiny": Workload("tiny", 64, _mk(256, 16, 4, 128, 128, 7.0, 0.0)),
    # Step-3.5-Flash-shaped prefill, 4096 tokens, no clipping
    "step35_prefill": Workload("step35_prefill", 4096, _mk(4096, 288, 8, 1280, 1280, 0.0, 0.0)),
    # Step-5-Preview-shaped prefill, one 8192-token sequence, limit 7 on both
    "step5_prefill": Workload("step5_prefill", 8192, _mk(4096, 352, 8, 1536, 1536, 7.0, 7.0)),
    # Step-5-Preview-shaped decode: 64 tokens, +1.0 bias on a seeded 10% of experts
    "step5_decode": Workload("step5_decode", 64, _mk(4096, 352, 8, 1536, 1536, 7.0, 7.0),
                             hot_fraction=0.1, hot_bias=1.0),
    # same decode with the hot bias calibrated so the hot experts take about
    # half of the selections (+1.0 gives them all of them)
    "step5_decode_half": Workload("step5_decode_half", 64, _mk(4096, 352, 8, 1536, 1536, 7.0, 7.0),
                                  hot_fraction=0.1, hot_bias=0.15),
    # one rank's share of the Step-5 prefill under 8-way expert parallelism:
    # 44 of the 352 experts, the 65,536 token-expert pairs of 8192 tokens
    # (about 1490 rows per expert, so the expert GEMMs are MFMA-bound)
    "ep_rank_proxy": Workload("ep_rank_proxy", 8192, _mk(4096, 44, 8, 1536, 1536, 7.0, 7.0)),
    # Step-5-Preview-shaped prefill with FP8 E4M3 routed experts
    "step5_fp8_prefill": Workload("step5_fp8_prefill", 8192,
                                  _mk(4096, 352, 8, 1536, 1536, 7.0, 7.0, expert_dtype="fp8")),
}


def _seed(base: int, name: str, idx: int = 0) -> int:
    return (base * 1_000_003 + zlib.crc32(name.encode()) * 4099 + idx) & 0x7FFF_FFFF_FFFF


def _gen(device, base: int, name: str, idx: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(base, name, idx))
    return g


def _normal(shape, std, device, base, name, idx=0):
    g = _gen(device, base, name, idx)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _uniform(shape, lo, hi, device, base, name, idx=0):
    g = _gen(device, base, name, idx)
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def fp8_block_quantise_weights(w: torch.Tensor, u: torch.Tensor):
    """Turn one expert's fp32 weight [N, K] into E4M3FN codes + 128x128 block scales.

    scale[b] = u[b] * absmax(block b) / 448; codes = E4M3FN(w / scale) with the
    ratio clamped to the finite range.  The conversion is torch's own float8
    cast (round to nearest even); the codes and scales are then *inputs*: both
    the oracle and the GPU path take them as given.
    """
    N, K = w.shape
    nb, kb = N // 128, K // 128
    blocks = w.reshape(nb, 128, kb, 128)
    amax = blocks.abs().amax(dim=(1, 3))                       # [nb, kb]
    scale = u * amax / 448.0
    scale = torch.where(scale > 0, scale, torch.ones_like(scale))
    q = (blocks / scale[:, None, :, None]).clamp(-448.0, 448.0)
    codes = q.reshape(N, K).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.contiguous()


def make_inputs(wl: Workload, device="cpu", seed: int = 0,
                experts: Optional[list] = None) -> Dict[str, torch.Tensor]:
    """Draw every tensor of the layer for workload ``wl`` on ``device``.

    Returns a dict with x [T,H] bf16, w_router [E,H] bf16, router_bias [E] f32,
    w13 [E,2I,H] (bf16, or uint8 E4M3FN codes), w13_scale [E,2I/128,H/128] f32
    (FP8 only), w2 [E,H,I], w2_scale [E,H/128,I/128] (FP8 only),
    ws13 [2Is,H] bf16, ws2 [H,Is] bf16, and hot_experts (long) when skewed.
    """
    c = wl.cfg
    T, H, E, I, Is = wl.T, c.hidden_size, c.num_experts, c.moe_intermediate_size, c.share_expert_dim
    bf = torch.bfloat16
    out: Dict[str, torch.Tensor] = {}
    out["x"] = (_normal((T, H), 1.0, device, seed, "x") * wl.x_scale).to(bf)
    out["w_router"] = _normal((E, H), 0.02, device, seed, "w_router").to(bf)
    bias = _uniform((E,), -0.1, 0.1, device, seed, "router_bias")
    if wl.hot_fraction > 0:
        n_hot = int(E * wl.hot_fraction)
        g = _gen("cpu", seed, "hot_set")
        hot = torch.randperm(E, generator=g)[:n_hot].to(device)
        bias[hot] += wl.hot_bias
        out["hot_experts"] = hot
    out["router_bias"] = bias.contiguous()
    fp8 = c.expert_dtype == "fp8"
    ex = range(E)
    w13 = torch.empty((E, 2 * I, H), dtype=torch.uint8 if fp8 else bf, device=device)
    w2 = torch.empty((E, H, I), dtype=torch.uint8 if fp8 else bf, device=device)
    if fp8:
        w13s = torch.empty((E, 2 * I // 128, H // 128), dtype=torch.float32, device=device)
        w2s = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device=device)
    for e in ex:
        if experts is not None and e not in experts:
            continue
        a = _normal((2 * I, H), 0.02, device, seed, "w13", e)
        b = _normal((H, I), 0.02, device, seed, "w2", e)
        if fp8:
            ua = _uniform((2 * I // 128, H // 128), 0.5, 2.0, device, seed, "w13_u", e)
            ub = _uniform((H // 128, I // 128), 0.5, 2.0, device, seed, "w2_u", e)
            w13[e], w13s[e] = fp8_block_quantise_weights(a, ua)
            w2[e], w2s[e] = fp8_block_quantise_weights(b, ub)
        else:
            w13[e] = a.to(bf)
            w2[e] = b.to(bf)
        del a, b
    out["w13"], out["w2"] = w13, w2
    if fp8:
        out["w13_scale"], out["w2_scale"] = w13s, w2s
    if Is > 0:
        out["ws13"] = _normal((2 * Is, H), 0.02, device, seed, "ws13").to(bf)
        out["ws2"] = _normal((H, Is), 0.02, device, seed, "ws2").to(bf)
    return out


RMS_NORM_EPS = 1e-5


def block_inputs(wl: Workload, device="cpu", seed: int = 0) -> Dict[str, object]:
    """The residual stream in front of the layer: resid [T,H] fp32, N(0,1)
    rows each scaled by 2^U(-2, 4) (rows of very different size, as the
    residual stream grows with depth), the stored zero-centred norm weight
    norm_weight [H] fp32 ~ N(0, 0.1), and eps."""
    T, H = wl.T, wl.cfg.hidden_size
    row = torch.exp2(_uniform((T, 1), -2.0, 4.0, device, seed, "resid_row_scale"))
    resid = (_normal((T, H), 1.0, device, seed, "resid") * row).contiguous()
    g = _normal((H,), 0.1, device, seed, "norm_weight").contiguous()
    return {"resid": resid, "norm_weight": g, "eps": RMS_NORM_EPS}


def random_expert_ids(wl: Workload, device="cpu", seed: int = 0) -> torch.Tensor:
    """A seeded stand-in for a replayed expert choice: [T,k] int32, k distinct
    experts per token drawn uniformly (the first k of a random permutation)."""
    c = wl.cfg
    g = _gen("cpu", seed, "replay_ids")
    keys = torch.rand((wl.T, c.num_experts), generator=g)
    return keys.argsort(dim=1)[:, :c.top_k].to(torch.int32).contiguous().to(device)


def workload(name: str, **overrides) -> Workload:
    wl = WORKLOADS[name]
    if not overrides:
        return wl
    cfg_fields = {f.name for f in dataclasses.fields(MoEConfig)}
    cfg_over = {k: v for k, v in overrides.items() if k in cfg_fields}
    wl_over = {k: v for k, v in overrides.items() if k not in cfg_fields}
    cfg = dataclasses.replace(wl.cfg, **cfg_over)
    return dataclasses.replace(wl, cfg=cfg, **wl_over)
