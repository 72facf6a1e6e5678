"""GPU parity of the training path: moe_layer_forward_train and
moe_layer_backward against the oracle's backward (bf16 pre-activations, the
mode in which the clamps decide on the same bf16 values as the kernels).

Both sides run the same expert choice: a seeded random choice replayed on
both, or the oracle's own routing replayed on both (full size), so no
near-tie can send the two to different experts.  Each gradient tensor is
compared element by element and by its RMS error (tolerances derived
below); experts without rows must get exact zeros.
"""
import sys

import numpy as np
import pytest
import torch

import moe_inputs as mi
import sparse_moe_layer_route_amd as moe
from oracle import oracle as orc
from parity import TOL_BF16, max_err_over_rms

pytestmark = pytest.mark.gpu

DEV = "cuda"

# Every product of the backward reads bf16 operands (dout scaled by the gate
# weight, dgu, the saved h and x) and accumulates in fp32.  A rounding to
# bf16 (round to nearest even, 8 significant bits) leaves a relative error
# uniform within half a unit, about 1.6e-3 standard deviation; the weight
# gradients and dx see two such roundings in series (dy, then dgu): about
# 2.3e-3, which is what the RMS error over a tensor comes to (TOL_GRAD_RMS =
# 5e-3 of the RMS value).  Element by element, an error is about that
# fraction of the element's terms: of its own size for a large element; for
# one that cancels to near zero, of the terms that cancel, which in a sum over
# few rows with many zero dgu (the clip-stress case: 16 rows per expert) can
# be many times the RMS.  The bound is TOL_GRAD_ABS x RMS + TOL_GRAD_REL x
# |value|, 5e-2 and 2e-2.  A wrong index, sign, term or clamp decision moves
# an element by order one of its size, and the RMS error with it.
TOL_GRAD_ABS = 5e-2
TOL_GRAD_REL = 2e-2
TOL_GRAD_RMS = 5e-3

GRADS = [("dx", "dx"), ("dw_router", "dw_router"), ("dw13", "dw13"), ("dw2", "dw2")]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    moe.load()


def host(inp):
    return {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inp.items()}


def dout_for(wl, seed=3):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((wl.T, wl.cfg.hidden_size), generator=g, dtype=torch.float32)


def compare(name, gpu, ref):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    err, rms = max_err_over_rms(g, r)
    d = np.abs(g - r)
    rel = float(np.sqrt((d ** 2).mean()) / rms)
    worst = float((d / (TOL_GRAD_ABS * rms + TOL_GRAD_REL * np.abs(r))).max())
    say(f"  {name}: max_err/rms = {err:.3e}, rms_err/rms = {rel:.3e}, worst/bound = {worst:.2f} (rms {rms:.3e})")
    assert worst <= 1.0 and rel <= TOL_GRAD_RMS, name


SMALL = {
    "tiny": dict(),
    "tiny_clip_stress": dict(x_scale=40.0),
    "one_token": dict(T=1),
    "ragged_130_tokens_20_experts": dict(T=130, num_experts=20, top_k=3),
    "no_shared": dict(share_expert_dim=0, T=96),
    "no_norm": dict(norm_expert_weight=False, router_scaling_factor=2.5),
    "limits_off": dict(swiglu_limit=0.0, swiglu_limit_shared=0.0, x_scale=8.0),
    "all_experts_chosen": dict(top_k=16, T=40),
    "multi_tile_600_tokens": dict(T=600, num_experts=32, top_k=2),
    "wide_512_320": dict(hidden_size=512, moe_intermediate_size=320, share_expert_dim=320, T=300, num_experts=12,
                         top_k=2),
    "narrow_64": dict(hidden_size=64, moe_intermediate_size=64, share_expert_dim=64, T=200),
}


def run_train(wl, inp, ids, dout):
    out, saved = moe.moe_layer_forward_train(wl.cfg, inp, topk_ids=None if ids is None else ids.to(DEV))
    grads = moe.moe_layer_backward(wl.cfg, inp, saved, dout.to(DEV))
    torch.cuda.synchronize()
    return out, saved, grads


@pytest.mark.parametrize("name", list(SMALL))
def test_backward_small(name):
    wl = mi.workload("tiny", **SMALL[name])
    cfg, T, E = wl.cfg, wl.T, wl.cfg.num_experts
    say(f"[backward_small] {name} T={T} cfg={cfg}")
    inp = mi.make_inputs(wl, DEV, seed=0)
    ids = mi.random_expert_ids(wl, seed=21)
    dout = dout_for(wl)
    out, saved, g = run_train(wl, inp, ids, dout)
    h = host(inp)
    fwd = orc.layer(cfg, h, ids_in=ids, round_gu=True)
    err, _ = max_err_over_rms(out.float().cpu().numpy(), fwd["out"])
    say(f"  forward_train out: max_err/rms = {err:.3e}")
    assert err <= TOL_BF16
    ref = orc.backward(cfg, h, dout, ids_in=ids, round_gu=True)
    pairs = GRADS + ([("dws13", "dws13"), ("dws2", "dws2")] if cfg.share_expert_dim else [])
    for gk, rk in pairs:
        compare(gk, g[gk].cpu().numpy(), ref[rk])
    empty = np.setdiff1d(np.arange(E), ids.numpy().reshape(-1))
    for e in empty.tolist():
        for key in ("dw13", "dw2", "dw_router"):
            assert not g[key][e].any(), f"expert {e} has no rows but a nonzero {key}"


def test_backward_own_routing():
    """Without replay the training forward routes itself; on this seed no
    token is near a tie, so the oracle's routing is the same choice."""
    wl = mi.workload("tiny")
    say("[backward_own_routing]")
    inp = mi.make_inputs(wl, DEV, seed=0)
    dout = dout_for(wl)
    out, saved, g = run_train(wl, inp, None, dout)
    h = host(inp)
    ref = orc.backward(wl.cfg, h, dout, round_gu=True)
    P = wl.T * wl.cfg.top_k
    gpu_ids = saved[:P * 4].view(torch.int32).cpu().numpy().reshape(wl.T, -1)
    assert np.array_equal(gpu_ids, ref["ids"])
    for gk, rk in GRADS + [("dws13", "dws13"), ("dws2", "dws2")]:
        compare(gk, g[gk].cpu().numpy(), ref[rk])


def test_backward_deterministic_and_reusable():
    """Two backward calls on one state give the same bits; a zero dout gives
    zero gradients."""
    wl = mi.workload("tiny", T=257)
    inp = mi.make_inputs(wl, DEV, seed=0)
    ids = mi.random_expert_ids(wl, seed=5).to(DEV)
    dout = dout_for(wl).to(DEV)
    _, saved = moe.moe_layer_forward_train(wl.cfg, inp, topk_ids=ids)
    a = moe.moe_layer_backward(wl.cfg, inp, saved, dout)
    b = moe.moe_layer_backward(wl.cfg, inp, saved, dout)
    z = moe.moe_layer_backward(wl.cfg, inp, saved, torch.zeros_like(dout))
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
        assert not z[key].any(), key


def test_backward_zero_tokens():
    wl = mi.workload("tiny", T=0)
    inp = mi.make_inputs(wl, DEV, seed=0)
    out, saved = moe.moe_layer_forward_train(wl.cfg, inp)
    g = moe.moe_layer_backward(wl.cfg, inp, saved, torch.zeros((0, wl.cfg.hidden_size), device=DEV))
    torch.cuda.synchronize()
    for key in ("dw13", "dw2", "dw_router", "dws13", "dws2"):
        assert not g[key].any(), key


def test_backward_full_size_step5_prefill():
    """8192 tokens, 352 experts, H 4096, I 1536, replaying the oracle's own
    routing on both sides: dx on a seeded token sample, the weight and router
    gradients of the expert with the most rows (several 256-row tiles), of a
    median one, and zeros for an expert without rows."""
    wl = mi.WORKLOADS["step5_prefill"]
    cfg, T, E, k = wl.cfg, wl.T, wl.cfg.num_experts, wl.cfg.top_k
    say(f"[backward_full] T={T}")
    inp = mi.make_inputs(wl, DEV, seed=0)
    h = host(inp)
    ids, _ = orc.route(cfg, h["x"], h["w_router"], h["router_bias"])
    ids = torch.from_numpy(ids)
    dout = dout_for(wl)
    out, saved, g = run_train(wl, inp, ids, dout)
    say("  gpu done")
    counts = np.bincount(ids.numpy().reshape(-1), minlength=E)
    order = np.argsort(counts)
    experts = [int(order[-1]), int(order[E // 2])]
    empty = np.nonzero(counts == 0)[0]
    rng = np.random.default_rng(4)
    toks = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 22, replace=False)]))
    ref = orc.backward(cfg, h, dout, tokens=toks, experts=experts, shared=False, ids_in=ids, round_gu=True)
    say(f"  experts {experts} with {counts[experts].tolist()} rows; {toks.size} tokens")
    compare("dx", g["dx"].cpu().numpy()[toks], ref["dx"])
    compare("dw_router", g["dw_router"].cpu().numpy()[experts], ref["dw_router"])
    for q, e in enumerate(experts):
        compare(f"dw13[{e}]", g["dw13"][e].cpu().numpy(), ref["dw13"][q])
        compare(f"dw2[{e}]", g["dw2"][e].cpu().numpy(), ref["dw2"][q])
    if empty.size:
        e = int(empty[0])
        assert not g["dw13"][e].any() and not g["dw2"][e].any() and not g["dw_router"][e].any()
