"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test pins one part of the layer (routing, activation, expert MLP, combine,
permutation, FP8 codec) to a closed form, a page-printed number, a brute-force
second implementation, or a library routine (torch.nn.functional, torch's
float8 cast, numpy's stable sort) that reduces to the same definition.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import moe_inputs as mi
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(a):
    return torch.as_tensor(a, dtype=torch.float32).to(torch.bfloat16)


def tiny(**over):
    return mi.workload("tiny", **over)


# --------------------------------------------------------------------------
# page-printed facts


def test_page_facts_fix_the_configs():
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    s35 = facts["step35_config"]
    c1 = mi.WORKLOADS["step35_prefill"].cfg
    assert (c1.num_experts, c1.top_k, c1.moe_intermediate_size, c1.share_expert_dim) == (
        s35["moe_num_experts"], s35["moe_top_k"], s35["moe_intermediate_size"], s35["share_expert_dim"])
    assert c1.router_scaling_factor == s35["moe_router_scaling_factor"]
    assert c1.norm_expert_weight == s35["norm_expert_weight"]
    s5 = facts["step5_architecture"]
    for name in ("step5_prefill", "step5_decode", "step5_fp8_prefill"):
        c = mi.WORKLOADS[name].cfg
        assert (c.hidden_size, c.num_experts, c.top_k, c.moe_intermediate_size, c.share_expert_dim) == (
            s5["hidden_size"], s5["routed_experts"], s5["top_k"], s5["expert_intermediate_size"],
            s5["shared_intermediate_size"])
        assert c.router_scaling_factor == facts["step5_routing"]["router_scaling_factor"]


def test_step35_hidden_size_follows_from_parameter_counts():
    """Expert parameters = (total - per_rank) * ep / (ep - 1); they are
    n_moe_layers * E * 3 * H * I, which fixes H = 4096 exactly."""
    f = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    pc, cfg, lay = f["step35_param_counts"], f["step35_config"], f["step35_layers"]
    ep = pc["ep"]
    diff = pc["total_parameters"] - pc["per_rank_parameters_ep8"]
    assert diff * ep % (ep - 1) == 0
    expert_params = diff * ep // (ep - 1)
    n_layers = lay["moe_layer_last"] - lay["moe_layer_first"] + 1
    per_h = n_layers * cfg["moe_num_experts"] * 3 * cfg["moe_intermediate_size"]
    assert expert_params % per_h == 0
    assert expert_params // per_h == 4096 == mi.WORKLOADS["step35_prefill"].cfg.hidden_size


def test_step5_expert_tensor_sizes_match_fused_layout():
    """The 12 and 24 MiB bf16 expert tensors are one expert's [H, I] down
    projection and fused [2I, H] gate|up projection."""
    f = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    H, I = f["step5_architecture"]["hidden_size"], f["step5_architecture"]["expert_intermediate_size"]
    assert sorted(f["step5_routing"]["fp8_expert_tensor_mib"]) == [H * I * 2 // 2**20, 2 * I * H * 2 // 2**20]


# --------------------------------------------------------------------------
# activation: closed-form scalars


@pytest.mark.parametrize("g,u,L,want", [
    (10.0, 10.0, 7.0, 49.0),                       # both factors clip
    (10.0, -10.0, 7.0, -49.0),                     # up clips from below
    (-10.0, 100.0, 7.0, 7.0 * -4.539786870243442e-04),  # silu(-10) * 7
    (1.0, 2.0, 7.0, 2.0 * 0.7310585786300049),    # nothing clips: 2 * silu(1)
    (1.0, 2.0, 0.0, 2.0 * 0.7310585786300049),
    (0.0, 5.0, 7.0, 0.0),
    (20.0, 3.0, 0.0, 60.0 * 0.9999999979388463),   # L = 0: no clip at all
])
def test_act_closed_forms(orc, g, u, L, want):
    assert orc.act(g, u, L) == pytest.approx(want, rel=1e-12, abs=1e-15)


def test_silu_closed_forms(orc):
    assert orc.lib().orc_silu(0.0) == 0.0
    assert orc.lib().orc_silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert orc.lib().orc_silu(-1.0) == pytest.approx(-0.2689414213699951, rel=1e-15)


def test_act_limit_zero_is_unclipped(orc):
    rng = np.random.default_rng(0)
    for g, u in rng.normal(0, 30, (200, 2)):
        want = float(F.silu(torch.tensor(g, dtype=torch.float64)) * u)
        assert orc.act(g, u, 0.0) == pytest.approx(want, rel=1e-13, abs=1e-13)


# --------------------------------------------------------------------------
# routing


def _inputs(wl, seed=0):
    return mi.make_inputs(wl, "cpu", seed)


def test_route_zero_input_picks_largest_bias(orc):
    """x = 0 -> logits 0 -> s = 0.5 -> c = 0.5 + b: the ids are the k largest
    biases; weights are scale/k with normalisation, scale*0.5 without."""
    wl = tiny()
    inp = _inputs(wl)
    x = torch.zeros_like(inp["x"])
    b = inp["router_bias"]
    ids, w = orc.route(wl.cfg, x, inp["w_router"], b)
    k = wl.cfg.top_k
    want = sorted(range(wl.cfg.num_experts), key=lambda e: (-float(b[e]), e))[:k]
    assert (ids == np.array(want, np.int32)[None, :]).all()
    assert np.allclose(w, 3.0 / k, rtol=0, atol=1e-7)
    cfg_nonorm = dataclasses.replace(wl.cfg, norm_expert_weight=False)
    _, w2 = orc.route(cfg_nonorm, x, inp["w_router"], b)
    assert np.allclose(w2, 1.5, rtol=0, atol=0)


def test_route_ties_go_to_lower_index(orc):
    wl = tiny()
    inp = _inputs(wl)
    x = torch.zeros_like(inp["x"])
    ids, _ = orc.route(wl.cfg, x, inp["w_router"], torch.zeros(wl.cfg.num_experts))
    assert (ids == np.arange(wl.cfg.top_k, dtype=np.int32)[None, :]).all()
    # duplicate router rows give exactly equal scores: the lower index wins
    wg = inp["w_router"].clone()
    wg[9] = wg[3]
    b = torch.zeros(wl.cfg.num_experts)
    b[3] = b[9] = 5.0
    ids, _ = orc.route(wl.cfg, inp["x"], wg, b)
    assert (ids[:, 0] == 3).all() and (ids[:, 1] == 9).all()


def test_route_weights_sum_to_scale(orc):
    wl = tiny()
    inp = _inputs(wl)
    ids, w = orc.route(wl.cfg, inp["x"], inp["w_router"], inp["router_bias"])
    assert np.abs(w.astype(np.float64).sum(1) - 3.0).max() < 1e-6
    assert all(len(set(r)) == wl.cfg.top_k for r in ids.tolist())


def test_route_matches_full_sort_of_fp64_scores(orc):
    """Brute force: score every expert in double precision with torch, sort
    all E of them, keep the first k (ties to the lower index)."""
    wl = tiny()
    inp = _inputs(wl)
    ids, w, lg, cs = orc.route(wl.cfg, inp["x"], inp["w_router"], inp["router_bias"], want_scores=True)
    logits = inp["x"].double() @ inp["w_router"].double().T
    s = torch.sigmoid(logits)
    c = s + inp["router_bias"].double()
    assert np.allclose(lg, logits.numpy(), rtol=1e-6, atol=1e-6)
    for t in range(wl.T):
        order = sorted(range(wl.cfg.num_experts), key=lambda e: (-float(c[t, e]), e))
        srt = sorted(float(v) for v in c[t])[::-1]
        gap = srt[wl.cfg.top_k - 1] - srt[wl.cfg.top_k]
        if gap > 1e-6:
            assert sorted(ids[t].tolist()) == sorted(order[:wl.cfg.top_k])
            assert ids[t].tolist() == order[:wl.cfg.top_k]       # descending order too
        sw = s[t, ids[t]]
        assert np.allclose(w[t], (3.0 * sw / sw.sum()).numpy(), rtol=1e-6)


def test_route_nan_inf_guard(orc):
    wl = tiny()
    inp = _inputs(wl)
    x = inp["x"].clone()
    x[0] = float("nan")
    x[1, 5] = float("inf")
    x[2, :] = float("-inf")
    wg = inp["w_router"].clone()
    wg[7, 3] = float("nan")
    ids, _ = orc.route(wl.cfg, x, wg, inp["router_bias"])
    assert ids.min() >= 0 and ids.max() < wl.cfg.num_experts
    assert ids[0].tolist() == list(range(wl.cfg.top_k))      # every score NaN -> lowest indices
    for r in ids.tolist():
        assert len(set(r)) == wl.cfg.top_k


# --------------------------------------------------------------------------
# expert MLPs and combine against torch library routines


def _torch_mlp(x, w13, w2, L):
    """Textbook SwiGLU MLP in float64 with torch: F.linear + F.silu."""
    I = w2.shape[1]
    gu = F.linear(x.double(), w13.double())
    g, u = gu[..., :I], gu[..., I:]
    sg = F.silu(g)
    if L:
        sg = sg.clamp(max=L)
        u = u.clamp(-L, L)
    return F.linear(sg * u, w2.double())


def test_single_expert_is_textbook_swiglu(orc):
    wl = tiny(num_experts=1, top_k=1, share_expert_dim=0, router_scaling_factor=1.0, swiglu_limit=0.0)
    inp = _inputs(wl)
    res = orc.layer(wl.cfg, inp)
    want = _torch_mlp(inp["x"], inp["w13"][0], inp["w2"][0], 0.0).numpy()
    assert (res["ids"] == 0).all() and np.allclose(res["w"], 1.0)
    assert np.abs(res["out"] - want).max() <= 1e-5 * np.abs(want).max()


def test_identical_experts_give_scaled_mlp_plus_shared(orc):
    wl = tiny()
    inp = _inputs(wl)
    inp["w13"][:] = inp["w13"][0]
    inp["w2"][:] = inp["w2"][0]
    res = orc.layer(wl.cfg, inp)
    want = 3.0 * _torch_mlp(inp["x"], inp["w13"][0], inp["w2"][0], wl.cfg.swiglu_limit) + \
        _torch_mlp(inp["x"], inp["ws13"], inp["ws2"], wl.cfg.swiglu_limit_shared)
    assert np.abs(res["out"] - want.numpy()).max() <= 1e-5 * np.abs(want.numpy()).max()


def test_output_is_the_explicit_sum_over_chosen_experts(orc):
    wl = tiny(x_scale=40.0)      # clip stress: many SwiGLU inputs beyond the limit
    inp = _inputs(wl)
    res = orc.layer(wl.cfg, inp, want_parts=True)
    x = inp["x"]
    ref = _torch_mlp(x, inp["ws13"], inp["ws2"], wl.cfg.swiglu_limit_shared)
    assert np.abs(res["y_shared"] - ref.numpy()).max() <= 1e-5 * ref.abs().max().item()
    out = ref.clone()
    for t in range(wl.T):
        for j, e in enumerate(res["ids"][t].tolist()):
            y = _torch_mlp(x[t], inp["w13"][e], inp["w2"][e], wl.cfg.swiglu_limit)
            assert np.abs(res["y_routed"][t, j] - y.numpy()).max() <= 1e-5 * y.abs().max().item()
            out[t] += float(res["w"][t, j]) * y
    assert np.abs(res["out"] - out.numpy()).max() <= 1e-5 * out.abs().max().item()


def test_clip_stress_actually_clips(orc):
    """At limit 7 with activations x40 a large share of gate/up values is
    beyond the limit, so the stress case exercises the clip branch."""
    wl = tiny(x_scale=40.0)
    inp = _inputs(wl)
    gu = F.linear(inp["x"].double(), inp["w13"][0].double())
    frac = (gu.abs() > wl.cfg.swiglu_limit).double().mean().item()
    assert frac > 0.2


def test_output_linear_in_scaling_factor(orc):
    wl3 = tiny(share_expert_dim=0)
    wl1 = tiny(share_expert_dim=0, router_scaling_factor=1.0)
    inp = _inputs(wl3)
    o3 = orc.layer(wl3.cfg, inp)["out"].astype(np.float64)
    o1 = orc.layer(wl1.cfg, inp)["out"].astype(np.float64)
    assert np.abs(o3 - 3.0 * o1).max() <= 1e-6 * np.abs(o3).max()


def test_token_subset_equals_full_rows(orc):
    wl = tiny()
    inp = _inputs(wl)
    full = orc.layer(wl.cfg, inp)
    sub = orc.layer(wl.cfg, inp, tokens=[5, 17, 63])
    assert np.array_equal(sub["out"], full["out"][[5, 17, 63]])
    assert np.array_equal(sub["ids"], full["ids"][[5, 17, 63]])


@pytest.mark.parametrize("x_scale", [1.0, 40.0])
def test_oracle_matches_brute_force(orc, x_scale):
    wl = tiny(x_scale=x_scale)
    inp = _inputs(wl)
    toks = [0, 1, 2, 31, 62, 63]
    res = orc.layer(wl.cfg, inp, tokens=toks)
    f = lambda t: t.double().tolist()
    x = f(inp["x"])
    args = (f(inp["w_router"]), f(inp["router_bias"]), f(inp["w13"]), f(inp["w2"]), f(inp["ws13"]), f(inp["ws2"]))
    for r, t in enumerate(toks):
        ids, w, out, c = brute.token_forward(wl.cfg, x[t], *args)
        srt = sorted(c, reverse=True)
        if srt[wl.cfg.top_k - 1] - srt[wl.cfg.top_k] > 1e-6:
            assert res["ids"][r].tolist() == ids
        out = np.array(out)
        assert np.abs(res["out"][r] - out).max() <= 1e-5 * np.abs(out).max()
        assert np.allclose(res["w"][r], w, rtol=1e-6)


# --------------------------------------------------------------------------
# routing replay and static balanced routing


def _replay_ids(wl, seed):
    """k distinct experts per token, drawn at random (not the router's choice)."""
    rng = np.random.default_rng(seed)
    E, k = wl.cfg.num_experts, wl.cfg.top_k
    return np.stack([rng.choice(E, k, replace=False) for _ in range(wl.T)]).astype(np.int32)


def test_replay_of_own_choice_reproduces_route(orc):
    """Replaying the router's own choice gives back its ids and weights
    exactly; the bias plays no part once the choice is given."""
    wl = tiny()
    inp = _inputs(wl)
    ids, w = orc.route(wl.cfg, inp["x"], inp["w_router"], inp["router_bias"])
    ids2, w2 = orc.route(wl.cfg, inp["x"], inp["w_router"], None, ids_in=ids)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
    rnd = _replay_ids(wl, 1)
    _, wa = orc.route(wl.cfg, inp["x"], inp["w_router"], None, ids_in=rnd)
    _, wb = orc.route(wl.cfg, inp["x"], inp["w_router"], inp["router_bias"] * 100, ids_in=rnd)
    assert np.array_equal(wa, wb)


def test_replay_weights_zero_input_closed_form(orc):
    """x = 0 -> every raw score is 0.5, whatever the replayed ids (duplicates
    included): weights scale/k with normalisation, scale/2 without."""
    wl = tiny()
    inp = _inputs(wl)
    x = torch.zeros_like(inp["x"])
    ids = _replay_ids(wl, 2)
    ids[0, 1] = ids[0, 0]
    got, w = orc.route(wl.cfg, x, inp["w_router"], None, ids_in=ids)
    assert np.array_equal(got, ids)
    assert np.allclose(w, 3.0 / wl.cfg.top_k, rtol=0, atol=1e-7)
    _, w2 = orc.route(dataclasses.replace(wl.cfg, norm_expert_weight=False), x, inp["w_router"], None,
                      ids_in=ids)
    assert np.array_equal(w2, np.full_like(w2, 1.5))


def test_replay_clamps_out_of_range_ids(orc):
    wl = tiny()
    inp = _inputs(wl)
    E = wl.cfg.num_experts
    ids = _replay_ids(wl, 3)
    bad = ids.copy()
    bad[:, 0] = -7
    bad[:, 1] = E + 5
    fixed = ids.copy()
    fixed[:, 0] = 0
    fixed[:, 1] = E - 1
    g1, w1 = orc.route(wl.cfg, inp["x"], inp["w_router"], None, ids_in=bad)
    g2, w2 = orc.route(wl.cfg, inp["x"], inp["w_router"], None, ids_in=fixed)
    assert np.array_equal(g1, fixed) and np.array_equal(w1, w2)
    r1 = orc.layer(wl.cfg, inp, ids_in=bad, tokens=[0, 9])
    r2 = orc.layer(wl.cfg, inp, ids_in=fixed, tokens=[0, 9])
    assert np.array_equal(r1["out"], r2["out"])


@pytest.mark.parametrize("x_scale", [1.0, 40.0])
def test_replayed_layer_matches_brute_force(orc, x_scale):
    wl = tiny(x_scale=x_scale)
    inp = _inputs(wl)
    ids_in = _replay_ids(wl, 4)
    toks = [0, 1, 30, 63]
    res = orc.layer(wl.cfg, inp, tokens=toks, ids_in=ids_in)
    f = lambda t: t.double().tolist()
    x = f(inp["x"])
    args = (f(inp["w_router"]), f(inp["router_bias"]), f(inp["w13"]), f(inp["w2"]), f(inp["ws13"]), f(inp["ws2"]))
    for r, t in enumerate(toks):
        ids, w, out, _ = brute.token_forward(wl.cfg, x[t], *args, ids=ids_in[t].tolist())
        assert res["ids"][r].tolist() == ids
        assert np.allclose(res["w"][r], w, rtol=1e-6)
        out = np.array(out)
        assert np.abs(res["out"][r] - out).max() <= 1e-5 * np.abs(out).max()


def test_replayed_layer_of_own_choice_equals_layer(orc):
    wl = tiny()
    inp = _inputs(wl)
    ref = orc.layer(wl.cfg, inp)
    rep = orc.layer(wl.cfg, inp, ids_in=ref["ids"])
    for key in ("out", "ids", "w"):
        assert np.array_equal(ref[key], rep[key])


def test_replay_with_identical_experts_is_independent_of_ids(orc):
    """All experts equal and weights normalised: the routed part is
    scale x the one MLP for any choice, so out = 3 MLP(x) + shared(x)."""
    wl = tiny()
    inp = _inputs(wl)
    inp["w13"][:] = inp["w13"][0]
    inp["w2"][:] = inp["w2"][0]
    res = orc.layer(wl.cfg, inp, ids_in=_replay_ids(wl, 5))
    want = 3.0 * _torch_mlp(inp["x"], inp["w13"][0], inp["w2"][0], wl.cfg.swiglu_limit) + \
        _torch_mlp(inp["x"], inp["ws13"], inp["ws2"], wl.cfg.swiglu_limit_shared)
    assert np.abs(res["out"] - want.numpy()).max() <= 1e-5 * np.abs(want.numpy()).max()


@pytest.mark.parametrize("T,k,E", [(8192, 8, 352), (64, 8, 352), (7, 3, 5), (5, 4, 4), (1, 1, 1), (0, 2, 3),
                                   (100, 8, 288)])
def test_balanced_ids_are_balanced_and_distinct(orc, T, k, E):
    ids = orc.balanced_ids(T, k, E)
    assert ids.shape == (T, k) and ids.dtype == np.int32
    counts = np.bincount(ids.reshape(-1), minlength=E)
    P = T * k
    assert counts.sum() == P and counts.min() == P // E and counts.max() == -(-P // E)
    assert all(len(set(r)) == k for r in ids.tolist())
    assert ids.min(initial=0) >= 0 and ids.max(initial=0) < E
    # static: the same for every call, and token t's choice does not depend on T
    assert np.array_equal(orc.balanced_ids(T + 3, k, E)[:T], ids)


# --------------------------------------------------------------------------
# the steps either side of the layer: zero-centred RMSNorm, fp32 residual


def test_bf16_round_matches_torch_cast(orc):
    """Round to nearest even against torch's own fp32 -> bfloat16 cast, on
    exact ties (half-way between two bf16 values, both parities), values
    just off them, subnormals, the overflow edge, infinities and random."""
    ties = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -130 * 3, 3.0e38]
    vals = np.array(ties + [np.nextafter(np.float32(t), np.float32(0)) for t in ties[:3]] +
                    [np.nextafter(np.float32(t), np.float32(np.inf)) for t in ties[:3]] +
                    [0.0, -0.0, 1e-40, -3e-39, 3.3895e38, 3.4e38, np.inf, -np.inf], np.float32)
    rng = np.random.default_rng(0)
    vals = np.concatenate([vals, (rng.standard_normal(4000) * np.exp2(rng.integers(-60, 60, 4000))).astype(np.float32)])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_round(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, want)
    assert orc.bf16_round(float("nan")) & 0x7FFF > 0x7F80


def test_rmsnorm_matches_torch_rms_norm(orc):
    """torch.nn.functional.rms_norm in float64 with weight 1 + g, then
    torch's casts to fp32 and bf16, is the same definition."""
    wl = tiny(T=200, hidden_size=320)
    b = mi.block_inputs(wl)
    x = orc.rmsnorm(b["resid"], b["norm_weight"], b["eps"])
    H = wl.cfg.hidden_size
    ref = F.rms_norm(b["resid"].double(), (H,), weight=1.0 + b["norm_weight"].double(), eps=b["eps"])
    ref = ref.float().bfloat16()
    assert torch.equal(x.view(torch.int16), ref.view(torch.int16))


def test_rmsnorm_closed_forms(orc):
    H = 256
    g = mi.block_inputs(tiny())["norm_weight"]
    # a constant row c with eps = 0 normalises to sign(c) (1 + g)
    r = torch.tensor([[3.0] * H, [-0.25] * H], dtype=torch.float32)
    x = orc.rmsnorm(r, g, 0.0)
    assert torch.equal(x[0], (1.0 + g).bfloat16()) and torch.equal(x[1], (-(1.0 + g)).bfloat16())
    # scaling a row by a power of two changes nothing when eps = 0
    r = mi.block_inputs(tiny())["resid"]
    x0 = orc.rmsnorm(r, g, 0.0)
    for j in (-20, -3, 5, 40):
        assert torch.equal(orc.rmsnorm(r * 2.0 ** j, g, 0.0), x0)
    # g = 0: every row has mean square 1 up to bf16 rounding
    x1 = orc.rmsnorm(r, torch.zeros(H), 0.0).double()
    assert (x1.pow(2).mean(1) - 1.0).abs().max() < 1e-2
    # eps: a zero row stays zero; a tiny row is damped, not blown up
    z = orc.rmsnorm(torch.zeros(1, H), g, 1e-5)
    assert (z.float() == 0).all()
    small = orc.rmsnorm(torch.full((1, H), 1e-4), torch.zeros(H), 1e-5).float()
    assert torch.allclose(small, torch.full((1, H), 1e-4 / math.sqrt(1e-8 + 1e-5)), rtol=1e-2)


def test_block_is_residual_plus_layer_of_normed_input(orc):
    """resid_out = resid + layer(rmsnorm(resid)), the add in fp32: checked
    against the brute-force layer on the normalised rows."""
    wl = tiny()
    inp = dict(_inputs(wl), **mi.block_inputs(wl))
    toks = [0, 7, 63]
    res = orc.block(wl.cfg, inp, tokens=toks)
    x = res["x"]
    f = lambda t: t.double().tolist()
    args = (f(inp["w_router"]), f(inp["router_bias"]), f(inp["w13"]), f(inp["w2"]), f(inp["ws13"]), f(inp["ws2"]))
    for r, t in enumerate(toks):
        ids, _, out, c = brute.token_forward(wl.cfg, f(x[t]), *args)
        srt = sorted(c, reverse=True)
        assert srt[wl.cfg.top_k - 1] - srt[wl.cfg.top_k] > 1e-6
        want = inp["resid"][t].double().numpy() + np.array(out)
        scale = np.abs(np.array(out)).max()
        assert np.abs(res["resid_out"][r] - want).max() <= 1e-5 * scale + 4e-7 * np.abs(want).max()


# --------------------------------------------------------------------------
# backward (bf16 experts)


def _torch_layer64(cfg, inp, ids, round_gu=False):
    """The layer in float64 with torch ops, the expert choice ``ids`` held
    fixed; returns out and the leaf tensors (x, router, experts, shared).
    round_gu: the pre-activations take their bf16-rounded values (torch's
    cast) with the gradient passed straight through the rounding."""
    leaf = lambda t: t.double().clone().requires_grad_(True)
    x, wg, w13, w2 = leaf(inp["x"]), leaf(inp["w_router"]), leaf(inp["w13"]), leaf(inp["w2"])
    Is, I, L = cfg.share_expert_dim, cfg.moe_intermediate_size, cfg.swiglu_limit
    ws13 = leaf(inp["ws13"]) if Is else None
    ws2 = leaf(inp["ws2"]) if Is else None
    ids_t = torch.as_tensor(ids, dtype=torch.long)

    def mlp(xr, a, b, n, lim):
        gu = F.linear(xr, a)
        if round_gu:
            gu = gu + (gu.float().bfloat16().double() - gu).detach()
        g, u = gu[..., :n], gu[..., n:]
        sg = F.silu(g)
        if lim:
            sg = torch.clamp(sg, max=lim)
            u = torch.clamp(u, -lim, lim)
        return F.linear(sg * u, b)

    s = torch.sigmoid(F.linear(x, wg))
    sc = torch.gather(s, 1, ids_t)
    w = sc / sc.sum(1, keepdim=True) if cfg.norm_expert_weight else sc
    w = w * cfg.router_scaling_factor
    rows = []
    for t in range(x.shape[0]):
        acc = 0.0
        for j in range(ids_t.shape[1]):
            e = int(ids_t[t, j])
            acc = acc + w[t, j] * mlp(x[t], w13[e], w2[e], I, L)
        rows.append(acc)
    out = torch.stack(rows)
    if Is:
        out = out + mlp(x, ws13, ws2, Is, cfg.swiglu_limit_shared)
    return out, dict(x=x, w_router=wg, w13=w13, w2=w2, ws13=ws13, ws2=ws2)


def _dout(wl, seed=3):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((wl.T, wl.cfg.hidden_size), generator=g, dtype=torch.float32)


@pytest.mark.parametrize("over", [dict(), dict(x_scale=40.0), dict(norm_expert_weight=False, router_scaling_factor=2.5),
                                  dict(share_expert_dim=0), dict(swiglu_limit=0.0, swiglu_limit_shared=0.0),
                                  dict(T=24, num_experts=6, top_k=6)])
def test_backward_matches_torch_autograd(orc, over):
    """torch's autograd of the same layer in float64 (library routines:
    F.linear, F.silu, torch.clamp, torch.sigmoid), choice held fixed."""
    wl = tiny(**over)
    inp = _inputs(wl)
    dout = _dout(wl)
    res = orc.backward(wl.cfg, inp, dout)
    out, leaves = _torch_layer64(wl.cfg, inp, res["ids"])
    (out * dout.double()).sum().backward()
    pairs = [("dx", "x"), ("dw_router", "w_router"), ("dw13", "w13"), ("dw2", "w2")]
    if wl.cfg.share_expert_dim:
        pairs += [("dws13", "ws13"), ("dws2", "ws2")]
    for mine, name in pairs:
        want = leaves[name].grad.numpy()
        got = res[mine].astype(np.float64)
        scale = np.abs(want).max()
        assert scale > 0, name
        assert np.abs(got - want).max() <= 1e-6 * scale, (mine, np.abs(got - want).max() / scale)


@pytest.mark.parametrize("x_scale", [1.0, 40.0])
def test_backward_with_bf16_preactivations_matches_autograd(orc, x_scale):
    wl = tiny(x_scale=x_scale)
    inp = _inputs(wl)
    dout = _dout(wl)
    res = orc.backward(wl.cfg, inp, dout, round_gu=True)
    plain = orc.backward(wl.cfg, inp, dout)
    out, leaves = _torch_layer64(wl.cfg, inp, res["ids"], round_gu=True)
    (out * dout.double()).sum().backward()
    for mine, name in [("dx", "x"), ("dw_router", "w_router"), ("dw13", "w13"), ("dw2", "w2"), ("dws13", "ws13"),
                       ("dws2", "ws2")]:
        want = leaves[name].grad.numpy()
        got = res[mine].astype(np.float64)
        assert np.abs(got - want).max() <= 1e-6 * np.abs(want).max(), mine
    assert not np.array_equal(res["dw13"], plain["dw13"])      # the rounding is really applied
    fwd = orc.layer(wl.cfg, inp, ids_in=res["ids"], round_gu=True)["out"]
    want = out.detach().numpy()
    assert np.abs(fwd - want).max() <= 1e-6 * np.abs(want).max()


def test_backward_matches_finite_differences(orc):
    """Central differences of the brute-force forward (pure Python doubles,
    none of the oracle's code) on single weights and inputs."""
    wl = tiny(T=4, x_scale=3.0)
    inp = _inputs(wl)
    dout = _dout(wl)
    res = orc.backward(wl.cfg, inp, dout)
    f = lambda t: t.double().tolist()
    base = {k: f(inp[k]) for k in ("x", "w_router", "router_bias", "w13", "w2", "ws13", "ws2")}
    d = dout.double().tolist()

    def loss(p):
        tot = 0.0
        for t in range(wl.T):
            ids, _, out, _ = brute.token_forward(wl.cfg, p["x"][t], p["w_router"], p["router_bias"], p["w13"],
                                                 p["w2"], p["ws13"], p["ws2"], ids=res["ids"][t].tolist())
            tot += math.fsum(o * g for o, g in zip(out, d[t]))
        return tot

    e0 = int(res["ids"][1, 0])
    probes = [("x", (1, 5), res["dx"][1, 5]), ("x", (2, 100), res["dx"][2, 100]),
              ("w_router", (e0, 7), res["dw_router"][e0, 7]),
              ("w13", (e0, 3, 11), res["dw13"][e0, 3, 11]), ("w13", (e0, 128 + 3, 11), res["dw13"][e0, 131, 11]),
              ("w2", (e0, 9, 4), res["dw2"][e0, 9, 4]), ("ws13", (5, 6), res["dws13"][5, 6]),
              ("ws2", (6, 5), res["dws2"][6, 5])]
    eps = 1e-5
    for name, idx, got in probes:
        vals = []
        for sgn in (1, -1):
            p = {k: v for k, v in base.items()}
            p[name] = json.loads(json.dumps(base[name]))
            ref = p[name]
            for i in idx[:-1]:
                ref = ref[i]
            ref[idx[-1]] += sgn * eps
            vals.append(loss(p))
        fd = (vals[0] - vals[1]) / (2 * eps)
        assert abs(fd - got) <= 1e-5 * max(1.0, abs(fd)), (name, idx, fd, got)


def test_backward_is_linear_in_dout(orc):
    wl = tiny()
    inp = _inputs(wl)
    d = _dout(wl)
    a = orc.backward(wl.cfg, inp, d)
    b = orc.backward(wl.cfg, inp, d * 2.0)
    z = orc.backward(wl.cfg, inp, torch.zeros_like(d))
    for key in ("dx", "dw_router", "dw13", "dw2", "dws13", "dws2"):
        assert np.array_equal(b[key], 2.0 * a[key]), key
        assert not z[key].any(), key


def test_backward_selections_and_replay(orc):
    """Token and expert selections return the rows of the full result, and
    replaying the router's own choice changes nothing."""
    wl = tiny()
    inp = _inputs(wl)
    d = _dout(wl)
    full = orc.backward(wl.cfg, inp, d)
    sub = orc.backward(wl.cfg, inp, d, tokens=[3, 40], experts=[2, 9], shared=False)
    assert np.array_equal(sub["dx"], full["dx"][[3, 40]])
    for key in ("dw_router", "dw13", "dw2"):
        assert np.array_equal(sub[key], full[key][[2, 9]]), key
    rep = orc.backward(wl.cfg, inp, d, ids_in=full["ids"])
    for key in ("dx", "dw_router", "dw13", "dw2", "dws13", "dws2"):
        assert np.array_equal(rep[key], full[key]), key


def test_act_grad_closed_forms_and_clamp_convention(orc):
    # no clip: d/dg silu(g) u at g = 0 is u/2; d/du is silu(g)
    assert orc.act_grad(0.0, 3.0, 0.0) == pytest.approx((1.5, 0.0))
    g = 1.3
    sg = 1 / (1 + math.exp(-g))
    assert orc.act_grad(g, 2.0, 0.0) == pytest.approx((2.0 * sg * (1 + g * (1 - sg)), g * sg), rel=1e-14)
    # clipped factors pass nothing; the clamp's ends pass the gradient (as torch's clamp does)
    assert orc.act_grad(20.0, 1.0, 7.0)[0] == 0.0           # silu(20) > 7
    assert orc.act_grad(1.0, 9.0, 7.0)[1] == 0.0            # |u| > 7
    assert orc.act_grad(1.0, -9.0, 7.0)[1] == 0.0
    for u in (7.0, -7.0):
        t = torch.tensor(u, dtype=torch.float64, requires_grad=True)
        torch.clamp(t, -7.0, 7.0).backward()
        assert float(t.grad) == 1.0
        assert orc.act_grad(1.0, u, 7.0)[1] == pytest.approx(1.0 / (1 + math.exp(-1.0)))


# --------------------------------------------------------------------------
# permutation


def test_permute_matches_stable_sort(orc):
    wl = tiny()
    inp = _inputs(wl)
    ids, _ = orc.route(wl.cfg, inp["x"], inp["w_router"], inp["router_bias"])
    E = wl.cfg.num_experts
    counts, offs, r2p, p2r = orc.permute(ids, E)
    flat = ids.reshape(-1)
    assert counts.sum() == flat.size
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offs[0] == 0 and np.array_equal(np.diff(offs), counts)
    assert np.array_equal(r2p, np.argsort(flat, kind="stable"))      # library stable sort
    assert np.array_equal(p2r[r2p], np.arange(flat.size))
    for e in range(E):
        seg = r2p[offs[e]:offs[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


# --------------------------------------------------------------------------
# FP8 E4M3FN codec and the FP8 layer


def test_e4m3_decode_all_codes_against_torch(orc):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double()
    for code in range(256):
        v = orc.e4m3_decode(code)
        if math.isnan(ref[code]):
            assert math.isnan(v) and code in (0x7F, 0xFF)
        else:
            assert v == ref[code].item(), code
    assert orc.e4m3_decode(0x7E) == 448.0 and orc.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_encode_rne_against_torch(orc):
    finite = sorted({orc.e4m3_decode(c) for c in range(0x7F)})
    mids = [(a + b) / 2 for a, b in zip(finite[:-1], finite[1:])]
    rng = np.random.default_rng(1)
    vals = finite + mids + list(rng.uniform(-448, 448, 3000)) + list(rng.normal(0, 0.01, 1000))
    vals = [float(np.float32(v)) for v in vals]
    vals += [-v for v in vals]
    ref = torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    got = [orc.e4m3_encode(v) for v in vals]
    assert got == ref.tolist()
    # saturation beyond the finite range (torch's cast gives NaN there)
    assert orc.e4m3_encode(500.0) == 0x7E and orc.e4m3_encode(-1e9) == 0xFE
    assert orc.e4m3_encode(float("nan")) == 0x7F


def _torch_fp8_reference(cfg, inp, ids, w):
    """The FP8-mode layer with torch's own float8 cast and matmuls."""
    def deq_w(codes, scale):
        v = codes.view(torch.float8_e4m3fn).double()
        return v * scale.double().repeat_interleave(128, 0).repeat_interleave(128, 1)

    def quant_act(a):
        a = a.float()
        g = a.reshape(*a.shape[:-1], -1, 128)
        amax = g.abs().amax(-1, keepdim=True)
        s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q = (g / s).to(torch.float8_e4m3fn).float()
        return (q * s).reshape(a.shape)

    I, L = cfg.moe_intermediate_size, cfg.swiglu_limit
    xq = quant_act(inp["x"].float()).double()
    out = _torch_mlp(inp["x"], inp["ws13"], inp["ws2"], cfg.swiglu_limit_shared)
    for t in range(xq.shape[0]):
        for j, e in enumerate(ids[t].tolist()):
            gu = F.linear(xq[t], deq_w(inp["w13"][e], inp["w13_scale"][e]))
            gu = gu.float().double()
            sg, u = F.silu(gu[:I]), gu[I:]
            if L:
                sg, u = sg.clamp(max=L), u.clamp(-L, L)
            h = quant_act((sg * u).float()).double()
            out[t] += float(w[t, j]) * F.linear(h, deq_w(inp["w2"][e], inp["w2_scale"][e]))
    return out


def test_fp8_layer_matches_torch_float8_reference(orc):
    wl = mi.workload("tiny", hidden_size=256, moe_intermediate_size=128, expert_dtype="fp8", T=8)
    inp = _inputs(wl)
    res = orc.layer(wl.cfg, inp)
    want = _torch_fp8_reference(wl.cfg, inp, res["ids"], res["w"]).numpy()
    # activation codes can differ by one step where fp32 and fp64 disagree on
    # a rounding midpoint; the bound covers a handful of such flips
    assert np.abs(res["out"] - want).max() <= 1e-3 * np.abs(want).max()
    assert np.sqrt(((res["out"] - want) ** 2).mean()) <= 1e-5 * np.abs(want).max()


def test_fp8_exact_values_equal_bf16_path(orc):
    """With unit block scales, integer weights and activations that quantise
    exactly (x = 1, gate/up rows of ones so that with limit 1 every h is
    exactly 1), the FP8 layer equals the bf16 layer up to the fp32 rounding
    of 1/448 in the activation scale."""
    base = dict(num_experts=1, top_k=1, share_expert_dim=0, router_scaling_factor=1.0,
                swiglu_limit=1.0, hidden_size=256, moe_intermediate_size=128, T=4)
    wl16 = mi.workload("tiny", **base)
    wl8 = mi.workload("tiny", expert_dtype="fp8", **base)
    inp = _inputs(wl16)
    rng = np.random.default_rng(3)
    x = torch.ones(4, 256)
    w13 = torch.ones(1, 256, 256)
    w2 = torch.tensor(rng.integers(-1, 2, (1, 256, 128)), dtype=torch.float32)
    r16 = orc.layer(wl16.cfg, dict(inp, x=x.bfloat16(), w13=w13.bfloat16(), w2=w2.bfloat16()))
    f8 = lambda t: t.to(torch.float8_e4m3fn).view(torch.uint8)
    r8 = orc.layer(wl8.cfg, dict(inp, x=x.bfloat16(), w13=f8(w13), w2=f8(w2),
                                 w13_scale=torch.ones(1, 2, 2), w2_scale=torch.ones(1, 2, 1)))
    want = w2[0].sum(-1).numpy()[None, :].repeat(4, 0)
    assert np.array_equal(r16["out"], want)
    assert np.abs(r8["out"] - want).max() <= 1e-6 * np.abs(want).max()
