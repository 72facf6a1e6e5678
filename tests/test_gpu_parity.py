"""GPU parity: every entry point of libmoe.so against the CPU oracle on
identical seeded inputs.

Small workloads (tiny, ragged and edge-case shapes spanning several tiles and
ragged tails) are compared on every token; the full-size Step-3.5-Flash and
Step-5-Preview workloads are run through moe_layer_forward exactly as the
benchmark runs them, with routing and per-expert counts checked on every token
and outputs on a sample of tokens built from the GPU's own permutation so that
it reaches every (expert, m-tile) work item of the grouped launches: the first
and last row of every tile, a random row of each, and every row of the
largest expert (rows are independent, so a sampled row is checked exactly).
"""
import sys

import numpy as np
import pytest
import torch

import moe_inputs as mi
import sparse_moe_layer_route_amd as moe
from oracle import oracle as orc
from parity import (TOL_BF16, TOL_FP8, check_counts, check_routing, decode_rows, exempt_tokens,
                    max_err_over_rms, tile_plan_sample)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    moe.load()


def gpu_inputs(wl, seed=0):
    return mi.make_inputs(wl, DEV, seed)


def host(inp):
    return {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in inp.items()}


def run_layer(wl, inp, ws=None):
    T, k, E = wl.T, wl.cfg.top_k, wl.cfg.num_experts
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    counts = torch.empty((E,), dtype=torch.int32, device=DEV)
    out = moe.moe_layer_forward(wl.cfg, inp, ws=ws, topk_ids=ids, topk_w=w, expert_counts=counts)
    torch.cuda.synchronize()
    return out, ids, w, counts


# ----------------------------------------------------------------------------------------
# small and edge-case workloads: every token

SMALL = {
    "tiny": dict(),
    "tiny_clip_stress": dict(x_scale=40.0),
    "one_token": dict(T=1),
    "three_tokens": dict(T=3),
    "ragged_130_tokens_20_experts": dict(T=130, num_experts=20, top_k=3),
    "top1": dict(top_k=1, T=77),
    "all_experts_chosen": dict(top_k=16, T=40),
    "no_norm": dict(norm_expert_weight=False, router_scaling_factor=2.5),
    "no_shared": dict(share_expert_dim=0, T=96),
    "limits_off": dict(swiglu_limit=0.0, swiglu_limit_shared=0.0, x_scale=8.0),
    "shared_clip": dict(swiglu_limit=0.5, swiglu_limit_shared=0.5, x_scale=8.0),
    "bf16_out": dict(out_dtype="bf16"),
    "narrow_64": dict(hidden_size=64, moe_intermediate_size=64, share_expert_dim=64, T=200),
    "wide_tiles": dict(hidden_size=512, moe_intermediate_size=320, share_expert_dim=192, T=300,
                       num_experts=12, top_k=2),
    "max_experts_max_k": dict(hidden_size=128, num_experts=1024, top_k=32, moe_intermediate_size=64,
                              share_expert_dim=64, T=64),
    # ~37 rows per expert: 64-row tiles, several for the larger experts
    "small_tiles_multi_tile": dict(T=600, num_experts=32, top_k=2),
    # shared width differs from the experts': the shared expert runs on its own
    "shared_width_differs": dict(moe_intermediate_size=192, share_expert_dim=128, T=100),
    # small-batch router with H / 8 = 576 > 512: its K loop runs two chunks of
    # 16 slices, the second ragged
    "router_two_chunks": dict(hidden_size=4608, T=24, num_experts=16, top_k=4, moe_intermediate_size=64,
                              share_expert_dim=64),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small(name):
    wl = mi.workload("tiny", **SMALL[name])
    say(f"[layer_small] {name} T={wl.T} cfg={wl.cfg}")
    inp = gpu_inputs(wl)
    out, ids, w, counts = run_layer(wl, inp)
    h = host(inp)
    ref = orc.layer(wl.cfg, h)
    _, _, _, corr = orc.route(wl.cfg, h["x"], h["w_router"], h["router_bias"], want_scores=True)
    ex = check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], corr, wl.cfg.top_k)
    check_counts(counts.cpu().numpy(), ref["ids"], ids.cpu().numpy(), ex, wl.cfg.num_experts)
    keep = ~ex
    err, rms = max_err_over_rms(out.float().cpu().numpy()[keep], ref["out"][keep])
    say(f"  max_err/rms = {err:.3e} (rms {rms:.3e}), exempt tokens {int(ex.sum())}")
    assert err <= TOL_BF16


@pytest.mark.parametrize("name", ["tiny", "ragged_130_tokens_20_experts", "wide_tiles"])
def test_steps_small(name):
    """Each entry point on its own: route, permute, grouped experts, shared
    expert, combine."""
    wl = mi.workload("tiny", **SMALL[name])
    cfg, T, k, E, H = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts, wl.cfg.hidden_size
    say(f"[steps_small] {name}")
    inp = gpu_inputs(wl)
    h = host(inp)
    ws = moe.workspace(cfg, T)
    ids, w = moe.moe_route(cfg, inp["x"], inp["w_router"], inp["router_bias"], ws=ws)
    counts, offsets, r2p, p2r = moe.moe_permute(cfg, ids, ws=ws)
    y_rows = moe.moe_grouped_swiglu(cfg, inp["x"], offsets, r2p, inp["w13"], inp["w2"], ws=ws)
    y_sh = moe.moe_shared_ffn(cfg, inp["x"], inp["ws13"], inp["ws2"], ws=ws)
    out = moe.moe_combine(cfg, y_rows, p2r, w, y_sh)
    torch.cuda.synchronize()
    ids_h = ids.cpu().numpy()
    # permutation: bit-exact against the oracle's stable grouping of the GPU's ids
    oc, oo, or2p, op2r = orc.permute(ids_h, E)
    assert np.array_equal(counts.cpu().numpy(), oc)
    assert np.array_equal(offsets.cpu().numpy(), oo)
    assert np.array_equal(r2p.cpu().numpy(), or2p)
    assert np.array_equal(p2r.cpu().numpy(), op2r)
    # experts: row r of y_rows is pair r2p[r]'s expert output, unweighted
    ref = orc.layer(cfg, h, want_parts=True)
    _, _, _, corr = orc.route(cfg, h["x"], h["w_router"], h["router_bias"], want_scores=True)
    ex = check_routing(ids_h, w.cpu().numpy(), ref["ids"], ref["w"], corr, k)
    yr = decode_rows(y_rows, H)
    pairs = or2p
    t_of, j_of = pairs // k, pairs % k
    keep = ~ex[t_of]
    # the oracle's slot order may differ from the GPU's only among near-ties
    orc_slot = {(t, e): j for t in range(T) for j, e in enumerate(ref["ids"][t].tolist())}
    ref_rows = np.stack([ref["y_routed"][t, orc_slot[(t, ids_h[t, j])]] for t, j in zip(t_of, j_of)])
    err, _ = max_err_over_rms(yr[keep], ref_rows[keep])
    say(f"  grouped rows max_err/rms = {err:.3e}")
    assert err <= TOL_BF16
    err, _ = max_err_over_rms(y_sh.cpu().numpy(), ref["y_shared"])
    say(f"  shared max_err/rms = {err:.3e}")
    assert err <= TOL_BF16
    # combine: exact fp32 sum of the GPU's own buffers, in slot order
    want = y_sh.double().cpu().numpy().copy()
    wh = w.double().cpu().numpy()
    p2r_h = p2r.cpu().numpy()
    for t in range(T):
        for j in range(k):
            want[t] += wh[t, j] * yr[p2r_h[t * k + j]]
    assert np.abs(out.cpu().numpy() - want).max() <= 1e-5 * np.abs(want).max()


@pytest.mark.parametrize("name", ["tiny", "small_tiles_multi_tile", "wide_tiles"])
def test_steps_shared_rows(name):
    """The split path with the shared expert inside the expert launches
    (moe_expert_up / moe_expert_down with its weights, combine of its scaled
    fp16 rows) equals moe_layer_forward bit for bit, and the oracle within
    tolerance; where the widths differ, the entry points refuse."""
    wl = mi.workload("tiny", **SMALL[name])
    cfg, T, k = wl.cfg, wl.T, wl.cfg.top_k
    say(f"[steps_shared_rows] {name}")
    inp = gpu_inputs(wl)
    ws = moe.workspace(cfg, T)
    ids, w = moe.moe_route(cfg, inp["x"], inp["w_router"], inp["router_bias"], ws=ws)
    counts, offsets, r2p, p2r = moe.moe_permute(cfg, ids, ws=ws)
    if not moe.binding.shared_fusable(cfg):
        with pytest.raises(moe.MoEError):
            moe.moe_expert_up(cfg, inp["x"], offsets, r2p, inp["w13"], ws=ws, ws13=inp["ws13"])
        return
    h = moe.moe_expert_up(cfg, inp["x"], offsets, r2p, inp["w13"], ws=ws, ws13=inp["ws13"])
    y_rows = moe.moe_expert_down(cfg, T, h, offsets, inp["w2"], ws=ws, ws2=inp["ws2"])
    out = moe.moe_combine(cfg, y_rows, p2r, w, shared_rows=y_rows[T * k:])
    ref_out = moe.moe_layer_forward(cfg, inp)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    ref = orc.layer(cfg, host(inp))
    _, _, _, corr = orc.route(cfg, *(inp[n].cpu() for n in ("x", "w_router", "router_bias")), want_scores=True)
    ex = check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], corr, k)
    err, _ = max_err_over_rms(out.cpu().numpy()[~ex], ref["out"][~ex])
    say(f"  max_err/rms = {err:.3e}")
    assert err <= TOL_BF16


def test_permute_arbitrary_ids_with_duplicates():
    """Stable grouping is defined for any ids in range, duplicates included."""
    wl = mi.workload("tiny", T=333, num_experts=37, top_k=5)
    g = torch.Generator().manual_seed(7)
    ids = torch.randint(0, 37, (333, 5), generator=g, dtype=torch.int32)
    counts, offsets, r2p, p2r = moe.moe_permute(wl.cfg, ids.to(DEV))
    torch.cuda.synchronize()
    oc, oo, or2p, op2r = orc.permute(ids.numpy(), 37)
    assert np.array_equal(counts.cpu().numpy(), oc) and np.array_equal(offsets.cpu().numpy(), oo)
    assert np.array_equal(r2p.cpu().numpy(), or2p) and np.array_equal(p2r.cpu().numpy(), op2r)


def test_nan_inf_inputs_keep_ids_in_range():
    wl = mi.workload("tiny")
    inp = gpu_inputs(wl)
    inp["x"][0] = float("nan")
    inp["x"][1, 5] = float("inf")
    inp["x"][2] = float("-inf")
    ids, w = moe.moe_route(wl.cfg, inp["x"], inp["w_router"], inp["router_bias"])
    torch.cuda.synchronize()
    ids = ids.cpu().numpy()
    assert ids.min() >= 0 and ids.max() < wl.cfg.num_experts
    assert ids[0].tolist() == list(range(wl.cfg.top_k))      # all scores NaN -> lowest indices
    ref_ids, _ = orc.route(wl.cfg, *(inp[n].cpu() for n in ("x", "w_router", "router_bias")))
    assert np.array_equal(ids[:3], ref_ids[:3])


@pytest.mark.parametrize("name", ["step5_decode", "tiny", "step35_prefill"])
def test_graph_replay_matches_eager(name):
    """moe_layer_forward captured into a HIP graph: every replay (with eager
    work and synchronisations between them) equals the eager result."""
    wl = mi.WORKLOADS[name]
    cfg, T, H = wl.cfg, wl.T, wl.cfg.hidden_size
    say(f"[graph_replay] {name}")
    inp = gpu_inputs(wl)
    ws = moe.workspace(cfg, T)
    want = moe.moe_layer_forward(cfg, inp, ws=ws)
    torch.cuda.synchronize()
    out = torch.empty((T, H), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        moe.moe_layer_forward(cfg, inp, out=out, ws=ws, stream=side)
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            moe.moe_layer_forward(cfg, inp, out=out, ws=ws, stream=side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        scratch = torch.randn(1 << 20, device=DEV) * 3.0      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {rep} differs from eager"
        del scratch


def test_many_tokens_small_dims():
    """1.6 M (token, expert) pairs through the multi-kernel permutation and
    several-tile experts: routing and counts on every token, outputs on a
    sample (index ranges well beyond the other cases)."""
    wl = mi.workload("tiny", T=200_000, hidden_size=128, num_experts=64, top_k=8, moe_intermediate_size=128,
                     share_expert_dim=128)
    cfg, T, k, E = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts
    say(f"[many_tokens] T={T} P={T * k}")
    inp = gpu_inputs(wl)
    out, ids, w, counts = run_layer(wl, inp)
    h = host(inp)
    o_ids, o_w, _, corr = orc.route(cfg, h["x"], h["w_router"], h["router_bias"], want_scores=True)
    ids_h = ids.cpu().numpy()
    ex = check_routing(ids_h, w.cpu().numpy(), o_ids, o_w, corr, k)
    check_counts(counts.cpu().numpy(), o_ids, ids_h, ex, E)
    rng = np.random.default_rng(3)
    cand = np.nonzero(~ex)[0]
    sample = np.unique(np.concatenate([cand[:3], cand[-3:], rng.choice(cand, 64, replace=False)]))
    ref = orc.layer(cfg, h, tokens=sample)
    err, _ = max_err_over_rms(out.cpu().numpy()[sample], ref["out"])
    say(f"  sampled {sample.size} tokens: max_err/rms = {err:.3e}")
    assert err <= TOL_BF16


def test_zero_tokens():
    wl = mi.workload("tiny", T=0)
    inp = gpu_inputs(wl)
    out = moe.moe_layer_forward(wl.cfg, inp)
    torch.cuda.synchronize()
    assert out.shape == (0, wl.cfg.hidden_size)


def test_deterministic():
    wl = mi.workload("tiny", T=257)
    inp = gpu_inputs(wl)
    a = run_layer(wl, inp)
    b = run_layer(wl, inp)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ----------------------------------------------------------------------------------------
# routing supplied by the caller: routing replay and the static balanced routing

def run_routed(wl, inp, ids, ws=None):
    E = wl.cfg.num_experts
    w = torch.empty(ids.shape, dtype=torch.float32, device=DEV)
    counts = torch.empty((E,), dtype=torch.int32, device=DEV)
    out = moe.moe_layer_forward_routed(wl.cfg, inp, ids, ws=ws, topk_w=w, expert_counts=counts)
    torch.cuda.synchronize()
    return out, w, counts


def check_weights(gpu_w, orc_w):
    """Weights of a given choice: no selection involved, so every slot is
    compared (fp32 sigmoid on the GPU vs double on the host)."""
    gpu_w = np.asarray(gpu_w, np.float64)
    orc_w = np.asarray(orc_w, np.float64)
    assert np.all(np.abs(gpu_w - orc_w) <= 1e-6 + 1e-5 * np.abs(orc_w))


REPLAY_SMALL = ["tiny", "tiny_clip_stress", "one_token", "ragged_130_tokens_20_experts", "top1",
                "all_experts_chosen", "no_norm", "no_shared", "bf16_out", "max_experts_max_k",
                "small_tiles_multi_tile", "shared_width_differs"]


@pytest.mark.parametrize("name", ["tiny", "ragged_130_tokens_20_experts", "no_norm", "max_experts_max_k",
                                  "step5_decode"])
def test_replay_of_own_choice_is_bit_exact(name):
    """Replaying moe_route's own ids gives its weights and the layer output
    of moe_layer_forward bit for bit."""
    wl = mi.WORKLOADS[name] if name in mi.WORKLOADS else mi.workload("tiny", **SMALL[name])
    say(f"[replay_own_choice] {name}")
    inp = gpu_inputs(wl)
    ws = moe.workspace(wl.cfg, wl.T)
    out, ids, w, counts = run_layer(wl, inp, ws=ws)
    w2 = moe.moe_route_replay(wl.cfg, inp["x"], inp["w_router"], ids, ws=ws)
    out2, w3, counts2 = run_routed(wl, inp, ids, ws=ws)
    assert torch.equal(w, w2) and torch.equal(w, w3)
    assert torch.equal(counts, counts2)
    assert torch.equal(out, out2)


def test_layer_rows_per_expert_at_tile_boundaries():
    """Few rows per expert (64-row tiles, each 16-row MFMA tile its own A
    block): experts given exactly 1, 15, 16, 17, 31, 32, 33, 48, 63 and 64
    rows, six experts none, through the routed entry point; every token
    against the oracle with the same choice."""
    counts_want = [1, 15, 16, 17, 31, 32, 33, 48, 63, 64, 0, 0, 0, 0, 0, 0]
    wl = mi.workload("tiny", T=80, num_experts=16, top_k=4)
    cfg, T, k, E = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts
    assert sum(counts_want) == T * k
    # pair p (expert-sorted) goes to token p % T, slot p // T: an expert's
    # pairs are consecutive and fewer than T, so a token's k experts differ
    flat = np.repeat(np.arange(E), counts_want)
    ids_np = np.empty((T, k), dtype=np.int32)
    for p_, e in enumerate(flat):
        ids_np[p_ % T, p_ // T] = e
    assert all(len(set(r)) == k for r in ids_np.tolist())
    say("[layer_rows_per_expert_at_tile_boundaries]")
    inp = gpu_inputs(wl)
    ids = torch.from_numpy(ids_np)
    out, w, counts = run_routed(wl, inp, ids.to(DEV))
    assert counts.cpu().tolist() == counts_want
    ref = orc.layer(cfg, host(inp), ids_in=ids)
    check_weights(w.cpu().numpy(), ref["w"])
    err, rms = max_err_over_rms(out.float().cpu().numpy(), ref["out"])
    say(f"  max_err/rms = {err:.3e} (rms {rms:.3e})")
    assert err <= TOL_BF16


# rows per expert at the boundaries of the 256-row tiles' per-wave counts of
# valid 16-row tiles (wave wm holds tiles wm, wm+4, wm+8, wm+12: 1..4 of them,
# or none), of the FP8 kernel's 128-row tiles, and of two and three m-tiles
ROWS_AT_WAVE_TILE_BOUNDARIES = [1, 16, 17, 48, 49, 64, 65, 112, 128, 129, 192, 193, 240, 241, 255, 256, 257, 300,
                                511, 512, 513, 1, 0, 0]


@pytest.mark.parametrize("expert_dtype", ["bf16", "fp8"])
def test_layer_rows_per_expert_at_wave_tile_boundaries(expert_dtype):
    """Prefill-sized tiles (256 rows bf16, 128 rows FP8) with experts given
    row counts at every boundary of a wave's valid 16-row tiles, through the
    routed entry point; every token against the oracle with the same
    choice."""
    counts_want = ROWS_AT_WAVE_TILE_BOUNDARIES
    E, k = len(counts_want), 4
    T = sum(counts_want) // k
    assert T * k == sum(counts_want) and max(counts_want) < T
    kw = dict(T=T, num_experts=E, top_k=k, hidden_size=256, moe_intermediate_size=128 if expert_dtype == "fp8" else 256)
    if expert_dtype == "fp8":
        kw["expert_dtype"] = "fp8"
    wl = mi.workload("tiny", **kw)
    cfg = wl.cfg
    flat = np.repeat(np.arange(E), counts_want)
    ids_np = np.empty((T, k), dtype=np.int32)
    for p_, e in enumerate(flat):
        ids_np[p_ % T, p_ // T] = e
    assert all(len(set(r)) == k for r in ids_np.tolist())
    say(f"[layer_rows_per_expert_at_wave_tile_boundaries] {expert_dtype} T={T} E={E}")
    inp = gpu_inputs(wl)
    ids = torch.from_numpy(ids_np)
    out, w, counts = run_routed(wl, inp, ids.to(DEV))
    assert counts.cpu().tolist() == counts_want
    ref = orc.layer(cfg, host(inp), ids_in=ids)
    check_weights(w.cpu().numpy(), ref["w"])
    err, rms = max_err_over_rms(out.float().cpu().numpy(), ref["out"])
    say(f"  max_err/rms = {err:.3e} (rms {rms:.3e})")
    assert err <= (TOL_FP8 if expert_dtype == "fp8" else TOL_BF16)


@pytest.mark.parametrize("name", REPLAY_SMALL)
def test_layer_replay_small(name):
    """A replayed choice that is not the router's (random distinct experts;
    on two tokens also a duplicate and out-of-range ids, which are clamped):
    weights and outputs on every token against the oracle's replay."""
    wl = mi.workload("tiny", **SMALL[name])
    cfg, T, k, E = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts
    say(f"[layer_replay_small] {name} T={T}")
    inp = gpu_inputs(wl)
    ids = mi.random_expert_ids(wl, seed=11)
    if k >= 2:
        ids[0, 1] = ids[0, 0]
    if T >= 2:
        ids[T - 1, 0] = -3
        ids[T - 1, k - 1] = E + 7
    out, w, counts = run_routed(wl, inp, ids.to(DEV))
    ref = orc.layer(cfg, host(inp), ids_in=ids)
    check_weights(w.cpu().numpy(), ref["w"])
    assert np.array_equal(counts.cpu().numpy(), np.bincount(ref["ids"].reshape(-1), minlength=E))
    err, rms = max_err_over_rms(out.float().cpu().numpy(), ref["out"])
    say(f"  max_err/rms = {err:.3e} (rms {rms:.3e})")
    assert err <= TOL_BF16


def test_layer_replay_fp8_small():
    wl = fp8_workload("fp8_ragged_130_tokens_20_experts")
    say("[layer_replay_fp8_small]")
    inp = gpu_inputs(wl)
    ids = mi.random_expert_ids(wl, seed=12)
    out, w, counts = run_routed(wl, inp, ids.to(DEV))
    ref = orc.layer(wl.cfg, host(inp), ids_in=ids)
    check_weights(w.cpu().numpy(), ref["w"])
    err, rms = max_err_over_rms(out.float().cpu().numpy(), ref["out"])
    say(f"  max_err/rms = {err:.3e} (rms {rms:.3e})")
    assert err <= TOL_FP8


@pytest.mark.parametrize("T,k,E", [(8192, 8, 288), (64, 8, 288), (8192, 8, 352), (7, 3, 5), (1, 1, 1),
                                   (300_000, 8, 64)])
def test_balanced_ids_bit_exact(T, k, E):
    wl = mi.workload("tiny", T=T, top_k=k, num_experts=E)
    ids = moe.moe_balanced_ids(wl.cfg, T)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), orc.balanced_ids(T, k, E))


@pytest.mark.parametrize("name", ["step5_prefill", "step5_decode"])
def test_layer_balanced_full_size(name):
    """The static balanced routing at full size, as the benchmark's
    balanced line runs it: ids bit-exact, counts exact, weights on every
    token, outputs on a seeded sample."""
    wl = mi.WORKLOADS[name]
    cfg, T, k, E = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts
    say(f"[layer_balanced_full] {name} T={T}")
    inp = gpu_inputs(wl)
    ids = moe.moe_balanced_ids(cfg, T)
    out, w, counts = run_routed(wl, inp, ids)
    o_ids = orc.balanced_ids(T, k, E)
    assert np.array_equal(ids.cpu().numpy(), o_ids)
    assert np.array_equal(counts.cpu().numpy(), np.bincount(o_ids.reshape(-1), minlength=E))
    say("  gpu done; copying inputs to host")
    h = host(inp)
    del inp
    torch.cuda.empty_cache()
    _, o_w = orc.route(cfg, h["x"], h["w_router"], None, ids_in=o_ids)
    check_weights(w.cpu().numpy(), o_w)
    sample = item_sample(cfg, T, ids, np.zeros(T, bool), seed=5)
    ref = orc.layer(cfg, h, tokens=sample, ids_in=o_ids)
    err, rms = max_err_over_rms(out.cpu().numpy()[sample], ref["out"])
    say(f"  sampled {sample.size} tokens: max_err/rms = {err:.3e} (rms {rms:.3e})")
    assert err <= TOL_BF16


# ----------------------------------------------------------------------------------------
# the steps either side of the layer: zero-centred RMSNorm and the fp32 residual

def check_bf16_close(gpu_x, orc_x):
    """bf16 rows computed in fp32 (GPU) and double (oracle): at most one
    unit in the last place apart, and rarely even that."""
    a = gpu_x.view(torch.int16).cpu().numpy().astype(np.int32)
    b = orc_x.view(torch.int16).cpu().numpy().astype(np.int32)
    sa = np.where(a < 0, -(a & 0x7FFF), a)            # sign-magnitude -> ordered integers
    sb = np.where(b < 0, -(b & 0x7FFF), b)
    d = np.abs(sa - sb)
    assert d.max() <= 1, f"max ulp difference {d.max()}"
    frac = float((d > 0).mean())
    assert frac < 2e-3, f"{frac:.2e} of the values differ by one ulp"
    return frac


@pytest.mark.parametrize("T,H", [(1, 64), (5, 320), (64, 4096), (8192, 4096), (3, 8192)])
def test_rmsnorm_vs_oracle(T, H):
    wl = mi.workload("tiny", T=T, hidden_size=H)
    b = mi.block_inputs(wl, DEV)
    b["resid"][0] *= 1e12                                    # a huge row (squares ~1e26: still finite)
    if T > 2:
        b["resid"][1] = 0.0                                  # a zero row stays zero
        b["resid"][2] *= 1e-12                               # a tiny row: eps dominates
    x = moe.moe_rmsnorm(wl.cfg, b["resid"], b["norm_weight"], b["eps"])
    torch.cuda.synchronize()
    ref = orc.rmsnorm(b["resid"].cpu(), b["norm_weight"].cpu(), b["eps"])
    frac = check_bf16_close(x, ref)
    say(f"[rmsnorm] T={T} H={H}: {frac:.2e} of values one ulp apart")
    if T > 2:
        assert (x[1].float() == 0).all()


NORM_ROUTE = {
    "tiny_64_tokens_two_steps": ("tiny", dict(T=64)),
    "tiny_600_tokens_fused": ("tiny", dict(T=600)),
    "ragged_777_tokens_fused": ("tiny", dict(T=777, num_experts=20, top_k=3)),
    "step35_prefill_fused": ("step35_prefill", {}),
    "step5_prefill_fused": ("step5_prefill", {}),
}


@pytest.mark.parametrize("name", list(NORM_ROUTE))
def test_rmsnorm_route_equals_its_steps(name):
    """moe_rmsnorm_route = moe_rmsnorm then moe_route, bit for bit (x, ids,
    weights), whether it runs fused (from 512 tokens) or as two steps; the
    routing itself is checked against the oracle's routing of those rows."""
    base, over = NORM_ROUTE[name]
    wl = mi.workload(base, **over)
    cfg = wl.cfg
    say(f"[norm_route] {name} T={wl.T}")
    inp = dict(gpu_inputs(wl), **mi.block_inputs(wl, DEV))
    x, ids, w = moe.moe_rmsnorm_route(cfg, inp["resid"], inp["norm_weight"], inp["eps"], inp["w_router"],
                                      inp["router_bias"])
    x2 = moe.moe_rmsnorm(cfg, inp["resid"], inp["norm_weight"], inp["eps"])
    ids2, w2 = moe.moe_route(cfg, x2, inp["w_router"], inp["router_bias"])
    torch.cuda.synchronize()
    assert torch.equal(x, x2)
    assert torch.equal(ids, ids2)
    assert torch.equal(w, w2)
    if wl.T <= 1024:
        h = host(inp)
        o_ids, o_w, _, corr = orc.route(cfg, x.cpu(), h["w_router"], h["router_bias"], want_scores=True)
        check_routing(ids.cpu().numpy(), w.cpu().numpy(), o_ids, o_w, corr, cfg.top_k)


BLOCK_SMALL = ["tiny", "ragged_130_tokens_20_experts", "no_shared", "shared_width_differs", "top1",
               "small_tiles_multi_tile"]


def run_block(wl, inp, resid_out=None):
    T, k, E = wl.T, wl.cfg.top_k, wl.cfg.num_experts
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    counts = torch.empty((E,), dtype=torch.int32, device=DEV)
    out = moe.moe_block_forward(wl.cfg, inp, resid_out=resid_out, topk_ids=ids, topk_w=w, expert_counts=counts)
    torch.cuda.synchronize()
    return out, ids, w, counts


# The block routes its own normalised rows, which may differ from the
# oracle's by one bf16 ulp in a few elements (at most 2e-3 of them, as the
# RMSNorm test asserts; about 1e-4 in practice).  One such element moves a
# logit by |w_router| * ulp(x) <= 0.08 * 2^-6 ~ 1.2e-3 at most (|x| < 4,
# |w| < 4 sigma), i.e. a raw score by <= 3e-4: hence a 1e-3 tie gap for the
# choice and 5e-3 relative for the weights in these tests; the outputs keep
# the usual tolerance.
BLOCK_GAP, BLOCK_W_RTOL = 1e-3, 5e-3


def check_block(wl, inp, out, ids, w, counts, tokens=None):
    """Routing against the oracle's routing of the GPU's own normalised rows
    at the usual 1e-6 tie gap and weight tolerance (the selection itself,
    with the inputs held equal), and against the oracle's own normalised
    rows at the widened gap; then the layer part (resid_out - resid) against
    the oracle's layer output."""
    cfg, k, E = wl.cfg, wl.cfg.top_k, wl.cfg.num_experts
    x_gpu = moe.moe_rmsnorm(cfg, inp["resid"], inp["norm_weight"], inp["eps"])
    torch.cuda.synchronize()
    h = host(inp)
    g_ids, g_w, _, g_corr = orc.route(cfg, x_gpu.cpu(), h["w_router"], h["router_bias"], want_scores=True)
    ex_own = check_routing(ids.cpu().numpy(), w.cpu().numpy(), g_ids, g_w, g_corr, k)
    check_counts(counts.cpu().numpy(), g_ids, ids.cpu().numpy(), ex_own, E)
    x_o = orc.rmsnorm(h["resid"], h["norm_weight"], h["eps"])
    o_ids, o_w, _, corr = orc.route(cfg, x_o, h["w_router"], h["router_bias"], want_scores=True)
    ids_h = ids.cpu().numpy()
    ex = check_routing(ids_h, w.cpu().numpy(), o_ids, o_w, corr, k, w_rtol=BLOCK_W_RTOL, gap=BLOCK_GAP)
    check_counts(counts.cpu().numpy(), o_ids, ids_h, ex, E)
    keep = np.nonzero(~ex)[0] if tokens is None else np.array([t for t in tokens if not ex[t]])
    ref = orc.block(cfg, h, tokens=keep)
    moe_part = out.double().cpu().numpy()[keep] - h["resid"].double().numpy()[keep]
    err, rms = max_err_over_rms(moe_part, ref["out"])
    full = np.abs(out.cpu().numpy()[keep] - ref["resid_out"]).max()
    say(f"  layer part max_err/rms = {err:.3e} (rms {rms:.3e}); resid_out max abs diff {full:.3e}; "
        f"exempt {int(ex.sum())}")
    assert err <= TOL_BF16
    assert full <= TOL_BF16 * rms + 1e-6 * np.abs(ref["resid_out"]).max()


@pytest.mark.parametrize("name", BLOCK_SMALL)
def test_block_small(name):
    wl = mi.workload("tiny", **SMALL[name])
    say(f"[block_small] {name} T={wl.T}")
    inp = dict(gpu_inputs(wl), **mi.block_inputs(wl, DEV))
    del inp["x"]
    out, ids, w, counts = run_block(wl, inp)
    check_block(wl, inp, out, ids, w, counts)
    # in place: the residual buffer itself receives the result, bit for bit
    r = inp["resid"].clone()
    run_block(wl, dict(inp, resid=r), resid_out=r)
    assert torch.equal(r, out)


BLOCK_STEPS = {
    "tiny": ("tiny", {}),
    "step5_decode": ("step5_decode", {}),
    "tiny_600_tokens": ("tiny", dict(T=600)),          # the dense router instance from 512 tokens
    "step35_prefill": ("step35_prefill", {}),
}


@pytest.mark.parametrize("name", list(BLOCK_STEPS))
def test_block_equals_its_steps(name):
    """moe_block_forward = resid + moe_layer_forward(moe_rmsnorm(resid)),
    bit for bit (the residual add is the combine's last fp32 add), and so is
    the split path ending in moe_combine with the residual as its output."""
    base, over = BLOCK_STEPS[name]
    wl = mi.workload(base, **over)
    cfg, T, k = wl.cfg, wl.T, wl.cfg.top_k
    say(f"[block_steps] {name}")
    inp = dict(gpu_inputs(wl), **mi.block_inputs(wl, DEV))
    out, *_ = run_block(wl, inp)
    x = moe.moe_rmsnorm(cfg, inp["resid"], inp["norm_weight"], inp["eps"])
    lay = moe.moe_layer_forward(cfg, dict(inp, x=x))
    torch.cuda.synchronize()
    assert torch.equal(out, inp["resid"] + lay)
    assert moe.binding.shared_fusable(cfg)
    ws = moe.workspace(cfg, T)
    ids, w = moe.moe_route(cfg, x, inp["w_router"], inp["router_bias"], ws=ws)
    counts, offsets, r2p, p2r = moe.moe_permute(cfg, ids, ws=ws)
    hbuf = moe.moe_expert_up(cfg, x, offsets, r2p, inp["w13"], ws=ws, ws13=inp["ws13"])
    y_rows = moe.moe_expert_down(cfg, T, hbuf, offsets, inp["w2"], ws=ws, ws2=inp["ws2"])
    r = inp["resid"].clone()
    moe.moe_combine(cfg, y_rows, p2r, w, shared_rows=y_rows[T * k:], out=r, residual=r)
    torch.cuda.synchronize()
    assert torch.equal(r, out)


@pytest.mark.parametrize("name", ["step5_prefill", "step5_decode"])
def test_block_full_size(name):
    wl = mi.WORKLOADS[name]
    say(f"[block_full] {name} T={wl.T}")
    inp = dict(gpu_inputs(wl), **mi.block_inputs(wl, DEV))
    del inp["x"]
    out, ids, w, counts = run_block(wl, inp)
    sample = item_sample(wl.cfg, wl.T, ids, np.zeros(wl.T, bool), seed=2)
    check_block(wl, inp, out, ids, w, counts, tokens=sample)


# ----------------------------------------------------------------------------------------
# full-size workloads through moe_layer_forward

FULL = ["step35_prefill", "step5_prefill", "step5_decode", "step5_decode_half"]


def tile_rows(cfg, T):
    """Row height of the grouped launches' tiles (the library's rule: FP8
    experts 128; bf16 64 when experts average under 48 rows, else 256)."""
    if cfg.expert_dtype == "fp8":
        return 128
    return 64 if T * cfg.top_k < 48 * cfg.num_experts else 256


def item_sample(cfg, T, ids, exempt, seed):
    """Tokens reaching every (expert, m-tile) work item of the grouped
    launches (from the GPU's own permutation of its ids), and every m-tile of
    the shared expert's group, less the near-tie tokens."""
    k = cfg.top_k
    _, offsets, r2p, _ = moe.moe_permute(cfg, ids)
    torch.cuda.synchronize()
    bm = tile_rows(cfg, T)
    rng = np.random.default_rng(seed)
    toks = [tile_plan_sample(offsets.cpu().numpy(), r2p.cpu().numpy(), k, bm, rng)]
    if cfg.share_expert_dim:
        mt = (T + bm - 1) // bm
        for m in range(mt):
            a, b = m * T // mt, (m + 1) * T // mt
            toks.append(np.array([a, b - 1, int(rng.integers(a, b))]))
    sample = np.unique(np.concatenate(toks))
    return sample[~exempt[sample]]


@pytest.mark.parametrize("name", FULL)
def test_layer_full_size(name):
    wl = mi.WORKLOADS[name]
    cfg, T, k, E = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts
    say(f"[layer_full] {name} T={T} E={E} k={k} H={cfg.hidden_size} I={cfg.moe_intermediate_size}")
    inp = gpu_inputs(wl)
    out, ids, w, counts = run_layer(wl, inp)
    out2, *_ = run_layer(wl, inp)
    assert torch.equal(out, out2), "repeat run differs"
    say("  gpu done; copying inputs to host")
    h = host(inp)
    del inp
    torch.cuda.empty_cache()
    o_ids, o_w, _, corr = orc.route(cfg, h["x"], h["w_router"], h["router_bias"], want_scores=True)
    ids_h = ids.cpu().numpy()
    ex = check_routing(ids_h, w.cpu().numpy(), o_ids, o_w, corr, k)
    check_counts(counts.cpu().numpy(), o_ids, ids_h, ex, E)
    say(f"  routing ok on all {T} tokens; exempt {int(ex.sum())}; experts touched "
        f"{int((counts.cpu().numpy() > 0).sum())}")
    sample = item_sample(cfg, T, ids, ex, seed=0)
    say(f"  comparing {sample.size} tokens that reach every work item")
    assert T < 500 or sample.size > 500
    ref = orc.layer(cfg, h, tokens=sample)
    assert np.array_equal(ref["ids"], o_ids[sample])
    err, rms = max_err_over_rms(out.cpu().numpy()[sample], ref["out"])
    say(f"  sampled {sample.size} tokens: max_err/rms = {err:.3e} (rms {rms:.3e})")
    assert err <= TOL_BF16


# ----------------------------------------------------------------------------------------
# FP8 E4M3 routed experts (128 x 128 block scales): oracle in its FP8 mode

FP8_SMALL = {
    "fp8_tiny": dict(),
    "fp8_ragged_130_tokens_20_experts": dict(T=130, num_experts=20, top_k=3),
    "fp8_top1": dict(top_k=1, T=77),
    "fp8_clip_stress": dict(x_scale=40.0),
    "fp8_limits_off": dict(swiglu_limit=0.0, swiglu_limit_shared=0.0, x_scale=8.0),
    # H = 384: the second projection's last 256-column tile is half outside
    "fp8_half_tile_384": dict(hidden_size=384, moe_intermediate_size=256, share_expert_dim=128, T=300,
                              num_experts=12, top_k=2),
    # 66 K blocks in the first projection: the weight-scale registers are reloaded
    "fp8_deep_k_66_blocks": dict(hidden_size=128 * 66, moe_intermediate_size=128, share_expert_dim=64, T=24,
                                 num_experts=4, top_k=2),
    "fp8_no_shared_bf16_out": dict(share_expert_dim=0, out_dtype="bf16", T=96),
    # more work items than blocks, so blocks walk several: with 8 K blocks in
    # both projections each item fetches the next one's first slices during
    # its last steps (about 640 and 320 items)
    "fp8_pipelined_items_k1024": dict(hidden_size=1024, moe_intermediate_size=1024, share_expert_dim=256, T=2400,
                                      num_experts=16, top_k=4),
    # the second projection's 4 K blocks are too few for that: its blocks
    # walk about 1000 items one after the other, each with its own prologue
    "fp8_unpipelined_items_k512": dict(hidden_size=2048, moe_intermediate_size=512, share_expert_dim=256, T=4000,
                                       num_experts=8, top_k=4),
}


# cases whose launches must hold more 128-row work items than the 256 blocks
# of the persistent grid (checked from the GPU's own expert counts)
FP8_MULTI_ITEM = {"fp8_pipelined_items_k1024", "fp8_unpipelined_items_k512"}


def fp8_items(cfg, counts):
    """Work items of the FP8 first and second projections: 128-row m-tiles
    times 256-column n-tiles (first: 2I gate/up columns, second: H)."""
    tiles = int(sum((int(c) + 127) // 128 for c in counts))
    return tiles * (2 * cfg.moe_intermediate_size // 256), tiles * ((cfg.hidden_size + 255) // 256)


def fp8_workload(name):
    kw = dict(hidden_size=256, moe_intermediate_size=128, expert_dtype="fp8")
    kw.update(FP8_SMALL[name])
    return mi.workload("tiny", **kw)


@pytest.mark.parametrize("name", list(FP8_SMALL))
def test_layer_fp8_small(name):
    wl = fp8_workload(name)
    say(f"[layer_fp8_small] {name} T={wl.T} cfg={wl.cfg}")
    inp = gpu_inputs(wl)
    inp["x"][0] = 0.0                               # an all-zero row: every group's scale is 1
    out, ids, w, counts = run_layer(wl, inp)
    if name in FP8_MULTI_ITEM:
        up_items, down_items = fp8_items(wl.cfg, counts.cpu().numpy())
        say(f"  work items: {up_items} first projection, {down_items} second")
        assert min(up_items, down_items) > 256
    h = host(inp)
    ref = orc.layer(wl.cfg, h)
    _, _, _, corr = orc.route(wl.cfg, h["x"], h["w_router"], h["router_bias"], want_scores=True)
    ex = check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], corr, wl.cfg.top_k)
    check_counts(counts.cpu().numpy(), ref["ids"], ids.cpu().numpy(), ex, wl.cfg.num_experts)
    keep = ~ex
    err, rms = max_err_over_rms(out.float().cpu().numpy()[keep], ref["out"][keep])
    say(f"  max_err/rms = {err:.3e} (rms {rms:.3e}), exempt tokens {int(ex.sum())}")
    assert err <= TOL_FP8


def test_fp8_expert_steps():
    """moe_expert_up then moe_expert_down in FP8 mode: every routed row
    against the oracle's per-expert output, and the split path equal to
    moe_grouped_swiglu bit for bit."""
    wl = fp8_workload("fp8_ragged_130_tokens_20_experts")
    cfg, T, k, E = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts
    say("[fp8_expert_steps]")
    inp = gpu_inputs(wl)
    h_in = host(inp)
    ws = moe.workspace(cfg, T)
    ids, w = moe.moe_route(cfg, inp["x"], inp["w_router"], inp["router_bias"], ws=ws)
    counts, offsets, r2p, p2r = moe.moe_permute(cfg, ids, ws=ws)
    hbuf = moe.moe_expert_up(cfg, inp["x"], offsets, r2p, inp["w13"], inp["w13_scale"], ws=ws)
    y_split = moe.moe_expert_down(cfg, T, hbuf, offsets, inp["w2"], inp["w2_scale"], ws=ws)
    y_fused = moe.moe_grouped_swiglu(cfg, inp["x"], offsets, r2p, inp["w13"], inp["w2"],
                                     w13_scale=inp["w13_scale"], w2_scale=inp["w2_scale"], ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(y_split, y_fused)
    # h scales: positive, one per (row, 128 columns), block-major after the codes
    P, I = T * k, cfg.moe_intermediate_size
    code_bytes = (P * I + 255) // 256 * 256
    hs = hbuf[code_bytes:code_bytes + (I // 128) * P * 4].view(torch.float32).cpu().numpy()
    assert np.all(hs > 0) and np.all(np.isfinite(hs))
    ids_h = ids.cpu().numpy()
    ref = orc.layer(cfg, h_in, want_parts=True)
    _, _, _, corr = orc.route(cfg, h_in["x"], h_in["w_router"], h_in["router_bias"], want_scores=True)
    ex = check_routing(ids_h, w.cpu().numpy(), ref["ids"], ref["w"], corr, k)
    pairs = r2p.cpu().numpy()
    t_of, j_of = pairs // k, pairs % k
    keep = ~ex[t_of]
    orc_slot = {(t, e): j for t in range(T) for j, e in enumerate(ref["ids"][t].tolist())}
    ref_rows = np.stack([ref["y_routed"][t, orc_slot[(t, ids_h[t, j])]] for t, j in zip(t_of, j_of)])
    err, _ = max_err_over_rms(decode_rows(y_split, cfg.hidden_size)[keep], ref_rows[keep])
    say(f"  routed rows max_err/rms = {err:.3e}")
    assert err <= TOL_FP8


def test_fp8_deterministic():
    wl = fp8_workload("fp8_ragged_130_tokens_20_experts")
    inp = gpu_inputs(wl)
    a = run_layer(wl, inp)
    b = run_layer(wl, inp)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_layer_fp8_full_size():
    wl = mi.WORKLOADS["step5_fp8_prefill"]
    cfg, T, k, E = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts
    say(f"[layer_fp8_full] T={T} E={E} k={k} H={cfg.hidden_size} I={cfg.moe_intermediate_size}")
    inp = gpu_inputs(wl)
    out, ids, w, counts = run_layer(wl, inp)
    say("  gpu done; copying inputs to host")
    h = host(inp)
    del inp
    torch.cuda.empty_cache()
    o_ids, o_w, _, corr = orc.route(cfg, h["x"], h["w_router"], h["router_bias"], want_scores=True)
    ids_h = ids.cpu().numpy()
    ex = check_routing(ids_h, w.cpu().numpy(), o_ids, o_w, corr, k)
    check_counts(counts.cpu().numpy(), o_ids, ids_h, ex, E)
    sample = item_sample(cfg, T, ids, ex, seed=1)
    say(f"  comparing {sample.size} tokens that reach every work item")
    assert sample.size > 500
    ref = orc.layer(cfg, h, tokens=sample)
    err, rms = max_err_over_rms(out.cpu().numpy()[sample], ref["out"])
    say(f"  sampled {sample.size} tokens: max_err/rms = {err:.3e} (rms {rms:.3e})")
    assert err <= TOL_FP8


# ----------------------------------------------------------------------------------------
# the expert rows' range: no clip (limit 0) with outputs far beyond fp16's
# range, and tiny outputs far below its normal range

def large_y_workload(fp8=False):
    # x scaled so that, with no clip, h ~ 0.1 x_scale^2 and the expert
    # outputs reach about 0.02 sqrt(I) h ~ 2e5, beyond fp16's largest (65504)
    kw = dict(swiglu_limit=0.0, swiglu_limit_shared=0.0, x_scale=3000.0, T=96)
    if fp8:
        kw.update(hidden_size=256, moe_intermediate_size=128, expert_dtype="fp8")
    return mi.workload("tiny", **kw)


@pytest.mark.parametrize("fp8", [False, True])
def test_layer_no_clip_outputs_beyond_fp16(fp8):
    """Limit 0 (no clip) with expert outputs above 65504: the whole layer
    against the oracle within the usual tolerance, and the expert rows'
    format kept (each 128-column group's largest fp16 magnitude in
    [2^14, 2^15))."""
    wl = large_y_workload(fp8)
    cfg, T, k, H = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.hidden_size
    say(f"[no_clip_beyond_fp16] fp8={fp8} T={T}")
    inp = gpu_inputs(wl)
    out, ids, w, counts = run_layer(wl, inp)
    h = host(inp)
    ref = orc.layer(cfg, h, want_parts=True)
    big = float(np.abs(ref["y_routed"]).max())
    say(f"  oracle max |expert output| = {big:.3e}")
    assert big > 65504.0, "the case must reach beyond fp16's range"
    _, _, _, corr = orc.route(cfg, h["x"], h["w_router"], h["router_bias"], want_scores=True)
    ex = check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], corr, k)
    err, rms = max_err_over_rms(out.float().cpu().numpy()[~ex], ref["out"][~ex])
    say(f"  max_err/rms = {err:.3e} (rms {rms:.3e})")
    assert np.isfinite(out.cpu().numpy()).all()
    assert err <= (TOL_FP8 if fp8 else TOL_BF16)
    # the rows themselves
    ws = moe.workspace(cfg, T)
    ids2, w2 = moe.moe_route(cfg, inp["x"], inp["w_router"], inp["router_bias"], ws=ws)
    _, offsets, r2p, _ = moe.moe_permute(cfg, ids2, ws=ws)
    y = moe.moe_grouped_swiglu(cfg, inp["x"], offsets, r2p, inp["w13"], inp["w2"], w13_scale=inp.get("w13_scale"),
                               w2_scale=inp.get("w2_scale"), ws=ws)
    torch.cuda.synchronize()
    vals = y[:, :2 * H].cpu().contiguous().view(torch.float16).float().abs().numpy()
    gmax = vals.reshape(vals.shape[0], -1, 128).max(axis=2)
    nz = gmax > 0
    assert np.all((gmax[nz] >= 2.0 ** 14) & (gmax[nz] <= 2.0 ** 15))   # rounding may carry to 2^15
    assert np.abs(decode_rows(y, H)).max() > 65504.0


def test_layer_tiny_outputs():
    """Inputs scaled by 1e-4 (expert outputs around 1e-8, below fp16's
    smallest normal number): the layer against the oracle within the usual
    tolerance of its (tiny) RMS."""
    wl = mi.workload("tiny", x_scale=1e-4, T=96)
    say("[tiny_outputs]")
    inp = gpu_inputs(wl)
    out, ids, w, counts = run_layer(wl, inp)
    h = host(inp)
    ref = orc.layer(wl.cfg, h)
    _, _, _, corr = orc.route(wl.cfg, h["x"], h["w_router"], h["router_bias"], want_scores=True)
    ex = check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], corr, wl.cfg.top_k)
    err, rms = max_err_over_rms(out.float().cpu().numpy()[~ex], ref["out"][~ex])
    say(f"  max_err/rms = {err:.3e} (rms {rms:.3e})")
    assert err <= TOL_BF16


# ----------------------------------------------------------------------------------------
# prefill-sized token counts with small dimensions: the whole-layer call
# equals its separate entry points bit for bit (the shared expert as group E
# of the routed launches, or in launches of its own when its width differs)

PREFILL_SMALL_DIMS = {
    # 8192 pairs over 352 experts (23 per expert): 64-row tiles at T = 1024
    "t1024_64_row_tiles": dict(T=1024, hidden_size=128, num_experts=352, top_k=8, moe_intermediate_size=128,
                               share_expert_dim=128),
    # 256-row tiles, the shared expert of another width in launches of its own
    "t2048_shared_width_differs": dict(T=2048, hidden_size=256, num_experts=8, top_k=2, moe_intermediate_size=256,
                                       share_expert_dim=128),
    # 256-row tiles, the shared expert as group E
    "t2048_shared_as_group": dict(T=2048, hidden_size=256, num_experts=8, top_k=2, moe_intermediate_size=256,
                                  share_expert_dim=256),
    # 256-row tiles over 1024 expert groups: the item table deals 128 rounds of groups to the XCDs
    "t1536_1024_experts": dict(T=1536, hidden_size=128, num_experts=1024, top_k=32, moe_intermediate_size=128,
                               share_expert_dim=128),
    # 37 groups (a ragged last round of the deal) and a ragged shared group of 3000 rows
    "t3000_37_experts": dict(T=3000, hidden_size=256, num_experts=37, top_k=4, moe_intermediate_size=256,
                             share_expert_dim=256),
}


@pytest.mark.parametrize("name", list(PREFILL_SMALL_DIMS))
def test_prefill_sizes_layer_equals_steps(name):
    wl = mi.workload("tiny", **PREFILL_SMALL_DIMS[name])
    cfg, T, k, E = wl.cfg, wl.T, wl.cfg.top_k, wl.cfg.num_experts
    say(f"[prefill_sizes_layer_equals_steps] {name}")
    inp = gpu_inputs(wl)
    out, ids, w, counts = run_layer(wl, inp)
    ws = moe.workspace(cfg, T)
    ids2, w2 = moe.moe_route(cfg, inp["x"], inp["w_router"], inp["router_bias"], ws=ws)
    counts2, offsets, r2p, p2r = moe.moe_permute(cfg, ids2, ws=ws)
    if moe.binding.shared_fusable(cfg):
        hb = moe.moe_expert_up(cfg, inp["x"], offsets, r2p, inp["w13"], ws=ws, ws13=inp["ws13"])
        y = moe.moe_expert_down(cfg, T, hb, offsets, inp["w2"], ws=ws, ws2=inp["ws2"])
        out2 = moe.moe_combine(cfg, y, p2r, w2, shared_rows=y[T * k:])
    else:
        y = moe.moe_grouped_swiglu(cfg, inp["x"], offsets, r2p, inp["w13"], inp["w2"], ws=ws)
        ysh = moe.moe_shared_ffn(cfg, inp["x"], inp["ws13"], inp["ws2"], ws=ws)
        out2 = moe.moe_combine(cfg, y, p2r, w2, ysh)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w, w2) and torch.equal(counts, counts2)
    assert torch.equal(out, out2)
    h = host(inp)
    ref = orc.layer(cfg, h)
    _, _, _, corr = orc.route(cfg, h["x"], h["w_router"], h["router_bias"], want_scores=True)
    ex = check_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], corr, k)
    err, rms = max_err_over_rms(out.cpu().numpy()[~ex], ref["out"][~ex])
    say(f"  max_err/rms = {err:.3e} (rms {rms:.3e})")
    assert err <= TOL_BF16
