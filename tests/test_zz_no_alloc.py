"""The allocation-free layer entry point against moe_layer_forward with a
workspace of its own: the same kernels on the same inputs give the same
bits.  Two calls in a row share the library's scratch array, the second with
fewer tokens, so leftovers of the first call must not reach the second."""
import sys

import pytest
import torch

import moe_inputs as mi
import sparse_moe_layer_route_amd as moe
from sparse_moe_layer_route_amd import binding as B

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    moe.load()


def slice_tokens(inp, T):
    out = dict(inp)
    out["x"] = inp["x"][:T].contiguous()
    return out


def outputs(cfg, T):
    k, E = cfg.top_k, cfg.num_experts
    return (torch.full((T, k), -1, dtype=torch.int32, device=DEV),
            torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV),
            torch.full((E,), -1, dtype=torch.int32, device=DEV))


def both(cfg, inp, T):
    """(with workspace, allocation-free) results for the first T tokens."""
    sub = slice_tokens(inp, T)
    ids0, w0, c0 = outputs(cfg, T)
    ref = B.moe_layer_forward(cfg, sub, topk_ids=ids0, topk_w=w0, expert_counts=c0)
    ids1, w1, c1 = outputs(cfg, T)
    got = B.moe_layer_forward_noalloc(cfg, sub, topk_ids=ids1, topk_w=w1, expert_counts=c1)
    torch.cuda.synchronize()
    return (ref, ids0, w0, c0), (got, ids1, w1, c1)


def assert_same(a, b, what):
    for name, x, y in zip(("out", "topk_ids", "topk_w", "expert_counts"), a, b):
        assert torch.equal(x, y), f"{what}: {name} differs"


# (workload, overrides, first T, second T): decode-sized batches of the
# Step-5 and Step-3.5 layers, bf16 and FP8 experts, and a small-dims case
CASES = {
    "step5_decode_64_then_17": ("step5_decode", {}, 64, 17),
    "step5_decode_609_then_1": ("step5_decode", dict(T=609), 609, 1),
    "step35_fp8_256_then_100": ("step35_prefill", dict(T=256, expert_dtype="fp8"), 256, 100),
    "tiny_64_then_3": ("tiny", {}, 64, 3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_workspace_entry(name):
    base, over, T1, T2 = CASES[name]
    wl = mi.workload(base, **over)
    say(f"noalloc {name}: T={T1} then T={T2}")
    inp = mi.make_inputs(wl, DEV, seed=11)
    assert B.moe_workspace_size(wl.cfg, T1) <= B.moe_noalloc_max_bytes()
    r1, g1 = both(wl.cfg, inp, T1)
    assert_same(r1, g1, f"{name} first call")
    r2, g2 = both(wl.cfg, inp, T2)
    assert_same(r2, g2, f"{name} second call")


def test_noalloc_rejects_oversize_batch():
    wl = mi.workload("step5_decode", T=1024)
    assert B.moe_workspace_size(wl.cfg, 1024) > B.moe_noalloc_max_bytes()
    inp = mi.make_inputs(wl, DEV, seed=3)
    out = torch.full((1024, wl.cfg.hidden_size), 7.0, device=DEV)
    with pytest.raises(B.MoEError) as e:
        B.moe_layer_forward_noalloc(wl.cfg, inp, out=out)
    assert e.value.status == B.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "nothing may be written when the batch is too large"


def test_noalloc_zero_tokens():
    wl = mi.workload("tiny")
    inp = slice_tokens(mi.make_inputs(wl, DEV, seed=1), 0)
    out = B.moe_layer_forward_noalloc(wl.cfg, inp)
    assert out.shape == (0, wl.cfg.hidden_size)
