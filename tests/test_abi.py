"""The C-ABI library on the host: it loads, exports every entry point the
header declares, and rejects bad arguments with the documented status before
anything is launched (these calls never reach the GPU)."""
import ctypes
import os
import re

import pytest

import moe_inputs as mi
import sparse_moe_layer_route_amd as moe
from sparse_moe_layer_route_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from sparse_moe_layer_route_amd import build
        build.build()
    return B.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status_t|const char\*|size_t)\s+(moe_\w+)\s*\(", text, re.M)))


def test_header_symbols_are_exported(lib):
    names = header_functions()
    assert set(names) == set(B.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s, want in [(0, "ok"), (1, "invalid argument"), (2, "unsupported shape or dtype"),
                    (3, "workspace too small"), (4, "HIP launch or runtime error")]:
        assert moe.status_string(s) == want


def cfg_of(**over):
    return B.make_config(mi.workload("tiny", **over).cfg)


def ws_size(c, T):
    n = ctypes.c_size_t(0)
    st = B.load().moe_workspace_size(ctypes.byref(c), T, ctypes.byref(n))
    return st, n.value


def test_workspace_size_grows_with_tokens(lib):
    c = cfg_of()
    st0, n0 = ws_size(c, 0)
    st1, n1 = ws_size(c, 64)
    st2, n2 = ws_size(c, 4096)
    assert st0 == st1 == st2 == 0 and n0 < n1 < n2


@pytest.mark.parametrize("field,value,status", [
    ("hidden_size", 0, 1), ("hidden_size", 100, 2), ("num_experts", 0, 1), ("num_experts", 2048, 2),
    ("top_k", 0, 1), ("top_k", 17, 1), ("moe_intermediate_size", 96, 2), ("share_expert_dim", -64, 1),
    ("share_expert_dim", 32, 2), ("swiglu_limit", -1.0, 1), ("swiglu_limit", float("nan"), 1),
    ("swiglu_limit_shared", float("inf"), 1), ("router_scaling_factor", float("nan"), 1),
    ("norm_expert_weight", 2, 1), ("expert_dtype", 7, 1), ("out_dtype", 2, 1), ("expert_dtype", 1, 1),
])
def test_config_validation(lib, field, value, status):
    c = cfg_of()
    setattr(c, field, value)
    assert ws_size(c, 64)[0] == status


def test_32bit_offset_limits(lib):
    # x of T x H bf16 and a 2I x H (or 2Is x H) weight panel must stay under 4 GiB
    c = cfg_of(hidden_size=4096)
    assert ws_size(c, (1 << 31) // 4096 - 1)[0] == 0
    assert ws_size(c, (1 << 31) // 4096)[0] == 2
    c = cfg_of(hidden_size=16384, moe_intermediate_size=65536)
    assert ws_size(c, 8)[0] == 2
    c = cfg_of(hidden_size=16384, moe_intermediate_size=64, share_expert_dim=65536)
    assert ws_size(c, 8)[0] == 2


def test_topk_above_32_unsupported(lib):
    c = cfg_of(num_experts=64, top_k=33)
    assert ws_size(c, 8)[0] == 2


def test_negative_tokens_and_null_out(lib):
    c = cfg_of()
    assert ws_size(c, -1)[0] == 1
    assert lib.moe_workspace_size(ctypes.byref(c), 4, None) == 1
    assert lib.moe_workspace_size(None, 4, ctypes.byref(ctypes.c_size_t())) == 1


FAKE = ctypes.c_void_p(0x1000)    # never dereferenced: every call below fails its checks first


def test_entry_points_reject_null_pointers(lib):
    c = ctypes.byref(cfg_of())
    assert lib.moe_route(c, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.moe_permute(c, 4, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.moe_grouped_swiglu(c, 4, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, 1 << 30,
                                  None) == 1
    assert lib.moe_shared_ffn(c, 4, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    assert lib.moe_combine(c, 4, FAKE, FAKE, None, None, None, None, FAKE, None) == 1
    assert lib.moe_layer_forward(c, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, None, FAKE, None,
                                 None, None, FAKE, 1 << 30, None) == 1   # shared weights missing
    assert lib.moe_route_replay(c, 4, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None) == 1    # ids missing
    assert lib.moe_balanced_ids(c, 4, None, None) == 1
    assert lib.moe_layer_forward_routed(c, 4, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
                                        None, None, FAKE, 1 << 30, None) == 1             # ids missing
    assert lib.moe_layer_forward_routed(c, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None, None, FAKE,
                                        None, None, FAKE, 1 << 30, None) == 1             # shared weights


def test_bf16_experts_reject_scales(lib):
    c = ctypes.byref(cfg_of())
    assert lib.moe_grouped_swiglu(c, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 30,
                                  None) == 1


def test_shared_ffn_needs_a_shared_expert(lib):
    c = ctypes.byref(cfg_of(share_expert_dim=0))
    assert lib.moe_shared_ffn(c, 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1


def test_small_workspace_is_reported(lib):
    c = ctypes.byref(cfg_of())
    assert lib.moe_route(c, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == 3
    assert lib.moe_permute(c, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == 3
    assert lib.moe_grouped_swiglu(c, 64, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, 16, None) == 3
    assert lib.moe_shared_ffn(c, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == 3
    st, need = ws_size(cfg_of(), 64)
    assert lib.moe_layer_forward(c, 64, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, None,
                                 None, None, FAKE, need - 1, None) == 3
    assert lib.moe_route_replay(c, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == 3
    assert lib.moe_layer_forward_routed(c, 64, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
                                        None, None, FAKE, need - 1, None) == 3


def test_zero_tokens_is_a_noop(lib):
    c = ctypes.byref(cfg_of())
    assert lib.moe_route(c, 0, None, None, None, None, None, None, 0, None) == 0
    assert lib.moe_grouped_swiglu(c, 0, None, None, None, None, None, None, None, None, None, 0, None) == 0
    assert lib.moe_combine(c, 0, None, None, None, None, None, None, None, None) == 0
    assert lib.moe_layer_forward(c, 0, None, None, None, None, None, None, None, None, None, None, None,
                                 None, None, None, 0, None) == 0
    assert lib.moe_route_replay(c, 0, None, None, None, None, None, 0, None) == 0
    assert lib.moe_balanced_ids(c, 0, None, None) == 0
    assert lib.moe_layer_forward_routed(c, 0, None, None, None, None, None, None, None, None, None, None,
                                        None, None, None, 0, None) == 0


def test_routed_entry_points_check_the_config(lib):
    c = cfg_of()
    c.top_k = c.num_experts + 1
    assert lib.moe_balanced_ids(ctypes.byref(c), 4, FAKE, None) == 1
    assert lib.moe_route_replay(ctypes.byref(c), 4, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    c = ctypes.byref(cfg_of())
    assert lib.moe_layer_forward_routed(c, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                        None, None, FAKE, 1 << 30, None) == 1             # bf16 + scale


def test_binding_refuses_cpu_tensors(lib):
    import torch
    wl = mi.workload("tiny")
    inp = mi.make_inputs(wl, "cpu")
    with pytest.raises(ValueError, match="GPU tensor"):
        moe.moe_route(wl.cfg, inp["x"], inp["w_router"], inp["router_bias"],
                      topk_ids=torch.empty(1), topk_w=torch.empty(1), ws=torch.empty(1))


def test_fp8_shape_and_scale_rules(lib):
    # FP8 experts need H and I multiples of 128
    assert ws_size(cfg_of(expert_dtype="fp8", hidden_size=192), 8)[0] == 2
    assert ws_size(cfg_of(expert_dtype="fp8", moe_intermediate_size=192), 8)[0] == 2
    assert ws_size(cfg_of(expert_dtype="fp8"), 8)[0] == 0
    c = ctypes.byref(cfg_of(expert_dtype="fp8"))
    # FP8 experts need both scale tensors
    assert lib.moe_grouped_swiglu(c, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                  None) == 1
    assert lib.moe_expert_up(c, 4, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.moe_expert_down(c, 4, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 1 << 30, None) == 1


def test_fp8_hidden_bytes(lib):
    c = cfg_of(expert_dtype="fp8")
    T = 100
    n = ctypes.c_size_t()
    assert lib.moe_hidden_bytes(ctypes.byref(c), T, ctypes.byref(n)) == 0
    P, I = T * c.top_k, c.moe_intermediate_size
    assert n.value == (P * I + 255) // 256 * 256 + (I // 128) * P * 4
    cb = cfg_of(share_expert_dim=0)
    assert lib.moe_hidden_bytes(ctypes.byref(cb), T, ctypes.byref(n)) == 0
    assert n.value == P * I * 2


def test_shared_rows_rules(lib):
    # the shared expert runs in the expert launches only with bf16 experts of its width
    ok = ctypes.byref(cfg_of())                                    # tiny: I = Is = 128
    assert lib.moe_expert_up(ok, 0, None, None, None, None, None, FAKE, None, None, 0, None) == 0
    differ = ctypes.byref(cfg_of(share_expert_dim=64))
    assert lib.moe_expert_up(differ, 4, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.moe_expert_down(differ, 4, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    fp8 = ctypes.byref(cfg_of(expert_dtype="fp8"))
    assert lib.moe_expert_up(fp8, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    # combine takes one shared term at most
    assert lib.moe_combine(ok, 4, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == 1


def test_hidden_bytes_cover_shared_rows(lib):
    T = 10
    n = ctypes.c_size_t()
    c = cfg_of()                                                   # fusable
    assert lib.moe_hidden_bytes(ctypes.byref(c), T, ctypes.byref(n)) == 0
    assert n.value == (T * c.top_k + T) * c.moe_intermediate_size * 2
    c = cfg_of(share_expert_dim=0)
    assert lib.moe_hidden_bytes(ctypes.byref(c), T, ctypes.byref(n)) == 0
    assert n.value == T * c.top_k * c.moe_intermediate_size * 2


def test_norm_and_block_argument_rules(lib):
    c = ctypes.byref(cfg_of())
    st, need = ws_size(cfg_of(), 64)
    # rmsnorm: eps must be >= 0 and finite; null pointers refused; T = 0 is a no-op
    assert lib.moe_rmsnorm(c, 4, FAKE, FAKE, -1e-5, FAKE, None) == 1
    assert lib.moe_rmsnorm(c, 4, FAKE, FAKE, float("nan"), FAKE, None) == 1
    assert lib.moe_rmsnorm(c, 4, FAKE, None, 1e-5, FAKE, None) == 1
    assert lib.moe_rmsnorm(c, 0, None, None, 1e-5, None, None) == 0
    # block: fp32 residual only, norm weight and bias required, workspace checked
    bf = ctypes.byref(cfg_of(out_dtype="bf16"))
    # w_router, router_bias, w13, w13_scale, w2, w2_scale, ws13, ws2, resid_out, ids, w, counts, ws
    args = (FAKE, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, None, None, None, FAKE)
    assert lib.moe_block_forward(bf, 64, FAKE, FAKE, 1e-5, *args, 1 << 30, None) == 1
    assert lib.moe_block_forward(c, 64, FAKE, None, 1e-5, *args, 1 << 30, None) == 1
    assert lib.moe_block_forward(c, 64, FAKE, FAKE, float("inf"), *args, 1 << 30, None) == 1
    assert lib.moe_block_forward(c, 64, FAKE, FAKE, 1e-5, *args, need - 1, None) == 3
    assert lib.moe_block_forward(c, 0, None, None, 1e-5, *((None,) * 13), 0, None) == 0
    # combine: a bf16 output may not overwrite the fp32 residual it reads
    assert lib.moe_combine(bf, 4, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == 1


def test_training_entry_points_rules(lib):
    n = ctypes.c_size_t(0)
    c = cfg_of()                                                   # tiny: Is == I, bf16
    assert lib.moe_saved_bytes(ctypes.byref(c), 64, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.moe_backward_workspace_size(ctypes.byref(c), 64, ctypes.byref(n)) == 0 and n.value > 0
    for bad in (cfg_of(expert_dtype="fp8"), cfg_of(share_expert_dim=64)):
        assert lib.moe_saved_bytes(ctypes.byref(bad), 64, ctypes.byref(n)) == 2
        assert lib.moe_backward_workspace_size(ctypes.byref(bad), 64, ctypes.byref(n)) == 2
    assert lib.moe_saved_bytes(ctypes.byref(cfg_of(share_expert_dim=0)), 64, ctypes.byref(n)) == 0
    cr = ctypes.byref(c)
    # training forward: no saved buffer; saved too small
    st, need = ws_size(cfg_of(), 64)
    assert lib.moe_layer_forward_train(cr, 64, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE,
                                       need, None) == 1
    assert lib.moe_layer_forward_train(cr, 64, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE,
                                       need, None) == 3
    # backward: missing gradient buffers; small state or scratch
    grads = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert lib.moe_layer_backward(cr, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, FAKE, FAKE, None, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.moe_layer_backward(cr, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, *grads, FAKE,
                                  1 << 30, None) == 3
    assert lib.moe_layer_backward(cr, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, FAKE, *grads, FAKE,
                                  16, None) == 3


def test_rmsnorm_route_argument_checks(lib):
    c = ctypes.byref(cfg_of())
    eps = ctypes.c_float(1e-5)
    # null x, a bad eps, a small workspace, zero tokens
    assert lib.moe_rmsnorm_route(c, 4, FAKE, FAKE, eps, FAKE, FAKE, None, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert lib.moe_rmsnorm_route(c, 4, FAKE, FAKE, ctypes.c_float(-1.0), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 1 << 30, None) == 1
    assert lib.moe_rmsnorm_route(c, 600, FAKE, FAKE, eps, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, None) == 3
    assert lib.moe_rmsnorm_route(c, 0, None, None, eps, None, None, None, None, None, None, 0, None) == 0


def test_noalloc_limit_is_exported(lib):
    assert B.moe_noalloc_max_bytes() == 64 << 20
    # a batch whose workspace exceeds the array is refused before any launch
    c = cfg_of(hidden_size=4096, num_experts=352, top_k=8, moe_intermediate_size=1536, share_expert_dim=1536)
    assert ws_size(c, 1024)[1] > B.moe_noalloc_max_bytes()
    assert lib.moe_layer_forward_noalloc(ctypes.byref(c), 1024, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                                         FAKE, FAKE, None, None, None, None) == 3
