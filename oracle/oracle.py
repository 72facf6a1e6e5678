"""Python access to the CPU oracle (``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP path.  The functions take numpy
arrays or CPU torch tensors (bf16 tensors are passed as their raw 16-bit
patterns) and return numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("I", ctypes.c_int32), ("Is", ctypes.c_int32), ("scale", ctypes.c_float),
                ("norm", ctypes.c_int32), ("limit", ctypes.c_float),
                ("limit_shared", ctypes.c_float), ("fp8", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.orc_route.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int64, P, P, P, P, P, P, P, P]
        L.orc_layer.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int64, P, P, P, P, P, P, P, P, P,
                                P, P, P, P, P, P, P, ctypes.c_int32]
        L.orc_balanced_ids.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P]
        L.orc_backward.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int64, P, P, P, P, P, P, P, P, P, P,
                                   ctypes.c_int64, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   P, P, P, P, P, P, P]
        L.orc_act_grad.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
        L.orc_rmsnorm.argtypes = [ctypes.c_int64, ctypes.c_int32, P, P, ctypes.c_float, P]
        L.orc_bf16_round.argtypes = [ctypes.c_float]
        L.orc_bf16_round.restype = ctypes.c_uint16
        L.orc_permute.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P]
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_act.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
        L.orc_act.restype = ctypes.c_double
        L.orc_silu.argtypes = [ctypes.c_double]
        L.orc_silu.restype = ctypes.c_double
        L.orc_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _cfg(cfg) -> _Cfg:
    return _Cfg(cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size,
                cfg.share_expert_dim, float(cfg.router_scaling_factor), int(bool(cfg.norm_expert_weight)),
                float(cfg.swiglu_limit), float(cfg.swiglu_limit_shared),
                int(cfg.expert_dtype == "fp8"))


def _np(a, dtype=None):
    """CPU numpy view of a tensor/array; bf16 becomes its uint16 bit pattern."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16)
            a = a.numpy()
            if a.dtype == np.int16:
                a = a.view(np.uint16)
    except ImportError:
        pass
    a = np.ascontiguousarray(a)
    if dtype is not None:
        assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def route(cfg, x, w_router, router_bias, want_scores=False, ids_in=None):
    """Routing of every token: ids [T,k] int32, weights [T,k] fp32
    (+ logits, corrected scores [T,E] fp32 when want_scores).  With ids_in
    [T,k] the expert choices are replayed (clamped to [0, E-1]) and only the
    weights come from the router; router_bias may then be None."""
    x = _np(x, np.uint16)
    wg = _np(w_router, np.uint16)
    b = None if router_bias is None else _np(router_bias, np.float32)
    ids_in = None if ids_in is None else _np(ids_in, np.int32)
    T = x.shape[0]
    E, k = cfg.num_experts, cfg.top_k
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    lg = np.zeros((T, E), np.float32) if want_scores else None
    cs = np.zeros((T, E), np.float32) if want_scores else None
    c = _cfg(cfg)
    if ids_in is not None:
        assert ids_in.shape == (T, k), ids_in.shape
    rc = lib().orc_route(ctypes.byref(c), T, _p(x), _p(wg), _p(b), _p(ids_in), _p(ids), _p(w), _p(lg),
                         _p(cs))
    assert rc == 0, rc
    if want_scores:
        return ids, w, lg, cs
    return ids, w


def layer(cfg, inp, tokens=None, want_parts=False, ids_in=None, round_gu=False):
    """Layer output for the given token rows (all rows if tokens is None).

    inp holds the tensors of ``moe_inputs.make_inputs``.  Returns a dict with
    out [n,H] fp32, ids [n,k], w [n,k] and, if want_parts, y_routed [n,k,H]
    and y_shared [n,H].  ids_in [T,k] (rows indexed like x) replays the given
    expert choices instead of selecting them.  round_gu: the pre-activations
    are rounded to bf16 before the activation (the training forward)."""
    x = _np(inp["x"], np.uint16)
    T = x.shape[0]
    tok = None if tokens is None else np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    n = T if tok is None else tok.shape[0]
    fp8 = cfg.expert_dtype == "fp8"
    H, k, Is = cfg.hidden_size, cfg.top_k, cfg.share_expert_dim
    wg = _np(inp["w_router"], np.uint16)
    b = _np(inp["router_bias"], np.float32)
    w13 = _np(inp["w13"], np.uint8 if fp8 else np.uint16)
    w2 = _np(inp["w2"], np.uint8 if fp8 else np.uint16)
    w13s = _np(inp["w13_scale"], np.float32) if fp8 else None
    w2s = _np(inp["w2_scale"], np.float32) if fp8 else None
    ws13 = _np(inp["ws13"], np.uint16) if Is > 0 else None
    ws2 = _np(inp["ws2"], np.uint16) if Is > 0 else None
    out = np.zeros((n, H), np.float32)
    ids = np.zeros((n, k), np.int32)
    w = np.zeros((n, k), np.float32)
    yr = np.zeros((n, k, H), np.float32) if want_parts else None
    ys = np.zeros((n, H), np.float32) if want_parts else None
    c = _cfg(cfg)
    ids_in = None if ids_in is None else _np(ids_in, np.int32)
    if ids_in is not None:
        assert ids_in.shape == (T, k), ids_in.shape
    rc = lib().orc_layer(ctypes.byref(c), n, _p(tok), _p(x), _p(wg), _p(b), _p(ids_in), _p(w13), _p(w13s),
                         _p(w2), _p(w2s), _p(ws13), _p(ws2), _p(out), _p(ids), _p(w), _p(yr), _p(ys),
                         int(bool(round_gu)))
    assert rc == 0, rc
    res = {"out": out, "ids": ids, "w": w}
    if want_parts:
        res["y_routed"], res["y_shared"] = yr, ys
    return res


def permute(ids, num_experts):
    """Counts, offsets, row_to_pair and pair_to_row for the given routing."""
    ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    T, k = ids.shape
    counts = np.zeros(num_experts, np.int32)
    offs = np.zeros(num_experts + 1, np.int32)
    r2p = np.zeros(T * k, np.int32)
    p2r = np.zeros(T * k, np.int32)
    rc = lib().orc_permute(T, k, num_experts, _p(ids), _p(counts), _p(offs), _p(r2p), _p(p2r))
    assert rc == 0, rc
    return counts, offs, r2p, p2r


def balanced_ids(T, top_k, num_experts):
    """The static balanced routing: pair t*k + j goes to expert (t*k + j) mod E."""
    ids = np.zeros((T, top_k), np.int32)
    rc = lib().orc_balanced_ids(T, top_k, num_experts, _p(ids))
    assert rc == 0, rc
    return ids


def act_grad(g: float, u: float, limit: float):
    """(d act/d g, d act/d u) of the clipped SwiGLU at (g, u)."""
    dg, du = ctypes.c_double(), ctypes.c_double()
    lib().orc_act_grad(g, u, limit, ctypes.byref(dg), ctypes.byref(du))
    return dg.value, du.value


def backward(cfg, inp, dout, tokens=None, experts=None, shared=None, ids_in=None, round_gu=False):
    """Gradients of the layer (bf16 experts) for the loss sum(out * dout).

    dout [T,H] fp32.  Returns a dict: dx [n_tok,H] for ``tokens`` (all if
    None), dw_router [n_exp,H], dw13 [n_exp,2I,H], dw2 [n_exp,H,I] for
    ``experts`` (all if None), dws13 [2Is,H] and dws2 [H,Is] (when ``shared``,
    default: when there is a shared expert), and ids [T,k], the choice used.
    round_gu: the pre-activations are rounded to bf16 before the activation
    and its derivative (a training forward that keeps them in bf16)."""
    assert cfg.expert_dtype == "bf16"
    x = _np(inp["x"], np.uint16)
    T = x.shape[0]
    H, E, k, I, Is = cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size, cfg.share_expert_dim
    shared = Is > 0 if shared is None else shared
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.ascontiguousarray(np.asarray(tokens, np.int64))
    exp = np.arange(E, dtype=np.int32) if experts is None else np.ascontiguousarray(np.asarray(experts, np.int32))
    d = _np(dout, np.float32)
    assert d.shape == (T, H)
    ids_in = None if ids_in is None else _np(ids_in, np.int32)
    out = {"dx": np.zeros((tok.size, H), np.float32), "dw_router": np.zeros((exp.size, H), np.float32),
           "dw13": np.zeros((exp.size, 2 * I, H), np.float32), "dw2": np.zeros((exp.size, H, I), np.float32),
           "ids": np.zeros((T, k), np.int32)}
    if shared:
        out["dws13"] = np.zeros((2 * Is, H), np.float32)
        out["dws2"] = np.zeros((H, Is), np.float32)
    c = _cfg(cfg)
    rc = lib().orc_backward(ctypes.byref(c), T, _p(x), _p(_np(inp["w_router"], np.uint16)),
                            _p(_np(inp["router_bias"], np.float32)), _p(ids_in),
                            _p(_np(inp["w13"], np.uint16)), _p(_np(inp["w2"], np.uint16)),
                            _p(_np(inp["ws13"], np.uint16) if Is else None),
                            _p(_np(inp["ws2"], np.uint16) if Is else None), _p(d),
                            _p(tok), tok.size, _p(exp), exp.size, int(bool(shared)), int(bool(round_gu)),
                            _p(out["dx"]), _p(out["dw_router"]), _p(out["dw13"]), _p(out["dw2"]),
                            _p(out.get("dws13")), _p(out.get("dws2")), _p(out["ids"]))
    assert rc == 0, rc
    return out


def bf16_round(v: float) -> int:
    """bf16 bit pattern of an fp32 value, round to nearest even."""
    return lib().orc_bf16_round(v)


def rmsnorm(resid, norm_weight, eps):
    """Zero-centred RMSNorm of the fp32 residual rows: bf16 x [T,H] (as a
    torch bfloat16 tensor, the layer's input)."""
    import torch
    r = _np(resid, np.float32)
    g = _np(norm_weight, np.float32)
    T, H = r.shape
    assert g.shape == (H,)
    x = np.zeros((T, H), np.uint16)
    rc = lib().orc_rmsnorm(T, H, _p(r), _p(g), float(eps), _p(x))
    assert rc == 0, rc
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)


def block(cfg, inp, tokens=None, ids_in=None):
    """The MoE sub-block around the layer: x = rmsnorm(resid), then
    resid_out = resid + layer(x) in fp32.  inp holds the layer's tensors
    plus resid [T,H] fp32, norm_weight [H] fp32 and eps.  Returns the
    layer's dict with x (bf16 [T,H]) and resid_out [n,H] added."""
    x = rmsnorm(inp["resid"], inp["norm_weight"], inp["eps"])
    res = layer(cfg, dict(inp, x=x), tokens=tokens, ids_in=ids_in)
    r = _np(inp["resid"], np.float32)
    rows = r if tokens is None else r[np.asarray(tokens, dtype=np.int64)]
    res["x"] = x
    res["resid_out"] = (rows + res["out"]).astype(np.float32)
    return res


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(code)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def act(g: float, u: float, limit: float) -> float:
    return lib().orc_act(g, u, limit)


def num_threads() -> int:
    return lib().orc_num_threads()
