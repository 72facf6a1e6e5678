"""Thin Python binding of ``libmoe.so`` (the C ABI in include/moe.h).

Argument marshalling only: every function checks the tensors it is given
(device, dtype, shape, contiguity), passes their device pointers and the
current HIP stream to the C entry point of the same name, and raises
``MoEError`` on a non-OK status.  All arithmetic runs in the library's HIP
kernels; there is no CPU or PyTorch fallback, and the functions raise if the
library has not been built.  PyTorch supplies device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_BF16, MOE_FP32, MOE_FP8_E4M3_B128 = range(3)

EXPORTED = ("moe_workspace_size", "moe_route", "moe_permute", "moe_grouped_swiglu", "moe_expert_up",
            "moe_expert_down", "moe_hidden_bytes", "moe_expert_rows_bytes", "moe_shared_ffn", "moe_combine", "moe_layer_forward",
            "moe_route_replay", "moe_balanced_ids", "moe_layer_forward_routed", "moe_rmsnorm", "moe_rmsnorm_route",
            "moe_block_forward",
            "moe_saved_bytes", "moe_backward_workspace_size", "moe_layer_forward_train", "moe_layer_backward",
            "moe_layer_forward_noalloc", "moe_noalloc_max_bytes", "moe_status_string")


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class CConfig(ctypes.Structure):
    """Mirror of moe_config_t."""
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("moe_intermediate_size", ctypes.c_int32),
                ("share_expert_dim", ctypes.c_int32), ("router_scaling_factor", ctypes.c_float),
                ("norm_expert_weight", ctypes.c_int32), ("swiglu_limit", ctypes.c_float),
                ("swiglu_limit_shared", ctypes.c_float), ("expert_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


_lib = None


def load(path: Optional[str] = None):
    """Load libmoe.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_moe_layer_route_amd.build`")
    L = ctypes.CDLL(path)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    C = ctypes.POINTER(CConfig)
    sig = {
        "moe_workspace_size": [C, I64, ctypes.POINTER(SZ)],
        "moe_route": [C, I64, P, P, P, P, P, P, SZ, P],
        "moe_permute": [C, I64, P, P, P, P, P, P, SZ, P],
        "moe_grouped_swiglu": [C, I64, P, P, P, P, P, P, P, P, P, SZ, P],
        "moe_expert_up": [C, I64, P, P, P, P, P, P, P, P, SZ, P],
        "moe_expert_down": [C, I64, P, P, P, P, P, P, P, SZ, P],
        "moe_hidden_bytes": [C, I64, ctypes.POINTER(SZ)],
        "moe_expert_rows_bytes": [C, I64, ctypes.POINTER(SZ)],
        "moe_shared_ffn": [C, I64, P, P, P, P, P, SZ, P],
        "moe_combine": [C, I64, P, P, P, P, P, P, P, P],
        "moe_rmsnorm": [C, I64, P, P, ctypes.c_float, P, P],
        "moe_rmsnorm_route": [C, I64, P, P, ctypes.c_float, P, P, P, P, P, P, SZ, P],
        "moe_saved_bytes": [C, I64, ctypes.POINTER(SZ)],
        "moe_backward_workspace_size": [C, I64, ctypes.POINTER(SZ)],
        "moe_layer_forward_train": [C, I64, P, P, P, P, P, P, P, P, P, P, SZ, P, SZ, P],
        "moe_layer_backward": [C, I64, P, P, P, P, P, P, P, SZ, P, P, P, P, P, P, P, P, SZ, P],
        "moe_block_forward": [C, I64, P, P, ctypes.c_float, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "moe_layer_forward": [C, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "moe_layer_forward_noalloc": [C, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, P],
        "moe_route_replay": [C, I64, P, P, P, P, P, SZ, P],
        "moe_balanced_ids": [C, I64, P, P],
        "moe_layer_forward_routed": [C, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.moe_noalloc_max_bytes.argtypes = []
    L.moe_noalloc_max_bytes.restype = ctypes.c_size_t
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return load().moe_status_string(status).decode()


def make_config(cfg) -> CConfig:
    """moe_config_t from any object with the MoEConfig field names."""
    dt = {"bf16": MOE_BF16, "fp8": MOE_FP8_E4M3_B128}[cfg.expert_dtype]
    ot = {"fp32": MOE_FP32, "bf16": MOE_BF16}[getattr(cfg, "out_dtype", "fp32")]
    return CConfig(cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size,
                   cfg.share_expert_dim, float(cfg.router_scaling_factor), int(bool(cfg.norm_expert_weight)),
                   float(cfg.swiglu_limit), float(cfg.swiglu_limit_shared), dt, ot)


# ---- marshalling helpers ---------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor], dtype=None, shape=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def _weights_dtype(cfg):
    return torch.uint8 if cfg.expert_dtype == "fp8" else torch.bfloat16


# ---- the entry points ------------------------------------------------------------------------

def moe_workspace_size(cfg, T: int) -> int:
    n = ctypes.c_size_t(0)
    c = make_config(cfg)
    _check(load().moe_workspace_size(ctypes.byref(c), T, ctypes.byref(n)), "moe_workspace_size")
    return n.value


def workspace(cfg, T: int, device="cuda") -> torch.Tensor:
    """A device byte buffer large enough for every entry point at T tokens."""
    return torch.empty(max(moe_workspace_size(cfg, T), 1), dtype=torch.uint8, device=device)


def moe_route(cfg, x, w_router, router_bias, topk_ids=None, topk_w=None, ws=None, stream=None):
    T, H, E, k = x.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k
    topk_ids = topk_ids if topk_ids is not None else torch.empty((T, k), dtype=torch.int32, device=x.device)
    topk_w = topk_w if topk_w is not None else torch.empty((T, k), dtype=torch.float32, device=x.device)
    ws = ws if ws is not None else workspace(cfg, T, x.device)
    c = make_config(cfg)
    st = load().moe_route(ctypes.byref(c), T, _ptr(x, torch.bfloat16, (T, H), "x"),
                          _ptr(w_router, torch.bfloat16, (E, H), "w_router"),
                          _ptr(router_bias, torch.float32, (E,), "router_bias"),
                          _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
                          _ptr(topk_w, torch.float32, (T, k), "topk_w"),
                          _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_route")
    return topk_ids, topk_w


def moe_route_replay(cfg, x, w_router, topk_ids, topk_w=None, ws=None, stream=None):
    """Weights of the caller's expert choice topk_ids [T,k] under the current
    router; returns topk_w [T,k] fp32."""
    T, H, E, k = x.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k
    topk_w = topk_w if topk_w is not None else torch.empty((T, k), dtype=torch.float32, device=x.device)
    ws = ws if ws is not None else workspace(cfg, T, x.device)
    c = make_config(cfg)
    st = load().moe_route_replay(ctypes.byref(c), T, _ptr(x, torch.bfloat16, (T, H), "x"),
                                 _ptr(w_router, torch.bfloat16, (E, H), "w_router"),
                                 _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
                                 _ptr(topk_w, torch.float32, (T, k), "topk_w"),
                                 _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_route_replay")
    return topk_w


def moe_balanced_ids(cfg, T: int, topk_ids=None, device="cuda", stream=None):
    """The static balanced routing: topk_ids [T,k] int32, pair t*k+j -> expert (t*k+j) mod E."""
    k = cfg.top_k
    topk_ids = topk_ids if topk_ids is not None else torch.empty((T, k), dtype=torch.int32, device=device)
    c = make_config(cfg)
    st = load().moe_balanced_ids(ctypes.byref(c), T, _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
                                 _stream(stream))
    _check(st, "moe_balanced_ids")
    return topk_ids


def moe_permute(cfg, topk_ids, ws=None, stream=None):
    T, k, E = topk_ids.shape[0], cfg.top_k, cfg.num_experts
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    r2p = torch.empty(T * k, dtype=torch.int32, device=dev)
    p2r = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws = ws if ws is not None else workspace(cfg, T, dev)
    c = make_config(cfg)
    st = load().moe_permute(ctypes.byref(c), T, _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
                            _ptr(counts), _ptr(offsets), _ptr(r2p), _ptr(p2r),
                            _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_permute")
    return counts, offsets, r2p, p2r


def moe_expert_rows_bytes(cfg, rows: int) -> int:
    """Bytes of ``rows`` expert output rows (scaled fp16 row format)."""
    n = ctypes.c_size_t(0)
    c = make_config(cfg)
    _check(load().moe_expert_rows_bytes(ctypes.byref(c), rows, ctypes.byref(n)), "moe_expert_rows_bytes")
    return n.value


def expert_rows(cfg, rows: int, device) -> torch.Tensor:
    """A uint8 [rows, row bytes] tensor for expert output rows."""
    return torch.empty((rows, moe_expert_rows_bytes(cfg, 1)), dtype=torch.uint8, device=device)


def _rows_ptr(cfg, t, rows, name):
    return _ptr(t, torch.uint8, (rows, moe_expert_rows_bytes(cfg, 1)), name)


def moe_grouped_swiglu(cfg, x, expert_offsets, row_to_pair, w13, w2, w13_scale=None, w2_scale=None,
                       y_rows=None, ws=None, stream=None):
    """Both projections of the routed experts; y_rows: T*k expert output rows
    (uint8 [T*k, row bytes], scaled fp16 row format)."""
    T, H, E, k, I = x.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size
    wdt = _weights_dtype(cfg)
    y_rows = y_rows if y_rows is not None else expert_rows(cfg, T * k, x.device)
    ws = ws if ws is not None else workspace(cfg, T, x.device)
    fp8 = cfg.expert_dtype == "fp8"
    c = make_config(cfg)
    st = load().moe_grouped_swiglu(
        ctypes.byref(c), T, _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(row_to_pair, torch.int32, (T * k,), "row_to_pair"),
        _ptr(w13, wdt, (E, 2 * I, H), "w13"),
        _ptr(w13_scale, torch.float32, (E, 2 * I // 128, H // 128) if fp8 else None, "w13_scale"),
        _ptr(w2, wdt, (E, H, I), "w2"),
        _ptr(w2_scale, torch.float32, (E, H // 128, I // 128) if fp8 else None, "w2_scale"),
        _rows_ptr(cfg, y_rows, T * k, "y_rows"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_grouped_swiglu")
    return y_rows


def moe_hidden_bytes(cfg, T: int) -> int:
    n = ctypes.c_size_t(0)
    c = make_config(cfg)
    _check(load().moe_hidden_bytes(ctypes.byref(c), T, ctypes.byref(n)), "moe_hidden_bytes")
    return n.value


def shared_fusable(cfg) -> bool:
    """True when the shared expert can run inside the routed experts'
    launches (bf16 experts, shared width equal to the experts')."""
    return (cfg.expert_dtype == "bf16" and cfg.share_expert_dim > 0
            and cfg.share_expert_dim == cfg.moe_intermediate_size)


def moe_expert_up(cfg, x, expert_offsets, row_to_pair, w13, w13_scale=None, h=None, ws=None, stream=None,
                  ws13=None):
    """First projection + clipped SwiGLU of the routed experts (and, with
    ws13, of the shared expert as T more rows); h is a byte buffer of
    moe_hidden_bytes() (bf16 [T*k (+T), I] for bf16 experts)."""
    T, H, E, k, I = x.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size
    fp8 = cfg.expert_dtype == "fp8"
    nb = moe_hidden_bytes(cfg, T)
    h = h if h is not None else torch.empty(max(nb, 1), dtype=torch.uint8, device=x.device)
    if h.numel() * h.element_size() < nb:
        raise ValueError(f"h must hold {nb} bytes")
    ws = ws if ws is not None else workspace(cfg, T, x.device)
    c = make_config(cfg)
    Is = cfg.share_expert_dim
    st = load().moe_expert_up(
        ctypes.byref(c), T, _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(row_to_pair, torch.int32, (T * k,), "row_to_pair"),
        _ptr(w13, _weights_dtype(cfg), (E, 2 * I, H), "w13"),
        _ptr(w13_scale, torch.float32, (E, 2 * I // 128, H // 128) if fp8 else None, "w13_scale"),
        _ptr(ws13, torch.bfloat16, (2 * Is, H), "ws13"),
        _ptr(h, None, None, "h"), _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_expert_up")
    return h


def moe_expert_down(cfg, T, h, expert_offsets, w2, w2_scale=None, y_rows=None, ws=None, stream=None, ws2=None):
    """Second projection: T*k expert output rows (with ws2: T*k + T, the
    shared expert's rows last), uint8 [rows, row bytes] in the scaled fp16
    row format."""
    H, E, k, I = cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size
    fp8 = cfg.expert_dtype == "fp8"
    if h.numel() * h.element_size() < moe_hidden_bytes(cfg, T):
        raise ValueError("h is smaller than moe_hidden_bytes()")
    rows = T * k + (T if ws2 is not None else 0)
    y_rows = y_rows if y_rows is not None else expert_rows(cfg, rows, h.device)
    ws = ws if ws is not None else workspace(cfg, T, h.device)
    c = make_config(cfg)
    Is = cfg.share_expert_dim
    st = load().moe_expert_down(
        ctypes.byref(c), T, _ptr(h, None, None, "h"),
        _ptr(expert_offsets, torch.int32, (E + 1,), "expert_offsets"),
        _ptr(w2, _weights_dtype(cfg), (E, H, I), "w2"),
        _ptr(w2_scale, torch.float32, (E, H // 128, I // 128) if fp8 else None, "w2_scale"),
        _ptr(ws2, torch.bfloat16, (H, Is), "ws2"),
        _rows_ptr(cfg, y_rows, rows, "y_rows"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_expert_down")
    return y_rows


def moe_shared_ffn(cfg, x, ws13, ws2, y_shared=None, ws=None, stream=None):
    T, H, Is = x.shape[0], cfg.hidden_size, cfg.share_expert_dim
    y_shared = y_shared if y_shared is not None else torch.empty((T, H), dtype=torch.float32, device=x.device)
    ws = ws if ws is not None else workspace(cfg, T, x.device)
    c = make_config(cfg)
    st = load().moe_shared_ffn(ctypes.byref(c), T, _ptr(x, torch.bfloat16, (T, H), "x"),
                               _ptr(ws13, torch.bfloat16, (2 * Is, H), "ws13"),
                               _ptr(ws2, torch.bfloat16, (H, Is), "ws2"),
                               _ptr(y_shared, torch.float32, (T, H), "y_shared"),
                               _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_shared_ffn")
    return y_shared


def _out_dtype(cfg):
    return torch.bfloat16 if getattr(cfg, "out_dtype", "fp32") == "bf16" else torch.float32


def moe_combine(cfg, y_rows, pair_to_row, topk_w, y_shared=None, out=None, stream=None, shared_rows=None,
                residual=None):
    """y_rows: at least T*k expert output rows (uint8 [rows, row bytes], the
    routed rows first); the shared term is y_shared (fp32 [T, H]) or
    shared_rows (T rows of the same format); residual (fp32 [T, H]) is added
    last and may also be ``out``."""
    T, H, k = topk_w.shape[0], cfg.hidden_size, cfg.top_k
    rb = moe_expert_rows_bytes(cfg, 1)
    if y_rows.dim() != 2 or y_rows.shape[0] < T * k or y_rows.shape[1] != rb or y_rows.dtype != torch.uint8:
        raise ValueError(f"y_rows must be uint8 [>= {T * k}, {rb}] (got {tuple(y_rows.shape)} {y_rows.dtype})")
    out = out if out is not None else torch.empty((T, H), dtype=_out_dtype(cfg), device=y_rows.device)
    c = make_config(cfg)
    st = load().moe_combine(ctypes.byref(c), T, _ptr(y_rows, torch.uint8, None, "y_rows"),
                            _ptr(pair_to_row, torch.int32, (T * k,), "pair_to_row"),
                            _ptr(topk_w, torch.float32, (T, k), "topk_w"),
                            _ptr(y_shared, torch.float32, (T, H), "y_shared"),
                            _ptr(shared_rows, torch.uint8, (T, rb), "shared_rows"),
                            _ptr(residual, torch.float32, (T, H), "residual"),
                            _ptr(out, _out_dtype(cfg), (T, H), "out"), _stream(stream))
    _check(st, "moe_combine")
    return out


def moe_layer_forward(cfg, inp: dict, out=None, ws=None, topk_ids=None, topk_w=None, expert_counts=None,
                      stream=None):
    """The whole layer on the tensors of ``inp`` (keys as produced by the
    input generator: x, w_router, router_bias, w13, w2, [w13_scale, w2_scale],
    [ws13, ws2]).  Returns out [T,H]."""
    x = inp["x"]
    T, H, E, k, I, Is = (x.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size,
                         cfg.share_expert_dim)
    wdt = _weights_dtype(cfg)
    fp8 = cfg.expert_dtype == "fp8"
    out = out if out is not None else torch.empty((T, H), dtype=_out_dtype(cfg), device=x.device)
    ws = ws if ws is not None else workspace(cfg, T, x.device)
    c = make_config(cfg)
    st = load().moe_layer_forward(
        ctypes.byref(c), T, _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(inp["w_router"], torch.bfloat16, (E, H), "w_router"),
        _ptr(inp["router_bias"], torch.float32, (E,), "router_bias"),
        _ptr(inp["w13"], wdt, (E, 2 * I, H), "w13"),
        _ptr(inp.get("w13_scale"), torch.float32, (E, 2 * I // 128, H // 128) if fp8 else None, "w13_scale"),
        _ptr(inp["w2"], wdt, (E, H, I), "w2"),
        _ptr(inp.get("w2_scale"), torch.float32, (E, H // 128, I // 128) if fp8 else None, "w2_scale"),
        _ptr(inp.get("ws13") if Is else None, torch.bfloat16, (2 * Is, H), "ws13"),
        _ptr(inp.get("ws2") if Is else None, torch.bfloat16, (H, Is), "ws2"),
        _ptr(out, _out_dtype(cfg), (T, H), "out"),
        _ptr(topk_ids, torch.int32, (T, k), "topk_ids"), _ptr(topk_w, torch.float32, (T, k), "topk_w"),
        _ptr(expert_counts, torch.int32, (E,), "expert_counts"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_layer_forward")
    return out


def moe_noalloc_max_bytes() -> int:
    """Size of the per-GPU scratch array that moe_layer_forward_noalloc uses."""
    return int(load().moe_noalloc_max_bytes())


def moe_layer_forward_noalloc(cfg, inp: dict, out=None, topk_ids=None, topk_w=None, expert_counts=None,
                              stream=None):
    """moe_layer_forward without a workspace argument: the library's own
    per-GPU scratch array serves as the workspace and nothing is allocated
    (the output is allocated here when ``out`` is None).  Raises MoeError
    (MOE_ERR_WORKSPACE) when the batch needs more scratch than the array has."""
    x = inp["x"]
    T, H, E, k, I, Is = (x.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size,
                         cfg.share_expert_dim)
    wdt = _weights_dtype(cfg)
    fp8 = cfg.expert_dtype == "fp8"
    out = out if out is not None else torch.empty((T, H), dtype=_out_dtype(cfg), device=x.device)
    c = make_config(cfg)
    st = load().moe_layer_forward_noalloc(
        ctypes.byref(c), T, _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(inp["w_router"], torch.bfloat16, (E, H), "w_router"),
        _ptr(inp["router_bias"], torch.float32, (E,), "router_bias"),
        _ptr(inp["w13"], wdt, (E, 2 * I, H), "w13"),
        _ptr(inp.get("w13_scale"), torch.float32, (E, 2 * I // 128, H // 128) if fp8 else None, "w13_scale"),
        _ptr(inp["w2"], wdt, (E, H, I), "w2"),
        _ptr(inp.get("w2_scale"), torch.float32, (E, H // 128, I // 128) if fp8 else None, "w2_scale"),
        _ptr(inp.get("ws13") if Is else None, torch.bfloat16, (2 * Is, H), "ws13"),
        _ptr(inp.get("ws2") if Is else None, torch.bfloat16, (H, Is), "ws2"),
        _ptr(out, _out_dtype(cfg), (T, H), "out"),
        _ptr(topk_ids, torch.int32, (T, k), "topk_ids"), _ptr(topk_w, torch.float32, (T, k), "topk_w"),
        _ptr(expert_counts, torch.int32, (E,), "expert_counts"), _stream(stream))
    _check(st, "moe_layer_forward_noalloc")
    return out


def moe_layer_forward_routed(cfg, inp: dict, topk_ids, out=None, ws=None, topk_w=None, expert_counts=None,
                             stream=None):
    """The whole layer with the expert choice topk_ids [T,k] int32 given by
    the caller (routing replay or the static balanced routing); the tensors
    of ``inp`` as for moe_layer_forward (router_bias is not used).  Returns
    out [T,H]."""
    x = inp["x"]
    T, H, E, k, I, Is = (x.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size,
                         cfg.share_expert_dim)
    wdt = _weights_dtype(cfg)
    fp8 = cfg.expert_dtype == "fp8"
    out = out if out is not None else torch.empty((T, H), dtype=_out_dtype(cfg), device=x.device)
    ws = ws if ws is not None else workspace(cfg, T, x.device)
    c = make_config(cfg)
    st = load().moe_layer_forward_routed(
        ctypes.byref(c), T, _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(inp["w_router"], torch.bfloat16, (E, H), "w_router"),
        _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
        _ptr(inp["w13"], wdt, (E, 2 * I, H), "w13"),
        _ptr(inp.get("w13_scale"), torch.float32, (E, 2 * I // 128, H // 128) if fp8 else None, "w13_scale"),
        _ptr(inp["w2"], wdt, (E, H, I), "w2"),
        _ptr(inp.get("w2_scale"), torch.float32, (E, H // 128, I // 128) if fp8 else None, "w2_scale"),
        _ptr(inp.get("ws13") if Is else None, torch.bfloat16, (2 * Is, H), "ws13"),
        _ptr(inp.get("ws2") if Is else None, torch.bfloat16, (H, Is), "ws2"),
        _ptr(out, _out_dtype(cfg), (T, H), "out"),
        _ptr(topk_w, torch.float32, (T, k), "topk_w"),
        _ptr(expert_counts, torch.int32, (E,), "expert_counts"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_layer_forward_routed")
    return out


def moe_rmsnorm(cfg, resid, norm_weight, eps, x=None, stream=None):
    """Zero-centred RMSNorm of the fp32 residual rows resid [T,H] with the
    stored weight norm_weight [H] fp32 (used as 1 + g): returns x [T,H] bf16."""
    T, H = resid.shape[0], cfg.hidden_size
    x = x if x is not None else torch.empty((T, H), dtype=torch.bfloat16, device=resid.device)
    c = make_config(cfg)
    st = load().moe_rmsnorm(ctypes.byref(c), T, _ptr(resid, torch.float32, (T, H), "resid"),
                            _ptr(norm_weight, torch.float32, (H,), "norm_weight"), float(eps),
                            _ptr(x, torch.bfloat16, (T, H), "x"), _stream(stream))
    _check(st, "moe_rmsnorm")
    return x


def moe_rmsnorm_route(cfg, resid, norm_weight, eps, w_router, router_bias, x=None, topk_ids=None, topk_w=None,
                      ws=None, stream=None):
    """moe_rmsnorm then moe_route on its output (one fused pass from 512
    tokens): returns x [T,H] bf16, topk_ids [T,k] int32, topk_w [T,k] fp32."""
    T, H, E, k = resid.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k
    dev = resid.device
    x = x if x is not None else torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    topk_ids = topk_ids if topk_ids is not None else torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_w = topk_w if topk_w is not None else torch.empty((T, k), dtype=torch.float32, device=dev)
    ws = ws if ws is not None else workspace(cfg, T, dev)
    c = make_config(cfg)
    st = load().moe_rmsnorm_route(ctypes.byref(c), T, _ptr(resid, torch.float32, (T, H), "resid"),
                                  _ptr(norm_weight, torch.float32, (H,), "norm_weight"), float(eps),
                                  _ptr(w_router, torch.bfloat16, (E, H), "w_router"),
                                  _ptr(router_bias, torch.float32, (E,), "router_bias"),
                                  _ptr(x, torch.bfloat16, (T, H), "x"),
                                  _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
                                  _ptr(topk_w, torch.float32, (T, k), "topk_w"),
                                  _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_rmsnorm_route")
    return x, topk_ids, topk_w


def moe_block_forward(cfg, inp: dict, resid_out=None, ws=None, topk_ids=None, topk_w=None, expert_counts=None,
                      stream=None):
    """The MoE sub-block: resid_out = resid + layer(rmsnorm(resid)).  inp
    holds the layer's weights (as for moe_layer_forward, without x) plus
    resid [T,H] fp32, norm_weight [H] fp32 and eps.  resid_out may be
    inp["resid"] (in-place).  Returns resid_out."""
    resid = inp["resid"]
    T, H, E, k, I, Is = (resid.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size,
                         cfg.share_expert_dim)
    wdt = _weights_dtype(cfg)
    fp8 = cfg.expert_dtype == "fp8"
    resid_out = resid_out if resid_out is not None else torch.empty((T, H), dtype=torch.float32,
                                                                    device=resid.device)
    ws = ws if ws is not None else workspace(cfg, T, resid.device)
    c = make_config(cfg)
    st = load().moe_block_forward(
        ctypes.byref(c), T, _ptr(resid, torch.float32, (T, H), "resid"),
        _ptr(inp["norm_weight"], torch.float32, (H,), "norm_weight"), float(inp["eps"]),
        _ptr(inp["w_router"], torch.bfloat16, (E, H), "w_router"),
        _ptr(inp["router_bias"], torch.float32, (E,), "router_bias"),
        _ptr(inp["w13"], wdt, (E, 2 * I, H), "w13"),
        _ptr(inp.get("w13_scale"), torch.float32, (E, 2 * I // 128, H // 128) if fp8 else None, "w13_scale"),
        _ptr(inp["w2"], wdt, (E, H, I), "w2"),
        _ptr(inp.get("w2_scale"), torch.float32, (E, H // 128, I // 128) if fp8 else None, "w2_scale"),
        _ptr(inp.get("ws13") if Is else None, torch.bfloat16, (2 * Is, H), "ws13"),
        _ptr(inp.get("ws2") if Is else None, torch.bfloat16, (H, Is), "ws2"),
        _ptr(resid_out, torch.float32, (T, H), "resid_out"),
        _ptr(topk_ids, torch.int32, (T, k), "topk_ids"), _ptr(topk_w, torch.float32, (T, k), "topk_w"),
        _ptr(expert_counts, torch.int32, (E,), "expert_counts"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_block_forward")
    return resid_out


def _size(fn, cfg, T):
    n = ctypes.c_size_t(0)
    c = make_config(cfg)
    _check(getattr(load(), fn)(ctypes.byref(c), T, ctypes.byref(n)), fn)
    return n.value


def moe_saved_bytes(cfg, T: int) -> int:
    return _size("moe_saved_bytes", cfg, T)


def moe_backward_workspace_size(cfg, T: int) -> int:
    return _size("moe_backward_workspace_size", cfg, T)


def moe_layer_forward_train(cfg, inp: dict, out=None, saved=None, ws=None, topk_ids=None, stream=None):
    """The layer's forward for training (bf16 experts): also keeps what
    moe_layer_backward needs in ``saved`` (uint8, moe_saved_bytes).  With
    topk_ids [T,k] int32 the expert choice is replayed.  Returns (out, saved)."""
    x = inp["x"]
    T, H, E, k, I, Is = (x.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size,
                         cfg.share_expert_dim)
    out = out if out is not None else torch.empty((T, H), dtype=_out_dtype(cfg), device=x.device)
    saved = saved if saved is not None else torch.empty(moe_saved_bytes(cfg, T), dtype=torch.uint8,
                                                       device=x.device)
    ws = ws if ws is not None else workspace(cfg, T, x.device)
    c = make_config(cfg)
    st = load().moe_layer_forward_train(
        ctypes.byref(c), T, _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(inp["w_router"], torch.bfloat16, (E, H), "w_router"),
        _ptr(inp["router_bias"], torch.float32, (E,), "router_bias"),
        _ptr(topk_ids, torch.int32, (T, k), "topk_ids"),
        _ptr(inp["w13"], torch.bfloat16, (E, 2 * I, H), "w13"), _ptr(inp["w2"], torch.bfloat16, (E, H, I), "w2"),
        _ptr(inp.get("ws13") if Is else None, torch.bfloat16, (2 * Is, H), "ws13"),
        _ptr(inp.get("ws2") if Is else None, torch.bfloat16, (H, Is), "ws2"),
        _ptr(out, _out_dtype(cfg), (T, H), "out"), _ptr(saved, torch.uint8, None, "saved"), saved.numel(),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_layer_forward_train")
    return out, saved


def moe_layer_backward(cfg, inp: dict, saved, dout, grads=None, ws=None, stream=None):
    """Gradients for the loss sum(out * dout) (dout [T,H] fp32) from the
    state ``saved`` by moe_layer_forward_train on the same inputs.  Returns a
    dict of fp32 tensors: dx [T,H], dw_router [E,H], dw13 [E,2I,H],
    dw2 [E,H,I] and, with a shared expert, dws13 [2Is,H], dws2 [H,Is]."""
    x = inp["x"]
    T, H, E, k, I, Is = (x.shape[0], cfg.hidden_size, cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size,
                         cfg.share_expert_dim)
    dev = x.device
    f32 = torch.float32
    if grads is None:
        grads = {"dx": torch.empty((T, H), dtype=f32, device=dev),
                 "dw_router": torch.empty((E, H), dtype=f32, device=dev),
                 "dw13": torch.empty((E, 2 * I, H), dtype=f32, device=dev),
                 "dw2": torch.empty((E, H, I), dtype=f32, device=dev)}
        if Is:
            grads["dws13"] = torch.empty((2 * Is, H), dtype=f32, device=dev)
            grads["dws2"] = torch.empty((H, Is), dtype=f32, device=dev)
    ws = ws if ws is not None else torch.empty(moe_backward_workspace_size(cfg, T), dtype=torch.uint8, device=dev)
    c = make_config(cfg)
    st = load().moe_layer_backward(
        ctypes.byref(c), T, _ptr(x, torch.bfloat16, (T, H), "x"),
        _ptr(inp["w_router"], torch.bfloat16, (E, H), "w_router"),
        _ptr(inp["w13"], torch.bfloat16, (E, 2 * I, H), "w13"), _ptr(inp["w2"], torch.bfloat16, (E, H, I), "w2"),
        _ptr(inp.get("ws13") if Is else None, torch.bfloat16, (2 * Is, H), "ws13"),
        _ptr(inp.get("ws2") if Is else None, torch.bfloat16, (H, Is), "ws2"),
        _ptr(saved, torch.uint8, None, "saved"), saved.numel(), _ptr(dout, torch.float32, (T, H), "dout"),
        _ptr(grads["dx"], f32, (T, H), "dx"), _ptr(grads["dw_router"], f32, (E, H), "dw_router"),
        _ptr(grads["dw13"], f32, (E, 2 * I, H), "dw13"), _ptr(grads["dw2"], f32, (E, H, I), "dw2"),
        _ptr(grads.get("dws13"), f32, (2 * Is, H), "dws13"), _ptr(grads.get("dws2"), f32, (H, Is), "dws2"),
        _ptr(ws, torch.uint8, None, "ws"), ws.numel(), _stream(stream))
    _check(st, "moe_layer_backward")
    return grads
