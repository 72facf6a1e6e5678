"""Brute-force second implementation of the MoE layer for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Pure Python floats (IEEE double) with no rounding
to fp32 anywhere, and top-k by a *full sort* of all experts instead of the C
oracle's k selection rounds.  It exists so the C oracle (``moe_oracle.c``) is
checked against an implementation that shares nothing with it but the
definition (page "MAX 中 Step-3.5-Flash 架构解析…", section
"MoE：共享专家、sigmoid 路由与激活裁剪"): sigmoid scores, bias-corrected top-k,
weights from raw scores, optional normalisation, router scaling, clipped
SwiGLU experts plus an always-on shared expert.
"""
from __future__ import annotations

import math


def _sigmoid(a: float) -> float:
    if a >= 0:
        return 1.0 / (1.0 + math.exp(-a))
    z = math.exp(a)
    return z / (1.0 + z)


def _swiglu_clipped(g: float, u: float, limit: float) -> float:
    sg = g * _sigmoid(g)
    if limit == 0.0:
        return sg * u
    return min(sg, limit) * max(-limit, min(u, limit))


def _matvec(rows, v):
    return [math.fsum(r[i] * v[i] for i in range(len(v))) for r in rows]


def token_forward(cfg, x, wg, bias, w13, w2, ws13=None, ws2=None, ids=None):
    """One token.  All arguments are nested Python lists of floats:
    x [H], wg [E][H], bias [E], w13 [E][2I][H], w2 [E][H][I], ws13 [2Is][H],
    ws2 [H][Is].  ids (optional, k ints in [0, E)) replays an expert choice
    instead of selecting one.  Returns (ids, weights, out[H], corrected
    scores)."""
    E, k, I = cfg.num_experts, cfg.top_k, cfg.moe_intermediate_size
    logits = _matvec(wg, x)
    s = [_sigmoid(a) for a in logits]
    c = [s[e] + bias[e] for e in range(E)]
    if ids is None:
        order = sorted(range(E), key=lambda e: (0 if c[e] == c[e] else 1,
                                                -c[e] if c[e] == c[e] else 0.0, e))
        ids = order[:k]
    ids = list(ids)
    w = [s[e] for e in ids]
    if cfg.norm_expert_weight:
        tot = math.fsum(w)
        w = [v / tot for v in w]
    w = [v * cfg.router_scaling_factor for v in w]
    out = [0.0] * len(x)
    for wj, e in zip(w, ids):
        gu = _matvec(w13[e], x)
        h = [_swiglu_clipped(gu[i], gu[I + i], cfg.swiglu_limit) for i in range(I)]
        y = _matvec(w2[e], h)
        out = [o + wj * yy for o, yy in zip(out, y)]
    if cfg.share_expert_dim > 0:
        Is = cfg.share_expert_dim
        gu = _matvec(ws13, x)
        h = [_swiglu_clipped(gu[i], gu[Is + i], cfg.swiglu_limit_shared) for i in range(Is)]
        y = _matvec(ws2, h)
        out = [o + yy for o, yy in zip(out, y)]
    return ids, w, out, c
