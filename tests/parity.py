"""Comparison rules shared by the GPU parity tests.

Routing: ids are compared per token as sets (weights paired by id) and in
order where the neighbouring corrected scores differ by more than the tie
gap.  A token whose k-th and (k+1)-th corrected scores (in the oracle's
fp32 values) are closer than GAP is exempt from the exact-set check: the GPU
set must then contain every expert scoring above c_k + GAP and only experts
scoring at least c_(k+1) - GAP.

Outputs: max |gpu - oracle| <= tol * RMS(oracle output) over the compared
tokens, with tol = 2e-2 for bf16 experts and 6e-2 for FP8 experts.
"""
import numpy as np

GAP = 1e-6
TOL_BF16 = 2e-2
TOL_FP8 = 6e-2


def exempt_tokens(corrected: np.ndarray, k: int, gap: float = GAP) -> np.ndarray:
    """Boolean [T]: True where the k-th / (k+1)-th gap is below ``gap``."""
    c = np.where(np.isnan(corrected), -np.inf, corrected.astype(np.float64))
    if c.shape[1] <= k:
        return np.zeros(c.shape[0], bool)
    part = -np.sort(-c, axis=1)
    return (part[:, k - 1] - part[:, k]) < gap


def check_routing(gpu_ids, gpu_w, orc_ids, orc_w, corrected, k, w_rtol=1e-5, w_atol=1e-6, gap=GAP):
    """Asserts the routing rules; returns the exempt-token mask.  ``gap``
    widens the tie gap where the two sides route slightly different inputs."""
    gpu_ids = np.asarray(gpu_ids)
    gpu_w = np.asarray(gpu_w)
    ex = exempt_tokens(corrected, k, gap)
    c = corrected.astype(np.float64)
    T = gpu_ids.shape[0]
    assert gpu_ids.min() >= 0 and gpu_ids.max() < corrected.shape[1]
    for t in range(T):
        g, o = gpu_ids[t].tolist(), orc_ids[t].tolist()
        assert len(set(g)) == k, f"token {t}: duplicate ids {g}"
        if ex[t]:
            srt = np.sort(c[t])[::-1]
            ck, ck1 = srt[k - 1], srt[k]
            must = set(np.nonzero(c[t] > ck + gap)[0].tolist())
            may = set(np.nonzero(c[t] >= ck1 - gap)[0].tolist())
            assert must <= set(g) <= may, f"token {t}: exempt set rule violated"
            continue
        assert set(g) == set(o), f"token {t}: gpu {g} oracle {o}"
        # order: adjacent choices must agree unless their scores nearly tie
        for j in range(k):
            if g[j] != o[j]:
                assert abs(c[t, g[j]] - c[t, o[j]]) < gap, f"token {t}: order {g} vs {o}"
        gw = dict(zip(g, gpu_w[t].tolist()))
        for j, e in enumerate(o):
            assert abs(gw[e] - orc_w[t, j]) <= w_atol + w_rtol * abs(orc_w[t, j]), \
                f"token {t}: weight of expert {e}: {gw[e]} vs {orc_w[t, j]}"
    return ex


def check_counts(gpu_counts, orc_ids, gpu_ids, exempt, E):
    """Per-expert counts bit-exact once exempt tokens are taken out of both."""
    gpu_counts = np.asarray(gpu_counts).astype(np.int64)
    keep = ~exempt
    want = np.bincount(np.asarray(orc_ids)[keep].reshape(-1), minlength=E)
    gpu_ex = np.bincount(np.asarray(gpu_ids)[exempt].reshape(-1), minlength=E)
    assert gpu_counts.sum() == np.asarray(gpu_ids).size
    assert np.array_equal(gpu_counts - gpu_ex, want)


def max_err_over_rms(gpu_out, orc_out):
    gpu_out = np.asarray(gpu_out, dtype=np.float64)
    orc_out = np.asarray(orc_out, dtype=np.float64)
    rms = np.sqrt((orc_out ** 2).mean())
    return float(np.abs(gpu_out - orc_out).max() / rms), rms


def decode_rows(y_rows, H):
    """Expert output rows in the scaled fp16 row format (uint8 [rows, row
    bytes]: H fp16 values, then one int8 exponent per 128 columns) as
    float64 [rows, H]: value = fp16 * 2^exponent."""
    import torch
    y = y_rows.cpu()
    vals = y[:, :2 * H].contiguous().view(torch.float16).double().numpy()
    G = (H + 127) // 128
    ex = y[:, 2 * H:2 * H + G].contiguous().view(torch.int8).numpy().astype(np.int64)
    return vals * np.exp2(np.repeat(ex, 128, axis=1)[:, :H].astype(np.float64))


def tile_plan_sample(offsets, r2p, k, bm, rng, per_tile=1):
    """Tokens whose rows reach every (expert, m-tile) work item of a grouped
    launch with bm-row tiles (a group's rows split evenly over ceil(rows/bm)
    tiles): the first and last row of every tile, ``per_tile`` random rows
    of each, and every row of the largest expert.  Returns sorted unique
    token indices."""
    offsets = np.asarray(offsets, dtype=np.int64)
    r2p = np.asarray(r2p, dtype=np.int64)
    rows = []
    cnt = np.diff(offsets)
    for e in np.nonzero(cnt)[0]:
        n, base = int(cnt[e]), int(offsets[e])
        mt = (n + bm - 1) // bm
        for m in range(mt):
            a, b = base + m * n // mt, base + (m + 1) * n // mt
            rows += [a, b - 1] + rng.integers(a, b, per_tile).tolist()
    big = int(np.argmax(cnt))
    rows += list(range(int(offsets[big]), int(offsets[big + 1])))
    return np.unique(r2p[np.asarray(rows, dtype=np.int64)] // k)
