"""Gates that compare the GPU library's outputs with the oracle.

Tolerances (written here, used by every GPU parity test):
  * top-k: index sets bit-exact against the oracle's fp64 ranking, except
    entries whose oracle score lies within 1e-5 (relative) of the k-th largest
    score: those are ambiguous at fp32 precision, excluded and counted.
  * indexer scores: |gpu - oracle| <= (D_I + H_I + 8) * 2^-24 * sum_h |w_h|
    sum_d |q_hd k_d|, the fp32 accumulation bound of the products.
  * attention, bf16 I/O: max-abs <= 2e-2, mean-abs <= 2e-3, and per-query
    relative L2 error <= 1e-2 (the absolute gates alone are loose at small
    output magnitudes); fp32 I/O: max-abs <= 1e-5 and relative L2 <= 1e-5.
  * compression: |gpu - oracle| <= one output ulp + (m + 8) 2^-24 sum_i w_i |x_i|
    (fp32 output: 1e-6 relative to sum_i w_i |x_i|).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOPK_REL_BAND = 1e-5


def np64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a GPU/CPU tensor (bf16 by its bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return oracle.from_bf16_bits(t.contiguous().view(torch.int16).numpy().view(np.uint16))
    if t.dtype in (torch.float32, torch.float64):
        return t.numpy().astype(np.float64)
    return t.numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(np.int64) - 7)


def check_topk(gpu_idx: np.ndarray, scores64: np.ndarray, visible: int, k: int,
               rel: float = TOPK_REL_BAND):
    """Gate one query's top-k.  Returns the number of ambiguous (excluded) entries."""
    gpu_idx = np.asarray(gpu_idx, dtype=np.int64)
    want_n = min(k, visible)
    sel = gpu_idx[:want_n]
    assert np.all(gpu_idx[want_n:] == -1), "padding must be -1"
    assert np.all(sel >= 0) and np.all(sel < visible), "selected entry out of the visible range"
    assert np.all(np.diff(sel) > 0), "indices must be strictly ascending"
    if visible <= k:
        assert np.array_equal(sel, np.arange(visible))
        return 0
    s = scores64[:visible] + 0.0
    ref = oracle.topk_select(s, visible, k)
    kth = np.sort(s)[::-1][k - 1]
    amb = np.abs(s - kth) <= rel * np.maximum(np.abs(s), abs(kth))
    g = np.zeros(visible, bool)
    g[sel] = True
    o = np.zeros(visible, bool)
    o[ref[ref >= 0]] = True
    diff = g != o
    assert not np.any(diff & ~amb), (
        f"top-k differs outside the ambiguity band at entries {np.nonzero(diff & ~amb)[0][:10]}")
    return int(amb.sum()) if diff.any() else 0


def score_bound(q64, w64, k64, D_I, H_I):
    """Per-entry fp32 accumulation bound for index scores (see module doc)."""
    a = np.abs(q64) @ np.abs(k64).T            # [H, N]
    return (D_I + H_I + 8) * 2.0 ** -24 * (np.abs(w64) @ a)


def check_attention(o_gpu: np.ndarray, o_ref: np.ndarray, dtype: str, what: str = ""):
    """Gate attention outputs [..., H, D]; returns (max_abs, mean_abs, worst_rel_l2)."""
    err = np.abs(o_gpu - o_ref)
    max_abs, mean_abs = float(err.max()), float(err.mean())
    num = np.sqrt((err ** 2).sum(axis=-1))
    den = np.sqrt((o_ref ** 2).sum(axis=-1))
    rel = num / np.maximum(den, 1e-30)
    rel = np.where(den > 0, rel, num)
    worst = float(rel.max())
    if dtype == "bf16":
        assert max_abs <= 2e-2, f"{what} max-abs {max_abs}"
        assert mean_abs <= 2e-3, f"{what} mean-abs {mean_abs}"
        assert worst <= 1e-2, f"{what} rel-L2 {worst}"
    else:
        assert max_abs <= 1e-5, f"{what} max-abs {max_abs}"
        assert worst <= 1e-5, f"{what} rel-L2 {worst}"
    return max_abs, mean_abs, worst


# bf16 attention sums the softmax probabilities after rounding each to bf16
# (relative error at most 2^-9 per term, so at most 2^-9 for the sum: one term
# dominates a sharp softmax), and lse = max + log(sum); logits come from exact
# bf16 products accumulated in fp32 (error ~1e-4 at the sharp inputs' scale).
LSE_TOL_BF16 = 2.0 ** -8


def check_lse(lse_gpu: np.ndarray, lse_ref: np.ndarray, tol: float):
    lse_gpu, lse_ref = np.asarray(lse_gpu), np.asarray(lse_ref)
    empty = np.isneginf(lse_gpu)
    assert np.array_equal(empty, np.isneginf(lse_ref)), "empty-set rows differ"
    d = np.abs(lse_gpu[~empty] - lse_ref[~empty])
    assert d.size == 0 or d.max() <= tol, f"lse error {d.max()}"


def check_compress(out_gpu: np.ndarray, x64: np.ndarray, z64: np.ndarray, m: int, dtype: str):
    """Gate pooled entries [nb, C] against the oracle pooling of x64 [nb*m, C]."""
    ref = oracle.pool(x64, z64, m)
    nb = ref.shape[0]
    w = np.zeros((nb, m))
    for j in range(nb):
        e = np.exp(z64[m * j: m * j + m] - z64[m * j: m * j + m].max())
        w[j] = e / e.sum()
    mag = np.einsum("jm,jmc->jc", w, np.abs(x64[: nb * m].reshape(nb, m, -1)))
    err = np.abs(out_gpu - ref)
    if dtype == "bf16":
        allowed = bf16_ulp(ref) + (m + 8) * 2.0 ** -24 * mag
    else:
        allowed = 1e-6 * mag + 1e-30
    bad = err > allowed
    assert not bad.any(), f"compress error {err[bad][:5]} > {allowed[bad][:5]}"
    rounded = oracle.round_to_bf16(ref) if dtype == "bf16" else ref
    return float(np.mean(out_gpu != rounded))
