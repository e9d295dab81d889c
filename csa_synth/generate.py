"""Seeded generators for the workloads in ``workloads.py``.

Recipe (every tensor is independent, so any subset can be regenerated):

* Generator: ``torch.Generator`` on the target device, seeded with
  ``workload.seed * 1000 + tensor_id`` (ids below).  CPU and GPU draws of
  the same seed differ; parity tests always hand the oracle the exact bits
  that the GPU consumed, so that does not matter.
* Draws are float32 ``standard_normal`` times the tensor's std, then stored:
  fp32 as is, bf16 by round-to-nearest-even, FP4 by ``fp4_quantize`` (fp32
  block scales) or ``mx4_quantize`` (E8M0 block scales).
* Distributions: pooling logits N(0, 1); Q, K, V, indexer q / k
  N(0, 1)/sqrt(dim); indexer head weights N(0, w_std) in fp32.

Tensor ids: 1 raw tokens (K | V | K_I channels; drawn sequence by sequence
from one generator), 2 pooling logits,
3 cached K_c, 4 cached V_c, 5 cached K_I, 6 q, 7 q_I, 8 w_I.
"""
from __future__ import annotations

from typing import Dict

import numpy as np
import torch

from .workloads import Workload, std_for_dim

TENSOR_IDS = {"raw": 1, "logits": 2, "k_cache": 3, "v_cache": 4, "ki_cache": 5,
              "q": 6, "q_idx": 7, "w_idx": 8}


# ---------------------------------------------------------------- storage formats
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# E2M1 magnitude grid, indexed by the 3 low code bits (exponent bias 1, one
# mantissa bit; code 1 is the subnormal 0.5).
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
_E2M1_MIDS = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2


def _e2m1_pack(y: np.ndarray, shape) -> np.ndarray:
    """Round float32 ``y`` to the nearest E2M1 value (ties to the even code,
    saturating at +-6) and pack pairs, element 2i in the low nibble."""
    a = np.abs(y)
    lo = np.searchsorted(_E2M1_MIDS, a, side="left")    # midpoints strictly below a
    hi = np.searchsorted(_E2M1_MIDS, a, side="right")   # midpoints at or below a
    tie = lo != hi                                      # a sits exactly on a midpoint
    idx = np.where(tie, np.where(lo % 2 == 0, lo, lo + 1), lo)
    idx = np.minimum(idx, 7).astype(np.uint8)
    sign = (np.signbit(y)).astype(np.uint8) << 3
    code = (idx | sign).reshape(shape)
    return (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)


def fp4_quantize(x: torch.Tensor, block: int = 32):
    """Encode the last dim of ``x`` as FP4 E2M1 codes with one fp32 scale per block.

    scale = amax(block) / 6 (1.0 for an all-zero block); code = x / scale rounded
    to the nearest E2M1 value, ties to the even code, saturating at +-6.
    Returns (codes uint8 [..., dim/2] with element 2i in the low nibble,
    scales float32 [..., dim/block]).
    """
    xs = x.detach().to("cpu", torch.float32).numpy()
    dim = xs.shape[-1]
    assert dim % block == 0 and dim % 2 == 0
    xb = xs.reshape(xs.shape[:-1] + (dim // block, block))
    amax = np.abs(xb).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(6.0), np.float32(1.0)).astype(np.float32)
    y = (xb / scale[..., None]).astype(np.float32)
    return torch.from_numpy(_e2m1_pack(y, xs.shape)), torch.from_numpy(scale)


def mx4_quantize(x: torch.Tensor, block: int = 32):
    """Encode the last dim of ``x`` as MX FP4: E2M1 codes with one E8M0 scale
    byte per block, as the OCP Microscaling formats define it.

    Shared exponent e = floor(log2(amax)) - 2 (2 is the largest E2M1
    exponent), clamped to [-127, 127]; an all-zero block takes -127.  Code =
    x / 2**e rounded to the nearest E2M1 value, ties to the even code,
    saturating at +-6 (amax / 2**e lies in [4, 8)).  Scale byte = e + 127.
    Returns (codes uint8 [..., dim/2], scale bytes uint8 [..., dim/block]).
    """
    xs = x.detach().to("cpu", torch.float32).numpy()
    dim = xs.shape[-1]
    assert dim % block == 0 and dim % 2 == 0
    xb = xs.reshape(xs.shape[:-1] + (dim // block, block))
    amax = np.abs(xb).max(axis=-1).astype(np.float64)
    _, k = np.frexp(amax)                     # amax = f * 2**k, 0.5 <= f < 1: floor(log2) = k - 1
    e = np.where(amax > 0, k - 1 - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    y = (xb.astype(np.float64) * np.ldexp(1.0, -e)[..., None]).astype(np.float32)
    return (torch.from_numpy(_e2m1_pack(y, xs.shape)),
            torch.from_numpy((e + 127).astype(np.uint8)))


# ---------------------------------------------------------------- drawing
def _gen(w: Workload, tensor: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + TENSOR_IDS[tensor])
    return g


def _normal(w: Workload, tensor: str, shape, std: float, device) -> torch.Tensor:
    g = _gen(w, tensor, device)
    out = torch.empty(shape, dtype=torch.float32, device=device)
    out.normal_(0.0, 1.0, generator=g)
    if std != 1.0:
        out.mul_(std)
    return out


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return x.to(torch.bfloat16)   # round to nearest even
    raise ValueError(dtype)


def make_inputs(w: Workload, device="cpu", parts=None,
                keep_unquantised: bool = False) -> Dict[str, torch.Tensor]:
    """Draw the inputs of workload ``w`` on ``device``.

    Returns a dict of tensors (names below); ``parts`` limits which are drawn.
      raw       [B, n_raw, C]   K | V | K_I channels of the tokens to pool
      logits    [B, n_raw]      fp32 pooling logits
      k_cache   [B, N, D]       cached compressed K (rows >= n_cache left zero
      v_cache   [B, N, D]       for the compress stage to fill)
      ki_cache  [B, N, D_I]     cached compressed indexer keys (bf16 / f32)
      ki_codes  [B, N, D_I/2]   (fp4, mx4) E2M1 codes, ki_scale [B, N, D_I/32]
                                fp32 (fp4) or E8M0 bytes (mx4)
      q         [B, Tq, H, D]
      q_idx     [B, Tq, H_I, D_I] (fp4, mx4: q_codes / q_scale)
      w_idx     [B, Tq, H_I]    fp32
      q_pos     [B, Tq] int32, n_entries [B] int32
    keep_unquantised (fp4, mx4): also return the fp32 draws before encoding,
      ki_unquantised [B, N, D_I] and q_idx_unquantised [B, Tq, H_I, D_I].
    """
    want = set(parts) if parts is not None else None

    def need(name):
        return want is None or name in want

    out: Dict[str, torch.Tensor] = {}
    B, N, D = w.B, w.N, w.D
    if w.n_raw and need("raw"):
        # Drawn one sequence at a time from one generator (no full-size fp32
        # temporary); per-channel-group std: K and V by D, K_I by D_I.
        g = _gen(w, "raw", device)
        tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        raw = torch.empty((B, w.n_raw, w.C), dtype=tdt, device=device)
        for b in range(B):
            xb = torch.empty((w.n_raw, w.C), dtype=torch.float32, device=device)
            xb.normal_(0.0, 1.0, generator=g)
            xb[:, : 2 * D].mul_(std_for_dim(D))
            if w.kind == "csa":
                xb[:, 2 * D:].mul_(std_for_dim(w.D_I))
            raw[b] = _store(xb, w.dtype)
            del xb
        out["raw"] = raw
    if w.n_raw and need("logits"):
        out["logits"] = _normal(w, "logits", (B, w.n_raw), 1.0, device)
    if need("k_cache"):
        kc = torch.zeros((B, N, D), dtype=torch.float32, device=device)
        if w.n_cache:
            kc[:, : w.n_cache] = _normal(w, "k_cache", (B, w.n_cache, D), std_for_dim(D), device)
        out["k_cache"] = _store(kc, w.dtype)
        del kc
    if need("v_cache"):
        vc = torch.zeros((B, N, D), dtype=torch.float32, device=device)
        if w.n_cache:
            vc[:, : w.n_cache] = _normal(w, "v_cache", (B, w.n_cache, D), std_for_dim(D), device)
        out["v_cache"] = _store(vc, w.dtype)
        del vc
    if w.kind == "csa" and need("ki_cache"):
        kic = torch.zeros((B, N, w.D_I), dtype=torch.float32, device=device)
        if w.n_cache:
            kic[:, : w.n_cache] = _normal(w, "ki_cache", (B, w.n_cache, w.D_I),
                                          std_for_dim(w.D_I), device)
        if w.index_dtype in ("fp4", "mx4"):
            codes, scale = (fp4_quantize if w.index_dtype == "fp4" else mx4_quantize)(kic)
            out["ki_codes"] = codes.to(device)
            out["ki_scale"] = scale.to(device)
            if keep_unquantised:
                out["ki_unquantised"] = kic.clone()
        else:
            out["ki_cache"] = _store(kic, w.index_dtype)
        del kic
    if need("q"):
        out["q"] = _store(_normal(w, "q", (B, w.Tq, w.H, D), std_for_dim(D), device), w.dtype)
    if w.kind == "csa" and need("q_idx"):
        qi = _normal(w, "q_idx", (B, w.Tq, w.H_I, w.D_I), std_for_dim(w.D_I), device)
        if w.index_dtype in ("fp4", "mx4"):
            codes, scale = (fp4_quantize if w.index_dtype == "fp4" else mx4_quantize)(qi)
            out["q_codes"] = codes.to(device)
            out["q_scale"] = scale.to(device)
            if keep_unquantised:
                out["q_idx_unquantised"] = qi
        else:
            out["q_idx"] = _store(qi, w.index_dtype)
    if w.kind == "csa" and need("w_idx"):
        out["w_idx"] = _normal(w, "w_idx", (B, w.Tq, w.H_I), w.w_std, device)
    if need("q_pos"):
        pos = torch.arange(w.q_pos0, w.q_pos0 + w.Tq, dtype=torch.int32, device=device)
        out["q_pos"] = pos.unsqueeze(0).repeat(B, 1).contiguous()
    if need("n_entries"):
        out["n_entries"] = torch.full((B,), N, dtype=torch.int32, device=device)
    return out


# Sliding-window decode inputs: B sequences with a cache of n_tokens
# uncompressed tokens each (K, V ~ N(0,1)/sqrt(D), bf16) and one query token
# at the last position (q ~ N(0,1)/sqrt(D), H heads).
SWA_DECODE = dict(B=32, n_tokens=131072, H=64, D=128, window=4096, seed=5)


def make_swa_inputs(B: int, n_tokens: int, H: int, D: int, seed: int,
                    device="cpu") -> Dict[str, torch.Tensor]:
    out = {}
    std = 1.0 / np.sqrt(D)
    for i, (name, shape) in enumerate((("q", (B, 1, H, D)), ("k", (B, n_tokens, D)),
                                       ("v", (B, n_tokens, D)))):
        g = torch.Generator(device=device)
        g.manual_seed(seed * 1000 + 100 + i)
        x = torch.empty(shape, dtype=torch.float32, device=device)
        x.normal_(0.0, 1.0, generator=g)
        out[name] = (x * std).to(torch.bfloat16)
    out["q_pos"] = torch.full((B, 1), n_tokens - 1, dtype=torch.int32, device=device)
    out["n_tokens"] = torch.full((B,), n_tokens, dtype=torch.int32, device=device)
    return out


def sharp_variant(x: torch.Tensor, factor: float) -> torch.Tensor:
    """Scale a stored bf16/fp32 tensor by ``factor`` (re-rounded): used to draw
    'sharp' attention inputs whose softmax is far from uniform."""
    return (x.float() * factor).to(x.dtype)
