"""Plain fp64 CPU definition of CSA and HCA.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark
use this module.  It is deliberately slow and literal: each function is the
definition written out with NumPy in float64, with a library matmul / sort
as the only building blocks, no blocking and no reordering.

Source: the technical review "DeepSeek V4 技术解读" (takeshell.com):
  * §2.1 CSA: the KV entries of every m consecutive tokens are merged into one
    entry by a weighted aggregation (sequence length becomes n/m); a Lightning
    Indexer forms indexer queries for each query token, scores them against
    the compressed entries and keeps the top-k compressed blocks; core
    attention runs only over those k entries.  V4-Pro parameters: m = 4,
    64 indexer heads of dimension 128, top-k = 1024.
  * §2.2 HCA: m' = 128 tokens per entry, then full attention over all
    compressed entries with no sparse selection.
  * §5 (FP4 quantisation-aware training): the indexer's QK path runs in FP4
    E2M1, dequantised to FP8 E4M3 without loss.

Where the pages are silent this module takes these readings (each is used
below and listed with its reason in the design notes):
  R1 pooling weights: one logit per raw token; a block's weights are the
     softmax of its m logits; the same weights pool every channel
     (core K, core V and the indexer key).
  R2 one shared KV head (K and V separate) for all query heads, and one
     shared indexer key per compressed entry.
  R3 index score s(t, j) = sum_h w[t, h] * max(0, q_I[t, h] . k_I[j]),
     unscaled.
  R4 causality: entry j is visible to query position t iff m (j + 1) <= t + 1,
     so V(t) = min(N, floor((t + 1) / m)); no raw tokens are attended.
  R5 top-k: rank by (score descending, index ascending), -0.0 equal to +0.0;
     keep min(k, V(t)) entries; return them in ascending index order padded
     with -1.  One set per query token, shared by all heads.
  R6 attention: softmax scale 1/sqrt(D) unless given; an empty set gives
     output 0 and log-sum-exp -inf.
  R7 FP4: E2M1 codes (sign, 2 exponent bits with bias 1, 1 mantissa bit),
     element 2i in the low nibble, one fp32 scale per 32 consecutive
     elements; the value is code value times scale.
  R8 FP4 with power-of-two block scales (the MX-native variant): the same
     codes with one E8M0 scale byte per 32 elements (value 2**(byte - 127),
     byte 255 is NaN), the encoding of the OCP Microscaling formats.  §5's
     claim that FP4 dequantises to FP8 E4M3 without loss while the scale
     stays within a threshold is exact for such scales: every E2M1 value
     times 2**e is an E4M3 value for -8 <= e <= 6.
  R9 sliding window (§2.3's first layers): a query at position p attends the
     uncompressed tokens max(0, P - window) .. P - 1 with P = min(p + 1,
     tokens cached), i.e. its own token and the window - 1 before it; the
     pages give no window size, so it is an argument.
  R10 combining branches (§2.3, the local window kept next to the compressed
     global retrieval): two attention results over disjoint key sets, each
     given as (output, log-sum-exp) under the same softmax scale, combine
     into the attention over the union of the sets.
  R11 appending to the cache: after token t (0-based) is added, a block is
     complete when (t + 1) is a multiple of m; its entry j = (t + 1) / m - 1
     pools tokens m j .. m j + m - 1 (R1) and the sequence then holds j + 1
     entries.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np

NEG_INF = -np.inf


# ------------------------------------------------------------------ number formats
def from_bf16_bits(bits) -> np.ndarray:
    """bf16 bit patterns (any integer array) -> float64 values (exact)."""
    u = np.asarray(bits).astype(np.uint32) & 0xFFFF
    return (u << 16).view(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even (fp64 result).

    bf16 has 8 significant bits and fp32's exponent range; below 2**-126 the
    spacing is fixed at 2**-133.  Overflow goes to +-inf.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])                      # x = f * 2**e, 0.5 <= |f| < 1
    ulp = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    r = np.rint(x[fin] / ulp) * ulp              # rint: half to even
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, r), r)
    out[fin] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e = (code >> 1) & 3
    mbit = code & 1
    mag = 0.5 * mbit if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * mbit)
    return sign * mag


def e4m3_value(byte: int) -> float:
    """Value of an 8-bit E4M3 byte (OCP FP8: bias 7, S.1111.111 is NaN, no infinities)."""
    sign = -1.0 if (byte >> 7) & 1 else 1.0
    e = (byte >> 3) & 15
    mant = byte & 7
    if e == 15 and mant == 7:
        return math.nan
    if e == 0:
        mag = (mant / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + mant / 8.0) * 2.0 ** (e - 7)
    return sign * mag


def e2m1_to_e4m3(code: int) -> int:
    """The E4M3 byte that holds exactly the value of an E2M1 code (same sign).

    Found by searching all 256 E4M3 bytes, so it is the definition itself;
    §5 of the review says this dequantisation loses nothing.
    """
    v = e2m1_value(code)
    want_sign = (code >> 3) & 1
    for b in range(256):
        if (b >> 7) == want_sign and e4m3_value(b) == v:
            return b
    raise ValueError(f"E2M1 code {code} has no exact E4M3 encoding")


def fp4_dequantize(codes, scales, block: int = 32) -> np.ndarray:
    """Packed E2M1 codes [..., D/2] and fp32 scales [..., D/block] -> float64 [..., D]."""
    c = np.asarray(codes, dtype=np.uint8)
    lo = c & 0xF
    hi = c >> 4
    nib = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.uint8)
    nib[..., 0::2] = lo
    nib[..., 1::2] = hi
    table = np.array([e2m1_value(i) for i in range(16)], dtype=np.float64)
    vals = table[nib]
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    D = vals.shape[-1]
    return vals * np.repeat(s, block, axis=-1)[..., :D]


def e8m0_value(byte: int) -> float:
    """R8: value of an E8M0 scale byte (OCP MX): 2**(byte - 127); 255 is NaN."""
    byte = int(byte)
    if not 0 <= byte <= 255:
        raise ValueError(byte)
    return math.nan if byte == 255 else math.ldexp(1.0, byte - 127)


def e2m1_scaled_to_e4m3(code: int, e: int) -> Optional[int]:
    """R8 / §5: the E4M3 byte holding exactly e2m1_value(code) * 2**e, or None.

    Found by searching all 256 E4M3 bytes (the definition itself)."""
    v = math.ldexp(e2m1_value(code), e)
    want_sign = (code >> 3) & 1
    for b in range(256):
        if (b >> 7) == want_sign and e4m3_value(b) == v:
            return b
    return None


def mx4_quantize(x, block: int = 32):
    """R8: MX FP4 encoding of the last dim of x (OCP Microscaling formats).

    Per block of 32 elements: shared exponent e = floor(log2(amax)) - 2 (2 is
    the largest E2M1 exponent), clamped to [-127, 127], -127 for an all-zero
    block; scale byte e + 127.  Each element's magnitude |x| / 2**e goes to
    the nearest E2M1 magnitude, a tie to the code with an even mantissa bit,
    anything above 5 to 6 (saturation); the sign bit is x's own, so -0.0 and
    values that round to zero from below keep it.  Element 2i is the low
    nibble of byte i.  Returns (codes uint8 [..., D/2], scale bytes uint8
    [..., D/32]).
    """
    xs = np.asarray(x, dtype=np.float64)
    D = xs.shape[-1]
    if D % block or D % 2:
        raise ValueError(D)
    xb = xs.reshape(xs.shape[:-1] + (D // block, block))
    amax = np.abs(xb).max(axis=-1)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    e[nz] = np.frexp(amax[nz])[1] - 1 - 2         # amax = f 2^p, f in [0.5, 1): floor(log2) = p - 1
    e = np.clip(e, -127, 127)
    a = np.abs(xb) * np.ldexp(1.0, -e)[..., None]
    # magnitude index 0..7 over {0, .5, 1, 1.5, 2, 3, 4, 6}: strict '>' where the
    # tie belongs to the lower (even) code, '>=' where it belongs to the upper
    mag = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) +
           (a > 2.5) + (a >= 3.5) + (a > 5.0)).astype(np.uint8)
    code = (mag | (np.signbit(xb).astype(np.uint8) << 3)).reshape(xs.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def mx4_dequantize(codes, scale_bytes, block: int = 32) -> np.ndarray:
    """R8: packed E2M1 codes [..., D/2] and E8M0 scale bytes [..., D/block] -> float64 [..., D]."""
    sb = np.asarray(scale_bytes, dtype=np.uint8)
    table = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)
    c = np.asarray(codes, dtype=np.uint8)
    nib = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.uint8)
    nib[..., 0::2] = c & 0xF
    nib[..., 1::2] = c >> 4
    vals = np.array([e2m1_value(i) for i in range(16)], dtype=np.float64)[nib]
    D = vals.shape[-1]
    return vals * np.repeat(table[sb], block, axis=-1)[..., :D]


# ------------------------------------------------------------------ CSA / HCA steps
def visible_count(t: int, m: int, n_entries: int) -> int:
    """R4: number of compressed entries query position t may see."""
    return max(0, min(int(n_entries), (int(t) + 1) // int(m)))


def pool(x, z, m: int) -> np.ndarray:
    """§2.1 / §2.2 compression: entry j = sum_i w_i x[m j + i] with w = softmax(z block) (R1).

    x [n, C] (float64 or convertible), z [n] -> [n // m, C] float64.  Only
    complete blocks are produced.
    """
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    n_blocks = x.shape[0] // m
    out = np.zeros((n_blocks, x.shape[1]), dtype=np.float64)
    for j in range(n_blocks):
        zb = z[m * j: m * j + m]
        e = np.exp(zb - zb.max())
        w = e / e.sum()
        out[j] = w @ x[m * j: m * j + m]
    return out


def index_scores(q_idx, w_idx, k_idx, visible: int) -> np.ndarray:
    """§2.1 Lightning Indexer score of one query token against every entry (R3).

    q_idx [H_I, D_I], w_idx [H_I], k_idx [N, D_I] -> s [N] float64 with
    s[j] = sum_h w[h] max(0, q_idx[h] . k_idx[j]) for j < visible, -inf after.
    """
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w_idx, dtype=np.float64)
    K = np.asarray(k_idx, dtype=np.float64)
    s = np.full(K.shape[0], NEG_INF)
    if visible > 0:
        dots = q @ K[:visible].T                   # [H_I, visible]
        s[:visible] = w @ np.maximum(dots, 0.0)
    return s


def topk_select(scores, visible: int, k: int) -> np.ndarray:
    """§2.1 top-k of the visible entries (R5): int64 [k], ascending, -1 padded."""
    s = np.asarray(scores, dtype=np.float64)[:visible] + 0.0   # -0.0 -> +0.0
    order = np.lexsort((np.arange(visible), -s))               # key (-s, j)
    take = np.sort(order[: min(k, visible)])
    out = np.full(k, -1, dtype=np.int64)
    out[: take.size] = take
    return out


def attend(q, k_cache, v_cache, selected: Iterable[int], scale: Optional[float] = None):
    """§2.1 core attention over the selected entries only (R2, R6).

    q [H, D], k_cache / v_cache [N, D], ``selected`` entry indices (entries
    outside [0, N) are ignored).  Returns (o [H, D], lse [H]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(k_cache, dtype=np.float64)
    Vc = np.asarray(v_cache, dtype=np.float64)
    N = K.shape[0]
    sel = np.array([int(j) for j in selected if 0 <= int(j) < N], dtype=np.int64)
    H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if sel.size == 0:
        return np.zeros((H, D)), np.full(H, NEG_INF)
    logits = scale * (q @ K[sel].T)                # [H, |S|]
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ Vc[sel]) / l
    lse = (mx + np.log(l))[:, 0]
    return o, lse


def hca_attend(q, k_cache, v_cache, visible: int, scale: Optional[float] = None):
    """§2.2 HCA: attention over every visible compressed entry, no selection."""
    return attend(q, k_cache, v_cache, range(visible), scale)


def swa_attend(q, k_cache, v_cache, q_pos: int, n_tokens: int, window: int,
               scale: Optional[float] = None):
    """R9 sliding-window attention ("DeepSeek V4 技术解读", §2.3, the first
    layers): over uncompressed tokens, the query's own token and the
    window - 1 tokens before it (window is an argument; the pages give none)."""
    P = min(q_pos + 1, n_tokens)
    return attend(q, k_cache, v_cache, range(max(0, P - window), P), scale)


def merge_attention(o1, lse1, o2, lse2):
    """R10: the attention over S1 u S2 from the results over disjoint S1 and S2.

    o1, o2 [H, D], lse1, lse2 [H] (natural log, -inf for an empty set) ->
    (o [H, D], lse [H]) in float64: lse = log(exp(lse1) + exp(lse2)) and
    o = exp(lse1 - lse) o1 + exp(lse2 - lse) o2; both sets empty gives 0, -inf.
    """
    o1, o2 = np.asarray(o1, dtype=np.float64), np.asarray(o2, dtype=np.float64)
    l1, l2 = np.asarray(lse1, dtype=np.float64), np.asarray(lse2, dtype=np.float64)
    H = l1.shape[0]
    o = np.zeros_like(o1)
    lse = np.full(H, NEG_INF)
    for h in range(H):
        if l1[h] == NEG_INF and l2[h] == NEG_INF:
            continue
        mx = max(l1[h], l2[h])
        e1 = math.exp(l1[h] - mx) if l1[h] != NEG_INF else 0.0
        e2 = math.exp(l2[h] - mx) if l2[h] != NEG_INF else 0.0
        lse[h] = mx + math.log(e1 + e2)
        o[h] = (e1 * o1[h] + e2 * o2[h]) / (e1 + e2)
    return o, lse


def append_block(x_block, z_block, t: int, m: int):
    """R11: the entry that appending token t completes, or None.

    x_block [m, C], z_block [m]: the m most recent tokens (t - m + 1 .. t) ->
    (entry index j, pooled row [C] float64) when (t + 1) % m == 0, else None.
    """
    if (t + 1) % m:
        return None
    return (t + 1) // m - 1, pool(x_block, z_block, m)[0]


# ------------------------------------------------------------------ whole path
def csa_reference(*, q, q_idx, w_idx, k_cache, v_cache, k_idx, q_pos: int, m: int,
                  k: int, n_entries: int, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """One query token through the §2.1 pipeline on already-compressed caches."""
    V = visible_count(q_pos, m, n_entries)
    s = index_scores(q_idx, w_idx, k_idx, V)
    idx = topk_select(s, V, k)
    o, lse = attend(q, k_cache, v_cache, idx, scale)
    return {"visible": V, "scores": s, "idx": idx, "o": o, "lse": lse}
