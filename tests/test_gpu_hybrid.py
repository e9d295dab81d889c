"""GPU parity for the pieces around the decode step: incremental compression
(entries formed as tokens arrive), merging a sliding-window branch with a
compressed branch, and two invariants of the indexer selection (scaling the
head weights by 2 and permuting the entries)."""
import math
import sys

import numpy as np
import pytest
import torch

import long_context_attention_24_amd as csa
import oracle
from parity import LSE_TOL_BF16, bf16_ulp, check_attention, check_lse, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _randn(shape, std, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.empty(shape, device=DEV, dtype=torch.float32).normal_(0, 1, generator=g)
    return (x * std).to(dtype)


def _check_rows(got, x64, z64, m, dtype, what):
    """got [C] against the oracle pooling of one block (bound as in csa_compress)."""
    ref = oracle.pool(x64, z64, m)[0]
    e = np.exp(z64 - z64.max())
    w = e / e.sum()
    mag = w @ np.abs(x64)
    err = np.abs(got - ref)
    if dtype == torch.bfloat16:
        allowed = bf16_ulp(ref) + (m + 8) * 2.0 ** -24 * mag
    else:
        allowed = 1e-6 * mag + 1e-30
    assert np.all(err <= allowed), f"{what}: error {err.max()}"


@pytest.mark.parametrize("dtype,m,C,ring", [(torch.bfloat16, 4, 384, True),
                                            (torch.bfloat16, 4, 384, False),
                                            (torch.float32, 128, 256, True),
                                            (torch.bfloat16, 1, 64, False)])
def test_compress_append_matches_oracle(dtype, m, C, ring):
    """Tokens arrive one at a time, each sequence at its own position; every
    completed block becomes the next cache row (oracle append rule), the
    entry counts follow, and nothing else is written."""
    B, n = 3, 3 * m + m // 2 + 2
    _say(f"compress append: {dtype} m={m} C={C} ring={ring}")
    xs = _randn((B, n + 8, C), 1 / math.sqrt(C), dtype, 71)
    zs = _randn((B, n + 8), 1.0, torch.float32, 72)
    N_max = n // m + 2
    cache = torch.full((B, N_max, C), 7.0, dtype=dtype, device=DEV)
    n_ent = torch.zeros((B,), dtype=torch.int32, device=DEV)
    R = m if ring else n + 8
    xb = torch.zeros((B, R, C), dtype=dtype, device=DEV)
    zb = torch.zeros((B, R), dtype=torch.float32, device=DEV)
    lag = [0, 1, m + 1]                        # sequence b is lag[b] tokens behind
    for step in range(n + max(lag)):
        t = torch.tensor([step - lag[b] for b in range(B)], dtype=torch.int32, device=DEV)
        for b in range(B):
            tb = step - lag[b]
            if 0 <= tb < n:
                xb[b, tb % R] = xs[b, tb]
                zb[b, tb % R] = zs[b, tb]
        t = torch.where(t < n, t, torch.full_like(t, -1))
        csa.compress_append(xb, zb, t, m, cache, n_ent)
    torch.cuda.synchronize()
    X, Z, Cc = np64(xs), np64(zs), np64(cache)
    assert n_ent.tolist() == [n // m] * B
    for b in range(B):
        for j in range(n // m):
            _check_rows(Cc[b, j], X[b, m * j: m * j + m], Z[b, m * j: m * j + m], m, dtype,
                        f"b={b} j={j}")
        assert np.all(Cc[b, n // m:] == 7.0), "rows past the completed blocks were written"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_attend_merge_matches_oracle(dtype):
    rows, H, D = 37, 64, 128
    _say(f"attend merge {dtype}")
    oa = _randn((rows, H, D), 1.0, dtype, 81)
    ob = _randn((rows, H, D), 1.0, dtype, 82)
    la = _randn((rows, H), 3.0, torch.float32, 83)
    lb = _randn((rows, H), 3.0, torch.float32, 84)
    la[0, :5] = -math.inf                      # one side empty
    lb[1, 3:9] = -math.inf
    la[2, 7] = lb[2, 7] = -math.inf            # both empty
    lb[3, 10] = la[3, 10] + 80.0               # one side dominates completely
    out, lse = csa.attend_merge(oa, la, ob, lb, with_lse=True)
    inplace = oa.clone()
    csa.attend_merge(inplace, la, ob, lb, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(inplace, out)
    OA, OB, LA, LB, O, L = (np64(t) for t in (oa, ob, la, lb, out, lse))
    for r in range(rows):
        o_ref, l_ref = oracle.merge_attention(OA[r], LA[r], OB[r], LB[r])
        if dtype == torch.bfloat16:
            err = np.abs(O[r] - o_ref)
            assert np.all(err <= bf16_ulp(o_ref) + 1e-6 * np.abs(o_ref) + 1e-30), (r, err.max())
        else:
            np.testing.assert_allclose(O[r], o_ref, rtol=2e-6, atol=1e-6)
        check_lse(L[r], l_ref, 2e-6 * np.abs(l_ref[np.isfinite(l_ref)]).max(initial=1.0))
    assert np.all(O[2, 7] == 0) and np.isneginf(L[2, 7])


def test_window_and_compressed_branches_merge_to_one_softmax():
    """swa_attend over the last tokens of a raw cache and csa_attend over
    selected compressed entries, merged: the attention over the window's
    keys and the selected entries' keys together (oracle: one softmax over
    the concatenated key and value rows)."""
    B, n_raw, N, H, D, W, k = 3, 3000, 800, 64, 128, 200, 300
    bf = torch.bfloat16
    _say("hybrid: window branch + compressed branch")
    q = _randn((B, 1, H, D), 2.0 / math.sqrt(D), bf, 91)
    kr = _randn((B, n_raw, D), 1.0, bf, 92)
    vr = _randn((B, n_raw, D), 1.0, bf, 93)
    kc = _randn((B, N, D), 1.0, bf, 94)
    vc = _randn((B, N, D), 1.0, bf, 95)
    g = torch.Generator(device=DEV).manual_seed(96)
    idx = torch.stack([torch.randperm(N, generator=g, device=DEV)[:k] for _ in range(B)])
    idx = torch.sort(idx, dim=1).values.to(torch.int32).unsqueeze(1).contiguous()
    pos = torch.tensor([[n_raw - 1], [1500], [W // 2]], dtype=torch.int32, device=DEV)
    n_tok = torch.full((B,), n_raw, dtype=torch.int32, device=DEV)
    n_ent = torch.full((B,), N, dtype=torch.int32, device=DEV)
    ow, lw = csa.swa_attend(q, kr, vr, pos, n_tok, W, with_lse=True)
    oc, lc = csa.attend(q, kc, vc, idx, n_ent, with_lse=True)
    o, lse = csa.attend_merge(ow, lw, oc, lc, with_lse=True)
    torch.cuda.synchronize()
    Q, KR, VR, KC, VC, I, O, L = (np64(t) for t in (q, kr, vr, kc, vc, idx, o, lse))
    P = pos.cpu().numpy()
    for b in range(B):
        p = int(P[b, 0]) + 1
        win = np.arange(max(0, p - W), p)
        sel = I[b, 0]
        Kcat = np.concatenate([KR[b][win], KC[b][sel]])
        Vcat = np.concatenate([VR[b][win], VC[b][sel]])
        o_ref, l_ref = oracle.attend(Q[b, 0], Kcat, Vcat, range(Kcat.shape[0]))
        check_attention(O[b, 0], o_ref, "bf16", f"hybrid b={b}")
        check_lse(L[b, 0], l_ref, LSE_TOL_BF16)


def test_index_topk_invariants():
    """Scaling every head weight by 2 scales every score exactly by 2, so the
    selection is bitwise the same; permuting the cache entries permutes the
    selected indices (rows whose k-th and (k+1)-th scores tie are skipped)."""
    B, N, k, m = 6, 32768, 1024, 4
    bf = torch.bfloat16
    _say("index_topk: w x 2 and entry permutation")
    qi = _randn((B, 1, 64, 128), 1 / math.sqrt(128), bf, 101)
    ki = _randn((B, N, 128), 1 / math.sqrt(128), bf, 102)
    wi = _randn((B, 1, 64), 1 / 8, torch.float32, 103)
    pos = torch.full((B, 1), 4 * N, dtype=torch.int32, device=DEV)
    ne = torch.full((B,), N, dtype=torch.int32, device=DEV)
    idx = csa.index_topk(qi, wi, ki, pos, ne, m, k)
    idx2 = csa.index_topk(qi, wi * 2.0, ki, pos, ne, m, k)
    s1 = csa.index_score(qi, wi, ki, pos, ne, m)
    s2 = csa.index_score(qi, wi * 2.0, ki, pos, ne, m)
    g = torch.Generator(device=DEV).manual_seed(104)
    perm = torch.randperm(N, generator=g, device=DEV)
    idxp = csa.index_topk(qi, wi, ki[:, perm].contiguous(), pos, ne, m, k)
    torch.cuda.synchronize()
    assert torch.equal(s2, s1 * 2.0), "scores did not scale exactly"
    assert torch.equal(idx, idx2), "w x 2 changed the selection"
    S, I, IP, PERM = np64(s1), np64(idx), np64(idxp), perm.cpu().numpy()
    checked = 0
    for b in range(B):
        srt = np.sort(S[b, 0])[::-1]
        if srt[k - 1] == srt[k]:
            continue
        assert np.array_equal(np.sort(PERM[IP[b, 0]]), I[b, 0]), f"permutation b={b}"
        checked += 1
    assert checked >= B - 1


@pytest.mark.parametrize("dtype,B,n,C,d_mx,m", [(torch.bfloat16, 2, 4096, 384, 128, 4),
                                                (torch.bfloat16, 1, 4 * 77 + 3, 384, 128, 4),
                                                (torch.float32, 2, 1024, 160, 32, 4),
                                                (torch.bfloat16, 2, 1024 * 128, 256, 256, 128)])
def test_compress_mx4_is_compress_then_mx_encoding(dtype, B, n, C, d_mx, m):
    """The fused encoder's codes and scale bytes equal the oracle's MX
    encoding of csa_compress's fp32 pooled values (fp32 compression of the
    same inputs: the same arithmetic), byte for byte; the leading channels
    equal csa_compress's bitwise."""
    _say(f"compress mx4: {dtype} B={B} n={n} C={C} d_mx={d_mx} m={m}")
    x = _randn((B, n, C), 1 / math.sqrt(128), dtype, 111)
    x[0, : 4 * m, C - d_mx: C - d_mx + 32] = 0.0          # all-zero blocks
    x[0, 4 * m: 8 * m, C - 32:] *= 1e-20                   # tiny blocks (small exponents)
    z = _randn((B, n), 1.0, torch.float32, 112)
    out, codes, scales = csa.compress_mx4(x, z, m, d_mx)
    ref_dt = csa.compress(x, z, m)
    ref32 = csa.compress(x.float(), z, m)
    torch.cuda.synchronize()
    if out is not None:
        assert torch.equal(out, ref_dt[..., : C - d_mx]), "leading channels differ"
    c_ref, s_ref = oracle.mx4_quantize(np64(ref32[..., C - d_mx:]))
    assert np.array_equal(codes.cpu().numpy(), c_ref), "codes differ"
    assert np.array_equal(scales.cpu().numpy(), s_ref), "scale bytes differ"
