"""Pins for the oracle's top-k selection and attention."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle


# ---------------------------------------------------------------- top-k
def _brute_topk(s, V, k):
    """Max-sum k-subset of the visible entries, lexicographically smallest
    index set among ties.  Scores are integers so every sum is exact."""
    kk = min(k, V)
    best_sum, best = None, None
    for sub in itertools.combinations(range(V), kk):
        tot = sum(int(s[j]) for j in sub)
        if best_sum is None or tot > best_sum or (tot == best_sum and sub < best):
            best_sum, best = tot, sub
    out = np.full(k, -1, dtype=np.int64)
    out[:kk] = best
    return out


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(5)
    for trial in range(200):
        V = int(rng.integers(0, 11))
        N = V + int(rng.integers(0, 3))
        k = int(rng.integers(1, 8))
        s = rng.integers(-3, 4, size=N).astype(np.float64)   # many ties
        s[V:] = -np.inf
        got = oracle.topk_select(s, V, k)
        assert np.array_equal(got, _brute_topk(s, V, k)), (trial, s, V, k)


def test_topk_rules():
    # k >= visible: everything visible, ascending, padded
    s = np.array([0.3, -1.0, 2.0, 5.0, -np.inf])
    assert list(oracle.topk_select(s, 4, 6)) == [0, 1, 2, 3, -1, -1]
    # -0.0 and +0.0 tie: lower index wins
    s = np.array([1.0, -0.0, 0.0, 0.0, -2.0])
    assert list(oracle.topk_select(s, 5, 2)) == [0, 1]
    s = np.array([1.0, 0.0, -0.0, -2.0])
    assert list(oracle.topk_select(s, 4, 2)) == [0, 1]
    # output is ascending by index, not by score
    s = np.array([1.0, 9.0, 3.0, 7.0])
    assert list(oracle.topk_select(s, 4, 2)) == [1, 3]
    # nothing visible
    assert list(oracle.topk_select(s, 0, 3)) == [-1, -1, -1]


def test_topk_permutation_and_needles():
    rng = np.random.default_rng(6)
    N, k = 500, 40
    s = rng.standard_normal(N)
    base = set(oracle.topk_select(s, N, k).tolist())
    perm = rng.permutation(N)
    # entry perm[i] of the permuted row is entry i of the original... map back
    s_perm = s[perm]
    got = {int(perm[j]) for j in oracle.topk_select(s_perm, N, k)}
    assert got == base
    # planted needles are always selected
    s2 = s.copy()
    needles = [3, 77, 499]
    s2[needles] = 100.0
    assert set(needles) <= set(oracle.topk_select(s2, N, k).tolist())


# ---------------------------------------------------------------- attention
def _sdpa_causal(q, k, v, scale):
    """torch's scaled_dot_product_attention on CPU in float64 (library routine)."""
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]       # [1, H, T, D]
    tk = torch.from_numpy(k)[None, None].expand(1, q.shape[1], -1, -1)
    tv = torch.from_numpy(v)[None, None].expand(1, q.shape[1], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    return o[0].permute(1, 0, 2).numpy()                    # [T, H, D]


def test_m1_full_k_is_causal_attention():
    """m = 1 and k >= n: CSA reduces to standard causal attention."""
    rng = np.random.default_rng(7)
    T, H, D, HI, DI = 12, 3, 8, 2, 4
    q = rng.standard_normal((T, H, D))
    kr = rng.standard_normal((T, D))
    vr = rng.standard_normal((T, D))
    z = rng.standard_normal(T)
    kc = oracle.pool(kr, z, 1)
    vc = oracle.pool(vr, z, 1)
    ki = rng.standard_normal((T, DI))
    want = _sdpa_causal(q, kr, vr, 1 / math.sqrt(D))
    for t in range(T):
        r = oracle.csa_reference(q=q[t], q_idx=rng.standard_normal((HI, DI)),
                                 w_idx=rng.standard_normal(HI), k_cache=kc, v_cache=vc,
                                 k_idx=ki, q_pos=t, m=1, k=T, n_entries=T)
        assert r["visible"] == t + 1
        assert np.allclose(r["o"], want[t], atol=1e-12)


def test_hca_m1_is_causal_attention():
    rng = np.random.default_rng(8)
    T, H, D = 10, 2, 6
    q = rng.standard_normal((T, H, D))
    kr = rng.standard_normal((T, D))
    vr = rng.standard_normal((T, D))
    want = _sdpa_causal(q, kr, vr, 0.37)
    kc = oracle.pool(kr, rng.standard_normal(T), 1)
    vc = oracle.pool(vr, rng.standard_normal(T), 1)
    for t in range(T):
        o, _ = oracle.hca_attend(q[t], kc, vc, oracle.visible_count(t, 1, T), 0.37)
        assert np.allclose(o, want[t], atol=1e-12)


def test_swa_is_banded_causal_attention():
    """Sliding-window attention equals torch's scaled_dot_product_attention with
    a banded causal mask (a library routine, fp64 CPU); window >= p + 1 is full
    causal attention; window = 1 returns the token's own value row."""
    rng = np.random.default_rng(10)
    T, H, D, W = 14, 3, 8, 4
    q = rng.standard_normal((T, H, D))
    kr = rng.standard_normal((T, D))
    vr = rng.standard_normal((T, D))
    i = torch.arange(T)
    band = (i[None, :] <= i[:, None]) & (i[None, :] > i[:, None] - W)     # [T_q, T_k]
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(kr)[None, None].expand(1, H, -1, -1)
    tv = torch.from_numpy(vr)[None, None].expand(1, H, -1, -1)
    want = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=band, scale=0.4)[0].permute(1, 0, 2).numpy()
    full = _sdpa_causal(q, kr, vr, 0.4)
    for t in range(T):
        o, _ = oracle.swa_attend(q[t], kr, vr, t, T, W, 0.4)
        assert np.allclose(o, want[t], atol=1e-12)
        o, _ = oracle.swa_attend(q[t], kr, vr, t, T, T, 0.4)
        assert np.allclose(o, full[t], atol=1e-12)
        o, lse = oracle.swa_attend(q[t], kr, vr, t, T, 1, 0.4)
        assert np.array_equal(o, np.tile(vr[t], (H, 1)))
        assert np.allclose(lse, 0.4 * q[t] @ kr[t], atol=1e-13)
    # fewer tokens cached than the position implies: the window ends at the cache end
    o, _ = oracle.swa_attend(q[5], kr, vr, 9, 6, 3, 0.4)
    o2, _ = oracle.attend(q[5], kr, vr, [3, 4, 5], 0.4)
    assert np.array_equal(o, o2)


def test_attend_closed_forms():
    rng = np.random.default_rng(9)
    H, D, N = 4, 8, 16
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((N, D))
    Vc = rng.standard_normal((N, D))
    # one selected entry: output is that value row, lse is its logit
    o, lse = oracle.attend(q, K, Vc, [5, -1, -1], 0.5)
    assert np.allclose(o, np.tile(Vc[5], (H, 1)), atol=1e-14)
    assert np.allclose(lse, 0.5 * q @ K[5], atol=1e-14)
    # empty selection
    o, lse = oracle.attend(q, K, Vc, [-1, -1])
    assert np.all(o == 0) and np.all(lse == -np.inf)
    # lse equals scipy's logsumexp of the logits; output is a convex combination
    from scipy.special import logsumexp, softmax
    sel = [1, 2, 9, 15]
    o, lse = oracle.attend(q, K, Vc, sel, 0.3)
    logits = 0.3 * q @ K[sel].T
    assert np.allclose(lse, logsumexp(logits, axis=1), atol=1e-12)
    assert np.allclose(o, softmax(logits, axis=1) @ Vc[sel], atol=1e-12)
    # the order and duplicates of indices: order does not matter
    o2, _ = oracle.attend(q, K, Vc, sel[::-1], 0.3)
    assert np.allclose(o, o2, atol=1e-14)


def test_csa_with_large_k_equals_hca():
    """k >= visible entries: CSA is dense attention over the visible compressed entries."""
    rng = np.random.default_rng(10)
    N, H, D, HI, DI, m = 30, 4, 8, 3, 6, 4
    kc = rng.standard_normal((N, D))
    vc = rng.standard_normal((N, D))
    ki = rng.standard_normal((N, DI))
    for t in [0, 3, 17, 64, 200]:
        q = rng.standard_normal((H, D))
        r = oracle.csa_reference(q=q, q_idx=rng.standard_normal((HI, DI)),
                                 w_idx=rng.standard_normal(HI), k_cache=kc, v_cache=vc,
                                 k_idx=ki, q_pos=t, m=m, k=64, n_entries=N)
        o, lse = oracle.hca_attend(q, kc, vc, oracle.visible_count(t, m, N))
        assert np.allclose(r["o"], o, atol=1e-13)
        assert np.allclose(r["lse"], lse, atol=1e-13) or r["visible"] == 0


def test_selected_entries_dominate_sharp_attention():
    """Needle: an entry aligned with every query head is selected and dominates the output."""
    rng = np.random.default_rng(11)
    N, H, D, HI, DI = 64, 2, 16, 4, 16
    kc = rng.standard_normal((N, D)) * 0.1
    vc = rng.standard_normal((N, D))
    ki = rng.standard_normal((N, DI)) * 0.1
    qi = rng.standard_normal((HI, DI))
    needle = 41
    ki[needle] = 10 * qi.sum(axis=0)
    q = np.tile(kc[needle] * 0 + 1.0, (H, 1))
    kc[needle] = 50.0
    r = oracle.csa_reference(q=q, q_idx=qi, w_idx=np.ones(HI), k_cache=kc, v_cache=vc,
                             k_idx=ki, q_pos=4 * N, m=4, k=4, n_entries=N)
    assert needle in r["idx"]
    assert np.allclose(r["o"], np.tile(vc[needle], (H, 1)), atol=1e-6)


# ---------------------------------------------------------------- combining two branches (R10)
def test_merge_of_disjoint_sets_is_attention_over_the_union():
    """merge(attend(S1), attend(S2)) = attend(S1 u S2) for disjoint S1, S2,
    the union computed in one softmax; either order; an empty side returns
    the other side; both empty gives 0 / -inf."""
    rng = np.random.default_rng(21)
    H, D, N = 6, 16, 300
    for trial in range(20):
        q = rng.standard_normal((H, D)) * 2.0
        K = rng.standard_normal((N, D))
        V = rng.standard_normal((N, D))
        perm = rng.permutation(N)
        cut = int(rng.integers(1, N))
        S1, S2 = perm[:cut], perm[cut:]
        o1, l1 = oracle.attend(q, K, V, S1)
        o2, l2 = oracle.attend(q, K, V, S2)
        o, lse = oracle.merge_attention(o1, l1, o2, l2)
        o_ref, l_ref = oracle.attend(q, K, V, np.concatenate([S1, S2]))
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12)
        ob, lb = oracle.merge_attention(o2, l2, o1, l1)
        np.testing.assert_allclose(ob, o_ref, rtol=0, atol=1e-12)
    oe, le = oracle.attend(q, K, V, [])
    o, lse = oracle.merge_attention(o1, l1, oe, le)
    assert np.array_equal(o, o1) and np.array_equal(lse, l1)
    o, lse = oracle.merge_attention(oe, le, oe, le)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # a window branch and a compressed branch over different key tensors:
    # the merge equals one softmax over the concatenated keys
    Kw, Vw = rng.standard_normal((40, D)), rng.standard_normal((40, D))
    ow, lw = oracle.attend(q, Kw, Vw, range(40))
    oc, lc = oracle.attend(q, K, V, S1)
    o, lse = oracle.merge_attention(ow, lw, oc, lc)
    Kcat, Vcat = np.concatenate([Kw, K[S1]]), np.concatenate([Vw, V[S1]])
    o_ref, l_ref = oracle.attend(q, Kcat, Vcat, range(Kcat.shape[0]))
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-12)
