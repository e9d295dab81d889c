"""Pins for the oracle's compression (pooling), visibility and indexer score."""
import math

import numpy as np
import pytest

import oracle
from csa_synth import WORKLOADS


def _parse_rows(txt):
    return np.array([[float(v) for v in r.split(",")] for r in txt.split(";")])


def test_pool_worked_examples(golden):
    for row in golden("pool_worked.txt"):
        _, m, logits, rows, want = (p.strip() for p in row.split("|"))
        z = np.array([float(v) for v in logits.split()])
        x = _parse_rows(rows)
        got = oracle.pool(x, z, int(m))
        assert np.allclose(got, _parse_rows(want), rtol=0, atol=1e-12)


def test_pool_closed_forms():
    rng = np.random.default_rng(1)
    n, C, m = 32, 5, 4
    x = rng.standard_normal((n, C))
    z = rng.standard_normal(n)
    out = oracle.pool(x, z, m)
    assert out.shape == (n // m, C)
    # constant rows -> the constant
    xc = np.tile(np.arange(C, dtype=np.float64), (n, 1))
    assert np.allclose(oracle.pool(xc, z, m), xc[: n // m], atol=1e-14)
    # m = 1 is the identity
    assert np.array_equal(oracle.pool(x, z, 1), x)
    # adding a constant to the logits of one block changes nothing
    z2 = z.copy()
    z2[8:12] += 3.7
    assert np.allclose(oracle.pool(x, z2, m), out, atol=1e-14)
    # one dominant logit selects that token
    z3 = np.zeros(n)
    z3[5] = 800.0
    assert np.allclose(oracle.pool(x, z3, m)[1], x[5], atol=1e-14)
    # an incomplete tail block is dropped
    assert oracle.pool(x[:30], z[:30], m).shape == (7, C)


def test_pool_against_scalar_loop():
    rng = np.random.default_rng(2)
    n, C, m = 24, 3, 8
    x = rng.standard_normal((n, C))
    z = rng.standard_normal(n) * 3
    got = oracle.pool(x, z, m)
    for j in range(n // m):
        ws = [math.exp(z[m * j + i]) for i in range(m)]
        tot = sum(ws)
        for c in range(C):
            want = sum(ws[i] / tot * x[m * j + i, c] for i in range(m))
            assert abs(got[j, c] - want) < 1e-12


def test_visibility_tiny(golden):
    w = WORKLOADS["tiny_csa"]
    for row in golden("visibility_tiny.txt"):
        t, want = (int(v) for v in row.split())
        assert oracle.visible_count(t, 4, 64) == want
        assert w.visible(t) == want


def test_visibility_workloads():
    # decode at 128K: 131072 tokens of context -> 32768 entries all visible
    w = WORKLOADS["csa_decode_128k"]
    assert oracle.visible_count(w.q_pos0, w.m, w.N) == 32768
    w = WORKLOADS["hca_decode_1m"]
    assert oracle.visible_count(w.q_pos0, w.m, w.N) == 8192
    w = WORKLOADS["csa_prefill_chunk"]
    assert oracle.visible_count(w.q_pos0, w.m, w.N) == 65536
    assert oracle.visible_count(w.q_pos0 + 3, w.m, w.N) == 65537
    assert oracle.visible_count(w.q_pos0 + 4095, w.m, w.N) == 66560


def test_params_match_pages(golden):
    p = dict(r.split() for r in golden("v4pro_params.txt"))
    w = WORKLOADS["csa_decode_128k"]
    assert (w.m, w.H_I, w.D_I, w.k) == (int(p["csa_m"]), int(p["indexer_heads"]),
                                       int(p["indexer_head_dim"]), int(p["top_k"]))
    assert WORKLOADS["hca_decode_1m"].m == int(p["hca_m"])


def test_index_scores_brute_force():
    rng = np.random.default_rng(3)
    H, D, N, V = 3, 5, 9, 7
    q = rng.standard_normal((H, D))
    w = rng.standard_normal(H)
    K = rng.standard_normal((N, D))
    s = oracle.index_scores(q, w, K, V)
    for j in range(N):
        if j >= V:
            assert s[j] == -np.inf
            continue
        want = 0.0
        for h in range(H):
            dot = sum(q[h, d] * K[j, d] for d in range(D))
            want += w[h] * (dot if dot > 0 else 0.0)
        assert abs(s[j] - want) < 1e-12


def test_index_scores_special_cases():
    rng = np.random.default_rng(4)
    D, N = 8, 20
    q = np.abs(rng.standard_normal((1, D)))
    K = np.abs(rng.standard_normal((N, D)))     # all dots positive: ReLU is inactive
    s = oracle.index_scores(q, np.array([1.0]), K, N)
    assert np.allclose(s, K @ q[0], atol=1e-13)
    # all dots negative -> exactly zero
    s = oracle.index_scores(-q, np.array([2.5]), K, N)
    assert np.all(s == 0.0)
    # scaling the head weights by 2 scales every score by exactly 2
    q = rng.standard_normal((4, D))
    w = rng.standard_normal(4)
    K = rng.standard_normal((N, D))
    assert np.array_equal(oracle.index_scores(q, 2 * w, K, N), 2 * oracle.index_scores(q, w, K, N))
    # nothing visible
    assert np.all(oracle.index_scores(q, w, K, 0) == -np.inf)


@pytest.mark.parametrize("H", [1, 4])
def test_index_scores_relu_is_per_head(H):
    # two heads whose dots cancel: without a per-head ReLU the score would be 0
    q = np.array([[1.0, 0.0], [-1.0, 0.0]])
    K = np.array([[2.0, 0.0]])
    s = oracle.index_scores(q, np.array([1.0, 1.0]), K, 1)
    assert s[0] == 2.0


def test_append_block_completes_exactly_the_blocks_of_the_whole_pool():
    """R11: appending tokens one at a time completes entry j exactly when
    token m j + m - 1 arrives, and the pooled rows equal pooling the whole
    sequence at once (every entry, every m)."""
    rng = np.random.default_rng(31)
    for m in (1, 4, 7, 128):
        n, C = 3 * m + m // 2 + 1, 5
        x = rng.standard_normal((n, C))
        z = rng.standard_normal(n)
        whole = oracle.pool(x, z, m)
        got = []
        for t in range(n):
            lo = max(0, t - m + 1)
            r = oracle.append_block(x[lo:t + 1], z[lo:t + 1], t, m) if t + 1 >= m else None
            if (t + 1) % m == 0:
                assert r is not None and r[0] == (t + 1) // m - 1
                got.append(r[1])
            else:
                assert r is None
        assert len(got) == n // m
        np.testing.assert_allclose(np.array(got), whole, rtol=0, atol=0)
