"""The allocation-free decode step (csa_index_topk_attend_noalloc) against the
workspace entry point (csa_index_topk_attend) through the C ABI: identical
indices, outputs and lse on consecutive calls of different shapes, the
scratch left ready for the next call, the oracle on sampled rows, and the
size limit rejected on the host."""
import math
import sys

import numpy as np
import pytest
import torch

import long_context_attention_24_amd as csa
import oracle
from parity import LSE_TOL_BF16, check_attention, check_lse, check_topk, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _randn(shape, std, dtype, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.empty(shape, device=DEV, dtype=torch.float32).normal_(0, 1, generator=g)
    return (x * std).to(dtype)


def _case(B, N, seed, mx4=False):
    bf = torch.bfloat16
    c = dict(q=_randn((B, 1, 64, 128), 3 / math.sqrt(128), bf, seed),
             kc=_randn((B, N, 128), 1 / math.sqrt(128), bf, seed + 1),
             vc=_randn((B, N, 128), 1 / math.sqrt(128), bf, seed + 2),
             wi=_randn((B, 1, 64), 1 / 8, torch.float32, seed + 5))
    if mx4:
        g = torch.Generator(device=DEV).manual_seed(seed + 3)
        c["qi"] = torch.randint(0, 256, (B, 1, 64, 64), generator=g, device=DEV, dtype=torch.uint8)
        c["ki"] = torch.randint(0, 256, (B, N, 64), generator=g, device=DEV, dtype=torch.uint8)
        c["qs"] = torch.randint(122, 130, (B, 1, 64, 4), generator=g, device=DEV, dtype=torch.uint8)
        c["ks"] = torch.randint(122, 130, (B, N, 4), generator=g, device=DEV, dtype=torch.uint8)
    else:
        c["qi"] = _randn((B, 1, 64, 128), 1 / math.sqrt(128), bf, seed + 3)
        c["ki"] = _randn((B, N, 128), 1 / math.sqrt(128), bf, seed + 4)
        c["qs"] = c["ks"] = None
    c["pos"] = torch.full((B, 1), 4 * N + 3, dtype=torch.int32, device=DEV)
    c["ne"] = torch.tensor([N - 37 * b for b in range(B)], dtype=torch.int32, device=DEV)
    return c


def _run(c, k, noalloc):
    B = c["q"].shape[0]
    lse = torch.empty((B, 1, 64), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    if noalloc:
        o = csa.index_topk_attend_noalloc(c["qi"], c["wi"], c["ki"], c["q"], c["kc"], c["vc"],
                                          c["pos"], c["ne"], 4, k, q_scale=c["qs"],
                                          k_scale=c["ks"], lse=lse, idx_out=idx)
    else:
        o, lse, idx = csa.index_topk_attend(c["qi"], c["wi"], c["ki"], c["q"], c["kc"], c["vc"],
                                            c["pos"], c["ne"], 4, k, q_scale=c["qs"],
                                            k_scale=c["ks"], with_lse=True, with_idx=True)
    torch.cuda.synchronize()
    return o, lse, idx


def _same(a, b, what):
    (o1, l1, i1), (o2, l2, i2) = a, b
    assert torch.equal(i1, i2), f"{what}: top-k lists differ"
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"{what}: outputs differ"
    assert torch.equal(l1, l2), f"{what}: lse differs"


def _oracle_rows(c, res, k, rows):
    o, lse, idx = res
    I, Q, K, Vv, O, L = (np64(t) for t in (idx, c["q"], c["kc"], c["vc"], o, lse))
    QI, KI, W = np64(c["qi"]), np64(c["ki"]), np64(c["wi"])
    ne = c["ne"].cpu().numpy()
    for b in rows:
        V = int(ne[b])
        check_topk(I[b, 0], oracle.index_scores(QI[b, 0], W[b, 0], KI[b], V), V, k)
        o_ref, l_ref = oracle.attend(Q[b, 0], K[b], Vv[b], I[b, 0])
        check_attention(O[b, 0], o_ref, "bf16", f"noalloc b={b}")
        check_lse(L[b, 0], l_ref, LSE_TOL_BF16)


def test_noalloc_step_matches_workspace_step():
    assert csa.load_library().csa_index_topk_attend_noalloc_max_bytes() == 32 << 20
    _say("noalloc: call 1, B=8 N=32768 k=1024 (streamed rows, 8 splits)")
    big = _case(8, 32768, 500)
    r1 = _run(big, 1024, noalloc=True)
    _same(r1, _run(big, 1024, noalloc=False), "call 1")
    _oracle_rows(big, r1, 1024, [0, 7])
    _say("noalloc: call 2, B=3 N=5000 k=300 (smaller, ragged)")
    small = _case(3, 5000, 600)
    r2 = _run(small, 300, noalloc=True)
    _same(r2, _run(small, 300, noalloc=False), "call 2")
    _oracle_rows(small, r2, 300, [0, 1, 2])
    _say("noalloc: call 1 again (the scratch left ready: same bits)")
    _same(_run(big, 1024, noalloc=True), r1, "call 1 repeated")


def test_noalloc_long_rows_and_limits():
    _say("noalloc: MX FP4 indexer, B=2 N=262144 (filtered long rows)")
    c = _case(2, 262144, 700, mx4=True)
    _same(_run(c, 1024, noalloc=True), _run(c, 1024, noalloc=False), "long rows")
    _say("noalloc: more query rows than the scratch serves -> unsupported")
    q = torch.zeros((4097, 1, 64, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((4097, 8, 128), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((4097, 1, 64), dtype=torch.float32, device=DEV)
    pos = torch.zeros((4097, 1), dtype=torch.int32, device=DEV)
    ne = torch.zeros((4097,), dtype=torch.int32, device=DEV)
    with pytest.raises(csa.CsaError) as e:
        csa.index_topk_attend_noalloc(q, w, kv, q, kv, kv, pos, ne, 4, 4)
    assert e.value.status == 2 and "4097" in e.value.message


def test_noalloc_many_query_rows():
    """Many query rows per sequence (the prefill score kernel: 8 queries and
    4096 keys per workgroup, blocks loaded straight into LDS) through the
    allocation-free step, against the workspace step; two calls in a row,
    the second smaller."""
    bf = torch.bfloat16
    for B, Tq, N, k, seed in ((2, 37, 9000, 512, 800), (1, 12, 3000, 256, 900)):
        _say(f"noalloc: B={B} Tq={Tq} N={N} k={k} (prefill score kernel)")
        c = dict(q=_randn((B, Tq, 64, 128), 3 / math.sqrt(128), bf, seed),
                 kc=_randn((B, N, 128), 1 / math.sqrt(128), bf, seed + 1),
                 vc=_randn((B, N, 128), 1 / math.sqrt(128), bf, seed + 2),
                 qi=_randn((B, Tq, 64, 128), 1 / math.sqrt(128), bf, seed + 3),
                 ki=_randn((B, N, 128), 1 / math.sqrt(128), bf, seed + 4),
                 wi=_randn((B, Tq, 64), 1 / 8, torch.float32, seed + 5), qs=None, ks=None)
        # causal positions across the cache, some seeing fewer than k entries
        pos = [[4 * (N - 61 * t) + (t % 4) for t in range(Tq)] for _ in range(B)]
        pos[0][-1] = 4 * (k // 2)
        c["pos"] = torch.tensor(pos, dtype=torch.int32, device=DEV)
        c["ne"] = torch.tensor([N - 101 * b for b in range(B)], dtype=torch.int32, device=DEV)
        lse = torch.empty((B, Tq, 64), dtype=torch.float32, device=DEV)
        idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
        o = csa.index_topk_attend_noalloc(c["qi"], c["wi"], c["ki"], c["q"], c["kc"], c["vc"],
                                          c["pos"], c["ne"], 4, k, lse=lse, idx_out=idx)
        o2, lse2, idx2 = csa.index_topk_attend(c["qi"], c["wi"], c["ki"], c["q"], c["kc"],
                                               c["vc"], c["pos"], c["ne"], 4, k, with_lse=True,
                                               with_idx=True)
        torch.cuda.synchronize()
        _same((o, lse, idx), (o2, lse2, idx2), f"Tq={Tq}")
        I, Q, K, Vv, O = (np64(t) for t in (idx, c["q"], c["kc"], c["vc"], o))
        QI, KI, W = np64(c["qi"]), np64(c["ki"]), np64(c["wi"])
        ne = c["ne"].cpu().numpy()
        for b, t in ((0, 0), (0, Tq - 1), (B - 1, Tq // 2)):
            Vis = oracle.visible_count(pos[b][t], 4, int(ne[b]))
            check_topk(I[b, t], oracle.index_scores(QI[b, t], W[b, t], KI[b], Vis), Vis, k)
            o_ref, _ = oracle.attend(Q[b, t], K[b], Vv[b], I[b, t])
            check_attention(O[b, t], o_ref, "bf16", f"noalloc b={b} t={t}")
