"""GPU parity on small inputs: the tiny fp32 workload stage by stage, the
generic (VALU) kernels, ragged shapes and the method's degenerate cases.

Every case is checked against the oracle on the exact input bits the GPU
consumed (stage-wise: each stage's oracle uses the GPU's previous output)."""
import math
import sys

import numpy as np
import pytest
import torch

import long_context_attention_24_amd as csa
import oracle
from csa_synth import WORKLOADS, make_inputs
from parity import (LSE_TOL_BF16, check_attention, check_compress, check_lse, check_topk, np64,
                    score_bound)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gen(seed):
    return torch.Generator(device=DEV).manual_seed(seed)


def _randn(shape, std, dtype, seed):
    x = torch.empty(shape, device=DEV, dtype=torch.float32).normal_(0, 1, generator=_gen(seed))
    return (x * std).to(dtype)


def test_tiny_csa_stagewise():
    w = WORKLOADS["tiny_csa"]
    _say("tiny_csa: compress")
    inp = make_inputs(w, device=DEV)
    raw, z = inp["raw"], inp["logits"]
    cache = csa.compress(raw, z, w.m)                    # [1, 64, 160] = K | V | K_I
    torch.cuda.synchronize()
    frac = check_compress(np64(cache)[0], np64(raw)[0], np64(z)[0], w.m, "f32")
    kc, vc, ki = cache[..., :64], cache[..., 64:128], cache[..., 128:]
    q, qi, wi = inp["q"], inp["q_idx"], inp["w_idx"]
    q_pos, n_ent = inp["q_pos"], inp["n_entries"]

    _say("tiny_csa: index scores / top-k")
    scores = csa.index_score(qi, wi, ki, q_pos, n_ent, w.m)
    idx, sel_scores = csa.index_topk(qi, wi, ki, q_pos, n_ent, w.m, w.k, with_scores=True)
    idx2 = csa.topk(scores, q_pos, n_ent, w.m, w.k)
    torch.cuda.synchronize()
    S = np64(scores)[0]
    I = np64(idx)[0]
    ki64, qi64, wi64 = np64(ki)[0], np64(qi)[0], np64(wi)[0]
    assert np.array_equal(I, np64(idx2)[0])
    n_amb = 0
    for t in range(w.Tq):
        V = oracle.visible_count(t, w.m, w.N)
        s_ref = oracle.index_scores(qi64[t], wi64[t], ki64, V)
        assert np.all(np.isneginf(S[t, V:]))
        bound = score_bound(qi64[t], wi64[t], ki64[:V], w.D_I, w.H_I)
        assert np.all(np.abs(S[t, :V] - s_ref[:V]) <= bound + 1e-30)
        # selection of the GPU's own fp32 scores is exact
        assert np.array_equal(I[t], oracle.topk_select(S[t], V, w.k))
        n_amb += check_topk(I[t], s_ref, V, w.k)
        sel = I[t][I[t] >= 0]
        assert np.array_equal(np64(sel_scores)[0, t, : sel.size], S[t, sel])
    _say(f"tiny_csa: ambiguous top-k entries {n_amb}")

    _say("tiny_csa: attention")
    o, lse = csa.attend(q, kc, vc, idx, n_ent, with_lse=True)
    oh, lseh = csa.hca_attend(q, kc, vc, q_pos, n_ent, w.m, with_lse=True)
    torch.cuda.synchronize()
    kc64, vc64, q64 = np64(kc)[0], np64(vc)[0], np64(q)[0]
    o_ref = np.zeros_like(q64)
    l_ref = np.zeros(q64.shape[:2])
    oh_ref = np.zeros_like(q64)
    lh_ref = np.zeros(q64.shape[:2])
    for t in range(w.Tq):
        o_ref[t], l_ref[t] = oracle.attend(q64[t], kc64, vc64, I[t])
        oh_ref[t], lh_ref[t] = oracle.hca_attend(q64[t], kc64, vc64, oracle.visible_count(t, w.m, w.N))
    check_attention(np64(o)[0], o_ref, "f32", "csa")
    check_lse(np64(lse)[0], l_ref, 1e-5)
    check_attention(np64(oh)[0], oh_ref, "f32", "hca")
    check_lse(np64(lseh)[0], lh_ref, 1e-5)
    # positions 0..2 see nothing: zero output, -inf lse, all -1 indices
    assert np.all(I[:3] == -1) and np.all(np64(o)[0, :3] == 0)
    # at t >= 63 every query sees at least k entries
    assert np.all(I[63:] >= 0)
    _say(f"tiny_csa: ok (compress off-by-rounding fraction {frac:.2e})")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("H,D,HI,DI", [(8, 64, 16, 64), (3, 32, 5, 128), (64, 128, 7, 32)])
def test_generic_shapes_ragged(dtype, H, D, HI, DI):
    """Ragged caches: per-sequence valid rows, mixed query positions, odd sizes."""
    B, Tq, N_max, m, k = 3, 5, 517, 4, 37
    tag = "f32" if dtype == torch.float32 else "bf16"
    _say(f"generic {tag} H={H} D={D} HI={HI} DI={DI}")
    seed = 100 + H + D + HI
    q = _randn((B, Tq, H, D), 1 / math.sqrt(D), dtype, seed)
    kc = _randn((B, N_max, D), 1 / math.sqrt(D), dtype, seed + 1)
    vc = _randn((B, N_max, D), 1 / math.sqrt(D), dtype, seed + 2)
    qi = _randn((B, Tq, HI, DI), 1 / math.sqrt(DI), dtype, seed + 3)
    ki = _randn((B, N_max, DI), 1 / math.sqrt(DI), dtype, seed + 4)
    wi = _randn((B, Tq, HI), 0.5, torch.float32, seed + 5)
    q_pos = torch.tensor([[0, 3, 150, 700, 5000], [10, 11, 12, 400, 2067],
                          [2067, 4, 999, 1, 77]], dtype=torch.int32, device=DEV)
    n_ent = torch.tensor([517, 300, 0], dtype=torch.int32, device=DEV)
    scale = 0.3
    idx, sel = csa.index_topk(qi, wi, ki, q_pos, n_ent, m, k, with_scores=True)
    o, lse = csa.attend(q, kc, vc, idx, n_ent, scale=scale, with_lse=True)
    oh, lseh = csa.hca_attend(q, kc, vc, q_pos, n_ent, m, scale=scale, with_lse=True)
    torch.cuda.synchronize()
    I = np64(idx)
    Q, K, Vv, QI, KI, W = (np64(t) for t in (q, kc, vc, qi, ki, wi))
    qp, ne = q_pos.cpu().numpy(), n_ent.cpu().numpy()
    O, L, OH, LH = np64(o), np64(lse), np64(oh), np64(lseh)
    for b in range(B):
        for t in range(Tq):
            V = oracle.visible_count(int(qp[b, t]), m, int(ne[b]))
            s_ref = oracle.index_scores(QI[b, t], W[b, t], KI[b], V)
            check_topk(I[b, t], s_ref, V, k)
            o_ref, l_ref = oracle.attend(Q[b, t], K[b], Vv[b], I[b, t], scale)
            check_attention(O[b, t], o_ref, tag, f"csa b={b} t={t}")
            check_lse(L[b, t], l_ref, 1e-5 if tag == "f32" else 2.5e-3)
            oh_ref, lh_ref = oracle.hca_attend(Q[b, t], K[b], Vv[b], V, scale)
            check_attention(OH[b, t], oh_ref, tag, f"hca b={b} t={t}")
            check_lse(LH[b, t], lh_ref, 1e-5 if tag == "f32" else 2.5e-3)
    # sequence 2 has no valid rows: nothing selected, zero output
    assert np.all(I[2] == -1) and np.all(O[2] == 0) and np.all(np.isneginf(L[2]))


def test_tuned_kernels_ragged():
    """bf16 64 x 128 (the MFMA kernels) on ragged sizes: partial tiles, V < k,
    partially valid caches, an empty sequence."""
    B, Tq, N_max, m, k = 4, 2, 1000 + 3 * 8, 4, 300
    _say("tuned ragged bf16 64x128")
    q = _randn((B, Tq, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 7)
    kc = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 8)
    vc = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 9)
    qi = _randn((B, Tq, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 10)
    ki = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 11)
    wi = _randn((B, Tq, 64), 1 / 8, torch.float32, 12)
    q_pos = torch.tensor([[5000, 2], [803, 1200], [4095, 100000], [9, 3]], dtype=torch.int32,
                         device=DEV)
    n_ent = torch.tensor([N_max, 777, 1001, 0], dtype=torch.int32, device=DEV)
    scores = csa.index_score(qi, wi, ki, q_pos, n_ent, m)
    idx = csa.index_topk(qi, wi, ki, q_pos, n_ent, m, k)
    o, lse = csa.attend(q, kc, vc, idx, n_ent, with_lse=True)
    oh, lseh = csa.hca_attend(q, kc, vc, q_pos, n_ent, m, with_lse=True)
    torch.cuda.synchronize()
    S, I = np64(scores), np64(idx)
    Q, K, Vv, QI, KI, W = (np64(t) for t in (q, kc, vc, qi, ki, wi))
    qp, ne = q_pos.cpu().numpy(), n_ent.cpu().numpy()
    O, L, OH, LH = np64(o), np64(lse), np64(oh), np64(lseh)
    for b in range(B):
        for t in range(Tq):
            V = oracle.visible_count(int(qp[b, t]), m, int(ne[b]))
            s_ref = oracle.index_scores(QI[b, t], W[b, t], KI[b], V)
            assert np.all(np.isneginf(S[b, t, V:]))
            if V:
                bound = score_bound(QI[b, t], W[b, t], KI[b, :V], 128, 64)
                assert np.all(np.abs(S[b, t, :V] - s_ref[:V]) <= bound)
            check_topk(I[b, t], s_ref, V, k)
            o_ref, l_ref = oracle.attend(Q[b, t], K[b], Vv[b], I[b, t])
            check_attention(O[b, t], o_ref, "bf16", f"csa b={b} t={t}")
            check_lse(L[b, t], l_ref, 2.5e-3)
            oh_ref, lh_ref = oracle.hca_attend(Q[b, t], K[b], Vv[b], V)
            check_attention(OH[b, t], oh_ref, "bf16", f"hca b={b} t={t}")
            check_lse(LH[b, t], lh_ref, 2.5e-3)


@pytest.mark.parametrize("N_max", [1037, 2600, 4999])
def test_decode_scores_odd_chunk_counts(N_max):
    """The decode score kernel gives each wave two strided 256-key chunks; with
    an odd chunk count the last wave has one.  Scores against the oracle, -inf
    past the visible count (which ends inside either chunk of a wave), and the
    selection (through the chunk reports) against the oracle's top-k."""
    B, Tq, m, k = 3, 2, 4, 200
    _say(f"decode scores, odd chunk counts: N_max={N_max}")
    qi = _randn((B, Tq, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 121)
    ki = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 122)
    wi = _randn((B, Tq, 64), 1 / 8, torch.float32, 123)
    pos = [[4 * N_max + 3, 4 * (N_max // 2) + 1], [4 * 300, 4 * (N_max - 40)], [4 * 257, 7]]
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    n_ent = torch.tensor([N_max, N_max - 5, N_max], dtype=torch.int32, device=DEV)
    scores = csa.index_score(qi, wi, ki, q_pos, n_ent, m)
    idx = csa.index_topk(qi, wi, ki, q_pos, n_ent, m, k)
    torch.cuda.synchronize()
    S, I, QI, KI, W = np64(scores), np64(idx), np64(qi), np64(ki), np64(wi)
    ne = n_ent.cpu().numpy()
    for b in range(B):
        for t in range(Tq):
            V = oracle.visible_count(pos[b][t], m, int(ne[b]))
            s_ref = oracle.index_scores(QI[b, t], W[b, t], KI[b], V)
            assert np.all(np.isneginf(S[b, t, V:])), (b, t, V)
            if V:
                bound = score_bound(QI[b, t], W[b, t], KI[b, :V], 128, 64)
                assert np.all(np.abs(S[b, t, :V] - s_ref[:V]) <= bound), (b, t, V)
            check_topk(I[b, t], s_ref, V, k)


def test_hca_multi_split_ragged():
    """HCA on the tuned kernel with visible counts that end exactly on, just
    past and just before split boundaries, several splits per query, a
    sharp softmax in one sequence, one entry and none."""
    B, Tq, N_max, m = 3, 3, 3100, 128
    _say("hca multi-split ragged bf16 64x128")
    q = _randn((B, Tq, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 31)
    q[2] *= 24.0                                           # logit std ~3
    kc = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 32)
    vc = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 33)
    vis = [[1024, 1025, 2048], [2047, 3100, 1], [3073, 31, 0]]
    q_pos = torch.tensor([[m * v + m - 2 for v in row] for row in vis], dtype=torch.int32,
                         device=DEV)
    n_ent = torch.tensor([N_max, N_max, 3090], dtype=torch.int32, device=DEV)
    oh, lseh = csa.hca_attend(q, kc, vc, q_pos, n_ent, m, with_lse=True)
    torch.cuda.synchronize()
    Q, K, Vv, OH, LH = np64(q), np64(kc), np64(vc), np64(oh), np64(lseh)
    qp, ne = q_pos.cpu().numpy(), n_ent.cpu().numpy()
    for b in range(B):
        for t in range(Tq):
            V = oracle.visible_count(int(qp[b, t]), m, int(ne[b]))
            assert V == min(vis[b][t], int(ne[b]))
            oh_ref, lh_ref = oracle.hca_attend(Q[b, t], K[b], Vv[b], V)
            check_attention(OH[b, t], oh_ref, "bf16", f"hca b={b} t={t} V={V}")
            check_lse(LH[b, t], lh_ref, LSE_TOL_BF16 if b == 2 else 2.5e-3)
    assert np.all(OH[2, 2] == 0) and np.all(np.isneginf(LH[2, 2]))
    assert np.array_equal(OH[1, 2], np.tile(Vv[1, 0], (64, 1)))


def test_visible_count_extremes():
    """Query positions at the edges of the visible-count rule, through every
    decode kernel that reads them: q_pos = -1 and far below 0 (nothing
    visible), the largest int32 (visible count capped by n_entries, below
    N_max), and a count inside the second HCA split.  The decode kernels
    issue their first loads before q_pos and n_entries arrive, so these rows
    check that the masks applied afterwards are right.  bf16, MX and FP4
    scores with the selection, CSA attention over the selection, HCA and the
    sliding window, each against the oracle."""
    from csa_synth import mx4_quantize
    from csa_synth.generate import fp4_quantize
    B, N_max, m, k, win = 4, 2500, 4, 300, 700
    _say("visible-count extremes: bf16 / MX / FP4 scores, selection, CSA, HCA, window")
    pos = [-1, -1000, 2 ** 31 - 1, 4 * 1300 + 3]
    ne = [N_max, N_max, N_max - 37, N_max]
    q_pos = torch.tensor([[p] for p in pos], dtype=torch.int32, device=DEV)
    n_ent = torch.tensor(ne, dtype=torch.int32, device=DEV)
    vis = [oracle.visible_count(p, m, n) for p, n in zip(pos, ne)]
    assert vis == [0, 0, N_max - 37, 1301]
    qi = _randn((B, 1, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 131)
    ki = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 132)
    wi = _randn((B, 1, 64), 1 / 8, torch.float32, 133)
    q = _randn((B, 1, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 134)
    kc = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 135)
    vc = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 136)
    scores = csa.index_score(qi, wi, ki, q_pos, n_ent, m)
    idx = csa.index_topk(qi, wi, ki, q_pos, n_ent, m, k)
    o, lse = csa.attend(q, kc, vc, idx, n_ent, with_lse=True)
    oh, lseh = csa.hca_attend(q, kc, vc, q_pos, n_ent, m, with_lse=True)
    ow, lsew = csa.swa_attend(q, kc, vc, q_pos, n_ent, win, with_lse=True)
    qf, kf = qi.float(), ki.float()
    quant = {}
    for name, fn, deq in (("mx4", mx4_quantize, oracle.mx4_dequantize),
                          ("fp4", fp4_quantize, oracle.fp4_dequantize)):
        qc, qs = (t.to(DEV) for t in fn(qf))
        kcq, ksq = (t.to(DEV) for t in fn(kf))
        sq = csa.index_score(qc, wi, kcq, q_pos, n_ent, m, q_scale=qs, k_scale=ksq)
        iq = csa.index_topk(qc, wi, kcq, q_pos, n_ent, m, k, q_scale=qs, k_scale=ksq)
        quant[name] = (sq, iq, deq(qc.cpu().numpy(), qs.cpu().numpy()),
                       deq(kcq.cpu().numpy(), ksq.cpu().numpy()))
    torch.cuda.synchronize()
    W, Q, K, Vv = np64(wi), np64(q), np64(kc), np64(vc)
    runs = [("bf16", np64(scores), np64(idx), np64(qi), np64(ki))]
    runs += [(n, np64(sq), np64(iq), qd, kd) for n, (sq, iq, qd, kd) in quant.items()]
    O, L, OH, LH, OW, LW = (np64(t) for t in (o, lse, oh, lseh, ow, lsew))
    for b in range(B):
        V = vis[b]
        for name, S, I, QI, KI in runs:
            s_ref = oracle.index_scores(QI[b, 0], W[b, 0], KI[b], V)
            assert np.all(np.isneginf(S[b, 0, V:])), (name, b, V)
            if V:
                bound = score_bound(QI[b, 0], W[b, 0], KI[b, :V], 128, 64)
                assert np.all(np.abs(S[b, 0, :V] - s_ref[:V]) <= bound), (name, b, V)
            check_topk(I[b, 0], s_ref, V, k)
        o_ref, l_ref = oracle.attend(Q[b, 0], K[b], Vv[b], runs[0][2][b, 0])
        check_attention(O[b, 0], o_ref, "bf16", f"csa b={b}")
        check_lse(L[b, 0], l_ref, 2.5e-3)
        oh_ref, lh_ref = oracle.hca_attend(Q[b, 0], K[b], Vv[b], V)
        check_attention(OH[b, 0], oh_ref, "bf16", f"hca b={b}")
        check_lse(LH[b, 0], lh_ref, 2.5e-3)
        ow_ref, lw_ref = oracle.swa_attend(Q[b, 0], K[b], Vv[b], pos[b], ne[b], win)
        check_attention(OW[b, 0], ow_ref, "bf16", f"swa b={b}")
        check_lse(LW[b, 0], lw_ref, 2.5e-3)
    for i in (0, 1):                                       # nothing visible
        assert np.all(OH[i, 0] == 0) and np.all(np.isneginf(LH[i, 0]))
        assert np.all(np.asarray(runs[0][2][i, 0]) == -1)


def test_tuned_prefill_scores_ragged():
    """bf16 64 x 128 with many queries per sequence (the prefill score
    kernel: 8 queries per workgroup, 4096 keys per workgroup): a query count
    that is not a multiple of 8, three key blocks with a ragged tail, visible
    counts from 0 to all (ending on and next to block boundaries), a
    partially valid cache.  Scores, the chunk bounds (through the selection)
    and the selection are checked."""
    B, Tq, N_max, m, k = 2, 13, 2 * 4096 + 300, 4, 300
    _say("tuned prefill bf16 64x128 ragged")
    qi = _randn((B, Tq, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 31)
    ki = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 32)
    wi = _randn((B, Tq, 64), 1 / 8, torch.float32, 33)
    pos = [[4 * N_max + 7, 2, 3, 4 * 1024 - 1, 4 * 2048 - 1, 4 * 8192 - 1, 4 * 8192 + 3, 4 * 4000,
            4 * 4095 + 3, 4 * 4096 - 1, 4 * 4100, 4 * 300 + 2, 4 * 37],
           [4 * 1000, 4 * 2500, 4 * 4300, 1, 4 * 257, 4 * 256 - 1, 4 * 512, 4 * 3000, 4 * 3500,
            4 * 4000, 4 * 4200, 4 * 4390, 4 * 100]]
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    n_ent = torch.tensor([N_max, 3333], dtype=torch.int32, device=DEV)
    scores = csa.index_score(qi, wi, ki, q_pos, n_ent, m)
    idx = csa.index_topk(qi, wi, ki, q_pos, n_ent, m, k)
    torch.cuda.synchronize()
    S, I = np64(scores), np64(idx)
    QI, KI, W = np64(qi), np64(ki), np64(wi)
    ne = n_ent.cpu().numpy()
    for b in range(B):
        for t in range(Tq):
            V = oracle.visible_count(pos[b][t], m, int(ne[b]))
            s_ref = oracle.index_scores(QI[b, t], W[b, t], KI[b], V)
            assert np.all(np.isneginf(S[b, t, V:])), (b, t, V)
            if V:
                bound = score_bound(QI[b, t], W[b, t], KI[b, :V], 128, 64)
                assert np.all(np.abs(S[b, t, :V] - s_ref[:V]) <= bound), (b, t, V)
            check_topk(I[b, t], s_ref, V, k)


def _low_chunks(ki, chunks, scale):
    """Scale the keys of the given 256-entry chunks down (their chunk reports
    become the row's lowest, as for freshly pooled entries)."""
    for c in chunks:
        ki[:, 256 * c:256 * (c + 1)] *= scale
    return ki


@pytest.mark.parametrize("Tq,N_max,k,chunks", [
    (72, 40000, 256, (3, 50, 151, 155)),        # streamed rows: c = 2, r = 128 of ~157 reports
    (1, 100000, 1024, (0, 7, 200, 389)),        # few long rows: c = 3, r = 342 of 391 reports
])
def test_topk_bound_rth_report(Tq, N_max, k, chunks):
    """Selection with more chunk reports than the bound needs (the bound is
    the r-th largest report, r = ceil(k / c), found by bisection), some
    chunks' keys scaled down so that their reports are the row's lowest:
    the selected sets against the oracle's exact top-k."""
    B = 2 if Tq == 1 else 1
    _say(f"top-k bound: Tq={Tq} N_max={N_max} k={k}")
    qi = _randn((B, Tq, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 41)
    ki = _low_chunks(_randn((B, N_max, 128), 1 / math.sqrt(128), torch.float32, 42), chunks, 0.3)
    ki = ki.to(torch.bfloat16)
    wi = _randn((B, Tq, 64), 1 / 8, torch.float32, 43)
    pos = [[4 * N_max - 1 - 4 * 37 * t for t in range(Tq)] for _ in range(B)]
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    n_ent = torch.tensor([N_max] * B, dtype=torch.int32, device=DEV)
    idx = csa.index_topk(qi, wi, ki, q_pos, n_ent, 4, k)
    torch.cuda.synchronize()
    I, QI, KI, W = np64(idx), np64(qi), np64(ki), np64(wi)
    rows = [(b, t) for b in range(B) for t in range(0, Tq, 7)]
    for b, t in rows:
        V = oracle.visible_count(pos[b][t], 4, N_max)
        s_ref = oracle.index_scores(QI[b, t], W[b, t], KI[b], V)
        check_topk(I[b, t], s_ref, V, k)


def test_fused_selection_ragged_rows_and_reuse():
    """Few long rows (the selection's workgroups share each row and the last
    to finish selects): visible counts that end mid-segment, leave whole
    segments invisible, fall below k and reach zero, over two calls on one
    zero-filled workspace with different head weights.  Each selection
    against the oracle's exact top-k; the row counters at the front of the
    workspace are zero again after each call."""
    N_max, k, m = 140000, 1024, 4
    bf = torch.bfloat16
    qi = _randn((5, 1, 64, 128), 1 / math.sqrt(128), bf, 111)
    ki = _randn((5, N_max, 128), 1 / math.sqrt(128), bf, 112)
    pos = [4 * N_max + 3, 4 * 70000 + 1, 4 * 90000, 4 * N_max, 2]
    ne = [N_max, 100001, 6000, 3, 100]
    q_pos = torch.tensor([[p_] for p_ in pos], dtype=torch.int32, device=DEV)
    n_ent = torch.tensor(ne, dtype=torch.int32, device=DEV)
    ws = csa.new_workspace(csa.index_topk_workspace_bytes(5, 1, N_max, k), DEV)
    QI, KI = np64(qi), np64(ki)
    for call in range(2):
        _say(f"fused selection, ragged rows: call {call}")
        wi = _randn((5, 1, 64), 1 / 8, torch.float32, 113 + call)
        idx = csa.index_topk(qi, wi, ki, q_pos, n_ent, m, k, workspace=ws)
        torch.cuda.synchronize()
        assert not ws[:4096].any(), "selection counters left non-zero"
        I, W = np64(idx), np64(wi)
        for b in range(5):
            V = oracle.visible_count(pos[b], m, ne[b])
            s_ref = oracle.index_scores(QI[b, 0], W[b, 0], KI[b], V)
            check_topk(I[b, 0], s_ref, V, k)


def test_fused_selection_crowded_segment():
    """Few long rows where one 4096-entry stretch holds far more survivors
    than a segment keeps (3,500 of its keys scaled by 8: the positive-scoring
    ones, some 1,400, clear the row bound): that row takes the exact
    fallback, the other row the shared path.  Both against the oracle's exact
    top-k."""
    N_max, k, m = 140000, 1024, 4
    bf = torch.bfloat16
    _say("fused selection: a crowded segment")
    qi = _randn((2, 1, 64, 128), 1 / math.sqrt(128), bf, 121)
    ki = _randn((2, N_max, 128), 1 / math.sqrt(128), torch.float32, 122)
    ki[0, 8192:8192 + 3500] *= 8.0
    ki = ki.to(bf)
    wi = _randn((2, 1, 64), 1 / 8, torch.float32, 123)
    q_pos = torch.full((2, 1), 4 * N_max + 3, dtype=torch.int32, device=DEV)
    n_ent = torch.full((2,), N_max, dtype=torch.int32, device=DEV)
    idx = csa.index_topk(qi, wi, ki, q_pos, n_ent, m, k)
    torch.cuda.synchronize()
    I, QI, KI, W = np64(idx), np64(qi), np64(ki), np64(wi)
    for b in range(2):
        s_ref = oracle.index_scores(QI[b, 0], W[b, 0], KI[b], N_max)
        check_topk(I[b, 0], s_ref, N_max, k)
    hot = (I[0, 0] >= 8192) & (I[0, 0] < 8192 + 3500)
    assert hot.sum() > 500, "the crowded stretch should dominate row 0's selection"


@pytest.mark.parametrize("B,Tq,N_max,k", [
    (2, 13, 2 * 2048 + 300, 300),   # prefill kernel; rows with and without a bound
    (3, 1, 70000, 1024),            # decode kernel; few long rows (shared by workgroups)
    (1, 1, 20000, 2048),            # no bound (c > 16): the row overflows the LDS list
])
def test_index_topk_bf16_scores_exact(B, Tq, N_max, k):
    """BF16 index scores: the selection equals the oracle's top-k of the GPU's
    own fp32 scores rounded to bf16 (nearest, ties to even), index for index,
    and the returned scores are those rounded values.  The fp32 scores come
    from csa_index_score, whose kernels compute the same sums (the bf16 path
    differs only in how it stores them)."""
    _say(f"bf16 index scores: B={B} Tq={Tq} N_max={N_max} k={k}")
    qi = _randn((B, Tq, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 61)
    ki = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 62)
    wi = _randn((B, Tq, 64), 1 / 8, torch.float32, 63)
    pos = [[4 * N_max - 1 - 4 * 301 * t - 4 * 999 * b for t in range(Tq)] for b in range(B)]
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    n_ent = torch.tensor([N_max - 17 * b for b in range(B)], dtype=torch.int32, device=DEV)
    idx, val = csa.index_topk_bf16(qi, wi, ki, q_pos, n_ent, 4, k, with_scores=True)
    s32 = csa.index_score(qi, wi, ki, q_pos, n_ent, 4)
    torch.cuda.synchronize()
    I, VAL, S = np64(idx), np64(val), np64(s32)
    ne = n_ent.cpu().numpy()
    for b in range(B):
        for t in range(Tq):
            V = oracle.visible_count(pos[b][t], 4, int(ne[b]))
            r = oracle.round_to_bf16(S[b, t, :V])
            want = oracle.topk_select(r, V, k)
            assert np.array_equal(I[b, t], want), (b, t, V)
            n = int((want >= 0).sum())
            assert np.array_equal(VAL[b, t, :n], r[want[:n]]), (b, t)
            assert np.all(np.isneginf(VAL[b, t, n:]))


@pytest.mark.parametrize("window", [1, 100, 1500, 6000])
@pytest.mark.parametrize("dtype,H,D", [(torch.bfloat16, 64, 128), (torch.float32, 3, 32)])
def test_swa_attend_ragged(window, dtype, H, D):
    """Sliding-window attention: windows of one token, inside one split, over
    several splits and beyond the cache; queries near the start (window
    clipped at token 0), at the end, and past the tokens cached (window ends
    at the cache end).  Outputs and lse against the oracle."""
    B, Tq, N_max = 2, 5, 5000
    _say(f"swa window={window} {dtype} H={H} D={D}")
    q = _randn((B, Tq, H, D), 1 / math.sqrt(D), dtype, 71)
    kc = _randn((B, N_max, D), 1 / math.sqrt(D), dtype, 72)
    vc = _randn((B, N_max, D), 1 / math.sqrt(D), dtype, 73)
    pos = [[0, 57, 1499, 3000, N_max - 1], [4, 2047, 2600, 4000, 4500]]
    n_tok = [N_max, 3001]
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    n_t = torch.tensor(n_tok, dtype=torch.int32, device=DEV)
    o, lse = csa.swa_attend(q, kc, vc, q_pos, n_t, window, with_lse=True)
    torch.cuda.synchronize()
    O, L, Q, K, Vv = np64(o), np64(lse), np64(q), np64(kc), np64(vc)
    kind = "bf16" if dtype == torch.bfloat16 else "f32"
    for b in range(B):
        for t in range(Tq):
            o_ref, l_ref = oracle.swa_attend(Q[b, t], K[b], Vv[b], pos[b][t], n_tok[b], window)
            check_attention(O[b, t], o_ref, kind, f"swa b={b} t={t}")
            check_lse(L[b, t], l_ref, 2.5e-3 if kind == "bf16" else 1e-5)


def test_fp4_scores_ragged():
    """FP4 indexer (E2M1 codes, one fp32 scale per 32 elements) on ragged
    sizes: a partial last load unit and chunk, visible counts inside the first
    unit, a partially valid cache.  Scores against the oracle fed the same
    quantised inputs (fp32 accumulation bound), then the selection."""
    from csa_synth.generate import fp4_quantize
    B, N_max, m, k = 3, 1000 + 37, 4, 300
    _say("fp4 ragged scores")
    qi = _randn((B, 1, 64, 128), 1 / math.sqrt(128), torch.float32, 81)
    ki = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.float32, 82)
    wi = _randn((B, 1, 64), 1 / 8, torch.float32, 83)
    qc, qs = (t.to(DEV) for t in fp4_quantize(qi))
    kc, ks = (t.to(DEV) for t in fp4_quantize(ki))
    pos = [4 * N_max + 3, 4 * 50 + 1, 4 * 777]
    q_pos = torch.tensor([[p] for p in pos], dtype=torch.int32, device=DEV)
    ne = [N_max, 900, 1001]
    n_ent = torch.tensor(ne, dtype=torch.int32, device=DEV)
    scores = csa.index_score(qc, wi, kc, q_pos, n_ent, m, q_scale=qs, k_scale=ks)
    idx = csa.index_topk(qc, wi, kc, q_pos, n_ent, m, k, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    S, I, W = np64(scores), np64(idx), np64(wi)
    QI = oracle.fp4_dequantize(qc.cpu().numpy(), qs.cpu().numpy())
    KI = oracle.fp4_dequantize(kc.cpu().numpy(), ks.cpu().numpy())
    for b in range(B):
        V = oracle.visible_count(pos[b], m, ne[b])
        s_ref = oracle.index_scores(QI[b, 0], W[b, 0], KI[b], V)
        assert np.all(np.isneginf(S[b, 0, V:])), (b, V)
        bound = score_bound(QI[b, 0], W[b, 0], KI[b, :V], 128, 64)
        assert np.all(np.abs(S[b, 0, :V] - s_ref[:V]) <= bound), (b, V)
        check_topk(I[b, 0], s_ref, V, k)


def test_mx4_scores_ragged():
    """MX FP4 indexer (E2M1 codes, one E8M0 scale byte per 32 elements, the
    hardware's block scales) on ragged sizes, with block exponents spread far
    apart on both sides (so a scale applied to the wrong block shows), an
    all-zero key block (scale byte 0) and a partially valid cache.  Scores
    against the oracle fed the same quantised inputs, then the selection."""
    from csa_synth import mx4_quantize
    B, N_max, m, k = 3, 1000 + 37, 4, 300
    _say("mx4 ragged scores")
    qi = _randn((B, 1, 64, 128), 1 / math.sqrt(128), torch.float32, 91)
    ki = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.float32, 92)
    wi = _randn((B, 1, 64), 1 / 8, torch.float32, 93)
    ki[:, :, 32:64] *= 2.0 ** 10
    ki[:, :, 96:128] *= 2.0 ** -12
    ki[:, 5:300:7, 64:96] = 0.0
    qi[:, :, 7, 0:32] *= 2.0 ** 20
    qi[:, :, 40, 96:128] *= 2.0 ** -30
    qi[:, :, 1::3, 32:64] *= 2.0 ** -9
    qc, qs = (t.to(DEV) for t in mx4_quantize(qi))
    kc, ks = (t.to(DEV) for t in mx4_quantize(ki))
    assert ks.dtype == torch.uint8 and int(ks.min()) == 0
    pos = [4 * N_max + 3, 4 * 50 + 1, 4 * 777]
    q_pos = torch.tensor([[p] for p in pos], dtype=torch.int32, device=DEV)
    ne = [N_max, 900, 1001]
    n_ent = torch.tensor(ne, dtype=torch.int32, device=DEV)
    scores = csa.index_score(qc, wi, kc, q_pos, n_ent, m, q_scale=qs, k_scale=ks)
    idx = csa.index_topk(qc, wi, kc, q_pos, n_ent, m, k, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    S, I, W = np64(scores), np64(idx), np64(wi)
    QI = oracle.mx4_dequantize(qc.cpu().numpy(), qs.cpu().numpy())
    KI = oracle.mx4_dequantize(kc.cpu().numpy(), ks.cpu().numpy())
    for b in range(B):
        V = oracle.visible_count(pos[b], m, ne[b])
        s_ref = oracle.index_scores(QI[b, 0], W[b, 0], KI[b], V)
        assert np.all(np.isneginf(S[b, 0, V:])), (b, V)
        bound = score_bound(QI[b, 0], W[b, 0], KI[b, :V], 128, 64)
        assert np.all(np.abs(S[b, 0, :V] - s_ref[:V]) <= bound), (b, V)
        check_topk(I[b, 0], s_ref, V, k)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,D", [(1, 32), (37, 128), (300, 256)])
def test_quantize_mx4_bit_exact(dtype, rows, D):
    """GPU MX FP4 encoder against the oracle's encoder, byte for byte: blocks
    spread over many binades, exact ties on the E2M1 grid, all-zero and
    signed-zero blocks, values rounding to -0, subnormal fp32 inputs, values
    near the fp32 maximum and saturating ones."""
    _say(f"quantize mx4 {dtype} rows={rows} D={D}")
    g = torch.Generator().manual_seed(rows * 1000 + D)
    x = torch.randn((rows, D), generator=g, dtype=torch.float64)
    x *= torch.exp2(torch.randint(-40, 40, (rows, D // 32), generator=g).double()).repeat_interleave(32, 1)
    x = x.to(torch.float32)
    x[0, :32] = 0.0
    x[0, :8] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0])      # ties, amax 6
    if rows > 1:
        x[1, :32] = -0.0
    if rows > 2:
        x[2, :32] = -1e-30
        x[2, 5] = 4.0
    if rows > 3:
        x[3, :32] = 1e-40                                   # fp32 subnormals
        x[3, 7] = -3e-39
    if rows > 4:
        x[4, :32] = 3.0e38
        x[4, 1] = -2.5e38
        x[4, 2] = 7.0                                       # tiny next to huge
    if rows > 5:
        x[5, :32] = 1.0
        x[5, 0] = 7.9                                       # amax / 2^e near 8: saturates
    if dtype == torch.bfloat16:
        x = x.to(torch.bfloat16).to(torch.float32)          # exact bf16 values, finite
        x = torch.nan_to_num(x, posinf=3.0e38, neginf=-3.0e38)
    xd = x.to(DEV, dtype)
    codes, scales = csa.quantize_mx4(xd)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mx4_quantize(xd.float().cpu().numpy())
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)


def _mx4_edge_blocks():
    """32-element blocks at the edges of the MX FP4 encoding, as fp32 lists."""
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    eps = 2.0 ** -10
    grid = [4.0] + ties + [t + eps for t in ties] + [t - eps for t in ties] + \
        [-t for t in ties] + [-0.0, 0.0, 6.0]
    blocks = [[v * 2.0 ** k for v in grid] for k in (3, -20, 100, -120)]
    pad = lambda b: b + [0.0] * (32 - len(b))
    blocks += [
        pad([7.99, 5.0, 5.01, -7.5, 6.0, -6.0, -5.0, 4.99]),            # saturation at 6
        [0.0] * 32, [-0.0] * 32, [0.0, -0.0] * 16,
        # e = -127 with non-zero codes: amax below 2^-125
        pad([2.0 ** -126, 2.0 ** -127, 3 * 2.0 ** -128, -(2.0 ** -149), 2.0 ** -149,
             1.5 * 2.0 ** -127, -(2.0 ** -128), 5 * 2.0 ** -130, 7 * 2.0 ** -131]),
        pad([1.5 * 2.0 ** -125, 2.0 ** -125, -(2.0 ** -127), 2.0 ** -129, 1.25 * 2.0 ** -126]),
        # e = -126: subnormal inputs next to the smallest normal scale
        pad([2.0 ** -124, 2.0 ** -127, -(2.0 ** -127), 2.0 ** -128, 3 * 2.0 ** -128,
             -(2.0 ** -149), 2.0 ** -126]),
        pad([1.0, 1e-40, -1e-40, 2.0 ** -149, -(2.0 ** -149), -0.0]),     # subnormals, e = -2
        pad([3.0e38, -3.0e38, 1.0e38, 2.0 ** 127, 2.0 ** 100, -(2.0 ** 126)]),
    ]
    if len(blocks) % 2:
        blocks.append([0.0] * 32)
    return blocks


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_mx4_edge_blocks(dtype):
    """GPU MX FP4 encoder on hand-made edge blocks, byte for byte against the
    oracle: ties and near-ties on the E2M1 grid in several binades,
    saturation, signed zeros, the clamped exponent -127 with non-zero codes,
    subnormal inputs under the smallest normal scale, values near the fp32
    maximum."""
    _say(f"quantize mx4 edge blocks {dtype}")
    x = torch.tensor(_mx4_edge_blocks(), dtype=torch.float32).reshape(-1, 64)
    assert torch.isfinite(x).all()
    xd = x.to(DEV, dtype)
    codes, scales = csa.quantize_mx4(xd)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mx4_quantize(xd.float().cpu().numpy())
    assert (s_ref == 0).any() and (c_ref[s_ref.repeat(16, 1) == 0] & 0x77).any()
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)


def test_quantize_mx4_then_score():
    """Indexer inputs encoded on the GPU feed the MX score path: scores and
    selection against the oracle on the GPU's own codes."""
    B, N_max, m, k = 2, 2048 + 77, 4, 256
    _say("quantize mx4 on the GPU, then MX scores")
    qi = _randn((B, 1, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 95)
    ki = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 96)
    wi = _randn((B, 1, 64), 1 / 8, torch.float32, 97)
    qc, qs = csa.quantize_mx4(qi)
    kc, ks = csa.quantize_mx4(ki)
    pos = [4 * N_max + 1, 4 * 1500]
    q_pos = torch.tensor([[p] for p in pos], dtype=torch.int32, device=DEV)
    ne = [N_max, 2000]
    n_ent = torch.tensor(ne, dtype=torch.int32, device=DEV)
    scores = csa.index_score(qc, wi, kc, q_pos, n_ent, m, q_scale=qs, k_scale=ks)
    idx = csa.index_topk(qc, wi, kc, q_pos, n_ent, m, k, q_scale=qs, k_scale=ks)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mx4_quantize(np64(ki))
    assert np.array_equal(kc.cpu().numpy(), c_ref) and np.array_equal(ks.cpu().numpy(), s_ref)
    QI = oracle.mx4_dequantize(qc.cpu().numpy(), qs.cpu().numpy())
    KI = oracle.mx4_dequantize(kc.cpu().numpy(), ks.cpu().numpy())
    S, I, W = np64(scores), np64(idx), np64(wi)
    for b in range(B):
        V = oracle.visible_count(pos[b], m, ne[b])
        s_ref_b = oracle.index_scores(QI[b, 0], W[b, 0], KI[b], V)
        bound = score_bound(QI[b, 0], W[b, 0], KI[b, :V], 128, 64)
        assert np.all(np.abs(S[b, 0, :V] - s_ref_b[:V]) <= bound), b
        check_topk(I[b, 0], s_ref_b, V, k)


def test_bounded_selection_ties_and_degenerate():
    """The bounded selection (chunk bounds + survivor list) on inputs far from
    Gaussian, where ties decide: all scores equal (more survivors than the
    list holds, and fewer), two distinct key rows (one value fills the
    threshold bin), integer-valued inputs (exact scores with many ties).
    The scores are exact or their distinct values far apart, so the set must
    equal the oracle's exactly (ties to the lower index)."""
    m = 4
    bf = torch.bfloat16

    def run(qi, wi, ki, ne, k):
        B, N = ki.shape[0], ki.shape[1]
        pos = torch.full((B, 1), 4 * N + 3, dtype=torch.int32, device=DEV)
        n_ent = torch.tensor(ne, dtype=torch.int32, device=DEV)
        idx = csa.index_topk(qi, wi, ki, pos, n_ent, m, k)
        torch.cuda.synchronize()
        I, QI, KI, W = np64(idx), np64(qi), np64(ki), np64(wi)
        for b in range(B):
            V = oracle.visible_count(4 * N + 3, m, ne[b])
            s = oracle.index_scores(QI[b, 0], W[b, 0], KI[b], V)
            ref = oracle.topk_select(s, V, k)
            assert np.array_equal(I[b, 0], ref), (b, V, k, np.nonzero(I[b, 0] != ref)[0][:8])

    _say("bounded selection: all scores equal")
    N = 32768
    qi = _randn((2, 1, 64, 128), 1 / math.sqrt(128), bf, 61)
    ki = _randn((2, N, 128), 1 / math.sqrt(128), bf, 62)
    run(qi, torch.zeros((2, 1, 64), dtype=torch.float32, device=DEV), ki, [N, 12000], 1024)

    _say("bounded selection: two distinct key rows")
    N = 16384
    qi = _randn((2, 1, 64, 128), 1 / math.sqrt(128), bf, 63)
    wi = _randn((2, 1, 64), 1 / 8, torch.float32, 64).abs()
    kv = _randn((2, 2, 128), 1 / math.sqrt(128), bf, 65)
    QI, W, KV = np64(qi), np64(wi), np64(kv)
    rng = np.random.default_rng(66)
    ki = torch.empty((2, N, 128), dtype=bf, device=DEV)
    for b in range(2):
        s2 = [float(W[b, 0] @ np.maximum(QI[b, 0] @ KV[b, j], 0.0)) for j in (0, 1)]
        assert abs(s2[0] - s2[1]) > 1e-3 * max(abs(s2[0]), abs(s2[1]))
        hi_j = int(s2[1] > s2[0])
        pick = np.where(rng.random(N) < 0.05, hi_j, 1 - hi_j)
        ki[b] = kv[b][torch.from_numpy(pick).to(DEV)]
    run(qi, wi, ki, [N, N - 5], 1024)
    run(qi, wi, ki, [N, N - 5], 512)

    _say("bounded selection: integer-valued inputs")
    N = 32768
    qi = torch.round(_randn((2, 1, 64, 128), 1.0, torch.float32, 67)).to(bf)
    ki = torch.round(_randn((2, N, 128), 1.5, torch.float32, 68)).to(bf)
    wi = torch.full((2, 1, 64), 1 / 64, dtype=torch.float32, device=DEV)
    run(qi, wi, ki, [N, 30001], 1024)

    _say("bounded selection: one outlier key, keys spread over many binades")
    N = 32768
    qi = _randn((2, 1, 64, 128), 1 / math.sqrt(128), bf, 69)
    wi = _randn((2, 1, 64), 1 / 8, torch.float32, 70).abs()
    kf = _randn((2, N, 128), 1 / math.sqrt(128), torch.float32, 71)
    kf[0, 1234] *= 4096.0                         # one score far above the rest
    kf[1] *= torch.pow(2.0, -(torch.arange(N, device=DEV) % 48).float())[:, None]
    ki = kf.to(bf)
    pos = torch.full((2, 1), 4 * N, dtype=torch.int32, device=DEV)
    n_ent = torch.tensor([N, N], dtype=torch.int32, device=DEV)
    idx = csa.index_topk(qi, wi, ki, pos, n_ent, m, 1024)
    torch.cuda.synchronize()
    I, QI, KI, W = np64(idx), np64(qi), np64(ki), np64(wi)
    for b in range(2):
        s_ref = oracle.index_scores(QI[b, 0], W[b, 0], KI[b], N)
        check_topk(I[b, 0], s_ref, N, 1024)


@pytest.mark.parametrize("B,Tq,N", [(2, 1, 262144), (1, 72, 66560)])
def test_bounded_selection_all_equal_long_rows(B, Tq, N):
    """Every score equal (zero head weights) on rows far longer than the LDS
    survivor list: the selection falls back to the whole row, where the
    counts of entries equal to the threshold exceed 16 bits.  The top-k of a
    constant row is its first k entries (ties to the lower index).  (2, 1,
    262144): few long rows, each shared by several workgroups; (1, 72,
    66560): more rows than that path takes, one workgroup per row."""
    m, k = 4, 1024
    bf = torch.bfloat16
    _say(f"all-equal rows: B={B} Tq={Tq} N={N}")
    qi = _randn((B, Tq, 64, 128), 1 / math.sqrt(128), bf, 81)
    ki = _randn((B, N, 128), 1 / math.sqrt(128), bf, 82)
    wi = torch.zeros((B, Tq, 64), dtype=torch.float32, device=DEV)
    pos = torch.full((B, Tq), 4 * N + 3, dtype=torch.int32, device=DEV)
    n_ent = torch.full((B,), N, dtype=torch.int32, device=DEV)
    idx = csa.index_topk(qi, wi, ki, pos, n_ent, m, k)
    torch.cuda.synchronize()
    I, QI, KI, W = np64(idx), np64(qi), np64(ki), np64(wi)
    for b in range(B):
        for t in sorted({0, Tq - 1}):
            s = oracle.index_scores(QI[b, t], W[b, t], KI[b], N)
            assert np.array_equal(I[b, t], oracle.topk_select(s, N, k)), (b, t)
    assert np.array_equal(I.reshape(-1, k), np.tile(np.arange(k), (B * Tq, 1)))


def test_step_graph_replay_matches_eager():
    """The decode step (index_topk + attend, and hca_attend) captured in a HIP
    graph with caller-owned workspaces: every replay, with eager work and
    synchronisations between replays, reproduces the eager results bitwise."""
    B, N, k, m = 4, 8192 + 96, 1024, 4
    bf = torch.bfloat16
    _say("graph capture of the decode step")
    q = _randn((B, 1, 64, 128), 1 / math.sqrt(128), bf, 71)
    kc = _randn((B, N, 128), 1 / math.sqrt(128), bf, 72)
    vc = _randn((B, N, 128), 1 / math.sqrt(128), bf, 73)
    qi = _randn((B, 1, 64, 128), 1 / math.sqrt(128), bf, 74)
    ki = _randn((B, N, 128), 1 / math.sqrt(128), bf, 75)
    wi = _randn((B, 1, 64), 1 / 8, torch.float32, 76)
    pos = torch.tensor([[4 * N], [4 * N - 9], [4000], [4 * 5000 + 1]], dtype=torch.int32, device=DEV)
    ne = torch.tensor([N, N, N, 6000], dtype=torch.int32, device=DEV)
    u8 = torch.uint8
    ws_t = csa.new_workspace(csa.index_topk_workspace_bytes(B, 1, N, k), DEV)
    ws_a = csa.new_workspace(csa.attend_workspace_bytes(bf, B, 1, 64, 128, k), DEV)
    ws_h = csa.new_workspace(csa.hca_workspace_bytes(bf, B, 1, 64, 128, N), DEV)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    o, oh = torch.empty_like(q), torch.empty_like(q)

    def step():
        csa.index_topk(qi, wi, ki, pos, ne, m, k, workspace=ws_t, out=idx)
        csa.attend(q, kc, vc, idx, ne, workspace=ws_a, out=o)
        csa.hca_attend(q, kc, vc, pos, ne, m, workspace=ws_h, out=oh)

    step()
    torch.cuda.synchronize()
    ref = (idx.clone(), o.clone(), oh.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        idx.fill_(-7)
        o.zero_()
        oh.zero_()
        ws_t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref[0]) and torch.equal(o, ref[1]) and torch.equal(oh, ref[2]), rep


def test_attention_sharp_and_single_entry():
    """Sharp softmax (logit std ~3) where the absolute gates bite, repeated and
    invalid indices, and a single selected entry (output = that value row)."""
    B, Tq, N_max, k = 2, 3, 4096, 1024
    _say("sharp attention bf16 64x128")
    q = _randn((B, Tq, 64, 128), 3.0, torch.bfloat16, 21)
    kc = _randn((B, N_max, 128), 1.0, torch.bfloat16, 22)
    vc = _randn((B, N_max, 128), 1.0, torch.bfloat16, 23)
    g = _gen(24)
    idx = torch.randint(-50, N_max + 50, (B, Tq, k), generator=g, device=DEV, dtype=torch.int32)
    idx[1, 2] = -1
    idx[1, 2, 17] = 3000                                   # single valid entry
    idx[0, 1, :512] = idx[0, 1, 512:]                      # repeated entries
    n_ent = torch.tensor([N_max, 3500], dtype=torch.int32, device=DEV)
    o, lse = csa.attend(q, kc, vc, idx, n_ent, with_lse=True)
    torch.cuda.synchronize()
    Q, K, Vv, I = np64(q), np64(kc), np64(vc), np64(idx)
    O, L = np64(o), np64(lse)
    ne = n_ent.cpu().numpy()
    for b in range(B):
        for t in range(Tq):
            sel = [j for j in I[b, t] if 0 <= j < ne[b]]
            o_ref, l_ref = oracle.attend(Q[b, t], K[b], Vv[b], sel)
            check_attention(O[b, t], o_ref, "bf16", f"sharp b={b} t={t}")
            check_lse(L[b, t], l_ref, LSE_TOL_BF16)
    assert np.array_equal(O[1, 2], np.tile(Vv[1, 3000], (64, 1)))


def _step_case(B, Tq, N_max, k, seed, wzero=False, pos=None, ne=None):
    bf = torch.bfloat16
    q = _randn((B, Tq, 64, 128), 3 / math.sqrt(128), bf, seed)
    kc = _randn((B, N_max, 128), 1 / math.sqrt(128), bf, seed + 1)
    vc = _randn((B, N_max, 128), 1 / math.sqrt(128), bf, seed + 2)
    qi = _randn((B, Tq, 64, 128), 1 / math.sqrt(128), bf, seed + 3)
    ki = _randn((B, N_max, 128), 1 / math.sqrt(128), bf, seed + 4)
    wi = _randn((B, Tq, 64), 1 / 8, torch.float32, seed + 5)
    if wzero:
        wi.zero_()
    if pos is None:
        pos = [[4 * N_max + 3] * Tq] * B
    if ne is None:
        ne = [N_max] * B
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    n_ent = torch.tensor(ne, dtype=torch.int32, device=DEV)
    return q, kc, vc, qi, ki, wi, q_pos, n_ent


@pytest.mark.parametrize("name,B,Tq,N_max,k,wzero,pos,ne", [
    # decode rows: several splits, V < k, no valid rows, k not a multiple of 128
    ("ragged", 4, 2, 5000, 300, False,
     [[4 * 5000 + 3, 2], [4 * 777, 4 * 200], [4 * 4000 + 1, 4 * 4500], [9, 4 * 5000]],
     [5000, 777, 4300, 0]),
    # rows of 2000 .. 12000 visible entries: no chunk bound (k > 16 * full chunks)
    ("unbounded", 2, 3, 12000, 1024, False,
     [[4 * 12000, 4 * 2000, 4 * 9000], [4 * 11999 + 3, 4 * 6000, 4 * 1025]], [12000, 12000]),
    # every score equal: the survivor list overflows, the whole row is selected from
    ("all_equal", 2, 1, 32768, 1024, True, None, None),
    # many query rows (the prefill score kernel)
    ("many_rows", 1, 520, 3000, 512, False, [[4 * 3000 + i for i in range(520)]], None),
])
def test_index_topk_attend_matches_separate(name, B, Tq, N_max, k, wzero, pos, ne):
    """csa_index_topk_attend (score -> top-k -> attention in one call, the
    index lists kept in its workspace) equals csa_index_topk followed by
    csa_attend bitwise (indices, outputs, lse), and matches the oracle stage
    by stage."""
    _say(f"index_topk_attend: {name}")
    q, kc, vc, qi, ki, wi, q_pos, n_ent = _step_case(B, Tq, N_max, k, 400, wzero, pos, ne)
    o, lse, idx = csa.index_topk_attend(qi, wi, ki, q, kc, vc, q_pos, n_ent, 4, k, with_lse=True,
                                        with_idx=True)
    idx2 = csa.index_topk(qi, wi, ki, q_pos, n_ent, 4, k)
    o2, lse2 = csa.attend(q, kc, vc, idx2, n_ent, with_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "top-k lists differ from csa_index_topk"
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)), "outputs differ from csa_attend"
    assert torch.equal(lse, lse2), "lse differs from csa_attend"
    I, Q, K, Vv, QI, KI, W = (np64(t) for t in (idx, q, kc, vc, qi, ki, wi))
    O, L = np64(o), np64(lse)
    P, NE = q_pos.cpu().numpy(), n_ent.cpu().numpy()
    rows = [(b, t) for b in range(B) for t in range(Tq)]
    for b, t in rows[:: max(1, len(rows) // 12)]:
        V = oracle.visible_count(int(P[b, t]), 4, int(NE[b]))
        s = oracle.index_scores(QI[b, t], W[b, t], KI[b], V)
        if wzero:
            assert np.array_equal(I[b, t], oracle.topk_select(s, V, k))
        else:
            check_topk(I[b, t], s, V, k)
        o_ref, l_ref = oracle.attend(Q[b, t], K[b], Vv[b], I[b, t])
        check_attention(O[b, t], o_ref, "bf16", f"{name} b={b} t={t}")
        check_lse(L[b, t], l_ref, LSE_TOL_BF16)


ATTEND_SYNC_BYTES = 32 * 4 * 65536                  # merge counters at the front


def test_attention_workspace_reuse_across_shapes():
    """One zero-filled workspace serves split attention calls of different
    shapes in a row (CSA with many and with one split, HCA, a sliding
    window): each result matches the oracle, and the merge counters at the
    front of the workspace are zero again after every call."""
    bf = torch.bfloat16
    N_max = 5000
    kc = _randn((4, N_max, 128), 1 / math.sqrt(128), bf, 91)
    vc = _randn((4, N_max, 128), 1 / math.sqrt(128), bf, 92)
    q = _randn((4, 2, 64, 128), 3 / math.sqrt(128), bf, 93)
    n_ent = torch.tensor([N_max, 4000, 77, 1], dtype=torch.int32, device=DEV)
    nbytes = max(csa.attend_workspace_bytes(bf, 4, 2, 64, 128, 1024),
                 csa.hca_workspace_bytes(bf, 4, 2, 64, 128, N_max),
                 csa.swa_workspace_bytes(bf, 4, 2, 64, 128, N_max, 3000))
    ws = csa.new_workspace(nbytes, DEV)
    K, Vv, Q = np64(kc), np64(vc), np64(q)
    ne = n_ent.cpu().numpy()
    g = _gen(94)
    for case, (B, k) in enumerate([(4, 1024), (2, 100), (3, 300)]):
        _say(f"workspace reuse: csa B={B} k={k}")
        idx = torch.randint(-3, N_max, (B, 2, k), generator=g, device=DEV, dtype=torch.int32)
        o, lse = csa.attend(q[:B], kc[:B], vc[:B], idx, n_ent[:B], with_lse=True, workspace=ws)
        torch.cuda.synchronize()
        assert not ws[:ATTEND_SYNC_BYTES].any(), "merge counters left non-zero"
        I, O, L = np64(idx), np64(o), np64(lse)
        for b in range(B):
            for t in range(2):
                o_ref, l_ref = oracle.attend(Q[b, t], K[b], Vv[b], [j for j in I[b, t] if j < ne[b]])
                check_attention(O[b, t], o_ref, "bf16", f"reuse csa case={case} b={b} t={t}")
                check_lse(L[b, t], l_ref, LSE_TOL_BF16)
    _say("workspace reuse: hca and swa")
    pos = torch.tensor([[4 * 4999 + 3, 700], [4 * 3000, 9], [500, 4 * 77 + 3], [2, 3]],
                       dtype=torch.int32, device=DEV)
    oh, lh = csa.hca_attend(q, kc, vc, pos, n_ent, 4, with_lse=True, workspace=ws)
    torch.cuda.synchronize()
    assert not ws[:ATTEND_SYNC_BYTES].any(), "merge counters left non-zero"
    os_, ls_ = csa.swa_attend(q, kc, vc, pos, n_ent, 3000, with_lse=True, workspace=ws)
    torch.cuda.synchronize()
    assert not ws[:ATTEND_SYNC_BYTES].any(), "merge counters left non-zero"
    P = pos.cpu().numpy()
    OH, LH, OS, LS = np64(oh), np64(lh), np64(os_), np64(ls_)
    for b in range(4):
        for t in range(2):
            V = oracle.visible_count(int(P[b, t]), 4, int(ne[b]))
            o_ref, l_ref = oracle.hca_attend(Q[b, t], K[b], Vv[b], V)
            check_attention(OH[b, t], o_ref, "bf16", f"reuse hca b={b} t={t}")
            check_lse(LH[b, t], l_ref, LSE_TOL_BF16)
            o_ref, l_ref = oracle.swa_attend(Q[b, t], K[b], Vv[b], int(P[b, t]), int(ne[b]), 3000)
            check_attention(OS[b, t], o_ref, "bf16", f"reuse swa b={b} t={t}")
            check_lse(LS[b, t], l_ref, LSE_TOL_BF16)


def test_compress_edge_cases():
    _say("compress edge cases")
    g = _gen(31)
    # m = 1 is an exact copy; a ragged tail of n % m tokens is ignored
    x = torch.randn((2, 37, 64), generator=g, device=DEV).to(torch.bfloat16)
    z = torch.randn((2, 37), generator=g, device=DEV)
    out = csa.compress(x, z, 1)
    torch.cuda.synchronize()
    assert torch.equal(out, x)
    out = csa.compress(x, z, 4)
    torch.cuda.synchronize()
    assert out.shape == (2, 9, 64)
    for b in range(2):
        check_compress(np64(out)[b], np64(x)[b][:36], np64(z)[b][:36], 4, "bf16")
    # large pooling factor, strided output rows, fp32
    x = torch.randn((1, 8192, 32), generator=g, device=DEV)
    z = torch.randn((1, 8192), generator=g, device=DEV) * 4
    dst = torch.zeros((1, 2, 48), device=DEV)
    csa.compress(x, z, 4096, out=dst[..., :32])
    torch.cuda.synchronize()
    check_compress(np64(dst)[0, :, :32], np64(x)[0], np64(z)[0], 4096, "f32")
    assert np.all(np64(dst)[0, :, 32:] == 0)


def test_batch_invariance_and_determinism():
    """A sequence's results are bitwise identical alone, in a batch, and with
    different batch-mates; repeated runs are bitwise identical."""
    _say("batch invariance")
    N, k = 8192 + 96, 1024
    def draw(B, seed):
        return dict(
            q=_randn((B, 1, 64, 128), 1 / math.sqrt(128), torch.bfloat16, seed),
            kc=_randn((B, N, 128), 1 / math.sqrt(128), torch.bfloat16, seed + 1),
            vc=_randn((B, N, 128), 1 / math.sqrt(128), torch.bfloat16, seed + 2),
            qi=_randn((B, 1, 64, 128), 1 / math.sqrt(128), torch.bfloat16, seed + 3),
            ki=_randn((B, N, 128), 1 / math.sqrt(128), torch.bfloat16, seed + 4),
            wi=_randn((B, 1, 64), 1 / 8, torch.float32, seed + 5))
    def run(d, m=4):
        B = d["q"].shape[0]
        pos = torch.full((B, 1), 4 * N, dtype=torch.int32, device=DEV)
        ne = torch.full((B,), N, dtype=torch.int32, device=DEV)
        idx = csa.index_topk(d["qi"], d["wi"], d["ki"], pos, ne, m, k)
        o = csa.attend(d["q"], d["kc"], d["vc"], idx, ne)
        oh = csa.hca_attend(d["q"], d["kc"], d["vc"], pos, ne, m)
        torch.cuda.synchronize()
        return idx, o, oh
    a = draw(4, 40)
    b = draw(4, 50)
    mix = {key: torch.cat([a[key][:1], b[key][1:]]) for key in a}
    alone = {key: a[key][:1].contiguous() for key in a}
    r1, r2, r3, r4 = run(a), run(a), run(mix), run(alone)
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)
    for x, y, z in zip(r1, r3, r4):
        assert torch.equal(x[:1], y[:1]) and torch.equal(x[:1], z)


@pytest.mark.parametrize("B,Tq,N_max", [(3, 9, 70), (2, 16, 300), (1, 8, 1)])
def test_prefill_kernel_tiny_and_empty(B, Tq, N_max):
    """The prefill score kernel (Tq >= 8) on caches shorter than one 256-key
    block and one 32-key tile, with an empty sequence, queries that see
    nothing and a partially valid cache: scores (-inf past the visible
    entries), and the selection with k above and below the visible count."""
    _say(f"prefill kernel tiny: B={B} Tq={Tq} N_max={N_max}")
    m = 4
    qi = _randn((B, Tq, 64, 128), 1 / math.sqrt(128), torch.bfloat16, 60 + B)
    ki = _randn((B, N_max, 128), 1 / math.sqrt(128), torch.bfloat16, 61 + B)
    wi = _randn((B, Tq, 64), 1 / 8, torch.float32, 62 + B)
    pos = [[(7 * t * t + 3 * b) % (4 * N_max + 9) for t in range(Tq)] for b in range(B)]
    pos[0][0] = -1
    q_pos = torch.tensor(pos, dtype=torch.int32, device=DEV)
    ne = [N_max, 0, max(N_max // 2, 1)][:B]
    n_ent = torch.tensor(ne, dtype=torch.int32, device=DEV)
    scores = csa.index_score(qi, wi, ki, q_pos, n_ent, m)
    for k in (1, 16):
        idx = csa.index_topk(qi, wi, ki, q_pos, n_ent, m, k)
        torch.cuda.synchronize()
        S, I = np64(scores), np64(idx)
        QI, KI, W = np64(qi), np64(ki), np64(wi)
        for b in range(B):
            for t in range(Tq):
                V = oracle.visible_count(pos[b][t], m, ne[b])
                s_ref = oracle.index_scores(QI[b, t], W[b, t], KI[b], V)
                assert np.all(np.isneginf(S[b, t, V:])), (b, t, V)
                if V:
                    bound = score_bound(QI[b, t], W[b, t], KI[b, :V], 128, 64)
                    assert np.all(np.abs(S[b, t, :V] - s_ref[:V]) <= bound), (b, t, V)
                check_topk(I[b, t], s_ref, V, k)
