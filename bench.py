"""Benchmark: CSA decode at 128K context on one MI355X.

One step = the whole decode hot path for one batch of 16 sequences, each with
a 131072-token context compressed 4:1 into 32768 entries and one new query
token: Lightning Indexer scores (64 heads x 128, bf16) -> top-1024 selection
-> sparse core attention (64 heads x 128, bf16) over the selected entries.

Inputs are synthetic, seeded and resident in HBM before timing.  The decode
working set (~143 MB) fits the 256 MB Infinity Cache, so consecutive steps
rotate through independent input copies (4 x 403 MB) and every step streams
from HBM.

Prints one JSON line.  Options: --steps K --warmup W --gpus N (only 1),
--graph (also time the step captured in a HIP graph), --no-cpu-baseline,
--workload NAME (another workload's own line instead of the headline one:
hca_decode_1m, csa_decode_1m_fp4, csa_decode_1m_mx4, csa_prefill_chunk (also
timing the step with bf16 index scores) or swa_decode_128k; see other_workload),
--score-only (launch only the indexer score kernel, for hardware-counter
runs), --copy-calibration (run only a plain device copy of known size, for
scaling the FETCH_SIZE / WRITE_SIZE counters).

roofline.traffic is read from the counter summary committed under profiles/;
it is null when the score kernel's source no longer matches the one the
counters were taken on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA decode tokens/sec + achieved HBM GB/s at 128K context, 1 MI355X"
WORKLOAD = "csa_decode_128k"
HBM_PEAK_GBS = 8000.0
N_COPIES = 4
SCORE_KERNEL = "score_bf16_h64d128_kernel"
SCORE_SOURCE = os.path.join(ROOT, "long_context_attention_24_amd", "csrc", "index_score.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "score_bf16_h64d128_csa_decode_128k_traffic.txt")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--graph", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calibration", action="store_true")
    p.add_argument("--score-only", action="store_true")
    p.add_argument("--workload", default=WORKLOAD)
    return p.parse_args()


def algorithmic_bytes(w):
    """Bytes the method must move per step and per score-kernel launch."""
    B, N, H, D, HI, DI, k = w.B, w.N, w.H, w.D, w.H_I, w.D_I, w.k
    ki = B * N * DI * 2                       # indexer keys, bf16
    gathers = B * k * D * 2 * 2               # selected K and V rows
    q = B * H * D * 2
    qi = B * HI * DI * 2
    wi = B * HI * 4
    o = B * H * D * 2
    idx = B * k * 4 * 2                       # written by top-k, read by attention
    step = ki + gathers + q + qi + wi + o + idx
    score_kernel = ki + qi + wi + B * N * 4   # + the fp32 scores it writes
    return step, score_kernel


def stage_bytes(w):
    """Algorithmic bytes of the selection and attention stages of one step
    (the score workspace is counted where it is read)."""
    B, N, H, D, k = w.B, w.N, w.H, w.D, w.k
    select = B * N * 4 + B * k * 4                 # scores read, indices written
    attend = B * k * D * 2 * 2 + B * H * D * 2 * 2 + B * k * 4   # K/V gathers, q, o, indices
    return select, attend


def _calibrate_sleep() -> float:
    """Spin-kernel cycles per millisecond on this GPU."""
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 2_000_000
    e0.record()
    torch.cuda._sleep(n)
    e1.record()
    torch.cuda.synchronize()
    return n / max(e0.elapsed_time(e1), 1e-3)


def copy_calibration():
    """A plain elementwise copy (x * 1.0) of 2**28 fp32 values: 1 GiB read and
    1 GiB written per launch, for scaling hardware byte counters."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 4 * n, "bytes_written": 4 * n, "launches": 5}))


def cpu_baseline(w, inputs, seconds):
    """The oracle as it stands, on this host: passes over the batch's
    sequences (one decode token each) until about `seconds` have elapsed."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info

    f64 = lambda t: oracle.from_bf16_bits(t.cpu().view(torch.int16).numpy().view(np.uint16)) \
        if t.dtype == torch.bfloat16 else t.cpu().double().numpy()
    host = {k: f64(v) for k, v in inputs.items() if v.dtype != torch.int32}
    done, t0 = 0, time.perf_counter()
    while True:
        b = done % w.B
        oracle.csa_reference(q=host["q"][b, 0], q_idx=host["q_idx"][b, 0], w_idx=host["w_idx"][b, 0],
                             k_cache=host["k_cache"][b], v_cache=host["v_cache"][b],
                             k_idx=host["ki_cache"][b], q_pos=w.q_pos0, m=w.m, k=w.k, n_entries=w.N)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} decode tokens ({done / w.B:.1f} passes over the {w.B} sequences of "
                      f"{WORKLOAD}), fp64 NumPy oracle, {el:.1f} s"}


def recorded_traffic():
    """HBM bytes per score-kernel launch from the committed counter summary,
    or None if it is missing or was taken on a different kernel source."""
    import hashlib
    try:
        lines = open(TRAFFIC_SUMMARY).read().splitlines()
    except OSError:
        return None
    kv = {}
    for ln in lines:
        if ":" in ln and not ln.startswith(" "):
            key, val = ln.split(":", 1)
            kv[key.strip()] = val.strip()
    src = hashlib.sha256(open(SCORE_SOURCE, "rb").read()).hexdigest()
    if kv.get("source_sha256") != src or "hbm_bytes_per_launch" not in kv:
        return None
    return int(kv["hbm_bytes_per_launch"])


def _timer():
    """(hold_gpu(ms), timed(fn, steps, warmup) -> ms per call) as in main()."""
    cycles_per_ms = _calibrate_sleep()

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(cycles_per_ms * (20.0 + 0.05 * steps)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    return timed


def other_workload(args):
    """One JSON line for a workload other than the headline one.

    hca_decode_1m: compress the 1M-token raw stream 128:1 (timed once per
      sequence batch, reported), then HCA decode steps (32 tokens) over the
      compressed caches; roofline: the attention's K/V stream against HBM.
    csa_decode_1m_fp4: FP4 indexer scores + top-k + sparse attention for 4
      decode tokens at 1M context; roofline: the FP4 score kernel's bytes.
    csa_decode_1m_mx4: the same with MX FP4 indexer inputs (one E8M0 scale
      byte per 32 elements); roofline: the MX score kernel's bytes.
    csa_prefill_chunk: compress the 4096 new tokens, score / select / attend
      all 4096 queries; roofline: the prefill score kernel's FLOPs against the
      bf16 MFMA peak.
    swa_decode_128k: sliding-window attention (window 4096) for 32 decode
      tokens over uncompressed 128K-token caches; roofline: the window's K/V
      bytes against HBM.
    """
    import long_context_attention_24_amd as csa
    from csa_synth import SWA_DECODE, WORKLOADS, make_inputs, make_swa_inputs

    dev = "cuda"
    timed = _timer()
    base = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if args.workload == "swa_decode_128k":
        p = SWA_DECODE
        B, N, H, D, W = p["B"], p["n_tokens"], p["H"], p["D"], p["window"]
        copies = [make_swa_inputs(B, N, H, D, p["seed"] + c, device=dev) for c in range(N_COPIES)]
        ws = torch.empty(csa.swa_workspace_bytes(torch.bfloat16, B, 1, H, D, N, W),
                         dtype=torch.uint8, device=dev)
        out = torch.empty_like(copies[0]["q"])

        def step(i):
            c = copies[i % N_COPIES]
            csa.swa_attend(c["q"], c["k"], c["v"], c["q_pos"], c["n_tokens"], W, workspace=ws,
                           out=out)
        ms = timed(step, args.steps, args.warmup)
        step_bytes = B * W * D * 2 * 2 + 2 * B * H * D * 2
        gbs = step_bytes / (ms * 1e-3) / 1e9
        base.update(dict(
            metric="Sliding-window decode tokens/sec (window 4096 at 128K context), 1 MI355X",
            value=round(B / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 5),
            config={"workload": "swa_decode_128k", "batch": B, "context_tokens": N,
                    "window": W, "heads": f"{H}x{D}"},
            roofline={"kernel": "attend_split_kernel<HCA, window> + combine", "bound": "hbm",
                      "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}))
        print(json.dumps(base))
        return
    w = WORKLOADS[args.workload]
    if w.name == "hca_decode_1m":
        inp = make_inputs(w, device=dev, parts=["raw", "logits", "q", "q_pos", "n_entries"])
        caches = []
        comp_ms = None
        for c in range(N_COPIES):
            kv = torch.empty((w.B, w.N, 2 * w.D), dtype=torch.bfloat16, device=dev)
            if c == 0:
                comp_ms = timed(lambda i: csa.compress(inp["raw"], inp["logits"], w.m, out=kv), 3, 1)
            else:
                csa.compress(inp["raw"], inp["logits"], w.m, out=kv)
            caches.append(kv)
        del inp["raw"]
        ws = torch.empty(csa.hca_workspace_bytes(torch.bfloat16, w.B, 1, w.H, w.D, w.N),
                         dtype=torch.uint8, device=dev)
        out = torch.empty_like(inp["q"])

        def step(i):
            kv = caches[i % N_COPIES]
            csa.hca_attend(inp["q"], kv[..., :w.D], kv[..., w.D:], inp["q_pos"], inp["n_entries"],
                           w.m, workspace=ws, out=out)
        ms = timed(step, args.steps, args.warmup)
        kv_bytes = w.B * w.N * w.D * 2 * 2
        step_bytes = kv_bytes + 2 * w.B * w.H * w.D * 2
        gbs = step_bytes / (ms * 1e-3) / 1e9
        raw_bytes = w.B * w.n_raw * (2 * w.D * 2 + 4) + w.B * w.N * 2 * w.D * 2
        res = dict(metric="HCA decode tokens/sec at 1M context (m'=128), 1 MI355X",
                   value=round(w.B / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 5),
                   config={"workload": w.name, "batch": w.B, "context_tokens": w.q_pos0,
                           "compressed_entries": w.N, "m": w.m, "heads": f"{w.H}x{w.D}"},
                   roofline={"kernel": "attend_split_kernel<HCA> + combine", "bound": "hbm",
                             "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
                   compress_ms=round(comp_ms, 4),
                   compress_gbs=round(raw_bytes / (comp_ms * 1e-3) / 1e9, 1))
    elif w.name in ("csa_decode_1m_fp4", "csa_decode_1m_mx4"):
        mx = w.name == "csa_decode_1m_mx4"
        # one quantised draw; the other copies hold its entries rolled along
        # the entry axis (distinct memory for the cache rotation)
        first = make_inputs(w, device=dev)
        copies = [first]
        for c in range(1, N_COPIES):
            cp = dict(first)
            for name in ("ki_codes", "ki_scale", "k_cache", "v_cache"):
                cp[name] = torch.roll(first[name], shifts=997 * c, dims=1)
            copies.append(cp)
        ws_topk = torch.empty(csa.index_topk_workspace_bytes(w.B, 1, w.N, w.k), dtype=torch.uint8,
                              device=dev)
        ws_attn = torch.empty(csa.attend_workspace_bytes(torch.bfloat16, w.B, 1, w.H, w.D, w.k),
                              dtype=torch.uint8, device=dev)
        idx = torch.empty((w.B, 1, w.k), dtype=torch.int32, device=dev)
        out = torch.empty_like(copies[0]["q"])
        scores = torch.empty((w.B, 1, w.N), dtype=torch.float32, device=dev)

        def step(i):
            c = copies[i % N_COPIES]
            csa.index_topk(c["q_codes"], c["w_idx"], c["ki_codes"], c["q_pos"], c["n_entries"], w.m,
                           w.k, q_scale=c["q_scale"], k_scale=c["ki_scale"], workspace=ws_topk,
                           out=idx)
            csa.attend(c["q"], c["k_cache"], c["v_cache"], idx, c["n_entries"], workspace=ws_attn,
                       out=out)

        def score_only(i):
            c = copies[i % N_COPIES]
            csa.index_score(c["q_codes"], c["w_idx"], c["ki_codes"], c["q_pos"], c["n_entries"], w.m,
                            q_scale=c["q_scale"], k_scale=c["ki_scale"], out=scores)
        ms = timed(step, args.steps, args.warmup)
        sms = timed(score_only, args.steps, args.warmup)
        extra = {}
        if mx:
            # the MX encoder on the GPU: a whole bf16 indexer-key cache
            # [B, N, 128] -> codes + scale bytes (HBM stream)
            kb = torch.randn((w.B, w.N, w.D_I), device=dev).to(torch.bfloat16)
            kcd = torch.empty((w.B, w.N, w.D_I // 2), dtype=torch.uint8, device=dev)
            ksd = torch.empty((w.B, w.N, w.D_I // 32), dtype=torch.uint8, device=dev)
            qms = timed(lambda i: csa.quantize_mx4(kb, codes=kcd, scales=ksd), 20, 3)
            qbytes = w.B * w.N * (w.D_I * 2 + w.D_I // 2 + w.D_I // 32)
            extra = {"quantize_kcache_ms": round(qms, 4),
                     "quantize_kcache_gbs": round(qbytes / (qms * 1e-3) / 1e9, 1)}
            del kb, kcd, ksd
        # per (row, entry): 64 B codes + the scales (16 B fp32 or 4 E8M0 bytes)
        # + 4 B score; per row the query codes, scales and head weights
        sc_b = 4 if mx else 16
        score_bytes = w.B * w.N * (64 + sc_b + 4) + w.B * w.H_I * (64 + sc_b + 4)
        gbs = score_bytes / (sms * 1e-3) / 1e9
        res = dict(metric=("CSA decode tokens/sec at 1M context, MX FP4 indexer (E8M0 scales), "
                           "1 MI355X") if mx else
                          "CSA decode tokens/sec at 1M context, FP4 indexer, 1 MI355X",
                   value=round(w.B / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 5),
                   config={"workload": w.name, "batch": w.B, "context_tokens": w.q_pos0,
                           "compressed_entries": w.N, "m": w.m,
                           "indexer": "64x128 FP4 E2M1, E8M0 block scales" if mx else
                                      "64x128 FP4 E2M1", "top_k": w.k},
                   roofline={"kernel": "score_mx4_h64d128_kernel" if mx else
                                       "score_fp4_h64d128_kernel", "bound": "hbm",
                             "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                             "algorithmic_bytes_per_launch": score_bytes,
                             "avg_launch_ms": round(sms, 5)}, **extra)
    elif w.name == "csa_prefill_chunk":
        inp = make_inputs(w, device=dev)
        cache = torch.empty((1, w.N, 384), dtype=torch.bfloat16, device=dev)
        cache[..., :128] = inp["k_cache"]
        cache[..., 128:256] = inp["v_cache"]
        cache[..., 256:] = inp["ki_cache"]
        kc, vc, ki = cache[..., :128], cache[..., 128:256], cache[..., 256:]
        ws_topk = torch.empty(csa.index_topk_workspace_bytes(1, w.Tq, w.N, w.k), dtype=torch.uint8,
                              device=dev)
        ws_attn = torch.empty(csa.attend_workspace_bytes(torch.bfloat16, 1, w.Tq, w.H, w.D, w.k),
                              dtype=torch.uint8, device=dev)
        idx = torch.empty((1, w.Tq, w.k), dtype=torch.int32, device=dev)
        out = torch.empty_like(inp["q"])
        scores = torch.empty((1, w.Tq, w.N), dtype=torch.float32, device=dev)

        def step(i):
            csa.compress(inp["raw"], inp["logits"], w.m, out=cache[:, w.n_cache:])
            csa.index_topk(inp["q_idx"], inp["w_idx"], ki, inp["q_pos"], inp["n_entries"], w.m, w.k,
                           workspace=ws_topk, out=idx)
            csa.attend(inp["q"], kc, vc, idx, inp["n_entries"], workspace=ws_attn, out=out)

        def score_only(i):
            csa.index_score(inp["q_idx"], inp["w_idx"], ki, inp["q_pos"], inp["n_entries"], w.m,
                            out=scores)
        ws_topk16 = torch.empty(csa.index_topk_bf16_workspace_bytes(1, w.Tq, w.N, w.k),
                                dtype=torch.uint8, device=dev)

        def step_bf16_scores(i):   # the same step with the score matrix held in bf16
            csa.compress(inp["raw"], inp["logits"], w.m, out=cache[:, w.n_cache:])
            csa.index_topk_bf16(inp["q_idx"], inp["w_idx"], ki, inp["q_pos"], inp["n_entries"],
                                w.m, w.k, workspace=ws_topk16, out=idx)
            csa.attend(inp["q"], kc, vc, idx, inp["n_entries"], workspace=ws_attn, out=out)
        steps, warm = max(1, min(args.steps, 10)), max(1, min(args.warmup, 2))
        ms = timed(step, steps, warm)
        sms = timed(score_only, steps, warm)
        ms16 = timed(step_bf16_scores, steps, warm)
        # visible (query, entry) pairs x 64 heads x 128 dims x 2
        vis = sum(w.n_cache + (i + 1) // w.m for i in range(w.Tq))
        flop = vis * w.H_I * w.D_I * 2
        tfs = flop / (sms * 1e-3) / 1e12
        res = dict(metric="CSA prefill tokens/sec (4096-token chunk at 256K context), 1 MI355X",
                   value=round(w.Tq / (ms * 1e-3), 1), unit="tokens/s", ms_per_step=round(ms, 5),
                   config={"workload": w.name, "batch": 1, "chunk_tokens": w.Tq,
                           "context_tokens": w.q_pos0, "compressed_entries": w.N, "m": w.m,
                           "top_k": w.k},
                   roofline={"kernel": "score_prefill_bf16_h64d128_kernel", "bound": "mfma",
                             "achieved": round(tfs, 1), "peak": 2500.0, "unit": "TFLOP/s",
                             "frac": round(tfs / 2500.0, 4), "traffic": None,
                             "algorithmic_flop_per_launch": flop, "avg_launch_ms": round(sms, 4)},
                   bf16_index_scores={"ms_per_step": round(ms16, 5),
                                      "tokens_per_s": round(w.Tq / (ms16 * 1e-3), 1)})
        base["steps"], base["warmup"] = steps, warm
    else:
        print(f"unknown workload {w.name}", file=sys.stderr)
        sys.exit(2)
    base.update(res)
    print(json.dumps(base))


def _stages(w, score_ms, index_topk_ms, attend_ms, score_bytes):
    """Per-stage time, algorithmic bytes and HBM fraction (selection = the
    index_topk call minus the score kernel, so it includes one launch gap)."""
    sel_b, att_b = stage_bytes(w)
    out = {}
    for name, ms, b in (("score", score_ms, score_bytes),
                        ("selection", index_topk_ms - score_ms, sel_b),
                        ("attention", attend_ms, att_b)):
        gbs = b / (ms * 1e-3) / 1e9 if ms > 0 else 0.0
        out[name] = {"ms": round(ms, 5), "algorithmic_bytes": b, "gbs": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    if args.workload != WORKLOAD:
        other_workload(args)
        return

    import long_context_attention_24_amd as csa
    from csa_synth import WORKLOADS, make_inputs

    w = WORKLOADS[WORKLOAD]
    dev = "cuda"
    copies = [make_inputs(w.scaled(seed=w.seed + 1000 * c), device=dev) for c in range(N_COPIES)]
    ws_topk = torch.empty(csa.index_topk_workspace_bytes(w.B, 1, w.N, w.k), dtype=torch.uint8, device=dev)
    ws_attn = torch.empty(csa.attend_workspace_bytes(torch.bfloat16, w.B, 1, w.H, w.D, w.k),
                          dtype=torch.uint8, device=dev)
    idx = [torch.empty((w.B, 1, w.k), dtype=torch.int32, device=dev) for _ in range(N_COPIES)]
    out = [torch.empty_like(c["q"]) for c in copies]
    scores = torch.empty((w.B, 1, w.N), dtype=torch.float32, device=dev)

    def step(i):
        c = copies[i % N_COPIES]
        csa.index_topk(c["q_idx"], c["w_idx"], c["ki_cache"], c["q_pos"], c["n_entries"], w.m, w.k,
                       workspace=ws_topk, out=idx[i % N_COPIES])
        csa.attend(c["q"], c["k_cache"], c["v_cache"], idx[i % N_COPIES], c["n_entries"],
                   workspace=ws_attn, out=out[i % N_COPIES])

    def score_only(i):
        c = copies[i % N_COPIES]
        csa.index_score(c["q_idx"], c["w_idx"], c["ki_cache"], c["q_pos"], c["n_entries"], w.m,
                        out=scores)

    def index_topk_only(i):
        c = copies[i % N_COPIES]
        csa.index_topk(c["q_idx"], c["w_idx"], c["ki_cache"], c["q_pos"], c["n_entries"], w.m, w.k,
                       workspace=ws_topk, out=idx[i % N_COPIES])

    def attend_only(i):
        c = copies[i % N_COPIES]
        csa.attend(c["q"], c["k_cache"], c["v_cache"], idx[i % N_COPIES], c["n_entries"],
                   workspace=ws_attn, out=out[i % N_COPIES])

    # Host launch overhead (Python + ctypes) is comparable to a kernel's
    # duration, so every timed region is enqueued behind a spin kernel that
    # keeps the GPU busy until the whole region is queued: the events then
    # measure back-to-back GPU execution only.
    cycles_per_ms = _calibrate_sleep()

    def hold_gpu(ms):
        torch.cuda._sleep(int(cycles_per_ms * ms))

    def timed(fn, steps, warmup, per_launch=False):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        hold_gpu(20.0 + 0.05 * steps)
        if per_launch:
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for i in range(steps):
                ev[i][0].record()
                fn(i)
                ev[i][1].record()
            torch.cuda.synchronize()
            times = [a.elapsed_time(b) for a, b in ev]
            if per_launch == "quantiles":
                times.sort()
                return [times[int(q * (steps - 1))] for q in (0.1, 0.5, 0.9)]
            return sum(times) / steps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps          # ms per call

    graph_ms = None
    if args.graph:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(N_COPIES):
                step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(N_COPIES):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(i)
            graphs.append(g)
        graph_ms = timed(lambda i: graphs[i % N_COPIES].replay(), args.steps, args.warmup)

    if args.score_only:
        ms = timed(score_only, args.steps, args.warmup, per_launch=True)
        print(json.dumps({"score_only_ms": round(ms, 5), "launches": args.steps + args.warmup}))
        return
    ms = timed(step, args.steps, args.warmup)
    step_q = timed(step, args.steps, args.warmup, per_launch="quantiles")
    score_ms = timed(score_only, args.steps, args.warmup, per_launch=True)
    index_topk_ms = timed(index_topk_only, args.steps, args.warmup, per_launch=True)
    attend_ms = timed(attend_only, args.steps, args.warmup, per_launch=True)
    best_ms = min(ms, graph_ms) if graph_ms else ms

    step_bytes, score_bytes = algorithmic_bytes(w)
    tok_s = w.B / (best_ms * 1e-3)
    score_gbs = score_bytes / (score_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(best_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": w.B, "context_tokens": w.q_pos0,
                   "compressed_entries": w.N, "m": w.m, "indexer": f"{w.H_I}x{w.D_I} bf16",
                   "top_k": w.k, "core_attention": f"{w.H}x{w.D} bf16, 1 shared KV head",
                   "input_copies_rotated": N_COPIES,
                   "timing": "hip graph" if graph_ms and graph_ms <= ms else "eager launches"},
        "step_achieved_gbs": round(step_bytes / (best_ms * 1e-3) / 1e9, 1),
        "step_algorithmic_bytes": step_bytes,
        "ms_per_step_eager": round(ms, 5),
        "step_ms_p10_p50_p90": [round(x, 5) for x in step_q],
        "ms_per_step_graph": round(graph_ms, 5) if graph_ms else None,
        "call_ms": {"index_score": round(score_ms, 5),
                    "index_topk (score + selection)": round(index_topk_ms, 5),
                    "attend (split + combine)": round(attend_ms, 5)},
        "stages": _stages(w, score_ms, index_topk_ms, attend_ms, score_bytes),
        "roofline": {"kernel": SCORE_KERNEL, "bound": "hbm",
                     "achieved": round(score_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(score_gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(),
                     "algorithmic_bytes_per_launch": score_bytes,
                     "avg_launch_ms": round(score_ms, 5)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, copies[0], args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
