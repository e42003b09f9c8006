"""Benchmark of the CSA / HCA hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-graph] [--no-cpu-baseline]

Default workload: CSA decode at a 131,072-token context (batch 32, 32,768 compressed entries
per sequence, c = 512, 128 query heads, fp8 e4m3 indexer 64 x 128, top-k 1024).  One step =
index + top-k + sparse MQA for one new token per sequence; every m-th step (m = 4) the new
token completes a block, and that step first compresses the block's KV entry (bf16) and
index-key entry (fp8) from the decode state into the caches.  A run of m consecutive steps is
captured once in a HIP graph and replayed between two synchronisations (K is rounded up to a
multiple of m); inputs are resident in HBM before timing.

Prints one JSON line: whole-step throughput (query tokens/s), the roofline of the dominant
kernel (timed with HIP events on the stream it runs on), and the CPU oracle's throughput on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA query tokens/s (compress+index+top-k+MQA) at 128K ctx; % of roofline"
# the compressor-only workload counts raw tokens compressed, not query tokens
METRIC_COMPRESS = "CSA raw tokens compressed/s (csa_compress over a 1M-token sequence); % of HBM roofline"


def mxfp4_recall_record():
    """Mean / min / max per-sequence recall of the fp8 top-k by the MXFP4 top-k (both the
    oracle's, on the 128K decode draws), from tests/golden/mxfp4_recall_cfg2.txt; None if absent."""
    path = os.path.join(ROOT, "tests", "golden", "mxfp4_recall_cfg2.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and parts[0] in ("recall_mean", "recall_min", "recall_max"):
            rec[parts[0][len("recall_"):]] = float(parts[1])
    rec["source"] = "tests/golden/mxfp4_recall_cfg2.txt"
    return rec


def metric_for(cfg) -> str:
    """The metric string of a workload: the headline one for 128K-context decode, else a label
    that names what that workload's tokens/s counts."""
    if cfg.kind == "csa_compress":
        return METRIC_COMPRESS
    if cfg.kind == "csa_decode":
        ctx = cfg.q_pos0   # tokens before the query
        if ctx == 1 << 17:
            return METRIC
        return METRIC.replace("at 128K ctx", "at %s ctx" % ("1M" if ctx == 1 << 20 else str(ctx)))
    if cfg.kind == "csa_prefill":
        return "CSA prefill query tokens/s (compress+index+top-k+MQA) over a %d-token chunk; %% of roofline" % cfg.T
    return ("HCA query tokens/s (compress+dense MQA) for a %d-query chunk ending at position %d; %% of roofline"
            % (cfg.T, cfg.q_pos0 + cfg.T))
HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_PEAK = {"bf16": 2.5e15, "fp8": 5.0e15}
# MXFP4: a 4-bit value plus a 1-byte scale per 32; mixed KV rows: 448 fp8 + 64 bf16 per 512
DT_BYTES = {0: 4, 1: 2, 2: 1, 3: 17 / 32, 4: 576 / 512}
DT_NAME = {0: "f32", 1: "bf16", 2: "fp8_e4m3", 3: "mxfp4", 4: "kv_fp8_bf16"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------- algorithmic work
def stage_work(cfg):
    """Per-stage algorithmic bytes / flops of one step (each input byte read once, each output
    written once; flops over visible or selected pairs only)."""
    B, c, H = cfg.batch, cfg.c, cfg.H
    e = DT_BYTES[cfg.dt]
    st = {}
    if cfg.kind == "csa_compress":
        n = cfg.n
        st["compress"] = dict(bytes=4 * B * n * c * e + B * (n // cfg.m) * c * e + 2 * cfg.m * c * 4, flops=0,
                              bound="hbm")
        return st
    if cfg.kind == "csa_decode":
        # one decode-step compression (both caches, every sequence): the a-streams' current
        # block and the b-streams' previous block (m tokens each), the biases, one entry out
        m, cI = cfg.m, cfg.c_I
        e_kI = DT_BYTES[cfg.qk_dt]
        st["compress_step"] = dict(bytes=4 * B * m * (c + cI) * e + B * (c * e + cI * e_kI) + 2 * m * (c + cI) * 4,
                                   flops=0, bound="hbm")
    if cfg.kind in ("csa_decode", "csa_prefill"):
        T, N, HI, cI, k = cfg.T, cfg.N, cfg.H_I, cfg.c_I, cfg.k
        eq = DT_BYTES[cfg.qk_dt]
        pos = cfg.q_pos0 + np.arange(T)
        vis = np.minimum(N, (pos + 1) // cfg.m)          # visible entries per query
        pairs = int(vis.sum()) * B
        sel = int(np.minimum(vis, k).sum()) * B
        if cfg.kind == "csa_prefill":
            n = cfg.n
            st["compress_kv"] = dict(bytes=4 * B * n * c * e + B * (n // cfg.m) * c * e + 2 * cfg.m * c * 4, flops=0,
                                     bound="hbm")
            st["compress_kI"] = dict(bytes=4 * B * n * cI * e + B * (n // cfg.m) * cI * e + 2 * cfg.m * cI * 4,
                                     flops=0, bound="hbm")
        idx_bytes = B * N * cI * eq + B * T * HI * (cI * eq + 4) + pairs * 4
        st["index"] = dict(bytes=idx_bytes, flops=2 * pairs * HI * cI,
                           bound="hbm" if cfg.kind == "csa_decode" else "mfma")
        st["topk"] = dict(bytes=pairs * 4 + B * T * k * 8, flops=0, bound="hbm")
        # decode gathers distinct rows per sequence from HBM; prefill re-gathers from a cache
        # that stays in L2/MALL, so its HBM bytes are the cache read once
        ekv = DT_BYTES[cfg.dt if cfg.kv_dt < 0 else cfg.kv_dt]
        kv_bytes = sel * c * ekv if cfg.kind == "csa_decode" else B * N * c * e
        st["mqa"] = dict(bytes=kv_bytes + 2 * B * T * H * c * e + B * T * k * 4, flops=4 * sel * H * c,
                         bound="hbm" if cfg.kind == "csa_decode" else "mfma")
    else:
        n, mp, T, N = cfg.n, cfg.m_prime, cfg.T, cfg.N
        pos = cfg.q_pos0 + np.arange(T)
        vis = np.minimum(N, (pos + 1) // mp)
        pairs = int(vis.sum()) * B
        st["compress"] = dict(bytes=2 * B * n * c * e + B * N * c * e + mp * c * 4, flops=0, bound="hbm")
        st["mqa"] = dict(bytes=B * N * c * e + 2 * B * T * H * c * e, flops=4 * pairs * H * c, bound="mfma")
    return st


def peak_for(cfg, stage, bound):
    if bound == "hbm":
        return HBM_PEAK, "GB/s"
    if stage == "index" and cfg.qk_dt == 2:
        return MFMA_PEAK["fp8"], "TFLOP/s"
    return MFMA_PEAK["bf16"], "TFLOP/s"


# ---------------------------------------------------------------------------- CPU baseline
def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, host, budget_s=10.0):
    """The oracle on a bounded sample of the workload, repeated until about budget_s seconds of
    CPU work have been timed."""
    reps, tokens, elapsed = 0, 0, 0.0
    while elapsed < budget_s:
        r = _cpu_sample(cfg, host)
        reps += 1
        tokens += r["tokens"]
        elapsed += r["seconds"]
        sample = r["sample"]
    import oracle

    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{sample}; {reps} repetitions", "seconds": round(elapsed, 3), "cpu_model": cpu_model()}


def _cpu_sample(cfg, host):
    import oracle

    t0 = time.perf_counter()
    if cfg.kind == "csa_decode":
        nseq = cfg.batch
        sub = {k: host[k][:nseq] for k in ("kv", "q", "w")}
        if cfg.kv_dt == 4:   # mixed fp8 / bf16 KV rows: the oracle decodes them
            sub["kv"] = oracle.decode_kv_fp8_bf16(sub["kv"], cfg.c)
        if cfg.qk_dt == 3:   # MXFP4 storage: the oracle decodes it (shape from the config)
            sub["qI"] = oracle.decode_mxfp4(host["qI"], (cfg.batch, cfg.T, cfg.H_I, cfg.c_I))
            sub["kI"] = oracle.decode_mxfp4(host["kI"], (cfg.batch, cfg.N, cfg.c_I))
        else:
            sub["qI"], sub["kI"] = host["qI"][:nseq], host["kI"][:nseq]
        sc = oracle.index_scores(sub["qI"], sub["w"], sub["kI"], cfg.m, q_pos0=cfg.q_pos0, qk_dtype=cfg.qk_dt)
        idx, _ = oracle.topk(sc, cfg.m, cfg.k, q_pos0=cfg.q_pos0)
        oracle.sparse_mqa(sub["q"], sub["kv"], idx, cfg.scale, dtype=cfg.dt)
        what = "index + top-k + MQA"
        if "Ca" in host and "ICa" in host:   # one block's entries per sequence (every m steps)
            oracle.csa_compress(host["Ca"], host["Cb"], host["Za"], host["Zb"], host["Ba"], host["Bb"], cfg.m,
                                in_dtype=cfg.dt, out_dtype=cfg.dt)
            oracle.csa_compress(host["ICa"], host["ICb"], host["IZa"], host["IZb"], host["IBa"], host["IBb"], cfg.m,
                                in_dtype=cfg.dt, out_dtype=cfg.qk_dt)
            what = "index + top-k + MQA, plus one step's compression of the KV and index-key entries"
        tokens = nseq * cfg.T
        sample = f"all {nseq} sequences x {cfg.T} token ({what}, float64)"
    elif cfg.kind == "csa_compress":
        nt = 1 << 16
        oracle.csa_compress(*(host[k][:, :nt] for k in ("Ca", "Cb", "Za", "Zb")), host["Ba"], host["Bb"], cfg.m,
                            in_dtype=cfg.dt, out_dtype=cfg.dt)
        tokens = nt
        sample = f"the first {nt} tokens of the sequence (CSA compression, float64)"
    elif cfg.kind == "csa_prefill":
        rows = np.arange(cfg.T - 64, cfg.T)
        dt = cfg.dt
        kv = oracle.csa_compress(host["Ca"], host["Cb"], host["Za"], host["Zb"], host["Ba"], host["Bb"], cfg.m,
                                 in_dtype=dt, out_dtype=dt)
        kI = oracle.csa_compress(host["ICa"], host["ICb"], host["IZa"], host["IZb"], host["IBa"], host["IBb"], cfg.m,
                                 in_dtype=dt, out_dtype=dt)
        qpos = cfg.q_pos0 + rows
        sc = oracle.index_scores(host["qI"][:, rows], host["w"][:, rows], kI, cfg.m, qk_dtype=cfg.qk_dt, qpos=qpos)
        idx, _ = oracle.topk(sc, cfg.m, cfg.k, qpos=qpos)
        oracle.sparse_mqa(host["q"][:, rows], kv, idx, cfg.scale, dtype=dt)
        tokens = len(rows)
        sample = f"full compression + the last {len(rows)} query rows (index + top-k + MQA), float64"
    else:
        rows = np.arange(cfg.T - 8, cfg.T)
        kv = oracle.hca_compress(host["C"], host["Z"], host["B"], cfg.m_prime, in_dtype=cfg.dt, out_dtype=cfg.dt)
        oracle.hca_dense_mqa(host["q"][:, rows], kv, cfg.m_prime, cfg.scale, dtype=cfg.dt, qpos=cfg.q_pos0 + rows)
        tokens = len(rows)
        sample = f"full HCA compression + {len(rows)} query rows of dense MQA, float64"
    return {"tokens": tokens, "sample": sample, "seconds": time.perf_counter() - t0}


# ---------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="cfg2_csa_decode_128k")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stage-reps", type=int, default=0, help="launches per stage for kernel timing (0: = steps)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run device-to-device copies of BYTES (HBM counter calibration) and exit")
    ap.add_argument("--rope", action="store_true",
                    help="only time csa_rope (the last 64 channels) on a copy of the workload's q and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_calibration, "copies": 5}), flush=True)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import long_context_sparse_08_amd as csa
    from long_context_sparse_08_amd.pipeline import CsaCompress, CsaDecode, CsaPrefill, HcaChunk
    from workloads import CONFIGS, make_inputs, shapes

    cfg = CONFIGS[args.config]
    torch.cuda.set_device(0)
    if args.rope:
        # partial RoPE in place on a copy of q (bf16 [batch, T, H, c]); HBM-bound: each rotated
        # channel is read and written once
        q = torch.randn((cfg.batch, cfg.T, cfg.H, cfg.c), device="cuda").to(torch.bfloat16)
        d = 64
        fn = lambda: csa.csa_rope(q, cfg.q_pos0, 1, d)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        reps = max(args.steps, 10)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        byt = 2 * cfg.batch * cfg.T * cfg.H * d * 2
        print(json.dumps({"rope": {"workload": cfg.name, "rows": cfg.batch * cfg.T, "heads": cfg.H, "d": d,
                                   "ms_per_call": round(ms, 5), "bytes": byt,
                                   "hbm_frac": round(byt / (ms * 1e-3) / HBM_PEAK, 4)}}), flush=True)
        return
    log(f"[bench] generating inputs for {cfg.name}")
    host = make_inputs(cfg)
    sh = shapes(cfg)
    dev = {}
    for k, v in host.items():
        t = torch.from_numpy(v)
        if sh[k][1] == 1:
            t = t.view(torch.bfloat16)
        if sh[k][1] == 3:
            dev[k] = csa.MXFP4(t.cuda(), sh[k][0])
        elif sh[k][1] == 4:
            dev[k] = csa.KVFp8Bf16(t.cuda(), sh[k][0][-1])
        else:
            dev[k] = t.cuda()
    torch.cuda.synchronize()
    log("[bench] inputs resident on the GPU")

    if cfg.kind == "csa_decode":
        pipe = CsaDecode(dev, cfg.m, cfg.k, cfg.q_pos0)
    elif cfg.kind == "csa_prefill":
        pipe = CsaPrefill(dev, cfg.m, cfg.k, cfg.q_pos0)
    elif cfg.kind == "csa_compress":
        pipe = CsaCompress(dev, cfg.m)
    else:
        pipe = HcaChunk(dev, cfg.m_prime, cfg.q_pos0)

    # the timed unit: one step, or (decode with a state) a run of m steps whose last one
    # compresses the entries of the block its token completes
    with_compress = cfg.kind == "csa_decode" and pipe.can_compress()
    unit_fn = pipe.run_steps if with_compress else pipe.run
    per_unit = cfg.m if with_compress else 1

    def capture(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        return g

    def timed(fn, units):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(units):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    for _ in range(max(1, args.warmup // per_unit)):
        unit_fn()
    torch.cuda.synchronize()
    graph = None if args.no_graph else capture(unit_fn)

    # ---- timed region: K whole steps (K rounded up to whole units)
    units = (args.steps + per_unit - 1) // per_unit
    steps = units * per_unit
    log(f"[bench] timing {steps} steps ({'graph' if graph else 'eager'})")
    ms = timed(graph.replay if graph is not None else unit_fn, units) / steps
    tokens = cfg.batch * cfg.T
    value = tokens / (ms * 1e-3)
    # the same m-step units without the compression, for comparison
    ms_plain = None
    if with_compress:
        plain = lambda: pipe.run_steps(compress=False)
        g1 = None if args.no_graph else capture(plain)
        ms_plain = timed(g1.replay if g1 is not None else plain, units) / steps

    # ---- per-stage time: back-to-back launches of each stage's library call, HIP events on the
    # stream the launches go to (torch's current stream).  Each stage is one of the step's own
    # calls, plus the indexer alone (csa_index_scores launches exactly the indexer kernel the
    # step runs), so every single-kernel figure below is that kernel's launch duration.
    reps = args.stage_reps or args.steps
    i = dev
    stages = {}   # name -> (callable, kernels it launches, work key or None)
    if cfg.kind == "csa_decode":
        scores = torch.empty((cfg.batch, cfg.T, cfg.N), dtype=torch.float32, device="cuda")
        split = csa.csa_sparse_mqa_workspace_size(cfg.batch, cfg.T, cfg.H, cfg.c, cfg.k, cfg.dt) > 0
        stages["index"] = (lambda: csa.csa_index_scores(i["qI"], i["w"], i["kI"], cfg.q_pos0, cfg.m, scores=scores),
                           ["index_scores_mfma"], "index")
        stages["select"] = (pipe.select, ["index_scores_mfma", "topk"], None)
        # (decode launches have at most one workgroup per CU: the warp-specialised kernel)
        stages["attend"] = (pipe.attend, ["mqa_sparse_ws"] + (["mqa_combine"] if split else []), "mqa")
        if with_compress:   # the decode-step compression of the KV and index-key entries (one launch)
            stages["compress_step"] = (pipe.compress, ["compress_pair_kernel"], "compress_step")
    elif cfg.kind == "csa_compress":
        stages["compress"] = (pipe.run, ["compress_kernel"], "compress")
    elif cfg.kind == "csa_prefill":
        scores = torch.empty((cfg.batch, cfg.T, cfg.N), dtype=torch.float32, device="cuda")
        stages["compress_kv"] = (lambda: csa.csa_compress(i["Ca"], i["Cb"], i["Za"], i["Zb"], i["Ba"], i["Bb"], cfg.m,
                                                          out=pipe.kv), ["compress_kernel"], "compress_kv")
        stages["compress_kI"] = (lambda: csa.csa_compress(i["ICa"], i["ICb"], i["IZa"], i["IZb"], i["IBa"], i["IBb"],
                                                          cfg.m, out=pipe.kI), ["compress_kernel"], "compress_kI")
        stages["index"] = (lambda: csa.csa_index_scores(i["qI"], i["w"], pipe.kI, cfg.q_pos0, cfg.m, scores=scores),
                           ["index_scores_prefill"], "index")
        stages["select"] = (pipe.select, ["index_scores_prefill", "topk"], None)
        stages["attend"] = (pipe.attend, ["mqa_sparse_mfma"], "mqa")
    else:
        stages["compress"] = (pipe.compress, ["compress_kernel"], "compress")
        stages["attend"] = (pipe.attend, ["mqa_sparse_mfma"], "mqa")
    work = stage_work(cfg)
    stage_ms = {}
    # stages whose kernels are too short to time by launches from Python (the host would be
    # the limit): timed as a captured graph of back-to-back calls
    graph_stages = {"compress_step"}
    for name, (fn, _, _) in stages.items():
        fn()
        torch.cuda.synchronize()
        n_rep = max(3, reps if cfg.kind != "hca_chunk" else min(reps, 20))
        if name in graph_stages and not args.no_graph:
            def many(fn=fn):
                for _ in range(20):
                    fn()
            g = capture(many)
            stage_ms[name] = timed(g.replay, max(1, n_rep // 20)) / (20 * max(1, n_rep // 20))
            continue
        stage_ms[name] = timed(fn, n_rep) / n_rep
    # every stage's fraction of its own roofline (a stage of several kernels over its call
    # time; top-k alone as select - index)
    def frac(wk, t_ms):
        wv = work[wk]
        if wv["bound"] == "hbm":
            return wv["bytes"] / (t_ms * 1e-3) / HBM_PEAK
        return wv["flops"] / (t_ms * 1e-3) / peak_for(cfg, wk, "mfma")[0]

    stage_frac = {n: round(frac(wk, stage_ms[n]), 4) for n, (_, _, wk) in stages.items() if wk is not None}
    if "select" in stage_ms and "index" in stage_ms and stage_ms["select"] > stage_ms["index"]:
        stage_ms["topk (select - index)"] = stage_ms["select"] - stage_ms["index"]
        stage_frac["topk (select - index)"] = round(frac("topk", stage_ms["topk (select - index)"]), 4)
    # roofline of the dominant kernel: the longest stage that is a single kernel
    single = [n for n, (_, ks, wk) in stages.items() if len(ks) == 1 and wk is not None]
    dom = max(single, key=stage_ms.get)
    kernel, wkey = stages[dom][1][0], stages[dom][2]
    w = work[wkey]
    peak, unit = peak_for(cfg, wkey, w["bound"])
    t_s = stage_ms[dom] * 1e-3
    from long_context_sparse_08_amd.profiling import traffic_for, utilization_for
    tr = traffic_for(kernel, cfg.name)
    if w["bound"] == "hbm":
        achieved = w["bytes"] / t_s
        roof = {"bound": "hbm", "achieved": round(achieved / 1e9, 1), "peak": peak / 1e9, "unit": unit,
                "frac": round(achieved / peak, 4)}
    else:
        achieved = w["flops"] / t_s
        roof = {"bound": "mfma", "achieved": round(achieved / 1e12, 1), "peak": peak / 1e12, "unit": unit,
                "frac": round(achieved / peak, 4)}
    roof["traffic"] = None if tr is None else tr["traffic_bytes"]
    # the matrix cores' busy time from committed hardware counters (rocprofv3 MfmaUtil), for a
    # kernel bound by them; null when there is no summary for this kernel's current source
    util = utilization_for(kernel, cfg.name)
    if w["bound"] == "mfma":
        roof["mfma_util_pct"] = None if util is None or "MfmaUtil" not in util else util["MfmaUtil"]
    roof["kernel"] = kernel
    roof["ms_per_launch"] = round(stage_ms[dom], 5)
    roof["algorithmic_bytes"] = int(w["bytes"])
    roof["algorithmic_flops"] = int(w["flops"])
    # ideal step time: every stage at its roofline (the decode-step compression once every m steps)
    ideal = sum(max(v["bytes"] / HBM_PEAK, v["flops"] / peak_for(cfg, k, "mfma")[0]) / (cfg.m if k == "compress_step" else 1)
                for k, v in work.items() if k != "compress_step" or with_compress)

    result = {
        "metric": metric_for(cfg),
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {2: "bf16+fp8", 3: "bf16+mxfp4"}.get(cfg.qk_dt, "bf16"),
        "data": "synthetic (seeded SplitMix64 normals/uniforms; no dataset)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "query_tokens_per_seq": cfg.T, "q_pos0": cfg.q_pos0,
                   "entries": cfg.N, "c": cfg.c, "heads": cfg.H, "H_I": cfg.H_I, "c_I": cfg.c_I, "k": cfg.k,
                   "m": cfg.m if cfg.kind != "hca_chunk" else cfg.m_prime, "kv_dtype": DT_NAME[cfg.dt if cfg.kv_dt < 0 else cfg.kv_dt],
                   "qk_dtype": DT_NAME[cfg.qk_dt] if cfg.kind != "hca_chunk" else None,
                   "graph": graph is not None},
        "roofline": roof,
        "stage_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        "stage_roofline_frac": stage_frac,
        "stage_kernels": {k: v[1] for k, v in stages.items()},
        "step_roofline_frac": round(ideal / (ms * 1e-3), 4),
    }
    # hardware counters of the stages' kernels from committed summaries (MfmaUtil etc.)
    hw = {}
    for n, (_, ks, wk) in stages.items():
        if len(ks) == 1:
            u = utilization_for(ks[0], cfg.name)
            if u is not None:
                hw[n] = u
    if hw:
        result["stage_counters"] = hw
    if cfg.qk_dt == 3:
        # selection quality of the MXFP4 indexer: the committed record of how much of the fp8
        # oracle selection the MXFP4 oracle selection keeps on these draws (oracle-only figures)
        rec = mxfp4_recall_record()
        if rec is not None:
            result["mxfp4_recall_vs_fp8"] = rec
    if with_compress:
        # the step above includes one compression every m steps; the same steps without it
        result["ms_per_step_without_compress"] = round(ms_plain, 5)
        result["compress_ms_per_step_amortised"] = round(ms - ms_plain, 5)
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(cfg, host)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
