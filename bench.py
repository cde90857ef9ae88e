"""Benchmark: one context-parallel rank's DSA prefill hot path on one MI355X.

A step = CP-local metadata -> lightning-indexer scores + causal top-k -> sparse MLA attention
with sink (+ the round-robin rerange of a [T, 576] bf16 buffer for workloads that have one),
through the C ABI of libdsa, on torch's current stream, inputs resident in HBM.

Default workload: contiguous split, cp 8, last rank: 1024 local queries over an 8192-token
KV stream; 128 heads x 576/512 bf16 attention, 64 x 128 bf16 indexer, top-k 2048.

Before each timed region the step runs untimed, back to back, for --settle-ms (150 ms): after an
idle gap the GPU's clocks ramp up over the first ~40 ms of work (steps run up to 15% slower), and
the figures reported are the sustained ones.

Prints ONE JSON line (rank 0). --gpus N > 1 is refused: this path runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill query tokens/sec per rank (indexer+top-k+sparse attn) + MFMA util"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32
PEAK_HBM_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="inseq_cp8_last_8k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU time budget of the oracle sample")
    p.add_argument("--profile-only", action="store_true", help="no CPU baseline, fewer prints (for rocprofv3)")
    p.add_argument("--no-graph", action="store_true", help="time eager ABI calls instead of a captured HIP graph")
    p.add_argument("--settle-ms", type=float, default=150.0,
                   help="before each timed region, untimed steps run back to back for at least this long: after "
                        "an idle gap the GPU's clocks ramp up over the first ~40 ms of work, and the figures "
                        "reported are the sustained ones")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain copy of MIB MiB (the rerange kernel in its identity mode) three times; "
                        "its FETCH_SIZE / WRITE_SIZE counters scale the HBM traffic of the other kernels")
    return p.parse_args()


def settle(run, ms):
    """Run untimed steps back to back for at least `ms` milliseconds of wall time (synchronising
    every 8 steps, so the host clock follows the GPU). Returns the number of steps run."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            run()
        n += 8
        torch.cuda.synchronize()
    return n


def src_hash(name):
    path = os.path.join(ROOT, "sparse_attention_prefill_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this hot path runs on one GPU: the inter-rank all-gather / all-to-all are "
                                   "out of scope, so --gpus must be 1"}))
        sys.exit(2)
    import torch
    import sparse_attention_prefill_amd as D
    import synthetic as S

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n // 1152, 576, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            D.rerange(src, src.shape[0], 1, 0, False, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel() * 2, "launches": 3}))
        return
    wl = S.WORKLOADS[args.workload]
    mode = 0 if wl.mode == "in_seq" else 1

    # ---------------- setup (untimed): inputs for the rank's tokens, resident in HBM -------------
    qsl_d = torch.tensor(wl.qsl, dtype=torch.int32, device=dev)
    lens_d = torch.tensor(wl.seq_lens, dtype=torch.int32, device=dev)
    tpr, n_real, rows_concat = D.cp_sizes(wl.T, wl.cp, wl.rank, mode, wl.pad)
    meta0 = D.build_cp_metadata(qsl_d, lens_d, wl.T, wl.cp, wl.rank, mode, wl.pad)
    torch.cuda.synchronize()
    toks = meta0["token_map"].cpu().numpy()[:n_real]
    inp = S.stream_inputs(wl)
    qin = S.query_inputs(wl, toks)

    def dev_t(a, kind):
        a = np.ascontiguousarray(a)
        if kind == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        if kind == "fp8":
            return torch.from_numpy(a).to(dev)
        if kind == "f32":
            return torch.from_numpy(a.astype(np.float32)).to(dev)
        return torch.from_numpy(a.astype(np.int32)).to(dev)

    ik, ak = wl.idx_dtype, wl.attn_dtype
    q_idx, w_d, k_d = dev_t(qin["q_idx"], ik), dev_t(qin["w"], "f32"), dev_t(inp["k_idx"], ik)
    q_scale = dev_t(qin["q_scale"], "f32") if "q_scale" in qin else None
    k_scale = dev_t(inp["k_scale"], "f32") if "k_scale" in inp else None
    q_d, kv_d, sink_d = dev_t(qin["q"], ak), dev_t(inp["kv"], ak), dev_t(inp["sink"], "f32")
    kv_cmp = dev_t(inp["kv_cmp_start"], "i32") if wl.compress > 1 else None
    max_kv = int(wl.seq_lens.max())
    scale = 1.0 / np.sqrt(wl.Dqk)
    # outputs / workspace, allocated once
    meta = {k: torch.empty_like(v) if v is not None else None for k, v in meta0.items()}
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    idx = torch.empty(n_real, wl.k_tot, dtype=torch.int32, device=dev)
    out = torch.empty(n_real, wl.H, wl.Dv, dtype=q_d.dtype, device=dev)
    stride = wl.cp if wl.mode == "round_robin" else 1

    def ikw(m):
        return dict(topk=wl.topk, q_stride=stride, compress_ratio=wl.compress, kv_row_base=wl.n_kv if wl.compress > 1 else 0,
                    window=wl.window, window_kv_start=m["local_kv_start_loc"] if wl.window else None,
                    q_scale=q_scale, k_scale=k_scale, err_flag=err)

    cu_kv0 = kv_cmp if kv_cmp is not None else meta0["local_kv_start_loc"]
    ws_bytes = D.indexer_topk_workspace(q_idx, w_d, k_d, meta0["local_query_start_loc"], meta0["local_seq_lens"],
                                        cu_kv0, max_kv, **ikw(meta0))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    rr_in = rr_out = None
    if wl.rerange:
        rr_in = dev_t(S.rerange_buffer(wl, rows_concat).view(np.uint16), "bf16")
        rr_out = torch.empty(wl.T, wl.Dqk, dtype=torch.bfloat16, device=dev)

    L = D.lib()
    import ctypes

    def step(ev=None):
        """One pass of the hot path; ev: list of events to record between the ABI calls."""
        if ev:
            ev[0].record()
        m = D.build_cp_metadata(qsl_d, lens_d, wl.T, wl.cp, wl.rank, mode, wl.pad, err_flag=err)
        if ev:
            ev[1].record()
        cu_kv = kv_cmp if kv_cmp is not None else m["local_kv_start_loc"]
        D.indexer_topk(q_idx, w_d, k_d, m["local_query_start_loc"], m["local_seq_lens"], cu_kv, max_kv,
                       topk_idx=idx, workspace=ws, **ikw(m))
        if ev:
            ev[2].record()
        D.sparse_attn(q_d, kv_d, idx, sink_d, scale, wl.Dv, out=out, err_flag=err)
        if ev:
            ev[3].record()
        if rr_in is not None:
            D.rerange(rr_in, wl.T, wl.cp, mode, wl.pad, out=rr_out)
        if ev:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if err.item() != 0:
        print(json.dumps({"error": f"device error flag {err.item():#x}"}))
        sys.exit(1)
    idx_eager, out_eager = idx.clone(), out.clone()

    # The step is captured once into a HIP graph (every kernel of the path, in order, on one
    # stream) and replayed, so host launch overhead does not sit between the kernels. Each replay
    # of the timed region is checked bitwise against the eager step (the path is deterministic).
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

    def run_step():
        if graph is not None:
            graph.replay()
        else:
            step()

    # ---------------- timed region ------------------------------------------------------------
    settle_steps = settle(run_step, args.settle_ms)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    if graph is not None and not (torch.equal(idx, idx_eager) and torch.equal(out.view(torch.int16),
                                                                          out_eager.view(torch.int16))):
        print(json.dumps({"error": "graph replay differs from the eager step"}))
        sys.exit(1)

    # per-ABI-call durations (HIP events on the kernels' stream, eager calls, same work)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    settle(step, args.settle_ms)
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    stage = {name: float(np.mean([e[a].elapsed_time(e[b]) for e in evs]))
             for name, a, b in (("metadata", 0, 1), ("indexer_topk", 1, 2), ("sparse_attn", 2, 3), ("rerange", 3, 4))}

    # Stage split through the two-stage entry points (indexer score rows, then top-k over them) on a
    # score matrix of their own. For rows longer than max(32768, K) the fused call above selects
    # from candidate lists instead, so there indexer_topk is not the sum of these two.
    vis_max = max_kv // wl.compress if wl.compress > 1 else max_kv
    scores = torch.empty(max(n_real, 1), (vis_max + 63) // 64 * 64, dtype=torch.float32, device=dev)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    reps = max(3, args.steps // 2)
    split_ms = {"indexer": [], "topk": []}
    for _ in range(reps):
        e[0].record()
        D.indexer_scores(q_idx, w_d, k_d, meta0["local_query_start_loc"], meta0["local_seq_lens"], cu_kv0, max_kv,
                         scores, **ikw(meta0))
        e[1].record()
        D.topk_from_scores(q_idx, w_d, k_d, meta0["local_query_start_loc"], meta0["local_seq_lens"], cu_kv0, max_kv,
                           scores, topk_idx=idx, **ikw(meta0))
        e[2].record()
        torch.cuda.synchronize()
        split_ms["indexer"].append(e[0].elapsed_time(e[1]))
        split_ms["topk"].append(e[1].elapsed_time(e[2]))
    indexer_ms = float(np.mean(split_ms["indexer"]))
    topk_ms = float(np.mean(split_ms["topk"]))

    # ---------------- algorithmic work (per launch) ---------------------------------------------
    m = {k: (v.cpu().numpy() if v is not None else None) for k, v in meta0.items()}
    lqsl, lsl = m["local_query_start_loc"], m["local_seq_lens"]
    ext = []
    for b in range(len(wl.lens)):
        nb = int(lqsl[b + 1] - lqsl[b])
        ext += [int(lsl[b]) - (nb - 1 - j) * stride for j in range(nb)]
    ext = np.asarray(ext, dtype=np.int64)
    vis = ext // wl.compress if wl.compress > 1 else ext
    pairs = int(vis.sum())
    sel_topk = np.minimum(vis, wl.topk)
    sel_win = np.minimum(ext, wl.window) if wl.window else np.zeros_like(ext)
    selected = int((sel_topk + sel_win).sum())
    attn_flops = 2.0 * wl.H * (wl.Dqk + wl.Dv) * selected
    idx_flops = 2.0 * wl.Hi * wl.Di * pairs
    topk_bytes = 4.0 * pairs + 4.0 * wl.k_tot * n_real
    attn_s = stage["sparse_attn"] * 1e-3
    attn_peak = PEAK_BF16_TFLOPS if ak == "bf16" else PEAK_FP32_TFLOPS
    idx_peak = {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS, "f32": PEAK_FP32_TFLOPS}[ik]
    path_s = (stage["metadata"] + stage["indexer_topk"] + stage["sparse_attn"]) * 1e-3
    tokens_per_s = n_real / (ms_per_step * 1e-3)

    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_sparse_attn_mla_bf16_{wl.name}.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile))
        if t.get("attention_hip_sha") == src_hash("attention.hip"):
            traffic = t.get("bytes_per_launch")

    roofline = {"bound": "mfma", "kernel": "sparse_attn_mla_bf16" if ak == "bf16" else "sparse_attn_generic",
                "achieved": attn_flops / attn_s / 1e12, "peak": attn_peak, "unit": "TFLOP/s",
                "frac": attn_flops / attn_s / 1e12 / attn_peak, "traffic": traffic,
                "flops_per_launch": attn_flops, "avg_launch_ms": stage["sparse_attn"]}

    res = {
        "metric": METRIC, "value": tokens_per_s, "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": {"ms": args.settle_ms, "steps": settle_steps}, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": ak if ik == ak else f"{ak}+{ik}-indexer", "data": "synthetic",
        "timing": "HIP graph replay of the whole step" if graph is not None else "eager ABI calls",
        "config": {"workload": wl.name, "tokens": wl.T, "requests": len(wl.lens), "cp_size": wl.cp,
                   "cached_prefix_tokens": int(wl.n_kv - wl.T),
                   "cp_rank": wl.rank, "split": wl.mode, "padded": wl.pad, "local_queries": n_real,
                   "heads": wl.H, "d_qk": wl.Dqk, "d_v": wl.Dv, "indexer": f"{wl.Hi}x{wl.Di} {ik}", "topk": wl.topk,
                   "window": wl.window, "compress": wl.compress},
        "roofline": roofline,
        "mfma_util": {"path_bf16_peak_frac": (attn_flops + idx_flops) / path_s / 1e12 / PEAK_BF16_TFLOPS,
                      "sparse_attn_frac": attn_flops / attn_s / 1e12 / attn_peak,
                      "indexer_frac": idx_flops / (indexer_ms * 1e-3) / 1e12 / idx_peak},
        "stages_ms": {**stage, "indexer": indexer_ms, "topk": topk_ms},
        "indexer_topk_selection": "candidate lists" if vis_max > max(98304, wl.topk) else "score rows",
        "topk_hbm_frac": topk_bytes / (topk_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "work": {"indexer_pairs": pairs, "selected_rows": selected, "attn_gflop": attn_flops / 1e9,
                 "indexer_gflop": idx_flops / 1e9, "topk_mbytes": topk_bytes / 1e6},
        "note": "the pages publish no throughput figures for this path",
    }
    if wl.rerange:
        rr_bytes = 2.0 * wl.T * wl.Dqk * 2
        res["rerange_hbm_frac"] = rr_bytes / (stage["rerange"] * 1e-3) / 1e9 / PEAK_HBM_GBS

    # ---------------- CPU baseline: the oracle on a bounded sample of the same work -------------
    if not args.no_cpu_baseline and not args.profile_only:
        res["cpu_baseline"] = cpu_baseline(wl, m, inp, qin, args.cpu_seconds)
    print(json.dumps(res))


def cpu_baseline(wl, meta_np, inp, qin, budget_s):
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    m = O.cp_metadata(wl.qsl, wl.seq_lens, wl.cp, wl.rank, wl.mode, wl.pad)
    n = m["n_local_real"]
    order = np.random.default_rng(0).permutation(n)
    done = 0
    t0 = time.perf_counter()
    while done < n and (time.perf_counter() - t0 < budget_s or done < 4):
        chunk = order[done:done + 4]
        O.run_path(m, {**inp, **qin}, wl, rows=chunk)
        done += len(chunk)
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "query tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {n} local queries (random, seed 0): float64 indexer + top-k + sparse attention, "
                      f"{dt:.1f} s"}


if __name__ == "__main__":
    main()
