"""Benchmark: one context-parallel rank's DSA prefill hot path on one MI355X.

A step = CP-local metadata -> lightning-indexer scores + causal top-k -> sparse MLA attention
with sink (+ the round-robin rerange of a [T, 576] bf16 buffer for workloads that have one),
through the C ABI of libdsa, on torch's current stream, inputs resident in HBM.

Default workload: the long prefill, one 131072-token sequence split contiguously over 8 ranks,
last rank: 16384 local queries over the whole 131072-token stream; 128 heads x 576/512 bf16
attention, 64 x 128 fp8 E4M3 indexer (per-token key scale, per-(token, head) query scale),
top-k 2048.

Timing protocol:
  * warm-up steps, then untimed steps back to back for --settle-ms (after an idle gap the GPU's
    clocks ramp up over the first ~40 ms of work);
  * --steps timed iterations, each preceded (outside its events) by a write of --flush-mib MiB of
    scratch, so no input or intermediate of the previous step is still in the 256 MB last-level
    cache; each iteration is bracketed by HIP events on the kernels' stream, with events between
    the ABI calls (stages) and at every kernel boundary inside the indexer + top-k call;
  * value = local queries / median step time; the minimum is reported beside it;
  * after each timed iteration (outside its events) a one-wave probe reads the shader-clock and
    100 MHz real-time counters over a 200 us spin: the graphics clock (SCLK) the step ran at;
  * separately, the whole step captured in a HIP graph and replayed back to back with no flush.

Prints ONE JSON line. --gpus N > 1 is refused: this path runs on one GPU.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
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

# kernel -> the sources its code comes from (a traffic summary is valid while their hash holds)
KERNEL_SOURCES = {
    "sparse_attn_mla_bf16": ("attention.hip", "dsa_internal.h"),
    "indexer_mfma<fp8,candidates>": ("indexer.hip", "index_score.h", "dsa_internal.h"),
    "indexer_mfma<bf16>": ("indexer.hip", "index_score.h", "dsa_internal.h"),
    "indexer_mfma<fp8>": ("indexer.hip", "index_score.h", "dsa_internal.h"),
    "indexer_mfma<bf16,candidates>": ("indexer.hip", "index_score.h", "dsa_internal.h"),
}
# kernel name as the library's timing hook reports it -> its name in a rocprofv3 trace
TRACE_NAME = {
    "indexer_mfma<fp8,candidates>": "indexer_mfma<true, true>",
    "indexer_mfma<fp8>": "indexer_mfma<true, false>",
    "indexer_mfma<bf16,candidates>": "indexer_mfma<false, true>",
    "indexer_mfma<bf16>": "indexer_mfma<false, false>",
    "sparse_attn_mla_bf16": "sparse_attn_mla_bf16",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="long_131k_fp8")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU time budget of the oracle sample")
    p.add_argument("--profile-only", action="store_true", help="no CPU baseline and no two-stage split (rocprofv3)")
    p.add_argument("--flush-mib", type=int, default=1024, help="scratch written before each timed iteration")
    p.add_argument("--settle-ms", type=float, default=150.0,
                   help="before each timed region, untimed steps run back to back for at least this long")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain copy of MIB MiB (the rerange kernel in its identity mode) three times; "
                        "its FETCH_SIZE / WRITE_SIZE counters scale the HBM traffic of the other kernels")
    p.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                   help="write profiles/traffic_<kernel>_<workload>.json from four rocprofv3 --pmc output "
                        "directories (the benchmark's FETCH_SIZE and WRITE_SIZE passes, then the copy calibration's) "
                        "and exit; --workload names the workload, --kernel the kernel")
    p.add_argument("--kernel", default=None, help="kernel of --summarize-counters (timing-hook name)")
    p.add_argument("--copy-mib", type=int, default=512, help="size of the copy calibration, for --summarize-counters")
    return p.parse_args()


def src_hash(names):
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(ROOT, "sparse_attention_prefill_amd", "csrc", n), "rb").read())
    return h.hexdigest()[:16]


def settle(run, ms):
    """Run untimed steps back to back for at least `ms` milliseconds of wall time (synchronising
    every 4 steps, so the host clock follows the GPU). Returns the number of steps run."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            run()
        n += 4
        torch.cuda.synchronize()
    return n


def short_kernel_name(name):
    """A profiler's demangled kernel name without return type, namespaces and argument list:
    'void dsa::(anonymous namespace)::indexer_mfma<true, true>(unsigned char const*, ...)' ->
    'indexer_mfma<true, true>'."""
    name = re.sub(r"^void ", "", name)
    name = re.sub(r"^dsa::\(anonymous namespace\)::", "", name)
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def summarize_counters(args):
    """profiles/traffic_<kernel>_<workload>.json from rocprofv3 --pmc CSV output directories."""
    def per_dispatch(d, counter, trace_name):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                if row.get("Counter_Name") != counter:
                    continue
                name = short_kernel_name(row.get("Kernel_Name", ""))
                if trace_name is not None and not name.startswith(trace_name):
                    continue
                key = (f, row.get("Dispatch_Id"))
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
        if not vals:
            raise SystemExit(f"no {counter} values for {trace_name} under {d}")
        return float(np.median(list(vals.values()))), len(vals)

    kname = args.kernel
    tname = TRACE_NAME[kname]
    fetch_kib, nf = per_dispatch(args.summarize_counters[0], "FETCH_SIZE", tname)
    write_kib, nw = per_dispatch(args.summarize_counters[1], "WRITE_SIZE", tname)
    cal_f, _ = per_dispatch(args.summarize_counters[2], "FETCH_SIZE", "rerange_kernel")
    cal_w, _ = per_dispatch(args.summarize_counters[3], "WRITE_SIZE", "rerange_kernel")
    copy_bytes = (args.copy_mib * (1 << 20) // 1152) * 1152
    f_factor = copy_bytes / (cal_f * 1024.0)
    w_factor = copy_bytes / (cal_w * 1024.0)
    out = {"kernel": kname, "trace_name": tname, "workload": args.workload,
           "src_sha": src_hash(KERNEL_SOURCES[kname]), "sources": list(KERNEL_SOURCES[kname]),
           "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib, "dispatches": [nf, nw],
           "copy_bytes": copy_bytes, "fetch_factor": f_factor, "write_factor": w_factor,
           "fetch_bytes": fetch_kib * 1024.0 * f_factor, "write_bytes": write_kib * 1024.0 * w_factor}
    out["bytes_per_launch"] = out["fetch_bytes"] + out["write_bytes"]
    path = os.path.join(ROOT, "profiles", f"traffic_{kname.replace('<', '_').replace('>', '').replace(',', '_')}_"
                                          f"{args.workload}.json")
    json.dump(out, open(path, "w"), indent=1)
    print(json.dumps(out))


def traffic_for(kname, workload):
    path = os.path.join(ROOT, "profiles", f"traffic_{kname.replace('<', '_').replace('>', '').replace(',', '_')}_"
                                          f"{workload}.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("src_sha") != src_hash(KERNEL_SOURCES[kname]):
        return None
    return t.get("bytes_per_launch")


def med_min(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(xs)), "min": float(xs.min()), "mean": float(xs.mean())}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "this hot path runs on one GPU: the inter-rank all-gather / all-to-all are "
                                   "out of scope, so --gpus must be 1"}))
        sys.exit(2)
    if args.summarize_counters:
        summarize_counters(args)
        return
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
    print(f"bench: workload {wl.name}: generating inputs", file=sys.stderr, flush=True)

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
    flush = torch.empty(max(args.flush_mib, 1) << 20, dtype=torch.uint8, device=dev)
    probe = torch.zeros(args.steps, 4, dtype=torch.int64, device=dev)

    N_TAP = 8

    def step(ev=None, taps=None, names=None):
        """One pass of the hot path; ev: 5 events recorded between the ABI calls; taps: events at
        the kernel boundaries inside the indexer + top-k call (their kernel names go to `names`)."""
        if ev:
            ev[0].record()
        m = D.build_cp_metadata(qsl_d, lens_d, wl.T, wl.cp, wl.rank, mode, wl.pad, err_flag=err)
        if ev:
            ev[1].record()
        cu_kv = kv_cmp if kv_cmp is not None else m["local_kv_start_loc"]
        if taps is None:
            D.indexer_topk(q_idx, w_d, k_d, m["local_query_start_loc"], m["local_seq_lens"], cu_kv, max_kv,
                           topk_idx=idx, workspace=ws, **ikw(m))
        else:
            k = D.indexer_topk_timed(q_idx, w_d, k_d, m["local_query_start_loc"], m["local_seq_lens"], cu_kv,
                                     max_kv, taps, topk_idx=idx, workspace=ws, **ikw(m))
            if names is not None:
                names[:] = k
        if ev:
            ev[2].record()
        D.sparse_attn(q_d, kv_d, idx, sink_d, scale, wl.Dv, out=out, err_flag=err)
        if ev:
            ev[3].record()
        if rr_in is not None:
            D.rerange(rr_in, wl.T, wl.cp, mode, wl.pad, out=rr_out)
        if ev:
            ev[4].record()

    print(f"bench: {n_real} local queries; warm-up", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if err.item() != 0:
        print(json.dumps({"error": f"device error flag {err.item():#x}"}))
        sys.exit(1)
    idx_eager, out_eager = idx.clone(), out.clone()

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record()  # torch creates the HIP event on its first record
        return evs

    # ---------------- timed region: flushed iterations, events per stage and per kernel --------
    K = args.steps
    step_ev = [new_events(2) for _ in range(K)]
    stage_ev = [new_events(5) for _ in range(K)]
    tap_ev = [new_events(N_TAP) for _ in range(K)]
    torch.cuda.synchronize()
    kernel_names = []
    settle_steps = settle(step, args.settle_ms)
    print("bench: timed iterations", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        flush.fill_(k % 251)              # evict the last-level cache, outside the events
        step_ev[k][0].record()
        step(stage_ev[k], tap_ev[k], kernel_names)
        step_ev[k][1].record()
        D.clock_probe(probe[k], 20000)    # 200 us, outside the events
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    mhz = np.array([D.probe_mhz(r) for r in probe.cpu().numpy()])
    if err.item() != 0:
        print(json.dumps({"error": f"device error flag {err.item():#x}"}))
        sys.exit(1)
    if not (torch.equal(idx, idx_eager) and torch.equal(out.view(torch.int16), out_eager.view(torch.int16))):
        print(json.dumps({"error": "timed steps differ from the warm-up step"}))
        sys.exit(1)
    step_ms = [e[0].elapsed_time(e[1]) for e in step_ev]
    stage_ms = {name: med_min([e[a].elapsed_time(e[b]) for e in stage_ev])
                for name, a, b in (("metadata", 0, 1), ("indexer_topk", 1, 2), ("sparse_attn", 2, 3),
                                   ("rerange", 3, 4))}
    nk = len(kernel_names)
    kernel_ms = {}
    for j, kn in enumerate(kernel_names):
        kernel_ms[f"{j}:{kn}"] = med_min([e[j].elapsed_time(e[j + 1]) for e in tap_ev])
    kernel_mean = {kn: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in tap_ev]))
                   for j, kn in enumerate(kernel_names)}
    step_stats = med_min(step_ms)

    # ---------------- back to back: the whole step in a HIP graph, no flush ---------------------
    print("bench: graph replays", file=sys.stderr, flush=True)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    settle(graph.replay, args.settle_ms)
    torch.cuda.synchronize()
    g0 = time.perf_counter()
    for _ in range(K):
        graph.replay()
    torch.cuda.synchronize()
    b2b_ms = (time.perf_counter() - g0) * 1e3 / K
    if not (torch.equal(idx, idx_eager) and torch.equal(out.view(torch.int16), out_eager.view(torch.int16))):
        print(json.dumps({"error": "graph replay differs from the eager step"}))
        sys.exit(1)
    del graph
    attn_kernel = "sparse_attn_mla_bf16" if ak == "bf16" and wl.H == 128 else "sparse_attn_generic"
    ceiling = lds_mfma_ceiling(D, dev) if attn_kernel == "sparse_attn_mla_bf16" and not args.profile_only else None

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
    pairs_scored = int(vis[vis > wl.topk].sum())     # rows with at most K keys are taken whole, unscored
    sel_topk = np.minimum(vis, wl.topk)
    sel_win = np.minimum(ext, wl.window) if wl.window else np.zeros_like(ext)
    selected = int((sel_topk + sel_win).sum())
    attn_flops = 2.0 * wl.H * (wl.Dqk + wl.Dv) * selected
    idx_flops = 2.0 * wl.Hi * wl.Di * pairs_scored
    topk_bytes = 4.0 * pairs + 4.0 * wl.k_tot * n_real
    attn_peak = PEAK_BF16_TFLOPS if ak == "bf16" else PEAK_FP32_TFLOPS
    idx_peak = {"bf16": PEAK_BF16_TFLOPS, "fp8": PEAK_FP8_TFLOPS, "f32": PEAK_FP32_TFLOPS}[ik]
    value = n_real / (step_stats["median"] * 1e-3)

    attn_ms = stage_ms["sparse_attn"]["mean"]
    idx_kernel = next((kn for kn in kernel_names if kn.startswith("indexer")), None)
    idx_ms = kernel_mean.get(idx_kernel) if idx_kernel else None

    def roof(kname, flops, ms, peak):
        ach = flops / (ms * 1e-3) / 1e12
        r = {"bound": "mfma", "kernel": kname, "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
             "traffic": traffic_for(kname, wl.name) if kname in KERNEL_SOURCES else None,
             "flops_per_launch": flops, "avg_launch_ms": ms}
        if kname.startswith("indexer") and ik == "fp8":
            r["frac_of_bf16_peak"] = ach / PEAK_BF16_TFLOPS
        return r

    roofs = [roof(attn_kernel, attn_flops, attn_ms, attn_peak)]
    if ceiling:
        # what one wave per SIMD can issue, in shader cycles, scaled by the clock the run held
        c = ceiling["mla_half_tile_1wave"] * float(np.median(mhz)) / 2400.0
        roofs[0]["lds_mfma_ceiling"] = ceiling
        roofs[0]["ceiling_frac_of_peak"] = c
        roofs[0]["frac_of_ceiling"] = roofs[0]["frac"] / c
    if idx_kernel and idx_ms:
        roofs.append(roof(idx_kernel, idx_flops, idx_ms, idx_peak))
    roofs.sort(key=lambda r: -r["avg_launch_ms"])  # the dominant kernel first

    res = {
        "metric": METRIC, "value": value, "unit": "query tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": step_stats["median"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": ak if ik == ak else f"{ak}+{ik}-indexer", "data": "synthetic",
        "timing": f"median of {K} event-timed steps (eager ABI calls on one stream), each after a "
                  f"{args.flush_mib} MiB scratch write outside its events",
        "step_ms": step_stats, "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "wall_ms_per_iteration_incl_flush_and_probe": wall_s * 1e3 / K,
        "b2b_graph": {"ms_per_step": b2b_ms, "value": n_real / (b2b_ms * 1e-3),
                      "note": "whole step captured in a HIP graph, replayed back to back, no flush"},
        "sclk": {"mhz_median": float(np.median(mhz)), "mhz_min": float(mhz.min()), "mhz_max": float(mhz.max()),
                 "source": "shader-clock counter / 100 MHz real-time counter over a 200 us probe after each step"},
        "config": {"workload": wl.name, "tokens": wl.T, "requests": len(wl.lens), "cp_size": wl.cp,
                   "cached_prefix_tokens": int(wl.n_kv - wl.T),
                   "cp_rank": wl.rank, "split": wl.mode, "padded": wl.pad, "local_queries": n_real,
                   "heads": wl.H, "d_qk": wl.Dqk, "d_v": wl.Dv, "indexer": f"{wl.Hi}x{wl.Di} {ik}", "topk": wl.topk,
                   "window": wl.window, "compress": wl.compress},
        "roofline": roofs[0],
        "roofline_secondary": roofs[1] if len(roofs) > 1 else None,
        # time the step's MFMA work would take at each kernel's own dtype peak, over the step time
        "mfma_util": {"path_peak_frac": (attn_flops / (attn_peak * 1e12) + idx_flops / (idx_peak * 1e12))
                      / (step_stats["median"] * 1e-3),
                      "sparse_attn_frac": roofs[[r["kernel"] for r in roofs].index(attn_kernel)]["frac"],
                      "indexer_frac": (idx_flops / (idx_ms * 1e-3) / 1e12 / idx_peak) if idx_ms else None},
        "stages_ms": stage_ms,
        "indexer_topk_kernels_ms": kernel_ms,
        "indexer_topk_selection": "candidate lists" if any("cand" in k for k in kernel_names) else "score rows",
        "work": {"indexer_pairs": pairs, "indexer_pairs_scored": pairs_scored, "selected_rows": selected,
                 "attn_gflop": attn_flops / 1e9, "indexer_gflop": idx_flops / 1e9, "topk_mbytes": topk_bytes / 1e6},
        "note": "the pages publish no throughput figures for this path",
    }
    if nk >= N_TAP - 1:
        res["note_kernels"] = f"the call launched more than {N_TAP - 1} kernels; later ones are unbracketed"
    topk_kernels = [k for k in kernel_ms if "topk" in k]
    if res["indexer_topk_selection"] == "score rows" and topk_kernels:
        tk = kernel_ms[topk_kernels[0]]["median"]
        res["topk_hbm_frac"] = topk_bytes / (tk * 1e-3) / 1e9 / PEAK_HBM_GBS
    if wl.rerange:
        rr_bytes = 2.0 * wl.T * wl.Dqk * 2
        res["rerange_hbm_frac"] = rr_bytes / (stage_ms["rerange"]["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS

    # ---------------- CPU baseline: the oracle on a bounded sample of the same work -------------
    if not args.no_cpu_baseline and not args.profile_only:
        print("bench: CPU baseline (oracle sample)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, inp, qin, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def lds_mfma_ceiling(D, dev, iters=200):
    """MFMA busy fraction one SIMD reaches when its 32x32x16 bf16 MFMAs take their A operand from
    LDS in the MLA kernel's K form (one 16-byte read) or V form (two transposed 8-byte reads), with
    one or two waves per SIMD (the library's LDS-fed MFMA probe); mla_half_tile_1wave weighs the
    two forms as one half-tile of the kernel does (36 logit MFMAs, 32 P.V MFMAs)."""
    import torch
    cyc = torch.zeros(2048, dtype=torch.int64, device=dev)
    sink = torch.empty(256 * 512, dtype=torch.float32, device=dev)
    out = {}
    for name, op in (("k_form", 0), ("v_form", 1), ("registers", 2)):
        for w in (1, 2):
            D.lds_mfma_probe(op, w, iters, cyc, sink)
            torch.cuda.synchronize()
            out[f"{name}_{w}wave"] = round(D.lds_mfma_busy(cyc.cpu().numpy(), w, iters), 4)
    out["mla_half_tile_1wave"] = round(68.0 / (36.0 / out["k_form_1wave"] + 32.0 / out["v_form_1wave"]), 4)
    return out


def cpu_baseline(wl, inp, qin, budget_s):
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
        chunk = order[done:done + 8]
        O.run_path(m, {**inp, **qin}, wl, rows=chunk)
        done += len(chunk)
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "query tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {n} local queries (random, seed 0), 8 per oracle call: float64 indexer + top-k + "
                      f"sparse attention, {dt:.1f} s"}


if __name__ == "__main__":
    main()
