"""End-to-end GPU parity of one rank's hot path: metadata -> indexer + top-k -> sparse attention.

Each workload runs through the C ABI in the order and launch configuration the benchmark uses.
The oracle checks: metadata bit-exact; top-k sets bit-exact on integer-valued inputs and within
the tie band on Gaussian inputs; attention within tolerance on every checked row: end to end where
the sets match, and on the oracle's own set (the attention entry point alone) where they differ.
Full-size workloads are checked on at least 256 sampled rows, the first and last included;
reduced ones on every row or 200 evenly spread rows.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from dsa_testlib import gpu, to_dev, to_f64, assert_attn_close, check_topk_rows, SCORE_TOL, TIE_BAND

pytestmark = pytest.mark.gpu


def gpu_rank_path(wl, variant, dev, rank=None, keep_scores=False):
    """Run the rank's share through the library. Returns host copies of everything."""
    import sparse_attention_prefill_amd as D
    rank = wl.rank if rank is None else rank
    mode = 0 if wl.mode == O.IN_SEQ else 1
    inp = S.stream_inputs(wl, variant)
    qsl_d = to_dev(wl.qsl, "i32", dev)
    lens_d = to_dev(wl.seq_lens, "i32", dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    meta = D.build_cp_metadata(qsl_d, lens_d, wl.T, wl.cp, rank, mode, wl.pad, err_flag=err)
    torch.cuda.synchronize()
    tpr, n_real, _ = D.cp_sizes(wl.T, wl.cp, rank, mode, wl.pad)
    toks = meta["token_map"].cpu().numpy()[:n_real]
    qin = S.query_inputs(wl, toks, variant)
    ik = wl.idx_dtype
    max_kv = int(wl.seq_lens.max())
    cu_kv = to_dev(inp["kv_cmp_start"], "i32", dev) if wl.compress > 1 else meta["local_kv_start_loc"]
    q_idx = to_dev(qin["q_idx"], ik, dev)
    kw = dict(topk=wl.topk, q_stride=int(meta["scalars"][4].item()), compress_ratio=wl.compress,
              kv_row_base=wl.n_kv if wl.compress > 1 else 0, window=wl.window,
              window_kv_start=meta["local_kv_start_loc"] if wl.window else None,
              q_scale=to_dev(qin["q_scale"], "f32", dev) if "q_scale" in qin else None,
              k_scale=to_dev(inp["k_scale"], "f32", dev) if "k_scale" in inp else None, err_flag=err)
    w_d = to_dev(qin["w"], "f32", dev)
    k_d = to_dev(inp["k_idx"], ik, dev)
    print(f"case {wl.name} {variant} lens={wl.lens[:4]} cp={wl.cp} r={rank} K={wl.topk} nq={n_real}", flush=True)
    nbytes = D.indexer_topk_workspace(q_idx, w_d, k_d, meta["local_query_start_loc"], meta["local_seq_lens"], cu_kv,
                                      max_kv, **kw)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    idx = D.indexer_topk(q_idx, w_d, k_d, meta["local_query_start_loc"], meta["local_seq_lens"], cu_kv, max_kv,
                         workspace=ws, **kw)
    q_d, kv_d, sink_d = to_dev(qin["q"], wl.attn_dtype, dev), to_dev(inp["kv"], wl.attn_dtype, dev), \
        to_dev(inp["sink"], "f32", dev)
    out = D.sparse_attn(q_d, kv_d, idx, sink_d, 1.0 / np.sqrt(wl.Dqk), wl.Dv, err_flag=err)
    torch.cuda.synchronize()
    res = dict(meta={k: (v.cpu().numpy() if v is not None else None) for k, v in meta.items()}, err=err.item(),
               idx=idx.cpu().numpy(), out=out, toks=toks, inp=inp, qin=qin, n_real=n_real, tpr=tpr,
               q_d=q_d, kv_d=kv_d, sink_d=sink_d)
    if keep_scores:  # full score rows from the two-stage entry point (the fused call may keep none)
        vis = max_kv // wl.compress if wl.compress > 1 else max_kv
        sc = torch.empty(max(n_real, 1), (vis + 63) // 64 * 64, dtype=torch.float32, device=dev)
        D.indexer_scores(q_idx, w_d, k_d, meta["local_query_start_loc"], meta["local_seq_lens"], cu_kv, max_kv, sc,
                         **{k: v for k, v in kw.items() if k not in ("window", "window_kv_start", "kv_row_base")})
        torch.cuda.synchronize()
        res["scores_dev"] = sc
    return res


def sampled_rows(n, count):
    """count evenly spread rows of n, always with the first two and the last two."""
    return np.unique(np.concatenate([[0, 1, n - 2, n - 1], np.linspace(0, n - 1, count).astype(int)]))


def check_against_oracle(wl, variant, res, rows=None, min_same=0.99):
    m = O.cp_metadata(wl.qsl, wl.seq_lens, wl.cp, wl.rank, wl.mode, wl.pad)
    assert res["err"] == 0
    for k in ("local_query_start_loc", "local_seq_lens", "local_kv_start_loc", "token_map"):
        assert np.array_equal(res["meta"][k], m[k]), k
    n = m["n_local_real"]
    rows = list(range(n)) if rows is None else list(rows)
    ora = O.run_path(m, {**res["inp"], **{k: v for k, v in res["qin"].items()}}, wl, rows=rows, want_scores=True)
    K = wl.topk
    views = O.query_views(m)
    base = [((wl.n_kv + res["inp"]["kv_cmp_start"][views[i][0]]) if wl.compress > 1 else views[i][2]) for i in rows]
    gpu_topk = [res["idx"][i, :K] for i in rows]
    if variant == "int":
        for n_, i in enumerate(rows):
            g = gpu_topk[n_][gpu_topk[n_] >= 0]
            assert np.array_equal(g, ora["topk_ids"][n_]), f"row {i}: integer-valued top-k differs"
        same = len(rows)
    else:
        same = check_topk_rows(gpu_topk, ora["topk_ids"], ora["scores"], K, base, rows=rows,
                               delta_rel=TIE_BAND[wl.idx_dtype])
    assert same >= min_same * len(rows), f"only {same}/{len(rows)} rows with identical sets"
    if wl.window:
        for n_, i in enumerate(rows):
            w = res["idx"][i, K:]
            assert np.array_equal(w[w >= 0], ora["window_ids"][n_]), f"row {i}: window rows"
    got = to_f64(res["out"])
    keep = [n_ for n_, i in enumerate(rows)
            if np.array_equal(np.sort(gpu_topk[n_][gpu_topk[n_] >= 0]), ora["topk_ids"][n_])]
    assert_attn_close(got[[rows[k] for k in keep]], ora["out"][keep], wl.attn_dtype, wl.name)
    # rows whose sets differ (near-ties at the cut): the attention entry point alone on the oracle's set
    diff = [n_ for n_ in range(len(rows)) if n_ not in set(keep)]
    if diff:
        import sparse_attention_prefill_amd as D
        dev = res["q_d"].device
        idx_o = np.full((len(diff), wl.k_tot), -1, dtype=np.int32)
        for j, n_ in enumerate(diff):
            sel = np.concatenate([ora["topk_ids"][n_], ora["window_ids"][n_]])
            idx_o[j, :len(sel)] = sel
        q_rows = res["q_d"][torch.as_tensor([rows[n_] for n_ in diff], device=dev)].contiguous()
        o_iso = D.sparse_attn(q_rows, res["kv_d"], to_dev(idx_o, "i32", dev), res["sink_d"], 1.0 / np.sqrt(wl.Dqk),
                              wl.Dv)
        torch.cuda.synchronize()
        assert_attn_close(to_f64(o_iso), ora["out"][diff], wl.attn_dtype, f"{wl.name} (oracle's sets)")
    print(f"checked {len(rows)} rows: {same} identical top-k sets, {len(diff)} attended on the oracle's set",
          flush=True)
    return ora


REDUCED = [
    ("tiny_fp32_cp1", {}),
    ("inseq_cp8_last_8k", {"lens": (4096,)}),
    ("rr_cp8_r3_batch4", {"lens": (4400, 2600, 800, 5)}),
    ("long_131k_fp8", {"lens": (4096,)}),
    ("rr_cp4_r1_var8_cmp4", {"lens": (3000, 9001, 700, 1234)}),
    ("rr_cp4_r1_var8_cmp128", {"lens": (3000, 9001, 700, 1234)}),
    # x128 blocks with a small K, so that rows past 16 visible blocks run the selection
    ("rr_cp4_r1_var8_cmp128", {"lens": (3000, 9001, 700, 1234), "topk": 16}),
]


@pytest.mark.parametrize("name,kw", REDUCED)
def test_path_reduced_every_row(name, kw):
    dev = gpu()
    wl = S.WORKLOADS[name].with_(**kw)
    res = gpu_rank_path(wl, "normal", dev)
    n = res["n_real"]
    rows = range(n) if n <= 200 else np.unique(np.linspace(0, n - 1, 200).astype(int))
    check_against_oracle(wl, "normal", res, rows=rows)


@pytest.mark.parametrize("name,kw", REDUCED)
def test_path_integer_inputs_topk_exact(name, kw):
    dev = gpu()
    wl = S.WORKLOADS[name].with_(**kw)
    res = gpu_rank_path(wl, "int", dev)
    n = res["n_real"]
    rows = range(n) if n <= 120 else np.unique(np.linspace(0, n - 1, 120).astype(int))
    check_against_oracle(wl, "int", res, rows=rows)


@pytest.mark.parametrize("name", ["inseq_cp8_last_8k", "rr_cp8_r3_batch4", "long_131k_fp8", "rr_cp4_r1_var8_cmp4",
                                  "chunk_inseq_cp8_last_8k_p56k", "rr_cp4_r1_var8_cmp128"])
def test_path_full_size_integer_inputs_sampled(name):
    """Full-size workloads with integer-valued indexer inputs: every score is exact on both sides,
    so the top-k rows must be identical (the 131072-token rank selects from candidate lists)."""
    dev = gpu()
    wl = S.WORKLOADS[name]
    res = gpu_rank_path(wl, "int", dev)
    check_against_oracle(wl, "int", res, rows=sampled_rows(res["n_real"], 256))


@pytest.mark.parametrize("name", ["inseq_cp8_last_8k", "rr_cp8_r3_batch4", "rr_cp4_r1_var8_cmp4", "long_131k_fp8",
                                  "chunk_inseq_cp8_last_8k_p56k", "rr_cp4_r1_var8_cmp128"])
def test_path_full_size_sampled(name):
    dev = gpu()
    wl = S.WORKLOADS[name]
    res = gpu_rank_path(wl, "normal", dev, keep_scores=True)
    rows = sampled_rows(res["n_real"], 256)
    ora = check_against_oracle(wl, "normal", res, rows=rows, min_same=0.9)
    got = res.pop("scores_dev")[torch.as_tensor(rows, device=res["q_d"].device)].cpu().numpy()
    worst = 0.0
    for n_, i in enumerate(rows):  # the score rows themselves (rows the top-k keeps whole have none)
        ref = ora["scores"][n_]
        g = got[n_, :len(ref)].astype(np.float64)
        if len(ref) > wl.topk:
            dev_rel = np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-30)
            worst = max(worst, dev_rel)
            assert dev_rel <= SCORE_TOL[wl.idx_dtype], (name, i, dev_rel)
    print(f"worst score deviation / max|score|: {worst:.3e}", flush=True)


@pytest.mark.parametrize("name,kw", [("rr_cp8_r3_batch4", {"lens": (2100, 900, 300, 5), "topk": 256}),
                                     ("rr_cp4_r1_var8_cmp4", {"lens": (1500, 2222, 77, 901), "topk": 256}),
                                     ("inseq_cp8_last_8k", {"lens": (1000, 3001), "topk": 512})])
def test_all_ranks_reranged_equal_cp1_bitwise(name, kw):
    """Every rank's share run in turn, concatenated by rank and reranged == the cp = 1 run."""
    dev = gpu()
    import sparse_attention_prefill_amd as D
    wl = S.WORKLOADS[name].with_(**kw)
    mode = 0 if wl.mode == O.IN_SEQ else 1
    full = gpu_rank_path(wl.with_(cp=1, rank=0), "normal", dev)["out"]
    parts = []
    for r in range(wl.cp):
        res = gpu_rank_path(wl, "normal", dev, rank=r)
        rows = res["tpr"] if wl.pad else res["n_real"]
        part = torch.zeros(rows, wl.H, wl.Dv, dtype=res["out"].dtype, device=dev)
        part[:res["n_real"]] = res["out"]
        parts.append(part)
    concat = torch.cat(parts)
    back = D.rerange(concat.view(concat.shape[0], -1), wl.T, wl.cp, mode, wl.pad).view(wl.T, wl.H, wl.Dv)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), full.view(torch.int16))


def test_path_is_deterministic():
    dev = gpu()
    wl = S.WORKLOADS["rr_cp8_r3_batch4"].with_(lens=(3000, 1000, 17))
    a = gpu_rank_path(wl, "normal", dev)
    b = gpu_rank_path(wl, "normal", dev)
    assert np.array_equal(a["idx"], b["idx"])
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))


# Chunked prefill: every request carries a cached prefix ahead of its queries (its KV segment is
# prefix + queries long).  Reduced sizes that still span several tiles and a ragged tail.
CHUNKED = [
    ("chunk_inseq_cp8_last_8k_p56k", {"lens": (2048,), "prefix": (6000,)}),
    ("rr_cp8_r3_batch4", {"lens": (1500, 700, 130, 5), "prefix": (3000, 0, 517, 20)}),
    ("long_131k_fp8", {"lens": (2048,), "prefix": (9001,)}),
    ("rr_cp4_r1_var8_cmp4", {"lens": (1000, 2001, 300), "prefix": (4000, 3, 0)}),
]


@pytest.mark.parametrize("name,kw", CHUNKED)
def test_chunked_prefill_every_row(name, kw):
    dev = gpu()
    wl = S.WORKLOADS[name].with_(**kw)
    res = gpu_rank_path(wl, "normal", dev)
    n = res["n_real"]
    rows = range(n) if n <= 160 else np.unique(np.linspace(0, n - 1, 160).astype(int))
    # Rows of 10k+ fp8-scored keys put more near-equal scores at the cut: every differing id is
    # still checked against the tie band, only the floor on identical sets is lower.
    check_against_oracle(wl, "normal", res, rows=rows, min_same=0.95 if wl.idx_dtype == "fp8" else 0.99)


@pytest.mark.parametrize("name,kw", CHUNKED)
def test_chunked_prefill_integer_inputs_topk_exact(name, kw):
    dev = gpu()
    wl = S.WORKLOADS[name].with_(**kw)
    res = gpu_rank_path(wl, "int", dev)
    n = res["n_real"]
    rows = range(n) if n <= 100 else np.unique(np.linspace(0, n - 1, 100).astype(int))
    check_against_oracle(wl, "int", res, rows=rows)


@pytest.mark.parametrize("mode,cp,rank,pad", [(O.IN_SEQ, 4, 3, False), (O.ROUND_ROBIN, 3, 1, True)])
def test_chunked_prefill_equals_the_whole_requests_bitwise(mode, cp, rank, pad):
    """The last chunks of two requests, run after their cached prefixes on one rank, give the
    same top-k rows and the same output bits as the whole requests run at cp 1."""
    dev = gpu()
    whole = S.WORKLOADS["inseq_cp8_last_8k"].with_(lens=(3000, 1100), cp=1, rank=0, mode=O.IN_SEQ, pad=False,
                                                    topk=512)
    full = gpu_rank_path(whole, "normal", dev)
    prefix = (1900, 37)
    chunk = whole.with_(lens=(1100, 1063), prefix=prefix, cp=cp, rank=rank, mode=mode, pad=pad)
    assert list(chunk.seq_lens) == list(whole.lens)
    res = gpu_rank_path(chunk, "normal", dev)
    assert res["err"] == 0
    toks = res["toks"]
    b = np.searchsorted(chunk.qsl, toks, side="right") - 1
    whole_rows = whole.qsl[b] + np.asarray(prefix)[b] + toks - chunk.qsl[b]
    assert np.array_equal(res["idx"], full["idx"][whole_rows])
    got = res["out"].view(torch.int16).cpu().numpy()
    want = full["out"].view(torch.int16).cpu().numpy()[whole_rows]
    assert np.array_equal(got, want)
