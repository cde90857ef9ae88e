"""GPU parity of each kernel in isolation, on inputs the oracle also sees.

  top-k (3):     same fp32 score rows -> identical ascending id lists (bit-exact)
  indexer (2):   same stored q/k/w -> scores within fp32 rounding; exact on integer inputs
  attention (4): same index sets -> outputs within the attention tolerance
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from dsa_testlib import gpu, to_dev, to_f64, assert_attn_close, SCORE_TOL

pytestmark = pytest.mark.gpu


def _meta_dev(lens, cp, rank, mode, dev):
    qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    m = O.cp_metadata(qsl, lens, cp, rank, mode, False)
    d = {k: to_dev(m[k], "i32", dev) for k in ("local_query_start_loc", "local_seq_lens", "local_kv_start_loc")}
    return m, d


def _run_topk(scores, m, d, K, dev, ratio=1, window=0, win_start=None, kv_row_base=0, nk=None):
    """Top-k of given score rows. The indexer inputs are unused placeholders, except that k_idx
    has the nk rows (default: the KV stream's) every row's extent must fit, as for the indexer."""
    import sparse_attention_prefill_amd as D
    nq = m["n_local_real"]
    ld = scores.shape[1]
    max_kv = int(m["local_seq_lens"].max())
    nk = max(1, int(m["local_kv_start_loc"][-1]) if nk is None else nk)
    dummy_q = torch.zeros(nq, 1, 8, dtype=torch.float32, device=dev)
    dummy_k = torch.zeros(nk, 8, dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dummy_w = torch.zeros(nq, 1, dtype=torch.float32, device=dev)
    out = D.topk_from_scores(dummy_q, dummy_w, dummy_k, d["local_query_start_loc"], d["local_seq_lens"],
                             d["local_kv_start_loc"], max_kv, to_dev(scores, "f32", dev), topk=K,
                             q_stride=m["stride"], compress_ratio=ratio, window=window,
                             window_kv_start=win_start, kv_row_base=kv_row_base, err_flag=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    return out.cpu().numpy()


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "const", "narrow"])
@pytest.mark.parametrize("lens,cp,rank,K", [
    # at most 1024 rows: keys in registers
    ([700], 1, 0, 64),              # E = 1..700, short rows take everything; 256 x 16
    ([6000], 6, 5, 2048),           # 4096 < E <= 6000: 512 x 16 in registers
    ([9000], 9, 8, 2048),           # 8192 < E <= 9000: 1024 x 16 in registers
    ([20000], 30, 29, 2048),        # E ~ 20000: 1024 x 32 in registers, two workgroups per CU
    ([30000], 200, 199, 2048),      # E ~ 30000: 1024 x 32 in registers
    ([3000], 1, 0, 2048),           # 3000 rows, E crosses K: rows of up to 4096 keys stay in registers
    # more than 1024 rows of more than 4096 keys: the sampled kernel
    ([6000], 3, 2, 2048),           # 2000 rows, rows of up to 3584 keys are their own list, longer sampled
    ([9000], 8, 7, 2048),           # 1125 rows of 7876 .. 9000 keys
    ([30000], 16, 15, 2048),        # 1875 rows (more than four per CU): the sampled kernel; rows
                                    # of up to 3584 keys are their own list, longer rows are sampled
                                    # ("ties", "const" and "narrow" overflow the list: exact select
                                    # over the row); checked on 300 rows
    ([3300, 9000], 2, 1, 2048),     # 6150 rows, sampled kernel, two requests
    ([40000], 4000, 3999, 2048),    # E ~ 40000: streamed; "ties", "const" and "narrow" overflow the
                                    # candidate list and refine over the row itself
    ([131072], 16384, 16383, 2048), # E ~ 131072: streamed path, longest rows
    ([50, 1, 300], 3, 1, 7),        # several requests, round-robin below
])
def test_topk_bit_exact(kind, lens, cp, rank, K):
    dev = gpu()
    for mode in (O.IN_SEQ, O.ROUND_ROBIN):
        m, d = _meta_dev(lens, cp, rank, mode, dev)
        views = O.query_views(m)
        if not views:
            continue
        ld = (max(E for _, E, _ in views) + 3) // 4 * 4
        scores = S.score_rows(len(lens) * 1000 + K, len(views), ld, kind)
        got = _run_topk(scores, m, d, K, dev)
        check = range(len(views)) if len(views) <= 2200 else np.unique(np.linspace(0, len(views) - 1, 300).astype(int))
        for i in check:
            b, E, kv0 = views[i]
            want = kv0 + O.topk_positions(scores[i, :E], K)
            row = got[i]
            assert np.array_equal(row[:len(want)], want), (kind, i, E)
            assert np.all(row[len(want):] == -1)


def test_topk_compressed_and_window():
    """x4-compressed keys (Ev = floor(E/4)) plus the 128-token window, round-robin, padded rank."""
    dev = gpu()
    lens = [700, 9, 3, 1300]
    qsl = np.concatenate([[0], np.cumsum(lens)])
    T = int(qsl[-1])
    m, d = _meta_dev(lens, 4, 1, O.ROUND_ROBIN, dev)
    ccs = np.concatenate([[0], np.cumsum([l // 4 for l in lens])]).astype(np.int32)
    d["local_kv_start_loc"] = to_dev(ccs, "i32", dev)
    views = O.query_views(m)
    ld = (max(E // 4 for _, E, _ in views) + 4) // 4 * 4
    scores = S.score_rows(77, len(views), ld, "ties")
    K = 64
    got = _run_topk(scores, m, d, K, dev, ratio=4, window=128, win_start=to_dev(qsl, "i32", dev), kv_row_base=T,
                    nk=int(ccs[-1]))
    for i, (b, E, _) in enumerate(views):
        want = T + ccs[b] + O.topk_positions(scores[i, :E // 4], K)
        assert np.array_equal(got[i, :len(want)], want) and np.all(got[i, len(want):K] == -1), i
        win = qsl[b] + O.window_positions(E, 128)
        assert np.array_equal(got[i, K:K + len(win)], win) and np.all(got[i, K + len(win):] == -1), i


def _indexer_case(wl, variant, dev, rows_cap=None):
    import sparse_attention_prefill_amd as D
    m = O.cp_metadata(wl.qsl, wl.seq_lens, wl.cp, wl.rank, wl.mode, wl.pad)
    toks = m["token_map"][m["token_map"] >= 0]
    inp = S.stream_inputs(wl, variant)
    qin = S.query_inputs(wl, toks, variant)
    kind = {"f32": "f32", "bf16": "bf16", "fp8": "fp8"}[wl.idx_dtype]
    cu_kv = inp["kv_cmp_start"] if wl.compress > 1 else m["local_kv_start_loc"]
    max_kv = int(m["local_seq_lens"].max())
    ev_max = max_kv // wl.compress if wl.compress > 1 else max_kv
    ld = (ev_max + 63) // 64 * 64
    nq = len(toks)
    scores = torch.full((nq, ld), float("nan"), dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    D.indexer_scores(to_dev(qin["q_idx"], kind, dev), to_dev(qin["w"], "f32", dev), to_dev(inp["k_idx"], kind, dev),
                     to_dev(m["local_query_start_loc"], "i32", dev), to_dev(m["local_seq_lens"], "i32", dev),
                     to_dev(cu_kv, "i32", dev), max_kv, scores, q_stride=m["stride"], compress_ratio=wl.compress,
                     q_scale=to_dev(qin["q_scale"], "f32", dev) if "q_scale" in qin else None,
                     k_scale=to_dev(inp["k_scale"], "f32", dev) if "k_scale" in inp else None, err_flag=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    got = scores.cpu().numpy()
    k_hat = O.dequant_k(inp["k_idx"], inp.get("k_scale"), wl.idx_dtype)
    views = O.query_views(m)
    rows = range(nq) if rows_cap is None else np.unique(np.linspace(0, nq - 1, rows_cap).astype(int))
    for i in rows:
        b, E, kv0 = views[i]
        q_hat = O.dequant_q(qin["q_idx"][i], qin["q_scale"][i] if "q_scale" in qin else None, wl.idx_dtype)
        if wl.compress > 1:
            ev = E // wl.compress
            ref = O.indexer_scores_row(q_hat, qin["w"][i], k_hat[cu_kv[b]:cu_kv[b] + ev])
        else:
            ev = E
            ref = O.indexer_scores_row(q_hat, qin["w"][i], k_hat[kv0:kv0 + E])
        g = got[i, :ev].astype(np.float64)
        if ev == 0:
            continue
        if variant == "int":
            assert np.array_equal(g, ref), (wl.name, i)
            assert not np.any(np.signbit(g[g == 0])), "negative zero score"
        else:
            tol = SCORE_TOL[wl.idx_dtype] * max(np.abs(ref).max(), 1e-30)
            assert np.abs(g - ref).max() <= tol, (wl.name, i, np.abs(g - ref).max(), tol)


@pytest.mark.parametrize("variant", ["normal", "int"])
@pytest.mark.parametrize("name,kw", [
    ("tiny_fp32_cp1", {}),
    ("inseq_cp8_last_8k", {"lens": (3000,)}),
    ("rr_cp8_r3_batch4", {"lens": (1500, 700, 130, 5)}),
    ("long_131k_fp8", {"lens": (3000,)}),
    ("rr_cp4_r1_var8_cmp4", {"lens": (1100, 1900, 13, 640)}),
    # groups of 8 queries that straddle a request boundary: their union key range is longer than
    # any single range and ends just past a multiple of the 2048-key chunk
    ("inseq_cp8_last_8k", {"lens": (2046, 3), "cp": 2, "rank": 1}),
    ("long_131k_fp8", {"lens": (2045, 50), "cp": 8, "rank": 7}),
    # chunked prefill: queries start deep into their request's KV segment
    ("chunk_inseq_cp8_last_8k_p56k", {"lens": (1500,), "prefix": (3333,), "cp": 2, "rank": 0}),
    ("rr_cp8_r3_batch4", {"lens": (700, 130, 5), "prefix": (2500, 1, 90)}),
    ("long_131k_fp8", {"lens": (1000, 9), "prefix": (5000, 4100), "cp": 2, "rank": 1}),
    # x128-compressed keys: whole 128-token blocks become visible one at a time
    ("rr_cp4_r1_var8_cmp128", {"lens": (5000, 300, 17000)}),
])
def test_indexer_scores(name, kw, variant):
    dev = gpu()
    _indexer_case(S.WORKLOADS[name].with_(**kw), variant, dev)


# Scaling every weight by 2^k scales every score by exactly 2^k (each step of the score's
# arithmetic commutes with a power-of-two scale while nothing over- or underflows: the halved
# weights, the head sums, fp8's split c = sum_h (w_h/2) q_h and its scale exponent, the final FMA),
# so the GPU scores must match bit for bit and the candidate-list ids must not move. The scales
# reach magnitudes the Gaussian cases never do, where a wrong exponent or clamp in the split of c
# would show.
@pytest.mark.parametrize("name,kw", [
    ("long_131k_fp8", {"lens": (3000,)}),
    ("long_131k_fp8", {"lens": (100000,)}),          # candidate lists (rows > 98 304 keys)
    ("inseq_cp8_last_8k", {"lens": (3000,)}),        # bf16
])
def test_indexer_scores_scale_exactly_with_the_weights(name, kw):
    import sparse_attention_prefill_amd as D
    dev = gpu()
    wl = S.WORKLOADS[name].with_(**kw)
    m = O.cp_metadata(wl.qsl, wl.seq_lens, wl.cp, wl.rank, wl.mode, wl.pad)
    toks = m["token_map"][m["token_map"] >= 0]
    inp = S.stream_inputs(wl, "normal")
    qin = S.query_inputs(wl, toks, "normal", indexer_only=True)
    kind = wl.idx_dtype
    max_kv = int(m["local_seq_lens"].max())
    ld = (max_kv + 63) // 64 * 64
    base = [to_dev(qin["q_idx"], kind, dev), None, to_dev(inp["k_idx"], kind, dev),
            to_dev(m["local_query_start_loc"], "i32", dev), to_dev(m["local_seq_lens"], "i32", dev),
            to_dev(m["local_kv_start_loc"], "i32", dev), max_kv]
    kw_ = dict(q_stride=m["stride"],
               q_scale=to_dev(qin["q_scale"], "f32", dev) if "q_scale" in qin else None,
               k_scale=to_dev(inp["k_scale"], "f32", dev) if "k_scale" in inp else None)
    w = qin["w"].astype(np.float32)
    nq = len(toks)
    rows = np.arange(nq) if nq <= 512 else np.unique(np.concatenate([np.arange(32), np.arange(nq - 32, nq),
                                                                      np.linspace(0, nq - 1, 64).astype(int)]))
    sel = torch.from_numpy(rows).to(dev)
    res = {}
    for k in (0, -40, 40):
        args = list(base)
        args[1] = to_dev(np.ldexp(w, k).astype(np.float32), "f32", dev)
        scores = torch.empty(nq, ld, dtype=torch.float32, device=dev)
        D.indexer_scores(*args, scores, **kw_)
        ids = D.indexer_topk(*args, topk=wl.topk, **kw_)
        torch.cuda.synchronize()
        res[k] = (scores[sel].cpu().numpy(), ids.cpu().numpy())
        del scores
    views = O.query_views(m)
    for k in (-40, 40):
        for n, i in enumerate(rows):
            E = views[i][1]
            assert np.array_equal(res[k][0][n, :E], np.ldexp(res[0][0][n, :E], k)), (name, k, int(i))
        assert np.array_equal(res[k][1], res[0][1]), (name, k)


# Head dimensions that take the generic indexer's other paths: not a multiple of 4 or over 64
# (key rows re-read per head), 48 (held in registers, a 64-slot row with the tail unused), and
# bf16 rows of 64 read 4 elements at a time.
@pytest.mark.parametrize("Hi,Di,kind", [(4, 30, "f32"), (2, 100, "f32"), (4, 48, "f32"), (8, 64, "bf16")])
def test_generic_indexer_shapes(Hi, Di, kind):
    wl = S.WORKLOADS["tiny_fp32_cp1"].with_(lens=(300,), Hi=Hi, Di=Di, idx_dtype=kind)
    _indexer_case(wl, "normal", gpu())


def _rand_idx(g, nq, k_tot, n_rows, frac_missing=0.1, empty_rows=()):
    idx = g.integers(0, n_rows, size=(nq, k_tot)).astype(np.int32)
    idx[g.random((nq, k_tot)) < frac_missing] = -1
    for r in empty_rows:
        idx[r] = -1
    return idx


@pytest.mark.parametrize("variant", ["normal", "unit"])
@pytest.mark.parametrize("name,nq,k_tot,n_rows", [
    ("tiny_fp32_cp1", 37, 64, 512),
    ("tiny_fp32_cp1", 5, 100, 300),
    ("inseq_cp8_last_8k", 24, 2048, 8192),
    ("inseq_cp8_last_8k", 9, 2176, 5000),
    ("inseq_cp8_last_8k", 7, 100, 130),
    ("inseq_cp8_last_8k", 4, 1, 3),
])
def test_attention_on_given_sets(name, nq, k_tot, n_rows, variant):
    _attention_case(S.WORKLOADS[name].with_(lens=(n_rows,)), nq, k_tot, n_rows, variant)


# Shapes that take the generic kernel's other load paths: a head dimension that is not a multiple
# of 4 (element loads, zeroed pad columns), bf16 rows loaded 4 elements at a time, and the largest
# head dimension the kernel accepts (a tile's loads fill every slot of the per-thread batch).
@pytest.mark.parametrize("H,Dqk,Dv,dtype", [(8, 70, 64, "f32"), (16, 160, 128, "bf16"), (8, 512, 256, "f32")])
def test_generic_attention_shapes(H, Dqk, Dv, dtype):
    wl = S.WORKLOADS["tiny_fp32_cp1"].with_(lens=(300,), H=H, Dqk=Dqk, Dv=Dv, attn_dtype=dtype)
    _attention_case(wl, 11, 70, 300, "normal")


def _attention_case(wl, nq, k_tot, n_rows, variant):
    dev = gpu()
    import sparse_attention_prefill_amd as D
    name = wl.name
    inp = S.stream_inputs(wl, variant)
    qin = S.query_inputs(wl, np.arange(nq) * 7 % n_rows, variant)
    g = np.random.default_rng(nq * 1000 + k_tot)
    idx = _rand_idx(g, nq, k_tot, n_rows, empty_rows=(nq - 1,) if nq > 2 else ())
    scale = 1.0 / np.sqrt(wl.Dqk)
    kind = wl.attn_dtype
    lse = torch.empty(nq, wl.H, dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    out = D.sparse_attn(to_dev(qin["q"], kind, dev), to_dev(inp["kv"], kind, dev), to_dev(idx, "i32", dev),
                        to_dev(inp["sink"], "f32", dev), scale, wl.Dv, lse=lse, err_flag=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    kv = O.decode(inp["kv"], kind)
    sink = inp["sink"].astype(np.float64)
    ref = np.zeros((nq, wl.H, wl.Dv))
    ref_lse = np.zeros((nq, wl.H))
    for i in range(nq):
        sel = idx[i][idx[i] >= 0]
        ref[i], ref_lse[i] = O.sparse_attention_row(O.decode(qin["q"][i], kind), kv[sel], sink, scale, wl.Dv)
    assert_attn_close(to_f64(out), ref, kind, f"{name} {variant}")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() < (1e-4 if kind == "f32" else 2e-3)


def test_attention_every_key_is_dense_causal():
    """Index sets = all positions 0..t: the sparse kernel reproduces dense causal attention."""
    dev = gpu()
    import sparse_attention_prefill_amd as D
    T = 70
    wl = S.WORKLOADS["inseq_cp8_last_8k"].with_(lens=(T,))
    inp = S.stream_inputs(wl, "unit")
    qin = S.query_inputs(wl, np.arange(T), "unit")
    idx = np.full((T, 2048), -1, dtype=np.int32)
    for t in range(T):
        idx[t, :t + 1] = np.arange(t + 1)[::-1]
    scale = 1.0 / np.sqrt(576)
    out = D.sparse_attn(to_dev(qin["q"], "bf16", dev), to_dev(inp["kv"], "bf16", dev), to_dev(idx, "i32", dev),
                        to_dev(inp["sink"], "f32", dev), scale, 512)
    torch.cuda.synchronize()
    dense = O.dense_causal_attention(O.decode_bf16(qin["q"]), O.decode_bf16(inp["kv"]),
                                     inp["sink"].astype(np.float64), scale, 512)
    assert_attn_close(to_f64(out), dense, "bf16", "dense causal")


def test_attention_flags_bad_rows():
    dev = gpu()
    import sparse_attention_prefill_amd as D
    wl = S.WORKLOADS["inseq_cp8_last_8k"].with_(lens=(64,))
    inp = S.stream_inputs(wl)
    qin = S.query_inputs(wl, np.arange(2))
    idx = np.zeros((2, 64), dtype=np.int32)
    idx[0, 3] = 64  # one past the end
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    D.sparse_attn(to_dev(qin["q"], "bf16", dev), to_dev(inp["kv"], "bf16", dev), to_dev(idx, "i32", dev),
                  to_dev(inp["sink"], "f32", dev), 0.05, 512, err_flag=err)
    torch.cuda.synchronize()
    assert err.item() & 0x40


def test_attention_reruns_when_a_late_logit_is_far_above_the_first_rows():
    """The kernel takes each head's reference max from the first 32 selected rows (and the sink);
    a later row whose logit exceeds it by more than 64 (log2 units) makes the workgroup rerun the
    query with the exact max. Query 0 meets such a row at selection position 150 (third 64-row
    tile), 173 log2 units above the first rows: without the rerun its probabilities would overflow
    fp32. Query 1 meets an equally large logit at position 5, inside the first rows (no rerun);
    query 2 has neither. All three must match the oracle."""
    dev = gpu()
    import sparse_attention_prefill_amd as D
    n_rows, k_tot, nq = 512, 256, 3
    wl = S.WORKLOADS["inseq_cp8_last_8k"].with_(lens=(n_rows,))
    inp = S.stream_inputs(wl, "unit")
    qin = S.query_inputs(wl, np.arange(nq) * 5, "unit")
    scale = 1.0 / np.sqrt(wl.Dqk)
    q = O.decode(qin["q"], "bf16")
    kv_bits = inp["kv"].copy()
    big = {0: (7, 3, 150), 1: (11, 5, 5)}  # query: (kv row, head it aligns with, selection position)
    for i, (row, head, _) in big.items():
        # rope columns along q[i, head]'s: they add 120 nats to the logit of (i, head) on this row
        # and, not being value columns, leave the outputs O(1)
        r = q[i, head, wl.Dv:]
        kv_row = O.decode(kv_bits[row], "bf16").copy()
        kv_row[wl.Dv:] = 120.0 / (scale * np.linalg.norm(r)) * r / np.linalg.norm(r)
        kv_bits[row] = S.f64_to_bf16_bits(kv_row)
    g = np.random.default_rng(5)
    others = np.setdiff1d(np.arange(n_rows), [row for row, _, _ in big.values()])
    idx = np.stack([g.permutation(others)[:k_tot] for _ in range(nq)]).astype(np.int32)
    for i, (row, _, pos) in big.items():
        idx[i, pos] = row
    kv = O.decode(kv_bits, "bf16")
    sink = inp["sink"].astype(np.float64)
    first = [float((q[i] @ kv[idx[i, :32]].T).max() * scale) for i in range(nq)]
    late = [float((q[i] @ kv[idx[i, 32:]].T).max() * scale) for i in range(nq)]
    assert (late[0] - max(first[0], sink.max())) / np.log(2) > 128  # query 0 overflows without the rerun
    assert (late[1] - max(first[1], sink.max())) / np.log(2) < 64  # query 1 does not
    lse = torch.empty(nq, wl.H, dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    out = D.sparse_attn(to_dev(qin["q"], "bf16", dev), to_dev(kv_bits, "bf16", dev), to_dev(idx, "i32", dev),
                        to_dev(inp["sink"], "f32", dev), scale, wl.Dv, lse=lse, err_flag=err)
    torch.cuda.synchronize()
    assert err.item() == 0
    ref = np.zeros((nq, wl.H, wl.Dv))
    ref_lse = np.zeros((nq, wl.H))
    for i in range(nq):
        ref[i], ref_lse[i] = O.sparse_attention_row(q[i], kv[idx[i]], sink, scale, wl.Dv)
    assert_attn_close(to_f64(out), ref, "bf16", "late large logit")
    assert np.abs(lse.cpu().numpy() - ref_lse).max() < 2e-3


def test_attention_largest_selection_and_one_past_it():
    """k_tot = 2304 (the most selected rows per query the MLA kernel holds) matches the oracle;
    2305 is refused before any launch."""
    dev = gpu()
    import sparse_attention_prefill_amd as D
    n_rows, nq = 4096, 3
    wl = S.WORKLOADS["inseq_cp8_last_8k"].with_(lens=(n_rows,))
    inp = S.stream_inputs(wl)
    qin = S.query_inputs(wl, np.arange(nq) * 11)
    scale = 1.0 / np.sqrt(wl.Dqk)
    g = np.random.default_rng(9)
    idx = np.stack([g.permutation(n_rows)[:2304] for _ in range(nq)]).astype(np.int32)
    idx[2, 2300:] = -1  # a ragged last tile
    q_d, kv_d, s_d = to_dev(qin["q"], "bf16", dev), to_dev(inp["kv"], "bf16", dev), to_dev(inp["sink"], "f32", dev)
    out = D.sparse_attn(q_d, kv_d, to_dev(idx, "i32", dev), s_d, scale, wl.Dv)
    torch.cuda.synchronize()
    kv = O.decode(inp["kv"], "bf16")
    sink = inp["sink"].astype(np.float64)
    ref = np.stack([O.sparse_attention_row(O.decode(qin["q"][i], "bf16"), kv[idx[i][idx[i] >= 0]], sink, scale,
                                           wl.Dv)[0] for i in range(nq)])
    assert_attn_close(to_f64(out), ref, "bf16", "k_tot 2304")
    with pytest.raises(D.DsaError, match="2304"):
        D.sparse_attn(q_d, kv_d, to_dev(np.zeros((nq, 2305), np.int32), "i32", dev), s_d, scale, wl.Dv)


@pytest.mark.parametrize("name", ["inseq_cp8_last_8k", "tiny_fp32_cp1"])
def test_attention_without_sink(name):
    """sink = NULL drops the e^(sink) term: the oracle with sink = -inf; a query whose selection is
    empty gives out = 0 and lse = -inf."""
    dev = gpu()
    import sparse_attention_prefill_amd as D
    n_rows, nq = 300, 5
    wl = S.WORKLOADS[name].with_(lens=(n_rows,))
    inp = S.stream_inputs(wl, "unit")
    qin = S.query_inputs(wl, np.arange(nq) * 3, "unit")
    kind = wl.attn_dtype
    k_tot = 100 if kind == "bf16" else 64
    idx = _rand_idx(np.random.default_rng(3), nq, k_tot, n_rows, empty_rows=(2,))
    scale = 1.0 / np.sqrt(wl.Dqk)
    lse = torch.empty(nq, wl.H, dtype=torch.float32, device=dev)
    out = D.sparse_attn(to_dev(qin["q"], kind, dev), to_dev(inp["kv"], kind, dev), to_dev(idx, "i32", dev), None,
                        scale, wl.Dv, lse=lse)
    torch.cuda.synchronize()
    kv = O.decode(inp["kv"], kind)
    no_sink = np.full(wl.H, -np.inf)
    ref = np.zeros((nq, wl.H, wl.Dv))
    ref_lse = np.zeros((nq, wl.H))
    for i in range(nq):
        ref[i], ref_lse[i] = O.sparse_attention_row(O.decode(qin["q"][i], kind), kv[idx[i][idx[i] >= 0]], no_sink,
                                                    scale, wl.Dv)
    assert_attn_close(to_f64(out), ref, kind, f"{name} no sink")
    got_lse = lse.cpu().numpy()
    assert np.all(np.isneginf(got_lse[2])) and np.all(np.isneginf(ref_lse[2]))
    live = np.arange(nq) != 2
    assert np.abs(got_lse[live] - ref_lse[live]).max() < (1e-4 if kind == "f32" else 2e-3)


def test_attention_every_partial_tile_size():
    """Query j selects j + 1 rows (1 .. 64) and a few more around two and three half-tiles, so the
    last tile's mask is exercised at every fill level of both 32-row halves."""
    dev = gpu()
    import sparse_attention_prefill_amd as D
    n_rows, k_tot = 400, 160
    sizes = list(range(1, 65)) + [65, 95, 96, 97, 127, 128, 129, 160]
    nq = len(sizes)
    wl = S.WORKLOADS["inseq_cp8_last_8k"].with_(lens=(n_rows,))
    inp = S.stream_inputs(wl, "unit")
    qin = S.query_inputs(wl, np.arange(nq) * 5 % n_rows, "unit")
    g = np.random.default_rng(11)
    idx = np.full((nq, k_tot), -1, dtype=np.int32)
    for j, n in enumerate(sizes):
        slots = np.sort(g.permutation(k_tot)[:n])  # the -1 entries sit anywhere in the row
        idx[j, slots] = g.permutation(n_rows)[:n]
    scale = 1.0 / np.sqrt(wl.Dqk)
    out = D.sparse_attn(to_dev(qin["q"], "bf16", dev), to_dev(inp["kv"], "bf16", dev), to_dev(idx, "i32", dev),
                        to_dev(inp["sink"], "f32", dev), scale, wl.Dv)
    torch.cuda.synchronize()
    kv = O.decode(inp["kv"], "bf16")
    sink = inp["sink"].astype(np.float64)
    ref = np.stack([O.sparse_attention_row(O.decode(qin["q"][j], "bf16"), kv[idx[j][idx[j] >= 0]], sink, scale,
                                           wl.Dv)[0] for j in range(nq)])
    got = to_f64(out)
    for j, n in enumerate(sizes):
        assert_attn_close(got[j], ref[j], "bf16", f"{n} selected rows")
