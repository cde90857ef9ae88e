"""GPU: indexer + top-k in candidate mode against the two-stage path, bit for bit.

In a launch whose longest row has more than 98304 visible keys, rows with more than
max(32768, K) visible keys are selected from lists of their best scores (a sampled threshold
decides what the indexer keeps) instead of from full score rows; a row whose list falls short
of K or overflows is recomputed and selected from a full row. Either
way the ids must be exactly those of dsa_topk_from_scores over dsa_indexer_scores, which are
checked against the oracle elsewhere. Cases: long rows in bf16 and fp8, short and long rows in
one batch, several requests in round-robin order, compressed keys with a window, and inputs
that force the recomputation (a K close to the list size, all-zero keys with every score tied,
and a K larger than 32768). The threshold itself is checked against its definition over the
indexer's score rows.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from dsa_testlib import gpu, to_dev

pytestmark = pytest.mark.gpu


def _both(wl, variant, dev, zero_keys=False):
    import sparse_attention_prefill_amd as D
    m = O.cp_metadata(wl.qsl, wl.seq_lens, wl.cp, wl.rank, wl.mode, wl.pad)
    toks = m["token_map"][m["token_map"] >= 0]
    inp = S.stream_inputs(wl, variant)
    qin = S.query_inputs(wl, toks, variant, indexer_only=True)
    ik = wl.idx_dtype
    k_idx = np.zeros_like(inp["k_idx"]) if zero_keys else inp["k_idx"]
    cu_kv = inp["kv_cmp_start"] if wl.compress > 1 else m["local_kv_start_loc"]
    max_kv = int(m["local_seq_lens"].max())
    vis = max_kv // wl.compress if wl.compress > 1 else max_kv
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    lkv = to_dev(m["local_kv_start_loc"], "i32", dev)
    args = [to_dev(qin["q_idx"], ik, dev), to_dev(qin["w"], "f32", dev), to_dev(k_idx, ik, dev),
            to_dev(m["local_query_start_loc"], "i32", dev), to_dev(m["local_seq_lens"], "i32", dev),
            to_dev(cu_kv, "i32", dev), max_kv]
    kw = dict(topk=wl.topk, q_stride=m["stride"], compress_ratio=wl.compress,
              kv_row_base=wl.n_kv if wl.compress > 1 else 0, window=wl.window,
              window_kv_start=lkv if wl.window else None,
              q_scale=to_dev(qin["q_scale"], "f32", dev) if "q_scale" in qin else None,
              k_scale=to_dev(inp["k_scale"], "f32", dev) if "k_scale" in inp else None, err_flag=err)
    print(f"case {wl.name} lens={wl.lens[:4]} cp={wl.cp} r={wl.rank} K={wl.topk} nq={len(toks)} max_vis={vis}",
          flush=True)
    fused = D.indexer_topk(*args, **kw)
    torch.cuda.synchronize()
    assert err.item() == 0
    scores = torch.empty(len(toks), (vis + 63) // 64 * 64, dtype=torch.float32, device=dev)
    skw = {k: v for k, v in kw.items() if k not in ("window", "window_kv_start", "kv_row_base")}
    D.indexer_scores(*args, scores, **skw)
    ref = D.topk_from_scores(*args, scores, **kw)
    torch.cuda.synchronize()
    assert err.item() == 0
    return fused.cpu().numpy(), ref.cpu().numpy(), vis


CASES = [
    ("inseq_cp8_last_8k", {"lens": (100000,)}, "normal"),
    ("inseq_cp8_last_8k", {"lens": (100000,)}, "int"),
    ("long_131k_fp8", {}, "normal"),
    # short and long rows in one batch: request 1 rows stay under 32768 keys
    ("long_131k_fp8", {"lens": (100000, 20000), "cp": 4, "rank": 3, "mode": "round_robin"}, "normal"),
    ("rr_cp8_r3_batch4", {"lens": (110000, 36000, 5), "cp": 4, "rank": 1}, "normal"),
    ("chunk_inseq_cp8_last_8k_p56k", {"prefix": (100000,)}, "normal"),
    # x4 keys (visible = extent / 4) with a window; short and long rows
    ("rr_cp4_r1_var8_cmp4", {"lens": (420000,), "cp": 16, "rank": 5}, "normal"),
]


@pytest.mark.parametrize("name,kw,variant", CASES)
def test_candidate_lists_match_score_rows(name, kw, variant):
    dev = gpu()
    fused, ref, vis = _both(S.WORKLOADS[name].with_(**kw), variant, dev)
    assert vis > 98304
    assert np.array_equal(fused, ref)


@pytest.mark.parametrize("name,kw,zero", [
    ("inseq_cp8_last_8k", {"lens": (100000,), "topk": 16000}, False),   # lists overflow: every row recomputed
    ("inseq_cp8_last_8k", {"lens": (100000,)}, True),                    # every score 0.0: ties at the cut
    ("inseq_cp8_last_8k", {"lens": (100000,), "cp": 4, "rank": 3, "topk": 40000}, False),  # K above 32768
    # fp8: the recomputation repeats the indexer's fp8 arithmetic (|x| head sum + split c . k)
    ("long_131k_fp8", {"lens": (100000,), "topk": 16000}, False),
    ("long_131k_fp8", {"lens": (100000,)}, True),
])
def test_recomputed_rows_match_score_rows(name, kw, zero):
    dev = gpu()
    fused, ref, _ = _both(S.WORKLOADS[name].with_(**kw), "normal", dev, zero_keys=zero)
    assert np.array_equal(fused, ref)


@pytest.mark.parametrize("name,kw", [
    ("inseq_cp8_last_8k", {"lens": (9000,), "topk": 512}),     # score rows
    ("inseq_cp8_last_8k", {"lens": (100000,)}),                 # candidate lists
    ("rr_cp4_r1_var8_cmp4", {"lens": (6000, 9000)}),            # x4 keys, window
])
def test_rows_outside_the_key_buffer_are_cleared_and_flagged(name, kw):
    """A key buffer shorter than some rows' extents: those rows get -1 everywhere (window included)
    and DSA_DEVERR_EXTENT; the other rows are exactly those of the full buffer."""
    dev = gpu()
    import sparse_attention_prefill_amd as D
    wl = S.WORKLOADS[name].with_(**kw)
    m = O.cp_metadata(wl.qsl, wl.seq_lens, wl.cp, wl.rank, wl.mode, wl.pad)
    toks = m["token_map"][m["token_map"] >= 0]
    inp = S.stream_inputs(wl)
    qin = S.query_inputs(wl, toks, indexer_only=True)
    ik = wl.idx_dtype
    cu_kv = inp["kv_cmp_start"] if wl.compress > 1 else m["local_kv_start_loc"]
    max_kv = int(m["local_seq_lens"].max())
    k_full = inp["k_idx"]
    nk_short = k_full.shape[0] - 37
    views = O.query_views(m)
    vis = [E // wl.compress if wl.compress > 1 else E for (_, E, _) in views]
    kv0 = [int(cu_kv[b]) for (b, _, _) in views]
    bad = np.array([k0 + e > nk_short for k0, e in zip(kv0, vis)])
    assert bad.any() and not bad.all()
    lkv = to_dev(m["local_kv_start_loc"], "i32", dev)
    outs, errs = [], []
    for k_idx in (k_full, k_full[:nk_short]):
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        out = torch.full((len(toks), wl.k_tot), -7, dtype=torch.int32, device=dev)  # no valid entry is -7
        print(f"case {name} nk={k_idx.shape[0]} nq={len(toks)}", flush=True)
        D.indexer_topk(to_dev(qin["q_idx"], ik, dev), to_dev(qin["w"], "f32", dev), to_dev(k_idx, ik, dev),
                       to_dev(m["local_query_start_loc"], "i32", dev), to_dev(m["local_seq_lens"], "i32", dev),
                       to_dev(cu_kv, "i32", dev), max_kv, topk_idx=out, topk=wl.topk, q_stride=m["stride"],
                       compress_ratio=wl.compress, kv_row_base=wl.n_kv if wl.compress > 1 else 0,
                       window=wl.window, window_kv_start=lkv if wl.window else None, err_flag=err)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
        errs.append(err.item())
    assert errs[0] == 0 and errs[1] & 0x20
    assert np.all(outs[1][bad] == -1)
    assert np.array_equal(outs[1][~bad], outs[0][~bad])
    assert not np.any(outs[0] == -7) and not np.any(outs[1] == -7)


def _order_keys(scores):
    """Order-preserving 32-bit keys of float32 scores (-0.0 and +0.0 share 2^31)."""
    u = np.ascontiguousarray(scores, dtype=np.float32).view(np.uint32).astype(np.int64)
    m = u & 0x7FFFFFFF
    return np.where(u >> 31, 0x80000000 - m, 0x80000000 + m)


@pytest.mark.parametrize("name,kw", [
    ("long_131k_fp8", {}),                                                          # fp8, every group shared
    ("long_131k_fp8", {"lens": (100000, 20000), "cp": 4, "rank": 3, "mode": "round_robin"}),
    ("inseq_cp8_last_8k", {"lens": (100000,)}),                                     # bf16
    ("rr_cp8_r3_batch4", {"lens": (110000, 36000, 5), "cp": 4, "rank": 1}),         # bf16, three requests
])
def test_theta_is_the_sample_rank_prefix_of_the_score_rows(name, kw):
    """White-box check of the candidate threshold (it lives in the call's workspace, after the
    lists: nq x 16384 entries of 8 bytes). For a candidate row of extent ev in a group of 8 rows
    (rows 8g .. 8g + 7) the sample is 16 tiles of 128 consecutive keys starting at
    t * (ev_s - 128) // 15, with ev_s the shortest extent of the group when all 8 are candidate rows
    of one request (else the row's own), and theta is the top 22 bits of the order key of the
    sample's r-th largest score, r = min(2048, ceil((2.75 + sqrt(2.75^2 + 2048 K / ev))^2)). The
    sample scores are recomputed here from the indexer's own score rows, so theta must match bit
    for bit wherever the kernel computes them with the indexer's arithmetic: bf16 rows, and fp8
    rows of shared groups (fp8 rows of other groups keep the ReLU form, which moves theta by
    rounding only, and are not compared)."""
    import math
    import sparse_attention_prefill_amd as D
    dev = gpu()
    wl = S.WORKLOADS[name].with_(**kw)
    m = O.cp_metadata(wl.qsl, wl.seq_lens, wl.cp, wl.rank, wl.mode, wl.pad)
    toks = m["token_map"][m["token_map"] >= 0]
    nq = len(toks)
    inp = S.stream_inputs(wl)
    qin = S.query_inputs(wl, toks, indexer_only=True)
    ik = wl.idx_dtype
    max_kv = int(m["local_seq_lens"].max())
    args = [to_dev(qin["q_idx"], ik, dev), to_dev(qin["w"], "f32", dev), to_dev(inp["k_idx"], ik, dev),
            to_dev(m["local_query_start_loc"], "i32", dev), to_dev(m["local_seq_lens"], "i32", dev),
            to_dev(m["local_kv_start_loc"], "i32", dev), max_kv]
    kw2 = dict(topk=wl.topk, q_stride=m["stride"],
               q_scale=to_dev(qin["q_scale"], "f32", dev) if "q_scale" in qin else None,
               k_scale=to_dev(inp["k_scale"], "f32", dev) if "k_scale" in inp else None)
    print(f"case {name} lens={wl.lens[:4]} nq={nq} max_vis={max_kv}", flush=True)
    assert max_kv > 98304
    ws = torch.zeros(D.indexer_topk_workspace(*args, **kw2), dtype=torch.uint8, device=dev)
    D.indexer_topk(*args, workspace=ws, **kw2)
    off = nq * 16384 * 8
    theta = ws[off:off + 4 * nq].view(torch.int32).cpu().numpy().view(np.uint32).astype(np.int64)
    scores = torch.empty(nq, (max_kv + 63) // 64 * 64, dtype=torch.float32, device=dev)
    D.indexer_scores(*args, scores, **kw2)
    torch.cuda.synchronize()

    views = O.query_views(m)
    ev = np.array([E for (_, E, _) in views])
    kv0 = np.array([k for (_, _, k) in views])
    fuse_above = max(32768, wl.topk)
    cand = ev > fuse_above
    checked = 0
    pos, rows, rank = [], [], []
    for g in range((nq + 7) // 8):
        grp = range(8 * g, min(8 * g + 8, nq))
        shared = len(grp) == 8 and all(cand[j] for j in grp) and len({kv0[j] for j in grp}) == 1
        for i in grp:
            if not cand[i] or (ik == "fp8" and not shared):
                continue
            ev_s = min(ev[j] for j in grp) if shared else ev[i]
            starts = [t * (ev_s - 128) // 15 for t in range(16)]
            pos.append(np.concatenate([np.arange(s, s + 128) for s in starts]))
            rows.append(i)
            sr = 2.75 + math.sqrt(2.75 * 2.75 + wl.topk * 2048 / ev[i])
            rank.append(min(2048, math.ceil(sr * sr)))
    assert rows
    flat = np.asarray(rows, dtype=np.int64)[:, None] * scores.shape[1] + np.stack(pos)
    samples = scores.view(-1)[torch.as_tensor(flat, device=dev)].cpu().numpy()
    keys = -np.sort(-_order_keys(samples), axis=1)
    want = np.array([keys[k, r - 1] for k, r in enumerate(rank)]) >> 10 << 10
    got = theta[rows]
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} of {len(rows)} rows differ, first row {rows[bad[0]]}: {got[bad[0]]:#x} vs {want[bad[0]]:#x}"
