"""GPU: indexer + top-k in candidate mode against the two-stage path, bit for bit.

In a launch whose longest row has more than 98304 visible keys, rows with more than
max(32768, K) visible keys are selected from lists of their best scores (a sampled threshold
decides what the indexer keeps) instead of from full score rows; a row whose list falls short
of K or overflows is recomputed and selected from a full row. Either
way the ids must be exactly those of dsa_topk_from_scores over dsa_indexer_scores, which are
checked against the oracle elsewhere. Cases: long rows in bf16 and fp8, short and long rows in
one batch, several requests in round-robin order, compressed keys with a window, and inputs
that force the recomputation (a K close to the list size, all-zero keys with every score tied,
and a K larger than 32768).
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
