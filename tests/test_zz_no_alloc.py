"""GPU: dsa_indexer_topk_noalloc (for callers that cannot allocate) against dsa_indexer_topk with a
caller workspace, bit for bit, on two calls in a row (the second smaller, so it runs over what the
first left in the shared static scratch), and its rejection of calls larger than the scratch."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from dsa_testlib import gpu, to_dev

pytestmark = pytest.mark.gpu


def _inputs(wl, dev):
    m = O.cp_metadata(wl.qsl, wl.seq_lens, wl.cp, wl.rank, wl.mode, wl.pad)
    toks = m["token_map"][m["token_map"] >= 0]
    inp = S.stream_inputs(wl)
    qin = S.query_inputs(wl, toks, indexer_only=True)
    ik = wl.idx_dtype
    cu_kv = inp["kv_cmp_start"] if wl.compress > 1 else m["local_kv_start_loc"]
    args = [to_dev(qin["q_idx"], ik, dev), to_dev(qin["w"], "f32", dev), to_dev(inp["k_idx"], ik, dev),
            to_dev(m["local_query_start_loc"], "i32", dev), to_dev(m["local_seq_lens"], "i32", dev),
            to_dev(cu_kv, "i32", dev), int(m["local_seq_lens"].max())]
    kw = dict(topk=wl.topk, q_stride=m["stride"], compress_ratio=wl.compress,
              kv_row_base=wl.n_kv if wl.compress > 1 else 0, window=wl.window,
              window_kv_start=to_dev(m["local_kv_start_loc"], "i32", dev) if wl.window else None,
              q_scale=to_dev(qin["q_scale"], "f32", dev) if "q_scale" in qin else None,
              k_scale=to_dev(inp["k_scale"], "f32", dev) if "k_scale" in inp else None)
    return args, kw, len(toks)


def test_noalloc_equals_the_workspace_call_on_two_calls_in_a_row():
    dev = gpu()
    import sparse_attention_prefill_amd as D
    cases = [
        S.WORKLOADS["inseq_cp8_last_8k"],                                     # 1024 rows x 8192 keys: 32 MiB
        S.WORKLOADS["rr_cp4_r1_var8_cmp4"].with_(lens=(1100, 1900, 13, 640)),  # 914 rows, x4 keys + window: 2 MiB
    ]
    for wl in cases:
        args, kw, nq = _inputs(wl, dev)
        print(f"case {wl.name} lens={wl.lens[:4]} nq={nq}", flush=True)
        err_ref = torch.zeros(1, dtype=torch.int32, device=dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        need = D.indexer_topk_workspace(*args, **kw)
        assert need <= 64 << 20
        ref = D.indexer_topk(*args, err_flag=err_ref, **kw)
        got = torch.full((nq, wl.k_tot), -7, dtype=torch.int32, device=dev)  # no valid entry is -7
        D.indexer_topk_noalloc(*args, got, err_flag=err, **kw)
        torch.cuda.synchronize()
        assert err_ref.item() == 0 and err.item() == 0
        assert torch.equal(got, ref)


def test_noalloc_rejects_calls_larger_than_its_scratch():
    dev = gpu()
    import sparse_attention_prefill_amd as D
    nq, max_kv = 4096, 8192  # score rows of 4096 x 8192 floats: 128 MiB
    qi = torch.zeros(nq, 64, 128, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(nq, 64, dtype=torch.float32, device=dev)
    ki = torch.zeros(max_kv, 128, dtype=torch.bfloat16, device=dev)
    cu_q = torch.tensor([0, nq], dtype=torch.int32, device=dev)
    used = torch.tensor([max_kv], dtype=torch.int32, device=dev)
    cu_kv = torch.tensor([0, max_kv], dtype=torch.int32, device=dev)
    out = torch.full((nq, 2048), -7, dtype=torch.int32, device=dev)
    with pytest.raises(D.DsaError, match="static scratch"):
        D.indexer_topk_noalloc(qi, w, ki, cu_q, used, cu_kv, max_kv, out, topk=2048)
    torch.cuda.synchronize()
    assert bool((out == -7).all())  # nothing was launched
