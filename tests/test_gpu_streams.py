"""The library keeps no state between calls (only a per-thread error string): two different steps
enqueued on two streams at once, each with its own workspace and outputs, give exactly the results
of the same steps run one after the other on one stream."""
import numpy as np
import pytest
import torch

import synthetic as S
from dsa_testlib import gpu, to_dev

pytestmark = pytest.mark.gpu


def _case(name, kw, dev):
    import sparse_attention_prefill_amd as D
    wl = S.WORKLOADS[name].with_(**kw)
    mode = 0 if wl.mode == "in_seq" else 1
    qsl_d, lens_d = to_dev(wl.qsl, "i32", dev), to_dev(wl.seq_lens, "i32", dev)
    _, n_real, _ = D.cp_sizes(wl.T, wl.cp, wl.rank, mode, wl.pad)
    meta0 = D.build_cp_metadata(qsl_d, lens_d, wl.T, wl.cp, wl.rank, mode, wl.pad)
    torch.cuda.synchronize()
    toks = meta0["token_map"].cpu().numpy()[:n_real]
    inp, qin = S.stream_inputs(wl), S.query_inputs(wl, toks)
    t = dict(qi=to_dev(qin["q_idx"], "bf16", dev), w=to_dev(qin["w"], "f32", dev), ki=to_dev(inp["k_idx"], "bf16", dev),
             q=to_dev(qin["q"], "bf16", dev), kv=to_dev(inp["kv"], "bf16", dev), sink=to_dev(inp["sink"], "f32", dev),
             qsl=qsl_d, lens=lens_d)
    kv_cmp = to_dev(inp["kv_cmp_start"], "i32", dev) if wl.compress > 1 else None
    ws = torch.empty(D.indexer_topk_workspace(t["qi"], t["w"], t["ki"], meta0["local_query_start_loc"],
                                              meta0["local_seq_lens"],
                                              kv_cmp if kv_cmp is not None else meta0["local_kv_start_loc"],
                                              int(wl.seq_lens.max()), topk=wl.topk, window=wl.window,
                                              window_kv_start=meta0["local_kv_start_loc"], compress_ratio=wl.compress),
                     dtype=torch.uint8, device=dev)
    idx = torch.empty(n_real, wl.k_tot, dtype=torch.int32, device=dev)
    out = torch.empty(n_real, wl.H, wl.Dv, dtype=torch.bfloat16, device=dev)

    def step(stream):
        m = D.build_cp_metadata(t["qsl"], t["lens"], wl.T, wl.cp, wl.rank, mode, wl.pad, stream=stream)
        D.indexer_topk(t["qi"], t["w"], t["ki"], m["local_query_start_loc"], m["local_seq_lens"],
                       kv_cmp if kv_cmp is not None else m["local_kv_start_loc"], int(wl.seq_lens.max()), topk_idx=idx,
                       workspace=ws, topk=wl.topk, q_stride=wl.cp if mode else 1, compress_ratio=wl.compress,
                       kv_row_base=wl.n_kv if wl.compress > 1 else 0, window=wl.window,
                       window_kv_start=m["local_kv_start_loc"] if wl.window else None, stream=stream)
        D.sparse_attn(t["q"], t["kv"], idx, t["sink"], 1.0 / np.sqrt(wl.Dqk), wl.Dv, out=out, stream=stream)
        return m

    return step, idx, out


def test_two_streams_equal_serial():
    dev = gpu()
    cases = [_case("inseq_cp8_last_8k", {"lens": (6000,)}, dev),
             _case("rr_cp4_r1_var8_cmp4", {"lens": (3000, 901, 2200)}, dev)]
    # serial, on the current stream
    cur = torch.cuda.current_stream()
    refs = []
    for step, idx, out in cases:
        step(cur)
        torch.cuda.synchronize()
        refs.append((idx.clone(), out.clone()))
    for rep in range(3):
        for _, idx, out in cases:
            idx.fill_(-7)
            out.zero_()
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream() for _ in cases]  # default priority
        metas = []
        for (step, _, _), s in zip(cases, streams):
            with torch.cuda.stream(s):  # the metadata tensors are allocated on the stream that uses them
                metas.append(step(s))
        torch.cuda.synchronize()
        for (_, idx, out), (ridx, rout) in zip(cases, refs):
            assert torch.equal(idx, ridx), f"rep {rep}: top-k differs"
            assert torch.equal(out.view(torch.int16), rout.view(torch.int16)), f"rep {rep}: attention differs"
