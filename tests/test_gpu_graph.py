"""The rank's path captured in a HIP graph (as the benchmark times it): every replay, with eager
work and synchronisations between replays, equals the eager run bit for bit."""
import numpy as np
import pytest
import torch

import synthetic as S
from dsa_testlib import gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw", [("inseq_cp8_last_8k", {"lens": (4096,)}),
                                     ("rr_cp4_r1_var8_cmp4", {"lens": (3000, 901, 2200)}),
                                     # rows past 98304 keys: the candidate-list kernels in the graph
                                     ("inseq_cp8_last_8k", {"lens": (100000,)})])
def test_graph_replays_equal_eager(name, kw):
    dev = gpu()
    import sparse_attention_prefill_amd as D
    wl = S.WORKLOADS[name].with_(**kw)
    mode = 0 if wl.mode == "in_seq" else 1
    qsl_d, lens_d = to_dev(wl.qsl, "i32", dev), to_dev(wl.seq_lens, "i32", dev)
    _, n_real, _ = D.cp_sizes(wl.T, wl.cp, wl.rank, mode, wl.pad)
    meta0 = D.build_cp_metadata(qsl_d, lens_d, wl.T, wl.cp, wl.rank, mode, wl.pad)
    torch.cuda.synchronize()
    toks = meta0["token_map"].cpu().numpy()[:n_real]
    inp, qin = S.stream_inputs(wl), S.query_inputs(wl, toks)
    qi, w, ki = to_dev(qin["q_idx"], "bf16", dev), to_dev(qin["w"], "f32", dev), to_dev(inp["k_idx"], "bf16", dev)
    q, kv, sink = to_dev(qin["q"], "bf16", dev), to_dev(inp["kv"], "bf16", dev), to_dev(inp["sink"], "f32", dev)
    kv_cmp = to_dev(inp["kv_cmp_start"], "i32", dev) if wl.compress > 1 else None
    idx = torch.empty(n_real, wl.k_tot, dtype=torch.int32, device=dev)
    out = torch.empty(n_real, wl.H, wl.Dv, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(D.indexer_topk_workspace(qi, w, ki, meta0["local_query_start_loc"], meta0["local_seq_lens"],
                                              kv_cmp if kv_cmp is not None else meta0["local_kv_start_loc"],
                                              int(wl.seq_lens.max()), topk=wl.topk, window=wl.window,
                                              window_kv_start=meta0["local_kv_start_loc"],
                                              compress_ratio=wl.compress), dtype=torch.uint8, device=dev)

    def step():
        m = D.build_cp_metadata(qsl_d, lens_d, wl.T, wl.cp, wl.rank, mode, wl.pad)
        D.indexer_topk(qi, w, ki, m["local_query_start_loc"], m["local_seq_lens"],
                       kv_cmp if kv_cmp is not None else m["local_kv_start_loc"], int(wl.seq_lens.max()), topk_idx=idx,
                       workspace=ws, topk=wl.topk, q_stride=wl.cp if mode else 1, compress_ratio=wl.compress,
                       kv_row_base=wl.n_kv if wl.compress > 1 else 0, window=wl.window,
                       window_kv_start=m["local_kv_start_loc"] if wl.window else None)
        D.sparse_attn(q, kv, idx, sink, 1.0 / np.sqrt(wl.Dqk), wl.Dv, out=out)

    step()
    torch.cuda.synchronize()
    idx_ref, out_ref = idx.clone(), out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        idx.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref), f"replay {rep}: top-k differs"
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), f"replay {rep}: attention differs"
        _ = (q.float() * 2).sum().item()  # eager work between replays
