"""The C-ABI library: it loads on a machine without a GPU, exports every symbol the header
declares, and its host-side checks reject bad arguments before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_hot_path_calls():
    names = declared_functions()
    for f in ("dsa_build_cp_metadata", "dsa_indexer_topk", "dsa_sparse_attn", "dsa_rerange"):
        assert f in names


def test_library_exports_every_declared_symbol():
    import sparse_attention_prefill_amd as D
    L = D.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_host_sizes():
    import sparse_attention_prefill_amd as D
    assert D.cp_sizes(8000, 8, 7, 0, False) == (1000, 1000, 8000)
    assert D.cp_sizes(43013, 8, 3, 1, False) == (5377, 5377, 43013)
    assert D.cp_sizes(11, 3, 2, 0, True) == (4, 3, 12)
    assert D.cp_sizes(11, 3, 2, 1, False) == (4, 3, 11)
    with pytest.raises(D.DsaError):
        D.cp_sizes(10, 4, 4, 0, False)


def test_host_checks_reject_before_launch():
    import sparse_attention_prefill_amd as D
    L = D.lib()
    # rerange: row bytes not a multiple of 16, bad mode, rank-less sizes
    assert L.dsa_rerange(None, None, 10, 24, 2, 0, 0, 0, None) == 1
    assert L.dsa_rerange(None, None, 10, 32, 2, 7, 0, 0, None) == 1
    assert L.dsa_rerange(None, None, 0, 32, 2, 1, 0, 0, None) == 0          # nothing to do
    assert L.dsa_rerange(ctypes.c_void_p(16), ctypes.c_void_p(32), 10, 32, 2, 1, 0, 0, None) == 1  # overlap
    assert b"overlap" in L.dsa_last_error()
    # metadata: rank out of range
    assert L.dsa_build_cp_metadata(None, None, 1, 8, 2, 2, 0, 0, None, None, None, None, None, None, None) == 1
    # attention: NULL args, bad dtype
    assert L.dsa_sparse_attn(None, None) == 1
    a = D.binding.AttnArgs()
    a.nq, a.n_rows, a.n_heads, a.d_qk, a.d_v, a.k_tot, a.dtype = 2, 4, 128, 576, 512, 8, 2
    assert L.dsa_sparse_attn(ctypes.byref(a), None) == 2
    a.dtype = 1
    assert L.dsa_sparse_attn(ctypes.byref(a), None) == 1                      # NULL pointers
    # indexer: top-k < 1, fp8 without scales
    g = D.binding.IndexerArgs()
    g.nq, g.nk, g.n_heads, g.head_dim, g.batch, g.topk, g.q_stride, g.compress_ratio = 4, 8, 64, 128, 1, 0, 1, 1
    assert L.dsa_indexer_topk(ctypes.byref(g), None) == 1
    g.topk, g.dtype = 16, 2
    g.q_idx = g.weights = g.k_idx = g.cu_seqlens_q = g.seqused_kv = g.cu_seqlens_kv = g.topk_idx = 256
    assert L.dsa_indexer_topk(ctypes.byref(g), None) == 1
    assert b"scale" in L.dsa_last_error()
    g.q_scale = g.k_scale = 256
    g.max_seqlen_kv = 8
    assert L.dsa_indexer_topk(ctypes.byref(g), None) == 3                     # no workspace
    assert L.dsa_indexer_topk_workspace(ctypes.byref(g)) == 4 * 64 * 4
    g.max_seqlen_kv = 200000
    assert L.dsa_indexer_topk(ctypes.byref(g), None) == 2                     # rows too long


def test_missing_library_fails_loudly(monkeypatch):
    import sparse_attention_prefill_amd.binding as B
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "library_path", "/nonexistent/libdsa.so")
    with pytest.raises(B.DsaError):
        B.lib()


def test_indexer_workspace_sizes_follow_the_selection_mode():
    """Host-only sizing: score rows up to 98304 visible keys; above that (64 x 128 bf16/fp8 indexer)
    one 128 KB list slot per row plus thresholds, segment counts, row status and 256 scratch rows."""
    import torch
    import sparse_attention_prefill_amd as D
    nq = 1000
    qi = torch.zeros(nq, 64, 128, dtype=torch.bfloat16)
    w = torch.zeros(nq, 64)
    ki = torch.zeros(200000, 128, dtype=torch.bfloat16)
    cu_q = torch.tensor([0, nq], dtype=torch.int32)
    used = torch.tensor([98304], dtype=torch.int32)
    cu_kv = torch.tensor([0, 200000], dtype=torch.int32)
    rows = D.indexer_topk_workspace(qi, w, ki, cu_q, used, cu_kv, 98304, topk=2048)
    assert rows == nq * 98304 * 4
    lists = D.indexer_topk_workspace(qi, w, ki, cu_q, used, cu_kv, 98305, topk=2048)
    ld = (98305 + 63) // 64 * 64
    assert nq * 131072 + nq * 4 * 3 + 256 * ld * 4 <= lists <= nq * 131072 + nq * 4 * (2 + 64) + 256 * ld * 4 + 1024
    # a K above the launch bound keeps score rows; so does the generic (non 64 x 128) indexer
    assert D.indexer_topk_workspace(qi, w, ki, cu_q, used, cu_kv, 100000, topk=100000) == nq * 100032 * 4
    qs = torch.zeros(nq, 32, 128, dtype=torch.bfloat16)
    assert D.indexer_topk_workspace(qs, w[:, :32], ki, cu_q, used, cu_kv, 100000, topk=2048) == nq * 100032 * 4


def test_binding_rejects_tensors_the_library_cannot_read():
    """Marshalling checks: host tensors, non-contiguous views, mixed dtypes, padded score columns."""
    import torch
    import sparse_attention_prefill_amd as D
    nq = 4
    qi = torch.zeros(nq, 64, 128, dtype=torch.bfloat16)
    w = torch.zeros(nq, 64)
    cu = torch.tensor([0, nq], dtype=torch.int32)
    used = torch.tensor([16], dtype=torch.int32)
    with pytest.raises(D.DsaError, match="GPU"):
        D.indexer_topk(qi, w, torch.zeros(16, 128, dtype=torch.bfloat16), cu, used, cu, 16, topk=8)
    with pytest.raises(D.DsaError, match="dtype"):
        D.indexer_topk_workspace(qi, w, torch.zeros(16, 128, dtype=torch.float32), cu, used, cu, 16, topk=8)
    with pytest.raises(D.DsaError, match="dtype"):
        D.indexer_topk_workspace(qi, w.double(), torch.zeros(16, 128, dtype=torch.bfloat16), cu, used, cu, 16)
    with pytest.raises(D.DsaError, match="dense rows"):
        D.indexer_scores(qi, w, qi[0], cu, used, cu, 16, torch.zeros(16, nq).t())
    q = torch.zeros(2, 128, 576, dtype=torch.bfloat16)
    with pytest.raises(D.DsaError, match="GPU"):
        D.sparse_attn(q, torch.zeros(8, 576, dtype=torch.bfloat16), torch.zeros(2, 4, dtype=torch.int32),
                      None, 0.1, 512)
    with pytest.raises(D.DsaError, match="GPU|contiguous"):
        D.rerange(torch.zeros(8, 64, dtype=torch.bfloat16)[:, ::2], 8, 2, 1, False)


def test_timed_indexer_rejects_missing_events_before_launch():
    import sparse_attention_prefill_amd as D
    L = D.lib()
    g = D.binding.IndexerArgs()
    n = ctypes.c_int32(-1)
    assert L.dsa_indexer_topk_timed(ctypes.byref(g), None, None, 4, ctypes.byref(n), None) == 1
    ev = (ctypes.c_void_p * 3)(16, None, 32)
    assert L.dsa_indexer_topk_timed(ctypes.byref(g), None, ev, 3, ctypes.byref(n), None) == 1
    assert b"NULL event" in L.dsa_last_error() and n.value == -1


def test_measurement_probes_reject_bad_arguments_before_launch():
    import sparse_attention_prefill_amd as D
    L = D.lib()
    assert L.dsa_clock_probe(None, 100, None) == 1
    assert L.dsa_clock_probe(ctypes.c_void_p(256), 0, None) == 1
    p = ctypes.c_void_p(256)
    assert L.dsa_lds_mfma_probe(3, 1, 10, p, 2048, p, 65536, None) == 1       # operand
    assert L.dsa_lds_mfma_probe(0, 3, 10, p, 2048, p, 65536, None) == 1       # waves per SIMD
    assert L.dsa_lds_mfma_probe(0, 1, 0, p, 2048, p, 65536, None) == 1        # iterations
    assert L.dsa_lds_mfma_probe(1, 1, 10, p, 2047, p, 65536, None) == 1       # short cycle buffer
    assert L.dsa_lds_mfma_probe(1, 2, 10, p, 2048, p, 65536, None) == 1       # sink for 512 threads
    assert b"sink" in L.dsa_last_error()


def test_checked_library_exports_every_declared_symbol():
    import sparse_attention_prefill_amd as D
    with D.library(D.checked_library_path) as L:
        missing = [n for n in declared_functions() if not hasattr(L, n)]
        assert not missing, missing
        assert L.dsa_sparse_attn(None, None) == 1      # the same host checks
    assert D.lib()._name == D.library_path
