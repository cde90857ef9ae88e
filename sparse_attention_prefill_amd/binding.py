"""ctypes binding of libdsa.so: argument marshalling only (no compute, no fallback).

Tensors are torch device tensors; the HIP stream is torch's current stream unless one is
given. Every call raises DsaError with the library's message when the C call fails.
bf16 tensors are torch.bfloat16; fp8 E4M3FN tensors are torch.uint8 (raw bytes) or
torch.float8_e4m3fn.
"""
import contextlib
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(HERE, "libdsa.so")
# the same sources built with DSA_CHECKED: bounds-checked indices, failures in err_flag (tests only)
checked_library_path = os.path.join(HERE, "libdsa_checked.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
IN_SEQ, ROUND_ROBIN = 0, 1

c_i32, c_i64, c_p, c_f32, c_size = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t


class DsaError(RuntimeError):
    pass


class IndexerArgs(ctypes.Structure):
    _fields_ = [
        ("q_idx", c_p), ("q_scale", c_p), ("weights", c_p), ("k_idx", c_p), ("k_scale", c_p),
        ("dtype", c_i32), ("nq", c_i32), ("nk", c_i32), ("n_heads", c_i32), ("head_dim", c_i32), ("batch", c_i32),
        ("cu_seqlens_q", c_p), ("seqused_kv", c_p), ("cu_seqlens_kv", c_p),
        ("max_seqlen_kv", c_i32), ("q_stride", c_i32), ("compress_ratio", c_i32), ("topk", c_i32),
        ("kv_row_base", c_i32), ("window", c_i32), ("window_kv_start", c_p), ("topk_idx", c_p),
        ("workspace", c_p), ("workspace_bytes", c_size), ("err_flag", c_p),
    ]


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("q", c_p), ("kv", c_p), ("idx", c_p), ("sink", c_p), ("out", c_p), ("lse", c_p), ("err_flag", c_p),
        ("softmax_scale", c_f32), ("dtype", c_i32), ("nq", c_i32), ("n_rows", c_i32), ("n_heads", c_i32),
        ("d_qk", c_i32), ("d_v", c_i32), ("k_tot", c_i32),
    ]


_lib = None


@contextlib.contextmanager
def library(path):
    """Route the calls made inside the block to the library at `path` (e.g. checked_library_path);
    the previous library is used again afterwards. Not for concurrent use from several threads."""
    global _lib, library_path
    saved = (_lib, library_path)
    _lib, library_path = None, path
    try:
        yield lib()
    finally:
        _lib, library_path = saved


def lib():
    """The loaded libdsa.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise DsaError(f"{library_path} is missing: build it with `python -m sparse_attention_prefill_amd.build`")
        L = ctypes.CDLL(library_path)
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_version.restype = ctypes.c_char_p
        L.dsa_cp_sizes.argtypes = [c_i32] * 5 + [ctypes.POINTER(c_i32)] * 3
        L.dsa_build_cp_metadata.argtypes = [c_p, c_p] + [c_i32] * 6 + [c_p] * 7
        L.dsa_indexer_topk_workspace.argtypes = [ctypes.POINTER(IndexerArgs)]
        L.dsa_indexer_topk_workspace.restype = c_size
        L.dsa_indexer_topk.argtypes = [ctypes.POINTER(IndexerArgs), c_p]
        L.dsa_indexer_topk_noalloc.argtypes = [ctypes.POINTER(IndexerArgs), c_p]
        L.dsa_indexer_topk_timed.argtypes = [ctypes.POINTER(IndexerArgs), c_p, ctypes.POINTER(c_p), c_i32,
                                             ctypes.POINTER(c_i32), ctypes.POINTER(ctypes.c_char_p)]
        L.dsa_indexer_scores.argtypes = [ctypes.POINTER(IndexerArgs), c_p, c_i64, c_p]
        L.dsa_topk_from_scores.argtypes = [ctypes.POINTER(IndexerArgs), c_p, c_i64, c_p]
        L.dsa_sparse_attn.argtypes = [ctypes.POINTER(AttnArgs), c_p]
        L.dsa_clock_probe.argtypes = [c_p, c_i64, c_p]
        L.dsa_lds_mfma_probe.argtypes = [c_i32, c_i32, c_i32, c_p, c_i64, c_p, c_i64, c_p]
        L.dsa_rerange.argtypes = [c_p, c_p, c_i32, c_i64, c_i32, c_i32, c_i32, c_i32, c_p]
        for f in ("dsa_cp_sizes", "dsa_build_cp_metadata", "dsa_indexer_topk", "dsa_indexer_topk_noalloc",
                  "dsa_indexer_topk_timed",
                  "dsa_indexer_scores",
                  "dsa_topk_from_scores", "dsa_sparse_attn", "dsa_rerange", "dsa_clock_probe",
                  "dsa_lds_mfma_probe"):
            getattr(L, f).restype = c_i32
        _lib = L
    return _lib


def version():
    return lib().dsa_version().decode()


def _check(status, what):
    if status != 0:
        raise DsaError(f"{what} failed ({status}): {lib().dsa_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dense(name, t, dtype=None, optional=False, memory=True):
    """A device tensor the library may read as dense row-major memory: on a GPU, contiguous and,
    when given, of `dtype` (a torch dtype or a tuple of them). None is allowed when optional.
    memory=False (host-only size queries, which read no tensor memory) checks the dtype only."""
    if t is None:
        if optional:
            return
        raise DsaError(f"{name} is required")
    if memory and not t.is_cuda:
        raise DsaError(f"{name} must be a GPU tensor")
    if memory and not t.is_contiguous():
        raise DsaError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise DsaError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _rows(name, t, dtype):
    """Score rows: a GPU tensor whose rows are dense (stride(1) == 1); rows may be padded."""
    if not t.is_cuda or t.dim() != 2 or t.dtype != dtype or t.stride(1) != 1:
        raise DsaError(f"{name} must be a 2-D {dtype} GPU tensor with dense rows (stride(1) == 1)")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DSA_FP8_E4M3
    raise DsaError(f"unsupported dtype {t.dtype}")


def _mode(mode):
    return {"in_seq": IN_SEQ, "round_robin": ROUND_ROBIN, IN_SEQ: IN_SEQ, ROUND_ROBIN: ROUND_ROBIN}[mode]


def cp_sizes(num_tokens, cp_size, cp_rank, mode, pad_to_cp):
    """(tokens_per_rank, n_local_real, num_rows_concat) of a rank (host only)."""
    a, b, c = c_i32(), c_i32(), c_i32()
    _check(lib().dsa_cp_sizes(num_tokens, cp_size, cp_rank, _mode(mode), int(pad_to_cp), ctypes.byref(a),
                              ctypes.byref(b), ctypes.byref(c)), "dsa_cp_sizes")
    return a.value, b.value, c.value


def build_cp_metadata(query_start_loc, seq_lens, num_tokens, cp_size, cp_rank, mode, pad_to_cp=False,
                      token_map=True, err_flag=None, stream=None):
    """Run the metadata kernel; returns a dict of int32 device tensors."""
    dev = query_start_loc.device
    _dense("query_start_loc", query_start_loc, torch.int32)
    _dense("seq_lens", seq_lens, torch.int32)
    _dense("err_flag", err_flag, torch.int32, optional=True)
    B = seq_lens.numel()
    tpr, _, _ = cp_sizes(num_tokens, cp_size, cp_rank, mode, pad_to_cp)
    out = {
        "local_query_start_loc": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "local_seq_lens": torch.empty(max(B, 1), dtype=torch.int32, device=dev),
        "local_kv_start_loc": torch.empty(B + 1, dtype=torch.int32, device=dev),
        "scalars": torch.empty(8, dtype=torch.int32, device=dev),
        "token_map": torch.empty(max(tpr, 1), dtype=torch.int32, device=dev) if token_map else None,
    }
    _check(lib().dsa_build_cp_metadata(
        _ptr(query_start_loc), _ptr(seq_lens), B, num_tokens, cp_size, cp_rank, _mode(mode), int(pad_to_cp),
        _ptr(out["local_query_start_loc"]), _ptr(out["local_seq_lens"]), _ptr(out["local_kv_start_loc"]),
        _ptr(out["scalars"]), _ptr(out["token_map"]), _ptr(err_flag), _stream(stream)), "dsa_build_cp_metadata")
    out["local_seq_lens"] = out["local_seq_lens"][:B]
    if token_map:
        out["token_map"] = out["token_map"][:tpr]
    return out


def _indexer_args(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv, q_stride=1,
                  compress_ratio=1, topk=2048, kv_row_base=0, window=0, window_kv_start=None, q_scale=None,
                  k_scale=None, topk_idx=None, workspace=None, err_flag=None, memory=True):
    _dense("q_idx", q_idx, memory=memory)
    _dense("k_idx", k_idx, q_idx.dtype, memory=memory)
    _dense("weights", weights, torch.float32, memory=memory)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("seqused_kv", seqused_kv), ("cu_seqlens_kv", cu_seqlens_kv)):
        _dense(name, t, torch.int32, memory=memory)
    _dense("window_kv_start", window_kv_start, torch.int32, optional=True, memory=memory)
    _dense("q_scale", q_scale, torch.float32, optional=True, memory=memory)
    _dense("k_scale", k_scale, torch.float32, optional=True, memory=memory)
    _dense("topk_idx", topk_idx, torch.int32, optional=True, memory=memory)
    _dense("workspace", workspace, optional=True, memory=memory)
    _dense("err_flag", err_flag, torch.int32, optional=True, memory=memory)
    if topk_idx is not None and tuple(topk_idx.shape) != (q_idx.shape[0], int(topk) + int(window)):
        raise DsaError(f"topk_idx must be [{q_idx.shape[0]}, {int(topk) + int(window)}], got {tuple(topk_idx.shape)}")
    a = IndexerArgs()
    a.q_idx, a.q_scale, a.weights = _ptr(q_idx), _ptr(q_scale), _ptr(weights)
    a.k_idx, a.k_scale = _ptr(k_idx), _ptr(k_scale)
    a.dtype = _dtype_code(q_idx)
    a.nq, a.n_heads, a.head_dim = q_idx.shape[0], q_idx.shape[1], q_idx.shape[2]
    a.nk = k_idx.shape[0]
    a.batch = seqused_kv.numel()
    a.cu_seqlens_q, a.seqused_kv, a.cu_seqlens_kv = _ptr(cu_seqlens_q), _ptr(seqused_kv), _ptr(cu_seqlens_kv)
    a.max_seqlen_kv, a.q_stride, a.compress_ratio = int(max_seqlen_kv), int(q_stride), int(compress_ratio)
    a.topk, a.kv_row_base, a.window = int(topk), int(kv_row_base), int(window)
    a.window_kv_start, a.topk_idx = _ptr(window_kv_start), _ptr(topk_idx)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.err_flag = _ptr(err_flag)
    return a


def indexer_topk_workspace(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv, **kw):
    """Workspace bytes of indexer_topk (host only: no tensor memory is read)."""
    a = _indexer_args(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv, memory=False,
                      **kw)
    n = lib().dsa_indexer_topk_workspace(ctypes.byref(a))
    if n == 0:
        raise DsaError(lib().dsa_last_error().decode())
    return n


def indexer_topk(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv, topk_idx=None,
                 workspace=None, stream=None, **kw):
    """Indexer scores + top-k into topk_idx [nq, topk + window] (allocated if not given)."""
    topk = kw.get("topk", 2048)
    window = kw.get("window", 0)
    if topk_idx is None:
        topk_idx = torch.empty(q_idx.shape[0], topk + window, dtype=torch.int32, device=q_idx.device)
    if workspace is None:
        n = indexer_topk_workspace(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv, **kw)
        workspace = torch.empty(n, dtype=torch.uint8, device=q_idx.device)
    a = _indexer_args(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv,
                      topk_idx=topk_idx, workspace=workspace, **kw)
    _check(lib().dsa_indexer_topk(ctypes.byref(a), _stream(stream)), "dsa_indexer_topk")
    return topk_idx


def indexer_topk_noalloc(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv, topk_idx,
                         stream=None, **kw):
    """indexer_topk for callers that cannot allocate: the library's static per-GPU scratch (64 MiB)
    instead of a workspace; topk_idx [nq, topk + window] int32 must be given. Calls that overlap on
    one GPU race. Allocates nothing."""
    if topk_idx is None:
        raise DsaError("indexer_topk_noalloc: topk_idx must be given (this call allocates nothing)")
    a = _indexer_args(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv,
                      topk_idx=topk_idx, **kw)
    _check(lib().dsa_indexer_topk_noalloc(ctypes.byref(a), _stream(stream)), "dsa_indexer_topk_noalloc")
    return topk_idx


def indexer_topk_timed(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv, events,
                       topk_idx, workspace, stream=None, **kw):
    """indexer_topk with events[k] recorded right before the k-th kernel it launches and events[n]
    right after the last; returns the n kernel names. events: torch.cuda.Event(enable_timing=True)
    objects that have been recorded once already (torch creates the HIP event on first record)."""
    handles = [int(e.cuda_event) for e in events]
    if len(handles) < 2 or not all(handles):
        raise DsaError("indexer_topk_timed: need at least 2 events, each recorded once before")
    arr = (c_p * len(handles))(*handles)
    names = (ctypes.c_char_p * len(handles))()
    n = c_i32(0)
    a = _indexer_args(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv,
                      topk_idx=topk_idx, workspace=workspace, **kw)
    _check(lib().dsa_indexer_topk_timed(ctypes.byref(a), _stream(stream), arr, len(handles), ctypes.byref(n), names),
           "dsa_indexer_topk_timed")
    return [names[k].decode() for k in range(n.value)]


def indexer_scores(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv, scores,
                   stream=None, **kw):
    _rows("scores", scores, torch.float32)
    a = _indexer_args(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv, **kw)
    _check(lib().dsa_indexer_scores(ctypes.byref(a), _ptr(scores), scores.stride(0), _stream(stream)),
           "dsa_indexer_scores")
    return scores


def topk_from_scores(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv, scores,
                     topk_idx=None, stream=None, **kw):
    topk = kw.get("topk", 2048)
    window = kw.get("window", 0)
    if topk_idx is None:
        topk_idx = torch.empty(q_idx.shape[0], topk + window, dtype=torch.int32, device=scores.device)
    _rows("scores", scores, torch.float32)
    a = _indexer_args(q_idx, weights, k_idx, cu_seqlens_q, seqused_kv, cu_seqlens_kv, max_seqlen_kv,
                      topk_idx=topk_idx, **kw)
    _check(lib().dsa_topk_from_scores(ctypes.byref(a), _ptr(scores), scores.stride(0), _stream(stream)),
           "dsa_topk_from_scores")
    return topk_idx


def clock_probe(out, ticks=20000, stream=None):
    """Enqueue the clock probe: out (uint64 or int64 GPU tensor of 4) receives the shader-clock and
    100 MHz real-time counters before and after a spin of `ticks` real-time ticks."""
    _dense("out", out, (torch.int64,))
    if out.numel() < 4:
        raise DsaError("clock_probe: out needs 4 entries")
    _check(lib().dsa_clock_probe(_ptr(out), int(ticks), _stream(stream)), "dsa_clock_probe")
    return out


def probe_mhz(out):
    """The shader clock in MHz from a clock_probe result (host copy of its 4 counters)."""
    c0, c1, r0, r1 = (int(x) for x in out[:4])
    return 100.0 * (c1 - c0) / max(r1 - r0, 1)


def lds_mfma_probe(operand, waves_per_simd, iters, cycles, sink, stream=None):
    """Enqueue the LDS-fed MFMA probe (operand 0: K-form reads, 1: V-form transposed reads, 2: none);
    cycles (int64 GPU tensor, >= 2048) receives per-wave shader-clock cycles at [8 * block + wave],
    sink (float32 GPU tensor, >= 256 * 256 * waves_per_simd) keeps the MFMA chains live."""
    _dense("cycles", cycles, (torch.int64,))
    _dense("sink", sink, torch.float32)
    _check(lib().dsa_lds_mfma_probe(int(operand), int(waves_per_simd), int(iters), _ptr(cycles), cycles.numel(),
                                    _ptr(sink), sink.numel(), _stream(stream)), "dsa_lds_mfma_probe")
    return cycles


def lds_mfma_busy(cycles, waves_per_simd, iters):
    """MFMA busy fraction per SIMD from a lds_mfma_probe result (host array of the 2048 counts):
    the median over workgroups of the slowest wave's loop."""
    import numpy as np
    c = np.asarray(cycles, dtype=np.int64).reshape(256, 8)[:, :4 * waves_per_simd].max(axis=1)
    return 32.0 * 32 * iters * waves_per_simd / float(np.median(c))


def sparse_attn(q, kv, idx, sink, softmax_scale, d_v, out=None, lse=None, err_flag=None, stream=None):
    """Sparse attention of q [nq, H, D_qk] over kv rows idx [nq, k_tot]; returns out [nq, H, d_v]."""
    nq, H, Dqk = q.shape
    if out is None:
        out = torch.empty(nq, H, d_v, dtype=q.dtype, device=q.device)
    _dense("q", q)
    _dense("kv", kv, q.dtype)
    _dense("idx", idx, torch.int32, optional=True)
    _dense("sink", sink, torch.float32, optional=True)
    _dense("out", out, q.dtype)
    _dense("lse", lse, torch.float32, optional=True)
    _dense("err_flag", err_flag, torch.int32, optional=True)
    if tuple(out.shape) != (nq, H, d_v):
        raise DsaError(f"out must be [{nq}, {H}, {d_v}], got {tuple(out.shape)}")
    if idx is not None and (idx.dim() != 2 or idx.shape[0] != nq):
        raise DsaError(f"idx must be [{nq}, k_tot], got {tuple(idx.shape)}")
    if sink is not None and sink.numel() != H:
        raise DsaError(f"sink must hold {H} values, got {sink.numel()}")
    if lse is not None and tuple(lse.shape) != (nq, H):
        raise DsaError(f"lse must be [{nq}, {H}], got {tuple(lse.shape)}")
    a = AttnArgs()
    a.q, a.kv, a.idx, a.sink, a.out, a.lse, a.err_flag = (_ptr(q), _ptr(kv), _ptr(idx), _ptr(sink), _ptr(out),
                                                          _ptr(lse), _ptr(err_flag))
    a.softmax_scale = float(softmax_scale)
    a.dtype = _dtype_code(q)
    a.nq, a.n_rows, a.n_heads, a.d_qk, a.d_v = nq, kv.shape[0], H, Dqk, d_v
    a.k_tot = idx.shape[1] if idx is not None else 0
    _check(lib().dsa_sparse_attn(ctypes.byref(a), _stream(stream)), "dsa_sparse_attn")
    return out


def rerange(x, num_tokens, cp_size, mode, pad_to_cp, inverse=False, out=None, stream=None):
    """Rank-concatenated rows -> logical order (inverse=False), or the split (inverse=True)."""
    _, _, rows_concat = cp_sizes(num_tokens, cp_size, 0, mode, pad_to_cp)
    n_out = rows_concat if inverse else num_tokens
    if out is None:
        out = torch.empty((n_out,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    _dense("x", x)
    _dense("out", out, x.dtype)
    n_in = num_tokens if inverse else rows_concat
    if x.shape[0] < n_in or out.shape[0] < n_out or tuple(x.shape[1:]) != tuple(out.shape[1:]):
        raise DsaError(f"rerange: x needs {n_in} rows and out {n_out} rows of the same shape")
    row_bytes = x[0].numel() * x.element_size() if x.shape[0] else out[0].numel() * out.element_size()
    _check(lib().dsa_rerange(_ptr(x), _ptr(out), num_tokens, row_bytes, cp_size, _mode(mode), int(pad_to_cp),
                             int(inverse), _stream(stream)), "dsa_rerange")
    return out
