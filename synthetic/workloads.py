"""The five synthetic DSA-prefill workloads and their seeded input tensors.

Shapes follow the pages' long-prefill scenarios with DeepSeek-V3.2/V4 attention shapes:
128 query heads over a 576-wide shared latent row (512 latent + 64 rope, value = the first
512 columns), a 64-head x 128 lightning indexer and top-k 2048, plus one tiny fp32 case.

Recipe (every workload): values are drawn in float64 from numpy's PCG64, seeded by
SeedSequence([workload_id, tensor_id, block]) and rounded once (RNE) to the storage dtype.
  q, kv         ~ N(0,1)/sqrt(D_qk)        q_idx, k_idx ~ N(0,1)/sqrt(D_i)
  w             ~ N(0,1)/sqrt(H_i)         sink         ~ N(0,1)
Per-query tensors (q, q_idx, w, q_scale) are seeded per token, by the KV-stream row the token
occupies, so any rank's rows can be drawn alone, every rank sees the same value for the same
token, and a chunk of a request carries the same values as that part of the whole request.
Full-stream tensors (kv, k_idx, k_scale) are seeded per block of 64 KV rows.

Chunked prefill: request b may carry a cached prefix of prefix[b] tokens.  Its KV segment
then holds prefix[b] + lens[b] rows (prefix first) and the segments follow one another in
request order; the queries are the lens[b] new tokens only.

Variants: "normal" (above), "unit" (q, kv, q_idx, k_idx ~ N(0,1): logits of order one) and
"int" (q_idx, k_idx integers in [-4,4], w integers in [-2,2], fp8 scales powers of two, so
every indexer score is an exact small integer multiple of a power of two in fp32 and fp64).
"""
from dataclasses import dataclass, field
import numpy as np

from .encode import f64_to_bf16_bits, f64_to_e4m3fn_bytes, E4M3FN_MAX

T_KV, T_KIDX, T_KSCALE, T_SINK, T_Q, T_QIDX, T_W, T_QSCALE, T_RR, T_SCORES = range(1, 11)
STREAM_BLOCK = 64


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed id
    lens: tuple              # query tokens per request (the new tokens)
    cp: int
    rank: int
    mode: str                # "in_seq" | "round_robin"
    pad: bool                # pad the flattened stream to a multiple of cp
    H: int
    Dqk: int
    Dv: int
    attn_dtype: str          # "f32" | "bf16"
    Hi: int
    Di: int
    idx_dtype: str           # "f32" | "bf16" | "fp8"
    topk: int
    window: int = 0          # sliding-window rows appended to the top-k rows
    compress: int = 1        # indexer runs over keys compressed by this ratio
    rerange: bool = False    # also permute a rank-concatenated [T, D_qk] buffer
    notes: str = ""
    prefix: tuple = ()       # cached tokens before each request's queries (empty: none)

    @property
    def T(self):
        return int(sum(self.lens))

    @property
    def qsl(self):
        return np.concatenate([[0], np.cumsum(np.asarray(self.lens, dtype=np.int64))]).astype(np.int32)

    @property
    def seq_lens(self):
        """KV tokens per request: cached prefix plus the new tokens."""
        p = self.prefix or (0,) * len(self.lens)
        return (np.asarray(self.lens, dtype=np.int64) + np.asarray(p, dtype=np.int64)).astype(np.int32)

    @property
    def kvsl(self):
        """Start row of each request's KV segment, [B+1]."""
        return np.concatenate([[0], np.cumsum(self.seq_lens.astype(np.int64))]).astype(np.int32)

    @property
    def n_kv(self):
        return int(self.seq_lens.astype(np.int64).sum())

    @property
    def k_tot(self):
        return self.topk + self.window

    def with_(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def _var_lens():
    rng = np.random.default_rng(np.random.SeedSequence([5, 0]))
    return tuple(int(v) for v in rng.integers(1024, 16385, size=8))


WORKLOADS = {
    "tiny_fp32_cp1": Workload(
        "tiny_fp32_cp1", 1, (512,), 1, 0, "in_seq", False, 16, 160, 128, "f32", 4, 32, "f32", 64,
        notes="1 x 512 tokens, cp 1; 16 heads over 128+32 latent, 4x32 fp32 indexer, top-k 64"),
    "inseq_cp8_last_8k": Workload(
        "inseq_cp8_last_8k", 2, (8192,), 8, 7, "in_seq", False, 128, 576, 512, "bf16", 64, 128, "bf16", 2048,
        notes="contiguous split, cp 8, last rank: 1024 queries over 8192 KV"),
    "rr_cp8_r3_batch4": Workload(
        "rr_cp8_r3_batch4", 3, (32768, 8192, 2048, 5), 8, 3, "round_robin", False, 128, 576, 512, "bf16",
        64, 128, "bf16", 2048, rerange=True,
        notes="round-robin cp 8, rank 3, requests 32768/8192/2048/5; rerange of [T,576] bf16"),
    "long_131k_fp8": Workload(
        "long_131k_fp8", 4, (131072,), 8, 7, "in_seq", False, 128, 576, 512, "bf16", 64, 128, "fp8", 2048,
        notes="131072 tokens, contiguous cp 8 last rank (16384 queries); fp8 e4m3 indexer"),
    "chunk_inseq_cp8_last_8k_p56k": Workload(
        "chunk_inseq_cp8_last_8k_p56k", 6, (8192,), 8, 7, "in_seq", False, 128, 576, 512, "bf16", 64, 128,
        "bf16", 2048, prefix=(57344,),
        notes="chunked prefill: an 8192-token chunk after a 57344-token cached prefix, contiguous cp 8, "
              "last rank: 1024 queries over up to 65536 KV"),
    "rr_cp4_r1_var8_cmp4": Workload(
        "rr_cp4_r1_var8_cmp4", 5, _var_lens(), 4, 1, "round_robin", True, 128, 576, 512, "bf16", 64, 128,
        "bf16", 2048, window=128, compress=4,
        notes="8 requests U[1024,16384], padded round-robin cp 4 rank 1; x4-compressed indexer, top-k 2048 "
              "plus a 128-token window"),
    "rr_cp4_r1_var8_cmp128": Workload(
        "rr_cp4_r1_var8_cmp128", 7, _var_lens(), 4, 1, "round_robin", True, 128, 576, 512, "bf16", 64, 128,
        "bf16", 2048, window=128, compress=128,
        notes="the same 8 requests and split with x128-compressed keys: at most 128 visible blocks per query, "
              "so the top-k 2048 keeps every one, plus a 128-token window"),
}


def _rng(wid, tid, block, variant):
    vtag = {"normal": 0, "unit": 1, "int": 2}[variant]
    return np.random.default_rng(np.random.SeedSequence([wid, tid, vtag, int(block)]))


def _store(x, dtype):
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    raise ValueError(dtype)


def bf16_bits_to_f64(b):
    """Widen stored bfloat16 bit patterns (input preparation only: the compressor stand-in)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _stream_rows(wl, tid, n_rows, width, draw):
    out = np.empty((n_rows, width), dtype=np.float64)
    for blk in range((n_rows + STREAM_BLOCK - 1) // STREAM_BLOCK):
        a = blk * STREAM_BLOCK
        b = min(n_rows, a + STREAM_BLOCK)
        out[a:b] = draw(_rng(wl.wid, tid, blk, wl._variant), (b - a, width))
    return out


def _normal(scale):
    return lambda g, shape: g.standard_normal(shape) * scale


def _ints(lo, hi):
    return lambda g, shape: g.integers(lo, hi + 1, size=shape).astype(np.float64)


def _quant_fp8_rows(x):
    """Per-row scale amax/448 (float32, positive) and E4M3FN codes of x/scale."""
    amax = np.max(np.abs(x), axis=-1, keepdims=True)
    scale = np.maximum(amax / E4M3FN_MAX, 2.0 ** -60).astype(np.float32)
    codes = f64_to_e4m3fn_bytes(x / scale.astype(np.float64))
    return codes, scale[..., 0]


class _WL:
    """Workload plus the chosen variant (kept out of the frozen dataclass)."""

    def __init__(self, wl, variant):
        self.__dict__.update(wl.__dict__)
        self._variant = variant
        self.T = wl.T
        self.qsl = wl.qsl
        self.seq_lens = wl.seq_lens
        self.kvsl = wl.kvsl
        self.n_kv = wl.n_kv


def stream_inputs(wl: Workload, variant="normal"):
    """Full-stream tensors: kv rows, indexer keys (+ fp8 scales), sink; compressed stand-ins.

    Returns a dict of numpy arrays in storage dtype (N = n_kv KV rows, = T without prefixes):
      kv      [N + Nc, D_qk]  (Nc compressed latent rows follow the N token rows when compress > 1)
      k_idx   [N or Nc, D_i]  (compressed keys only when compress > 1)
      k_scale [N] float32     (fp8 only)
      sink    [H] float32
      kv_cmp_start [B+1] int32 (compress > 1: offset of request b's compressed rows)
    """
    w = _WL(wl, variant)
    T = wl.n_kv
    unit = variant == "unit"
    out = {"qsl": wl.qsl, "seq_lens": wl.seq_lens}
    kv = _stream_rows(w, T_KV, T, wl.Dqk, _normal(1.0 if unit else 1.0 / np.sqrt(wl.Dqk)))
    if variant == "int":
        kidx = _stream_rows(w, T_KIDX, T, wl.Di, _ints(-4, 4))
    else:
        kidx = _stream_rows(w, T_KIDX, T, wl.Di, _normal(1.0 if unit else 1.0 / np.sqrt(wl.Di)))
    out["sink"] = _rng(wl.wid, T_SINK, 0, variant).standard_normal(wl.H).astype(np.float32)

    kv_st = _store(kv, wl.attn_dtype)
    if wl.idx_dtype == "fp8":
        if variant == "int":
            codes = f64_to_e4m3fn_bytes(kidx)
            sc = np.ldexp(1.0, -_stream_rows(w, T_KSCALE, T, 1, _ints(0, 3))[:, 0].astype(np.int64))
            out["k_idx"], out["k_scale"] = codes, sc.astype(np.float32)
        else:
            out["k_idx"], out["k_scale"] = _quant_fp8_rows(kidx)
    else:
        out["k_idx"] = _store(kidx, wl.idx_dtype)

    if wl.compress > 1:
        # Compressor stand-in: mean of each non-overlapping block of `compress` tokens of a
        # request's KV segment (trailing partial block dropped), computed in float64 from the
        # stored values and rounded once.  The pages name a compressor but do not define it.
        r = wl.compress
        kvsl = wl.kvsl
        nblk = [int(l) // r for l in wl.seq_lens]
        kv_dec = kv_st.astype(np.float64) if wl.attn_dtype == "f32" else bf16_bits_to_f64(kv_st)
        kidx_dec = out["k_idx"].astype(np.float64) if wl.idx_dtype == "f32" else bf16_bits_to_f64(out["k_idx"])
        kv_c, ki_c = [], []
        for b in range(len(wl.lens)):
            s = int(kvsl[b])
            n = nblk[b]
            kv_c.append(kv_dec[s:s + n * r].reshape(n, r, wl.Dqk).mean(axis=1))
            ki_c.append(kidx_dec[s:s + n * r].reshape(n, r, wl.Di).mean(axis=1))
        kv_c = np.concatenate(kv_c) if kv_c else np.zeros((0, wl.Dqk))
        ki_c = np.concatenate(ki_c) if ki_c else np.zeros((0, wl.Di))
        kv_st = np.concatenate([kv_st, _store(kv_c, wl.attn_dtype)])
        out["k_idx"] = _store(ki_c, wl.idx_dtype)
        out["kv_cmp_start"] = np.concatenate([[0], np.cumsum(nblk)]).astype(np.int32)
    out["kv"] = kv_st
    return out


def query_inputs(wl: Workload, tokens, variant="normal", indexer_only=False):
    """Per-query tensors for the given global token ids (pads: id < 0 give zero rows).

    Returns q [n,H,D_qk], q_idx [n,H_i,D_i], w [n,H_i] float32, and q_scale [n,H_i] for fp8,
    filled token by token straight into the storage dtype.  Token t of request b is seeded by
    its KV row kvsl[b] + prefix[b] + (t - qsl[b]) (= t without prefixes).  indexer_only: q is
    left out (the indexer tensors are the same values either way).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    n = len(tokens)
    qsl = wl.qsl.astype(np.int64)
    req = np.clip(np.searchsorted(qsl, tokens, side="right") - 1, 0, max(len(wl.lens) - 1, 0))
    kv_row = (wl.kvsl.astype(np.int64)[req] + (wl.seq_lens.astype(np.int64) - np.diff(qsl))[req]
              + tokens - qsl[req]) if len(wl.lens) else tokens
    unit = variant == "unit"
    sq = 1.0 if unit else 1.0 / np.sqrt(wl.Dqk)
    si = 1.0 if unit else 1.0 / np.sqrt(wl.Di)
    q = np.zeros((0 if indexer_only else n, wl.H, wl.Dqk), dtype=np.float32 if wl.attn_dtype == "f32" else np.uint16)
    fp8 = wl.idx_dtype == "fp8"
    qi = np.zeros((n, wl.Hi, wl.Di), dtype={"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[wl.idx_dtype])
    w = np.zeros((n, wl.Hi), dtype=np.float32)
    qs = np.ones((n, wl.Hi), dtype=np.float32)
    for j, t in enumerate(tokens):
        if t < 0:
            continue
        row = int(kv_row[j])
        if not indexer_only:
            g = _rng(wl.wid, T_Q, row, variant)
            q[j] = _store(g.standard_normal((wl.H, wl.Dqk)) * sq, wl.attn_dtype)
        g = _rng(wl.wid, T_QIDX, row, variant)
        if variant == "int":
            x = g.integers(-4, 5, size=(wl.Hi, wl.Di)).astype(np.float64)
            w[j] = g.integers(-2, 3, size=wl.Hi)
            if fp8:
                qs[j] = np.ldexp(1.0, -g.integers(0, 4, size=wl.Hi))
        else:
            x = g.standard_normal((wl.Hi, wl.Di)) * si
            w[j] = g.standard_normal(wl.Hi) / np.sqrt(wl.Hi)
        if fp8:
            if variant == "int":
                qi[j] = f64_to_e4m3fn_bytes(x)
            else:
                qi[j], qs[j] = _quant_fp8_rows(x)
        else:
            qi[j] = _store(x, wl.idx_dtype)
    out = {"q": q, "w": w, "q_idx": qi}
    if fp8:
        out["q_scale"] = qs
    return out


def rerange_buffer(wl: Workload, n_rows, width=None, variant="normal"):
    """A [n_rows, width] bf16 buffer of random rows (content is irrelevant to a permutation)."""
    width = width or wl.Dqk
    g = _rng(wl.wid, T_RR, 0, variant)
    return g.integers(0, 1 << 16, size=(n_rows, width), dtype=np.uint16)


def score_rows(seed, n_rows, length, kind="normal"):
    """Random fp32 score rows for isolated top-k tests.

    kind: "normal" (distinct values), "ties" (few distinct values, many exact ties),
          "zeros" (mixture of +0.0 and -0.0 and a few positives), "const" (all equal),
          "narrow" (mostly distinct values packed into [1, 1 + 2^-10), so that they share their
          sign, exponent and leading mantissa bits).
    """
    g = np.random.default_rng(np.random.SeedSequence([seed, T_SCORES, {"normal": 0, "ties": 1, "zeros": 2,
                                                                     "const": 3, "narrow": 4}[kind]]))
    if kind == "normal":
        x = g.standard_normal((n_rows, length)).astype(np.float32)
    elif kind == "ties":
        x = g.integers(-3, 4, size=(n_rows, length)).astype(np.float32) * np.float32(0.25)
    elif kind == "zeros":
        x = np.where(g.random((n_rows, length)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        pos = g.random((n_rows, length)) < 0.01
        x = np.where(pos, g.random((n_rows, length)).astype(np.float32), x).astype(np.float32)
    elif kind == "narrow":
        x = (np.float32(1.0) + g.random((n_rows, length)).astype(np.float32) * np.float32(2.0 ** -10)).astype(np.float32)
    else:
        x = np.full((n_rows, length), 1.5, dtype=np.float32)
    return x


def make_inputs(wl: Workload, tokens, variant="normal"):
    """Stream tensors plus the per-query tensors of `tokens` (global ids, -1 = pad row)."""
    d = stream_inputs(wl, variant)
    d.update(query_inputs(wl, tokens, variant))
    return d
