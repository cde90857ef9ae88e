"""Plain, slow, obviously-correct CPU oracle for DSA sparse-attention prefill on one CP rank.

TEST INFRASTRUCTURE ONLY.  Only tests/, the package smoke check and the benchmark's
CPU-baseline leg may import or call this module.  It shares no code with the HIP path.

Arithmetic: integers in int64; floating point decoded exactly from the stored bytes
(float32, bfloat16, OCP fp8 E4M3FN) and computed in float64.  A library matmul / sort /
exp is used as a step where the definition calls for one; nothing is blocked or fused.

Pages cited (by title and section):
  [xLLM-CP]    "feat: DeepSeek-V4 DSA context-parallel on NPU" (xLLM pull request page)
  [CP-blog]    "[DeepSeek v3.2] context parallel explained" (blog post on SGLang's NSA prefill CP)
  [CP-gathers] "The role of the two all-gathers in NSA prefill CP" (SGLang design note)

Readings of points the pages leave open are tagged R-n; they are listed with their reasons
in the design notes of this repository:
  R-1  in-seq local_start/local_end clamp to T; trailing ranks may hold only pad rows.
  R-2  every request keeps its entry; in-seq local_seq_lens[b] = P_b + clamp(local_end - qs_b, 0, len_b)
       (P_b = the cached prefix of R-17, 0 in pure prefill).
  R-3  multi-request in-seq split cuts the flattened stream.
  R-4  round-robin padding appends pad rows at the end of the flattened stream.
  R-5  round-robin local_seq_lens = extent of the request's last local query (P_b without one);
       local_kv_start_loc = where each request's KV segment starts (the global query_start_loc
       in pure prefill); per-query extents step by cp.
  R-6  a query sees itself (position p sees keys 0..p).
  R-7  one indexer key per token, shared by all indexer heads; weights per (token, head).
  R-8  fp8: q_hat = q8 * q_scale[token, head], k_hat = k8 * k_scale[token], scales > 0.
  R-9  -0.0 scores are canonicalised to +0.0 before ranking.
  R-10 top-k ties go to the lower key index; extent <= K keeps every key; ids are absolute rows.
  R-11 sink = natural-log logit per head, in the denominator only; V = first D_v columns.
  R-12 compressed indexer: attend the selected compressed rows plus the window's original rows.
  R-13 window = the last `window` positions up to and including the query.
  R-16 unpadded round-robin rerange: rank r's rows start at sum_{r'<r} ceil((T - r')/cp).
  R-17 seq_lens[b] >= the query length n_b; the difference P_b is a cached prefix (chunked
       prefill).  Request b's KV segment holds seq_lens[b] rows, prefix first, and the
       segments follow one another in request order; query g (0-based) of the request sits at
       KV position P_b + g.  Pure prefill is P_b = 0.
  R-18 local rows are ordered by global token index; pad rows come last.
"""
import numpy as np

IN_SEQ = "in_seq"
ROUND_ROBIN = "round_robin"


# ---------------------------------------------------------------------------------------------
# Decoding stored values (exact)
# ---------------------------------------------------------------------------------------------

def decode_bf16(bits):
    """bfloat16 bit patterns -> float64: sign, 8-bit exponent (bias 127), 7-bit mantissa."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    mag = np.where(e == 0, m * 2.0 ** (-133), (128 + m) * np.exp2(e.astype(np.float64) - 134))
    if np.any(e == 0xFF):
        raise ValueError("non-finite bfloat16 input")
    return sign * mag


def decode_e4m3fn(codes):
    """OCP fp8 E4M3FN bytes -> float64: bias 7, no infinities, S.1111.111 is NaN (rejected)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    if np.any((e == 15) & (m == 7)):
        raise ValueError("fp8 NaN input")
    mag = np.where(e == 0, m * 2.0 ** (-9), (8 + m) * np.exp2(e.astype(np.float64) - 10))
    return sign * mag


def decode(x, dtype):
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(x)
    if dtype == "fp8":
        return decode_e4m3fn(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------------------------
# O1  CP-local metadata
#   [xLLM-CP] Implementation §2 (CP-local metadata: num_tokens_pad, tokens_per_rank,
#   local_start/local_end, intersection with the global cu-seqlens, local_kv_start_loc as the
#   right-aligned cumsum of local_seq_lens; cp_size 1 is the identity view) and Design,
#   key points (local queries see a right-aligned KV extent; the last rank sees all of it).
#   [CP-blog] §2B (token t goes to rank t % cp_size; per-rank cu-seqlens are recomputed) and
#   Part 3.1 (per-rank counts differ by at most one).
# ---------------------------------------------------------------------------------------------

def check_lengths(qsl, seq_lens):
    qsl = np.asarray(qsl, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    if qsl.ndim != 1 or len(qsl) != len(seq_lens) + 1 or qsl[0] != 0:
        raise ValueError("query_start_loc must be [B+1] starting at 0")
    if np.any(np.diff(qsl) < 0):
        raise ValueError("query_start_loc must be non-decreasing")
    if np.any(seq_lens < np.diff(qsl)):                       # R-17
        raise ValueError("seq_lens must be at least the query lengths")
    return qsl, seq_lens


def kv_start_loc(seq_lens):
    """Row where each request's KV segment starts in the full stream (R-17): [B+1]."""
    return np.concatenate([[0], np.cumsum(np.asarray(seq_lens, dtype=np.int64))])


def local_tokens(T, cp_size, cp_rank, mode):
    """Global ids of the real tokens a rank owns, ascending (R-1, R-18)."""
    tpr = -(-T // cp_size) if T > 0 else 0
    if mode == IN_SEQ:
        a = min(cp_rank * tpr, T)
        b = min((cp_rank + 1) * tpr, T)
        return np.arange(a, b, dtype=np.int64)
    if mode == ROUND_ROBIN:
        return np.arange(cp_rank, T, cp_size, dtype=np.int64)
    raise ValueError(mode)


def cp_metadata(qsl, seq_lens, cp_size, cp_rank, mode, pad_to_cp):
    """The rank's local view of a batch of prefill requests.

    Returns a dict of numpy int64 arrays / ints:
      num_tokens_pad, tokens_per_rank, local_start, local_end, stride, n_local_real,
      max_seqlen_q, num_local_reqs,
      local_query_start_loc [B+1], local_seq_lens [B], local_kv_start_loc [B+1],
      token_map [tokens_per_rank] (global token id of each local row, -1 for pad rows).
    """
    qsl, seq_lens = check_lengths(qsl, seq_lens)
    if not (0 <= cp_rank < cp_size):
        raise ValueError("need 0 <= cp_rank < cp_size")
    B = len(seq_lens)
    T = int(qsl[B])
    num_tokens_pad = -(-T // cp_size) * cp_size
    tpr = num_tokens_pad // cp_size
    toks = local_tokens(T, cp_size, cp_rank, mode)
    if mode == IN_SEQ:
        stride = 1
        local_start = min(cp_rank * tpr, T)
        local_end = min((cp_rank + 1) * tpr, T)
    else:
        stride = cp_size
        local_start = min(cp_rank, T)
        local_end = int(toks[-1]) + 1 if len(toks) else local_start

    n_b = np.zeros(B, dtype=np.int64)
    lsl = np.zeros(B, dtype=np.int64)
    for b in range(B):
        qs, qe = int(qsl[b]), int(qsl[b + 1])
        prefix = int(seq_lens[b]) - (qe - qs)                        # R-17
        mine = toks[(toks >= qs) & (toks < qe)]
        n_b[b] = len(mine)
        if mode == IN_SEQ:                                           # R-2
            lsl[b] = prefix + min(max(local_end - qs, 0), qe - qs)
        else:                                                        # R-5
            lsl[b] = prefix + ((int(mine[-1]) - qs + 1) if len(mine) else 0)
    lqsl = np.concatenate([[0], np.cumsum(n_b)])
    if mode == IN_SEQ:
        lkv = np.concatenate([[0], np.cumsum(lsl)])                  # right-aligned cumsum
    else:
        lkv = kv_start_loc(seq_lens)                                 # R-5
    token_map = np.full(tpr, -1, dtype=np.int64)
    token_map[:len(toks)] = toks                                     # R-18: pads last
    # Unpadded round-robin: rows past the rank's real tokens are not rows at all; the map still
    # has tokens_per_rank entries and marks them -1.
    return dict(num_tokens_pad=num_tokens_pad, tokens_per_rank=tpr, local_start=local_start,
                local_end=local_end, stride=stride, n_local_real=len(toks),
                max_seqlen_q=int(n_b.max()) if B else 0, num_local_reqs=int((n_b > 0).sum()),
                local_query_start_loc=lqsl, local_seq_lens=lsl, local_kv_start_loc=lkv,
                token_map=token_map, n_per_req=n_b, pad_to_cp=bool(pad_to_cp), mode=mode)


def query_views(meta):
    """Per local real row i (in local order): request b, causal extent E, KV offset kv0.

    Right alignment generalised to stride cp: local query j of request b (0-based among the
    n_b local queries of b) sees E = local_seq_lens[b] - (n_b - 1 - j) * stride keys starting
    at row local_kv_start_loc[b] of the full stream ([xLLM-CP] Design, key points; R-5).
    """
    lqsl = meta["local_query_start_loc"]
    lsl = meta["local_seq_lens"]
    lkv = meta["local_kv_start_loc"]
    stride = meta["stride"]
    rows = []
    for b in range(len(lsl)):
        nb = int(lqsl[b + 1] - lqsl[b])
        for j in range(nb):
            rows.append((b, int(lsl[b] - (nb - 1 - j) * stride), int(lkv[b])))
    return rows


# ---------------------------------------------------------------------------------------------
# O2  Split and rerange
#   [CP-blog] §2B (split keeps rows cp_rank, cp_rank + cp, ...), Part 3 step B (after the
#   all-gather the rows are concatenated by rank, e.g. T0,T4,T1,T5,...; the rerange restores
#   T0,T1,T2,...).  [CP-gathers] Gather #1 (the helper restores logical order for both the
#   round-robin and the in-seq split).
# ---------------------------------------------------------------------------------------------

def rank_row_counts(T, cp_size, mode, pad_to_cp):
    """Rows each rank contributes to the rank-concatenated buffer."""
    tpr = -(-T // cp_size) if T > 0 else 0
    if pad_to_cp:
        return [tpr] * cp_size
    return [len(local_tokens(T, cp_size, r, mode)) for r in range(cp_size)]    # R-16


def split_concat(x, T, cp_size, mode, pad_to_cp):
    """Rank-concatenated buffer split_0 || ... || split_{cp-1} of the logical rows x[:T].

    Padded: every rank contributes tokens_per_rank rows; pad rows are zero.
    """
    x = np.asarray(x)
    parts = []
    counts = rank_row_counts(T, cp_size, mode, pad_to_cp)
    for r in range(cp_size):
        toks = local_tokens(T, cp_size, r, mode)
        part = np.zeros((counts[r],) + x.shape[1:], dtype=x.dtype)
        part[:len(toks)] = x[toks]
        parts.append(part)
    return np.concatenate(parts) if parts else x[:0]


def rerange(concat, T, cp_size, mode, pad_to_cp):
    """Logical-order rows from a rank-concatenated buffer: out[t] = concat[off(rank(t)) + k(t)]."""
    counts = rank_row_counts(T, cp_size, mode, pad_to_cp)
    off = np.concatenate([[0], np.cumsum(counts)])
    out = np.empty((T,) + concat.shape[1:], dtype=concat.dtype)
    for r in range(cp_size):
        toks = local_tokens(T, cp_size, r, mode)
        out[toks] = concat[off[r]:off[r] + len(toks)]
    return out


# ---------------------------------------------------------------------------------------------
# O3  Lightning-indexer scores
#   [xLLM-CP] Design, data-flow step (3) and Implementation §4: the indexer query, weights and
#   top-k run on the local rows, the index keys on the full stream.  Score of local query i
#   against key s:  sum_h w[i,h] * max(0, q_idx[i,h,:] . k_idx[s,:])   (R-7, R-8, R-9)
# ---------------------------------------------------------------------------------------------

def dequant_q(q_idx, q_scale, dtype):
    q = decode(q_idx, dtype)
    if dtype == "fp8":
        q = q * np.asarray(q_scale, dtype=np.float32).astype(np.float64)[..., None]
    return q


def dequant_k(k_idx, k_scale, dtype):
    k = decode(k_idx, dtype)
    if dtype == "fp8":
        k = k * np.asarray(k_scale, dtype=np.float32).astype(np.float64)[:, None]
    return k


def indexer_scores_row(q_hat, w, k_hat_rows):
    """q_hat [H_i, D_i], w [H_i], k_hat_rows [n, D_i] (float64) -> scores [n] float64."""
    per_head = k_hat_rows @ q_hat.T                       # [n, H_i]
    s = np.maximum(per_head, 0.0) @ np.asarray(w, dtype=np.float64)
    return s + 0.0                                        # R-9: -0.0 + 0.0 == +0.0


def visible_keys(E, compress):
    """Keys a query of causal extent E may score: E tokens, or floor(E/ratio) whole blocks."""
    return E // compress if compress > 1 else E


# ---------------------------------------------------------------------------------------------
# O4  Per-query causal top-k (+ sliding window)
#   [xLLM-CP] Design, step (3) and Implementation §5 (if the indexer metadata is not localised
#   the top-k collapses to position 0: the selection is per query, over its causal keys).
# ---------------------------------------------------------------------------------------------

def topk_positions(scores, K):
    """Positions of the K best scores: score descending, then position ascending (R-10)."""
    scores = np.asarray(scores, dtype=np.float64) + 0.0
    n = len(scores)
    if n <= K:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -scores))           # primary: -score, secondary: position
    return np.sort(order[:K])


def window_positions(E, window):
    """Positions max(0, p - window + 1) .. p of a query at position p = E - 1 (R-13)."""
    p = E - 1
    return np.arange(max(0, p - window + 1), p + 1, dtype=np.int64)


# ---------------------------------------------------------------------------------------------
# O5  Sparse attention with a per-head sink
#   [xLLM-CP] Design, data-flow step (4): attention of the local queries, all heads, over the
#   shared KV rows the indexer picked, output [T_local, heads, head_dim]; key points: the
#   attention sink is loaded for all heads (R-11).
# ---------------------------------------------------------------------------------------------

def sparse_attention_row(q_i, kv_rows, sink, scale, Dv):
    """q_i [H, D_qk], kv_rows [n, D_qk], sink [H] (float64) -> (out [H, D_v], lse [H]).

    l_s = scale * q . kv_s;  m = max(max_s l_s, sink);  Z = e^(sink-m) + sum_s e^(l_s-m);
    out = sum_s e^(l_s-m) kv_s[:D_v] / Z;  lse = m + ln Z.   An empty set gives out = 0.
    """
    sink = np.asarray(sink, dtype=np.float64)
    if len(kv_rows) == 0:
        return np.zeros((q_i.shape[0], Dv)), sink.copy()
    logits = scale * (q_i @ kv_rows.T)                    # [H, n]
    m = np.maximum(logits.max(axis=1), sink)
    p = np.exp(logits - m[:, None])
    Z = np.exp(sink - m) + p.sum(axis=1)
    out = (p @ kv_rows[:, :Dv]) / Z[:, None]
    return out, m + np.log(Z)


# ---------------------------------------------------------------------------------------------
# O7  Dense causal attention with sink, by brute force (an independent second path)
# ---------------------------------------------------------------------------------------------

def dense_causal_attention(q, kv, sink, scale, Dv):
    """One request, every position: q [T, H, D_qk], kv [T, D_qk] -> out [T, H, D_v].

    The sink is an extra key column with logit sink_h and a zero value row; position i sees
    keys 0..i.  Softmax over the T+1 columns is taken row by row in textbook form.
    """
    T, H, _ = q.shape
    logits = scale * np.einsum("thd,sd->hts", q, kv)      # [H, T, T]
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    logits[:, mask] = -np.inf
    full = np.concatenate([logits, np.broadcast_to(np.asarray(sink, np.float64)[:, None, None],
                                                   (H, T, 1))], axis=2)
    full = full - full.max(axis=2, keepdims=True)
    e = np.exp(full)
    probs = e / e.sum(axis=2, keepdims=True)
    values = np.concatenate([kv[:, :Dv], np.zeros((1, Dv))], axis=0)   # sink value = 0
    out = np.einsum("hts,sd->thd", probs, values)
    return out


# ---------------------------------------------------------------------------------------------
# The whole path for chosen local rows
# ---------------------------------------------------------------------------------------------

def run_path(meta, inputs, wl, rows=None, scale=None, want_scores=False):
    """Indexer -> top-k (+window) -> sparse attention for local rows `rows` (default: all).

    inputs: dict of stored arrays (q, q_idx, w, q_scale?, kv, k_idx, k_scale?, sink, seq_lens,
            kv_cmp_start? for compressed keys); q/q_idx/w/q_scale indexed by local row.
            kv holds the token rows of every request's KV segment (R-17), then, with
            compressed keys, the compressed rows.
    Returns dict with per-row lists: topk_ids (absolute KV rows, ascending), window_ids,
    out [n, H, D_v] float64, lse [n, H], and optionally the float64 score rows.
    """
    views = query_views(meta)
    if rows is None:
        rows = range(len(views))
    rows = list(rows)
    scale = (1.0 / np.sqrt(wl.Dqk)) if scale is None else scale
    kv = decode(inputs["kv"], wl.attn_dtype)
    k_hat = dequant_k(inputs["k_idx"], inputs.get("k_scale"), wl.idx_dtype)
    sink = np.asarray(inputs["sink"], dtype=np.float32).astype(np.float64)
    kvsl = kv_start_loc(inputs["seq_lens"])                   # R-17: request b's KV segment
    n_kv = int(kvsl[-1])
    res = dict(topk_ids=[], window_ids=[], out=np.zeros((len(rows), wl.H, wl.Dv)),
               lse=np.zeros((len(rows), wl.H)), scores=[])
    for n, i in enumerate(rows):
        b, E, kv0 = views[i]
        q_hat = dequant_q(inputs["q_idx"][i], None if "q_scale" not in inputs else inputs["q_scale"][i],
                          wl.idx_dtype)
        if wl.compress > 1:
            c0 = int(inputs["kv_cmp_start"][b])
            nvis = visible_keys(E, wl.compress)
            krows = k_hat[c0:c0 + nvis]
            sc = indexer_scores_row(q_hat, inputs["w"][i], krows)
            ids = n_kv + c0 + topk_positions(sc, wl.topk)  # compressed rows follow the token rows
        else:
            krows = k_hat[kv0:kv0 + E]
            sc = indexer_scores_row(q_hat, inputs["w"][i], krows)
            ids = kv0 + topk_positions(sc, wl.topk)
        win = (int(kvsl[b]) + window_positions(E, wl.window)) if wl.window else np.zeros(0, np.int64)
        res["topk_ids"].append(ids)
        res["window_ids"].append(win)
        if want_scores:
            res["scores"].append(sc)
        sel = np.concatenate([ids, win])
        q_i = decode(inputs["q"][i], wl.attn_dtype)
        o, lse = sparse_attention_row(q_i, kv[sel], sink, scale, wl.Dv)
        res["out"][n] = o
        res["lse"][n] = lse
    return res
