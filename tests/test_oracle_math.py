"""Pins of the oracle's indexer scores, top-k and sparse attention.

Each pin is a closed form, an invariant, a special case that reduces to a library routine, a
property that characterises the result, or an independent brute-force path, chosen so that
a dropped term, a wrong sign, a wrong index or a transposed operand fails at least one.
"""
import numpy as np
import pytest
from scipy.special import softmax, expit

import oracle as O
import synthetic as S


# ----------------------------------------------------------------------------- decoding

def test_decode_bf16_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3F81, 0x7F7F, 0x0001, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 1.0 + 2 ** -7, (2 - 2 ** -7) * 2 ** 127, 2 ** -133, 3.140625]
    got = O.decode_bf16(bits)
    assert list(got) == want
    assert np.signbit(got[3])


def test_decode_e4m3fn_known_values():
    # OCP 8-bit floating point spec, E4M3: bias 7, max normal 448 = S.1111.110, min
    # subnormal 2^-9, no infinities, S.1111.111 is NaN.
    codes = np.array([0x38, 0x7E, 0xFE, 0x01, 0x08, 0x40, 0xC4, 0x00, 0x80, 0x3C], dtype=np.uint8)
    want = [1.0, 448.0, -448.0, 2 ** -9, 2 ** -6, 2.0, -3.0, 0.0, -0.0, 1.5]
    assert list(O.decode_e4m3fn(codes)) == want
    with pytest.raises(ValueError):
        O.decode_e4m3fn(np.array([0x7F], dtype=np.uint8))


def test_storage_round_trips():
    g = np.random.default_rng(0)
    x = g.standard_normal(2000)
    b = S.f64_to_bf16_bits(x)
    xb = O.decode_bf16(b)
    assert np.all(np.abs(xb - x) <= np.abs(x) * 2.0 ** -8)
    assert np.array_equal(S.f64_to_bf16_bits(xb), b)          # representable values are fixed points
    q = S.f64_to_e4m3fn_bytes(x * 100)
    xq = O.decode_e4m3fn(q)
    assert np.all(np.abs(xq) <= 448)
    assert np.array_equal(S.f64_to_e4m3fn_bytes(xq), q)


# ----------------------------------------------------------------------------- indexer

def test_indexer_closed_form_when_every_dot_is_positive():
    """All q, k > 0 and w >= 0: ReLU is the identity and the score is (sum_h w_h q_h) . k."""
    g = np.random.default_rng(1)
    q = g.random((4, 8)) + 0.1
    k = g.random((11, 8)) + 0.1
    w = g.random(4)
    got = O.indexer_scores_row(q, w, k)
    want = k @ (w @ q)
    assert np.allclose(got, want, rtol=1e-14, atol=0)


def test_indexer_relu_comes_before_the_weight():
    """Dots all negative: every score is exactly +0.0, whatever the sign of w."""
    q = np.array([[1.0, 2.0], [0.5, 1.0]])
    k = -np.array([[1.0, 1.0], [3.0, 0.5]])
    w = np.array([-2.0, -1.0])
    s = O.indexer_scores_row(q, w, k)
    assert list(s) == [0.0, 0.0] and not np.any(np.signbit(s))


def test_indexer_single_head_single_key_and_sign_of_weight():
    q = np.array([[1.0, -2.0, 3.0]])
    k = np.array([[2.0, 1.0, 1.0], [0.0, 1.0, 0.0]])
    assert list(O.indexer_scores_row(q, np.array([-1.5]), k)) == [-4.5, 0.0]
    assert list(O.indexer_scores_row(q, np.array([2.0]), k)) == [6.0, 0.0]


def test_indexer_head_and_key_permutations():
    g = np.random.default_rng(2)
    q, k, w = g.standard_normal((6, 5)), g.standard_normal((9, 5)), g.standard_normal(6)
    s = O.indexer_scores_row(q, w, k)
    ph, pk = g.permutation(6), g.permutation(9)
    assert np.allclose(O.indexer_scores_row(q[ph], w[ph], k), s, rtol=1e-13, atol=1e-15)
    assert np.allclose(O.indexer_scores_row(q, w, k[pk]), s[pk], rtol=0, atol=0)
    # linear in w, positively homogeneous in q
    w2 = g.standard_normal(6)
    assert np.allclose(O.indexer_scores_row(q, w + w2, k), s + O.indexer_scores_row(q, w2, k), atol=1e-13)
    assert np.allclose(O.indexer_scores_row(3 * q, w, k), 3 * s, atol=1e-13)


def test_indexer_integer_inputs_are_exact_integers():
    g = np.random.default_rng(3)
    q = g.integers(-4, 5, size=(64, 128)).astype(np.float64)
    k = g.integers(-4, 5, size=(50, 128)).astype(np.float64)
    w = g.integers(-2, 3, size=64).astype(np.float64)
    s = O.indexer_scores_row(q, w, k)
    assert np.array_equal(s, np.round(s))
    # brute force for two keys, head by head, in exact integer arithmetic
    qi, ki, wi = q.astype(np.int64), k.astype(np.int64), w.astype(np.int64)
    for j in (0, 49):
        exact = sum(int(wi[h]) * max(0, int(qi[h] @ ki[j])) for h in range(64))
        assert s[j] == exact


def test_fp8_dequantisation_uses_both_scales():
    """q8 * q_scale[head] and k8 * k_scale[token]: equal to the same values given unscaled."""
    g = np.random.default_rng(4)
    q8 = S.f64_to_e4m3fn_bytes(g.integers(-4, 5, size=(3, 16)))
    k8 = S.f64_to_e4m3fn_bytes(g.integers(-4, 5, size=(7, 16)))
    qs = np.array([0.5, 2.0, 0.25], dtype=np.float32)
    ks = np.array([1, 2, 4, 8, 0.5, 0.25, 1], dtype=np.float32)
    w = np.array([1.0, -1.0, 0.5])
    qh = O.dequant_q(q8, qs, "fp8")
    kh = O.dequant_k(k8, ks, "fp8")
    assert np.array_equal(qh, O.decode_e4m3fn(q8) * qs[:, None].astype(np.float64))
    assert np.array_equal(kh, O.decode_e4m3fn(k8) * ks[:, None].astype(np.float64))
    base = O.indexer_scores_row(O.decode_e4m3fn(q8), w * qs.astype(np.float64), O.decode_e4m3fn(k8))
    assert np.allclose(O.indexer_scores_row(qh, w, kh), base * ks.astype(np.float64), rtol=1e-15, atol=0)


def test_compressed_visibility_is_whole_blocks():
    """Block c of a request (tokens 4c..4c+3) is visible to position p iff 4c + 3 <= p."""
    for E in range(1, 40):
        p = E - 1
        n = O.visible_keys(E, 4)
        assert n == sum(1 for c in range(20) if 4 * c + 3 <= p)
    assert O.visible_keys(17, 1) == 17


# ----------------------------------------------------------------------------- top-k

def _check_topk_property(scores, K, pos):
    """The defining property: K picks (or all), and every pick beats every non-pick by
    (score desc, position asc)."""
    scores = np.asarray(scores, np.float64) + 0.0
    n = len(scores)
    assert len(pos) == min(n, K) and len(set(pos.tolist())) == len(pos)
    chosen = np.zeros(n, bool)
    chosen[pos] = True
    for s in np.flatnonzero(chosen):
        others = np.flatnonzero(~chosen)
        assert np.all((scores[s] > scores[others]) | ((scores[s] == scores[others]) & (s < others)))


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "const"])
def test_topk_satisfies_its_definition(kind):
    rows = S.workloads.score_rows(11, 12, 300, kind)
    for K in (1, 7, 64, 299, 300, 500):
        for r in rows:
            _check_topk_property(r, K, O.topk_positions(r, K))


def test_topk_small_examples():
    assert list(O.topk_positions([1, 3, 3, 2, 3], 2)) == [1, 2]
    assert list(O.topk_positions([1, 3, 3, 2, 3], 4)) == [1, 2, 3, 4]
    assert list(O.topk_positions([5.0, 6.0], 8)) == [0, 1]
    assert list(O.topk_positions([-0.0, 0.0, -1.0], 1)) == [0]
    assert list(O.topk_positions([0.0, -0.0, -1.0], 1)) == [0]
    assert list(O.topk_positions([], 3)) == []


def test_window_positions():
    assert list(O.window_positions(1, 128)) == [0]
    assert list(O.window_positions(200, 128)) == list(range(72, 200))
    assert len(O.window_positions(128, 128)) == 128 and O.window_positions(128, 128)[0] == 0


# ----------------------------------------------------------------------------- attention

def _rand_attn(seed, H=3, n=7, D=10, Dv=6, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal((H, D)) * scale, g.standard_normal((n, D)) * scale, g.standard_normal(H), Dv


def test_attention_without_sink_is_softmax_attention():
    q, kv, _, Dv = _rand_attn(20)
    sink = np.full(q.shape[0], -np.inf)
    o, lse = O.sparse_attention_row(q, kv, sink, 0.7, Dv)
    p = softmax(0.7 * q @ kv.T, axis=1)
    assert np.allclose(o, p @ kv[:, :Dv], rtol=1e-13, atol=1e-14)
    from scipy.special import logsumexp
    assert np.allclose(lse, logsumexp(0.7 * q @ kv.T, axis=1), rtol=1e-14)


def test_attention_one_key_is_a_logistic_gate():
    q, kv, sink, Dv = _rand_attn(21, n=1)
    o, lse = O.sparse_attention_row(q, kv, sink, 0.5, Dv)
    l = 0.5 * (q @ kv[0])
    assert np.allclose(o, expit(l - sink)[:, None] * kv[0, :Dv][None, :], rtol=1e-13, atol=1e-15)
    assert np.allclose(lse, np.logaddexp(l, sink), rtol=1e-14)


def test_attention_set_semantics_and_empty_set():
    q, kv, sink, Dv = _rand_attn(22, n=9)
    o, lse = O.sparse_attention_row(q, kv, sink, 0.3, Dv)
    perm = np.random.default_rng(0).permutation(9)
    o2, lse2 = O.sparse_attention_row(q, kv[perm], sink, 0.3, Dv)
    assert np.allclose(o, o2, rtol=1e-13, atol=1e-15) and np.allclose(lse, lse2, rtol=1e-14)
    o0, lse0 = O.sparse_attention_row(q, kv[:0], sink, 0.3, Dv)
    assert not o0.any() and np.array_equal(lse0, sink)


def test_attention_value_columns_are_the_leading_ones():
    """V = the first D_v columns; the logit uses every D_qk column (R-11). Hand-worked values."""
    kv = np.array([[1.0, 2.0, 3.0, 4.0], [5.0, 6.0, 7.0, 8.0]])
    # q = 0: both logits are 0, so out = (v_0 + v_1) / (e^0 + 2) with v = the first two columns
    o, lse = O.sparse_attention_row(np.zeros((1, 4)), kv, np.array([0.0]), 1.0, 2)
    assert np.allclose(o, [[2.0, 8.0 / 3.0]], rtol=1e-15, atol=0)
    assert np.isclose(lse[0], np.log(3.0), rtol=1e-15)
    # q reads the last column only: logits 4 and 8 come from columns the value does not use
    o, lse = O.sparse_attention_row(np.array([[0.0, 0.0, 0.0, 1.0]]), kv, np.array([0.0]), 1.0, 2)
    z = 1.0 + np.exp(4.0) + np.exp(8.0)
    assert np.allclose(o, [[(np.exp(4.0) * 1 + np.exp(8.0) * 5) / z, (np.exp(4.0) * 2 + np.exp(8.0) * 6) / z]],
                       rtol=1e-14, atol=0)
    assert np.isclose(lse[0], np.log(z), rtol=1e-15)


def test_attention_is_stable_at_large_logits():
    """Logits far past exp's float64 range: adding c to every logit and to the sink leaves the
    output unchanged and shifts lse by c; one logit 1000 above the rest returns its value row."""
    g = np.random.default_rng(24)
    v = g.standard_normal((6, 3))
    l = g.standard_normal(6)
    q = np.array([[0.0, 0.0, 0.0, 1.0]])
    sink = np.array([0.3])
    o, lse = O.sparse_attention_row(q, np.column_stack([v, l]), sink, 1.0, 3)
    for c in (800.0, -800.0, 1e5):
        o2, lse2 = O.sparse_attention_row(q, np.column_stack([v, l + c]), sink + c, 1.0, 3)
        assert np.allclose(o2, o, rtol=1e-9, atol=1e-12) and np.isclose(lse2[0], lse[0] + c, rtol=1e-13)
    l_dom = np.zeros(6)
    l_dom[2] = 1000.0
    o3, lse3 = O.sparse_attention_row(q, np.column_stack([v, l_dom]), np.array([0.0]), 1.0, 3)
    assert np.array_equal(o3[0], v[2]) and lse3[0] == 1000.0


@pytest.mark.parametrize("seed", [30, 31])
def test_sparse_with_every_key_equals_dense_causal_brute_force(seed):
    """top-k >= extent: the sparse path over all visible keys is dense causal attention."""
    g = np.random.default_rng(seed)
    T, H, D, Dv = 19, 3, 12, 8
    q = g.standard_normal((T, H, D))
    kv = g.standard_normal((T, D))
    sink = g.standard_normal(H)
    dense = O.dense_causal_attention(q, kv, sink, 0.4, Dv)
    for t in range(T):
        o, _ = O.sparse_attention_row(q[t], kv[:t + 1], sink, 0.4, Dv)
        assert np.allclose(o, dense[t], rtol=1e-12, atol=1e-14)


def test_dense_brute_force_sink_column():
    """Position 0 with one key: brute force agrees with the logistic closed form."""
    g = np.random.default_rng(32)
    q = g.standard_normal((1, 2, 4))
    kv = g.standard_normal((1, 4))
    sink = g.standard_normal(2)
    d = O.dense_causal_attention(q, kv, sink, 1.0, 3)
    assert np.allclose(d[0], expit(q[0] @ kv[0] - sink)[:, None] * kv[0, :3], rtol=1e-13)


# ----------------------------------------------------------------------------- whole path

def _tiny_wl(mode, cp, rank, pad, lens=(13, 7, 22), topk=6, compress=1, window=0):
    base = S.WORKLOADS["tiny_fp32_cp1"]
    return base.with_(lens=tuple(lens), cp=cp, rank=rank, mode=mode, pad=pad, H=4, Dqk=24, Dv=16,
                      Hi=3, Di=8, topk=topk, compress=compress, window=window)


@pytest.mark.parametrize("mode,pad,compress,window", [(O.IN_SEQ, False, 1, 0), (O.ROUND_ROBIN, False, 1, 0),
                                                       (O.ROUND_ROBIN, True, 4, 5)])
def test_all_ranks_reranged_equal_the_single_rank_run(mode, pad, compress, window):
    """Each rank's share computed alone, concatenated by rank and reranged, equals cp = 1."""
    wl1 = _tiny_wl(mode, 1, 0, pad, compress=compress, window=window)
    T = wl1.T
    inp = S.stream_inputs(wl1)
    m1 = O.cp_metadata(wl1.qsl, wl1.lens, 1, 0, mode, pad)
    full = O.run_path(m1, {**inp, **S.query_inputs(wl1, m1["token_map"])}, wl1)
    cp = 3
    parts = []
    for r in range(cp):
        wl = wl1.with_(cp=cp, rank=r)
        m = O.cp_metadata(wl.qsl, wl.lens, cp, r, mode, pad)
        res = O.run_path(m, {**inp, **S.query_inputs(wl, m["token_map"])}, wl)
        nrows = m["tokens_per_rank"] if pad else m["n_local_real"]
        part = np.zeros((nrows, wl.H, wl.Dv))
        part[:m["n_local_real"]] = res["out"]
        parts.append(part)
    back = O.rerange(np.concatenate(parts), T, cp, mode, pad)
    assert np.allclose(back, full["out"], rtol=1e-12, atol=1e-15)


def test_selected_rows_are_causal_and_absolute():
    wl = _tiny_wl(O.ROUND_ROBIN, 3, 1, False, topk=4)
    m = O.cp_metadata(wl.qsl, wl.lens, 3, 1, O.ROUND_ROBIN, False)
    inp = {**S.stream_inputs(wl), **S.query_inputs(wl, m["token_map"])}
    res = O.run_path(m, inp, wl)
    toks = m["token_map"][m["token_map"] >= 0]
    for t, ids in zip(toks, res["topk_ids"]):
        b = np.searchsorted(wl.qsl, t, side="right") - 1
        assert len(ids) == min(4, t - wl.qsl[b] + 1)
        assert np.all((ids >= wl.qsl[b]) & (ids <= t))


@pytest.mark.parametrize("mode,cp,rank,pad,compress,window", [
    (O.IN_SEQ, 1, 0, False, 1, 0), (O.IN_SEQ, 3, 2, False, 1, 0), (O.ROUND_ROBIN, 3, 1, False, 1, 0),
    (O.ROUND_ROBIN, 2, 1, True, 4, 5), (O.IN_SEQ, 2, 1, True, 4, 5)])
def test_chunked_prefill_equals_the_rows_of_the_whole_requests(mode, cp, rank, pad, compress, window):
    """R-17: the last chunk of each request, run after its cached prefix, gives exactly the rows
    the whole requests give at the same KV positions (same keys, same top-k, same output).

    The whole run is cp 1 pure prefill, whose rows are pinned above; a wrong prefix offset,
    extent or KV segment start in the chunked metadata changes the keys a row sees.
    """
    whole = _tiny_wl(O.IN_SEQ, 1, 0, False, lens=(13, 7, 22), topk=4, compress=compress, window=window)
    m1 = O.cp_metadata(whole.qsl, whole.seq_lens, 1, 0, O.IN_SEQ, False)
    inp = S.stream_inputs(whole)
    full = O.run_path(m1, {**inp, **S.query_inputs(whole, m1["token_map"])}, whole, want_scores=True)
    prefix = (9, 0, 17)
    chunk = whole.with_(lens=tuple(l - p for l, p in zip(whole.lens, prefix)), prefix=prefix,
                        mode=mode, cp=cp, rank=rank, pad=pad)
    assert list(chunk.seq_lens) == list(whole.lens)
    cinp = S.stream_inputs(chunk)
    for k in ("kv", "k_idx", "kv_cmp_start"):
        if k in inp:
            assert np.array_equal(cinp[k], inp[k]), k
    m = O.cp_metadata(chunk.qsl, chunk.seq_lens, cp, rank, mode, pad)
    toks = m["token_map"][m["token_map"] >= 0]
    assert len(toks) > 0
    res = O.run_path(m, {**cinp, **S.query_inputs(chunk, m["token_map"])}, chunk, want_scores=True)
    for n, t in enumerate(toks):
        b = int(np.searchsorted(chunk.qsl, t, side="right") - 1)
        row = int(whole.qsl[b]) + prefix[b] + int(t - chunk.qsl[b])    # KV row = whole-run row
        assert np.array_equal(res["scores"][n], full["scores"][row])
        assert np.array_equal(res["topk_ids"][n], full["topk_ids"][row])
        assert np.array_equal(res["window_ids"][n], full["window_ids"][row])
        assert np.array_equal(res["out"][n], full["out"][row])
        assert np.array_equal(res["lse"][n], full["lse"][row])


@pytest.mark.parametrize("mode,pad", [(O.IN_SEQ, False), (O.ROUND_ROBIN, True)])
def test_all_ranks_reranged_equal_the_single_rank_run_with_prefixes(mode, pad):
    """The rank reconstruction holds for chunked prefill too (R-17)."""
    wl1 = _tiny_wl(mode, 1, 0, pad, lens=(5, 7, 12), compress=4, window=3).with_(prefix=(8, 0, 10))
    inp = S.stream_inputs(wl1)
    m1 = O.cp_metadata(wl1.qsl, wl1.seq_lens, 1, 0, mode, pad)
    full = O.run_path(m1, {**inp, **S.query_inputs(wl1, m1["token_map"])}, wl1)
    cp = 3
    parts = []
    for r in range(cp):
        wl = wl1.with_(cp=cp, rank=r)
        m = O.cp_metadata(wl.qsl, wl.seq_lens, cp, r, mode, pad)
        res = O.run_path(m, {**inp, **S.query_inputs(wl, m["token_map"])}, wl)
        nrows = m["tokens_per_rank"] if pad else m["n_local_real"]
        part = np.zeros((nrows, wl.H, wl.Dv))
        part[:m["n_local_real"]] = res["out"]
        parts.append(part)
    back = O.rerange(np.concatenate(parts), wl1.T, cp, mode, pad)
    assert np.allclose(back, full["out"], rtol=1e-12, atol=1e-15)
