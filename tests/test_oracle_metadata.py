"""Pins of the oracle's CP-local metadata and split/rerange against what the pages fix.

Pages: [xLLM-CP] "feat: DeepSeek-V4 DSA context-parallel on NPU" (Implementation §2 and §8
unit tests: per-rank views, ranks partition the query tokens, cp_size 1 is the identity,
padding and boundary-crossing requests; Design key points: right-aligned KV extent, the last
rank sees the whole stream).  [CP-blog] "[DeepSeek v3.2] context parallel explained"
(Part 1 contiguous example, Part 3 round-robin example, counts differ by at most one).
"""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _qsl(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _random_batches(seed, n):
    g = np.random.default_rng(seed)
    for _ in range(n):
        B = int(g.integers(1, 6))
        lens = g.integers(0, 40, size=B)
        lens[g.integers(0, B)] = max(1, lens[0])
        yield [int(x) for x in lens]


MODES = [(O.IN_SEQ, False), (O.IN_SEQ, True), (O.ROUND_ROBIN, False), (O.ROUND_ROBIN, True)]


def test_golden_contiguous_8000_on_8():
    g = json.load(open(os.path.join(GOLDEN, "inseq_8000_cp8.json")))
    qsl = _qsl(g["lens"])
    for r, (a, b) in enumerate(g["rank_first_last_token"]):
        m = O.cp_metadata(qsl, g["lens"], g["cp_size"], r, O.IN_SEQ, False)
        assert list(m["token_map"]) == list(range(a, b + 1))
        assert list(m["local_query_start_loc"]) == [0, b + 1 - a]
        # right-aligned extent: the rank's queries see the stream up to its last token
        assert list(m["local_seq_lens"]) == [b + 1]
        assert list(m["local_kv_start_loc"]) == [0, b + 1]


def test_golden_round_robin_8_on_4():
    g = json.load(open(os.path.join(GOLDEN, "round_robin_t8_cp4.json")))
    qsl = _qsl(g["lens"])
    T = int(qsl[-1])
    for r, toks in enumerate(g["rank_tokens"]):
        m = O.cp_metadata(qsl, g["lens"], g["cp_size"], r, O.ROUND_ROBIN, False)
        assert list(m["token_map"][m["token_map"] >= 0]) == toks
        # Q_r and Q_{r+4} see keys 0..r and 0..r+4 (a query sees itself)
        assert [E for (_, E, _) in O.query_views(m)] == [t + 1 for t in toks]
    x = np.arange(T)
    concat = O.split_concat(x, T, g["cp_size"], O.ROUND_ROBIN, False)
    assert list(concat) == g["gathered_order"]
    assert list(O.rerange(concat, T, g["cp_size"], O.ROUND_ROBIN, False)) == g["logical_order"]


@pytest.mark.parametrize("mode,pad", MODES)
def test_cp1_is_identity(mode, pad):
    for lens in _random_batches(1, 30):
        qsl = _qsl(lens)
        m = O.cp_metadata(qsl, lens, 1, 0, mode, pad)
        T = int(qsl[-1])
        assert m["tokens_per_rank"] == T and m["num_tokens_pad"] == T
        assert list(m["local_query_start_loc"]) == list(qsl)
        assert list(m["local_seq_lens"]) == list(lens)
        assert list(m["local_kv_start_loc"]) == list(qsl)
        assert list(m["token_map"]) == list(range(T))


@pytest.mark.parametrize("mode,pad", MODES)
def test_ranks_partition_the_query_tokens(mode, pad):
    for lens in _random_batches(2, 30):
        qsl = _qsl(lens)
        T = int(qsl[-1])
        for cp in (1, 2, 3, 4, 8):
            seen = []
            per_req = np.zeros(len(lens), dtype=np.int64)
            for r in range(cp):
                m = O.cp_metadata(qsl, lens, cp, r, mode, pad)
                assert m["num_tokens_pad"] % cp == 0 and m["num_tokens_pad"] >= T
                assert m["num_tokens_pad"] - T < cp
                assert len(m["token_map"]) == m["tokens_per_rank"] == m["num_tokens_pad"] // cp
                seen += list(m["token_map"][m["token_map"] >= 0])
                per_req += np.diff(m["local_query_start_loc"])
                assert m["n_local_real"] == int((m["token_map"] >= 0).sum())
            assert sorted(seen) == list(range(T)) and len(seen) == T
            assert list(per_req) == list(lens)


@pytest.mark.parametrize("pad", [False, True])
def test_round_robin_counts_differ_by_at_most_one(pad):
    for lens in _random_batches(3, 30):
        qsl = _qsl(lens)
        for cp in (2, 3, 4, 8):
            counts = [O.cp_metadata(qsl, lens, cp, r, O.ROUND_ROBIN, pad)["n_local_real"] for r in range(cp)]
            assert max(counts) - min(counts) <= 1


@pytest.mark.parametrize("mode,pad", MODES)
def test_extents_are_positions_plus_one(mode, pad):
    """Every local query sees exactly the keys of its request up to and including itself."""
    for lens in _random_batches(4, 30):
        qsl = _qsl(lens)
        for cp in (1, 2, 3, 5):
            for r in range(cp):
                m = O.cp_metadata(qsl, lens, cp, r, mode, pad)
                toks = m["token_map"][m["token_map"] >= 0]
                views = O.query_views(m)
                assert len(views) == len(toks)
                for t, (b, E, kv0) in zip(toks, views):
                    assert qsl[b] <= t < qsl[b + 1]
                    assert E == t - qsl[b] + 1
                    assert kv0 == qsl[b]


def test_last_rank_sees_the_full_stream():
    for lens in _random_batches(5, 30):
        qsl = _qsl(lens)
        for cp in (2, 3, 4, 8):
            m = O.cp_metadata(qsl, lens, cp, cp - 1, O.IN_SEQ, False)
            assert list(m["local_seq_lens"]) == list(lens)
            assert list(m["local_kv_start_loc"]) == list(qsl)


def test_hand_worked_padding_and_boundary_crossing():
    """seq_lens [5,3,3] (T=11), cp 3: num_tokens_pad 12, tokens_per_rank 4.

    Contiguous: rank r owns [4r, 4r+4) clipped to 11, so rank 1 holds token 4 of request 0
    (position 4: extent 5) and all of request 1; rank 2 holds request 2 and one pad row.
    Round-robin: rank 0 {0,3,6,9}, rank 1 {1,4,7,10}, rank 2 {2,5,8}.
    """
    lens = [5, 3, 3]
    qsl = _qsl(lens)
    want_in_seq = {
        0: ([0, 4, 4, 4], [4, 0, 0], [0, 4, 4, 4], [0, 1, 2, 3]),
        1: ([0, 1, 4, 4], [5, 3, 0], [0, 5, 8, 8], [4, 5, 6, 7]),
        2: ([0, 0, 0, 3], [5, 3, 3], [0, 5, 8, 11], [8, 9, 10, -1]),
    }
    for r, (lq, ls, lk, tm) in want_in_seq.items():
        m = O.cp_metadata(qsl, lens, 3, r, O.IN_SEQ, False)
        assert m["num_tokens_pad"] == 12 and m["tokens_per_rank"] == 4
        assert (list(m["local_query_start_loc"]), list(m["local_seq_lens"]),
                list(m["local_kv_start_loc"]), list(m["token_map"])) == (lq, ls, lk, tm)
    want_rr = {
        0: ([0, 2, 3, 4], [4, 2, 2], [0, 3, 6, 9, ]),
        1: ([0, 2, 3, 4], [5, 3, 3], [1, 4, 7, 10]),
        2: ([0, 1, 2, 3], [3, 1, 1], [2, 5, 8, -1]),
    }
    for r, (lq, ls, tm) in want_rr.items():
        m = O.cp_metadata(qsl, lens, 3, r, O.ROUND_ROBIN, False)
        assert list(m["local_query_start_loc"]) == lq
        assert list(m["local_seq_lens"]) == ls
        assert list(m["local_kv_start_loc"]) == [0, 5, 8, 11]
        assert list(m["token_map"]) == tm
    concat = O.split_concat(np.arange(11), 11, 3, O.ROUND_ROBIN, False)
    assert list(concat) == [0, 3, 6, 9, 1, 4, 7, 10, 2, 5, 8]
    assert list(O.rerange(concat, 11, 3, O.ROUND_ROBIN, False)) == list(range(11))


def test_round_robin_batch_of_four_rank3():
    """Requests 32768/8192/2048/5, cp 8, rank 3: rank 3 owns tokens 3, 11, 19, ...

    Request starts 0, 32768, 40960, 43008 are multiples of 8, so each request's local tokens
    are positions 3, 11, ... within it: 4096, 1024, 256 and 1 queries whose last positions are
    32763, 8187, 2043 and 3.
    """
    lens = [32768, 8192, 2048, 5]
    qsl = _qsl(lens)
    m = O.cp_metadata(qsl, lens, 8, 3, O.ROUND_ROBIN, False)
    assert list(m["local_query_start_loc"]) == [0, 4096, 5120, 5376, 5377]
    assert list(m["local_seq_lens"]) == [32764, 8188, 2044, 4]
    assert list(m["local_kv_start_loc"]) == [0, 32768, 40960, 43008, 43013]
    assert m["tokens_per_rank"] == 5377 and m["num_tokens_pad"] == 43016
    assert m["max_seqlen_q"] == 4096 and m["num_local_reqs"] == 4


@pytest.mark.parametrize("mode,pad", MODES)
def test_rerange_inverts_split(mode, pad):
    g = np.random.default_rng(6)
    for lens in _random_batches(7, 20):
        T = int(sum(lens))
        x = g.integers(0, 1 << 16, size=(T, 3)).astype(np.uint16)
        for cp in (1, 2, 3, 4, 8):
            concat = O.split_concat(x, T, cp, mode, pad)
            assert len(concat) == (cp * (-(-T // cp)) if pad else T)
            assert np.array_equal(O.rerange(concat, T, cp, mode, pad), x)
            y = g.integers(0, 1 << 16, size=concat.shape).astype(np.uint16)
            again = O.split_concat(O.rerange(y, T, cp, mode, pad), T, cp, mode, pad)
            counts = O.rank_row_counts(T, cp, mode, pad)
            off = np.concatenate([[0], np.cumsum(counts)])
            for r in range(cp):
                nreal = len(O.local_tokens(T, cp, r, mode))
                assert np.array_equal(again[off[r]:off[r] + nreal], y[off[r]:off[r] + nreal])
                assert not again[off[r] + nreal:off[r + 1]].any()


def test_in_seq_rerange_is_identity():
    x = np.arange(23)
    for cp in (2, 4, 5):
        for pad in (False, True):
            concat = O.split_concat(x, 23, cp, O.IN_SEQ, pad)
            assert list(O.rerange(concat, 23, cp, O.IN_SEQ, pad)) == list(range(23))
            if not pad:
                assert list(concat) == list(range(23))


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        O.cp_metadata([0, 4, 6], [4, 1], 2, 0, O.IN_SEQ, False)      # seq_lens below the query length
    with pytest.raises(ValueError):
        O.cp_metadata([0, 4, 6], [4, 2], 2, 2, O.IN_SEQ, False)      # rank out of range
    with pytest.raises(ValueError):
        O.cp_metadata([1, 4, 6], [3, 2], 2, 0, O.IN_SEQ, False)      # qsl[0] != 0


# ----------------------------------------------------------------------------- chunked prefill
# R-17: request b carries P_b = seq_lens[b] - n_b cached tokens; its KV segment is
# seq_lens[b] rows long (prefix first), segments follow in request order, and query g of the
# request sits at KV position P_b + g.  With P_b = 0 every rule above is unchanged.

def _random_prefixed(seed, n):
    g = np.random.default_rng(seed)
    for lens in _random_batches(seed, n):
        yield lens, [int(x) for x in g.integers(0, 30, size=len(lens))]


def test_hand_worked_chunked_prefill():
    """Queries [5,3,3] after cached prefixes [2,0,4] (seq_lens [7,3,7]), cp 3, tokens_per_rank 4.

    KV segments start at rows 0, 7, 10 (17 rows in all).  Contiguous: rank 0 holds tokens 0..3,
    the first four queries of request 0 at KV positions 2..5, so its last query sees 6 keys; a
    later request contributes only its cached prefix (request 1 none, request 2 four rows);
    rank 1 holds token 4 (position 6: 7 keys) and request 1; rank 2 holds request 2, whose last
    query sees 4 + 3 keys, so the last rank sees every segment whole.
    Round-robin: rank 0 {0,3,6,9}: last local queries of the requests sit at positions 5, 1, 5.
    """
    lens, prefix = [5, 3, 3], [2, 0, 4]
    seq = [l + p for l, p in zip(lens, prefix)]
    qsl = _qsl(lens)
    want_in_seq = {
        0: ([0, 4, 4, 4], [6, 0, 4], [0, 6, 6, 10], [3, 4, 5, 6]),
        1: ([0, 1, 4, 4], [7, 3, 4], [0, 7, 10, 14], [7, 1, 2, 3]),
        2: ([0, 0, 0, 3], [7, 3, 7], [0, 7, 10, 17], [5, 6, 7]),
    }
    for r, (lq, ls, lk, ext) in want_in_seq.items():
        m = O.cp_metadata(qsl, seq, 3, r, O.IN_SEQ, False)
        assert (list(m["local_query_start_loc"]), list(m["local_seq_lens"]),
                list(m["local_kv_start_loc"])) == (lq, ls, lk)
        assert [E for (_, E, _) in O.query_views(m)] == ext
    want_rr = {
        0: ([0, 2, 3, 4], [6, 2, 6], [3, 6, 2, 6]),
        1: ([0, 2, 3, 4], [7, 3, 7], [4, 7, 3, 7]),
        2: ([0, 1, 2, 3], [5, 1, 5], [5, 1, 5]),
    }
    for r, (lq, ls, ext) in want_rr.items():
        m = O.cp_metadata(qsl, seq, 3, r, O.ROUND_ROBIN, False)
        assert list(m["local_query_start_loc"]) == lq
        assert list(m["local_seq_lens"]) == ls
        assert list(m["local_kv_start_loc"]) == [0, 7, 10, 17]
        assert [E for (_, E, _) in O.query_views(m)] == ext


@pytest.mark.parametrize("mode,pad", MODES)
def test_extents_with_prefixes_are_kv_positions_plus_one(mode, pad):
    """Every local query sees its request's KV segment up to and including its own position."""
    for lens, prefix in _random_prefixed(8, 30):
        qsl = _qsl(lens)
        seq = [l + p for l, p in zip(lens, prefix)]
        kv_start = _qsl(seq)
        for cp in (1, 2, 3, 5):
            for r in range(cp):
                m = O.cp_metadata(qsl, seq, cp, r, mode, pad)
                toks = m["token_map"][m["token_map"] >= 0]
                views = O.query_views(m)
                assert len(views) == len(toks)
                for t, (b, E, kv0) in zip(toks, views):
                    assert qsl[b] <= t < qsl[b + 1]
                    assert E == prefix[b] + (t - qsl[b]) + 1
                    assert kv0 == kv_start[b]


def test_last_rank_sees_every_segment_with_prefixes():
    for lens, prefix in _random_prefixed(9, 30):
        seq = [l + p for l, p in zip(lens, prefix)]
        for cp in (1, 2, 4):
            m = O.cp_metadata(_qsl(lens), seq, cp, cp - 1, O.IN_SEQ, False)
            assert list(m["local_seq_lens"]) == seq
            assert list(m["local_kv_start_loc"]) == list(_qsl(seq))
