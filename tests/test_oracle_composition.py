"""Hand-worked pins of the rows the oracle's whole path attends with compressed index keys and a
sliding window (readings R-12, R-13, R-17).

Page: [xLLM-CP] "feat: DeepSeek-V4 DSA context-parallel on NPU", Background (the attention mixes a
sliding window, compressed KV and an indexer top-k over the compressed keys) and Implementation §4
(the indexer's full side is the compressed key stream, addressed by its own cu-seqlens).

Every expected row id below is written out by hand from these facts, not computed by the code
under test:
  * request b's KV segment holds its tokens, segments in request order; the compressed rows of
    all requests follow the last token row, request by request (block c of request b is row
    n_kv + kv_cmp_start[b] + c, where n_kv = sum of seq_lens);
  * compressed block c (tokens 4c .. 4c+3 of the segment) is visible to KV position p iff
    4c + 3 <= p, i.e. the first floor((p + 1) / 4) blocks;
  * the window of position p is the segment rows max(0, p - 2) .. p (window 3);
  * the attended set is the selected compressed rows plus the window rows, in one softmax with
    the sink (R-12).
The compressed index keys are chosen so that each block's score is a known number, and the
output is checked against a softmax over the hand-listed rows, written out term by term.
"""
import math

import numpy as np
import pytest

import oracle as O
import synthetic as S

SINK = 0.5


def _wl(lens, prefix, K, mode=O.IN_SEQ, cp=1, rank=0):
    base = S.WORKLOADS["tiny_fp32_cp1"]
    return base.with_(lens=tuple(lens), prefix=tuple(prefix), cp=cp, rank=rank, mode=mode, pad=False,
                      H=1, Dqk=2, Dv=1, Hi=1, Di=1, idx_dtype="f32", attn_dtype="f32",
                      topk=K, compress=4, window=3)


def _kv_row(r):
    """Row r of the KV buffer: value column r + 1, logit column 0.25 * (r mod 3)."""
    return [float(r + 1), 0.25 * (r % 3)]


def _inputs(n_kv, cmp_start, cmp_keys, seq_lens, n_rows):
    n_cmp = len(cmp_keys)
    return {
        "kv": np.array([_kv_row(r) for r in range(n_kv + n_cmp)], dtype=np.float32),
        "k_idx": np.array([[k] for k in cmp_keys], dtype=np.float32),
        "sink": np.array([SINK], dtype=np.float32),
        "seq_lens": np.array(seq_lens, dtype=np.int32),
        "kv_cmp_start": np.array(cmp_start, dtype=np.int32),
        # every query: q = [0, 1] (its logit reads the second column), indexer q = 1, w = 1, so a
        # block's score is its compressed key
        "q": np.tile(np.array([[[0.0, 1.0]]], dtype=np.float32), (n_rows, 1, 1)),
        "q_idx": np.ones((n_rows, 1, 1), dtype=np.float32),
        "w": np.ones((n_rows, 1), dtype=np.float32),
    }


def _softmax_over(rows):
    """out = sum_s e^(l_s) v_s / (e^sink + sum_s e^(l_s)), l_s = kv[s] . [0, 1], v_s = kv[s][0]."""
    num = 0.0
    den = math.exp(SINK)
    for r in rows:
        v, l = _kv_row(r)
        num += math.exp(l) * v
        den += math.exp(l)
    return num / den


# Requests of 9 and 6 tokens, no cached prefix.  n_kv = 15; request 0 has blocks 0, 1 (tokens
# 0-3, 4-7; token 8 is in no whole block) at rows 15, 16; request 1 has block 0 (its tokens
# 0-3 = rows 9-12) at row 17.  Compressed keys: 1, 3 (request 0), 2 (request 1).
# Table: (request, position) -> (scores of the visible blocks, ids with K = 1, ids with K = 2,
# window rows).
PURE = {
    (0, 0): ([], [], [], [0]),
    (0, 1): ([], [], [], [0, 1]),
    (0, 2): ([], [], [], [0, 1, 2]),
    (0, 3): ([1.0], [15], [15], [1, 2, 3]),
    (0, 4): ([1.0], [15], [15], [2, 3, 4]),
    (0, 5): ([1.0], [15], [15], [3, 4, 5]),
    (0, 6): ([1.0], [15], [15], [4, 5, 6]),
    (0, 7): ([1.0, 3.0], [16], [15, 16], [5, 6, 7]),
    (0, 8): ([1.0, 3.0], [16], [15, 16], [6, 7, 8]),
    (1, 0): ([], [], [], [9]),
    (1, 1): ([], [], [], [9, 10]),
    (1, 2): ([], [], [], [9, 10, 11]),
    (1, 3): ([2.0], [17], [17], [10, 11, 12]),
    (1, 4): ([2.0], [17], [17], [11, 12, 13]),
    (1, 5): ([2.0], [17], [17], [12, 13, 14]),
}

# The same requests, request 1 now after a 2-token cached prefix (R-17): seq_lens (9, 8),
# n_kv = 17, request 1's segment is rows 9-16 (prefix rows 9, 10; its 6 queries sit at KV
# positions 2..7).  Blocks: request 0 rows 17, 18 (keys 1, 3); request 1 blocks 0 (rows 9-12)
# and 1 (rows 13-16) at rows 19, 20 (keys 2, 5).  Request 1's rows are keyed by query index g.
CHUNKED = {
    (0, 0): ([], [], [], [0]),
    (0, 1): ([], [], [], [0, 1]),
    (0, 2): ([], [], [], [0, 1, 2]),
    (0, 3): ([1.0], [17], [17], [1, 2, 3]),
    (0, 4): ([1.0], [17], [17], [2, 3, 4]),
    (0, 5): ([1.0], [17], [17], [3, 4, 5]),
    (0, 6): ([1.0], [17], [17], [4, 5, 6]),
    (0, 7): ([1.0, 3.0], [18], [17, 18], [5, 6, 7]),
    (0, 8): ([1.0, 3.0], [18], [17, 18], [6, 7, 8]),
    (1, 0): ([], [], [], [9, 10, 11]),               # KV position 2
    (1, 1): ([2.0], [19], [19], [10, 11, 12]),        # position 3: block 0 complete
    (1, 2): ([2.0], [19], [19], [11, 12, 13]),
    (1, 3): ([2.0], [19], [19], [12, 13, 14]),
    (1, 4): ([2.0], [19], [19], [13, 14, 15]),
    (1, 5): ([2.0, 5.0], [20], [19, 20], [14, 15, 16]),  # position 7: block 1 complete
}

CASES = {
    "pure": (PURE, (9, 6), (0, 0), 15, [0, 2, 3], [1.0, 3.0, 2.0], (9, 6)),
    "chunked": (CHUNKED, (9, 6), (0, 2), 17, [0, 2, 4], [1.0, 3.0, 2.0, 5.0], (9, 8)),
}


def _run(case, K, mode, cp, rank):
    table, lens, prefix, n_kv, cmp_start, keys, seq_lens = CASES[case]
    wl = _wl(lens, prefix, K, mode, cp, rank)
    assert wl.n_kv == n_kv and list(wl.seq_lens) == list(seq_lens)
    m = O.cp_metadata(wl.qsl, wl.seq_lens, cp, rank, mode, False)
    toks = m["token_map"][m["token_map"] >= 0]
    inp = _inputs(n_kv, cmp_start, keys, seq_lens, len(toks))
    res = O.run_path(m, inp, wl, scale=1.0, want_scores=True)
    qsl = np.concatenate([[0], np.cumsum(lens)])
    keyed = [(int(b), int(t - qsl[b])) for t in toks for b in [np.searchsorted(qsl, t, side="right") - 1]]
    return table, keyed, res


@pytest.mark.parametrize("case", ["pure", "chunked"])
@pytest.mark.parametrize("K", [1, 2])
@pytest.mark.parametrize("mode,cp,rank", [(O.IN_SEQ, 1, 0), (O.ROUND_ROBIN, 2, 1), (O.ROUND_ROBIN, 3, 0),
                                          (O.IN_SEQ, 2, 1)])
def test_compressed_ids_window_and_output_are_the_hand_worked_rows(case, K, mode, cp, rank):
    table, keyed, res = _run(case, K, mode, cp, rank)
    assert len(keyed) == len(res["topk_ids"]) > 0
    for n, key in enumerate(keyed):
        scores, ids1, ids2, win = table[key]
        ids = ids1 if K == 1 else ids2
        assert list(res["scores"][n]) == scores, (key, "scores of the visible blocks")
        assert list(res["topk_ids"][n]) == ids, (key, "selected compressed rows")
        assert list(res["window_ids"][n]) == win, (key, "window rows")
        assert np.isclose(res["out"][n][0, 0], _softmax_over(ids + win), rtol=1e-14, atol=0), key


def test_every_table_row_is_reached():
    """The rank splits above together visit every (request, position) of both tables."""
    for case in CASES:
        seen = set()
        for mode, cp in ((O.IN_SEQ, 1), (O.ROUND_ROBIN, 2), (O.ROUND_ROBIN, 3)):
            for rank in range(cp):
                table, keyed, _ = _run(case, 1, mode, cp, rank)
                seen.update(keyed)
        assert seen == set(CASES[case][0])
