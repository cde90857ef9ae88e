"""The seeded input generator: determinism, rank-consistency, storage encodings, stand-ins."""
import numpy as np

import oracle as O
import synthetic as S


def test_query_rows_do_not_depend_on_which_rows_are_drawn():
    wl = S.WORKLOADS["rr_cp8_r3_batch4"].with_(lens=(40, 9), H=2, Dqk=8, Dv=4, Hi=2, Di=4)
    a = S.query_inputs(wl, [3, 11, 19, 27])
    b = S.query_inputs(wl, [27, -1, 11])
    assert np.array_equal(a["q"][3], b["q"][0]) and np.array_equal(a["q"][1], b["q"][2])
    assert not b["q"][1].any()
    assert np.array_equal(a["q_idx"][1], b["q_idx"][2]) and np.array_equal(a["w"][3], b["w"][0])


def test_stream_is_deterministic_and_sized():
    wl = S.WORKLOADS["tiny_fp32_cp1"]
    a, b = S.stream_inputs(wl), S.stream_inputs(wl)
    for k in ("kv", "k_idx", "sink"):
        assert np.array_equal(a[k], b[k])
    assert a["kv"].shape == (512, 160) and a["kv"].dtype == np.float32
    assert abs(a["kv"].std() * np.sqrt(160) - 1) < 0.02


def test_compressed_stand_in_is_the_block_mean():
    wl = S.WORKLOADS["rr_cp4_r1_var8_cmp4"].with_(lens=(9, 4, 3, 13), H=2, Dqk=16, Dv=8, Hi=2, Di=8)
    d = S.stream_inputs(wl)
    T = wl.T
    assert list(d["kv_cmp_start"]) == [0, 2, 3, 3, 6]
    assert d["kv"].shape == (T + 6, 16) and d["k_idx"].shape == (6, 8)
    full_k = S.stream_inputs(wl.with_(compress=1))["k_idx"]
    kv = O.decode_bf16(d["kv"])
    kf = O.decode_bf16(full_k)
    qsl = wl.qsl
    for b, start in enumerate(qsl[:-1]):
        for c in range(wl.lens[b] // 4):
            row = int(d["kv_cmp_start"][b]) + c
            blk = slice(int(start) + 4 * c, int(start) + 4 * c + 4)
            assert np.array_equal(d["kv"][T + row], S.f64_to_bf16_bits(kv[blk].mean(axis=0)))
            assert np.array_equal(d["k_idx"][row], S.f64_to_bf16_bits(kf[blk].mean(axis=0)))


def test_fp8_inputs_respect_the_range_and_scales():
    wl = S.WORKLOADS["long_131k_fp8"].with_(lens=(300,), H=2, Dqk=8, Dv=4)
    d = S.stream_inputs(wl)
    q = S.query_inputs(wl, np.arange(5))
    k = O.decode_e4m3fn(d["k_idx"])
    assert d["k_idx"].dtype == np.uint8 and d["k_scale"].shape == (300,)
    assert np.all(np.abs(k).max(axis=1) == 448.0)      # per-token amax maps to the largest code
    assert np.all(d["k_scale"] > 0) and np.all(q["q_scale"] > 0)
    assert q["q_scale"].shape == (5, 64)


def test_var_batch_lengths_are_seeded():
    lens = S.WORKLOADS["rr_cp4_r1_var8_cmp4"].lens
    assert len(lens) == 8 and all(1024 <= l <= 16384 for l in lens)


def test_indexer_only_query_inputs_draw_the_same_values():
    wl = S.WORKLOADS["long_131k_fp8"].with_(lens=(300,))
    a = S.query_inputs(wl, [0, 7, 299], indexer_only=True)
    b = S.query_inputs(wl, [0, 7, 299])
    assert a["q"].shape[0] == 0
    for k in ("q_idx", "w", "q_scale"):
        assert np.array_equal(a[k], b[k]), k
