"""GPU parity: CP-local metadata (1) and rerange (5) against the oracle, bit-exact."""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from dsa_testlib import gpu, to_dev, mode_code

pytestmark = pytest.mark.gpu


def _batches():
    g = np.random.default_rng(100)
    yield [5, 3, 3]
    yield [8]
    yield [8000]
    yield [32768, 8192, 2048, 5]
    yield list(S.WORKLOADS["rr_cp4_r1_var8_cmp4"].lens)
    yield [1]
    yield [0, 4, 0, 7]
    for _ in range(12):
        B = int(g.integers(1, 40))
        yield [int(x) for x in g.integers(0, 300, size=B)]
    for B in (64, 65, 300):  # the single-wave path's limit, just past it, several waves
        yield [int(x) for x in g.integers(0, 50, size=B)]
    yield [int(x) for x in g.integers(0, 9, size=1100)]  # more requests than one workgroup pass
    yield []


@pytest.mark.parametrize("mode", [O.IN_SEQ, O.ROUND_ROBIN])
@pytest.mark.parametrize("prefixed", [False, True])
def test_metadata_matches_oracle(mode, prefixed):
    """prefixed: every request also carries a random cached prefix (chunked prefill)."""
    dev = gpu()
    import sparse_attention_prefill_amd as D
    g = np.random.default_rng(101)
    for lens in _batches():
        qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        T = int(qsl[-1])
        seq = np.asarray(lens, dtype=np.int64)
        if prefixed:
            seq = seq + g.integers(0, 5000, size=len(lens))
        for cp in (1, 2, 3, 4, 8):
            for pad in (False, True):
                for r in sorted({0, cp // 2, cp - 1}):
                    ref = O.cp_metadata(qsl, seq, cp, r, mode, pad)
                    err = torch.zeros(1, dtype=torch.int32, device=dev)
                    m = D.build_cp_metadata(to_dev(qsl, "i32", dev), to_dev(seq, "i32", dev), T, cp, r,
                                            mode_code(mode), pad, err_flag=err)
                    torch.cuda.synchronize()
                    tag = f"lens={lens[:6]}.. seq={list(seq[:6])}.. cp={cp} r={r} pad={pad}"
                    assert err.item() == 0, tag
                    for k in ("local_query_start_loc", "local_seq_lens", "local_kv_start_loc", "token_map"):
                        assert np.array_equal(m[k].cpu().numpy(), ref[k]), f"{k} {tag}"
                    sc = m["scalars"].cpu().numpy()
                    want = [ref["num_tokens_pad"], ref["tokens_per_rank"], ref["local_start"], ref["local_end"],
                            ref["stride"], ref["n_local_real"], ref["max_seqlen_q"], ref["num_local_reqs"]]
                    assert list(sc) == want, f"scalars {tag}: {list(sc)} vs {want}"


def test_metadata_flags_bad_inputs():
    dev = gpu()
    import sparse_attention_prefill_amd as D
    qsl = to_dev(np.array([0, 4, 9]), "i32", dev)
    for seq, T, bit in (([4, 3], 9, 0x4), ([3, 5], 9, 0x4), ([4, 5], 10, 0x8)):
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        D.build_cp_metadata(qsl, to_dev(np.array(seq), "i32", dev), T, 2, 0, 0, False, err_flag=err)
        torch.cuda.synchronize()
        assert err.item() & bit, (seq, T, err.item())
    with pytest.raises(D.DsaError):
        D.build_cp_metadata(qsl, to_dev(np.array([4, 5]), "i32", dev), 9, 2, 2, 0, False)


@pytest.mark.parametrize("mode", [O.IN_SEQ, O.ROUND_ROBIN])
@pytest.mark.parametrize("pad", [False, True])
def test_rerange_matches_oracle(mode, pad):
    dev = gpu()
    import sparse_attention_prefill_amd as D
    g = np.random.default_rng(7)
    for T in (1, 7, 8, 11, 1000, 4099):
        for cp in (1, 2, 3, 4, 8):
            for width in (8, 576):
                x = g.integers(0, 1 << 16, size=(T, width), dtype=np.uint16)
                concat = O.split_concat(x, T, cp, mode, pad)
                xd = to_dev(concat, "bf16", dev)
                back = D.rerange(xd, T, cp, mode_code(mode), pad, inverse=False)
                split = D.rerange(to_dev(x, "bf16", dev), T, cp, mode_code(mode), pad, inverse=True)
                torch.cuda.synchronize()
                assert np.array_equal(back.view(torch.int16).cpu().numpy().view(np.uint16), x), (T, cp, width)
                assert np.array_equal(split.view(torch.int16).cpu().numpy().view(np.uint16), concat), (T, cp, width)


def test_rerange_full_size_round_robin_batch4():
    """Rank-concatenated [43013, 576] bf16 (requests 32768/8192/2048/5 on 8 ranks) -> logical order."""
    dev = gpu()
    import sparse_attention_prefill_amd as D
    wl = S.WORKLOADS["rr_cp8_r3_batch4"]
    T = wl.T
    x = S.rerange_buffer(wl, T)
    concat = O.split_concat(x, T, 8, O.ROUND_ROBIN, False)
    out = D.rerange(to_dev(concat, "bf16", dev), T, 8, 1, False)
    torch.cuda.synchronize()
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), x)
