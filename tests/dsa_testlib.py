"""Helpers for the GPU parity tests: device transfer, running the HIP path, comparisons.

The HIP path is always reached through the C ABI via the package binding; the oracle is
always the CPU reference. This module holds no method arithmetic.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S


# Indexer score parity, as a fraction of the row's largest |oracle score| (R-15): the GPU sums its
# products in float32 in an order of its own (fp8: inside the matrix cores, whose sums are not
# float32-exact), the oracle in float64. Each bound is twice the worst deviation measured over every
# test row's full score row and 1026 full rows of the 131072-key fp8 workload (fp8 3.79e-5, bf16
# 1.30e-6, f32 7.35e-7 of the row maximum; each inside an any-order float32 summation bound).
SCORE_TOL = {"f32": 1.4e-6, "bf16": 2.6e-6, "fp8": 7.5e-5}
# A top-k id may differ from the oracle's only if its oracle score lies within this fraction of the
# row's largest |score| of the K-th best: GPU and oracle order two keys differently only when their
# oracle scores are closer than the sum of the two keys' errors, at most twice the worst error.
TIE_BAND = dict(SCORE_TOL)


def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import sparse_attention_prefill_amd as D  # noqa: F401  (raises if libdsa.so is missing)
    return torch.device("cuda:0")


def to_dev(a, kind, device):
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if kind == "fp8":
        return torch.from_numpy(a.view(np.uint8)).to(device)
    if kind == "f32":
        return torch.from_numpy(a.astype(np.float32)).to(device)
    if kind == "i32":
        return torch.from_numpy(a.astype(np.int32)).to(device)
    raise ValueError(kind)


def to_f64(t):
    """Device tensor (f32 / bf16) -> numpy float64."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def mode_code(mode):
    return 0 if mode == O.IN_SEQ else 1


def assert_attn_close(got, ref, dtype, what=""):
    """bf16: max-abs <= 2e-2, relative Frobenius < 1e-2, max-abs / max|ref| < 1e-2; f32: max-abs <= 1e-4."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    if dtype == "f32":
        assert err.max() <= 1e-4, f"{what}: max-abs {err.max():.3e}"
        return
    scale = max(np.abs(ref).max(), 1e-30)
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err.max() <= 2e-2, f"{what}: max-abs {err.max():.3e}"
    assert fro < 1e-2, f"{what}: relative Frobenius {fro:.3e}"
    assert err.max() / scale < 1e-2, f"{what}: max-abs/max|ref| {err.max() / scale:.3e}"


def check_topk_rows(gpu_ids, ora_ids, ora_scores, K, base_of_row, rows=None, delta_rel=1e-5):
    """Top-k parity with the tie band: equal sets, or every differing id's oracle score lies within
    delta of the oracle's K-th best score (scores near the cut can swap under fp32 rounding).
    Returns the number of rows whose sets are identical."""
    same = 0
    rows = range(len(ora_ids)) if rows is None else rows
    for n, i in enumerate(rows):
        g = np.sort(gpu_ids[n][gpu_ids[n] >= 0])
        r = np.sort(ora_ids[n])
        if len(g) == len(r) and np.array_equal(g, r):
            same += 1
            continue
        assert len(g) == len(r) == K, f"row {i}: {len(g)} vs {len(r)} ids"
        sc = ora_scores[n]
        kth = np.sort(sc)[::-1][K - 1]
        delta = delta_rel * max(np.abs(sc).max(), 1e-30)
        diff = np.setxor1d(g, r) - base_of_row[n]
        assert np.all((diff >= 0) & (diff < len(sc))), f"row {i}: id outside the causal extent"
        assert np.all(np.abs(sc[diff] - kth) <= delta), f"row {i}: differing ids far from the cut"
    return same
