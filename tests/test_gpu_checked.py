"""The checked build (libdsa_checked.so: the same sources compiled with DSA_CHECKED, every gathered
row id and data-dependent index verified before use) on the paths the benchmark workloads take:
no index fails its check (err_flag stays 0, so no DSA_DEVERR_BOUNDS), and the results equal the
product library's bit for bit."""
import numpy as np
import pytest
import torch

import synthetic as S
import sparse_attention_prefill_amd as D
from dsa_testlib import gpu
from test_gpu_path import gpu_rank_path

pytestmark = pytest.mark.gpu

# each case reaches a different set of kernels
CASES = [
    ("tiny_fp32_cp1", {}),                                          # generic indexer and attention
    ("inseq_cp8_last_8k", {}),                                      # bf16 indexer, register top-k, MLA attention
    ("rr_cp8_r3_batch4", {}),                                       # sampled top-k (5377 rows up to 32K keys)
    ("rr_cp4_r1_var8_cmp4", {"lens": (3000, 9001, 700, 1234)}),     # compressed keys + window rows
    ("chunk_inseq_cp8_last_8k_p56k", {"lens": (2048,), "prefix": (40000,)}),  # streamed top-k (> 32K keys)
    ("long_131k_fp8", {"lens": (1024,), "prefix": (110000,)}),      # fp8, candidate lists (> 96K keys)
]


@pytest.mark.parametrize("name,kw", CASES)
def test_checked_build_flags_nothing_and_matches(name, kw):
    dev = gpu()
    wl = S.WORKLOADS[name].with_(**kw) if kw else S.WORKLOADS[name]
    ref = gpu_rank_path(wl, "normal", dev)
    assert ref["err"] == 0, f"product library: device error flag {ref['err']:#x}"
    print(f"checked library: {name} {kw}", flush=True)
    with D.library(D.checked_library_path):
        got = gpu_rank_path(wl, "normal", dev)
    assert got["err"] == 0, f"checked library: device error flag {got['err']:#x}"
    assert np.array_equal(got["idx"], ref["idx"])
    assert torch.equal(got["out"].view(torch.int16) if got["out"].dtype == torch.bfloat16 else got["out"],
                       ref["out"].view(torch.int16) if ref["out"].dtype == torch.bfloat16 else ref["out"])


def test_checked_library_is_a_separate_build():
    gpu()
    with D.library(D.checked_library_path) as L:
        assert L._name.endswith("libdsa_checked.so")
    assert D.lib()._name.endswith("libdsa.so")
