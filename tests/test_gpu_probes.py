"""The measurement hooks on the GPU: the clock probe returns a plausible shader clock and the
LDS-fed MFMA probe returns busy fractions in (0, 1], ordered as its read forms require (a chain
fed from registers is at least as busy as one fed from LDS)."""
import pytest
import torch

import sparse_attention_prefill_amd as D
from dsa_testlib import gpu

pytestmark = pytest.mark.gpu


def test_clock_probe_reports_a_plausible_clock():
    dev = gpu()
    out = torch.zeros(4, dtype=torch.int64, device=dev)
    D.clock_probe(out, 20000)
    torch.cuda.synchronize()
    mhz = D.probe_mhz(out.cpu().numpy())
    print(f"shader clock {mhz:.0f} MHz", flush=True)
    assert 300.0 < mhz < 3000.0


def test_lds_mfma_probe_fractions():
    dev = gpu()
    cyc = torch.zeros(2048, dtype=torch.int64, device=dev)
    sink = torch.empty(256 * 512, dtype=torch.float32, device=dev)
    busy = {}
    for op in (0, 1, 2):
        for w in (1, 2):
            cyc.zero_()
            D.lds_mfma_probe(op, w, 50, cyc, sink)
            torch.cuda.synchronize()
            c = cyc.cpu().numpy().reshape(256, 8)
            assert (c[:, :4 * w] > 0).all() and (c[:, 4 * w:] == 0).all()
            busy[(op, w)] = D.lds_mfma_busy(c.reshape(-1), w, 50)
    print({f"operand{k[0]}_{k[1]}wave": round(v, 3) for k, v in busy.items()}, flush=True)
    for v in busy.values():
        assert 0.05 < v <= 1.05
    for w in (1, 2):
        assert busy[(2, w)] >= 0.95 * max(busy[(0, w)], busy[(1, w)])
