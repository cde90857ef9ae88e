"""bench.py's counter-summary helpers (CPU only): profiler kernel names reduce to the names the
traffic files use, and a traffic file stops counting once its kernel's sources change."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_short_kernel_names():
    n = bench.short_kernel_name
    assert n("void dsa::(anonymous namespace)::indexer_mfma<true, true>(unsigned char const*, float const*)") == \
        "indexer_mfma<true, true>"
    assert n("dsa::(anonymous namespace)::sparse_attn_mla_bf16(unsigned short const*, int)") == "sparse_attn_mla_bf16"
    assert n("void dsa::(anonymous namespace)::topk_reg_kernel<256, 16>(float const*, long)") == \
        "topk_reg_kernel<256, 16>"
    assert n("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"
    for k, t in bench.TRACE_NAME.items():
        assert k in bench.KERNEL_SOURCES and t == n("void dsa::(anonymous namespace)::" + t + "(int)")


def test_traffic_is_dropped_when_sources_change(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    csrc = tmp_path / "sparse_attention_prefill_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    for f in ("attention.hip", "dsa_internal.h"):
        (csrc / f).write_text("// v1\n")
    sha = bench.src_hash(bench.KERNEL_SOURCES["sparse_attn_mla_bf16"])
    (tmp_path / "profiles" / "traffic_sparse_attn_mla_bf16_w.json").write_text(
        json.dumps({"src_sha": sha, "bytes_per_launch": 123.0}))
    assert bench.traffic_for("sparse_attn_mla_bf16", "w") == 123.0
    assert bench.traffic_for("sparse_attn_mla_bf16", "other") is None
    (csrc / "dsa_internal.h").write_text("// v2\n")
    assert bench.traffic_for("sparse_attn_mla_bf16", "w") is None


def test_committed_traffic_files_match_the_sources():
    """Every committed traffic file belongs to the current sources of its kernel (else bench.py
    would report null traffic for it)."""
    prof = os.path.join(ROOT, "profiles")
    names = [f for f in os.listdir(prof) if f.startswith("traffic_") and f.endswith(".json")]
    assert names
    for f in names:
        t = json.load(open(os.path.join(prof, f)))
        assert t["src_sha"] == bench.src_hash(bench.KERNEL_SOURCES[t["kernel"]]), f
