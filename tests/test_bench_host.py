"""Host-side logic of bench.py (no GPU): source hashes per path, the stored
traffic summaries and the algorithmic byte counts of each kernel."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from token_level_head_block_amd import synth  # noqa: E402


def test_source_hash_per_path():
    shas = {p: bench.kernel_source_sha(p) for p in bench.KERNEL_SOURCES}
    assert all(len(s) == 64 for s in shas.values())
    assert shas["3kernel"] == shas["fused"]
    assert shas["causal"] != shas["3kernel"]   # the causal kernel's source is part of its hash


def test_measured_traffic_reads_or_ignores(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    for name in ("token_level_head_block_amd",):
        os.symlink(os.path.join(ROOT, name), tmp_path / name)
    assert bench.measured_traffic("nothing-here", "3kernel") == {}
    body = ["source_sha256: {sha}", "fetch_scale: 2.0", "write_scale: 0.5",
            "query_apply fetch_kib: 10", "query_apply write_kib: 4"]
    f = tmp_path / "profiles" / "traffic_w.txt"
    f.write_text("\n".join(body).format(sha=bench.kernel_source_sha("3kernel")) + "\n")
    assert bench.measured_traffic("w", "3kernel") == {"query_apply": 10 * 1024 * 2 + 4 * 1024 // 2}
    assert bench.measured_traffic("w", "causal") == {}   # another path's sources: stale
    f.write_text("\n".join(body).format(sha="0" * 64) + "\n")
    assert bench.measured_traffic("w", "3kernel") == {}


@pytest.mark.parametrize("idx", range(len(synth.CONFIGS)))
def test_kernel_bytes_are_compulsory_traffic(idx):
    p = synth.CONFIGS[idx]
    kb = bench.kernel_bytes(p, p.elem_bytes)
    tensor = p.batch * p.n_tokens * p.heads * p.head_dim * p.elem_bytes
    assert kb["block_kv_summary"] > 2 * tensor
    assert kb["query_apply"] > 2 * tensor
    assert kb["query_apply_causal"] > 4 * tensor
