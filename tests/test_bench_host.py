"""Host-side pieces of bench.py: which committed traffic measurement a run may
use (the code of its decode path's sources must hash as when it was taken)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_code_tokens_ignore_comments_and_layout():
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* no\n overflow */ }\n"
    b = "int f(int x)\n{\n    return 2 * x;\n}"
    assert bench.code_tokens(a) == bench.code_tokens(b)
    assert bench.code_tokens(a) != bench.code_tokens(b.replace("2 *", "3 *"))


@pytest.mark.parametrize("key,family", [("c2", "grouped"), ("c3", "grouped"), ("c4", "grouped"),
                                        ("c5", "latent"), ("c3_mfma", "mfma"),
                                        ("c3_mxfp8", "mxfp8")])
def test_traffic_family(key, family):
    assert bench.traffic_family(key) == family


def test_each_path_hashes_its_own_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "paged_kv_cache_58_amd" / "csrc"
    csrc.mkdir(parents=True)
    names = sorted({n for srcs in bench.KERNEL_SOURCES.values() for n in srcs})
    for n in names:
        (csrc / n).write_text(f"int {n.replace('.', '_')}_v = 1;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    before = {f: bench.kernel_source_hash(f) for f in bench.KERNEL_SOURCES}
    # a comment changes nothing
    (csrc / "latent_decode.hip").write_text("int latent_decode_hip_v = 1;  // note\n")
    assert {f: bench.kernel_source_hash(f) for f in bench.KERNEL_SOURCES} == before
    # code of one path changes that path's hash only
    (csrc / "latent_decode.hip").write_text("int latent_decode_hip_v = 2;\n")
    after = {f: bench.kernel_source_hash(f) for f in bench.KERNEL_SOURCES}
    assert after["latent"] != before["latent"]
    assert all(after[f] == before[f] for f in ("grouped", "mfma", "mxfp8"))
    # shared code changes every path
    (csrc / "device_common.h").write_text("int device_common_h_v = 2;\n")
    shared = {f: bench.kernel_source_hash(f) for f in bench.KERNEL_SOURCES}
    assert all(shared[f] != after[f] for f in bench.KERNEL_SOURCES)
