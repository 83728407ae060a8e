"""Host-side pieces of bench.py: the source hash that gates stored counter readings."""
import os
import shutil

import bench
from tensor_mlp_shard_amd import build


def _copy_sources(dst):
    for src in list(build.SOURCES) + ["device_common.h", "tpm_internal.h"]:
        shutil.copy(os.path.join(build.CSRC, src), os.path.join(dst, src))


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    monkeypatch.setattr(build, "CSRC", str(tmp_path))
    base = bench.kernel_source_hash()
    assert base == bench.kernel_source_hash()
    k = tmp_path / "k_reduce.hip"
    text = k.read_text(encoding="utf-8")
    k.write_text("// a new line comment\n/* and a\n block comment */\n" + text, encoding="utf-8")
    assert bench.kernel_source_hash() == base
    k.write_text(text + "\nnamespace { constexpr int kUnusedForHash = 1; }\n", encoding="utf-8")
    assert bench.kernel_source_hash() != base
