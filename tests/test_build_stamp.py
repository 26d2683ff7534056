"""The build stamp: each built library records a hash of the sources and
flags it was built from (exact_attention_26_amd.build.source_stamp), so that
the GPU tests refuse a library that is older than the sources in the tree."""
import os

import pytest

import exact_attention_26_amd as fa
from exact_attention_26_amd import build


def test_stamp_depends_on_flags_and_sources(tmp_path, monkeypatch):
    base = build.source_stamp([])
    assert base == build.source_stamp([])  # deterministic
    assert base != build.source_stamp(["-DFA_DEBUG_TRACE"])
    # A copy of the sources with one byte changed gives another stamp.
    for sub, src in (("csrc", build.CSRC), ("include", build.INCLUDE)):
        os.makedirs(tmp_path / sub)
        for name in os.listdir(src):
            with open(os.path.join(src, name), "rb") as f:
                (tmp_path / sub / name).write_bytes(f.read())
    monkeypatch.setattr(build, "CSRC", str(tmp_path / "csrc"))
    monkeypatch.setattr(build, "INCLUDE", str(tmp_path / "include"))
    assert build.source_stamp([]) == base  # the same bytes at another path
    hdr = tmp_path / "include" / "fa.h"
    hdr.write_bytes(hdr.read_bytes() + b"\n")
    assert build.source_stamp([]) != base


def test_missing_stamp_is_not_current(tmp_path):
    assert not build.is_current(str(tmp_path / "libfa.so"))


@pytest.mark.parametrize("path", [fa.LIB_PATH, fa.POISON_LIB_PATH, fa.TRACE_LIB_PATH])
def test_built_libraries_are_current(path):
    if not os.path.exists(path):
        pytest.skip(f"{os.path.basename(path)} is not built")
    assert build.is_current(path), f"{os.path.basename(path)} is older than its sources"
