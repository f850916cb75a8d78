"""The loader refuses, or rebuilds, a libep.so whose recorded source hash
does not match the current sources (CPU only; the library is loaded, no
kernel runs)."""
import os
import shutil

import pytest

from combine_group_limited_amd import _lib, build


@pytest.fixture
def fresh_loader(monkeypatch):
    # a loader with nothing cached, restored afterwards
    monkeypatch.setattr(_lib, "_lib", None)
    yield
    _lib._lib = None


def test_hash_tracks_content_not_time(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("int a;\n")
    h0 = build.source_hash([str(src)])
    os.utime(src, (1, 1))                       # another time stamp, same bytes
    assert build.source_hash([str(src)]) == h0
    src.write_text("int b;\n")                  # same length, other bytes
    assert build.source_hash([str(src)]) != h0


def test_current_library_is_not_stale():
    build.build()
    assert not build.is_stale()
    assert build.built_hash() == build.source_hash()


def test_edited_source_makes_the_loader_rebuild(tmp_path, monkeypatch, fresh_loader):
    # a copy of one source stands in for an edit of it
    edited = tmp_path / "gate.hip"
    shutil.copy(os.path.join(build.CSRC, "gate.hip"), edited)
    inputs = [p for p in build._inputs() if not p.endswith("gate.hip")] + [str(edited)]
    monkeypatch.setattr(build, "_inputs", lambda: inputs)
    monkeypatch.setattr(build, "HASH_PATH", str(tmp_path / "libep.so.sources"))
    with open(build.HASH_PATH, "w") as f:
        f.write(build.source_hash() + "\n")
    assert not build.is_stale()
    edited.write_text(edited.read_text() + "// edited\n")
    assert build.is_stale()
    calls = []

    def fake_build(verbose=False):
        calls.append(1)
        with open(build.HASH_PATH, "w") as f:
            f.write(build.source_hash() + "\n")
        return build.LIB_PATH

    monkeypatch.setattr(build, "build", fake_build)
    L = _lib.lib()
    assert calls == [1] and L.ep_abi_version() > 0
    assert not build.is_stale()


def test_stale_library_without_hipcc_is_refused(tmp_path, monkeypatch, fresh_loader):
    monkeypatch.setattr(build, "HASH_PATH", str(tmp_path / "libep.so.sources"))
    with open(build.HASH_PATH, "w") as f:
        f.write("0" * 64 + "\n")                # built from other sources
    monkeypatch.setattr(build, "hipcc_available", lambda: False)
    with pytest.raises(RuntimeError, match="other sources"):
        _lib.lib()
