"""Properties of the device code that hipcc shows without a GPU: each HIP
source is compiled to gfx950 assembly with the library's own flags, and
every kernel must use no scratch memory (no register spills), no packed
fp32 arithmetic may appear, and no store, atomic, write-back or discard may
go through the scalar data cache (stores are vector stores only)."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest
import yaml

from combine_group_limited_amd import build as B

HIPCC = B.HIPCC if os.path.exists(B.HIPCC) else shutil.which("hipcc")
pytestmark = pytest.mark.skipif(not HIPCC, reason="hipcc not found")

PACKED_FP32 = re.compile(r"^\s+v_pk_(add|mul|fma)_f32\b", re.M)
SCALAR_WRITE = re.compile(r"^\s+s_(store|atomic|buffer_store|scratch_store|dcache_wb|dcache_discard)\w*", re.M)


def _isa(src: str, out_dir: str) -> str:
    flags = [f for f in B.HIPFLAGS if f not in ("-fPIC", "-Wall")]
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    r = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", "-o", out, src], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return open(out).read()


@pytest.fixture(scope="module")
def isa():
    with tempfile.TemporaryDirectory() as d:
        names = B.SOURCES + B.PROBE_SOURCES + B.CHECK_SOURCES
        srcs = [os.path.join(B.CSRC, f) for f in names]
        with cf.ThreadPoolExecutor(max_workers=min(6, len(srcs))) as ex:
            return dict(zip(names, ex.map(lambda s: _isa(s, d), srcs)))


def _kernels(text):
    """The kernel descriptors of one assembly file (its YAML metadata)."""
    m = re.search(r"^\s*\.amdgpu_metadata\s*$(.*?)^\s*\.end_amdgpu_metadata", text, re.M | re.S)
    assert m, "no metadata"
    return yaml.safe_load(m.group(1))["amdhsa.kernels"]


def test_no_scratch_and_no_vgpr_spills(isa):
    # (an SGPR spill lands in VGPR lanes, not in memory, so it is allowed)
    kernels = 0
    for name, text in isa.items():
        for k in _kernels(text):
            kernels += 1
            assert k[".private_segment_fixed_size"] == 0, (name, k[".name"])
            assert k.get(".vgpr_spill_count", 0) == 0, (name, k[".name"])
    assert kernels >= 20, kernels


def test_no_packed_fp32_arithmetic(isa):
    for name, text in isa.items():
        assert not PACKED_FP32.search(text), name


def test_no_scalar_cache_writes(isa):
    for name, text in isa.items():
        hit = SCALAR_WRITE.search(text)
        assert hit is None, (name, hit.group(0) if hit else None)
