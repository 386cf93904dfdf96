"""Kernel resources of the built library, read from its gfx950 code object's metadata.

Host-only: the HIP library embeds its device code as clang offload bundles in the
``.hip_fatbin`` section; ``llvm-readelf --notes`` prints each kernel's metadata.
Every kernel must run without scratch memory (no register spills to memory) and fit
the 160 KB of LDS a gfx950 workgroup may use.
"""
import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

from ring_attention_ringattn_amd import _lib

READELF = shutil.which("llvm-readelf") or "/opt/rocm/llvm/bin/llvm-readelf"
LDS_LIMIT = 160 * 1024


def _sections(data):
    shoff = struct.unpack_from("<Q", data, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)
    secs = [struct.unpack_from("<IIQQQQIIQQ", data, shoff + i * shentsize) for i in range(shnum)]
    strtab = secs[shstrndx][4]

    def name(off):
        return data[strtab + off: data.index(b"\0", strtab + off)].decode()
    return {name(s[0]): (s[4], s[5]) for s in secs}


def _code_objects(path):
    """The gfx950 code objects of every offload bundle in the library's fat binary."""
    data = open(path, "rb").read()
    off, size = _sections(data)[".hip_fatbin"]
    blob = data[off: off + size]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    i = blob.find(magic)
    while i >= 0:
        n = struct.unpack_from("<Q", blob, i + 24)[0]
        p = i + 32
        for _ in range(n):
            eoff, esize, tlen = struct.unpack_from("<QQQ", blob, p)
            p += 24
            triple = blob[p: p + tlen].decode()
            p += tlen
            if "gfx950" in triple and esize:
                yield blob[i + eoff: i + eoff + esize]
        i = blob.find(magic, i + 1)


def _kernels(path):
    """{kernel symbol: {metadata key: int}} for the keys this test checks."""
    keys = ("group_segment_fixed_size", "private_segment_fixed_size", "vgpr_spill_count", "vgpr_count")
    out = {}
    for co in _code_objects(path):
        with tempfile.NamedTemporaryFile(suffix=".co", delete=False) as f:
            f.write(co)
        try:
            notes = subprocess.run([READELF, "--notes", f.name], capture_output=True, text=True, check=True).stdout
        finally:
            os.unlink(f.name)
        # each kernel is one list item of the metadata; its keys are sorted, so split at
        # the item markers and read the keys of each item
        for item in re.split(r"\n\s*-\s+\.agpr_count:", notes)[1:]:
            m = re.search(r"\.name:\s+(\S+)", item)
            if not m:
                continue
            out[m.group(1)] = {k: int(v) for k, v in re.findall(r"\.(%s):\s+(\d+)" % "|".join(keys), item)}
    return out


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("the HIP library is not built")
    if not os.path.exists(READELF):
        pytest.skip("llvm-readelf is not available")
    ks = _kernels(_lib.LIB_PATH)
    assert ks, "no gfx950 kernels found in the library's fat binary"
    return ks


def test_every_hot_kernel_is_present(kernels):
    names = " ".join(kernels)
    for k in ("fwd_bf16_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "merge_kernel", "bwd_pre_kernel",
              "vt_transpose_kernel", "tile_ranges_batch_kernel", "fwd_f32_kernel", "bwd_dq_f32_kernel",
              "bwd_dkdv_f32_kernel"):
        assert k in names, k


def test_no_kernel_uses_scratch_memory(kernels):
    bad = {k: v for k, v in kernels.items()
           if v.get("private_segment_fixed_size", 0) != 0 or v.get("vgpr_spill_count", 0) != 0}
    assert not bad, bad


def test_lds_fits_a_workgroup(kernels):
    for k, v in kernels.items():
        assert v.get("group_segment_fixed_size", 0) <= LDS_LIMIT, (k, v)
