"""Register and scratch budget of every kernel in the built library.

The library's gfx950 code objects carry, per kernel, the bytes of private
(scratch) memory each lane uses and the registers the compiler spilled.  A
weight stream whose buffers land in scratch memory (an array indexed at run
time, a spill) sends every element through the vector-memory pipeline twice
more and runs several times slower, with correct results, so no parity test
notices it.  This test reads the metadata out of the built library (offload
bundles in its .hip_fatbin section, the AMDGPU metadata note of each code
object) and holds every kernel to no scratch memory, except the two whose use
is known and bounded below.
"""
import os
import struct

import pytest

from speculative_decode_verification_router_amd import binding as bd

msgpack = pytest.importorskip("msgpack")

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NT_AMDGPU_METADATA = 32

# kernel name fragment -> (max private bytes per lane, max VGPR spills)
KNOWN = {
    # the run-time-shape instance of the GEMM down + shared kernel (model
    # shapes without a compiled instance); the compiled one spills nothing
    "k_gemm_down_sharedILi0ELi0E": (160, 48),
    # a few SGPR spills of the routing kernel
    "k_routeI": (48, 0),
}


def _bundles(blob):
    """(triple, code object bytes) of every offload bundle in `blob`."""
    out, at = [], blob.find(BUNDLE_MAGIC)
    while at >= 0:
        n, = struct.unpack_from("<Q", blob, at + 24)
        p = at + 32
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", blob, p)
            triple = blob[p + 24:p + 24 + tlen].decode()
            p += 24 + tlen
            out.append((triple, blob[at + off:at + off + size]))
        at = blob.find(BUNDLE_MAGIC, at + 1)
    return out


def _metadata(elf):
    """The AMDGPU metadata map of one ELF64 code object."""
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum = struct.unpack_from("<HH", elf, 0x3A)
    for i in range(shnum):
        sh = shoff + i * shentsize
        sh_type, = struct.unpack_from("<I", elf, sh + 4)
        if sh_type != 7:  # SHT_NOTE
            continue
        off, size = struct.unpack_from("<QQ", elf, sh + 0x18)
        p, end = off, off + size
        while p < end:
            namesz, descsz, ntype = struct.unpack_from("<III", elf, p)
            name = elf[p + 12:p + 12 + namesz].rstrip(b"\0")
            desc_at = p + 12 + ((namesz + 3) & ~3)
            if name == b"AMDGPU" and ntype == NT_AMDGPU_METADATA:
                return msgpack.unpackb(elf[desc_at:desc_at + descsz], raw=False)
            p = desc_at + ((descsz + 3) & ~3)
    raise AssertionError("no AMDGPU metadata note")


def _kernels():
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("library not built")
    blob = open(bd.LIB_PATH, "rb").read()
    kernels = []
    for triple, obj in _bundles(blob):
        if "gfx950" in triple and obj[:4] == b"\x7fELF":
            kernels += _metadata(obj)["amdhsa.kernels"]
    return kernels


def test_every_kernel_keeps_its_buffers_in_registers():
    kernels = _kernels()
    assert len(kernels) > 20  # every source's gfx950 code object was found
    names = [k[".name"] for k in kernels]
    for frag in ("k_ffn_small", "k_gate_up_mid", "k_down_mid", "k_one_launch", "k_lm_argmax", "k_gemm_gate_up"):
        assert any(frag in n for n in names), frag
    for k in kernels:
        name, priv = k[".name"], k[".private_segment_fixed_size"]
        spills = k.get(".vgpr_spill_count", 0)
        limit = next((v for f, v in KNOWN.items() if f in name), (0, 0))
        assert priv <= limit[0] and spills <= limit[1], (name, priv, spills)
