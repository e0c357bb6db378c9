"""The built gfx950 kernels use no scratch memory.

"mmaemu backends" (Building fatbins) makes its build fail when the compiler
reports spill bytes. The same gate here reads the kernel descriptors of the
code objects inside the built libmmfp8.so: every kernel must report zero VGPR
and SGPR spills and no private (scratch) segment. The code objects are the
gfx950 entries of the clang offload bundles the HIP link places in the
library; their AMDGPU metadata note (msgpack) lists each kernel's resources.
"""
import struct

import msgpack
import pytest

import block_scaled_gemm_amd as mm

MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
NT_AMDGPU_METADATA = 32


def code_objects(blob: bytes):
    """The gfx950 code objects of every offload bundle in blob."""
    pos = 0
    while True:
        i = blob.find(MAGIC, pos)
        if i < 0:
            return
        n, = struct.unpack_from("<Q", blob, i + 24)
        off = i + 32
        for _ in range(n):
            eo, es, ts = struct.unpack_from("<QQQ", blob, off)
            off += 24
            triple = blob[off:off + ts].decode()
            off += ts
            if "gfx950" in triple:
                yield blob[i + eo:i + eo + es]
        pos = i + len(MAGIC)


def kernel_metadata(co: bytes):
    """amdhsa.kernels of an ELF64 code object (from its PT_NOTE segments)."""
    assert co[:4] == b"\x7fELF" and co[4] == 2, "not an ELF64 code object"
    phoff, = struct.unpack_from("<Q", co, 32)
    phentsize, phnum = struct.unpack_from("<HH", co, 54)
    out = []
    for p in range(phnum):
        ptype, _, poff, _, _, pfsz = struct.unpack_from("<IIQQQQ", co, phoff + p * phentsize)
        if ptype != 4:  # PT_NOTE
            continue
        q = poff
        while q < poff + pfsz:
            namesz, descsz, ntype = struct.unpack_from("<III", co, q)
            dstart = q + 12 + ((namesz + 3) & ~3)
            if ntype == NT_AMDGPU_METADATA:
                out += msgpack.unpackb(co[dstart:dstart + descsz], raw=False).get("amdhsa.kernels", [])
            q = dstart + ((descsz + 3) & ~3)
    return out


@pytest.fixture(scope="module")
def kernels():
    blob = open(mm.LIB_PATH, "rb").read()
    ks = [k for co in code_objects(blob) for k in kernel_metadata(co)]
    assert ks, "no gfx950 kernels found in the library"
    return {k[".name"]: k for k in ks}


def test_every_kernel_family_is_present(kernels):
    names = " ".join(kernels)
    for family in ("gemm_tile", "gemm_skinny", "gemm_skinny_k", "gemm_ksplit", "transpose_kernel", "group_pack_kernel",
                   "amax_init", "amax_finalize", "debug_convert"):
        assert family in names, family


def test_no_kernel_spills_to_memory(kernels):
    bad = {n: (k.get(".vgpr_spill_count"), k.get(".private_segment_fixed_size"))
           for n, k in kernels.items() if k.get(".vgpr_spill_count", 0) or k.get(".private_segment_fixed_size", 0)}
    assert not bad, f"kernels with VGPR spills or scratch memory (vgpr spills, private bytes): {bad}"


def test_sgpr_spills_stay_in_vgpr_lanes(kernels):
    """SGPR spills are written to lanes of a VGPR (v_writelane / v_readlane, no memory traffic): a kernel that
    has them must still have no private segment. (The block-scaled and MX tile kernels have them: their
    per-step scale and LDS-DMA offsets are scalar.)"""
    for n, k in kernels.items():
        if k.get(".sgpr_spill_count", 0):
            assert k.get(".private_segment_fixed_size", 0) == 0, n
            assert "gemm_tile" in n, n


def test_kernels_fit_the_register_file(kernels):
    # 512 VGPRs (arch + acc) per lane at one wave per SIMD; the descriptors report what each kernel allocates
    for n, k in kernels.items():
        assert k.get(".vgpr_count", 0) + k.get(".agpr_count", 0) <= 512, n
