"""Register budget of the built kernels (no kernel runs): every gfx950 kernel
in libslt.so compiles without VGPR spills, without a private (scratch)
segment and without a dynamic stack.  A VGPR spill turns register traffic
into memory traffic in the hot loop or epilogue; the 256 x 256 GEMM sits at
the 256-VGPR limit, so a small epilogue change can push it over without any
change in results.  SGPR spills are allowed while the private segment stays
empty: they go to VGPR lanes, not to memory.

The code objects are read from the library's .hip_fatbin section (clang
offload bundles, one per compiled source) and their AMDGPU metadata notes are
printed by llvm-readelf."""
import os
import re
import shutil
import struct
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "scratch_llama_transformer_amd", "libslt.so")
READELF = next((p for p in ("/opt/rocm/llvm/bin/llvm-readelf", shutil.which("llvm-readelf")) if p and os.path.exists(p)),
               None)

pytestmark = [pytest.mark.skipif(not os.path.exists(LIB), reason="libslt.so not built"),
              pytest.mark.skipif(READELF is None, reason="llvm-readelf not found")]

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def fatbin_section(blob):
    """Bytes of the .hip_fatbin section of a 64-bit little-endian ELF file."""
    shoff = struct.unpack_from("<Q", blob, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", blob, 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQIIQQ", blob, shoff + i * shentsize) for i in range(shnum)]
    strtab = hdrs[shstrndx][4]
    for h in hdrs:
        name = blob[strtab + h[0]:blob.index(b"\0", strtab + h[0])]
        if name == b".hip_fatbin":
            return blob[h[4]:h[4] + h[5]]
    raise AssertionError("no .hip_fatbin section")


def device_code_objects(sec, arch="gfx950"):
    """The device entries of every offload bundle: magic, entry count, then
    per entry its offset, size, target-triple length and triple."""
    out = []
    for m in re.finditer(re.escape(BUNDLE_MAGIC), sec):
        base = m.start()
        n = struct.unpack_from("<Q", sec, base + len(BUNDLE_MAGIC))[0]
        q = base + len(BUNDLE_MAGIC) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", sec, q)
            q += 24
            triple = sec[q:q + tlen].decode()
            q += tlen
            if arch in triple:
                out.append(sec[base + off:base + off + size])
    return out


def kernel_resources():
    sec = fatbin_section(open(LIB, "rb").read())
    objs = device_code_objects(sec)
    assert objs, "no gfx950 code object in the library"
    res = {}
    with tempfile.TemporaryDirectory() as d:
        for i, co in enumerate(objs):
            path = os.path.join(d, f"k{i}.co")
            with open(path, "wb") as f:
                f.write(co)
            notes = subprocess.run([READELF, "--notes", path], capture_output=True, text=True, check=True).stdout
            for blk in re.split(r"\n\s*- \.agpr_count:", notes)[1:]:
                field = lambda k: re.search(rf"\.{k}:\s+(\S+)", blk).group(1)
                res[field("name")] = {"vgpr": int(field("vgpr_count")), "vgpr_spill": int(field("vgpr_spill_count")),
                                      "sgpr_spill": int(field("sgpr_spill_count")),
                                      "private": int(field("private_segment_fixed_size")),
                                      "dynamic_stack": field("uses_dynamic_stack") == "true"}
    return res


def test_no_kernel_spills_vgprs_or_uses_scratch():
    res = kernel_resources()
    # the GEMM, attention and row kernels are all there
    for part in ("gemm_w8_k", "gemm_d64_k", "gemm_dl_k", "fl_fwd_k", "fl_dq_k", "fl_dkdv2_k", "norm_bwd_k", "adamw_k"):
        assert any(part in k for k in res), part
    bad = {k: v for k, v in res.items() if v["vgpr_spill"] or v["private"] or v["dynamic_stack"]}
    assert not bad, bad
    assert max(v["vgpr"] for v in res.values()) <= 512
