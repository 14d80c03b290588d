"""Resource gates of the built gfx950 kernels (no GPU needed): register
spills, the per-lane register total and the LDS size of each kernel, read
from the AMDGPU metadata of the code objects inside libsage.so.  The
kernels' occupancy is part of their design -- three attention blocks per CU
hide one another's MFMA and VALU phases, two decode blocks share a CU -- so a
change that spills registers or pushes a kernel past its budget fails here
rather than only showing up as a slower benchmark.  MI355X: 160 KiB of LDS
per CU, 512 registers per SIMD lane (VGPRs and AGPRs together)."""
import os
import re
import shutil
import subprocess

import pytest

LLVM = "/opt/rocm/llvm/bin"
LDS_PER_CU = 160 * 1024
REGS_PER_LANE = 512


def _kernels(tmp_dir):
    """{demangled name: metadata dict} of every kernel in libsage.so."""
    from quantized_attention_block_amd import sage
    if not os.path.exists(sage.LIB_PATH):
        from quantized_attention_block_amd import build
        build.build()
    objdump, readelf, cxxfilt = (os.path.join(LLVM, "llvm-objdump"), os.path.join(LLVM, "llvm-readelf"),
                                 shutil.which("c++filt"))
    if not (os.path.exists(objdump) and os.path.exists(readelf) and cxxfilt):
        pytest.skip("llvm-objdump / llvm-readelf / c++filt not available")
    lib = os.path.join(tmp_dir, "libsage.so")
    shutil.copy(sage.LIB_PATH, lib)
    # writes lib.<i>.<target> next to the copy, one file per offload bundle
    subprocess.run([objdump, "--offloading", lib], check=True, capture_output=True, cwd=tmp_dir)
    kernels = {}
    for fn in sorted(os.listdir(tmp_dir)):
        if not fn.endswith("gfx950"):
            continue
        notes = subprocess.run([readelf, "--notes", os.path.join(tmp_dir, fn)], check=True,
                               capture_output=True, text=True).stdout
        cur = None
        for line in notes.splitlines():
            if re.match(r"^\s+- \.agpr_count:", line):   # first key of a kernel's map
                cur = {}
                line = line.replace("- ", "  ", 1)
            m = re.match(r"^\s+\.(\w+):\s+(\S+)\s*$", line)
            if cur is not None and m:
                cur[m.group(1)] = m.group(2)
                if m.group(1) == "name" and not m.group(2).endswith(".kd"):
                    kernels[m.group(2)] = cur
    if not kernels and os.environ.get("SAGE_LIBRARY"):
        pytest.skip("SAGE_LIBRARY selects a build without gfx950 code objects (the host-only sanitizer build)")
    names = subprocess.run([cxxfilt], input="\n".join(kernels), capture_output=True, text=True,
                           check=True).stdout.split("\n")
    return {d: kernels[m] for m, d in zip(kernels, names)}


@pytest.fixture(scope="module")
def K(tmp_path_factory):
    return _kernels(str(tmp_path_factory.mktemp("code_objects")))


def _pick(K, pattern):
    got = {n: v for n, v in K.items() if re.search(pattern, n)}
    assert got, f"no kernel matches {pattern}"
    return got


def _i(meta, key):
    return int(meta.get(key, 0))


def test_metadata_read(K):
    assert len(K) >= 40
    for n, m in K.items():
        assert "vgpr_count" in m and "group_segment_fixed_size" in m, n


def test_attention_int8_three_blocks_per_cu_without_spills(K):
    for n, m in _pick(K, r"k_attn_fwd<(64|128), false, (true|false)>").items():
        assert _i(m, "vgpr_spill_count") == 0 and _i(m, "private_segment_fixed_size") == 0, n
        assert _i(m, "vgpr_count") <= 168, n                        # 3 waves per SIMD
        assert 3 * _i(m, "group_segment_fixed_size") <= LDS_PER_CU, n


def test_attention_mxfp4_three_blocks_per_cu(K):
    for n, m in _pick(K, r"k_attn_fwd<128, true, (true|false)>").items():
        # the fused form keeps one dword in scratch, outside the KV loop
        assert _i(m, "vgpr_spill_count") <= 1, n
        assert _i(m, "vgpr_count") <= 168, n
        assert 3 * _i(m, "group_segment_fixed_size") <= LDS_PER_CU, n


def test_attention_pingpong_two_waves_per_simd(K):
    for n, m in _pick(K, r"k_attn_fwd_pp").items():
        assert _i(m, "vgpr_spill_count") == 0, n
        assert 2 * _i(m, "vgpr_count") <= REGS_PER_LANE, n
        assert _i(m, "group_segment_fixed_size") <= LDS_PER_CU, n


def test_decode_two_blocks_per_cu_at_head_dim_128(K):
    for n, m in _pick(K, r"k_paged_decode<\d+, (true|false), 128, (true|false)>").items():
        assert _i(m, "vgpr_spill_count") == 0, n
        assert 2 * _i(m, "vgpr_count") <= REGS_PER_LANE, n         # 2 waves per SIMD
        assert 2 * _i(m, "group_segment_fixed_size") <= LDS_PER_CU, n
    for n, m in _pick(K, r"k_paged_decode<\d+, (true|false), 256, (true|false)>").items():
        assert _i(m, "vgpr_spill_count") == 0, n
        assert _i(m, "vgpr_count") <= REGS_PER_LANE // 2, n
        assert _i(m, "group_segment_fixed_size") <= LDS_PER_CU, n
    for n, m in _pick(K, r"k_decode_merge<").items():
        assert _i(m, "vgpr_spill_count") == 0 and _i(m, "private_segment_fixed_size") == 0, n


def test_quantizers_spill_at_most_their_known_count(K):
    for n, m in _pick(K, r"k_(quant|mean|v_amax|v_quant)").items():
        limit = 2 if re.search(r"k_quant_qk_fused<128", n) else 0
        assert _i(m, "vgpr_spill_count") <= limit, n
        assert _i(m, "group_segment_fixed_size") <= LDS_PER_CU, n
