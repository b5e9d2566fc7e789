"""Compile the GEMM for gfx950 and check the hot kernels' register use.

A VGPR spill in the GEMM main loop costs ~8x (scratch traffic per MFMA); the
kernels the training passes launch (fprop NT act x block, dgrad NN act x
block, wgrad NT act x act -- the 8-wave float32-scale kernel and the 4-wave
power-of-two kernel -- and the 1x32 MXFP8 NT kernel) must compile without
spills, and the power-of-two kernels must keep their accumulators in the
AGPR file.  CPU only (hipcc cross-compiles)."""
import os
import re
import shutil
import subprocess

import pytest

from blockwise_fp8_gemm_bfp8_amd import build as bfp8_build

HOT = {
    "fprop NT act x block": r"111gemm_kernelILb0ELb0ELi0ELi1ELi256EE",
    "dgrad NN act x block": r"111gemm_kernelILb0ELb1ELi0ELi1ELi256EE",
    "wgrad NT act x act": r"111gemm_kernelILb0ELb0ELi0ELi0ELi256EE",
    # 256 x 192 tiles (the 2048 x 6144 wgrad output), K-block-major act scales
    "wgrad NT act x act, 192 columns": r"111gemm_kernelILb0ELb0ELi3ELi3ELi192EE",
    # power-of-two (E8M0) scales, hardware-scaled MFMA, 4 waves
    "mx fprop NT act x block": r"gemm_mx4_kernelILb0ELb0ELi0ELi1EE",
    "mx dgrad NN act x block": r"gemm_mx4_kernelILb0ELb1ELi0ELi1EE",
    "mx wgrad NT act x act": r"gemm_mx4_kernelILb0ELb0ELi0ELi0EE",
    "mx32 NT 1x32 x 1x32": r"gemm_mx4_kernelILb0ELb0ELi2ELi2EE",
}


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    cmd = [bfp8_build.hipcc(), *bfp8_build.compile_flags(), "-x", "hip", "-S", "--cuda-device-only",
           os.path.join(bfp8_build.CSRC, "gemm.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def kernel_meta(asm, pattern):
    meta = asm[asm.index("amdhsa.kernels:"):]
    for blk in re.split(r"\n  - ", meta)[1:]:
        name = re.search(r"\.name:\s+(\S+)", blk)
        if name and re.search(pattern, name.group(1)):
            get = lambda k: int(re.search(r"\." + k + r":\s+(\d+)", blk).group(1))
            return {k: get(k) for k in ("vgpr_count", "agpr_count", "vgpr_spill_count",
                                        "sgpr_spill_count", "private_segment_fixed_size",
                                        "group_segment_fixed_size")}
    raise AssertionError(f"kernel {pattern} not found")


@pytest.mark.parametrize("role", list(HOT))
def test_hot_gemm_kernels_do_not_spill(gemm_asm, role):
    m = kernel_meta(gemm_asm, HOT[role])
    assert m["vgpr_spill_count"] == 0, (role, m)
    assert m["private_segment_fixed_size"] == 0, (role, m)
    assert m["group_segment_fixed_size"] <= 160 * 1024, (role, m)
    if "mx" in role:
        assert m["agpr_count"] == 256, (role, m)
