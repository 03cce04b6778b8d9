"""The probe-matched GEMM's toward-zero slice additions, checked in the
device assembly of gemm.hip built with the package's own flags (CPU only:
hipcc cross-compiles for gfx950). Every probe-mode kernel must open and close
a single-precision round-toward-zero window around each k tile's slice
additions, and every v_add_f32 of those kernels must lie inside a window: an
fp32 addition moved across a MODE write would round to nearest. The default
kernels must contain no MODE write to the single-precision field."""
import os
import re
import shutil
import subprocess

import pytest

from fp4_block_scaled_fp4q_amd import build

OPEN = "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 3"
CLOSE = "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0"


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not available")
def test_probe_mode_additions_inside_toward_zero_windows(tmp_path):
    out = str(tmp_path / "gemm.s")
    cmd = [build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S", os.path.join(build.CSRC, "gemm.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = open(out).read().split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_ZN\S*gemm_kernel\S*:", l)]
    assert starts
    probe_kernels = 0
    for s in starts:
        name = lines[s].split(":")[0]
        e = next(i for i in range(s, len(lines)) if "s_endpgm" in lines[i])
        body = lines[s:e]
        # template argument 8 (kProbe) of gemm_kernel<kBM, kBN, kFullK, kF32Out, kWM, kWN, kSwz, kProbe, ...>
        args = re.search(r"gemm_kernelI(.*)EEvPKh", name).group(1)
        probe = re.findall(r"L[ib](\d+)E", args)[7] == "1"
        inside, windows, n, adds_in, adds_out = False, [], 0, 0, 0
        for l in body:
            if OPEN in l:
                assert not inside, f"{name}: nested window"
                inside, n = True, 0
            elif CLOSE in l:
                assert inside, f"{name}: window closed without opening"
                windows.append(n)
                inside = False
            elif "v_add_f32" in l:
                if inside:
                    n += 1
                else:
                    adds_out += 1
        assert not inside, f"{name}: window left open"
        if probe:
            probe_kernels += 1
            assert windows and all(w == windows[0] and w > 0 for w in windows), f"{name}: windows {windows}"
            assert adds_out == 0, f"{name}: {adds_out} fp32 additions outside the toward-zero windows"
        else:
            assert not windows, f"{name}: a default kernel writes the rounding field"
    assert probe_kernels >= 4
