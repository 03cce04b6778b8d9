"""The GEMM kernels' device assembly, built from gemm.hip with the
package's own flags (CPU only: hipcc cross-compiles for gfx950).

The probe-matched GEMM's toward-zero slice additions: every probe-mode
kernel must open and close a single-precision round-toward-zero window
around each k tile's slice additions, and every v_add_f32 of those kernels
must lie inside a window: an fp32 addition moved across a MODE write would
round to nearest. The default kernels must contain no MODE write to the
single-precision field.

The default kernels' instruction choice and registers: the whole-K kernels
contract on v_mfma_f32_16x16x32_f16 and the others on
v_mfma_f32_32x32x16_f16, and no GEMM kernel spills registers (a spill in
the k loop would put scratch traffic under every MFMA)."""
import os
import re
import subprocess

import pytest

from fp4_block_scaled_fp4q_amd import build

OPEN = "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 3"
CLOSE = "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0"


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("gemm_asm") / "gemm.s")
    cmd = [build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S", os.path.join(build.CSRC, "gemm.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


def _kernels(text):
    """(name, template arguments, body lines) of every gemm_kernel."""
    lines = text.split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_ZN\S*gemm_kernel\S*:", l)]
    assert starts
    out = []
    for s in starts:
        name = lines[s].split(":")[0]
        e = next(i for i in range(s, len(lines)) if "s_endpgm" in lines[i])
        # gemm_kernel<kBM, kBN, kFullK, kF32Out, kWM, kWN, kSwz, kProbe, kFmt, kK64>
        args = re.findall(r"L[ib](\d+)E", re.search(r"gemm_kernelI(.*)EEvPKh", name).group(1))
        out.append((name, args, lines[s:e]))
    return out


def test_probe_mode_additions_inside_toward_zero_windows(gemm_asm):
    probe_kernels = 0
    for name, args, body in _kernels(gemm_asm):
        probe = args[7] == "1"
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


def test_default_kernels_mfma_shape_and_no_spills(gemm_asm):
    kernels = _kernels(gemm_asm)
    n16 = 0
    for name, args, body in kernels:
        text = "\n".join(body)
        full_k, probe, fmt = args[2] == "1", args[7] == "1", args[8] == "1"
        if full_k and not probe and not fmt:
            n16 += 1
            assert "v_mfma_f32_16x16x32_f16" in text and "v_mfma_f32_32x32x16" not in text, name
        else:
            assert "v_mfma_f32_16x16x32" not in text and "v_mfma_f32_32x32x16" in text, name
    assert n16 == 4  # {bf16, fp32 output} x {row-major, K64}
    counts = re.findall(r"\.vgpr_spill_count:\s+(\d+)", gemm_asm)
    assert counts and all(c == "0" for c in counts), counts
