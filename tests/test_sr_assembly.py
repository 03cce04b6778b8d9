"""The stochastic-rounding quantize kernels' hand-scheduled pieces, checked
in the device assembly of quantize.hip built with the package's own flags
(CPU only: hipcc cross-compiles for gfx950).

- Every fused multiply-add of the SR decision and every conversion of a
  Philox word to binary32 runs inside a single-precision round-toward-zero
  window (a MODE write to 3 ... a MODE write to 0), and the windows hold
  nothing else that rounds: an operation outside would round to nearest,
  one inside that is not meant to would round toward zero.
- Each window's opening write is followed by wait states before its first
  instruction.
- The byte-select conversions that pack four pairs of codes write one
  destination register, and every one that writes a byte other than the
  lowest is followed by a wait state (as the compiler schedules the
  round-to-nearest form of the same chain).
- The round-to-nearest kernels hold no MODE write and no stochastic
  conversion.
- No quantize kernel spills registers."""
import os
import re
import subprocess

import pytest

from fp4_block_scaled_fp4q_amd import build

OPEN = "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 3"
CLOSE = "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0"
CVT_SR = "v_cvt_scalef32_sr_pk_fp4_f32"
# floating-point operations whose rounding the MODE field governs and that
# may appear inside a window
IN_WINDOW = ("v_fma_f32", "v_cvt_f32_u32")
# the SR decision's two multiply-adds: |v| - q' s2 (an abs modifier on the
# addend) and s2 * 0.5 + t
SR_FMA = (re.compile(r"^v_fma_f32 v\d+, -v\d+, v\d+, \|v\d+\|$"), re.compile(r"^v_fma_f32 v\d+, v\d+, 0\.5, v\d+$"))


def _kernels(lines, pattern):
    for s, l in enumerate(lines):
        m = re.match(r"^(_ZN\S*" + pattern + r"\S*):", l)
        if m:
            e = next(i for i in range(s, len(lines)) if "s_endpgm" in lines[i])
            yield m.group(1), [x.strip() for x in lines[s:e]]


@pytest.mark.skipif(not os.path.exists(build.HIPCC), reason="hipcc not available")
def test_sr_windows_and_conversion_chains(tmp_path):
    out = str(tmp_path / "quantize.s")
    cmd = [build.HIPCC, *build.FLAGS, "--cuda-device-only", "-S", os.path.join(build.CSRC, "quantize.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = open(out).read()
    lines = text.split("\n")
    spills = re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)
    assert spills and all(c == "0" for c in spills), spills
    sr_kernels = rne_kernels = 0
    for name, body in _kernels(lines, r"quant_(row|dual|tile|tile32)_kernel"):
        # template arguments <kBF16, kSR, ...>: the second is kSR
        flags = re.findall(r"Lb(\d)E", name)
        sr = flags[1] == "1"
        ins = [l for l in body if l and not l.startswith((".", ";")) and not l.split()[0].endswith(":")]
        if not sr:
            rne_kernels += 1
            assert not any(OPEN in l or CLOSE in l for l in ins), f"{name}: MODE write in an RNE kernel"
            assert not any(CVT_SR in l for l in ins), f"{name}: stochastic conversion in an RNE kernel"
            continue
        sr_kernels += 1
        inside, windows, content = False, 0, []
        for i, l in enumerate(ins):
            op = l.split()[0]
            if OPEN in l:
                assert not inside, f"{name}: nested window"
                inside, content = True, []
                assert ins[i + 1].startswith("s_nop"), f"{name}: no wait states after the MODE write"
            elif CLOSE in l:
                assert inside, f"{name}: window closed without opening"
                inside = False
                windows += 1
                # a window converts 8 words, or takes 4 elements' two
                # multiply-adds each
                kinds = sorted(x.split()[0] for x in content)
                assert kinds in (["v_cvt_f32_u32"] * 8, ["v_fma_f32"] * 8), f"{name}: window holds {kinds}"
                if kinds[0] == "v_fma_f32":
                    assert all(any(p.match(x) for p in SR_FMA) for x in content), f"{name}: {content}"
            elif inside:
                assert op in IN_WINDOW or op.startswith("s_nop"), f"{name}: {op} inside a toward-zero window"
                if op in IN_WINDOW:
                    content.append(l)
            else:
                # other fp32 arithmetic (the tensor scale's division) rounds
                # to nearest, outside; the SR multiply-adds never do
                assert not any(p.match(l) for p in SR_FMA), f"{name}: {l} outside the toward-zero windows"
        assert not inside, f"{name}: window left open"
        assert windows > 0, f"{name}: no toward-zero window"
        # the conversion chains: 4 consecutive conversions (with wait states
        # between them) into one register, byte selects 0, 1, 2, 3
        cv = [i for i, l in enumerate(ins) if l.startswith(CVT_SR)]
        assert cv and len(cv) % 4 == 0, f"{name}: {len(cv)} stochastic conversions"
        for c in range(0, len(cv), 4):
            chain = [ins[i] for i in cv[c:c + 4]]
            dsts = {l.split()[1].rstrip(",") for l in chain}
            assert len(dsts) == 1, f"{name}: chain writes {dsts}"
            sels = [re.search(r"op_sel:\[0,0,(\d),(\d)\]", l) for l in chain]
            assert [0 if m is None else int(m.group(1)) + 2 * int(m.group(2)) for m in sels] == [0, 1, 2, 3], \
                f"{name}: byte selects of {chain}"
            for i in cv[c + 1:c + 4]:
                assert ins[i + 1].startswith("s_nop"), f"{name}: no wait state after {ins[i]}"
            assert cv[c + 3] - cv[c] <= 5, f"{name}: chain not contiguous"
    assert sr_kernels >= 8 and rne_kernels >= 8, (sr_kernels, rne_kernels)
