"""GPU parity of amax, quantize and dequant against the oracle: bit-exact
codes, scales, tensor scale, repair counts and amax.

Inputs are seeded and synthetic (shapes span several workgroups and end in
ragged tails); the exhaustive cases enumerate every bf16 input of a range."""
import numpy as np
import pytest
import torch

import oracle
from fp4_block_scaled_fp4q_amd import api, inputs
from parity_util import DEV, assert_quant_equal, dev_scalar, host_view, quant_both

pytestmark = pytest.mark.gpu


def _t3(shape, seed, dtype=torch.bfloat16, outliers=True):
    rng = np.random.default_rng(seed)
    cols = inputs.outlier_columns(rng, shape[1]) if outliers else np.array([], int)
    x = inputs.activation(rng, shape[0], shape[1], cols)
    return inputs.to_bf16(x) if dtype == torch.bfloat16 else torch.from_numpy(x)


def _grad(shape, seed, dtype=torch.bfloat16):
    x = inputs.loguniform_grad(np.random.default_rng(seed), *shape)
    return inputs.to_bf16(x) if dtype == torch.bfloat16 else torch.from_numpy(x)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape,pad", [((1, 16), 0), ((37, 4104), 0), ((300, 520), 8),
                                        ((4096, 1024), 0), ((0, 64), 0)])
def test_amax(dtype, shape, pad):
    x = _t3(shape, 1, dtype) if shape[0] else torch.zeros(shape, dtype=dtype)
    if pad:
        buf = torch.zeros((shape[0], shape[1] + pad), dtype=dtype)
        buf[:, :shape[1]] = x
        xd = buf.to(DEV)[:, :shape[1]]
    else:
        xd = x.to(DEV)
    got = api.amax(xd).cpu().numpy()[0]
    want = oracle.amax(host_view(x))
    assert np.float32(got).view(np.uint32) == np.float32(want).view(np.uint32)


CASES = [("row16", (37, 4128)), ("row16", (16, 64)), ("col16", (48, 1048)), ("col16", (32, 4104)),
         ("col16", (208, 4104)), ("tile", (48, 1056)), ("tile", (64, 4128)), ("tile", (208, 528)),
         ("row16+col16", (48, 1056)), ("row16+col16", (208, 4128))]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("layout,shape", CASES)
def test_quantize_parity(layout, shape, rnd, dtype):
    x = _grad(shape, 3, dtype) if rnd else _t3(shape, 2, dtype)
    a = float(oracle.amax(host_view(x)))
    both = layout == "row16+col16"
    lay = "row16" if both else layout
    for held, T in ((a, 448.0), (a * 0.01, 448.0), (a * 300.0, 2048.0)):
        g, o = quant_both(x, held, lay, rnd, T, seed=0x5EED_0001_0000_0007, subseq=2,
                          transposed=(layout == "tile" or both))
        assert_quant_equal(g, o, f"{layout} {shape} rnd={rnd} held={held} T={T}")


def test_quantize_strided_rows():
    x = _t3((64, 256), 4)
    g, o = quant_both(x, 3.0, "row16", ld_pad=64)
    assert_quant_equal(g, o)
    g, o = quant_both(x, 3.0, "col16", ld_pad=8)
    assert_quant_equal(g, o)
    g, o = quant_both(x, 3.0, "tile", transposed=True, ld_pad=16)
    assert_quant_equal(g, o)
    g, o = quant_both(x, 3.0, "row16", transposed=True, ld_pad=24)
    assert_quant_equal(g, o)


def test_hand_worked_blocks_on_gpu():
    rows = [
        ([6, -3, 1.5, 0.75, 0.25, -0.25, 1.25, 1.75, 2.5, 3.5, 5, -5, 0, -0.0, 4, 0.5], 6.0),
        ([1.0, 0.3, -0.5, 0.05], 10.0),
        ([1e-6, -1e-7], 1e6),
        ([200, 100, -50, 1], 1.0),
    ]
    for vals, held in rows:
        x = torch.zeros((1, 16), dtype=torch.float32)
        x[0, :len(vals)] = torch.tensor(vals, dtype=torch.float32)
        g, o = quant_both(x, held, "row16")
        assert_quant_equal(g, o, str(vals))


def _all_bf16(lo_abs, hi_abs):
    """Every finite bf16 value v with lo_abs <= |v| <= hi_abs, both signs."""
    bits = np.arange(0x8000, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) >= lo_abs) & (np.abs(vals) <= hi_abs)
    pos = bits[keep].astype(np.uint16)
    return np.concatenate([pos, pos | 0x8000])


@pytest.mark.parametrize("rnd", [0, 1])
def test_exhaustive_bf16_payloads(rnd):
    # rows of 16: an anchor 6 (held A = 6, T = 448 -> S = 448, scale 448,
    # r = 1) and 15 enumerated values, so every bf16 input in [-8, 8] is
    # encoded directly by the payload rule
    v = _all_bf16(0.0, 8.0)
    n = (len(v) + 14) // 15
    body = np.zeros(n * 15, np.uint16)
    body[:len(v)] = v
    bits = np.zeros((n, 16), np.uint16)
    bits[:, 0] = 0x40C0  # bf16 6.0
    bits[:, 1:] = body.reshape(n, 15)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    g, o = quant_both(x, 6.0, "row16", rnd, seed=77)
    assert_quant_equal(g, o, "payload sweep")


@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("held,T", [(1.0, 448.0), (1e-3, 448.0), (3e4, 2048.0), (2.5e-30, 448.0)])
def test_exhaustive_block_scales(held, T, rnd):
    # one block per positive finite bf16 bamax: exercises both per-block
    # divisions, the UE5M3 rounding (incl. ties), zero/saturation repair and
    # the overflowing-multiplier path; with held = 2.5e-30 the saturated
    # scales let x * r overflow to +-Inf for the largest inputs, which both
    # roundings must encode as +-6
    v = _all_bf16(0.0, 3.4e38)
    v = v[(v & 0x8000) == 0]
    v = v[v != 0]
    bits = np.zeros((len(v), 16), np.uint16)
    bits[:, 0] = v
    bits[:, 1] = v | 0x8000
    bits[:, 2] = (v.astype(np.uint32) - 1).clip(0).astype(np.uint16)  # just below bamax
    bits[:, 3] = (v >> 1)                                               # about sqrt-ish smaller
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    g, o = quant_both(x, held, "row16", rnd, T, seed=11)
    assert_quant_equal(g, o, f"held={held} T={T} rnd={rnd}")


@pytest.mark.parametrize("held", [0.0, float("inf"), float("nan"), 1e-40, 1e-36])
def test_degenerate_tensor_scales(held):
    x = _t3((32, 64), 5, torch.float32)
    x[3] = 0.0                          # all-zero blocks
    x[4, :16] = 1e-30
    for layout, tr in (("row16", False), ("row16", True), ("col16", False), ("tile", True)):
        for rnd in (0, 1):
            g, o = quant_both(x, held, layout, rnd, transposed=tr)
            assert_quant_equal(g, o, f"held={held} {layout} tr={tr} rnd={rnd}")


def test_empty_quantize_writes_scale():
    x = torch.zeros((0, 32), dtype=torch.bfloat16, device=DEV)
    q, _, diag = api.quantize(x, dev_scalar(6.0), with_diag=True)
    torch.cuda.synchronize()
    assert q.enc_scale.item() == 448.0 and diag.cpu().tolist() == [0, 0]


@pytest.mark.parametrize("layout", ["row16", "tile"])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_dequant_parity(layout, out):
    x = _t3((48, 1056), 6)
    a = float(oracle.amax(host_view(x)))
    g, o = quant_both(x, a * 0.5, layout)
    got = api.dequant(g["q"], out).float().cpu().numpy()
    want = oracle.dequant_f32(o.q)
    if out == torch.bfloat16:
        want = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_sr_same_word_row_and_col_on_gpu():
    x = _grad((64, 128), 9)
    xd = x.to(DEV)
    # the held amax both sides use is the oracle's
    a_held = float(oracle.amax(host_view(x)))
    a = dev_scalar(a_held)
    qr, _, _ = api.quantize(xd, a, rnd=api.SR, seed=123)
    qc, _, _ = api.quantize(xd, a, rnd=api.SR, seed=123, layout=api.COL16)
    # decoding both orientations and comparing sign-and-rounding direction
    # is covered by the oracle parity; here: both match the oracle at once
    o_r = oracle.quantize(host_view(x), a_held, rnd=oracle.SR, seed=123).q
    o_c = oracle.quantize(host_view(x), a_held, rnd=oracle.SR, seed=123, layout=oracle.COL16).q
    np.testing.assert_array_equal(qr.codes.cpu().numpy(), o_r.codes)
    np.testing.assert_array_equal(qc.codes.cpu().numpy(), o_c.codes)


def test_quantize_deterministic():
    x = _grad((256, 4096), 10).to(DEV)
    a = api.amax(x)
    r1 = api.quantize(x, a, rnd=api.SR, seed=9, layout=api.COL16)[0]
    r2 = api.quantize(x, a, rnd=api.SR, seed=9, layout=api.COL16)[0]
    assert torch.equal(r1.codes, r2.codes) and torch.equal(r1.scales, r2.scales)


def test_input_beyond_4gib():
    # A 4.3 GB bf16 input (2^21 + 16 rows of 1024): amax, the ROW16 kernel
    # (RNE and SR) and the one-pass ROW16 + COL16 kernel address past 2^32
    # bytes. The input is drawn on the device with torch's seeded generator
    # (normal, 0.5 scale) and its largest magnitude, 1000, is planted in the
    # last element, so the amax is known. Under the held amax 1000 each
    # 16-row band quantizes independently of the others (the SR word index
    # is placed by the oracle's origin), so bands at the start, the middle
    # and the end are checked against the oracle.
    R, C = (1 << 21) + 16, 1024
    g = torch.Generator(device=DEV).manual_seed(7)
    X = torch.randn((R, C), generator=g, device=DEV, dtype=torch.bfloat16).mul_(0.5)
    X[-1, -1] = 1000.0
    a = api.amax(X)
    assert a.item() == 1000.0
    held = dev_scalar(1000.0)
    q, qt, _ = api.quantize(X, held, transposed=True)
    qr = api.quantize(X, held)[0]
    qs = api.quantize(X, held, rnd=api.SR, seed=3, subseq=1)[0]
    torch.cuda.synchronize()
    for b in (0, (R // 32) * 16, R - 16):
        band = host_view(X[b:b + 16].cpu())
        o_row = oracle.quantize(band, 1000.0, 448.0, oracle.ROW16)
        o_col = oracle.quantize(band, 1000.0, 448.0, oracle.COL16)
        o_sr = oracle.quantize(band, 1000.0, 448.0, oracle.ROW16, oracle.SR, 3, 1, origin=(b, 0, C))
        for got in (q, qr):
            np.testing.assert_array_equal(got.codes[b:b + 16].cpu().numpy(), o_row.q.codes, err_msg=str(b))
            np.testing.assert_array_equal(got.scales[b:b + 16].cpu().numpy(), o_row.q.scales, err_msg=str(b))
        np.testing.assert_array_equal(qt.codes[:, b // 2:b // 2 + 8].cpu().numpy(), o_col.q.codes,
                                      err_msg=str(b))
        np.testing.assert_array_equal(qt.scales[:, b // 16:b // 16 + 1].cpu().numpy(), o_col.q.scales,
                                      err_msg=str(b))
        np.testing.assert_array_equal(qs.codes[b:b + 16].cpu().numpy(), o_sr.q.codes, err_msg=str(b))
        np.testing.assert_array_equal(qs.scales[b:b + 16].cpu().numpy(), o_sr.q.scales, err_msg=str(b))


def _fp32_neighbourhoods(span: int) -> np.ndarray:
    """Every binary32 value within +-span units in the last place of each
    E2M1 level (0, 0.5, 1, 1.5, 2, 3, 4, 6) and of each rounding midpoint
    between levels (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5), both signs."""
    pts = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    d = np.arange(-span, span + 1, dtype=np.int64)
    bits = [np.arange(0, span + 1, dtype=np.int64)]  # 0 and the smallest subnormals
    for p in pts:
        bits.append(int(np.float32(p).view(np.uint32)) + d)
    u = np.unique(np.concatenate(bits)).astype(np.uint32)
    return np.concatenate([u, u | np.uint32(0x80000000)]).view(np.float32)


def _latin_anchor_tensor(vals: np.ndarray, cols: int) -> torch.Tensor:
    """An fp32 tensor whose every 16-element row block and every 16-row column
    block holds exactly one 6.0 (at column 16 j + r % 16 of row r), the other
    positions filled with vals in order (then zeros). With held amax 6 and
    T = 448, S = 448 and every block (row, column or 16 x 16 tile) has bamax
    within 0.6% of 6, so its scale is 448 and r = RN(S / dec) = 1: the payload
    rule sees each value itself."""
    per_row = cols - cols // 16
    rows = -(-len(vals) // per_row)
    rows = -(-rows // 64) * 64
    x = np.zeros((rows, cols), np.float32)
    anchor = np.zeros((rows, cols), bool)
    r = np.arange(rows)[:, None]
    anchor[r, 16 * np.arange(cols // 16)[None, :] + (r % 16)] = True
    body = np.zeros(rows * per_row, np.float32)
    body[:len(vals)] = vals
    x[anchor] = 6.0
    x[~anchor] = body
    return torch.from_numpy(x)


@pytest.mark.parametrize("layout", ["row16", "row16+col16", "tile"])
@pytest.mark.parametrize("rnd", [0, 1])
def test_fp32_payload_neighbourhoods(layout, rnd):
    # fp32 inputs with full 24-bit significands: each E2M1 level and each
    # midpoint between levels +-2^16 ulps (and the subnormals next to zero),
    # through the ROW16 kernel, the one-pass ROW16 + COL16 kernel and the
    # 16 x 16 tile kernel, RNE and SR, bit-exact against the oracle. The
    # hardware RNE conversion and the stochastic-rounding threshold are
    # thereby checked where a wrong tie rule or a lost low bit would show.
    x = _latin_anchor_tensor(_fp32_neighbourhoods(1 << 16), 1024)
    both = layout == "row16+col16"
    g, o = quant_both(x, 6.0, "row16" if both else layout, rnd, 448.0, seed=0xC0FFEE, subseq=9,
                      transposed=(both or layout == "tile"))
    assert g["S"] == np.float32(448.0)
    assert (o.q.scales == 0xBE).all()
    assert_quant_equal(g, o, f"{layout} rnd={rnd}")


@pytest.mark.parametrize("layout", ["row16", "row16+col16", "tile"])
def test_sr_decision_boundaries(layout):
    # every element exactly at the last value that rounds down or the first
    # that rounds up for its own Philox word (tests/sr_threshold.py), in every
    # E2M1 interval, through the ROW16, one-pass ROW16 + COL16 and tile
    # kernels: bit-exact against the oracle. A word conversion or threshold
    # off by one unit anywhere flips codes here.
    from sr_threshold import threshold_tensor
    seed, subseq = 0x1234_5678_9ABC, 11
    x, want = threshold_tensor(128, 512, seed, subseq)
    both = layout == "row16+col16"
    g, o = quant_both(torch.from_numpy(x), 6.0, "row16" if both else layout, 1, 448.0, seed=seed,
                      subseq=subseq, transposed=(both or layout == "tile"))
    if layout != "tile":
        codes = np.zeros(x.shape, np.int64)
        codes[:, 0::2] = o.q.codes & 0xF
        codes[:, 1::2] = o.q.codes >> 4
        np.testing.assert_array_equal(codes & 7, want)
    assert_quant_equal(g, o, layout)
