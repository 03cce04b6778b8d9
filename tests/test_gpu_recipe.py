"""FP4Linear (the autograd module over the C ABI) and its recipe state on the
GPU, against the oracle ("UE5M3 FP4 Block Scaling for Stable Language Model
Pretraining", §5.1-§5.2): forward and both gradients, sample-and-hold
refreshes every D steps, the targeted dY override for wgrad, per-(module,
step) stochastic-rounding streams, and inference's once-measured weight
amax."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from fp4_block_scaled_fp4q_amd import api, inputs
from fp4_block_scaled_fp4q_amd.recipe import Fp4Recipe, FP4Linear
from parity_util import DEV, GEMM_TOL, rel_fro, round_out

pytestmark = pytest.mark.gpu

M, K, N = 256, 512, 384


def make(seed=0):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(inputs.activation(rng, M, K, inputs.outlier_columns(rng, K))).to(torch.bfloat16)
    w = torch.from_numpy(inputs.gaussian(rng, N, K, 0.02))
    dy = torch.from_numpy(inputs.loguniform_grad(rng, M, N)).to(torch.bfloat16)
    return x, w, dy


def oracle_step(x, w, dy, A_x, A_w, A_dy, r: Fp4Recipe, subseq: int):
    """The layer's three products from the oracle's own quantizations."""
    xv, dyv = inputs.bf16_bits(x), inputs.bf16_bits(dy)
    wv = w.numpy()
    kw = dict(block=r.block, scale_fmt=r.scale_fmt)
    xq = oracle.quantize(xv, A_x, r.target, oracle.ROW16, **kw).q
    xqt = oracle.quantize(xv, A_x, r.target, oracle.COL16, **kw).q
    wq = oracle.quantize(wv, A_w, r.target, oracle.TILE16, transposed=True, **kw)
    dyq = oracle.quantize(dyv, A_dy, r.target, oracle.ROW16, oracle.SR, r.seed, subseq, **kw).q
    dyqt = oracle.quantize(dyv, A_dy, r.t_dy_wgrad(), oracle.COL16, oracle.SR, r.seed, subseq, **kw).q
    return oracle.gemm(xq, wq.q), oracle.gemm(dyq, wq.qt), oracle.gemm(dyqt, xqt)


def run(layer, x, dy):
    xd = x.to(DEV).requires_grad_(True)
    y = layer(xd)
    y.backward(dy.to(DEV))
    torch.cuda.synchronize()
    return y.detach(), xd.grad, layer.weight.grad


def close(got, ref, what):
    err = rel_fro(got.float().cpu().numpy(), round_out(ref, got.dtype))
    assert err <= GEMM_TOL, f"{what}: {err:.3e}"


@pytest.mark.parametrize("recipe", [Fp4Recipe(seed=3), Fp4Recipe(seed=3, target_dy_wgrad=2048.0),
                                    Fp4Recipe(seed=5, block=32, scale_fmt=api.E4M3)])
def test_forward_and_gradients_match_oracle(recipe):
    x, w, dy = make()
    layer = FP4Linear(K, N, recipe, device=DEV)
    with torch.no_grad():
        layer.weight.copy_(w.to(DEV))
    y, dx, dw = run(layer, x, dy)
    A = [float(oracle.amax(v)) for v in (inputs.bf16_bits(x), w.numpy(), inputs.bf16_bits(dy))]
    held = layer.held_amax()
    for k, a in zip(("x", "w", "dy"), A):
        assert float(held[k].cpu()[0]) == a, k  # a refresh step samples the current maxima
    ry, rdx, rdw = oracle_step(x, w, dy, *A, recipe, subseq=0)
    close(y, ry, "fwd")
    close(dx, rdx, "dgrad")
    close(dw, rdw, "wgrad")
    assert dw.dtype == torch.float32 and dx.dtype == torch.bfloat16


def test_sample_and_hold_refreshes_every_d_steps():
    D = 3
    x, w, dy = make(1)
    layer = FP4Linear(K, N, Fp4Recipe(refresh_period=D), device=DEV)
    with torch.no_grad():
        layer.weight.copy_(w.to(DEV))
    held_x, held_dy = [], []
    for t in range(5):
        f = float(t + 1)  # every step's tensors grow, so a refresh is visible
        run(layer, (x.float() * f).to(torch.bfloat16), (dy.float() * f).to(torch.bfloat16))
        h = layer.held_amax()
        held_x.append(float(h["x"].cpu()[0]))
        held_dy.append(float(h["dy"].cpu()[0]))
        layer.weight.grad = None
    ax = [float(oracle.amax(inputs.bf16_bits((x.float() * (t + 1)).to(torch.bfloat16)))) for t in range(5)]
    ady = [float(oracle.amax(inputs.bf16_bits((dy.float() * (t + 1)).to(torch.bfloat16)))) for t in range(5)]
    # refreshes at steps 0 and 3; held in between
    assert held_x == [ax[0], ax[0], ax[0], ax[3], ax[3]]
    assert held_dy == [ady[0], ady[0], ady[0], ady[3], ady[3]]
    assert layer.step == 5


def test_held_amax_is_used_between_refreshes():
    # at step 1 (not a refresh) the module quantizes with step 0's maxima
    D = 4
    x, w, dy = make(2)
    r = Fp4Recipe(refresh_period=D, seed=9)
    layer = FP4Linear(K, N, r, device=DEV)
    with torch.no_grad():
        layer.weight.copy_(w.to(DEV))
    run(layer, x, dy)
    layer.weight.grad = None
    x2 = (x.float() * 3.0).to(torch.bfloat16)
    dy2 = (dy.float() * 0.5).to(torch.bfloat16)
    y, dx, dw = run(layer, x2, dy2)
    A0 = [float(oracle.amax(v)) for v in (inputs.bf16_bits(x), w.numpy(), inputs.bf16_bits(dy))]
    ry, rdx, rdw = oracle_step(x2, w, dy2, *A0, r, subseq=1)
    close(y, ry, "fwd")
    close(dx, rdx, "dgrad")
    close(dw, rdw, "wgrad")


def test_stochastic_rounding_streams():
    x, w, dy = make(3)
    outs = {}
    for seed in (1, 2):
        layer = FP4Linear(K, N, Fp4Recipe(seed=seed), device=DEV)
        with torch.no_grad():
            layer.weight.copy_(w.to(DEV))
        y0, _, dw0 = run(layer, x, dy)
        dw0 = dw0.clone()
        layer.weight.grad = None
        _, _, dw1 = run(layer, x, dy)   # next step: another Philox subsequence
        outs[seed] = (y0.clone(), dw0, dw1.clone())
    assert torch.equal(outs[1][0], outs[2][0])          # RNE forward: seed-independent
    assert not torch.equal(outs[1][1], outs[2][1])      # different module seeds
    assert not torch.equal(outs[1][1], outs[1][2])      # different steps
    layer = FP4Linear(K, N, Fp4Recipe(seed=1), device=DEV)
    with torch.no_grad():
        layer.weight.copy_(w.to(DEV))
    _, _, dw = run(layer, x, dy)
    assert torch.equal(dw, outs[1][1])                  # same seed, same step: identical


def test_inference_measures_weight_amax_once():
    x, w, _ = make(4)
    layer = FP4Linear(K, N, Fp4Recipe(refresh_period=2), device=DEV)
    with torch.no_grad():
        layer.weight.copy_(w.to(DEV))
    layer.eval()
    with torch.no_grad():
        layer(x.to(DEV))
        aw0 = float(layer.held_amax()["w"].cpu()[0])
        layer.weight.mul_(4.0)
        for _ in range(3):
            y = layer(x.to(DEV))
        torch.cuda.synchronize()
    assert float(layer.held_amax()["w"].cpu()[0]) == aw0
    # the held weight amax is the first weight's; the output uses it (the
    # scaled weight under the old S)
    aw_oracle = float(oracle.amax(w.numpy()))
    assert aw0 == aw_oracle
    w4 = (w * 4.0).numpy()
    xq = oracle.quantize(inputs.bf16_bits(x), float(oracle.amax(inputs.bf16_bits(x)))).q
    wq = oracle.quantize(w4, aw_oracle, layout=oracle.TILE16).q
    close(y, oracle.gemm(xq, wq), "inference fwd")


@pytest.mark.parametrize("m,k,n", [(96, 80, 48), (128, 192, 320)])
def test_packing_follows_the_shapes(m, k, n):
    # K64 wherever every contraction length (K, N, M) is a multiple of 64,
    # row-major otherwise; the results match the oracle either way
    rng = np.random.default_rng(m + k + n)
    x = torch.from_numpy(inputs.activation(rng, m, k, inputs.outlier_columns(rng, k))).to(torch.bfloat16)
    w = torch.from_numpy(inputs.gaussian(rng, n, k, 0.02))
    dy = torch.from_numpy(inputs.loguniform_grad(rng, m, n)).to(torch.bfloat16)
    r = Fp4Recipe(seed=4)
    layer = FP4Linear(k, n, r, device=DEV)
    with torch.no_grad():
        layer.weight.copy_(w.to(DEV))
    y, dx, dw = run(layer, x, dy)
    A = [float(oracle.amax(v)) for v in (inputs.bf16_bits(x), w.numpy(), inputs.bf16_bits(dy))]
    ry, rdx, rdw = oracle_step(x, w, dy, *A, r, subseq=0)
    close(y, ry, "fwd")
    close(dx, rdx, "dgrad")
    close(dw, rdw, "wgrad")


def test_fp32_activations_and_gradients_quantized_directly():
    # fp32 X gives an fp32 output, so autograd hands the backward an fp32
    # dY, which reaches the quantizer as it is: all three outputs (fp32)
    # lie within the elementwise fp32-accumulation bound of the oracle's
    # contraction of its own quantizations of the fp32 tensors (a bf16
    # rounding of dY before its stochastic rounding moves codes by far more
    # than that bound)
    from parity_util import check_gemm_elementwise, gemm_ref_and_bound
    rng = np.random.default_rng(11)
    x = torch.from_numpy(inputs.activation(rng, M, K, inputs.outlier_columns(rng, K)))
    w = torch.from_numpy(inputs.gaussian(rng, N, K, 0.02))
    dy = torch.from_numpy(inputs.loguniform_grad(rng, M, N))
    r = Fp4Recipe(seed=9)
    layer = FP4Linear(K, N, r, device=DEV)
    with torch.no_grad():
        layer.weight.copy_(w.to(DEV))
    y, dx, dw = run(layer, x, dy)
    assert y.dtype == torch.float32 and dx.dtype == torch.float32 and dw.dtype == torch.float32
    A = [float(oracle.amax(v.numpy())) for v in (x, w, dy)]
    xq = oracle.quantize(x.numpy(), A[0], r.target, oracle.ROW16).q
    xqt = oracle.quantize(x.numpy(), A[0], r.target, oracle.COL16).q
    wq = oracle.quantize(w.numpy(), A[1], r.target, oracle.TILE16, transposed=True)
    dyq = oracle.quantize(dy.numpy(), A[2], r.target, oracle.ROW16, oracle.SR, r.seed, 0).q
    dyqt = oracle.quantize(dy.numpy(), A[2], r.target, oracle.COL16, oracle.SR, r.seed, 0).q
    ref, bound = gemm_ref_and_bound(xq, wq.q, torch.float32)
    check_gemm_elementwise(y, ref, bound, "fwd")
    ref, bound = gemm_ref_and_bound(dyq, wq.qt, torch.float32)
    check_gemm_elementwise(dx, ref, bound, "dgrad")
    ref, bound = gemm_ref_and_bound(dyqt, xqt, torch.float32)
    check_gemm_elementwise(dw, ref, bound, "wgrad")
