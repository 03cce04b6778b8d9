"""Recipe state around the emulated FP4 linear layer, and a torch autograd
module over the C ABI ("UE5M3 FP4 Block Scaling for Stable Language Model
Pretraining", §5.1-§5.2 and the quantized-inference appendix).

* Sample-and-hold tensor maxima (§5.1): every operand (activation, weight,
  upstream gradient) of every module keeps its own held amax on the device.
  It is re-sampled from the current tensor on refresh steps only, every D
  optimizer steps (D = 50 in the page's recipe), and reused in between.
* A tunable UE5M3 target T per operand (§5.2), with the page's targeted
  override: T = 2048 for dY in the weight-gradient GEMM of chosen modules.
* Stochastic rounding for dY only; one Philox stream per (module, step):
  key = the module's seed, subsequence = the step counter, so no two steps
  or modules share random words.
* Inference: a weight's amax is measured once and then held; activations
  use a delayed cache started from the first batch (refreshed on the same
  period, counted over inference calls).
* Operands are stored in the K64 packing (contiguous 64-element k tiles,
  which the GEMM reads in one run per tile) whenever every contraction
  length involved is a multiple of 64, else row-major; the packing changes
  no value.

Everything on the data path runs in libfp4q.so (fp4q_amax, fp4q_quantize*,
fp4q_linear_*); this module only keeps state and calls it. Nothing here
synchronizes the device.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import api


@dataclass
class Fp4Recipe:
    """Configuration of the FP4 recipe for one module."""
    refresh_period: int = 50          # D: optimizer steps between tensor-maximum refreshes
    target: float = 448.0             # T for X, W and dY (dgrad)
    target_dy_wgrad: float | None = None  # the targeted override for dY in wgrad (e.g. 2048)
    block: int = 16                   # 16, or 32 (the block-32 variant)
    scale_fmt: int = api.UE5M3        # UE5M3, or E4M3 (NVFP4's scale format)
    seed: int = 0                     # Philox key of this module's dY stochastic rounding
    pack: int = api.PACK_K64          # memory packing (row-major where a length is not % 64)

    def t_dy_wgrad(self) -> float:
        return self.target if self.target_dy_wgrad is None else float(self.target_dy_wgrad)


def is_refresh(step: int, period: int) -> bool:
    """Refresh steps of the sample-and-hold schedule: 0, D, 2D, ..."""
    if period < 1:
        raise ValueError("refresh period must be >= 1")
    return step % period == 0


class HeldAmax:
    """One operand's held tensor maximum (a device float32 scalar)."""

    def __init__(self, device: torch.device | str):
        self.value = torch.zeros(1, dtype=torch.float32, device=device)
        self.sampled = False

    def update(self, x: torch.Tensor, refresh: bool) -> torch.Tensor:
        """On a refresh step (or before the first sample) re-sample the held
        value from x; return the held value either way."""
        if refresh or not self.sampled:
            api.fp4q_amax(x, self.value)
            self.sampled = True
        return self.value


@dataclass
class _State:
    amax_x: HeldAmax
    amax_w: HeldAmax
    amax_dy: HeldAmax
    step: int = 0          # training forward calls so far
    eval_calls: int = 0    # inference forward calls so far
    weight_measured: bool = False


class _Fp4LinearFn(torch.autograd.Function):
    """y = x W^T with every GEMM operand FP4-quantized; gradients by the
    dgrad and wgrad GEMMs of the same layer."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, weight: torch.Tensor, module: "FP4Linear", need_grad: bool):
        r = module.recipe
        st = module.state
        training = module.training
        # inference keeps its own delayed schedule, started from the first batch
        refresh = is_refresh(st.step if training else st.eval_calls, r.refresh_period)
        x2 = x.reshape(-1, x.shape[-1])
        if not x2.is_contiguous():
            x2 = x2.contiguous()
        M, K, N = x2.shape[0], x2.shape[1], weight.shape[0]
        # every contraction the packing must serve: K (fwd), and with a
        # backward N (dgrad) and M (wgrad)
        lengths = (K, N, M) if need_grad else (K,)
        pack = api.PACK_K64 if r.pack == api.PACK_K64 and all(n % 64 == 0 for n in lengths) else api.PACK_ROWS
        kw = dict(block=r.block, scale_fmt=r.scale_fmt, pack=pack)
        # each operand's amax is followed by its own quantization, which then
        # re-reads a tensor the amax has just streamed through the cache
        ax = st.amax_x.update(x2, refresh)
        # X: ROW (fwd) and, when a backward follows, COL (wgrad) in one pass
        xq, xqt, _ = api.quantize(x2, ax, r.target, api.ROW16, api.RNE, transposed=need_grad, **kw)
        if training or not st.weight_measured:
            aw = st.amax_w.update(weight, refresh)
            st.weight_measured = True
        else:
            aw = st.amax_w.value  # inference: the weight's amax is measured once
        wq, wqt, _ = api.quantize(weight, aw, r.target, api.TILE16x16, api.RNE, transposed=need_grad,
                                  **kw)
        # the output (and, in backward, dX) in the activation's dtype: fp32
        # activations get fp32 outputs, so their upstream gradients arrive in
        # fp32 and are quantized without a bf16 rounding first
        out_dtype = torch.float32 if x.dtype == torch.float32 else torch.bfloat16
        y = torch.empty((x2.shape[0], weight.shape[0]), dtype=out_dtype, device=x.device)
        api.fp4q_linear_fwd(xq, wq, y)
        if need_grad:
            ctx.module = module
            ctx.step = st.step
            ctx.refresh = refresh
            ctx.x_shape = x.shape
            ctx.x_dtype = x.dtype
            ctx.w_dtype = weight.dtype
            ctx.xqt, ctx.wqt = xqt, wqt
            ctx.pack = pack
        if training:
            st.step += 1
        else:
            st.eval_calls += 1
        return y.reshape(*x.shape[:-1], weight.shape[0])

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        module = ctx.module
        r = module.recipe
        st = module.state
        dy2 = dy.reshape(-1, dy.shape[-1])
        # bf16 and fp32 gradients are quantized as they come (no extra
        # rounding step); other dtypes widen exactly to fp32 first
        if dy2.dtype not in (torch.bfloat16, torch.float32):
            dy2 = dy2.to(torch.float32)
        if not dy2.is_contiguous():
            dy2 = dy2.contiguous()
        ady = st.amax_dy.update(dy2, ctx.refresh)
        kw = dict(block=r.block, scale_fmt=r.scale_fmt, pack=ctx.pack)
        seed, subseq = r.seed, ctx.step & 0xFFFFFFFF
        t_wg = r.t_dy_wgrad()
        if t_wg == r.target:
            # one pass: ROW (dgrad) and COL (wgrad), one Philox word per element
            dyq, dyqt, _ = api.quantize(dy2, ady, r.target, api.ROW16, api.SR, seed, subseq,
                                        transposed=True, **kw)
        else:
            # the targeted override: the wgrad operand under its own target
            # (same seed and subsequence, so the same random word per element)
            dyq, _, _ = api.quantize(dy2, ady, r.target, api.ROW16, api.SR, seed, subseq, **kw)
            dyqt, _, _ = api.quantize(dy2, ady, t_wg, api.COL16, api.SR, seed, subseq, **kw)
        M, N = dy2.shape
        K = ctx.wqt.rows
        dx = torch.empty((M, K), dtype=torch.float32 if ctx.x_dtype == torch.float32 else torch.bfloat16,
                         device=dy.device)
        dw = torch.empty((N, K), dtype=torch.float32, device=dy.device)
        api.fp4q_linear_dgrad(dyq, ctx.wqt, dx)
        api.fp4q_linear_wgrad(dyqt, ctx.xqt, dw)
        ctx.xqt = ctx.wqt = None
        return dx.reshape(ctx.x_shape).to(ctx.x_dtype), dw.to(ctx.w_dtype), None, None


class FP4Linear(torch.nn.Module):
    """A bias-free linear layer y = x W^T whose three GEMMs (fwd, dgrad,
    wgrad) run on FP4-quantized operands (E2M1 payloads, block scales, held
    FP32 tensor scales) through libfp4q.so.

    weight: [out_features, in_features], float32 or bfloat16 (quantized from
    that dtype; its gradient comes back in it). Inputs are bfloat16 or float32
    (the output and the input's gradient come in the same dtype: bf16 for
    bf16 inputs, fp32 for fp32 inputs, whose upstream gradients are then
    quantized in fp32)
    with in_features a multiple of the block size and of 16; the token count
    must be a multiple of the block size in training (the wgrad operands are
    blocked along tokens).
    """

    def __init__(self, in_features: int, out_features: int, recipe: Fp4Recipe | None = None,
                 device: torch.device | str = "cuda", dtype: torch.dtype = torch.float32):
        super().__init__()
        self.in_features = in_features
        self.out_features = out_features
        self.recipe = recipe or Fp4Recipe()
        self.weight = torch.nn.Parameter(torch.empty((out_features, in_features), device=device,
                                                     dtype=dtype))
        torch.nn.init.normal_(self.weight, std=0.02)
        self.state = _State(HeldAmax(device), HeldAmax(device), HeldAmax(device))

    @property
    def step(self) -> int:
        return self.state.step

    def held_amax(self) -> dict:
        """The held tensor maxima (device scalars) of X, W and dY."""
        return {"x": self.state.amax_x.value, "w": self.state.amax_w.value,
                "dy": self.state.amax_dy.value}

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        # a backward follows only in training with autograd on (the COL
        # quantizations for wgrad are produced only then)
        need_grad = self.training and torch.is_grad_enabled() and (x.requires_grad or self.weight.requires_grad)
        return _Fp4LinearFn.apply(x, self.weight, self, need_grad)

    def extra_repr(self) -> str:
        r = self.recipe
        return (f"in_features={self.in_features}, out_features={self.out_features}, D={r.refresh_period}, "
                f"T={r.target}, T_dy_wgrad={r.t_dy_wgrad()}, block={r.block}, scale_fmt={r.scale_fmt}, "
                f"pack={r.pack}")
