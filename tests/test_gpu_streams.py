"""Every launch of a C ABI call goes to the stream the call is given.

The whole path of one linear layer (three amaxes, the RNE and SR
quantizations with their second orientations, fwd, dgrad and a wgrad whose
fp32 tiles run as split K halves behind a zeroing launch) is enqueued once on
torch's default stream and once on a side stream of default priority; the
two runs agree bit for bit. A launch that went to another stream than the
one passed would race with its neighbours in the side-stream run."""
import numpy as np
import pytest
import torch

from fp4_block_scaled_fp4q_amd import api, inputs
from parity_util import DEV

pytestmark = pytest.mark.gpu


def _layer(X, W, dY, pack):
    M, K = X.shape
    N = W.shape[0]
    ax, aw, ady = api.amax(X), api.amax(W), api.amax(dY)
    qx, qxt, _ = api.quantize(X, ax, transposed=True, pack=pack)
    qw, qwt, _ = api.quantize(W, aw, layout=api.TILE16x16, transposed=True, pack=pack)
    qdy, qdyt, _ = api.quantize(dY, ady, rnd=api.SR, seed=7, subseq=3, transposed=True, pack=pack)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    dx = torch.full((M, K), float("nan"), dtype=torch.bfloat16, device=DEV)
    dw = torch.full((N, K), float("nan"), dtype=torch.float32, device=DEV)
    api.fp4q_linear_fwd(qx, qw, y)
    api.fp4q_linear_dgrad(qdy, qwt, dx)
    api.fp4q_linear_wgrad(qdyt, qxt, dw)
    out = {"ax": ax, "aw": aw, "ady": ady, "y": y, "dx": dx, "dw": dw}
    for name, q in (("x", qx), ("xt", qxt), ("w", qw), ("wt", qwt), ("dy", qdy), ("dyt", qdyt)):
        out[name + ".codes"], out[name + ".scales"], out[name + ".S"] = q.codes, q.scales, q.enc_scale
    return out


@pytest.mark.parametrize("pack", [api.PACK_ROWS, api.PACK_K64])
def test_side_stream_matches_default_stream(pack):
    # wgrad: dW [1024, 1024] is 16 fp32 tiles, a multiple of 8 that leaves
    # the last round of workgroups at most half full, so all of them run as
    # split K halves behind the zeroing launch
    M, N, K = 512, 1024, 1024
    rng = np.random.default_rng(5)
    X = inputs.to_bf16(inputs.activation(rng, M, K, inputs.outlier_columns(rng, K))).to(DEV)
    W = inputs.to_bf16(inputs.gaussian(rng, N, K, 0.02)).to(DEV)
    dY = inputs.to_bf16(inputs.loguniform_grad(rng, M, N)).to(DEV)
    ref = _layer(X, W, dY, pack)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = _layer(X, W, dY, pack)
    side.synchronize()
    for name, t in ref.items():
        assert torch.equal(got[name].view(torch.uint8), t.view(torch.uint8)), name
