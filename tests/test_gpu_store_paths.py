"""The two ways a GEMM epilogue stores an fp16 Y agree bit for bit.

A wave quarter that lies inside Y, with Y's rows 16-byte aligned, goes out
through LDS in whole cache lines; any other quarter, and every quarter of a Y
whose rows are not 16-byte aligned, is stored straight from the matrix-core
layout. Each format's layer is run into a contiguous Y (aligned rows: the
staged store wherever a quarter fits, the direct one at the ragged edges) and
into a view whose row stride is N + 3 halves (never aligned: the direct store
everywhere). Both results must be equal, and the view's padding columns and
the rows around it untouched.
"""
from __future__ import annotations

import numpy as np
import pytest

from gpu_common import dev, torch_mod

pytestmark = pytest.mark.gpu

M, K, N, R = 300, 256, 200, 32      # full quarters for every format's tile, ragged edges too


def _inputs(seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, 3, replace=False)] *= 20
    X = X.astype(np.float16)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    return X, W, b


def _two_ways(run):
    torch = torch_mod()
    Ya = torch.empty((M, N), dtype=torch.float16, device="cuda")
    run(Ya)
    Ybig = torch.full((M + 2, N + 3), -7.0, dtype=torch.float16, device="cuda")
    Yv = Ybig[1:M + 1, :N]
    assert (Yv.stride(0) * 2) % 16 != 0
    run(Yv)
    torch.cuda.synchronize()
    a = Ya.cpu().numpy()
    big = Ybig.cpu().numpy()
    assert np.all(np.isfinite(a))
    assert np.array_equal(big[1:M + 1, :N].view(np.uint16), a.view(np.uint16))
    assert np.all(big[0] == -7.0) and np.all(big[M + 1] == -7.0) and np.all(big[:, N:] == -7.0)


@pytest.mark.parametrize("fmt,act", [("int4", None), ("int4", "gelu_tanh"),
                                     ("mxfp4", None), ("mxfp4", "gelu_tanh"), ("w4a16", None)])
def test_staged_and_direct_stores_agree(fmt, act):
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    X, W, b = _inputs(seed=len(fmt) * 7 + (act is not None))
    Xd, bd = dev(X), dev(b)
    if fmt == "w4a16":
        p = sq.prepare_weights_w4a16(W)
        ct, st = sq.pack_w4a16_tiles(p.w_codes, p.w_scales, K)
        wc, ws = dev(ct), dev(st)
        buf = torch.empty(sq.w4a16_x_tiled_bytes(M, K), dtype=torch.uint8, device="cuda")
        _two_ways(lambda Y: sq.linear_w4a16(Xd, wc, ws, bd, Y, buf))
        return
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    if fmt == "int4":
        p = sq.prepare_weights(W, lam, R)
        wc, ws = dev(p.w_codes), dev(p.w_scales)
        buf = torch.empty(sq.linear_workspace_bytes(M, K, R), dtype=torch.uint8, device="cuda")
        layer = sq.linear
    else:
        p = sq.prepare_weights_mx(W, lam, R)
        ct, et = sq.pack_mx_tiles(p.w_codes, p.w_scales, K)
        wc, ws = dev(ct), dev(et)
        buf = torch.empty(sq.linear_mx_workspace_bytes(M, K, R), dtype=torch.uint8,
                          device="cuda")
        layer = sq.linear_mx
    inv, L1p, L2t = dev(p.inv_smooth), dev(p.L1p), dev(p.L2t)
    _two_ways(lambda Y: layer(Xd, inv, L1p, L2t, R, wc, ws, bd, Y, buf, activation=act))
