"""K1 with two 16-row tiles per workgroup on ragged row counts.

Once there are more 16-row tiles than compute units, a row holds at least 16
groups of 64 channels and the rank is at most 64, K1 gives each workgroup 32
rows (two groups in flight per wave, three on rows of at least 96 groups);
with M not a multiple of 32 the last workgroup's second tile, or part of its
first, lies past M. The cases cover both ring depths, and rank 96 (16-row
workgroups of four waves) with fp32 X on a ragged M. On such row counts the INT4 codes and scales, and
the MXFP4 tiled codes and exponents, must be bit-exact against the oracle's
quantizer on every row, D must stay within the down-projection's bound, and
the INT4 output rows past M must stay untouched (canary bytes).
"""
from __future__ import annotations

import numpy as np
import pytest

import int4_tiles
import oracle as O
from gpu_common import dev, host_u16, oracle_prep, rel_err, torch_mod
from test_gpu_mx import MxDevice, _oracle_w, read_act

pytestmark = pytest.mark.gpu

CASES = [(4100, 1024, 32, "f16"), (4113, 1024, 96, "f32"), (4127, 6144, 16, "f16")]


def _inputs(M, K, xdt, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, 3, replace=False)] *= 20
    X = X.astype(np.float16 if xdt == "f16" else np.float32)
    W = (rng.standard_normal((K, 128)) * 0.02).astype(np.float32)
    return X, W


def _check_d(Dg, xh, L1, K, f16_out=False):
    """fp32 accumulation bound; with f16_out, plus D's one fp16 rounding (half an
    fp16 ulp: 2^-11 relative, 2^-25 absolute below the normal range)."""
    Do = O.down_projection(xh, L1)
    env = np.abs(O.to_f16(xh).astype(np.float64)) @ np.abs(np.asarray(L1, np.float64))
    tol = K * 2.0 ** -23 * env + 2.0 ** -24 * np.abs(Do) + 1e-30
    if f16_out:
        tol = tol + 2.0 ** -11 * np.abs(Do) + 2.0 ** -25
    assert np.all(np.abs(Dg - Do) <= tol)
    assert rel_err(Dg, Do) <= 1e-3


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}_r{c[2]}_{c[3]}")
def test_int4_two_row_tiles_ragged(case):
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K, R, xdt = case
    X, W = _inputs(M, K, xdt, seed=M + K + R)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, R)
    _, inv_o, _, _ = oracle_prep(X, W, p, R)
    pad = 40
    codes = torch.full((M + pad, K // 2), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((M + pad, K // 64), 0x5A5A, dtype=torch.int16, device="cuda")
    D = torch.full((M + pad, R), -3.0, dtype=torch.float32, device="cuda")
    sq.quantize_act_lowrank_down(dev(X), dev(p.inv_smooth), dev(p.L1p), R, codes[:M], scales[:M],
                                 D[:M])
    torch.cuda.synchronize()
    a_codes, a_scales, xh = O.quantize_activation(X, inv_o)
    got_c = codes.cpu().numpy()
    got_s = host_u16(scales)
    assert np.array_equal(got_c[:M], a_codes)
    assert np.array_equal(got_s[:M], a_scales.view(np.uint16))
    assert np.all(got_c[M:] == 0x5A) and np.all(got_s[M:] == 0x5A5A)
    Dg = D.cpu().numpy()
    assert np.all(Dg[M:] == -3.0)
    _check_d(Dg[:M].astype(np.float64), xh, p.L1, K)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}_r{c[2]}_{c[3]}")
def test_mx_two_row_tiles_ragged(case):
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K, R, xdt = case
    X, W = _inputs(M, K, xdt, seed=M + K + R + 1)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights_mx(W, lam, R)
    inv, _, _ = _oracle_w(X, W, p, R)
    d = MxDevice(X, p, None)
    d.k1()
    torch.cuda.synchronize()
    a_codes, a_e8, xh = O.mx_quantize_activation(X, inv)
    got_c, got_e = read_act(d)
    assert np.array_equal(got_c, a_codes)
    assert np.array_equal(got_e, a_e8)
    Dg = int4_tiles.untile_d(d.D.cpu().numpy(), M, R).astype(np.float64)
    _check_d(Dg, xh, p.L1, K, f16_out=True)


# Long rows (at least 96 groups) with more 16-row tiles than compute units:
# with the optional workspace the tiled and MXFP4 pre-kernels split each
# 32-row tile's groups over several workgroups and sum the partial D tiles in
# a second pass; without it they run unsplit. Both must give the oracle's
# codes and scales bit for bit, and D within the down-projection's bound plus
# its one fp16 rounding, on ragged row counts.
SPLIT = [(4100, 6144, 16, "f16"), (4113, 6144, 32, "f32")]


@pytest.mark.parametrize("split", [True, False], ids=["split", "unsplit"])
@pytest.mark.parametrize("case", SPLIT, ids=lambda c: f"{c[0]}x{c[1]}_r{c[2]}_{c[3]}")
def test_tiled_long_rows_split_and_unsplit(case, split):
    import bit_post_quantized_smooth_amd as sq
    from test_gpu_tiled import TiledLayer, _check_k1_tiled
    torch = torch_mod()
    M, K, R, xdt = case
    X, W = _inputs(M, K, xdt, seed=M + K + R + 2)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, R)
    _, inv_o, _, _ = oracle_prep(X, W, p, R)
    assert sq.quantize_act_workspace_bytes(M, K, R) > 0      # the shape splits on MI355X
    d = TiledLayer(X, p, None, "f16", k1_workspace=split)
    d.k1()
    torch.cuda.synchronize()
    _check_k1_tiled(X, inv_o, p, K, d)


@pytest.mark.parametrize("split", [True, False], ids=["split", "unsplit"])
@pytest.mark.parametrize("case", SPLIT, ids=lambda c: f"{c[0]}x{c[1]}_r{c[2]}_{c[3]}")
def test_mx_long_rows_split_and_unsplit(case, split):
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K, R, xdt = case
    X, W = _inputs(M, K, xdt, seed=M + K + R + 3)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights_mx(W, lam, R)
    inv, _, _ = _oracle_w(X, W, p, R)
    d = MxDevice(X, p, None, k1_workspace=split)
    d.k1()
    torch.cuda.synchronize()
    a_codes, a_e8, xh = O.mx_quantize_activation(X, inv)
    got_c, got_e = read_act(d)
    assert np.array_equal(got_c, a_codes)
    assert np.array_equal(got_e, a_e8)
    Dg = int4_tiles.untile_d(d.D.cpu().numpy(), M, R).astype(np.float64)
    _check_d(Dg, xh, p.L1, K, f16_out=True)

