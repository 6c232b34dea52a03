"""GPU parity of the convolution path (K1 on the implicit patch matrix of an
NHWC image, then K2) against the oracle's linear layer on its im2col.

Bit-exact: activation codes and scales against the oracle's quantizer on the
patch matrix, and codes, scales, D and Y against the linear entry points run
on the same patch matrix materialised in device memory (the two must agree to
the bit: the same values reach the same arithmetic). Within 2e-3 * max|Y| and
the strict element-wise bound: Y against the oracle, on every element for the
small cases and on sampled output pixels at the UNet sizes. The tiled INT4
convolution (K1 writing the operand tiles, then K2T) is held to the same bar
against the tiled linear path and the oracle, and the MXFP4 convolution (K1-MX
on the patches, K2-MX) against the oracle's MXFP4 functions."""
import numpy as np
import pytest

import oracle as O
import int4_tiles
import workloads as wl
from gpu_common import (TOL_Y, assert_y_strict, d_stat_bound, dev, host_u16, oracle_rows,
                        oracle_rows_exact, rel_err, sample_rows, torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_post_quantized_smooth_amd  # noqa: F401  (raises if the library is missing)


class _Prep:
    """The oracle's smoothing and residual codes for the library's fp16 factors."""

    def __init__(self, Xcol, Wm, p):
        lam = O.smoothing_factors(O.channel_absmax(Xcol), Wm)
        self.inv = O.inv_smoothing(lam)
        self.wc, self.ws = O.quantize_residual_from_factors(Wm, lam, p.L1, p.L2)


def _setup(L: wl.ConvLayer, X, Wc, bias):
    """Library prep from the implicit patch matrix's statistics; oracle prep from im2col."""
    import bit_post_quantized_smooth_amd as sq
    Wm = O.conv_weight_matrix(Wc)
    lam = sq.smoothing_factors(sq.conv_patch_absmax(X, L.KH, L.KW, L.stride, L.pad), Wm)
    p = sq.prepare_weights(Wm, lam, L.rank)
    Xcol = O.im2col_nhwc(X, L.KH, L.KW, L.stride, L.pad)
    o = _Prep(Xcol, Wm, p)
    assert np.array_equal(o.inv, p.inv_smooth)
    assert np.array_equal(o.wc, p.w_codes) and np.array_equal(o.ws.view(np.uint16), p.w_scales)
    return p, Xcol, o


def _run(L: wl.ConvLayer, X, p, bias):
    """K1-conv alone, and the whole convolution; returns device tensors."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K, R = L.M, L.K, p.rank
    Xd = dev(X)
    inv, L1p = dev(p.inv_smooth), (dev(p.L1p) if R else None)
    a_codes = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    a_scales = torch.empty((M, K // 64), dtype=torch.int16, device="cuda")
    D = torch.empty((M, max(R, 1)), dtype=torch.float32, device="cuda")
    sq.quantize_act_lowrank_down_conv(Xd, L.KH, L.KW, L.stride, L.pad, inv, L1p, R, a_codes,
                                      a_scales, D if R else None)
    conv = sq.Conv2d(p, L.KH, L.KW, L.stride, L.pad, bias,
                     out_dtype=torch.float16 if L.y_dtype == "f16" else torch.float32)
    Y = conv(Xd)
    torch.cuda.synchronize()
    assert Y.shape == (L.batch, L.OH, L.OW, p.N)
    return a_codes, a_scales, D, Y


def _linear_on_patches(Xcol, p, bias, y_dtype):
    """The linear entry points on the materialised patch matrix."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K = Xcol.shape
    R = p.rank
    Xd = dev(Xcol)
    inv, L1p = dev(p.inv_smooth), (dev(p.L1p) if R else None)
    a_codes = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    a_scales = torch.empty((M, K // 64), dtype=torch.int16, device="cuda")
    D = torch.empty((M, max(R, 1)), dtype=torch.float32, device="cuda")
    sq.quantize_act_lowrank_down(Xd, inv, L1p, R, a_codes, a_scales, D if R else None)
    lin = sq.Linear(p, bias, out_dtype=torch.float16 if y_dtype == "f16" else torch.float32)
    Y = lin(Xd)
    torch.cuda.synchronize()
    return a_codes, a_scales, D, Y


def _check_against_linear(L, Xcol, p, bias, got):
    a_codes, a_scales, D, Y = got
    lc, ls, lD, lY = _linear_on_patches(Xcol, p, bias, L.y_dtype)
    assert torch_mod().equal(a_codes, lc)
    assert torch_mod().equal(a_scales, ls)
    if p.rank:
        assert torch_mod().equal(D[:, :p.rank], lD[:, :p.rank])
    assert torch_mod().equal(Y.reshape(L.M, p.N).view(torch_mod().uint8), lY.view(torch_mod().uint8))


# small convolutions, every element: stride 1-3, padding 0-2, a 1x1 kernel, a
# kernel wider than the image, output pixels whose patch lies wholly in the
# padding, ragged row tiles, ranks 0-48, both dtypes
EDGE = [
    # batch, H, W, C, N, KH, KW, stride, pad, rank, x, y
    wl.ConvLayer(1, 8, 8, 64, 64, 3, 3, 1, 1, 16, "f32", "f32", "tiny"),
    wl.ConvLayer(1, 5, 7, 64, 48, 3, 3, 2, 1, 16, "f16", "f16", "s2 ragged"),
    wl.ConvLayer(2, 6, 6, 128, 96, 1, 1, 1, 0, 0, "f16", "f32", "1x1 rank0"),
    wl.ConvLayer(1, 9, 5, 64, 40, 3, 3, 1, 0, 32, "f16", "f16", "no pad"),
    wl.ConvLayer(1, 4, 4, 64, 33, 5, 5, 1, 2, 16, "f32", "f16", "5x5 on 4x4"),
    wl.ConvLayer(3, 9, 7, 192, 70, 3, 2, 3, 1, 48, "f16", "f16", "s3 3x2"),
    wl.ConvLayer(1, 2, 2, 64, 16, 1, 1, 1, 2, 16, "f32", "f32", "pad only rows"),
    # 4225 patch rows: more 16-row tiles than CUs, so K1 takes 32 rows per
    # workgroup, and the last workgroup holds a single row
    wl.ConvLayer(1, 65, 65, 64, 32, 3, 3, 1, 1, 32, "f16", "f16", "two row tiles"),
]


def _edge_inputs(L: wl.ConvLayer, seed: int):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((L.batch, L.H, L.W, L.C))
    X[..., rng.choice(L.C, max(1, L.C // 50), replace=False)] *= 20
    X = X.astype(np.float16 if L.x_dtype == "f16" else np.float32)
    Wc = (rng.standard_normal((L.KH, L.KW, L.C, L.N)) * 0.02).astype(np.float32)
    b = (rng.standard_normal(L.N) * 0.1).astype(np.float32)
    return X, Wc, b


@pytest.mark.parametrize("L", EDGE, ids=lambda L: L.name.replace(" ", "_"))
def test_conv_edge_every_element(L):
    X, Wc, b = _edge_inputs(L, seed=L.H * 131 + L.W * 7 + L.C + L.KH + L.stride)
    p, Xcol, o = _setup(L, X, Wc, b)
    got = _run(L, X, p, b)
    a_codes, a_scales, D, Y = got
    oc, osc, xh = O.quantize_activation(Xcol, o.inv)
    assert np.array_equal(a_codes.cpu().numpy(), oc)
    assert np.array_equal(host_u16(a_scales), osc.view(np.uint16))
    if p.rank:
        Dg = D.cpu().numpy()[:, :p.rank].astype(np.float64)
        Do = O.down_projection(xh, p.L1)
        assert float(np.max(np.abs(Dg - Do) / (d_stat_bound(xh, p.L1, L.K) + 1e-30))) <= 1.0
    Yg = Y.cpu().numpy().reshape(L.M, L.N)
    Yo = O.linear(Xcol, o.inv, p.L1, p.L2, o.wc, o.ws, b, L.y_dtype)
    assert rel_err(Yg, Yo) <= TOL_Y
    Ye, env, jump = oracle_rows_exact(Xcol, o.inv, p, o.wc, o.ws, b, np.arange(L.M))
    assert_y_strict(Yg, Ye, env, jump, L.y_dtype, L.K // 64, p.rank)
    _check_against_linear(L, Xcol, p, b, got)
    if L.name == "pad only rows":
        # 1x1 kernel, pad 2: output pixels off the image see only zeros
        img = np.zeros((L.OH, L.OW), dtype=bool)
        img[2:2 + L.H, 2:2 + L.W] = True
        off = ~img.reshape(-1)
        assert np.all(host_u16(a_scales)[off] == 0) and np.all(a_codes.cpu().numpy()[off] == 0)
        assert np.array_equal(Yg[off], np.broadcast_to(b, (int(off.sum()), L.N)))


@pytest.mark.parametrize("idx", range(1, len(wl.CONV_LAYERS)),
                         ids=lambda i: wl.CONV_LAYERS[i].name.replace(" ", "_"))
def test_conv_unet_sizes(idx):
    """UNet layers at full size: whole tensors against the linear path on the
    materialised patch matrix, sampled output pixels against the oracle."""
    L, X, Wc = wl.conv_inputs(idx)
    b = wl.bias(wl.CONV_CFG, idx, L.N)
    p, Xcol, o = _setup(L, X, Wc, b)
    got = _run(L, X, p, b)
    a_codes, a_scales, D, Y = got
    rows = sample_rows(L.M, seed=idx)
    # include output pixels on the image border (padding taps) of both images
    border = [0, L.OW - 1, (L.OH - 1) * L.OW, L.OH * L.OW - 1, L.OH * L.OW, L.M - 1]
    rows = np.unique(np.concatenate([rows, border]))
    oc, osc, xh = O.quantize_activation(Xcol[rows], o.inv)
    assert np.array_equal(a_codes.cpu().numpy()[rows], oc)
    assert np.array_equal(host_u16(a_scales)[rows], osc.view(np.uint16))
    Dg = D.cpu().numpy()[rows, :p.rank].astype(np.float64)
    Do = O.down_projection(xh, p.L1)
    assert float(np.max(np.abs(Dg - Do) / (d_stat_bound(xh, p.L1, L.K) + 1e-30))) <= 1.0
    Yg = Y.cpu().numpy().reshape(L.M, L.N)
    Yo = oracle_rows(Xcol, o.inv, p, o.wc, o.ws, b, rows, L.y_dtype)
    assert rel_err(Yg[rows], Yo) <= TOL_Y
    Ye, env, jump = oracle_rows_exact(Xcol, o.inv, p, o.wc, o.ws, b, rows)
    assert_y_strict(Yg[rows], Ye, env, jump, L.y_dtype, L.K // 64, p.rank)
    assert np.all(np.isfinite(Yg))
    _check_against_linear(L, Xcol, p, b, got)


def test_conv_workspace_reuse_smaller_image():
    """One Conv2d called on a large then a smaller image: the second result does
    not depend on what the first left in the workspace."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    big = wl.ConvLayer(2, 20, 18, 128, 64, 3, 3, 1, 1, 32, "f16", "f16", "big")
    small = wl.ConvLayer(1, 7, 5, 128, 64, 3, 3, 1, 1, 32, "f16", "f16", "small")
    Xb, Wc, b = _edge_inputs(big, seed=11)
    Xs, _, _ = _edge_inputs(small, seed=12)
    p, _, _ = _setup(big, Xb, Wc, b)
    conv = sq.Conv2d(p, 3, 3, 1, 1, b)
    conv(dev(Xb))
    Ys = conv(dev(Xs))
    torch.cuda.synchronize()
    Ys2 = sq.Conv2d(p, 3, 3, 1, 1, b)(dev(Xs))
    torch.cuda.synchronize()
    assert torch.equal(Ys.view(torch.uint8), Ys2.view(torch.uint8))
    Xcol = O.im2col_nhwc(Xs, 3, 3, 1, 1)
    lam = O.smoothing_factors(O.channel_absmax(O.im2col_nhwc(Xb, 3, 3, 1, 1)),
                              O.conv_weight_matrix(Wc))
    inv = O.inv_smoothing(lam)
    wc, ws = O.quantize_residual_from_factors(O.conv_weight_matrix(Wc), lam, p.L1, p.L2)
    Yo = O.linear(Xcol, inv, p.L1, p.L2, wc, ws, b, "f16")
    assert rel_err(Ys.cpu().numpy().reshape(small.M, 64), Yo) <= TOL_Y


# ---------------------------------------------------------------------------
# the tiled INT4 convolution: K1 on the implicit patch matrix writing K2T's
# operand tiles, then K2T


def _run_tiled(L: wl.ConvLayer, X, p, bias):
    """Tiled K1-conv alone (outputs prefilled with canaries), and the whole
    convolution through Conv2d(tiled=True)."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K, R = L.M, L.K, p.rank
    Xd = dev(X)
    ops = torch.full((sq.int4_act_tiled_bytes(M, K),), 0x5A, dtype=torch.uint8, device="cuda")
    sc = torch.full((sq.int4_act_scales_tiled_bytes(M, K) // 4,), float("nan"),
                    dtype=torch.float32, device="cuda")
    Dt = _dt_buffer(M, R)
    sq.quantize_act_lowrank_down_conv_tiled(Xd, L.KH, L.KW, L.stride, L.pad, dev(p.inv_smooth),
                                            dev(p.L1p) if R else None, R, ops, sc,
                                            Dt if R else None)
    conv = sq.Conv2d(p, L.KH, L.KW, L.stride, L.pad, bias, tiled=True,
                     out_dtype=torch.float16 if L.y_dtype == "f16" else torch.float32)
    Y = conv(Xd)
    torch.cuda.synchronize()
    assert Y.shape == (L.batch, L.OH, L.OW, p.N)
    return ops, sc, Dt, Y


def _check_tiled_against_linear(L, Xcol, p, bias, got):
    """The tiled linear entry points on the materialised patch matrix (the
    pre-kernel without a workspace: unsplit, as the convolution's; the GEMM with
    its workspace, split along K where Conv2d splits it) give the same bits:
    operand tiles, scales, D_t and Y."""
    from test_gpu_tiled import TiledLayer
    torch = torch_mod()
    ops, sc, Dt, Y = got
    d = TiledLayer(Xcol, p, bias, L.y_dtype, k1_workspace=False, k2_workspace=True)
    d.k1()
    d.k2()
    torch.cuda.synchronize()
    assert torch.equal(ops, d.ops)
    assert torch.equal(sc.view(torch.int32), d.scales.view(torch.int32))
    if p.rank:
        assert torch.equal(Dt, d.D)
    assert torch.equal(Y.reshape(L.M, p.N).view(torch.uint8), d.Y.view(torch.uint8))


@pytest.mark.parametrize("L", EDGE, ids=lambda L: L.name.replace(" ", "_"))
def test_conv_tiled_edge_every_element(L):
    X, Wc, b = _edge_inputs(L, seed=L.H * 131 + L.W * 7 + L.C + L.KH + L.stride + 5)
    p, Xcol, o = _setup(L, X, Wc, b)
    got = _run_tiled(L, X, p, b)
    _check_tiled_against_linear(L, Xcol, p, b, got)
    Yg = got[3].cpu().numpy().reshape(L.M, L.N)
    Yo = O.linear(Xcol, o.inv, p.L1, p.L2, o.wc, o.ws, b, L.y_dtype)
    assert rel_err(Yg, Yo) <= TOL_Y
    Ye, env, jump = oracle_rows_exact(Xcol, o.inv, p, o.wc, o.ws, b, np.arange(L.M))
    assert_y_strict(Yg, Ye, env, jump, L.y_dtype, L.K // 64, p.rank)


@pytest.mark.parametrize("idx", range(1, len(wl.CONV_LAYERS)),
                         ids=lambda i: wl.CONV_LAYERS[i].name.replace(" ", "_"))
def test_conv_tiled_unet_sizes(idx):
    """UNet layers at full size on the tiled path: whole tensors against the tiled
    linear path on the materialised patch matrix, sampled output pixels (with the
    image borders) against the oracle."""
    L, X, Wc = wl.conv_inputs(idx)
    b = wl.bias(wl.CONV_CFG, idx, L.N)
    p, Xcol, o = _setup(L, X, Wc, b)
    got = _run_tiled(L, X, p, b)
    _check_tiled_against_linear(L, Xcol, p, b, got)
    rows = sample_rows(L.M, seed=idx + 7)
    border = [0, L.OW - 1, (L.OH - 1) * L.OW, L.OH * L.OW - 1, L.OH * L.OW, L.M - 1]
    rows = np.unique(np.concatenate([rows, border]))
    Yg = got[3].cpu().numpy().reshape(L.M, L.N)
    Yo = oracle_rows(Xcol, o.inv, p, o.wc, o.ws, b, rows, L.y_dtype)
    assert rel_err(Yg[rows], Yo) <= TOL_Y
    Ye, env, jump = oracle_rows_exact(Xcol, o.inv, p, o.wc, o.ws, b, rows)
    assert_y_strict(Yg[rows], Ye, env, jump, L.y_dtype, L.K // 64, p.rank)
    assert np.all(np.isfinite(Yg))


# ---------------------------------------------------------------------------
# the MXFP4 convolution: K1-MX on the implicit patch matrix, then K2-MX

import mx_tiles as T  # noqa: E402
from test_gpu_mx import _assert_strict, _exact_rows  # noqa: E402


def _setup_mx(L: wl.ConvLayer, X, Wc):
    import bit_post_quantized_smooth_amd as sq
    Wm = O.conv_weight_matrix(Wc)
    lam = sq.smoothing_factors(sq.conv_patch_absmax(X, L.KH, L.KW, L.stride, L.pad), Wm)
    p = sq.prepare_weights_mx(Wm, lam, L.rank)
    Xcol = O.im2col_nhwc(X, L.KH, L.KW, L.stride, L.pad)
    lam_o = O.smoothing_factors(O.channel_absmax(Xcol), Wm)
    inv = O.inv_smoothing(lam_o)
    wc, we = O.mx_quantize_residual_from_factors(Wm, lam_o, p.L1, p.L2)
    assert np.array_equal(inv, p.inv_smooth)
    assert np.array_equal(wc, p.w_codes) and np.array_equal(we, p.w_scales)
    return p, Xcol, inv, wc, we


def _dt_buffer(M, R):
    """A D_t buffer (fp16 D in operand order) filled with NaN bits."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    return torch.full((max(sq.int4_d_tiled_bytes(M, R), 2) // 2,), -1, dtype=torch.int16,
                      device="cuda")


def _assert_d_t(Dt, rows, xh, L1, K, M, R):
    """fp16(D) from D_t against the oracle's D of `rows`: the pre-kernel's bound
    plus half an fp16 ulp of its one rounding (2^-11 relative, 2^-25 below the
    normal range)."""
    Dg = int4_tiles.untile_d(Dt.cpu().numpy(), M, R)[rows].astype(np.float64)
    Do = O.down_projection(xh, L1)
    tol = d_stat_bound(xh, L1, K) + 2.0 ** -11 * np.abs(Do) + 2.0 ** -25
    assert float(np.max(np.abs(Dg - Do) / tol)) <= 1.0
    assert np.all(np.isfinite(Dg))


def _run_mx(L: wl.ConvLayer, X, p, bias):
    """K1-MX on the patches (tiled outputs read back as canonical codes and
    exponents), and the whole MXFP4 convolution."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K, R = L.M, L.K, p.rank
    Xd = dev(X)
    ct = torch.full((sq.mx_codes_tiled_bytes(M, K),), 0x5A, dtype=torch.uint8, device="cuda")
    et = torch.full((sq.mx_exps_tiled_bytes(M, K),), 0x5A, dtype=torch.uint8, device="cuda")
    D = _dt_buffer(M, R)
    sq.quantize_act_lowrank_down_conv_mx(Xd, L.KH, L.KW, L.stride, L.pad, dev(p.inv_smooth),
                                         dev(p.L1p) if R else None, R, ct, et, D if R else None)
    conv = sq.Conv2d(p, L.KH, L.KW, L.stride, L.pad, bias,
                     out_dtype=torch.float16 if L.y_dtype == "f16" else torch.float32)
    Y = conv(Xd)
    torch.cuda.synchronize()
    c = T.untile_codes(ct.cpu().numpy(), M, K)
    e = T.untile_exps(et.cpu().numpy(), M, K)
    if K % 128:
        assert not c[:M, K // 2:].any() and np.all(e[:M, K // 32:] == 127)
    return c[:M, :K // 2], e[:M, :K // 32], D, Y, (ct, et)


def _check_mx_against_linear(L, Xcol, p, bias, tiles, D, Y):
    """K1-MX and the MXFP4 linear layer on the materialised patch matrix give the same bits."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K, R = L.M, L.K, p.rank
    Xd = dev(Xcol)
    ct = torch.full((sq.mx_codes_tiled_bytes(M, K),), 0x5A, dtype=torch.uint8, device="cuda")
    et = torch.full((sq.mx_exps_tiled_bytes(M, K),), 0x5A, dtype=torch.uint8, device="cuda")
    D2 = _dt_buffer(M, R)
    sq.quantize_act_lowrank_down_mx(Xd, dev(p.inv_smooth), dev(p.L1p) if R else None, R, ct, et,
                                    D2 if R else None)
    lin = sq.Linear(p, bias, out_dtype=torch.float16 if L.y_dtype == "f16" else torch.float32)
    Y2 = lin(Xd)
    torch.cuda.synchronize()
    assert torch.equal(ct, tiles[0]) and torch.equal(et, tiles[1])
    if R:
        assert torch.equal(D, D2)
    assert torch.equal(Y.reshape(M, p.N).view(torch.uint8), Y2.view(torch.uint8))


MX_EDGE = [EDGE[0], EDGE[1], EDGE[3], EDGE[4], EDGE[5], EDGE[6], EDGE[7]]


@pytest.mark.parametrize("L", MX_EDGE, ids=lambda L: "mx_" + L.name.replace(" ", "_"))
def test_conv_mx_edge_every_element(L):
    X, Wc, b = _edge_inputs(L, seed=L.H * 131 + L.W * 7 + L.C + L.KH + L.stride + 1)
    p, Xcol, inv, wc, we = _setup_mx(L, X, Wc)
    c, e, D, Y, tiles = _run_mx(L, X, p, b)
    oc, oe, xh = O.mx_quantize_activation(Xcol, inv)
    assert np.array_equal(c, oc)
    assert np.array_equal(e, oe)
    if p.rank:
        _assert_d_t(D, np.arange(L.M), xh, p.L1, L.K, L.M, p.rank)
    Yg = Y.cpu().numpy().reshape(L.M, L.N)
    Yo = O.mx_linear(Xcol, inv, p.L1, p.L2, wc, we, b, L.y_dtype)
    assert rel_err(Yg, Yo) <= TOL_Y
    Ye, env, jump = _exact_rows(Xcol, inv, p, wc, we, b, np.arange(L.M))
    _assert_strict(Yg, Ye, env, jump, L.y_dtype, L.K, p.rank)
    _check_mx_against_linear(L, Xcol, p, b, tiles, D, Y)


@pytest.mark.parametrize("idx", [1, 3], ids=lambda i: "mx_" + wl.CONV_LAYERS[i].name.replace(" ", "_"))
def test_conv_mx_unet_sizes(idx):
    L, X, Wc = wl.conv_inputs(idx)
    b = wl.bias(wl.CONV_CFG, idx, L.N)
    p, Xcol, inv, wc, we = _setup_mx(L, X, Wc)
    c, e, D, Y, tiles = _run_mx(L, X, p, b)
    rows = sample_rows(L.M, seed=idx + 50)
    border = [0, L.OW - 1, (L.OH - 1) * L.OW, L.OH * L.OW - 1, L.OH * L.OW, L.M - 1]
    rows = np.unique(np.concatenate([rows, border]))
    oc, oe, xh = O.mx_quantize_activation(Xcol[rows], inv)
    assert np.array_equal(c[rows], oc)
    assert np.array_equal(e[rows], oe)
    _assert_d_t(D, rows, xh, p.L1, L.K, L.M, p.rank)
    Yg = Y.cpu().numpy().reshape(L.M, L.N)
    Yo = np.concatenate([O.mx_linear(Xcol[rows[i:i + 16]], inv, p.L1, p.L2, wc, we, b, L.y_dtype)
                         for i in range(0, len(rows), 16)])
    assert rel_err(Yg[rows], Yo) <= TOL_Y
    Ye, env, jump = _exact_rows(Xcol, inv, p, wc, we, b, rows)
    _assert_strict(Yg[rows], Ye, env, jump, L.y_dtype, L.K, p.rank)
    assert np.all(np.isfinite(Yg))
    _check_mx_against_linear(L, Xcol, p, b, tiles, D, Y)
