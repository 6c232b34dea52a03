"""GPU parity of the 4-bit weight-only baseline (W4A16) through the C ABI
against the CPU oracle's w4a16_linear.

Bit-exact: the tiled fp16 activation (whole tensors, against the index
formulas of svdq.h in tests/w16_tiles.py). Within 2e-3 * max|Y| and within an
element-wise rounding bound (one output ulp plus two fp32 roundings per step of
32 along K, each at most 2^-24 of |fp16(X)| . |fp16(s q)|^T + |b|): the layer
output on sampled rows at the full sizes, and on every element for small and
ragged shapes (K an odd multiple of 64, M and N not multiples of the tiles,
fp32 X or Y, no bias)."""
import functools

import numpy as np
import pytest

import oracle as O
import w16_tiles as T
import workloads as wl
from gpu_common import TOL_Y, dev, rel_err, sample_rows, torch_mod

pytestmark = pytest.mark.gpu

SPECS = [(0, 0), (1, 0), (2, 0), (2, 1), (3, 0), (3, 2), (3, 4), (4, 0)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_post_quantized_smooth_amd  # noqa: F401  (raises if the library is missing)


@functools.lru_cache(maxsize=3)
def _layer(cfg: int, li: int):
    import bit_post_quantized_smooth_amd as sq
    L, X, W = wl.layer_inputs(cfg, li)
    return L, X, W, sq.prepare_weights_w4a16(W)


def _run(X, p, bias, y_dtype):
    """(x_t, Y) from the two kernels, and Y again from the one-call layer."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K = X.shape
    ct, st = sq.pack_w4a16_tiles(p.w_codes, p.w_scales, K)
    wc, ws = dev(ct), dev(st)
    Xd = dev(X)
    bd = dev(bias) if bias is not None else None
    ydt = torch.float16 if y_dtype == "f16" else torch.float32
    x_t = torch.full((sq.w4a16_x_tiled_bytes(M, K) // 2,), 0x5A5A, dtype=torch.int16, device="cuda")
    Y = torch.empty((M, p.N), dtype=ydt, device="cuda")
    sq.w4a16_tile_activation(Xd, x_t)
    sq.w4a16_gemm(x_t, wc, ws, bd, Y, K)
    Y2 = torch.empty_like(Y)
    wsp = torch.empty(sq.w4a16_x_tiled_bytes(M, K), dtype=torch.uint8, device="cuda")
    sq.linear_w4a16(Xd, wc, ws, bd, Y2, wsp)
    torch.cuda.synchronize()
    Yg = Y.cpu().numpy()
    assert np.array_equal(Yg.view(np.uint8), Y2.cpu().numpy().view(np.uint8))
    return x_t.cpu().numpy().view(np.uint16), Yg


def _assert_strict(Yg, X, p, bias, rows, out_dtype, K):
    Ye = O.w4a16_linear(X[rows], p.w_codes, p.w_scales.view(np.float16), bias, "f64")
    env = (np.abs(O.to_f16(X[rows]).astype(np.float64))
           @ np.abs(O.w4a16_dequant(p.w_codes, p.w_scales.view(np.float16)).astype(np.float64)).T)
    if bias is not None:
        env += np.abs(np.asarray(bias, np.float64))[None, :]
    a = np.abs(Ye)
    if out_dtype == "f16":
        ulp = np.maximum(np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -14))) - 10), 2.0 ** -24)
    else:
        ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 23)
    tol = ulp + (2 * (K // 32) + 4) * 2.0 ** -24 * env
    ratio = np.abs(np.asarray(Yg, np.float64) - Ye) / tol
    assert float(ratio.max()) <= 1.0, (int(np.count_nonzero(ratio > 1)), float(ratio.max()))


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: f"c{s[0]}l{s[1]}")
def test_w4a16_matches_oracle(spec):
    L, X, W, p = _layer(*spec)
    bias = wl.bias(spec[0], spec[1], L.N)
    wc, ws = O.w4a16_prepare(W)
    assert np.array_equal(wc, p.w_codes) and np.array_equal(ws.view(np.uint16), p.w_scales)
    x_t, Yg = _run(X, p, bias, L.y_dtype)
    assert np.array_equal(x_t, T.tile_x(O.to_f16(X)))
    assert np.all(np.isfinite(Yg))
    rows = sample_rows(L.M, seed=spec[0] * 100 + spec[1] + 11)
    Yo = O.w4a16_linear(X[rows], wc, ws, bias, L.y_dtype)
    err = rel_err(Yg[rows], Yo)
    assert err <= TOL_Y, err
    _assert_strict(Yg[rows], X, p, bias, rows, L.y_dtype, L.K)


EDGE = [
    # M, K, N, x_dtype, y_dtype, bias
    (1, 64, 1, "f32", "f32", True),
    (17, 192, 130, "f16", "f16", True),
    (129, 320, 257, "f16", "f32", False),
    (200, 384, 320, "f32", "f16", True),
    (64, 1024, 512, "f16", "f16", True),
    (300, 640, 136, "f16", "f16", False),
    (33, 128, 600, "f32", "f16", True),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "x".join(map(str, c[:3])) + f"_{c[3]}_{c[4]}")
def test_w4a16_edge_shapes_every_element(case):
    import bit_post_quantized_smooth_amd as sq
    M, K, N, xdt, ydt, use_bias = case
    rng = np.random.default_rng(M * 13 + K + N)
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    X = X.astype(np.float16 if xdt == "f16" else np.float32)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    W[rng.choice(K, max(1, K // 100), replace=False)] *= 10
    bias = (rng.standard_normal(N) * 0.1).astype(np.float32) if use_bias else None
    p = sq.prepare_weights_w4a16(W)
    wc, ws = O.w4a16_prepare(W)
    assert np.array_equal(wc, p.w_codes) and np.array_equal(ws.view(np.uint16), p.w_scales)
    x_t, Yg = _run(X, p, bias, ydt)
    assert np.array_equal(x_t, T.tile_x(O.to_f16(X)))
    Yo = O.w4a16_linear(X, wc, ws, bias, ydt)
    assert rel_err(Yg, Yo) <= TOL_Y
    _assert_strict(Yg, X, p, bias, np.arange(M), ydt, K)


def test_w4a16_linear_class_and_streams():
    """Linear(prep of fmt w4a16) gives the same bits on the current and a side stream."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    L, X, W, p = _layer(0, 0)
    lin = sq.Linear(p, wl.bias(0, 0, L.N), out_dtype=torch.float32)
    Xd = dev(X)
    Y1 = lin(Xd)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Y2 = lin(Xd)
    s.synchronize()
    torch.cuda.synchronize()
    assert np.array_equal(Y1.cpu().numpy().view(np.uint32), Y2.cpu().numpy().view(np.uint32))
    Yo = O.w4a16_linear(X, p.w_codes, p.w_scales.view(np.float16), wl.bias(0, 0, L.N), "f32")
    assert rel_err(Y1.cpu().numpy(), Yo) <= TOL_Y
