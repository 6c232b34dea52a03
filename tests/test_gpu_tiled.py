"""GPU parity of the tiled INT4 path (svdq_quantize_act_lowrank_down_tiled,
svdq_w4a4_gemm_lowrank_up_tiled, svdq_linear_tiled) through the C ABI against
the CPU oracle.

Bit-exact: the activation operands and fp32 scales the tiled pre-kernel
writes (read back with the layout formulas of svdq.h, tests/int4_tiles.py),
and the tiled GEMM's own int32 group partials, exposed through Y with
power-of-two scales as in test_gpu_k2_partials.py. Within 2e-3 of max|Y| and
within the element-wise rounding bound of gpu_common.assert_y_strict: the
whole layer at the full sizes of every workload (sampled rows) and on the
ragged edge shapes (every element)."""
import numpy as np
import pytest

import oracle as O
import int4_tiles as T
from gpu_common import (TOL_Y, assert_y_strict, d_stat_bound, dev, host_u16, layer, oracle_prep,
                        oracle_rows, oracle_rows_exact, rel_err, sample_rows, torch_mod)
from test_gpu_parity import EDGE, SPECS, _edge_inputs, _ids

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_post_quantized_smooth_amd  # noqa: F401  (raises if the library is missing)


def sq_mod():
    import bit_post_quantized_smooth_amd as sq
    return sq


class TiledLayer:
    """Device buffers of one layer on the tiled path (weights packed by the library)."""

    def __init__(self, X, p, bias, y_dtype="f16", k1_workspace=True, k2_workspace=False):
        torch = torch_mod()
        sq = sq_mod()
        self.M, self.K = X.shape
        self.N, self.R = p.N, p.rank
        self.X = dev(X)
        self.inv = dev(p.inv_smooth)
        self.L1p = dev(p.L1p) if self.R else None
        self.L2t = dev(p.L2t) if self.R else None
        ct, st = sq.pack_w4a4_tiles(p.w_codes, p.w_scales, self.K)
        self.wc, self.ws = dev(ct), dev(st)
        self.bias = dev(bias) if bias is not None else None
        self.ops = torch.full((sq.int4_act_tiled_bytes(self.M, self.K),), 0x5A, dtype=torch.uint8,
                              device="cuda")
        self.scales = torch.full((sq.int4_act_scales_tiled_bytes(self.M, self.K) // 4,),
                                 float("nan"), dtype=torch.float32, device="cuda")
        self.D = torch.full((max(sq.int4_d_tiled_bytes(self.M, self.R), 2) // 2,), -1,
                            dtype=torch.int16, device="cuda")
        self.Y = torch.full((self.M, self.N), float("nan"),
                            dtype=torch.float16 if y_dtype == "f16" else torch.float32,
                            device="cuda")

        # the optional pre-kernel workspace (long rows run split, as in
        # svdq_linear_tiled), filled with garbage
        need = sq.quantize_act_workspace_bytes(self.M, self.K, self.R)
        self.k1ws = (torch.full((max(need, 256),), 0xA5, dtype=torch.uint8, device="cuda")
                     if k1_workspace else None)
        # the GEMM's optional workspace (an under-filled long-K shape runs split
        # along K), filled with garbage
        need = sq.gemm_tiled_workspace_bytes(self.M, self.N, self.K)
        self.k2ws = (torch.full((max(need, 256),), 0xA5, dtype=torch.uint8, device="cuda")
                     if k2_workspace else None)

    def k1(self):
        sq_mod().quantize_act_lowrank_down_tiled(self.X, self.inv, self.L1p, self.R, self.ops,
                                                 self.scales, self.D if self.R else None,
                                                 workspace=self.k1ws)

    def k2(self, activation=None):
        sq_mod().w4a4_gemm_lowrank_up_tiled(self.ops, self.scales, self.wc, self.ws,
                                            self.D if self.R else None, self.L2t, self.R,
                                            self.bias, self.Y, self.K, activation=activation,
                                            workspace=self.k2ws)


def _check_k1_tiled(X, inv_o, p, K, d):
    """The tiled pre-kernel's outputs against the oracle's codes, scales and D."""
    M = X.shape[0]
    a_codes, a_scales, xh = O.quantize_activation(X, inv_o)
    q = T.untile_act_ops(d.ops.cpu().numpy(), M, K)
    ref = T.unpack(a_codes)
    nbad = int(np.count_nonzero(q[:M] != ref))
    assert nbad == 0, f"{nbad} activation operands differ"
    assert np.all(q[M:] == ref[M - 1]), "rows past M must repeat the last row"
    sc = d.scales.cpu().numpy()
    idx = T.act_scale_index(M, K)
    exp = T.tile_act_scales(a_scales, M, K)
    assert np.array_equal(sc[idx[:M]].view(np.uint32), exp[idx[:M]].view(np.uint32))
    Mb16 = ((M + 15) // 16) * 16
    if Mb16 > M:
        assert np.array_equal(sc[idx[M:Mb16]], np.repeat(sc[idx[M - 1:M]], Mb16 - M, 0))
    if p.rank:
        # D_t: fp16(D) in operand order; its one fp16 rounding adds up to half an
        # fp16 ulp of |D| (2^-11 relative, 2^-25 absolute below the normal range)
        Dg = T.untile_d(d.D.cpu().numpy(), M, p.rank).astype(np.float64)
        Do = O.down_projection(xh, p.L1)
        tol = d_stat_bound(xh, p.L1, K) + 2.0 ** -11 * np.abs(Do) + 2.0 ** -25
        worst = float(np.max(np.abs(Dg - Do) / tol))
        assert worst <= 1.0, worst
        assert np.all(np.isfinite(Dg))


@pytest.mark.parametrize("spec", SPECS, ids=_ids)
def test_k1_tiled_bit_exact(spec):
    torch = torch_mod()
    L, X, W, lam, p, bias = layer(*spec)
    _, inv_o, wc, ws = oracle_prep(X, W, p, L.rank)
    d = TiledLayer(X, p, bias, L.y_dtype)
    d.k1()
    torch.cuda.synchronize()
    _check_k1_tiled(X, inv_o, p, L.K, d)


def _run_k2t(a_codes, w_codes, sx, sw, M, N, K, pad=3):
    """The tiled GEMM at rank 0 on operands tiled by the test's own layout code."""
    torch = torch_mod()
    Ybig = torch.full((M, N + pad), float("nan"), dtype=torch.float32, device="cuda")
    Ybig[:, N:] = -3.0
    ct, st = T.tile_w(w_codes, np.asarray(sw, dtype=np.float16).view(np.uint16), N, K)
    sq_mod().w4a4_gemm_lowrank_up_tiled(dev(T.tile_act_ops(a_codes, M, K)),
                                        dev(T.tile_act_scales(sx, M, K)), dev(ct), dev(st), None, None,
                                        0, None, Ybig[:, :N], K)
    torch.cuda.synchronize()
    Yh = Ybig.cpu().numpy()
    assert np.all(Yh[:, N:] == -3.0), "K2T wrote past column N"
    return Yh[:, :N]


def _partials_checks(a_codes, w_codes, M, N, K, groups):
    G = K // 64
    for g in groups:
        sx = np.zeros((M, G), dtype=np.float16)
        sw = np.zeros((N, G), dtype=np.float16)
        sx[:, g] = np.exp2(-(np.arange(M) % 3))
        sw[:, g] = np.exp2(-(np.arange(N) % 5))
        Y = _run_k2t(a_codes, w_codes, sx, sw, M, N, K)
        sl = slice(32 * g, 32 * (g + 1))
        P = O.group_partials(a_codes[:, sl], w_codes[:, sl])[:, :, 0].astype(np.float64)
        ref = P * np.exp2(-(np.arange(M) % 3))[:, None] * np.exp2(-(np.arange(N) % 5))[None, :]
        bad = np.count_nonzero(Y.astype(np.float64) != ref)
        assert bad == 0, f"group {g}: {bad} of {M * N} outputs differ"
    s = np.full((M, G), 2.0 ** -4, dtype=np.float16)
    t = np.full((N, G), 2.0 ** -4, dtype=np.float16)
    Y = _run_k2t(a_codes, w_codes, s, t, M, N, K)
    Psum = O.group_partials(a_codes, w_codes, group=K)[:, :, 0].astype(np.float64)
    bad = np.count_nonzero(Y.astype(np.float64) * 256.0 != Psum)
    assert bad == 0, f"uniform scales: {bad} of {M * N} outputs differ"


@pytest.mark.parametrize("spec", SPECS, ids=_ids)
def test_k2_tiled_partials_bit_exact(spec):
    L, X, W, lam, p, _ = layer(*spec)
    _, inv_o, wc, _ = oracle_prep(X, W, p, L.rank)
    a_codes, _, _ = O.quantize_activation(X, inv_o)
    G = L.K // 64
    _partials_checks(a_codes, wc, L.M, L.N, L.K, sorted({0, 1 % G, G // 2, G - 1}))


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "x".join(map(str, c[:3])))
def test_k2_tiled_partials_edge_shapes(case):
    M, K, N = case[0], case[1], case[2]
    rng = np.random.default_rng(M + 7 * N + 1)
    a_codes = O.pack_nibbles(rng.integers(-7, 8, size=(M, K)))
    w_codes = O.pack_nibbles(rng.integers(-7, 8, size=(N, K)))
    _partials_checks(a_codes, w_codes, M, N, K, sorted({0, K // 64 - 1}))


@pytest.mark.parametrize("sign", [1, -1])
def test_k2_tiled_partials_extreme_codes(sign):
    M, K, N = 130, 12288, 200
    _partials_checks(O.pack_nibbles(np.full((M, K), 7)), O.pack_nibbles(np.full((N, K), 7 * sign)),
                     M, N, K, [0, 191])


@pytest.mark.parametrize("spec", SPECS, ids=_ids)
def test_linear_tiled_matches_oracle(spec):
    sq = sq_mod()
    torch = torch_mod()
    L, X, W, lam, p, bias = layer(*spec, with_bias=True)
    _, inv_o, wc, ws = oracle_prep(X, W, p, L.rank)
    d = TiledLayer(X, p, bias, L.y_dtype)
    d.k1()
    d.k2()
    # the whole layer in one call gives the same bits as the two kernels
    Y2 = torch.full_like(d.Y, float("nan"))
    wsb = torch.empty(sq.linear_tiled_workspace_bytes(L.M, L.K, p.rank), dtype=torch.uint8,
                      device="cuda")
    sq.linear_tiled(d.X, d.inv, d.L1p, d.L2t, p.rank, d.wc, d.ws, d.bias, Y2, wsb)
    torch.cuda.synchronize()
    Yg = d.Y.cpu().numpy()
    assert np.array_equal(Yg.view(np.uint8), Y2.cpu().numpy().view(np.uint8))
    assert np.all(np.isfinite(Yg))
    rows = sample_rows(L.M, seed=spec[0] * 100 + spec[1] + 1)
    Yo = oracle_rows(X, inv_o, p, wc, ws, bias, rows, L.y_dtype)
    err = rel_err(Yg[rows], Yo)
    assert err <= TOL_Y, err
    Ye, env, jump = oracle_rows_exact(X, inv_o, p, wc, ws, bias, rows)
    assert_y_strict(Yg[rows], Ye, env, jump, L.y_dtype, L.K // 64, p.rank)


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "x".join(map(str, c[:4])) + f"_{c[4]}_{c[5]}")
def test_linear_tiled_edge_shapes_every_element(case):
    sq = sq_mod()
    torch = torch_mod()
    M, K, N, R, xdt, ydt, use_bias = case
    X, W, b = _edge_inputs(M, K, N, R, xdt, seed=M * 31 + K + N + R)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, R)
    bias = b if use_bias else None
    _, inv_o, wc, ws = oracle_prep(X, W, p)
    d = TiledLayer(X, p, bias, ydt)
    d.k1()
    d.k2()
    torch.cuda.synchronize()
    _check_k1_tiled(X, inv_o, p, K, d)
    Yo = O.linear(X, inv_o, p.L1, p.L2, wc, ws, bias, ydt)
    assert rel_err(d.Y.cpu().numpy(), Yo) <= TOL_Y
    Ye, env, jump = oracle_rows_exact(X, inv_o, p, wc, ws, bias, np.arange(M))
    assert_y_strict(d.Y.cpu().numpy(), Ye, env, jump, ydt, K // 64, R)


def test_linear_tiled_strided_output_and_gelu():
    """ldy > N (a column slice of a wider output), ragged M and N, fused GELU:
    the padding columns and the rows around Y keep their canary."""
    sq = sq_mod()
    torch = torch_mod()
    M, K, N, R = 300, 640, 200, 32
    X, W, b = _edge_inputs(M, K, N, R, "f16", seed=21)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, R)
    _, inv_o, wc, ws = oracle_prep(X, W, p)
    ct, st = sq.pack_w4a4_tiles(p.w_codes, p.w_scales, K)
    Ybig = torch.full((M + 2, N + 56), -7.0, dtype=torch.float16, device="cuda")
    Y = Ybig[1:M + 1, :N]
    wsb = torch.empty(sq.linear_tiled_workspace_bytes(M, K, R), dtype=torch.uint8, device="cuda")
    sq.linear_tiled(dev(X), dev(p.inv_smooth), dev(p.L1p), dev(p.L2t), R, dev(ct), dev(st), dev(b),
                    Y, wsb, activation="gelu_tanh")
    torch.cuda.synchronize()
    Yb = Ybig.cpu().numpy()
    assert np.all(Yb[0] == -7.0) and np.all(Yb[M + 1] == -7.0) and np.all(Yb[:, N:] == -7.0)
    Go = O.linear(X, inv_o, p.L1, p.L2, wc, ws, b, "f16", activation="gelu_tanh")
    assert rel_err(Yb[1:M + 1, :N], Go) <= TOL_Y


def test_mlp_chain_tiled_fused_gelu():
    """The DiT MLP pair on the tiled path, GELU fused into the up-projection's
    epilogue, against the oracle's chain (the same 1e-2 bound as the other
    chain tests: the down layer re-quantizes an intermediate that agrees with
    the oracle's to about one fp16 ulp)."""
    sq = sq_mod()
    torch = torch_mod()
    Lu, X, Wu, _, pu, _ = layer(2, 0)
    Ld, Xd_cal, Wd, _, pd, _ = layer(2, 1)
    rows = np.arange(0, Lu.M, 97)[:48]
    _, inv_u, wcu, wsu = oracle_prep(X, Wu, pu, Lu.rank)
    _, inv_d, wcd, wsd = oracle_prep(Xd_cal, Wd, pd, Ld.rank)
    Hu = np.concatenate([O.linear(X[rows[i:i + 16]], inv_u, pu.L1, pu.L2, wcu, wsu, None, "f16",
                                  activation="gelu_tanh") for i in range(0, len(rows), 16)])
    Yo = oracle_rows(Hu, inv_d, pd, wcd, wsd, None, np.arange(len(rows)), "f16")
    up = sq.Linear(pu, activation="gelu_tanh", tiled=True)
    down = sq.Linear(pd, tiled=True)
    Yd = down(up(dev(X)))
    torch.cuda.synchronize()
    assert rel_err(Yd.cpu().numpy()[rows], Yo) <= 1e-2


# Under-filled long-K GEMMs (at most half of the resident workgroup slots,
# at least 32 groups) run split along K when the GEMM gets its workspace:
# slice s of a tile sums groups s*G/S .. (s+1)*G/S - 1 (slice 0 with the
# low-rank term) into an fp32 partial tile, and a second pass sums the slices
# in order before the bias, the activation and the rounding. Y must meet the
# oracle's element-wise bound, the fused entry point with room for the split
# must give the same bits as the two calls, and the unsplit kernel the same
# bound (its sums run in another order).
SPLITK = [
    # M, K, N, R, x, y, bias, activation: 16 x 5 tiles, S = 4; 8 x 5 tiles, S = 2
    (2000, 4096, 600, 32, "f16", "f16", True, None),
    (1024, 2560, 640, 16, "f32", "f32", False, "gelu_tanh"),
]


@pytest.mark.parametrize("case", SPLITK, ids=lambda c: "x".join(map(str, c[:4])) + f"_{c[5]}")
def test_gemm_split_along_k(case):
    sq = sq_mod()
    torch = torch_mod()
    M, K, N, R, xdt, ydt, use_bias, act = case
    X, W, b = _edge_inputs(M, K, N, R, xdt, seed=M + K + N + R + 9)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, R)
    bias = b if use_bias else None
    _, inv_o, wc, ws = oracle_prep(X, W, p)
    assert sq.gemm_tiled_workspace_bytes(M, N, K) > 0        # the shape splits on MI355X
    d = TiledLayer(X, p, bias, ydt, k2_workspace=True)
    d.k1()
    d.k2(activation=act)
    torch.cuda.synchronize()
    Yg = d.Y.cpu().numpy()
    assert np.all(np.isfinite(Yg))
    rows = sample_rows(M, seed=M + N)
    if act is None:
        Ye, env, jump = oracle_rows_exact(X, inv_o, p, wc, ws, bias, rows)
        assert_y_strict(Yg[rows], Ye, env, jump, ydt, K // 64, R)
    Yo = O.linear(X[rows], inv_o, p.L1, p.L2, wc, ws, bias, ydt, activation=act)
    assert rel_err(Yg[rows], Yo) <= TOL_Y
    # the fused entry point with room for the split: the same bits
    need = sq.linear_tiled_workspace_bytes(M, K, R) + sq.gemm_tiled_workspace_bytes(M, N, K)
    wsb = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    Y2 = torch.full_like(d.Y, float("nan"))
    sq.linear_tiled(d.X, d.inv, d.L1p, d.L2t, R, d.wc, d.ws, d.bias, Y2, wsb, activation=act)
    torch.cuda.synchronize()
    assert torch.equal(d.Y.view(torch.uint8), Y2.view(torch.uint8))
    # unsplit: the same bound
    d2 = TiledLayer(X, p, bias, ydt, k2_workspace=False)
    d2.k1()
    d2.k2(activation=act)
    torch.cuda.synchronize()
    Yu = d2.Y.cpu().numpy()
    if act is None:
        assert_y_strict(Yu[rows], Ye, env, jump, ydt, K // 64, R)
    assert rel_err(Yu, Yg) <= TOL_Y
