"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: activation codes and scales (whole tensors), integer group partials
(sampled row slices, including the tails). Within 2e-3 * max|Y|: the layer
output on sampled rows at the full sizes of the five workloads, and on every
element for the small and edge-case shapes."""
import numpy as np
import pytest

import oracle as O
import workloads as wl
from gpu_common import (TOL_Y, DeviceLayer, assert_y_strict, d_stat_bound, dev, host_u16, layer,
                        oracle_prep, oracle_rows, oracle_rows_exact,
                        rel_err, sample_rows, torch_mod)

pytestmark = pytest.mark.gpu

# (config, layer) pairs at their full sizes
SPECS = [(0, 0), (1, 0), (2, 0), (2, 1), (3, 0), (3, 1), (3, 2), (3, 3), (3, 4), (4, 0), (4, 18)]


def _ids(s):
    return f"c{s[0]}l{s[1]}"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_post_quantized_smooth_amd  # noqa: F401  (raises if the library is missing)


def _d_tolerance(xh, L1, K):
    """|D_gpu - D_oracle| <= K * 2^-23 * (|fp16(xh)| . |L1|) + 2^-24 * |D| (fp32 sums)."""
    env = np.abs(O.to_f16(xh).astype(np.float64)) @ np.abs(np.asarray(L1, np.float64))
    return K * 2.0 ** -23 * env


@pytest.mark.parametrize("spec", SPECS, ids=_ids)
def test_k1_codes_scales_bit_exact(spec):
    torch = torch_mod()
    L, X, W, lam, p, bias = layer(*spec)
    lam_o, inv_o, wc, ws = oracle_prep(X, W, p, L.rank)
    assert np.array_equal(inv_o, p.inv_smooth)
    assert np.array_equal(wc, p.w_codes) and np.array_equal(ws.view(np.uint16), p.w_scales)
    d = DeviceLayer(X, p, bias, L.y_dtype)
    d.k1()
    torch.cuda.synchronize()
    a_codes, a_scales, xh = O.quantize_activation(X, inv_o)
    got_c = d.a_codes.cpu().numpy()
    got_s = host_u16(d.a_scales)
    nbad = int(np.count_nonzero(got_c != a_codes))
    assert nbad == 0, f"{nbad} code bytes differ"
    assert np.array_equal(got_s, a_scales.view(np.uint16))
    if p.rank:
        Dg = d.D.cpu().numpy()[:, :p.rank].astype(np.float64)
        Do = O.down_projection(xh, p.L1)
        tol = _d_tolerance(xh, p.L1, L.K) + 1e-30
        assert np.all(np.abs(Dg - Do) <= tol + 2.0 ** -24 * np.abs(Do))
        assert rel_err(Dg, Do) <= 1e-3
        # The bound above is the worst case (every fp32 addition rounding the
        # same way). Rounding that random-walks over the K/64 accumulating
        # matrix instructions stays near sqrt(K/64) * 2^-24 of the envelope;
        # 16x that still catches a corrupted operand (seen once at 2e-5).
        worst = float(np.max(np.abs(Dg - Do) / (d_stat_bound(xh, p.L1, L.K) + 1e-30)))
        assert worst <= 1.0, worst


@pytest.mark.parametrize("spec", SPECS, ids=_ids)
def test_group_partials_bit_exact(spec):
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    L, X, W, lam, p, bias = layer(*spec)
    _, inv_o, wc, ws = oracle_prep(X, W, p, L.rank)
    d = DeviceLayer(X, p, bias, L.y_dtype)
    d.k1()
    a_codes, _, _ = O.quantize_activation(X, inv_o)
    G = L.K // 64
    M = L.M
    slices = [(0, min(16, M)), (max(0, min(M, 136) - 17), min(17, M)), (max(0, M - 33), min(33, M))]
    for row0, rows in slices:
        P = torch.empty((rows, L.N, G), dtype=torch.int32, device="cuda")
        sq.debug_group_partials(d.a_codes, d.wc, M, L.N, L.K, row0, rows, P)
        torch.cuda.synchronize()
        ref = O.group_partials(a_codes[row0:row0 + rows], wc)
        assert np.array_equal(P.cpu().numpy(), ref.astype(np.int32)), (row0, rows)


@pytest.mark.parametrize("spec", SPECS, ids=_ids)
def test_linear_matches_oracle(spec):
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    L, X, W, lam, p, bias = layer(*spec, with_bias=True)
    _, inv_o, wc, ws = oracle_prep(X, W, p, L.rank)
    d = DeviceLayer(X, p, bias, L.y_dtype)
    d.k1()
    d.k2()
    # the whole layer in one call must give the same bits as the two kernels
    Y2 = torch.empty_like(d.Y)
    ws_buf = torch.empty(sq.linear_workspace_bytes(L.M, L.K, p.rank), dtype=torch.uint8,
                         device="cuda")
    sq.linear(d.X, d.inv, d.L1p, d.L2t, p.rank, d.wc, d.ws, d.bias, Y2, ws_buf)
    torch.cuda.synchronize()
    Yg = d.Y.cpu().numpy()
    assert np.array_equal(Yg.view(np.uint8), Y2.cpu().numpy().view(np.uint8))
    assert np.all(np.isfinite(Yg))
    rows = sample_rows(L.M, seed=spec[0] * 100 + spec[1])
    Yo = oracle_rows(X, inv_o, p, wc, ws, bias, rows, L.y_dtype)
    err = rel_err(Yg[rows], Yo)
    assert err <= TOL_Y, err
    Ye, env, jump = oracle_rows_exact(X, inv_o, p, wc, ws, bias, rows)
    assert_y_strict(Yg[rows], Ye, env, jump, L.y_dtype, L.K // 64, p.rank)


# small and ragged shapes, compared on every element
EDGE = [
    # M, K, N, R, x_dtype, y_dtype, bias
    (1, 64, 1, 0, "f32", "f32", True),
    (17, 128, 130, 16, "f16", "f16", True),
    (129, 192, 257, 48, "f16", "f32", False),
    (200, 320, 320, 32, "f32", "f16", True),
    (64, 1024, 512, 256, "f16", "f16", True),
    (300, 640, 136, 80, "f16", "f16", False),
    (33, 64, 600, 16, "f32", "f16", True),
    # ranks whose column-block count (7, 9) has no kernel of its own
    (50, 256, 200, 112, "f16", "f16", True),
    (40, 384, 150, 144, "f32", "f16", False),
]


def _edge_inputs(M, K, N, R, xdt, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    X[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20
    X = X.astype(np.float16 if xdt == "f16" else np.float32)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    W[rng.choice(K, max(1, K // 100), replace=False)] *= 10
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    return X, W, b


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "x".join(map(str, c[:4])) + f"_{c[4]}_{c[5]}")
def test_edge_shapes_every_element(case):
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K, N, R, xdt, ydt, use_bias = case
    X, W, b = _edge_inputs(M, K, N, R, xdt, seed=M * 31 + K + N + R)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, R)
    bias = b if use_bias else None
    _, inv_o, wc, ws = oracle_prep(X, W, p)
    d = DeviceLayer(X, p, bias, ydt)
    d.k1()
    d.k2()
    torch.cuda.synchronize()
    a_codes, a_scales, xh = O.quantize_activation(X, inv_o)
    assert np.array_equal(d.a_codes.cpu().numpy(), a_codes)
    assert np.array_equal(host_u16(d.a_scales), a_scales.view(np.uint16))
    Yo = O.linear(X, inv_o, p.L1, p.L2, wc, ws, bias, ydt)
    err = rel_err(d.Y.cpu().numpy(), Yo)
    assert err <= TOL_Y, err
    Ye, env, jump = oracle_rows_exact(X, inv_o, p, wc, ws, bias, np.arange(M))
    assert_y_strict(d.Y.cpu().numpy(), Ye, env, jump, ydt, K // 64, R)
    P = torch.empty((M, N, K // 64), dtype=torch.int32, device="cuda")
    sq.debug_group_partials(d.a_codes, d.wc, M, N, K, 0, M, P)
    torch.cuda.synchronize()
    assert np.array_equal(P.cpu().numpy(), O.group_partials(a_codes, wc).astype(np.int32))


def test_strided_buffers_and_canaries():
    """ldx > K and ldy > N: padding columns of X are ignored and those of Y untouched."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K, N, R = 70, 256, 100, 32
    X, W, b = _edge_inputs(M, K, N, R, "f16", seed=5)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, R)
    _, inv_o, wc, ws = oracle_prep(X, W, p)
    Xpad = np.full((M, K + 64), np.float16(1000.0), dtype=np.float16)
    Xpad[:, :K] = X
    Xd = dev(Xpad)[:, :K]
    Ybig = torch.full((M + 2, N + 28), -7.0, dtype=torch.float16, device="cuda")
    Y = Ybig[1:M + 1, :N]                     # row stride N + 28 (16-byte multiple)
    wsb = torch.empty(sq.linear_workspace_bytes(M, K, R), dtype=torch.uint8, device="cuda")
    sq.linear(Xd, dev(p.inv_smooth), dev(p.L1p), dev(p.L2t), R, dev(p.w_codes), dev(p.w_scales),
              dev(b), Y, wsb)
    torch.cuda.synchronize()
    Yb = Ybig.cpu().numpy()
    assert np.all(Yb[0] == -7.0) and np.all(Yb[M + 1] == -7.0) and np.all(Yb[:, N:] == -7.0)
    Yo = O.linear(X, inv_o, p.L1, p.L2, wc, ws, b, "f16")
    assert rel_err(Yb[1:M + 1, :N], Yo) <= TOL_Y


def test_zero_activation_rows():
    """All-zero groups give zero scales and codes; output is the bias plus the branch (0)."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K, N, R = 48, 192, 64, 16
    X, W, b = _edge_inputs(M, K, N, R, "f16", seed=8)
    X[5] = 0
    X[:, 64:128] = 0
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, R)
    _, inv_o, wc, ws = oracle_prep(X, W, p)
    d = DeviceLayer(X, p, b, "f32")
    d.k1()
    d.k2()
    torch.cuda.synchronize()
    s = host_u16(d.a_scales)
    assert np.all(s[5] == 0) and np.all(s[:, 1] == 0)
    assert np.all(d.a_codes.cpu().numpy()[5] == 0)
    Y = d.Y.cpu().numpy()
    assert np.array_equal(Y[5], b)
    assert rel_err(Y, O.linear(X, inv_o, p.L1, p.L2, wc, ws, b, "f32")) <= TOL_Y


def test_lora_adds_exactly_its_term():
    """The LoRA-merged DiT layer: Y(L1', L2') - Y(L1, L2) = X.A.B up to the fp16 roundings
    of the branch, checked on the difference itself (the term is small next to Y)."""
    torch = torch_mod()
    L, X, W, lam, p_lora, _ = layer(4, 0)
    _, _, _, _, p_base, _ = layer(4, 0, use_lora=False)
    A, B = wl.lora(4, 0, L.K, L.N, L.lora_rank)
    outs = []
    for p in (p_base, p_lora):
        d = DeviceLayer(X, p, None, "f32")
        d.k1()
        d.k2()
        torch.cuda.synchronize()
        outs.append(d.Y.cpu().numpy().astype(np.float64))
    assert np.array_equal(p_base.w_codes, p_lora.w_codes)
    rows = sample_rows(L.M, seed=3, n_random=32)
    delta = outs[1][rows] - outs[0][rows]
    ref = X[rows].astype(np.float64) @ A.astype(np.float64) @ B.astype(np.float64)
    env = np.abs(X[rows].astype(np.float64)) @ np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    # three fp16 roundings in the branch, fp32 sums, and the fp32 rounding of two outputs
    bound = 3.2 * 2.0 ** -11 * env + 2.0 ** -21 * (np.abs(outs[0][rows]) + np.abs(outs[1][rows])) \
        + L.K * 2.0 ** -23 * env
    assert np.all(np.abs(delta - ref) <= bound)
    assert np.max(np.abs(ref)) > 0.01


def test_gelu_within_one_ulp():
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    L = wl.CONFIGS[2].layers[1]
    Z = wl.preactivation(2, 1, 1024, L.K)
    Zf = Z.reshape(-1)
    n = Zf.size - 3                                    # ragged length: vector body + tail
    x = dev(Zf)
    y = torch.full_like(x, 65504.0)                   # canary bits 0x7BFF
    sq.gelu_tanh_f16(x[:n], y[:n])
    torch.cuda.synchronize()
    got = host_u16(y)[:n].astype(np.int32)
    ref = O.gelu_tanh(Zf[:n]).view(np.uint16).astype(np.int32)
    # compare as ordered integers: sign-magnitude fp16 bits -> monotone integers
    def ordered(h):
        return np.where(h & 0x8000, -(h & 0x7FFF), h)
    assert np.max(np.abs(ordered(got) - ordered(ref))) <= 1
    assert np.all(host_u16(y)[n:] == 0x7BFF)


TOL_CHAIN = 1e-2


def test_dit_mlp_chain():
    """Up-projection -> GELU -> down-projection on the GPU against the same chain in
    the oracle, on sampled rows. The down layer is calibrated offline on the seeded
    GELU input of the MLP workload. Each layer on its own is held to 2e-3 above;
    here the intermediate H agrees with the oracle's only to about one fp16 ulp
    (fp32 against fp64 accumulation, then GELU), and the down layer quantizes H
    again, so a code whose value sits near a rounding boundary can move by one
    step (up to s_x*s_w*|q_w| per flip). Two layers with re-quantization in
    between are therefore held to 1e-2 of max|Y|."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    Lu, X, Wu, _, pu, _ = layer(2, 0)
    Ld, Xd_cal, Wd, _, pd, _ = layer(2, 1)
    rows = np.arange(0, Lu.M, 97)[:48]
    _, inv_u, wcu, wsu = oracle_prep(X, Wu, pu, Lu.rank)
    _, inv_d, wcd, wsd = oracle_prep(Xd_cal, Wd, pd, Ld.rank)
    Hu = O.gelu_tanh(oracle_rows(X, inv_u, pu, wcu, wsu, None, rows, "f16"))
    Yo = oracle_rows(Hu, inv_d, pd, wcd, wsd, None, np.arange(len(rows)), "f16")
    up = sq.Linear(pu)
    down = sq.Linear(pd)
    H = up(dev(X))
    sq.gelu_tanh_f16(H, H)
    Yd = down(H)
    torch.cuda.synchronize()
    assert rel_err(Yd.cpu().numpy()[rows], Yo) <= TOL_CHAIN


def test_fused_gelu_epilogue():
    """K2 with the GELU of a DiT MLP's first layer fused into its epilogue, on the
    MLP up-projection (sampled rows): GELU(Y) against the oracle's GELU of the
    unrounded Y. Besides the 2e-3 bound: one fp16 step of the result, plus the
    layer's own bound (see assert_y_strict) times GELU's largest slope (< 1.13),
    plus the fp32 evaluation of GELU itself (a few roundings inside exp's
    argument, each amplified at most |v|/4)."""
    torch = torch_mod()
    L, X, W, lam, p, bias = layer(2, 0, with_bias=True)
    _, inv_o, wc, ws = oracle_prep(X, W, p, L.rank)
    d = DeviceLayer(X, p, bias, L.y_dtype)
    d.k1()
    import bit_post_quantized_smooth_amd as sq
    sq.w4a4_gemm_lowrank_up(d.a_codes, d.a_scales, d.wc, d.ws, d.D, d.L2t, d.R, d.bias, d.Y, d.K,
                            activation="gelu_tanh")
    torch.cuda.synchronize()
    Yg = d.Y.cpu().numpy().astype(np.float64)
    rows = sample_rows(L.M, seed=7)[:40]
    Go = np.concatenate([O.linear(X[rows[i:i + 8]], inv_o, p.L1, p.L2, wc, ws, bias, "f16",
                                  activation="gelu_tanh") for i in range(0, len(rows), 8)])
    assert rel_err(Yg[rows], Go) <= TOL_Y
    Ye, env, jump = oracle_rows_exact(X, inv_o, p, wc, ws, bias, rows)
    G = L.K // 64
    tol_y = (G + p.rank / 16 + 4) * 2.0 ** -24 * env + jump
    Ge = O.gelu_tanh_f64(Ye)
    step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(Ge), 2.0 ** -14))) - 10), 2.0 ** -24)
    tol = step + 1.13 * tol_y + 2.0 ** -18 * (1.0 + np.abs(Ye) ** 3)
    ratio = np.abs(Yg[rows] - Ge) / tol
    assert float(ratio.max()) <= 1.0, (int(np.count_nonzero(ratio > 1)), float(ratio.max()))
    assert np.min(Yg[rows]) >= -0.2      # GELU's minimum is about -0.17


def test_dit_mlp_chain_fused_gelu():
    """The MLP chain with the GELU fused into the up-projection's epilogue: the
    intermediate is written once, in fp16, already activated. Same tolerance as
    the unfused chain."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    Lu, X, Wu, _, pu, _ = layer(2, 0)
    Ld, Xd_cal, Wd, _, pd, _ = layer(2, 1)
    rows = np.arange(0, Lu.M, 97)[:48]
    _, inv_u, wcu, wsu = oracle_prep(X, Wu, pu, Lu.rank)
    _, inv_d, wcd, wsd = oracle_prep(Xd_cal, Wd, pd, Ld.rank)
    Hu = np.concatenate([O.linear(X[rows[i:i + 16]], inv_u, pu.L1, pu.L2, wcu, wsu, None, "f16",
                                  activation="gelu_tanh") for i in range(0, len(rows), 16)])
    Yo = oracle_rows(Hu, inv_d, pd, wcd, wsd, None, np.arange(len(rows)), "f16")
    up = sq.Linear(pu, activation="gelu_tanh")
    down = sq.Linear(pd)
    Yd = down(up(dev(X)))
    torch.cuda.synchronize()
    assert rel_err(Yd.cpu().numpy()[rows], Yo) <= TOL_CHAIN


def test_repeatable_and_any_stream():
    """Same inputs -> same bits, also on a side stream."""
    torch = torch_mod()
    L, X, W, lam, p, bias = layer(0, 0, with_bias=True)
    d = DeviceLayer(X, p, bias, "f32")
    d.k1()
    d.k2()
    torch.cuda.synchronize()
    y1 = d.Y.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        d.Y.zero_()
        d.k1()
        d.k2()
    s.synchronize()
    assert torch.equal(y1, d.Y)
