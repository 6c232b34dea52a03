"""Bit-exact integer partials of the GEMM kernels themselves, read through Y.

The int32 per-group partial sums P[m,n,g] = sum over k in group g of
qx[m,k] * qw[n,k] are the integer core of the W4A4 layer (SVDQuant abstract on
ai-digest.ru: both operands at 4 bits; chattools.cn overview, section
"SVDQuant的主要功能", quantization item). K2 never stores them: it rescales
each one by s_x[m,g] * s_w[n,g] in fp32 and sums over g. With scales that are
powers of two every step of that rescale is exact, so Y shows P itself:

* one-hot: s_x = 2^-(m % 3) and s_w = 2^-(n % 5) on group g, 0 on every other
  group, so Y[m,n] = P[m,n,g] * 2^-(m%3 + n%5) exactly (P has at most 12 bits);
* uniform: s_x = s_w = 2^-4 on every group, so 256 * Y = sum_g P[m,n,g]
  exactly (|sum| < 2^24 for K <= 12288).

These run svdq_w4a4_gemm_lowrank_up (rank 0, no bias, fp32 Y) on the oracle's
codes, at the full sizes of every workload and on ragged edge shapes, so the
loader, the LDS layout, the software pipeline, the banded tile order, the
quarter tiles of the last round and the M/N tails are all on the path. Y is
NaN-filled first and written with a row stride past N; the padding columns
must keep their canary.

The MXFP4 GEMM has no integer partials (its matrix core sums E2M1 products in
fp32); with every E8M0 exponent at 127 (or one of 126..128 while K is small
enough) the products are multiples of 1/16 and the sums stay below 2^24 units,
so its Y is exact too and is compared bit for bit with the oracle's
dequantized product."""
import numpy as np
import pytest

import oracle as O
import mx_tiles as T
from gpu_common import dev, layer, oracle_prep, torch_mod
from test_gpu_parity import EDGE, SPECS, _edge_inputs, _ids

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_post_quantized_smooth_amd  # noqa: F401  (raises if the library is missing)


def _codes(X, W, p, base_rank):
    """The oracle's activation and residual codes for this layer."""
    _, inv_o, wc, _ = oracle_prep(X, W, p, base_rank)
    a_codes, _, _ = O.quantize_activation(X, inv_o)
    return a_codes, wc


def _f16_bits(v):
    return np.asarray(v, dtype=np.float16).view(np.uint16)


def _run_k2(a_codes, w_codes, sx, sw, M, N, K, pad=3):
    """K2 at rank 0 with the given fp16 scales; returns Y (fp32, M x N) after
    checking the canary columns of a row stride N + pad."""
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    Ybig = torch.full((M, N + pad), float("nan"), dtype=torch.float32, device="cuda")
    Ybig[:, N:] = -3.0
    Y = Ybig[:, :N]
    sq.w4a4_gemm_lowrank_up(dev(a_codes), dev(_f16_bits(sx)), dev(w_codes), dev(_f16_bits(sw)),
                            None, None, 0, None, Y, K)
    torch.cuda.synchronize()
    Yh = Ybig.cpu().numpy()
    assert np.all(Yh[:, N:] == -3.0), "K2 wrote past column N"
    return Yh[:, :N]


def _onehot_scales(M, N, G, g):
    sx = np.zeros((M, G), dtype=np.float16)
    sw = np.zeros((N, G), dtype=np.float16)
    sx[:, g] = np.exp2(-(np.arange(M) % 3))
    sw[:, g] = np.exp2(-(np.arange(N) % 5))
    return sx, sw


def _check_onehot(a_codes, w_codes, M, N, K, groups):
    G = K // 64
    for g in groups:
        sx, sw = _onehot_scales(M, N, G, g)
        Y = _run_k2(a_codes, w_codes, sx, sw, M, N, K)
        sl = slice(32 * g, 32 * (g + 1))                 # group g's 32 bytes of packed codes
        P = O.group_partials(a_codes[:, sl], w_codes[:, sl])[:, :, 0].astype(np.float64)
        ref = P * np.exp2(-(np.arange(M) % 3))[:, None] * np.exp2(-(np.arange(N) % 5))[None, :]
        bad = np.count_nonzero(Y.astype(np.float64) != ref)
        assert bad == 0, f"group {g}: {bad} of {M * N} outputs differ"


def _check_uniform(a_codes, w_codes, M, N, K):
    G = K // 64
    s = np.full((M, G), 2.0 ** -4, dtype=np.float16)
    t = np.full((N, G), 2.0 ** -4, dtype=np.float16)
    Y = _run_k2(a_codes, w_codes, s, t, M, N, K)
    # the sum over all groups: the oracle's partials with one group spanning K
    Psum = O.group_partials(a_codes, w_codes, group=K)[:, :, 0].astype(np.float64)
    bad = np.count_nonzero(Y.astype(np.float64) * 256.0 != Psum)
    assert bad == 0, f"{bad} of {M * N} outputs differ"


@pytest.mark.parametrize("spec", SPECS, ids=_ids)
def test_k2_partials_bit_exact(spec):
    L, X, W, lam, p, _ = layer(*spec)
    a_codes, wc = _codes(X, W, p, L.rank)
    G = L.K // 64
    _check_onehot(a_codes, wc, L.M, L.N, L.K, sorted({0, 1 % G, G // 2, G - 1}))
    _check_uniform(a_codes, wc, L.M, L.N, L.K)


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "x".join(map(str, c[:3])))
def test_k2_partials_edge_shapes(case):
    M, K, N, R, xdt, _, _ = case
    X, W, _ = _edge_inputs(M, K, N, R, xdt, seed=M * 31 + K + N + R)
    rng = np.random.default_rng(M + 7 * N)
    # random codes in [-7, 7] on both sides (every code value, both signs)
    a_codes = O.pack_nibbles(rng.integers(-7, 8, size=(M, K)))
    w_codes = O.pack_nibbles(rng.integers(-7, 8, size=(N, K)))
    G = K // 64
    _check_onehot(a_codes, w_codes, M, N, K, sorted({0, G - 1}))
    _check_uniform(a_codes, w_codes, M, N, K)


@pytest.mark.parametrize("sign", [1, -1])
def test_k2_partials_extreme_codes(sign):
    """Every code at +-7 on both sides: each partial is +-3136 (the largest), the
    sum over 192 groups +-602112: the seeded accumulator and the fp32 sum stay exact."""
    M, K, N = 130, 12288, 200
    a_codes = O.pack_nibbles(np.full((M, K), 7))
    w_codes = O.pack_nibbles(np.full((N, K), 7 * sign))
    _check_onehot(a_codes, w_codes, M, N, K, [0, 191])
    _check_uniform(a_codes, w_codes, M, N, K)


MX_SPECS = [(0, 0), (1, 0), (2, 1), (3, 0), (3, 4), (4, 0)]


@pytest.mark.parametrize("spec", MX_SPECS, ids=_ids)
def test_k2_mx_products_bit_exact(spec):
    """K2-MX with power-of-two block exponents near 1: Y = the exact product of the
    dequantized codes, compared bit for bit (oracle MXFP4 codes on both sides)."""
    import bit_post_quantized_smooth_amd as sq
    from test_gpu_mx import _mx_layer
    torch = torch_mod()
    L, X, W, lam, p = _mx_layer(*spec)
    M, K, N = L.M, L.K, L.N
    lam_o = O.smoothing_factors(O.channel_absmax(X), W)
    a_codes, _, _ = O.mx_quantize_activation(X, O.inv_smoothing(lam_o))
    wc, _ = O.mx_quantize_residual_from_factors(W, lam_o, p.L1[:, :L.rank], p.L2[:L.rank])
    rng = np.random.default_rng(spec[0] * 10 + spec[1])
    if K <= 6144:      # products are multiples of 1/16 up to 144: sums exact below 2^24 units
        ae = rng.integers(126, 129, size=(M, K // 32)).astype(np.uint8)
        we = rng.integers(126, 129, size=(N, K // 32)).astype(np.uint8)
    else:
        ae = np.full((M, K // 32), 127, dtype=np.uint8)
        we = np.full((N, K // 32), 127, dtype=np.uint8)
    Ybig = torch.full((M, N + 5), float("nan"), dtype=torch.float32, device="cuda")
    Ybig[:, N:] = -3.0
    sq.mx_gemm_lowrank_up(dev(T.tile_codes(a_codes, K)), dev(T.tile_exps(ae, K)),
                          dev(T.tile_codes(wc, K)), dev(T.tile_exps(we, K)), None, None, 0, None,
                          Ybig[:, :N], K)
    torch.cuda.synchronize()
    Yh = Ybig.cpu().numpy()
    assert np.all(Yh[:, N:] == -3.0), "K2-MX wrote past column N"
    A = O.mx_dequantize_blocks(O.unpack_codes4(a_codes), ae)
    B = O.mx_dequantize_blocks(O.unpack_codes4(wc), we)
    ref = A @ B.T
    bad = np.count_nonzero(Yh[:, :N].astype(np.float64) != ref)
    assert bad == 0, f"{bad} of {M * N} outputs differ"
