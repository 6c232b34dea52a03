"""svdq_linear_noalloc, the entry point for callers that cannot allocate
device memory, against svdq_linear (the same layer with a caller workspace).

Both run the same kernels, so their outputs must agree bit for bit; the
layer is also held to the oracle's 2e-3 bound on sampled rows. Three calls in
a row share the library's static buffer: the DiT QKV layer in full, then the
first 777 rows of it, then a small ragged layer with bias, GELU and fp32
output, so the later, smaller calls run over what the earlier ones left in
the buffer."""
import numpy as np
import pytest

import oracle as O
from gpu_common import TOL_Y, dev, layer, oracle_prep, rel_err, sample_rows, torch_mod
from test_gpu_parity import _edge_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_post_quantized_smooth_amd  # noqa: F401  (raises if the library is missing)


def _run_both(X, p, bias, y_dtype, activation=None):
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    M, K = X.shape
    N, R = p.N, p.rank
    yt = torch.float16 if y_dtype == "f16" else torch.float32
    Xd, inv = dev(X), dev(p.inv_smooth)
    L1p = dev(p.L1p) if R else None
    L2t = dev(p.L2t) if R else None
    wc, ws = dev(p.w_codes), dev(p.w_scales)
    b = dev(bias) if bias is not None else None
    Y_ref = torch.full((M, N), float("nan"), dtype=yt, device="cuda")
    wsb = torch.empty(sq.linear_workspace_bytes(M, K, R), dtype=torch.uint8, device="cuda")
    sq.linear(Xd, inv, L1p, L2t, R, wc, ws, b, Y_ref, wsb, activation=activation)
    Y = torch.full((M, N), float("nan"), dtype=yt, device="cuda")
    sq.linear_noalloc(Xd, inv, L1p, L2t, R, wc, ws, b, Y, activation=activation)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), Y_ref.cpu().numpy()


def test_noalloc_matches_linear_on_successive_calls():
    L, X, W, lam, p, bias = layer(1, 0, with_bias=True)
    _, inv_o, wc, ws = oracle_prep(X, W, p, L.rank)
    for rows in (L.M, 777):
        Xr = np.ascontiguousarray(X[:rows])
        Y, Y_ref = _run_both(Xr, p, bias, "f16")
        assert np.array_equal(Y.view(np.uint16), Y_ref.view(np.uint16)), rows
        r = sample_rows(rows, seed=rows, n_random=24)
        Yo = np.concatenate([O.linear(Xr[r[i:i + 16]], inv_o, p.L1, p.L2, wc, ws, bias, "f16")
                             for i in range(0, len(r), 16)])
        assert rel_err(Y[r], Yo) <= TOL_Y
    # a third, smaller layer of another shape: ragged M and N, fp32 out, GELU
    import bit_post_quantized_smooth_amd as sq
    M, K, N, R = 300, 640, 136, 80
    X2, W2, b2 = _edge_inputs(M, K, N, R, "f16", seed=11)
    lam2 = sq.smoothing_factors(sq.channel_absmax(X2), W2)
    p2 = sq.prepare_weights(W2, lam2, R)
    Y, Y_ref = _run_both(X2, p2, b2, "f32", activation="gelu_tanh")
    assert np.array_equal(Y.view(np.uint32), Y_ref.view(np.uint32))
    _, inv2, wc2, ws2 = oracle_prep(X2, W2, p2)
    Yo = O.linear(X2, inv2, p2.L1, p2.L2, wc2, ws2, b2, "f32", activation="gelu_tanh")
    assert rel_err(Y, Yo) <= TOL_Y
