"""The layer captured in a HIP graph and replayed: a serving loop issues the
pre-kernel and the GEMM as one graph launch instead of one host call per
kernel. Every entry point on the step's path launches its kernels on the
caller's stream with no allocation, no memset and no synchronization, so the
graph holds only the kernels. Each test replays the graph several times, with
eager work on the same stream and synchronizations between the replays, after
refilling every output with garbage, and checks every replay bit for bit
against the eager result of the same calls."""
import pytest

from gpu_common import layer, torch_mod
from test_gpu_tiled import TiledLayer

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_post_quantized_smooth_amd  # noqa: F401  (raises if the library is missing)


def _bits(t):
    torch = torch_mod()
    return t.view(torch.int16 if t.dtype == torch.float16 else torch.int32).clone()


def _replay_and_check(step, outputs, refill):
    """Capture step() once, then replay it REPLAYS times; before each replay
    refill the outputs, run unrelated eager work, synchronize; after it compare
    every output with its eager bits."""
    torch = torch_mod()
    step()
    torch.cuda.synchronize()
    ref = [_bits(o) for o in outputs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    a = torch.randn(256, 256, device="cuda")
    for rep in range(REPLAYS):
        refill()
        b = a @ a                                  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        c = b.sum()                                # and behind the replay
        torch.cuda.synchronize()
        assert bool(torch.isfinite(c))
        for o, r in zip(outputs, ref):
            assert torch.equal(_bits(o), r), f"replay {rep} differs from the eager result"
    del g


@pytest.mark.parametrize("spec", [(0, 0), (3, 1), (4, 0)], ids=lambda s: f"c{s[0]}l{s[1]}")
def test_tiled_kernels_replay_in_a_graph(spec):
    torch = torch_mod()
    L, X, W, lam, p, bias = layer(*spec, with_bias=True)
    d = TiledLayer(X, p, bias, L.y_dtype)

    def step():
        d.k1()
        d.k2()

    def refill():
        d.ops.fill_(0x5A)
        d.scales.fill_(float("nan"))
        d.D.fill_(-1)
        d.Y.fill_(float("nan"))

    outs = [d.Y, d.scales] + ([d.D] if p.rank else [])
    _replay_and_check(step, outs, refill)
    assert bool(torch.all(torch.isfinite(d.Y.float())))


@pytest.mark.parametrize("spec", [(1, 0), (3, 0)], ids=lambda s: f"c{s[0]}l{s[1]}")
def test_fused_tiled_entry_replays_in_a_graph(spec):
    import bit_post_quantized_smooth_amd as sq
    torch = torch_mod()
    L, X, W, lam, p, bias = layer(*spec, with_bias=True)
    d = TiledLayer(X, p, bias, L.y_dtype)
    ws = torch.empty(sq.linear_tiled_workspace_bytes(L.M, L.K, p.rank), dtype=torch.uint8,
                     device="cuda")

    def step():
        sq.linear_tiled(d.X, d.inv, d.L1p, d.L2t, p.rank, d.wc, d.ws, d.bias, d.Y, ws)

    def refill():
        ws.fill_(0xA5)
        d.Y.fill_(float("nan"))

    _replay_and_check(step, [d.Y], refill)


@pytest.mark.parametrize("spec", [(0, 0), (3, 2)], ids=lambda s: f"c{s[0]}l{s[1]}")
def test_canonical_entry_replays_in_a_graph(spec):
    import bit_post_quantized_smooth_amd as sq
    from gpu_common import dev
    torch = torch_mod()
    L, X, W, lam, p, bias = layer(*spec, with_bias=True)
    Xd, inv = dev(X), dev(p.inv_smooth)
    L1p = dev(p.L1p) if p.rank else None
    L2t = dev(p.L2t) if p.rank else None
    wc, wsc = dev(p.w_codes), dev(p.w_scales)
    bd = dev(bias)
    Y = torch.empty((L.M, L.N), dtype=torch.float16 if L.y_dtype == "f16" else torch.float32,
                    device="cuda")
    ws = torch.empty(sq.linear_workspace_bytes(L.M, L.K, p.rank), dtype=torch.uint8,
                     device="cuda")

    def step():
        sq.linear(Xd, inv, L1p, L2t, p.rank, wc, wsc, bd, Y, ws)

    def refill():
        ws.fill_(0xA5)
        Y.fill_(float("nan"))

    _replay_and_check(step, [Y], refill)


@pytest.mark.parametrize("shape", [(4100, 6144, 256, 16), (2000, 4096, 600, 32)],
                         ids=["k1_split_long_rows", "k2_split_along_k"])
def test_split_paths_replay_in_a_graph(shape):
    """The split pre-kernel (long rows) and the GEMM split along K (a quarter-
    filled long-K grid) each launch a second, reducing kernel; captured with
    their workspaces, they replay to the eager bits."""
    import bit_post_quantized_smooth_amd as sq
    from test_gpu_parity import _edge_inputs
    M, K, N, R = shape
    X, W, b = _edge_inputs(M, K, N, R, "f16", seed=M + K)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, R)
    d = TiledLayer(X, p, b, "f16", k1_workspace=True, k2_workspace=True)
    assert (sq.quantize_act_workspace_bytes(M, K, R) > 0) or (sq.gemm_tiled_workspace_bytes(M, N, K) > 0)

    def step():
        d.k1()
        d.k2()

    def refill():
        d.ops.fill_(0x5A)
        d.scales.fill_(float("nan"))
        d.D.fill_(-1)
        d.Y.fill_(float("nan"))
        d.k1ws.fill_(0xA5)
        d.k2ws.fill_(0xA5)

    _replay_and_check(step, [d.Y, d.scales, d.D], refill)
