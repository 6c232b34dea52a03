"""The Python binding's argument checks, on the CPU.

The device kernels trust the sizes they are given, so the binding compares
every tensor with the others before the library call: a weight buffer of the
wrong size, an output of the wrong shape, a strided inner dimension, an fp16
bias or a CPU tensor must raise, not reach a kernel. The checks run in that
order (shapes, dtypes and strides first, the device last), so with CPU tensors
a correct call stops exactly at the device check."""
import pytest

torch = pytest.importorskip("torch")
sq = pytest.importorskip("bit_post_quantized_smooth_amd")

M, K, N, R = 40, 128, 48, 16
G = K // 64
u8, i16, f16, f32 = torch.uint8, torch.int16, torch.float16, torch.float32


def z(*shape, dtype):
    return torch.zeros(*shape, dtype=dtype)


def k2_args(**over):
    a = dict(a_codes=z(M, K // 2, dtype=u8), a_scales=z(M, G, dtype=i16),
             w_codes=z(N, K // 2, dtype=u8), w_scales=z(N, G, dtype=i16), D=z(M, R, dtype=f32),
             L2t=z(N, R, dtype=i16), R=R, bias=z(N, dtype=f32), Y=z(M, N, dtype=f16), K=K)
    a.update(over)
    return a


def k1_args(**over):
    a = dict(X=z(M, K, dtype=f16), inv_smooth=z(K, dtype=f32), L1p=z(R * K, dtype=i16), R=R,
             a_codes=z(M, K // 2, dtype=u8), a_scales=z(M, G, dtype=i16), D=z(M, R, dtype=f32))
    a.update(over)
    return a


def lin_args(**over):
    ws = z(sq.linear_workspace_bytes(M, K, R), dtype=u8)
    a = dict(X=z(M, K, dtype=f16), inv_smooth=z(K, dtype=f32), L1p=z(R * K, dtype=i16),
             L2t=z(N, R, dtype=i16), R=R, w_codes=z(N, K // 2, dtype=u8),
             w_scales=z(N, G, dtype=i16), bias=z(N, dtype=f32), Y=z(M, N, dtype=f16), ws=ws)
    a.update(over)
    return a


def test_correct_cpu_arguments_stop_at_the_device_check():
    for f, a in ((sq.w4a4_gemm_lowrank_up, k2_args()), (sq.quantize_act_lowrank_down, k1_args()),
                 (sq.linear, lin_args())):
        with pytest.raises(ValueError, match="GPU"):
            f(**a)


@pytest.mark.parametrize("over,match", [
    (dict(w_codes=z(N, K // 2 - 16, dtype=u8)), "w_codes"),           # weights of another K
    (dict(w_scales=z(N + 1, G, dtype=i16)), "w_scales"),               # weights of another N
    (dict(L2t=z(N, R + 16, dtype=i16)), "L2t"),                        # another rank
    (dict(bias=z(N, dtype=f16)), "bias"),                              # fp16 bias
    (dict(bias=z(N + 3, dtype=f32)), "bias"),                          # bias of another N
    (dict(a_codes=z(M - 1, K // 2, dtype=u8)), "a_codes"),             # activation codes too short
    (dict(a_scales=z(M, G - 1, dtype=i16)), "a_scales"),
    (dict(D=z(M, R - 1, dtype=f32)), "D"),
    (dict(Y=z(M, 2 * N, dtype=f16)[:, ::2]), "inner stride"),          # strided columns
    (dict(Y=z(M, N, dtype=torch.float64)), "Y"),                       # unsupported output type
    (dict(K=K + 32), "multiple of 64"),
    (dict(a_codes=z(M, K // 2, dtype=f32)), "a_codes"),                # wrong element type
])
def test_k2_mismatches_raise(over, match):
    with pytest.raises((ValueError, TypeError), match=match):
        sq.w4a4_gemm_lowrank_up(**k2_args(**over))


@pytest.mark.parametrize("over,match", [
    (dict(X=z(M, K + 64, dtype=f16)), "inv_smooth"),                   # X of another K
    (dict(L1p=z(R * K - 8, dtype=i16)), "L1p"),
    (dict(a_scales=z(M - 2, G, dtype=i16)), "a_scales"),
    (dict(X=z(M, 2 * K, dtype=f16)[:, ::2]), "inner stride"),
    (dict(inv_smooth=z(K, dtype=f16)), "inv_smooth"),
])
def test_k1_mismatches_raise(over, match):
    with pytest.raises((ValueError, TypeError), match=match):
        sq.quantize_act_lowrank_down(**k1_args(**over))


@pytest.mark.parametrize("over,match", [
    (dict(X=z(M, K + 64, dtype=f16)), "inv_smooth"),
    (dict(Y=z(M + 1, N, dtype=f16)), "Y"),
    (dict(Y=z(M, N + 8, dtype=f16)), "w_codes"),                       # wider Y than the weights
    (dict(ws=z(64, dtype=u8)), "ws"),
    (dict(bias=z(N, dtype=f16)), "bias"),
])
def test_linear_mismatches_raise(over, match):
    with pytest.raises((ValueError, TypeError), match=match):
        sq.linear(**lin_args(**over))


def test_mx_and_conv_and_gelu_mismatches_raise():
    ct, et = sq.mx_codes_tiled_bytes(N, K), sq.mx_exps_tiled_bytes(N, K)
    with pytest.raises(ValueError, match="w_codes_t"):
        sq.mx_gemm_lowrank_up(z(sq.mx_codes_tiled_bytes(M, K), dtype=u8),
                              z(sq.mx_exps_tiled_bytes(M, K), dtype=u8), z(ct - 1024, dtype=u8),
                              z(et, dtype=u8), None, None, 0, None, z(M, N, dtype=f16), K)
    X = z(2, 8, 8, 64, dtype=f16)
    Kc = 9 * 64
    ws = z(sq.linear_workspace_bytes(128, Kc, 0), dtype=u8)
    with pytest.raises(ValueError, match="Y"):
        sq.conv2d(X, 3, 3, 1, 1, z(Kc, dtype=f32), None, None, 0, z(N, Kc // 2, dtype=u8),
                  z(N, Kc // 64, dtype=i16), None, z(2, 8, 7, N, dtype=f16), ws)
    with pytest.raises(ValueError, match="y"):
        sq.gelu_tanh_f16(z(100, dtype=f16), z(99, dtype=f16))
