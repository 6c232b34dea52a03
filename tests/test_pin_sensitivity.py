"""Plant a plausible mistake in the oracle (on the CPU) and show that at least
one pin catches it. Each mutation is undone by ``monkeypatch``."""
import numpy as np
import pytest

import oracle.svdq_ref as R
import pins


def _fails(checks):
    failed = []
    for c in checks:
        try:
            c(R)
        except AssertionError:
            failed.append(c.__name__)
    return failed


def _orig(name):
    return getattr(R, name)


def mut_scale_div8(mp):
    orig = _orig("quantize_groups")

    def q(v, group=64):
        return orig(np.asarray(v, dtype=np.float32) * np.float32(7.0 / 8.0), group)
    mp.setattr(R, "quantize_groups", q)


def mut_ties_away(mp):
    mp.setattr(R.np, "rint", lambda x: np.floor(np.abs(x) + 0.5) * np.sign(x), raising=True)


def mut_nibble_order(mp):
    def pack(q):
        q = np.asarray(q, dtype=np.int16)
        return ((q[..., 1::2] & 0xF) | ((q[..., 0::2] & 0xF) << 4)).astype(np.uint8)
    mp.setattr(R, "pack_nibbles", pack)


def mut_smoothing_inverted(mp):
    orig = _orig("smoothing_factors")
    mp.setattr(R, "smoothing_factors", lambda xa, W: (np.float32(1.0) / orig(xa, W)).astype(np.float32))


def mut_sigma_unsplit(mp):
    def f(U, S, Vt, r):
        return U[:, :r] * S[None, :r], Vt[:r, :].copy()
    mp.setattr(R, "lowrank_factors_f64", f)


def mut_smallest_singulars(mp):
    def f(U, S, Vt, r):
        if r == 0:
            return U[:, :0], Vt[:0, :]
        h = np.sqrt(S[-r:])
        return U[:, -r:] * h[None, :], h[:, None] * Vt[-r:, :]
    mp.setattr(R, "lowrank_factors_f64", f)


def mut_residual_sign(mp):
    mp.setattr(R, "residual", lambda What, L1, L2: np.asarray(What, np.float64) + (
        np.asarray(L1, np.float64) @ np.asarray(L2, np.float64)))


def mut_partials_group_shift(mp):
    orig = _orig("group_partials")

    def f(a, w, group=64):
        P = orig(a, w, group)
        return np.roll(P, 1, axis=2)
    mp.setattr(R, "group_partials", f)


def mut_drop_weight_scale(mp):
    def f(P, sx, sw):
        return np.einsum("mng,mg->mn", np.asarray(P, np.float64), np.asarray(sx, np.float64))
    mp.setattr(R, "scaled_group_sum", f)


def mut_drop_bias(mp):
    orig = _orig("finalize")
    mp.setattr(R, "finalize", lambda acc, lr, bias, od: orig(acc, lr, None, od))


def mut_down_no_f16(mp):
    mp.setattr(R, "down_projection", lambda xh, L1: np.asarray(xh, np.float64) @ np.asarray(L1, np.float64))


def mut_up_no_f16(mp):
    mp.setattr(R, "lowrank_up", lambda D, L2: np.asarray(D, np.float64) @ np.asarray(L2, np.float64))


def mut_lora_no_lambda(mp):
    orig = _orig("concat_lora")
    mp.setattr(R, "concat_lora", lambda L1, L2, lam, A, B, scale=1.0: orig(L1, L2, np.ones_like(lam), A, B, scale))


def mut_f16_via_f32(mp):
    mp.setattr(R, "to_f16", lambda x: np.asarray(x).astype(np.float32).astype(np.float16))


def mut_smooth_multiplies_lambda(mp):
    def f(X, inv):
        lam = (np.float32(1.0) / np.asarray(inv, np.float32)).astype(np.float32)
        return (np.asarray(X, np.float32) * lam[None, :]).astype(np.float32)
    mp.setattr(R, "smooth_activation", f)


def mut_transposed_weight_groups(mp):
    def f(Rm, group=64):
        q, s = R.quantize_groups(np.asarray(Rm, np.float32), group)   # groups along N, not K
        return R.pack_nibbles(q), s
    mp.setattr(R, "quantize_weight", f)


def mut_clamp_8(mp):
    orig_clip = np.clip
    mp.setattr(R.np, "clip", lambda a, lo, hi: orig_clip(a, -8, 8))


def mut_gelu_before_bias(mp):
    """The fused activation applied to the sum without the bias, bias added after."""
    orig = _orig("linear")

    def lin(X, inv, L1, L2, wc, ws, bias=None, out_dtype="f16", group=64, return_parts=False,
            activation=None):
        if activation != "gelu_tanh" or bias is None:
            return orig(X, inv, L1, L2, wc, ws, bias, out_dtype, group, return_parts, activation)
        y = orig(X, inv, L1, L2, wc, ws, None, "f32", group, False, None).astype(np.float64)
        y = R.gelu_tanh_f64(y) + np.asarray(bias, dtype=np.float64)[None, :]
        return y.astype(np.float16 if out_dtype == "f16" else np.float32)
    mp.setattr(R, "linear", lin)


def _mx_blocks_with(e_of_amax=None, round_fn=None, bias=127):
    """An MXFP4 block quantizer with one step replaced (the rest as the oracle's)."""
    def q(v32, block=32):
        v = np.asarray(v32, dtype=np.float32)
        sh = v.shape
        vb = v.reshape(sh[:-1] + (sh[-1] // block, block)).astype(np.float64)
        amax = np.max(np.abs(vb), axis=-1)
        if e_of_amax is None:
            e = np.where(amax > 0, np.frexp(amax)[1] - 3, -127)
        else:
            e = e_of_amax(amax)
        e = np.clip(e, -127, 127)
        codes = (round_fn or R.e2m1_round)(vb / np.ldexp(1.0, e)[..., None])
        return codes.reshape(sh), (e + bias).astype(np.uint8)
    return q


def mut_mx_ties_up(mp):
    """E2M1 midpoints rounded up (away from zero) instead of to the even code."""
    def rnd(x):
        m = np.abs(x)
        c = sum((m >= t).astype(np.int64) for t in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0))
        return (c + 8 * np.signbit(x)).astype(np.uint8)
    mp.setattr(R, "mx_quantize_blocks", _mx_blocks_with(round_fn=rnd))


def mut_mx_exponent_ceil(mp):
    """Shared exponent from ceil(log2 amax) instead of floor."""
    mp.setattr(R, "mx_quantize_blocks", _mx_blocks_with(
        e_of_amax=lambda a: np.where(a > 0, np.ceil(np.log2(np.where(a > 0, a, 1))) - 2, -127)
        .astype(np.int64)))


def mut_mx_exponent_nearest(mp):
    """Shared exponent rounded from log2(amax / 6) (amax mapped near 6, not floored)."""
    mp.setattr(R, "mx_quantize_blocks", _mx_blocks_with(
        e_of_amax=lambda a: np.where(a > 0, np.rint(np.log2(np.where(a > 0, a, 6) / 6)), -127)
        .astype(np.int64)))


def mut_mx_negative_zero_dropped(mp):
    """Negative values that round to zero get code 0 instead of the -0 code."""
    orig = _orig("e2m1_round")
    mp.setattr(R, "e2m1_round", lambda x: np.where(orig(x) == 8, 0, orig(x)).astype(np.uint8))


def mut_mx_bias_128(mp):
    """E8M0 stored with bias 128 (and read back the same way, so Y is unchanged)."""
    mp.setattr(R, "mx_quantize_blocks", _mx_blocks_with(bias=128))
    orig = _orig("mx_dequantize_blocks")
    mp.setattr(R, "mx_dequantize_blocks",
               lambda c, e8, block=32: orig(c, np.asarray(e8, np.int64) - 1, block))


def mut_mx_nibble_order(mp):
    def pack(c):
        c = np.asarray(c, dtype=np.uint8) & 15
        return (c[..., 1::2] | (c[..., 0::2] << 4)).astype(np.uint8)
    mp.setattr(R, "pack_codes4", pack)


def mut_mx_weight_blocks_along_n(mp):
    """R's 32-blocks taken along the output dimension instead of down K."""
    def f(W, lam32, L1, L2):
        R32 = R.to_f32(R.residual(R.smooth_weight(W, lam32), L1, L2))
        Np = -(-R32.shape[1] // 32) * 32
        pad = np.zeros((R32.shape[0], Np), dtype=np.float32)
        pad[:, :R32.shape[1]] = R32
        codes, _ = R.mx_quantize_blocks(pad)
        codes = codes[:, :R32.shape[1]].T
        _, e8 = R.mx_quantize_blocks(R32.T)
        return R.pack_codes4(codes), e8
    mp.setattr(R, "mx_quantize_residual_from_factors", f)


def mut_mx_unsmoothed_activation(mp):
    """The activation quantized before smoothing (X instead of Xhat)."""
    orig = _orig("mx_quantize_activation")
    mp.setattr(R, "mx_quantize_activation",
               lambda X, inv: orig(X, np.ones_like(np.asarray(inv, np.float32))))


def mut_w4a16_unrounded_dequant(mp):
    """The weight-only baseline's dequantized weights kept in fp64 (no fp16 rounding)."""
    def f(wc, ws, group=64):
        q = R.unpack_nibbles(wc).astype(np.float64)
        s = np.asarray(ws, dtype=np.float16).astype(np.float64)
        N, K = q.shape
        return (q.reshape(N, K // group, group) * s[:, :, None]).reshape(N, K)
    mp.setattr(R, "w4a16_dequant", f)


def mut_w4a16_scale_group_shift(mp):
    """Each group dequantized with its neighbour's scale."""
    orig = _orig("w4a16_dequant")
    mp.setattr(R, "w4a16_dequant",
               lambda wc, ws, group=64: orig(wc, np.roll(np.asarray(ws), 1, axis=1), group))


def mut_im2col_channel_major(mp):
    """Patch columns ordered (c, kh, kw) instead of (kh, kw, c)."""
    orig = _orig("im2col_nhwc")

    def f(X, KH, KW, stride, pad):
        cols = orig(X, KH, KW, stride, pad)
        C = np.asarray(X).shape[3]
        return cols.reshape(cols.shape[0], KH * KW, C).transpose(0, 2, 1).reshape(cols.shape[0], -1)
    mp.setattr(R, "im2col_nhwc", f)


def mut_im2col_no_padding_shift(mp):
    """Taps not shifted by the padding (output (oh, ow) reads from (oh + kh, ow + kw) - 0)."""
    orig = _orig("im2col_nhwc")

    def f(X, KH, KW, stride, pad):
        X = np.asarray(X)
        if pad == 0:
            return orig(X, KH, KW, stride, pad)
        Xs = np.zeros_like(X)
        Xs[:, pad:, pad:, :] = X[:, :X.shape[1] - pad, :X.shape[2] - pad, :]
        return orig(Xs, KH, KW, stride, pad)
    mp.setattr(R, "im2col_nhwc", f)


MUTATIONS = [mut_scale_div8, mut_ties_away, mut_nibble_order, mut_smoothing_inverted,
             mut_sigma_unsplit, mut_smallest_singulars, mut_residual_sign,
             mut_partials_group_shift, mut_drop_weight_scale, mut_drop_bias,
             mut_down_no_f16, mut_up_no_f16, mut_lora_no_lambda, mut_f16_via_f32,
             mut_smooth_multiplies_lambda, mut_transposed_weight_groups, mut_clamp_8,
             mut_gelu_before_bias, mut_mx_ties_up, mut_mx_exponent_ceil,
             mut_mx_exponent_nearest, mut_mx_negative_zero_dropped, mut_mx_bias_128,
             mut_mx_nibble_order, mut_mx_weight_blocks_along_n, mut_mx_unsmoothed_activation,
             mut_w4a16_unrounded_dequant, mut_w4a16_scale_group_shift,
             mut_im2col_channel_major, mut_im2col_no_padding_shift]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__)
def test_mutation_is_caught(mutation, monkeypatch):
    mutation(monkeypatch)
    failed = _fails(pins.ALL_CHECKS)
    assert failed, f"no pin caught {mutation.__name__}"
