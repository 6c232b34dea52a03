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


MUTATIONS = [mut_scale_div8, mut_ties_away, mut_nibble_order, mut_smoothing_inverted,
             mut_sigma_unsplit, mut_smallest_singulars, mut_residual_sign,
             mut_partials_group_shift, mut_drop_weight_scale, mut_drop_bias,
             mut_down_no_f16, mut_up_no_f16, mut_lora_no_lambda, mut_f16_via_f32,
             mut_smooth_multiplies_lambda, mut_transposed_weight_groups, mut_clamp_8,
             mut_gelu_before_bias]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__)
def test_mutation_is_caught(mutation, monkeypatch):
    mutation(monkeypatch)
    failed = _fails(pins.ALL_CHECKS)
    assert failed, f"no pin caught {mutation.__name__}"
