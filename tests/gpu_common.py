"""Shared helpers of the GPU parity tests: seeded layers, device buffers and
the oracle side of each comparison. The oracle's inputs are the seeded
inputs and the host-side factors; nothing here feeds a GPU result to it."""
from __future__ import annotations

import functools

import numpy as np

import oracle as O
import workloads as wl

TOL_Y = 2e-3          # max |Y_gpu - Y_oracle| / max |Y_oracle|


def torch_mod():
    import torch
    return torch


def dev(a: np.ndarray):
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host_u16(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def layer(cfg: int, li: int, with_bias: bool = False, use_lora: bool = True):
    """(Layer, X, W, lam, prep, bias) with the library's host prep."""
    L, X, W, lam, p = _layer(cfg, li, use_lora)
    bias = wl.bias(cfg, li, L.N) if with_bias else None
    return L, X, W, lam, p, bias


@functools.lru_cache(maxsize=6)
def _layer(cfg: int, li: int, use_lora: bool):
    import bit_post_quantized_smooth_amd as sq
    L, X, W = wl.layer_inputs(cfg, li)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, L.rank)
    if L.lora_rank and use_lora:
        A, B = wl.lora(cfg, li, L.K, L.N, L.lora_rank)
        p = sq.concat_lora(p, lam, A, B, 1.0)
    return L, X, W, lam, p


class DeviceLayer:
    def __init__(self, X, p, bias, y_dtype="f16"):
        torch = torch_mod()
        self.M, self.K = X.shape
        self.N, self.R = p.N, p.rank
        self.X = dev(X)
        self.inv = dev(p.inv_smooth)
        self.L1p = dev(p.L1p) if self.R else None
        self.L2t = dev(p.L2t) if self.R else None
        self.wc = dev(p.w_codes)
        self.ws = dev(p.w_scales)
        self.bias = dev(bias) if bias is not None else None
        G = self.K // 64
        self.a_codes = torch.empty((self.M, self.K // 2), dtype=torch.uint8, device="cuda")
        self.a_scales = torch.empty((self.M, G), dtype=torch.int16, device="cuda")
        self.D = torch.empty((self.M, max(self.R, 1)), dtype=torch.float32, device="cuda")
        self.Y = torch.empty((self.M, self.N),
                             dtype=torch.float16 if y_dtype == "f16" else torch.float32, device="cuda")

    def k1(self):
        import bit_post_quantized_smooth_amd as sq
        sq.quantize_act_lowrank_down(self.X, self.inv, self.L1p, self.R, self.a_codes,
                                     self.a_scales, self.D if self.R else None)

    def k2(self):
        import bit_post_quantized_smooth_amd as sq
        sq.w4a4_gemm_lowrank_up(self.a_codes, self.a_scales, self.wc, self.ws,
                                self.D if self.R else None, self.L2t, self.R, self.bias, self.Y,
                                self.K)


def sample_rows(M: int, seed: int = 0, n_random: int = 48):
    """First tile, tile boundaries, the last rows (the tail) and random rows."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(M, 16)))
    for b in (127, 128, 129, 255, 256):
        if b < M:
            rows.add(b)
    rows.update(range(max(0, M - 17), M))
    rows.update(int(r) for r in rng.choice(M, min(M, n_random), replace=False))
    return np.array(sorted(rows))


def oracle_prep(X, W, p, base_rank=None):
    """The oracle's own smoothing, 1/lambda and residual codes, for the library's
    fp16 factors (the factors are an input shared by both sides, like X).

    With a LoRA concatenated onto the SVD factors, the residual belongs to the
    first ``base_rank`` columns only (the codes are not re-quantized)."""
    lam = O.smoothing_factors(O.channel_absmax(X), W)
    inv = O.inv_smoothing(lam)
    r = p.rank if base_rank is None else base_rank
    wc, ws = O.quantize_residual_from_factors(W, lam, p.L1[:, :r], p.L2[:r])
    return lam, inv, wc, ws


def oracle_rows(X, inv, p, wc, ws, bias, rows, out_dtype, chunk=16):
    """Oracle Y for the given rows, in chunks of rows (rows are independent)."""
    Ys = []
    for i in range(0, len(rows), chunk):
        r = rows[i:i + chunk]
        Ys.append(O.linear(X[r], inv, p.L1, p.L2, wc, ws, bias, out_dtype))
    return np.concatenate(Ys, axis=0)


def d_stat_bound(xh, L1, K):
    """Per-element bound on |D_gpu - D| that the pre-kernel must meet: rounding
    that random-walks over the K/64 accumulating matrix instructions,
    2^-20 sqrt(K/64) of the envelope |fp16(Xhat)| . |L1| (about 16x the typical
    error; the worst case K 2^-23 of the envelope is far looser)."""
    env = np.abs(O.to_f16(xh).astype(np.float64)) @ np.abs(np.asarray(L1, np.float64))
    return 2.0 ** -20 * np.sqrt(K / 64) * env


def oracle_rows_exact(X, inv, p, wc, ws, bias, rows, chunk=16):
    """For the given rows: the oracle's Y before its final rounding (fp64), the
    magnitude envelope sum_g |s_x s_w P| + |fp16(D)| . |L2| + |b|, and the
    largest legitimate change of the low-rank term: where D lies within the
    pre-kernel's error bound of an fp16 rounding boundary, the device may round
    it to the neighbouring fp16 value, which moves Y by that step times |L2|."""
    Ys, envs, jumps = [], [], []
    K = X.shape[1]
    L2a = np.abs(np.asarray(p.L2, dtype=np.float64))
    swa = np.abs(np.asarray(ws, dtype=np.float16).astype(np.float64))
    for i in range(0, len(rows), chunk):
        r = rows[i:i + chunk]
        _, parts = O.linear(X[r], inv, p.L1, p.L2, wc, ws, bias, "f32", return_parts=True)
        y = parts["acc"] + parts["lr"]
        sxa = np.abs(np.asarray(parts["a_scales"], dtype=np.float16).astype(np.float64))
        env = np.einsum("mng,mg,ng->mn", np.abs(parts["P"]).astype(np.float64), sxa, swa,
                        optimize=True)
        env += np.abs(O.to_f16(parts["D"]).astype(np.float64)) @ L2a
        if bias is not None:
            y = y + np.asarray(bias, dtype=np.float64)[None, :]
            env += np.abs(np.asarray(bias, dtype=np.float64))[None, :]
        D = parts["D"]
        delta = d_stat_bound(parts["xhat"], p.L1, K)
        step = np.abs(O.to_f16(D + delta).astype(np.float64) - O.to_f16(D - delta).astype(np.float64))
        Ys.append(y)
        envs.append(env)
        jumps.append(step @ L2a)
    return (np.concatenate(Ys, axis=0), np.concatenate(envs, axis=0),
            np.concatenate(jumps, axis=0))


def assert_y_strict(Yg, Y_exact, env, jump, out_dtype, G, R):
    """Element-wise bound for a correct kernel: one ulp of the output type (the
    final rounding, crossing at most one rounding boundary) plus one fp32
    rounding per group, per 16 ranks of the low-rank sum and a few more, each
    at most 2^-24 of the envelope, plus the low-rank step where fp16(D) may
    legitimately round the other way. A corrupted operand or a wrongly rounded
    intermediate lands far outside this while staying inside 2e-3 of max|Y|."""
    Yg = np.asarray(Yg, dtype=np.float64)
    a = np.abs(Y_exact)
    if out_dtype == "f16":
        ulp = np.maximum(np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -14))) - 10), 2.0 ** -24)
    else:
        ulp = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 23)
    tol = ulp + (G + R / 16 + 4) * 2.0 ** -24 * env + jump
    ratio = np.abs(Yg - Y_exact) / tol
    assert float(ratio.max()) <= 1.0, (int(np.count_nonzero(ratio > 1)), float(ratio.max()))


def rel_err(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-30))
