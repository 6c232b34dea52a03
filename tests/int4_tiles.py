"""The tiled INT4 layouts of include/svdq.h ("Tiled INT4 path"), written out in
numpy from the documented index formulas, for the tests: to check the host
packing of the weights and to read back (and build) the activation operands
and scale pairs of the tiled kernels."""
from __future__ import annotations

import numpy as np

# order of the 16 codes of a lane's k-chunk inside its 16 operand bytes:
# byte t holds code PERM[t] (even codes of each 8, then the odd ones)
PERM = np.array([0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15])


def unpack(codes: np.ndarray) -> np.ndarray:
    """rows x K/2 canonical bytes -> rows x K int8 codes (two's complement nibbles)."""
    b = np.asarray(codes, dtype=np.int16)
    lo, hi = b & 15, (b >> 4) & 15
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int16)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out.astype(np.int8)


def tile_act_ops(codes: np.ndarray, M: int, K: int) -> np.ndarray:
    """canonical activation codes (M x K/2) -> a_ops_t bytes (rows past M in the
    last block repeat row M-1)."""
    G, nb = K // 64, (M + 15) // 16
    q = unpack(codes).astype(np.int16)                       # M x K
    rows = np.minimum(np.arange(nb * 16), M - 1)
    q = q[rows]                                              # nb*16 x K
    # [b, r, g, chunk, 16] -> [b, g, chunk, r, 16] (lane = 16*chunk + r)
    t = q.reshape(nb, 16, G, 4, 16)[..., PERM].transpose(0, 2, 3, 1, 4)
    return ((16 * t) & 0xFF).astype(np.uint8).reshape(-1)


def untile_act_ops(ops: np.ndarray, M: int, K: int) -> np.ndarray:
    """a_ops_t bytes -> (nb*16) x K int8 codes, after checking every byte is 16*q."""
    G, nb = K // 64, (M + 15) // 16
    v = np.asarray(ops, dtype=np.uint8)[:nb * G * 1024].view(np.int8).astype(np.int16)
    assert np.all(v % 16 == 0), "operand bytes must be multiples of 16"
    v = (v // 16).reshape(nb, G, 4, 16, 16)                  # [b, g, chunk, r, byte]
    inv = np.argsort(PERM)
    v = v[..., inv].transpose(0, 3, 1, 2, 4)                 # [b, r, g, chunk, code]
    return v.reshape(nb * 16, K).astype(np.int8)


def act_scale_index(M: int, K: int):
    """(row, group) -> flat float index of the row's scale in a_scales_t."""
    G = K // 64
    rows = np.arange(((M + 127) // 128) * 128)
    t, i, r = rows // 128, (rows % 128) // 16, rows % 16
    return t[:, None] * G * 128 + np.arange(G)[None, :] * 128 + (64 * (i // 4) + 4 * r + i % 4)[:, None]


def tile_act_scales(scales: np.ndarray, M: int, K: int) -> np.ndarray:
    """fp16 activation scales (M x G) -> a_scales_t floats; rows past M get zeros."""
    G = K // 64
    nt = (M + 127) // 128
    s = np.zeros((nt * 128, G), dtype=np.float32)
    s[:M] = np.asarray(scales, dtype=np.float16).astype(np.float32)
    out = np.zeros(nt * G * 128, dtype=np.float32)
    out[act_scale_index(M, K)] = s
    return out


def tile_w(w_codes: np.ndarray, w_scales: np.ndarray, N: int, K: int):
    """canonical weight codes (N x K/2) and fp16 scale bits (N x G) -> (w_codes_t
    bytes, w_scales_t fp32 pairs (s/256, -12582912 s/256)), zero past N."""
    G, ns = K // 64, (N + 31) // 32
    c = np.zeros((ns * 32, K // 2), dtype=np.uint8)
    c[:N] = w_codes
    # [s, j, r, g, q, 8] -> [s, g, q, r, j, 8]  (lane = 16q + r, bytes 8j .. 8j+7)
    ct = c.reshape(ns, 2, 16, G, 4, 8).transpose(0, 3, 4, 2, 1, 5)
    sc = np.zeros((ns * 32, G), dtype=np.float64)
    bits = np.asarray(w_scales)
    bits = bits if bits.dtype == np.uint16 else bits.view(np.uint16)
    sc[:N] = bits.view(np.float16).astype(np.float64)
    # column 32s + 16j + 4q + e -> entries 16q + 8j + 2e (+1) of block (s, g)
    st = sc.reshape(ns, 2, 4, 4, G).transpose(0, 4, 2, 1, 3)      # s, g, q, j, e
    pairs = np.stack([st / 256.0, st * (-12582912.0 / 256.0)], axis=-1).astype(np.float32)
    return np.ascontiguousarray(ct).reshape(-1), np.ascontiguousarray(pairs).reshape(-1)


def untile_d(dt: np.ndarray, M: int, R: int) -> np.ndarray:
    """D_t (fp16 bits, the tiled low-rank down-projection) -> M x R fp16."""
    nb, rc = (M + 15) // 16, (R + 31) // 32
    v = np.asarray(dt).view(np.uint16)[:nb * rc * 512].reshape(nb, rc, 4, 16, 8)  # b, c, q, r, j
    v = v.transpose(0, 3, 1, 2, 4).reshape(nb * 16, rc * 32)                      # [16b + r][32c + 8q + j]
    return v[:M, :R].view(np.float16)


def tile_d(d16: np.ndarray, M: int, R: int) -> np.ndarray:
    """M x R fp16 -> D_t fp16 bits (entries past M or R zero)."""
    nb, rc = (M + 15) // 16, (R + 31) // 32
    full = np.zeros((nb * 16, rc * 32), dtype=np.float16)
    full[:M, :R] = d16
    v = full.view(np.uint16).reshape(nb, 16, rc, 4, 8).transpose(0, 2, 3, 1, 4)   # b, c, q, r, j
    return np.ascontiguousarray(v).reshape(-1)
