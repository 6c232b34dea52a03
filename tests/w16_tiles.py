"""The tiled device layouts of the 4-bit weight-only baseline (include/svdq.h),
written out in numpy from the documented index formulas, for the tests."""
from __future__ import annotations

import numpy as np

ORDER = [0, 4, 1, 5, 2, 6, 3, 7]        # element order inside a lane's 8 values


def tile_x(X16: np.ndarray) -> np.ndarray:
    """M x K fp16 -> flat uint16 tiles; rows past M repeat row M-1."""
    M, K = X16.shape
    nb, S = (M + 15) // 16, K // 32
    Xp = np.empty((nb * 16, K), dtype=np.float16)
    Xp[:M] = X16
    Xp[M:] = X16[M - 1]
    # block (b, s), lane 16q + r, slot e  <-  row 16b + r, k = 32s + 8q + ORDER[e]
    t = Xp.reshape(nb, 16, S, 4, 8)[..., ORDER].transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(t).view(np.uint16).reshape(-1)


def tile_w_codes(codes: np.ndarray, K: int) -> np.ndarray:
    """N x K/2 canonical codes -> flat tiles, each nibble + 8 (columns past N: code 0)."""
    N = codes.shape[0]
    nb, S = (N + 15) // 16, K // 32
    full = np.full((nb * 16, K // 2), 0x00, dtype=np.uint8)
    full[:N] = codes
    t = (full ^ 0x88).reshape(nb, 16, S, 4, 4).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(t).reshape(-1)


def tile_w_scales(scales_bits: np.ndarray, K: int) -> np.ndarray:
    """N x K/64 fp16 bits -> flat uint16 tiles (columns past N: 0)."""
    N = scales_bits.shape[0]
    nc, G = (N + 63) // 64, K // 64
    full = np.zeros((nc * 64, G), dtype=np.uint16)
    full[:N] = scales_bits
    # block (c, g), entry 4r + j  <-  column 64c + 16j + r
    t = full.reshape(nc, 4, 16, G).transpose(0, 3, 2, 1)
    return np.ascontiguousarray(t).reshape(-1)
