"""The tiled MXFP4 device layouts of include/svdq.h, written out in numpy
(reshapes and transposes of the documented index formulas) for the tests:
to check the host packing and to read back what K1-MX writes."""
from __future__ import annotations

import numpy as np


def n_chunks(K: int) -> int:
    return (K + 127) // 128


def tile_codes(codes: np.ndarray, K: int) -> np.ndarray:
    """rows x K/2 canonical codes -> flat tiled codes (zero padding)."""
    rows = codes.shape[0]
    nb, C = (rows + 15) // 16, n_chunks(K)
    full = np.zeros((nb * 16, C * 64), dtype=np.uint8)
    full[:rows, :K // 2] = codes
    # block (b, c), lane 16q + r, byte j  <-  row 16b + r, byte 64c + 16q + j
    t = full.reshape(nb, 16, C, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(t).reshape(-1)


def tile_exps(e8m0: np.ndarray, K: int) -> np.ndarray:
    """rows x K/32 canonical exponents -> flat tiled exponents (padding 127)."""
    rows = e8m0.shape[0]
    ng, C = (rows + 63) // 64, n_chunks(K)
    full = np.full((ng * 64, C * 4), 127, dtype=np.uint8)
    full[:rows, :K // 32] = e8m0
    # block (g, c), byte 4(16q + r) + i  <-  row 64g + 16i + r, block 4c + q
    t = full.reshape(ng, 4, 16, C, 4).transpose(0, 3, 4, 2, 1)
    return np.ascontiguousarray(t).reshape(-1)


def untile_codes(codes_t: np.ndarray, rows: int, K: int) -> np.ndarray:
    """flat tiled codes -> (padded rows) x (C * 64) bytes, canonical order."""
    nb, C = (rows + 15) // 16, n_chunks(K)
    t = np.asarray(codes_t, dtype=np.uint8)[:nb * C * 1024].reshape(nb, C, 4, 16, 16)
    return np.ascontiguousarray(t.transpose(0, 3, 1, 2, 4)).reshape(nb * 16, C * 64)


def untile_exps(exps_t: np.ndarray, rows: int, K: int) -> np.ndarray:
    """flat tiled exponents -> (padded rows) x (C * 4) bytes, canonical order."""
    ng, C = (rows + 63) // 64, n_chunks(K)
    t = np.asarray(exps_t, dtype=np.uint8)[:ng * C * 256].reshape(ng, C, 4, 16, 4)
    return np.ascontiguousarray(t.transpose(0, 4, 3, 1, 2)).reshape(ng * 64, C * 4)
