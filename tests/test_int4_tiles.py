"""The tiled INT4 weight layouts on the CPU: the library's packer against the
layout formulas of svdq.h written out in numpy (tests/int4_tiles.py), and the
numpy helpers' own round trips (they build and read the GPU tests' operands)."""
import numpy as np
import pytest

import int4_tiles as T

sq = pytest.importorskip("bit_post_quantized_smooth_amd")


@pytest.mark.parametrize("N,K", [(1, 64), (31, 192), (32, 64), (33, 128), (100, 320), (257, 640)])
def test_pack_w4a4_tiles_matches_the_layout(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    wc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    # every finite non-negative fp16 scale pattern is possible (zero and subnormals included)
    ws = rng.integers(0, 0x7C00, size=(N, K // 64), dtype=np.uint16)
    ws[0, 0] = 0x7BFF                                   # 65504, the largest scale
    ct, st = sq.pack_w4a4_tiles(wc, ws, K)
    ect, est = T.tile_w(wc, ws, N, K)
    assert ct.size == sq.int4_w_codes_tiled_bytes(N, K) == ect.size
    assert st.dtype == np.float32
    assert st.size * 4 == sq.int4_w_scales_tiled_bytes(N, K) == est.size * 4
    assert np.array_equal(ct, ect) and np.array_equal(st.view(np.uint32), est.view(np.uint32))
    # the pair is exact: s/256 and -12582912 s/256 times 256 give back s and -12582912 s
    s64 = ws.view(np.float16).astype(np.float64)
    col = 0
    assert st[0] * 256.0 == s64[col, 0] and st[1] == s64[col, 0] * -49152.0
    # a permutation with zero padding: every canonical byte appears exactly once
    assert np.array_equal(np.sort(ct)[-wc.size:], np.sort(wc.reshape(-1)))
    assert np.count_nonzero(ct) <= np.count_nonzero(wc)


@pytest.mark.parametrize("M,K", [(1, 64), (17, 128), (129, 192), (300, 640)])
def test_activation_tile_helpers_round_trip(M, K):
    rng = np.random.default_rng(M + K)
    q = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    codes = ((q[:, 0::2] & 15) | ((q[:, 1::2] & 15) << 4)).astype(np.uint8)
    ops = T.tile_act_ops(codes, M, K)
    assert ops.size == sq.int4_act_tiled_bytes(M, K)
    back = T.untile_act_ops(ops, M, K)
    assert np.array_equal(back[:M], q)
    assert np.all(back[M:] == q[M - 1])
    s = np.abs(rng.standard_normal((M, K // 64))).astype(np.float16)
    p = T.tile_act_scales(s, M, K)
    assert p.size * 4 == sq.int4_act_scales_tiled_bytes(M, K)
    idx = T.act_scale_index(M, K)
    assert np.array_equal(p[idx[:M]], s.astype(np.float32))
    assert np.all(p[idx[M:]] == 0)
    # the index formula is a bijection onto the blocks
    assert np.array_equal(np.sort(idx.reshape(-1)), np.arange(p.size))
    # row 128t + 16i + r, group g at (t G + g) 128 + 64 (i/4) + 4 r + i%4
    for r_ in {min(M - 1, 137), min(M - 1, 77), M - 1}:
        g_ = K // 64 - 1
        t, i, r = r_ // 128, (r_ % 128) // 16, r_ % 16
        assert idx[r_, g_] == (t * (K // 64) + g_) * 128 + 64 * (i // 4) + 4 * r + i % 4


@pytest.mark.parametrize("M,R", [(1, 16), (17, 32), (130, 48), (300, 96)])
def test_d_tile_helpers(M, R):
    """D_t: element 8l + j of block (b, c), l = 16q + r, is D[16b + r][32c + 8q + j]."""
    rng = np.random.default_rng(M * 7 + R)
    d = rng.standard_normal((M, R)).astype(np.float16)
    t = T.tile_d(d, M, R)
    assert t.size * 2 == sq.int4_d_tiled_bytes(M, R)
    assert np.array_equal(T.untile_d(t, M, R).view(np.uint16), d.view(np.uint16))
    rc = (R + 31) // 32
    for m, k in {(0, 0), (M - 1, R - 1), (min(M - 1, 21), min(R - 1, 13))}:
        b, r, c, q, j = m // 16, m % 16, k // 32, (k % 32) // 8, k % 8
        assert t[((b * rc + c) * 64 + 16 * q + r) * 8 + j] == d.view(np.uint16)[m, k]
