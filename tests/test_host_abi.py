"""The C ABI on the CPU: exported symbols, argument checks and the host prep
(smoothing, SVD split, residual codes, LoRA concat) against the oracle.

No test here launches GPU work: the device entry points are only called with
arguments that fail validation (which runs before any HIP call), or, on a
machine without a GPU, with arguments that pass it (they must report
SVDQ_ERR_NO_DEVICE)."""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O
import workloads as wl

sq = pytest.importorskip("bit_post_quantized_smooth_amd")
from bit_post_quantized_smooth_amd import _lib  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(svdq_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert len(names) >= 13, names
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(svdq_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        getattr(_lib.lib, n)


def header_prototypes():
    """{name: (return type, [parameter types])} parsed from include/svdq.h."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for m in re.finditer(r"^\s*((?:const\s+)?[\w]+\s*\**)\s*\b(svdq_\w+)\s*\(([^)]*)\)\s*;",
                         src, flags=re.M):
        ret, name, params = m.group(1), m.group(2), m.group(3)
        plist = [] if params.strip() in ("", "void") else [p.strip() for p in params.split(",")]
        types = [re.sub(r"\s*\b\w+$", "", p) if not p.endswith("*") else p for p in plist]
        out[name] = (ret.strip(), types)
    return out


def _ctype_of(t: str):
    """The ctypes type a C parameter of type t is passed as."""
    t = t.replace("const ", "").strip()
    if t.endswith("*") or t == "hipStream_t":
        return C.c_void_p
    return {"int": C.c_int, "int32_t": C.c_int32, "int64_t": C.c_int64, "size_t": C.c_size_t,
            "float": C.c_float}[t]


def test_ctypes_signatures_match_the_header():
    """Every binding signature agrees with the header's prototype in arity, order
    and kind of each argument (an argument out of step would pass a size where a
    pointer is expected, or the reverse)."""
    protos = header_prototypes()
    assert set(protos) == set(header_functions())
    for name, (res, args) in _lib._SIGS.items():
        assert name in protos, name
        ret, ptypes = protos[name]
        want = [_ctype_of(t) for t in ptypes]
        assert list(args) == want, (name, ptypes)
        if ret.endswith("*"):
            assert res in (C.c_char_p, C.c_void_p), name
        else:
            assert res == _ctype_of(ret), (name, ret)
    assert set(protos) == set(_lib._SIGS), set(protos) ^ set(_lib._SIGS)


def test_one_hip_runtime_is_mapped():
    """The library and torch share one HIP runtime (a second copy would be handed
    the other's stream and device-memory handles)."""
    maps = open("/proc/self/maps").read()
    paths = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(paths) <= 1, paths


def test_version_and_status_strings():
    assert _lib.abi_version() == 12
    for s in range(12):
        assert _lib.status_str(s) and _lib.status_str(s) != "unknown status"
    assert _lib.status_str(99) == "unknown status"


def test_channel_absmax_and_smoothing_bit_exact():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((37, 192)).astype(np.float32)
    X[:, 5] = 0.0
    W = (rng.standard_normal((192, 40)) * 0.02).astype(np.float32)
    W[7] = 0.0
    for Xd in (X, X.astype(np.float16)):
        xa = sq.channel_absmax(Xd)
        assert np.array_equal(xa, O.channel_absmax(Xd).astype(np.float32))
        lam = sq.smoothing_factors(xa, W)
        assert np.array_equal(lam, O.smoothing_factors(O.channel_absmax(Xd), W))
    assert lam[5] == 1.0 and lam[7] == 1.0


@pytest.mark.parametrize("geom", [
    # batch, H, W, C, KH, KW, stride, pad
    (1, 8, 8, 64, 3, 3, 1, 1), (2, 5, 7, 128, 3, 3, 2, 1), (1, 6, 4, 64, 1, 1, 1, 0),
    (1, 4, 4, 64, 5, 5, 1, 2), (3, 9, 5, 192, 3, 2, 3, 0), (1, 2, 2, 64, 1, 1, 1, 2)])
def test_conv_patch_absmax_bit_exact(geom):
    """Column maxima of the implicit patch matrix = those of the oracle's im2col."""
    B, H, W, Cc, KH, KW, st, pad = geom
    rng = np.random.default_rng(sum(geom))
    X = rng.standard_normal((B, H, W, Cc)).astype(np.float32)
    X[..., 3] *= 30
    for Xd in (X, X.astype(np.float16)):
        got = sq.conv_patch_absmax(Xd, KH, KW, st, pad)
        ref = O.channel_absmax(O.im2col_nhwc(Xd, KH, KW, st, pad)).astype(np.float32)
        assert got.shape == (KH * KW * Cc,)
        assert np.array_equal(got, ref)
    assert sq.conv_out_size(H, KH, st, pad) == (H + 2 * pad - KH) // st + 1


@pytest.mark.parametrize("K,N,r", [(64, 16, 0), (128, 96, 16), (256, 64, 32), (192, 300, 48),
                                   (512, 512, 16)])
def test_prepare_codes_bit_exact(K, N, r):
    rng = np.random.default_rng(K * 7 + N + r)
    X = rng.standard_normal((64, K)).astype(np.float32)
    X[:, rng.choice(K, 3, replace=False)] *= 20
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    W[rng.choice(K, 2, replace=False)] *= 10
    lam = O.smoothing_factors(O.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, r, want_sigma=True)
    assert np.array_equal(p.inv_smooth, O.inv_smoothing(lam))
    # the residual codes that the oracle derives from the library's own factors
    wc, ws = O.quantize_residual_from_factors(W, lam, p.L1, p.L2)
    assert np.array_equal(p.w_codes, wc)
    assert np.array_equal(p.w_scales, ws.view(np.uint16))
    # singular values against LAPACK
    S = np.linalg.svd(O.smooth_weight(W, lam), compute_uv=False)
    assert np.allclose(p.sigma, S, rtol=0, atol=1e-10 * S[0])
    if r:
        # Eckart-Young-Mirsky: the library's fp16 pair cannot beat the optimum and
        # stays within the fp16 rounding of the factors
        What = O.smooth_weight(W, lam)
        L1 = p.L1.astype(np.float64)
        L2 = p.L2.astype(np.float64)
        e = np.linalg.norm(What - L1 @ L2)
        tail = np.sqrt(np.sum(S[r:] ** 2))
        rnd = 2.0 ** -11 * (np.linalg.norm(L1) * np.linalg.norm(L2, 2) +
                            np.linalg.norm(L1, 2) * np.linalg.norm(L2)) * 1.01
        assert tail * (1 - 1e-12) <= e <= tail + rnd
        # the balanced split: L1^T L1 ~ diag(sigma_r)
        G1 = L1.T @ L1
        assert np.allclose(np.diag(G1), S[:r], rtol=4e-3)
        # canonical sign: the largest-magnitude entry of each column of L1 is positive
        idx = np.argmax(np.abs(L1), axis=0)
        assert np.all(L1[idx, np.arange(r)] > 0)


@pytest.mark.parametrize("K,N,r", [(64, 16, 0), (128, 96, 16), (320, 40, 32), (512, 512, 16)])
def test_prepare_mx_bit_exact(K, N, r):
    """MXFP4 prep: the same factors as the INT4 prep, and residual codes and
    E8M0 exponents equal to the oracle's for those factors."""
    rng = np.random.default_rng(K * 5 + N + r)
    X = rng.standard_normal((64, K)).astype(np.float32)
    X[:, rng.choice(K, 3, replace=False)] *= 20
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    W[rng.choice(K, 2, replace=False)] *= 10
    W[:, 3 % N] = 0.0                                  # an all-zero column: E8M0 0, codes 0
    lam = O.smoothing_factors(O.channel_absmax(X), W)
    p = sq.prepare_weights_mx(W, lam, r)
    assert p.fmt == "mxfp4" and p.w_scales.shape == (N, K // 32) and p.w_codes.shape == (N, K // 2)
    pi = sq.prepare_weights(W, lam, r)
    assert np.array_equal(p.L1t, pi.L1t) and np.array_equal(p.L2t, pi.L2t)
    assert np.array_equal(p.inv_smooth, pi.inv_smooth)
    wc, we = O.mx_quantize_residual_from_factors(W, lam, p.L1, p.L2)
    assert np.array_equal(p.w_codes, wc)
    assert np.array_equal(p.w_scales, we)


def test_prepare_mx_extreme_values():
    """Columns that are tiny (subnormal fp32), huge, exactly on E2M1 midpoints, or
    signed zeros: host codes equal the oracle's."""
    K, N = 128, 6
    W = np.zeros((K, N), dtype=np.float32)
    rng = np.random.default_rng(77)
    W[:, 0] = rng.standard_normal(K) * 1e-41          # subnormal
    W[:, 1] = rng.standard_normal(K) * 1e37
    W[:, 2] = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], K) * rng.choice([-1, 1], K)
    W[:, 3] = -0.0
    W[::2, 4] = -0.0
    W[1::2, 4] = 1e-3
    W[:, 5] = rng.standard_normal(K)
    lam = np.ones(K, dtype=np.float32)
    p = sq.prepare_weights_mx(W, lam, 0)
    wc, we = O.mx_quantize_residual_from_factors(W, lam, np.zeros((K, 0), np.float16),
                                                 np.zeros((0, N), np.float16))
    assert np.array_equal(p.w_codes, wc)
    assert np.array_equal(p.w_scales, we)
    assert np.all(p.w_scales[3] == 0) and np.all(p.w_codes[3] == 0x88)   # -0 keeps its sign


@pytest.mark.parametrize("rows,K", [(1, 64), (16, 128), (100, 320), (130, 1024), (64, 192)])
def test_pack_mx_tiles_is_the_documented_layout(rows, K):
    """svdq_pack_mx_tiles against the index formulas of svdq.h, written out in
    numpy (tests/mx_tiles.py) and checked entry by entry on a sample; padding
    rows and the missing half of the last chunk hold zero codes and exponent 127."""
    import mx_tiles as T
    rng = np.random.default_rng(rows * 7 + K)
    c = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    e = rng.integers(0, 255, (rows, K // 32), dtype=np.uint8)
    ct, et = sq.pack_mx_tiles(c, e, K)
    C = (K + 127) // 128
    assert ct.size == ((rows + 15) // 16) * C * 1024 == sq.mx_codes_tiled_bytes(rows, K)
    assert et.size == ((rows + 63) // 64) * C * 256 == sq.mx_exps_tiled_bytes(rows, K)
    assert np.array_equal(ct, T.tile_codes(c, K)) and np.array_equal(et, T.tile_exps(e, K))
    assert np.array_equal(T.untile_codes(ct, rows, K)[:rows, :K // 2], c)
    assert np.array_equal(T.untile_exps(et, rows, K)[:rows, :K // 32], e)
    for _ in range(200):
        b, cc, l = rng.integers(0, (rows + 15) // 16), rng.integers(0, C), rng.integers(0, 64)
        j, g, i = rng.integers(0, 16), rng.integers(0, (rows + 63) // 64), rng.integers(0, 4)
        row, byte = 16 * b + l % 16, 64 * cc + 16 * (l // 16) + j
        want = c[row, byte] if row < rows and byte < K // 2 else 0
        assert ct[((b * C + cc) * 64 + l) * 16 + j] == want
        row, blk = 64 * g + 16 * i + l % 16, 4 * cc + l // 16
        want = e[row, blk] if row < rows and blk < K // 32 else 127
        assert et[((g * C + cc) * 64 + l) * 4 + i] == want


@pytest.mark.parametrize("K,N", [(64, 1), (128, 40), (320, 70), (1024, 256)])
def test_w4a16_prep_and_tiles(K, N):
    """The weight-only baseline's weights equal the oracle's Q(W), and their tiled
    layouts follow the index formulas of svdq.h (numpy statement in
    tests/w16_tiles.py, spot-checked entry by entry)."""
    import w16_tiles as T
    rng = np.random.default_rng(K + 3 * N)
    W = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    W[rng.integers(0, K)] *= 10
    p = sq.prepare_weights_w4a16(W)
    wc, ws = O.w4a16_prepare(W)
    assert p.fmt == "w4a16" and np.array_equal(p.w_codes, wc)
    assert np.array_equal(p.w_scales, ws.view(np.uint16))
    ct, st = sq.pack_w4a16_tiles(p.w_codes, p.w_scales, K)
    assert np.array_equal(ct, T.tile_w_codes(p.w_codes, K))
    assert np.array_equal(st, T.tile_w_scales(p.w_scales, K))
    S, G = K // 32, K // 64
    for _ in range(100):
        b, s, l, j = rng.integers(0, (N + 15) // 16), rng.integers(0, S), rng.integers(0, 64), rng.integers(0, 4)
        n = 16 * b + l % 16
        want = (p.w_codes[n, 16 * s + 4 * (l // 16) + j] ^ 0x88) if n < N else 0x88
        assert ct[((b * S + s) * 64 + l) * 4 + j] == want
        c, g, r = rng.integers(0, (N + 63) // 64), rng.integers(0, G), rng.integers(0, 16)
        n = 64 * c + 16 * j + r
        want = p.w_scales[n, g] if n < N else 0
        assert st[(c * G + g) * 64 + 4 * r + j] == want


def test_prepare_full_rank_reconstructs():
    rng = np.random.default_rng(5)
    K, N = 64, 48
    W = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    lam = np.ones(K, dtype=np.float32)
    p = sq.prepare_weights(W, lam, min(K, N))
    L1 = p.L1.astype(np.float64)
    L2 = p.L2.astype(np.float64)
    E = O.smooth_weight(W, lam) - L1 @ L2
    rnd = 2.0 ** -11 * (np.linalg.norm(L1) * np.linalg.norm(L2, 2) +
                        np.linalg.norm(L1, 2) * np.linalg.norm(L2)) * 1.01
    assert np.linalg.norm(E) <= rnd


@pytest.mark.slow
def test_prepare_dit_qkv_full_size_bit_exact():
    """The 3072 x 9216 DiT QKV weight: residual codes bit-exact at full size."""
    L, X, W = wl.layer_inputs(1, 0)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, L.rank)
    wc, ws = O.quantize_residual_from_factors(W, lam, p.L1, p.L2)
    assert np.array_equal(p.w_codes, wc)
    assert np.array_equal(p.w_scales, ws.view(np.uint16))


def test_concat_lora_bit_exact():
    rng = np.random.default_rng(9)
    K, N, r, rl = 128, 80, 16, 8
    X = rng.standard_normal((16, K)).astype(np.float32)
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    lam = O.smoothing_factors(O.channel_absmax(X), W)
    p = sq.prepare_weights(W, lam, r)
    A = (rng.standard_normal((K, rl)) * 0.01).astype(np.float16)
    B = (rng.standard_normal((rl, N)) * 0.01).astype(np.float16)
    for scale in (1.0, 0.37):
        q = sq.concat_lora(p, lam, A, B, scale)
        L1o, L2o = O.concat_lora(p.L1, p.L2, lam, A, B, scale)
        assert np.array_equal(q.L1.view(np.uint16), L1o.view(np.uint16))
        assert np.array_equal(q.L2.view(np.uint16), L2o.view(np.uint16))
        assert np.array_equal(q.w_codes, p.w_codes) and q.rank == r + rl


@pytest.mark.parametrize("K,R", [(64, 16), (192, 48), (1024, 112)])
def test_pack_lowrank_down_is_the_documented_permutation(K, R):
    """svdq_pack_lowrank_down against the index formula of the header, written
    here as a reshape: L1t[c*16 + rl, g*64 + q*16 + h*8 + j] goes to operand
    (g, c, h), lane q*16 + rl, element j."""
    rng = np.random.default_rng(K + R)
    L1t = rng.integers(0, 1 << 16, size=(R, K), dtype=np.uint16)
    got = sq.pack_lowrank_down(L1t)
    ref = (L1t.reshape(R // 16, 16, K // 64, 4, 2, 8)     # c, rl, g, q, h, j
              .transpose(2, 0, 4, 3, 1, 5)                 # g, c, h, q, rl, j
              .reshape(-1))
    assert got.shape == (R * K,) and np.array_equal(got, ref)
    # spot check one element by the formula itself
    g, c, h, q, rl, j = K // 64 - 1, R // 16 - 1, 1, 2, 5, 3
    idx = (((g * (R // 16) + c) * 2 + h) * 64 + q * 16 + rl) * 8 + j
    assert got[idx] == L1t[c * 16 + rl, g * 64 + q * 16 + h * 8 + j]


@pytest.mark.parametrize("K,N,R", [(64, 1, 16), (192, 130, 48), (1024, 300, 112)])
def test_pack_lowrank_takes_the_canonical_factors(K, N, R):
    """svdq_pack_lowrank on L1 (K x R) and L2 (R x N), the oracle's shapes: L1p by
    the header's index formula (a reshape of L1's transpose), L2t = L2 transposed;
    the factors of an oracle preparation go through unchanged."""
    rng = np.random.default_rng(K + N + R)
    L1 = rng.integers(0, 1 << 16, size=(K, R), dtype=np.uint16)
    L2 = rng.integers(0, 1 << 16, size=(R, N), dtype=np.uint16)
    L1p, L2t = sq.pack_lowrank(L1, L2)
    ref = (L1.T.reshape(R // 16, 16, K // 64, 4, 2, 8)    # c, rl, g, q, h, j
              .transpose(2, 0, 4, 3, 1, 5)                 # g, c, h, q, rl, j
              .reshape(-1))
    assert np.array_equal(L1p, ref)
    g, c, h, q, rl, j = K // 64 - 1, R // 16 - 1, 1, 3, 14, 7
    idx = (((g * (R // 16) + c) * 2 + h) * 64 + q * 16 + rl) * 8 + j
    assert L1p[idx] == L1[g * 64 + q * 16 + h * 8 + j, c * 16 + rl]
    assert L2t.shape == (N, R) and np.array_equal(L2t, L2.T)
    # the same packing as svdq_pack_lowrank_down on the transpose
    assert np.array_equal(L1p, sq.pack_lowrank_down(np.ascontiguousarray(L1.T)))


def test_pack_lowrank_of_an_oracle_preparation():
    rng = np.random.default_rng(11)
    K, N, R = 128, 96, 16
    W = rng.standard_normal((K, N)).astype(np.float32)
    X = rng.standard_normal((32, K)).astype(np.float32)
    lam = O.smoothing_factors(O.channel_absmax(X), W)
    pr = O.prepare(W, lam, R)
    assert pr["L1"].shape == (K, R) and pr["L2"].shape == (R, N)
    L1p, L2t = sq.pack_lowrank(pr["L1"].view(np.uint16), pr["L2"].view(np.uint16))
    assert np.array_equal(L2t.view(np.float16), pr["L2"].T)
    assert L1p[0] == pr["L1"].view(np.uint16)[0, 0]


def test_host_errors():
    L = _lib.lib
    W = np.zeros((128, 8), dtype=np.float32)
    lam = np.ones(128, dtype=np.float32)
    buf = np.zeros(1 << 16, dtype=np.uint8)
    bp = buf.ctypes.data
    assert L.svdq_prepare_weights(None, lam.ctypes.data, 128, 8, 4, 64, bp, bp, bp, bp, bp, None) == _lib.ERR_NULL
    assert L.svdq_prepare_weights(W.ctypes.data, lam.ctypes.data, 128, 8, 4, 32, bp, bp, bp, bp, bp, None) == _lib.ERR_GROUP
    assert L.svdq_prepare_weights(W.ctypes.data, lam.ctypes.data, 100, 8, 4, 64, bp, bp, bp, bp, bp, None) == _lib.ERR_GROUP
    assert L.svdq_prepare_weights(W.ctypes.data, lam.ctypes.data, 128, 8, 9, 64, bp, bp, bp, bp, bp, None) == _lib.ERR_RANK
    assert "rank" in _lib.last_error()
    assert L.svdq_channel_absmax(bp, 3, 4, 4, 4, bp) == _lib.ERR_DTYPE
    assert L.svdq_channel_absmax(bp, 2, 4, 8, 4, bp) == _lib.ERR_SHAPE
    assert L.svdq_concat_lora(None, None, 64, 8, 0, lam.ctypes.data, bp, bp, 0, 1.0, bp, bp) == _lib.ERR_RANK
    assert L.svdq_smoothing_factors(None, bp, 4, 4, bp) == _lib.ERR_NULL
    assert L.svdq_pack_lowrank_down(None, 64, 16, bp) == _lib.ERR_NULL
    assert L.svdq_pack_lowrank_down(bp, 96, 16, bp) == _lib.ERR_GROUP
    assert L.svdq_pack_lowrank_down(bp, 64, 24, bp) == _lib.ERR_RANK
    assert L.svdq_pack_lowrank_down(bp, 64, 0, bp) == _lib.ERR_RANK
    assert L.svdq_pack_lowrank(None, bp, 64, 8, 16, bp, bp) == _lib.ERR_NULL
    assert L.svdq_pack_lowrank(bp, bp, 96, 8, 16, bp, bp) == _lib.ERR_GROUP
    assert L.svdq_pack_lowrank(bp, bp, 64, 0, 16, bp, bp) == _lib.ERR_SHAPE
    assert L.svdq_pack_lowrank(bp, bp, 64, 8, 24, bp, bp) == _lib.ERR_RANK
    # weight-only baseline
    assert L.svdq_prepare_weights_w4a16(None, 64, 8, bp, bp) == _lib.ERR_NULL
    assert L.svdq_prepare_weights_w4a16(W.ctypes.data, 96, 8, bp, bp) == _lib.ERR_GROUP
    assert L.svdq_pack_w4a16_tiles(bp, bp, 0, 64, bp, bp) == _lib.ERR_SHAPE
    assert L.svdq_w4a16_codes_tiled_bytes(4, 96) == 0 and L.svdq_w4a16_x_tiled_bytes(0, 64) == 0
    # MXFP4 tiles
    assert L.svdq_pack_mx_tiles(None, bp, 4, 64, bp, bp) == _lib.ERR_NULL
    assert L.svdq_pack_mx_tiles(bp, bp, 4, 96, bp, bp) == _lib.ERR_GROUP
    assert L.svdq_pack_mx_tiles(bp, bp, 0, 64, bp, bp) == _lib.ERR_SHAPE
    assert L.svdq_mx_codes_tiled_bytes(0, 64) == 0 and L.svdq_mx_exps_tiled_bytes(4, 96) == 0
    # MXFP4 prep
    assert L.svdq_prepare_weights_mx(W.ctypes.data, lam.ctypes.data, 128, 8, 4, bp, bp, bp, bp, None, None) == _lib.ERR_NULL
    assert L.svdq_prepare_weights_mx(W.ctypes.data, lam.ctypes.data, 96, 8, 4, bp, bp, bp, bp, bp, None) == _lib.ERR_GROUP
    assert L.svdq_prepare_weights_mx(W.ctypes.data, lam.ctypes.data, 128, 0, 0, bp, bp, bp, bp, bp, None) == _lib.ERR_SHAPE
    assert L.svdq_prepare_weights_mx(W.ctypes.data, lam.ctypes.data, 128, 8, 9, bp, bp, bp, bp, bp, None) == _lib.ERR_RANK


# Fake device addresses: never dereferenced because validation rejects the call
# (or, on a machine without a GPU, the device check does).
A16 = 0x10000
MIS = 0x10008


def test_device_entry_points_reject_bad_arguments():
    L = _lib.lib
    # K1
    assert L.svdq_quantize_act_lowrank_down(None, 1, 16, 64, 64, A16, A16, 16, 64, A16, A16, A16, None) == _lib.ERR_NULL
    assert L.svdq_quantize_act_lowrank_down(A16, 7, 16, 64, 64, A16, A16, 16, 64, A16, A16, A16, None) == _lib.ERR_DTYPE
    assert L.svdq_quantize_act_lowrank_down(A16, 1, 16, 96, 96, A16, A16, 16, 64, A16, A16, A16, None) == _lib.ERR_GROUP
    assert L.svdq_quantize_act_lowrank_down(A16, 1, 16, 64, 64, A16, A16, 24, 64, A16, A16, A16, None) == _lib.ERR_RANK
    assert L.svdq_quantize_act_lowrank_down(A16, 1, 16, 64, 64, A16, A16, 512, 64, A16, A16, A16, None) == _lib.ERR_RANK
    assert L.svdq_quantize_act_lowrank_down(A16, 1, 0, 64, 64, A16, A16, 16, 64, A16, A16, A16, None) == _lib.ERR_SHAPE
    assert L.svdq_quantize_act_lowrank_down(A16, 1, 16, 64, 32, A16, A16, 16, 64, A16, A16, A16, None) == _lib.ERR_SHAPE
    # rows longer than 2^25 elements would overflow the kernel's 32-bit offsets
    assert L.svdq_quantize_act_lowrank_down(A16, 1, 16, 64, (1 << 25) + 64, A16, A16, 16, 64, A16, A16, A16, None) == _lib.ERR_SHAPE
    assert L.svdq_quantize_act_lowrank_down(MIS, 1, 16, 64, 64, A16, A16, 16, 64, A16, A16, A16, None) == _lib.ERR_ALIGN
    assert L.svdq_quantize_act_lowrank_down(A16, 1, 16, 64, 68, A16, A16, 16, 64, A16, A16, A16, None) == _lib.ERR_ALIGN
    assert L.svdq_quantize_act_lowrank_down(A16, 1, 16, 64, 64, A16, None, 16, 64, A16, A16, A16, None) == _lib.ERR_NULL
    # K2
    args = [A16, A16, A16, A16, A16, A16, 16, None, A16, 1, 16, 16, 64, 16, 64, 0, None]
    bad = list(args); bad[8] = None
    assert L.svdq_w4a4_gemm_lowrank_up(*bad) == _lib.ERR_NULL
    bad = list(args); bad[9] = 5
    assert L.svdq_w4a4_gemm_lowrank_up(*bad) == _lib.ERR_DTYPE
    bad = list(args); bad[13] = 8
    assert L.svdq_w4a4_gemm_lowrank_up(*bad) == _lib.ERR_SHAPE
    bad = list(args); bad[8] = 0x10001          # fp16 Y on an odd address
    assert L.svdq_w4a4_gemm_lowrank_up(*bad) == _lib.ERR_ALIGN
    bad = list(args); bad[7] = 0x10002          # bias not 4-byte aligned
    assert L.svdq_w4a4_gemm_lowrank_up(*bad) == _lib.ERR_ALIGN
    bad = list(args); bad[0] = MIS              # codes
    assert L.svdq_w4a4_gemm_lowrank_up(*bad) == _lib.ERR_ALIGN
    bad = list(args); bad[14] = 128
    assert L.svdq_w4a4_gemm_lowrank_up(*bad) == _lib.ERR_GROUP
    bad = list(args); bad[15] = 7                # activation code
    assert L.svdq_w4a4_gemm_lowrank_up(*bad) == _lib.ERR_ACT
    # whole layer: workspace
    need = L.svdq_linear_workspace_bytes(16, 64, 16, 64)
    assert need >= 16 * 32 + 16 * 2 + 16 * 16 * 4 and need % 256 == 0
    assert L.svdq_linear_workspace_bytes(16, 60, 16, 64) == 0
    la = [A16, 1, 64, A16, A16, A16, 16, A16, A16, None, A16, 1, 16, 16, 64, 16, 64, A16, need - 1, 0,
          None]
    assert L.svdq_linear(*la) == _lib.ERR_WORKSPACE
    la[18] = need
    la[19] = 2
    assert L.svdq_linear(*la) == _lib.ERR_ACT
    la[19] = 1
    la[17] = 0x10080
    assert L.svdq_linear(*la) == _lib.ERR_ALIGN
    # MXFP4 K1 / K2 / layer
    assert L.svdq_quantize_act_lowrank_down_mx(A16, 1, 16, 64, 64, A16, A16, 16, A16, None, A16, None, 0, None) == _lib.ERR_NULL
    assert L.svdq_quantize_act_lowrank_down_mx(A16, 1, 16, 96, 96, A16, A16, 16, A16, A16, A16, None, 0, None) == _lib.ERR_GROUP
    assert L.svdq_quantize_act_lowrank_down_mx(A16, 1, 16, 64, 64, A16, A16, 24, A16, A16, A16, None, 0, None) == _lib.ERR_RANK
    assert L.svdq_quantize_act_lowrank_down_mx(A16, 1, 16, 64, 64, A16, A16, 16, A16, MIS, A16, None, 0, None) == _lib.ERR_ALIGN
    assert L.svdq_quantize_act_lowrank_down_mx(A16, 3, 16, 64, 64, A16, A16, 16, A16, A16, A16, None, 0, None) == _lib.ERR_DTYPE
    # the pre-kernels' optional workspace (split long rows): too small, misaligned
    big = (4608, 12288, 32)
    need_k1 = L.svdq_quantize_act_workspace_bytes(*big)
    assert need_k1 > 0
    k1t = [A16, 1, big[0], big[1], big[1], A16, A16, big[2], A16, A16, A16, 0x10000, need_k1 - 1,
           None]
    assert L.svdq_quantize_act_lowrank_down_tiled(*k1t) == _lib.ERR_WORKSPACE
    assert "workspace" in _lib.last_error()
    assert L.svdq_quantize_act_lowrank_down_mx(*k1t) == _lib.ERR_WORKSPACE
    k1t[11], k1t[12] = 0x10040, need_k1
    assert L.svdq_quantize_act_lowrank_down_tiled(*k1t) == _lib.ERR_ALIGN
    assert L.svdq_quantize_act_lowrank_down_mx(*k1t) == _lib.ERR_ALIGN
    mxa = [A16, A16, A16, A16, A16, A16, 16, None, A16, 1, 16, 16, 64, 16, 0, None]
    bad = list(mxa); bad[3] = None
    assert L.svdq_mx_gemm_lowrank_up(*bad) == _lib.ERR_NULL
    bad = list(mxa); bad[1] = MIS                # activation exponents
    assert L.svdq_mx_gemm_lowrank_up(*bad) == _lib.ERR_ALIGN
    bad = list(mxa); bad[12] = 160
    assert L.svdq_mx_gemm_lowrank_up(*bad) == _lib.ERR_GROUP
    bad = list(mxa); bad[13] = 15
    assert L.svdq_mx_gemm_lowrank_up(*bad) == _lib.ERR_SHAPE
    bad = list(mxa); bad[14] = 3
    assert L.svdq_mx_gemm_lowrank_up(*bad) == _lib.ERR_ACT
    need_mx = L.svdq_linear_mx_workspace_bytes(16, 64, 16)
    assert need_mx >= 16 * 32 + 16 * 2 + 16 * 16 * 4 and need_mx % 256 == 0
    assert L.svdq_linear_mx_workspace_bytes(16, 96, 16) == 0
    lm = [A16, 1, 64, A16, A16, A16, 16, A16, A16, None, A16, 1, 16, 16, 64, 16, A16, need_mx - 1, 0,
          None]
    assert L.svdq_linear_mx(*lm) == _lib.ERR_WORKSPACE
    lm[17] = need_mx
    lm[18] = 9
    assert L.svdq_linear_mx(*lm) == _lib.ERR_ACT
    lm[18] = 0
    lm[16] = 0x10080
    assert L.svdq_linear_mx(*lm) == _lib.ERR_ALIGN
    # weight-only baseline, device side
    assert L.svdq_w4a16_tile_activation(None, 1, 16, 64, 64, A16, None) == _lib.ERR_NULL
    assert L.svdq_w4a16_tile_activation(A16, 9, 16, 64, 64, A16, None) == _lib.ERR_DTYPE
    assert L.svdq_w4a16_tile_activation(A16, 1, 16, 64, 68, A16, None) == _lib.ERR_ALIGN
    assert L.svdq_w4a16_tile_activation(A16, 1, 16, 96, 96, A16, None) == _lib.ERR_GROUP
    wg = [A16, A16, A16, None, A16, 1, 16, 16, 64, 16, None]
    bad = list(wg); bad[1] = None
    assert L.svdq_w4a16_gemm(*bad) == _lib.ERR_NULL
    bad = list(wg); bad[9] = 8
    assert L.svdq_w4a16_gemm(*bad) == _lib.ERR_SHAPE
    bad = list(wg); bad[2] = MIS
    assert L.svdq_w4a16_gemm(*bad) == _lib.ERR_ALIGN
    need16 = L.svdq_w4a16_x_tiled_bytes(16, 64)
    assert need16 == 2 * 1024
    lw = [A16, 1, 64, A16, A16, None, A16, 1, 16, 16, 64, 16, A16, need16 - 1, None]
    assert L.svdq_linear_w4a16(*lw) == _lib.ERR_WORKSPACE
    # convolutions: geometry checks come before any pointer is used
    geo = [1, 8, 8, 64, 3, 3, 1, 1]
    assert L.svdq_conv_patch_absmax(None, 2, *geo, A16) == _lib.ERR_NULL
    for bad_geo in ([1, 8, 8, 96, 3, 3, 1, 1],     # C not a multiple of 64
                    [1, 8, 8, 0, 3, 3, 1, 1],
                    [0, 8, 8, 64, 3, 3, 1, 1],
                    [1, 8, 8, 64, 3, 3, 0, 1],     # stride 0
                    [1, 8, 8, 64, 3, 3, 1, -1],    # negative pad
                    [1, 2, 8, 64, 5, 3, 1, 1],     # kernel taller than the padded image
                    [1, 8, 8, 64, 65, 1, 1, 40],   # kernel beyond 64
                    [1 << 16, 128, 128, 64, 3, 3, 1, 1]):   # image past 2^31 elements
        assert L.svdq_conv_patch_absmax(A16, 2, *bad_geo, A16) == _lib.ERR_SHAPE, bad_geo
        assert L.svdq_quantize_act_lowrank_down_conv(A16, 1, *bad_geo, A16, A16, 16, A16, A16, A16,
                                                     None) == _lib.ERR_SHAPE, bad_geo
        assert L.svdq_conv2d(A16, 1, *bad_geo, A16, A16, A16, 16, A16, A16, None, A16, 1, 16, A16,
                             1 << 20, 0, None) == _lib.ERR_SHAPE, bad_geo
    assert L.svdq_conv_patch_absmax(A16, 5, *geo, A16) == _lib.ERR_DTYPE
    assert L.svdq_quantize_act_lowrank_down_conv(MIS, 1, *geo, A16, A16, 16, A16, A16, A16, None) == _lib.ERR_ALIGN
    assert L.svdq_quantize_act_lowrank_down_conv(A16, 1, *geo, A16, A16, 24, A16, A16, A16, None) == _lib.ERR_RANK
    assert L.svdq_quantize_act_lowrank_down_conv(A16, 1, *geo, A16, None, 16, A16, A16, A16, None) == _lib.ERR_NULL
    # patch matrix 64 x 576: the workspace is that of the linear layer
    need_c = L.svdq_linear_workspace_bytes(64, 576, 16, 64)
    ca = [A16, 1, *geo, A16, A16, A16, 16, A16, A16, None, A16, 1, 16, A16, need_c - 1, 0, None]
    assert L.svdq_conv2d(*ca) == _lib.ERR_WORKSPACE
    ca[21] = need_c
    ca[22] = 4
    assert L.svdq_conv2d(*ca) == _lib.ERR_ACT
    ca[22] = 0
    ca[20] = 0x10080
    assert L.svdq_conv2d(*ca) == _lib.ERR_ALIGN
    ca[20] = None
    assert L.svdq_conv2d(*ca) == _lib.ERR_NULL
    # the MXFP4 convolution: same geometry checks, the MXFP4 workspace
    assert L.svdq_quantize_act_lowrank_down_conv_mx(A16, 1, 1, 8, 8, 96, 3, 3, 1, 1, A16, A16, 16, A16, A16, A16, None) == _lib.ERR_SHAPE
    assert L.svdq_quantize_act_lowrank_down_conv_mx(A16, 1, *geo, A16, A16, 16, A16, MIS, A16, None) == _lib.ERR_ALIGN
    need_cm = L.svdq_linear_mx_workspace_bytes(64, 576, 16)
    cm = [A16, 1, *geo, A16, A16, A16, 16, A16, A16, None, A16, 1, 16, A16, need_cm - 1, 0, None]
    assert L.svdq_conv2d_mx(*cm) == _lib.ERR_WORKSPACE
    cm[21] = need_cm
    cm[22] = 5
    assert L.svdq_conv2d_mx(*cm) == _lib.ERR_ACT
    cm[2] = 0
    cm[22] = 0
    assert L.svdq_conv2d_mx(*cm) == _lib.ERR_SHAPE
    # partials hook: slice outside the rows
    assert L.svdq_debug_group_partials(A16, A16, 16, 16, 64, 64, 10, 7, A16, None) == _lib.ERR_SHAPE
    assert L.svdq_gelu_tanh_f16(A16, MIS, 8, None) == _lib.ERR_ALIGN
    assert L.svdq_gelu_tanh_f16(A16, A16, 0, None) == _lib.OK          # empty: nothing to do


def test_pre_kernel_workspace_sizes():
    """The split pre-kernel's partial tiles: S slices x rows rounded up to 32 x R
    fp32 on long rows with more 16-row tiles than compute units (256 here:
    without a device the library assumes MI355X's), nothing otherwise, and the
    fused entry points' workspaces grow by exactly that (256-byte aligned)."""
    L = _lib.lib
    ws = L.svdq_quantize_act_workspace_bytes
    # 4608 x 12288: 144 tiles of 32 rows, S = ceil(4 * 256 / 144) = 8
    assert ws(4608, 12288, 32) == 8 * 4608 * 32 * 4
    # 4100 x 6144: 129 tiles, ceil(1024 / 129) = 8, capped at G / 16 = 6; rows
    # rounded up to 4128
    assert ws(4100, 6144, 16) == 6 * 4128 * 16 * 4
    # 8200 rows: 257 tiles, S = ceil(1024 / 257) = 4
    assert ws(8200, 6144, 32) == 4 * 8224 * 32 * 4
    # ranks 80 and 96 split whatever the row length: 4608 x 12288 as above
    # (S = 8); 9216 x 3072 (48 groups): 288 tiles, ceil(1024 / 288) = 4,
    # capped at G / 16 = 3
    assert ws(4608, 12288, 96) == 8 * 4608 * 96 * 4
    assert ws(9216, 3072, 96) == 3 * 9216 * 96 * 4
    assert ws(9216, 3072, 80) == 3 * 9216 * 80 * 4
    for shape in [(4608, 3072, 32),     # short rows: 48 groups
                  (4096, 12288, 32),    # 256 tiles of 16 rows: one per compute unit
                  (4608, 12288, 0),     # no D
                  (4608, 12288, 112),   # rank above 96
                  (4096, 3072, 96),     # rank 96, one 16-row tile per compute unit
                  (4608, 12280, 32), (0, 12288, 32), (4608, 12288, 24)]:
        assert ws(*shape) == 0, shape
    for M, K, R in [(4608, 12288, 32), (4608, 3072, 32), (4100, 6144, 16)]:
        extra = (ws(M, K, R) + 255) // 256 * 256
        base_t = (((M + 15) // 16) * (K // 64) * 1024 + ((M + 127) // 128) * (K // 64) * 512
                  + (((M + 15) // 16) * ((R + 31) // 32) * 1024 + 255) // 256 * 256)
        assert L.svdq_linear_tiled_workspace_bytes(M, K, R) == base_t + extra
        C = (K + 127) // 128
        base_m = (((M + 15) // 16) * C * 1024 + ((M + 63) // 64) * C * 256
                  + (((M + 15) // 16) * ((R + 31) // 32) * 1024 + 255) // 256 * 256)
        assert L.svdq_linear_mx_workspace_bytes(M, K, R) == base_m + extra


def test_gemm_tiled_workspace_sizes():
    """The tiled GEMM's split along K: S partial 128 x 128 fp32 tiles per tile
    when the tiles fill at most a quarter of the resident slots and K holds at
    least 32 groups, S = slots / tiles capped at G / 16 and 8. Without a device the
    library takes 512 slots (2 per compute unit of MI355X); the GPU uses the
    kernel's own occupancy. A workspace below the size is refused."""
    L = _lib.lib
    ws = L.svdq_gemm_tiled_workspace_bytes
    # 16 x 8 tiles = a quarter of 512 slots, 180 groups: S = min(512 // 128, 11, 8) = 4
    assert ws(2048, 1024, 11520) == 4 * 128 * 128 * 128 * 4
    # 16 x 10 tiles: more than a quarter of 512 (on MI355X's 768 slots it splits)
    assert ws(2048, 1280, 11520) == 0
    # 8 x 5 tiles, K = 2560 (40 groups): S = min(12, 2, 8) = 2
    assert ws(1024, 640, 2560) == 2 * 40 * 128 * 128 * 4
    for shape in [(4608, 9216, 3072),    # 2592 tiles: no room to split
                  (2048, 1280, 1280),    # 20 groups
                  (2048, 1280, 1000), (0, 64, 4096), (64, 0, 4096)]:
        assert ws(*shape) == 0, shape
    need = ws(1024, 640, 2560)
    args = [A16, A16, A16, A16, A16, A16, 16, None, A16, 1, 1024, 640, 2560, 640, 0, 0x10000,
            need - 1, None]
    assert L.svdq_w4a4_gemm_lowrank_up_tiled(*args) == _lib.ERR_WORKSPACE
    args[15], args[16] = 0x10040, need
    assert L.svdq_w4a4_gemm_lowrank_up_tiled(*args) == _lib.ERR_ALIGN


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="only meaningful where no GPU is present")
def test_device_entry_points_report_no_device():
    L = _lib.lib
    assert L.svdq_quantize_act_lowrank_down(A16, 1, 16, 64, 64, A16, A16, 16, 64, A16, A16, A16, None) == _lib.ERR_NO_DEVICE
    assert _lib.last_error()
    args = [A16, A16, A16, A16, A16, A16, 16, None, A16, 1, 16, 16, 64, 16, 64, 0, None]
    assert L.svdq_w4a4_gemm_lowrank_up(*args) == _lib.ERR_NO_DEVICE
    assert L.svdq_gelu_tanh_f16(A16, A16, 8, None) == _lib.ERR_NO_DEVICE
    assert L.svdq_quantize_act_lowrank_down_mx(A16, 1, 16, 64, 64, A16, A16, 16, A16, A16, A16, None, 0, None) == _lib.ERR_NO_DEVICE
    assert L.svdq_mx_gemm_lowrank_up(A16, A16, A16, A16, A16, A16, 16, None, A16, 1, 16, 16, 64, 16, 0, None) == _lib.ERR_NO_DEVICE
    geo = [1, 8, 8, 64, 3, 3, 1, 1]
    assert L.svdq_quantize_act_lowrank_down_conv(A16, 1, *geo, A16, A16, 16, A16, A16, A16, None) == _lib.ERR_NO_DEVICE
    need_c = L.svdq_linear_workspace_bytes(64, 576, 16, 64)
    assert L.svdq_conv2d(A16, 1, *geo, A16, A16, A16, 16, A16, A16, None, A16, 1, 16, 0x10000,
                         need_c, 0, None) == _lib.ERR_NO_DEVICE
    assert L.svdq_quantize_act_lowrank_down_conv_mx(A16, 1, *geo, A16, A16, 16, A16, A16, A16, None) == _lib.ERR_NO_DEVICE
    assert L.svdq_quantize_act_lowrank_down_conv_tiled(A16, 1, *geo, A16, A16, 16, A16, A16, A16,
                                                       None) == _lib.ERR_NO_DEVICE
    need_ct = L.svdq_linear_tiled_workspace_bytes(64, 576, 16)
    assert L.svdq_conv2d_tiled(A16, 1, *geo, A16, A16, A16, 16, A16, A16, None, A16, 1, 16,
                               0x10000, need_ct, 0, None) == _lib.ERR_NO_DEVICE
    assert L.svdq_conv2d_tiled(A16, 1, *geo, A16, A16, A16, 16, A16, A16, None, A16, 1, 16,
                               0x10000, need_ct - 1, 0, None) == _lib.ERR_WORKSPACE
    need_cm = L.svdq_linear_mx_workspace_bytes(64, 576, 16)
    assert L.svdq_conv2d_mx(A16, 1, *geo, A16, A16, A16, 16, A16, A16, None, A16, 1, 16, 0x10000,
                            need_cm, 0, None) == _lib.ERR_NO_DEVICE


def test_noalloc_rejects_layers_beyond_its_buffer():
    """svdq_linear_noalloc refuses, before any HIP call, a layer whose
    intermediates exceed its static buffer, and reports bad sizes as svdq_linear."""
    lib = _lib.lib
    M, K = 1 << 20, 4096                       # 2 GiB of codes alone
    assert lib.svdq_linear_workspace_bytes(M, K, 0, 64) > _lib.NOALLOC_MAX_BYTES
    s = lib.svdq_linear_noalloc(None, _lib.F16, K, None, None, None, 0, None, None, None, None,
                                _lib.F16, 64, M, K, 64, 64, 0, None)
    assert s == _lib.ERR_WORKSPACE and "static buffer" in _lib.last_error()
    s = lib.svdq_linear_noalloc(None, _lib.F16, 64, None, None, None, 0, None, None, None, None,
                                _lib.F16, 64, 16, 60, 64, 64, 0, None)
    assert s == _lib.ERR_GROUP and _lib.last_error().startswith("svdq_linear_noalloc")
