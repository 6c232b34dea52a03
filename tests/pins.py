"""Pins for the CPU oracle: checks against facts the oracle itself does not encode.

Each ``check_*`` takes the oracle module ``O`` and raises AssertionError when
the oracle disagrees with a closed form, an invariant, a hand-derived golden
value or an independent brute-force computation. ``test_oracle_pins.py`` runs
them on the real oracle; ``test_pin_sensitivity.py`` plants mistakes in the
oracle (on the CPU) and shows that some check fails for each.

The brute-force helpers below are written in plain Python (``struct`` for the
IEEE roundings, ``round`` for half-to-even) and call nothing in the oracle.
"""
from __future__ import annotations

import math
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# plain-Python IEEE helpers (independent of numpy and of the oracle)


def py_f32(x: float) -> float:
    """Round a Python float (binary64) to binary32, nearest-even."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def py_f16(x: float) -> float:
    """Round a Python float (binary64) to binary16, nearest-even."""
    return struct.unpack("<e", struct.pack("<e", x))[0]


def py_f16_bits(x: float) -> int:
    return struct.unpack("<H", struct.pack("<e", x))[0]


def bits_f32(h: int) -> float:
    return struct.unpack("<f", struct.pack("<I", h))[0]


def bits_f16(h: int) -> float:
    return struct.unpack("<e", struct.pack("<H", h))[0]


def py_quantize_group(vals):
    """One group through the quantizer reading, using only Python floats.

    fp32 division and multiplication are done in binary64 and rounded to
    binary32: for a quotient or product of two binary32 values, binary64
    carries more than 2*24+2 bits, so this double rounding equals the
    correctly rounded binary32 result."""
    v = [py_f32(x) for x in vals]
    a = max(abs(x) for x in v)
    s32 = min(py_f32(a / 7.0), 65504.0)
    s = py_f16(s32)
    inv = 0.0 if s == 0.0 else py_f32(1.0 / s)
    q = []
    for x in v:
        t = py_f32(x * inv)
        r = round(t)            # Python rounds half to even
        q.append(max(-7, min(7, int(r))))
    return q, s


# --------------------------------------------------------------------------
# golden fixtures


def load_quantizer_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "quantizer_cases.txt")) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = dict(name=tok[1], v=[0.0] * 64, scale=None, codes=[0] * 64, bytes=[0] * 32)
            elif tok[0] == "v":
                cur["v"][int(tok[1])] = bits_f32(int(tok[2], 16))
            elif tok[0] == "scale":
                cur["scale"] = int(tok[1], 16)
            elif tok[0] == "codes":
                for t in tok[1:]:
                    i, c = t.split(":")
                    cur["codes"][int(i)] = int(c)
            elif tok[0] == "bytes":
                for t in tok[1:]:
                    i, c = t.split(":")
                    cur["bytes"][int(i)] = int(c, 16)
            elif tok[0] == "end":
                cases.append(cur)
                cur = None
    return cases


def check_golden_quantizer(O):
    cases = load_quantizer_cases()
    assert len(cases) >= 8
    V = np.array([c["v"] for c in cases], dtype=np.float32)
    q, s = O.quantize_groups(V)
    packed = O.pack_nibbles(q)
    for i, c in enumerate(cases):
        got_s = int(np.asarray(s[i, 0], dtype=np.float16).view(np.uint16))
        assert got_s == c["scale"], (c["name"], hex(got_s), hex(c["scale"]))
        assert list(q[i]) == c["codes"], (c["name"], list(q[i]))
        assert list(packed[i]) == c["bytes"], (c["name"], [hex(b) for b in packed[i]])


def check_golden_smoothing(O):
    rows = []
    with open(os.path.join(GOLDEN, "smoothing_cases.txt")) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                rows.append([float(t) for t in line.split()])
    xa = np.array([r[0] for r in rows])
    # a W whose row maxima are the fixture values, sign mixed on purpose
    W = np.zeros((len(rows), 3), dtype=np.float32)
    for j, r in enumerate(rows):
        W[j, j % 3] = -r[1] if j % 2 else r[1]
        W[j, (j + 1) % 3] = 0.5 * r[1]
    lam = O.smoothing_factors(xa, W)
    inv = O.inv_smoothing(lam)
    for j, r in enumerate(rows):
        assert float(lam[j]) == r[2], (j, float(lam[j]), r[2])
        assert float(inv[j]) == py_f32(r[3]), (j, float(inv[j]), r[3])


def check_golden_tiny_linear(O):
    d = {}
    with open(os.path.join(GOLDEN, "linear_tiny.txt")) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                tok = line.split()
                d.setdefault(tok[0], []).append(tok[1:])
    X = np.zeros((1, 64), dtype=np.float32)
    for i, v in d["x"]:
        X[0, int(i)] = float(v)
    W = np.zeros((64, 1), dtype=np.float32)
    for i, h in d["w"]:
        W[int(i), 0] = bits_f32(int(h, 16))
    lam = np.ones(64, dtype=np.float32)
    prep = O.prepare(W, lam, rank=0)
    ws = int(np.asarray(prep["w_scales"][0, 0], dtype=np.float16).view(np.uint16))
    assert ws == int(d["w_scale"][0][0], 16), hex(ws)
    codes = O.unpack_nibbles(prep["w_codes"])[0]
    for t in d["w_codes"][0]:
        i, c = t.split(":")
        assert int(codes[int(i)]) == int(c)
    Y, parts = O.linear(X, prep["inv_smooth"], prep["L1"], prep["L2"], prep["w_codes"],
                        prep["w_scales"], None, "f32", return_parts=True)
    assert int(parts["P"][0, 0, 0]) == int(d["P"][0][0])
    assert float(Y[0, 0]) == float(d["y"][0][0]), float(Y[0, 0])


# --------------------------------------------------------------------------
# rounding


def check_fp16_single_rounding(O):
    """fp64 -> fp16 must round once (not through fp32)."""
    x = 1.0 + 2.0 ** -11 + 2.0 ** -30         # just above the halfway point
    assert float(O.to_f16(np.float64(x))) == 1.0 + 2.0 ** -10
    assert float(O.to_f16(np.float64(1.0 + 2.0 ** -11))) == 1.0               # tie -> even
    assert float(O.to_f16(np.float64(1.0 + 3 * 2.0 ** -11))) == 1.0 + 2.0 ** -9  # tie -> even
    assert float(O.to_f16(np.float64(65519.99))) == 65504.0


# --------------------------------------------------------------------------
# quantizer


def _random_groups(rng, n):
    """Groups spanning normal, tiny (subnormal-scale), huge (saturating) and tie-heavy values."""
    out = []
    for i in range(n):
        kind = i % 5
        if kind == 0:
            v = rng.standard_normal(64)
        elif kind == 1:
            v = rng.standard_normal(64) * 1e-6
        elif kind == 2:
            v = rng.standard_normal(64) * 3e5
        elif kind == 3:
            v = rng.integers(-14, 15, 64) * 0.5          # many exact .5 ties at scale 1
            v[0] = 7.0
        else:
            v = rng.standard_normal(64) * 10.0 ** rng.uniform(-3, 3)
            v[rng.integers(0, 64, 3)] = 0.0
        out.append(v)
    return np.array(out, dtype=np.float32)


def check_quantizer_bruteforce(O, n=300, seed=7):
    V = _random_groups(np.random.default_rng(seed), n)
    q, s = O.quantize_groups(V)
    for i in range(n):
        qq, ss = py_quantize_group([float(x) for x in V[i]])
        assert list(q[i]) == qq, (i, list(q[i]), qq)
        assert float(s[i, 0]) == ss, (i, float(s[i, 0]), ss)


def check_roundtrip_bound(O, seed=11):
    """|v - s q| <= (s/2)(1 + 2^-19) wherever s is a normal fp16 and not saturated."""
    rng = np.random.default_rng(seed)
    V = (rng.standard_normal((400, 64)) * 10.0 ** rng.uniform(-3, 3, (400, 1))).astype(np.float32)
    q, s = O.quantize_groups(V)
    sf = s.astype(np.float64)[:, 0]
    normal = (sf >= 2.0 ** -14) & (sf < 65504.0)
    assert normal.sum() > 300
    err = np.abs(V.astype(np.float64) - sf[:, None] * q.astype(np.float64))
    bound = 0.5 * sf[:, None] * (1 + 2.0 ** -19)
    assert np.all(err[normal] <= bound[normal])
    # the largest element of each group maps to +-7 or +-6 (s rounds to fp16,
    # so a/s lies in [7(1-2^-11), 7(1+2^-11)])
    amax = np.abs(q[normal]).max(axis=1)
    assert np.all(amax == 7)


def check_invariants(O, seed=13):
    rng = np.random.default_rng(seed)
    V = (rng.standard_normal((64, 64)) * 0.3).astype(np.float32)
    q, s = O.quantize_groups(V)
    qn, sn = O.quantize_groups(-V)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for k in (-3, 2, 5):                       # power-of-two scaling, normal range
        qk, sk = O.quantize_groups(V * np.float32(2.0 ** k))
        assert np.array_equal(qk, q)
        assert np.array_equal(sk.astype(np.float64), s.astype(np.float64) * 2.0 ** k)
    z = np.zeros((1, 64), dtype=np.float32)
    qz, sz = O.quantize_groups(z)
    assert not qz.any() and float(sz[0, 0]) == 0.0
    one = np.zeros((2, 64), dtype=np.float32)
    one[0, 17], one[1, 40] = 0.123, -5.5
    q1, _ = O.quantize_groups(one)
    assert q1[0, 17] == 7 and q1[1, 40] == -7 and np.count_nonzero(q1) == 2
    # codes of one group do not depend on any other group
    W2 = V.reshape(1, -1)
    qa, sa = O.quantize_groups(W2)
    assert np.array_equal(qa.reshape(64, 64), q)


def check_pack_roundtrip(O):
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = O.unpack_nibbles(b)
    assert q.min() == -8 and q.max() == 7
    assert np.array_equal(O.pack_nibbles(q), b)
    # element 2j is the low nibble
    qq = np.array([[1, 2, -1, -8]], dtype=np.int8)
    assert list(O.pack_nibbles(qq)[0]) == [0x21, 0x8F]


# --------------------------------------------------------------------------
# SVD split


def _smoothed(rng, K, N):
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    W[rng.choice(K, max(1, K // 50), replace=False)] *= 10
    X = rng.standard_normal((32, K)).astype(np.float32)
    X[:, rng.choice(K, max(1, K // 50), replace=False)] *= 20
    lam = None
    return X, W, lam


def check_eym(O, seed=17):
    """Eckart-Young-Mirsky: the rank-r truncation leaves exactly the dropped
    singular values (chattools.cn overview, technical principles, EYM item)."""
    rng = np.random.default_rng(seed)
    for (K, N, r) in [(96, 64, 8), (64, 160, 16), (128, 128, 32)]:
        X, W, _ = _smoothed(rng, K, N)
        lam = O.smoothing_factors(np.abs(X).max(0), W)
        What = O.smooth_weight(W, lam)
        U, S, Vt = O.svd_canonical(What)
        # the singular values against an independent symmetric eigen-solver
        ev = np.sort(np.linalg.eigvalsh(What.T @ What if K >= N else What @ What.T))[::-1]
        assert np.allclose(S ** 2, ev[:len(S)], rtol=1e-9, atol=1e-12 * ev[0])
        L1, L2 = O.lowrank_factors_f64(U, S, Vt, r)
        E = What - L1 @ L2
        tail = math.sqrt(float(np.sum(S[r:] ** 2)))
        assert abs(np.linalg.norm(E) - tail) <= 1e-10 * tail
        assert abs(np.linalg.norm(E, 2) - S[r]) <= 1e-10 * S[r]
        # any rank-r pair, including the fp16 pair, cannot beat the optimum,
        # and the fp16 pair stays within the fp16 rounding of the optimum
        H1, H2 = O.lowrank_factors(U, S, Vt, r)
        Eh = O.residual(What, H1, H2)
        rnd = np.linalg.norm(H1.astype(np.float64) @ H2.astype(np.float64) - L1 @ L2)
        assert np.linalg.norm(Eh) >= tail * (1 - 1e-12)
        assert np.linalg.norm(Eh) <= tail + rnd + 1e-12
        # canonical sign: the largest-magnitude entry of each u_i is positive
        idx = np.argmax(np.abs(U), axis=0)
        assert np.all(U[idx, np.arange(U.shape[1])] > 0)


def check_sigma_split(O, seed=19):
    """The branch carries Sigma^(1/2) on each side: L1^T L1 = L2 L2^T = Sigma_r."""
    rng = np.random.default_rng(seed)
    _, W, _ = _smoothed(rng, 128, 96)
    U, S, Vt = O.svd_canonical(W.astype(np.float64))
    L1, L2 = O.lowrank_factors_f64(U, S, Vt, 12)
    assert np.allclose(L1.T @ L1, np.diag(S[:12]), atol=1e-12 * S[0])
    assert np.allclose(L2 @ L2.T, np.diag(S[:12]), atol=1e-12 * S[0])


def check_full_rank(O, seed=23):
    """r = min(K, N) with fp64 factors reconstructs What, and the smoothing cancels
    (Xhat . What = X . W up to the fp32 rounding of 1/lam)."""
    rng = np.random.default_rng(seed)
    for (K, N) in [(64, 48), (48, 80)]:
        X, W, _ = _smoothed(rng, K, N)
        lam = O.smoothing_factors(np.abs(X).max(0), W)
        What = O.smooth_weight(W, lam)
        U, S, Vt = O.svd_canonical(What)
        L1, L2 = O.lowrank_factors_f64(U, S, Vt, min(K, N))
        assert np.linalg.norm(What - L1 @ L2) <= 1e-12 * np.linalg.norm(What)
        inv = O.inv_smoothing(lam)
        xh = X.astype(np.float64) * inv.astype(np.float64)[None, :]
        ref = X.astype(np.float64) @ W.astype(np.float64)
        got = xh @ What
        assert np.max(np.abs(got - ref)) <= 2e-7 * np.max(np.abs(X) @ np.abs(W))
        # and with the oracle's own fp32 Xhat
        xh32 = O.smooth_activation(X, inv).astype(np.float64)
        assert np.max(np.abs(xh32 @ What - ref)) <= 4e-7 * np.max(np.abs(X) @ np.abs(W))


def check_reconstruction(O, seed=29):
    """L1.L2 + R = What to fp64 precision, for any rank."""
    rng = np.random.default_rng(seed)
    X, W, _ = _smoothed(rng, 128, 64)
    lam = O.smoothing_factors(np.abs(X).max(0), W)
    for r in (0, 1, 7, 32):
        p = O.prepare(W, lam, r)
        rec = p["L1"].astype(np.float64) @ p["L2"].astype(np.float64) + p["R"]
        assert np.max(np.abs(rec - p["What"])) <= 1e-14 * np.max(np.abs(p["What"]))
        assert p["L1"].shape == (128, r) and p["L2"].shape == (r, 64)
        assert p["w_codes"].shape == (64, 64) and p["w_scales"].shape == (64, 2)


# --------------------------------------------------------------------------
# online part: brute force on tiny shapes


def _py_unpack(b):
    out = []
    for byte in b:
        lo, hi = int(byte) & 15, (int(byte) >> 4) & 15
        out += [lo - 16 if lo >= 8 else lo, hi - 16 if hi >= 8 else hi]
    return out


def check_partials_bruteforce(O, seed=31):
    """Triple loops in Python give the same P, D and Y as the oracle."""
    rng = np.random.default_rng(seed)
    for (M, K, N, r) in [(8, 64, 16, 4), (5, 128, 7, 2)]:
        X = (rng.standard_normal((M, K)) * 2).astype(np.float32)
        W = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
        lam = O.smoothing_factors(np.abs(X).max(0), W)
        p = O.prepare(W, lam, r)
        bias = (rng.standard_normal(N) * 0.1).astype(np.float32)
        Y, parts = O.linear(X, p["inv_smooth"], p["L1"], p["L2"], p["w_codes"], p["w_scales"],
                            bias, "f32", return_parts=True)
        G = K // 64
        inv = [float(t) for t in p["inv_smooth"]]
        L1 = p["L1"].astype(np.float64).tolist()
        L2 = p["L2"].astype(np.float64).tolist()
        wq = [_py_unpack(p["w_codes"][n]) for n in range(N)]
        ws = p["w_scales"].astype(np.float64).tolist()
        for m in range(M):
            xh = [py_f32(float(X[m, k]) * inv[k]) for k in range(K)]
            qs = [py_quantize_group(xh[64 * g:64 * g + 64]) for g in range(G)]
            qx = sum((t[0] for t in qs), [])
            sx = [t[1] for t in qs]
            x16 = [py_f16(v) for v in xh]
            D = [sum(x16[k] * L1[k][j] for k in range(K)) for j in range(r)]
            D16 = [py_f16(d) for d in D]
            for n in range(N):
                acc = 0.0
                for g in range(G):
                    Pg = sum(qx[k] * wq[n][k] for k in range(64 * g, 64 * g + 64))
                    assert Pg == int(parts["P"][m, n, g]), (m, n, g)
                    acc += sx[g] * ws[n][g] * Pg
                lr = sum(D16[j] * L2[j][n] for j in range(r))
                y = acc + lr + float(bias[n])
                assert abs(y - float(Y[m, n])) <= 1e-6 * max(1.0, abs(y)), (m, n, y, float(Y[m, n]))
            for j in range(r):
                assert abs(D[j] - parts["D"][m, j]) <= 1e-12 * max(1.0, abs(D[j]))


def check_dense_identity(O, seed=37):
    """sum_g s_x s_w P equals the dense product of the dequantized operands."""
    rng = np.random.default_rng(seed)
    M, K, N = 24, 192, 40
    X = rng.standard_normal((M, K)).astype(np.float32)
    W = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    lam = O.smoothing_factors(np.abs(X).max(0), W)
    p = O.prepare(W, lam, 4)
    _, parts = O.linear(X, p["inv_smooth"], p["L1"], p["L2"], p["w_codes"], p["w_scales"],
                        None, "f32", return_parts=True)
    xq = O.dequantize_groups(O.unpack_nibbles(parts["a_codes"]), parts["a_scales"])
    wq = O.dequantize_groups(O.unpack_nibbles(p["w_codes"]), p["w_scales"])      # N x K
    dense = xq @ wq.T
    assert np.max(np.abs(dense - parts["acc"])) <= 1e-12 * np.max(np.abs(dense))


def check_lora(O, seed=41):
    """LoRA joins the branch without touching the codes, and adds exactly X.A.B.scale
    up to the fp16 roundings of Xhat, lam(.)A and D (chattools.cn overview, main
    features, LoRA item; SVDQuant abstract)."""
    rng = np.random.default_rng(seed)
    M, K, N, r, rl, scale = 16, 128, 48, 8, 6, 0.75
    X = rng.standard_normal((M, K)).astype(np.float32)
    X[:, 3] *= 20
    W = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    lam = O.smoothing_factors(np.abs(X).max(0), W)
    p = O.prepare(W, lam, r)
    A = (rng.standard_normal((K, rl)) * 0.05).astype(np.float16)
    B = (rng.standard_normal((rl, N)) * 0.05).astype(np.float16)
    L1n, L2n = O.concat_lora(p["L1"], p["L2"], lam, A, B, scale)
    assert np.array_equal(L1n[:, :r], p["L1"]) and np.array_equal(L2n[:r], p["L2"])
    # the prep's codes are reused as they are
    Y0, parts0 = O.linear(X, p["inv_smooth"], p["L1"], p["L2"], p["w_codes"], p["w_scales"],
                          None, "f32", return_parts=True)
    Y1, parts1 = O.linear(X, p["inv_smooth"], L1n, L2n, p["w_codes"], p["w_scales"],
                          None, "f32", return_parts=True)
    assert np.array_equal(parts0["a_codes"], parts1["a_codes"])
    delta = parts1["lr"] - parts0["lr"]
    ref = X.astype(np.float64) @ A.astype(np.float64) @ B.astype(np.float64) * scale
    env = (np.abs(X.astype(np.float64)) @ np.abs(A.astype(np.float64) * scale)
           @ np.abs(B.astype(np.float64)))
    # three fp16 roundings (x-hat, lam(.)A, D) and the fp32 1/lam: < 3.2 * 2^-11 relative
    assert np.all(np.abs(delta - ref) <= 3.2 * 2.0 ** -11 * env + 1e-12)
    assert np.max(np.abs(ref)) > 0.05 * np.max(np.abs(delta))


def check_method_sanity(O):
    """On the tiny workload (256 x 512 x 512, r = 16), the low-rank branch lowers
    the error against the exact X.W (SVDQuant abstract: the branch absorbs the
    outliers that make 4-bit quantization hard)."""
    import workloads as wl
    L, X, W = wl.layer_inputs(0, 0)
    lam = O.smoothing_factors(np.abs(X.astype(np.float64)).max(0), W)
    ref = X.astype(np.float64) @ W.astype(np.float64)
    errs = {}
    for r in (0, L.rank):
        p = O.prepare(W, lam, r)
        Y = O.linear(X, p["inv_smooth"], p["L1"], p["L2"], p["w_codes"], p["w_scales"], None, "f32")
        errs[r] = float(np.linalg.norm(Y.astype(np.float64) - ref) / np.linalg.norm(ref))
    assert errs[L.rank] < 0.9 * errs[0], errs


def check_method_sanity_dit(O):
    """E8 on the DiT fused-QKV workload (4608 x 3072 x 9216, r = 32): the
    low-rank branch lowers the error against the exact X.W on the same sampled
    rows. Smoothing is calibrated on all rows; one SVD serves both ranks."""
    import workloads as wl
    L, X, W = wl.layer_inputs(1, 0)
    lam = O.smoothing_factors(O.channel_absmax(X), W)
    svd = O.svd_canonical(O.smooth_weight(W, lam))
    rows = np.random.default_rng(8).choice(L.M, 48, replace=False)
    Xs = X[rows]
    ref = Xs.astype(np.float64) @ W.astype(np.float64)
    errs = {}
    for r in (0, L.rank):
        p = O.prepare(W, lam, r, svd=svd)
        Y = O.linear(Xs, p["inv_smooth"], p["L1"], p["L2"], p["w_codes"], p["w_scales"], None,
                     "f32")
        errs[r] = float(np.linalg.norm(Y.astype(np.float64) - ref) / np.linalg.norm(ref))
    assert errs[L.rank] < 0.95 * errs[0], errs


def check_gelu(O):
    x = np.array([0.0, 1.0, -1.0, 3.0, -3.0, 20.0, -20.0], dtype=np.float64)
    g = O.gelu_tanh(x).astype(np.float64)
    c = math.sqrt(2.0 / math.pi)
    for xi, gi in zip(x, g):
        ref = 0.5 * xi * (1.0 + math.tanh(c * (xi + 0.044715 * xi ** 3)))
        assert gi == py_f16(ref)
        # the tanh form stays within 1e-3 of the exact erf form
        exact = 0.5 * xi * (1.0 + math.erf(xi / math.sqrt(2.0)))
        assert abs(gi - exact) <= 1e-3 + 2 ** -10 * abs(exact)
    assert g[0] == 0.0 and g[5] == 20.0 and g[6] == 0.0


def check_linear_gelu(O):
    """The fused activation: GELU of the unrounded layer output, rounded once.
    Checked against an independent composition: the fp32 layer output, then a
    pure-Python tanh GELU, rounded to fp16 (double rounding, so at most one
    fp16 step apart, and equal almost everywhere)."""
    import workloads as wl
    L, X, W = wl.layer_inputs(0, 0)
    b = wl.bias(0, 0, L.N)
    lam = O.smoothing_factors(O.channel_absmax(X), W)
    p = O.prepare(W, lam, L.rank)
    args = (X[:24], p["inv_smooth"], p["L1"], p["L2"], p["w_codes"], p["w_scales"], b)
    Yg = O.linear(*args, "f16", activation="gelu_tanh").astype(np.float64)
    Y32 = O.linear(*args, "f32").astype(np.float64)
    c = math.sqrt(2.0 / math.pi)
    ref = np.array([[py_f16(0.5 * v * (1.0 + math.tanh(c * (v + 0.044715 * v ** 3)))) for v in row]
                    for row in Y32])
    diff = np.abs(Yg - ref)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14))) - 10)
    assert np.all(diff <= step), float(np.max(diff / step))
    assert np.mean(diff == 0) > 0.99
    # and it is not the plain layer: GELU changes the negative outputs
    assert np.any(np.abs(Yg - O.linear(*args, "f16").astype(np.float64)) > 0.1)


ALL_CHECKS = [
    check_fp16_single_rounding, check_golden_quantizer, check_golden_smoothing,
    check_golden_tiny_linear, check_quantizer_bruteforce, check_roundtrip_bound,
    check_invariants, check_pack_roundtrip, check_eym, check_sigma_split, check_full_rank,
    check_reconstruction, check_partials_bruteforce, check_dense_identity, check_lora,
    check_method_sanity, check_gelu, check_linear_gelu,
]

# pins too slow to repeat under every planted mutation (one full-size SVD)
SLOW_CHECKS = [check_method_sanity_dit]


# --------------------------------------------------------------------------
# MXFP4 variant (OCP Microscaling v1.0 reading of the pages' 4-bit float
# variant; taicenter.com news page on SVDQuant, hardware co-design section)

PY_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def py_e2m1_code(t: float) -> int:
    """E2M1 code of the Python float t: nearest magnitude by threshold
    comparisons (midpoints go to the even encoding), saturating, sign bit kept."""
    m = abs(t)
    # (midpoint, goes up on a tie): ties go to the even code of the two
    code = 0
    for mid, up_on_tie in ((0.25, False), (0.75, True), (1.25, False), (1.75, True),
                           (2.5, False), (3.5, True), (5.0, False)):
        if m > mid or (up_on_tie and m == mid):
            code += 1
    return code | (8 if math.copysign(1.0, t) < 0 else 0)


def py_mx_block(vals):
    """One 32-block through the MXFP4 reading in plain Python: (codes, e8m0)."""
    v = [py_f32(x) for x in vals]
    a = max(abs(x) for x in v)
    if a == 0.0:
        e = -127
    else:
        e = math.frexp(a)[1] - 1 - 2          # floor(log2 a) - 2
        e = max(-127, min(127, e))
    return [py_e2m1_code(x / 2.0 ** e) for x in v], e + 127


def load_mx_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "mx_cases.txt")) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = dict(name=tok[1], v=[0.0] * 32, codes=[0] * 32, bytes=[0] * 16)
            elif tok[0] == "v":
                cur["v"][int(tok[1])] = bits_f32(int(tok[2], 16))
            elif tok[0] == "e8m0":
                cur["e8m0"] = int(tok[1])
            elif tok[0] in ("codes", "bytes"):
                for t in tok[1:]:
                    i, c = t.split(":")
                    cur[tok[0]][int(i)] = int(c, 0)
            elif tok[0] == "end":
                cases.append(cur)
                cur = None
    return cases


def check_golden_mx(O):
    cases = load_mx_cases()
    assert len(cases) >= 7
    V = np.array([c["v"] for c in cases], dtype=np.float32)
    codes, e8 = O.mx_quantize_blocks(V)
    packed = O.pack_codes4(codes)
    for i, c in enumerate(cases):
        assert int(e8[i, 0]) == c["e8m0"], (c["name"], int(e8[i, 0]))
        assert list(codes[i]) == c["codes"], (c["name"], list(codes[i]))
        assert list(packed[i]) == c["bytes"], (c["name"], [hex(b) for b in packed[i]])
        # decoding: every nonzero code is +-magnitude * 2^(byte-127)
        dec = O.mx_dequantize_blocks(codes[i:i + 1], e8[i:i + 1])[0]
        for k in range(32):
            cc = c["codes"][k]
            want = (-1 if cc & 8 else 1) * PY_E2M1[cc & 7] * 2.0 ** (c["e8m0"] - 127)
            assert dec[k] == want, (c["name"], k, dec[k], want)


def check_golden_mx_linear(O):
    d = {}
    with open(os.path.join(GOLDEN, "mx_linear_tiny.txt")) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                tok = line.split()
                d.setdefault(tok[0], []).append(tok[1:])
    X = np.zeros((1, 64), dtype=np.float32)
    for i, v in d["x"]:
        X[0, int(i)] = float(v)
    W = np.zeros((64, 1), dtype=np.float32)
    for i, h in d["w"]:
        W[int(i), 0] = bits_f32(int(h, 16))
    lam = np.ones(64, dtype=np.float32)
    p = O.mx_prepare(W, lam, rank=0)
    assert [int(t) for t in p["w_e8m0"][0]] == [int(t) for t in d["w_e8m0"][0]]
    wc = O.unpack_codes4(p["w_codes"])[0]
    want = [0] * 64
    for t in d["w_codes"][0]:
        i, c = t.split(":")
        want[int(i)] = int(c)
    assert list(wc) == want
    Y, parts = O.mx_linear(X, p["inv_smooth"], p["L1"], p["L2"], p["w_codes"], p["w_e8m0"],
                           None, "f32", return_parts=True)
    assert [int(t) for t in parts["a_e8m0"][0]] == [int(t) for t in d["x_e8m0"][0]]
    xc = O.unpack_codes4(parts["a_codes"])[0]
    want = [0] * 64
    for t in d["x_codes"][0]:
        i, c = t.split(":")
        want[int(i)] = int(c)
    assert list(xc) == want
    assert float(Y[0, 0]) == float(d["y"][0][0]), float(Y[0, 0])


def _random_mx_blocks(rng, n):
    """Blocks of normal, tiny, huge, midpoint-heavy and signed-zero values."""
    out = []
    for i in range(n):
        kind = i % 6
        if kind == 0:
            v = rng.standard_normal(32)
        elif kind == 1:
            v = rng.standard_normal(32) * 1e-30
        elif kind == 2:
            v = rng.standard_normal(32) * 1e30
        elif kind == 3:   # exact midpoints and grid points at one scale
            v = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 3.0], 32)
            v *= rng.choice([-1.0, 1.0], 32) * 2.0 ** int(rng.integers(-20, 20))
        elif kind == 4:
            v = rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 6)
            v[rng.integers(0, 32, 4)] = -0.0
        else:
            v = rng.standard_normal(32) * 1e-40       # subnormal fp32
        out.append(v)
    return np.array(out, dtype=np.float32)


def check_mx_bruteforce(O, n=360, seed=43):
    V = _random_mx_blocks(np.random.default_rng(seed), n)
    codes, e8 = O.mx_quantize_blocks(V)
    for i in range(n):
        cc, ee = py_mx_block([float(x) for x in V[i]])
        assert list(codes[i]) == cc, (i, list(codes[i]), cc)
        assert int(e8[i, 0]) == ee, (i, int(e8[i, 0]), ee)


def check_mx_roundtrip_bound(O, seed=47):
    """|v - deq| <= max(2^e / 4, |v| / 4): half an E2M1 step below 2, a quarter
    of |v| from 2 up, and under |v|/4 in the saturated band (6, 8) * 2^e."""
    rng = np.random.default_rng(seed)
    V = (rng.standard_normal((500, 32)) * 10.0 ** rng.uniform(-8, 8, (500, 1))).astype(np.float32)
    codes, e8 = O.mx_quantize_blocks(V)
    deq = O.mx_dequantize_blocks(codes, e8)
    s = np.ldexp(1.0, e8.astype(np.int64) - 127)
    v = V.astype(np.float64)
    err = np.abs(v - deq)
    bound = np.maximum(np.repeat(s, 32, axis=1) / 4, np.abs(v) / 4)
    assert np.all(err <= bound)
    # the block maximum lands in [4, 8) * 2^e, so its code is 6 or 7
    amax_code = (codes & 7).max(axis=1)
    assert np.all(amax_code >= 6)


def check_mx_invariants(O, seed=53):
    rng = np.random.default_rng(seed)
    V = (rng.standard_normal((40, 64)) * 0.3).astype(np.float32)
    c, e = O.mx_quantize_blocks(V)
    assert c.shape == (40, 64) and e.shape == (40, 2)
    cn, en = O.mx_quantize_blocks(-V)
    assert np.array_equal(cn, c ^ 8) and np.array_equal(en, e)      # sign is bit 3
    for k in (-9, 3, 40):                     # power-of-two scaling shifts only e
        ck, ek = O.mx_quantize_blocks(V * np.float32(2.0 ** k))
        assert np.array_equal(ck, c)
        assert np.array_equal(ek.astype(np.int64), e.astype(np.int64) + k)
    # blocks are independent, and run along the last axis
    c2, _ = O.mx_quantize_blocks(V.reshape(-1, 32))
    assert np.array_equal(c2.reshape(40, 64), c)
    Vb = V.copy()
    Vb[:, 32:] *= 1000
    cb, eb = O.mx_quantize_blocks(Vb)
    assert np.array_equal(cb[:, :32], c[:, :32]) and np.array_equal(eb[:, 0], e[:, 0])
    # pack: element 2j in the low nibble
    assert list(O.pack_codes4(np.array([[1, 2, 15, 8]], np.uint8))[0]) == [0x21, 0x8F]
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(O.pack_codes4(O.unpack_codes4(b)), b)


def check_mx_linear_bruteforce(O, seed=59):
    """Python loops over the plain-Python block quantizer give the oracle's
    codes, exponents and Y; R's blocks run down K for each output column."""
    rng = np.random.default_rng(seed)
    for (M, K, N, r) in [(4, 64, 6, 3), (3, 128, 5, 0)]:
        X = (rng.standard_normal((M, K)) * 2).astype(np.float32)
        X[:, 5] *= 30
        W = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
        lam = O.smoothing_factors(np.abs(X).max(0), W)
        p = O.mx_prepare(W, lam, r)
        bias = (rng.standard_normal(N) * 0.1).astype(np.float32)
        Y, parts = O.mx_linear(X, p["inv_smooth"], p["L1"], p["L2"], p["w_codes"], p["w_e8m0"],
                               bias, "f32", return_parts=True)
        inv = [float(t) for t in p["inv_smooth"]]
        lamf = [float(t) for t in lam]
        L1 = p["L1"].astype(np.float64).tolist()
        L2 = p["L2"].astype(np.float64).tolist()
        nb = K // 32

        def deq(codes, e8):
            return [(-1 if c & 8 else 1) * PY_E2M1[c & 7] * 2.0 ** (e8[k // 32] - 127)
                    for k, c in enumerate(codes)]

        wdeq = []
        for n in range(N):
            Rcol = [py_f32(lamf[k] * float(W[k, n]) - sum(L1[k][j] * L2[j][n] for j in range(r)))
                    for k in range(K)]
            cs, es = [], []
            for b in range(nb):
                cc, ee = py_mx_block(Rcol[32 * b:32 * b + 32])
                cs += cc
                es.append(ee)
            assert list(O.unpack_codes4(p["w_codes"][n])) == cs, n
            assert [int(t) for t in p["w_e8m0"][n]] == es, n
            wdeq.append(deq(cs, es))
        for m in range(M):
            xh = [py_f32(float(X[m, k]) * inv[k]) for k in range(K)]
            cs, es = [], []
            for b in range(nb):
                cc, ee = py_mx_block(xh[32 * b:32 * b + 32])
                cs += cc
                es.append(ee)
            assert list(O.unpack_codes4(parts["a_codes"][m])) == cs, m
            assert [int(t) for t in parts["a_e8m0"][m]] == es, m
            xd = deq(cs, es)
            D16 = [py_f16(sum(py_f16(xh[k]) * L1[k][j] for k in range(K))) for j in range(r)]
            for n in range(N):
                y = (sum(xd[k] * wdeq[n][k] for k in range(K))
                     + sum(D16[j] * L2[j][n] for j in range(r)) + float(bias[n]))
                assert abs(y - float(Y[m, n])) <= 1e-6 * max(1.0, abs(y)), (m, n, y, float(Y[m, n]))


def check_mx_method_sanity(O):
    """MXFP4 on the tiny workload: the low-rank branch lowers the error against
    the exact X.W, and the error is of the same order as the INT4 path's."""
    import workloads as wl
    L, X, W = wl.layer_inputs(0, 0)
    lam = O.smoothing_factors(np.abs(X.astype(np.float64)).max(0), W)
    ref = X.astype(np.float64) @ W.astype(np.float64)
    errs = {}
    for r in (0, L.rank):
        p = O.mx_prepare(W, lam, r)
        Y = O.mx_linear(X, p["inv_smooth"], p["L1"], p["L2"], p["w_codes"], p["w_e8m0"], None, "f32")
        errs[r] = float(np.linalg.norm(Y.astype(np.float64) - ref) / np.linalg.norm(ref))
    p = O.prepare(W, lam, L.rank)
    Yi = O.linear(X, p["inv_smooth"], p["L1"], p["L2"], p["w_codes"], p["w_scales"], None, "f32")
    e_int4 = float(np.linalg.norm(Yi.astype(np.float64) - ref) / np.linalg.norm(ref))
    assert errs[L.rank] < 0.9 * errs[0], errs
    assert 0.25 * e_int4 < errs[L.rank] < 4 * e_int4, (errs, e_int4)


ALL_CHECKS += [check_golden_mx, check_golden_mx_linear, check_mx_bruteforce,
               check_mx_roundtrip_bound, check_mx_invariants, check_mx_linear_bruteforce,
               check_mx_method_sanity]


# --------------------------------------------------------------------------
# 4-bit weight-only baseline (W4A16): reading of the SVDQuant abstract's
# comparison baseline (ai-digest.ru page)


def check_golden_w4a16(O):
    d = {}
    with open(os.path.join(GOLDEN, "w4a16_tiny.txt")) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                tok = line.split()
                d.setdefault(tok[0], []).append(tok[1:])
    X = np.zeros((1, 64), dtype=np.float16)
    for i, v in d["x"]:
        X[0, int(i)] = float(v)
    W = np.zeros((64, 1), dtype=np.float32)
    for i, h in d["w"]:
        W[int(i), 0] = bits_f32(int(h, 16))
    wc, ws = O.w4a16_prepare(W)
    deq = O.w4a16_dequant(wc, ws).astype(np.float64)
    assert [float(deq[0, 0]), float(deq[0, 1])] == [float(t) for t in d["deq"][0]]
    Y = O.w4a16_linear(X, wc, ws, None, "f32")
    assert float(Y[0, 0]) == float(d["y"][0][0]), float(Y[0, 0])


def check_w4a16_bruteforce(O, seed=61):
    """Python loops: the group quantizer of pins.py, fp16(s q) by struct, exact sums."""
    rng = np.random.default_rng(seed)
    for (M, K, N) in [(3, 64, 5), (2, 128, 3)]:
        X = (rng.standard_normal((M, K)) * 2).astype(np.float16)
        W = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
        W[3] *= 10
        bias = (rng.standard_normal(N) * 0.1).astype(np.float32)
        wc, ws = O.w4a16_prepare(W)
        Y = O.w4a16_linear(X, wc, ws, bias, "f32")
        for n in range(N):
            deq = []
            for g in range(K // 64):
                q, s = py_quantize_group([float(W[k, n]) for k in range(64 * g, 64 * g + 64)])
                deq += [py_f16(s * qq) for qq in q]
            for m in range(M):
                y = sum(float(X[m, k]) * deq[k] for k in range(K)) + float(bias[n])
                assert abs(y - float(Y[m, n])) <= 1e-6 * max(1.0, abs(y)), (m, n, y, float(Y[m, n]))


def check_w4a16_grid_identity(O, seed=67):
    """Weights already on the quantization grid (fp16 scale times an integer in
    -7..7, each product exact in fp16) come back unchanged, so the layer equals
    fp16(X) . W exactly."""
    rng = np.random.default_rng(seed)
    K, N, M = 128, 6, 4
    s = np.array([2.0 ** -6, 0.125, 0.75, 2.0 ** -10, 1.0, 0.5])
    q = rng.integers(-7, 8, size=(K, N)).astype(np.float64)
    q[0] = 7                                    # each group's absmax is 7 s ...
    q[64] = -7
    W = (q * s[None, :]).astype(np.float32)     # ... so Q recovers s and q exactly
    wc, ws = O.w4a16_prepare(W)
    deq = O.w4a16_dequant(wc, ws).astype(np.float64)
    assert np.array_equal(deq, W.T.astype(np.float64))
    X = rng.standard_normal((M, K)).astype(np.float16)
    Y = O.w4a16_linear(X, wc, ws, None, "f32").astype(np.float64)
    ref = (X.astype(np.float64) @ W.astype(np.float64)).astype(np.float32).astype(np.float64)
    assert np.array_equal(Y, ref)


def check_w4a16_sanity(O):
    """Against the W4A4 layer with lam = 1 and rank 0, whose weight codes are
    the same (Q of W itself): the weight-only layer, which does not quantize
    the activations, is closer to X.W on the tiny workload. (Against the
    smoothed W4A4 layer it is not: the outlier rows of W dominate its groups.)"""
    import workloads as wl
    L, X, W = wl.layer_inputs(0, 0)
    ref = X.astype(np.float16).astype(np.float64) @ W.astype(np.float64)
    wc, ws = O.w4a16_prepare(W)
    ones = np.ones(W.shape[0], dtype=np.float32)
    p = O.prepare(W, ones, 0)
    assert np.array_equal(p["w_codes"], wc) and np.array_equal(p["w_scales"], ws)
    e16 = np.linalg.norm(O.w4a16_linear(X, wc, ws, None, "f32").astype(np.float64) - ref)
    e44 = np.linalg.norm(O.linear(X, p["inv_smooth"], p["L1"], p["L2"], p["w_codes"],
                                  p["w_scales"], None, "f32").astype(np.float64) - ref)
    assert e16 < 0.8 * e44, (e16, e44)


ALL_CHECKS += [check_golden_w4a16, check_w4a16_bruteforce, check_w4a16_grid_identity,
               check_w4a16_sanity]


# --------------------------------------------------------------------------
# Convolutions as implicit GEMMs (reading of the pages' UNet applicability)


def _py_conv_direct(X, Wc, stride, pad):
    """Direct convolution by loops (Python floats)."""
    B, H, W, C = X.shape
    KH, KW, _, N = Wc.shape
    OH = (H + 2 * pad - KH) // stride + 1
    OW = (W + 2 * pad - KW) // stride + 1
    Y = np.zeros((B, OH, OW, N))
    for b in range(B):
        for oh in range(OH):
            for ow in range(OW):
                for n in range(N):
                    acc = 0.0
                    for kh in range(KH):
                        ih = oh * stride + kh - pad
                        if ih < 0 or ih >= H:
                            continue
                        for kw in range(KW):
                            iw = ow * stride + kw - pad
                            if iw < 0 or iw >= W:
                                continue
                            for c in range(C):
                                acc += float(X[b, ih, iw, c]) * float(Wc[kh, kw, c, n])
                    Y[b, oh, ow, n] = acc
    return Y


def check_im2col_is_the_convolution(O, seed=71):
    """X_col . W equals a direct convolution by loops (zero padding, strides 1
    and 2, odd sizes), and a 1 x 1 stride-1 convolution's X_col is X itself."""
    rng = np.random.default_rng(seed)
    for (B, H, W, C, N, KH, KW, s, p) in [(1, 5, 4, 3, 2, 3, 3, 1, 1), (2, 6, 7, 2, 3, 3, 3, 2, 1),
                                          (1, 4, 5, 2, 2, 2, 3, 1, 0)]:
        X = rng.standard_normal((B, H, W, C))
        Wc = rng.standard_normal((KH, KW, C, N))
        Y = O.im2col_nhwc(X, KH, KW, s, p) @ O.conv_weight_matrix(Wc)
        ref = _py_conv_direct(X, Wc, s, p).reshape(Y.shape)
        assert np.allclose(Y, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))
    X = rng.standard_normal((2, 3, 5, 4))
    assert np.array_equal(O.im2col_nhwc(X, 1, 1, 1, 0), X.reshape(-1, 4))
    # padding entries are exact zeros, and the column order is (kh, kw, c)
    cols = O.im2col_nhwc(np.ones((1, 2, 2, 1)), 3, 3, 1, 1)
    assert cols.shape == (4, 9)
    assert list(cols[0]) == [0, 0, 0, 0, 1, 1, 0, 1, 1]     # output (0, 0): taps hit rows/cols -1
    assert list(cols[3]) == [1, 1, 0, 1, 1, 0, 0, 0, 0]     # output (1, 1)


ALL_CHECKS += [check_im2col_is_the_convolution]
