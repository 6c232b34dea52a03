"""Benchmark of the SVDQuant W4A4 + low-rank linear layer on one MI355X.

One step = the whole hot path on one batch: K1 (smoothing, 4-bit quantization
and the low-rank down-projection of X) then K2 (the W4A4 GEMM with the fused
up-projection and bias). The default workload is the DiT fused-QKV projection:
X fp16 4608 x 3072 (4096 image + 512 text tokens), W 3072 x 9216, rank 32,
groups of 64, Y fp16. Inputs are seeded synthetic data with outlier channels;
weights are prepared on the host by the library before timing.

Prints one JSON line. ``value`` is the effective throughput 2*M*N*K / t of the
whole step (TOPS); ``roofline`` reports the dominant kernel (K2) against the
dense INT8 matrix-core peak, timed with HIP events on the stream it runs on;
``cpu_baseline`` times the CPU oracle on a bounded row sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense FP4 / FP6 MFMA
FP16_PEAK_TFLOPS = 2500.0      # MI355X dense fp16 MFMA
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
# HBM traffic of the GEMM kernel from committed rocprofv3 FETCH/WRITE passes,
# used only while the kernel's sources are unchanged since they were taken
PROFILE_PMC = {"int4": os.path.join(ROOT, "profiles", "k2_dit_qkv_pmc.json"),
               "mxfp4": os.path.join(ROOT, "profiles", "k2mx_dit_qkv_pmc.json"),
               "w4a16": os.path.join(ROOT, "profiles", "k2w16_dit_qkv_pmc.json")}
_CSRC = "bit_post_quantized_smooth_amd/csrc/"
K2_SOURCES = {"int4": [_CSRC + "k2_w4a4_gemm.hip", _CSRC + "k2_common.hpp",
                       _CSRC + "device_common.hpp"],
              "mxfp4": [_CSRC + "k2_mx_gemm.hip", _CSRC + "k2_common.hpp",
                        _CSRC + "device_common.hpp"],
              "w4a16": [_CSRC + "k2_w4a16_gemm.hip", _CSRC + "k2_common.hpp",
                        _CSRC + "device_common.hpp"]}


def k2_source_hash(fmt: str = "int4") -> str:
    h = hashlib.sha256()
    for p in K2_SOURCES[fmt]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=1, help="workload index (1 = DiT QKV)")
    ap.add_argument("--layer", type=int, default=0)
    ap.add_argument("--sets", type=int, default=4, help="rotating buffer sets (cold MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-overhead", action="store_true", help="skip the rank-0 comparison run")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain fp32 copy kernel of known size (for PMC scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--mlp", action="store_true",
                    help="time the DiT MLP pair instead: up-projection with the GELU fused into "
                         "its epilogue, then the down-projection")
    ap.add_argument("--format", choices=["int4", "mxfp4", "w4a16"], default="int4",
                    help="mxfp4: the MXFP4 variant (E2M1 codes, E8M0 exponent per 32) on the "
                         "scaled FP4 matrix core; w4a16: the 4-bit weight-only baseline of the "
                         "pages' speed comparison (fp16 activations, no low-rank branch)")
    ap.add_argument("--unfused-gelu", action="store_true",
                    help="with --mlp: plain up-projection, then the separate GELU kernel")
    ap.add_argument("--conv", type=int, default=None,
                    help="time UNet convolution I instead (NHWC, K1 on the implicit patch matrix, "
                         "then K2; INT4 format)")
    return ap.parse_args()


class Sets:
    """`n` independent device copies of one layer's inputs, weights and outputs."""

    def __init__(self, torch, X, prep, bias, n, y_dtype):
        import bit_post_quantized_smooth_amd as sq
        self.sq = sq
        self.mx = prep.fmt == "mxfp4"
        self.w16 = prep.fmt == "w4a16"
        M, K = X.shape
        self.M, self.K, self.N, self.R = M, K, prep.N, prep.rank
        G = K // 64
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16
                                       else np.ascontiguousarray(a)).to("cuda")
        if self.mx:
            wct, wet = sq.pack_mx_tiles(prep.w_codes, prep.w_scales, K)
        if self.w16:
            wct, wet = sq.pack_w4a16_tiles(prep.w_codes, prep.w_scales, K)
        self.sets = []
        for _ in range(n):
            s = dict(
                X=d(X), inv=d(prep.inv_smooth),
                L1p=d(prep.L1p) if self.R else None, L2t=d(prep.L2t) if self.R else None,
                b=None if bias is None else d(bias),
                D=torch.empty((M, max(self.R, 1)), dtype=torch.float32, device="cuda"),
                Y=torch.empty((M, self.N), dtype=torch.float16 if y_dtype == "f16" else torch.float32,
                              device="cuda"))
            if self.w16:
                s.update(wc=d(wct), ws=d(wet),
                         ac=torch.empty(sq.w4a16_x_tiled_bytes(M, K) // 2, dtype=torch.int16,
                                        device="cuda"), asc=None)
            elif self.mx:
                s.update(wc=d(wct), ws=d(wet),
                         ac=torch.empty(sq.mx_codes_tiled_bytes(M, K), dtype=torch.uint8, device="cuda"),
                         asc=torch.empty(sq.mx_exps_tiled_bytes(M, K), dtype=torch.uint8, device="cuda"))
            else:
                s.update(wc=d(prep.w_codes), ws=d(prep.w_scales),
                         ac=torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
                         asc=torch.empty((M, G), dtype=torch.int16, device="cuda"))
            self.sets.append(s)

    def k1(self, i):
        s = self.sets[i % len(self.sets)]
        if self.w16:
            self.sq.w4a16_tile_activation(s["X"], s["ac"])
            return
        f = (self.sq.quantize_act_lowrank_down_mx if self.mx
             else self.sq.quantize_act_lowrank_down)
        f(s["X"], s["inv"], s["L1p"], self.R, s["ac"], s["asc"], s["D"] if self.R else None)

    def k2(self, i):
        s = self.sets[i % len(self.sets)]
        if self.w16:
            self.sq.w4a16_gemm(s["ac"], s["wc"], s["ws"], s["b"], s["Y"], self.K)
            return
        f = self.sq.mx_gemm_lowrank_up if self.mx else self.sq.w4a4_gemm_lowrank_up
        f(s["ac"], s["asc"], s["wc"], s["ws"], s["D"] if self.R else None, s["L2t"], self.R, s["b"],
          s["Y"], self.K)


def time_steps(torch, sets, steps, warmup):
    """Two passes of `steps` steps after `warmup` untimed ones. The first,
    bracketed by synchronizations, is the step time: plain launches and
    nothing else on the stream. The second records HIP events around each
    launch on the launch stream for the per-kernel durations; an event record
    costs the stream a few microseconds, so that pass is not the step time."""
    for i in range(warmup):
        sets.k1(i)
        sets.k2(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        sets.k1(i)
        sets.k2(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        e0, e1, e2 = ev[i]
        e0.record()
        sets.k1(i)
        e1.record()
        sets.k2(i)
        e2.record()
    torch.cuda.synchronize()
    k1 = np.array([a.elapsed_time(b) for a, b, _ in ev]) * 1e-3
    k2 = np.array([b.elapsed_time(c) for _, b, c in ev]) * 1e-3
    return (t1 - t0) / steps, k1, k2


def copy_probe(torch):
    """A plain copy of known size (256 Mi fp32: 1 GiB read + 1 GiB written, more
    than the last-level cache), whose FETCH_SIZE and WRITE_SIZE counters scale
    the GEMM's and the pre-kernel's to bytes."""
    n = 256 << 20
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()


def event_gap(torch, reps=50):
    """Median time between two HIP events recorded back to back on the current
    stream with nothing between them: the overhead one event pair adds to a
    kernel timed between them."""
    gaps = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        gaps.append((a, b))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in gaps])) * 1e-3


def cpu_baseline(X, W, prep, bias, budget_s):
    """The oracle's online part (quantize X, down-projection, integer partials,
    scaled sum, up-projection, bias; or its MXFP4 counterpart) on chunks of rows
    until ~budget_s seconds."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    lam = O.smoothing_factors(O.channel_absmax(X), W)
    inv = O.inv_smoothing(lam)
    mx = prep.fmt == "mxfp4"
    w16 = prep.fmt == "w4a16"
    if w16:
        wc, ws = O.w4a16_prepare(W)
    elif mx:
        wc, ws = O.mx_quantize_residual_from_factors(W, lam, prep.L1, prep.L2)
    else:
        wc, ws = O.quantize_residual_from_factors(W, lam, prep.L1, prep.L2)
    M, K = X.shape
    N = W.shape[1]
    chunk = 32
    rows = 0
    t0 = time.perf_counter()
    while rows < M and time.perf_counter() - t0 < budget_s:
        r = slice(rows, min(M, rows + chunk))
        if w16:
            O.w4a16_linear(X[r], wc, ws, bias, "f16")
        else:
            (O.mx_linear if mx else O.linear)(X[r], inv, prep.L1, prep.L2, wc, ws, bias, "f16")
        rows = r.stop
    t = time.perf_counter() - t0
    return dict(value=2.0 * rows * N * K / t / 1e12, unit="TFLOPS" if (mx or w16) else "TOPS",
                cores=int(cores), kind="oracle",
                sample=f"first {rows} of {M} rows of the same layer, online part only "
                       f"({t:.1f} s, numpy fp64, chunks of {chunk} rows)")


def mlp_main(args, torch, sq, wl):
    """Step = the DiT MLP pair on one batch: K1 + K2 (+GELU) of the up-projection
    4608 x 3072 -> 12288, then K1 + K2 of the down-projection 12288 -> 3072."""
    (Lu, Xu, Wu), (Ld, _, Wd) = wl.layer_inputs(2, 0), wl.layer_inputs(2, 1)
    import oracle as O   # input synthesis only: GELU of the seeded pre-activations
    Xd_cal = O.gelu_tanh(wl.preactivation(2, 1, Ld.M, Ld.K, Ld.x_outlier_frac, Ld.x_outlier_scale))
    lam_u = sq.smoothing_factors(sq.channel_absmax(Xu), Wu)
    lam_d = sq.smoothing_factors(sq.channel_absmax(Xd_cal), Wd)
    up = sq.Linear(sq.prepare_weights(Wu, lam_u, Lu.rank),
                   activation=None if args.unfused_gelu else "gelu_tanh")
    down = sq.Linear(sq.prepare_weights(Wd, lam_d, Ld.rank))
    n = args.sets
    X = [torch.from_numpy(Xu).to("cuda") for _ in range(n)]
    H = [torch.empty((Lu.M, Lu.N), dtype=torch.float16, device="cuda") for _ in range(n)]
    Y = [torch.empty((Ld.M, Ld.N), dtype=torch.float16, device="cuda") for _ in range(n)]

    def step(i):
        j = i % n
        up(X[j], H[j])
        if args.unfused_gelu:
            sq.gelu_tanh_f16(H[j], H[j])
        down(H[j], Y[j])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / args.steps
    ops = 2.0 * Lu.M * Lu.N * Lu.K + 2.0 * Ld.M * Ld.N * Ld.K
    value = ops / t / 1e12
    print(json.dumps({
        "metric": "effective TOPS of the DiT MLP pair (SVDQuant W4A4+rank-32 up, GELU, down)",
        "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": "dit_mlp: X f16 4608x3072 -> 12288 (GELU-tanh) -> 3072, rank 32",
                   "gelu": "separate kernel" if args.unfused_gelu else "fused into the up epilogue",
                   "buffer_sets": n},
        "pct_int8_peak": round(100.0 * value / INT8_PEAK_TOPS, 2)}), flush=True)


def conv_cpu_baseline(L, X, Wm, prep, bias, budget_s):
    """The oracle's convolution (im2col of the whole image, then its linear layer
    on chunks of patch rows) until ~budget_s seconds."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    t0 = time.perf_counter()
    Xcol = O.im2col_nhwc(X, L.KH, L.KW, L.stride, L.pad)
    lam = O.smoothing_factors(O.channel_absmax(Xcol), Wm)
    inv = O.inv_smoothing(lam)
    mx = prep.fmt == "mxfp4"
    if mx:
        wc, ws = O.mx_quantize_residual_from_factors(Wm, lam, prep.L1, prep.L2)
    else:
        wc, ws = O.quantize_residual_from_factors(Wm, lam, prep.L1, prep.L2)
    t_setup = time.perf_counter() - t0
    chunk, rows = 32, 0
    t0 = time.perf_counter()
    while rows < L.M and time.perf_counter() - t0 < budget_s:
        r = slice(rows, min(L.M, rows + chunk))
        (O.mx_linear if mx else O.linear)(Xcol[r], inv, prep.L1, prep.L2, wc, ws, bias,
                                          L.y_dtype)
        rows = r.stop
    t = time.perf_counter() - t0
    return dict(value=2.0 * rows * L.N * L.K / t / 1e12, unit="TFLOPS" if mx else "TOPS",
                cores=int(cores),
                kind="oracle",
                sample=f"first {rows} of {L.M} output pixels of the same convolution, online "
                       f"part only ({t:.1f} s, numpy fp64, chunks of {chunk}; the im2col and "
                       f"calibration before it took {t_setup:.1f} s and are not counted)")


def conv_main(args, torch, sq, wl):
    """Step = one UNet convolution on one batch: K1 on the implicit patch matrix
    of the NHWC image, then K2 (the same kernels as svdq_conv2d, or with
    --format mxfp4 their MXFP4 versions, as svdq_conv2d_mx)."""
    L, X, Wc = wl.conv_inputs(args.conv)
    mx = args.format == "mxfp4"
    if args.format == "w4a16":
        raise SystemExit("--conv runs the INT4 or MXFP4 format")
    Wm = Wc.reshape(L.K, L.N)
    bias = wl.bias(wl.CONV_CFG, args.conv, L.N)
    lam = sq.smoothing_factors(sq.conv_patch_absmax(X, L.KH, L.KW, L.stride, L.pad), Wm)
    prep = (sq.prepare_weights_mx if mx else sq.prepare_weights)(Wm, lam, L.rank)
    M, K, N, R = L.M, L.K, L.N, prep.rank
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16
                                   else np.ascontiguousarray(a)).to("cuda")
    if mx:
        wct, wet = sq.pack_mx_tiles(prep.w_codes, prep.w_scales, K)
    else:
        wct, wet = prep.w_codes, prep.w_scales
    ydt = torch.float16 if L.y_dtype == "f16" else torch.float32
    sets = []
    for _ in range(args.sets):
        s = dict(X=d(X), inv=d(prep.inv_smooth), L1p=d(prep.L1p), L2t=d(prep.L2t), wc=d(wct),
                 ws=d(wet), b=d(bias), D=torch.empty((M, R), dtype=torch.float32, device="cuda"),
                 Y=torch.empty((L.batch, L.OH, L.OW, N), dtype=ydt, device="cuda"))
        if mx:
            s.update(ac=torch.empty(sq.mx_codes_tiled_bytes(M, K), dtype=torch.uint8, device="cuda"),
                     asc=torch.empty(sq.mx_exps_tiled_bytes(M, K), dtype=torch.uint8, device="cuda"))
        else:
            s.update(ac=torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
                     asc=torch.empty((M, K // 64), dtype=torch.int16, device="cuda"))
        sets.append(s)
    k1f = sq.quantize_act_lowrank_down_conv_mx if mx else sq.quantize_act_lowrank_down_conv
    k2f = sq.mx_gemm_lowrank_up if mx else sq.w4a4_gemm_lowrank_up

    class _Step:
        def k1(self, i):
            s = sets[i % len(sets)]
            k1f(s["X"], L.KH, L.KW, L.stride, L.pad, s["inv"], s["L1p"], R, s["ac"], s["asc"],
                s["D"])

        def k2(self, i):
            s = sets[i % len(sets)]
            k2f(s["ac"], s["asc"], s["wc"], s["ws"], s["D"], s["L2t"], R, s["b"],
                s["Y"].view(M, N), K)

    t_step, t1, t2 = time_steps(torch, _Step(), args.steps, args.warmup)
    gap = event_gap(torch)
    k1_avg = float(np.mean(t1)) - gap
    k2_avg = float(np.mean(t2)) - gap
    ops = 2.0 * M * N * K
    value = ops / t_step / 1e12
    xb = 2 if L.x_dtype == "f16" else 4
    yb = 2 if L.y_dtype == "f16" else 4
    img = L.batch * L.H * L.W * L.C
    meta = (K // 32) if mx else 2 * (K // 64)           # exponent or scale bytes per row
    # K1: the image once, the patch matrix's codes, scales (or exponents) and D out
    k1_bytes = img * xb + M * K // 2 + M * meta + 4 * M * R + 2 * K * R + 4 * K
    k2_bytes = (M + N) * K // 2 + (M + N) * meta + 4 * M * R + 2 * R * N + M * N * yb
    peak, unit, kname, dtype = ((FP4_PEAK_TFLOPS, "TFLOPS", "k2_mx_kernel", "fp4") if mx else
                                (INT8_PEAK_TOPS, "TOPS", "k2_w4a4_kernel", "int8"))
    fmt_txt = "MXFP4 (E2M1, E8M0 per 32)" if mx else "INT4 per-64 groups"
    out = {
        "metric": (f"effective {unit} of an SVDQuant {'MXFP4' if mx else 'W4A4'}+rank-32 UNet "
                   f"convolution (implicit GEMM), % of {'FP4' if mx else 'INT8'} MFMA peak"),
        "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t_step * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": f"{L.name}: X {L.x_dtype} NHWC {L.batch}x{L.H}x{L.W}x{L.C}, "
                               f"{L.KH}x{L.KW} stride {L.stride} pad {L.pad} -> {N} channels "
                               f"(patch matrix {M}x{K}), rank {R}, {fmt_txt}, Y {L.y_dtype}",
                   "M": M, "K": K, "N": N, "rank": R, "format": args.format,
                   "buffer_sets": args.sets},
        ("pct_fp4_peak" if mx else "pct_int8_peak"): round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "kernel": kname,
                     "achieved": round(ops / k2_avg / 1e12, 2), "peak": peak,
                     "unit": unit, "frac": round(ops / k2_avg / 1e12 / peak, 4),
                     "traffic": None, "algorithmic_bytes": k2_bytes,
                     "avg_ms": round(k2_avg * 1e3, 4),
                     "timing": "HIP events around each launch in a second pass of the same "
                               "steps, on the launch stream, less the gap of an empty "
                               "event pair",
                     "event_gap_us": round(gap * 1e6, 2)},
        "k1": {"kernel": "k1_quant_down_kernel (convolution instance)",
               "avg_ms": round(k1_avg * 1e3, 4), "algorithmic_bytes": k1_bytes,
               "achieved_gbs": round(k1_bytes / k1_avg / 1e9, 1), "peak_gbs": HBM_PEAK_GBS,
               "frac": round(k1_bytes / k1_avg / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if args.copy_probe:
        copy_probe(torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = conv_cpu_baseline(L, X, Wm, prep, bias, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built and measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_post_quantized_smooth_amd as sq
    import workloads as wl

    if args.mlp:
        mlp_main(args, torch, sq, wl)
        return
    if args.conv is not None:
        conv_main(args, torch, sq, wl)
        return
    cfg = wl.CONFIGS[args.config]
    L = cfg.layers[args.layer]
    Lx, X, W = wl.layer_inputs(args.config, args.layer)
    if X is None:
        import oracle as O   # input synthesis only: GELU of the seeded pre-activations
        X = O.gelu_tanh(wl.preactivation(args.config, args.layer, L.M, L.K, L.x_outlier_frac,
                                         L.x_outlier_scale))
    bias = None
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    mx = args.format == "mxfp4"
    w16 = args.format == "w4a16"
    prepare = sq.prepare_weights_mx if mx else sq.prepare_weights
    prep = sq.prepare_weights_w4a16(W) if w16 else prepare(W, lam, L.rank)
    if L.lora_rank and not w16:
        A, B = wl.lora(args.config, args.layer, L.K, L.N, L.lora_rank)
        prep = sq.concat_lora(prep, lam, A, B, 1.0)
    M, K, N, R = L.M, L.K, L.N, prep.rank
    sets = Sets(torch, X, prep, bias, args.sets, L.y_dtype)
    t_step, k1, k2 = time_steps(torch, sets, args.steps, args.warmup)
    ops = 2.0 * M * N * K
    value = ops / t_step / 1e12
    gap = event_gap(torch)
    k1_avg = float(np.mean(k1)) - gap
    k2_avg = float(np.mean(k2)) - gap
    xb = 2 if L.x_dtype == "f16" else 4
    yb = 2 if L.y_dtype == "f16" else 4
    meta = (K // 32) if mx else 2 * (K // 64)          # exponent or scale bytes per row
    if w16:   # tiling pass: read X, write fp16 tiles; GEMM: fp16 tiles, codes, scales, Y
        k1_bytes = M * K * xb + 2 * M * K
        k2_bytes = 2 * M * K + N * K // 2 + N * meta + M * N * yb
    else:
        k1_bytes = M * K * xb + M * K // 2 + M * meta + 4 * M * R + 2 * K * R + 4 * K
        k2_bytes = (M + N) * K // 2 + (M + N) * meta + 4 * M * R + 2 * R * N + M * N * yb

    traffic = None
    if os.path.exists(PROFILE_PMC[args.format]):
        try:
            pm = json.load(open(PROFILE_PMC[args.format]))
            if (pm.get("k2_source_hash") == k2_source_hash(args.format)
                    and pm.get("config") == args.config):
                traffic = pm.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    overhead = None
    if not args.no_overhead and R > 0 and not w16:
        prep0 = prepare(W, lam, 0)
        sets0 = Sets(torch, X, prep0, bias, args.sets, L.y_dtype)
        t0_step, _, k2_0 = time_steps(torch, sets0, args.steps, args.warmup)
        k2_0 = float(np.mean(k2_0)) - gap
        overhead = dict(step_ms_rank0=t0_step * 1e3, k2_ms_rank0=k2_0 * 1e3,
                        frac=(t_step - t0_step) / k2_0)
        del sets0

    if args.copy_probe:
        copy_probe(torch)

    if w16:
        metric = "effective TFLOPS of the 4-bit weight-only (W4A16) baseline linear, % of fp16 MFMA peak"
        peak, unit, kname, dtype = FP16_PEAK_TFLOPS, "TFLOPS", "k2_w4a16_kernel", "fp16"
        fmt_txt = "W4A16 baseline (INT4 weights per-64 groups, fp16 activations, no low-rank)"
    elif mx:
        metric = "effective TFLOPS of the SVDQuant MXFP4+rank-32 linear, % of FP4 MFMA peak"
        peak, unit, kname, dtype = FP4_PEAK_TFLOPS, "TFLOPS", "k2_mx_kernel", "fp4"
        fmt_txt = "MXFP4 (E2M1, E8M0 per 32)"
    else:
        metric = "effective TOPS of SVDQuant W4A4+rank-32 linear, % of INT8 MFMA peak"
        peak, unit, kname, dtype = INT8_PEAK_TOPS, "TOPS", "k2_w4a4_kernel", "int8"
        fmt_txt = "INT4 per-64 groups"
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} layer {args.layer}: X {L.x_dtype} {M}x{K}, "
                               f"W {K}x{N}, rank {R}, {fmt_txt}, Y {L.y_dtype}",
                   "M": M, "K": K, "N": N, "rank": R, "format": args.format,
                   "buffer_sets": args.sets},
        ("pct_fp16_peak" if w16 else "pct_fp4_peak" if mx else "pct_int8_peak"):
            round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "kernel": kname,
                     "achieved": round(ops / k2_avg / 1e12, 2), "peak": peak,
                     "unit": unit, "frac": round(ops / k2_avg / 1e12 / peak, 4),
                     "traffic": traffic, "algorithmic_bytes": k2_bytes,
                     "avg_ms": round(k2_avg * 1e3, 4),
                     "timing": "HIP events around each launch in a second pass of the same "
                               "steps, on the launch stream, less the gap of an empty "
                               "event pair",
                     "event_gap_us": round(gap * 1e6, 2)},
        "k1": {"kernel": "tile_x_kernel" if w16 else "k1_quant_down_kernel",
               "avg_ms": round(k1_avg * 1e3, 4),
               "algorithmic_bytes": k1_bytes, "achieved_gbs": round(k1_bytes / k1_avg / 1e9, 1),
               "peak_gbs": HBM_PEAK_GBS, "frac": round(k1_bytes / k1_avg / 1e9 / HBM_PEAK_GBS, 4)},
        "lowrank_overhead": None if overhead is None else {
            k: round(v, 4) for k, v in overhead.items()},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(X, W, prep, bias, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
