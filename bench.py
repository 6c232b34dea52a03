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
``clock`` is the shader clock sampled during the timed steps; ``cpu_baseline``
times the CPU oracle on a bounded row sample.

``--layer all`` times a whole workload instead of one layer: the five UNet
linears back to back (config 3), the 19-layer LoRA stack as a chain in which
each layer's output is the next one's input (config 4), or the DiT MLP pair
(config 2, the same as ``--mlp``).
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
               "int4t": os.path.join(ROOT, "profiles", "k2t_dit_qkv_pmc.json"),
               "mxfp4": os.path.join(ROOT, "profiles", "k2mx_dit_qkv_pmc.json"),
               "w4a16": os.path.join(ROOT, "profiles", "k2w16_dit_qkv_pmc.json")}
_CSRC = "bit_post_quantized_smooth_amd/csrc/"
K2_SOURCES = {"int4": [_CSRC + "k2_w4a4_gemm.hip", _CSRC + "k2_common.hpp",
                       _CSRC + "device_common.hpp"],
              "int4t": [_CSRC + "k2_w4a4_tiled.hip", _CSRC + "k2_common.hpp",
                        _CSRC + "device_common.hpp"],
              "mxfp4": [_CSRC + "k2_mx_gemm.hip", _CSRC + "k2_common.hpp",
                        _CSRC + "device_common.hpp"],
              "w4a16": [_CSRC + "k2_w4a16_gemm.hip", _CSRC + "k2_common.hpp",
                        _CSRC + "device_common.hpp"]}
TIMING_NOTE = ("HIP events around each launch in a second pass of the same steps, on the "
               "launch stream, less the gap of an empty event pair")
GRAPH_TIMING_NOTE = ("HIP events around replays of a graph of one launch over the buffer sets, "
                     "less the gap of an empty event pair, per launch")


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
    ap.add_argument("--layer", default="0",
                    help="layer index, or 'all': the whole workload (config 2: the MLP pair, "
                         "3: the five UNet linears back to back, 4: the 19-layer chain)")
    ap.add_argument("--sets", type=int, default=4, help="rotating buffer sets (cold MALL)")
    ap.add_argument("--graph", action="store_true",
                    help="run the steps as replays of a HIP graph of --sets steps (one host "
                         "call per graph instead of one per kernel)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-overhead", action="store_true", help="skip the rank-0 comparison run")
    ap.add_argument("--no-clock", action="store_true",
                    help="no shader-clock probe (a replica of the timed steps)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain fp32 copy kernel of known size (for PMC scaling)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="run the step for this long before the counted warm-up steps, so the "
                         "shader clock has left its idle level (reported as settle_ms)")
    ap.add_argument("--mlp", action="store_true",
                    help="time the DiT MLP pair instead: up-projection with the GELU fused into "
                         "its epilogue, then the down-projection")
    ap.add_argument("--format", choices=["int4", "mxfp4", "w4a16"], default="int4",
                    help="mxfp4: the MXFP4 variant (E2M1 codes, E8M0 exponent per 32) on the "
                         "scaled FP4 matrix core; w4a16: the 4-bit weight-only baseline of the "
                         "pages' speed comparison (fp16 activations, no low-rank branch)")
    ap.add_argument("--path", choices=["tiled", "canonical"], default="tiled",
                    help="INT4 only: the tiled path (pre-kernel writing the GEMM's operand "
                         "tiles, svdq_linear_tiled) or the canonical-layout kernels")
    ap.add_argument("--unfused-gelu", action="store_true",
                    help="with --mlp: plain up-projection, then the separate GELU kernel")
    ap.add_argument("--conv", type=int, default=None,
                    help="time UNet convolution I instead (NHWC, K1 on the implicit patch matrix, "
                         "then K2; INT4 format)")
    return ap.parse_args()


# --------------------------------------------------------------------------
# timing


class ClockProbe:
    """The shader clock over a replica of the timed steps: svdq_clock_probe
    (one wave on a side stream, sampling the shader-clock cycle counter
    against the constant wall counter every INTERVAL_US) runs from just before
    the replica's first launch until svdq_clock_mark, queued behind its last
    launch, sets the stop flag; the final synchronize waits for the probe to
    see the flag (at most one interval). The replica runs right after the
    timed pass, with the same launches: run beside the timed pass itself, the
    probe wave slowed its steps (c1: 240 against 222 us per step on one box)."""
    INTERVAL_US = 10.0

    def __init__(self, torch, sq):
        self.torch, self.sq = torch, sq
        self.wall_khz, self.peak_khz = sq.clock_rates()
        self.ticks = max(1, int(round(self.INTERVAL_US * self.wall_khz / 1000.0)))
        n = 1 << 18                                       # 2.6 s of samples at 10 us
        self.samples = torch.zeros(1 + 2 * n, dtype=torch.int64, device="cuda")
        self.stop = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.stamp = torch.zeros(1, dtype=torch.int64, device="cuda")
        self.side = torch.cuda.Stream()                   # default priority

    def arm(self):
        """Before the synchronize that opens the timed window."""
        self.stop.zero_()
        self.samples[0].zero_()

    def launch(self):
        """Right after that synchronize, before the first timed launch."""
        self.sq.clock_probe(self.samples, self.stop, self.ticks, stream=self.side)

    def end(self):
        """Right after the last timed launch, before the closing synchronize."""
        self.sq.clock_mark(self.stamp, self.stop)

    def result(self):
        s = self.samples.cpu().numpy().view(np.uint64)
        n = int(s[0])
        if n < 2:
            return {"sclk_mhz": None, "samples": n}
        c = s[1:1 + 2 * n:2].astype(np.float64)
        w = s[2:2 + 2 * n:2].astype(np.float64)
        wall_mhz = self.wall_khz / 1000.0
        mean = (c[-1] - c[0]) / (w[-1] - w[0]) * wall_mhz
        # per-millisecond windows for the spread
        step = max(1, int(round(1000.0 / self.INTERVAL_US)))
        idx = np.arange(0, n, step)
        if idx[-1] != n - 1:
            idx = np.append(idx, n - 1)
        dc, dw = np.diff(c[idx]), np.diff(w[idx])
        per = dc[dw > 0] / dw[dw > 0] * wall_mhz
        return {"sclk_mhz": round(float(mean), 1),
                "ms_per_step_replica": (round(self.step_s * 1e3, 4)
                                        if getattr(self, "step_s", None) else None),
                "sclk_mhz_min_1ms": round(float(per.min()), 1) if per.size else None,
                "sclk_mhz_max_1ms": round(float(per.max()), 1) if per.size else None,
                "peak_mhz": round(self.peak_khz / 1000.0, 1),
                "window_ms": round((w[-1] - w[0]) / self.wall_khz, 3), "samples": n,
                "how": "shader-clock counter against the constant wall counter, one wave on a "
                       "side stream during a replica of the timed steps run right after them"}


def settle(torch, runner, ms):
    """Run whole steps for about `ms` milliseconds (untimed, before the counted
    warm-up): right after idle the shader clock sits well below its loaded
    level for longer than a few steps (measured on c1: 1.85 GHz averaged over
    the first 7 ms against 2.2 GHz once settled)."""
    if ms <= 0:
        return 0.0
    t0 = time.perf_counter()
    i = 0
    while True:
        for _, f in runner.launches(i):
            f()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms:
                break
    return (time.perf_counter() - t0) * 1e3


def time_steps(torch, runner, steps, warmup, probe=None, graph_period=0):
    """Passes of `steps` steps after `warmup` untimed ones. The first,
    bracketed by synchronizations, is the step time: plain launches and
    nothing else on the GPU. With a clock probe, a replica of it follows with
    the probe beside it (ClockProbe). The last records HIP events around each
    launch on the launch stream for the per-kernel durations; an event record
    costs the stream a few microseconds, so that pass is not the step time.
    With graph_period = P > 0 the steps run as replays of one HIP graph of P
    consecutive steps (every buffer set once), captured after the warm-up, so
    the host issues one call per P steps instead of one per kernel; the
    per-kernel pass then replays, for each launch of a step, a graph of that
    launch over the P steps between two events. Returns (step seconds, launch
    names, per-launch seconds as a rows x launches array)."""
    for i in range(warmup):
        for _, f in runner.launches(i):
            f()
    torch.cuda.synchronize()
    names = [n for n, _ in runner.launches(0)]
    if graph_period > 0:
        P = graph_period
        reps = max(1, steps // P)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(P):
                for _, f in runner.launches(i):
                    f()
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if probe is not None:
            probe.arm()
            torch.cuda.synchronize()
            probe.launch()
            r0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            probe.end()
            torch.cuda.synchronize()
            probe.step_s = (time.perf_counter() - r0) / (reps * P)
        gap = event_gap(torch)
        per = np.zeros((reps, len(names)))
        for j in range(len(names)):
            gj = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gj):
                for i in range(P):
                    runner.launches(i)[j][1]()
            gj.replay()
            evs = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                gj.replay()
                b.record()
                evs.append((a, b))
            torch.cuda.synchronize()
            # the callers subtract one event gap per launch: leave it in once
            per[:, j] = [(a.elapsed_time(b) * 1e-3 - gap) / P + gap for a, b in evs]
            del gj
        del g
        return (t1 - t0) / (reps * P), names, per
    t0 = time.perf_counter()
    for i in range(steps):
        for _, f in runner.launches(i):
            f()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if probe is not None:
        probe.arm()
        torch.cuda.synchronize()
        probe.launch()
        r0 = time.perf_counter()
        for i in range(steps):
            for _, f in runner.launches(i):
                f()
        probe.end()
        torch.cuda.synchronize()
        probe.step_s = (time.perf_counter() - r0) / steps
    evs = []
    for i in range(steps):
        ls = runner.launches(i)
        es = [torch.cuda.Event(enable_timing=True) for _ in range(len(ls) + 1)]
        for j, (_, f) in enumerate(ls):
            es[j].record()
            f()
        es[-1].record()
        evs.append(es)
    torch.cuda.synchronize()
    per = np.array([[es[j].elapsed_time(es[j + 1]) for j in range(len(names))] for es in evs])
    return (t1 - t0) / steps, names, per * 1e-3


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


def kernel_stats(per_col, gap):
    """(mean, median) seconds of one launch over the event pass, less the event gap."""
    return float(np.mean(per_col)) - gap, float(np.median(per_col)) - gap


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


def host_cores():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count()


# --------------------------------------------------------------------------
# algorithmic bytes (per launch)


def k1_bytes(M, K, R, xb, meta_per_row, tiled=False, db=4):
    """Read X once; write codes, scales (or exponents) and D (db bytes an entry:
    fp32, or fp16 on the MXFP4 path); read L1 and 1/lambda.
    tiled: the activation side as the tiled path stores it (one int8 operand byte
    per code, an fp32 scale per row and group, D in fp16)."""
    if tiled:
        return M * K * xb + M * K + 4 * M * (K // 64) + 2 * M * R + 2 * K * R + 4 * K
    act = M * K // 2 + M * meta_per_row
    return M * K * xb + act + db * M * R + 2 * K * R + 4 * K


def k2_bytes(M, N, K, R, yb, meta_per_row, tiled=False, db=4):
    """Codes and scales of both operands, D (db bytes an entry), L2, Y (bias not
    counted: zero in the configs).
    tiled: as the tiled path stores them (int8 activation operands and fp32 scales,
    the weight scales as 8-byte fp32 pairs, D in fp16)."""
    if tiled:
        G = K // 64
        return (M * K + 4 * M * G + N * K // 2 + 8 * N * G + 2 * M * R + 2 * R * N
                + M * N * yb)
    act = M * K // 2 + M * meta_per_row
    return act + N * K // 2 + N * meta_per_row + db * M * R + 2 * R * N + M * N * yb


# --------------------------------------------------------------------------
# one layer


class Sets:
    """`n` independent device copies of one layer's inputs, weights and outputs."""

    def __init__(self, torch, X, prep, bias, n, y_dtype, tiled=False):
        import bit_post_quantized_smooth_amd as sq
        self.sq = sq
        self.mx = prep.fmt == "mxfp4"
        self.w16 = prep.fmt == "w4a16"
        self.tiled = tiled and prep.fmt == "int4"
        M, K = X.shape
        self.M, self.K, self.N, self.R = M, K, prep.N, prep.rank
        G = K // 64
        d = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16
                                       else np.ascontiguousarray(a)).to("cuda")
        if self.mx:
            wct, wet = sq.pack_mx_tiles(prep.w_codes, prep.w_scales, K)
        if self.w16:
            wct, wet = sq.pack_w4a16_tiles(prep.w_codes, prep.w_scales, K)
        if self.tiled:
            wct, wet = sq.pack_w4a4_tiles(prep.w_codes, prep.w_scales, K)
        self.sets = []
        for _ in range(n):
            s = dict(
                X=d(X), inv=d(prep.inv_smooth),
                L1p=d(prep.L1p) if self.R else None, L2t=d(prep.L2t) if self.R else None,
                b=None if bias is None else d(bias),
                D=(torch.empty(max(sq.int4_d_tiled_bytes(M, self.R), 2) // 2, dtype=torch.int16,
                               device="cuda") if self.tiled or self.mx else
                   torch.empty((M, max(self.R, 1)), dtype=torch.float32, device="cuda")),
                Y=torch.empty((M, self.N), dtype=torch.float16 if y_dtype == "f16" else torch.float32,
                              device="cuda"))
            if self.w16:
                s.update(wc=d(wct), ws=d(wet),
                         ac=torch.empty(sq.w4a16_x_tiled_bytes(M, K) // 2, dtype=torch.int16,
                                        device="cuda"), asc=None)
            elif self.tiled:
                s.update(wc=d(wct), ws=d(wet),
                         ac=torch.empty(sq.int4_act_tiled_bytes(M, K), dtype=torch.uint8,
                                        device="cuda"),
                         asc=torch.empty(sq.int4_act_scales_tiled_bytes(M, K) // 4, dtype=torch.float32,
                                         device="cuda"))
            elif self.mx:
                s.update(wc=d(wct), ws=d(wet),
                         ac=torch.empty(sq.mx_codes_tiled_bytes(M, K), dtype=torch.uint8, device="cuda"),
                         asc=torch.empty(sq.mx_exps_tiled_bytes(M, K), dtype=torch.uint8, device="cuda"))
            else:
                s.update(wc=d(prep.w_codes), ws=d(prep.w_scales),
                         ac=torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
                         asc=torch.empty((M, G), dtype=torch.int16, device="cuda"))
            self.sets.append(s)
        # the pre-kernel's optional workspace (long rows run split), shared by
        # the sets: the launches of one stream never overlap
        need = sq.quantize_act_workspace_bytes(M, K, self.R) if (self.tiled or self.mx) else 0
        self.k1ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
        # the tiled GEMM's optional workspace (an under-filled long-K GEMM runs
        # split along K)
        need = sq.gemm_tiled_workspace_bytes(M, self.N, K) if self.tiled else 0
        self.k2ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None

    def k1(self, i, X=None):
        s = self.sets[i % len(self.sets)]
        X = s["X"] if X is None else X
        if self.w16:
            self.sq.w4a16_tile_activation(X, s["ac"])
            return
        f = (self.sq.quantize_act_lowrank_down_mx if self.mx
             else self.sq.quantize_act_lowrank_down_tiled if self.tiled
             else self.sq.quantize_act_lowrank_down)
        if self.tiled or self.mx:
            f(X, s["inv"], s["L1p"], self.R, s["ac"], s["asc"], s["D"] if self.R else None,
              workspace=self.k1ws)
        else:
            f(X, s["inv"], s["L1p"], self.R, s["ac"], s["asc"], s["D"] if self.R else None)

    def k2(self, i, Y=None):
        s = self.sets[i % len(self.sets)]
        Y = s["Y"] if Y is None else Y
        if self.w16:
            self.sq.w4a16_gemm(s["ac"], s["wc"], s["ws"], s["b"], Y, self.K)
            return
        f = (self.sq.mx_gemm_lowrank_up if self.mx
             else self.sq.w4a4_gemm_lowrank_up_tiled if self.tiled
             else self.sq.w4a4_gemm_lowrank_up)
        if self.tiled:
            f(s["ac"], s["asc"], s["wc"], s["ws"], s["D"] if self.R else None, s["L2t"], self.R,
              s["b"], Y, self.K, workspace=self.k2ws)
        else:
            f(s["ac"], s["asc"], s["wc"], s["ws"], s["D"] if self.R else None, s["L2t"], self.R,
              s["b"], Y, self.K)

    def launches(self, i):
        return [("k1", lambda: self.k1(i)), ("k2", lambda: self.k2(i))]


def cpu_baseline(X, W, prep, bias, budget_s, out_dtype="f16"):
    """The oracle's online part (quantize X, down-projection, integer partials,
    scaled sum, up-projection, bias; or its MXFP4 counterpart) on chunks of rows
    until ~budget_s seconds. Returns (dict, seconds per row)."""
    import oracle as O
    lam = O.smoothing_factors(O.channel_absmax(X), W)
    inv = O.inv_smoothing(lam)
    mx = prep.fmt == "mxfp4"
    w16 = prep.fmt == "w4a16"
    if w16:
        wc, ws = O.w4a16_prepare(W)
    elif mx:
        wc, ws = O.mx_quantize_residual_from_factors(W, lam, prep.L1, prep.L2)
    else:
        base = prep.rank if getattr(prep, "base_rank", None) is None else prep.base_rank
        wc, ws = O.quantize_residual_from_factors(W, lam, prep.L1[:, :base], prep.L2[:base])
    M, K = X.shape
    N = W.shape[1]
    chunk = 32
    rows = 0
    t0 = time.perf_counter()
    while rows < M and time.perf_counter() - t0 < budget_s:
        r = slice(rows, min(M, rows + chunk))
        if w16:
            O.w4a16_linear(X[r], wc, ws, bias, out_dtype)
        else:
            (O.mx_linear if mx else O.linear)(X[r], inv, prep.L1, prep.L2, wc, ws, bias, out_dtype)
        rows = r.stop
    t = time.perf_counter() - t0
    return (dict(value=2.0 * rows * N * K / t / 1e12, unit="TFLOPS" if (mx or w16) else "TOPS",
                 cores=int(host_cores()), kind="oracle",
                 sample=f"first {rows} of {M} rows of the same layer, online part only "
                        f"({t:.1f} s, numpy fp64, chunks of {chunk} rows)"), t / rows)


def prepare_layer(sq, wl, cfg, li, fmt, rank=None):
    """(Layer, X, W, lam, prep) with the library's host prep (LoRA concatenated
    for the configs that carry one); rank overrides the SVD rank (0: bare GEMM)."""
    L, X, W = wl.layer_inputs(cfg, li)
    lam = sq.smoothing_factors(sq.channel_absmax(X), W)
    r = L.rank if rank is None else rank
    if fmt == "w4a16":
        return L, X, W, lam, sq.prepare_weights_w4a16(W)
    prep = (sq.prepare_weights_mx if fmt == "mxfp4" else sq.prepare_weights)(W, lam, r)
    if L.lora_rank and rank is None:
        A, B = wl.lora(cfg, li, L.K, L.N, L.lora_rank)
        base = prep.rank
        prep = sq.concat_lora(prep, lam, A, B, 1.0)
        prep.base_rank = base
    return L, X, W, lam, prep


FORMATS = {
    "int4": dict(metric="effective TOPS of SVDQuant W4A4+rank-32 linear, % of INT8 MFMA peak",
                 peak=INT8_PEAK_TOPS, unit="TOPS", kname="k2_w4a4_kernel", dtype="int8",
                 text="INT4 per-64 groups", pct="pct_int8_peak"),
    "mxfp4": dict(metric="effective TFLOPS of the SVDQuant MXFP4+rank-32 linear, % of FP4 MFMA peak",
                  peak=FP4_PEAK_TFLOPS, unit="TFLOPS", kname="k2_mx_kernel", dtype="fp4",
                  text="MXFP4 (E2M1, E8M0 per 32)", pct="pct_fp4_peak"),
    "w4a16": dict(metric="effective TFLOPS of the 4-bit weight-only (W4A16) baseline linear, "
                         "% of fp16 MFMA peak",
                  peak=FP16_PEAK_TFLOPS, unit="TFLOPS", kname="k2_w4a16_kernel", dtype="fp16",
                  text="W4A16 baseline (INT4 weights per-64 groups, fp16 activations, no "
                       "low-rank)", pct="pct_fp16_peak"),
}


def meta_bytes(K, fmt):
    return (K // 32) if fmt == "mxfp4" else 2 * (K // 64)


def single_layer_main(args, torch, sq, wl, probe):
    cfg = wl.CONFIGS[args.config]
    li = int(args.layer)
    fmt = args.format
    F = FORMATS[fmt]
    L, X, W, lam, prep = prepare_layer(sq, wl, args.config, li, fmt)
    bias = None
    M, K, N, R = L.M, L.K, L.N, prep.rank
    tiled = args.path == "tiled" and fmt == "int4"
    sets = Sets(torch, X, prep, bias, args.sets, L.y_dtype, tiled)
    settled = settle(torch, sets, args.settle_ms)
    t_step, _, per = time_steps(torch, sets, args.steps, args.warmup, probe,
                                 args.sets if args.graph else 0)
    clock = probe.result() if probe is not None else None
    ops = 2.0 * M * N * K
    value = ops / t_step / 1e12
    gap = event_gap(torch)
    k1_avg, k1_med = kernel_stats(per[:, 0], gap)
    k2_avg, k2_med = kernel_stats(per[:, 1], gap)
    xb = 2 if L.x_dtype == "f16" else 4
    yb = 2 if L.y_dtype == "f16" else 4
    meta = meta_bytes(K, fmt)
    if fmt == "w4a16":   # tiling pass: read X, write fp16 tiles; GEMM: fp16 tiles, codes, scales, Y
        b1 = M * K * xb + 2 * M * K
        b2 = 2 * M * K + N * K // 2 + N * meta + M * N * yb
    else:
        db = 2 if fmt == "mxfp4" else 4
        b1 = k1_bytes(M, K, R, xb, meta, db=db)
        b2 = k2_bytes(M, N, K, R, yb, meta, db=db)
    # the bytes the tiled path's layouts move (the fractions use the method's
    # algorithmic bytes above, which are fewer)
    b1_layout = k1_bytes(M, K, R, xb, meta, tiled) if tiled else b1
    b2_layout = k2_bytes(M, N, K, R, yb, meta, tiled) if tiled else b2

    traffic = None
    pkey = "int4t" if tiled else fmt
    if os.path.exists(PROFILE_PMC[pkey]):
        try:
            with open(PROFILE_PMC[pkey]) as f:
                pm = json.load(f)
            if (pm.get("k2_source_hash") == k2_source_hash(pkey)
                    and pm.get("config") == args.config):
                traffic = pm.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    overhead = None
    if not args.no_overhead and R > 0 and fmt != "w4a16":
        _, _, _, _, prep0 = prepare_layer(sq, wl, args.config, li, fmt, rank=0)
        sets0 = Sets(torch, X, prep0, bias, args.sets, L.y_dtype, tiled)
        settle(torch, sets0, args.settle_ms)     # the clock fell while the rank-0 layer was made
        t0_step, _, per0 = time_steps(torch, sets0, args.steps, args.warmup, None,
                                       args.sets if args.graph else 0)
        k2_0 = float(np.median(per0[:, 1])) - gap
        overhead = dict(step_ms_rank0=t0_step * 1e3, k2_ms_rank0=k2_0 * 1e3,
                        frac=(t_step - t0_step) / k2_0)
        del sets0

    if args.copy_probe:
        copy_probe(torch)

    out = {
        "metric": F["metric"],
        "value": round(value, 2),
        "unit": F["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": round(settled, 1),
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": F["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} layer {li}: X {L.x_dtype} {M}x{K}, "
                               f"W {K}x{N}, rank {R}, {F['text']}, Y {L.y_dtype}",
                   "M": M, "K": K, "N": N, "rank": R, "format": fmt,
                   "path": "tiled" if tiled else "canonical", "buffer_sets": args.sets,
                   "launch": "hip graph" if args.graph else "eager"},
        F["pct"]: round(100.0 * value / F["peak"], 2),
        "roofline": {"bound": "mfma", "kernel": "k2t_w4a4_kernel" if tiled else F["kname"],
                     "achieved": round(ops / k2_avg / 1e12, 2), "peak": F["peak"],
                     "unit": F["unit"], "frac": round(ops / k2_avg / 1e12 / F["peak"], 4),
                     "traffic": traffic, "algorithmic_bytes": b2, "layout_bytes": b2_layout,
                     "avg_ms": round(k2_avg * 1e3, 4), "median_ms": round(k2_med * 1e3, 4),
                     "frac_median": round(ops / k2_med / 1e12 / F["peak"], 4),
                     "timing": GRAPH_TIMING_NOTE if args.graph else TIMING_NOTE,
                     "event_gap_us": round(gap * 1e6, 2)},
        "k1": {"kernel": "tile_x_kernel" if fmt == "w4a16" else "k1_quant_down_kernel",
               "avg_ms": round(k1_avg * 1e3, 4), "median_ms": round(k1_med * 1e3, 4),
               "layout_bytes": b1_layout,
               "algorithmic_bytes": b1, "achieved_gbs": round(b1 / k1_avg / 1e9, 1),
               "peak_gbs": HBM_PEAK_GBS, "frac": round(b1 / k1_avg / 1e9 / HBM_PEAK_GBS, 4),
               "frac_median": round(b1 / k1_med / 1e9 / HBM_PEAK_GBS, 4)},
        "lowrank_overhead": None if overhead is None else {
            k: round(v, 4) for k, v in overhead.items()},
        "clock": clock,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(X, W, prep, bias, args.cpu_seconds, L.y_dtype)[0]
    return out


# --------------------------------------------------------------------------
# whole workloads


class Chain:
    """A whole workload as one step. chain=True: layer l reads layer l-1's output
    (the LoRA stack, K = N for every layer); else every layer has its own input
    (the UNet batch, run back to back)."""

    def __init__(self, torch, layers, n_sets, chain, tiled=False):
        self.chain = chain
        self.layers = [Sets(torch, X, prep, None, n_sets if (li == 0 or not chain) else 1,
                            L.y_dtype, tiled) for li, (L, X, prep) in enumerate(layers)]
        if chain:
            M, N = layers[0][0].M, layers[0][0].N
            self.act = [torch.empty((M, N), dtype=torch.float16, device="cuda") for _ in range(2)]

    def launches(self, i):
        out = []
        for li, s in enumerate(self.layers):
            if self.chain and li > 0:
                x_in, y_out = self.act[(li - 1) % 2], self.act[li % 2]
                out.append((f"k1[{li}]", lambda s=s, x=x_in: s.k1(0, X=x)))
                out.append((f"k2[{li}]", lambda s=s, y=y_out: s.k2(0, Y=y)))
            elif self.chain:
                y0 = self.act[0]
                out.append((f"k1[{li}]", lambda s=s, i=i: s.k1(i)))
                out.append((f"k2[{li}]", lambda s=s, i=i, y=y0: s.k2(i, Y=y)))
            else:
                out.append((f"k1[{li}]", lambda s=s, i=i: s.k1(i)))
                out.append((f"k2[{li}]", lambda s=s, i=i: s.k2(i)))
        return out


def whole_config_main(args, torch, sq, wl, probe):
    cfg = wl.CONFIGS[args.config]
    fmt = args.format
    if fmt == "w4a16":
        raise SystemExit("--layer all runs the INT4 or MXFP4 format")
    F = FORMATS[fmt]
    chain = args.config == 4
    prepped = []
    for li in range(len(cfg.layers)):
        prepped.append(prepare_layer(sq, wl, args.config, li, fmt))
        print(f"prepared layer {li + 1} of {len(cfg.layers)}", file=sys.stderr, flush=True)
    layers = [(L, X, prep) for (L, X, W, lam, prep) in prepped]
    tiled = args.path == "tiled" and fmt == "int4"
    runner = Chain(torch, layers, args.sets, chain, tiled)
    settled = settle(torch, runner, args.settle_ms)
    t_step, names, per = time_steps(torch, runner, args.steps, args.warmup, probe,
                                     args.sets if args.graph else 0)
    clock = probe.result() if probe is not None else None
    gap = event_gap(torch)
    ops_total = sum(2.0 * L.M * L.N * L.K for L, _, _ in layers)
    rows, k2_total, k2_total_med = [], 0.0, 0.0
    for li, (L, X, prep) in enumerate(layers):
        M, K, N, R = L.M, L.K, L.N, prep.rank
        k1_avg, k1_med = kernel_stats(per[:, 2 * li], gap)
        k2_avg, k2_med = kernel_stats(per[:, 2 * li + 1], gap)
        k2_total += k2_avg
        k2_total_med += k2_med
        xb = 2 if L.x_dtype == "f16" else 4
        yb = 2 if L.y_dtype == "f16" else 4
        meta = meta_bytes(K, fmt)
        db = 2 if fmt == "mxfp4" else 4
        b1 = k1_bytes(M, K, R, xb, meta, db=db)
        b2 = k2_bytes(M, N, K, R, yb, meta, db=db)
        ops = 2.0 * M * N * K
        attainable = min(F["peak"], ops / b2 * HBM_PEAK_GBS / 1e3)   # TOPS at 8 TB/s
        rows.append({"layer": li, "M": M, "K": K, "N": N, "rank": R,
                     "k1_us": round(k1_med * 1e6, 2), "k2_us": round(k2_med * 1e6, 2),
                     "k2_tops": round(ops / k2_med / 1e12, 1),
                     "k2_pct_peak": round(100.0 * ops / k2_med / 1e12 / F["peak"], 2),
                     "k2_attainable": round(attainable, 1),
                     "k2_pct_attainable": round(100.0 * ops / k2_med / 1e12 / attainable, 2),
                     "k1_gbs": round(b1 / k1_med / 1e9, 1),
                     "k1_pct_hbm": round(100.0 * b1 / k1_med / 1e9 / HBM_PEAK_GBS, 2)})
    overhead = None
    if not args.no_overhead:
        p0 = [prepare_layer(sq, wl, args.config, li, fmt, rank=0) for li in range(len(cfg.layers))]
        runner0 = Chain(torch, [(L, X, prep) for (L, X, W, lam, prep) in p0], args.sets, chain,
                        tiled)
        settle(torch, runner0, args.settle_ms)   # the clock fell while the rank-0 layers were made
        t0_step, _, per0 = time_steps(torch, runner0, args.steps, args.warmup, None,
                                       args.sets if args.graph else 0)
        k2_0 = sum(float(np.median(per0[:, 2 * li + 1])) - gap for li in range(len(p0)))
        overhead = dict(step_ms_rank0=t0_step * 1e3, k2_ms_rank0=k2_0 * 1e3,
                        frac=(t_step - t0_step) / k2_0)
        del runner0
    value = ops_total / t_step / 1e12
    desc = ("19 chained layers (each output is the next input)" if chain else
            f"{len(layers)} layers back to back")
    out = {
        "metric": F["metric"].replace("linear", f"workload ({desc})"),
        "value": round(value, 2), "unit": F["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": round(settled, 1),
        "ms_per_step": round(t_step * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": F["dtype"], "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {desc}; {cfg.note}", "format": fmt,
                   "layers": len(layers), "buffer_sets": args.sets,
                   "launch": "hip graph" if args.graph else "eager"},
        F["pct"]: round(100.0 * value / F["peak"], 2),
        "roofline": {"bound": "mfma", "kernel": F["kname"] + " (all layers)",
                     "achieved": round(ops_total / k2_total / 1e12, 2), "peak": F["peak"],
                     "unit": F["unit"], "frac": round(ops_total / k2_total / 1e12 / F["peak"], 4),
                     "frac_median": round(ops_total / k2_total_med / 1e12 / F["peak"], 4),
                     "traffic": None,
                     "timing": GRAPH_TIMING_NOTE if args.graph else TIMING_NOTE,
                     "event_gap_us": round(gap * 1e6, 2)},
        "layers": rows,
        "lowrank_overhead": None if overhead is None else {
            k: round(v, 4) for k, v in overhead.items()},
        "clock": clock,
    }
    if not args.no_cpu_baseline:
        # the oracle on a row sample of each distinct layer shape, scaled to the whole workload
        t_cpu, desc_cpu, seen = 0.0, [], {}
        budget = args.cpu_seconds / (1 if chain else len(prepped))
        for li, (L, X, W, lam, prep) in enumerate(prepped):
            key = (L.M, L.K, L.N)
            if chain and key in seen:
                t_cpu += seen[key]
                continue
            d, per_row = cpu_baseline(X, W, prep, None, budget, L.y_dtype)
            seen[key] = per_row * L.M
            t_cpu += per_row * L.M
            desc_cpu.append(d["sample"])
        out["cpu_baseline"] = dict(value=ops_total / t_cpu / 1e12, unit=F["unit"],
                                   cores=int(host_cores()), kind="oracle",
                                   sample="; ".join(desc_cpu) + " -- scaled to every row of every "
                                          "layer (rows are independent)")
    return out


def mlp_main(args, torch, sq, wl, probe):
    """Step = the DiT MLP pair on one batch: K1 + K2 (+GELU) of the up-projection
    4608 x 3072 -> 12288, then K1 + K2 of the down-projection 12288 -> 3072, each
    one call of the layer's fused entry point (svdq_linear_tiled on the tiled
    INT4 path, svdq_linear on the canonical one, svdq_linear_mx for MXFP4)."""
    if args.format == "w4a16":
        raise SystemExit("the MLP pair runs the INT4 or MXFP4 format")
    mx = args.format == "mxfp4"
    tiled = args.path == "tiled" and not mx
    prep_fn = sq.prepare_weights_mx if mx else sq.prepare_weights
    Lu, Xu, Wu = wl.layer_inputs(2, 0)
    Ld, Xd_cal, Wd = wl.layer_inputs(2, 1)
    lam_u = sq.smoothing_factors(sq.channel_absmax(Xu), Wu)
    lam_d = sq.smoothing_factors(sq.channel_absmax(Xd_cal), Wd)
    up = sq.Linear(prep_fn(Wu, lam_u, Lu.rank),
                   activation=None if args.unfused_gelu else "gelu_tanh", tiled=tiled)
    down = sq.Linear(prep_fn(Wd, lam_d, Ld.rank), tiled=tiled)
    n = args.sets
    X = [torch.from_numpy(Xu).to("cuda") for _ in range(n)]
    H = [torch.empty((Lu.M, Lu.N), dtype=torch.float16, device="cuda") for _ in range(n)]
    Y = [torch.empty((Ld.M, Ld.N), dtype=torch.float16, device="cuda") for _ in range(n)]

    class _Runner:
        def launches(self, i):
            j = i % n
            ls = [("up", lambda: up(X[j], H[j]))]
            if args.unfused_gelu:
                ls.append(("gelu", lambda: sq.gelu_tanh_f16(H[j], H[j])))
            ls.append(("down", lambda: down(H[j], Y[j])))
            return ls

    settled = settle(torch, _Runner(), args.settle_ms)
    t, names, per = time_steps(torch, _Runner(), args.steps, args.warmup, probe)
    clock = probe.result() if probe is not None else None
    gap = event_gap(torch)
    ops = 2.0 * Lu.M * Lu.N * Lu.K + 2.0 * Ld.M * Ld.N * Ld.K
    value = ops / t / 1e12
    F = FORMATS[args.format]
    return {
        "metric": (f"effective {F['unit']} of the DiT MLP pair (SVDQuant "
                   f"{'MXFP4' if mx else 'W4A4'}+rank-32 up, GELU, down)"),
        "value": round(value, 2), "unit": F["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": round(settled, 1),
        "ms_per_step": round(t * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": F["dtype"], "data": "synthetic",
        "config": {"workload": "dit_mlp: X f16 4608x3072 -> 12288 (GELU-tanh) -> 3072, rank 32",
                   "gelu": "separate kernel" if args.unfused_gelu else "fused into the up epilogue",
                   "format": args.format,
                   "path": "tiled" if tiled else ("mxfp4" if mx else "canonical"),
                   "buffer_sets": n},
        F["pct"]: round(100.0 * value / F["peak"], 2),
        "launch_median_us": {nm: round((float(np.median(per[:, j])) - gap) * 1e6, 2)
                             for j, nm in enumerate(names)},
        "clock": clock}


def conv_cpu_baseline(L, X, Wm, prep, bias, budget_s):
    """The oracle's convolution (im2col of the whole image, then its linear layer
    on chunks of patch rows) until ~budget_s seconds."""
    import oracle as O
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
                cores=int(host_cores()),
                kind="oracle",
                sample=f"first {rows} of {L.M} output pixels of the same convolution, online "
                       f"part only ({t:.1f} s, numpy fp64, chunks of {chunk}; the im2col and "
                       f"calibration before it took {t_setup:.1f} s and are not counted)")


def conv_main(args, torch, sq, wl, probe):
    """Step = one UNet convolution on one batch: K1 on the implicit patch matrix
    of the NHWC image, then K2 (the same kernels as svdq_conv2d_tiled on the
    tiled INT4 path, svdq_conv2d with --path canonical, or with --format mxfp4
    their MXFP4 versions, as svdq_conv2d_mx)."""
    L, X, Wc = wl.conv_inputs(args.conv)
    mx = args.format == "mxfp4"
    tiled = args.path == "tiled" and not mx
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
    elif tiled:
        wct, wet = sq.pack_w4a4_tiles(prep.w_codes, prep.w_scales, K)
    else:
        wct, wet = prep.w_codes, prep.w_scales
    ydt = torch.float16 if L.y_dtype == "f16" else torch.float32
    sets = []
    for _ in range(args.sets):
        s = dict(X=d(X), inv=d(prep.inv_smooth), L1p=d(prep.L1p), L2t=d(prep.L2t), wc=d(wct),
                 ws=d(wet), b=d(bias),
                 D=(torch.empty(max(sq.int4_d_tiled_bytes(M, R), 2) // 2, dtype=torch.int16,
                                device="cuda") if mx or tiled else
                    torch.empty((M, R), dtype=torch.float32, device="cuda")),
                 Y=torch.empty((L.batch, L.OH, L.OW, N), dtype=ydt, device="cuda"))
        if tiled:
            s.update(ac=torch.empty(sq.int4_act_tiled_bytes(M, K), dtype=torch.uint8,
                                    device="cuda"),
                     asc=torch.empty(sq.int4_act_scales_tiled_bytes(M, K) // 4,
                                     dtype=torch.float32, device="cuda"))
        elif mx:
            s.update(ac=torch.empty(sq.mx_codes_tiled_bytes(M, K), dtype=torch.uint8, device="cuda"),
                     asc=torch.empty(sq.mx_exps_tiled_bytes(M, K), dtype=torch.uint8, device="cuda"))
        else:
            s.update(ac=torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
                     asc=torch.empty((M, K // 64), dtype=torch.int16, device="cuda"))
        sets.append(s)
    k1f = (sq.quantize_act_lowrank_down_conv_mx if mx else
           sq.quantize_act_lowrank_down_conv_tiled if tiled else sq.quantize_act_lowrank_down_conv)
    k2f = (sq.mx_gemm_lowrank_up if mx else sq.w4a4_gemm_lowrank_up_tiled if tiled else
           sq.w4a4_gemm_lowrank_up)
    # the tiled GEMM's split along K on under-filled shapes (as svdq_conv2d_tiled
    # with a workspace that holds it)
    need = sq.gemm_tiled_workspace_bytes(M, N, K) if tiled else 0
    k2kw = dict(workspace=torch.empty(need, dtype=torch.uint8, device="cuda")) if need else {}

    class _Runner:
        def launches(self, i):
            s = sets[i % len(sets)]
            return [("k1", lambda: k1f(s["X"], L.KH, L.KW, L.stride, L.pad, s["inv"], s["L1p"], R,
                                       s["ac"], s["asc"], s["D"])),
                    ("k2", lambda: k2f(s["ac"], s["asc"], s["wc"], s["ws"], s["D"], s["L2t"], R,
                                       s["b"], s["Y"].view(M, N), K, **k2kw))]

    settled = settle(torch, _Runner(), args.settle_ms)
    t_step, _, per = time_steps(torch, _Runner(), args.steps, args.warmup, probe)
    clock = probe.result() if probe is not None else None
    gap = event_gap(torch)
    k1_avg, k1_med = kernel_stats(per[:, 0], gap)
    k2_avg, k2_med = kernel_stats(per[:, 1], gap)
    ops = 2.0 * M * N * K
    value = ops / t_step / 1e12
    xb = 2 if L.x_dtype == "f16" else 4
    yb = 2 if L.y_dtype == "f16" else 4
    img = L.batch * L.H * L.W * L.C
    meta = meta_bytes(K, args.format)
    # K1: the image once, the patch matrix's codes, scales (or exponents) and D out
    db = 2 if args.format == "mxfp4" else 4
    b1 = img * xb + M * K // 2 + M * meta + db * M * R + 2 * K * R + 4 * K
    b2 = k2_bytes(M, N, K, R, yb, meta, db=db)
    F = FORMATS[args.format]
    fmt_txt = F["text"]
    out = {
        "metric": (f"effective {F['unit']} of an SVDQuant {'MXFP4' if mx else 'W4A4'}+rank-32 UNet "
                   f"convolution (implicit GEMM), % of {'FP4' if mx else 'INT8'} MFMA peak"),
        "value": round(value, 2), "unit": F["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": round(settled, 1),
        "ms_per_step": round(t_step * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": F["dtype"], "data": "synthetic",
        "config": {"workload": f"{L.name}: X {L.x_dtype} NHWC {L.batch}x{L.H}x{L.W}x{L.C}, "
                               f"{L.KH}x{L.KW} stride {L.stride} pad {L.pad} -> {N} channels "
                               f"(patch matrix {M}x{K}), rank {R}, {fmt_txt}, Y {L.y_dtype}",
                   "M": M, "K": K, "N": N, "rank": R, "format": args.format,
                   "path": "tiled" if tiled else ("mxfp4" if mx else "canonical"),
                   "buffer_sets": args.sets},
        F["pct"]: round(100.0 * value / F["peak"], 2),
        "roofline": {"bound": "mfma", "kernel": "k2t_w4a4_kernel" if tiled else F["kname"],
                     "achieved": round(ops / k2_avg / 1e12, 2), "peak": F["peak"],
                     "unit": F["unit"], "frac": round(ops / k2_avg / 1e12 / F["peak"], 4),
                     "traffic": None, "algorithmic_bytes": b2,
                     "avg_ms": round(k2_avg * 1e3, 4), "median_ms": round(k2_med * 1e3, 4),
                     "timing": TIMING_NOTE, "event_gap_us": round(gap * 1e6, 2)},
        "k1": {"kernel": "k1_quant_down_kernel (convolution instance)",
               "avg_ms": round(k1_avg * 1e3, 4), "median_ms": round(k1_med * 1e3, 4),
               "algorithmic_bytes": b1,
               "achieved_gbs": round(b1 / k1_avg / 1e9, 1), "peak_gbs": HBM_PEAK_GBS,
               "frac": round(b1 / k1_avg / 1e9 / HBM_PEAK_GBS, 4)},
        "clock": clock,
    }
    if args.copy_probe:
        copy_probe(torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = conv_cpu_baseline(L, X, Wm, prep, bias, args.cpu_seconds)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer is built and measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_post_quantized_smooth_amd as sq
    import workloads as wl

    probe = None if args.no_clock else ClockProbe(torch, sq)
    if args.mlp or (args.layer == "all" and args.config == 2):
        out = mlp_main(args, torch, sq, wl, probe)
    elif args.conv is not None:
        out = conv_main(args, torch, sq, wl, probe)
    elif args.layer == "all" and len(wl.CONFIGS[args.config].layers) > 1:
        out = whole_config_main(args, torch, sq, wl, probe)
    else:
        if args.layer == "all":
            args.layer = "0"
        out = single_layer_main(args, torch, sq, wl, probe)
    print(json.dumps(out), flush=True)
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
