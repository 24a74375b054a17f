"""Benchmark of the GEMM hot path on one MI355X.

One step = one 8192^3 bf16 GEMM (A row-major, B column-major, entries
N(0, 0.02^2) rounded to bf16, fp32 accumulate, bf16 output, alpha 1, beta 0)
through the library's default entry point (gemm_bf16), inputs resident in
HBM.  This is the configuration the 70%-of-peak target is stated on, so
`value` is that GEMM's TFLOP/s alone.  The 8192^3 MX block-scaled fp8 GEMM
(E4M3 entries from U[-448, 448], one E8M0 scale per 32 K elements with
exponents uniform in -8..8, bf16 output) is timed the same way in its own
loop and reported in `mx_fp8` with its fraction of the fp8 peak; no figure
mixes the two precisions.

Prints ONE JSON line.  `roofline` covers the bf16 kernel, timed with HIP
events on the stream it runs on; `cpu_baseline` times the fp64 oracle on a
bounded row sample of the bf16 GEMM on the host cores and checks those rows
of the GPU result.  `clocks` holds the GFX clock and socket power sampled
(amdsmi, every few ms) during a sustained window of back-to-back launches of
each kernel and of the matrix-core loop; `matrix_core_loop` is the rate of a
pure matrix-core loop per instruction shape (no memory traffic), the
power-limited ceiling the GEMMs run under.

Modes for profiling (no JSON): --only bf16|mxfp8|copy|e4m3|e5m2|e2m3|e3m2|e2m1
--reps R runs just that kernel R times after one warm-up (--level L: at level
L instead of the default one; copy: a 1 GiB
device-to-device copy, the calibration of the HBM byte counters; the MX
element-format names: the 8192^3 MX GEMM in that format; cfg1-cfg3: the
single-tile, 4096^3 and ragged workloads; skinny64 / skinny1: the 64 x 8192
x 8192 and 1 x 8192 x 8192 bf16 GEMMs; skinny64mx / skinny1mx: the same in
MX E4M3).  --only loop prints the matrix-core loop rates alone.  --configs
prints one JSON line timing every standard workload and the skinny shapes
against their own rooflines; --levels one line timing every level of the
ladder on every standard workload.  These modes (and --mx-formats,
--tile-orders and the attention timings) run each case back to back for a
quarter of a second before its W warm-up and K timed launches, so that it
is timed at sustained clocks rather than on the way up from idle.
--mx-formats prints one JSON line instead: the 8192^3 MX GEMM in every
element format at its default level, with W warm-up and K timed launches.
--tile-orders prints one JSON line timing the 8192^3 bf16 and MX GEMMs
under each tile walk (XCD-major or dispatch order, several group sizes).
--attention prints one JSON line timing the fused attention forward on the
16k-token workloads (4 x 4096 tokens, 16 heads of 128; causal and full),
with the oracle timed on a row sample beside it; --only attn-causal|attn-full
runs one of them R times for profiling.  The default line carries the same
timings in `attention`.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2516.6     # TFLOP/s dense: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_FP8 = 5033.2      # TFLOP/s dense: 256 CU x 8192 flop/clk x 2.4 GHz
PEAK_FP4 = 10066.3     # TFLOP/s dense fp6 / fp4: 256 CU x 16384 flop/clk x 2.4 GHz
PEAK_HBM = 8000.0      # GB/s
METRIC = "GEMM TFLOP/s and % of dense MFMA peak (bf16, MX-fp8) at 8192³ on 1 MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_bf16_8192.txt")
KERNEL_SOURCES = ["matrix_core_engineering_amd/csrc/kernels_fast.hpp",
                  "matrix_core_engineering_amd/csrc/k_fast_bf16.hip",
                  "matrix_core_engineering_amd/csrc/common.hpp",
                  "matrix_core_engineering_amd/csrc/sched.hpp",
                  "matrix_core_engineering_amd/csrc/epilogue.hpp",
                  "matrix_core_engineering_amd/csrc/ring_plan.hpp"]


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=["bf16", "mxfp8", "copy", "loop", "cfg1", "cfg2", "cfg3",
                                       "attn-causal", "attn-full", "skinny64", "skinny1", "skinny64mx",
                                       "skinny1mx"]
                    + list(MX_FORMAT_NAMES),
                    default=None)
    ap.add_argument("--levels", action="store_true",
                    help="time every level on every standard workload (one JSON line)")
    ap.add_argument("--configs", action="store_true",
                    help="time every standard workload against its roofline (one JSON line)")
    ap.add_argument("--mx-formats", action="store_true",
                    help="time the 8192^3 MX GEMM in every element format (one JSON line)")
    ap.add_argument("--attention", action="store_true",
                    help="time the fused attention workloads (one JSON line)")
    ap.add_argument("--tile-orders", action="store_true",
                    help="time the 8192^3 GEMMs under each tile walk (one JSON line)")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--level", type=int, default=None,
                    help="with --only bf16|mxfp8|cfgN: run that level instead of the default")
    ap.add_argument("--order", type=str, default=None,
                    help="with --only bf16|mxfp8: tile walk 'X,G' (X 1 XCD-major or 0 dispatch "
                         "order, G tile rows per group) through gemm_bf16_order / gemm_mx_order")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


class Workload:
    """One standard workload's operands resident on the device."""

    def __init__(self, cfg, dev):
        import torch
        from matrix_core_engineering_amd.inputs import config_problem, skinny_problem
        self.p = p = config_problem(cfg) if isinstance(cfg, int) else skinny_problem(cfg)

        def up(a):
            v = {1: np.uint8, 2: np.int16, 4: np.int32}[a.dtype.itemsize]
            return torch.from_numpy(np.ascontiguousarray(a).view(v)).to(dev)

        self.A, self.B = up(p.A), up(p.B)
        self.SA = up(p.SA) if p.SA is not None else None
        self.SB = up(p.SB) if p.SB is not None else None
        self.C = torch.zeros((p.M, p.ldc), dtype=torch.int16 if p.c_dtype == 1 else torch.float32,
                             device=dev)

    def run(self, stream):
        import matrix_core_engineering_amd as mce
        p = self.p
        if p.SA is None:
            return mce.gemm_bf16(p.M, p.N, p.K, self.A, p.lda, p.a_col_major, self.B, p.ldb,
                                 p.b_col_major, self.C, p.ldc, p.c_col_major, p.c_dtype,
                                 p.alpha, p.beta, stream=stream)
        return mce.gemm_mxfp8(p.M, p.N, p.K, self.A, p.lda, p.a_col_major, self.SA, p.ld_sa,
                              self.B, p.ldb, p.b_col_major, self.SB, p.ld_sb, self.C, p.ldc,
                              p.c_col_major, p.c_dtype, p.alpha, p.beta, stream=stream)

    def run_level(self, level, stream):
        """The same call at a fixed level; returns the library's status."""
        import matrix_core_engineering_amd as mce
        p = self.p
        if p.SA is None:
            return mce.gemm_bf16_level(level, p.M, p.N, p.K, self.A, p.lda, p.a_col_major, self.B,
                                       p.ldb, p.b_col_major, self.C, p.ldc, p.c_col_major,
                                       p.c_dtype, p.alpha, p.beta, stream=stream,
                                       raise_on_error=False)
        return mce.gemm_mxfp8_level(level, p.M, p.N, p.K, self.A, p.lda, p.a_col_major, self.SA,
                                    p.ld_sa, self.B, p.ldb, p.b_col_major, self.SB, p.ld_sb,
                                    self.C, p.ldc, p.c_col_major, p.c_dtype, p.alpha, p.beta,
                                    stream=stream, raise_on_error=False)

    def run_order(self, xcd, group_m, stream):
        """The default level with a chosen tile walk; returns the status."""
        import matrix_core_engineering_amd as mce
        p = self.p
        if p.SA is None:
            return mce.gemm_bf16_order(0, xcd, group_m, p.M, p.N, p.K, self.A, p.lda, p.a_col_major,
                                       self.B, p.ldb, p.b_col_major, self.C, p.ldc, p.c_col_major,
                                       p.c_dtype, p.alpha, p.beta, stream=stream,
                                       raise_on_error=False)
        return mce.gemm_mx_order(0, xcd, group_m, mce.MCE_MX_E4M3, p.M, p.N, p.K, self.A, p.lda,
                                 p.a_col_major, self.SA, p.ld_sa, self.B, p.ldb, p.b_col_major,
                                 self.SB, p.ld_sb, self.C, p.ldc, p.c_col_major, p.c_dtype, p.alpha,
                                 p.beta, stream=stream, raise_on_error=False)

    def level(self):
        import matrix_core_engineering_amd as mce
        p = self.p
        if p.SA is None:
            return mce.gemm_bf16_pick_level(p.M, p.N, p.K, self.A, p.lda, p.a_col_major, self.B,
                                            p.ldb, p.b_col_major)
        return mce.gemm_mxfp8_pick_level(p.M, p.N, p.K, self.A, p.lda, p.a_col_major, self.B,
                                         p.ldb, p.b_col_major)


# MX element formats: name -> (generator format, library code, dense peak)
MX_FORMAT_NAMES = ("e4m3", "e5m2", "e2m3", "e3m2", "e2m1")


def mx_format_table():
    import matrix_core_engineering_amd as mce
    from matrix_core_engineering_amd.inputs import E2M1, E2M3, E3M2, E4M3FN, E5M2
    return {"e4m3": (E4M3FN, mce.MCE_MX_E4M3, PEAK_FP8), "e5m2": (E5M2, mce.MCE_MX_E5M2, PEAK_FP8),
            "e2m3": (E2M3, mce.MCE_MX_E2M3, PEAK_FP4), "e3m2": (E3M2, mce.MCE_MX_E3M2, PEAK_FP4),
            "e2m1": (E2M1, mce.MCE_MX_E2M1, PEAK_FP4)}


class MxFormatWorkload:
    """The 8192^3 MX workload (A row-major, B column-major, one E8M0 scale
    per 32 K with exponents -8..8, bf16 out) in one element format: 8-bit
    codes from U[-448, 448], the packed formats every code equally likely."""

    def __init__(self, name, dev, a_col_major=False, b_col_major=True):
        import torch
        from matrix_core_engineering_amd.inputs import E4M3FN, E5M2, OUT_BF16, make_problem
        gfmt, self.code, self.peak = mx_format_table()[name]
        kw = (dict(dist="uniform", lo=-448.0, hi=448.0) if gfmt in (E4M3FN, E5M2)
              else dict(dist="codes"))
        self.a_cm, self.b_cm = int(a_col_major), int(b_col_major)
        self.p = p = make_problem(8192, 8192, 8192, fmt=gfmt, a_col_major=a_col_major,
                                  b_col_major=b_col_major, c_dtype=OUT_BF16, seed=5,
                                  name=f"mx_{name}_8192", **kw)

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        self.A, self.B, self.SA, self.SB = up(p.A), up(p.B), up(p.SA), up(p.SB)
        self.C = torch.zeros((p.M, p.ldc), dtype=torch.int16, device=dev)

    def run(self, stream):
        import matrix_core_engineering_amd as mce
        p = self.p
        return mce.gemm_mx(self.code, p.M, p.N, p.K, self.A, p.lda, self.a_cm, self.SA, p.ld_sa,
                           self.B, p.ldb, self.b_cm, self.SB, p.ld_sb, self.C, p.ldc, 0, p.c_dtype,
                           p.alpha, p.beta, stream=stream)

    def level(self):
        import matrix_core_engineering_amd as mce
        p = self.p
        return mce.gemm_mx_pick_level(self.code, p.M, p.N, p.K, self.A, p.lda, self.a_cm, self.SA,
                                      p.ld_sa, self.B, p.ldb, self.b_cm, self.SB, p.ld_sb)


def mx_formats(args, dev, stream):
    """One JSON line: each element format's 8192^3 GEMM at its default level
    (and the 8-bit formats with MN-major operands: A column-major, or A
    column-major and B row-major), HIP events on the launch stream around
    each launch."""
    import torch
    res = {}
    cases = [(n, n, False, True) for n in MX_FORMAT_NAMES]
    cases += [(f"{n}_a_col", n, True, True) for n in ("e4m3", "e5m2")]
    cases += [(f"{n}_a_col_b_row", n, True, False) for n in ("e4m3", "e5m2")]
    for key, name, a_cm, b_cm in cases:
        w = MxFormatWorkload(name, dev, a_cm, b_cm)
        prewarm(lambda: w.run(stream))
        for _ in range(args.warmup):
            w.run(stream)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record(stream)
        for s in range(args.steps):
            w.run(stream)
            ev[s + 1].record(stream)
        torch.cuda.synchronize()
        us = float(np.mean([ev[s].elapsed_time(ev[s + 1]) for s in range(args.steps)])) * 1e3
        tf = w.p.flops / (us * 1e-6) / 1e12
        res[key] = {"level": w.level(), "us_per_launch": us, "tflops": tf, "peak_tflops": w.peak,
                    "frac_of_peak": tf / w.peak}
        del w
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "MX GEMM TFLOP/s by element format, 8192^3, bf16 out",
                      "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "data": "synthetic", "per_format": res}), flush=True)


CEILING_SHAPES = (("bf16_32x32x16", 0, "bf16", PEAK_BF16),
                  ("bf16_16x16x32", 1, "bf16", PEAK_BF16),
                  ("mxfp8_32x32x64", 2, "e4m3", PEAK_FP8),
                  ("mxfp4_32x32x64", 3, "e2m1", PEAK_FP4),
                  ("mxfp6_32x32x64", 4, "e2m3", PEAK_FP4))


def matrix_core_ceiling(dev, stream, iters=2000, reps=3):
    """Sustained rate of the pure matrix-core loop (mce_matrix_core_loop, one
    workgroup per CU, one wave per SIMD, no memory traffic in the loop) per
    instruction shape, on the bench workloads' value distributions (bf16 from
    N(0, 0.02^2), E4M3 from U[-448, 448]): the power-limited ceiling that the
    GEMM kernels run under."""
    import torch
    import matrix_core_engineering_amd as mce
    g = torch.Generator().manual_seed(7)
    nfrag = 1 << 16
    bufs = {"bf16": (torch.randn(nfrag * 8, generator=g) * 0.02).to(torch.bfloat16)
                    .view(torch.int16).to(dev),
            "e4m3": (torch.rand(nfrag * 32, generator=g) * 896.0 - 448.0)
                    .to(torch.float8_e4m3fn).view(torch.uint8).to(dev),
            # every E2M1 code equally likely, two per byte (no NaN or Inf codes)
            "e2m1": torch.randint(0, 256, (nfrag * 32,), generator=g, dtype=torch.uint8).to(dev),
            # every E2M3 code equally likely, four per three bytes (no NaN or
            # Inf codes in the 6-bit formats)
            "e2m3": torch.randint(0, 256, (nfrag * 32,), generator=g, dtype=torch.uint8).to(dev)}
    blocks = 256
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    flops = blocks * 4 * iters * float(1 << 21)
    res = {}
    for name, shape, data, peak in CEILING_SHAPES:
        mce.mce_matrix_core_loop(shape, bufs[data], nfrag, out, blocks, iters // 4, stream=stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            mce.mce_matrix_core_loop(shape, bufs[data], nfrag, out, blocks, iters, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        tf = flops / (us * 1e-6) / 1e12
        res[name] = {"tflops": tf, "frac_of_peak": tf / peak, "us_per_launch": us}
    return res


def algorithmic_bytes(p):
    """HBM bytes a GEMM must move at least: A, B and the MX scales read once,
    C read when beta != 0, C written once."""
    elt = 1 if p.SA is not None else 2
    c_elt = 2 if p.c_dtype == 1 else 4
    scales = (p.M + p.N) * ((p.K + 31) // 32) if p.SA is not None else 0
    c_bytes = p.M * p.N * c_elt
    return p.M * p.K * elt + p.K * p.N * elt + scales + c_bytes * (2 if p.beta != 0 else 1)


def prewarm(run, seconds=0.25):
    """Runs `run` back to back for about `seconds` of wall time.  From idle
    (input generation on the host leaves the GPU idle for a second or more)
    the GPU takes tens of milliseconds of work to reach its sustained
    clocks; a 4096^3 GEMM measured 118 us after 20 warm-up launches (2 ms)
    and 102-106 us after 300 (30 ms) on the same boxes."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            run()
        torch.cuda.synchronize()


def configs(args, dev, stream):
    """One JSON line: every standard workload and the skinny shapes through
    the default entry point, each against the roofline that bounds it
    (matrix cores, or HBM when its flops per algorithmic byte are below the
    ridge; a square-ish problem of fewer 128x128 tiles than CUs occupies
    part of one CU set and is reported as latency-bound, with no roofline
    fraction).  HBM-bound workloads are timed cold: a 512 MiB fill before
    every launch evicts L2 and the Infinity Cache, and only the GEMM is
    timed."""
    import torch
    from matrix_core_engineering_amd.inputs import SKINNY
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    res = {}
    for cfg in (1, 2, 3, 4, 5) + tuple(SKINNY):
        w = Workload(cfg, dev)
        p = w.p
        peak = PEAK_FP8 if p.SA is not None else PEAK_BF16
        nbytes = algorithmic_bytes(p)
        skinny = min(p.M, p.N) <= 256 and max(p.M, p.N) >= 4096
        latency = not skinny and ((p.M + 127) // 128) * ((p.N + 127) // 128) < 256
        hbm_bound = not latency and p.flops / nbytes < peak * 1e12 / (PEAK_HBM * 1e9)
        prewarm(lambda: w.run(stream))
        for _ in range(args.warmup):
            w.run(stream)
        torch.cuda.synchronize()
        # launches back to back (the scrub fill, when there is one, runs on
        # the same stream just before each launch); events around each launch
        evs = []
        for _ in range(args.steps):
            if hbm_bound:
                scrub.fill_(len(res) + 1)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            w.run(stream)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        times = [e0.elapsed_time(e1) * 1e3 for e0, e1 in evs]
        us = float(np.median(times))
        tf = p.flops / (us * 1e-6) / 1e12
        gbs = nbytes / (us * 1e-6) / 1e9
        res[p.name] = {"level": w.level(), "us_median": us, "us_min": float(min(times)),
                       "tflops": tf, "algorithmic_bytes": nbytes, "gb_per_s": gbs,
                       "bound": "latency" if latency else "hbm" if hbm_bound else "mfma",
                       "frac": None if latency else gbs / PEAK_HBM if hbm_bound else tf / peak,
                       "peak": None if latency else PEAK_HBM if hbm_bound else peak,
                       "timed": "cold (512 MiB scrub before each launch)" if hbm_bound else "warm"}
        del w
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "GEMM time per standard workload vs its roofline", "n_gpus": 1,
                      "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
                      "per_config": res}), flush=True)


def levels(args, dev, stream):
    """One JSON line: every level of the ladder on every standard workload
    (warm, back to back, events around each launch, median), null where the
    level declines the problem."""
    import torch
    import matrix_core_engineering_amd as mce
    res = {}
    for cfg in (1, 2, 3, 4, 5):
        w = Workload(cfg, dev)
        p = w.p
        row = {}
        for level in (1, 2, 3, 4, 5, 6, 7, 9):
            if w.run_level(level, stream) != mce.MCE_OK:
                row[str(level)] = None
                continue
            prewarm(lambda: w.run_level(level, stream))
            for _ in range(args.warmup):
                w.run_level(level, stream)
            evs = []
            for _ in range(args.steps):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                w.run_level(level, stream)
                e1.record(stream)
                evs.append((e0, e1))
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))
            row[str(level)] = {"us_median": us, "tflops": p.flops / (us * 1e-6) / 1e12}
        res[p.name] = row
        del w
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "GEMM time per level and standard workload", "n_gpus": 1,
                      "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
                      "per_config": res}), flush=True)


def read_traffic(level):
    """HBM bytes per launch of the bf16 kernel from the committed counter
    summary, or None if it is missing, was taken on other kernel code or on
    another level's kernel."""
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_hash") != kernel_source_hash():
            return None
        if int(kv.get("kernel_level", -1)) != level:
            return None
        return float(kv["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class AttentionWorkload:
    """One attention workload (bf16 Q, K, V resident on the device, bf16 O)
    through attention_bf16."""

    def __init__(self, name, dev):
        import torch
        from matrix_core_engineering_amd.inputs import (ATTENTION_WORKLOADS, attention_flops,
                                                        attention_inputs)
        self.name = name
        self.w = w = dict(ATTENTION_WORKLOADS[name])
        self.shape = (w["batch"], w["heads"], w["seq_q"], w["seq_k"], w["dim"])
        self.host = attention_inputs(*self.shape, seed=7)
        self.Q, self.K, self.V = (torch.from_numpy(x.view(np.int16)).to(dev) for x in self.host)
        self.O = torch.zeros_like(self.Q)
        self.scale = 1.0 / float(np.sqrt(w["dim"]))
        self.flops = attention_flops(*self.shape, w["causal"])

    def run(self, stream):
        import matrix_core_engineering_amd as mce
        return mce.attention_bf16(*self.shape, self.Q, self.K, self.V, self.O, mce.MCE_OUT_BF16,
                                  self.scale, self.w["causal"], stream=stream)

    def describe(self):
        B, H, S, T, D = self.shape
        return (f"attention forward, {B} x {S} queries and keys, {H} heads of {D}, "
                f"{'causal' if self.w['causal'] else 'full'}, N(0,1) bf16 Q/K/V, bf16 out")


def attention_cpu_baseline(work, target_s):
    """The oracle on the first query rows of the flattened batch x heads x
    seq_q order of an attention workload, sized to about target_s seconds,
    with those rows of the GPU result checked; flops counted as the
    kernel's (4 dim per visible query-key pair)."""
    import oracle
    B, H, S, T, D = work.shape
    causal = work.w["causal"]
    q, k, v = work.host

    def pairs(r0, r1):
        i = np.arange(r0, r1) % S
        if not causal:
            return float(len(i) * T)
        return float(np.clip(i + T - S + 1, 0, T).sum())

    cal = min(B * H * S, 2 * S)      # two whole heads: every row length
    t0 = time.perf_counter()
    oracle.attention(B, H, S, T, D, q, k, v, np.float32(work.scale), causal, 0, cal)
    per_pair = max((time.perf_counter() - t0) / pairs(0, cal), 1e-12)
    rows = int(min(B * H * S, max(cal, target_s / (per_pair * pairs(0, S)) * S)))
    t0 = time.perf_counter()
    oref, pv, smax = oracle.attention(B, H, S, T, D, q, k, v, np.float32(work.scale), causal,
                                      0, rows)
    secs = time.perf_counter() - t0
    got = work.O.reshape(-1, D)[:rows].cpu().numpy().view(np.uint16)
    got = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ok, worst, _ = oracle.check_attention(got, oref, pv, smax, T, True)
    return {"value": 4.0 * D * pairs(0, rows) / secs / 1e12, "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the first {rows} of {B * H * S} query rows (batch x head x query order), "
                      f"fp64, {secs:.1f} s",
            "seconds": secs, "sample_rows_checked_ok": bool(ok),
            "sample_worst_err_over_tol": worst}


def attention_timings(dev, stream, warmup, steps, cpu_seconds=None):
    out = {}
    for name in ("causal", "full"):
        work = AttentionWorkload(name, dev)
        prewarm(lambda: work.run(stream))
        t, _ = timed_steps(work, warmup, steps, stream)
        ms = float(np.mean(t))
        tf = work.flops / (ms * 1e-3) / 1e12
        out[name] = {"workload": work.describe(), "flops_per_launch": work.flops,
                     "us_per_launch": ms * 1e3, "us_median": float(np.median(t)) * 1e3,
                     "tflops": tf, "peak_tflops": PEAK_BF16, "frac_of_peak": tf / PEAK_BF16}
        if cpu_seconds:
            out[name]["cpu_baseline"] = attention_cpu_baseline(work, cpu_seconds)
        del work
    return out


def cpu_baseline(work, target_s):
    """Times the oracle on rows [0, R) of the bf16 workload (R sized for
    about target_s seconds) and checks those rows of the GPU result."""
    import oracle
    import torch
    p = work.p
    kw = p.oracle_kwargs()
    # two calibration runs separate the fixed cost (decoding all of B) from
    # the per-row cost; then the sample
    t0 = time.perf_counter()
    oracle.gemm_rows(row_begin=0, row_end=16, **kw)
    t16 = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.gemm_rows(row_begin=0, row_end=64, **kw)
    t64 = time.perf_counter() - t0
    per_row = max((t64 - t16) / 48, 1e-5)
    fixed = max(t16 - 16 * per_row, 0.0)
    rows = int(min(p.M, max(64, (target_s - fixed) / per_row)))
    t0 = time.perf_counter()
    cref, tsum = oracle.gemm_rows(row_begin=0, row_end=rows, **kw)
    secs = time.perf_counter() - t0
    got_bits = work.C[:rows, :p.N].cpu().numpy().view(np.uint16)
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ok, worst, bad = oracle.check(got, cref, tsum, out_bf16=True)
    flops = 2.0 * rows * p.N * p.K
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"rows 0..{rows - 1} of the 8192^3 bf16 GEMM (all 8192 columns, full K), "
                      f"fp64, {secs:.1f} s",
            "seconds": secs, "sample_rows_checked_ok": bool(ok),
            "sample_worst_err_over_tol": worst}


def timed_steps(work, warmup, steps, stream):
    """W untimed launches, then K launches with HIP events on the launch
    stream around each; returns (per-launch ms list, wall seconds)."""
    import torch
    for _ in range(warmup):
        work.run(stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for s in range(steps):
        work.run(stream)
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [ev[s].elapsed_time(ev[s + 1]) for s in range(steps)], wall


class ClockSampler:
    """Samples the GFX clock (MHz) and the socket power (W) of GPU 0 through
    the amdsmi Python module every few milliseconds in a thread.  Where
    amdsmi cannot be used the samples stay empty and the reason is kept."""

    def __init__(self, period_s=0.005):
        import threading
        self.period = period_s
        self.sclk, self.power, self.error = [], [], None
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            try:
                h = amdsmi.amdsmi_get_processor_handles()[0]
                while not self._stop.is_set():
                    clk = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
                    pw = amdsmi.amdsmi_get_power_info(h)
                    c = clk.get("clk", clk.get("cur_clk"))
                    p = pw.get("socket_power", pw.get("current_socket_power"))
                    if isinstance(c, (int, float)):
                        self.sclk.append(float(c))
                    if isinstance(p, (int, float)):
                        self.power.append(float(p))
                    self._stop.wait(self.period)
            finally:
                amdsmi.amdsmi_shut_down()
        except Exception as e:   # reported, never fatal to the benchmark
            self.error = f"{type(e).__name__}: {e}"

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self):
        def stats(v):
            if not v:
                return None
            return {"median": float(np.median(v)), "min": float(np.min(v)),
                    "max": float(np.max(v)), "samples": len(v)}
        return {"sclk_mhz": stats(self.sclk), "socket_power_w": stats(self.power),
                "error": self.error}


def sustained_window(work, stream, seconds=2.0):
    """Back-to-back launches for about `seconds` with the clock sampler on;
    returns the sampled clock and power with the window's own rate."""
    import torch
    t_one, _ = timed_steps(work, 2, 5, stream)
    n = max(10, int(seconds / (np.mean(t_one) * 1e-3)))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with ClockSampler() as cs:
        e0.record(stream)
        for _ in range(n):
            work.run(stream)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    out = cs.summary()
    out.update({"launches": n, "us_per_launch": ms * 1e3,
                "tflops": work.p.flops / (ms * 1e-3) / 1e12})
    return out


def sustained_loop(dev, stream, shape, seconds=2.0):
    """The matrix-core loop (one instruction shape) for about `seconds` with
    the clock sampler on."""
    import torch
    import matrix_core_engineering_amd as mce
    g = torch.Generator().manual_seed(7)
    nfrag = 1 << 16
    frags = (torch.randn(nfrag * 8, generator=g) * 0.02).to(torch.bfloat16).view(torch.int16).to(dev)
    blocks, iters = 256, 2000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    flops = blocks * 4 * iters * float(1 << 21)
    mce.mce_matrix_core_loop(shape, frags, nfrag, out, blocks, iters // 4, stream=stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    mce.mce_matrix_core_loop(shape, frags, nfrag, out, blocks, iters, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    n = max(3, int(seconds / (e0.elapsed_time(e1) * 1e-3)))
    with ClockSampler() as cs:
        e0.record(stream)
        for _ in range(n):
            mce.mce_matrix_core_loop(shape, frags, nfrag, out, blocks, iters, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    res = cs.summary()
    res.update({"launches": n, "us_per_launch": ms * 1e3, "tflops": flops / (ms * 1e-3) / 1e12})
    return res


def tile_orders(args, dev, stream):
    """One JSON line: the 8192^3 bf16 and MX GEMMs at their default level
    under each tile walk (XCD-major or dispatch-order workgroup slots, tile
    rows per group), warm, interleaved rounds of launches, HIP events."""
    import torch
    import matrix_core_engineering_amd as mce
    orders = [(1, 8), (1, 4), (1, 2), (1, 16), (1, 32), (1, 1), (0, 8), (0, 4)]
    res = {}
    for cfg, name in ((4, "bf16_8192"), (5, "mxfp8_8192")):
        w = Workload(cfg, dev)
        p = w.p

        def run(xcd, gm):
            st = w.run_order(xcd, gm, stream)
            assert st == mce.MCE_OK, mce.gemm_status_string(st)

        times = {o: [] for o in orders}
        prewarm(lambda: run(1, 8))
        for _ in range(args.warmup):
            run(1, 8)
        for rnd in range(5):
            for o in orders:
                evs = []
                for _ in range(max(1, args.steps // 5)):
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    run(*o)
                    e1.record(stream)
                    evs.append((e0, e1))
                torch.cuda.synchronize()
                times[o] += [a.elapsed_time(b) * 1e3 for a, b in evs]
        res[name] = {f"{'xcd' if o[0] else 'dispatch'}_g{o[1]}":
                     {"us_median": float(np.median(t)), "us_min": float(np.min(t)),
                      "tflops": p.flops / (float(np.median(t)) * 1e-6) / 1e12}
                     for o, t in times.items()}
        del w
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "8192^3 GEMM time per tile walk", "n_gpus": 1,
                      "steps": args.steps, "warmup": args.warmup, "data": "synthetic",
                      "per_workload": res}), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {args.gpus} requested); "
              "the multi-GPU split of the GEMM is a design note, not a measured path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import matrix_core_engineering_amd as mce
    mce.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.only == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.reps + 1):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {args.reps + 1} x {n} bytes", flush=True)
        return
    if args.mx_formats:
        mx_formats(args, dev, stream)
        return
    if args.configs:
        configs(args, dev, stream)
        return
    if args.levels:
        levels(args, dev, stream)
        return
    if args.tile_orders:
        tile_orders(args, dev, stream)
        return
    if args.attention:
        res = attention_timings(dev, stream, args.warmup, args.steps,
                                None if args.no_cpu_baseline else args.cpu_seconds)
        print(json.dumps({"attention": res}), flush=True)
        return
    if args.only in ("attn-causal", "attn-full"):
        work = AttentionWorkload(args.only[5:], dev)
        for _ in range(args.reps + 1):
            work.run(stream)
        torch.cuda.synchronize()
        print(f"ran {args.only} x {args.reps + 1}", flush=True)
        return
    if args.only == "loop":
        res = matrix_core_ceiling(dev, stream, reps=args.reps)
        print(json.dumps({"matrix_core_loop": res}), flush=True)
        return
    if args.only in MX_FORMAT_NAMES:
        work = MxFormatWorkload(args.only, dev)
        for _ in range(args.reps + 1):
            work.run(stream)
        torch.cuda.synchronize()
        print(f"ran {args.only} level {work.level()} x {args.reps + 1}", flush=True)
        return
    if args.only:
        work = Workload({"bf16": 4, "mxfp8": 5, "cfg1": 1, "cfg2": 2, "cfg3": 3,
                         "skinny64": "skinny_64x8192x8192_bf16",
                         "skinny1": "skinny_1x8192x8192_bf16",
                         "skinny64mx": "skinny_64x8192x8192_mxfp8",
                         "skinny1mx": "skinny_1x8192x8192_mxfp8"}[args.only], dev)
        for _ in range(args.reps + 1):
            if args.order is not None:
                xcd, gm = (int(v) for v in args.order.split(","))
                if work.run_order(xcd, gm, stream) != mce.MCE_OK:
                    print(f"order {args.order} declined", file=sys.stderr, flush=True)
                    sys.exit(2)
            elif args.level is None:
                work.run(stream)
            elif work.run_level(args.level, stream) != mce.MCE_OK:
                print(f"level {args.level} declines {args.only}", file=sys.stderr, flush=True)
                sys.exit(2)
        torch.cuda.synchronize()
        lvl = work.level() if args.level is None else args.level
        print(f"ran {args.only} level {lvl} x {args.reps + 1}", flush=True)
        return

    bf16 = Workload(4, dev)
    mx = Workload(5, dev)
    # measurements reported beside the headline, taken first: the clock and
    # power of each kernel over a 2 s window of back-to-back launches, and
    # the matrix-core loop rates; they also bring the clocks to their
    # sustained state before the timed steps
    clocks = {"bf16_8192": sustained_window(bf16, stream),
              "mxfp8_8192": sustained_window(mx, stream),
              "matrix_core_loop_bf16_16x16x32": sustained_loop(dev, stream, 1)}
    ceiling = matrix_core_ceiling(dev, stream)
    # the headline: W warm-up launches, then K timed launches (HIP events)
    t_bf16, wall = timed_steps(bf16, args.warmup, args.steps, stream)
    t_mx, _ = timed_steps(mx, args.warmup, args.steps, stream)
    ms_per_step = float(np.mean(t_bf16))
    value = bf16.p.flops / (ms_per_step * 1e-3) / 1e12
    tf_mx = mx.p.flops / (float(np.mean(t_mx)) * 1e-3) / 1e12
    attention = attention_timings(dev, stream, args.warmup, args.steps)
    traffic = read_traffic(bf16.level())
    # the default bf16 kernel for whole 256x256 bf16 tiles runs 16x16x32
    loop_bf16 = ceiling["bf16_16x16x32"]["tflops"]
    loop_mx = ceiling["mxfp8_32x32x64"]["tflops"]
    roofline = {"bound": "mfma", "achieved": value, "peak": PEAK_BF16, "unit": "TFLOP/s",
                "frac": value / PEAK_BF16, "traffic": traffic,
                "traffic_counters": "FETCH_SIZE + WRITE_SIZE per launch: bytes between the "
                                    "L2 (TCC) and the fabric, so reads served by the "
                                    "Infinity Cache count too; scaled by a 1 GiB copy",
                "kernel": f"bf16_8192 (level {bf16.level()})",
                "flops_per_launch": bf16.p.flops, "us_per_launch": ms_per_step * 1e3,
                "sustained_loop_tflops": loop_bf16,
                "frac_of_sustained_loop": value / loop_bf16}
    out = {"metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "8192^3 bf16 GEMM, N(0, 0.02^2) entries, A row-major, "
                                  "B column-major, fp32 accumulate, bf16 out",
                      "M": 8192, "N": 8192, "K": 8192, "alpha": 1.0, "beta": 0.0},
           "us_min": float(np.min(t_bf16)) * 1e3, "us_median": float(np.median(t_bf16)) * 1e3,
           "roofline": roofline,
           "mx_fp8": {"workload": "8192^3 MX GEMM, E4M3 from U[-448, 448], E8M0 exponents "
                                  "-8..8 per 32 K, A row-major, B column-major, bf16 out",
                      "dtype": "mxfp8-e4m3", "level": mx.level(), "tflops": tf_mx,
                      "peak_tflops": PEAK_FP8, "frac_of_peak": tf_mx / PEAK_FP8,
                      "us_per_launch": float(np.mean(t_mx)) * 1e3,
                      "us_median": float(np.median(t_mx)) * 1e3,
                      "sustained_loop_tflops": loop_mx, "frac_of_sustained_loop": tf_mx / loop_mx},
           "attention": attention,
           "clocks": clocks, "matrix_core_loop": ceiling, "wall_s_timed": wall}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(bf16, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
