"""Benchmark of the W8A8 INT8 linear layer on one MI355X.

Headline: INT8 TOPS of one step = per-token quantization + INT8 GEMM with the
dequant epilogue on the prefill workload with outlier channels (X bf16
[2048, 4096], W int8 [4096, 4096], bf16 out); ops = 2 M N K per step.  Also
measured in the same run: HBM GB/s of the decode linear at M = 1 (X bf16
[1, 4096], W int8 [4096, 14336]; bytes = W + s_ch + X + out per call).

Inputs are seeded synthetic tensors resident in HBM before timing starts.
Before the W warmup steps the captured steps are replayed for --settle-seconds
(default 0.2 s): after idling, the GPU takes tens of milliseconds to reach its
steady clock, and a short warmup would time that ramp instead.
Each step uses the next of R buffer sets (R x ~59 MB > the 256 MB Infinity
Cache plus L2), so weights and activations come from HBM, not cache.  Steps
are captured in HIP graphs and replayed, so the GPU is not left waiting for
per-launch Python work; exactly K steps are timed with HIP events on the
replay stream.

Prints one JSON line (rank 0; one GPU only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0     # MI355X dense INT8 MFMA, published
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
FP8_PEAK_TFLOPS = 5000.0    # MI355X dense FP8 MFMA, published
CSRC = os.path.join(ROOT, "w8a8_int8_quantized_qk_amd", "csrc")
# the 2048 x 4096 x 4096 GEMM (128 tiles of 256 x 256, fewer than the CUs; k a
# multiple of 128) runs the 256 x 128 kernel with separate transfer and
# matrix-core waves
GEMM_KERNEL = "gemm_i8_spec_kernel"
GEMM_TRAFFIC = (os.path.join(ROOT, "profiles", "gemm_spec_prefill_outliers_traffic.txt"),
                [os.path.join(CSRC, f) for f in ("gemm_spec.hip", "gemm_tile.h", "lds_dma.h")])
GEMV_TRAFFIC = (os.path.join(ROOT, "profiles", "gemv_decode_m1_traffic.txt"),
                [os.path.join(CSRC, f) for f in ("gemv.hip", "quant_math.h", "lds_dma.h")])
FP8_TRAFFIC = (os.path.join(ROOT, "profiles", "gemm_fp8_prefill_outliers_traffic.txt"),
               [os.path.join(CSRC, f) for f in ("gemm_slice.hip", "gemm_tile.h", "lds_dma.h")])
GROUPED_TRAFFIC = (os.path.join(ROOT, "profiles", "gemm_grouped128_prefill_outliers_traffic.txt"),
                   [os.path.join(CSRC, f) for f in ("gemm_slice.hip", "gemm_tile.h", "lds_dma.h")])
# the MoE up-projection (4096 routed rows x 14336) takes the 256 x 256 tiles
MOE_KERNEL = "gemm_i8_wide_moe_kernel"
MOE_TRAFFIC = (os.path.join(ROOT, "profiles", "gemm_wide_moe_up_traffic.txt"),
               [os.path.join(CSRC, f) for f in ("gemm_wide.hip", "gemm_tile.h", "lds_dma.h")])
# the zero-point GEMM at the prefill shape takes the kernel with transfer waves too
ASYM_KERNEL = "gemm_i8_spec_asym_kernel"
ASYM_TRAFFIC = (os.path.join(ROOT, "profiles", "gemm_spec_asym_prefill_outliers_traffic.txt"),
                [os.path.join(CSRC, f) for f in ("gemm_spec.hip", "gemm_tile.h", "lds_dma.h")])
STATIC_TRAFFIC = (os.path.join(ROOT, "profiles", "quant_static_prefill_outliers_traffic.txt"),
                  [os.path.join(CSRC, f) for f in ("quant_static.hip", "quant_math.h")])
GEMV_M8_TRAFFIC = (os.path.join(ROOT, "profiles", "gemv_mfma_decode_m8_traffic.txt"),
                   [os.path.join(CSRC, f) for f in ("gemv.hip", "quant_math.h", "lds_dma.h")])


def _args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--repeats", type=int, default=5,
                   help="timed blocks of exactly --steps steps each; the median is reported")
    p.add_argument("--ring", type=int, default=8, help="buffer sets cycled through")
    p.add_argument("--settle-seconds", type=float, default=0.2,
                   help="replay the captured steps this long before the warmup steps: the GPU "
                        "takes tens of milliseconds to reach its steady clock after idling")
    p.add_argument("--decode-calls", type=int, default=400)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target duration of the CPU oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-fp8", action="store_true", help="skip the FP8 layer at the prefill shape")
    p.add_argument("--no-moe", action="store_true", help="skip the MoE grouped GEMM")
    p.add_argument("--moe-per-expert", action="store_true",
                   help="also time the MoE work as one plain GEMM launch per expert")
    p.add_argument("--no-static-asym", action="store_true",
                   help="skip the static and asymmetric variants")
    p.add_argument("--no-grouped", action="store_true",
                   help="skip the INT8 GEMM with per-group weight scales at the prefill shape")
    p.add_argument("--no-other-configs", action="store_true",
                   help="skip the other workload shapes (8-row decode, gated down, MLP up)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain copy kernel of known size (for counter scaling)")
    return p.parse_args()


def _code_sha(paths):
    """SHA-256 prefix of a kernel's source files (concatenated in order) with
    comments and blank lines removed, so that a comment edit does not orphan
    counter data taken on that code."""
    code = []
    for path in paths:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
        code.append("\n".join(ln for ln in lines if ln.strip()))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def _traffic_from_profile(which):
    """Memory bytes per launch (L2 fetches + writes, scaled by a plain copy's
    counts) from the committed counter summary, if it was taken on the current
    kernel code (comments aside); else None."""
    summary, srcs = which
    if not os.path.exists(summary):
        return None
    text = open(summary).read()
    m = re.search(r"kernel_code_sha256_16:\s*([0-9a-f]{16})", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != _code_sha(srcs):
        return None
    return float(t.group(1))


def _clock_now(table):
    """Current clock in MHz from the amdgpu driver's sysfs table `table`
    (pp_dpm_sclk: shader, pp_dpm_mclk: memory; the level marked '*'), or None
    where it cannot be read."""
    import glob
    for path in sorted(glob.glob(f"/sys/class/drm/card*/device/{table}")):
        try:
            for line in open(path).read().splitlines():
                if line.rstrip().endswith("*"):
                    mhz = re.search(r"(\d+)\s*[Mm]hz", line)
                    if mhz:
                        return int(mhz.group(1))
        except OSError:
            continue
    return None


class _ClockSampler:
    """Samples the shader and memory clocks every ~2 ms in a thread while a
    timed region runs."""

    def __init__(self):
        import threading
        self.samples = {"pp_dpm_sclk": [], "pp_dpm_mclk": []}
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            got = False
            for table, vals in self.samples.items():
                v = _clock_now(table)
                if v is not None:
                    vals.append(v)
                    got = True
            if not got:
                return
            self._stop.wait(0.002)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self, table="pp_dpm_sclk"):
        v = sorted(self.samples[table])
        if not v:
            return None
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1],
                "samples": len(v), "source": f"sysfs {table} during the timed repeats"}


def main():
    args = _args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for "
              f"--gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import w8a8_int8_quantized_qk_amd as qk
    from w8a8_int8_quantized_qk_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qk.library()
    stream = torch.cuda.Stream(dev)  # default priority (capture needs a non-default stream)

    def timed_replays(step_fns, k_steps, warmup, repeats=None, stats=None):
        """Capture one HIP graph per buffer set (one step each) plus one graph of
        a whole ring, then run `repeats` timed blocks of exactly k_steps steps by
        replay, each timed with HIP events on the replay stream.  Returns (median
        ms per step, wall seconds of the median block); `stats`, when given,
        receives every block's ms per step and their min / median / max."""
        repeats = args.repeats if repeats is None else repeats
        R = len(step_fns)
        with torch.cuda.stream(stream):
            for f in step_fns:  # eager warm-up: first-use setup stays out of capture
                f()
        torch.cuda.synchronize()
        singles = []
        for f in step_fns:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                f()
            singles.append(g)
        ring = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ring, stream=stream):
            for f in step_fns:
                f()
        torch.cuda.synchronize()

        def run(n):
            with torch.cuda.stream(stream):
                for _ in range(n // R):
                    ring.replay()
                for i in range(n % R):
                    singles[i].replay()

        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < args.settle_seconds:
            run(8 * R)
            torch.cuda.synchronize()
        run(warmup)
        torch.cuda.synchronize()
        blocks = []
        for _ in range(max(1, repeats)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record(stream)
            run(k_steps)
            e1.record(stream)
            torch.cuda.synchronize()
            blocks.append((e0.elapsed_time(e1) / k_steps, time.perf_counter() - t0))
        order = sorted(blocks)
        ms, wall = order[len(order) // 2]
        if stats is not None:
            stats.update({"repeats": len(blocks), "steps_each": k_steps,
                          "ms_per_step_each": [round(b[0], 6) for b in blocks],
                          "min_ms": round(order[0][0], 6), "median_ms": round(ms, 6),
                          "max_ms": round(order[-1][0], 6)})
        return ms, wall

    # ---------------- prefill: quant + GEMM (headline) ----------------
    wcfg = wl.WORKLOADS["prefill_outliers"]
    m, k, n = wcfg.m, wcfg.k, wcfg.n
    sets = []
    for r in range(args.ring):
        d = wl.generate(wcfg, seed=r)
        sets.append({
            "x": d["x"].to(dev), "w": torch.from_numpy(d["w"]).to(dev),
            "s_ch": torch.from_numpy(d["s_ch"]).to(dev),
            "q": torch.empty((m, k), dtype=torch.int8, device=dev),
            "s": torch.empty((m,), dtype=torch.float32, device=dev),
            "out": torch.empty((m, n), dtype=torch.bfloat16, device=dev),
        })

    def step_fn(bs):
        def f():
            qk.quant_per_token(bs["x"], bs["q"], bs["s"])
            qk.gemm_i8_scaled(bs["q"], bs["w"], bs["s"], bs["s_ch"], out=bs["out"])
        return f

    def gemm_fn(bs):
        return lambda: qk.gemm_i8_scaled(bs["q"], bs["w"], bs["s"], bs["s_ch"], out=bs["out"])

    def quant_fn(bs):
        return lambda: qk.quant_per_token(bs["x"], bs["q"], bs["s"])

    step_stats, gemm_stats, quant_stats = {}, {}, {}
    with _ClockSampler() as sclk:
        ms_per_step, wall = timed_replays([step_fn(b) for b in sets], args.steps, args.warmup,
                                          stats=step_stats)
    gemm_ms, _ = timed_replays([gemm_fn(b) for b in sets], args.steps, args.warmup, stats=gemm_stats)
    quant_ms, _ = timed_replays([quant_fn(b) for b in sets], args.steps, args.warmup,
                                stats=quant_stats)
    ops = 2.0 * m * n * k
    tops = ops / (ms_per_step * 1e-3) / 1e12
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    traffic = _traffic_from_profile(GEMM_TRAFFIC)

    result = {
        "metric": "INT8 TOPS (quant+GEMM) at M=2048,K=N=4096; HBM GB/s at decode M=1",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "prefill_outliers", "m": m, "k": k, "n": n, "x_dtype": "bf16",
                   "w_layout": "[K,N]", "out_dtype": "bf16", "outlier_cols": wcfg.outlier_cols,
                   "ring_sets": args.ring,
                   "step": "qk_quant_per_token + qk_gemm_i8_scaled, replayed from HIP graphs"},
        "roofline": {"bound": "mfma", "kernel": GEMM_KERNEL,
                     "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": traffic,
                     "traffic_source": ("rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of this kernel "
                                        "code, copy-kernel scaled, from "
                                        "profiles/" + os.path.basename(GEMM_TRAFFIC[0])
                                        if traffic is not None else
                                        "none: no counter summary taken on this kernel code"),
                     "avg_launch_us": round(gemm_ms * 1e3, 3),
                     "algorithmic_ops_per_launch": ops},
        "step_frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
        "timing": {"step": step_stats, "gemm": gemm_stats, "quant": quant_stats,
                   "rule": "each block times exactly --steps replayed steps with HIP events; "
                           "value and ms_per_step are the median block"},
        "sclk": sclk.summary("pp_dpm_sclk"),
        "mclk": sclk.summary("pp_dpm_mclk"),
        "quant_kernel_us": round(quant_ms * 1e3, 3),
        "wall_s_timed_region": round(wall, 4),
        "settle_s_before_warmup": args.settle_seconds,
    }

    # ---------------- decode: M = 1 linear (second metric) ----------------
    if not args.no_decode:
        dcfg = wl.WORKLOADS["decode_m1"]
        dm, dk, dn = dcfg.m, dcfg.k, dcfg.n
        ws = qk.new_workspace(qk.gemm_workspace_size(dm, dn, dk), dev)
        dsets = []
        for r in range(args.ring):
            d = wl.generate(dcfg, seed=r)
            dsets.append({
                "x": d["x"].to(dev), "w": torch.from_numpy(d["w"]).to(dev),
                "s_ch": torch.from_numpy(d["s_ch"]).to(dev),
                "out": torch.empty((dm, dn), dtype=torch.bfloat16, device=dev),
            })

        def dstep_fn(bs):
            return lambda: qk.linear_w8a8(bs["x"], bs["w"], bs["s_ch"], out=bs["out"], workspace=ws)

        dstats = {}
        dms, _ = timed_replays([dstep_fn(b) for b in dsets], args.decode_calls, args.warmup,
                               stats=dstats)
        dbytes = dk * dn + 4 * dn + 2 * dm * dk + 2 * dm * dn
        gbs = dbytes / (dms * 1e-3) / 1e9
        result["decode"] = {
            "metric": "HBM GB/s at decode M=1 (quantization + GEMV in one launch)",
            "workload": "decode_m1", "m": dm, "k": dk, "n": dn,
            "value": round(gbs, 1), "unit": "GB/s",
            "us_per_call": round(dms * 1e3, 3), "algorithmic_bytes_per_call": dbytes,
            "timing": dstats,
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "kernel": "gemv_kernel (fused quantization)",
                         "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "avg_launch_us": round(dms * 1e3, 3),
                         "algorithmic_bytes_per_launch": dbytes,
                         "traffic": _traffic_from_profile(GEMV_TRAFFIC)},
        }

    # ---------------- the FP8 layer at the prefill shape ----------------
    # per-token e4m3fn quantization + FP8 GEMM (binary32 accumulation): the
    # same activations, e4m3fn weights
    if not args.no_fp8:
        fsets = []
        for r in range(args.ring):
            d = wl.generate(wcfg, seed=r, weight="fp8")
            fsets.append({"x": d["x"].to(dev), "w": torch.from_numpy(d["w"]).to(dev).view(torch.float8_e4m3fn),
                          "s_ch": torch.from_numpy(d["s_ch"]).to(dev),
                          "q": torch.empty((m, k), dtype=torch.float8_e4m3fn, device=dev),
                          "s": torch.empty((m,), dtype=torch.float32, device=dev),
                          "out": torch.empty((m, n), dtype=torch.bfloat16, device=dev)})

        def fquant(bs):
            qk.quant_per_token_fp8(bs["x"], 0.0, bs["q"], bs["s"])

        def fgemm(bs):
            qk.gemm_fp8_scaled(bs["q"], bs["w"], bs["s"], bs["s_ch"], out=bs["out"])

        fstep_ms, _ = timed_replays([(lambda bs=b: (fquant(bs), fgemm(bs))) for b in fsets], args.steps, args.warmup)
        fgemm_ms, _ = timed_replays([(lambda bs=b: fgemm(bs)) for b in fsets], args.steps, args.warmup)
        fquant_ms, _ = timed_replays([(lambda bs=b: fquant(bs)) for b in fsets], args.steps, args.warmup)
        fops = 2.0 * m * n * k
        ftf = fops / (fgemm_ms * 1e-3) / 1e12
        result["fp8_prefill"] = {
            "metric": "FP8 TFLOP/s (quant+GEMM) at M=2048,K=N=4096",
            "workload": "prefill_outliers with e4m3fn weights", "m": m, "k": k, "n": n,
            "x_dtype": "bf16", "w": "e4m3fn [K,N]", "out_dtype": "bf16",
            "value": round(fops / (fstep_ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(fstep_ms, 5),
            "step": "qk_quant_per_token_fp8 + qk_gemm_fp8_scaled, replayed from HIP graphs",
            "quant_kernel_us": round(fquant_ms * 1e3, 3),
            "roofline": {"bound": "mfma", "kernel": "gemm_slice_kernel (FP8)",
                         "achieved": round(ftf, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ftf / FP8_PEAK_TFLOPS, 4),
                         "traffic": _traffic_from_profile(FP8_TRAFFIC),
                         "avg_launch_us": round(fgemm_ms * 1e3, 3),
                         "algorithmic_flops_per_launch": fops},
        }
        del fsets
        torch.cuda.empty_cache()

    # ---------------- INT8 with per-group weight scales at the prefill shape ----------------
    # per-token INT8 quantization + the GEMM whose weight carries one scale per
    # group of 128 (and 64) consecutive k of each column
    if not args.no_grouped:
        gsets = []
        for r in range(args.ring):
            d = wl.generate(wcfg, seed=r)
            grng = np.random.default_rng(1000 + r)
            gsets.append({"x": d["x"].to(dev), "w": torch.from_numpy(d["w"]).to(dev),
                          "sg128": torch.from_numpy(wl.random_group_scales(grng, k // 128, n)).to(dev),
                          "sg64": torch.from_numpy(wl.random_group_scales(grng, k // 64, n)).to(dev),
                          "q": torch.empty((m, k), dtype=torch.int8, device=dev),
                          "s": torch.empty((m,), dtype=torch.float32, device=dev),
                          "out": torch.empty((m, n), dtype=torch.bfloat16, device=dev)})
        grouped = {}
        for group in (128, 64):
            def ggemm(bs, group=group):
                qk.gemm_i8_grouped(bs["q"], bs["w"], bs["s"], bs[f"sg{group}"], group, out=bs["out"])

            def gstep(bs, group=group):
                qk.quant_per_token(bs["x"], bs["q"], bs["s"])
                ggemm(bs, group)

            gstep_ms, _ = timed_replays([(lambda bs=b: gstep(bs)) for b in gsets], args.steps, args.warmup)
            ggemm_ms, _ = timed_replays([(lambda bs=b: ggemm(bs)) for b in gsets], args.steps, args.warmup)
            gops = 2.0 * m * n * k
            gt = gops / (ggemm_ms * 1e-3) / 1e12
            grouped[f"group_{group}"] = {
                "value": round(gops / (gstep_ms * 1e-3) / 1e12, 2), "unit": "TOPS",
                "ms_per_step": round(gstep_ms, 5),
                "roofline": {"bound": "mfma", "kernel": f"gemm_slice_kernel (INT8, groups of {group})",
                             "achieved": round(gt, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                             "frac": round(gt / INT8_PEAK_TOPS, 4),
                             "traffic": _traffic_from_profile(GROUPED_TRAFFIC) if group == 128 else None,
                             "avg_launch_us": round(ggemm_ms * 1e3, 3),
                             "algorithmic_ops_per_launch": gops,
                             "valu_wave_instructions_per_launch": 2 * m * n * (k // group) // 64}}
        result["grouped_prefill"] = {
            "metric": "INT8 TOPS (quant+GEMM) with per-group weight scales at M=2048,K=N=4096",
            "workload": "prefill_outliers with group scales [K/G, N]", "m": m, "k": k, "n": n,
            "step": "qk_quant_per_token + qk_gemm_i8_grouped, replayed from HIP graphs", **grouped}
        del gsets
        torch.cuda.empty_cache()

    # ---------------- static and asymmetric variants at the prefill shape ----------------
    if not args.no_static_asym:
        vsets = []
        for r in range(args.ring):
            d = wl.generate(wcfg, seed=r)
            w_dev = torch.from_numpy(d["w"]).to(dev)
            amax = float(d["x"].float().abs().max())
            vsets.append({"x": d["x"].to(dev), "w": w_dev, "s_ch": torch.from_numpy(d["s_ch"]).to(dev),
                          "wsum": qk.weight_colsum(w_dev),
                          "s_static": torch.tensor([amax / 127.0], dtype=torch.float32, device=dev),
                          "q": torch.empty((m, k), dtype=torch.int8, device=dev),
                          "out": torch.empty((m, n), dtype=torch.bfloat16, device=dev)})
        torch.cuda.synchronize()

        def vstatic(bs):
            qk.quant_static(bs["x"], bs["s_static"], q=bs["q"])

        def vasym_q(bs):
            bs["qa"] = qk.quant_per_token_asym(bs["x"])

        for bs in vsets:
            vasym_q(bs)

        def vasym_gemm(bs):
            q, s, z = bs["qa"]
            qk.library().qk_gemm_i8_asym(m, n, k, qk._ptr(q), qk._ptr(z), qk._ptr(bs["w"]),
                                         qk._ptr(bs["wsum"]), None, qk._ptr(s), qk._ptr(bs["s_ch"]),
                                         1.0, qk._ptr(bs["out"]), qk.BF16, qk.B_KN,
                                         qk._stream(dev))

        st_ms, _ = timed_replays([(lambda bs=b: vstatic(bs)) for b in vsets], args.steps, args.warmup)
        aq_ms, _ = timed_replays([(lambda bs=b: qk.library().qk_quant_per_token_asym(
            m, k, qk._ptr(bs["x"]), qk.BF16, qk._ptr(bs["qa"][0]), qk._ptr(bs["qa"][1]),
            qk._ptr(bs["qa"][2]), qk._stream(dev))) for b in vsets], args.steps, args.warmup)
        ag_ms, _ = timed_replays([(lambda bs=b: vasym_gemm(bs)) for b in vsets], args.steps, args.warmup)
        qbytes = m * k * 2 + m * k
        aops = 2.0 * m * n * k
        agt = aops / (ag_ms * 1e-3) / 1e12
        result["static_asym_prefill"] = {
            "workload": "prefill_outliers", "m": m, "k": k, "n": n,
            "static_quant": {"us": round(st_ms * 1e3, 3), "unit": "GB/s",
                             "value": round(qbytes / (st_ms * 1e-3) / 1e9, 1),
                             "roofline": {"bound": "hbm", "achieved": round(qbytes / (st_ms * 1e-3) / 1e9, 1),
                                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                          "frac": round(qbytes / (st_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                          "traffic": _traffic_from_profile(STATIC_TRAFFIC),
                                          "algorithmic_bytes_per_launch": qbytes}},
            "asym_quant": {"us": round(aq_ms * 1e3, 3), "unit": "GB/s",
                           "value": round((qbytes + 8 * m) / (aq_ms * 1e-3) / 1e9, 1)},
            "asym_gemm": {"us": round(ag_ms * 1e3, 3), "unit": "TOPS", "value": round(agt, 2),
                          "roofline": {"bound": "mfma", "kernel": ASYM_KERNEL,
                                       "achieved": round(agt, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                                       "frac": round(agt / INT8_PEAK_TOPS, 4),
                                       "traffic": _traffic_from_profile(ASYM_TRAFFIC),
                                       "avg_launch_us": round(ag_ms * 1e3, 3),
                                       "algorithmic_ops_per_launch": aops}},
        }
        del vsets
        torch.cuda.empty_cache()

    # ---------------- MoE grouped GEMM: all experts in one launch ----------------
    if not args.no_moe:
        msets = []
        for r in range(2):  # the weights (470 MB per set) exceed the Infinity Cache already
            d = wl.generate_moe(seed=r)
            msets.append({"x": d["x"].to(dev), "w": torch.from_numpy(d["w"]).to(dev),
                          "s_ch": torch.from_numpy(d["s_ch"]).to(dev),
                          "off": torch.from_numpy(d["offsets"]).to(dev), "off_host": d["offsets"],
                          "q": torch.empty((d["rows"], d["k"]), dtype=torch.int8, device=dev),
                          "s": torch.empty((d["rows"],), dtype=torch.float32, device=dev),
                          "out": torch.empty((d["rows"], d["n"]), dtype=torch.bfloat16, device=dev)})
        mrows, mk, mn, mexp = d["rows"], d["k"], d["n"], d["experts"]
        del d

        def mgemm(bs):
            qk.moe_gemm_i8_scaled(bs["q"], bs["w"], bs["off"], bs["s"], bs["s_ch"], out=bs["out"])

        def mstep(bs):
            qk.quant_per_token(bs["x"], bs["q"], bs["s"])
            mgemm(bs)

        def per_expert(bs):  # the same work as one GEMM launch per expert
            o = bs["off_host"]
            for e in range(mexp):
                r0, r1 = int(o[e]), int(o[e + 1])
                if r1 > r0:
                    qk.gemm_i8_scaled(bs["q"][r0:r1], bs["w"][e], bs["s"][r0:r1], bs["s_ch"][e],
                                      out=bs["out"][r0:r1], kernel="mfma")

        msteps = max(4, args.steps // 10)
        mstep_ms, _ = timed_replays([(lambda bs=b: mstep(bs)) for b in msets], msteps, 2)
        mgemm_ms, _ = timed_replays([(lambda bs=b: mgemm(bs)) for b in msets], msteps, 2)
        mper_ms = None
        if args.moe_per_expert:  # launches the plain GEMM at the experts' shapes
            mper_ms, _ = timed_replays([(lambda bs=b: per_expert(bs)) for b in msets], msteps, 2)
        mops = 2.0 * mrows * mn * mk
        mt = mops / (mgemm_ms * 1e-3) / 1e12
        result["moe_up"] = {
            "metric": "INT8 TOPS (quant+MoE GEMM), 8 experts, 2048 tokens x top-2, 4096 -> 14336",
            "experts": mexp, "rows": mrows, "k": mk, "n": mn,
            "rows_per_expert": [int(x) for x in np.diff(msets[0]["off_host"])],
            "value": round(mops / (mstep_ms * 1e-3) / 1e12, 2), "unit": "TOPS",
            "ms_per_step": round(mstep_ms, 5),
            "step": "qk_quant_per_token + qk_moe_gemm_i8_scaled (one launch for all experts)",
            "one_launch_per_expert_us": round(mper_ms * 1e3, 2) if mper_ms is not None else None,
            "roofline": {"bound": "mfma", "kernel": MOE_KERNEL,
                         "achieved": round(mt, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                         "frac": round(mt / INT8_PEAK_TOPS, 4), "traffic": _traffic_from_profile(MOE_TRAFFIC),
                         "avg_launch_us": round(mgemm_ms * 1e3, 3),
                         "algorithmic_ops_per_launch": mops},
        }
        del msets
        torch.cuda.empty_cache()

    # ---------------- the other workload shapes (reported, not the metric) ----------------
    if not args.no_other_configs:
        others = {}
        # 8-row decode: the fused linear, HBM-bound like the 1-row one
        ocfg = wl.WORKLOADS["decode_m8"]
        om, ok, on = ocfg.m, ocfg.k, ocfg.n
        ows = qk.new_workspace(qk.gemm_workspace_size(om, on, ok), dev)
        osets = []
        for r in range(args.ring):
            d = wl.generate(ocfg, seed=r)
            osets.append({"x": d["x"].to(dev), "w": torch.from_numpy(d["w"]).to(dev),
                          "s_ch": torch.from_numpy(d["s_ch"]).to(dev),
                          "out": torch.empty((om, on), dtype=torch.bfloat16, device=dev)})
        oms, _ = timed_replays([(lambda bs=b: qk.linear_w8a8(bs["x"], bs["w"], bs["s_ch"], out=bs["out"],
                                                             workspace=ows)) for b in osets],
                               200, args.warmup)
        obytes = ok * on + 4 * on + 2 * om * ok + 2 * om * on
        ogbs = obytes / (oms * 1e-3) / 1e9
        others["decode_m8"] = {"m": om, "k": ok, "n": on, "us_per_call": round(oms * 1e3, 3),
                               "value": round(ogbs, 1), "unit": "GB/s",
                               "frac_of_hbm_peak": round(ogbs / HBM_PEAK_GBS, 4),
                               "roofline": {"bound": "hbm", "kernel": "gemv_mfma_kernel (fused quantization)",
                                            "achieved": round(ogbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                            "frac": round(ogbs / HBM_PEAK_GBS, 4),
                                            "algorithmic_bytes_per_launch": obytes,
                                            "traffic": _traffic_from_profile(GEMV_M8_TRAFFIC)}}
        del osets, ows
        torch.cuda.empty_cache()

        # one GPU's share under 8-way column (tensor) parallelism: the 1-row
        # decode and the prefill with N / 8 output columns (weights from a ring
        # larger than the Infinity Cache: 48 x 7.3 MB and 8 x 2.1 MB + inputs)
        gen = torch.Generator(device=dev)
        gen.manual_seed(0)
        shard = {}
        for sname, (sm, sk, sn, nsets, ssteps) in (("decode_m1_n1792", (1, 4096, 1792, 48, 480)),
                                                     ("prefill_n512", (2048, 4096, 512, 8, 80))):
            ssets = []
            for r in range(nsets):
                if sm == 1:
                    x = torch.randn((sm, sk), generator=gen, device=dev).to(torch.bfloat16)
                else:  # the prefill activations, outlier columns included
                    x = wl.generate(wcfg, seed=r)["x"].to(dev)
                ssets.append({"x": x,
                              "w": torch.randint(-127, 128, (sk, sn), generator=gen, device=dev,
                                                 dtype=torch.int8),
                              "s_ch": torch.empty(sn, device=dev).uniform_(1e-3, 1e-2, generator=gen),
                              "out": torch.empty((sm, sn), dtype=torch.bfloat16, device=dev)})
            sws = qk.new_workspace(qk.gemm_workspace_size(sm, sn, sk), dev)
            sms, _ = timed_replays([(lambda bs=b: qk.linear_w8a8(bs["x"], bs["w"], bs["s_ch"],
                                                                 out=bs["out"], workspace=sws))
                                    for b in ssets], ssteps, args.warmup)
            if sm == 1:
                sbytes = sk * sn + 4 * sn + 2 * sk + 2 * sn
                shard[sname] = {"m": sm, "k": sk, "n": sn, "us_per_call": round(sms * 1e3, 3),
                                "value": round(sbytes / (sms * 1e-3) / 1e9, 1), "unit": "GB/s",
                                "frac_of_hbm_peak": round(sbytes / (sms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            else:
                sops = 2.0 * sm * sn * sk
                shard[sname] = {"m": sm, "k": sk, "n": sn, "us_per_step": round(sms * 1e3, 3),
                                "value": round(sops / (sms * 1e-3) / 1e12, 1), "unit": "TOPS",
                                "step": "quantization + GEMM (qk_linear_w8a8)"}
            del ssets, sws
            torch.cuda.empty_cache()
        others["tp8_column_shard"] = shard

        # gated down-projection and MLP up-projection: quantization + GEMM, and
        # the GEMM alone; two buffer sets each (both exceed the 256 MB Infinity
        # Cache already)
        for name, steps in (("gated_down", 20), ("mlp_up", 8)):
            gcfg = wl.WORKLOADS[name]
            gm, gk, gn = gcfg.m, gcfg.k, gcfg.n
            odt = torch.float32 if gcfg.out_dtype == "f32" else torch.bfloat16
            gsets = []
            for r in range(2):
                d = wl.generate(gcfg, seed=r)
                bs = {"w": torch.from_numpy(d["w"]).to(dev), "s_ch": torch.from_numpy(d["s_ch"]).to(dev),
                      "q": torch.empty((gm, gk), dtype=torch.int8, device=dev),
                      "s": torch.empty((gm,), dtype=torch.float32, device=dev),
                      "out": torch.empty((gm, gn), dtype=odt, device=dev)}
                bs["in"] = (d["h"] if gcfg.gated else d["x"]).to(dev)
                gsets.append(bs)
                del d

            def quant(bs, gated=gcfg.gated):
                if gated:
                    qk.silu_mul_quant_per_token(bs["in"], bs["q"], bs["s"])
                else:
                    qk.quant_per_token(bs["in"], bs["q"], bs["s"])

            def gemm(bs):
                qk.gemm_i8_scaled(bs["q"], bs["w"], bs["s"], bs["s_ch"], out=bs["out"])

            step_ms, _ = timed_replays([(lambda bs=b: (quant(bs), gemm(bs))) for b in gsets], steps, 2)
            gemm_only_ms, _ = timed_replays([(lambda bs=b: gemm(bs)) for b in gsets], steps, 2)
            ops = 2 * gm * gn * gk
            others[name] = {"m": gm, "k": gk, "n": gn, "out_dtype": gcfg.out_dtype,
                            "quantization": "silu(gate)*up fused" if gcfg.gated else "per-token",
                            "us_per_step": round(step_ms * 1e3, 2),
                            "step_tops": round(ops / (step_ms * 1e-3) / 1e12, 1),
                            "gemm_us": round(gemm_only_ms * 1e3, 2),
                            "gemm_tops": round(ops / (gemm_only_ms * 1e-3) / 1e12, 1),
                            "gemm_frac_of_int8_peak": round(ops / (gemm_only_ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)}
            del gsets
            torch.cuda.empty_cache()
        result["other_configs"] = others

    if args.copy_calibration:
        nbytes = 256 << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        result["copy_calibration_bytes_each_way"] = nbytes

    # ---------------- CPU oracle baseline (reported, not the target) ----------------
    if not args.no_cpu_baseline:
        cores = len(os.sched_getaffinity(0))
        os.environ.setdefault("OMP_NUM_THREADS", str(cores))
        import oracle

        d0 = wl.generate(wcfg, seed=0)
        xb = wl.bits(d0["x"])

        def run_rows(rows):
            t = time.perf_counter()
            oracle.linear(xb[:rows], oracle.BF16, d0["w"], d0["s_ch"])
            return time.perf_counter() - t

        # a sample of about --cpu-seconds of oracle work: the first `rows` rows,
        # or, when the whole workload takes less, whole passes over it
        probe_rows = 32
        tp = run_rows(probe_rows)
        rows = int(min(m, max(probe_rows, probe_rows * args.cpu_seconds / max(tp, 1e-3))))
        rows = max(16, rows // 16 * 16)
        tc = run_rows(rows)
        passes = 1
        if rows == m and tc < args.cpu_seconds:
            passes = int(min(30, max(1, round(args.cpu_seconds / max(tc, 1e-3)))))
            if passes > 1:
                tc = sum(run_rows(rows) for _ in range(passes))
        cpu_tops = 2.0 * rows * n * k * passes / tc / 1e12
        what = (f"rows 0..{rows - 1}" if passes == 1 else f"{passes} passes over all {rows} rows")
        result["cpu_baseline"] = {
            "value": round(cpu_tops, 5), "unit": "TOPS", "cores": int(os.environ["OMP_NUM_THREADS"]),
            "kind": "oracle",
            "sample": f"{what} of prefill_outliers ({rows}x{k}x{n}): widen, per-token "
                      f"quant, int8 GEMM, float64 dequant; {tc:.2f} s",
            "seconds": round(tc, 3), "gpu_speedup": round(tops / cpu_tops, 1),
        }

    props = torch.cuda.get_device_properties(dev)
    result["env"] = {"gpu": getattr(props, "gcnArchName", props.name), "cus": props.multi_processor_count,
                     "torch": torch.__version__, "hip": torch.version.hip,
                     "host_cpu": platform.processor() or platform.machine(),
                     "host_cores": len(os.sched_getaffinity(0)), "lib": qk.build_info()}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
