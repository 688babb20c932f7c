"""Benchmark: FNO spectral-conv throughput on one MI355X through libfno.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload train2d_512] [--no-cpu-baseline]

A step is one pass of the workload's whole hot path over one batch of synthetic input
already resident in HBM.  The default workload is the 2D FNO training step: 4 spectral
blocks of width 64 on a 512x512 grid, batch 8, modes 32x32 per corner, tanh pre-activation
and bf16 spectral operands with fp32 accumulation, forward + MSE + backward (input, weight,
bypass and bias gradients).  Throughput is grid points x channels x batch x blocks per second
(the forward and backward of a block count once).

Printed: one JSON line with the metric, the per-kernel breakdown measured with HIP events on
the stream libfno launches on, the roofline of the dominant kernel, and the fp64 oracle timed
on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F32_TFLOPS = 157.3        # dense fp32 matrix cores (= fp32 vector peak)
MFMA_HALF_TFLOPS = 2516.6      # dense bf16 / fp16 matrix cores
METRIC = "FNO spectral-conv fwd+bwd grid-pts·ch/s per MI355X; % HBM/MFMA roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="train2d_512")
    ap.add_argument("--spectral-precision", choices=["f32", "bf16", "f16"], default=None,
                    help="run the workload's plan at this spectral precision, tanh kept as the "
                         "workload has it (e.g. f32: a mixed run after a precision-schedule "
                         "switch)")
    ap.add_argument("--last-axis", choices=["auto", "fft", "dense"], default="auto",
                    help="float32 plans: forward transform of the contiguous axis by FFT or by "
                         "dense matrix-core products (auto: the plan's choice for its shape)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-batch", type=int, default=3)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    return ap.parse_args()


def copy_calibration(nbytes: int, reps: int = 3):
    """A plain device-to-device copy of a known size, used to scale the HBM byte counters."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"kind": "copy", "bytes_read": 4 * n, "bytes_written": 4 * n,
                      "launches": reps, "avg_ms": dt * 1e3,
                      "GBps_rw": 8 * n / dt / 1e9}), flush=True)


def _fft_flops(n: int) -> float:
    """Flops of one real FFT row of n points, the usual 2.5 n log2 n estimate."""
    return 2.5 * n * math.log2(n)


def _outer_lines(wl, j: int) -> int:
    """Lines of the truncated DFT along outer axis j: the transforms run innermost outer axis
    first, so axes before j are still whole and axes after j already truncated."""
    N, m, d = wl.grid, wl.modes, wl.ndim
    lines = wl.batch * wl.width * m[-1]
    for i in range(d - 1):
        if i < j:
            lines *= N[i]
        elif i > j:
            lines *= 2 * m[i]
    return lines


def _weight_bytes(wl) -> int:
    """Bytes of one block's spectral weight: the dense corners, or the Tucker core + factors."""
    C, m, d = wl.width, wl.modes, wl.ndim
    if wl.tucker_ranks:
        r = list(wl.tucker_ranks)
        ext = [C, C] + [2 * v for v in m[:-1]] + [m[-1]]
        core = 1
        for v in r:
            core *= v
        return 8 * (core + sum(e * v for e, v in zip(ext, r)))
    mp = 1
    for v in m:
        mp *= v
    return 8 * (1 << (d - 1)) * C * C * mp


def method_work(wl):
    """The method's compulsory HBM bytes and flops of one step of the workload.

    Bytes: per block, the input and output fields, W and Wb once (forward: 8 B per element +
    |W|); a training step adds the incoming gradient, the input again, grad_x, W again and dW
    (20 B per element + 3 |W|), and the loss target once; lift and projection read and write
    their fields.  Flops: a real FFT of the contiguous axis (2.5 N log2 N per row) and truncated
    DFTs along the outer axes (8 N 2m per line) in each direction, the per-mode mix (8 B C^2 K),
    in the spectral dtype; the 1x1 bypass (2 C^2 per point, 3x with the backward), lift and
    projection in float32."""
    B, C, P, nb = wl.batch, wl.width, wl.points, wl.blocks
    U = B * C * P
    N, m, d = wl.grid, wl.modes, wl.ndim
    K = m[-1]
    for j in range(d - 1):
        K *= 2 * m[j]
    per_dir = U / N[-1] * _fft_flops(N[-1]) + sum(
        8 * N[j] * 2 * m[j] * _outer_lines(wl, j) for j in range(d - 1))
    mix = 8 * B * C * C * K
    bypass = 2 * C * C * P * B
    wbytes = _weight_bytes(wl)
    wb_bytes = 4 * C * C + 4 * C
    if wl.train:
        nbytes = nb * (20 * U + 3 * wbytes + 3 * wb_bytes) + 4 * U
        spec = nb * (4 * per_dir + 3 * mix)
        pw = nb * 3 * bypass
    else:
        nbytes = nb * (8 * U + wbytes + wb_bytes)
        spec = nb * (2 * per_dir + mix)
        pw = nb * bypass
    if wl.lift_in:
        nbytes += 4 * B * P * (wl.lift_in + C) + 4 * B * P * (C + wl.proj_out)
        pw += 2 * B * P * (wl.lift_in * C + C * wl.proj_hidden + wl.proj_hidden * wl.proj_out)
    return {"bytes": nbytes, "flops_spectral": spec, "flops_pointwise": pw}


def step_roofline(wl, prec, ms_per_step):
    """Both floors of one step: HBM time of the compulsory bytes at 8 TB/s, and matrix-core
    time of the method's flops (spectral flops at the peak of the spectral dtype, pointwise
    flops at the float32 peak); t_roof is the larger, frac = t_roof / measured step time."""
    w = method_work(wl)
    t_hbm = w["bytes"] / (HBM_PEAK_GBS * 1e9)
    peak_spec = MFMA_F32_TFLOPS if prec == "f32" else MFMA_HALF_TFLOPS
    t_flop = w["flops_spectral"] / (peak_spec * 1e12) + w["flops_pointwise"] / (
        MFMA_F32_TFLOPS * 1e12)
    t_roof = max(t_hbm, t_flop)
    return {"alg_bytes": w["bytes"], "alg_flops_spectral": w["flops_spectral"],
            "alg_flops_pointwise": w["flops_pointwise"], "t_hbm_us": round(t_hbm * 1e6, 1),
            "t_flop_us": round(t_flop * 1e6, 1), "t_roof_us": round(t_roof * 1e6, 1),
            "bound": "hbm" if t_hbm >= t_flop else "mfma",
            "frac": round(t_roof / (ms_per_step * 1e-3), 4)}


def kernel_model(wl, prec):
    """Algorithmic bytes and flops per launch of each libfno kernel for this workload:
    name -> (bytes, spectral flops, pointwise flops, pointwise on the bf16 matrix cores).

    Bytes: every input and output buffer of the kernel once (fields, spectra, weights).
    Flops: the method's, as in method_work (FFT count for the contiguous axis, dense truncated
    DFTs along outer axes, the mix, the bypass).  On half plans with a multiple of 32 channels
    the line epilogues run the bypass products as three bf16 products of split operands."""
    B, C = wl.batch, wl.width
    P = wl.points
    d = wl.ndim
    U = B * C * P
    N = list(wl.grid)
    m = list(wl.modes)
    Na, Nb, ma, mb = N[-2], N[-1], m[-2], m[-1]
    K = mb
    for j in range(d - 1):
        K *= 2 * m[j]
    ncorner = 1 << (d - 1)
    half = prec != "f32"
    spec = B * C * K * 8
    wbytes = _weight_bytes(wl) if not wl.tucker_ranks else 0
    mprod = 1
    for v in m:
        mprod *= v
    wdense = 8 * ncorner * C * C * mprod
    lines = P // Nb
    # the spectrum after the outer inverses: complex float32, or the half format on half plans
    # of width 64 (the width-64 line epilogues take it so)
    T = B * C * lines * mb * (4 if (half and C == 64) else 8)
    O = P // (Na * Nb)
    plane_spec = B * C * O * 2 * ma * mb * 8
    fft_last = U / Nb * _fft_flops(Nb)            # real row <-> retained bins, per direction
    dft_a = 8 * Na * 2 * ma * _outer_lines(wl, d - 2)
    bypass = 2 * C * C * P * B
    mixf = 8 * B * C * C * K
    split = half and C % 32 == 0
    model = {
        "plane_fwd": (4 * U + plane_spec, fft_last + dft_a, 0, False),
        "plane_fwd_tanh": (4 * U + plane_spec, fft_last + dft_a, 0, False),
        "plane_fwd_gelu": (4 * U + plane_spec, fft_last + dft_a, 0, False),
        "plane_fwd_tanh_gelu": (4 * U + plane_spec, fft_last + dft_a, 0, False),
        "plane_fwd_gelugrad": (8 * U + plane_spec, fft_last + dft_a, 0, False),
        "mix_fwd": (max(wbytes, wdense) + 2 * spec, mixf, 0, False),
        "mix_bwd_dx": (max(wbytes, wdense) + 2 * spec, mixf, 0, False),
        "mix_bwd_dw": (max(wbytes, wdense) + 2 * spec, mixf, 0, False),
        # both gradients in one launch: W in, dW out, the spectra (g, x in, g_x out)
        "mix_bwd": (2 * max(wbytes, wdense) + 3 * spec, 2 * mixf, 0, False),
        # x in, y out (+ z saved for the backward)
        "epilogue_fwd": (8 * U + T, fft_last, bypass, split),
        "epilogue_fwd_zsave": (12 * U + T, fft_last, bypass, split),
        # short rows: the epilogue also inverts axis a, from the [2ma][mb] spectrum per plane
        "epilogue_rows_fwd": (8 * U + plane_spec, fft_last + dft_a, bypass, False),
        "epilogue_rows_fwd_zsave": (12 * U + plane_spec, fft_last + dft_a, bypass, False),
        # g and x in, grad_x out (+ z in for GELU' when the block applies the output GELU)
        "epilogue_bwd": (12 * U + T, fft_last, 2 * bypass, split),
        "epilogue_bwd_gelu": (16 * U + T, fft_last, 2 * bypass, split),
        "mse": (12 * U, 0, 3 * U, False),
        # the last block's forward fused with the loss: x and the target in, grad_z out
        "epilogue_fwd_mse": (12 * U + T, fft_last, bypass, split),
        # the same where the line epilogue does not apply: z and the target in, grad_z out
        "mse_preact": (12 * U, 0, 3 * U, False),
    }
    return model


def kernel_floor(model_row, prec):
    """(t_hbm, t_flop) of one launch: bytes at 8 TB/s; spectral flops at the spectral dtype's
    matrix-core peak; pointwise flops at the float32 peak, or as three bf16 products each at the
    bf16 peak where the kernel splits its operands."""
    b, fs, fp, split = model_row
    peak_spec = MFMA_F32_TFLOPS if prec == "f32" else MFMA_HALF_TFLOPS
    peak_pw = MFMA_HALF_TFLOPS / 3 if split else MFMA_F32_TFLOPS
    return b / (HBM_PEAK_GBS * 1e9), fs / (peak_spec * 1e12) + fp / (peak_pw * 1e12)


def dominant_kernel(wl, kern):
    """The kernel with the most time among those the byte model covers (kern: timer report);
    without a report, the one with the most algorithmic bytes per step."""
    model = kernel_model(wl, configs_precision(wl))
    if kern:
        cands = [n for n in kern if model.get(n, (None,))[0]]
        if cands:
            return max(cands, key=lambda n: kern[n][1])
    return max(model, key=lambda n: model[n][0])


def bench_gpu(wl, steps, warmup, precision=None, last_axis=None):
    """Warm-up (every launch timed: names the dominant kernel), the timed region (events only
    around the dominant kernel's launches, so the other launches run as in production), then
    `steps` more untimed steps with every launch timed for the per-kernel breakdown."""
    import torch

    from fno_spectral_convolution_amd import binding as L
    from fno_spectral_convolution_amd.stack import StackRunner

    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    runner = StackRunner(wl, device="cuda:0", last_axis=last_axis)
    if precision is not None:
        runner.set_precision(precision)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    print(f"[bench] {wl.name}: inputs on device in {setup_s:.1f}s; warmup {warmup}", flush=True)
    # the first warm-up step pays one-time costs (first launches), so the dominant kernel is
    # named from the later warm-up steps (from the byte model when there are none)
    L.fno_timing_reset()
    L.fno_timing_select(None)
    for i in range(warmup):
        # the first step also pays one-time costs: it names the kernel only when it is the
        # only warm-up step
        L.fno_timing_enable(i > 0 or warmup == 1)
        runner.step()
    torch.cuda.synchronize()
    L.fno_timing_enable(False)
    # without warm-up steps every launch of the timed region is timed and the dominant kernel
    # is named from it
    dom = dominant_kernel(wl, L.timing_report()) if warmup > 0 else None
    L.fno_timing_reset()
    L.fno_timing_select(dom)
    L.fno_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        runner.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    L.fno_timing_enable(False)
    kern_dom = L.timing_report()
    if dom is None:
        dom = dominant_kernel(wl, kern_dom)
    print(f"[bench] timed {steps} steps in {wall:.3f}s (events around {dom})", flush=True)
    L.fno_timing_reset()
    L.fno_timing_select(None)
    L.fno_timing_enable(True)
    for _ in range(steps):
        runner.step()
    torch.cuda.synchronize()
    L.fno_timing_enable(False)
    kern_all = L.timing_report()
    L.fno_timing_reset()
    return runner, wall, dom, kern_dom, kern_all


def configs_precision(wl):
    from fno_spectral_convolution_amd import configs
    return configs.precision(wl)


def roofline(wl, prec, dom, kern_dom, kern_all):
    """Roofline of the dominant kernel from its events in the timed region (bound: the larger of
    its HBM and matrix-core floors); the per-kernel rows from the breakdown steps."""
    model = kernel_model(wl, prec)

    def row(name, launches, total_ms, share):
        avg_s = total_ms / 1e3 / max(launches, 1)
        mr = model.get(name)
        b = mr[0] if mr else None
        return {"launches": launches, "avg_us": avg_s * 1e6, "share": share, "alg_bytes": b,
                "GBps": (b / avg_s / 1e9) if b else None}

    tot = max(sum(v[1] for v in kern_all.values()), 1e-12)
    rows = {n: row(n, c, ms, ms / tot) for n, (c, ms) in kern_all.items()}
    launches, total_ms = kern_dom[dom]
    r = row(dom, launches, total_ms, None)
    avg_s = r["avg_us"] / 1e6
    b, fs, fp, _ = model[dom]
    t_hbm, t_flop = kernel_floor(model[dom], prec)
    traffic = measured_traffic(wl, dom)
    out = {"kernel": dom}
    if t_hbm >= t_flop:
        ach = b / avg_s / 1e9
        out.update({"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4)})
    else:
        ach = (fs + fp) / avg_s / 1e12
        peak = (fs + fp) / t_flop / 1e12  # the kernel's own dtype mix
        out.update({"bound": "mfma", "achieved": round(ach, 2), "peak": round(peak, 1),
                    "unit": "TFLOP/s", "frac": round(ach / peak, 4)})
    out.update({"traffic": traffic, "alg_bytes_per_launch": b,
                "alg_flops_per_launch": fs + fp, "t_hbm_us": round(t_hbm * 1e6, 1),
                "t_flop_us": round(t_flop * 1e6, 1), "avg_launch_us": round(r["avg_us"], 2),
                "timed_launches": launches})
    return out, rows


def measured_traffic(wl, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the counter's reading for a plain copy of known
    size), or None when there is none for this workload or the kernel's source (or a header it
    includes) has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"counters_{wl.name}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))["kernels"][kernel]
        h = hashlib.sha256()
        for f in rec["sources"]:  # the kernel's source file and the headers it includes
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except (KeyError, OSError, ValueError):
        return None
    if h.hexdigest() != rec["sources_sha256"]:
        return None
    return round(rec["fetch_bytes"] + rec["write_bytes"])


def cpu_baseline(wl, sample_batch, min_seconds=10.0, max_reps=12):
    """The fp64 oracle, as it stands, on a bounded sample: one block's forward + backward for
    `sample_batch` batch entries of the workload (full grid and width)."""
    import numpy as np

    import oracle.fno_oracle as O
    from fno_spectral_convolution_amd import inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    sb = min(sample_batch, wl.batch)
    g = np.random.default_rng(np.random.SeedSequence([wl.cfg_id, 99]))
    shape = (sb, wl.width) + tuple(wl.grid)
    x = g.standard_normal(shape).astype(np.float32)
    gy = g.standard_normal(shape).astype(np.float32) * 1e-3
    blk = inputs.block_params(wl, 1)[0]
    what = "fwd+bwd" if wl.train else "fwd"
    reps = 0
    t0 = time.perf_counter()
    # repeat the sample until about min_seconds of host work (bounded by max_reps)
    while True:
        tanh = bool(wl.mixed)
        if "core" in blk:  # Tucker-factorised weights
            if wl.train:
                O.tucker_block_bwd(x, blk["core"], blk["factors"], blk["wb"], blk["bias"],
                                   wl.modes, gy, tanh=tanh)
            else:
                O.tucker_block_fwd(x, blk["core"], blk["factors"], blk["wb"], blk["bias"],
                                   wl.modes, tanh=tanh)
        elif wl.train:
            O.block_bwd(x, blk["w"], blk["wb"], blk["bias"], wl.modes, gy, tanh=tanh)
        else:
            O.block_fwd(x, blk["w"], blk["wb"], blk["bias"], wl.modes, tanh=tanh)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    units = reps * sb * wl.width * wl.points
    return {"value": units / dt, "unit": "grid-pts·ch/s", "cores": threads, "kind": "oracle",
            "sample": f"one block {what} (fp64 numpy oracle), batch {sb} of {wl.batch}, "
                      f"width {wl.width}, grid {list(wl.grid)}, modes {list(wl.modes)}, "
                      f"repeated {reps}x: {dt:.2f} s",
            "seconds": round(dt, 3), "host_cpus": os.cpu_count()}


def main():
    args = parse()
    if args.copy_bytes:
        copy_calibration(args.copy_bytes)
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design only).", file=sys.stderr, flush=True)
        sys.exit(2)
    from fno_spectral_convolution_amd import configs
    wl = configs.get(args.workload)
    last_axis = None if args.last_axis == "auto" else args.last_axis
    runner, wall, dom, kern_dom, kern_all = bench_gpu(wl, args.steps, args.warmup,
                                                      args.spectral_precision, last_axis)
    dtype = runner.precision
    switched = dtype != configs.precision(wl)
    tucker_order = runner.tk.order if runner.tk is not None else None
    ms = wall / args.steps * 1e3
    value = wl.units / (wall / args.steps)
    roof, rows = roofline(wl, dtype, dom, kern_dom, kern_all)
    if switched:  # the committed counters were taken at the workload's own precision
        roof["traffic"] = None
    del runner
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", flush=True)
        cpu = cpu_baseline(wl, args.cpu_sample_batch)
    rec = {
        "metric": METRIC, "value": value, "unit": "grid-pts·ch/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {wl.notes}", "batch": wl.batch, "width": wl.width,
                   "grid": list(wl.grid), "modes": list(wl.modes), "blocks": wl.blocks,
                   "spectral_precision": (f"{dtype} operands, fp32 accumulate"
                                          if dtype != "f32" else "fp32")
                   + (f" (switched from {configs.precision(wl)}, tanh "
                      f"{'kept' if wl.mixed else 'off'})" if switched else ""),
                   "pointwise_precision": "fp32",
                   **({"spectral_weight": f"Tucker ranks {list(wl.tucker_ranks)}, contraction "
                                          f"order '{tucker_order}'"}
                      if wl.tucker_ranks else {})},
        "roofline": roof,
        "step_roofline": step_roofline(wl, dtype, ms),
        "cpu_baseline": cpu,
        "kernels": {k: {"launches": v["launches"], "avg_us": round(v["avg_us"], 2),
                        "share": round(v["share"], 4),
                        "GBps": round(v["GBps"], 1) if v["GBps"] else None}
                    for k, v in sorted(rows.items(), key=lambda kv: -kv[1]["share"])},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
