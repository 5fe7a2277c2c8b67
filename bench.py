"""Benchmark: full BigVGAN decode throughput on one MI355X.

Workload (default): the MiniMax-H3-shaped decoder at full size, latent
[2, 32, 400] (two mono passes of 10 s at 40 frames/s) -> waveform
[2, 320000] at 32 kHz, He-initialised synthetic weights, float32 throughout.
``--workload 5`` runs the LTX-2.5-shaped vocoder ([2, 64, 2000] log-mel ->
[2, 320000] at 16 kHz) instead.

One step = one whole decode (every kernel of the path) of the batch, inputs
already resident in HBM.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense FP32 matrix


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4, choices=(4, 5))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-frames", type=int, default=120,
                    help="latent frames of the oracle's bounded CPU sample (one pass)")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the other full decoder config's figure (workload 5 or 4)")
    ap.add_argument("--no-bwe", action="store_true",
                    help="skip the LTX bandwidth-extension tail figure (workload 7)")
    ap.add_argument("--no-dav", action="store_true",
                    help="skip the Music-3 DAV decoder figure (workload 6)")
    ap.add_argument("--stream-tile", type=int, default=100,
                    help="latent frames per tile of the streaming-decode figure (0: skip it)")
    ap.add_argument("--serial-mrf", action="store_true",
                    help="run each stage's AMP blocks one after the other on one stream "
                         "(default: overlapped on the decoder's side streams)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the figures of configs 1-3 (AMP blocks and one upsample stage)")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the oracle parity figures (sampled windows) in the JSON line")
    ap.add_argument("--timed-only", action="store_true",
                    help="warm-up, timed and profiled steps of the headline schedule only, then "
                         "print the line (the command behind the kernel-trace profile)")
    ap.add_argument("--only", choices=("act1d", "configs"),
                    help="run one figure alone and print it (for counter profiles): "
                         "act1d = avae_act1d on [2,512,65536]; configs = configs 1-3")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="also run one plain 256 MiB device-to-device copy, whose "
                         "FETCH_SIZE / WRITE_SIZE counters calibrate the traffic figures")
    return ap.parse_args()


def cpu_baseline(spec, z, t, frames):
    """The float64 oracle, as it stands, on a bounded sample: one pass of the
    first `frames` latent frames of the same workload."""
    import numpy as np
    from oracle import avae_oracle as O
    from tests.helpers import decoder_params
    p = decoder_params(spec, t)
    zs = np.ascontiguousarray(z[:1, :, :frames])
    t0 = time.perf_counter()
    c0 = time.process_time()
    y = O.decode(zs, p)
    dt = time.perf_counter() - t0
    cpu = time.process_time() - c0
    samples = y.shape[-1]
    return {"value": samples / dt, "unit": "samples/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"one mono pass of the first {frames} latent frames "
                      f"({samples} output samples) in {dt:.1f} s",
            "nproc": nproc(), "cpu_seconds": cpu, "mean_busy_threads": cpu / dt}


def nproc():
    """Host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except Exception:
        return os.cpu_count() or 1


def blas_threads():
    """Threads the oracle's library matrix products run on (its only
    multi-threaded step; the rest of the oracle is single-threaded numpy)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] + [1]))
    except Exception:
        return 1


def dominant_kernel(kernels):
    """The kernel with the largest share of the decode's roofline sum: its
    algorithmic time max(flops / MFMA peak, bytes / HBM peak), summed over its
    launches.  (Summed event durations would rank the kernels by how long
    they waited beside other streams' kernels, not by their work.)"""
    return max(kernels, key=lambda n: max(kernels[n]["flops"] / FP32_MFMA_PEAK_TFLOPS,
                                          kernels[n]["bytes"] / HBM_PEAK_GBPS * 1e-3))


def roofline(kernels, steps, name=None):
    """Roofline entry for one kernel (default: the dominant one): achieved =
    algorithmic flops (matrix kernels) or bytes (Activation1d) per launch /
    average launch duration, against MI355X's published peak."""
    if name is None:
        name = dominant_kernel(kernels)
    k = kernels[name]
    avg_s = k["total_ms"] / 1e3 / k["launches"]
    if _hbm_bound(name, k):
        achieved = k["bytes"] / k["launches"] / avg_s / 1e9
        peak, unit, bound = HBM_PEAK_GBPS, "GB/s", "hbm"
    else:
        achieved = k["flops"] / k["launches"] / avg_s / 1e12
        peak, unit, bound = FP32_MFMA_PEAK_TFLOPS, "TFLOP/s", "mfma"
    return {"kernel": name, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": traffic_for(name),
            "launches_per_step": k["launches"] / steps, "avg_launch_us": avg_s * 1e6,
            "algorithmic_per_launch": (k["bytes"] if bound == "hbm" else k["flops"]) / k["launches"]}


def _hbm_bound(name, k):
    """Whether a kernel's algorithmic bound is HBM bandwidth: its bytes at the
    HBM peak take longer than its flops at the FP32 matrix peak (the
    activations, the FFT convolution's transforms, the MRF sum)."""
    return k["bytes"] / (HBM_PEAK_GBPS * 1e9) > k["flops"] / (FP32_MFMA_PEAK_TFLOPS * 1e12)


def traffic_for(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        import hashlib
        d = json.load(open(path))
        e = d.get("kernels", {}).get(name)
        if not e:
            return None
        src = os.path.join(ROOT, e["source"])
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if sha != e["source_sha256"]:
            return None
        return e["hbm_bytes_per_launch"]
    except Exception:
        return None


def act1d_standalone(torch, avae, W, steps):
    """avae_act1d alone on workload 2's shape [2, 512, 65536]: HBM GB/s."""
    dev = torch.device("cuda:0")
    x, la, lb, _ = W.workload2()
    xd = torch.from_numpy(x).to(dev)
    lad = torch.from_numpy(la).to(dev)
    lbd = torch.from_numpy(lb).to(dev)
    yd = torch.empty_like(xd)
    # Warm-up on the kernel's own load: after an idle gap the compute clock
    # ramps up over ~20 ms of continuous Activation1d work (launch times fall
    # 118 -> 93 us over 300 back-to-back launches, while a copy of the same
    # tensor runs at its steady rate from the start), so ~30 ms of launches
    # come first and the timed launches see the steady clock.
    warm = 300
    for _ in range(warm):
        avae.act1d(xd, lad, lbd, out=yd)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n = max(steps, 10)
    e0.record(s)
    for _ in range(n):
        avae.act1d(xd, lad, lbd, out=yd)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    gbps = 8.0 * x.size / (ms / 1e3) / 1e9
    # a plain device-to-device copy of the same tensor: the HBM rate this
    # machine delivers to a read-once / write-once stream
    for _ in range(3):
        yd.copy_(xd)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(n):
        yd.copy_(xd)
    e1.record(s)
    torch.cuda.synchronize()
    copy_gbps = 8.0 * x.size / (e0.elapsed_time(e1) / n / 1e3) / 1e9
    # the library's streaming copy (one float4 per thread, every load of the
    # grid in flight at once): faster than the runtime's copy, so the honest
    # measured HBM ceiling for a read-once / write-once kernel
    for _ in range(3):
        avae.probe_copy(xd, yd)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(n):
        avae.probe_copy(xd, yd)
    e1.record(s)
    torch.cuda.synchronize()
    stream_gbps = 8.0 * x.size / (e0.elapsed_time(e1) / n / 1e3) / 1e9
    return {"shape": list(x.shape), "warmup_launches": warm, "timed_launches": n, "ms": ms,
            "GBps": gbps, "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS,
            "copy_GBps": copy_gbps, "frac_of_copy": gbps / copy_gbps,
            "stream_copy_GBps": stream_gbps, "frac_of_stream_copy": gbps / stream_gbps}


def mfma_probe(torch, avae):
    """The FP32 rate the matrix cores deliver (avae_probe_mfma, no memory
    traffic): 16 independent accumulator chains per wave at one wave per SIMD
    (the instruction's full rate), and 8 chains at two waves per SIMD (the
    shape of the convolution kernels' work).  Each grid is exactly one
    resident wave of blocks (256 CUs x waves per SIMD), so no partial second
    round skews the rate, and a warm-up launch of a few ms comes first."""
    dev = torch.device("cuda:0")
    s = torch.cuda.current_stream()
    out = {}
    for key, chains, blocks, iters in (("16_chains_1_wave_per_simd", 16, 256, 20000),
                                       ("8_chains_2_waves_per_simd", 8, 512, 10000)):
        sink = torch.empty(blocks * 256, device=dev)
        avae.probe_mfma(chains, blocks, iters, sink)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        avae.probe_mfma(chains, blocks, iters, sink)
        e1.record(s)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        out[key] = blocks * 4.0 * iters * chains * 2048.0 / (ms / 1e3) / 1e12
    out["unit"] = "TFLOP/s"
    return out


def direct_form_flops(spec, B, frames):
    """The decode's convolution flops counted in the direct form (2 Cout Cin K
    per output sample for every Conv1d, 2 Cin Cout K per input sample for
    every ConvTranspose1d): the algorithmic count of the pages' layers,
    whatever form a kernel evaluates them in."""
    w = spec.widths()
    T = frames
    f = 2.0 * spec.c_in * w[0] * spec.k_pre * T * B
    for i, r in enumerate(spec.rates):
        f += 2.0 * w[i] * w[i + 1] * spec.up_k[i] * T * B
        T *= r
        c = w[i + 1]
        for k, dil in zip(spec.rb_k, spec.rb_d):
            f += len(dil) * 2 * (2.0 * c * c * k * T * B)
    f += 2.0 * w[-1] * spec.k_post * T * B
    return f


def roofline_sum(kernels, steps):
    """Sum over the decode's kernels of max(flops / MFMA peak, bytes / HBM
    peak), per step (aggregated per kernel name; every launch of a name has
    the same bound)."""
    t = 0.0
    for k in kernels.values():
        t += max(k["flops"] / (FP32_MFMA_PEAK_TFLOPS * 1e12), k["bytes"] / (HBM_PEAK_GBPS * 1e9))
    return t * 1e3 / steps


def cpu_amp_block_one_core(W):
    """The oracle on one core: workload 1 (one AMP block, [1, 32, 4096])
    whole, and bounded samples of workload 2."""
    import numpy as np
    from oracle import avae_oracle as O
    from tests.helpers import amp_params
    x, t = W.workload1()
    p = amp_params(t, "block", 3, (1, 3, 5))
    xs = np.asarray(x, np.float64)
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    ctx = threadpool_limits(1) if threadpool_limits else None
    t0 = time.perf_counter()
    if ctx is not None:
        with ctx:
            O.amp_block(xs, p)
    else:
        O.amp_block(xs, p)
    dt = time.perf_counter() - t0
    res = {"workload": "one AMP block, [1,32,4096], k=3, d=(1,3,5)", "seconds": dt,
           "samples_per_s": x.shape[-1] / dt, "cores": 1}
    # workload 2 on one core, on a bounded sample: one pass (B = 1) of the
    # 512-channel block and of the standalone Activation1d over the first
    # 2048 samples (the full [2, 512, 65536] block is 1.24 TFLOP of float64
    # work); samples/s scale linearly with the length at this size
    x2, la, lb, t2 = W.workload2()
    xs = np.asarray(x2[:1, :, :2048], np.float64)
    p2 = amp_params(t2, "block", 3, (1, 3, 5))
    ctx = threadpool_limits(1) if threadpool_limits else None
    t0 = time.perf_counter()
    if ctx is not None:
        with ctx:
            O.amp_block(xs, p2)
    else:
        O.amp_block(xs, p2)
    dt2 = time.perf_counter() - t0
    h = O.kaiser_sinc()
    t0 = time.perf_counter()
    O.act1d(xs[0], np.asarray(la, np.float64), np.asarray(lb, np.float64), h, h)
    dt3 = time.perf_counter() - t0
    res["workload2_amp_block_sample"] = {
        "sample": "one pass, [1, 512, 2048] of workload 2, k=3, d=(1,3,5)", "seconds": dt2,
        "samples_per_s": 2048 / dt2, "cores": 1,
        "full_config_estimate_s": dt2 * (2 * 65536) / 2048}
    res["workload2_act1d_sample"] = {
        "sample": "one pass, [512, 2048] of workload 2", "seconds": dt3,
        "elements_per_s": 512 * 2048 / dt3, "GBps": 8.0 * 512 * 2048 / dt3 / 1e9, "cores": 1}
    return res


def _timed(torch, fn, n):
    """Average ms of fn() over n calls, timed with events on the current
    stream (the library launches on it); two warm-up calls first."""
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(n):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _profiled(avae, fn, n, per_call):
    """Per-kernel event figures of n calls of fn() from the library's
    launch profiler (each launch bracketed by events on its own stream)."""
    avae.profile_begin(n * per_call + 64)
    for _ in range(n):
        fn()
    kernels, _ = avae.profile_end()
    return kernels


def _kernel_rows(kernels, n):
    """Per kernel name: launches and ms per call, algorithmic rate and its
    fraction of the MI355X peak (FP32 matrix for the convolutions, HBM for
    the activations)."""
    rows = {}
    for name, k in sorted(kernels.items(), key=lambda kv: -kv[1]["total_ms"]):
        sec = k["total_ms"] / 1e3
        row = {"launches_per_call": k["launches"] / n, "ms_per_call": k["total_ms"] / n,
               "avg_launch_us": 1e6 * sec / max(k["launches"], 1)}
        if _hbm_bound(name, k):
            row["GBps"] = k["bytes"] / sec / 1e9
            row["frac_of_hbm_peak"] = row["GBps"] / HBM_PEAK_GBPS
        else:
            row["TFLOPs"] = k["flops"] / sec / 1e12
            row["frac_of_fp32_mfma_peak"] = row["TFLOPs"] / FP32_MFMA_PEAK_TFLOPS
        rows[name] = row
    return rows


def _amp_lists(td, prefix, n):
    return ([td[f"{prefix}.convs1.{q}.weight"] for q in range(n)],
            [td[f"{prefix}.convs1.{q}.bias"] for q in range(n)],
            [td[f"{prefix}.convs2.{q}.weight"] for q in range(n)],
            [td[f"{prefix}.convs2.{q}.bias"] for q in range(n)],
            [td[f"{prefix}.activations.{q}.act.alpha"] for q in range(2 * n)],
            [td[f"{prefix}.activations.{q}.act.beta"] for q in range(2 * n)])


def _rel_err(got, ref):
    import numpy as np
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / rms


def amp_configs(torch, avae, W, steps, parity):
    """Configs 1-3 of the workload table, each timed as a whole (events on
    the stream) and per kernel (the library's launch profiler), with the
    roofline sum of its kernels and, with `parity`, max|err|/RMS against
    the float64 oracle (whole output for config 1; windows recomputed from
    crops wider than the block's reach for configs 2 and 3)."""
    import numpy as np
    dev = torch.device("cuda:0")
    out = {}
    dil = (1, 3, 5)
    n = max(steps // 2, 5)

    def finish(key, ms, kernels, flops_call, extra):
        fig = {"ms": ms, "kernels": _kernel_rows(kernels, n)}
        t_roof = roofline_sum(kernels, n)
        fig["roofline_sum_ms"] = t_roof
        fig["frac_of_roofline_sum"] = t_roof / ms
        fig["TFLOPs_overall"] = flops_call / (ms / 1e3) / 1e12
        fig.update(extra)
        out[key] = fig

    # config 1: one AMP block [1, 32, 4096], k=3
    x, t = W.workload1()
    td = {k: torch.from_numpy(v).to(dev) for k, v in t.items()}
    xd = torch.from_numpy(x).to(dev)
    yd = torch.empty_like(xd)
    ws = torch.empty(avae.amp_block_workspace_bytes(*x.shape), dtype=torch.uint8, device=dev)
    lists = _amp_lists(td, "block", 3)
    call = lambda: avae.amp_block(xd, 3, dil, *lists, out=yd, workspace=ws)
    ms = _timed(torch, call, n)
    kernels = _profiled(avae, call, n, 16)
    B, C, T = x.shape
    extra = {"workload": "one AMP block, [1,32,4096], k=3, d=(1,3,5)",
             "samples_per_s": B * T / (ms / 1e3)}
    if parity:
        from oracle import avae_oracle as O
        from tests.helpers import amp_params
        call()
        torch.cuda.synchronize()
        extra["parity_max_err_over_rms"] = _rel_err(yd.cpu().numpy(),
                                                    O.amp_block(x, amp_params(t, "block", 3, dil)))
        extra["parity_scope"] = "whole output"
    finish("config1_amp_block", ms, kernels, 6 * 2.0 * C * C * 3 * T * B, extra)
    del td, xd, yd, ws

    # config 2: one AMP block [2, 512, 65536], k=3 (the 3-tap 512-channel convs)
    x, _, _, t = W.workload2()
    td = {k: torch.from_numpy(v).to(dev) for k, v in t.items()}
    xd = torch.from_numpy(x).to(dev)
    yd = torch.empty_like(xd)
    # the direct kernels first (workspace of avae_amp_block_workspace_bytes),
    # then the frequency-domain convolutions (the larger workspace selects them)
    lists = _amp_lists(td, "block", 3)
    ws = torch.empty(avae.amp_block_workspace_bytes(*x.shape), dtype=torch.uint8, device=dev)
    ms_direct = _timed(torch, lambda: avae.amp_block(xd, 3, dil, *lists, out=yd, workspace=ws), n)
    del ws
    ws = torch.empty(avae.amp_block_fft_workspace_bytes(*x.shape, 3, dil), dtype=torch.uint8,
                     device=dev)
    call = lambda: avae.amp_block(xd, 3, dil, *lists, out=yd, workspace=ws)
    ms = _timed(torch, call, n)
    kernels = _profiled(avae, call, n, 32)  # 6 convolutions x (packing + 3)
    B, C, T = x.shape
    convs = {k: v for k, v in kernels.items() if k.startswith(("conv1d", "fft_"))}
    cf = 6 * 2.0 * C * C * 3 * T * B * n  # direct-form multiply-adds x 2
    ct = sum(v["total_ms"] for v in convs.values()) / 1e3
    extra = {"workload": "one AMP block, [2,512,65536], k=3, d=(1,3,5)",
             "samples_per_s": B * T / (ms / 1e3),
             "direct_kernels_ms": ms_direct,
             "conv_direct_form_TFLOPs": cf / ct / 1e12,
             "conv_ms_per_call": ct * 1e3 / n}
    if parity:
        from oracle import avae_oracle as O
        from tests.helpers import amp_params, amp_reach
        call()
        torch.cuda.synchronize()
        y = yd.cpu().numpy()
        p = amp_params(t, "block", 3, dil)
        m = amp_reach(3, dil) + 8
        errs = []
        for a0 in (0, 30000, T - 256):
            lo, hi = max(a0 - m, 0), min(a0 + 256 + m, T)
            ref = O.amp_block(x[..., lo:hi], p)[..., a0 - lo:a0 - lo + 256]
            errs.append(_rel_err(y[..., a0:a0 + 256], ref))
        extra["parity_max_err_over_rms"] = max(errs)
        extra["parity_scope"] = "all 512 channels of both passes, time windows [0,256), " \
                                "[30000,30256), [65280,65536)"
    finish("config2_amp_block", ms, kernels, 6 * 2.0 * C * C * 3 * T * B, extra)
    del td, xd, yd, ws
    torch.cuda.empty_cache()

    # config 3: ConvTranspose1d 1024 -> 512 (k=10, s=5) on [2,1024,8000], then
    # the MRF of blocks k=(3,7,11) accumulated into one output
    x, t = W.workload3()
    td = {k: torch.from_numpy(v).to(dev) for k, v in t.items()}
    xd = torch.from_numpy(x).to(dev)
    up = avae.convtr1d(xd, td["ups.0.weight"], td["ups.0.bias"], stride=5)
    yd = torch.empty_like(up)
    ws = torch.empty(max(avae.amp_block_fft_workspace_bytes(*up.shape, k, dil) for k in (3, 7, 11)),
                     dtype=torch.uint8, device=dev)
    blists = [_amp_lists(td, f"resblocks.{j}", 3) for j in range(3)]

    def stage():
        avae.convtr1d(xd, td["ups.0.weight"], td["ups.0.bias"], stride=5, out=up)
        for j, k in enumerate((3, 7, 11)):
            avae.amp_block(up, k, dil, *blists[j], out_scale=1.0 / 3.0, accumulate=j > 0,
                           out=yd, workspace=ws)
    ms = _timed(torch, stage, n)
    kernels = _profiled(avae, stage, n, 96)  # 1 + 18 convolutions x (packing + 3)
    B, Cin, Tin = x.shape
    _, C, T = up.shape
    flops = 2.0 * Cin * C * 10 * Tin * B + sum(6 * 2.0 * C * C * k * T * B for k in (3, 7, 11))
    extra = {"workload": "ConvTranspose1d 1024->512 k=10 s=5 on [2,1024,8000], then the MRF "
                         "(3,7,11)x(1,3,5) -> [2,512,40001]",
             "samples_per_s": B * T / (ms / 1e3)}
    if parity:
        from oracle import avae_oracle as O
        from tests.helpers import amp_params, amp_reach
        stage()
        torch.cuda.synchronize()
        y = yd.cpu().numpy()
        xo = O.convtr1d(x, t["ups.0.weight"], t["ups.0.bias"], stride=5)
        e_up = _rel_err(up.cpu().numpy(), xo)
        blocks = [amp_params(t, f"resblocks.{j}", k, dil) for j, k in enumerate((3, 7, 11))]
        m = max(amp_reach(k, dil) for k in (3, 7, 11)) + 8
        errs = []
        for a0 in (0, T - 200):
            lo, hi = max(a0 - m, 0), min(a0 + 200 + m, T)
            ref = O.mrf(xo[..., lo:hi], blocks)[..., a0 - lo:a0 - lo + 200]
            errs.append(_rel_err(y[..., a0:a0 + 200], ref))
        extra["parity_max_err_over_rms"] = max(errs)
        extra["parity_convtr1d_max_err_over_rms"] = e_up
        extra["parity_scope"] = "ConvTranspose1d output whole; MRF output on all 512 channels " \
                                "of both passes, time windows [0,200) and [39801,40001)"
    finish("config3_upsample_stage", ms, kernels, flops, extra)
    del td, xd, up, yd, ws
    torch.cuda.empty_cache()
    return out


def decode_parity(torch, dec, spec, z, t, B, F):
    """max|err|/RMS of the full-size decode against the float64 oracle on a
    4-frame window in the middle of the last pass, the oracle decoding a
    latent crop whose margin exceeds the receptive-field bound: on the
    conv_post output before the final nonlinearity (the decode's bar) and on
    the waveform."""
    import numpy as np
    from oracle import avae_oracle as O
    from tests.helpers import decoder_params, decoder_reach_frames
    wave, stages = dec.decode(torch.from_numpy(z).to("cuda:0"), trace=True)
    torch.cuda.synchronize()
    pre = stages[-1][B - 1].cpu().numpy()
    w = wave[B - 1].cpu().numpy()
    R = decoder_reach_frames(spec)
    a = F // 2
    lo, hi = max(a - R, 0), min(a + 4 + R, F)
    p = decoder_params(spec, t)
    t0 = time.perf_counter()
    wref = O.decode(z[B - 1:B, :, lo:hi], p, record=True)[0]
    dt = time.perf_counter() - t0
    hop = spec.hop
    off = (a - lo) * hop
    pre_ref = p.stages[-1][0, 0, off:off + 4 * hop]
    return {"workload": f"{spec.name}, pass {B - 1}, latent frames [{a}, {a + 4}) "
                        f"from a crop [{lo}, {hi})",
            "pre_final_max_err_over_rms": _rel_err(pre[a * hop:(a + 4) * hop], pre_ref),
            "wave_max_abs_err": float(np.max(np.abs(w[a * hop:(a + 4) * hop] -
                                                    wref[off:off + 4 * hop]))),
            "bar": 1e-3, "oracle_seconds": dt}


def other_decoder(torch, avae, W, which, steps):
    """The other full decoder config, timed like the main step: workload 5
    (LTX-2.5-shaped, [2,64,2000] log-mel -> [2,320000] at 16 kHz) when the
    main step is workload 4, and the reverse."""
    dev = torch.device("cuda:0")
    z, t = W.workload5() if which == 5 else W.workload4()
    spec = W.LTX if which == 5 else W.H3
    dec = avae.Decoder(spec, {k: torch.from_numpy(v).to(dev) for k, v in t.items()})
    B, _, F = z.shape
    L = dec.output_length(F)
    zd = torch.from_numpy(z).to(dev)
    ws = torch.empty(dec.workspace_bytes(B, F), dtype=torch.uint8, device=dev)
    out = torch.empty((B, L), dtype=torch.float32, device=dev)
    for _ in range(3):
        dec.decode(zd, out=out, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        dec.decode(zd, out=out, workspace=ws)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    res = {"workload": f"{spec.name} decode, latent [{B},{spec.c_in},{F}] -> wave [{B},{L}] "
                       f"at {spec.sample_rate} Hz",
           "ms": ms, "samples_per_s": B * L / (ms / 1e3),
           "x_realtime": (L / spec.sample_rate) / (ms / 1e3)}
    # roofline sum over its kernels, each launch alone on the GPU (blocks
    # serialized for the profiled pass), against the timed step
    dec.set_concurrent(False)
    n = max(steps // 2, 3)
    kernels = _profiled(avae, lambda: dec.decode(zd, out=out, workspace=ws), n, 400)
    dec.set_concurrent(True)
    t_roof = roofline_sum(kernels, n)
    res["roofline_sum_ms"] = t_roof
    res["frac_of_roofline_sum"] = t_roof / ms
    top = sorted(kernels.items(), key=lambda kv: -kv[1]["total_ms"])[:8]
    res["kernels"] = _kernel_rows(dict(top), n)
    return res


def streaming(torch, dec, zd, out, tile, steps):
    """avae_bigvgan_decode_streaming over the same batch in tiles of `tile`
    frames with the receptive-field halo: throughput and recompute overhead."""
    B, _, F = zd.shape
    ws = torch.empty(dec.streaming_workspace_bytes(B, min(tile, F)), dtype=torch.uint8,
                     device=zd.device)
    for _ in range(2):
        dec.decode_streaming(zd, tile, out=out, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n = max(steps // 2, 3)
    e0.record(s)
    for _ in range(n):
        dec.decode_streaming(zd, tile, out=out, workspace=ws)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    R = dec.reach_frames()
    tiles = -(-F // tile)
    # the end tiles decode min(tile + R, F) frames, inner tiles min(tile + 2 R, F)
    if tiles == 1:
        decoded = F
    else:
        decoded = 2 * min(tile + R, F) + (tiles - 2) * min(tile + 2 * R, F)
    return {"tile_frames": tile, "halo_frames": R, "tiles": tiles, "ms": ms,
            "samples_per_s": out.numel() / (ms / 1e3), "decoded_frames_ratio": decoded / F,
            "workspace_MB": ws.numel() / 1e6}


def dav_figure(torch, avae, W, steps):
    """The Music-3 DAV decoder on workload 6: stereo latent [1,128,862] ->
    interleaved [1, 2*441344] at 44.1 kHz (10 s), timed like the main step,
    with its per-kernel split from the library's launch profiler."""
    dev = torch.device("cuda:0")
    z, t = W.workload6()
    dav = avae.DavDecoder(W.DAV, {k: torch.from_numpy(v).to(dev) for k, v in t.items()})
    B, _, F = z.shape
    L = dav.output_length(F)
    zd = torch.from_numpy(z).to(dev)
    ws = torch.empty(dav.workspace_bytes(B, F), dtype=torch.uint8, device=dev)
    out = torch.empty((B, 2 * L), dtype=torch.float32, device=dev)
    for _ in range(2):
        dav.decode(zd, out=out, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n = max(steps // 2, 3)
    e0.record(s)
    for _ in range(n):
        dav.decode(zd, out=out, workspace=ws)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    avae.profile_begin(n * 200 + 64)
    for _ in range(n):
        dav.decode(zd, out=out, workspace=ws)
    kernels, _ = avae.profile_end()
    top = sorted(kernels.items(), key=lambda kv: -kv[1]["total_ms"])[:6]
    t_roof = roofline_sum(kernels, n)
    return {"workload": f"music3-dav decode, latent [{B},128,{F}] -> [{B},{2 * L}] "
                        f"interleaved stereo at {W.DAV.sample_rate} Hz",
            "ms": ms, "samples_per_s": out.numel() / (ms / 1e3),
            "x_realtime": (L / W.DAV.sample_rate) / (ms / 1e3),
            "roofline_sum_ms": t_roof, "frac_of_roofline_sum": t_roof / ms,
            "kernels": _kernel_rows(dict(top), n)}


def bwe_figure(torch, avae, W, steps):
    """The LTX bandwidth-extension tail on workload 7: 16 kHz [2,320000] ->
    48 kHz [2,960000] (log-mel, generator, Hann-sinc skip, clamp)."""
    dev = torch.device("cuda:0")
    low, t = W.workload7()
    dec = avae.BweDecoder(W.BWE, {k: torch.from_numpy(v).to(dev) for k, v in t.items()})
    B, T = low.shape
    ld = torch.from_numpy(low).to(dev)
    ws = torch.empty(dec.workspace_bytes(B, T), dtype=torch.uint8, device=dev)
    out = torch.empty((B, 3 * T), dtype=torch.float32, device=dev)
    for _ in range(2):
        dec.decode(ld, out=out, workspace=ws)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n = max(steps // 2, 3)
    e0.record(s)
    for _ in range(n):
        dec.decode(ld, out=out, workspace=ws)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    avae.profile_begin(n * 300 + 64)
    for _ in range(n):
        dec.decode(ld, out=out, workspace=ws)
    kernels, _ = avae.profile_end()
    top = sorted(kernels.items(), key=lambda kv: -kv[1]["total_ms"])[:6]
    t_roof = roofline_sum(kernels, n)
    return {"workload": f"ltx bandwidth extension, [{B},{T}] at 16 kHz -> [{B},{3 * T}] at 48 kHz",
            "ms": ms, "samples_per_s": out.numel() / (ms / 1e3),
            "x_realtime": (T / 16000.0) / (ms / 1e3),
            "roofline_sum_ms": t_roof, "frac_of_roofline_sum": t_roof / ms,
            "kernels": _kernel_rows(dict(top), n),
            "mel_stft_ms": kernels.get("mel_stft_kernel", {}).get("total_ms", 0.0) / n,
            "combine_ms": kernels.get("bwe_combine_kernel", {}).get("total_ms", 0.0) / n}


def pmc_calibration_copy(torch, res):
    """One plain 256 MiB device-to-device copy: its FETCH_SIZE / WRITE_SIZE
    counters (known bytes) calibrate the traffic figures of a counter run."""
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    res["pmc_calibration_copy_bytes"] = src.numel() * 4


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the decoder's "
              "multi-GPU split is a design note, not part of this build", file=sys.stderr)
        sys.exit(2)
    import torch
    from bigvgan_waveform_decoder_amd import avae
    from bigvgan_waveform_decoder_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.only:
        res = {"only": args.only}
        if args.only == "act1d":
            res["act1d_workload2"] = act1d_standalone(torch, avae, W, args.steps)
        else:
            res["configs"] = amp_configs(torch, avae, W, args.steps, not args.no_parity)
        if args.pmc_calibration:
            pmc_calibration_copy(torch, res)
        print(json.dumps(res), flush=True)
        return
    if args.workload == 4:
        z, t = W.workload4()
        spec = W.H3
    else:
        z, t = W.workload5()
        spec = W.LTX
    B, _, F = z.shape
    td = {k: torch.from_numpy(v).to(dev) for k, v in t.items()}
    dec = avae.Decoder(spec, td)
    if args.serial_mrf:
        dec.set_concurrent(False)
    L = dec.output_length(F)
    zd = torch.from_numpy(z).to(dev)
    ws = torch.empty(dec.workspace_bytes(B, F), dtype=torch.uint8, device=dev)
    out = torch.empty((B, L), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        dec.decode(zd, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        dec.decode(zd, out=out, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    value = B * L / (ms / 1e3)
    xrt = (L / spec.sample_rate) / (ms / 1e3)

    res = {
        "metric": "BigVGAN decode output samples/s (x-realtime) at 1 GPU",
        "value": value,
        "unit": "samples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "x_realtime": xrt,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded latents, He-initialised random weights)",
        "config": {"workload": f"{spec.name} decode, latent [{B},{spec.c_in},{F}] -> "
                               f"wave [{B},{L}] at {spec.sample_rate} Hz",
                   "global_batch": B, "frames": F, "parallelism": "none (1 GPU)"},
    }
    # Profiled passes over the same number of steps: per-kernel event timing
    # inside the library (the clean timed region above carries no events).
    def profiled():
        avae.profile_begin(args.steps * 400 + 64)
        for _ in range(args.steps):
            dec.decode(zd, out=out, workspace=ws)
        return avae.profile_end()

    kernels, phases = profiled()
    res["mrf_blocks"] = "serial" if args.serial_mrf else "concurrent (3 streams)"
    # with overlapped AMP blocks the kernel times add up to more than a step
    res["kernel_ms_per_step_sum"] = sum(k["total_ms"] for k in kernels.values()) / args.steps
    res["phases_ms_per_step"] = {k: v / args.steps for k, v in phases.items()}
    # The headline roofline is the dominant kernel as it runs in the timed
    # schedule (its launches' events in the profiled pass of the same steps,
    # on the streams they run on).  With the AMP blocks overlapped a launch
    # shares the CUs with the other blocks' kernels and lasts longer than its
    # own work needs, so the same kernel with every launch alone on the GPU
    # follows as roofline_isolated (a further pass with the blocks serialized).
    if args.timed_only:
        res["roofline"] = roofline(kernels, args.steps)
        res["roofline"]["measured"] = ("timed schedule: " + res["mrf_blocks"] +
                                       " (profiled pass of the same steps)")
        if args.pmc_calibration:
            pmc_calibration_copy(torch, res)
        print(json.dumps(res), flush=True)
        return
    if args.serial_mrf:
        iso = kernels
    else:
        dec.set_concurrent(False)
        # the single-stream schedule, timed like the headline
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            dec.decode(zd, out=out, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        ms1 = e0.elapsed_time(e1) / args.steps
        res["single_stream"] = {"ms_per_step": ms1, "samples_per_s": B * L / (ms1 / 1e3)}
        iso, _ = profiled()
        dec.set_concurrent(True)
    dom = dominant_kernel(iso)
    res["roofline"] = roofline(kernels, args.steps, dom)
    res["roofline"]["measured"] = ("timed schedule: " + res["mrf_blocks"] +
                                   " (profiled pass of the same steps)")
    res["roofline_isolated"] = roofline(iso, args.steps, dom)
    res["roofline_isolated"]["measured"] = ("AMP blocks serialized: every launch alone on the "
                                            "GPU")
    probe = mfma_probe(torch, avae)
    res["mfma_probe"] = probe
    for key in ("roofline", "roofline_isolated"):
        if res[key]["unit"] == "TFLOP/s":
            res[key]["frac_of_probe_peak"] = (res[key]["achieved"] /
                                              probe["16_chains_1_wave_per_simd"])
    # roofline sum over the decode's kernels vs the timed step (and vs the
    # single-stream step, whose launches are the same ones one after another)
    t_roof = roofline_sum(iso, args.steps)
    single_ms = ms if args.serial_mrf else res["single_stream"]["ms_per_step"]
    res["decode_roofline_sum"] = {"ms": t_roof, "frac_of_timed": t_roof / ms,
                                  "frac_of_single_stream": t_roof / single_ms}
    # the whole step's rate of executed flops (the frequency-domain
    # convolutions count their complex products, not the direct form's taps)
    res["decode_TFLOPs"] = sum(k["flops"] for k in iso.values()) / args.steps / (ms / 1e3) / 1e12
    # the same step against the direct form's flop count: above the matrix
    # peak where the transforms save more multiply-adds than they cost
    res["decode_direct_form_TFLOPs"] = (direct_form_flops(spec, B, F) / (ms / 1e3) / 1e12)
    acts = [v for k, v in iso.items() if k.startswith("act1d")]
    if acts:
        ab = sum(v["bytes"] for v in acts)
        at = sum(v["total_ms"] for v in acts)
        res["act1d_in_decode_GBps"] = ab / (at / 1e3) / 1e9
    res["act1d_workload2"] = act1d_standalone(torch, avae, W, args.steps)
    res["kernels"] = {k: {"launches_per_step": v["launches"] / args.steps,
                          "ms_per_step": v["total_ms"] / args.steps,
                          "avg_us": 1e3 * v["total_ms"] / max(v["launches"], 1)}
                      for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["total_ms"])}
    if not args.no_dav:
        res["dav"] = dav_figure(torch, avae, W, args.steps)
    if not args.no_bwe:
        res["bwe"] = bwe_figure(torch, avae, W, args.steps)
    if not args.no_other:
        res["other_decoder"] = other_decoder(torch, avae, W, 5 if args.workload == 4 else 4,
                                             args.steps)
    if args.stream_tile > 0:
        res["streaming"] = streaming(torch, dec, zd, out, args.stream_tile, args.steps)
    if not args.no_configs:
        res["configs"] = amp_configs(torch, avae, W, args.steps, not args.no_parity)
    if not args.no_parity:
        res["parity"] = decode_parity(torch, dec, spec, z, t, B, F)
    res["seeds"] = {"generator": "numpy PCG64, one stream per tensor, seed = master ^ "
                                 "FNV-1a-64(tensor name); normals drawn in float64, rounded "
                                 "to float32",
                    "master": {f"workload{i}": hex(W.master_seed(i)) for i in range(1, 8)}}
    if args.pmc_calibration:
        pmc_calibration_copy(torch, res)
    # the same step with the latent coming from pinned host memory and the
    # waveform going back to it (PCIe both ways), for context
    zh = torch.from_numpy(z).pin_memory()
    oh = torch.empty((B, L), dtype=torch.float32).pin_memory()
    for _ in range(2):
        zd.copy_(zh, non_blocking=True)
        dec.decode(zd, out=out, workspace=ws)
        oh.copy_(out, non_blocking=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        zd.copy_(zh, non_blocking=True)
        dec.decode(zd, out=out, workspace=ws)
        oh.copy_(out, non_blocking=True)
    e1.record(stream)
    torch.cuda.synchronize()
    msh = e0.elapsed_time(e1) / args.steps
    res["with_host_copies"] = {"ms_per_step": msh, "samples_per_s": B * L / (msh / 1e3)}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, z, t, args.cpu_frames)
        res["cpu_amp_block_one_core"] = cpu_amp_block_one_core(W)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
