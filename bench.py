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
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    p = decoder_params(spec, t)
    zs = np.ascontiguousarray(z[:1, :, :frames])
    t0 = time.perf_counter()
    y = O.decode(zs, p)
    dt = time.perf_counter() - t0
    samples = y.shape[-1]
    return {"value": samples / dt, "unit": "samples/s", "cores": int(cores), "kind": "oracle",
            "sample": f"one mono pass of the first {frames} latent frames "
                      f"({samples} output samples) in {dt:.1f} s"}


def roofline(kernels, steps):
    """Roofline entry for the kernel with the largest share of decode time:
    achieved = algorithmic flops (matrix kernels) or bytes (Activation1d)
    per launch / average launch duration, against MI355X's published peak."""
    name, k = max(kernels.items(), key=lambda kv: kv[1]["total_ms"])
    avg_s = k["total_ms"] / 1e3 / k["launches"]
    if name.startswith("act1d") or name.startswith("channel_affine"):
        achieved = k["bytes"] / k["launches"] / avg_s / 1e9
        peak, unit, bound = HBM_PEAK_GBPS, "GB/s", "hbm"
    else:
        achieved = k["flops"] / k["launches"] / avg_s / 1e12
        peak, unit, bound = FP32_MFMA_PEAK_TFLOPS, "TFLOP/s", "mfma"
    return {"kernel": name, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": traffic_for(name),
            "launches_per_step": k["launches"] / steps, "avg_launch_us": avg_s * 1e6,
            "algorithmic_per_launch": (k["bytes"] if bound == "hbm" else k["flops"]) / k["launches"]}


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
    for _ in range(3):
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
    return {"shape": list(x.shape), "ms": ms, "GBps": gbps, "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS,
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


def roofline_sum(kernels, steps):
    """Sum over the decode's kernels of max(flops / MFMA peak, bytes / HBM
    peak), per step (aggregated per kernel name; every launch of a name has
    the same bound)."""
    t = 0.0
    for k in kernels.values():
        t += max(k["flops"] / (FP32_MFMA_PEAK_TFLOPS * 1e12), k["bytes"] / (HBM_PEAK_GBPS * 1e9))
    return t * 1e3 / steps


def cpu_amp_block_one_core(W):
    """The oracle on workload 1 (one AMP block, [1, 32, 4096]) on one core."""
    import numpy as np
    from oracle import avae_oracle as O
    from tests.helpers import amp_params
    x, t = W.workload1()
    p = amp_params(t, "block", 3, (1, 3, 5))
    xs = np.asarray(x, np.float64)
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(1)
    except Exception:
        ctx = None
    t0 = time.perf_counter()
    if ctx is not None:
        with ctx:
            O.amp_block(xs, p)
    else:
        O.amp_block(xs, p)
    dt = time.perf_counter() - t0
    return {"workload": "one AMP block, [1,32,4096], k=3, d=(1,3,5)", "seconds": dt,
            "samples_per_s": x.shape[-1] / dt, "cores": 1}


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
    return {"workload": f"{spec.name} decode, latent [{B},{spec.c_in},{F}] -> wave [{B},{L}] "
                        f"at {spec.sample_rate} Hz",
            "ms": ms, "samples_per_s": B * L / (ms / 1e3),
            "x_realtime": (L / spec.sample_rate) / (ms / 1e3)}


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
    return {"workload": f"music3-dav decode, latent [{B},128,{F}] -> [{B},{2 * L}] "
                        f"interleaved stereo at {W.DAV.sample_rate} Hz",
            "ms": ms, "samples_per_s": out.numel() / (ms / 1e3),
            "x_realtime": (L / W.DAV.sample_rate) / (ms / 1e3),
            "kernels_ms": {k: v["total_ms"] / n for k, v in top}}


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
    return {"workload": f"ltx bandwidth extension, [{B},{T}] at 16 kHz -> [{B},{3 * T}] at 48 kHz",
            "ms": ms, "samples_per_s": out.numel() / (ms / 1e3),
            "x_realtime": (T / 16000.0) / (ms / 1e3),
            "kernels_ms": {k: v["total_ms"] / n for k, v in top},
            "mel_stft_ms": kernels.get("mel_stft_kernel", {}).get("total_ms", 0.0) / n,
            "combine_ms": kernels.get("bwe_combine_kernel", {}).get("total_ms", 0.0) / n}


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
    # The roofline is taken with every launch alone on the GPU (a launch that
    # shares the CUs with another block's kernels lasts longer than its own
    # work needs); the same kernel's figure in the timed arrangement follows.
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
    res["roofline"] = roofline(iso, args.steps)
    probe = mfma_probe(torch, avae)
    res["mfma_probe"] = probe
    if res["roofline"]["unit"] == "TFLOP/s":
        res["roofline"]["frac_of_probe_peak"] = (res["roofline"]["achieved"] /
                                                 probe["16_chains_1_wave_per_simd"])
    # roofline sum over the decode's kernels vs the timed step (and vs the
    # single-stream step, whose launches are the same ones one after another)
    t_roof = roofline_sum(iso, args.steps)
    single_ms = ms if args.serial_mrf else res["single_stream"]["ms_per_step"]
    res["decode_roofline_sum"] = {"ms": t_roof, "frac_of_timed": t_roof / ms,
                                  "frac_of_single_stream": t_roof / single_ms}
    res["roofline"]["measured"] = "AMP blocks serialized for this pass: each launch alone on the GPU"
    kname = res["roofline"]["kernel"]
    if kname in kernels and not args.serial_mrf:
        k = kernels[kname]
        avg = k["total_ms"] / 1e3 / k["launches"]
        res["roofline"]["overlapped"] = {
            "avg_launch_us": avg * 1e6,
            "achieved": k["flops"] / k["launches"] / avg / 1e12
            if res["roofline"]["unit"] == "TFLOP/s" else k["bytes"] / k["launches"] / avg / 1e9}
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
    if args.pmc_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["pmc_calibration_copy_bytes"] = src.numel() * 4
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
