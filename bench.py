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
    ap.add_argument("--cpu-frames", type=int, default=24,
                    help="latent frames of the oracle's bounded CPU sample (one pass)")
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
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, z, t, args.cpu_frames)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
