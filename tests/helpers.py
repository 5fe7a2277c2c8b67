"""Test glue: turns the seeded tensors of a workload into the oracle's
parameter objects, and the error metric every parity test uses."""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np

from oracle import avae_oracle as O


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def amp_params(t: Dict[str, np.ndarray], prefix: str, k: int, dil: Sequence[int]) -> O.AmpParams:
    n = len(dil)
    return O.AmpParams(
        k=k, dil=list(dil),
        w1=[f64(t[f"{prefix}.convs1.{q}.weight"]) for q in range(n)],
        b1=[f64(t[f"{prefix}.convs1.{q}.bias"]) for q in range(n)],
        w2=[f64(t[f"{prefix}.convs2.{q}.weight"]) for q in range(n)],
        b2=[f64(t[f"{prefix}.convs2.{q}.bias"]) for q in range(n)],
        la=[f64(t[f"{prefix}.activations.{q}.act.alpha"]) for q in range(2 * n)],
        lb=[f64(t[f"{prefix}.activations.{q}.act.beta"]) for q in range(2 * n)],
    )


def decoder_params(spec, t: Dict[str, np.ndarray]) -> O.DecoderParams:
    nk = len(spec.rb_k)
    blocks = []
    for i in range(len(spec.rates)):
        blocks.append([amp_params(t, f"resblocks.{i * nk + j}", spec.rb_k[j], spec.rb_d[j])
                       for j in range(nk)])
    return O.DecoderParams(
        conv_pre_w=f64(t["conv_pre.weight"]), conv_pre_b=f64(t["conv_pre.bias"]),
        up_w=[f64(t[f"ups.{i}.weight"]) for i in range(len(spec.rates))],
        up_b=[f64(t[f"ups.{i}.bias"]) for i in range(len(spec.rates))],
        rates=list(spec.rates), blocks=blocks,
        post_la=f64(t["activation_post.act.alpha"]), post_lb=f64(t["activation_post.act.beta"]),
        conv_post_w=f64(t["conv_post.weight"]), conv_post_b=f64(t["conv_post.bias"]),
        final=spec.final,
        latent_mean=f64(t["latents_mean"]) if "latents_mean" in t else None,
        latent_std=f64(t["latents_std"]) if "latents_std" in t else None,
        dec_in_w=f64(t["dec_in.weight"]) if "dec_in.weight" in t else None,
        dec_in_b=f64(t["dec_in.bias"]) if "dec_in.bias" in t else None,
    )


def rel_err(got, ref) -> float:
    """max|got - ref| / RMS(ref): the parity metric, in float64."""
    got = f64(got)
    ref = f64(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(got - ref))) if got.size else 0.0
    return float(np.max(np.abs(got - ref))) / rms if got.size else 0.0


def decoder_reach_frames(spec) -> int:
    """Upper bound, in latent frames, on how far an output sample's
    dependence reaches into the latent on either side.  Per layer, in that
    layer's input samples: Activation1d reads x[t-5 .. t+5]; a "same" Conv1d
    (k, d) reaches (k-1)d/2; a ConvTranspose1d output reads inputs within
    ceil(k/s) + 1.  Each reach is divided by the upsampling factor already
    applied, and the sum is rounded up (plus one frame of slack)."""
    import math
    reach = (spec.k_pre - 1) / 2.0
    rate = 1
    for r, k in zip(spec.rates, spec.up_k):
        reach += (math.ceil(k / r) + 1) / rate
        rate *= r
        mrf = max(sum(5 + (kj - 1) * d / 2.0 + 5 + (kj - 1) / 2.0 for d in dj)
                  for kj, dj in zip(spec.rb_k, spec.rb_d))
        reach += mrf / rate
    reach += (5 + (spec.k_post - 1) / 2.0) / rate
    return int(math.ceil(reach)) + 1


def amp_reach(k, dil) -> int:
    """Samples an AMP block's output reaches on either side (same rule)."""
    return int(sum(5 + (k - 1) * d // 2 + 5 + (k - 1) // 2 for d in dil))


def dav_params(spec, t: Dict[str, np.ndarray]) -> O.DavParams:
    """The DAV decoder's weights (H3 page names) as oracle parameters."""
    stages = []
    for i, s in enumerate(spec.strides):
        p = f"mvae.decoder.model.{i + 1}"
        units = []
        for u, d in enumerate(spec.unit_dil):
            q = f"{p}.block.{u + 2}"
            units.append(O.DavUnitParams(
                dilation=d, a1=f64(t[f"{q}.block.0.alpha"]),
                w1=f64(t[f"{q}.block.1.weight"]), b1=f64(t[f"{q}.block.1.bias"]),
                a2=f64(t[f"{q}.block.2.alpha"]),
                w2=f64(t[f"{q}.block.3.weight"]), b2=f64(t[f"{q}.block.3.bias"])))
        stages.append(O.DavStageParams(
            stride=s, alpha=f64(t[f"{p}.block.0.alpha"]), up_w=f64(t[f"{p}.block.1.weight"]),
            up_b=f64(t[f"{p}.block.1.bias"]), units=units))
    n = len(spec.strides)
    return O.DavParams(
        dec_in_w=f64(t["mvae.dec_in_proj.weight"]), dec_in_b=f64(t["mvae.dec_in_proj.bias"]),
        conv_pre_w=f64(t["mvae.decoder.model.0.weight"]),
        conv_pre_b=f64(t["mvae.decoder.model.0.bias"]), stages=stages,
        post_alpha=f64(t[f"mvae.decoder.model.{n + 1}.alpha"]),
        conv_post_w=f64(t[f"mvae.decoder.model.{n + 2}.weight"]),
        conv_post_b=f64(t[f"mvae.decoder.model.{n + 2}.bias"]))


def dav_reach_frames(spec) -> int:
    """Latent frames an output sample of the DAV decoder can depend on, on
    either side: conv_pre (k-1)/2 frames; per stage a transposed conv
    (within ceil(k/s) + 1 of its input samples) and the units' dilated convs
    ((k-1)d/2 samples each, the 1-tap convs and Snake add nothing); conv_post
    (k-1)/2 output samples; each divided by the upsampling already applied,
    rounded up plus one frame of slack."""
    import math
    reach = (spec.k_pre - 1) / 2.0
    rate = 1
    for s, k in zip(spec.strides, spec.up_k):
        reach += (math.ceil(k / s) + 1) / rate
        rate *= s
        reach += sum((spec.unit_k - 1) * d / 2.0 for d in spec.unit_dil) / rate
    reach += (spec.k_post - 1) / 2.0 / rate
    return int(math.ceil(reach)) + 1


def runs_fft_convs(spec) -> bool:
    """Whether the library may run some of this decoder's AMP convolutions in
    the frequency domain (overlap-save, 256-point transforms): widths a
    multiple of 16 with (K-1) d <= 128, from 48 channels with 7 or more taps,
    from 192 to 512 channels with 3 (those only on long enough rows).  The
    block framing then follows the sequence start, so decodes of crops
    (streaming tiles) round differently from the whole sequence there."""
    chans = [spec.c0 // (2 ** (i + 1)) for i in range(len(spec.rates))]
    for c in chans:
        if c % 16:
            continue
        for k, dil in zip(spec.rb_k, spec.rb_d):
            if not any((k - 1) * d <= 128 for d in tuple(dil) + (1,)):
                continue
            if (k >= 7 and c >= 48) or (k >= 3 and 192 <= c <= 512):
                return True
    return False
