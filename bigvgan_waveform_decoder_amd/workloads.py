"""Seeded synthetic workloads: shapes, distributions and the generator.

This module holds no arithmetic of the decoder itself -- only tensor shapes,
the distributions they are drawn from, and a seeded generator -- so that the
HIP path and the float64 oracle can be fed byte-identical inputs without
sharing any of the method's code.

Generator: one numpy PCG64 stream per tensor, seeded with
``master ^ fnv1a64(tensor name)`` where ``master = 0xB1C00000 + workload id``.
Normals are drawn in float64 and rounded to float32.  ``N(mu, v)`` in the
workload descriptions is read with ``v`` as the variance.

Workloads (the shapes of the MiniMax-H3 audio VAE decoder and the LTX-2.5
vocoder pages):
  1  one AMP block, 32 ch x 4096, k=3, d=(1,3,5), W ~ N(0, 1/96)
  2  Activation1d and one AMP block at 512 ch x 65536, stereo (B=2)
  3  one upsample stage: ConvTranspose1d 1024->512, s=5, k=10 on [2,1024,8000],
     then the MRF of AMP blocks k=(3,7,11) x d=(1,3,5); He weights
  4  full H3-shaped decode: latent [2,32,400] -> [2,320000] at 32 kHz
  5  LTX-shaped vocoder: log-mel [2,64,2000] ~ N(-4,2) -> [2,320000] at 16 kHz
  6  Music-3 DAV decoder: stereo latent [1,128,862] ~ N(0,1) -> interleaved
     [1, 2*441344] at 44.1 kHz (10 s); plain-Snake alphas ~ N(1, 0.01)
  7  LTX bandwidth-extension tail: 16 kHz signal [2,320000] ~ N(0, 0.01)
     -> 48 kHz [2,960000]; STFT basis DFT x Hann (L = 512), slaney mel basis
     (64 mels, 0-8 kHz), BWE generator rates (6,5,2,2,2), c0 = 512, He
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(name: str) -> int:
    h = FNV_OFFSET
    for byte in name.encode("utf-8"):
        h ^= byte
        h = (h * FNV_PRIME) & MASK64
    return h


def master_seed(workload: int) -> int:
    return 0xB1C00000 + int(workload)


def normal(workload: int, name: str, shape: Sequence[int], mean: float = 0.0,
           var: float = 1.0) -> np.ndarray:
    """float32 array of N(mean, var) draws from the tensor's own stream."""
    seed = master_seed(workload) ^ fnv1a64(name)
    rng = np.random.Generator(np.random.PCG64(seed))
    z = rng.standard_normal(size=tuple(int(s) for s in shape), dtype=np.float64)
    return (z * math.sqrt(var) + mean).astype(np.float32)


def he_var(fan_in: int) -> float:
    """He (Kaiming-normal) variance 2/fan_in; fan_in = Cin*k for Conv1d and
    for ConvTranspose1d weights [Cin, Cout, k] alike."""
    return 2.0 / float(fan_in)


# --------------------------------------------------------------------------
# Decoder architecture descriptions (shapes only)
# --------------------------------------------------------------------------

@dataclass
class DecoderSpec:
    name: str
    c_in: int
    c0: int
    rates: Tuple[int, ...]
    up_k: Tuple[int, ...]
    rb_k: Tuple[int, ...] = (3, 7, 11)
    rb_d: Tuple[Tuple[int, ...], ...] = ((1, 3, 5), (1, 3, 5), (1, 3, 5))
    k_pre: int = 7
    k_post: int = 7
    final: str = "tanh"          # 'none' | 'tanh' | 'clamp'
    sample_rate: int = 32000
    latent_affine: bool = False
    dec_in: int = 0              # >0: a 1x1 conv from c_in to this many channels first

    @property
    def hop(self) -> int:
        h = 1
        for r in self.rates:
            h *= r
        return h

    def widths(self) -> List[int]:
        """Channel width entering each stage, then the last width
        (halving per stage, as both pages' decoders do)."""
        w = [self.c0]
        for _ in self.rates:
            w.append(w[-1] // 2)
        return w


H3 = DecoderSpec(name="minimax-h3", c_in=32, c0=1536, rates=(5, 5, 2, 2, 2, 2, 2),
                 up_k=(11, 11, 4, 4, 4, 4, 4), final="tanh", sample_rate=32000)
LTX = DecoderSpec(name="ltx-2.5-vocoder", c_in=64, c0=1024, rates=(5, 2, 2, 2, 2, 2),
                  up_k=(11, 4, 4, 4, 4, 4), final="clamp", sample_rate=16000)


def decoder_tensors(spec: DecoderSpec, workload: int, *, snake_var: float = 0.1,
                    bias_var: float = 0.01, weight_var=None) -> Dict[str, np.ndarray]:
    """All decoder weights by name (the H3 page's naming scheme).
    ``weight_var(fan_in)`` defaults to He."""
    wv = weight_var or he_var
    t: Dict[str, np.ndarray] = {}
    w = spec.widths()
    cin = spec.c_in
    if spec.latent_affine:
        t["latents_mean"] = normal(workload, "latents_mean", [cin], 0.0, 0.01)
        t["latents_std"] = (1.0 + 0.1 * normal(workload, "latents_std", [cin])).astype(np.float32)
    if spec.dec_in:
        t["dec_in.weight"] = normal(workload, "dec_in.weight", [spec.dec_in, cin, 1], 0.0, wv(cin))
        t["dec_in.bias"] = normal(workload, "dec_in.bias", [spec.dec_in], 0.0, bias_var)
        cin = spec.dec_in
    t["conv_pre.weight"] = normal(workload, "conv_pre.weight", [w[0], cin, spec.k_pre], 0.0,
                                  wv(cin * spec.k_pre))
    t["conv_pre.bias"] = normal(workload, "conv_pre.bias", [w[0]], 0.0, bias_var)
    nk = len(spec.rb_k)
    for i, (r, k) in enumerate(zip(spec.rates, spec.up_k)):
        ci, co = w[i], w[i + 1]
        t[f"ups.{i}.weight"] = normal(workload, f"ups.{i}.weight", [ci, co, k], 0.0, wv(ci * k))
        t[f"ups.{i}.bias"] = normal(workload, f"ups.{i}.bias", [co], 0.0, bias_var)
        for j, (kj, dj) in enumerate(zip(spec.rb_k, spec.rb_d)):
            p = f"resblocks.{i * nk + j}"
            for q in range(len(dj)):
                for conv in ("convs1", "convs2"):
                    t[f"{p}.{conv}.{q}.weight"] = normal(workload, f"{p}.{conv}.{q}.weight",
                                                         [co, co, kj], 0.0, wv(co * kj))
                    t[f"{p}.{conv}.{q}.bias"] = normal(workload, f"{p}.{conv}.{q}.bias", [co],
                                                       0.0, bias_var)
            for q in range(2 * len(dj)):
                t[f"{p}.activations.{q}.act.alpha"] = normal(
                    workload, f"{p}.activations.{q}.act.alpha", [co], 0.0, snake_var)
                t[f"{p}.activations.{q}.act.beta"] = normal(
                    workload, f"{p}.activations.{q}.act.beta", [co], 0.0, snake_var)
    cl = w[-1]
    t["activation_post.act.alpha"] = normal(workload, "activation_post.act.alpha", [cl], 0.0, snake_var)
    t["activation_post.act.beta"] = normal(workload, "activation_post.act.beta", [cl], 0.0, snake_var)
    t["conv_post.weight"] = normal(workload, "conv_post.weight", [1, cl, spec.k_post], 0.0,
                                   wv(cl * spec.k_post))
    t["conv_post.bias"] = normal(workload, "conv_post.bias", [1], 0.0, bias_var)
    return t


def amp_tensors(workload: int, prefix: str, c: int, k: int, dil: Sequence[int], *,
                weight_var: float, bias_var: float = 0.01, snake_var: float = 0.1
                ) -> Dict[str, np.ndarray]:
    """Weights of one AMP block (names as in the H3 page)."""
    t: Dict[str, np.ndarray] = {}
    for q in range(len(dil)):
        for conv in ("convs1", "convs2"):
            t[f"{prefix}.{conv}.{q}.weight"] = normal(workload, f"{prefix}.{conv}.{q}.weight",
                                                      [c, c, k], 0.0, weight_var)
            t[f"{prefix}.{conv}.{q}.bias"] = normal(workload, f"{prefix}.{conv}.{q}.bias", [c],
                                                    0.0, bias_var)
    for q in range(2 * len(dil)):
        t[f"{prefix}.activations.{q}.act.alpha"] = normal(
            workload, f"{prefix}.activations.{q}.act.alpha", [c], 0.0, snake_var)
        t[f"{prefix}.activations.{q}.act.beta"] = normal(
            workload, f"{prefix}.activations.{q}.act.beta", [c], 0.0, snake_var)
    return t


@dataclass
class DavSpec:
    """The Music-3 DAV decoder (the H3 page's Music3Dav).  Channel widths are
    not on the page: c0 halves at every stage, like the H3 decoder."""
    name: str = "music3-dav"
    c_side: int = 64             # latent channels per stereo side
    dec_in: int = 64             # 1-tap projection width
    c0: int = 1536
    strides: Tuple[int, ...] = (8, 8, 4, 2)
    unit_k: int = 7
    unit_dil: Tuple[int, ...] = (1, 3, 9)
    k_pre: int = 7
    k_post: int = 7
    sample_rate: int = 44100

    @property
    def up_k(self) -> Tuple[int, ...]:
        return tuple(2 * s for s in self.strides)

    @property
    def hop(self) -> int:
        return int(np.prod(self.strides))

    def widths(self) -> List[int]:
        return [self.c0 // (2 ** i) for i in range(len(self.strides) + 1)]


DAV = DavSpec()


def dav_tensors(spec: DavSpec, workload: int, *, alpha_var: float = 0.01,
                bias_var: float = 0.01) -> Dict[str, np.ndarray]:
    """All DAV decoder weights by the H3 page's names; He weights, Snake
    alphas ~ N(1, alpha_var)."""
    t: Dict[str, np.ndarray] = {}
    w = spec.widths()
    cs, d = spec.c_side, spec.dec_in

    def conv(name, cout, cin, k):
        t[f"{name}.weight"] = normal(workload, f"{name}.weight", [cout, cin, k], 0.0,
                                     he_var(cin * k))
        t[f"{name}.bias"] = normal(workload, f"{name}.bias", [cout], 0.0, bias_var)

    def snake_alpha(name, c):
        t[f"{name}.alpha"] = normal(workload, f"{name}.alpha", [c], 1.0, alpha_var)

    conv("mvae.dec_in_proj", d, cs, 1)
    conv("mvae.decoder.model.0", w[0], d, spec.k_pre)
    for i, (s, k) in enumerate(zip(spec.strides, spec.up_k)):
        p = f"mvae.decoder.model.{i + 1}"
        ci, co = w[i], w[i + 1]
        snake_alpha(f"{p}.block.0", ci)
        t[f"{p}.block.1.weight"] = normal(workload, f"{p}.block.1.weight", [ci, co, k], 0.0,
                                          he_var(ci * k))
        t[f"{p}.block.1.bias"] = normal(workload, f"{p}.block.1.bias", [co], 0.0, bias_var)
        for u in range(len(spec.unit_dil)):
            q = f"{p}.block.{u + 2}"
            snake_alpha(f"{q}.block.0", co)
            conv(f"{q}.block.1", co, co, spec.unit_k)
            snake_alpha(f"{q}.block.2", co)
            conv(f"{q}.block.3", co, co, 1)
    snake_alpha(f"mvae.decoder.model.{len(spec.strides) + 1}", w[-1])
    conv(f"mvae.decoder.model.{len(spec.strides) + 2}", 1, w[-1], spec.k_post)
    return t


def scaled_dav(c0: int, **kw) -> DavSpec:
    d = dict(DAV.__dict__)
    d.update(kw)
    d["c0"] = c0
    d["name"] = f"music3-dav-c{c0}"
    return DavSpec(**d)


# --------------------------------------------------------------------------
# The workloads
# --------------------------------------------------------------------------

def workload1(T: int = 4096, C: int = 32, B: int = 1):
    """Single AMP block: x ~ N(0,1) [B, C, T], k=3, d=(1,3,5), W ~ N(0, 1/(C*3))."""
    x = normal(1, "x", [B, C, T])
    w = amp_tensors(1, "block", C, 3, (1, 3, 5), weight_var=1.0 / (C * 3))
    return x, w


def workload2(T: int = 65536, C: int = 512, B: int = 2):
    """Activation1d alone and one AMP block at production width."""
    x = normal(2, "x", [B, C, T])
    la = normal(2, "act.alpha", [C], 0.0, 0.1)
    lb = normal(2, "act.beta", [C], 0.0, 0.1)
    w = amp_tensors(2, "block", C, 3, (1, 3, 5), weight_var=1.0 / (C * 3))
    return x, la, lb, w


def workload3(T: int = 8000, cin: int = 1024, cout: int = 512, B: int = 2, k_up: int = 10,
              stride: int = 5):
    """ConvTranspose1d cin->cout (k=10, s=5) then the MRF (3,7,11)x(1,3,5), He weights."""
    x = normal(3, "x", [B, cin, T])
    t = {
        "ups.0.weight": normal(3, "ups.0.weight", [cin, cout, k_up], 0.0, he_var(cin * k_up)),
        "ups.0.bias": normal(3, "ups.0.bias", [cout], 0.0, 0.01),
    }
    for j, k in enumerate((3, 7, 11)):
        t.update(amp_tensors(3, f"resblocks.{j}", cout, k, (1, 3, 5), weight_var=he_var(cout * k)))
    return x, t


def workload4(frames: int = 400, B: int = 2, spec: DecoderSpec = H3):
    """Full H3-shaped decode; latent ~ N(0,1) [B, 32, frames]."""
    z = normal(4, "latent", [B, spec.c_in, frames])
    return z, decoder_tensors(spec, 4)


def workload5(frames: int = 2000, B: int = 2, spec: DecoderSpec = LTX):
    """LTX-shaped vocoder; log-mel ~ N(-4, 2) [B, 64, frames]."""
    z = normal(5, "mel", [B, spec.c_in, frames], -4.0, 2.0)
    return z, decoder_tensors(spec, 5)


def scaled_spec(spec: DecoderSpec, c0: int, name: Optional[str] = None, **kw) -> DecoderSpec:
    """Same architecture at a reduced width (for tests that the oracle must
    finish in seconds)."""
    d = dict(spec.__dict__)
    d.update(kw)
    d["c0"] = c0
    d["name"] = name or f"{spec.name}-c{c0}"
    return DecoderSpec(**d)


def workload6(frames: int = 862, B: int = 1, spec: DavSpec = DAV):
    """Music-3 DAV decode: stereo latent ~ N(0,1) [B, 2*64, frames] (10 s)."""
    z = normal(6, "latent", [B, 2 * spec.c_side, frames])
    return z, dav_tensors(spec, 6)


# --------------------------------------------------------------------------
# LTX bandwidth-extension tail (the checkpoint's STFT and mel bases are not
# on the pages: a DFT x Hann basis and a slaney mel basis stand in)
# --------------------------------------------------------------------------

BWE = DecoderSpec(name="ltx-bwe", c_in=64, c0=512, rates=(6, 5, 2, 2, 2),
                  up_k=(12, 11, 4, 4, 4), final="none", sample_rate=48000)
BWE_HOP = 80
BWE_NFFT = 512
BWE_MELS = 64


def stft_basis(n_fft: int) -> np.ndarray:
    """[2 (n_fft/2+1), n_fft]: rows r = cos(2 pi r j / n) w(j), rows n/2+1+r =
    -sin(2 pi r j / n) w(j), w the periodic Hann window (float32)."""
    nf = n_fft // 2 + 1
    j = np.arange(n_fft, dtype=np.float64)
    win = 0.5 - 0.5 * np.cos(2.0 * np.pi * j / n_fft)
    r = np.arange(nf, dtype=np.float64)[:, None]
    ang = 2.0 * np.pi * r * j[None, :] / n_fft
    return np.concatenate([np.cos(ang) * win, -np.sin(ang) * win]).astype(np.float32)


def slaney_mel_basis(sr: float, n_fft: int, n_mels: int, fmin: float, fmax: float) -> np.ndarray:
    """[n_mels, n_fft/2+1] triangular filters on the slaney mel scale with
    unit-area normalisation (float32)."""
    nf = n_fft // 2 + 1
    f_log, m_log, step = 1000.0, 15.0, math.log(6.4) / 27.0

    def hz2mel(f):
        return np.where(f >= f_log, m_log + np.log(np.maximum(f, 1e-9) / f_log) / step, 3.0 * f / 200.0)

    def mel2hz(m):
        return np.where(m >= m_log, f_log * np.exp((m - m_log) * step), m * 200.0 / 3.0)

    m0, m1 = hz2mel(np.array(fmin)), hz2mel(np.array(fmax))
    pts = mel2hz(m0 + (m1 - m0) * np.arange(n_mels + 2) / (n_mels + 1))
    freqs = sr * np.arange(nf) / n_fft
    fb = np.zeros((n_mels, nf))
    for m in range(n_mels):
        lo, c, hi = pts[m], pts[m + 1], pts[m + 2]
        up = (freqs - lo) / max(c - lo, 1e-12)
        dn = (hi - freqs) / max(hi - c, 1e-12)
        fb[m] = np.maximum(0.0, np.minimum(up, dn)) * (2.0 / (hi - lo))
    return fb.astype(np.float32)


def bwe_tensors(workload: int, spec: DecoderSpec = BWE) -> Dict[str, np.ndarray]:
    t = decoder_tensors(spec, workload)
    t["mel_stft.forward_basis"] = stft_basis(BWE_NFFT)
    t["mel_stft.mel_basis"] = slaney_mel_basis(16000.0, BWE_NFFT, BWE_MELS, 0.0, 8000.0)
    return t


def workload7(T: int = 320000, B: int = 2, spec: DecoderSpec = BWE):
    """The bandwidth-extension tail on a 16 kHz signal ~ N(0, 0.01) [B, T]."""
    low = normal(7, "low16k", [B, T], 0.0, 0.01)
    return low, bwe_tensors(7, spec)
