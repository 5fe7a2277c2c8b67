"""Plain, slow, float64 CPU oracle for the alias-free BigVGAN decoder.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP library (different language,
different filter designer, different loops) and imports nothing from the
package next to it.

Every function takes float arrays (normally float32 values promoted to
float64) and computes in float64 throughout, with no intermediate float32
rounding, by the plain definition the pages give.  Library primitives serve
as single steps (a matrix product per convolution tap); there is no tiling,
fusion or reordering beyond the definitions.

Sources (cited by page and item, never by line):
  [H3]  docs.rs source page of ``cortiq_engine/audiovae.rs`` (cortiq-engine
        0.5.74) -- MiniMax-H3 audio VAE decoder, the authority.
  [LTX] docs.rs source page of ``cortiq_engine/ltxaudio.rs`` (cortiq-engine
        0.6.3) -- LTX-2.5 BigVGAN v2 vocoder, second source.
  The [H3] page also holds the MiniMax-Music-3 DAV decoder (items Snake,
  DavUnit, DavStage, Music3Dav); the [LTX] page the bandwidth-extension tail
  (items MelStft, hann_sinc_upsample, AudioStack::decode_from_mel).  Both
  are sections at the end of this module.

Readings taken where the pages are silent or disagree are listed in the
function docstrings (and in the design notes of the repository).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

FILTER_LEN = 12  # [H3] constant FILTER_LEN: both resampling filters have 12 taps


# --------------------------------------------------------------------------
# Filter design  ([H3] bessel_i0, sinc, kaiser_sinc)
# --------------------------------------------------------------------------

def bessel_i0(x: float) -> float:
    """Modified Bessel function of the first kind, order 0 ([H3] ``bessel_i0``
    sums its power series; here numpy's ``np.i0`` is the library step)."""
    return float(np.i0(float(x)))


def kaiser_params(half_width: float, k: int) -> Tuple[float, float]:
    """Stop-band attenuation A (dB) and Kaiser's beta for the design of
    [H3] ``kaiser_sinc``.

    The page estimates A with Kaiser's length rule for a filter of k/2 taps
    and transition width 4 half_width (in units of pi): A = 2.285 (k/2 - 1)
    pi (4 half_width) + 7.95.  beta follows Kaiser's empirical formula:
    0.1102 (A - 8.7) above 50 dB, 0.5842 (A - 21)^0.4 + 0.07886 (A - 21) from
    21 to 50 dB, and 0 (a rectangular window) below.
    """
    atten = 2.285 * (k // 2 - 1) * math.pi * (4.0 * half_width) + 7.95
    if atten > 50.0:
        return atten, 0.1102 * (atten - 8.7)
    if atten >= 21.0:
        return atten, 0.5842 * (atten - 21.0) ** 0.4 + 0.07886 * (atten - 21.0)
    return atten, 0.0


def kaiser_sinc_f64(cutoff: float, half_width: float, k: int) -> np.ndarray:
    """Kaiser-windowed sinc lowpass, unit sum, unrounded float64 ([H3] ``kaiser_sinc``).

    The ideal lowpass impulse response 2 cutoff sinc(2 cutoff t) (cutoff in
    cycles per sample, normalised sinc) is sampled at the k tap positions
    t = i - (k - 1)/2 (half-integers for even k), multiplied by the Kaiser
    window I0(beta sqrt(1 - (2t/(k-1))^2)) / I0(beta), and scaled to unit sum.
    """
    _, beta = kaiser_params(half_width, k)
    pos = np.arange(k, dtype=np.float64) - (k - 1) / 2.0
    rel = 2.0 * pos / (k - 1)
    window = np.i0(beta * np.sqrt(np.clip(1.0 - rel * rel, 0.0, None))) / np.i0(beta)
    h = 2.0 * cutoff * np.sinc(2.0 * cutoff * pos) * window
    return h / h.sum()


def kaiser_sinc(cutoff: float = 0.25, half_width: float = 0.3, k: int = FILTER_LEN) -> np.ndarray:
    """The designed taps as the model stores them: float64 design rounded to
    float32 ([H3] ``kaiser_sinc`` ends with a cast to f32).  Returned as float64
    holding float32 values."""
    return kaiser_sinc_f64(cutoff, half_width, k).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Activation1d  ([H3] Activation1d::apply, fir_pad, SnakeBeta;
#                [LTX] Aliasing::upsample / downsample, SnakeBeta::forward)
# --------------------------------------------------------------------------

def _clamp_index(n_out: int, shift: int, n: int) -> np.ndarray:
    return np.clip(np.arange(n_out) - shift, 0, n - 1)


def upsample2(x: np.ndarray, up: np.ndarray, ratio: int = 2) -> np.ndarray:
    """Anti-aliased x2 upsample over the last axis ([LTX] ``Aliasing::upsample``,
    [H3] first half of ``Activation1d::apply``).

    pad = K/ratio - 1 replicate samples each side; transposed convolution with
    the filter at stride ``ratio`` and gain ``ratio``:
    u[ratio*i + j] += ratio * xp[i] * up[j]; then trim
    pad*ratio + (K-ratio)//2 on the left and pad*ratio + ceil((K-ratio)/2) on
    the right, leaving ratio*T samples.
    """
    x = np.asarray(x, dtype=np.float64)
    up = np.asarray(up, dtype=np.float64)
    k = up.shape[0]
    n = x.shape[-1]
    pad = k // ratio - 1
    pad_l = pad * ratio + (k - ratio) // 2
    pad_r = pad * ratio + (k - ratio + 1) // 2
    tp = n + 2 * pad
    xp = x[..., _clamp_index(tp, pad, n)]
    full = (tp - 1) * ratio + k
    u = np.zeros(x.shape[:-1] + (full,), dtype=np.float64)
    for j in range(k):
        # positions ratio*i + j for i in [0, tp)
        u[..., j: j + ratio * (tp - 1) + 1: ratio] += ratio * xp * up[j]
    return u[..., pad_l: full - pad_r]


def snake_beta(v: np.ndarray, log_alpha: np.ndarray, log_beta: np.ndarray) -> np.ndarray:
    """SnakeBeta with log-scale parameters ([H3] ``SnakeBeta``, [LTX] ``SnakeBeta::forward``):
    v + sin(exp(a_c) v)^2 / (exp(b_c) + 1e-9), channel c on axis -2."""
    v = np.asarray(v, dtype=np.float64)
    a = np.exp(np.asarray(log_alpha, dtype=np.float64))[:, None]
    b = np.exp(np.asarray(log_beta, dtype=np.float64))[:, None]
    s = np.sin(a * v)
    return v + s * s / (b + 1e-9)


def downsample2(m: np.ndarray, down: np.ndarray, ratio: int = 2) -> np.ndarray:
    """Lowpass x2 downsample over the last axis ([H3] ``fir_pad`` as called by
    ``Activation1d::apply``, [LTX] ``Aliasing::downsample``).

    Replicate-pad K/2 - 1 on the left (even K) and K/2 on the right, then the
    FIR at stride ``ratio``: y[t] = sum_j down[j] * buf[ratio*t + j], with
    (n + pad_l + pad_r - K)/ratio + 1 outputs.
    """
    m = np.asarray(m, dtype=np.float64)
    down = np.asarray(down, dtype=np.float64)
    k = down.shape[0]
    n = m.shape[-1]
    pad_l = k // 2 - (1 if k % 2 == 0 else 0)
    pad_r = k // 2
    padded = n + pad_l + pad_r
    buf = m[..., _clamp_index(padded, pad_l, n)]
    out_n = (padded - k) // ratio + 1
    y = np.zeros(m.shape[:-1] + (out_n,), dtype=np.float64)
    for j in range(k):
        y += down[j] * buf[..., j: j + ratio * (out_n - 1) + 1: ratio]
    return y


def act1d(x: np.ndarray, log_alpha, log_beta, up=None, down=None) -> np.ndarray:
    """Alias-free activation, ``[..., C, T] -> [..., C, T]`` ([H3] ``Activation1d::apply``):
    upsample x2, SnakeBeta at the doubled rate, lowpass-downsample x2.
    ``up``/``down`` default to the designed taps ([H3] ``Activation1d::load``
    falls back to ``kaiser_sinc(0.25, 0.3, 12)`` for both)."""
    if up is None:
        up = kaiser_sinc()
    if down is None:
        down = kaiser_sinc()
    mid = upsample2(x, up)
    mid = snake_beta(mid, log_alpha, log_beta)
    return downsample2(mid, down)


# --------------------------------------------------------------------------
# Convolutions  ([H3] Conv1d::apply, ConvT1d::apply; [LTX] Conv1d, ConvT1d)
# --------------------------------------------------------------------------

def conv1d(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None, dilation: int = 1,
           pad: Optional[int] = None, residual: Optional[np.ndarray] = None) -> np.ndarray:
    """Dilated correlation with zero padding ([H3] ``Conv1d::apply``).

    x ``[B, Cin, n]``, w ``[Cout, Cin, k]``; out length n + 2 pad - d (k - 1);
    y[o, t] = b[o] + sum_i sum_j w[o, i, j] x[i, t + j d - pad] (zero outside).
    ``pad`` defaults to the "same" padding (k d - d) / 2 ([H3] ``get_padding``).
    ``residual`` (same shape as y) is added afterwards: the AMP residual
    ``cur += xt`` of [H3] ``AmpBlock::apply``.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    cout, cin, k = w.shape
    assert x.shape[-2] == cin
    n = x.shape[-1]
    if pad is None:
        pad = (k * dilation - dilation) // 2
    out_n = n + 2 * pad - dilation * (k - 1)
    assert out_n >= 0
    xp = np.zeros(x.shape[:-1] + (n + 2 * pad,), dtype=np.float64)
    xp[..., pad: pad + n] = x
    y = np.zeros(x.shape[:-2] + (cout, out_n), dtype=np.float64)
    for j in range(k):
        # tap j reads x[i, t + j d - pad] = xp[i, t + j d]
        # (contiguous operands keep numpy's matmul on BLAS)
        wj = np.ascontiguousarray(w[:, :, j])
        xj = np.ascontiguousarray(xp[..., j * dilation: j * dilation + out_n])
        y += np.matmul(wj, xj)
    if b is not None:
        y += np.asarray(b, dtype=np.float64)[:, None]
    if residual is not None:
        y += np.asarray(residual, dtype=np.float64)
    return y


def convtr1d(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray], stride: int,
             pad: Optional[int] = None) -> np.ndarray:
    """Transposed convolution by scatter and crop ([H3] ``ConvT1d::apply``).

    x ``[B, Cin, n]``, w ``[Cin, Cout, k]``; pad defaults to (k - stride) // 2
    ([H3] ``ConvT1d::load``); out length (n - 1) stride + k - 2 pad;
    out[o, t stride + j - pad] += x[i, t] w[i, o, j], plus b[o].
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    cin, cout, k = w.shape
    assert x.shape[-2] == cin
    n = x.shape[-1]
    if pad is None:
        pad = (k - stride) // 2
    full = (n - 1) * stride + k
    out_n = full - 2 * pad
    buf = np.zeros(x.shape[:-2] + (cout, full), dtype=np.float64)
    for j in range(k):
        # input t lands at t*stride + j
        buf[..., j: j + stride * (n - 1) + 1: stride] += np.matmul(
            np.ascontiguousarray(w[:, :, j].T), np.ascontiguousarray(x))
    y = buf[..., pad: pad + out_n].copy()
    if b is not None:
        y += np.asarray(b, dtype=np.float64)[:, None]
    return y


# --------------------------------------------------------------------------
# AMP block, MRF, decoder  ([H3] AmpBlock::apply, AudioVae::decode;
#                           [LTX] AmpBlock::forward, Vocoder::forward)
# --------------------------------------------------------------------------

@dataclass
class AmpParams:
    """One AMP residual block with kernel size k and dilations ``dil``.
    w1[q], b1[q]: convs1 (dilation dil[q]); w2[q], b2[q]: convs2 (dilation 1);
    la[q], lb[q] for q < 2 len(dil): activation q's log alpha / log beta."""
    k: int
    dil: Sequence[int]
    w1: List[np.ndarray]
    b1: List[Optional[np.ndarray]]
    w2: List[np.ndarray]
    b2: List[Optional[np.ndarray]]
    la: List[np.ndarray]
    lb: List[np.ndarray]


def amp_block(x: np.ndarray, p: AmpParams, up=None, down=None) -> np.ndarray:
    """[H3] ``AmpBlock::apply``: for each dilation q,
    cur += conv2_q(act_{2q+1}(conv1_q(act_{2q}(cur))))."""
    cur = np.asarray(x, dtype=np.float64)
    for q, d in enumerate(p.dil):
        xt = act1d(cur, p.la[2 * q], p.lb[2 * q], up, down)
        xt = conv1d(xt, p.w1[q], p.b1[q], dilation=d, pad=(p.k * d - d) // 2)
        xt = act1d(xt, p.la[2 * q + 1], p.lb[2 * q + 1], up, down)
        cur = conv1d(xt, p.w2[q], p.b2[q], dilation=1, pad=(p.k - 1) // 2, residual=cur)
    return cur


def mrf(x: np.ndarray, blocks: Sequence[AmpParams], up=None, down=None) -> np.ndarray:
    """Multi-receptive-field fusion ([H3] ``AudioVae::decode`` stage loop):
    the AMP blocks of a stage all read the same input and their outputs are
    summed, then divided by the number of blocks."""
    acc = None
    for p in blocks:
        r = amp_block(x, p, up, down)
        acc = r if acc is None else acc + r
    return acc / len(blocks)


@dataclass
class DecoderParams:
    """Weights of a BigVGAN decoder.  ``final`` is 'none', 'tanh' or 'clamp'."""
    conv_pre_w: np.ndarray                 # [C0, Cin, k_pre]
    conv_pre_b: Optional[np.ndarray]
    up_w: List[np.ndarray]                 # stage i: [C_i, C_{i+1}, k_i]
    up_b: List[Optional[np.ndarray]]
    rates: Sequence[int]
    blocks: List[List[AmpParams]]          # [stage][kernel]
    post_la: np.ndarray
    post_lb: np.ndarray
    conv_post_w: np.ndarray                # [1, C_last, k_post]
    conv_post_b: Optional[np.ndarray]
    final: str = "tanh"
    latent_mean: Optional[np.ndarray] = None
    latent_std: Optional[np.ndarray] = None
    dec_in_w: Optional[np.ndarray] = None  # [Cin', Cin, 1]
    dec_in_b: Optional[np.ndarray] = None
    stages: List[np.ndarray] = field(default_factory=list)  # filled by decode(record=True)


def decode(latent: np.ndarray, p: DecoderParams, up=None, down=None,
           record: bool = False) -> np.ndarray:
    """One BigVGAN decode ([H3] ``AudioVae::decode``, [LTX] ``Vocoder::forward``).

    latent ``[B, Cin, F]``; each of the B rows is an independent mono pass
    (the stereo channels of [H3] are two such passes).  Steps: optional
    latent affine z*std + mean and optional 1x1 ``dec_in`` conv; ``conv_pre``
    ("same" padding); per stage a transposed conv at the stage's rate
    followed by the MRF average; ``act_post``; ``conv_post``; the final
    nonlinearity (tanh, clamp to [-1, 1], or none).
    With ``record`` the per-stage outputs and the pre-final conv_post output
    are kept in ``p.stages`` for stage-by-stage comparison.
    """
    x = np.asarray(latent, dtype=np.float64)
    if p.latent_std is not None:
        x = x * np.asarray(p.latent_std, np.float64)[:, None]
    if p.latent_mean is not None:
        x = x + np.asarray(p.latent_mean, np.float64)[:, None]
    if p.dec_in_w is not None:
        x = conv1d(x, p.dec_in_w, p.dec_in_b, dilation=1, pad=0)
    kp = p.conv_pre_w.shape[2]
    x = conv1d(x, p.conv_pre_w, p.conv_pre_b, dilation=1, pad=(kp - 1) // 2)
    if record:
        p.stages = [x]
    for i, r in enumerate(p.rates):
        x = convtr1d(x, p.up_w[i], p.up_b[i], stride=r)
        x = mrf(x, p.blocks[i], up, down)
        if record:
            p.stages.append(x)
    x = act1d(x, p.post_la, p.post_lb, up, down)
    kq = p.conv_post_w.shape[2]
    y = conv1d(x, p.conv_post_w, p.conv_post_b, dilation=1, pad=(kq - 1) // 2)
    if record:
        p.stages.append(y)
    if p.final == "tanh":
        y = np.tanh(y)
    elif p.final == "clamp":
        y = np.clip(y, -1.0, 1.0)
    elif p.final != "none":
        raise ValueError(p.final)
    return y[..., 0, :]


# --------------------------------------------------------------------------
# Music-3 DAV decoder  ([H3] page, items Snake, DavUnit, DavStage, Music3Dav)
# --------------------------------------------------------------------------

DAV_STRIDES = (8, 8, 4, 2)   # [H3] Music3Dav::STRIDES
DAV_HOP = 512                # [H3] Music3Dav::HOP = 8 * 8 * 4 * 2
DAV_UNIT_DILATIONS = (1, 3, 9)  # [H3] DavStage::load


def snake(x: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """Plain Snake ([H3] ``Snake::apply``), per channel c of ``[..., C, T]``:
    x + sin^2(alpha_c x) / (alpha_c + 1e-9), alpha used as stored (no
    exponential, unlike SnakeBeta)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.asarray(alpha, dtype=np.float64)[:, None]
    return x + np.sin(a * x) ** 2 / (a + 1e-9)


@dataclass
class DavUnitParams:
    """One residual unit: a1, c1 (k taps at ``dilation``, "same" padding
    (k-1)/2 * dilation), a2, c2 (1 tap)."""
    dilation: int
    a1: np.ndarray
    w1: np.ndarray            # [C, C, k]
    b1: Optional[np.ndarray]
    a2: np.ndarray
    w2: np.ndarray            # [C, C, 1]
    b2: Optional[np.ndarray]


def dav_unit(x: np.ndarray, p: DavUnitParams) -> np.ndarray:
    """[H3] ``DavUnit::apply``: x + c2(snake(c1(snake(x, a1)), a2)).  The page
    loads c1 with padding 3 * dilation for its 7 taps, i.e. "same"."""
    k = p.w1.shape[2]
    h = snake(x, p.a1)
    h = conv1d(h, p.w1, p.b1, dilation=p.dilation, pad=(k - 1) // 2 * p.dilation)
    h = snake(h, p.a2)
    return conv1d(h, p.w2, p.b2, dilation=1, pad=0, residual=x)


@dataclass
class DavStageParams:
    """Snake (alpha over the stage's input channels), a transposed conv at
    ``stride`` (weight [Cin, Cout, k], padding (k - stride) // 2 as in
    [H3] ``ConvT1d::load``), then the residual units in order."""
    stride: int
    alpha: np.ndarray
    up_w: np.ndarray
    up_b: Optional[np.ndarray]
    units: List[DavUnitParams]


def dav_stage(x: np.ndarray, p: DavStageParams) -> np.ndarray:
    """[H3] ``DavStage::apply``."""
    h = snake(x, p.alpha)
    h = convtr1d(h, p.up_w, p.up_b, stride=p.stride)
    for u in p.units:
        h = dav_unit(h, u)
    return h


@dataclass
class DavParams:
    """Weights of the DAV decoder.  dec_in is the 1-tap input projection of
    one side's latent, conv_pre and conv_post use "same" padding."""
    dec_in_w: np.ndarray      # [D, C_side, 1]
    dec_in_b: Optional[np.ndarray]
    conv_pre_w: np.ndarray    # [C0, D, k]
    conv_pre_b: Optional[np.ndarray]
    stages: List[DavStageParams]
    post_alpha: np.ndarray
    conv_post_w: np.ndarray   # [1, C_last, k]
    conv_post_b: Optional[np.ndarray]
    trace: List[np.ndarray] = field(default_factory=list)  # filled by dav_decode(record=True)


def dav_decode(latent: np.ndarray, p: DavParams, record: bool = False) -> np.ndarray:
    """[H3] ``Music3Dav::decode``: latent ``[B, 2 C_side, F]`` -> interleaved
    stereo ``[B, 2 F hop]``.

    The latent channels are a stereo pair: channels [0, C_side) are the left
    side and [C_side, 2 C_side) the right, each decoded as an independent mono
    pass: dec_in, conv_pre, the stages, Snake, conv_post, tanh.  The result
    interleaves the sides sample by sample: out[b, 2 i + side].  With
    ``record`` the per-stage outputs (conv_pre, each stage) and the
    pre-tanh conv_post output of the ``[2 B, ...]`` side batch are kept in
    ``p.trace``.
    """
    z = np.asarray(latent, dtype=np.float64)
    B, C2, F = z.shape
    cs = p.dec_in_w.shape[1]
    assert C2 == 2 * cs, "the latent is a stereo pair of sides"
    x = z.reshape(B * 2, cs, F)          # row 2 b + side
    x = conv1d(x, p.dec_in_w, p.dec_in_b, dilation=1, pad=0)
    kp = p.conv_pre_w.shape[2]
    x = conv1d(x, p.conv_pre_w, p.conv_pre_b, dilation=1, pad=(kp - 1) // 2)
    if record:
        p.trace = [x]
    for st in p.stages:
        x = dav_stage(x, st)
        if record:
            p.trace.append(x)
    x = snake(x, p.post_alpha)
    kq = p.conv_post_w.shape[2]
    y = conv1d(x, p.conv_post_w, p.conv_post_b, dilation=1, pad=(kq - 1) // 2)[:, 0, :]
    if record:
        p.trace.append(y)
    y = np.tanh(y)
    L = y.shape[-1]
    out = np.empty((B, 2 * L), dtype=np.float64)
    out[:, 0::2] = y[0::2]
    out[:, 1::2] = y[1::2]
    return out


# --------------------------------------------------------------------------
# LTX bandwidth-extension tail  ([LTX] MelStft, hann_sinc_upsample,
#                               AudioStack::decode_from_mel)
# --------------------------------------------------------------------------

def mel_stft(x: np.ndarray, forward_basis: np.ndarray, mel_basis: np.ndarray,
             hop: int) -> np.ndarray:
    """[LTX] ``MelStft::forward``: causal log-mel of ``x [B, T]`` ->
    ``[B, n_mels, frames]`` (mel-major, the layout the generator reads).

    forward_basis ``[2 n_freqs, L]`` (rows r: real part, rows n_freqs + r:
    imaginary part), mel_basis ``[n_mels, n_freqs]``.  The signal is padded
    with L - hop zeros on the left (causal) and none on the right; frame f
    starts at f hop of the padded signal; frames = (T + L - hop - L) // hop + 1.
    Each frame: magnitude sqrt(re^2 + im^2) per frequency, the mel
    projection, then ln(max(., 1e-5)).
    """
    x = np.asarray(x, dtype=np.float64)
    fb = np.asarray(forward_basis, dtype=np.float64)
    mb = np.asarray(mel_basis, dtype=np.float64)
    nf2, L = fb.shape
    nf = nf2 // 2
    left = max(L - hop, 0)
    B, T = x.shape
    padded = T + left
    frames = (padded - L) // hop + 1 if padded >= L else 0
    xp = np.concatenate([np.zeros((B, left)), x], axis=1)
    out = np.empty((B, mb.shape[0], frames))
    for f in range(frames):
        seg = xp[:, f * hop: f * hop + L]            # [B, L]
        z = seg @ fb.T                               # [B, 2 nf]
        mag = np.sqrt(z[:, :nf] ** 2 + z[:, nf:] ** 2)
        out[:, :, f] = np.log(np.maximum(mag @ mb.T, 1e-5))
    return out


def hann_sinc_filter_f64(ratio: int, rolloff: float = 0.99, lpw: float = 6.0) -> np.ndarray:
    """The x``ratio`` Hann-windowed sinc interpolator of [LTX]
    ``hann_sinc_upsample``, unrounded float64: k = 2 w ratio + 1 taps,
    w = ceil(lpw / rolloff); tap i at t = (i / ratio - w) * rolloff:
    sinc(t) cos^2(pi clamp(t) / (2 lpw)) * rolloff / ratio."""
    w = math.ceil(lpw / rolloff)
    k = 2 * w * ratio + 1
    i = np.arange(k, dtype=np.float64)
    ta = (i / ratio - w) * rolloff
    tc = np.clip(ta, -lpw, lpw)
    win = np.cos(tc * math.pi / lpw / 2.0) ** 2
    s = np.where(ta == 0.0, 1.0, np.sin(math.pi * ta) / np.where(ta == 0.0, 1.0, math.pi * ta))
    return s * win * rolloff / ratio


def hann_sinc_filter(ratio: int, rolloff: float = 0.99, lpw: float = 6.0) -> np.ndarray:
    """The interpolator's taps as [LTX] ``hann_sinc_upsample`` uses them:
    designed in float64, then cast to float32 (returned as float64 holding
    float32 values), like ``kaiser_sinc``."""
    return hann_sinc_filter_f64(ratio, rolloff, lpw).astype(np.float32).astype(np.float64)


def hann_sinc_upsample(x: np.ndarray, ratio: int, filt: Optional[np.ndarray] = None) -> np.ndarray:
    """[LTX] ``hann_sinc_upsample``: ``x [B, T]`` -> ``[B, ratio T]``.
    Replicate-pad w samples each side, scale by ``ratio``, transposed FIR
    with the filter at stride ``ratio``, keep [2 w ratio, full - (k - ratio))."""
    x = np.asarray(x, dtype=np.float64)
    if filt is None:
        filt = hann_sinc_filter(ratio)
    filt = np.asarray(filt, dtype=np.float64)
    k = filt.shape[0]
    w = (k - 1) // (2 * ratio)
    B, T = x.shape
    idx = np.clip(np.arange(-w, T + w), 0, T - 1)
    xp = x[:, idx] * ratio
    tp = T + 2 * w
    full = (tp - 1) * ratio + k
    acc = np.zeros((B, full))
    for a in range(k):
        acc[:, a: a + ratio * (tp - 1) + 1: ratio] += xp * filt[a]
    lo, hi = 2 * w * ratio, full - (k - ratio)
    return acc[:, lo:hi]


def bwe_tail(low: np.ndarray, forward_basis: np.ndarray, mel_basis: np.ndarray, hop: int,
             bwe: DecoderParams, ratio: int = 3, skip_filter: Optional[np.ndarray] = None
             ) -> np.ndarray:
    """[LTX] ``AudioStack::decode_from_mel`` after the first vocoder: the
    16 kHz ``low [B, T]`` is zero-padded to whole hops, its causal log-mel
    drives the bandwidth-extension generator (a BigVGAN whose output is a
    residual, no final nonlinearity), the padded signal is upsampled x``ratio``
    by the Hann-sinc interpolator, and the sum is clamped to [-1, 1] over
    min(len(residual), len(skip), ratio T) samples."""
    low = np.asarray(low, dtype=np.float64)
    B, T = low.shape
    rem = T % hop
    padded = low if rem == 0 else np.concatenate([low, np.zeros((B, hop - rem))], axis=1)
    m = mel_stft(padded, forward_basis, mel_basis, hop)
    residual = decode(m, bwe)
    skip = hann_sinc_upsample(padded, ratio, skip_filter)
    t = min(residual.shape[-1], skip.shape[-1], T * ratio)
    return np.clip(residual[:, :t] + skip[:, :t], -1.0, 1.0)
