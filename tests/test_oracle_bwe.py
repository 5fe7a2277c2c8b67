"""Pins for the oracle's LTX bandwidth-extension tail ([LTX] page, items
MelStft, hann_sinc_upsample, AudioStack::decode_from_mel), checked against
numpy's FFT, continuous sinusoids and closed-form lengths."""
import math

import numpy as np
import pytest

from bigvgan_waveform_decoder_amd import workloads as W
from oracle import avae_oracle as O
from tests.helpers import decoder_params


def test_mel_stft_matches_numpy_rfft():
    """With an identity mel basis the oracle's frames are ln(max(|rfft(w x)|,
    1e-5)) of the causally framed signal (numpy's FFT, not the basis)."""
    n, hop = 64, 16
    fb = W.stft_basis(n)
    nf = n // 2 + 1
    x = W.normal(7, "stft/x", [2, 200]).astype(np.float64)
    got = O.mel_stft(x, fb, np.eye(nf), hop)
    left = n - hop
    xp = np.concatenate([np.zeros((2, left)), x], axis=1)
    win = 0.5 - 0.5 * np.cos(2 * np.pi * np.arange(n) / n)
    frames = (200 + left - n) // hop + 1
    assert got.shape == (2, nf, frames)
    for f in range(frames):
        seg = xp[:, f * hop: f * hop + n] * win
        ref = np.maximum(np.abs(np.fft.rfft(seg, axis=1)), 1e-5)
        # the basis is float32: compare magnitudes against the frame's scale
        assert np.max(np.abs(np.exp(got[:, :, f]) - ref)) <= 1e-6 * np.max(ref)


def test_mel_stft_causal_framing_and_floor():
    """An impulse at sample s reaches exactly the frames whose window
    [f hop - (L - hop), f hop + hop) covers it; silence is ln(1e-5)."""
    L, hop = 512, 80
    fb = W.stft_basis(L)
    mb = W.slaney_mel_basis(16000.0, L, 64, 0.0, 8000.0)
    x = np.zeros((1, 1600))
    z = O.mel_stft(x, fb, mb, hop)
    assert z.shape == (1, 64, 20) and np.all(z == math.log(1e-5))
    s = 700
    x[0, s] = 1.0
    z = O.mel_stft(x, fb, mb, hop)
    hit = np.nonzero(np.any(z[0] > math.log(1e-5) + 1e-9, axis=0))[0]
    left = L - hop
    expect = [f for f in range(20) if f * hop - left <= s < f * hop - left + L]
    assert hit.tolist() == expect


def test_hann_sinc_filter_shape_and_centre():
    f = O.hann_sinc_filter_f64(3)
    w = math.ceil(6.0 / 0.99)
    assert f.shape == (2 * w * 3 + 1,)
    assert abs(f[w * 3] - 0.99 / 3) < 1e-15
    assert np.allclose(f, f[::-1], rtol=0, atol=1e-15)


def test_hann_sinc_filter_taps_are_float32_like_the_page():
    """[LTX] hann_sinc_upsample builds its taps in float64 and stores them as
    f32: every tap the oracle uses is a float32 value, the nearest one to
    the float64 design (within half a float32 ulp), mirror-symmetric."""
    f64 = O.hann_sinc_filter_f64(3)
    f = O.hann_sinc_filter(3)
    assert np.array_equal(f, f.astype(np.float32).astype(np.float64))
    half_ulp = 0.5 * np.spacing(np.abs(f64).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(f - f64) <= half_ulp)
    assert np.array_equal(f, f[::-1])
    assert f[3 * math.ceil(6.0 / 0.99)] == np.float32(0.99 / 3)


def test_hann_sinc_upsample_interpolates_a_sinusoid():
    """A 700 Hz tone at 16 kHz, upsampled x3, matches the tone sampled at
    48 kHz away from the ends (the interpolator's passband ends near 7.9 kHz)."""
    T = 1600
    t = np.arange(T) / 16000.0
    x = np.sin(2 * np.pi * 700 * t + 0.3)[None]
    y = O.hann_sinc_upsample(x, 3)
    assert y.shape == (1, 3 * T)
    t3 = np.arange(3 * T) / 48000.0
    ref = np.sin(2 * np.pi * 700 * t3 + 0.3)
    mid = slice(300, 3 * T - 300)
    assert np.max(np.abs(y[0, mid] - ref[mid])) < 2e-3


def test_hann_sinc_upsample_constant_and_length():
    """Replicate padding: a constant stays constant (to the filter's DC
    gain, within 1e-3) up to both ends; length is exactly 3 T."""
    for T in (1, 7, 50):
        y = O.hann_sinc_upsample(np.full((1, T), 0.5), 3)
        assert y.shape == (1, 3 * T)
        assert np.max(np.abs(y - 0.5)) < 1e-3


SMALL = W.scaled_spec(W.BWE, 32)


@pytest.mark.parametrize("T", [800, 845])
def test_bwe_tail_with_silent_generator_is_the_clamped_skip(T):
    """A generator with all-zero weights and biases adds nothing: the tail is
    clamp(hann_sinc_upsample(padded)) over 3 T samples."""
    t = W.bwe_tensors(7, SMALL)
    zero = {k: (np.zeros_like(v) if not k.startswith("mel_stft") and "act." not in k else v)
            for k, v in t.items()}
    p = decoder_params(SMALL, zero)
    p.final = "none"
    low = np.clip(W.normal(7, "tail/low", [2, T], 0.0, 0.5), -1, 1).astype(np.float64)
    out = O.bwe_tail(low, t["mel_stft.forward_basis"], t["mel_stft.mel_basis"], 80, p)
    assert out.shape == (2, 3 * T)
    pad = (-T) % 80
    padded = np.concatenate([low, np.zeros((2, pad))], axis=1)
    skip = O.hann_sinc_upsample(padded, 3)[:, :3 * T]
    assert np.array_equal(out, np.clip(skip, -1, 1))


def test_bwe_generator_geometry():
    """Mel frames at hop 80 through rates (6,5,2,2,2) give 240 samples a
    frame: three 48 kHz samples per 16 kHz sample of the padded signal."""
    assert int(np.prod(W.BWE.rates)) == 3 * 80
    t = W.bwe_tensors(7, SMALL)
    p = decoder_params(SMALL, t)
    p.final = "none"
    m = np.zeros((1, 64, 4))
    assert O.decode(m, p).shape == (1, 4 * 240)
