"""Pins for the float64 oracle: each test ties it to something other than
itself -- values the pages print, library routines that compute the same
quantity by another route, closed forms and invariants of the mathematics.

[H3]  = docs.rs source page of cortiq_engine/audiovae.rs (cortiq-engine 0.5.74)
[LTX] = docs.rs source page of cortiq_engine/ltxaudio.rs (cortiq-engine 0.6.3)
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch
import torch.nn.functional as F

from oracle import avae_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")
PAGE = json.load(open(GOLDEN))

RNG = np.random.default_rng(1234)


# ----------------------------------------------------------------- filter design

def test_bessel_i0_page_values():
    """[H3] test bessel_i0_matches_known_values (values in tests/golden)."""
    g = PAGE["bessel_i0"]
    for x, want in g["values"]:
        got = O.bessel_i0(x)
        assert abs(got - want) < g["rel_tol"] * max(want, 1.0), (x, got, want)


def test_bessel_i0_matches_scipy():
    """Library routine: scipy.special.i0 over the range the design uses."""
    for x in np.linspace(0.0, 8.0, 81):
        assert O.bessel_i0(float(x)) == pytest.approx(float(scipy.special.i0(x)), rel=1e-14)


def test_taps_page_invariants():
    """[H3] test the_resampling_filter_is_the_references (tests/golden)."""
    g = PAGE["filter"]
    f = O.kaiser_sinc(g["cutoff"], g["half_width"], g["len"]).astype(np.float32)
    assert f.shape == (g["len"],)
    assert abs(float(f.sum(dtype=np.float32)) - 1.0) < g["sum_tol"]
    for i in range(g["len"] // 2):
        assert abs(f[i] - f[g["len"] - 1 - i]) < g["sym_tol"]
    assert abs(f[g["peak_index"]] - f.max()) < 1e-6


def test_kaiser_beta_matches_scipy_design_formulas():
    """Kaiser's attenuation and beta formulas as scipy implements them:
    A = kaiser_atten(numtaps=k/2, width=4*half_width), beta = kaiser_beta(A)."""
    a, beta = O.kaiser_params(0.3, 12)
    assert a == pytest.approx(scipy.signal.kaiser_atten(6, 1.2), rel=1e-15)
    assert beta == pytest.approx(scipy.signal.kaiser_beta(a), rel=1e-15)
    assert a > 50.0  # the high-attenuation branch is the one taken
    assert beta == pytest.approx(4.663800, abs=5e-7)


def test_taps_match_scipy_firwin():
    """Library routine: a 12-tap Kaiser-window lowpass at cutoff 0.25 cycles
    per sample (0.5 of Nyquist), scaled to unit DC gain, is scipy's firwin."""
    _, beta = O.kaiser_params(0.3, 12)
    ref = scipy.signal.firwin(12, 0.5, window=("kaiser", beta), scale=True)
    np.testing.assert_allclose(O.kaiser_sinc_f64(0.25, 0.3, 12), ref, rtol=0, atol=1e-15)


def test_window_is_numpy_kaiser():
    """The window inside the design is numpy's Kaiser window: dividing the
    taps by the plain sinc recovers np.kaiser(12, beta) up to one scale."""
    _, beta = O.kaiser_params(0.3, 12)
    t = np.arange(12) - 5.5
    raw = O.kaiser_sinc_f64(0.25, 0.3, 12) / (0.5 * np.sinc(0.5 * t))
    win = np.kaiser(12, beta)
    np.testing.assert_allclose(raw / raw.max(), win / win.max(), rtol=1e-13)


def test_polyphase_halves_each_sum_to_half():
    """Symmetric even-length taps: the even- and odd-index taps are mirror
    images, so each half sums to exactly 1/2.  This is why a constant passes
    the x2 upsampler (gain 2 per phase) unchanged."""
    h = O.kaiser_sinc_f64(0.25, 0.3, 12)
    assert h[0::2].sum() == pytest.approx(0.5, abs=1e-15)
    assert h[1::2].sum() == pytest.approx(0.5, abs=1e-15)


# ----------------------------------------------------------------- Activation1d

def _snake_closed_form(c, la, lb):
    return c + np.sin(np.exp(la) * c) ** 2 / (np.exp(lb) + 1e-9)


@pytest.mark.parametrize("T", [1, 2, 5, 11, 64])
def test_act1d_constant_closed_form_everywhere(T):
    """A constant row c maps to the SnakeBeta of c at every sample, the
    replicate-padded edges included (unit-sum filters, x2 gain per phase)."""
    h = O.kaiser_sinc_f64(0.25, 0.3, 12)
    C = 4
    c = np.array([0.3, -1.7, 2.5, 40.0])
    la = np.array([0.1, -0.2, 0.3, 0.0])
    lb = np.array([-0.1, 0.25, 0.0, 0.5])
    x = np.repeat(c[:, None], T, axis=1)
    y = O.act1d(x, la, lb, h, h)
    assert y.shape == (C, T)
    want = _snake_closed_form(c, la, lb)[:, None]
    np.testing.assert_allclose(y, np.broadcast_to(want, y.shape), rtol=0, atol=1e-13)


@pytest.mark.parametrize("T", [1, 2, 3, 5, 11, 100, 4096])
def test_act1d_length_preserving(T):
    x = RNG.standard_normal((3, T))
    y = O.act1d(x, np.zeros(3), np.zeros(3))
    assert y.shape == (3, T)


def test_act1d_interior_is_textbook_multirate_chain():
    """Away from the edges the operator is: zero-stuff by 2, convolve with
    2*up, SnakeBeta pointwise, convolve with down, keep every other sample.
    With two symmetric 12-tap filters the group delays add to 11 samples at
    the doubled rate, so y[t] = w[2t + 11] (np.convolve, full mode)."""
    h = O.kaiser_sinc_f64(0.25, 0.3, 12)
    T = 300
    x = RNG.standard_normal(T) * 2.0
    la, lb = 0.37, -0.21
    y = O.act1d(x[None, :], np.array([la]), np.array([lb]), h, h)[0]
    z = np.zeros(2 * T)
    z[0::2] = x
    u = np.convolve(z, 2.0 * h)
    u = u + np.sin(np.exp(la) * u) ** 2 / (np.exp(lb) + 1e-9)
    w = np.convolve(u, h)
    ref = w[2 * np.arange(T) + 11]
    inner = slice(8, T - 8)  # the edges see replicate padding instead
    np.testing.assert_allclose(y[inner], ref[inner], rtol=0, atol=1e-12)


@pytest.mark.parametrize("f", [0.01, 0.05, 0.12])
def test_act1d_linear_limit_sinusoid_response(f):
    """With log beta = 60 the snake term is ~1e-26 and the operator is LTI.
    A sinusoid at f cycles/sample comes out scaled by
    A(f) = sum_{k=0,1} H(f/2 + k/2)^2 exp(2 pi i (f/2 + k/2) 11),
    H the DTFT of the taps (derivation: zero-stuffing splits the input into
    the baseband and its image, both filtered twice, decimation folds them
    back).  A low-frequency sinusoid survives upsample-then-downsample."""
    h = O.kaiser_sinc_f64(0.25, 0.3, 12)
    j = np.arange(12)

    def H(nu):
        return np.sum(h * np.exp(-2j * np.pi * nu * j))

    A = sum(H(f / 2 + k / 2) ** 2 * np.exp(2j * np.pi * (f / 2 + k / 2) * 11) for k in (0, 1))
    assert abs(A.imag) < 1e-12
    T = 2000
    t = np.arange(T)
    x = np.cos(2 * np.pi * f * t + 0.3)
    y = O.act1d(x[None, :], np.zeros(1), np.array([60.0]), h, h)[0]
    inner = slice(20, T - 20)
    np.testing.assert_allclose(y[inner], A.real * x[inner], rtol=0, atol=1e-12)
    if f <= 0.01:
        assert np.max(np.abs(y[inner] - x[inner])) < 1e-4


def test_act1d_commutes_with_time_reversal():
    """Symmetric taps and the pages' pad/trim amounts (up: 5 and 5, trim
    15 and 15; down: 5 left, 6 right on the doubled signal) make the whole
    operator commute with time reversal -- edges included.  A wrong pad or
    trim offset breaks this at the ends."""
    h = O.kaiser_sinc(0.25, 0.3, 12)
    for T in (1, 2, 7, 50):
        x = RNG.standard_normal((2, T)) * 3
        la = RNG.standard_normal(2) * 0.3
        lb = RNG.standard_normal(2) * 0.3
        y = O.act1d(x, la, lb, h, h)
        yr = O.act1d(x[:, ::-1], la, lb, h, h)[:, ::-1]
        np.testing.assert_allclose(y, yr, rtol=0, atol=1e-12)


def test_act1d_impulse_response_linear_limit():
    """Linear limit: the impulse response is 11 taps long (support +-5 around
    the impulse), symmetric, and its sum is the DC gain 1."""
    h = O.kaiser_sinc_f64(0.25, 0.3, 12)
    T = 64
    x = np.zeros(T)
    x[32] = 1.0
    y = O.act1d(x[None, :], np.zeros(1), np.array([60.0]), h, h)[0]
    nz = np.nonzero(np.abs(y) > 1e-15)[0]
    assert nz.min() == 27 and nz.max() == 37
    np.testing.assert_allclose(y[27:38], y[27:38][::-1], atol=1e-15)
    assert y.sum() == pytest.approx(1.0, abs=1e-14)


# ----------------------------------------------------------------- convolutions

@pytest.mark.parametrize("cin,cout,k,d,T", [(3, 5, 3, 1, 17), (4, 2, 7, 3, 40), (6, 6, 11, 5, 64),
                                            (5, 1, 7, 1, 9), (2, 3, 1, 1, 5), (3, 4, 3, 5, 4)])
def test_conv1d_matches_torch(cin, cout, k, d, T):
    """Library routine: torch's float64 CPU conv1d with the same dilation and
    'same' padding (k d - d)/2 ([H3] get_padding)."""
    x = RNG.standard_normal((2, cin, T))
    w = RNG.standard_normal((cout, cin, k))
    b = RNG.standard_normal(cout)
    r = RNG.standard_normal((2, cout, T))
    p = (k * d - d) // 2
    y = O.conv1d(x, w, b, dilation=d, pad=p, residual=r)
    ref = F.conv1d(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b),
                   padding=p, dilation=d).numpy() + r
    assert y.shape == (2, cout, T)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_conv1d_k1_is_matrix_product():
    x = RNG.standard_normal((1, 7, 13))
    w = RNG.standard_normal((5, 7, 1))
    y = O.conv1d(x, w, None, dilation=1, pad=0)
    np.testing.assert_allclose(y[0], w[:, :, 0] @ x[0], rtol=1e-13, atol=1e-13)


def test_conv1d_impulse_returns_taps():
    """A unit impulse in channel i at time t0 returns w[:, i, ::-1] around t0."""
    k, d = 7, 3
    x = np.zeros((1, 2, 60))
    x[0, 1, 30] = 1.0
    w = RNG.standard_normal((3, 2, k))
    y = O.conv1d(x, w, None, dilation=d)
    p = (k * d - d) // 2
    for j in range(k):
        np.testing.assert_allclose(y[0, :, 30 + p - j * d], w[:, 1, j], atol=1e-15)


@pytest.mark.parametrize("cin,cout,k,s,T", [(4, 3, 10, 5, 9), (3, 2, 11, 5, 7), (5, 4, 4, 2, 12),
                                            (2, 2, 3, 1, 6), (3, 2, 3, 5, 6)])
def test_convtr1d_matches_torch(cin, cout, k, s, T):
    """Library routine: torch's float64 conv_transpose1d with padding
    (k - s)//2 ([H3] ConvT1d::load), weights [Cin, Cout, k]."""
    x = RNG.standard_normal((2, cin, T))
    w = RNG.standard_normal((cin, cout, k))
    b = RNG.standard_normal(cout)
    p = (k - s) // 2 if k >= s else 0
    y = O.convtr1d(x, w, b, stride=s, pad=p)
    ref = F.conv_transpose1d(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b),
                             stride=s, padding=p).numpy()
    assert y.shape == ref.shape == (2, cout, (T - 1) * s + k - 2 * p)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_convtr1d_adjoint_of_strided_conv():
    """<ConvT_W(x), y> = <x, StridedConv_W(y)>: pins the [Cin, Cout, k] weight
    layout against torch's strided conv1d (the adjoint), no bias."""
    cin, cout, k, s, T = 3, 4, 11, 5, 9
    p = (k - s) // 2
    x = RNG.standard_normal((1, cin, T))
    w = RNG.standard_normal((cin, cout, k))
    yt = O.convtr1d(x, w, None, stride=s, pad=p)
    y = RNG.standard_normal(yt.shape)
    lhs = float(np.sum(yt * y))
    adj = F.conv1d(torch.from_numpy(y), torch.from_numpy(w), stride=s, padding=p).numpy()
    adj = adj[..., :T]
    rhs = float(np.sum(x * adj))
    assert lhs == pytest.approx(rhs, rel=1e-12)


def test_convtr1d_output_length_h3_stages():
    """k = 11 at rate 5 and k = 4 at rate 2 give exactly T * rate: the H3
    decoder's frames x hop geometry."""
    for k, s in ((11, 5), (4, 2)):
        x = RNG.standard_normal((1, 2, 13))
        w = RNG.standard_normal((2, 2, k))
        assert O.convtr1d(x, w, None, stride=s).shape[-1] == 13 * s


# ----------------------------------------------------------------- AMP / MRF / decode

def _amp_params(C, k, dil, scale=0.3, zero_conv2=False, zero_all=False):
    w1 = [RNG.standard_normal((C, C, k)) * scale for _ in dil]
    b1 = [RNG.standard_normal(C) * 0.1 for _ in dil]
    w2 = [RNG.standard_normal((C, C, k)) * scale for _ in dil]
    b2 = [RNG.standard_normal(C) * 0.1 for _ in dil]
    if zero_conv2 or zero_all:
        w2 = [np.zeros_like(w) for w in w2]
        b2 = [np.zeros_like(b) for b in b2]
    if zero_all:
        w1 = [np.zeros_like(w) for w in w1]
        b1 = [np.zeros_like(b) for b in b1]
    la = [RNG.standard_normal(C) * 0.3 for _ in range(2 * len(dil))]
    lb = [RNG.standard_normal(C) * 0.3 for _ in range(2 * len(dil))]
    return O.AmpParams(k, list(dil), w1, b1, w2, b2, la, lb)


def test_amp_identity_when_second_convs_vanish():
    x = RNG.standard_normal((2, 4, 50))
    p = _amp_params(4, 3, (1, 3, 5), zero_conv2=True)
    np.testing.assert_array_equal(O.amp_block(x, p), x)


def test_mrf_identity_when_all_convs_vanish():
    x = RNG.standard_normal((1, 3, 40))
    blocks = [_amp_params(3, k, (1, 3, 5), zero_all=True) for k in (3, 7, 11)]
    np.testing.assert_allclose(O.mrf(x, blocks), x, rtol=0, atol=1e-15)


def test_amp_receptive_field():
    """One AMP block with k and dilations d: perturbing x[t0] changes outputs
    only within sum over units of (2*5 + (k-1)d/2 + 2*5 + (k-1)/2)... bounded
    support, and nothing beyond it."""
    C, k, dil = 2, 3, (1, 3, 5)
    p = _amp_params(C, k, dil)
    x = RNG.standard_normal((1, C, 200))
    x2 = x.copy()
    x2[0, 0, 100] += 1.0
    dy = np.abs(O.amp_block(x2, p) - O.amp_block(x, p))[0].max(axis=0)
    reach = sum(5 + (k - 1) * d // 2 + 5 + (k - 1) // 2 for d in dil)
    assert dy[100] > 0
    assert np.all(dy[: 100 - reach] == 0) and np.all(dy[100 + reach + 1:] == 0)
