"""Pins for the oracle's Music-3 DAV decoder ([H3] page, items Snake,
DavUnit, DavStage, Music3Dav and the test of its geometry), checked against
values and identities the page and the mathematics fix, not against the
oracle's own formulas."""
import math

import numpy as np
import pytest

from bigvgan_waveform_decoder_amd import workloads as W
from oracle import avae_oracle as O
from tests.helpers import dav_params, dav_reach_frames


def test_snake_uses_alpha_as_stored():
    """alpha = 2 at x = pi/4: sin^2(pi/2) = 1, so the value is pi/4 + 1/2
    (up to the 1e-9 of the denominator).  An exponentiated alpha (the
    SnakeBeta convention) would give pi/4 + sin^2(e^2 pi/4)/e^2 instead."""
    y = O.snake(np.array([[math.pi / 4]]), np.array([2.0]))[0, 0]
    assert abs(y - (math.pi / 4 + 1.0 / (2.0 + 1e-9))) < 1e-15
    assert abs(y - (math.pi / 4 + math.sin(math.e ** 2 * math.pi / 4) ** 2 / math.e ** 2)) > 0.1
    assert O.snake(np.zeros((1, 3)), np.array([0.7]))[0].tolist() == [0.0, 0.0, 0.0]


def test_snake_equals_snakebeta_with_log_parameters():
    """SnakeBeta with log alpha = log beta = log a is plain Snake with alpha a
    (two independently written functions of the oracle)."""
    rng = np.random.default_rng(3)
    a = rng.uniform(0.3, 3.0, size=5)
    x = rng.standard_normal((2, 5, 40)) * 3
    got = O.snake(x, a)
    ref = O.snake_beta(x, np.log(a), np.log(a))
    assert np.max(np.abs(got - ref)) < 1e-12


def test_snake_periodicity_and_bounds():
    """snake(x) - x has period pi/alpha and lies in [0, 1/alpha]."""
    rng = np.random.default_rng(4)
    a = rng.uniform(0.5, 2.0, size=4)
    x = rng.standard_normal((4, 100)) * 5
    d0 = O.snake(x, a) - x
    xs = x + math.pi / a[:, None]
    d1 = O.snake(xs, a) - xs
    assert np.max(np.abs(d0 - d1)) < 1e-9
    assert np.all(d0 >= 0) and np.all(d0 <= 1.0 / a[:, None] + 1e-12)


def _unit(C, k, d, rng, zero=False):
    z = (lambda *s: np.zeros(s)) if zero else (lambda *s: rng.standard_normal(s) * 0.2)
    return O.DavUnitParams(dilation=d, a1=rng.uniform(0.5, 1.5, C), w1=z(C, C, k), b1=z(C),
                           a2=rng.uniform(0.5, 1.5, C), w2=z(C, C, 1), b2=z(C))


def test_dav_unit_identity_and_bias():
    """All-zero convolutions leave the unit the identity (the residual); a
    zero 1-tap weight with bias c adds exactly c."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 6, 50))
    u = _unit(6, 7, 3, rng, zero=True)
    assert np.array_equal(O.dav_unit(x, u), x)
    u.b2 = np.full(6, 0.25)
    assert np.max(np.abs(O.dav_unit(x, u) - (x + 0.25))) == 0.0


def test_dav_unit_receptive_field():
    """An impulse reaches (k-1) d / 2 samples each way through the dilated
    conv and no further (Snake and the 1-tap conv are pointwise)."""
    rng = np.random.default_rng(6)
    C, T, k, d = 4, 120, 7, 9
    u = _unit(C, k, d, rng)
    x = rng.standard_normal((1, C, T))
    x2 = x.copy()
    x2[0, :, 60] += 1.0
    diff = np.abs(O.dav_unit(x2, u) - O.dav_unit(x, u)).max(axis=(0, 1))
    nz = np.nonzero(diff > 0)[0]
    assert nz.min() == 60 - (k - 1) // 2 * d and nz.max() == 60 + (k - 1) // 2 * d


@pytest.mark.parametrize("s", [8, 4, 2])
def test_dav_stage_length_is_stride_times_input(s):
    """k = 2 s with padding (k - s) / 2 gives exactly s output samples per
    input sample (the page's HOP = 8*8*4*2 = 512 needs it)."""
    rng = np.random.default_rng(7)
    C = 4
    st = O.DavStageParams(stride=s, alpha=rng.uniform(0.5, 1.5, C),
                          up_w=rng.standard_normal((C, 3, 2 * s)), up_b=np.zeros(3),
                          units=[_unit(3, 7, d, rng) for d in (1, 3, 9)])
    for n in (1, 5, 13):
        assert O.dav_stage(rng.standard_normal((1, C, n)), st).shape == (1, 3, n * s)


SMALL = W.scaled_dav(64)


def _page_latent(frames):
    """The page's structured latent: 0.4 sin(0.13 c + 0.7 t) over 128 x frames."""
    c = np.arange(128)[:, None]
    t = np.arange(frames)[None, :]
    return (0.4 * np.sin(c * 0.13 + t * 0.7))[None]


def test_dav_decode_reference_geometry():
    """The page's geometry test on synthetic weights: 512 samples a frame per
    side, interleaved; finite; within the tanh range; not silent; the two
    sides differ."""
    frames = 12
    p = dav_params(SMALL, W.dav_tensors(SMALL, 6))
    y = O.dav_decode(_page_latent(frames), p)
    assert y.shape == (1, frames * O.DAV_HOP * 2)
    assert np.all(np.isfinite(y)) and np.all(np.abs(y) <= 1.0)
    assert np.sqrt(np.mean(y ** 2)) > 1e-4
    assert np.max(np.abs(y[0, 0::2] - y[0, 1::2])) > 0.0


def test_dav_stereo_split_and_interleave():
    """Identical halves decode to identical sides; swapping the halves swaps
    the interleaved samples."""
    frames = 3
    p = dav_params(SMALL, W.dav_tensors(SMALL, 6))
    z = W.normal(6, "stereo", [1, 128, frames])
    same = np.concatenate([z[:, :64], z[:, :64]], axis=1)
    y = O.dav_decode(same, p)
    assert np.array_equal(y[0, 0::2], y[0, 1::2])
    a = O.dav_decode(z, p)
    b = O.dav_decode(np.concatenate([z[:, 64:], z[:, :64]], axis=1), p)
    assert np.array_equal(a[0, 0::2], b[0, 1::2]) and np.array_equal(a[0, 1::2], b[0, 0::2])


def test_dav_receptive_field_bound_holds():
    """Changing one latent frame changes output samples only within the
    reach bound used by the windowed full-size parity tests."""
    frames, f0 = 40, 20
    R = dav_reach_frames(SMALL)
    assert R <= 14
    p = dav_params(SMALL, W.dav_tensors(SMALL, 6))
    z = W.normal(6, "reach", [1, 128, frames])
    z2 = z.copy()
    z2[0, :, f0] += 1.0
    d = np.abs(O.dav_decode(z2, p) - O.dav_decode(z, p))[0]
    hop2 = 2 * O.DAV_HOP
    assert np.all(d[: (f0 - R) * hop2] == 0) and np.all(d[(f0 + R + 1) * hop2:] == 0)
    assert d[f0 * hop2: (f0 + 1) * hop2].max() > 0
