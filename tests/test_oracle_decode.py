"""Whole-decoder properties of the oracle, on narrow versions of the two
decoders (same rates, kernels and dilations; fewer channels) so that each
case finishes in seconds.

[H3]  = docs.rs source page of cortiq_engine/audiovae.rs (cortiq-engine 0.5.74)
[LTX] = docs.rs source page of cortiq_engine/ltxaudio.rs (cortiq-engine 0.6.3)
"""
import json
import os

import numpy as np
import pytest

from bigvgan_waveform_decoder_amd import workloads as W
from oracle import avae_oracle as O
from tests.helpers import decoder_params, rel_err

PAGE = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))

H3_SMALL = W.scaled_spec(W.H3, 128)
LTX_SMALL = W.scaled_spec(W.LTX, 64)


def _decode(spec, frames, B=2, workload=4, **kw):
    z = W.normal(workload, "latent", [B, spec.c_in, frames])
    t = W.decoder_tensors(spec, workload, **kw)
    p = decoder_params(spec, t)
    return z, p, O.decode(z, p)


def test_h3_geometry_is_page_geometry():
    """[H3] module doc: 800 samples a frame at 32 kHz, 40 frames a second,
    32 latent channels (tests/golden)."""
    g = PAGE["geometry"]
    assert W.H3.hop == g["h3_hop"]
    assert W.H3.sample_rate == g["h3_sample_rate"] == g["h3_frame_rate"] * g["h3_hop"]
    assert W.H3.c_in == g["h3_latent_channels"]
    assert list(W.LTX.rates) == g["ltx_vocoder_rates"]


@pytest.mark.parametrize("spec,frames", [(H3_SMALL, 3), (LTX_SMALL, 5)])
def test_decode_length_range_and_motion(spec, frames):
    """[H3] test music3_dav_decodes_to_the_reference_geometry, its checks
    reused: length = frames x hop, finite, within [-1, 1], not silent, and
    the two passes differ when their latents differ."""
    z, p, y = _decode(spec, frames)
    assert y.shape == (2, frames * spec.hop)
    assert np.all(np.isfinite(y))
    assert np.all(np.abs(y) <= 1.0)
    assert np.sqrt(np.mean(y * y)) > 1e-4
    assert np.max(np.abs(y[0] - y[1])) > 0.0


def test_decode_batched_equals_per_pass():
    """Stereo = independent mono passes ([H3] AudioVae::decode): decoding the
    batch equals decoding each row alone, exactly."""
    spec = H3_SMALL
    z, p, y = _decode(spec, 3)
    for b in range(2):
        yb = O.decode(z[b:b + 1], p)
        np.testing.assert_array_equal(yb[0], y[b])


def test_decode_locality():
    """The decoder is a finite, non-causal stack: changing the last latent
    frame leaves the first output samples untouched, and changes samples
    near that frame."""
    spec = W.scaled_spec(W.H3, 128, final="none")
    frames = 40
    z = W.normal(4, "latent", [1, spec.c_in, frames])
    p = decoder_params(spec, W.decoder_tensors(spec, 4))
    y0 = O.decode(z, p)
    z2 = z.copy()
    z2[0, :, -1] += 1.0
    y1 = O.decode(z2, p)
    d = np.abs(y1 - y0)[0]
    hop = spec.hop
    assert d[(frames - 1) * hop:].max() > 0
    # receptive field of the H3 geometry is ~31 frames; 40 frames back is untouched
    assert d[: 4 * hop].max() == 0.0


def test_decode_final_modes():
    """tanh and clamp finals are the pointwise maps of the pre-final output."""
    spec = W.scaled_spec(W.LTX, 64, final="none")
    z, p, y = _decode(spec, 3, workload=5)
    p.final = "tanh"
    np.testing.assert_allclose(O.decode(z, p), np.tanh(y), rtol=0, atol=0)
    p.final = "clamp"
    np.testing.assert_allclose(O.decode(z, p), np.clip(y, -1, 1), rtol=0, atol=0)


def test_decode_optional_affine_and_dec_in():
    """Latent denormalisation z*std + mean and the 1x1 dec_in conv ([H3]
    AudioVae::decode) equal explicit pre-processing followed by the plain
    decoder."""
    spec = W.scaled_spec(W.H3, 128, latent_affine=True, dec_in=16, final="none")
    t = W.decoder_tensors(spec, 4)
    z = W.normal(4, "latent", [1, spec.c_in, 3])
    p = decoder_params(spec, t)
    y = O.decode(z, p)
    lat = z.astype(np.float64) * t["latents_std"][:, None] + t["latents_mean"][:, None]
    lat = np.einsum("oi,bit->bot", t["dec_in.weight"][:, :, 0].astype(np.float64), lat) \
        + t["dec_in.bias"][:, None]
    p2 = decoder_params(spec, t)
    p2.latent_mean = p2.latent_std = p2.dec_in_w = p2.dec_in_b = None
    y2 = O.decode(lat, p2)
    assert rel_err(y, y2) < 1e-10  # only f64 summation order differs


@pytest.mark.parametrize("spec", [W.scaled_spec(W.H3, 128, final="none"),
                                  W.scaled_spec(W.LTX, 64, final="none")])
def test_receptive_field_bound_holds(spec):
    """The crop margin used by the full-size parity tests is a true bound:
    perturbing one latent frame changes no output sample more than
    decoder_reach_frames(spec) frames away."""
    from tests.helpers import decoder_reach_frames
    R = decoder_reach_frames(spec)
    frames = 2 * R + 5
    z = W.normal(4, "latent", [1, spec.c_in, frames])
    p = decoder_params(spec, W.decoder_tensors(spec, 4))
    y0 = O.decode(z, p)[0]
    f = R + 2
    z2 = z.copy()
    z2[0, :, f] += 1.0
    d = np.abs(O.decode(z2, p)[0] - y0)
    hop = spec.hop
    assert d[f * hop:(f + 1) * hop].max() > 0
    assert d[:max(0, (f - R) * hop)].max(initial=0.0) == 0.0
    assert d[(f + R + 1) * hop:].max(initial=0.0) == 0.0
