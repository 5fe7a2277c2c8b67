"""Parity of the fused Activation1d kernel (avae_act1d) with the float64
oracle: max|err| / RMS(ref) <= 1e-5 per kernel call."""
import numpy as np
import pytest

from bigvgan_waveform_decoder_amd import avae
from bigvgan_waveform_decoder_amd import workloads as W
from oracle import avae_oracle as O
from tests.gpu_util import announce, cuda, host
from tests.helpers import rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _inputs(tag, B, C, T, scale=1.0):
    x = W.normal(0, f"act/{tag}/x", [B, C, T]) * np.float32(scale)
    la = W.normal(0, f"act/{tag}/la", [C], 0.0, 0.1)
    lb = W.normal(0, f"act/{tag}/lb", [C], 0.0, 0.1)
    return x, la, lb


@pytest.mark.parametrize("B,C,T,scale", [
    (1, 1, 1, 1.0), (1, 3, 2, 1.0), (2, 3, 7, 3.0), (1, 2, 1023, 1.0), (1, 2, 1024, 1.0),
    (2, 2, 1025, 1.0), (1, 4, 3000, 10.0), (1, 2, 5000, 1000.0), (3, 5, 2049, 0.01),
    # T % 4 == 0: edge tiles on the vector path (first, last, partial, single)
    (1, 2, 4, 1.0), (2, 3, 8, 1.0), (1, 2, 12, 2.0), (1, 3, 2048, 1.0), (2, 2, 2052, 1.0),
    (1, 2, 4096, 1.0), (1, 2, 4104, 1.0), (1, 1, 6148, 1.0)])
def test_act1d_matches_oracle(B, C, T, scale):
    announce(f"act1d B={B} C={C} T={T} scale={scale}")
    x, la, lb = _inputs(f"{B}-{C}-{T}", B, C, T, scale)
    y = host(avae.act1d(cuda(x), cuda(la), cuda(lb)))
    ref = O.act1d(x, la, lb)
    assert y.shape == (B, C, T)
    assert rel_err(y, ref) <= TOL


def test_act1d_explicit_asymmetric_taps():
    """Caller-supplied taps (not symmetric, different up and down) exercise
    every tap index of both filters."""
    announce("act1d explicit taps")
    x, la, lb = _inputs("taps", 2, 3, 1500)
    up = W.normal(0, "act/taps/up", [12], 0.0, 0.05) + np.float32(1.0 / 12)
    down = W.normal(0, "act/taps/down", [12], 0.0, 0.05) + np.float32(1.0 / 12)
    y = host(avae.act1d(cuda(x), cuda(la), cuda(lb), up_taps=up, down_taps=down))
    ref = O.act1d(x, la, lb, up.astype(np.float64), down.astype(np.float64))
    assert rel_err(y, ref) <= TOL


def test_act1d_constant_rows_closed_form():
    """Constant rows map to SnakeBeta of the constant everywhere, edges included."""
    announce("act1d constants")
    C, T = 4, 3000
    c = np.array([0.3, -1.7, 2.5, 40.0], np.float32)
    x = np.repeat(c[:, None], T, axis=1)[None]
    la = np.array([0.1, -0.2, 0.3, 0.0], np.float32)
    lb = np.array([-0.1, 0.25, 0.0, 0.5], np.float32)
    y = host(avae.act1d(cuda(x), cuda(la), cuda(lb)))[0]
    want = (c + np.sin(np.exp(la.astype(np.float64)) * c) ** 2
            / (np.exp(lb.astype(np.float64)) + 1e-9))
    assert np.max(np.abs(y - want[:, None]) / np.abs(want)[:, None]) < 2e-6


def test_act1d_full_size_workload2_sampled_rows():
    """Workload 2 at full size, [2, 512, 65536], as bench.py launches it;
    the oracle recomputes 24 sampled (pass, channel) rows (the operation is
    per channel, so a row is exact on its own)."""
    announce("act1d workload2 full size")
    x, la, lb, _ = W.workload2()
    y = avae.act1d(cuda(x), cuda(la), cuda(lb))
    yh = host(y)
    rng = np.random.default_rng(7)
    rows = [(int(b), int(c)) for b, c in zip(rng.integers(0, 2, 24), rng.integers(0, 512, 24))]
    rows += [(0, 0), (1, 511)]
    for b, c in rows:
        ref = O.act1d(x[b, c][None], la[c:c + 1], lb[c:c + 1])[0]
        assert rel_err(yh[b, c], ref) <= TOL, (b, c)
    assert np.all(np.isfinite(yh))


def test_act1d_deterministic():
    announce("act1d determinism")
    x, la, lb = _inputs("det", 2, 8, 4097)
    a = host(avae.act1d(cuda(x), cuda(la), cuda(lb)))
    b = host(avae.act1d(cuda(x), cuda(la), cuda(lb)))
    np.testing.assert_array_equal(a, b)


def test_mfma_probe_runs_and_sums_are_finite():
    """The matrix-core probe bench.py times: it runs for both chain counts
    and writes one finite sum per thread."""
    import torch
    announce("mfma probe")
    for chains in (8, 16):
        sink = torch.full((4 * 256,), float("nan"), device="cuda:0")
        avae.probe_mfma(chains, 4, 10, sink)
        s10 = host(sink)
        assert np.all(np.isfinite(s10))
        # every iteration adds the same product to every chain, so the sums
        # are linear in iters; an odd count runs the loop's single-round tail
        avae.probe_mfma(chains, 4, 11, sink)
        s11 = host(sink)
        nz = np.abs(s10) > 1e-12
        assert nz.sum() > 0
        np.testing.assert_allclose(s11[nz], 1.1 * s10[nz], rtol=1e-4)


def test_probe_copy_is_exact():
    """The streaming-copy probe bench.py times copies every element, including
    a last partial block."""
    import torch
    announce("stream copy probe")
    for n in (4, 1024, 4 * 1000 + 8):
        x = torch.from_numpy(W.normal(0, f"copy/{n}", [n])).to("cuda:0")
        y = torch.full_like(x, float("nan"))
        avae.probe_copy(x, y)
        assert np.array_equal(host(y), host(x))
