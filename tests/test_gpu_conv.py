"""Parity of the FP32-MFMA Conv1d and polyphase ConvTranspose1d kernels
(avae_conv1d, avae_convtr1d) with the float64 oracle:
max|err| / RMS(ref) <= 1e-5 per kernel call."""
import numpy as np
import pytest

from bigvgan_waveform_decoder_amd import avae
from bigvgan_waveform_decoder_amd import workloads as W
from oracle import avae_oracle as O
from tests.gpu_util import announce, cuda, host
from tests.helpers import rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _conv_inputs(tag, B, Cin, Cout, T, K):
    x = W.normal(0, f"conv/{tag}/x", [B, Cin, T])
    w = W.normal(0, f"conv/{tag}/w", [Cout, Cin, K], 0.0, 1.0 / (Cin * K))
    b = W.normal(0, f"conv/{tag}/b", [Cout], 0.0, 0.01)
    return x, w, b


CONV_CASES = [
    # B, Cin, Cout, T, K, d, pad (None = same), residual
    (1, 8, 16, 100, 3, 1, None, False),
    (2, 13, 21, 257, 3, 3, None, True),
    (1, 32, 12, 1000, 7, 5, None, False),
    (2, 24, 130, 300, 11, 5, None, True),
    (1, 12, 1, 64, 7, 1, None, False),
    (1, 5, 7, 50, 5, 2, None, False),      # K outside the specialised set
    (1, 9, 9, 40, 3, 1, 0, False),          # "valid" padding: Tout = T - 2
    (1, 9, 9, 40, 3, 2, 5, False),          # more padding than "same"
    (1, 256, 256, 513, 3, 1, None, True),   # 128-row tiles
    (2, 512, 512, 700, 11, 3, None, False),
    (1, 768, 768, 260, 11, 5, None, True),  # H3 stage-1 width, long K
    (2, 1, 3, 33, 1, 1, None, False),
    (2, 48, 70, 300, 3, 2, None, True),     # LDS-DMA staging, Cout tail in a 64-row tile
    (1, 64, 100, 200, 7, 9, None, False),   # 7 taps at dilation 9 (wider staged halo)
    (1, 36, 64, 300, 11, 1, None, False),   # Cin not a multiple of 8: register staging
    # output-channel tiles in groups of two (weights of a tile ~1 MB), the
    # last group holding one tile
    (1, 384, 320, 600, 11, 1, None, True),
    # 64 x 160 tiles (one round of <= 768 blocks where 64 x 128 makes more;
    # ragged last time tile, Cout tail)
    (2, 16, 64, 59999, 11, 3, None, True),
    (1, 8, 100, 52700, 11, 1, None, False),
    (2, 16, 64, 59999, 7, 5, None, False),
    (1, 16, 100, 52700, 3, 1, None, True),
    # 64 x 96 tiles (one resident round of 384 blocks; ragged last time tile)
    (2, 64, 128, 9200, 11, 5, None, True),
    (2, 64, 64, 18400, 3, 1, None, False),
    (1, 128, 128, 18400, 7, 3, None, False),
    # 96 x 128 tiles (96-row channel tiles over grids of >= 2048 blocks;
    # ragged last time tile, three channel tiles)
    (1, 16, 96, 262100, 7, 3, None, True),
    (1, 16, 288, 90000, 3, 1, None, False),
]


@pytest.mark.parametrize("B,Cin,Cout,T,K,d,pad,res", CONV_CASES)
def test_conv1d_matches_oracle(B, Cin, Cout, T, K, d, pad, res):
    announce(f"conv1d B={B} Cin={Cin} Cout={Cout} T={T} K={K} d={d} pad={pad} res={res}")
    x, w, b = _conv_inputs(f"{B}-{Cin}-{Cout}-{T}-{K}-{d}-{pad}", B, Cin, Cout, T, K)
    p = (K * d - d) // 2 if pad is None else pad
    Tout = T + 2 * p - d * (K - 1)
    r = W.normal(0, f"conv/{Cin}-{Cout}-{T}/res", [B, Cout, Tout]) if res else None
    y = host(avae.conv1d(cuda(x), cuda(w), cuda(b), dilation=d, pad=p,
                         residual=cuda(r) if res else None))
    ref = O.conv1d(x, w, b, dilation=d, pad=p, residual=r)
    assert y.shape == ref.shape
    assert rel_err(y, ref) <= TOL


def test_conv1d_inplace_residual():
    """residual may be the output buffer itself (cur += conv(...))."""
    announce("conv1d in-place residual")
    x, w, b = _conv_inputs("inplace", 2, 64, 64, 777, 3)
    cur = W.normal(0, "conv/inplace/cur", [2, 64, 777])
    out = cuda(cur)
    avae.conv1d(cuda(x), cuda(w), cuda(b), dilation=3, residual=out, out=out)
    ref = O.conv1d(x, w, b, dilation=3, residual=cur)
    assert rel_err(host(out), ref) <= TOL


def _window_conv(x, w, b, d, a, e):
    """Oracle outputs y[..., a:e] of a 'same' conv, from the inputs it reads
    (zero beyond the signal)."""
    K = w.shape[2]
    p = (K * d - d) // 2
    T = x.shape[-1]
    lo, hi = a - p, e - p + (K - 1) * d
    xw = np.zeros(x.shape[:-1] + (hi - lo,), np.float64)
    s0, s1 = max(lo, 0), min(hi, T)
    xw[..., s0 - lo:s1 - lo] = x[..., s0:s1]
    return O.conv1d(xw, w, b, dilation=d, pad=0)


@pytest.mark.parametrize("d", [1, 5])
def test_conv1d_full_size_workload2_sampled_windows(d):
    """Workload 2's AMP conv at full size ([2, 512, 65536], 512 -> 512, k=3)
    on windows at both ends and inside, every output channel."""
    announce(f"conv1d workload2 full size d={d}")
    x, _, _, t = W.workload2()
    w = t["block.convs1.0.weight"]
    b = t["block.convs1.0.bias"]
    y = host(avae.conv1d(cuda(x), cuda(w), cuda(b), dilation=d))
    T = x.shape[-1]
    for a in (0, 12345, 40000, T - 300):
        ref = _window_conv(x, w, b, d, a, a + 300)
        assert rel_err(y[..., a:a + 300], ref) <= TOL, a


CONVT_CASES = [
    # B, Cin, Cout, Tin, K, s, pad (-1 = (K-s)/2)
    (1, 8, 16, 10, 10, 5, -1),
    (2, 24, 12, 33, 11, 5, -1),
    (1, 16, 8, 40, 4, 2, -1),
    (1, 70, 130, 17, 4, 2, -1),
    (2, 6, 5, 9, 3, 1, -1),
    (1, 4, 4, 6, 4, 2, 0),
    (1, 12, 6, 300, 11, 5, 4),
    (2, 96, 48, 1000, 4, 2, -1),
    (1, 32, 40, 50, 16, 8, -1),    # LDS-DMA staging, Cout tail in a 32-channel tile
    (1, 32, 20, 50, 11, 5, -1),    # short input: 16-channel tiles, LDS-DMA, Cout tail
    (2, 48, 20, 77, 8, 4, -1),
    (1, 16, 33, 29, 11, 5, -1),    # Cout*K not a multiple of 4: generic kernel
    (2, 48, 24, 300, 4, 2, -1),    # stride 2, Cout <= 32: 16 x 256 tiles (LDS DMA)
    (1, 24, 12, 500, 4, 2, -1),    # the same with Cin not a multiple of 16 (register staging)
    (2, 64, 96, 257, 4, 2, -1),    # stride 2, Cout 96: 32 x 128 tiles
]


@pytest.mark.parametrize("B,Cin,Cout,Tin,K,s,pad", CONVT_CASES)
def test_convtr1d_matches_oracle(B, Cin, Cout, Tin, K, s, pad):
    announce(f"convtr1d B={B} Cin={Cin} Cout={Cout} Tin={Tin} K={K} s={s} pad={pad}")
    x = W.normal(0, f"convt/{Cin}-{Cout}-{Tin}/x", [B, Cin, Tin])
    w = W.normal(0, f"convt/{Cin}-{Cout}-{Tin}/w", [Cin, Cout, K], 0.0, 2.0 / (Cin * K))
    b = W.normal(0, f"convt/{Cin}-{Cout}-{Tin}/b", [Cout], 0.0, 0.01)
    y = host(avae.convtr1d(cuda(x), cuda(w), cuda(b), stride=s, pad=pad))
    p = (K - s) // 2 if pad < 0 else pad
    ref = O.convtr1d(x, w, b, stride=s, pad=p)
    assert y.shape == ref.shape
    assert rel_err(y, ref) <= TOL


def test_convtr1d_full_size_workload3():
    """Workload 3's upsampler at full size: [2, 1024, 8000] -> [2, 512, 40001]."""
    announce("convtr1d workload3 full size")
    x, t = W.workload3()
    y = host(avae.convtr1d(cuda(x), cuda(t["ups.0.weight"]), cuda(t["ups.0.bias"]), stride=5))
    ref = O.convtr1d(x, t["ups.0.weight"], t["ups.0.bias"], stride=5)
    assert y.shape == (2, 512, 40001)
    assert rel_err(y, ref) <= TOL


def _random_conv_cases(n, seed):
    """Seeded shapes spread over the dispatch branches: tile rows 16/32/48/64/96,
    K in and outside the specialised set, dilations up to the staged halo,
    channel counts that are and are not multiples of the staging chunks."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        K = int(rng.choice([1, 3, 5, 7, 11]))
        d = int(rng.integers(1, 10 if K == 7 else 6))
        Cin = int(rng.choice([4, 8, 12, 16, 24, 32, 40, 48, 64, 72, 96, 128]))
        Cout = int(rng.choice([1, 5, 16, 24, 33, 48, 64, 70, 96, 128, 192]))
        T = int(rng.integers(max(1, (K - 1) * d // 2 + 1), 700))
        out.append((int(rng.integers(1, 3)), Cin, Cout, T, K, d, bool(rng.integers(0, 2))))
    return out


RANDOM_CONV = _random_conv_cases(24, 20261203)


@pytest.mark.parametrize("B,Cin,Cout,T,K,d,res", RANDOM_CONV)
def test_conv1d_random_shapes(B, Cin, Cout, T, K, d, res):
    announce(f"conv1d random B={B} Cin={Cin} Cout={Cout} T={T} K={K} d={d} res={res}")
    x, w, b = _conv_inputs(f"rnd-{B}-{Cin}-{Cout}-{T}-{K}-{d}", B, Cin, Cout, T, K)
    r = W.normal(0, f"conv/rnd-{Cin}-{Cout}-{T}-{K}/res", [B, Cout, T]) if res else None
    y = host(avae.conv1d(cuda(x), cuda(w), cuda(b), dilation=d,
                         residual=cuda(r) if res else None))
    ref = O.conv1d(x, w, b, dilation=d, pad=(K * d - d) // 2, residual=r)
    assert rel_err(y, ref) <= TOL


def _random_convt_cases(n, seed):
    """Seeded (K, stride) pairs of the specialised kernels and others, with
    Cin on and off the 16-channel chunk and Cout tails."""
    rng = np.random.default_rng(seed)
    pairs = [(11, 5), (10, 5), (4, 2), (16, 8), (8, 4), (3, 1), (6, 3), (5, 2)]
    out = []
    for _ in range(n):
        K, s = pairs[int(rng.integers(0, len(pairs)))]
        out.append((int(rng.integers(1, 3)), int(rng.choice([8, 16, 24, 32, 48, 64])),
                    int(rng.choice([4, 12, 16, 20, 32, 40, 64, 100])),
                    int(rng.integers(1, 300)), K, s))
    return out


RANDOM_CONVT = _random_convt_cases(16, 20261204)


@pytest.mark.parametrize("B,Cin,Cout,Tin,K,s", RANDOM_CONVT)
def test_convtr1d_random_shapes(B, Cin, Cout, Tin, K, s):
    announce(f"convtr1d random B={B} Cin={Cin} Cout={Cout} Tin={Tin} K={K} s={s}")
    x = W.normal(0, f"convt/rnd-{Cin}-{Cout}-{Tin}/x", [B, Cin, Tin])
    w = W.normal(0, f"convt/rnd-{Cin}-{Cout}-{Tin}/w", [Cin, Cout, K], 0.0, 2.0 / (Cin * K))
    b = W.normal(0, f"convt/rnd-{Cin}-{Cout}-{Tin}/b", [Cout], 0.0, 0.01)
    y = host(avae.convtr1d(cuda(x), cuda(w), cuda(b), stride=s))
    ref = O.convtr1d(x, w, b, stride=s, pad=(K - s) // 2)
    assert y.shape == ref.shape
    assert rel_err(y, ref) <= TOL
