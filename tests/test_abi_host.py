"""CPU-side checks of the C-ABI library: it loads, it exports every entry
point the header declares, its host-only filter designer agrees with the
oracle, and argument errors are reported before anything touches a device."""
import ctypes
import os
import re

import numpy as np
import pytest

from bigvgan_waveform_decoder_amd import avae
from oracle import avae_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "avae.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(avae_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = avae.lib()
    names = _declared_functions()
    assert len(names) >= 14, names
    for n in names:
        assert hasattr(L, n), f"libavae.so does not export {n}"


def test_version():
    assert avae.version() >= 100


def test_kaiser_sinc_matches_oracle():
    """The library's float64 designer (its own C++) rounds to the same float32
    taps as the oracle's design, for the decoder's filter and a few others."""
    for cutoff, hw, k in [(0.25, 0.3, 12), (0.25, 0.3, 16), (0.2, 0.25, 24), (0.4, 0.1, 8)]:
        got = avae.kaiser_sinc(cutoff, hw, k).astype(np.float64)
        ref = O.kaiser_sinc(cutoff, hw, k)
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= ulp), (cutoff, hw, k, got - ref)


def test_kaiser_sinc_rejects_bad_arguments():
    L = avae.lib()
    out = np.zeros(16, np.float32)
    assert L.avae_kaiser_sinc(0.25, 0.3, 11, out.ctypes.data) == -1
    assert L.avae_kaiser_sinc(0.0, 0.3, 12, out.ctypes.data) == -1
    assert L.avae_kaiser_sinc(0.25, 0.3, 12, None) == -1
    assert b"taps" in L.avae_last_error() or b"null" in L.avae_last_error()


def test_argument_errors_before_any_launch():
    """Null pointers and impossible shapes fail with a code and a message,
    without any device call (this runs where there is no GPU)."""
    L = avae.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: checks fail first
    assert L.avae_act1d(None, fake, 1, 1, 1, fake, fake, None, None, None) == -1
    assert L.avae_act1d(fake, fake, 0, 1, 1, fake, fake, None, None, None) == -1
    assert L.avae_conv1d(fake, fake, 1, 1, 1, 4, None, None, 3, 1, 1, None, None) == -1
    # Tout = 4 + 0 - 5*(3-1) < 1
    assert L.avae_conv1d(fake, ctypes.c_void_p(0x2000), 1, 1, 1, 4, fake, None, 3, 5, 0,
                         None, None) == -2
    assert L.avae_conv1d(fake, ctypes.c_void_p(0x2000), 1, 1, 1, 4, fake, None, 33, 1, 16,
                         None, None) == -2
    assert L.avae_convtr1d(fake, ctypes.c_void_p(0x2000), 1, 1, 1, 4, fake, None, 2, 5, -1,
                           None) == -2
    assert L.avae_convtr1d(fake, ctypes.c_void_p(0x2000), 1, 1, 1, 4, fake, None, 4, 0, -1,
                           None) == -1
    assert len(L.avae_last_error()) > 0
    # workspace too small
    dil = (ctypes.c_int * 1)(1)
    ptrs = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    rc = L.avae_amp_block(fake, ctypes.c_void_p(0x2000), 1, 4, 8, 3, 1, ctypes.addressof(dil),
                          ctypes.addressof(ptrs), None, ctypes.addressof(ptrs), None,
                          ctypes.addressof(ptrs), ctypes.addressof(ptrs), 1.0, 0, fake, 16, None)
    assert rc == -3
    assert L.avae_amp_block_workspace_bytes(2, 4, 8) >= 3 * 2 * 4 * 8 * 4
    assert L.avae_amp_block_workspace_bytes(0, 4, 8) == 0


def test_decoder_create_rejects_bad_config():
    L = avae.lib()
    cfg = avae.avae_config()
    w = avae.avae_weights()
    h = ctypes.c_void_p()
    assert L.avae_decoder_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)) in (-1, -2)
    assert not h.value
    assert L.avae_decoder_create(None, ctypes.byref(w), ctypes.byref(h)) == -1
    assert L.avae_decoder_workspace_bytes(None, 1, 1) == 0
    assert L.avae_decoder_set_concurrent(None, 1) == -1
    fake = ctypes.c_void_p(0x1000)
    assert L.avae_probe_mfma(8, 1, 1, None, None) == -1
    assert L.avae_probe_mfma(7, 1, 1, fake, None) == -1
    assert L.avae_probe_mfma(16, 0, 1, fake, None) == -1
    assert L.avae_probe_copy(None, fake, 16, None) == -1
    assert L.avae_probe_copy(fake, fake, 6, None) == -1
    assert L.avae_probe_copy(fake, ctypes.c_void_p(0x1004), 16, None) == -1


def test_streaming_rejects_bad_arguments():
    L = avae.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.avae_bigvgan_decode_streaming(None, fake, 1, 1, fake, 1, 0, fake, 16, None) == -1
    assert L.avae_decoder_streaming_workspace_bytes(None, 1, 1, 0) == 0
    assert L.avae_decoder_reach_frames(None, None) == -1


def test_dav_bwe_and_tail_ops_reject_bad_arguments():
    """The DAV decoder, the extension tail and their single ops check their
    arguments before any device work (this runs where there is no GPU)."""
    L = avae.lib()
    fake = ctypes.c_void_p(0x1000)
    assert L.avae_snake(None, fake, 1, 1, 1, fake, None) == -1
    assert L.avae_snake(fake, fake, 0, 1, 1, fake, None) == -1
    assert L.avae_mel_stft(fake, fake, 1, 800, fake, 257, 512, 80, None, 64, None) == -1
    # filter shorter than the hop, and a filter length that is not a multiple of 32
    assert L.avae_mel_stft(fake, fake, 1, 800, fake, 257, 64, 80, fake, 64, None) == -2
    assert L.avae_mel_stft(fake, fake, 1, 800, fake, 257, 500, 80, fake, 64, None) == -2
    assert L.avae_mel_stft(fake, fake, 1, 40, fake, 257, 512, 80, fake, 64, None) == -2
    assert L.avae_hann_sinc_upsample(fake, fake, 1, 10, 0, None) == -1
    assert L.avae_hann_sinc_upsample(fake, fake, 1, 10, 5, None) == -1
    cfg = avae.avae_dav_config()
    h = ctypes.c_void_p()
    assert L.avae_dav_create(ctypes.byref(cfg), ctypes.byref(avae.avae_dav_weights()),
                             ctypes.byref(h)) in (-1, -2)
    assert not h.value
    assert L.avae_dav_workspace_bytes(None, 1, 1) == 0
    assert L.avae_dav_decode(None, fake, 1, 1, fake, fake, 16, None) == -1
    bcfg = avae.avae_bwe_config()
    assert L.avae_bwe_create(ctypes.byref(bcfg), ctypes.byref(avae.avae_bwe_weights()),
                             ctypes.byref(h)) in (-1, -2)
    assert L.avae_bwe_workspace_bytes(None, 1, 1) == 0
    assert L.avae_bwe_decode(None, fake, 1, 1, fake, fake, 16, None) == -1


def test_kernel_names_in_the_profiler_are_stable():
    """bench.py's traffic lookup keys on the names the library's launch
    profiler gives its kernels, each with the source file it is built from."""
    import json
    d = json.load(open(os.path.join(ROOT, "profiles", "pmc_traffic.json")))
    src = {
        "conv.hip": (r"(conv1d_(pipe|dma|mfma)_kernel<\d+(,\d+)*(,d\d+)?(,snake)?>"
                     r"|convtr1d_(dma|poly|mfma)_kernel<\d+(,\d+)*>|conv_out1_kernel"
                     r"|sum_into_kernel)$"),
        "fftconv.hip": (r"(fft_fwd_kernel(<act>|<snake>)?|fft_inv_kernel|fft_pack_kernel"
                        r"|fft_gemm_kernel<\d>)$"),
        "act1d.hip": r"act1d_kernel$",
        "amp_unit.hip": r"(amp_unit_kernel<\d+,\d+>|pack_unit_weights_kernel)$",
    }
    for name, e in d["kernels"].items():
        f = os.path.basename(e["source"])
        assert f in src, (name, f)
        assert re.match(src[f], name), (name, f)
        assert os.path.exists(os.path.join(ROOT, e["source"]))
        text = open(os.path.join(ROOT, e["source"])).read()
        assert name.split("<")[0] in text, name


def test_amp_block_static_checks_before_any_launch():
    """The no-workspace AMP block rejects null pointers and sizes beyond its
    static scratch on the host (no device call: this runs without a GPU)."""
    L = avae.lib()
    cap = L.avae_amp_block_static_max_bytes()
    assert cap == 64 << 20
    fake = ctypes.c_void_p(0x1000)
    dil = (ctypes.c_int * 1)(1)
    ptrs = (ctypes.c_void_p * 2)(0x3000, 0x3000)
    C = 64
    T = cap // (3 * 4 * C) + 1024
    assert L.avae_amp_block_workspace_bytes(1, C, T) > cap
    rc = L.avae_amp_block_static(fake, ctypes.c_void_p(0x2000), 1, C, T, 3, 1,
                                 ctypes.addressof(dil), ctypes.addressof(ptrs),
                                 ctypes.addressof(ptrs), ctypes.addressof(ptrs),
                                 ctypes.addressof(ptrs), ctypes.addressof(ptrs),
                                 ctypes.addressof(ptrs), ctypes.c_float(1.0), 0, None)
    assert rc == -2
    assert b"scratch" in L.avae_last_error()
    rc = L.avae_amp_block_static(None, fake, 1, 4, 8, 3, 1, ctypes.addressof(dil),
                                 ctypes.addressof(ptrs), ctypes.addressof(ptrs),
                                 ctypes.addressof(ptrs), ctypes.addressof(ptrs),
                                 ctypes.addressof(ptrs), ctypes.addressof(ptrs),
                                 ctypes.c_float(1.0), 0, None)
    assert rc == -1


def test_amp_block_fft_workspace_sizes():
    """The workspace size that selects the AMP block's frequency-domain
    convolutions: the direct size where no convolution takes that path, room
    for three spectra slots and one packed weight otherwise, 0 for invalid
    arguments (host logic only)."""
    L = avae.lib()
    L.avae_amp_block_fft_workspace_bytes.restype = ctypes.c_size_t
    L.avae_amp_block_workspace_bytes.restype = ctypes.c_size_t
    dil = (ctypes.c_int * 3)(1, 3, 5)
    q = lambda B, C, T, K, n=3, d=ctypes.addressof(dil): int(
        L.avae_amp_block_fft_workspace_bytes(B, C, T, K, n, d))
    plain = lambda B, C, T: int(L.avae_amp_block_workspace_bytes(B, C, T))
    # narrow widths, 3 taps below 192 channels: the direct kernels only
    assert q(2, 12, 5000, 7) == plain(2, 12, 5000)
    assert q(2, 64, 5000, 3) == plain(2, 64, 5000)
    # 3 taps at 512 channels on long rows, 7 taps from 48 channels: spectra
    # of 128 slots x 2 floats per (channel, 16-padded column) in each of the
    # three slots, plus one convolution's 256 C^2 packed floats
    for B, C, T, K in ((2, 512, 65536, 3), (2, 48, 5000, 7), (1, 96, 9000, 11)):
        L_blk = 256 - (K - 1) * 5
        cols = B * -(-T // L_blk)
        spec_lb = 256 * C * (-(-cols // 16) * 16) * 4
        got = q(B, C, T, K)
        assert got >= 3 * spec_lb + 256 * C * C * 4, (B, C, T, K)
        assert got > plain(B, C, T)
    # 3 taps on short rows (fewer than 64 columns) stay direct
    assert q(1, 256, 2000, 3) == plain(1, 256, 2000)
    # invalid arguments
    assert q(0, 512, 100, 3) == 0
    assert q(1, 512, 100, 3, n=0) == 0
    assert q(1, 512, 100, 3, n=5) == 0
    assert q(1, 512, 100, 3, d=None) == 0
