"""Thin ctypes binding over libavae.so (see include/avae.h).

Argument marshalling only: every step of the decoder runs in the library's
HIP kernels.  PyTorch provides device memory (``tensor.data_ptr()``) and the
stream (``torch.cuda.current_stream().cuda_stream``).  There is no fallback:
if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# AVAE_LIB_PATH selects another build of the same library (the host-sanitized
# check build); a missing file raises like a missing default.
LIB_PATH = os.environ.get("AVAE_LIB_PATH") or os.path.join(_HERE, "libavae.so")

AVAE_FILTER_LEN = 12
AVAE_MAX_STAGES = 8
AVAE_MAX_KERNELS = 4
AVAE_MAX_DIL = 4
FINAL = {"none": 0, "tanh": 1, "clamp": 2}

c_int, c_float, c_double, c_size_t, c_void_p = (ctypes.c_int, ctypes.c_float, ctypes.c_double,
                                                ctypes.c_size_t, ctypes.c_void_p)
P = c_void_p


class AvaeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libavae error {code}: {msg}")
        self.code = code


class avae_config(ctypes.Structure):
    _fields_ = [
        ("c_in", c_int), ("dec_in_ch", c_int), ("has_latent_affine", c_int),
        ("k_pre", c_int), ("k_post", c_int), ("n_stages", c_int),
        ("ch", c_int * (AVAE_MAX_STAGES + 1)),
        ("rates", c_int * AVAE_MAX_STAGES), ("up_k", c_int * AVAE_MAX_STAGES),
        ("n_kernels", c_int), ("rb_k", c_int * AVAE_MAX_KERNELS), ("n_dil", c_int),
        ("rb_d", (c_int * AVAE_MAX_DIL) * AVAE_MAX_KERNELS), ("final_act", c_int),
    ]


_W3 = ((P * AVAE_MAX_DIL) * AVAE_MAX_KERNELS) * AVAE_MAX_STAGES
_A3 = ((P * (2 * AVAE_MAX_DIL)) * AVAE_MAX_KERNELS) * AVAE_MAX_STAGES


class avae_weights(ctypes.Structure):
    _fields_ = [
        ("latent_mean", P), ("latent_std", P), ("dec_in_w", P), ("dec_in_b", P),
        ("conv_pre_w", P), ("conv_pre_b", P),
        ("up_w", P * AVAE_MAX_STAGES), ("up_b", P * AVAE_MAX_STAGES),
        ("w1", _W3), ("b1", _W3), ("w2", _W3), ("b2", _W3),
        ("act_la", _A3), ("act_lb", _A3),
        ("post_la", P), ("post_lb", P), ("conv_post_w", P), ("conv_post_b", P),
    ]


class avae_dav_config(ctypes.Structure):
    _fields_ = [
        ("c_side", c_int), ("dec_in_ch", c_int), ("k_pre", c_int), ("k_post", c_int),
        ("n_stages", c_int), ("ch", c_int * (AVAE_MAX_STAGES + 1)),
        ("strides", c_int * AVAE_MAX_STAGES), ("up_k", c_int * AVAE_MAX_STAGES),
        ("unit_k", c_int), ("n_units", c_int), ("unit_dil", c_int * AVAE_MAX_DIL),
    ]


_U2 = (P * AVAE_MAX_DIL) * AVAE_MAX_STAGES


class avae_dav_weights(ctypes.Structure):
    _fields_ = [
        ("dec_in_w", P), ("dec_in_b", P), ("conv_pre_w", P), ("conv_pre_b", P),
        ("stage_alpha", P * AVAE_MAX_STAGES), ("up_w", P * AVAE_MAX_STAGES),
        ("up_b", P * AVAE_MAX_STAGES),
        ("a1", _U2), ("w1", _U2), ("b1", _U2), ("a2", _U2), ("w2", _U2), ("b2", _U2),
        ("post_alpha", P), ("conv_post_w", P), ("conv_post_b", P),
    ]


class avae_bwe_config(ctypes.Structure):
    _fields_ = [("gen", avae_config), ("filter_len", c_int), ("hop", c_int), ("n_freqs", c_int),
                ("n_mels", c_int), ("ratio", c_int)]


class avae_bwe_weights(ctypes.Structure):
    _fields_ = [("gen", avae_weights), ("forward_basis", P), ("mel_basis", P)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -m bigvgan_waveform_decoder_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    L.avae_last_error.restype = ctypes.c_char_p
    L.avae_last_error.argtypes = []
    L.avae_version.restype = c_int
    L.avae_kaiser_sinc.restype = c_int
    L.avae_kaiser_sinc.argtypes = [c_double, c_double, c_int, P]
    L.avae_act1d.restype = c_int
    L.avae_act1d.argtypes = [P, P, c_int, c_int, c_int, P, P, P, P, P]
    L.avae_conv1d.restype = c_int
    L.avae_conv1d.argtypes = [P, P, c_int, c_int, c_int, c_int, P, P, c_int, c_int, c_int, P, P]
    L.avae_conv1d_fft_weight_floats.restype = c_size_t
    L.avae_conv1d_fft_weight_floats.argtypes = [c_int, c_int]
    L.avae_conv1d_fft_pack.restype = c_int
    L.avae_conv1d_fft_pack.argtypes = [P, P, c_int, c_int, c_int, c_int, P]
    L.avae_conv1d_fft_workspace_bytes.restype = c_size_t
    L.avae_conv1d_fft_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int]
    L.avae_conv1d_fft.restype = c_int
    L.avae_conv1d_fft.argtypes = [P, P, c_int, c_int, c_int, c_int, P, P, c_int, c_int, P, P,
                                  c_size_t, P]
    L.avae_act_conv1d_fft.restype = c_int
    L.avae_act_conv1d_fft.argtypes = [P, P, c_int, c_int, c_int, c_int, P, P, P, P, c_int, c_int,
                                      P, P, c_size_t, P]
    L.avae_convtr1d.restype = c_int
    L.avae_convtr1d.argtypes = [P, P, c_int, c_int, c_int, c_int, P, P, c_int, c_int, c_int, P]
    L.avae_amp_block_workspace_bytes.restype = c_size_t
    L.avae_amp_block_workspace_bytes.argtypes = [c_int, c_int, c_int]
    L.avae_amp_block_fft_workspace_bytes.restype = c_size_t
    L.avae_amp_block_fft_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, P]
    L.avae_amp_block.restype = c_int
    L.avae_amp_block.argtypes = [P, P, c_int, c_int, c_int, c_int, c_int, P, P, P, P, P, P, P,
                                 c_float, c_int, P, c_size_t, P]
    L.avae_amp_block_static_max_bytes.restype = c_size_t
    L.avae_amp_block_static_max_bytes.argtypes = []
    L.avae_amp_block_static.restype = c_int
    L.avae_amp_block_static.argtypes = [P, P, c_int, c_int, c_int, c_int, c_int, P, P, P, P, P,
                                        P, P, c_float, c_int, P]
    L.avae_decoder_create.restype = c_int
    L.avae_decoder_create.argtypes = [ctypes.POINTER(avae_config), ctypes.POINTER(avae_weights),
                                      ctypes.POINTER(P)]
    L.avae_decoder_destroy.restype = None
    L.avae_decoder_destroy.argtypes = [P]
    L.avae_decoder_output_length.restype = c_int
    L.avae_decoder_output_length.argtypes = [P, c_int, ctypes.POINTER(c_int)]
    L.avae_decoder_workspace_bytes.restype = c_size_t
    L.avae_decoder_workspace_bytes.argtypes = [P, c_int, c_int]
    L.avae_decoder_set_concurrent.restype = c_int
    L.avae_decoder_set_concurrent.argtypes = [P, c_int]
    L.avae_probe_mfma.restype = c_int
    L.avae_probe_mfma.argtypes = [c_int, c_int, c_int, P, P]
    L.avae_probe_copy.restype = c_int
    L.avae_probe_copy.argtypes = [P, P, ctypes.c_longlong, P]
    L.avae_bigvgan_decode.restype = c_int
    L.avae_bigvgan_decode.argtypes = [P, P, c_int, c_int, P, P, c_size_t, P]
    L.avae_bigvgan_decode_traced.restype = c_int
    L.avae_bigvgan_decode_traced.argtypes = [P, P, c_int, c_int, P, P, c_size_t, P, P]
    L.avae_mel_stft.restype = c_int
    L.avae_mel_stft.argtypes = [P, P, c_int, c_int, P, c_int, c_int, c_int, P, c_int, P]
    L.avae_hann_sinc_upsample.restype = c_int
    L.avae_hann_sinc_upsample.argtypes = [P, P, c_int, c_int, c_int, P]
    L.avae_bwe_create.restype = c_int
    L.avae_bwe_create.argtypes = [P, P, P]
    L.avae_bwe_destroy.restype = None
    L.avae_bwe_destroy.argtypes = [P]
    L.avae_bwe_workspace_bytes.restype = c_size_t
    L.avae_bwe_workspace_bytes.argtypes = [P, c_int, c_int]
    L.avae_bwe_decode.restype = c_int
    L.avae_bwe_decode.argtypes = [P, P, c_int, c_int, P, P, c_size_t, P]
    L.avae_bwe_decode_traced.restype = c_int
    L.avae_bwe_decode_traced.argtypes = [P, P, c_int, c_int, P, P, c_size_t, P, P, P]
    L.avae_snake.restype = c_int
    L.avae_snake.argtypes = [P, P, c_int, c_int, c_int, P, P]
    L.avae_dav_create.restype = c_int
    L.avae_dav_create.argtypes = [P, P, P]
    L.avae_dav_destroy.restype = None
    L.avae_dav_destroy.argtypes = [P]
    L.avae_dav_output_length.restype = c_int
    L.avae_dav_output_length.argtypes = [P, c_int, ctypes.POINTER(c_int)]
    L.avae_dav_workspace_bytes.restype = c_size_t
    L.avae_dav_workspace_bytes.argtypes = [P, c_int, c_int]
    L.avae_dav_decode.restype = c_int
    L.avae_dav_decode.argtypes = [P, P, c_int, c_int, P, P, c_size_t, P]
    L.avae_dav_decode_traced.restype = c_int
    L.avae_dav_decode_traced.argtypes = [P, P, c_int, c_int, P, P, c_size_t, P, P]
    L.avae_decoder_reach_frames.restype = c_int
    L.avae_decoder_reach_frames.argtypes = [P, ctypes.POINTER(c_int)]
    L.avae_decoder_streaming_workspace_bytes.restype = c_size_t
    L.avae_decoder_streaming_workspace_bytes.argtypes = [P, c_int, c_int, c_int]
    L.avae_bigvgan_decode_streaming.restype = c_int
    L.avae_bigvgan_decode_streaming.argtypes = [P, P, c_int, c_int, P, c_int, c_int, P, c_size_t, P]
    L.avae_profile_begin.restype = c_int
    L.avae_profile_begin.argtypes = [c_int]
    L.avae_profile_end.restype = c_int
    L.avae_profile_end.argtypes = []
    L.avae_profile_count.restype = c_int
    L.avae_profile_count.argtypes = []
    L.avae_profile_entry.restype = c_int
    L.avae_profile_entry.argtypes = [c_int, ctypes.c_char_p, c_int,
                                     ctypes.POINTER(ctypes.c_longlong),
                                     ctypes.POINTER(c_double), ctypes.POINTER(c_double),
                                     ctypes.POINTER(c_double)]
    L.avae_profile_phases.restype = c_int
    L.avae_profile_phases.argtypes = [ctypes.POINTER(c_double)]
    _lib = L
    return L


def _check(rc: int):
    if rc != 0:
        raise AvaeError(rc, lib().avae_last_error().decode())


# ------------------------------------------------------------------ helpers

def _torch():
    import torch
    return torch


def _dev(t, name: str, shape: Optional[Sequence[int]] = None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if t.dtype != torch.float32:
        raise ValueError(f"{name}: must be float32, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _opt(t, name, shape=None):
    return None if t is None else _dev(t, name, shape)


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _host_taps(taps):
    if taps is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(taps, dtype=np.float32))
    if a.shape != (AVAE_FILTER_LEN,):
        raise ValueError(f"taps must have {AVAE_FILTER_LEN} entries")
    return a, a.ctypes.data


# ------------------------------------------------------------------ entry points

def version() -> int:
    return lib().avae_version()


PHASES = ("dec_in", "conv_pre", "upsamples", "resblocks", "act_post", "conv_post")


def profile_begin(max_launches: int):
    """Open a profiled region (avae_profile_begin)."""
    _check(lib().avae_profile_begin(int(max_launches)))


def profile_end():
    """Close the region; returns (per-kernel dict, per-phase ms dict).
    Per kernel: launches, total_ms, flops, bytes (algorithmic, summed)."""
    L = lib()
    _check(L.avae_profile_end())
    out = {}
    for i in range(L.avae_profile_count()):
        name = ctypes.create_string_buffer(256)
        n = ctypes.c_longlong()
        ms, fl, by = c_double(), c_double(), c_double()
        _check(L.avae_profile_entry(i, name, 256, ctypes.byref(n), ctypes.byref(ms),
                                    ctypes.byref(fl), ctypes.byref(by)))
        out[name.value.decode()] = {"launches": n.value, "total_ms": ms.value,
                                    "flops": fl.value, "bytes": by.value}
    ph = (c_double * 6)()
    _check(L.avae_profile_phases(ph))
    return out, dict(zip(PHASES, list(ph)))


def kaiser_sinc(cutoff: float = 0.25, half_width: float = 0.3, taps: int = 12) -> np.ndarray:
    out = np.zeros(max(int(taps), 1), dtype=np.float32)
    _check(lib().avae_kaiser_sinc(cutoff, half_width, int(taps), out.ctypes.data))
    return out


def act1d(x, log_alpha, log_beta, up_taps=None, down_taps=None, out=None, stream=None):
    """avae_act1d: [B, C, T] -> [B, C, T]."""
    torch = _torch()
    B, C, T = x.shape
    px = _dev(x, "x")
    if out is None:
        out = torch.empty_like(x)
    py = _dev(out, "out", (B, C, T))
    ua, up = _host_taps(up_taps)
    da, dp = _host_taps(down_taps)
    _check(lib().avae_act1d(px, py, B, C, T, _dev(log_alpha, "log_alpha", (C,)),
                            _dev(log_beta, "log_beta", (C,)), up, dp, _stream(stream)))
    return out


def conv1d(x, w, bias=None, dilation: int = 1, pad: Optional[int] = None, residual=None,
           out=None, stream=None):
    """avae_conv1d; pad defaults to the 'same' padding (K*d - d)/2."""
    torch = _torch()
    B, Cin, T = x.shape
    Cout, Cin_w, K = w.shape
    if Cin_w != Cin:
        raise ValueError(f"weight has {Cin_w} input channels, x has {Cin}")
    if pad is None:
        pad = (K * dilation - dilation) // 2
    Tout = T + 2 * pad - dilation * (K - 1)
    if out is None:
        out = torch.empty((B, Cout, max(Tout, 0)), device=x.device, dtype=torch.float32)
    _check(lib().avae_conv1d(_dev(x, "x"), _dev(out, "out", (B, Cout, Tout)), B, Cin, Cout, T,
                             _dev(w, "w"), _opt(bias, "bias", (Cout,)), K, dilation, pad,
                             _opt(residual, "residual", (B, Cout, Tout)), _stream(stream)))
    return out


def conv1d_fft_pack(w, dilation: int = 1, out=None, stream=None):
    """avae_conv1d_fft_pack: w [Cout, Cin, K] -> packed frequency-domain weights."""
    torch = _torch()
    Cout, Cin, K = w.shape
    n = int(lib().avae_conv1d_fft_weight_floats(Cin, Cout))
    if out is None:
        out = torch.empty((n,), device=w.device, dtype=torch.float32)
    _check(lib().avae_conv1d_fft_pack(_dev(w, "w"), _dev(out, "out", (n,)), Cin, Cout, K,
                                      dilation, _stream(stream)))
    return out


def conv1d_fft_workspace_bytes(B: int, Cin: int, Cout: int, T: int, K: int,
                               dilation: int = 1) -> int:
    return int(lib().avae_conv1d_fft_workspace_bytes(B, Cin, Cout, T, K, dilation))


def conv1d_fft(x, wp, Cout: int, K: int, bias=None, dilation: int = 1, residual=None, out=None,
               workspace=None, stream=None):
    """avae_conv1d_fft: 'same'-padded Conv1d with weights packed by conv1d_fft_pack."""
    torch = _torch()
    B, Cin, T = x.shape
    if out is None:
        out = torch.empty((B, Cout, T), device=x.device, dtype=torch.float32)
    need = conv1d_fft_workspace_bytes(B, Cin, Cout, T, K, dilation)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), device=x.device, dtype=torch.uint8)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise ValueError("workspace must be a uint8 device tensor")
    _check(lib().avae_conv1d_fft(_dev(x, "x"), _dev(out, "out", (B, Cout, T)), B, Cin, Cout, T,
                                 _dev(wp, "wp"), _opt(bias, "bias", (Cout,)), K, dilation,
                                 _opt(residual, "residual", (B, Cout, T)),
                                 workspace.data_ptr(), workspace.numel(),
                                 _stream(stream)))
    return out


def act_conv1d_fft(x, log_alpha, log_beta, wp, Cout: int, K: int, bias=None, dilation: int = 1,
                   residual=None, out=None, workspace=None, stream=None):
    """avae_act_conv1d_fft: conv1d_fft of act1d(x) (designed taps), one pass."""
    torch = _torch()
    B, Cin, T = x.shape
    if out is None:
        out = torch.empty((B, Cout, T), device=x.device, dtype=torch.float32)
    need = conv1d_fft_workspace_bytes(B, Cin, Cout, T, K, dilation)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), device=x.device, dtype=torch.uint8)
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise ValueError("workspace must be a uint8 device tensor")
    _check(lib().avae_act_conv1d_fft(
        _dev(x, "x"), _dev(out, "out", (B, Cout, T)), B, Cin, Cout, T,
        _dev(log_alpha, "log_alpha", (Cin,)), _dev(log_beta, "log_beta", (Cin,)), _dev(wp, "wp"),
        _opt(bias, "bias", (Cout,)), K, dilation, _opt(residual, "residual", (B, Cout, T)),
        workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out


def convtr1d(x, w, bias=None, stride: int = 1, pad: int = -1, out=None, stream=None):
    """avae_convtr1d; pad < 0 selects (K - stride)/2."""
    torch = _torch()
    B, Cin, Tin = x.shape
    Cin_w, Cout, K = w.shape
    if Cin_w != Cin:
        raise ValueError(f"weight has {Cin_w} input channels, x has {Cin}")
    p = (K - stride) // 2 if pad < 0 else pad
    Tout = (Tin - 1) * stride + K - 2 * p
    if out is None:
        out = torch.empty((B, Cout, max(Tout, 0)), device=x.device, dtype=torch.float32)
    _check(lib().avae_convtr1d(_dev(x, "x"), _dev(out, "out", (B, Cout, Tout)), B, Cin, Cout, Tin,
                               _dev(w, "w"), _opt(bias, "bias", (Cout,)), K, stride, pad,
                               _stream(stream)))
    return out


def amp_block_workspace_bytes(B: int, C: int, T: int) -> int:
    return int(lib().avae_amp_block_workspace_bytes(B, C, T))


def amp_block_fft_workspace_bytes(B: int, C: int, T: int, K: int, dil: Sequence[int]) -> int:
    n = len(dil)
    dil_a = (c_int * n)(*[int(d) for d in dil])
    return int(lib().avae_amp_block_fft_workspace_bytes(B, C, T, K, n, ctypes.addressof(dil_a)))


def amp_block(x, K: int, dil: Sequence[int], w1: List, b1: List, w2: List, b2: List,
              log_alpha: List, log_beta: List, out_scale: float = 1.0, accumulate: bool = False,
              out=None, workspace=None, stream=None, fft: bool = True):
    """avae_amp_block: out = [out +] out_scale * AMP(x).  Without a workspace,
    one is allocated: sized for the frequency-domain convolutions if fft,
    else for the direct ones."""
    torch = _torch()
    B, C, T = x.shape
    n = len(dil)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out tensor")
        out = torch.empty_like(x)
    if workspace is None:
        nb = (amp_block_fft_workspace_bytes(B, C, T, K, dil) if fft
              else amp_block_workspace_bytes(B, C, T))
        workspace = torch.empty(nb, dtype=torch.uint8, device=x.device)
    dil_a = (c_int * n)(*[int(d) for d in dil])
    arr = lambda ts, nm, shape: (P * len(ts))(*[_opt(t, nm, shape) for t in ts])
    w1a = arr(w1, "w1", (C, C, K))
    b1a = arr(b1, "b1", (C,))
    w2a = arr(w2, "w2", (C, C, K))
    b2a = arr(b2, "b2", (C,))
    laa = arr(log_alpha, "log_alpha", (C,))
    lba = arr(log_beta, "log_beta", (C,))
    if len(w1) != n or len(w2) != n or len(log_alpha) != 2 * n or len(log_beta) != 2 * n:
        raise ValueError("amp_block: per-dilation lists have the wrong length")
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise ValueError("workspace must be a uint8 device tensor")
    _check(lib().avae_amp_block(
        _dev(x, "x"), _dev(out, "out", (B, C, T)), B, C, T, K, n, ctypes.addressof(dil_a),
        ctypes.addressof(w1a), ctypes.addressof(b1a), ctypes.addressof(w2a),
        ctypes.addressof(b2a), ctypes.addressof(laa), ctypes.addressof(lba), float(out_scale),
        1 if accumulate else 0, workspace.data_ptr(), workspace.numel(), _stream(stream)))
    return out


def amp_block_static_max_bytes() -> int:
    return int(lib().avae_amp_block_static_max_bytes())


def amp_block_static(x, K: int, dil: Sequence[int], w1: List, b1: List, w2: List, b2: List,
                     log_alpha: List, log_beta: List, out_scale: float = 1.0,
                     accumulate: bool = False, out=None, stream=None):
    """avae_amp_block_static: avae_amp_block with the library's static device
    scratch instead of a workspace (nothing is allocated by the library;
    `out` is allocated here only when the caller passes none)."""
    torch = _torch()
    B, C, T = x.shape
    n = len(dil)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out tensor")
        out = torch.empty_like(x)
    if len(w1) != n or len(w2) != n or len(log_alpha) != 2 * n or len(log_beta) != 2 * n:
        raise ValueError("amp_block_static: per-dilation lists have the wrong length")
    dil_a = (c_int * n)(*[int(d) for d in dil])
    arr = lambda ts, nm, shape: (P * len(ts))(*[_opt(t, nm, shape) for t in ts])
    w1a = arr(w1, "w1", (C, C, K))
    b1a = arr(b1, "b1", (C,))
    w2a = arr(w2, "w2", (C, C, K))
    b2a = arr(b2, "b2", (C,))
    laa = arr(log_alpha, "log_alpha", (C,))
    lba = arr(log_beta, "log_beta", (C,))
    _check(lib().avae_amp_block_static(
        _dev(x, "x"), _dev(out, "out", (B, C, T)), B, C, T, K, n, ctypes.addressof(dil_a),
        ctypes.addressof(w1a), ctypes.addressof(b1a), ctypes.addressof(w2a),
        ctypes.addressof(b2a), ctypes.addressof(laa), ctypes.addressof(lba), float(out_scale),
        1 if accumulate else 0, _stream(stream)))
    return out


def _decoder_structs(spec, tensors: Dict[str, "object"]):
    """avae_config and avae_weights of a BigVGAN decoder spec, weights named
    as on the H3 page."""
    cfg = avae_config()
    cfg.c_in = spec.c_in
    cfg.dec_in_ch = int(spec.dec_in)
    cfg.has_latent_affine = 1 if spec.latent_affine else 0
    cfg.k_pre, cfg.k_post = spec.k_pre, spec.k_post
    ns = len(spec.rates)
    if ns > AVAE_MAX_STAGES:
        raise ValueError("too many stages")
    cfg.n_stages = ns
    for i, c in enumerate(spec.widths()):
        cfg.ch[i] = c
    for i, (r, k) in enumerate(zip(spec.rates, spec.up_k)):
        cfg.rates[i], cfg.up_k[i] = r, k
    nk = len(spec.rb_k)
    cfg.n_kernels = nk
    nd = len(spec.rb_d[0])
    cfg.n_dil = nd
    for j in range(nk):
        cfg.rb_k[j] = spec.rb_k[j]
        if len(spec.rb_d[j]) != nd:
            raise ValueError("every AMP block needs the same number of dilations")
        for q in range(nd):
            cfg.rb_d[j][q] = spec.rb_d[j][q]
    cfg.final_act = FINAL[spec.final]
    t = tensors
    g = lambda name: _dev(t[name], name) if name in t else None
    w = avae_weights()
    w.latent_mean, w.latent_std = g("latents_mean"), g("latents_std")
    w.dec_in_w, w.dec_in_b = g("dec_in.weight"), g("dec_in.bias")
    w.conv_pre_w, w.conv_pre_b = g("conv_pre.weight"), g("conv_pre.bias")
    for i in range(ns):
        w.up_w[i], w.up_b[i] = g(f"ups.{i}.weight"), g(f"ups.{i}.bias")
        for j in range(nk):
            p = f"resblocks.{i * nk + j}"
            for q in range(nd):
                w.w1[i][j][q] = g(f"{p}.convs1.{q}.weight")
                w.b1[i][j][q] = g(f"{p}.convs1.{q}.bias")
                w.w2[i][j][q] = g(f"{p}.convs2.{q}.weight")
                w.b2[i][j][q] = g(f"{p}.convs2.{q}.bias")
            for q in range(2 * nd):
                w.act_la[i][j][q] = g(f"{p}.activations.{q}.act.alpha")
                w.act_lb[i][j][q] = g(f"{p}.activations.{q}.act.beta")
    w.post_la, w.post_lb = g("activation_post.act.alpha"), g("activation_post.act.beta")
    w.conv_post_w, w.conv_post_b = g("conv_post.weight"), g("conv_post.bias")
    return cfg, w


class Decoder:
    """avae_decoder_create / avae_bigvgan_decode over device weight tensors
    named as on the H3 page (``conv_pre.weight``, ``ups.{i}.weight``,
    ``resblocks.{i*nk+j}.convs1.{q}.weight``,
    ``resblocks.{..}.activations.{q}.act.alpha`` ...)."""

    def __init__(self, spec, tensors: Dict[str, "object"]):
        cfg, w = _decoder_structs(spec, tensors)
        self.spec = spec
        self.cfg = cfg
        h = P()
        _check(lib().avae_decoder_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.avae_decoder_destroy(h)
            self._h = None

    def output_length(self, frames: int) -> int:
        n = c_int()
        _check(lib().avae_decoder_output_length(self._h, frames, ctypes.byref(n)))
        return n.value

    def workspace_bytes(self, B: int, frames: int) -> int:
        return int(lib().avae_decoder_workspace_bytes(self._h, B, frames))

    def set_concurrent(self, on: bool) -> None:
        """Run a stage's AMP blocks overlapped on side streams (default) or
        one after the other on the caller's stream."""
        _check(lib().avae_decoder_set_concurrent(self._h, 1 if on else 0))

    def stage_shapes(self, B: int, frames: int):
        """Shapes of the traced intermediates (conv_pre, each stage, pre-final)."""
        w = self.spec.widths()
        shapes = [(B, w[0], frames)]
        T = frames
        for i, (r, k) in enumerate(zip(self.spec.rates, self.spec.up_k)):
            T = (T - 1) * r + k - 2 * ((k - r) // 2)
            shapes.append((B, w[i + 1], T))
        shapes.append((B, self.output_length(frames)))
        return shapes

    def decode(self, latent, out=None, workspace=None, stream=None, trace: bool = False):
        """latent [B, c_in, F] -> wave [B, L]; with trace=True also returns
        the list of intermediates."""
        torch = _torch()
        B, C, F = latent.shape
        if C != self.spec.c_in:
            raise ValueError(f"latent has {C} channels, decoder expects {self.spec.c_in}")
        L = self.output_length(F)
        if out is None:
            out = torch.empty((B, L), device=latent.device, dtype=torch.float32)
        if workspace is None:
            workspace = torch.empty(self.workspace_bytes(B, F), dtype=torch.uint8,
                                    device=latent.device)
        if workspace.dtype != torch.uint8 or not workspace.is_cuda:
            raise ValueError("workspace must be a uint8 device tensor")
        if not trace:
            _check(lib().avae_bigvgan_decode(self._h, _dev(latent, "latent"), B, F,
                                             _dev(out, "out", (B, L)), workspace.data_ptr(),
                                             workspace.numel(), _stream(stream)))
            return out
        stages = [torch.empty(s, device=latent.device, dtype=torch.float32)
                  for s in self.stage_shapes(B, F)]
        arr = (P * len(stages))(*[s.data_ptr() for s in stages])
        _check(lib().avae_bigvgan_decode_traced(self._h, _dev(latent, "latent"), B, F,
                                                _dev(out, "out", (B, L)), workspace.data_ptr(),
                                                workspace.numel(), ctypes.addressof(arr),
                                                _stream(stream)))
        return out, stages

    def reach_frames(self) -> int:
        n = c_int()
        _check(lib().avae_decoder_reach_frames(self._h, ctypes.byref(n)))
        return n.value

    def streaming_workspace_bytes(self, B: int, tile_frames: int, halo_frames: int = -1) -> int:
        return int(lib().avae_decoder_streaming_workspace_bytes(self._h, B, tile_frames,
                                                                  halo_frames))

    def decode_streaming(self, latent, tile_frames: int, halo_frames: int = -1, out=None,
                         workspace=None, stream=None):
        """avae_bigvgan_decode_streaming: latent [B, c_in, F] -> wave [B, F*hop] in
        tiles of tile_frames frames (halo < 0: the decoder's receptive-field reach)."""
        torch = _torch()
        B, C, F = latent.shape
        if C != self.spec.c_in:
            raise ValueError(f"latent has {C} channels, decoder expects {self.spec.c_in}")
        L = F * self.spec.hop
        if out is None:
            out = torch.empty((B, L), device=latent.device, dtype=torch.float32)
        if workspace is None:
            workspace = torch.empty(self.streaming_workspace_bytes(B, min(tile_frames, F),
                                                                   halo_frames),
                                    dtype=torch.uint8, device=latent.device)
        _check(lib().avae_bigvgan_decode_streaming(
            self._h, _dev(latent, "latent"), B, F, _dev(out, "out", (B, L)), int(tile_frames),
            int(halo_frames), workspace.data_ptr(), workspace.numel(), _stream(stream)))
        return out



def probe_mfma(chains: int, blocks: int, iters: int, sink, stream=None) -> None:
    """avae_probe_mfma: a pure FP32-MFMA loop (measurement aid); the caller
    times it.  flops = blocks * 4 * iters * chains * 2048."""
    _check(lib().avae_probe_mfma(chains, blocks, iters, _dev(sink, "sink", (blocks * 256,)),
                                 _stream(stream)))

def probe_copy(x, out, stream=None) -> None:
    """avae_probe_copy: out = x by a streaming float4 copy (measurement
    aid); the caller times it.  bytes moved = 8 * x.numel()."""
    n = x.numel()
    _check(lib().avae_probe_copy(_dev(x, "x"), _dev(out, "out", tuple(x.shape)), n,
                                 _stream(stream)))


def snake(x, alpha, out=None, stream=None):
    """avae_snake: plain Snake with alpha as stored; out may be x."""
    torch = _torch()
    B, C, T = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check(lib().avae_snake(_dev(x, "x"), _dev(out, "out", (B, C, T)), B, C, T,
                            _dev(alpha, "alpha", (C,)), _stream(stream)))
    return out


class DavDecoder:
    """avae_dav_create / avae_dav_decode over device weight tensors named as on
    the H3 page (``mvae.dec_in_proj.weight``, ``mvae.decoder.model.{i}...``)."""

    def __init__(self, spec, tensors: Dict[str, "object"]):
        cfg = avae_dav_config()
        cfg.c_side, cfg.dec_in_ch = spec.c_side, spec.dec_in
        cfg.k_pre, cfg.k_post = spec.k_pre, spec.k_post
        ns = len(spec.strides)
        cfg.n_stages = ns
        for i, c in enumerate(spec.widths()):
            cfg.ch[i] = c
        for i, (st, k) in enumerate(zip(spec.strides, spec.up_k)):
            cfg.strides[i], cfg.up_k[i] = st, k
        cfg.unit_k = spec.unit_k
        cfg.n_units = len(spec.unit_dil)
        for u, d in enumerate(spec.unit_dil):
            cfg.unit_dil[u] = d
        self.spec, self.cfg = spec, cfg
        t = tensors
        g = lambda name: _dev(t[name], name) if name in t else None
        w = avae_dav_weights()
        w.dec_in_w, w.dec_in_b = g("mvae.dec_in_proj.weight"), g("mvae.dec_in_proj.bias")
        w.conv_pre_w, w.conv_pre_b = g("mvae.decoder.model.0.weight"), g("mvae.decoder.model.0.bias")
        for i in range(ns):
            p = f"mvae.decoder.model.{i + 1}"
            w.stage_alpha[i] = g(f"{p}.block.0.alpha")
            w.up_w[i], w.up_b[i] = g(f"{p}.block.1.weight"), g(f"{p}.block.1.bias")
            for u in range(len(spec.unit_dil)):
                q = f"{p}.block.{u + 2}"
                w.a1[i][u] = g(f"{q}.block.0.alpha")
                w.w1[i][u], w.b1[i][u] = g(f"{q}.block.1.weight"), g(f"{q}.block.1.bias")
                w.a2[i][u] = g(f"{q}.block.2.alpha")
                w.w2[i][u], w.b2[i][u] = g(f"{q}.block.3.weight"), g(f"{q}.block.3.bias")
        w.post_alpha = g(f"mvae.decoder.model.{ns + 1}.alpha")
        w.conv_post_w = g(f"mvae.decoder.model.{ns + 2}.weight")
        w.conv_post_b = g(f"mvae.decoder.model.{ns + 2}.bias")
        h = P()
        _check(lib().avae_dav_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.avae_dav_destroy(h)
            self._h = None

    def output_length(self, frames: int) -> int:
        """Samples per side."""
        n = c_int()
        _check(lib().avae_dav_output_length(self._h, frames, ctypes.byref(n)))
        return n.value

    def workspace_bytes(self, B: int, frames: int) -> int:
        return int(lib().avae_dav_workspace_bytes(self._h, B, frames))

    def stage_shapes(self, B: int, frames: int):
        """Traced intermediates of the [2B, ...] side batch."""
        w = self.spec.widths()
        shapes = [(2 * B, w[0], frames)]
        T = frames
        for i, (st, k) in enumerate(zip(self.spec.strides, self.spec.up_k)):
            T = (T - 1) * st + k - 2 * ((k - st) // 2)
            shapes.append((2 * B, w[i + 1], T))
        shapes.append((2 * B, self.output_length(frames)))
        return shapes

    def decode(self, latent, out=None, workspace=None, stream=None, trace: bool = False):
        """latent [B, 2 c_side, F] -> interleaved stereo [B, 2 L]."""
        torch = _torch()
        B, C, F = latent.shape
        if C != 2 * self.spec.c_side:
            raise ValueError(f"latent has {C} channels, the DAV decoder expects "
                             f"{2 * self.spec.c_side} (two sides)")
        L = self.output_length(F)
        if out is None:
            out = torch.empty((B, 2 * L), device=latent.device, dtype=torch.float32)
        if workspace is None:
            workspace = torch.empty(self.workspace_bytes(B, F), dtype=torch.uint8,
                                    device=latent.device)
        if not trace:
            _check(lib().avae_dav_decode(self._h, _dev(latent, "latent"), B, F,
                                         _dev(out, "out", (B, 2 * L)), workspace.data_ptr(),
                                         workspace.numel(), _stream(stream)))
            return out
        stages = [torch.empty(s, device=latent.device, dtype=torch.float32)
                  for s in self.stage_shapes(B, F)]
        arr = (P * len(stages))(*[s.data_ptr() for s in stages])
        _check(lib().avae_dav_decode_traced(self._h, _dev(latent, "latent"), B, F,
                                            _dev(out, "out", (B, 2 * L)), workspace.data_ptr(),
                                            workspace.numel(), ctypes.addressof(arr),
                                            _stream(stream)))
        return out, stages


def mel_stft(x, forward_basis, mel_basis, hop: int, out=None, stream=None):
    """avae_mel_stft: x [B, T] -> causal log-mel [B, n_mels, T // hop]."""
    torch = _torch()
    B, T = x.shape
    nf2, L = forward_basis.shape
    n_mels, nf = mel_basis.shape
    if nf2 != 2 * nf:
        raise ValueError("forward_basis needs 2 n_freqs rows")
    frames = T // hop
    if out is None:
        out = torch.empty((B, n_mels, frames), device=x.device, dtype=torch.float32)
    _check(lib().avae_mel_stft(_dev(x, "x"), _dev(out, "out", (B, n_mels, frames)), B, T,
                               _dev(forward_basis, "forward_basis"), nf, L, hop,
                               _dev(mel_basis, "mel_basis"), n_mels, _stream(stream)))
    return out


def hann_sinc_upsample(x, ratio: int = 3, out=None, stream=None):
    """avae_hann_sinc_upsample: x [B, T] -> [B, ratio T]."""
    torch = _torch()
    B, T = x.shape
    if out is None:
        out = torch.empty((B, ratio * T), device=x.device, dtype=torch.float32)
    _check(lib().avae_hann_sinc_upsample(_dev(x, "x"), _dev(out, "out", (B, ratio * T)), B, T,
                                         ratio, _stream(stream)))
    return out


class BweDecoder:
    """avae_bwe_create / avae_bwe_decode: the bandwidth-extension tail, the
    generator's weights named as for Decoder, the bases as
    ``mel_stft.forward_basis`` [2 nf, L] and ``mel_stft.mel_basis`` [n_mels, nf]."""

    def __init__(self, spec, tensors: Dict[str, "object"], hop: int = 80, ratio: int = 3):
        gcfg, gw = _decoder_structs(spec, tensors)
        fb, mb = tensors["mel_stft.forward_basis"], tensors["mel_stft.mel_basis"]
        cfg = avae_bwe_config()
        cfg.gen = gcfg
        cfg.filter_len, cfg.hop, cfg.ratio = fb.shape[1], hop, ratio
        cfg.n_mels, cfg.n_freqs = mb.shape
        w = avae_bwe_weights()
        w.gen = gw
        w.forward_basis, w.mel_basis = _dev(fb, "forward_basis"), _dev(mb, "mel_basis")
        self.spec, self.cfg = spec, cfg
        h = P()
        _check(lib().avae_bwe_create(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.avae_bwe_destroy(h)
            self._h = None

    def workspace_bytes(self, B: int, T: int) -> int:
        return int(lib().avae_bwe_workspace_bytes(self._h, B, T))

    def decode(self, low, out=None, workspace=None, stream=None, trace: bool = False):
        """low [B, T] at the input rate -> [B, ratio T]; trace=True also
        returns the log-mel and the generator's residual."""
        torch = _torch()
        B, T = low.shape
        r, hop = self.cfg.ratio, self.cfg.hop
        if out is None:
            out = torch.empty((B, r * T), device=low.device, dtype=torch.float32)
        if workspace is None:
            workspace = torch.empty(self.workspace_bytes(B, T), dtype=torch.uint8,
                                    device=low.device)
        if not trace:
            _check(lib().avae_bwe_decode(self._h, _dev(low, "low"), B, T,
                                         _dev(out, "out", (B, r * T)), workspace.data_ptr(),
                                         workspace.numel(), _stream(stream)))
            return out
        frames = -(-T // hop)
        mel = torch.empty((B, self.cfg.n_mels, frames), device=low.device, dtype=torch.float32)
        res = torch.empty((B, frames * hop * r), device=low.device, dtype=torch.float32)
        _check(lib().avae_bwe_decode_traced(self._h, _dev(low, "low"), B, T,
                                            _dev(out, "out", (B, r * T)), workspace.data_ptr(),
                                            workspace.numel(), mel.data_ptr(), res.data_ptr(),
                                            _stream(stream)))
        return out, mel, res
