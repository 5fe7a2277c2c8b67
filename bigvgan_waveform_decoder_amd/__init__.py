"""MI355X-native BigVGAN waveform decoder (alias-free AMP), gfx950.

The compute lives in ``libavae.so`` (HIP kernels behind a C-ABI, header
``include/avae.h``); ``bigvgan_waveform_decoder_amd.avae`` is the thin ctypes
binding with the same entry-point names.  Importing the package itself loads
nothing: the binding loads the library on first use and raises if it is
missing.
"""
__all__ = ["avae", "workloads"]
