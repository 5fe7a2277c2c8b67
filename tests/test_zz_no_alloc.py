"""avae_amp_block_static (the AMP block without a workspace argument, its
scratch a static device array of the library) against avae_amp_block with a
caller workspace of avae_amp_block_workspace_bytes (the direct kernels, which
the static entry point runs too): the outputs must be bit-identical.

Two calls in a row through the static scratch, the second on a smaller
input (and a narrower width, so it also takes the fused one-launch-per-step
path and packs its weights into the same array), each compared with the
workspace entry point on the same inputs; then an accumulate call; then the
size limit, which is rejected on the host before any launch."""
import numpy as np
import pytest

from bigvgan_waveform_decoder_amd import avae
from bigvgan_waveform_decoder_amd import workloads as W
from tests.gpu_util import announce, cuda, cuda_dict, host

pytestmark = pytest.mark.gpu


def _lists(td, prefix, n):
    return ([td[f"{prefix}.convs1.{q}.weight"] for q in range(n)],
            [td[f"{prefix}.convs1.{q}.bias"] for q in range(n)],
            [td[f"{prefix}.convs2.{q}.weight"] for q in range(n)],
            [td[f"{prefix}.convs2.{q}.bias"] for q in range(n)],
            [td[f"{prefix}.activations.{q}.act.alpha"] for q in range(2 * n)],
            [td[f"{prefix}.activations.{q}.act.beta"] for q in range(2 * n)])


def _case(B, C, T, K, dil, tag):
    x = W.normal(0, f"noalloc/{tag}/x", [B, C, T])
    t = W.amp_tensors(0, f"noalloc{tag}", C, K, dil, weight_var=2.0 / (C * K))
    return cuda(x), cuda_dict(t), f"noalloc{tag}"


def test_static_scratch_matches_workspace_two_calls():
    import torch
    runs = [(2, 48, 5000, 7, (1, 3, 5), "a"),   # separate launches, 3 slots of 1.9 MB
            (1, 12, 2100, 3, (1, 3, 5), "b")]   # smaller: fused unit, packed weights
    for B, C, T, K, dil, tag in runs:
        announce(f"amp_block_static B={B} C={C} T={T} K={K}")
        xd, td, prefix = _case(B, C, T, K, dil, tag)
        lists = _lists(td, prefix, len(dil))
        ref = avae.amp_block(xd, K, dil, *lists, fft=False)
        got = avae.amp_block_static(xd, K, dil, *lists)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(got), host(ref))
        assert np.all(np.isfinite(host(got)))


def test_static_scratch_accumulate_matches_workspace():
    import torch
    announce("amp_block_static accumulate")
    B, C, T, K, dil = 2, 24, 1500, 11, (1, 3, 5)
    xd, td, prefix = _case(B, C, T, K, dil, "c")
    lists = _lists(td, prefix, len(dil))
    o0 = W.normal(0, "noalloc/c/o", [B, C, T])
    ref = cuda(o0)
    got = cuda(o0)
    avae.amp_block(xd, K, dil, *lists, out_scale=0.25, accumulate=True, out=ref, fft=False)
    avae.amp_block_static(xd, K, dil, *lists, out_scale=0.25, accumulate=True, out=got)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), host(ref))


def test_static_scratch_rejects_oversize_before_launch():
    import torch
    announce("amp_block_static oversize rejected on the host")
    cap = avae.amp_block_static_max_bytes()
    assert cap == 64 << 20
    B, C, K, dil = 1, 64, 3, (1,)
    T = cap // (3 * 4 * C) + 1024          # three [B, C, T] slots exceed the array
    assert avae.amp_block_workspace_bytes(B, C, T) > cap
    x = torch.zeros((B, C, T), device="cuda:0")
    out = torch.full_like(x, 7.0)
    w = torch.zeros((C, C, K), device="cuda:0")
    p = torch.zeros((C,), device="cuda:0")
    with pytest.raises(avae.AvaeError) as ei:
        avae.amp_block_static(x, K, dil, [w], [p], [w], [p], [p, p], [p, p], out=out)
    assert ei.value.code == -2 and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())       # nothing was launched
