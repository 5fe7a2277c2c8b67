// Device math shared by the Activation1d kernels (act1d.hip, amp_unit.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace avae {

// SnakeBeta ([H3] = docs.rs page of cortiq_engine/audiovae.rs, item
// SnakeBeta): v + sin^2(alpha v) / (beta + 1e-9), with alpha_rev =
// alpha / (2 pi) and inv_beta = 1 / (beta + 1e-9) precomputed per channel.
// sin(alpha v) = sin(2 pi r), r = v * alpha_rev, by v_sin_f32, which takes
// revolutions and reduces the argument itself.  Measured on MI355X over
// 2^24 arguments up to |r| = 1e5: within 1.25e-7 of sin(2 pi frac(r)) in
// double, where reducing with v_fract_f32 first was within 3.5e-7 (a tiny
// negative r rounds to frac(r) = 1 - 2^-24) and costs one more instruction
// per evaluation.
__device__ __forceinline__ float snake_beta(float v, float alpha_rev, float inv_beta) {
    const float s = __builtin_amdgcn_sinf(v * alpha_rev);
    return fmaf(s * s, inv_beta, v);
}

// Plain Snake ([H3] page, item Snake, the Music-3 DAV decoder): alpha used
// as stored, v + sin^2(alpha v) / (alpha + 1e-9), the sine as above.
__device__ __forceinline__ float snake_plain(float v, float alpha) {
    const float s = __builtin_amdgcn_sinf(v * (alpha * 0.15915494309189535f));
    return fmaf(s * s, 1.0f / (alpha + 1e-9f), v);
}

// Per-channel SnakeBeta constants from the stored logarithms.
__device__ __forceinline__ float snake_alpha_rev(float log_alpha) {
    return expf(log_alpha) * 0.15915494309189535f;  // alpha / (2 pi)
}
__device__ __forceinline__ float snake_inv_beta(float log_beta) {
    return 1.0f / (expf(log_beta) + 1e-9f);
}

// Spreads consecutive block ids over the 8 XCDs so that each XCD works
// through a contiguous range of logical tiles (neighbouring tiles share
// their halos in that XCD's L2).
__device__ __forceinline__ int xcd_spread(int bid, int nblk) {
    const int q = nblk >> 3, r = nblk & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

}  // namespace avae
