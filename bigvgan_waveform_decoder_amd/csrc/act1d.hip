// Fused alias-free activation (Activation1d) for gfx950.
//
// Operation ([H3] = docs.rs page of cortiq_engine/audiovae.rs, items
// Activation1d::apply, SnakeBeta and fir_pad; [LTX] = docs.rs page of
// cortiq_engine/ltxaudio.rs, Aliasing::upsample/downsample):
//   x2 upsample by replicate pad 5 / transposed FIR (stride 2, gain 2) /
//   trim 15 each side, pointwise SnakeBeta at the doubled rate, then
//   replicate pad 5 left / 6 right of the doubled signal and a stride-2 FIR.
//
// Polyphase form used here (derived from those steps, 12-tap filters):
//   the doubled-rate sample m = 2q   is  sum_k up2[2k+1] * x[clamp(q+2-k)]
//   the doubled-rate sample m = 2q+1 is  sum_k up2[2k]   * x[clamp(q+3-k)]
//   y[t] = sum_k down[2k] * s[2(t+k-3)+1] + down[2k+1] * s[2(t+k-2)]
// where s = SnakeBeta(mid) and every index of s is clamped to [0, 2T-1]
// (the down-sampler's replicate padding acts on the post-snake doubled
// signal, not on an extended upsample).  Each output therefore reads
// x[t-5 .. t+5].
//
// One block owns one (b, c) row segment of kTile outputs: it stages the
// input window in LDS (coalesced loads along time), computes each doubled-
// rate sample and its SnakeBeta exactly once into two LDS phase arrays,
// then runs the stride-2 FIR from LDS and writes the outputs once.  HBM
// traffic is one read and one write of the row (8 bytes per element).
// kTile = 8*256 - 6 so that the kTile + 6 phase positions fill every lane
// of eight passes.
//
// SnakeBeta's sine: sin(alpha v) = sin(2 pi r) with r = v * (alpha / 2 pi);
// r is reduced to [0, 1) by v_fract_f32 (exact) and v_sin_f32 evaluates
// sin(2 pi r) directly in revolutions.  Against the reduced argument the
// hardware sine is within ~1.3e-7 (measured on MI355X over [0, 1)); the only
// other error is the float32 rounding of r itself, relative ~1e-7 of the
// phase, the same order as rounding alpha*v before any float32 sine.
#include "avae_internal.h"

namespace avae {
namespace {

constexpr int kThreads = 256;
constexpr int kQ = 8 * kThreads;   // phase positions q in [t0-3, t0+kTile+3)
constexpr int kTile = kQ - 6;      // outputs per block
constexpr int kX = kTile + 12;     // input window [t0-6, t0+kTile+6)

__device__ __forceinline__ float snake_beta(float v, float alpha_rev, float inv_beta) {
    const float r = v * alpha_rev;
    const float s = __builtin_amdgcn_sinf(__builtin_amdgcn_fractf(r));
    return fmaf(s * s, inv_beta, v);
}

__global__ __launch_bounds__(kThreads) void act1d_kernel(
    const float* __restrict__ x, float* __restrict__ y, int C, int T, int tiles,
    const float* __restrict__ log_alpha, const float* __restrict__ log_beta, ActTaps taps) {
    __shared__ float xs[kX];
    __shared__ float se[kQ];  // s at even doubled-rate positions 2q
    __shared__ float so[kQ];  // s at odd doubled-rate positions 2q+1

    const int row = blockIdx.x / tiles;  // b*C + c
    const int tile = blockIdx.x - row * tiles;
    const int c = row % C;
    const int t0 = tile * kTile;
    const size_t base = (size_t)row * (size_t)T;
    const float alpha_rev = expf(log_alpha[c]) * 0.15915494309189535f;  // alpha / (2 pi)
    const float inv_beta = 1.0f / (expf(log_beta[c]) + 1e-9f);

    // Stage x[clamp(t0-6+i)]: the clamp is the upsampler's replicate padding.
    // All of a thread's loads are issued before the first LDS write, so they
    // are in flight together.
    constexpr int kLoads = (kX + kThreads - 1) / kThreads;
    float xv[kLoads];
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
        const int i = threadIdx.x + r * kThreads;
        const int t = min(max(t0 - 6 + i, 0), T - 1);
        xv[r] = (i < kX) ? x[base + t] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
        const int i = threadIdx.x + r * kThreads;
        if (i < kX) xs[i] = xv[r];
    }
    __syncthreads();

#pragma unroll
    for (int i = threadIdx.x; i < kQ; i += kThreads) {
        const int q = t0 - 3 + i;
        const int qc = min(max(q, 0), T - 1);
        const int p = qc - (t0 - 6);  // xs index of x[qc]
        float e = 0.f, o = 0.f;
#pragma unroll
        for (int k = 0; k < 6; ++k) {
            e = fmaf(taps.up2[2 * k + 1], xs[p + 2 - k], e);
            o = fmaf(taps.up2[2 * k], xs[p + 3 - k], o);
        }
        // Positions before 0 replicate s[0] (even phase at q = 0); positions
        // past 2T-1 replicate s[2T-1] (odd phase at q = T-1).
        if (q < 0) o = e;
        if (q > T - 1) e = o;
        se[i] = snake_beta(e, alpha_rev, inv_beta);
        so[i] = snake_beta(o, alpha_rev, inv_beta);
    }
    __syncthreads();

#pragma unroll
    for (int i = threadIdx.x; i < kTile; i += kThreads) {
        const int t = t0 + i;
        if (t >= T) break;
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < 6; ++k) {
            acc = fmaf(taps.down[2 * k], so[i + k], acc);
            acc = fmaf(taps.down[2 * k + 1], se[i + k + 1], acc);
        }
        y[base + t] = acc;
    }
}

}  // namespace

hipError_t launch_act1d(const float* x, float* y, int B, int C, int T,
                        const float* log_alpha, const float* log_beta,
                        const ActTaps& taps, hipStream_t stream) {
    const int tiles = (T + kTile - 1) / kTile;
    const long long blocks = (long long)B * C * tiles;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    prof_pre(stream);
    hipLaunchKernelGGL(act1d_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, x, y, C,
                       T, tiles, log_alpha, log_beta, taps);
    const hipError_t e = hipGetLastError();
    // algorithmic: 24 FMA + 2 SnakeBeta (mul, fma) per output; one read, one write
    const double n = (double)B * C * T;
    prof_post(stream, "act1d_kernel", 52.0 * n, 8.0 * n);
    return e;
}

}  // namespace avae
