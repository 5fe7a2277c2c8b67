// Internal launch interface between the C-ABI layer and the HIP kernels.
// Not installed; include/avae.h is the public boundary.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace avae {

constexpr int kFilterLen = 12;

// Resampling taps passed by value to the activation kernel (they land in
// scalar registers).  up2 holds the upsampling taps already multiplied by
// the x2 gain of the transposed convolution (exact: a power of two).
struct ActTaps {
    float up2[kFilterLen];
    float down[kFilterLen];
};

// Epilogue of the Conv1d kernel:
//   v   = conv + bias[o], then Snake(v, snake_alpha[o]) if given, (+ residual[idx])
//   out = v * out_scale (+ out[idx] if accumulate)
// residual may alias out (same element read then written by one lane).
struct ConvEpilogue {
    const float* bias;         // [Cout] or null
    const float* residual;     // [B, Cout, Tout] or null
    float out_scale;
    int accumulate;
    const float* snake_alpha;  // [Cout] or null: plain Snake after the bias
    const float* in_alpha;     // [Cin] or null: plain Snake of the input as it is staged
};

// Launch profiler (profile.cpp).  prof_pre/prof_post bracket one launch;
// they do nothing unless a profiled region is open.  Phases: 0 dec_in,
// 1 conv_pre, 2 upsamples, 3 resblocks, 4 act_post, 5 conv_post, -1 none.
enum Phase { kPhaseNone = -1, kPhaseDecIn = 0, kPhaseConvPre = 1, kPhaseUpsamples = 2,
             kPhaseResblocks = 3, kPhaseActPost = 4, kPhaseConvPost = 5 };
void prof_set_phase(int phase);
void prof_pre(hipStream_t s);
void prof_post(hipStream_t s, const char* name, double flops, double bytes);

// Host-side float64 Kaiser-sinc design (filter_design.cpp).
void design_kaiser_sinc(double cutoff, double half_width, int taps, double* out);
// Host-side float64 Hann-sinc interpolator taps; returns the tap count
// (out may be null to query it).
int design_hann_sinc(int ratio, double rolloff, double lpw, double* out);

// y is written with non-temporal stores (not kept in the caches).
hipError_t launch_act1d(const float* x, float* y, int B, int C, int T,
                        const float* log_alpha, const float* log_beta,
                        const ActTaps& taps, hipStream_t stream);

// Returns hipErrorInvalidValue if the shape needs more LDS than a block has.
hipError_t launch_conv1d(const float* x, float* y, const float* w, int B, int Cin, int Cout,
                         int T, int Tout, int K, int dilation, int pad,
                         const ConvEpilogue& ep, hipStream_t stream);

// in_alpha: [Cin] or null, plain Snake applied to the input as it is staged.
hipError_t launch_convtr1d(const float* x, float* y, const float* w, const float* bias,
                           int B, int Cin, int Cout, int Tin, int Tout, int K, int stride,
                           int pad, hipStream_t stream, const float* in_alpha = nullptr);

// Conv1d through 256-point overlap-save transforms (fftconv.hip), "same"
// padding, shapes that plan::fft_supported takes.  wp holds
// fft_conv_weight_floats(Cin, Cout) floats from launch_fft_pack; xspec and
// yspec plan::fft_spectrum_bytes(B, Cin | Cout, T, K, d) bytes each.  With
// act_log_alpha, act_log_beta and act_taps all given, the convolution's
// input is Activation1d(x) (as launch_act1d computes it), evaluated inside
// the forward transforms; else with ep.in_alpha, the plain Snake of x there.
// ep.snake_alpha applies the plain Snake after the bias, as launch_conv1d.
size_t fft_conv_weight_floats(int Cin, int Cout);
hipError_t launch_fft_pack(const float* w, float* wp, int Cin, int Cout, int K, int dilation,
                           hipStream_t s);
hipError_t launch_conv1d_fft(const float* x, float* y, const float* wp, int B, int Cin, int Cout,
                             int T, int K, int dilation, const ConvEpilogue& ep, float* xspec,
                             float* yspec, hipStream_t s, const float* act_log_alpha = nullptr,
                             const float* act_log_beta = nullptr,
                             const ActTaps* act_taps = nullptr);

// Conv1d to a single output channel ("same" padding, odd K) followed by the
// final nonlinearity (0 none, 1 tanh, 2 clamp to [-1,1]).  pre_final, if not
// null, also receives the value before the nonlinearity ([B, T]).  With
// interleave2, input rows 2b and 2b+1 are the two stereo sides of output
// row b, written interleaved: y[b][2t + side].
hipError_t launch_conv_out1(const float* x, float* y, float* pre_final, const float* w,
                            const float* bias, int B, int Cin, int T, int K, int final_act,
                            int interleave2, hipStream_t stream,
                            const float* in_alpha = nullptr);

// Plain Snake (snake.hip): y = x + sin^2(alpha_c x) / (alpha_c + 1e-9).
hipError_t launch_snake(const float* x, float* y, int B, int C, int T, const float* alpha,
                        hipStream_t stream);

// Fused AMP unit (amp_unit.hip): y = x + conv2(act2(conv1(act1(x)))) for one
// dilation step, then y * out_scale (+ y_old if accumulate).  Narrow widths
// only (amp_unit_supported); the weights come packed by
// launch_pack_unit_weights into amp_unit_packed_floats(C, K) floats.  x and y
// must not overlap.
bool amp_unit_supported(int C, int K, int dilation);
size_t amp_unit_packed_floats(int C, int K);
hipError_t launch_pack_unit_weights(const float* w, float* wt, int C, int K, hipStream_t s);
// n <= 8 weights of one (C, K) packed in one launch.
hipError_t launch_pack_unit_weights_n(const float* const* w, float* const* wt, int n, int C,
                                      int K, hipStream_t s);
hipError_t launch_amp_unit(const float* x, float* y, const float* wt1, const float* b1,
                           const float* wt2, const float* b2, const float* la1, const float* lb1,
                           const float* la2, const float* lb2, int B, int C, int T, int K,
                           int dilation, float out_scale, int accumulate, const ActTaps& taps,
                           hipStream_t stream);

// Causal log-mel (bwe.hip): x [B, T] (zero beyond T) -> out [B, n_mels,
// frames], frame f covering padded samples [f hop, f hop + L) with L - hop
// zeros on the left; basis [2 nf, L], mel [n_mels, nf].
hipError_t launch_mel_stft(const float* x, float* out, int B, int T, int frames,
                           const float* basis, int nf, int L, int hop, const float* mel,
                           int n_mels, hipStream_t stream);
// out[b, t] (t < Lout) = [clamp](resid[b, t] + skip(t)), skip the x`ratio`
// interpolation (k host taps) of x zero-extended from T to Tp samples and
// replicate-padded; resid may be null (skip alone).
hipError_t launch_bwe_combine(const float* x, const float* resid, float* out, int B, int T,
                              int Tp, int Lres, int Lout, int ratio, const float* taps_host,
                              int k, int do_clamp, hipStream_t stream);

// y[i] += x[0][i] + ... + x[n-1][i] for i < count (n <= 3): the MRF sum of
// AMP blocks that ran concurrently into separate buffers.
hipError_t launch_sum_into(float* y, float* const* x, int n, size_t count, hipStream_t stream);

// Matrix-core throughput probe (probe.hip): `blocks` workgroups of 256
// threads, each wave running `chains` (8 or 16) independent FP32 MFMA
// accumulator chains for `iters` iterations; sink gets blocks*256 floats.
hipError_t launch_mfma_probe(int chains, int blocks, int iters, float* sink, hipStream_t s);
hipError_t launch_stream_copy(const float* x, float* y, long long n4, hipStream_t s);

// y[b,c,t] = x[b,c,t] * scale[c] + shift[c]
hipError_t launch_channel_affine(const float* x, float* y, const float* scale,
                                 const float* shift, int B, int C, int T, hipStream_t stream);

}  // namespace avae
