// LTX bandwidth-extension tail ([LTX] = docs.rs page of
// cortiq_engine/ltxaudio.rs, items MelStft, hann_sinc_upsample and
// AudioStack::decode_from_mel), gfx950.
//
// mel_stft_kernel: the causal log-mel the extension generator reads.  The
// STFT is a GEMM Z = basis [2 nf x L] . frames [L x F] with frame f of the
// (L - hop)-left-padded signal starting at f hop; a block owns 32 frames:
// it stages their samples (32 hop + L - hop floats) in LDS once, and each
// wave owns 16-frequency groups, accumulating the real rows r and the
// imaginary rows nf + r of a group in two MFMA tiles with the same lane
// layout, so |Z| is formed in registers.  The magnitudes go to LDS, the mel
// projection (n_mels x nf) and ln(max(., 1e-5)) run on the vector ALUs.
//
// bwe_combine_kernel: out = clamp(residual + skip, -1, 1), where skip is the
// x3 Hann-sinc interpolation of the hop-padded 16 kHz signal, evaluated in
// polyphase form straight from the signal: skip[t] = sum_m ratio * h[a_m] *
// x[clamp((t + ratio w - a_m) / ratio)], a_m = ((t + 2 ratio w) mod ratio)
// + ratio m (derived from the page's pad / transposed-FIR / crop steps).
#include <hip/hip_runtime.h>

#include "avae_internal.h"

namespace avae {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMT = 256;      // threads per block
constexpr int kMF = 32;       // frames per block
constexpr int kMaxTaps = 64;  // interpolator taps passed by value
constexpr int kRing = 8;      // STFT basis steps loaded ahead

__global__ __launch_bounds__(kMT) void mel_stft_kernel(
    const float* __restrict__ x, float* __restrict__ out, int T, int frames, int fblocks,
    const float* __restrict__ basis, int nf, int L, int hop, const float* __restrict__ mel,
    int n_mels, int xs_len) {
    extern __shared__ __align__(16) float sm[];
    float* xs = sm;                          // [xs_len]: padded signal from f0*hop
    float* mag = sm + ((xs_len + 3) & ~3);   // [nf][kMF]
    const int b = blockIdx.x / fblocks;
    const int f0 = (blockIdx.x - b * fblocks) * kMF;
    const int left = L - hop;
    const float* xb = x + (size_t)b * T;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    // padded index p = f0*hop + u  <->  signal index p - left (zero outside [0, T))
    for (int u = tid; u < xs_len; u += kMT) {
        const int s = f0 * hop + u - left;
        xs[u] = (s >= 0 && s < T) ? xb[s] : 0.f;
    }
    __syncthreads();
    const int groups = (nf + 15) / 16;
    for (int gq = wid; gq < groups; gq += 4) {
        const int r0 = gq * 16;
        f32x4 re[2], im[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            re[c] = f32x4{0.f, 0.f, 0.f, 0.f};
            im[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const int r = r0 + l16;  // A row of this lane
        const int rc = min(r, nf - 1);
        const float sel = r < nf ? 1.f : 0.f;
        // A (basis) comes from L2: kRing steps of it are loaded one ring ahead
        // of the MFMAs that use them (the copy at the end of a ring waits on
        // loads issued a whole ring earlier).  L is a multiple of 4 * kRing.
        const float* are = basis + (size_t)rc * L + g4;
        const float* aim = basis + (size_t)(nf + rc) * L + g4;
        float cre[kRing], cim[kRing], nre[kRing], nim[kRing];
#pragma unroll
        for (int i = 0; i < kRing; ++i) {
            cre[i] = are[4 * i];
            cim[i] = aim[4 * i];
        }
        for (int j0 = 0; j0 < L; j0 += 4 * kRing) {
            const int jn = j0 + 4 * kRing < L ? j0 + 4 * kRing : j0;
#pragma unroll
            for (int i = 0; i < kRing; ++i) {
                nre[i] = are[jn + 4 * i];
                nim[i] = aim[jn + 4 * i];
            }
#pragma unroll
            for (int i = 0; i < kRing; ++i) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    // B[k = g4][n = l16] = sample j0 + 4i + g4 of frame f0 + 16c + l16
                    const float bv = xs[(16 * c + l16) * hop + j0 + 4 * i + g4];
                    re[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(cre[i] * sel, bv, re[c], 0, 0, 0);
                    im[c] = __builtin_amdgcn_mfma_f32_16x16x4f32(cim[i] * sel, bv, im[c], 0, 0, 0);
                }
            }
#pragma unroll
            for (int i = 0; i < kRing; ++i) {
                cre[i] = nre[i];
                cim[i] = nim[i];
            }
        }
        // D[4 g4 + i][l16]: frequency r0 + 4 g4 + i, frame 16 c + l16
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = r0 + 4 * g4 + i;
                if (rr < nf)
                    mag[rr * kMF + 16 * c + l16] = sqrtf(re[c][i] * re[c][i] + im[c][i] * im[c][i]);
            }
    }
    __syncthreads();
    float* ob = out + (size_t)b * n_mels * frames;
    for (int e = tid; e < n_mels * kMF; e += kMT) {
        const int m = e / kMF, f = e - m * kMF;
        if (f0 + f >= frames) continue;
        const float* mr = mel + (size_t)m * nf;
        float acc = 0.f;
        for (int k = 0; k < nf; ++k) acc = fmaf(mr[k], mag[k * kMF + f], acc);
        ob[(size_t)m * frames + f0 + f] = logf(fmaxf(acc, 1e-5f));
    }
}

struct InterpTaps {
    float h[kMaxTaps];  // ratio * tap (the page scales the signal by ratio)
};

// x [B, T] holds the signal; xp is x zero-extended to Tp >= T.
__global__ __launch_bounds__(kMT) void bwe_combine_kernel(
    const float* __restrict__ x, const float* __restrict__ resid, float* __restrict__ out, int T,
    int Tp, int Lres, int Lout, int ratio, int w, int k, InterpTaps taps, int do_clamp) {
    const int b = blockIdx.y;
    const int t = blockIdx.x * kMT + threadIdx.x;
    if (t >= Lout) return;
    const float* xb = x + (size_t)b * T;
    // zero extension beyond T: evaluate on a bounded view
    const int a0 = (t + 2 * ratio * w) % ratio;
    float acc = 0.f;
    for (int a = a0; a < k; a += ratio) {
        const int q = min(max((t + ratio * w - a) / ratio, 0), Tp - 1);
        acc = fmaf(taps.h[a], q < T ? xb[q] : 0.f, acc);
    }
    float v = acc + (resid ? resid[(size_t)b * Lres + t] : 0.f);
    if (do_clamp) v = fminf(fmaxf(v, -1.f), 1.f);
    out[(size_t)b * Lout + t] = v;
}

}  // namespace

hipError_t launch_mel_stft(const float* x, float* out, int B, int T, int frames,
                           const float* basis, int nf, int L, int hop, const float* mel,
                           int n_mels, hipStream_t stream) {
    const int fblocks = (frames + kMF - 1) / kMF;
    const long long nblk = (long long)B * fblocks;
    if (nblk < 1 || nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    const int xs_len = (kMF - 1) * hop + L;
    const size_t lds = ((size_t)((xs_len + 3) & ~3) + (size_t)nf * kMF) * sizeof(float);
    if (lds > 64 * 1024 || L % (4 * kRing) != 0 || L < hop) return hipErrorInvalidValue;
    prof_pre(stream);
    hipLaunchKernelGGL(mel_stft_kernel, dim3((unsigned)nblk), dim3(kMT), lds, stream, x, out, T,
                       frames, fblocks, basis, nf, L, hop, mel, n_mels, xs_len);
    const hipError_t e = hipGetLastError();
    const double nfr = (double)B * frames;
    prof_post(stream, "mel_stft_kernel", nfr * (4.0 * nf * L + 2.0 * n_mels * nf),
              4.0 * ((double)B * T + nfr * n_mels));
    return e;
}

hipError_t launch_bwe_combine(const float* x, const float* resid, float* out, int B, int T,
                              int Tp, int Lres, int Lout, int ratio, const float* taps_host,
                              int k, int do_clamp, hipStream_t stream) {
    if (k > kMaxTaps || k < 1 || ratio < 1 || (k - 1) % (2 * ratio) != 0)
        return hipErrorInvalidValue;
    InterpTaps taps;
    for (int i = 0; i < kMaxTaps; ++i) taps.h[i] = i < k ? (float)ratio * taps_host[i] : 0.f;
    const int w = (k - 1) / (2 * ratio);
    dim3 grid((unsigned)((Lout + kMT - 1) / kMT), (unsigned)B);
    prof_pre(stream);
    hipLaunchKernelGGL(bwe_combine_kernel, grid, dim3(kMT), 0, stream, x, resid, out, T, Tp, Lres,
                       Lout, ratio, w, k, taps, do_clamp);
    const hipError_t e = hipGetLastError();
    const double n = (double)B * Lout;
    prof_post(stream, "bwe_combine_kernel", n * 2.0 * ((k + ratio - 1) / ratio),
              4.0 * ((double)B * T + n * (resid ? 2.0 : 1.0)));
    return e;
}

}  // namespace avae
