// Conv1d in the frequency domain (overlap-save, 256-point transforms) for
// gfx950: the same operation as the direct kernels in conv.hip, evaluated
// through the convolution theorem, so that the matrix cores do ~2 real
// multiply-adds per output and channel pair instead of K.
//
// Operation ([H3] = docs.rs page of cortiq_engine/audiovae.rs, Conv1d::apply
// and the dilated convolutions of AmpBlock::apply): "same" padding, odd K,
//   y[b,o,t] = bias[o] + sum_c sum_j w[o,c,j] x[b,c,t + j d - P],  P = (K-1)d/2,
// with x zero outside [0, T), then the epilogue of the direct kernels
// (+ residual, * out_scale, + previous y).
//
// Framing.  With span S = (K-1)d and L = N - S, output block n of a row,
// t in [nL, nL + L), only reads s_n[u] = x[nL - P + u], u in [0, N):
//   y[nL + v] = sum_j w_j s_n[v + j d],  v < L,
// a circular cross-correlation of s_n with g (g[j d] = w_j, else 0) that
// never wraps.  In the DFT domain (X_k = sum_u s[u] e^{-2 pi i k u / N}):
//   Y_k = sum_c conj(G_oc,k) X_c,k,   conj(G_k) = sum_j w_j e^{+2 pi i k j d / N},
// one complex matrix product per frequency, over the channels.  Real signals
// keep bins 0..N/2; bins 0 and N/2 are real and share slot 0 (re = bin 0,
// im = bin N/2), so there are N/2 = 128 slots, the other 127 holding bins
// 1..127.
//
// Three launches: fft_fwd_kernel (blocks of x -> X[slot][c][column]),
// fft_gemm_kernel (Y[slot] = W[slot] X[slot] on the matrix cores,
// v_mfma_f32_16x16x4_f32), fft_inv_kernel (Y -> y, epilogue).  A column is
// one (batch, block) pair, column = b nb + n.  The packed weights W come from
// fft_pack_kernel (double-precision sums, rounded once).
//
// The transforms are radix-4 Stockham FFTs (self-sorting: every stage reads
// a[j + r N/4] and writes b[4(j - k) + k + q Ns], k = j mod Ns), one wave per
// transform, lane j owning butterfly j of each of the four stages.  The
// first stage's inputs are lane j's own loads and the last stage's outputs
// are bins j + 64 q in lane j's registers, so only the three inner exchanges
// go through LDS.
#include <cstdio>

#include "act_math.h"
#include "avae_internal.h"
#include "plan.h"

namespace avae {
namespace {

constexpr int kN = 256;           // transform length
constexpr int kSlots = kN / 2;    // frequency slots (bins 0 and N/2 share slot 0)
constexpr int kCols = 16;         // transforms (columns) per transform workgroup
constexpr int kThreads = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
    return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }

// The factors of the three stages that have them (Ns = 4, 16, 64), stage by
// stage: tw[off + (r-1) Ns + k] = exp(-2 pi i r k step / N), step =
// N / (4 Ns), off = 0, 12, 60 (252 entries), from a double-precision sine
// and cosine.  Laid out by k, the lanes of a wave read consecutive entries
// (or the same one), never two entries on one LDS bank (indexed by r k step,
// up to four lanes' distinct entries shared a bank).
__device__ void init_twiddles(float2* tw) {
    for (int t = threadIdx.x; t < 252; t += blockDim.x) {
        const int Ns = t < 12 ? 4 : t < 60 ? 16 : 64;
        const int u = t - (t < 12 ? 0 : t < 60 ? 12 : 60);
        const int r = u / Ns + 1, k = u - (r - 1) * Ns;
        const int m = r * k * (kN / (4 * Ns));
        double s, c;
        sincospi(-2.0 * (double)m / (double)kN, &s, &c);
        tw[t] = make_float2((float)c, (float)s);
    }
}

// Lane j's twiddles for the three stages that have them: w[s][r-1] =
// exp(-2 pi i r k step / N), k = j mod Ns.  Read once per wave from the LDS
// table and reused for every transform of the wave.
struct LaneTwiddles {
    float2 w[3][3];
};

__device__ __forceinline__ LaneTwiddles lane_twiddles(int j, const float2* tw) {
    LaneTwiddles t;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int Ns = 4 << (2 * s);
        const int k = j & (Ns - 1);
        const int off = s == 0 ? 0 : s == 1 ? 12 : 60;
#pragma unroll
        for (int r = 1; r < 4; ++r) t.w[s][r - 1] = tw[off + (r - 1) * Ns + k];
    }
    return t;
}

// One radix-4 Stockham stage for butterfly j (sub-transform size Ns = 4^p,
// stage p; p = 0 has unit twiddles): v[r] = a[j + 64 r] on entry, the four
// outputs (positions 4(j - k) + k + q Ns, k = j mod Ns) on exit.
__device__ __forceinline__ void radix4(float2 (&v)[4], int p, const LaneTwiddles& lt) {
    if (p > 0) {
        v[1] = cmul(v[1], lt.w[p - 1][0]);
        v[2] = cmul(v[2], lt.w[p - 1][1]);
        v[3] = cmul(v[3], lt.w[p - 1][2]);
    }
    const float2 s0 = cadd(v[0], v[2]), s1 = csub(v[0], v[2]);
    const float2 s2 = cadd(v[1], v[3]), s3 = csub(v[1], v[3]);
    v[0] = cadd(s0, s2);
    v[2] = csub(s0, s2);
    v[1] = make_float2(s1.x + s3.y, s1.y - s3.x);  // s1 - i s3
    v[3] = make_float2(s1.x - s3.y, s1.y + s3.x);  // s1 + i s3
}

// Exchange-buffer index with its low four bits XORed by 5 x bits 4..5: a
// bijection on each 16-element block that puts the 16 lanes of every
// 8-byte LDS access of the exchanges of fft256 (the strided stage-0 and stage-1
// writes, the contiguous reads) on distinct banks.
__device__ __forceinline__ int swz(int i) { return i ^ (5 * ((i >> 4) & 3)); }

// Forward 256-point DFT by one wave.  Entry: lane j holds a[j + 64 r] in
// v[r]; exit: lane j holds A[j + 64 q] in v[q].  buf is this wave's own N
// complex of LDS.  LDS operations of one wave complete in issue order and
// every write depends on the reads before it, so the exchanges need no
// barrier; wave_barrier only keeps the compiler from moving them.
__device__ __forceinline__ void fft256(float2 (&v)[4], int j, float2* buf, const LaneTwiddles& lt) {
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const int Ns = 1 << (2 * p);
        radix4(v, p, lt);
        const int k = j & (Ns - 1);
        const int dst = 4 * (j - k) + k;
#pragma unroll
        for (int q = 0; q < 4; ++q) buf[swz(dst + q * Ns)] = v[q];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = buf[swz(j + 64 * r)];
        __builtin_amdgcn_wave_barrier();
    }
    radix4(v, 3, lt);  // Ns = 64, k = j: outputs j + 64 q stay in place
}

// ---------------------------------------------------------------------------
// Forward transforms.  grid (ceil(nb / kCols), C, B): workgroup = kCols
// consecutive blocks of row (b, c), four waves taking one block each in turn.
// Writes X[slot][c][b nb + n] (complex, NP columns per row).
//
// With ACT the transformed signal is Activation1d(x) ([H3] Activation1d::
// apply, SnakeBeta, fir_pad), evaluated on the block's window as it is
// loaded, in the polyphase form of act1d.hip: the doubled-rate pair at q is
//   e(q) = sum_k up2[2k+1] x[clamp(q+2-k)],  o(q) = sum_k up2[2k] x[clamp(q+3-k)],
// both through SnakeBeta (for q < 0 both phases are s[0] = e(0), for q > T-1
// both are s[2T-1] = o(T-1): the down-sampler's replicate padding), and
//   a(p) = sum_m down[2m] so(p+m-3) + down[2m+1] se(p+m-2).
// A window of 256 outputs p0 .. p0+255 needs q in [p0-3, p0+259) and x in
// [p0-6, p0+262).  The convolution's zero padding then applies to a.
constexpr int kActX = kN + 12;   // x window per transform (a multiple of 4)
constexpr int kActQ = kN + 8;    // phase pairs per transform (kN + 6, padded to 16 bytes)

struct ActIn {
    const float* log_alpha;    // [C] (mode 1)
    const float* log_beta;     // [C] (mode 1)
    ActTaps taps;              // (mode 1)
    const float* snake_alpha;  // [C] (mode 2)
};

// Input transform of the forward kernel: 0 none, 1 Activation1d (SnakeBeta
// between the resampling filters), 2 plain Snake ([H3] Snake, the DAV units:
// pointwise, alpha as stored).
template <int MODE>
__global__ __launch_bounds__(kThreads) void fft_fwd_kernel(const float* __restrict__ x,
                                                           float2* __restrict__ xf, int C, int T,
                                                           int L, int P, int nb, int NP,
                                                           ActIn act) {
    __shared__ float2 tw[kN];
    __shared__ float2 buf[kThreads / 64][kN];
    __shared__ float2 res[kSlots][kCols + 1];
    constexpr bool ACT = MODE == 1;
    __shared__ __align__(16) float aw[ACT ? kThreads / 64 : 1][ACT ? kActX + 2 * kActQ : 1];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int b = blockIdx.z, c = blockIdx.y, n0 = blockIdx.x * kCols;
    init_twiddles(tw);
    __syncthreads();
    const LaneTwiddles lt = lane_twiddles(lane, tw);
    const float* xr = x + ((size_t)b * C + c) * (size_t)T;
    constexpr int kPerWave = kCols / (kThreads / 64);
    // Two real blocks per complex transform: z = s1 + i s2, then
    // S1[k] = (Z[k] + conj(Z[N-k])) / 2, S2[k] = -i (Z[k] - conj(Z[N-k])) / 2.
    // Lane j holds Z[j + 64 q]; Z[N - j] and Z[N - 64 - j] are lane (64 - j)'s
    // q = 3 and q = 2 values (lane 0: its own), exchanged through its buffer.
    auto store_pair = [&](const float2 (&v)[4], int g1, int g2) {
        float2* bw = buf[wid];
        bw[lane] = v[2];
        bw[64 + lane] = v[3];
        __builtin_amdgcn_wave_barrier();
        const int pj = (64 - lane) & 63;
        const float2 w2 = bw[pj], w3 = bw[64 + pj];
        __builtin_amdgcn_wave_barrier();
        auto split = [&](float2 zk, float2 zm, int k) {
            // zm = Z[N - k]
            const float2 d = make_float2(zk.x - zm.x, zk.y + zm.y);  // Z[k] - conj(Z[N-k])
            res[k][g1] = make_float2(0.5f * (zk.x + zm.x), 0.5f * (zk.y - zm.y));
            res[k][g2] = make_float2(0.5f * d.y, -0.5f * d.x);
        };
        if (lane == 0) {
            // bins 0 and N/2 of both blocks are real: slot 0 = (bin 0, bin N/2)
            res[0][g1] = make_float2(v[0].x, v[2].x);
            res[0][g2] = make_float2(v[0].y, v[2].y);
            split(v[1], w3, 64);
        } else {
            split(v[0], w3, lane);
            split(v[1], w2, lane + 64);
        }
    };
    if constexpr (!ACT) {
        // every input of this wave's kCols / 4 transforms is loaded up front
        // (the loads of one transform alone leave HBM latency exposed)
        float xin[kPerWave][4];
#pragma unroll
        for (int it = 0; it < kPerWave; ++it) {
            const int u0 = (n0 + wid + (kThreads / 64) * it) * L - P + lane;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = u0 + 64 * r;
                xin[it][r] = (t >= 0 && t < T) ? xr[t] : 0.f;
            }
        }
        if constexpr (MODE == 2) {
            // plain Snake of the samples inside the row (the zero padding
            // outside stays zero)
            const float a = act.snake_alpha[c];
            const float arev = a * 0.15915494309189535f, inv = 1.0f / (a + 1e-9f);
#pragma unroll
            for (int it = 0; it < kPerWave; ++it) {
                const int u0 = (n0 + wid + (kThreads / 64) * it) * L - P + lane;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = u0 + 64 * r;
                    if (t >= 0 && t < T) xin[it][r] = snake_beta(xin[it][r], arev, inv);
                }
            }
        }
#pragma unroll
        for (int pr = 0; pr < kPerWave / 2; ++pr) {
            const int g1 = wid + (kThreads / 64) * (2 * pr), g2 = g1 + kThreads / 64;
            if (n0 + g1 >= nb) break;  // wave-uniform; no workgroup barrier until after the loop
            float2 v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = make_float2(xin[2 * pr][r], xin[2 * pr + 1][r]);
            fft256(v, lane, buf[wid], lt);
            store_pair(v, g1, g2);
        }
    } else {
        const float alpha_rev = snake_alpha_rev(act.log_alpha[c]);
        const float inv_beta = snake_inv_beta(act.log_beta[c]);
        float* xw = aw[wid];             // x[clamp(p0 - 6 + i)]
        float* se = xw + kActX;          // snake(e(q)), q = p0 - 3 + j
        float* so = se + kActQ;          // snake(o(q))
        constexpr int kXr = (kActX + 63) / 64;
        float xin[kPerWave][kXr];
#pragma unroll
        for (int it = 0; it < kPerWave; ++it) {
            const int p0 = (n0 + wid + (kThreads / 64) * it) * L - P;
#pragma unroll
            for (int r = 0; r < kXr; ++r)
                xin[it][r] = xr[min(max(p0 - 6 + lane + 64 * r, 0), T - 1)];
        }
        // the activated window of column it: av[r] = a(p0 + lane + 64 r)
        auto act_col = [&](int it, float (&av)[4]) {
            const int p0 = (n0 + wid + (kThreads / 64) * it) * L - P;
#pragma unroll
            for (int r = 0; r < kXr; ++r)
                if (lane + 64 * r < kActX) xw[lane + 64 * r] = xin[it][r];
            __builtin_amdgcn_wave_barrier();
            if (p0 >= 6 && p0 + kActX - 6 <= T) {
                // interior window: no index is clamped.  Lane l evaluates the
                // odd samples of pairs j = 4l .. 4l + 3 and the even samples of
                // pairs 4l + 1 .. 4l + 4 from xw[4l + 1 .. 4l + 9], kept one
                // pair apart (se[j] = s(2(q+1)) here, q = p0 - 3 + j), so that
                // the outputs u = 4l .. 4l + 3 read both from windows
                // so[4l .. 4l + 8], se[4l .. 4l + 8] that start on a 16-byte
                // boundary (16-byte LDS reads; a window starting one float
                // later is read 4 bytes at a time, two lanes to a bank); then
                // one LDS transposition gives the FFT its a[j + 64 r] order.
                const int j0 = 4 * lane;
                {
                    const float4* xp = reinterpret_cast<const float4*>(xw + j0);
                    const float4 w0 = xp[0], w1 = xp[1], w2 = xp[2];
                    // xw[4l] and xw[4l + 10 ..] are not used; marking them used
                    // keeps the three reads whole 16-byte LDS reads (trimmed,
                    // they become 4- and 8-byte reads that share banks)
                    asm volatile("" : : "v"(w0.x), "v"(w2.z), "v"(w2.w));
                    const float xwin[12] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y,
                                            w1.z, w1.w, w2.x, w2.y, w2.z, w2.w};
                    float ev[4], ov[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        float e = 0.f, o = 0.f;
#pragma unroll
                        for (int m = 0; m < 6; ++m) {
                            e = fmaf(act.taps.up2[2 * m + 1], xwin[k + 6 - m], e);
                            o = fmaf(act.taps.up2[2 * m], xwin[k + 6 - m], o);
                        }
                        ev[k] = snake_beta(e, alpha_rev, inv_beta);
                        ov[k] = snake_beta(o, alpha_rev, inv_beta);
                    }
                    *reinterpret_cast<float4*>(se + j0) = make_float4(ev[0], ev[1], ev[2], ev[3]);
                    *reinterpret_cast<float4*>(so + j0) = make_float4(ov[0], ov[1], ov[2], ov[3]);
                    if (lane < kActQ - 2 - kN) {  // j = 256 .. 261
                        const int j = kN + lane;
                        const float* xq = xw + j + 3;
                        float e = 0.f, o = 0.f;
#pragma unroll
                        for (int m = 0; m < 6; ++m) {
                            e = fmaf(act.taps.up2[2 * m + 1], xq[3 - m], e);
                            o = fmaf(act.taps.up2[2 * m], xq[3 - m], o);
                        }
                        se[j] = snake_beta(e, alpha_rev, inv_beta);
                        so[j] = snake_beta(o, alpha_rev, inv_beta);
                    }
                }
                __builtin_amdgcn_wave_barrier();
                {
                    const float4* op = reinterpret_cast<const float4*>(so + j0);
                    const float4* ep = reinterpret_cast<const float4*>(se + j0);
                    const float4 o0 = op[0], o1 = op[1], o2 = op[2];
                    const float4 e0 = ep[0], e1 = ep[1], e2 = ep[2];
                    // whole 16-byte reads, as above (only o2.x and e2.x are used)
                    asm volatile("" : : "v"(o2.y), "v"(o2.z), "v"(o2.w), "v"(e2.y), "v"(e2.z),
                                 "v"(e2.w));
                    const float sw[12] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y,
                                          o1.z, o1.w, o2.x, o2.y, o2.z, o2.w};
                    const float ew[12] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y,
                                          e1.z, e1.w, e2.x, e2.y, e2.z, e2.w};
                    float out[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        float acc = 0.f;
#pragma unroll
                        for (int m = 0; m < 6; ++m) {
                            acc = fmaf(act.taps.down[2 * m], sw[k + m], acc);
                            acc = fmaf(act.taps.down[2 * m + 1], ew[k + m], acc);
                        }
                        out[k] = acc;
                    }
                    // xw is free: the transposition goes through it
                    *reinterpret_cast<float4*>(xw + j0) =
                        make_float4(out[0], out[1], out[2], out[3]);
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int r = 0; r < 4; ++r) av[r] = xw[lane + 64 * r];
            } else {
                // a window at a row end: clamped indices, the boundary pairs
#pragma unroll
                for (int r = 0; r < (kActQ + 63) / 64; ++r) {
                    const int j = lane + 64 * r;
                    if (j < kActQ - 2) {
                        const int q = p0 - 3 + j;
                        const int qc = min(max(q, 0), T - 1);
                        const float* xq = xw + (qc - p0 + 6);
                        float e = 0.f, o = 0.f;
#pragma unroll
                        for (int k = 0; k < 6; ++k) {
                            e = fmaf(act.taps.up2[2 * k + 1], xq[2 - k], e);
                            o = fmaf(act.taps.up2[2 * k], xq[3 - k], o);
                        }
                        if (q < 0) o = e;
                        if (q > T - 1) e = o;
                        se[j] = snake_beta(e, alpha_rev, inv_beta);
                        so[j] = snake_beta(o, alpha_rev, inv_beta);
                    }
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int u = lane + 64 * r;
                    float acc = 0.f;
#pragma unroll
                    for (int m = 0; m < 6; ++m) {
                        acc = fmaf(act.taps.down[2 * m], so[u + m], acc);
                        acc = fmaf(act.taps.down[2 * m + 1], se[u + m + 1], acc);
                    }
                    const int p = p0 + u;
                    av[r] = (p >= 0 && p < T) ? acc : 0.f;
                }
            }
            __builtin_amdgcn_wave_barrier();
        };
#pragma unroll
        for (int pr = 0; pr < kPerWave / 2; ++pr) {
            const int g1 = wid + (kThreads / 64) * (2 * pr), g2 = g1 + kThreads / 64;
            if (n0 + g1 >= nb) break;  // wave-uniform
            float a1[4], a2[4] = {0.f, 0.f, 0.f, 0.f};
            act_col(2 * pr, a1);
            if (n0 + g2 < nb) act_col(2 * pr + 1, a2);
            float2 v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = make_float2(a1[r], a2[r]);
            fft256(v, lane, buf[wid], lt);
            store_pair(v, g1, g2);
        }
    }
    __syncthreads();
    const int ncol = min(kCols, nb - n0);
    float2* dst = xf + (size_t)c * NP + (size_t)b * nb + n0;
    const size_t plane = (size_t)C * NP;
    for (int i = threadIdx.x; i < kSlots * kCols; i += kThreads) {
        const int f = i / kCols, g = i - f * kCols;
        if (g < ncol) dst[f * plane + g] = res[f][g];
    }
}

// ---------------------------------------------------------------------------
// Inverse transforms and the epilogue.  grid (ceil(nb / kCols), Cout, B).
// y = IDFT(Y) = conj(DFT(conj(Y))) / N over the Hermitian spectrum; for a
// real result only the real part is formed.
__global__ __launch_bounds__(kThreads) void fft_inv_kernel(const float2* __restrict__ yf,
                                                           float* y, int Cout, int T, int L, int nb,
                                                           int NP, const float* __restrict__ bias,
                                                           const float* residual, float out_scale,
                                                           int accumulate,
                                                           const float* __restrict__ snake_alpha) {
    __shared__ float2 tw[kN];
    __shared__ float2 buf[kThreads / 64][kN];
    __shared__ float2 res[kSlots][kCols + 1];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int b = blockIdx.z, o = blockIdx.y, n0 = blockIdx.x * kCols;
    init_twiddles(tw);
    const int ncol = min(kCols, nb - n0);
    const float2* src = yf + (size_t)o * NP + (size_t)b * nb + n0;
    const size_t plane = (size_t)Cout * NP;
    {
        // all loads first, then the LDS writes
        constexpr int kLd = kSlots * kCols / kThreads;
        float2 ld[kLd];
#pragma unroll
        for (int k = 0; k < kLd; ++k) {
            const int i = threadIdx.x + kThreads * k;
            const int f = i / kCols, g = i - f * kCols;
            ld[k] = (g < ncol) ? src[f * plane + g] : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < kLd; ++k) {
            const int i = threadIdx.x + kThreads * k;
            res[i / kCols][i % kCols] = ld[k];
        }
    }
    __syncthreads();
    const LaneTwiddles lt = lane_twiddles(lane, tw);
    const float bo = bias ? bias[o] : 0.f;
    // plain Snake after the bias, as the direct kernels' epilogue
    const float sa = snake_alpha ? snake_alpha[o] : 0.f;
    const float sa_rev = sa * 0.15915494309189535f, sa_inv = 1.0f / (sa + 1e-9f);
    const size_t row = ((size_t)b * Cout + o) * (size_t)T;
    constexpr float inv_n = 1.0f / (float)kN;  // exact (power of two)
    // the residual and previous-output values of this wave's outputs are read
    // before any transform (each read otherwise waits out its own latency)
    constexpr int kPerWave = kCols / (kThreads / 64);
    float rv[kPerWave][4], ov[kPerWave][4];
#pragma unroll
    for (int it = 0; it < kPerWave; ++it) {
        const int n = n0 + wid + (kThreads / 64) * it;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int u = lane + 64 * q;
            const int t = n * L + u;
            const bool ok = n < nb && u < L && t < T;
            rv[it][q] = (ok && residual) ? residual[row + t] : 0.f;
            ov[it][q] = (ok && accumulate) ? y[row + t] : 0.f;
        }
    }
    // Z = conj(Y) on bins 0..N/2, Z_k = Y_{N-k} above, for column g in lane
    // j's order (k = j + 64 q)
    auto spectrum = [&](int g, float2 (&z)[4]) {
        const float2 s0 = res[0][g];
        if (lane == 0) {
            z[0] = make_float2(s0.x, 0.f);
            z[2] = make_float2(s0.y, 0.f);
        } else {
            const float2 a = res[lane][g];
            z[0] = make_float2(a.x, -a.y);
            z[2] = res[128 - lane][g];
        }
        const float2 a1 = res[lane + 64][g];
        z[1] = make_float2(a1.x, -a1.y);
        z[3] = res[64 - lane][g];
    };
    auto store = [&](int it, int n, int q, float val) {
        const int u = lane + 64 * q;
        const int t = n * L + u;
        if (u < L && t < T) {
            float v = fmaf(val, inv_n, bo);
            if (snake_alpha) v = snake_beta(v, sa_rev, sa_inv);
            y[row + t] = fmaf(v + rv[it][q], out_scale, ov[it][q]);
        }
    };
    // two blocks per transform: both results are real, so the transform of
    // Z1 + i Z2 carries block 1 in its real part and block 2 in its imaginary
    // part
#pragma unroll
    for (int pr = 0; pr < kPerWave / 2; ++pr) {
        const int g1 = wid + (kThreads / 64) * (2 * pr), g2 = g1 + kThreads / 64;
        const int n1 = n0 + g1, n2 = n0 + g2;
        if (n1 >= nb) break;  // wave-uniform
        float2 z1[4], z2[4], v[4];
        spectrum(g1, z1);
        spectrum(g2, z2);  // zeros past the row's last block
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = make_float2(z1[q].x - z2[q].y, z1[q].y + z2[q].x);
        fft256(v, lane, buf[wid], lt);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            store(2 * pr, n1, q, v[q].x);
            if (n2 < nb) store(2 * pr + 1, n2, q, v[q].y);
        }
    }
}

// ---------------------------------------------------------------------------
// Y[slot] = W[slot] X[slot]: per slot a complex [Cout x Cin] x [Cin x NP]
// product on the matrix cores.  Workgroup: one slot, 64 output rows (16 per
// wave; Cout a multiple of 16), NT = 16 NJ columns.  A operands (W) come
// pre-packed in MFMA fragment order, wp[slot][o/16][c/16][re,im][lane][4] (4 consecutive
// k-steps per lane per 16-byte load), read straight from memory one
// 16-channel chunk ahead.  B operands (X) go to LDS by LDS DMA
// (global_load_lds_dwordx4: no register round trip), 16 channels per chunk,
// double-buffered, rows of NT complex back to back; each wave reads its B
// fragments one k-step ahead of the matrix instructions that use them.
// Three real products per complex multiply-add (Gauss); slot 0 holds two
// real bins (re: bin 0, im: bin N/2), whose products are the first two.  The
// blockIdx -> tile map keeps each XCD on a contiguous range of slots, so a
// slot's X is fetched into one L2.
__device__ __forceinline__ void wait_vmem_all() {
    // s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int NJ>
__global__ __launch_bounds__(kThreads, 2) void fft_gemm_kernel(const float* __restrict__ wp,
                                                               const float2* __restrict__ xf,
                                                               float2* __restrict__ yf, int Cin,
                                                               int Cout, int NP, int ntiles) {
    constexpr int NT = 16 * NJ;
    constexpr int KC = 16;               // channels per chunk (4 k-steps)
    constexpr int kDma = KC * NT / 128;  // 1 KB wave instructions per chunk (2 NJ)
    // two buffers as two objects, so that the compiler sees the DMA into one
    // and the fragment reads from the other as independent
    __shared__ __align__(16) float2 bsA[KC * NT];
    __shared__ __align__(16) float2 bsB[KC * NT];

    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // XCD-contiguous tile order: workgroups are dealt to the 8 XCDs round robin
    const int mt = (Cout + 63) / 64;
    const int G = ntiles * mt * kSlots;
    const int id = blockIdx.x;
    const int lid = (id & 7) * (G >> 3) + (id >> 3);
    const int nt = lid % ntiles;
    const int om = (lid / ntiles) % mt;
    const int f = lid / (ntiles * mt);
    // a wave past the last 16-row tile (Cout % 64 != 0) computes on the last
    // tile's weights and stores nothing
    const int OT = Cout / 16;
    const int ot = om * 4 + wid;
    const bool rows_ok = ot < OT;
    const int n0 = nt * NT;
    const int S4 = Cin / 16;
    const int nchunk = Cin / KC;

    const f32x4* ap = reinterpret_cast<const f32x4*>(wp) +
                      ((size_t)(f * OT + min(ot, OT - 1)) * S4) * 128 + lane;
    const float2* xb = xf + (size_t)f * Cin * NP + n0;

    // chunk ch -> buf: float4 q = 64 i + lane of the chunk image, i = wid + 4 t;
    // the lane's offsets inside a chunk are the same for every chunk
    constexpr int kDmaW = (kDma + kThreads / 64 - 1) / (kThreads / 64);
    int doff[kDmaW];
#pragma unroll
    for (int t = 0; t < kDmaW; ++t) {
        const int q = 64 * (wid + (kThreads / 64) * t) + lane;
        const int kk = q / (NT / 2), c2 = q - kk * (NT / 2);
        doff[t] = kk * NP + 2 * c2;
    }
    auto issue_chunk = [&](int ch, float2* buf) {
        const float2* cb = xb + (size_t)KC * ch * NP;
#pragma unroll
        for (int t = 0; t < kDmaW; ++t) {
            const int i = wid + (kThreads / 64) * t;
            if (i < kDma)  // wave-uniform
                __builtin_amdgcn_global_load_lds((const void*)(cb + doff[t]),
                                                 (void*)(buf + 128 * i), 16, 0, 0);
        }
    };

    // Gauss's three real products per complex multiply-add:
    //   P1 = Wr Xr, P2 = Wi Xi, P3 = (Wr + Wi)(Xr + Xi);
    //   Re Y = P1 - P2, Im Y = P3 - P1 - P2
    // (the sums formed in registers, one add per operand).  Slot 0's two
    // real bins are P1 (bin 0) and P2 (bin N/2).
    f32x4 p1a[NJ], p2a[NJ], p3a[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) {
        p1a[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        p2a[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
        p3a[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int brow = lane >> 4, bcol = lane & 15;
    // one chunk: matrix work on chunk ch from Bc (weights ar, ai) while chunk
    // ch + 1 lands in Bn (weights nar, nai: the other register set, so no
    // copy between chunks)
    auto step = [&](int ch, const float2* Bc, float2* Bn, const f32x4& ar, const f32x4& ai,
                    f32x4& nar, f32x4& nai) {
        const bool more = ch + 1 < nchunk;
        if (more) {
            issue_chunk(ch + 1, Bn);
            nar = ap[(size_t)(ch + 1) * 128];
            nai = ap[(size_t)(ch + 1) * 128 + 64];
        }
        const float2* bb = Bc + brow * NT + bcol;
        float2 bv[2][NJ];
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) bv[0][jt] = bb[16 * jt];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = ks & 1;
            if (ks < 3) {
#pragma unroll
                for (int jt = 0; jt < NJ; ++jt) bv[c ^ 1][jt] = bb[(4 * (ks + 1)) * NT + 16 * jt];
            }
            __builtin_amdgcn_sched_barrier(0);
            const float wr = ar[ks], wi = ai[ks], ws = wr + wi;
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
                p1a[jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(wr, bv[c][jt].x, p1a[jt], 0, 0, 0);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
                p2a[jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(wi, bv[c][jt].y, p2a[jt], 0, 0, 0);
#pragma unroll
            for (int jt = 0; jt < NJ; ++jt)
                p3a[jt] = __builtin_amdgcn_mfma_f32_16x16x4f32(ws, bv[c][jt].x + bv[c][jt].y,
                                                               p3a[jt], 0, 0, 0);
        }
        // the next chunk's DMA and A operands have landed; every wave is done
        // with Bc before it is refilled
        wait_vmem_all();
        __syncthreads();
    };
    issue_chunk(0, bsA);
    f32x4 arE = ap[0], aiE = ap[64], arO = arE, aiO = aiE;
    wait_vmem_all();
    __syncthreads();
    for (int ch = 0; ch < nchunk; ch += 2) {
        step(ch, bsA, bsB, arE, aiE, arO, aiO);
        if (ch + 1 < nchunk) step(ch + 1, bsB, bsA, arO, aiO, arE, aiE);
    }
    // D layout: lane l holds rows 4 (l / 16) + i, column l % 16 of each tile
    if (!rows_ok) return;
    float2* yo = yf + ((size_t)f * Cout + 16 * ot + 4 * brow) * NP + n0 + bcol;
    const bool dc = (f == 0);
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = p1a[jt][i], b = p2a[jt][i];
            yo[(size_t)i * NP + 16 * jt] =
                dc ? make_float2(a, b) : make_float2(a - b, p3a[jt][i] - (a + b));
        }
}

// ---------------------------------------------------------------------------
// Packed frequency-domain weights: for slot f >= 1
//   W = sum_j w[o,c,j] e^{+2 pi i f j d / N},
// slot 0 = (sum_j w_j, sum_j (-1)^{j d} w_j) (bins 0 and N/2), summed in
// double and rounded once, stored in fft_gemm_kernel's fragment order.
// Workgroup: one 16 x 16 (output row, input channel) tile, kPackSlots
// consecutive slots; thread t owns the pair at float t of the tile's 256-float
// planes, reads its K taps once and keeps a sum per slot, and every slot's
// two planes are written as 1 KB runs.  The twiddles come from a double
// table in LDS, one index for the whole workgroup at a time (a broadcast).
constexpr int kPackSlots = 16;
__global__ __launch_bounds__(256) void fft_pack_kernel(const float* __restrict__ w,
                                                       float* __restrict__ wp, int Cin, int Cout,
                                                       int K, int d) {
    // double twiddles e^{+2 pi i m / N}, one per thread of the workgroup
    __shared__ double2 twd[kN];
    {
        double sn, cs;
        sincospi(2.0 * (double)threadIdx.x / (double)kN, &sn, &cs);
        twd[threadIdx.x] = make_double2(cs, sn);
    }
    __syncthreads();
    const int S4 = Cin / 16, OT = Cout / 16;
    const int ot = blockIdx.x / S4, s4 = blockIdx.x - ot * S4;
    const int f0 = blockIdx.y * kPackSlots;
    // float t of a (slot, ot, s4) plane: lane ln = t / 4 of k-step e = t % 4,
    // i.e. row ot 16 + ln % 16, channel s4 16 + 4 e + ln / 16
    const int t = threadIdx.x, e = t & 3, ln = t >> 2;
    const int o = ot * 16 + (ln & 15), c = s4 * 16 + e * 4 + (ln >> 4);
    const float* wr = w + ((size_t)o * Cin + c) * K;
    double re[kPackSlots], im[kPackSlots];
#pragma unroll
    for (int s = 0; s < kPackSlots; ++s) re[s] = im[s] = 0.0;
    for (int j = 0; j < K; ++j) {
        const double wj = (double)wr[j];
        const int jd = (j * d) & (kN - 1);
#pragma unroll
        for (int s = 0; s < kPackSlots; ++s) {
            const int f = f0 + s;
            if (f == 0) {
                re[s] += wj;
                im[s] = fma(wj, twd[(jd * (kN / 2)) & (kN - 1)].x, im[s]);  // (-1)^{j d}
            } else {
                const double2 tw = twd[(f * jd) & (kN - 1)];
                re[s] = fma(wj, tw.x, re[s]);
                im[s] = fma(wj, tw.y, im[s]);
            }
        }
    }
#pragma unroll
    for (int s = 0; s < kPackSlots; ++s) {
        const size_t g = ((size_t)(f0 + s) * OT + ot) * S4 + s4;
        wp[g * 512 + t] = (float)re[s];
        wp[g * 512 + 256 + t] = (float)im[s];
    }
}

template <int NJ>
void gemm_launch(const float* wp, const float2* xf, float2* yf, int Cin, int Cout, int NP,
                 int ntiles, hipStream_t s) {
    const int G = ntiles * ((Cout + 63) / 64) * kSlots;
    hipLaunchKernelGGL(fft_gemm_kernel<NJ>, dim3((unsigned)G), dim3(kThreads), 0, s, wp, xf, yf,
                       Cin, Cout, NP, ntiles);
}

}  // namespace

size_t fft_conv_weight_floats(int Cin, int Cout) {
    return (size_t)kSlots * (size_t)Cout * (size_t)Cin * 2;
}

hipError_t launch_fft_pack(const float* w, float* wp, int Cin, int Cout, int K, int dilation,
                           hipStream_t s) {
    if (!plan::fft_supported(Cin, Cout, K, dilation)) return hipErrorInvalidValue;
    const long long total = (long long)kSlots * Cout * Cin;
    const long long tiles = (long long)(Cout / 16) * (Cin / 16);
    if (tiles > 0x7fffffffLL) return hipErrorInvalidValue;
    prof_pre(s);
    hipLaunchKernelGGL(fft_pack_kernel, dim3((unsigned)tiles, kSlots / kPackSlots), dim3(256), 0, s,
                       w, wp, Cin, Cout, K, dilation);
    // reads w once, writes the 2 x 128 x Cout x Cin packed floats
    prof_post(s, "fft_pack_kernel", 4.0 * K * (double)total,
              4.0 * ((double)Cout * Cin * K + 2.0 * (double)total));
    return hipGetLastError();
}

hipError_t launch_conv1d_fft(const float* x, float* y, const float* wp, int B, int Cin, int Cout,
                             int T, int K, int dilation, const ConvEpilogue& ep, float* xspec,
                             float* yspec, hipStream_t s, const float* act_log_alpha,
                             const float* act_log_beta, const ActTaps* act_taps) {
    const bool act = act_log_alpha && act_log_beta && act_taps;
    if (!plan::fft_supported(Cin, Cout, K, dilation) || (act && ep.in_alpha))
        return hipErrorInvalidValue;
    const plan::FftShape sh = plan::fft_shape(B, T, K, dilation);
    if (sh.ntiles < 1 || sh.NJ < 1 || sh.NJ > 8) return hipErrorInvalidValue;
    const int P = (K - 1) * dilation / 2;
    float2* xf = reinterpret_cast<float2*>(xspec);
    float2* yf = reinterpret_cast<float2*>(yspec);
    const dim3 tg((unsigned)((sh.nb + kCols - 1) / kCols), 1, (unsigned)B);
    const double blocks = (double)sh.NB;

    ActIn ai{act_log_alpha, act_log_beta, {}, ep.in_alpha};
    if (act) ai.taps = *act_taps;
    const dim3 fg(tg.x, (unsigned)Cin, tg.z);
    prof_pre(s);
    if (act)
        hipLaunchKernelGGL(fft_fwd_kernel<1>, fg, dim3(kThreads), 0, s, x, xf, Cin, T, sh.L, P,
                           sh.nb, sh.NP, ai);
    else if (ep.in_alpha)
        hipLaunchKernelGGL(fft_fwd_kernel<2>, fg, dim3(kThreads), 0, s, x, xf, Cin, T, sh.L, P,
                           sh.nb, sh.NP, ai);
    else
        hipLaunchKernelGGL(fft_fwd_kernel<0>, fg, dim3(kThreads), 0, s, x, xf, Cin, T, sh.L, P,
                           sh.nb, sh.NP, ai);
    hipError_t e = hipGetLastError();
    // algorithmic: x read once (4 B per sample), the spectrum written once
    prof_post(s, act ? "fft_fwd_kernel<act>" : ep.in_alpha ? "fft_fwd_kernel<snake>" : "fft_fwd_kernel",
              act ? 52.0 * B * Cin * (double)T : ep.in_alpha ? 4.0 * B * Cin * (double)T : 0.0,
              4.0 * B * Cin * (double)T + 8.0 * kSlots * Cin * blocks);
    if (e != hipSuccess) return e;

    prof_pre(s);
    switch (sh.NJ) {
        case 1: gemm_launch<1>(wp, xf, yf, Cin, Cout, sh.NP, sh.ntiles, s); break;
        case 2: gemm_launch<2>(wp, xf, yf, Cin, Cout, sh.NP, sh.ntiles, s); break;
        case 3: gemm_launch<3>(wp, xf, yf, Cin, Cout, sh.NP, sh.ntiles, s); break;
        case 4: gemm_launch<4>(wp, xf, yf, Cin, Cout, sh.NP, sh.ntiles, s); break;
        case 5: gemm_launch<5>(wp, xf, yf, Cin, Cout, sh.NP, sh.ntiles, s); break;
        case 6: gemm_launch<6>(wp, xf, yf, Cin, Cout, sh.NP, sh.ntiles, s); break;
        case 7: gemm_launch<7>(wp, xf, yf, Cin, Cout, sh.NP, sh.ntiles, s); break;
        default: gemm_launch<8>(wp, xf, yf, Cin, Cout, sh.NP, sh.ntiles, s); break;
    }
    e = hipGetLastError();
    {
        // algorithmic: 127 complex slots (3 real products each, Gauss) + slot
        // 0 (2), one multiply-add = 2 flops, over the real columns
        static const char* names[8] = {"fft_gemm_kernel<1>", "fft_gemm_kernel<2>",
                                       "fft_gemm_kernel<3>", "fft_gemm_kernel<4>",
                                       "fft_gemm_kernel<5>", "fft_gemm_kernel<6>",
                                       "fft_gemm_kernel<7>", "fft_gemm_kernel<8>"};
        const double macs = (127.0 * 3.0 + 2.0) * Cout * (double)Cin * blocks;
        const double bytes = 8.0 * kSlots * (double)Cout * Cin +
                             8.0 * kSlots * (double)(Cin + Cout) * blocks;
        prof_post(s, names[sh.NJ - 1], 2.0 * macs, bytes);
    }
    if (e != hipSuccess) return e;

    prof_pre(s);
    hipLaunchKernelGGL(fft_inv_kernel, dim3(tg.x, (unsigned)Cout, tg.z), dim3(kThreads), 0, s, yf,
                       y, Cout, T, sh.L, sh.nb, sh.NP, ep.bias, ep.residual, ep.out_scale,
                       ep.accumulate, ep.snake_alpha);
    e = hipGetLastError();
    const double n = (double)B * Cout * T;
    prof_post(s, "fft_inv_kernel", 0.0,
              8.0 * kSlots * Cout * blocks + 4.0 * n * (1 + (ep.residual != nullptr) +
                                                        (ep.accumulate != 0)));
    return e;
}

}  // namespace avae
