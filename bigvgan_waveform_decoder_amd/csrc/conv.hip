// Conv1d and ConvTranspose1d as implicit GEMMs on the gfx950 FP32 matrix
// cores (v_mfma_f32_16x16x4_f32), plus the one-output-channel conv_post.
//
// Operations ([H3] = docs.rs page of cortiq_engine/audiovae.rs):
//   Conv1d::apply:  y[o,t] = b[o] + sum_i sum_j w[o,i,j] x[i, t + j d - pad]
//                   (zero padding).  The page notes that w is already the
//                   [Cout x Cin*K] GEMM operand of an im2col formulation.
//   ConvT1d::apply: y[o, t s + j - pad] += x[i,t] w[i,o,j], plus b[o].
//
// Conv1d: GEMM with M = Cout, N = time, K = Cin * taps.  There is no im2col
// buffer: a block stages kKC input channels of its time window plus the
// (K-1)*d halo in LDS once, and every tap j reads the same LDS rows shifted
// by j*d.  The weight slice [BM rows x kKC*K] is staged in LDS in the
// caller's [Cout, Cin, K] order (rows contiguous in global memory, so loads
// coalesce).
//
// ConvTranspose1d: polyphase gather.  Output t' = q*s + r - pad (phase r)
// receives sum_i sum_m w[i,o,r+s*m] * x[i, q-m], m < ceil((K-r)/s): one
// small GEMM per phase, no zero-stuffing and no atomics; each block owns
// one (Cout tile, phase, q tile).
//
// MFMA 16x16x4 f32 operand layout (wave64): lane l supplies A[l%16][l/16]
// and B[l/16][l%16]; the 4 accumulator registers of lane l hold
// D[4*(l/16) + r][l%16], r = 0..3.  Rows map to output channels and columns
// to time, so consecutive lanes store consecutive samples.
#include <algorithm>
#include <string>

#include "act_math.h"
#include "avae_internal.h"

namespace avae {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kKC = 8;  // input channels per K chunk: two MFMA k-steps of 4

// Workgroups are dispatched round-robin over the 8 XCDs; remap so that each
// XCD works through a contiguous range of logical tiles (neighbouring output
// channel tiles of one time window share the staged input in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
    const int q = nblk >> 3, r = nblk & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

__device__ __forceinline__ int floor_div(int a, int b) {
    int q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
    return q;
}

// Conv1d epilogue for an MT x NTL grid of 16x16 accumulator tiles whose
// top-left output is (o_base, t_base): bias, optional plain Snake, optional
// residual, scale, optional accumulate.  Every input of the epilogue is
// loaded before the first store: a store may alias the residual (the same
// element, read and written by the same lane), so a load issued after a
// store would wait for it, one memory latency per element.
template <int MT, int NTL, bool SN>
__device__ __forceinline__ void conv_epilogue(const f32x4 (&acc)[MT][NTL], float* y, int Cout,
                                              int Tout, int b, int o_base, int t_base, int l16,
                                              int g, const ConvEpilogue& ep) {
    float* yb = y + (size_t)b * Cout * Tout;
    const float* rb = ep.residual ? ep.residual + (size_t)b * Cout * Tout : nullptr;
    float bias[MT][4], alpha[MT][4];
    float res[MT][NTL][4], old[MT][NTL][4];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = o_base + a * 16 + g * 4 + r;
            bias[a][r] = (ep.bias && o < Cout) ? ep.bias[o] : 0.f;
            alpha[a][r] = (SN && ep.snake_alpha && o < Cout) ? ep.snake_alpha[o] : 1.f;
        }
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int cc = 0; cc < NTL; ++cc) {
            const int t = t_base + cc * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = o_base + a * 16 + g * 4 + r;
                const bool ok = o < Cout && t < Tout;
                const size_t idx = (size_t)o * Tout + t;
                res[a][cc][r] = (rb && ok) ? rb[idx] : 0.f;
                old[a][cc][r] = (ep.accumulate && ok) ? yb[idx] : 0.f;
            }
        }
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int cc = 0; cc < NTL; ++cc) {
            const int t = t_base + cc * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = o_base + a * 16 + g * 4 + r;
                if (o < Cout && t < Tout) {
                    float v = acc[a][cc][r];
                    if (ep.bias) v += bias[a][r];
                    if (SN && ep.snake_alpha) v = snake_plain(v, alpha[a][r]);
                    if (rb) v += res[a][cc][r];
                    v *= ep.out_scale;
                    if (ep.accumulate) v += old[a][cc][r];
                    yb[(size_t)o * Tout + t] = v;
                }
            }
        }
}

// ------------------------------------------------------------------ Conv1d

template <int BM, int BN, int WM, int WN, int KT>
__global__ __launch_bounds__(WM * WN * 64) void conv1d_mfma_kernel(
    const float* __restrict__ x, float* y, const float* __restrict__ w, int Cin, int Cout,
    int T, int Tout, int Kr, int dil, int pad, int m_tiles, int n_tiles, int nblk,
    int ws_stride, int xs_stride, int flush, ConvEpilogue ep) {
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 16, NTL = WTN / 16;
    static_assert(MT >= 1 && NTL >= 1, "wave tile must hold at least one 16x16 MFMA tile");
    const int K = KT > 0 ? KT : Kr;

    extern __shared__ float lds[];
    float* Ws = lds;                     // [BM][ws_stride]: col i*K + j
    float* Xs = lds + BM * ws_stride;    // [kKC][xs_stride]: col u <-> t0 - pad + u

    const int lid = xcd_remap(blockIdx.x, nblk);
    const int mt_i = lid % m_tiles;
    const int rest = lid / m_tiles;
    const int nt_i = rest % n_tiles;
    const int b = rest / n_tiles;
    const int o0 = mt_i * BM, t0 = nt_i * BN;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm0 = (wid / WN) * WTM, wn0 = (wid % WN) * WTN;
    const int l16 = lane & 15, g = lane >> 4;

    // Blocked accumulation: the matrix cores accumulate `flush` K chunks into
    // `part`, which is then added into `acc`.  This keeps every float32
    // running sum short (a few dozen MFMA steps plus Cin/(8*flush) block
    // additions instead of Cin*K/4 sequential MFMA steps).
    f32x4 acc[MT][NTL], part[MT][NTL];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int c = 0; c < NTL; ++c) {
            acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            part[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const int xw = BN + (K - 1) * dil;
    const int wrow = kKC * K;
    const float* xb = x + (size_t)b * Cin * T;

    int chunk = 0;
    for (int ic0 = 0; ic0 < Cin; ic0 += kKC, ++chunk) {
        for (int e = tid; e < BM * wrow; e += NT) {
            const int ol = e / wrow;
            const int f = e - ol * wrow;
            const int i = f / K;
            const int o = o0 + ol;
            float v = 0.f;
            if (o < Cout && ic0 + i < Cin) v = w[((size_t)o * Cin + ic0) * K + f];
            Ws[ol * ws_stride + f] = v;
        }
        for (int e = tid; e < kKC * xw; e += NT) {
            const int i = e / xw;
            const int u = e - i * xw;
            const int t = t0 - pad + u;
            float v = 0.f;
            if (ic0 + i < Cin && t >= 0 && t < T) {
                v = xb[(size_t)(ic0 + i) * T + t];
                if (ep.in_alpha) v = snake_plain(v, ep.in_alpha[ic0 + i]);
            }
            Xs[i * xs_stride + u] = v;
        }
        __syncthreads();

        for (int j = 0; j < K; ++j) {
#pragma unroll
            for (int kk = 0; kk < kKC / 4; ++kk) {
                float av[MT], bv[NTL];
#pragma unroll
                for (int a = 0; a < MT; ++a)
                    av[a] = Ws[(wm0 + a * 16 + l16) * ws_stride + (kk * 4 + g) * K + j];
#pragma unroll
                for (int c = 0; c < NTL; ++c)
                    bv[c] = Xs[(kk * 4 + g) * xs_stride + wn0 + c * 16 + l16 + j * dil];
#pragma unroll
                for (int a = 0; a < MT; ++a)
#pragma unroll
                    for (int c = 0; c < NTL; ++c)
                        part[a][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv[c],
                                                                          part[a][c], 0, 0, 0);
            }
        }
        if ((chunk + 1) % flush == 0 || ic0 + kKC >= Cin) {
#pragma unroll
            for (int a = 0; a < MT; ++a)
#pragma unroll
                for (int c = 0; c < NTL; ++c) {
                    acc[a][c] += part[a][c];
                    part[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
        __syncthreads();
    }

    conv_epilogue<MT, NTL, true>(acc, y, Cout, Tout, b, o0 + wm0, t0 + wn0, l16, g, ep);
}

// Pipelined Conv1d for the decoder's shapes (K in {1,3,7,11}, dilation <= 5,
// Cin a multiple of 4, 16-byte aligned weights).  Same GEMM and blocked
// accumulation as conv1d_mfma_kernel, plus:
//  - the next K chunk's weights (float4 loads) and input window are loaded
//    into registers while the matrix cores work on the current chunk from
//    LDS, so global latency hides behind the MFMA work of the same block;
//  - the input window is staged row by row (256/KC lanes per channel row),
//    no integer division per element;
//  - KC = 16 input channels per chunk for small K (more MFMA work between
//    barriers), 8 otherwise;
//  - `n_fastest` selects the tile walk within each XCD's range: output
//    channel tiles fastest (0: neighbouring blocks share the staged input)
//    or time tiles fastest (1: they share one weight slice).  Measured on
//    MI355X, channel-fastest is equal or better for every decoder shape.
// Largest dilation a pipelined kernel stages the halo for (its DM template
// parameter): 5 covers the BigVGAN units (d = 1, 3, 5); a second 7-tap
// instantiation with DM = 9 takes the DAV units' d = 9 (a wider halo costs
// the d <= 5 shapes staging work, so they keep DM = 5).
constexpr int kDilMax = 5;
constexpr int dil_max(int K) { return K == 7 ? 9 : kDilMax; }

constexpr int xs_stride_const(int xw) {
    return ((xw + 63) / 64 * 64 + 16) - 64 >= xw ? ((xw + 63) / 64 * 64 + 16) - 64
                                                   : (xw + 63) / 64 * 64 + 16;
}

// Minimum waves per SIMD requested from the register allocator: 3 for the
// tiles that measured faster at that occupancy (no or few spills), none for
// the 64-row tiles whose prefetch and accumulator registers would spill.
template <int BM, int BN, int KT>
constexpr int pipe_min_waves() {
    return (BM == 96 || BM == 48 || BM == 32 || (BM == 64 && BN == 64 && KT <= 3)) ? 3 : 1;
}

template <int BM, int BN, int WM, int WN, int KT, int KC, int DM, bool SN>
__global__ __launch_bounds__(WM * WN * 64, (pipe_min_waves<BM, BN, KT>())) void conv1d_pipe_kernel(
    const float* __restrict__ x, float* y, const float* __restrict__ w, int Cin, int Cout,
    int T, int Tout, int dil, int pad, int m_tiles, int n_tiles, int nblk, int flush,
    int n_fastest, ConvEpilogue ep) {
    constexpr int NT = WM * WN * 64;
    static_assert(NT == 256, "256 threads");
    static_assert(KC == 8 || KC == 16, "8 or 16 input channels per chunk");
    constexpr int kXLanes = NT / KC;  // lanes per staged input row
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 16, NTL = WTN / 16;
    constexpr int WROW = KC * KT;      // weight floats per row per chunk
    // row stride = 4 (mod 8) floats: each staged float4 is one ds_write_b128
    // (an odd stride split it into four conflicting scalar writes)
    constexpr int WS = (WROW % 8 == 0) ? WROW + 4 : WROW + 8;
    constexpr int WV = WROW / 4;        // float4 per row per chunk
    constexpr int WV_PT = (BM * WV + NT - 1) / NT;
    constexpr int XW_MAX = BN + (KT - 1) * DM;
    constexpr int XS = xs_stride_const(XW_MAX);
    constexpr int X_PT = (XW_MAX + kXLanes - 1) / kXLanes;
    static_assert(WROW % 4 == 0, "float4 weight rows");

    __shared__ __align__(16) float Ws[BM * WS];
    __shared__ __align__(16) float Xs[KC * XS];

    const int lid = xcd_remap(blockIdx.x, nblk);
    int mt_i, nt_i, b;
    if (n_fastest) {
        nt_i = lid % n_tiles;
        const int rest = lid / n_tiles;
        mt_i = rest % m_tiles;
        b = rest / m_tiles;
    } else {
        mt_i = lid % m_tiles;
        const int rest = lid / m_tiles;
        nt_i = rest % n_tiles;
        b = rest / n_tiles;
    }
    const int o0 = mt_i * BM, t0 = nt_i * BN;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm0 = (wid / WN) * WTM, wn0 = (wid % WN) * WTN;
    const int l16 = lane & 15, g = lane >> 4;
    const int xrow = tid / kXLanes, xcol = tid % kXLanes;

    f32x4 acc[MT][NTL], part[MT][NTL];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int c = 0; c < NTL; ++c) {
            acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            part[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const int xw = BN + (KT - 1) * dil;
    const float* xb = x + (size_t)b * Cin * T;
    const int nch = (Cin + KC - 1) / KC;

    float4 wr[WV_PT];
    float xr[X_PT];
    float xa = 1.f;  // Snake alpha of this thread's staged input row

    auto gload = [&](int ic0) {
        const int valid_f = (Cin - ic0 < KC ? Cin - ic0 : KC) * KT;  // multiple of 4
#pragma unroll
        for (int r = 0; r < WV_PT; ++r) {
            const int e4 = tid + r * NT;
            const int ol = e4 / WV;
            const int f4 = e4 - ol * WV;
            const int o = o0 + ol;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e4 < BM * WV && o < Cout && 4 * f4 < valid_f)
                v = *reinterpret_cast<const float4*>(w + ((size_t)o * Cin + ic0) * KT + 4 * f4);
            wr[r] = v;
        }
        const int ic = ic0 + xrow;
        const float* xrowp = xb + (size_t)ic * T;
#pragma unroll
        for (int r = 0; r < X_PT; ++r) {
            const int u = xcol + r * kXLanes;
            const int t = t0 - pad + u;
            float v = 0.f;
            if (u < xw && ic < Cin && t >= 0 && t < T) v = xrowp[t];
            xr[r] = v;
        }
        if (SN && ep.in_alpha) xa = ic < Cin ? ep.in_alpha[ic] : 1.f;
    };
    auto lstore = [&]() {
#pragma unroll
        for (int r = 0; r < WV_PT; ++r) {
            const int e4 = tid + r * NT;
            if (e4 < BM * WV) {
                const int ol = e4 / WV;
                const int f4 = e4 - ol * WV;
                *reinterpret_cast<float4*>(Ws + ol * WS + 4 * f4) = wr[r];
            }
        }
        if (SN && ep.in_alpha) {
            // plain Snake of the input as staged (zero padding stays zero)
            const float arev = xa * 0.15915494309189535f, inv = 1.0f / (xa + 1e-9f);
#pragma unroll
            for (int r = 0; r < X_PT; ++r) xr[r] = snake_beta(xr[r], arev, inv);
        }
#pragma unroll
        for (int r = 0; r < X_PT; ++r) {
            const int u = xcol + r * kXLanes;
            if (u < xw) Xs[xrow * XS + u] = xr[r];
        }
    };

    gload(0);
    lstore();
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch) gload((c + 1) * KC);
        // Several taps per iteration let the next taps' LDS reads overlap
        // the current tap's MFMAs (measured +5-25% for tiles of 48+ rows);
        // the small tiles keep one tap per iteration.
        constexpr int kTapUnroll = BM >= 48 ? 4 : 1;
#pragma unroll kTapUnroll
        for (int j = 0; j < KT; ++j) {
#pragma unroll
            for (int kk = 0; kk < KC / 4; ++kk) {
                float av[MT], bv[NTL];
#pragma unroll
                for (int a = 0; a < MT; ++a)
                    av[a] = Ws[(wm0 + a * 16 + l16) * WS + (kk * 4 + g) * KT + j];
#pragma unroll
                for (int cc = 0; cc < NTL; ++cc)
                    bv[cc] = Xs[(kk * 4 + g) * XS + wn0 + cc * 16 + l16 + j * dil];
#pragma unroll
                for (int a = 0; a < MT; ++a)
#pragma unroll
                    for (int cc = 0; cc < NTL; ++cc)
                        part[a][cc] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv[cc],
                                                                           part[a][cc], 0, 0, 0);
            }
        }
        if ((c + 1) % flush == 0 || c + 1 == nch) {
#pragma unroll
            for (int a = 0; a < MT; ++a)
#pragma unroll
                for (int cc = 0; cc < NTL; ++cc) {
                    acc[a][cc] += part[a][cc];
                    part[a][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
        __syncthreads();
        if (c + 1 < nch) {
            lstore();
            __syncthreads();
        }
    }

    conv_epilogue<MT, NTL, SN>(acc, y, Cout, Tout, b, o0 + wm0, t0 + wn0, l16, g, ep);
}

struct ConvTile {
    int bm, bn;
};

// LDS row strides: the weight rows get an odd stride; the input rows a
// stride = 16 (mod 64) so the four 16-lane groups of a fragment read fall in
// disjoint bank ranges.
inline int xs_stride_for(int xw) {
    int s = (xw + 63) / 64 * 64 + 16;
    if (s - 64 >= xw) s -= 64;
    return s;
}

template <int BM, int BN, int WM, int WN, int KT>
hipError_t run_conv1d(const float* x, float* y, const float* w, int B, int Cin, int Cout, int T,
                      int Tout, int K, int dil, int pad, const ConvEpilogue& ep,
                      hipStream_t stream) {
    const int m_tiles = (Cout + BM - 1) / BM;
    const int n_tiles = (Tout + BN - 1) / BN;
    const long long nblk = (long long)m_tiles * n_tiles * B;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    const int ws_stride = kKC * K + 1;
    const int xs_stride = xs_stride_for(BN + (K - 1) * dil);
    const size_t lds = (size_t)(BM * ws_stride + kKC * xs_stride) * sizeof(float);
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    auto kern = conv1d_mfma_kernel<BM, BN, WM, WN, KT>;
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    // about two dozen MFMA k-steps (2*K per chunk) between block additions
    const int flush = K >= 12 ? 1 : (24 / (2 * K) > 0 ? 24 / (2 * K) : 1);
    static const std::string name = "conv1d_mfma_kernel<" + std::to_string(BM) + "," +
                                    std::to_string(BN) + "," + std::to_string(WM) + "," +
                                    std::to_string(WN) + "," + std::to_string(KT) + ">";
    prof_pre(stream);
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(WM * WN * 64), lds, stream, x, y, w, Cin,
                       Cout, T, Tout, K, dil, pad, m_tiles, n_tiles, (int)nblk, ws_stride,
                       xs_stride, flush, ep);
    const hipError_t e = hipGetLastError();
    const double out_n = (double)B * Cout * Tout;
    prof_post(stream, name.c_str(), 2.0 * out_n * Cin * K,
              4.0 * ((double)B * Cin * T + out_n * (1 + (ep.residual ? 1 : 0) + ep.accumulate) +
                     (double)Cout * Cin * K));
    return e;
}

template <int BM, int BN, int WM, int WN, int KT, int DM = kDilMax, bool SN = false>
hipError_t run_conv1d_pipe(const float* x, float* y, const float* w, int B, int Cin, int Cout,
                           int T, int Tout, int dil, int pad, const ConvEpilogue& ep,
                           hipStream_t stream) {
    const int m_tiles = (Cout + BM - 1) / BM;
    const int n_tiles = (Tout + BN - 1) / BN;
    const long long nblk = (long long)m_tiles * n_tiles * B;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    // 16 input channels per chunk for K <= 3, and for K = 7 on the 64x128
    // tile (measured faster); 8 otherwise (larger chunks cost occupancy).
    constexpr int KC = (KT <= 3 || (KT == 7 && BM == 64 && BN == 128)) ? 16 : 8;
    // about two dozen MFMA k-steps (KC/4 per tap) between block additions
    const int flush = (24 / ((KC / 4) * KT)) > 0 ? 24 / ((KC / 4) * KT) : 1;
    const int n_fastest = 0;
    static const std::string name = "conv1d_pipe_kernel<" + std::to_string(BM) + "," +
                                    std::to_string(BN) + "," + std::to_string(WM) + "," +
                                    std::to_string(WN) + "," + std::to_string(KT) + "," +
                                    std::to_string(KC) +
                                    (DM == kDilMax ? std::string() : ",d" + std::to_string(DM)) +
                                    (SN ? ",snake" : "") + ">";
    prof_pre(stream);
    hipLaunchKernelGGL((conv1d_pipe_kernel<BM, BN, WM, WN, KT, KC, DM, SN>), dim3((unsigned)nblk),
                       dim3(WM * WN * 64), 0, stream, x, y, w, Cin, Cout, T, Tout, dil, pad,
                       m_tiles, n_tiles, (int)nblk, flush, n_fastest, ep);
    const hipError_t e = hipGetLastError();
    const double out_n = (double)B * Cout * Tout;
    prof_post(stream, name.c_str(), 2.0 * out_n * Cin * KT,
              4.0 * ((double)B * Cin * T + out_n * (1 + (ep.residual ? 1 : 0) + ep.accumulate) +
                     (double)Cout * Cin * KT));
    return e;
}

// Waits for every vector-memory operation of this wave, LDS DMA included
// (s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima).  Put before
// the barrier that publishes a DMA-staged buffer: the barrier alone does not
// wait for the DMA, and whether the compiler adds the wait depends on the
// schedule (a build with a different register budget dropped it).
__device__ __forceinline__ void wait_dma_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Conv1d with the weight tiles staged by LDS DMA (global_load_lds_dwordx4:
// each lane's 16 bytes go straight from global memory to LDS, no registers,
// no LDS store instructions) into two LDS buffers, so the next K chunk's
// weights stream in during the whole MFMA work on the current chunk, with one
// barrier per chunk.  The input window keeps the register path (its zero
// padding at the sequence ends needs a select), double-buffered in LDS too.
// The staging loads of the next chunk are spread over the k-steps of the
// current one, each pinned between two groups of MFMAs by a scheduling
// barrier (left alone, the compiler sinks them all to the end of the chunk,
// just before the barrier that waits for them); the loads take no lane masks
// (every lane of a wave that issues the last DMA instruction has an LDS slot,
// input offsets are clamped and out-of-range samples zeroed when stored).
// Same GEMM, LDS layouts (padded weight rows), blocked accumulation and
// epilogue as conv1d_pipe_kernel.  Cin must be a multiple of KC.  Used for
// the 96-, 64- and 48-row tiles (measured equal or up to 5% faster than the
// register-prefetch kernel on the 96- and 48-row ones); the 32- and 16-row
// tiles keep conv1d_pipe_kernel.
// Input channels per K chunk of conv1d_dma_kernel: 16 for up to 3 taps; 4 for
// 11 taps (on the 64x128 tile 33 KB of LDS and 142 VGPRs: three blocks per
// CU, which share the CUs better with the other AMP blocks' kernels running
// beside them), except on the 96-column tile, whose grids are one round of
// two blocks per CU (8: fewer barriers); 8 otherwise.  The 160-column tile
// (three blocks per CU, 150-168 VGPRs) takes 8 for up to 3 taps and 4
// otherwise.
template <int BN, int KT>
constexpr int dma_kc() {
    return BN == 160 ? (KT <= 3 ? 8 : 4) : KT <= 3 ? 16 : (KT == 11 && BN != 96) ? 4 : 8;
}

template <int BM, int BN, int WM, int WN, int KT, int KC, int DM, bool SN>
__global__ __launch_bounds__(WM * WN * 64, ((KT == 11 && KC == 4) || BN == 160) ? 3 : 2) void conv1d_dma_kernel(
    const float* __restrict__ x, float* y, const float* __restrict__ w, int Cin, int Cout,
    int T, int Tout, int dil, int pad, int m_tiles, int n_tiles, int nblk, int flush, int mg,
    ConvEpilogue ep) {
    constexpr int NT = WM * WN * 64;
    static_assert(NT == 256, "256 threads");
    constexpr int kXLanes = NT / KC;  // lanes per staged input row
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 16, NTL = WTN / 16;
    constexpr int WROW = KC * KT;                          // weight floats per row per chunk
    constexpr int WS = (WROW % 8 == 0) ? WROW + 4 : WROW + 8;  // padded LDS row (floats)
    constexpr int GR = WS / 4, GV = WROW / 4;              // 16-byte granules per row
    constexpr int NG = BM * GR;                            // granules per weight buffer
    constexpr int NI = (NG + NT - 1) / NT;                 // DMA instructions per thread
    // floats per weight buffer: every lane of a wave that takes part in the
    // last DMA instruction has a slot (waves wholly past the tile skip it)
    constexpr int WBUF = (NG + 63) / 64 * 64 * 4;
    constexpr int XW_MAX = BN + (KT - 1) * DM;
    constexpr int XS = xs_stride_const(XW_MAX);
    constexpr int X_PT = (XW_MAX + kXLanes - 1) / kXLanes;
    static_assert(WROW % 4 == 0, "float4 weight rows");
    static_assert(X_PT * kXLanes <= XS, "unconditional input stores stay inside the row");

    __shared__ __align__(16) float WsA[WBUF];
    __shared__ __align__(16) float WsB[WBUF];
    __shared__ __align__(16) float XsA[KC * XS];
    __shared__ __align__(16) float XsB[KC * XS];

    // Logical tiles in groups of mg output-channel tiles that sweep all time
    // tiles (channel tile fastest inside a group): an XCD's contiguous range
    // then needs the weights of about mg channel tiles, sized on the host to
    // stay in its L2, while neighbouring tiles still share the input window.
    const int lid = xcd_remap(blockIdx.x, nblk);
    const int nn_tiles = nblk / m_tiles;  // time tiles x batch
    const int grp = lid / (mg * nn_tiles);
    const int m_lo = grp * mg;
    const int mg_eff = min(mg, m_tiles - m_lo);
    const int r_in = lid - m_lo * nn_tiles;
    const int mt_i = m_lo + r_in % mg_eff;
    const int rest = r_in / mg_eff;
    const int nt_i = rest % n_tiles;
    const int b = rest / n_tiles;
    const int o0 = mt_i * BM, t0 = nt_i * BN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm0 = (wid / WN) * WTM, wn0 = (wid % WN) * WTN;
    const int l16 = lane & 15, g = lane >> 4;
    const int xrow = tid / kXLanes, xcol = tid % kXLanes;

    f32x4 acc[MT][NTL], part[MT][NTL];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int c = 0; c < NTL; ++c) {
            acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            part[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    unsigned woff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int q = i * NT + tid;
        const int row = q / GR;
        int f4 = q - row * GR;
        int o = o0 + row;
        if (row >= BM || o >= Cout) o = o0;
        if (f4 >= GV) f4 = 0;
        woff[i] = (unsigned)(o * Cin * KT + 4 * f4);
    }
    const int xw = BN + (KT - 1) * dil;
    const float* xb = x + (size_t)b * Cin * T;
    const int nch = Cin / KC;
    // clamped input offsets (the loads never leave the row; out-of-range
    // samples are zeroed when stored)
    int xoff[X_PT];
    bool xin[X_PT];
#pragma unroll
    for (int r = 0; r < X_PT; ++r) {
        const int u = xcol + r * kXLanes;
        const int t = t0 - pad + u;
        xin[r] = u < xw && t >= 0 && t < T;
        xoff[r] = min(max(t, 0), T - 1);
    }
    float xr[X_PT];
    float xa = 1.f;
    // Up to 3 taps with KC KT a multiple of 16: the chunk's k-steps go in
    // groups of four, and in group q lane g's four steps take the flattened
    // (channel, tap) indices f = 16 q + 4 g + t, t = 0..3 (any assignment of
    // the indices to (step, lane group) is the same sum), so that its four
    // weights are one aligned 16-byte LDS read; its input row for step s is
    // channel f / KT at tap offset (f % KT) dil.
    constexpr bool kGrouped = KT <= 3 && (KC * KT) % 16 == 0;
    constexpr int kSlotsG = kGrouped ? KC * KT / 4 : 1;
    int boff[kSlotsG];
#pragma unroll
    for (int s4 = 0; s4 < kSlotsG; ++s4) {
        const int f = 16 * (s4 >> 2) + 4 * g + (s4 & 3);
        boff[s4] = (f / KT) * XS + (f % KT) * dil;
    }

    auto dma_one = [&](const float* wc, float* wbuf, int i) {
        if (NG % NT == 0 || i + 1 < NI || i * NT + wid * 64 < NG)  // wave-uniform
            __builtin_amdgcn_global_load_lds((const void*)(wc + woff[i]),
                                             (void*)(wbuf + (i * NT + wid * 64) * 4), 16, 0, 0);
    };
    auto gx_one = [&](const float* xrowp, int r) { xr[r] = xrowp[xoff[r]]; };
    auto sx = [&](float* xbuf) {
        const float arev = xa * 0.15915494309189535f, inv = 1.0f / (xa + 1e-9f);
#pragma unroll
        for (int r = 0; r < X_PT; ++r) {
            float v = xin[r] ? xr[r] : 0.f;
            if (SN && ep.in_alpha) v = xin[r] ? snake_beta(v, arev, inv) : 0.f;
            xbuf[xrow * XS + xcol + r * kXLanes] = v;
        }
    };
    // one chunk: MFMA work on chunk c from (Wc, Xc) with the staging of the
    // next chunk into (Wn, Xn) spread evenly over its k-steps; the last
    // chunk re-stages itself into the free buffers (never read)
    auto step = [&](int c, const float* Wc, const float* Xc, float* Wn, float* Xn) {
        const int cn = (c + 1 < nch) ? c + 1 : c;
        const float* wc = w + (size_t)cn * KC * KT;
        const float* xrowp = xb + (size_t)(cn * KC + xrow) * T;
        if (SN && ep.in_alpha) xa = ep.in_alpha[cn * KC + xrow];
        constexpr int SLOTS = KT * (KC / 4);  // k-steps of the chunk
        constexpr int ITEMS = NI + X_PT;      // staging loads per thread
        // 3-tap chunks are short: their loads go into the first quarter
        constexpr int kSpread = KT <= 3 ? 4 : 1;
        // With 7 or more taps, the operands of k-step s + 1 are read from LDS
        // before the MFMAs of step s (two register sets; the scheduling
        // barrier keeps the compiler from sinking the reads back to their
        // use, where each step then waited on its own loads): 7-tap tiles
        // -4%, 11-tap -0.5%, measured on MI355X.  The 3-tap tiles, whose
        // chunks also carry the staging loads in their first quarter, were 3-4%
        // slower that way and keep loading each step's operands just before
        // use.
        if constexpr (KT > 3) {
            float av[2][MT], bv[2][NTL];
            auto ld = [&](int slot, int buf) {
                const int j = slot / (KC / 4), kk = slot - j * (KC / 4);
#pragma unroll
                for (int a = 0; a < MT; ++a)
                    av[buf][a] = Wc[(wm0 + a * 16 + l16) * WS + (kk * 4 + g) * KT + j];
#pragma unroll
                for (int cc = 0; cc < NTL; ++cc)
                    bv[buf][cc] = Xc[(kk * 4 + g) * XS + wn0 + cc * 16 + l16 + j * dil];
            };
            ld(0, 0);
#pragma unroll
            for (int j = 0; j < KT; ++j) {
#pragma unroll
                for (int kk = 0; kk < KC / 4; ++kk) {
                    const int slot = j * (KC / 4) + kk;
                    const int cb = slot & 1;
                    if (slot + 1 < SLOTS) ld(slot + 1, cb ^ 1);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int a = 0; a < MT; ++a)
#pragma unroll
                        for (int cc = 0; cc < NTL; ++cc)
                            part[a][cc] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                av[cb][a], bv[cb][cc], part[a][cc], 0, 0, 0);
#pragma unroll
                    for (int it = 0; it < ITEMS; ++it)
                        if ((it * SLOTS) / (kSpread * ITEMS) == slot) {
                            if (it < NI) dma_one(wc, Wn, it);
                            else gx_one(xrowp, it - NI);
                            // pin the load here: only VALU, SALU (not MFMA) and LDS
                            // reads may be scheduled across this point
                            __builtin_amdgcn_sched_barrier(0x106);
                        }
                }
            }
        } else if constexpr (kGrouped) {
#pragma unroll
            for (int q = 0; q < SLOTS / 4; ++q) {
                f32x4 a4[MT];
#pragma unroll
                for (int a = 0; a < MT; ++a)
                    a4[a] = *reinterpret_cast<const f32x4*>(Wc + (wm0 + a * 16 + l16) * WS +
                                                            16 * q + 4 * g);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int slot = 4 * q + t;
                    float bv[NTL];
#pragma unroll
                    for (int cc = 0; cc < NTL; ++cc)
                        bv[cc] = Xc[boff[slot] + wn0 + cc * 16 + l16];
#pragma unroll
                    for (int a = 0; a < MT; ++a)
#pragma unroll
                        for (int cc = 0; cc < NTL; ++cc)
                            part[a][cc] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                a4[a][t], bv[cc], part[a][cc], 0, 0, 0);
#pragma unroll
                    for (int it = 0; it < ITEMS; ++it)
                        if ((it * SLOTS) / (kSpread * ITEMS) == slot) {
                            if (it < NI) dma_one(wc, Wn, it);
                            else gx_one(xrowp, it - NI);
                            // pin the load here: only VALU, SALU (not MFMA) and LDS
                            // reads may be scheduled across this point
                            __builtin_amdgcn_sched_barrier(0x106);
                        }
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < KT; ++j) {
#pragma unroll
                for (int kk = 0; kk < KC / 4; ++kk) {
                    float av[MT], bv[NTL];
#pragma unroll
                    for (int a = 0; a < MT; ++a)
                        av[a] = Wc[(wm0 + a * 16 + l16) * WS + (kk * 4 + g) * KT + j];
#pragma unroll
                    for (int cc = 0; cc < NTL; ++cc)
                        bv[cc] = Xc[(kk * 4 + g) * XS + wn0 + cc * 16 + l16 + j * dil];
#pragma unroll
                    for (int a = 0; a < MT; ++a)
#pragma unroll
                        for (int cc = 0; cc < NTL; ++cc)
                            part[a][cc] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                av[a], bv[cc], part[a][cc], 0, 0, 0);
                    const int slot = j * (KC / 4) + kk;
#pragma unroll
                    for (int it = 0; it < ITEMS; ++it)
                        if ((it * SLOTS) / (kSpread * ITEMS) == slot) {
                            if (it < NI) dma_one(wc, Wn, it);
                            else gx_one(xrowp, it - NI);
                            // pin the load here: only VALU, SALU (not MFMA) and LDS
                            // reads may be scheduled across this point
                            __builtin_amdgcn_sched_barrier(0x106);
                        }
                }
            }
        }
        if ((c + 1) % flush == 0 || c + 1 == nch) {
#pragma unroll
            for (int a = 0; a < MT; ++a)
#pragma unroll
                for (int cc = 0; cc < NTL; ++cc) {
                    acc[a][cc] += part[a][cc];
                    part[a][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
        sx(Xn);
        wait_dma_all();
        __syncthreads();
    };

    {
        const float* xrowp = xb + (size_t)xrow * T;
        if (SN && ep.in_alpha) xa = ep.in_alpha[xrow];
#pragma unroll
        for (int i = 0; i < NI; ++i) dma_one(w, WsA, i);
#pragma unroll
        for (int r = 0; r < X_PT; ++r) gx_one(xrowp, r);
        sx(XsA);
        wait_dma_all();
        __syncthreads();
    }
    for (int c = 0; c < nch; c += 2) {
        step(c, WsA, XsA, WsB, XsB);
        if (c + 1 < nch) step(c + 1, WsB, XsB, WsA, XsA);
    }

    conv_epilogue<MT, NTL, SN>(acc, y, Cout, Tout, b, o0 + wm0, t0 + wn0, l16, g, ep);
}

template <int BM, int BN, int WM, int WN, int KT, int DM = kDilMax, bool SN = false>
hipError_t run_conv1d_dma(const float* x, float* y, const float* w, int B, int Cin, int Cout,
                          int T, int Tout, int dil, int pad, const ConvEpilogue& ep,
                          hipStream_t stream) {
    constexpr int KC = dma_kc<BN, KT>();
    const int m_tiles = (Cout + BM - 1) / BM;
    const int n_tiles = (Tout + BN - 1) / BN;
    const long long nblk = (long long)m_tiles * n_tiles * B;
    // (T >= 1: the kernel clamps its input offsets into [0, T-1])
    if (nblk > 0x7fffffffLL || T < 1 || Cin % KC != 0 ||
        (long long)Cout * Cin * KT >= (1LL << 31))
        return hipErrorInvalidValue;
    const int flush = (24 / ((KC / 4) * KT)) > 0 ? 24 / ((KC / 4) * KT) : 1;
    // channel tiles per group: their weights within ~2.5 MB (an XCD's L2 is 4 MB)
    const long long wtile = (long long)BM * Cin * KT * 4;
    const int mg = (int)std::max(1LL, std::min((long long)m_tiles, (5LL << 19) / wtile));
    static const std::string name = "conv1d_dma_kernel<" + std::to_string(BM) + "," +
                                    std::to_string(BN) + "," + std::to_string(WM) + "," +
                                    std::to_string(WN) + "," + std::to_string(KT) + "," +
                                    std::to_string(KC) +
                                    (DM == kDilMax ? std::string() : ",d" + std::to_string(DM)) +
                                    (SN ? ",snake" : "") + ">";
    prof_pre(stream);
    hipLaunchKernelGGL((conv1d_dma_kernel<BM, BN, WM, WN, KT, KC, DM, SN>), dim3((unsigned)nblk),
                       dim3(WM * WN * 64), 0, stream, x, y, w, Cin, Cout, T, Tout, dil, pad,
                       m_tiles, n_tiles, (int)nblk, flush, mg, ep);
    const hipError_t e = hipGetLastError();
    const double out_n = (double)B * Cout * Tout;
    prof_post(stream, name.c_str(), 2.0 * out_n * Cin * KT,
              4.0 * ((double)B * Cin * T + out_n * (1 + (ep.residual ? 1 : 0) + ep.accumulate) +
                     (double)Cout * Cin * KT));
    return e;
}

template <int BM, int BN, int WM, int WN>
hipError_t dispatch_pipe(const float* x, float* y, const float* w, int B, int Cin, int Cout,
                         int T, int Tout, int K, int dil, int pad, const ConvEpilogue& ep,
                         hipStream_t stream) {
    if constexpr (BM == 64 || BM == 96 || BM == 48) {
      if (Cin % (K <= 3 ? 16 : 8) == 0 && (long long)Cout * Cin * K < (1LL << 31)) {
        switch (K) {
            case 1: return run_conv1d_dma<BM, BN, WM, WN, 1>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
            case 3: return run_conv1d_dma<BM, BN, WM, WN, 3>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
            case 7:
                // the DAV units' first conv: both Snakes fused (input staging, epilogue)
                if (ep.in_alpha || ep.snake_alpha) {
                    if (dil > kDilMax)
                        return run_conv1d_dma<BM, BN, WM, WN, 7, 9, true>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
                    return run_conv1d_dma<BM, BN, WM, WN, 7, kDilMax, true>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
                }
                if (dil > kDilMax)
                    return run_conv1d_dma<BM, BN, WM, WN, 7, 9>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
                return run_conv1d_dma<BM, BN, WM, WN, 7>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
            default: return run_conv1d_dma<BM, BN, WM, WN, 11>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
        }
      }
    }
    switch (K) {
        case 1: return run_conv1d_pipe<BM, BN, WM, WN, 1>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
        case 3: return run_conv1d_pipe<BM, BN, WM, WN, 3>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
        case 7:
            // the DAV units' first conv: both Snakes fused (input staging, epilogue)
            if (ep.in_alpha || ep.snake_alpha) {
                if (dil > kDilMax)
                    return run_conv1d_pipe<BM, BN, WM, WN, 7, 9, true>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
                return run_conv1d_pipe<BM, BN, WM, WN, 7, kDilMax, true>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
            }
            if (dil > kDilMax)
                return run_conv1d_pipe<BM, BN, WM, WN, 7, 9>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
            return run_conv1d_pipe<BM, BN, WM, WN, 7>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
        default: return run_conv1d_pipe<BM, BN, WM, WN, 11>(x, y, w, B, Cin, Cout, T, Tout, dil, pad, ep, stream);
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t dispatch_k(const float* x, float* y, const float* w, int B, int Cin, int Cout, int T,
                      int Tout, int K, int dil, int pad, const ConvEpilogue& ep,
                      hipStream_t stream) {
    switch (K) {
        case 1: return run_conv1d<BM, BN, WM, WN, 1>(x, y, w, B, Cin, Cout, T, Tout, K, dil, pad, ep, stream);
        case 3: return run_conv1d<BM, BN, WM, WN, 3>(x, y, w, B, Cin, Cout, T, Tout, K, dil, pad, ep, stream);
        case 7: return run_conv1d<BM, BN, WM, WN, 7>(x, y, w, B, Cin, Cout, T, Tout, K, dil, pad, ep, stream);
        case 11: return run_conv1d<BM, BN, WM, WN, 11>(x, y, w, B, Cin, Cout, T, Tout, K, dil, pad, ep, stream);
        default: return run_conv1d<BM, BN, WM, WN, 0>(x, y, w, B, Cin, Cout, T, Tout, K, dil, pad, ep, stream);
    }
}

// ------------------------------------------------------------------ ConvTranspose1d

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void convtr1d_mfma_kernel(
    const float* __restrict__ x, float* __restrict__ y, const float* __restrict__ w,
    const float* __restrict__ bias, const float* __restrict__ in_alpha, int Cin, int Cout,
    int Tin, int Tout, int K, int s, int pad, int ntap_max, int m_tiles, int q_tiles, int nblk,
    int ws_stride, int xs_stride, int flush) {
    constexpr int NT = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int MT = WTM / 16, NTL = WTN / 16;

    extern __shared__ float lds[];
    float* Ws = lds;                   // [BM][ws_stride]: col i*ntap_max + m
    float* Xs = lds + BM * ws_stride;  // [kKC][xs_stride]: col u <-> x[q0-(ntap_max-1)+u]

    const int lid = xcd_remap(blockIdx.x, nblk);
    const int mt_i = lid % m_tiles;
    int rest = lid / m_tiles;
    const int r = rest % s;
    rest /= s;
    const int qt = rest % q_tiles;
    const int b = rest / q_tiles;

    const int ntap = (r < K) ? (K - r + s - 1) / s : 0;
    const int qmin = -floor_div(r - pad, s);             // ceil((pad - r)/s)
    const int qmax = floor_div(Tout - 1 + pad - r, s);
    const int q0 = qmin + qt * BN;
    if (q0 > qmax) return;  // uniform over the block, before any barrier
    const int o0 = mt_i * BM;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm0 = (wid / WN) * WTM, wn0 = (wid % WN) * WTN;
    const int l16 = lane & 15, g = lane >> 4;

    f32x4 acc[MT][NTL], part[MT][NTL];  // blocked accumulation, as in Conv1d
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int c = 0; c < NTL; ++c) {
            acc[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            part[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const int xw = BN + ntap_max - 1;
    const int wrow = kKC * ntap_max;
    const float* xb = x + (size_t)b * Cin * Tin;
    const int xbase = q0 - (ntap_max - 1);

    int chunk = 0;
    for (int ic0 = 0; ic0 < Cin; ic0 += kKC, ++chunk) {
        for (int e = tid; e < BM * wrow; e += NT) {
            const int ol = e / wrow;
            const int f = e - ol * wrow;
            const int i = f / ntap_max;
            const int m = f - i * ntap_max;
            const int o = o0 + ol, ic = ic0 + i;
            float v = 0.f;
            if (o < Cout && ic < Cin && m < ntap) v = w[((size_t)ic * Cout + o) * K + r + s * m];
            Ws[ol * ws_stride + f] = v;
        }
        for (int e = tid; e < kKC * xw; e += NT) {
            const int i = e / xw;
            const int u = e - i * xw;
            const int t = xbase + u;
            float v = 0.f;
            if (ic0 + i < Cin && t >= 0 && t < Tin) {
                v = xb[(size_t)(ic0 + i) * Tin + t];
                if (in_alpha) v = snake_plain(v, in_alpha[ic0 + i]);
            }
            Xs[i * xs_stride + u] = v;
        }
        __syncthreads();
        for (int m = 0; m < ntap; ++m) {
#pragma unroll
            for (int kk = 0; kk < kKC / 4; ++kk) {
                float av[MT], bv[NTL];
#pragma unroll
                for (int a = 0; a < MT; ++a)
                    av[a] = Ws[(wm0 + a * 16 + l16) * ws_stride + (kk * 4 + g) * ntap_max + m];
#pragma unroll
                for (int c = 0; c < NTL; ++c)
                    bv[c] = Xs[(kk * 4 + g) * xs_stride + wn0 + c * 16 + l16 + (ntap_max - 1 - m)];
#pragma unroll
                for (int a = 0; a < MT; ++a)
#pragma unroll
                    for (int c = 0; c < NTL; ++c)
                        part[a][c] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[a], bv[c],
                                                                          part[a][c], 0, 0, 0);
            }
        }
        if ((chunk + 1) % flush == 0 || ic0 + kKC >= Cin) {
#pragma unroll
            for (int a = 0; a < MT; ++a)
#pragma unroll
                for (int c = 0; c < NTL; ++c) {
                    acc[a][c] += part[a][c];
                    part[a][c] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
        __syncthreads();
    }

    float* yb = y + (size_t)b * Cout * Tout;
#pragma unroll
    for (int a = 0; a < MT; ++a) {
#pragma unroll
        for (int c = 0; c < NTL; ++c) {
            const int q = q0 + wn0 + c * 16 + l16;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int o = o0 + wm0 + a * 16 + g * 4 + rr;
                if (o < Cout && q <= qmax) {
                    float v = acc[a][c][rr];
                    if (bias) v += bias[o];
                    yb[(size_t)o * Tout + (q * s + r - pad)] = v;
                }
            }
        }
    }
}

// All-phase polyphase ConvTranspose1d for the decoder's (K, stride) pairs.
// One block owns BMo = 16*WM output channels x NQ consecutive q (input-rate
// positions) and computes every phase r of them: output t' = q*S + r - pad.
// Each wave owns 16 channels and all S phases (one 16-row MFMA tile per
// phase), so a phase with fewer taps (r + S*m >= K) simply issues fewer
// MFMAs.  The input window x[q0-NTAP+1 .. q0+NQ) and the weight slice
// w[ic][o0 .. o0+BMo)[0 .. K) (contiguous in the caller's [Cin, Cout, K]
// layout) are staged once per K chunk for all phases, with the next chunk
// prefetched into registers during the MFMA work, as in conv1d_pipe_kernel
// (convtr1d_dma_kernel below stages the weights by LDS DMA instead).
constexpr int kKCT = 16;  // input channels per ConvT K chunk

template <int WM, int WN, int NTL, int KT, int S>
__global__ __launch_bounds__(WM * WN * 64) void convtr1d_poly_kernel(
    const float* __restrict__ x, float* __restrict__ y, const float* __restrict__ w,
    const float* __restrict__ bias, const float* __restrict__ in_alpha, int Cin, int Cout,
    int Tin, int Tout, int pad, int qlo, int m_tiles, int q_tiles, int nblk, int flush) {
    constexpr int NT = WM * WN * 64;
    static_assert(NT == 256, "256 threads");
    constexpr int BMO = 16 * WM;              // output channels per block
    constexpr int NQ = 16 * NTL * WN;         // q positions per block
    constexpr int NTAP = (KT + S - 1) / S;    // taps of the longest phase
    constexpr int WROW = BMO * KT;            // weight floats per input channel
    constexpr int RS = (WROW % 32 <= 16) ? WROW - WROW % 32 + 16 : WROW - WROW % 32 + 48;
    static_assert(WROW % 4 == 0, "float4 weight slices");
    constexpr int WV = WROW / 4;              // float4 per input channel
    constexpr int W_PT = (kKCT * WV + NT - 1) / NT;
    constexpr int XW = NQ + NTAP - 1;
    constexpr int XS = xs_stride_const(XW);
    constexpr int XR = NT / kKCT;             // lanes per staged input row
    constexpr int X_PT = (XW + XR - 1) / XR;

    __shared__ float Ws[kKCT * RS];
    __shared__ float Xs[kKCT * XS];

    const int lid = xcd_remap(blockIdx.x, nblk);
    const int qt = lid % q_tiles;
    const int rest = lid / q_tiles;
    const int mt_i = rest % m_tiles;
    const int b = rest / m_tiles;
    const int o0 = mt_i * BMO;
    const int q0 = qlo + qt * NQ;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn0 = (wid % WN) * (16 * NTL);
    const int l16 = lane & 15, g = lane >> 4;
    const int xrow = tid / XR, xcol = tid % XR;

    f32x4 acc[S][NTL], part[S][NTL];
#pragma unroll
    for (int r = 0; r < S; ++r)
#pragma unroll
        for (int c = 0; c < NTL; ++c) {
            acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            part[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const float* xb = x + (size_t)b * Cin * Tin;
    const int xbase = q0 - (NTAP - 1);
    const int nch = (Cin + kKCT - 1) / kKCT;
    float4 wr[W_PT];
    float xr[X_PT];
    float xa = 1.f;  // Snake alpha of this thread's staged input row

    auto gload = [&](int ic0) {
#pragma unroll
        for (int k = 0; k < W_PT; ++k) {
            const int e = tid + k * NT;
            const int i = e / WV;
            const int f = 4 * (e - i * WV);  // (o - o0) * KT + j, multiple of 4
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (e < kKCT * WV && ic0 + i < Cin && o0 * KT + f < Cout * KT)
                v = *reinterpret_cast<const float4*>(w + ((size_t)(ic0 + i) * Cout + o0) * KT + f);
            wr[k] = v;
        }
        const int ic = ic0 + xrow;
#pragma unroll
        for (int k = 0; k < X_PT; ++k) {
            const int u = xcol + k * XR;
            const int t = xbase + u;
            float v = 0.f;
            if (u < XW && ic < Cin && t >= 0 && t < Tin) v = xb[(size_t)ic * Tin + t];
            xr[k] = v;
        }
        if (in_alpha) xa = ic < Cin ? in_alpha[ic] : 1.f;
    };
    auto lstore = [&]() {
#pragma unroll
        for (int k = 0; k < W_PT; ++k) {
            const int e = tid + k * NT;
            if (e < kKCT * WV) {
                const int i = e / WV;
                *reinterpret_cast<float4*>(Ws + i * RS + 4 * (e - i * WV)) = wr[k];
            }
        }
        if (in_alpha) {
            const float arev = xa * 0.15915494309189535f, inv = 1.0f / (xa + 1e-9f);
#pragma unroll
            for (int k = 0; k < X_PT; ++k) xr[k] = snake_beta(xr[k], arev, inv);
        }
#pragma unroll
        for (int k = 0; k < X_PT; ++k) {
            const int u = xcol + k * XR;
            if (u < XW) Xs[xrow * XS + u] = xr[k];
        }
    };

    gload(0);
    lstore();
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch) gload((c + 1) * kKCT);
#pragma unroll
        for (int m = 0; m < NTAP; ++m) {
#pragma unroll 1
            for (int kk = 0; kk < kKCT / 4; ++kk) {
                float bv[NTL];
#pragma unroll
                for (int cc = 0; cc < NTL; ++cc)
                    bv[cc] = Xs[(kk * 4 + g) * XS + wn0 + cc * 16 + l16 + (NTAP - 1 - m)];
#pragma unroll
                for (int r = 0; r < S; ++r) {
                    if (r + S * m < KT) {
                        const float av =
                            Ws[(kk * 4 + g) * RS + (wm * 16 + l16) * KT + r + S * m];
#pragma unroll
                        for (int cc = 0; cc < NTL; ++cc)
                            part[r][cc] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                av, bv[cc], part[r][cc], 0, 0, 0);
                    }
                }
            }
        }
        if ((c + 1) % flush == 0 || c + 1 == nch) {
#pragma unroll
            for (int r = 0; r < S; ++r)
#pragma unroll
                for (int cc = 0; cc < NTL; ++cc) {
                    acc[r][cc] += part[r][cc];
                    part[r][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
        __syncthreads();
        if (c + 1 < nch) {
            lstore();
            __syncthreads();
        }
    }

    float* yb = y + (size_t)b * Cout * Tout;
    // bias loaded before the first store (a store could alias it, which
    // would make every later load wait for it)
    float bv[4];
#pragma unroll
    for (int ri = 0; ri < 4; ++ri) {
        const int o = o0 + wm * 16 + g * 4 + ri;
        bv[ri] = (bias && o < Cout) ? bias[o] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < S; ++r) {
#pragma unroll
        for (int cc = 0; cc < NTL; ++cc) {
            const int q = q0 + wn0 + cc * 16 + l16;
            const int t = q * S + r - pad;
#pragma unroll
            for (int ri = 0; ri < 4; ++ri) {
                const int o = o0 + wm * 16 + g * 4 + ri;
                if (o < Cout && t >= 0 && t < Tout) {
                    float v = acc[r][cc][ri];
                    if (bias) v += bv[ri];
                    yb[(size_t)o * Tout + t] = v;
                }
            }
        }
    }
}

// convtr1d_poly_kernel with the weight slices staged by LDS DMA
// (global_load_lds_dwordx4) into two LDS buffers, as in conv1d_dma_kernel:
// the next K chunk's weights stream in during the MFMA work on the current
// chunk, one barrier per chunk; the input window keeps the register path
// (zero padding, optional Snake), also double-buffered.  Cin must be a
// multiple of kKCT.  Same GEMM, LDS layouts and summation order.
template <int WM, int WN, int NTL, int KT, int S>
__global__ __launch_bounds__(WM * WN * 64) void convtr1d_dma_kernel(
    const float* __restrict__ x, float* __restrict__ y, const float* __restrict__ w,
    const float* __restrict__ bias, const float* __restrict__ in_alpha, int Cin, int Cout,
    int Tin, int Tout, int pad, int qlo, int m_tiles, int q_tiles, int nblk) {
    constexpr int NT = WM * WN * 64;
    static_assert(NT == 256, "256 threads");
    constexpr int BMO = 16 * WM;              // output channels per block
    constexpr int NQ = 16 * NTL * WN;         // q positions per block
    constexpr int NTAP = (KT + S - 1) / S;    // taps of the longest phase
    constexpr int WROW = BMO * KT;            // weight floats per input channel
    constexpr int RS = (WROW % 32 <= 16) ? WROW - WROW % 32 + 16 : WROW - WROW % 32 + 48;
    static_assert(WROW % 4 == 0 && RS % 4 == 0, "float4 weight slices");
    constexpr int GR = RS / 4, GV = WROW / 4; // 16-byte granules per row: padded, valid
    constexpr int NG = kKCT * GR;             // granules per weight buffer
    constexpr int NI = (NG + NT - 1) / NT;    // DMA instructions per thread
    constexpr int XW = NQ + NTAP - 1;
    constexpr int XS = xs_stride_const(XW);
    constexpr int XR = NT / kKCT;             // lanes per staged input row
    constexpr int X_PT = (XW + XR - 1) / XR;

    __shared__ __align__(16) float WsA[NG * 4];
    __shared__ __align__(16) float WsB[NG * 4];
    __shared__ __align__(16) float XsA[kKCT * XS];
    __shared__ __align__(16) float XsB[kKCT * XS];

    const int lid = xcd_remap(blockIdx.x, nblk);
    const int qt = lid % q_tiles;
    const int rest = lid / q_tiles;
    const int mt_i = rest % m_tiles;
    const int b = rest / m_tiles;
    const int o0 = mt_i * BMO;
    const int q0 = qlo + qt * NQ;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid / WN, wn0 = (wid % WN) * (16 * NTL);
    const int l16 = lane & 15, g = lane >> 4;
    const int xrow = tid / XR, xcol = tid % XR;

    f32x4 acc[S][NTL], part[S][NTL];
#pragma unroll
    for (int r = 0; r < S; ++r)
#pragma unroll
        for (int c = 0; c < NTL; ++c) {
            acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
            part[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // Granule q = i*NT + tid of the padded [kKCT][GR] buffer: input channel
    // q / GR, float4 q % GR of its [BMO x KT] slice.  Pad granules and
    // granules past Cout re-fetch the slice's first float4 (in bounds; never
    // read, or masked by the epilogue); lanes past the buffer issue no DMA.
    int woff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int q = i * NT + tid;
        const int ic = q / GR;
        int f = q - ic * GR;
        if (f >= GV || o0 * KT + 4 * f >= Cout * KT) f = 0;
        woff[i] = (ic < kKCT ? ic : 0) * Cout * KT + o0 * KT + 4 * f;
    }
    const float* xb = x + (size_t)b * Cin * Tin;
    const int xbase = q0 - (NTAP - 1);
    const int nch = Cin / kKCT;
    float xr[X_PT];
    float xa = 1.f;  // Snake alpha of this thread's staged input row
    // this thread's input offsets, clamped into the row (the loads never
    // leave it; samples outside [0, Tin) and past the window are zeroed when
    // stored): the same for every chunk, so no index arithmetic per chunk
    int xoff[X_PT];
    bool xin[X_PT];
#pragma unroll
    for (int k = 0; k < X_PT; ++k) {
        const int u = xcol + k * XR;
        const int t = xbase + u;
        xin[k] = u < XW && t >= 0 && t < Tin;
        xoff[k] = min(max(t, 0), Tin - 1);
    }
    static_assert(X_PT * XR <= XS, "unconditional input stores stay inside the row");

    auto dma_w = [&](int ic0, float* wbuf) {
        const float* wc = w + (size_t)ic0 * Cout * KT;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            if ((i + 1) * NT <= NG || i * NT + tid < NG)
                __builtin_amdgcn_global_load_lds((const void*)(wc + woff[i]),
                                                 (void*)(wbuf + (i * NT + wid * 64) * 4), 16, 0,
                                                 0);
    };
    auto gx = [&](int ic0) {
        const int ic = ic0 + xrow;
        const float* xrowp = xb + (size_t)ic * Tin;
#pragma unroll
        for (int k = 0; k < X_PT; ++k) xr[k] = xrowp[xoff[k]];
        if (in_alpha) xa = in_alpha[ic];
    };
    auto sx = [&](float* xbuf) {
        if (in_alpha) {
            const float arev = xa * 0.15915494309189535f, inv = 1.0f / (xa + 1e-9f);
#pragma unroll
            for (int k = 0; k < X_PT; ++k) xr[k] = snake_beta(xr[k], arev, inv);
        }
#pragma unroll
        for (int k = 0; k < X_PT; ++k) xbuf[xrow * XS + xcol + k * XR] = xin[k] ? xr[k] : 0.f;
    };
    // K chunks summed on the matrix cores before each add into acc, fixed by
    // the tap count (the host computes the same value for the poly kernel).
    // With one or two the add sits at a fixed place in the two-chunk loop
    // body, so part stays in the accumulation registers across chunks
    // instead of being copied out and back each chunk (k=11 s=5: 266 ->
    // 257 us at 1536 -> 768 channels, same sums in the same order).
    constexpr int FL = 24 / (NTAP * (kKCT / 4)) > 0 ? 24 / (NTAP * (kKCT / 4)) : 1;
    auto step = [&](int c, const float* Wc, const float* Xc, float* Wn, float* Xn, bool fl) {
        if (c + 1 < nch) {
            dma_w((c + 1) * kKCT, Wn);
            gx((c + 1) * kKCT);
        }
        // The substeps (tap m, channels kk*4 .. kk*4+3), m outer, fully
        // unrolled, each substep's operands read from LDS before the previous
        // substep's MFMAs (two register sets, pinned by a scheduling
        // barrier), so the matrix work does not wait on its own reads: for
        // the tiles where that keeps the occupancy (one time tile per wave:
        // 168 VGPRs, three blocks per CU; the stride-2 tiles of two or four
        // channel tiles: 232-248, two blocks per CU as before).  Measured on
        // MI355X: k=11 s=5 16 x 64 tiles 272 -> 248 us at 1536 -> 768
        // channels; stride 2, 64 x 64 tiles 104 -> 95 us, 32 x 128 tiles 87
        // -> 75 us.  The others would drop to one block per CU (280 VGPRs)
        // and keep the rolled loop.
        if constexpr (NTL == 1 || (S == 2 && WM >= 2)) {
            constexpr int NSUB = NTAP * (kKCT / 4);
            float avb[2][S], bvb[2][NTL];
            auto ldo = [&](int sub, int buf) {
                const int m = sub / (kKCT / 4), kk = sub - m * (kKCT / 4);
#pragma unroll
                for (int cc = 0; cc < NTL; ++cc)
                    bvb[buf][cc] = Xc[(kk * 4 + g) * XS + wn0 + cc * 16 + l16 + (NTAP - 1 - m)];
#pragma unroll
                for (int r = 0; r < S; ++r)
                    if (r + S * m < KT)
                        avb[buf][r] = Wc[(kk * 4 + g) * RS + (wm * 16 + l16) * KT + r + S * m];
            };
            ldo(0, 0);
#pragma unroll
            for (int sub = 0; sub < NSUB; ++sub) {
                const int m = sub / (kKCT / 4);
                const int cb = sub & 1;
                if (sub + 1 < NSUB) ldo(sub + 1, cb ^ 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int r = 0; r < S; ++r)
                    if (r + S * m < KT) {
#pragma unroll
                        for (int cc = 0; cc < NTL; ++cc)
                            part[r][cc] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                avb[cb][r], bvb[cb][cc], part[r][cc], 0, 0, 0);
                    }
            }
        } else {
#pragma unroll
            for (int m = 0; m < NTAP; ++m) {
#pragma unroll 1
                for (int kk = 0; kk < kKCT / 4; ++kk) {
                    float bv[NTL];
#pragma unroll
                    for (int cc = 0; cc < NTL; ++cc)
                        bv[cc] = Xc[(kk * 4 + g) * XS + wn0 + cc * 16 + l16 + (NTAP - 1 - m)];
#pragma unroll
                    for (int r = 0; r < S; ++r) {
                        if (r + S * m < KT) {
                            const float av =
                                Wc[(kk * 4 + g) * RS + (wm * 16 + l16) * KT + r + S * m];
#pragma unroll
                            for (int cc = 0; cc < NTL; ++cc)
                                part[r][cc] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                                    av, bv[cc], part[r][cc], 0, 0, 0);
                        }
                    }
                }
            }
        }
        if (fl) {
#pragma unroll
            for (int r = 0; r < S; ++r)
#pragma unroll
                for (int cc = 0; cc < NTL; ++cc) {
                    acc[r][cc] += part[r][cc];
                    part[r][cc] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
        }
        if (c + 1 < nch) sx(Xn);
        // this wave's DMA of chunk c+1 has landed
        wait_dma_all();
        __syncthreads();
    };

    dma_w(0, WsA);
    gx(0);
    sx(XsA);
    wait_dma_all();
    __syncthreads();
    for (int c = 0; c < nch; c += 2) {
        if constexpr (FL <= 2) {
            step(c, WsA, XsA, WsB, XsB, FL == 1);
            if (c + 1 < nch) step(c + 1, WsB, XsB, WsA, XsA, true);
        } else {
            step(c, WsA, XsA, WsB, XsB, (c + 1) % FL == 0 || c + 1 == nch);
            if (c + 1 < nch)
                step(c + 1, WsB, XsB, WsA, XsA, (c + 2) % FL == 0 || c + 2 == nch);
        }
    }
    if constexpr (FL == 2) {
        // an odd chunk count leaves the last chunk in part (else part is 0)
#pragma unroll
        for (int r = 0; r < S; ++r)
#pragma unroll
            for (int cc = 0; cc < NTL; ++cc) acc[r][cc] += part[r][cc];
    }

    float* yb = y + (size_t)b * Cout * Tout;
    float bvv[4];
#pragma unroll
    for (int ri = 0; ri < 4; ++ri) {
        const int o = o0 + wm * 16 + g * 4 + ri;
        bvv[ri] = (bias && o < Cout) ? bias[o] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < S; ++r) {
#pragma unroll
        for (int cc = 0; cc < NTL; ++cc) {
            const int q = q0 + wn0 + cc * 16 + l16;
            const int t = q * S + r - pad;
#pragma unroll
            for (int ri = 0; ri < 4; ++ri) {
                const int o = o0 + wm * 16 + g * 4 + ri;
                if (o < Cout && t >= 0 && t < Tout) {
                    float v = acc[r][cc][ri];
                    if (bias) v += bvv[ri];
                    yb[(size_t)o * Tout + t] = v;
                }
            }
        }
    }
}

template <int WM, int WN, int NTL, int KT, int S>
hipError_t run_convtr1d_poly(const float* x, float* y, const float* w, const float* bias,
                             const float* in_alpha, int B, int Cin, int Cout, int Tin, int Tout,
                             int pad, hipStream_t stream) {
    constexpr int BMO = 16 * WM;
    constexpr int NQ = 16 * NTL * WN;
    // q = floor((t' + pad) / S) over all outputs t' in [0, Tout)
    const int qlo = pad / S;
    const int qhi = (Tout - 1 + pad) / S;
    const int m_tiles = (Cout + BMO - 1) / BMO;
    const int q_tiles = (qhi - qlo + 1 + NQ - 1) / NQ;
    const long long nblk = (long long)m_tiles * q_tiles * B;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    constexpr int NTAP = (KT + S - 1) / S;
    const int flush = 24 / (NTAP * (kKCT / 4)) > 0 ? 24 / (NTAP * (kKCT / 4)) : 1;
    // LDS-DMA staging when every K chunk is full and the offsets fit in int
    const bool dma = Cin % kKCT == 0 && (long long)Cin * Cout * KT < (1LL << 31);
    static const std::string tile = std::to_string(WM) + "," + std::to_string(WN) + "," +
                                    std::to_string(NTL) + "," + std::to_string(KT) + "," +
                                    std::to_string(S) + ">";
    static const std::string name_poly = "convtr1d_poly_kernel<" + tile;
    static const std::string name_dma = "convtr1d_dma_kernel<" + tile;
    prof_pre(stream);
    if (dma)
        hipLaunchKernelGGL((convtr1d_dma_kernel<WM, WN, NTL, KT, S>), dim3((unsigned)nblk),
                           dim3(WM * WN * 64), 0, stream, x, y, w, bias, in_alpha, Cin, Cout, Tin,
                           Tout, pad, qlo, m_tiles, q_tiles, (int)nblk);
    else
        hipLaunchKernelGGL((convtr1d_poly_kernel<WM, WN, NTL, KT, S>), dim3((unsigned)nblk),
                           dim3(WM * WN * 64), 0, stream, x, y, w, bias, in_alpha, Cin, Cout, Tin,
                           Tout, pad, qlo, m_tiles, q_tiles, (int)nblk, flush);
    const std::string& name = dma ? name_dma : name_poly;
    const hipError_t e = hipGetLastError();
    prof_post(stream, name.c_str(), 2.0 * B * Cin * Cout * (double)KT * Tin,
              4.0 * ((double)B * Cin * Tin + (double)B * Cout * Tout + (double)Cin * Cout * KT));
    return e;
}

// ------------------------------------------------------------------ conv_post (Cout = 1)

constexpr int kOutThreads = 256;
constexpr int kOutChunk = 16;

__global__ __launch_bounds__(kOutThreads) void conv_out1_kernel(
    const float* __restrict__ x, float* __restrict__ y, float* __restrict__ pre,
    const float* __restrict__ w, const float* __restrict__ bias,
    const float* __restrict__ in_alpha, int Cin, int T, int K, int final_act, int interleave2,
    int tiles) {
    extern __shared__ float sm[];
    const int xw = kOutThreads + K - 1;
    float* ws = sm;                 // [Cin*K]
    float* xs = sm + Cin * K;       // [kOutChunk][xw]
    const int b = blockIdx.x / tiles;
    const int t0 = (blockIdx.x - b * tiles) * kOutThreads;
    const int tid = threadIdx.x;
    const int pad = (K - 1) / 2;
    for (int e = tid; e < Cin * K; e += kOutThreads) ws[e] = w[e];
    float acc = 0.f;
    const float* xb = x + (size_t)b * Cin * T;
    for (int ic0 = 0; ic0 < Cin; ic0 += kOutChunk) {
        __syncthreads();
        for (int e = tid; e < kOutChunk * xw; e += kOutThreads) {
            const int i = e / xw;
            const int u = e - i * xw;
            const int t = t0 - pad + u;
            float v = 0.f;
            if (ic0 + i < Cin && t >= 0 && t < T) {
                v = xb[(size_t)(ic0 + i) * T + t];
                if (in_alpha) v = snake_plain(v, in_alpha[ic0 + i]);
            }
            xs[i * xw + u] = v;
        }
        __syncthreads();
        const int nc = min(kOutChunk, Cin - ic0);
        for (int i = 0; i < nc; ++i)
            for (int j = 0; j < K; ++j) acc = fmaf(ws[(ic0 + i) * K + j], xs[i * xw + tid + j], acc);
    }
    const int t = t0 + tid;
    if (t < T) {
        if (bias) acc += bias[0];
        if (pre) pre[(size_t)b * T + t] = acc;
        float v = acc;
        if (final_act == 1) v = tanhf(v);
        else if (final_act == 2) v = fminf(fmaxf(v, -1.f), 1.f);
        // interleave2: rows 2b and 2b+1 are the two sides of output row b
        const size_t yi = interleave2 ? (size_t)(b >> 1) * 2 * T + 2 * (size_t)t + (b & 1)
                                      : (size_t)b * T + t;
        y[yi] = v;
    }
}

__global__ void channel_affine_kernel(const float* __restrict__ x, float* __restrict__ y,
                                      const float* __restrict__ scale,
                                      const float* __restrict__ shift, int C, int T, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x) {
        const int c = (int)((i / (size_t)T) % (size_t)C);
        y[i] = fmaf(x[i], scale[c], shift[c]);
    }
}

}  // namespace

hipError_t launch_conv1d(const float* x, float* y, const float* w, int B, int Cin, int Cout,
                         int T, int Tout, int K, int dilation, int pad, const ConvEpilogue& ep,
                         hipStream_t stream) {
    // Snake in the prologue/epilogue: the 7-tap staged kernels (LDS-DMA or
    // register prefetch), else the generic one
    const bool snake = ep.in_alpha || ep.snake_alpha;
    const bool pipe_ok = (K == 1 || K == 3 || K == 7 || K == 11) && dilation <= dil_max(K) &&
                         (!snake || K == 7) &&
                         Cin % 4 == 0 && ((uintptr_t)w & 15) == 0;
    if (pipe_ok) {
        auto blocks = [&](int bm, int bn) {
            return (long long)((Cout + bm - 1) / bm) * ((Tout + bn - 1) / bn) * B;
        };
        // Cout tiles that divide the decoder's widths: 96 and 48 (H3's 96- and
        // 48-channel stages) avoid padding a 64-row tile.  Long grids (the
        // DAV decoder's 96-channel stage over 441344 samples: 6896 blocks)
        // take 96 x 128 tiles, whose rounds are many enough that only the
        // halved input re-staging counts; short ones keep 96 x 64 (H3 at
        // 40000 samples: 96 x 128 made 626 blocks, 1.2 rounds, 10% slower),
        // and so do 11 taps, which spill at 96 x 128.
        if (Cout % 96 == 0 && Cout % 64 != 0) {
            if (K != 11 && blocks(96, 128) >= 2048)
                return dispatch_pipe<96, 128, 2, 2>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
            return dispatch_pipe<96, 64, 2, 2>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
        }
        if (Cout == 48)
            return dispatch_pipe<48, 128, 1, 4>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
        if (Cout > 32) {
            // 64 x 128 tiles; when that would leave fewer than ~2.5 blocks per
            // CU on 256 CUs, 64 x 96 if those make one resident round of at
            // least 384 blocks (two 4-wave blocks per CU: 512 slots; e.g. 768
            // channels x 2 x 2000 samples: 504 blocks, where 64 x 64 tiles
            // make 768, a round and a half), else 64 x 64.
            // 64 x 160 tiles (three blocks per CU: 768 slots) when they make
            // one resident round where 64 x 128 would make more (384 channels
            // x 2 x 10000 samples: 756 blocks instead of 948; a launch alone
            // 558 -> 516 us at 11 taps, -6% at 7 and 3)
            if ((K == 11 || K == 7 || K == 3) && !snake && Cin % 8 == 0 && dilation <= kDilMax &&
                (long long)Cout * Cin * K < (1LL << 31) && blocks(64, 128) > 768 &&
                blocks(64, 160) <= 768 && blocks(64, 160) >= 600) {
                if (K == 11) return run_conv1d_dma<64, 160, 2, 2, 11>(x, y, w, B, Cin, Cout, T, Tout, dilation, pad, ep, stream);
                if (K == 7) return run_conv1d_dma<64, 160, 2, 2, 7>(x, y, w, B, Cin, Cout, T, Tout, dilation, pad, ep, stream);
                return run_conv1d_dma<64, 160, 2, 2, 3>(x, y, w, B, Cin, Cout, T, Tout, dilation, pad, ep, stream);
            }
            if (blocks(64, 128) >= 640)
                return dispatch_pipe<64, 128, 2, 2>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
            if (blocks(64, 96) >= 384 && blocks(64, 96) <= 512)
                return dispatch_pipe<64, 96, 2, 2>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
            return dispatch_pipe<64, 64, 2, 2>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
        }
        if (Cout > 16)
            return dispatch_pipe<32, 256, 1, 4>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
        return dispatch_pipe<16, 256, 1, 4>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
    }
    // Tile choice: the largest Cout tile that wastes little of the matrix
    // cores, shrunk while the grid would leave the 256 CUs under-filled.
    auto blocks = [&](int bm, int bn) {
        return (long long)((Cout + bm - 1) / bm) * ((Tout + bn - 1) / bn) * B;
    };
    int bm;
    if (Cout >= 256 && Cout % 128 == 0) bm = 128;
    else if (Cout >= 64) bm = 64;
    else if (Cout > 16) bm = 32;
    else bm = 16;
    if (bm == 128 && blocks(128, 128) < 512) bm = 64;
    if (bm == 64 && blocks(64, 128) < 256) bm = 32;
    switch (bm) {
        case 128: return dispatch_k<128, 128, 2, 2>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
        case 64: return dispatch_k<64, 128, 2, 2>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
        case 32: return dispatch_k<32, 256, 1, 4>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
        default: return dispatch_k<16, 256, 1, 4>(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep, stream);
    }
}

hipError_t launch_convtr1d(const float* x, float* y, const float* w, const float* bias, int B,
                           int Cin, int Cout, int Tin, int Tout, int K, int stride, int pad,
                           hipStream_t stream, const float* in_alpha) {
    // float4 weight slices need Cout*K % 4 == 0 and a 16-byte aligned base
    const bool vec = ((long long)Cout * K) % 4 == 0 && ((uintptr_t)w & 15) == 0;
    // 16-channel tiles of 64 positions (twice the blocks of the 32 x 128
    // ones, and the unrolled substep loop with operands read one substep
    // ahead): 1536 -> 768 at 400 positions 333 -> 248 us, 768 -> 384 at 2000
    // positions 279 -> 247 us against 32-channel tiles of 128 positions
    if (vec && stride == 5 && K == 11)
        return run_convtr1d_poly<1, 4, 1, 11, 5>(x, y, w, bias, in_alpha, B, Cin, Cout, Tin, Tout, pad, stream);
    if (vec && stride == 5 && K == 10)
        return run_convtr1d_poly<2, 2, 2, 10, 5>(x, y, w, bias, in_alpha, B, Cin, Cout, Tin, Tout, pad, stream);
    // stride 2: 64-channel tiles of 64 positions, narrower and longer tiles
    // for the narrow stages (Cout <= 32: 16 x 256, e.g. 24 -> 12 at 160000
    // positions 80 -> 37 us; Cout 96: 32 x 128, 100 -> 87 us)
    if (vec && stride == 2 && K == 4 && Cout <= 32)
        return run_convtr1d_poly<1, 4, 4, 4, 2>(x, y, w, bias, in_alpha, B, Cin, Cout, Tin, Tout, pad, stream);
    if (vec && stride == 2 && K == 4 && Cout % 32 == 0 && Cout % 64 != 0)
        return run_convtr1d_poly<2, 2, 4, 4, 2>(x, y, w, bias, in_alpha, B, Cin, Cout, Tin, Tout, pad, stream);
    if (vec && stride == 2 && K == 4)
        return run_convtr1d_poly<4, 1, 4, 4, 2>(x, y, w, bias, in_alpha, B, Cin, Cout, Tin, Tout, pad, stream);
    if (vec && stride == 8 && K == 16)
        return run_convtr1d_poly<2, 2, 1, 16, 8>(x, y, w, bias, in_alpha, B, Cin, Cout, Tin, Tout, pad, stream);
    if (vec && stride == 4 && K == 8)
        return run_convtr1d_poly<2, 2, 2, 8, 4>(x, y, w, bias, in_alpha, B, Cin, Cout, Tin, Tout, pad, stream);
    constexpr int BM = 64, BN = 64, WM = 2, WN = 2;
    const int ntap_max = (K + stride - 1) / stride;
    auto fdiv = [](int a, int b) { int q = a / b; if ((a % b != 0) && ((a < 0) != (b < 0))) --q; return q; };
    int nq = 0;
    for (int r = 0; r < stride; ++r) {
        const int qmin = -fdiv(r - pad, stride);
        const int qmax = fdiv(Tout - 1 + pad - r, stride);
        nq = qmax - qmin + 1 > nq ? qmax - qmin + 1 : nq;
    }
    const int m_tiles = (Cout + BM - 1) / BM;
    const int q_tiles = (nq + BN - 1) / BN;
    const long long nblk = (long long)m_tiles * stride * q_tiles * B;
    if (nblk > 0x7fffffffLL || nq < 1) return hipErrorInvalidValue;
    const int ws_stride = kKC * ntap_max + 1;
    const int xs_stride = xs_stride_for(BN + ntap_max - 1);
    const size_t lds = (size_t)(BM * ws_stride + kKC * xs_stride) * sizeof(float);
    if (lds > 64 * 1024) return hipErrorInvalidValue;
    const int flush = 24 / (2 * ntap_max) > 0 ? 24 / (2 * ntap_max) : 1;
    prof_pre(stream);
    hipLaunchKernelGGL((convtr1d_mfma_kernel<BM, BN, WM, WN>), dim3((unsigned)nblk),
                       dim3(WM * WN * 64), lds, stream, x, y, w, bias, in_alpha, Cin, Cout, Tin,
                       Tout, K, stride, pad, ntap_max, m_tiles, q_tiles, (int)nblk, ws_stride,
                       xs_stride, flush);
    const hipError_t e = hipGetLastError();
    prof_post(stream, "convtr1d_mfma_kernel<64,64,2,2>", 2.0 * B * Cin * Cout * (double)K * Tin,
              4.0 * ((double)B * Cin * Tin + (double)B * Cout * Tout + (double)Cin * Cout * K));
    return e;
}

hipError_t launch_conv_out1(const float* x, float* y, float* pre_final, const float* w,
                            const float* bias, int B, int Cin, int T, int K, int final_act,
                            int interleave2, hipStream_t stream, const float* in_alpha) {
    const int tiles = (T + kOutThreads - 1) / kOutThreads;
    const long long nblk = (long long)tiles * B;
    const size_t lds = (size_t)(Cin * K + kOutChunk * (kOutThreads + K - 1)) * sizeof(float);
    if (nblk > 0x7fffffffLL || lds > 64 * 1024) return hipErrorInvalidValue;
    prof_pre(stream);
    hipLaunchKernelGGL(conv_out1_kernel, dim3((unsigned)nblk), dim3(kOutThreads), lds, stream, x,
                       y, pre_final, w, bias, in_alpha, Cin, T, K, final_act, interleave2, tiles);
    const hipError_t e = hipGetLastError();
    prof_post(stream, "conv_out1_kernel", 2.0 * B * Cin * (double)K * T,
              4.0 * ((double)B * Cin * T + (double)B * T * (pre_final ? 2 : 1) + (double)Cin * K));
    return e;
}

__global__ __launch_bounds__(256) void sum_into_kernel(float* __restrict__ y, const float* __restrict__ a,
                                                      const float* __restrict__ b,
                                                      const float* __restrict__ c, size_t n4,
                                                      int n) {
    // float4 elements; the buffers are 256-byte aligned workspace slots
    for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
        float4 v = reinterpret_cast<float4*>(y)[i];
        const float4 p = reinterpret_cast<const float4*>(a)[i];
        v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
        if (n > 1) {
            const float4 q = reinterpret_cast<const float4*>(b)[i];
            v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
        }
        if (n > 2) {
            const float4 q = reinterpret_cast<const float4*>(c)[i];
            v.x += q.x; v.y += q.y; v.z += q.z; v.w += q.w;
        }
        reinterpret_cast<float4*>(y)[i] = v;
    }
}

hipError_t launch_sum_into(float* y, float* const* x, int n, size_t count, hipStream_t stream) {
    if (n < 1) return hipSuccess;
    if (n > 3 || count % 4 != 0) return hipErrorInvalidValue;
    const size_t n4 = count / 4;
    const unsigned blocks = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
    prof_pre(stream);
    hipLaunchKernelGGL(sum_into_kernel, dim3(blocks), dim3(256), 0, stream, y, x[0],
                       n > 1 ? x[1] : nullptr, n > 2 ? x[2] : nullptr, n4, n);
    const hipError_t e = hipGetLastError();
    prof_post(stream, "sum_into_kernel", (double)n * count, 4.0 * (n + 2) * count);
    return e;
}

hipError_t launch_channel_affine(const float* x, float* y, const float* scale, const float* shift,
                                 int B, int C, int T, hipStream_t stream) {
    const size_t n = (size_t)B * C * T;
    const unsigned blocks = (unsigned)((n + 255) / 256 > 65536 ? 65536 : (n + 255) / 256);
    prof_pre(stream);
    hipLaunchKernelGGL(channel_affine_kernel, dim3(blocks), dim3(256), 0, stream, x, y, scale,
                       shift, C, T, n);
    const hipError_t e = hipGetLastError();
    prof_post(stream, "channel_affine_kernel", 2.0 * n, 8.0 * n);
    return e;
}

}  // namespace avae
