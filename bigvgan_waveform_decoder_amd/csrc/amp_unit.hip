// Fused AMP unit for narrow channel counts (C <= 32), gfx950.
//
// Operation ([H3] = docs.rs page of cortiq_engine/audiovae.rs, item
// AmpBlock::apply; [LTX] = docs.rs page of cortiq_engine/ltxaudio.rs, the AMP
// block): one dilation step of an AMP block,
//   y = x + conv2(act2(conv1(act1(x))))
// where act is Activation1d (2x Kaiser-sinc upsample, SnakeBeta, 2x lowpass
// downsample, polyphase form as in act1d.hip), conv1 is the "same" Conv1d
// with K taps at dilation d and conv2 the one at dilation 1, both with zero
// padding and bias.  Epilogue as the Conv1d one: out = y * out_scale
// (+ out if accumulate), which carries the MRF average.
//
// Why fused: at C <= 32 channels the four separate launches stream six reads
// and four writes of [B, C, T] through HBM, and each convolution alone has
// too few flops per byte to keep the matrix cores busy.  Here one block owns
// a time tile of TT outputs of every channel of one batch row: it stages x
// over the tile plus the unit's halo (H = 10 + (K-1)(d+1)/2 per side) in LDS
// by LDS DMA (no register round trip), runs act1, conv1, act2 and conv2 out
// of LDS, and writes y once.  HBM traffic is one read of x (plus halo) and
// one write of y; the residual x is read again from L2 for the epilogue
// rather than held in registers through the activations.
//
// LDS holds two buffers of C rows.  P holds x, then conv1's output; Q holds
// act1's output, then act2's.  Ranges (global sample index):
//   x      [t0 - H,       t0 + TT + H)        P, NX  = TT + 2H
//   act1   [t0 - H + 5,   t0 + TT + H - 5)    Q, NA1 = NX - 10
//   conv1  [t0 - h2 - 5,  t0 + TT + h2 + 5)   P, N1  = TT + 2 h2 + 10
//   act2   [t0 - h2,      t0 + TT + h2)       Q, N2  = TT + 2 h2
//   y      [t0,           t0 + TT)
// with h1 = (K-1)d/2 and h2 = (K-1)/2 the convolutions' half widths.
//
// Sequence ends: x is staged replicate-padded (x[clamp(t)]); conv1's output
// is replicate-padded in LDS before act2 (the activation's own padding);
// doubled-rate samples outside [0, 2T) take the boundary sample (the
// down-sampler's replicate padding); activation outputs outside [0, T) are
// 0 (the convolutions' zero padding).  Interior tiles run a separate copy of
// the activation without any of this.
//
// Convolutions: implicit GEMM on v_mfma_f32_16x16x4_f32 with M = output
// channel (MT tiles of 16), N = time (16-wide tiles, NTW per wave, every
// tile's accumulator resident), K = tap x input channel.  The A operand
// (weights) is read from a packed copy wt[(j*C + i)*16*MT + o] (rows o >= C
// zero), so a lane's load is part of four contiguous 64-byte segments and is
// reused by all NTW tiles of the wave; the B operand comes from LDS with row
// strides = 16 (mod 32), which puts the four K rows of an MFMA operand in
// distinct bank groups.
#include "act_math.h"
#include "avae_internal.h"

#include <algorithm>
#include <atomic>

namespace avae {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kUT = 256;              // threads per block (4 waves)
// longest run length act_stage picks: 20 with MT = 1, 28 with MT = 2
constexpr int run_max(int MT) { return MT == 1 ? 20 : 28; }
constexpr int kLdsBudget = 80 * 1024; // two blocks per CU
// More co-resident blocks for narrower rows: smaller time tiles (more halo
// work) but more blocks to overlap the phases.  Measured on the decoders'
// stages, each launch alone: three blocks per CU -20% at C = 16 and -5% at
// C = 24 against two; four blocks per CU -7% at C = 12 against three, +6%
// at C = 16.
constexpr int kLdsBudget3 = 53 * 1024;
constexpr int kLdsBudget4 = 40 * 1024;
int unit_blocks_per_cu(int C) { return C <= 12 ? 4 : C <= 24 ? 3 : 2; }
size_t unit_lds_budget(int C) {
    return C <= 12 ? kLdsBudget4 : C <= 24 ? kLdsBudget3 : kLdsBudget;
}

struct UnitArgs {
    const float* x;
    float* y;
    const float* wt1;
    const float* b1;
    const float* wt2;
    const float* b2;
    const float* la1;
    const float* lb1;
    const float* la2;
    const float* lb2;
    int C, T, K, d, TT, tiles, nblk, SP, SQ;
    float out_scale;
    int accumulate;
};

// Activation1d over one LDS range: dst[c][m], m in [0, Nd), is the output at
// global position og + m; src[c][m + i], i in [0, 10], holds the input at
// og - 5 + m + i.  A run computes R consecutive outputs from a window of
// R + 10 inputs: the doubled-rate pairs e[u] = s(2(g-2+u)) and
// o[u] = s(2(g-3+u)+1) both read the inputs u .. u+5 of the window, and
// output r is sum_k down[2k] o[r+k] + down[2k+1] e[r+k] (g = og + m0).
// Runs start at multiples of R floats of 16-float-aligned rows, so an
// interior run reads its window with 16-byte LDS loads and writes a full run
// with them; an edge run (kEdge) reads every input at its clamped position.
template <int R, bool kEdge>
__device__ __forceinline__ void act_run(const float* __restrict__ src, int ss,
                                        float* __restrict__ dst, int ds, int c, int m0, int Nd,
                                        int og, int T, const float* arev, const float* ibeta,
                                        const ActTaps& taps) {
    constexpr int W = R + 12;  // window read (R + 10 used)
    const int g = og + m0;
    float out[R];
    if (kEdge && (g + R <= 0 || g >= T)) {
#pragma unroll
        for (int r = 0; r < R; ++r) out[r] = 0.f;
    } else {
        const float* srow = src + c * ss;
        float xw[W];
        if (!kEdge) {
            const float4* s4 = reinterpret_cast<const float4*>(srow + m0);
#pragma unroll
            for (int i = 0; i < W / 4; ++i) {
                const float4 q = s4[i];
                xw[4 * i] = q.x;
                xw[4 * i + 1] = q.y;
                xw[4 * i + 2] = q.z;
                xw[4 * i + 3] = q.w;
            }
        } else {
            // replicate padding: the input at global p is src at clamp(p)
#pragma unroll
            for (int i = 0; i < W; ++i) xw[i] = srow[min(max(g - 5 + i, 0), T - 1) - (og - 5)];
        }
        const float ar = arev[c], ib = ibeta[c];
        float e[R + 5], o[R + 5];
#pragma unroll
        for (int u = 0; u < R + 5; ++u) {
            float ev = 0.f, ov = 0.f;
#pragma unroll
            for (int k = 0; k < 6; ++k) {
                ev = fmaf(taps.up2[2 * k + 1], xw[u + 5 - k], ev);
                ov = fmaf(taps.up2[2 * k], xw[u + 5 - k], ov);
            }
            e[u] = snake_beta(ev, ar, ib);
            o[u] = snake_beta(ov, ar, ib);
        }
        if (kEdge) {
            const int base = 5 - og;  // src index of global position 0
            if (g < 3) {
                // s(0): the even sample at q = 0 from x[clamp(2 - k)]
                float v = 0.f;
#pragma unroll
                for (int k = 0; k < 6; ++k)
                    v = fmaf(taps.up2[2 * k + 1], srow[base + min(max(2 - k, 0), T - 1)], v);
                const float s0 = snake_beta(v, ar, ib);
#pragma unroll
                for (int u = 0; u < R + 5; ++u) {
                    if (g - 2 + u < 0) e[u] = s0;
                    if (g - 3 + u < 0) o[u] = s0;
                }
            }
            if (g + R + 2 > T - 1 && T - 1 < og + Nd + 5) {
                // s(2T-1): the odd sample at q = T-1 from x[clamp(T+2-k)]
                float v = 0.f;
#pragma unroll
                for (int k = 0; k < 6; ++k)
                    v = fmaf(taps.up2[2 * k], srow[base + min(max(T + 2 - k, 0), T - 1)], v);
                const float sl = snake_beta(v, ar, ib);
#pragma unroll
                for (int u = 0; u < R + 5; ++u) {
                    if (g - 2 + u > T - 1) e[u] = sl;
                    if (g - 3 + u > T - 1) o[u] = sl;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < 6; ++k) {
                acc = fmaf(taps.down[2 * k], o[r + k], acc);
                acc = fmaf(taps.down[2 * k + 1], e[r + k], acc);
            }
            out[r] = (kEdge && (g + r < 0 || g + r >= T)) ? 0.f : acc;
        }
    }
    float* drow = dst + c * ds + m0;
    if (m0 + R <= Nd) {
        float4* d4 = reinterpret_cast<float4*>(drow);
#pragma unroll
        for (int i = 0; i < R / 4; ++i)
            d4[i] = make_float4(out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]);
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (m0 + r < Nd) drow[r] = out[r];
    }
}

// The activation over all C rows of a range: runs of R outputs, one per
// thread per pass.
template <int R, bool kEdge>
__device__ __forceinline__ void act_pass(const float* __restrict__ src, int ss,
                                         float* __restrict__ dst, int ds, int C, int Nd, int og,
                                         int T, const float* arev, const float* ibeta,
                                         const ActTaps& taps) {
    const int runs = (Nd + R - 1) / R;
    const int items = C * runs;
    // (c, run) of item it, advanced by kUT items per pass without a division
    const int add_c = kUT / runs, add_r = kUT - add_c * runs;
    int c = threadIdx.x / runs, run = threadIdx.x - c * runs;
    for (int it = threadIdx.x; it < items; it += kUT) {
        act_run<R, kEdge>(src, ss, dst, ds, c, run * R, Nd, og, T, arev, ibeta, taps);
        c += add_c;
        run += add_r;
        if (run >= runs) {
            run -= runs;
            ++c;
        }
    }
}

// The run length of an interior range: a pass over the block costs about
// one run (R outputs from R + 5 doubled-rate pairs), and C * ceil(Nd / R)
// runs take ceil(C * ceil(Nd / R) / 256) passes; a range just over a
// multiple of 256 runs of 16 would leave most threads idle in its last pass,
// so the length with the fewest pass-pairs wins.  Run lengths are 12, 20 or
// 28 floats: the 64 lanes of a wave read windows R floats apart with 16-byte
// LDS loads, and for R = 4 (mod 8) every 8 consecutive lanes (one LDS cycle
// of 16-byte reads) land in distinct bank groups; R = 16 put 4 lanes, R = 24
// two lanes, on one group.  28 needs the register room of the
// two-blocks-per-CU kernels (kLong).  Edge tiles (two per row) run a
// separate copy with runs of 12: kept apart, the interior copy's window
// loads stay 16-byte vector loads (merged with the edge path's clamped
// reads, the compiler turns them all into 4-byte loads).
template <bool kLong>
__device__ __forceinline__ void act_stage(const float* __restrict__ src, int ss,
                                          float* __restrict__ dst, int ds, int C, int Nd, int og,
                                          int T, bool edge, const float* arev, const float* ibeta,
                                          const ActTaps& taps) {
    if (edge) {
        act_pass<12, true>(src, ss, dst, ds, C, Nd, og, T, arev, ibeta, taps);
        return;
    }
    auto cost = [&](int R) {
        const int items = C * ((Nd + R - 1) / R);
        return ((items + kUT - 1) / kUT) * (R + 5);
    };
    const int c12 = cost(12), c20 = cost(20), c28 = kLong ? cost(28) : 1 << 30;
    if (c28 < c20 && c28 < c12)
        act_pass<kLong ? 28 : 20, false>(src, ss, dst, ds, C, Nd, og, T, arev, ibeta, taps);
    else if (c20 <= c12)
        act_pass<20, false>(src, ss, dst, ds, C, Nd, og, T, arev, ibeta, taps);
    else
        act_pass<12, false>(src, ss, dst, ds, C, Nd, og, T, arev, ibeta, taps);
}

typedef const float __attribute__((address_space(1))) gfloat;

// One convolution of the unit: acc[m][s] = the 16x16 output tile (channel
// tile m, time tile wid + 4 s) of sum_{j,i} W[o][i][j] * Bs[i][n + j*dil].
// K steps run over (tap j, input channels i0 .. i0+3).  Steps go in pairs
// with separate registers for even and odd steps, so every operand is
// loaded one step (B, from LDS) or two steps (A, from L2) before the MFMAs
// that read it and no register copy or branch forces an early wait; an odd
// step count is padded with one step of zero weights (packed that way)
// times the last step's finite B.  Every time tile up to 4*NTW is computed
// (the LDS rows are long enough); callers store only the tiles they need.
template <int MT, int NTW>
__device__ __forceinline__ void conv_tiles(const float* __restrict__ Bs, int sb, int dil,
                                           const float* __restrict__ wt, int C, int K,
                                           f32x4 (&acc)[MT][NTW]) {
    constexpr int CP = 16 * MT;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < NTW; ++s) acc[m][s] = f32x4{0.f, 0.f, 0.f, 0.f};
    // step st = j*(C/4) + i0/4 reads A rows 4*st .. 4*st+3 (= j*C + i0 ..)
    const int steps = K * (C >> 2);
    const int nst = steps + (steps & 1);
    const float* wl = wt + g4 * CP + l16;
    const float* bl = Bs + g4 * sb + wid * 16 + l16;
    // A loads go through an opaque pointer: otherwise the compiler proves a
    // prefetched value equals a reload of its address and moves the load
    // (and a full wait) to the use.
    auto load_a = [&](int st, float (&a)[MT]) {
        const int sc = st < nst ? st : nst - 1;
        const gfloat* wq = (const gfloat*)wl;
        asm volatile("" : "+v"(wq));
#pragma unroll
        for (int m = 0; m < MT; ++m) a[m] = wq[4 * sc * CP + m * 16];
    };
    // (pi0, pj): coordinates of step ps, the next B to load (stops at the last)
    int pi0 = 0, pj = 0, ps = 0;
    auto load_b = [&](float (&b)[NTW]) {
        const float* brow = bl + pi0 * sb + pj;
#pragma unroll
        for (int s = 0; s < NTW; ++s) b[s] = brow[64 * s];
        if (ps + 1 < steps) {
            ++ps;
            pi0 += 4;
            if (pi0 >= C) {
                pi0 = 0;
                pj += dil;
            }
        }
    };
    auto mma = [&](const float (&a)[MT], const float (&b)[NTW]) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int s = 0; s < NTW; ++s)
                acc[m][s] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[m], b[s], acc[m][s], 0, 0, 0);
    };
    float aE[MT], aO[MT], bE[NTW], bO[NTW];
    load_a(0, aE);
    load_a(1, aO);
    load_b(bE);
    for (int st = 0; st < nst; st += 2) {
        load_b(bO);
        mma(aE, bE);
        load_a(st + 2, aE);
        load_b(bE);
        mma(aO, bO);
        load_a(st + 3, aO);
    }
}

// x[clamp(t0 - H + u)] for u in [0, NX) of every channel into P by LDS DMA
// (global_load_lds_dword: lane l's sample goes straight to LDS at the chunk
// start + l, no registers): each DMA instruction of a wave fills a chunk of
// 64 samples of one row.  A row's last chunk starts at NX - 64 and rewrites
// the overlap with the chunk before it with the same values, so no chunk
// crosses into the next row; a row shorter than 64 (NX >= 36) takes one
// chunk whose tail lands in the row's padding (SP >= 64 NTW >= 128).  The
// caller waits for the loads (vmcnt) before the barrier that publishes P.
__device__ __forceinline__ void stage_x(const float* __restrict__ xb, float* P, int SP, int C,
                                        int T, int t0, int H, int NX, int wid, int lane) {
    const int nch = (NX + 63) / 64;
    for (int k = wid; k < C * nch; k += kUT / 64) {
        const int c = k / nch, j = k - c * nch;
        const int u0 = (NX > 64 && j == nch - 1) ? NX - 64 : 64 * j;
        const int t = min(max(t0 - H + u0 + lane, 0), T - 1);
        __builtin_amdgcn_global_load_lds((const void*)(xb + (size_t)c * T + t),
                                         (void*)(P + c * SP + u0), 4, 0, 0);
    }
}

// Waits for this wave's outstanding vector memory operations (the LDS DMA
// of stage_x; also its stores).
__device__ __forceinline__ void wait_vmem() {
    // s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maxima
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int MT, int NTW>
// The register budget of up to four (MT = 1, NTW <= 6) or three (NTW <= 8 with
// MT = 1, NTW <= 4 with MT = 2) co-resident blocks, so that the register
// file does not undo the LDS plan.
__global__ __launch_bounds__(kUT, (MT == 1 && NTW <= 6) ? 4
                                  : (NTW <= 8 && (MT == 1 || NTW <= 4)) ? 3
                                                                        : 2) void amp_unit_kernel(UnitArgs a, ActTaps taps) {
    extern __shared__ __align__(16) float lds[];
    const int C = a.C, T = a.T, K = a.K, d = a.d, TT = a.TT, SP = a.SP, SQ = a.SQ;
    const int h1 = (K - 1) * d / 2, h2 = (K - 1) / 2, H = h1 + h2 + 10;
    const int NX = TT + 2 * H, NA1 = NX - 10, N1 = TT + 2 * h2 + 10, N2 = TT + 2 * h2;
    const int NT2 = TT >> 4;
    float* P = lds;
    float* Q = lds + C * SP;
    float* prm = Q + C * SQ;  // alpha/2pi and 1/beta of act1, then of act2

    const int lid = xcd_spread(blockIdx.x, a.nblk);
    const int b = lid / a.tiles;
    const int t0 = (lid - b * a.tiles) * TT;
    const size_t row0 = (size_t)b * C * T;
    const float* __restrict__ xb = a.x + row0;
    const bool edge = (t0 - H < 0) || (t0 + TT + H > T);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;

    // Biases at this lane's output channels, loaded while x streams in.
    float bias1[MT][4], bias2[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int o = m * 16 + 4 * g4 + r;
            bias1[m][r] = (a.b1 && o < C) ? a.b1[o] : 0.f;
            bias2[m][r] = (a.b2 && o < C) ? a.b2[o] : 0.f;
        }

    // 1. x[clamp(t0 - H + u)] for u in [0, NX) by LDS DMA; the activation
    //    constants.
    stage_x(xb, P, SP, C, T, t0, H, NX, wid, lane);
    if (tid < C) {
        prm[tid] = snake_alpha_rev(a.la1[tid]);
        prm[C + tid] = snake_inv_beta(a.lb1[tid]);
        prm[2 * C + tid] = snake_alpha_rev(a.la2[tid]);
        prm[3 * C + tid] = snake_inv_beta(a.lb2[tid]);
    }
    wait_vmem();
    __syncthreads();

    // 2. act1: P -> Q over [t0 - H + 5, +NA1)
    act_stage<MT == 2>(P, SP, Q, SQ, C, NA1, t0 - H + 5, T, edge, prm, prm + C, taps);
    __syncthreads();

    f32x4 acc[MT][NTW];

    // 3. conv1: Q -> P over [t0 - h2 - 5, +N1) (64 NTW columns), plus bias
    conv_tiles<MT, NTW>(Q, SQ, d, a.wt1, C, K, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < NTW; ++s) {
            const int nt = wid + 4 * s;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = m * 16 + 4 * g4 + r;
                if (o < C) P[o * SP + nt * 16 + l16] = acc[m][s][r] + bias1[m][r];
            }
        }
    __syncthreads();

    // 4. replicate-pad conv1's output outside [0, T) (edge tiles only)
    if (edge) {
        const int og1 = t0 - h2 - 5;
        for (int idx = tid; idx < C * N1; idx += kUT) {
            const int c = idx / N1;
            const int n = idx - c * N1;
            const int g = og1 + n;
            if (g < 0 || g >= T) P[c * SP + n] = P[c * SP + min(max(g, 0), T - 1) - og1];
        }
        __syncthreads();
    }

    // 5. act2: P -> Q over [t0 - h2, +N2)
    act_stage<MT == 2>(P, SP, Q, SQ, C, N2, t0 - h2, T, edge, prm + 2 * C, prm + 3 * C, taps);
    __syncthreads();

    // 6. conv2: Q -> y over [t0, t0 + TT), plus bias, residual x, epilogue
    // out = (conv2 + b2 + x) * out_scale (+ out): fold everything but the
    // sum into res before the matrix loop, x read again (from L2: this
    // block staged it) rather than kept in registers through the
    // activations, the old output read if accumulating.
    float* __restrict__ yb = a.y + row0;
    float res[MT][NTW][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < NTW; ++s) {
            const int nt = wid + 4 * s;
            const int t = t0 + nt * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = m * 16 + 4 * g4 + r;
                const bool in = nt < NT2 && t < T && o < C;
                const size_t idx = (size_t)o * T + t;
                const float xv = in ? xb[idx] : 0.f;
                const float old = (a.accumulate && in) ? yb[idx] : 0.f;
                res[m][s][r] = fmaf(xv + bias2[m][r], a.out_scale, old);
            }
        }
    conv_tiles<MT, NTW>(Q, SQ, 1, a.wt2, C, K, acc);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int s = 0; s < NTW; ++s) {
            const int nt = wid + 4 * s;
            const int t = t0 + nt * 16 + l16;
            if (nt < NT2 && t < T) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int o = m * 16 + 4 * g4 + r;
                    if (o < C)
                        __builtin_nontemporal_store(fmaf(acc[m][s][r], a.out_scale, res[m][s][r]),
                                                    yb + (size_t)o * T + t);
                }
            }
        }
}

// wt[(j*C + i)*CP + o] = w[o][i][j]; zero for o >= C and for padding rows.
__global__ void pack_unit_weights_kernel(const float* __restrict__ w, float* __restrict__ wt,
                                         int C, int K, int CP, int rows) {
    const int n = rows * CP;
    for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += gridDim.x * blockDim.x) {
        const int o = idx % CP;
        const int row = idx / CP;
        float v = 0.f;
        if (o < C && row < K * C) {
            const int j = row / C;
            const int i = row - j * C;
            v = w[((size_t)o * C + i) * K + j];
        }
        wt[idx] = v;
    }
}

// Several weights packed in one launch (blockIdx.y selects the pair).
struct PackList {
    const float* w[2 * 4];
    float* wt[2 * 4];
};
__global__ void pack_unit_weights_multi_kernel(PackList l, int C, int K, int CP, int rows) {
    const float* __restrict__ w = l.w[blockIdx.y];
    float* __restrict__ wt = l.wt[blockIdx.y];
    const int n = rows * CP;
    for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += gridDim.x * blockDim.x) {
        const int o = idx % CP;
        const int row = idx / CP;
        float v = 0.f;
        if (o < C && row < K * C) {
            const int j = row / C;
            const int i = row - j * C;
            v = w[((size_t)o * C + i) * K + j];
        }
        wt[idx] = v;
    }
}

// Rows of the packed weights: K*C, plus one zero step of 4 rows when the
// number of 4-row steps is odd.
int packed_rows(int C, int K) {
    const int steps = K * (C / 4);
    return 4 * (steps + (steps & 1));
}

// Smallest s >= n with s = 16 (mod 32).
int stride16(int n) {
    int s = (n + 15) / 16 * 16;
    if (s % 32 == 0) s += 16;
    return s;
}

struct UnitPlan {
    int MT, NTW, TT, SP, SQ;
    size_t lds;
};

// The largest time tile whose LDS fits unit_blocks_per_cu(C) blocks per CU
// (four for C <= 12, three for C <= 24, else two), with the per-wave tile
// count NTW chosen so that conv1's time tiles fill the four waves exactly,
// unless the grid of B rows of T samples would then be less than one
// resident round of blocks: then the largest tile that still fills one
// round, or the smallest one (short rows, such as a single [1, 32, 4096]
// block).  B = 0: the largest tile (the support check).
bool plan_unit(int C, int K, int d, int B, int T, UnitPlan* p) {
    if (C < 4 || C > 32 || C % 4 != 0 || K < 1 || K % 2 == 0 || d < 1) return false;
    if ((long long)(K - 1) * d > 4096) return false;
    const int MT = (C + 15) / 16;
    const int h1 = (K - 1) * d / 2, h2 = (K - 1) / 2, H = h1 + h2 + 10;
    static const int kNtw1[] = {11, 8, 6, 5, 4, 3, 2};
    static const int kNtw2[] = {6, 5, 4, 3, 2};
    const int* list = MT == 1 ? kNtw1 : kNtw2;
    const int n = MT == 1 ? 7 : 5;
    const long long slots = 256LL * unit_blocks_per_cu(C);
    bool found = false;
    for (int i = 0; i < n; ++i) {
        const int NTW = list[i];
        const int N1r = 64 * NTW;
        const int TT = (N1r - 2 * h2 - 10) / 16 * 16;
        if (TT < 32) continue;
        const int NX = TT + 2 * H;
        const int SP = stride16(std::max(NX + run_max(MT) + 4, N1r));
        const int SQ = stride16(N1r + 2 * h1);
        const size_t lds = ((size_t)C * (SP + SQ) + 4 * (size_t)C) * sizeof(float);
        if (lds > unit_lds_budget(C)) continue;
        *p = UnitPlan{MT, NTW, TT, SP, SQ, lds};
        found = true;
        if (B <= 0 || (long long)B * ((T + TT - 1) / TT) >= slots) return true;
    }
    return found;
}

template <int MT, int NTW>
hipError_t launch_unit_t(const UnitArgs& a, size_t lds, const ActTaps& taps, hipStream_t s) {
    auto kern = amp_unit_kernel<MT, NTW>;
    // Raise the kernel's dynamic-LDS limit to the plan budget once per
    // device (a per-launch attribute call costs tens of microseconds).
    static std::atomic<unsigned long long> raised{0};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const unsigned long long bit = 1ull << (dev & 63);
    if (!(raised.load(std::memory_order_acquire) & bit)) {
        e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kLdsBudget);
        if (e != hipSuccess) return e;
        raised.fetch_or(bit, std::memory_order_acq_rel);
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)a.nblk), dim3(kUT), lds, s, a, taps);
    return hipGetLastError();
}

}  // namespace

bool amp_unit_supported(int C, int K, int dilation) {
    UnitPlan p;
    return plan_unit(C, K, dilation, 0, 0, &p);
}

size_t amp_unit_packed_floats(int C, int K) {
    if (C < 4 || C > 32 || C % 4 != 0 || K < 1) return 0;
    return (size_t)packed_rows(C, K) * (16 * ((C + 15) / 16));
}

hipError_t launch_pack_unit_weights(const float* w, float* wt, int C, int K, hipStream_t s) {
    const int CP = 16 * ((C + 15) / 16);
    const int rows = packed_rows(C, K);
    const int blocks = (rows * CP + 255) / 256;
    hipLaunchKernelGGL(pack_unit_weights_kernel, dim3(blocks < 1 ? 1 : blocks), dim3(256), 0, s,
                       w, wt, C, K, CP, rows);
    return hipGetLastError();
}

hipError_t launch_pack_unit_weights_n(const float* const* w, float* const* wt, int n, int C,
                                      int K, hipStream_t s) {
    if (n < 1 || n > 8) return hipErrorInvalidValue;
    PackList l{};
    for (int i = 0; i < n; ++i) {
        l.w[i] = w[i];
        l.wt[i] = wt[i];
    }
    const int CP = 16 * ((C + 15) / 16);
    const int rows = packed_rows(C, K);
    const int blocks = (rows * CP + 255) / 256;
    hipLaunchKernelGGL(pack_unit_weights_multi_kernel, dim3(blocks < 1 ? 1 : blocks, n), dim3(256),
                       0, s, l, C, K, CP, rows);
    return hipGetLastError();
}

hipError_t launch_amp_unit(const float* x, float* y, const float* wt1, const float* b1,
                           const float* wt2, const float* b2, const float* la1, const float* lb1,
                           const float* la2, const float* lb2, int B, int C, int T, int K,
                           int dilation, float out_scale, int accumulate, const ActTaps& taps,
                           hipStream_t stream) {
    UnitPlan p;
    if (!plan_unit(C, K, dilation, B, T, &p)) return hipErrorInvalidValue;
    const int tiles = (T + p.TT - 1) / p.TT;
    const long long nblk = (long long)B * tiles;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidValue;
    UnitArgs a{x,   y,   wt1, b1,      wt2,      b2,        la1,       lb1,        la2,
               lb2, C,   T,   K,       dilation, p.TT,      tiles,     (int)nblk,  p.SP,
               p.SQ, out_scale, accumulate};
    prof_pre(stream);
    hipError_t e = hipErrorInvalidValue;
    const char* name = "";
    if (p.MT == 1) {
        switch (p.NTW) {
            case 11: e = launch_unit_t<1, 11>(a, p.lds, taps, stream); name = "amp_unit_kernel<1,11>"; break;
            case 8: e = launch_unit_t<1, 8>(a, p.lds, taps, stream); name = "amp_unit_kernel<1,8>"; break;
            case 6: e = launch_unit_t<1, 6>(a, p.lds, taps, stream); name = "amp_unit_kernel<1,6>"; break;
            case 5: e = launch_unit_t<1, 5>(a, p.lds, taps, stream); name = "amp_unit_kernel<1,5>"; break;
            case 4: e = launch_unit_t<1, 4>(a, p.lds, taps, stream); name = "amp_unit_kernel<1,4>"; break;
            case 3: e = launch_unit_t<1, 3>(a, p.lds, taps, stream); name = "amp_unit_kernel<1,3>"; break;
            case 2: e = launch_unit_t<1, 2>(a, p.lds, taps, stream); name = "amp_unit_kernel<1,2>"; break;
        }
    } else {
        switch (p.NTW) {
            case 6: e = launch_unit_t<2, 6>(a, p.lds, taps, stream); name = "amp_unit_kernel<2,6>"; break;
            case 5: e = launch_unit_t<2, 5>(a, p.lds, taps, stream); name = "amp_unit_kernel<2,5>"; break;
            case 4: e = launch_unit_t<2, 4>(a, p.lds, taps, stream); name = "amp_unit_kernel<2,4>"; break;
            case 3: e = launch_unit_t<2, 3>(a, p.lds, taps, stream); name = "amp_unit_kernel<2,3>"; break;
            case 2: e = launch_unit_t<2, 2>(a, p.lds, taps, stream); name = "amp_unit_kernel<2,2>"; break;
        }
    }
    // algorithmic: two C x C x K convolutions and two activations per sample;
    // one read of x and one write of y (plus the read of y when accumulating)
    const double n = (double)B * C * T;
    prof_post(stream, name, 4.0 * C * K * n + 2.0 * 52.0 * n, (accumulate ? 12.0 : 8.0) * n);
    return e;
}

}  // namespace avae
