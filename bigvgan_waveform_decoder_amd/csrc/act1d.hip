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
// One block owns one (b, c) row segment of kTile = 2048 outputs: it stages
// the input window in LDS, computes each doubled-rate sample and its
// SnakeBeta exactly once into two LDS phase arrays (even and odd positions),
// then runs the stride-2 FIR from LDS and writes the outputs once.  HBM
// traffic is one read and one write of the row (8 bytes per element).
//
// SnakeBeta's sine: sin(alpha v) = sin(2 pi r) with r = v * (alpha / 2 pi),
// evaluated by v_sin_f32 in revolutions, which reduces the argument itself:
// within ~1.3e-7 of sin(2 pi frac(r)) (measured on MI355X up to |r| = 1e5);
// the only other error is the float32 rounding of r itself, relative ~1e-7
// of the phase, the same order as rounding alpha*v before any float32 sine.
#include "act_math.h"
#include "avae_internal.h"

namespace avae {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 8 * kThreads;        // outputs per block
constexpr int kX = kTile + 16;             // staged input: x[t0-8 .. t0+kTile+8)
constexpr int kQ = kTile + 16;             // phase arrays: index j <-> q = t0 - 8 + j

// Source of the unconditional prefetch when the next tile is not interior
// (its loads must stay in bounds; the values are never used).
__device__ __align__(16) float g_zero_window[kX];


// The doubled-rate pair (2q, 2q+1) from x[q-3 .. q+3], xq pointing at x[q].
__device__ __forceinline__ void up_pair(const float* xq, const ActTaps& taps, float& e, float& o) {
    e = 0.f;
    o = 0.f;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        e = fmaf(taps.up2[2 * k + 1], xq[2 - k], e);
        o = fmaf(taps.up2[2 * k], xq[3 - k], o);
    }
}

// Interior tile: x[t0-8 .. t0+kTile+8) lies inside the row, every output
// exists, the row start is 16-byte aligned (T % 4 == 0).  Each thread owns
// two runs of 4 consecutive outputs, t0 + 4*tid + 1024*r + (0..3), so every
// global and LDS access is a float4 and the 64 lanes of a wave touch 1 KiB
// contiguously (no LDS bank conflicts).  A 12-value register window of x
// feeds a run's 4 polyphase pairs; two 12-value windows of the phase
// arrays feed its 4 stride-2 FIR outputs.
// Three 16-byte LDS reads of a 12-float window (16-byte aligned, in LDS).
// Written as one asm block because the compiler narrows float4 LDS loads to
// the elements it sees used, and the narrowed pieces (a 16-byte lane
// stride) conflict 4 ways in the LDS banks; full ds_read_b128 do not
// (measured: +10% Activation1d throughput).  The block waits for its own
// reads before it ends, so no output register is written after it, and its
// outputs are early-clobber: a read's destination must not overlap the
// address register, which a later read of the block may issue from after
// the earlier one's data has landed.
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load12(const float* p, float* w) {
    const unsigned addr = (unsigned)(uintptr_t)p;  // LDS byte offset of p
    f32x4v a, b, c;
    asm volatile(
        "ds_read_b128 %0, %3\n"
        "ds_read_b128 %1, %3 offset:16\n"
        "ds_read_b128 %2, %3 offset:32\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(b), "=&v"(c)
        : "v"(addr)
        : "memory");
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    w[8] = c.x; w[9] = c.y; w[10] = c.z; w[11] = c.w;
}

// The interior tile's input window x[t0-8 .. t0+kTile+8) (16-byte aligned)
// is two float4 per thread plus four for the tail, held in registers
// between the load and the LDS store so that its latency overlaps the
// previous tile's compute.  (Plain register variables: passed as a struct
// by reference, the window was kept in scratch memory and every prefetch
// waited for its load.)
// w points at the tile's first input (x + t0); the window starts 8 before.
__device__ __forceinline__ void act1d_window_load(const float* __restrict__ w, float4& a,
                                                  float4& b, float4& c) {
    const int tid = threadIdx.x;
    const float4* src = reinterpret_cast<const float4*>(w - 8);
    a = src[tid];
    b = src[tid + kThreads];
    // every lane loads (lanes >= 4 re-read one of the four tail float4 and
    // drop it): a load under a lane mask cannot be counted by the compiler,
    // which then waits for all memory operations, later stores included
    c = src[2 * kThreads + (tid & 3)];
}

__device__ __forceinline__ void act1d_interior_stage(float4 a, float4 b, float4 c, float* xs) {
    const int tid = threadIdx.x;
    float4* dst = reinterpret_cast<float4*>(xs);
    dst[tid] = a;
    dst[tid + kThreads] = b;
    if (tid < 4) dst[tid + 2 * kThreads] = c;
}

// Tile compute (input already staged in xs, replicate-padded on edge tiles)
// for rows with T % 4 == 0 and 16-byte aligned starts.  Each thread owns two
// runs of 4 consecutive outputs, t0 + 4*tid + 1024*r + (0..3), so every
// global and LDS access is a float4 and the 64 lanes of a wave touch 1 KiB
// contiguously.  A 12-value register window of x feeds a run's 4 polyphase
// pairs; two 12-value windows of the phase arrays feed its 4 stride-2 FIR
// outputs.  Edge tiles (the first and last of a row) take the same path:
// the doubled-rate samples before position 0 become s[0] and those past
// 2T-1 become s[2T-1] (the halo pairs directly, the ones past the row end
// in a fix-up pass), and only outputs t < T are stored (whole float4
// groups, T % 4 == 0).
// The thread's two output groups come back in out[0..1] (t0 + 4 tid and
// t0 + 4 tid + kTile/2); the caller stores them.
__device__ __forceinline__ void act1d_vec_compute(int T, int t0, bool edge, float alpha_rev,
                                                  float inv_beta, const ActTaps& taps,
                                                  const float* xs, float* se, float* so,
                                                  float4 (&res)[2]) {
    constexpr int kHalf = kTile / 2;
    const int tid = threadIdx.x;
    // Phase 1: q = t0 + 4 tid + kHalf r + k  <->  j = 8 + 4 tid + kHalf r + k.
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int j0 = 8 + 4 * tid + kHalf * r;
        float xw[12];  // xw[u] = xs[j0 - 4 + u] = x[q0 - 4 + u]
        load12(xs + j0 - 4, xw);
        float ev[4], ov[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float e, o;
            up_pair(xw + k + 4, taps, e, o);
            ev[k] = snake_beta(e, alpha_rev, inv_beta);
            ov[k] = snake_beta(o, alpha_rev, inv_beta);
        }
        *reinterpret_cast<float4*>(se + j0) = make_float4(ev[0], ev[1], ev[2], ev[3]);
        *reinterpret_cast<float4*>(so + j0) = make_float4(ov[0], ov[1], ov[2], ov[3]);
    }
    // halo: q = t0-3 .. t0-1 (j = 5, 6, 7) and q = t0+kTile .. +2 (j = kTile+8 .. +10);
    // outside the row, the pair at the clamped position with both phases
    // set to s[0] (q < 0) or s[2T-1] (q > T-1)
    if (tid < 6) {
        const int j = tid < 3 ? 5 + tid : kTile + 5 + tid;
        const int q = t0 - 8 + j;
        const int qc = min(max(q, 0), T - 1);
        float e, o;
        up_pair(xs + (qc - (t0 - 8)), taps, e, o);
        if (q < 0) o = e;
        if (q > T - 1) e = o;
        se[j] = snake_beta(e, alpha_rev, inv_beta);
        so[j] = snake_beta(o, alpha_rev, inv_beta);
    }
    __syncthreads();
    if (edge && t0 + kTile > T) {
        // pairs at q = T .. t0+kTile-1 take s[2T-1] = so at q = T-1
        const int jT = T - 1 - (t0 - 8);
        const float sl = so[jT];
        for (int j = jT + 1 + tid; j < kTile + 8; j += kThreads) {
            se[j] = sl;
            so[j] = sl;
        }
        __syncthreads();
    }

    // Phase 2: y[t] = sum_m down[2m] so[t+m-3] + down[2m+1] se[t+m-2] for
    // t = t0 + 4 tid + kHalf r + k; so index = j0 + k + m - 3, se index + 1.
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int j0 = 8 + 4 * tid + kHalf * r;
        float sw[12], ew[12];  // sw[u] = so[j0 - 4 + u], ew[u] = se[j0 - 4 + u]
        load12(so + j0 - 4, sw);
        load12(se + j0 - 4, ew);
        float out[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 6; ++m) {
                acc = fmaf(taps.down[2 * m], sw[k + m + 1], acc);
                acc = fmaf(taps.down[2 * m + 1], ew[k + m + 2], acc);
            }
            out[k] = acc;
        }
        res[r] = make_float4(out[0], out[1], out[2], out[3]);
    }
}

// Edge tile staging for the vector path: x[clamp(t0 - 8 + i)], i < kX, into
// xs (the replicate padding), all of a thread's loads before its first LDS
// write.
__device__ __forceinline__ void act1d_stage_clamped(const float* __restrict__ xrow, int T,
                                                    int t0, float* xs) {
    constexpr int kLoads = (kX + kThreads - 1) / kThreads;
    float xv[kLoads];
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
        const int i = threadIdx.x + r * kThreads;
        xv[r] = (i < kX) ? xrow[min(max(t0 - 8 + i, 0), T - 1)] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
        const int i = threadIdx.x + r * kThreads;
        if (i < kX) xs[i] = xv[r];
    }
}

// Scalar tile (rows with T % 4 != 0 or unaligned tensors): same arrays and
// index conventions, scalar and strided over the block, every index clamped
// to implement the replicate padding.
__device__ __forceinline__ void act1d_tile_edge(const float* __restrict__ xrow,
                                                float* __restrict__ yrow, int T, int t0,
                                                float alpha_rev, float inv_beta,
                                                const ActTaps& taps, float* xs, float* se,
                                                float* so) {
    // All of a thread's loads are issued before its first LDS write.
    constexpr int kLoads = (kX + kThreads - 1) / kThreads;
    float xv[kLoads];
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
        const int i = threadIdx.x + r * kThreads;
        xv[r] = (i < kX) ? xrow[min(max(t0 - 8 + i, 0), T - 1)] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
        const int i = threadIdx.x + r * kThreads;
        if (i < kX) xs[i] = xv[r];
    }
    __syncthreads();
    // q = t0 - 8 + j for j in [5, kTile + 11): q in [t0-3, t0+kTile+3)
#pragma unroll 3
    for (int j = 5 + threadIdx.x; j < kTile + 11; j += kThreads) {
        const int q = t0 - 8 + j;
        const int qc = min(max(q, 0), T - 1);
        float e, o;
        up_pair(xs + (qc - (t0 - 8)), taps, e, o);
        // Positions before 0 replicate s[0] (even phase at q = 0); positions
        // past 2T-1 replicate s[2T-1] (odd phase at q = T-1).
        if (q < 0) o = e;
        if (q > T - 1) e = o;
        se[j] = snake_beta(e, alpha_rev, inv_beta);
        so[j] = snake_beta(o, alpha_rev, inv_beta);
    }
    __syncthreads();
#pragma unroll 4
    for (int i = threadIdx.x; i < kTile; i += kThreads) {
        const int t = t0 + i;
        if (t >= T) break;
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < 6; ++m) {
            acc = fmaf(taps.down[2 * m], so[i + m + 5], acc);
            acc = fmaf(taps.down[2 * m + 1], se[i + m + 6], acc);
        }
        yrow[t] = acc;
    }
}

// A y tile's float4 store, non-temporal (the line is not kept in the caches
// on the way to HBM): a read-once / write-once stream of this size then
// reaches 97% of a plain copy's rate (measured on MI355X, [2, 512, 65536]:
// 102.3 -> 89.8 us; inside the H3-shaped decode, where the next convolution
// reads y, Activation1d 1.58 -> 1.45 ms per decode and the convolutions
// unchanged).  Non-temporal loads of x were slower.
__device__ __forceinline__ void store4_stream(float* p, float4 v) {
    typedef float nt4 __attribute__((ext_vector_type(4)));
    const nt4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<nt4*>(p));
}

// A block walks `per_block` consecutive tiles of the flattened (row, tile)
// order.  The next interior tile's input is loaded into registers right
// after the current tile is staged, so its HBM latency overlaps the current
// tile's compute.
// (six waves per SIMD: at most 80 VGPRs, six blocks' LDS per CU)
__global__ __launch_bounds__(kThreads, 6) void act1d_kernel(
    const float* __restrict__ x, float* __restrict__ y, int C, int T, int tiles, int total,
    int per_block, int vec_ok, const float* __restrict__ log_alpha,
    const float* __restrict__ log_beta, ActTaps taps) {
    __shared__ __align__(16) float xs[kX];
    __shared__ __align__(16) float se[kQ];  // s at even doubled-rate positions 2q
    __shared__ __align__(16) float so[kQ];  // s at odd doubled-rate positions 2q+1

    const int first = blockIdx.x * per_block;
    const int last = min(first + per_block, total);
    auto interior = [&](int t0) { return vec_ok && t0 >= 8 && t0 + kTile + 8 <= T; };

    // The next tile's window is loaded every tile, unconditionally: from the
    // row when the next tile is interior, else from a zero window that is
    // never used.  (A conditional load made the window a two-way merge that
    // the compiler resolved with register copies at the loop latch, each
    // waiting for every outstanding memory operation, the tile's own stores
    // included.)
    auto window = [&](int id) -> const float* {
        if (id < last) {
            const int row = id / tiles;
            const int t0 = (id - row * tiles) * kTile;
            if (interior(t0)) return x + (size_t)row * T + t0;
        }
        return g_zero_window + 8;
    };
    int cur_c = -1;
    float alpha_rev = 0.f, inv_beta = 0.f;
    auto set_channel = [&](int row) {
        const int c = row % C;
        if (c != cur_c) {
            cur_c = c;
            alpha_rev = snake_alpha_rev(log_alpha[c]);
            inv_beta = snake_inv_beta(log_beta[c]);
        }
    };
    // (two loops: with the float4 / scalar choice inside one, the window
    // registers were again a two-way merge)
    if (vec_ok) {
        // A tile's two output groups are stored a tile later, after the
        // next window's loads are issued: loads and stores share one wait
        // counter, and a wait for the window then never waits for stores
        // issued just before it (they have a whole tile's compute to land).
        float4 pa, pb, pc;
        float4 res[2];
        float* dst[2] = {nullptr, nullptr};
        auto store = [&]() {
#pragma unroll
            for (int r = 0; r < 2; ++r)
                if (dst[r]) store4_stream(dst[r], res[r]);
        };
        act1d_window_load(window(first), pa, pb, pc);
        for (int id = first; id < last; ++id) {
            const int row = id / tiles;
            const int t0 = (id - row * tiles) * kTile;
            set_channel(row);
            const size_t base = (size_t)row * (size_t)T;
            if (id > first) __syncthreads();  // previous tile done with xs, se, so
            const bool inner = interior(t0);
            if (inner) {
                act1d_interior_stage(pa, pb, pc, xs);
            } else {
                // the window was loaded (from the zero window) but is not
                // used: consume it here so that no load into these registers
                // is pending on either path when the next window overwrites
                // them (a pending one made the compiler wait for every memory
                // operation there, the stores just issued included)
                asm volatile("" ::"v"(pa.x), "v"(pa.y), "v"(pa.z), "v"(pa.w), "v"(pb.x),
                             "v"(pb.y), "v"(pb.z), "v"(pb.w), "v"(pc.x), "v"(pc.y), "v"(pc.z),
                             "v"(pc.w));
                act1d_stage_clamped(x + base, T, t0, xs);
            }
            act1d_window_load(window(id + 1), pa, pb, pc);
            store();  // the previous tile's outputs, behind the next window's loads
            __syncthreads();
            act1d_vec_compute(T, t0, !inner, alpha_rev, inv_beta, taps, xs, se, so, res);
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int t = t0 + 4 * (int)threadIdx.x + (kTile / 2) * r;
                dst[r] = (inner || t < T) ? y + base + t : nullptr;
            }
        }
        store();
    } else {
        for (int id = first; id < last; ++id) {
            const int row = id / tiles;
            const int t0 = (id - row * tiles) * kTile;
            set_channel(row);
            const size_t base = (size_t)row * (size_t)T;
            if (id > first) __syncthreads();
            act1d_tile_edge(x + base, y + base, T, t0, alpha_rev, inv_beta, taps, xs, se, so);
        }
    }
}

}  // namespace

hipError_t launch_act1d(const float* x, float* y, int B, int C, int T,
                        const float* log_alpha, const float* log_beta,
                        const ActTaps& taps, hipStream_t stream) {
    const int tiles = (T + kTile - 1) / kTile;
    const long long total = (long long)B * C * tiles;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    // Up to 4 tiles per block while the grid still gives ~6 blocks per CU
    // (256 CUs); short workloads keep one tile per block.
    int per_block = (int)(total / (256 * 6));
    per_block = per_block < 1 ? 1 : (per_block > 4 ? 4 : per_block);
    const long long blocks = (total + per_block - 1) / per_block;
    prof_pre(stream);
    // float4 rows need T % 4 == 0 and 16-byte aligned tensors
    const int vec_ok = (T % 4 == 0) && (((uintptr_t)x | (uintptr_t)y) & 15) == 0;
    hipLaunchKernelGGL(act1d_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, x, y, C,
                       T, tiles, (int)total, per_block, vec_ok, log_alpha, log_beta, taps);
    const hipError_t e = hipGetLastError();
    // algorithmic: 24 FMA + 2 SnakeBeta (mul, fma) per output; one read, one write
    const double n = (double)B * C * T;
    prof_post(stream, "act1d_kernel", 52.0 * n, 8.0 * n);
    return e;
}

}  // namespace avae
