// Measurement aids, not part of the decode path: a matrix-core throughput
// probe for the convolution kernels' roofline and a streaming copy that
// gives the HBM rate a plain read-and-write kernel reaches.
//
// Matrix-core probe:  Every wave runs N
// independent v_mfma_f32_16x16x4_f32 accumulator chains (the instruction
// the convolutions use) with no memory traffic inside the loop, so the
// achieved rate is what the matrix cores deliver for that many independent
// chains per wave at the occupancy the grid gives.
#include "avae_internal.h"

namespace avae {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int N>
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* __restrict__ sink, int iters) {
    f32x4 acc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // operands that the compiler cannot fold; tiny so the sums stay finite
    const float a = (float)threadIdx.x * 1e-6f, b = (float)blockIdx.x * 1e-6f;
    // two rounds of the N chains per trip: with one, the register allocator
    // rotates an accumulator through copies at the top of the loop, and the
    // copy waits for the previous trip's last MFMA (a stall per trip that
    // costs 8 chains about a fifth of the rate)
    int it = 0;
    for (; it + 1 < iters; it += 2) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < N; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i], 0, 0, 0);
    }
    if (it < iters) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[i], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// Streaming copy y = x of n4 float4: one float4 per thread, no loop, so every
// load of a wave is in flight at once and the grid streams HBM both ways;
// non-temporal stores (measured on MI355X, 512 MiB of random data: 7.4 TB/s
// against 6.0 with ordinary stores; two or four float4 per thread and
// non-temporal loads were slower).
__global__ __launch_bounds__(256) void stream_copy_kernel(const float4* __restrict__ x,
                                                          float4* __restrict__ y, long long n4) {
    typedef float nt4 __attribute__((ext_vector_type(4)));
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n4) {
        const float4 v = x[i];
        const nt4 w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<nt4*>(y) + i);
    }
}

}  // namespace

hipError_t launch_stream_copy(const float* x, float* y, long long n4, hipStream_t s) {
    const long long blocks = (n4 + 255) / 256;
    if (blocks < 1 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    prof_pre(s);
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(x), reinterpret_cast<float4*>(y), n4);
    const hipError_t e = hipGetLastError();
    prof_post(s, "stream_copy_kernel", 0.0, 32.0 * (double)n4);
    return e;
}

hipError_t launch_mfma_probe(int chains, int blocks, int iters, float* sink, hipStream_t s) {
    prof_pre(s);
    if (chains == 16)
        hipLaunchKernelGGL(mfma_probe_kernel<16>, dim3(blocks), dim3(256), 0, s, sink, iters);
    else
        hipLaunchKernelGGL(mfma_probe_kernel<8>, dim3(blocks), dim3(256), 0, s, sink, iters);
    const hipError_t e = hipGetLastError();
    prof_post(s, chains == 16 ? "mfma_probe_kernel<16>" : "mfma_probe_kernel<8>",
              (double)blocks * 4 * iters * chains * 2048.0, 4.0 * blocks * 256);
    return e;
}

}  // namespace avae
