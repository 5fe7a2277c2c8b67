// Plain Snake ([H3] = docs.rs page of cortiq_engine/audiovae.rs, item
// Snake, used by the Music-3 DAV decoder): per channel c,
//   y = x + sin^2(alpha_c x) / (alpha_c + 1e-9), alpha as stored.
// Pointwise and HBM-bound: 8 bytes per element.  A block walks float4s of
// one [B*C] row range; rows whose length is a multiple of 4 with 16-byte
// aligned bases use float4 loads and stores, others scalar ones.
#include "act_math.h"
#include "avae_internal.h"

namespace avae {
namespace {

constexpr int kSnakeThreads = 256;

__global__ __launch_bounds__(kSnakeThreads) void snake_kernel(const float* __restrict__ x,
                                                              float* __restrict__ y, int C, int T,
                                                              long long rows, int vec,
                                                              const float* __restrict__ alpha) {
    // one block per (row, 4096-element chunk)
    const int chunks = (T + 4095) / 4096;
    const long long row = blockIdx.x / chunks;
    const int t0 = (int)(blockIdx.x - row * chunks) * 4096;
    if (row >= rows) return;
    const float a = alpha[row % C];
    const float* xr = x + row * (long long)T;
    float* yr = y + row * (long long)T;
    const int t1 = min(t0 + 4096, T);
    if (vec) {
        for (int t = t0 + 4 * threadIdx.x; t < t1; t += 4 * kSnakeThreads) {
            const float4 v = *reinterpret_cast<const float4*>(xr + t);
            *reinterpret_cast<float4*>(yr + t) = make_float4(
                snake_plain(v.x, a), snake_plain(v.y, a), snake_plain(v.z, a), snake_plain(v.w, a));
        }
    } else {
        for (int t = t0 + threadIdx.x; t < t1; t += kSnakeThreads)
            __builtin_nontemporal_store(snake_plain(xr[t], a), yr + t);
    }
}

}  // namespace

hipError_t launch_snake(const float* x, float* y, int B, int C, int T, const float* alpha,
                        hipStream_t stream) {
    const long long rows = (long long)B * C;
    const long long blocks = rows * ((T + 4095) / 4096);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const int vec = (T % 4 == 0) && ((((uintptr_t)x) | ((uintptr_t)y)) & 15) == 0;
    prof_pre(stream);
    hipLaunchKernelGGL(snake_kernel, dim3((unsigned)blocks), dim3(kSnakeThreads), 0, stream, x, y,
                       C, T, rows, vec, alpha);
    const hipError_t e = hipGetLastError();
    const double n = (double)rows * T;
    prof_post(stream, "snake_kernel", 6.0 * n, 8.0 * n);
    return e;
}

}  // namespace avae
