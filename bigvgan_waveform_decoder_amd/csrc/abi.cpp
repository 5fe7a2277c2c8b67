// C-ABI of libavae.so: argument checking, error reporting, the AMP block
// sequence and the decoder plan.  Every check runs before the first launch;
// the compute calls never allocate or synchronise.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "avae.h"
#include "avae_internal.h"
#include "plan.h"

using avae::ActTaps;
using avae::ConvEpilogue;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(AVAE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define AVAE_TRY(expr, what)                                   \
    do {                                                       \
        hipError_t e_ = (expr);                                \
        if (e_ != hipSuccess) return hip_fail(e_, what);       \
    } while (0)

// The designed taps avae_kaiser_sinc(0.25, 0.3, 12), computed once.
const float* designed_taps() {
    static float taps[avae::kFilterLen];
    static std::once_flag once;
    std::call_once(once, [] {
        double d[avae::kFilterLen];
        avae::design_kaiser_sinc(0.25, 0.3, avae::kFilterLen, d);
        for (int i = 0; i < avae::kFilterLen; ++i) taps[i] = (float)d[i];
    });
    return taps;
}

ActTaps make_taps(const float* up, const float* down) {
    ActTaps t;
    const float* u = up ? up : designed_taps();
    const float* d = down ? down : designed_taps();
    for (int i = 0; i < avae::kFilterLen; ++i) {
        t.up2[i] = 2.0f * u[i];
        t.down[i] = d[i];
    }
    return t;
}

using avae::plan::round_up;

int conv_out_len(int T, int K, int dil, int pad) { return T + 2 * pad - dil * (K - 1); }

// One AMP block into y (y = scale*AMP(x) [+ y]); cur, t1, t2 are [B,C,T]
// scratch buffers.  Activations use `taps`.
// True if every dilation step of an AMP block of width C and K taps runs as
// one fused launch (amp_unit.hip).  The kernel takes C <= 32; it is used up
// to C = 24, the widths where it measured faster than the four separate
// launches on the decoders' long rows (at 32 channels the separate launches
// are a few percent faster there), and at 32 channels for short inputs
// (B T <= kFuseSmallBT samples per channel: one launch per step instead of
// four, each of which fills only part of the GPU).
constexpr int kFuseMaxC = 24;
constexpr long long kFuseSmallBT = 65536;
bool fuse_width(int B, int C, int T) {
    return C <= kFuseMaxC || (C <= 32 && (long long)B * T <= kFuseSmallBT);
}
bool amp_fusable(int C, int K, int n_dil, const int* dil) {
    if (C > 32) return false;
    for (int q = 0; q < n_dil; ++q)
        if (!avae::amp_unit_supported(C, K, dil[q])) return false;
    return true;
}

// One AMP block ([H3] AmpBlock::apply): for each dilation step q,
// cur <- cur + conv2_q(act(conv1_q(act(cur)))); the last step's result goes
// through the MRF epilogue (y = cur * out_scale, + y if accumulate).
// pw1/pw2 (packed weights, or null) select the fused one-launch-per-step
// path; otherwise each step is act1d, conv1d, act1d, conv1d launches.
// fw1/fw2 (per dilation step; null, or null entries, for the direct
// kernels) are frequency-domain weights from launch_fft_pack: where
// plan::fft_amp_use takes the shape, that
// activation + convolution then runs as launch_conv1d_fft with the
// activation inside its forward transforms, the spectra in t1 and t2 (slots
// of at least plan::fft_spectrum_bytes each).  fpack (or null): room for one
// convolution's frequency-domain weights, packed from w1/w2 just before use
// where fw1/fw2 give none.
int run_amp(const float* x, float* y, int B, int C, int T, int K, int n_dil, const int* dil,
            const float* const* w1, const float* const* b1, const float* const* w2,
            const float* const* b2, const float* const* la, const float* const* lb,
            const float* const* pw1, const float* const* pw2, const float* const* fw1,
            const float* const* fw2, float out_scale, int accumulate, float* cur, float* t1,
            float* t2, const ActTaps& taps, hipStream_t s, float* fpack = nullptr,
            int q_begin = 0, int q_end = -1) {
    // dilation steps [q_begin, q_end) (all by default): a caller interleaving
    // several blocks on their own streams runs them one step at a time
    const int qe = q_end < 0 ? n_dil : std::min(q_end, n_dil);
    if (pw1 && pw2) {
        float* bufs[2] = {t1, t2};
        for (int q = q_begin; q < qe; ++q) {
            const float* src = (q == 0) ? x : bufs[(q - 1) & 1];
            const bool last = (q == n_dil - 1);
            float* dst = last ? y : bufs[q & 1];
            AVAE_TRY(avae::launch_amp_unit(src, dst, pw1[q], b1[q], pw2[q], b2[q], la[2 * q],
                                           lb[2 * q], la[2 * q + 1], lb[2 * q + 1], B, C, T, K,
                                           dil[q], last ? out_scale : 1.0f, last ? accumulate : 0,
                                           taps, s),
                     "fused AMP unit");
        }
        return AVAE_OK;
    }
    for (int q = q_begin; q < qe; ++q) {
        const float* src = (q == 0) ? x : cur;
        const int d = dil[q];
        ConvEpilogue e1{b1[q], nullptr, 1.0f, 0};
        // h = conv1(act(src)) lands in t2 either way
        const bool f1 = ((fw1 && fw1[q]) || fpack) && avae::plan::fft_amp_use(B, C, T, K, d);
        const bool f2 = ((fw2 && fw2[q]) || fpack) && avae::plan::fft_amp_use(B, C, T, K, 1);
        if (f1) {
            const float* wp = (fw1 && fw1[q]) ? fw1[q] : fpack;
            if (wp == fpack)  // this call's weights, packed just before use
                AVAE_TRY(avae::launch_fft_pack(w1[q], fpack, C, C, K, d, s), "fft weight packing");
            // act(src) inside the transforms: spectrum in t1, product in t2,
            // output in t1
            AVAE_TRY(avae::launch_conv1d_fft(src, t1, wp, B, C, C, T, K, d, e1, t1, t2, s,
                                             la[2 * q], lb[2 * q], &taps),
                     "act + conv1d_fft (convs1)");
        } else {
            AVAE_TRY(avae::launch_act1d(src, t1, B, C, T, la[2 * q], lb[2 * q], taps, s),
                     "act1d");
            AVAE_TRY(avae::launch_conv1d(t1, t2, w1[q], B, C, C, T, T, K, d, (K * d - d) / 2, e1,
                                         s),
                     "conv1d (convs1)");
        }
        float* h = f1 ? t1 : t2;   // conv1's output
        float* fr = f1 ? t2 : t1;  // the other scratch slot
        const bool last = (q == n_dil - 1);
        ConvEpilogue e2{b2[q], src, last ? out_scale : 1.0f, last ? accumulate : 0};
        float* dst = last ? y : cur;
        if (f2) {
            const float* wp = (fw2 && fw2[q]) ? fw2[q] : fpack;
            if (wp == fpack)
                AVAE_TRY(avae::launch_fft_pack(w2[q], fpack, C, C, K, 1, s), "fft weight packing");
            // act(h) inside the transforms: spectrum in fr, product in h,
            // then dst (+ residual src)
            AVAE_TRY(avae::launch_conv1d_fft(h, dst, wp, B, C, C, T, K, 1, e2, fr, h, s,
                                             la[2 * q + 1], lb[2 * q + 1], &taps),
                     "act + conv1d_fft (convs2)");
        } else {
            AVAE_TRY(avae::launch_act1d(h, fr, B, C, T, la[2 * q + 1], lb[2 * q + 1], taps, s),
                     "act1d");
            AVAE_TRY(avae::launch_conv1d(fr, dst, w2[q], B, C, C, T, T, K, 1, (K - 1) / 2, e2, s),
                     "conv1d (convs2)");
        }
    }
    return AVAE_OK;
}

}  // namespace

// =========================================================================
// Small entry points
// =========================================================================

extern "C" const char* avae_last_error(void) { return g_err.c_str(); }

extern "C" int avae_version(void) { return 100; }

extern "C" int avae_kaiser_sinc(double cutoff, double half_width, int taps, float* out_host) {
    if (!out_host) return fail(AVAE_EINVAL, "avae_kaiser_sinc: out_host is null");
    if (taps < 2 || taps % 2 != 0 || taps > 1024)
        return fail(AVAE_EINVAL, "avae_kaiser_sinc: taps must be even in [2, 1024], got %d", taps);
    if (!(cutoff > 0.0 && cutoff <= 0.5) || !(half_width > 0.0 && half_width <= 0.5))
        return fail(AVAE_EINVAL, "avae_kaiser_sinc: cutoff and half_width must be in (0, 0.5]");
    std::vector<double> d(taps);
    avae::design_kaiser_sinc(cutoff, half_width, taps, d.data());
    for (int i = 0; i < taps; ++i) out_host[i] = (float)d[i];
    return AVAE_OK;
}

extern "C" int avae_act1d(const float* x, float* y, int B, int C, int T, const float* log_alpha,
                          const float* log_beta, const float* up_taps, const float* down_taps,
                          void* stream) {
    if (!x || !y || !log_alpha || !log_beta)
        return fail(AVAE_EINVAL, "avae_act1d: null tensor pointer");
    if (B < 1 || C < 1 || T < 1)
        return fail(AVAE_EINVAL, "avae_act1d: B, C, T must be >= 1 (got %d, %d, %d)", B, C, T);
    if (x == y) return fail(AVAE_EINVAL, "avae_act1d: x and y must not overlap");
    const ActTaps taps = make_taps(up_taps, down_taps);
    avae::prof_set_phase(avae::kPhaseNone);
    AVAE_TRY(avae::launch_act1d(x, y, B, C, T, log_alpha, log_beta, taps, (hipStream_t)stream),
             "avae_act1d launch");
    return AVAE_OK;
}

extern "C" int avae_conv1d(const float* x, float* y, int B, int Cin, int Cout, int T,
                           const float* w, const float* bias, int K, int dilation, int pad,
                           const float* residual, void* stream) {
    if (!x || !y || !w) return fail(AVAE_EINVAL, "avae_conv1d: null tensor pointer");
    if (B < 1 || Cin < 1 || Cout < 1 || T < 1 || K < 1 || dilation < 1 || pad < 0)
        return fail(AVAE_EINVAL, "avae_conv1d: bad size (B=%d Cin=%d Cout=%d T=%d K=%d d=%d pad=%d)",
                    B, Cin, Cout, T, K, dilation, pad);
    if (K > AVAE_MAX_TAPS) return fail(AVAE_ESHAPE, "avae_conv1d: K=%d > %d", K, AVAE_MAX_TAPS);
    if ((long long)(K - 1) * dilation > 4096)
        return fail(AVAE_ESHAPE, "avae_conv1d: receptive field (K-1)*d too large");
    const int Tout = conv_out_len(T, K, dilation, pad);
    if (Tout < 1) return fail(AVAE_ESHAPE, "avae_conv1d: output length %d < 1", Tout);
    if (x == y) return fail(AVAE_EINVAL, "avae_conv1d: x and y must not overlap");
    ConvEpilogue ep{bias, residual, 1.0f, 0};
    avae::prof_set_phase(avae::kPhaseNone);
    hipError_t e = avae::launch_conv1d(x, y, w, B, Cin, Cout, T, Tout, K, dilation, pad, ep,
                                       (hipStream_t)stream);
    if (e == hipErrorInvalidValue)
        return fail(AVAE_ESHAPE, "avae_conv1d: shape exceeds the kernel's LDS or grid limits");
    if (e != hipSuccess) return hip_fail(e, "avae_conv1d launch");
    return AVAE_OK;
}

extern "C" size_t avae_conv1d_fft_weight_floats(int Cin, int Cout) {
    if (Cin < 1 || Cout < 1) return 0;
    return avae::fft_conv_weight_floats(Cin, Cout);
}

extern "C" int avae_conv1d_fft_pack(const float* w, float* wp, int Cin, int Cout, int K,
                                    int dilation, void* stream) {
    if (!w || !wp) return fail(AVAE_EINVAL, "avae_conv1d_fft_pack: null pointer");
    if (Cin < 1 || Cout < 1 || K < 1 || dilation < 1)
        return fail(AVAE_EINVAL, "avae_conv1d_fft_pack: bad size (Cin=%d Cout=%d K=%d d=%d)", Cin,
                    Cout, K, dilation);
    if (!avae::plan::fft_supported(Cin, Cout, K, dilation))
        return fail(AVAE_ESHAPE,
                    "avae_conv1d_fft_pack: needs Cin and Cout multiples of 16, odd K, "
                    "(K-1)*d <= 128 (Cin=%d Cout=%d K=%d d=%d)",
                    Cin, Cout, K, dilation);
    AVAE_TRY(avae::launch_fft_pack(w, wp, Cin, Cout, K, dilation, (hipStream_t)stream),
             "avae_conv1d_fft_pack launch");
    return AVAE_OK;
}

extern "C" size_t avae_conv1d_fft_workspace_bytes(int B, int Cin, int Cout, int T, int K,
                                                  int dilation) {
    if (B < 1 || T < 1 || !avae::plan::fft_supported(Cin, Cout, K, dilation)) return 0;
    const size_t a = avae::plan::fft_spectrum_bytes(B, Cin, T, K, dilation);
    const size_t b = avae::plan::fft_spectrum_bytes(B, Cout, T, K, dilation);
    return (a == 0 || b == 0) ? 0 : a + b;
}

extern "C" int avae_conv1d_fft(const float* x, float* y, int B, int Cin, int Cout, int T,
                               const float* wp, const float* bias, int K, int dilation,
                               const float* residual, void* workspace, size_t ws_bytes,
                               void* stream) {
    if (!x || !y || !wp) return fail(AVAE_EINVAL, "avae_conv1d_fft: null tensor pointer");
    if (B < 1 || Cin < 1 || Cout < 1 || T < 1 || K < 1 || dilation < 1)
        return fail(AVAE_EINVAL, "avae_conv1d_fft: bad size (B=%d Cin=%d Cout=%d T=%d K=%d d=%d)",
                    B, Cin, Cout, T, K, dilation);
    if (x == y) return fail(AVAE_EINVAL, "avae_conv1d_fft: x and y must not overlap");
    if (!avae::plan::fft_supported(Cin, Cout, K, dilation))
        return fail(AVAE_ESHAPE,
                    "avae_conv1d_fft: needs Cin and Cout multiples of 16, odd K, "
                    "(K-1)*d <= 128 (Cin=%d Cout=%d K=%d d=%d)",
                    Cin, Cout, K, dilation);
    const size_t need = avae_conv1d_fft_workspace_bytes(B, Cin, Cout, T, K, dilation);
    if (!workspace || ws_bytes < need)
        return fail(AVAE_EWORKSPACE, "avae_conv1d_fft: workspace %zu bytes < %zu needed", ws_bytes,
                    need);
    float* xs = (float*)workspace;
    float* ys = (float*)((char*)workspace + avae::plan::fft_spectrum_bytes(B, Cin, T, K, dilation));
    ConvEpilogue ep{bias, residual, 1.0f, 0, nullptr, nullptr};
    avae::prof_set_phase(avae::kPhaseNone);
    AVAE_TRY(avae::launch_conv1d_fft(x, y, wp, B, Cin, Cout, T, K, dilation, ep, xs, ys,
                                     (hipStream_t)stream),
             "avae_conv1d_fft launch");
    return AVAE_OK;
}

extern "C" int avae_act_conv1d_fft(const float* x, float* y, int B, int Cin, int Cout, int T,
                                   const float* log_alpha, const float* log_beta,
                                   const float* wp, const float* bias, int K, int dilation,
                                   const float* residual, void* workspace, size_t ws_bytes,
                                   void* stream) {
    if (!x || !y || !wp || !log_alpha || !log_beta)
        return fail(AVAE_EINVAL, "avae_act_conv1d_fft: null tensor pointer");
    if (B < 1 || Cin < 1 || Cout < 1 || T < 1 || K < 1 || dilation < 1)
        return fail(AVAE_EINVAL,
                    "avae_act_conv1d_fft: bad size (B=%d Cin=%d Cout=%d T=%d K=%d d=%d)", B, Cin,
                    Cout, T, K, dilation);
    if (x == y) return fail(AVAE_EINVAL, "avae_act_conv1d_fft: x and y must not overlap");
    if (!avae::plan::fft_supported(Cin, Cout, K, dilation))
        return fail(AVAE_ESHAPE,
                    "avae_act_conv1d_fft: needs Cin and Cout multiples of 16, odd K, "
                    "(K-1)*d <= 128 (Cin=%d Cout=%d K=%d d=%d)",
                    Cin, Cout, K, dilation);
    const size_t need = avae_conv1d_fft_workspace_bytes(B, Cin, Cout, T, K, dilation);
    if (!workspace || ws_bytes < need)
        return fail(AVAE_EWORKSPACE, "avae_act_conv1d_fft: workspace %zu bytes < %zu needed",
                    ws_bytes, need);
    float* xs = (float*)workspace;
    float* ys = (float*)((char*)workspace + avae::plan::fft_spectrum_bytes(B, Cin, T, K, dilation));
    ConvEpilogue ep{bias, residual, 1.0f, 0, nullptr, nullptr};
    const ActTaps taps = make_taps(nullptr, nullptr);
    avae::prof_set_phase(avae::kPhaseNone);
    AVAE_TRY(avae::launch_conv1d_fft(x, y, wp, B, Cin, Cout, T, K, dilation, ep, xs, ys,
                                     (hipStream_t)stream, log_alpha, log_beta, &taps),
             "avae_act_conv1d_fft launch");
    return AVAE_OK;
}

extern "C" int avae_convtr1d(const float* x, float* y, int B, int Cin, int Cout, int Tin,
                             const float* w, const float* bias, int K, int stride, int pad,
                             void* stream) {
    if (!x || !y || !w) return fail(AVAE_EINVAL, "avae_convtr1d: null tensor pointer");
    if (B < 1 || Cin < 1 || Cout < 1 || Tin < 1 || K < 1 || stride < 1)
        return fail(AVAE_EINVAL, "avae_convtr1d: bad size (B=%d Cin=%d Cout=%d Tin=%d K=%d s=%d)",
                    B, Cin, Cout, Tin, K, stride);
    if (K > AVAE_MAX_TAPS) return fail(AVAE_ESHAPE, "avae_convtr1d: K=%d > %d", K, AVAE_MAX_TAPS);
    if (pad < 0) {
        if (K < stride) return fail(AVAE_ESHAPE, "avae_convtr1d: default pad needs K >= stride");
        pad = (K - stride) / 2;
    }
    const long long Tout = (long long)(Tin - 1) * stride + K - 2LL * pad;
    if (Tout < 1 || Tout > 0x7fffffffLL)
        return fail(AVAE_ESHAPE, "avae_convtr1d: output length %lld out of range", Tout);
    if (x == y) return fail(AVAE_EINVAL, "avae_convtr1d: x and y must not overlap");
    avae::prof_set_phase(avae::kPhaseNone);
    hipError_t e = avae::launch_convtr1d(x, y, w, bias, B, Cin, Cout, Tin, (int)Tout, K, stride,
                                         pad, (hipStream_t)stream);
    if (e == hipErrorInvalidValue)
        return fail(AVAE_ESHAPE, "avae_convtr1d: shape exceeds the kernel's LDS or grid limits");
    if (e != hipSuccess) return hip_fail(e, "avae_convtr1d launch");
    return AVAE_OK;
}

namespace {
// Packed-weight reserve of the standalone AMP block: room for every
// dilation step's two packed convolutions at the largest K.
size_t amp_pack_reserve(int B, int C, int T) {
    if (!fuse_width(B, C, T)) return 0;
    const size_t per = avae::amp_unit_packed_floats(C, AVAE_MAX_TAPS);
    return per ? 2 * AVAE_MAX_DIL * round_up(per * sizeof(float), 256) : 0;
}
}  // namespace

extern "C" size_t avae_amp_block_workspace_bytes(int B, int C, int T) {
    if (B < 1 || C < 1 || T < 1) return 0;
    const size_t slot = avae::plan::tensor_bytes(B, C, T);
    return slot ? 3 * slot + amp_pack_reserve(B, C, T) : 0;
}

namespace {
// Slot size and packing room of the AMP block's frequency-domain path (0, 0
// when none of its convolutions takes it).
void amp_fft_plan(int B, int C, int T, int K, int n_dil, const int* dil, size_t* slot,
                  size_t* pack) {
    *slot = 0;
    *pack = 0;
    size_t m = avae::plan::tensor_bytes(B, C, T);
    bool any = false;
    for (int q = 0; q <= n_dil; ++q) {
        const int d = q < n_dil ? dil[q] : 1;
        if (d < 1 || !avae::plan::fft_amp_use(B, C, T, K, d)) continue;
        const size_t f = avae::plan::fft_spectrum_bytes(B, C, T, K, d);
        if (f == 0 || m == 0) return;
        m = std::max(m, f);
        any = true;
    }
    if (!any) return;
    *slot = m;
    *pack = round_up(avae::fft_conv_weight_floats(C, C) * sizeof(float), 256);
}
}  // namespace

extern "C" size_t avae_amp_block_fft_workspace_bytes(int B, int C, int T, int K, int n_dil,
                                                    const int* dil) {
    if (B < 1 || C < 1 || T < 1 || !dil || n_dil < 1 || n_dil > AVAE_MAX_DIL) return 0;
    size_t slot, pack;
    amp_fft_plan(B, C, T, K, n_dil, dil, &slot, &pack);
    return slot ? 3 * slot + pack : avae_amp_block_workspace_bytes(B, C, T);
}

namespace {
// Argument checks shared by avae_amp_block and avae_amp_block_static
// (`who` names the entry point in the messages).
int amp_block_check(const char* who, const float* x, const float* y, int B, int C, int T, int K,
                    int n_dil, const int* dil, const float* const* w1, const float* const* w2,
                    const float* const* log_alpha, const float* const* log_beta) {
    if (!x || !y || !dil || !w1 || !w2 || !log_alpha || !log_beta)
        return fail(AVAE_EINVAL, "%s: null pointer", who);
    if (B < 1 || C < 1 || T < 1 || n_dil < 1) return fail(AVAE_EINVAL, "%s: bad size", who);
    if (n_dil > AVAE_MAX_DIL) return fail(AVAE_ESHAPE, "%s: n_dil > %d", who, AVAE_MAX_DIL);
    if (K < 1 || K % 2 == 0 || K > AVAE_MAX_TAPS)
        return fail(AVAE_ESHAPE, "%s: K must be odd and <= %d", who, AVAE_MAX_TAPS);
    if (x == y) return fail(AVAE_EINVAL, "%s: x and y must not overlap", who);
    for (int q = 0; q < n_dil; ++q) {
        if (dil[q] < 1) return fail(AVAE_EINVAL, "%s: dilation < 1", who);
        if ((long long)(K - 1) * dil[q] > 4096)
            return fail(AVAE_ESHAPE, "%s: receptive field too large", who);
        if (!w1[q] || !w2[q]) return fail(AVAE_EINVAL, "%s: null weight", who);
        if (!log_alpha[2 * q] || !log_alpha[2 * q + 1] || !log_beta[2 * q] || !log_beta[2 * q + 1])
            return fail(AVAE_EINVAL, "%s: null activation parameter", who);
    }
    return AVAE_OK;
}

// The AMP block on a checked call and a workspace of at least
// avae_amp_block_workspace_bytes(B, C, T) bytes: three [B, C, T] slots (cur,
// t1, t2), then the fused unit's packed weights.
int amp_block_run(const float* x, float* y, int B, int C, int T, int K, int n_dil,
                  const int* dil, const float* const* w1, const float* const* b1,
                  const float* const* w2, const float* const* b2,
                  const float* const* log_alpha, const float* const* log_beta, float out_scale,
                  int accumulate, void* workspace, hipStream_t s, size_t fft_slot = 0) {
    static const float* const kNull[AVAE_MAX_DIL] = {nullptr, nullptr, nullptr, nullptr};
    if (fft_slot) {
        // the frequency-domain path: three slots of fft_slot bytes, then one
        // convolution's packed weights
        char* ws = (char*)workspace;
        avae::prof_set_phase(avae::kPhaseNone);
        return run_amp(x, y, B, C, T, K, n_dil, dil, w1, b1 ? b1 : kNull, w2, b2 ? b2 : kNull,
                       log_alpha, log_beta, nullptr, nullptr, nullptr, nullptr, out_scale,
                       accumulate, (float*)ws, (float*)(ws + fft_slot),
                       (float*)(ws + 2 * fft_slot), make_taps(nullptr, nullptr), s,
                       (float*)(ws + 3 * fft_slot));
    }
    const size_t slot = avae::plan::tensor_bytes(B, C, T);
    char* ws = (char*)workspace;
    float* cur = (float*)ws;
    float* t1 = (float*)(ws + slot);
    float* t2 = (float*)(ws + 2 * slot);
    avae::prof_set_phase(avae::kPhaseNone);
    const float* pw1[AVAE_MAX_DIL] = {};
    const float* pw2[AVAE_MAX_DIL] = {};
    const bool fused = amp_pack_reserve(B, C, T) > 0 && amp_fusable(C, K, n_dil, dil);
    if (fused) {
        // pack this call's weights into the reserve (amp_unit.hip layout)
        char* pk = ws + 3 * slot;
        const size_t per = round_up(avae::amp_unit_packed_floats(C, K) * sizeof(float), 256);
        const float* src[2 * AVAE_MAX_DIL];
        float* dst[2 * AVAE_MAX_DIL];
        for (int q = 0; q < n_dil; ++q) {
            float* p1 = (float*)(pk + (2 * q) * per);
            float* p2 = (float*)(pk + (2 * q + 1) * per);
            src[2 * q] = w1[q];
            src[2 * q + 1] = w2[q];
            dst[2 * q] = p1;
            dst[2 * q + 1] = p2;
            pw1[q] = p1;
            pw2[q] = p2;
        }
        AVAE_TRY(avae::launch_pack_unit_weights_n(src, dst, 2 * n_dil, C, K, s), "weight packing");
    }
    return run_amp(x, y, B, C, T, K, n_dil, dil, w1, b1 ? b1 : kNull, w2, b2 ? b2 : kNull,
                   log_alpha, log_beta, fused ? pw1 : nullptr, fused ? pw2 : nullptr, nullptr,
                   nullptr, out_scale, accumulate, cur, t1, t2, make_taps(nullptr, nullptr), s);
}
}  // namespace

extern "C" int avae_amp_block(const float* x, float* y, int B, int C, int T, int K, int n_dil,
                              const int* dil, const float* const* w1, const float* const* b1,
                              const float* const* w2, const float* const* b2,
                              const float* const* log_alpha, const float* const* log_beta,
                              float out_scale, int accumulate, void* workspace, size_t ws_bytes,
                              void* stream) {
    int rc = amp_block_check("avae_amp_block", x, y, B, C, T, K, n_dil, dil, w1, w2, log_alpha,
                             log_beta);
    if (rc) return rc;
    const size_t need = avae_amp_block_workspace_bytes(B, C, T);
    if (need == 0) return fail(AVAE_ESHAPE, "avae_amp_block: workspace size overflows");
    if (!workspace || ws_bytes < need)
        return fail(AVAE_EWORKSPACE, "avae_amp_block: workspace %zu bytes < %zu needed", ws_bytes,
                    need);
    // a workspace that holds the frequency-domain path's spectra and packed
    // weights selects that path for the convolutions that take it
    size_t fslot, fpack;
    amp_fft_plan(B, C, T, K, n_dil, dil, &fslot, &fpack);
    const bool fft = fslot && workspace && ws_bytes >= 3 * fslot + fpack;
    return amp_block_run(x, y, B, C, T, K, n_dil, dil, w1, b1, w2, b2, log_alpha, log_beta,
                         out_scale, accumulate, workspace, (hipStream_t)stream, fft ? fslot : 0);
}

// -------------------------------------------------------------------------
// AMP block without a workspace argument, for callers that cannot allocate.
// Its scratch is one file-scope device array per GPU (loaded with the
// library's code object and held until the process ends).  In host code the
// array's name is only a host-side stand-in: its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and
// that address is what the kernels receive.
// -------------------------------------------------------------------------

namespace {
constexpr size_t kStaticScratchBytes = (size_t)AVAE_AMP_STATIC_SCRATCH_MB << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the
// first call there).
int static_scratch(void** out) {
    int dev = 0;
    AVAE_TRY(hipGetDevice(&dev), "avae_amp_block_static: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(AVAE_EINVAL, "avae_amp_block_static: device %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        AVAE_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                 "avae_amp_block_static: hipGetSymbolAddress(scratch)");
        if (!p) return fail(AVAE_EHIP, "avae_amp_block_static: null scratch address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return AVAE_OK;
}
}  // namespace

extern "C" size_t avae_amp_block_static_max_bytes(void) { return kStaticScratchBytes; }

extern "C" int avae_amp_block_static(const float* x, float* y, int B, int C, int T, int K,
                                     int n_dil, const int* dil, const float* const* w1,
                                     const float* const* b1, const float* const* w2,
                                     const float* const* b2, const float* const* log_alpha,
                                     const float* const* log_beta, float out_scale,
                                     int accumulate, void* stream) {
    int rc = amp_block_check("avae_amp_block_static", x, y, B, C, T, K, n_dil, dil, w1, w2,
                             log_alpha, log_beta);
    if (rc) return rc;
    const size_t need = avae_amp_block_workspace_bytes(B, C, T);
    if (need == 0 || need > kStaticScratchBytes)
        return fail(AVAE_ESHAPE,
                    "avae_amp_block_static: [%d, %d, %d] needs %zu bytes of scratch, more than "
                    "the library's static %zu (use avae_amp_block with a workspace)",
                    B, C, T, need, kStaticScratchBytes);
    void* ws = nullptr;
    rc = static_scratch(&ws);
    if (rc) return rc;
    return amp_block_run(x, y, B, C, T, K, n_dil, dil, w1, b1, w2, b2, log_alpha, log_beta,
                         out_scale, accumulate, ws, (hipStream_t)stream);
}

// =========================================================================
// Decoder
// =========================================================================

struct avae_decoder {
    avae_config cfg;
    avae_weights w;  // pointers into `blob`
    void* blob = nullptr;
    size_t blob_bytes = 0;
    // packed AMP weights for the stages that run the fused unit (else null)
    const float* pw1[AVAE_MAX_STAGES][AVAE_MAX_KERNELS][AVAE_MAX_DIL] = {};
    const float* pw2[AVAE_MAX_STAGES][AVAE_MAX_KERNELS][AVAE_MAX_DIL] = {};
    void* pblob = nullptr;
    // frequency-domain weights of the AMP convolutions that plan::fft_amp_pack
    // selects (else null)
    const float* fw1[AVAE_MAX_STAGES][AVAE_MAX_KERNELS][AVAE_MAX_DIL] = {};
    const float* fw2[AVAE_MAX_STAGES][AVAE_MAX_KERNELS][AVAE_MAX_DIL] = {};
    void* fblob = nullptr;
    // The AMP blocks of a stage are independent (they all read the ConvT
    // output): blocks 1.. run on side streams forked from and joined back to
    // the caller's stream with events, so one block's last partial wave of
    // workgroups overlaps the others' work.
    // The side streams and events belong to the decoder, so the enqueue of
    // one stage's fork .. join is held under `mu`: calls from several host
    // threads stay correct (their side work queues up on the same streams).
    hipStream_t side[AVAE_MAX_KERNELS - 1] = {};
    hipEvent_t fork = nullptr;
    hipEvent_t join[AVAE_MAX_KERNELS - 1] = {};
    bool has_side = false;     // streams and events exist (n_kernels > 1)
    bool concurrent = false;   // use them (avae_decoder_set_concurrent)
    mutable std::mutex mu;
    int device = 0;
    ActTaps taps;
};

namespace {

int check_config(const avae_config* c) {
    if (c->c_in < 1) return fail(AVAE_EINVAL, "config: c_in < 1");
    if (c->dec_in_ch < 0) return fail(AVAE_EINVAL, "config: dec_in_ch < 0");
    if (c->k_pre < 1 || c->k_pre % 2 == 0 || c->k_pre > AVAE_MAX_TAPS ||
        c->k_post < 1 || c->k_post % 2 == 0 || c->k_post > AVAE_MAX_TAPS)
        return fail(AVAE_ESHAPE, "config: k_pre/k_post must be odd and <= %d", AVAE_MAX_TAPS);
    if (c->n_stages < 1 || c->n_stages > AVAE_MAX_STAGES)
        return fail(AVAE_ESHAPE, "config: n_stages must be in [1, %d]", AVAE_MAX_STAGES);
    if (c->n_kernels < 1 || c->n_kernels > AVAE_MAX_KERNELS)
        return fail(AVAE_ESHAPE, "config: n_kernels must be in [1, %d]", AVAE_MAX_KERNELS);
    if (c->n_dil < 1 || c->n_dil > AVAE_MAX_DIL)
        return fail(AVAE_ESHAPE, "config: n_dil must be in [1, %d]", AVAE_MAX_DIL);
    for (int i = 0; i <= c->n_stages; ++i)
        if (c->ch[i] < 1) return fail(AVAE_EINVAL, "config: ch[%d] < 1", i);
    if (c->ch[c->n_stages] > 1024)
        return fail(AVAE_ESHAPE, "config: last width %d too wide for conv_post", c->ch[c->n_stages]);
    for (int i = 0; i < c->n_stages; ++i) {
        if (c->rates[i] < 1 || c->up_k[i] < c->rates[i] || c->up_k[i] > AVAE_MAX_TAPS)
            return fail(AVAE_ESHAPE, "config: stage %d needs 1 <= rate <= up_k <= %d", i,
                        AVAE_MAX_TAPS);
    }
    for (int j = 0; j < c->n_kernels; ++j) {
        if (c->rb_k[j] < 1 || c->rb_k[j] % 2 == 0 || c->rb_k[j] > AVAE_MAX_TAPS)
            return fail(AVAE_ESHAPE, "config: rb_k[%d] must be odd and <= %d", j, AVAE_MAX_TAPS);
        for (int q = 0; q < c->n_dil; ++q)
            if (c->rb_d[j][q] < 1 || (c->rb_k[j] - 1) * c->rb_d[j][q] > 4096)
                return fail(AVAE_ESHAPE, "config: bad dilation rb_d[%d][%d]", j, q);
    }
    if (c->final_act < AVAE_FINAL_NONE || c->final_act > AVAE_FINAL_CLAMP)
        return fail(AVAE_EINVAL, "config: bad final_act");
    return AVAE_OK;
}

using avae::plan::decode_slot_bytes;
using avae::plan::stage_lengths;

struct BlobPlan {
    std::vector<std::pair<const float**, std::pair<const float*, size_t>>> items;
    size_t total = 0;
    // dst: where the blob pointer goes; src: caller pointer; n: floats
    void add(const float** dst, const float* src, size_t n) {
        if (!src) {
            *dst = nullptr;
            return;
        }
        items.push_back({dst, {src, n}});
        total += round_up(n * sizeof(float), 256);
    }
};

}  // namespace

extern "C" int avae_decoder_create(const avae_config* cfg, const avae_weights* w,
                                   avae_decoder** out) {
    if (!cfg || !w || !out) return fail(AVAE_EINVAL, "avae_decoder_create: null argument");
    *out = nullptr;
    int rc = check_config(cfg);
    if (rc) return rc;
    const avae_config& c = *cfg;
    // required tensors
    if (!w->conv_pre_w || !w->conv_post_w || !w->post_la || !w->post_lb)
        return fail(AVAE_EINVAL, "avae_decoder_create: missing conv_pre/conv_post/act_post weights");
    if (c.has_latent_affine && (!w->latent_mean || !w->latent_std))
        return fail(AVAE_EINVAL, "avae_decoder_create: latent affine needs mean and std");
    if (c.dec_in_ch && !w->dec_in_w) return fail(AVAE_EINVAL, "avae_decoder_create: missing dec_in_w");
    for (int i = 0; i < c.n_stages; ++i) {
        if (!w->up_w[i]) return fail(AVAE_EINVAL, "avae_decoder_create: missing up_w[%d]", i);
        for (int j = 0; j < c.n_kernels; ++j) {
            for (int q = 0; q < c.n_dil; ++q)
                if (!w->w1[i][j][q] || !w->w2[i][j][q])
                    return fail(AVAE_EINVAL, "avae_decoder_create: missing conv weight [%d][%d][%d]",
                                i, j, q);
            for (int q = 0; q < 2 * c.n_dil; ++q)
                if (!w->act_la[i][j][q] || !w->act_lb[i][j][q])
                    return fail(AVAE_EINVAL, "avae_decoder_create: missing activation [%d][%d][%d]",
                                i, j, q);
        }
    }

    avae_decoder* d = new (std::nothrow) avae_decoder();
    if (!d) return fail(AVAE_ENOMEM, "avae_decoder_create: host allocation failed");
    d->cfg = c;
    d->taps = make_taps(nullptr, nullptr);
    std::memset(&d->w, 0, sizeof(d->w));

    BlobPlan plan;
    const int cin2 = c.dec_in_ch ? c.dec_in_ch : c.c_in;
    if (c.has_latent_affine) {
        plan.add(&d->w.latent_mean, w->latent_mean, c.c_in);
        plan.add(&d->w.latent_std, w->latent_std, c.c_in);
    }
    if (c.dec_in_ch) {
        plan.add(&d->w.dec_in_w, w->dec_in_w, (size_t)c.dec_in_ch * c.c_in);
        plan.add(&d->w.dec_in_b, w->dec_in_b, c.dec_in_ch);
    }
    plan.add(&d->w.conv_pre_w, w->conv_pre_w, (size_t)c.ch[0] * cin2 * c.k_pre);
    plan.add(&d->w.conv_pre_b, w->conv_pre_b, c.ch[0]);
    for (int i = 0; i < c.n_stages; ++i) {
        const size_t ci = c.ch[i], co = c.ch[i + 1];
        plan.add(&d->w.up_w[i], w->up_w[i], ci * co * c.up_k[i]);
        plan.add(&d->w.up_b[i], w->up_b[i], co);
        for (int j = 0; j < c.n_kernels; ++j) {
            for (int q = 0; q < c.n_dil; ++q) {
                plan.add(&d->w.w1[i][j][q], w->w1[i][j][q], co * co * c.rb_k[j]);
                plan.add(&d->w.b1[i][j][q], w->b1[i][j][q], co);
                plan.add(&d->w.w2[i][j][q], w->w2[i][j][q], co * co * c.rb_k[j]);
                plan.add(&d->w.b2[i][j][q], w->b2[i][j][q], co);
            }
            for (int q = 0; q < 2 * c.n_dil; ++q) {
                plan.add(&d->w.act_la[i][j][q], w->act_la[i][j][q], co);
                plan.add(&d->w.act_lb[i][j][q], w->act_lb[i][j][q], co);
            }
        }
    }
    const size_t cl = c.ch[c.n_stages];
    plan.add(&d->w.post_la, w->post_la, cl);
    plan.add(&d->w.post_lb, w->post_lb, cl);
    plan.add(&d->w.conv_post_w, w->conv_post_w, cl * c.k_post);
    plan.add(&d->w.conv_post_b, w->conv_post_b, 1);

    hipError_t e = hipGetDevice(&d->device);
    if (e != hipSuccess) {
        delete d;
        return hip_fail(e, "avae_decoder_create: hipGetDevice");
    }
    e = hipMalloc(&d->blob, plan.total);
    if (e != hipSuccess) {
        delete d;
        return fail(AVAE_ENOMEM, "avae_decoder_create: hipMalloc(%zu): %s", plan.total,
                    hipGetErrorString(e));
    }
    d->blob_bytes = plan.total;
    char* p = (char*)d->blob;
    for (auto& it : plan.items) {
        const size_t n = it.second.second;
        e = hipMemcpy(p, it.second.first, n * sizeof(float), hipMemcpyDefault);
        if (e != hipSuccess) {
            (void)hipFree(d->blob);
            delete d;
            return hip_fail(e, "avae_decoder_create: weight copy");
        }
        *it.first = (const float*)p;
        p += round_up(n * sizeof(float), 256);
    }
    // Packed copies of the AMP weights of every stage the fused unit takes.
    size_t pbytes = 0;
    for (int i = 0; i < c.n_stages; ++i)
        for (int j = 0; j < c.n_kernels; ++j)
            if (c.ch[i + 1] <= kFuseMaxC && amp_fusable(c.ch[i + 1], c.rb_k[j], c.n_dil, c.rb_d[j]))
                pbytes += 2 * c.n_dil *
                          round_up(avae::amp_unit_packed_floats(c.ch[i + 1], c.rb_k[j]) *
                                       sizeof(float), 256);
    if (pbytes) {
        e = hipMalloc(&d->pblob, pbytes);
        if (e != hipSuccess) {
            (void)hipFree(d->blob);
            delete d;
            return fail(AVAE_ENOMEM, "avae_decoder_create: hipMalloc(%zu): %s", pbytes,
                        hipGetErrorString(e));
        }
        char* pp = (char*)d->pblob;
        for (int i = 0; i < c.n_stages && e == hipSuccess; ++i)
            for (int j = 0; j < c.n_kernels && e == hipSuccess; ++j) {
                const int co = c.ch[i + 1], K = c.rb_k[j];
                if (co > kFuseMaxC || !amp_fusable(co, K, c.n_dil, c.rb_d[j])) continue;
                const size_t per = round_up(avae::amp_unit_packed_floats(co, K) * sizeof(float), 256);
                for (int q = 0; q < c.n_dil && e == hipSuccess; ++q) {
                    float* p1 = (float*)pp;
                    float* p2 = (float*)(pp + per);
                    pp += 2 * per;
                    e = avae::launch_pack_unit_weights(d->w.w1[i][j][q], p1, co, K, nullptr);
                    if (e == hipSuccess)
                        e = avae::launch_pack_unit_weights(d->w.w2[i][j][q], p2, co, K, nullptr);
                    d->pw1[i][j][q] = p1;
                    d->pw2[i][j][q] = p2;
                }
            }
        if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
        if (e != hipSuccess) {
            (void)hipFree(d->pblob);
            (void)hipFree(d->blob);
            delete d;
            return hip_fail(e, "avae_decoder_create: weight packing");
        }
    }
    // Frequency-domain copies of the wide AMP convolutions.
    size_t fbytes = 0;
    for (int i = 0; i < c.n_stages; ++i)
        for (int j = 0; j < c.n_kernels; ++j) {
            const int co = c.ch[i + 1], K = c.rb_k[j];
            const size_t per = round_up(avae::fft_conv_weight_floats(co, co) * sizeof(float), 256);
            for (int q = 0; q < c.n_dil; ++q) {
                if (avae::plan::fft_amp_pack(co, K, c.rb_d[j][q])) fbytes += per;
                if (avae::plan::fft_amp_pack(co, K, 1)) fbytes += per;
            }
        }
    if (fbytes) {
        e = hipMalloc(&d->fblob, fbytes);
        if (e != hipSuccess) {
            if (d->pblob) (void)hipFree(d->pblob);
            (void)hipFree(d->blob);
            delete d;
            return fail(AVAE_ENOMEM, "avae_decoder_create: hipMalloc(%zu): %s", fbytes,
                        hipGetErrorString(e));
        }
        char* fp = (char*)d->fblob;
        for (int i = 0; i < c.n_stages && e == hipSuccess; ++i)
            for (int j = 0; j < c.n_kernels && e == hipSuccess; ++j) {
                const int co = c.ch[i + 1], K = c.rb_k[j];
                const size_t per =
                    round_up(avae::fft_conv_weight_floats(co, co) * sizeof(float), 256);
                for (int q = 0; q < c.n_dil && e == hipSuccess; ++q) {
                    const int dq = c.rb_d[j][q];
                    if (avae::plan::fft_amp_pack(co, K, dq)) {
                        e = avae::launch_fft_pack(d->w.w1[i][j][q], (float*)fp, co, co, K, dq,
                                                  nullptr);
                        d->fw1[i][j][q] = (const float*)fp;
                        fp += per;
                    }
                    if (e == hipSuccess && avae::plan::fft_amp_pack(co, K, 1)) {
                        e = avae::launch_fft_pack(d->w.w2[i][j][q], (float*)fp, co, co, K, 1,
                                                  nullptr);
                        d->fw2[i][j][q] = (const float*)fp;
                        fp += per;
                    }
                }
            }
        if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
        if (e != hipSuccess) {
            (void)hipFree(d->fblob);
            if (d->pblob) (void)hipFree(d->pblob);
            (void)hipFree(d->blob);
            delete d;
            return hip_fail(e, "avae_decoder_create: frequency-domain weights");
        }
    }
    // side streams and events for the concurrent MRF blocks (non-blocking:
    // no implicit ordering with the null stream; default priority)
    if (c.n_kernels > 1) {
        bool ok = hipEventCreateWithFlags(&d->fork, hipEventDisableTiming) == hipSuccess;
        for (int j = 0; ok && j < c.n_kernels - 1; ++j)
            ok = hipStreamCreateWithFlags(&d->side[j], hipStreamNonBlocking) == hipSuccess &&
                 hipEventCreateWithFlags(&d->join[j], hipEventDisableTiming) == hipSuccess;
        d->has_side = d->concurrent = ok;
    }
    *out = d;
    return AVAE_OK;
}

extern "C" void avae_decoder_destroy(avae_decoder* dec) {
    if (!dec) return;
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(dec->device);
    for (int j = 0; j < AVAE_MAX_KERNELS - 1; ++j) {
        if (dec->side[j]) (void)hipStreamDestroy(dec->side[j]);
        if (dec->join[j]) (void)hipEventDestroy(dec->join[j]);
    }
    if (dec->fork) (void)hipEventDestroy(dec->fork);
    if (dec->blob) (void)hipFree(dec->blob);
    if (dec->pblob) (void)hipFree(dec->pblob);
    if (dec->fblob) (void)hipFree(dec->fblob);
    (void)hipSetDevice(cur);
    delete dec;
}

extern "C" int avae_decoder_output_length(const avae_decoder* dec, int frames, int* out_len) {
    if (!dec || !out_len) return fail(AVAE_EINVAL, "avae_decoder_output_length: null argument");
    if (frames < 1) return fail(AVAE_EINVAL, "avae_decoder_output_length: frames < 1");
    long long T[AVAE_MAX_STAGES + 1];
    if (stage_lengths(dec->cfg, frames, T))
        return fail(AVAE_ESHAPE, "avae_decoder_output_length: length overflow");
    *out_len = (int)T[dec->cfg.n_stages];
    return AVAE_OK;
}

namespace {
// Workspace slots: M and X, then per AMP block its own three scratch slots
// and (blocks after the first) its own output, when the blocks run
// concurrently; M, X and one block's scratch otherwise.
int decode_slots(const avae_decoder* dec) {
    return dec->has_side ? 1 + 4 * dec->cfg.n_kernels : 5;
}
}  // namespace

extern "C" int avae_decoder_set_concurrent(avae_decoder* dec, int on) {
    if (!dec) return fail(AVAE_EINVAL, "avae_decoder_set_concurrent: null decoder");
    if (on && !dec->has_side)
        return fail(AVAE_EINVAL, "avae_decoder_set_concurrent: this decoder has %s",
                    dec->cfg.n_kernels > 1 ? "no side streams (creation failed)"
                                           : "a single AMP block per stage");
    dec->concurrent = on != 0;
    return AVAE_OK;
}

extern "C" size_t avae_decoder_workspace_bytes(const avae_decoder* dec, int B, int frames) {
    if (!dec || B < 1 || frames < 1) return 0;
    long long T[AVAE_MAX_STAGES + 1];
    if (stage_lengths(dec->cfg, frames, T)) return 0;
    return decode_slots(dec) * decode_slot_bytes(dec->cfg, B, T);
}

namespace {

int decode_impl(const avae_decoder* dec, const float* latent, int B, int frames, float* wave,
                void* workspace, size_t ws_bytes, float* const* stage_out, hipStream_t s) {
    if (!dec || !latent || !wave) return fail(AVAE_EINVAL, "avae_bigvgan_decode: null argument");
    if (B < 1 || frames < 1) return fail(AVAE_EINVAL, "avae_bigvgan_decode: B, frames must be >= 1");
    const avae_config& c = dec->cfg;
    const avae_weights& w = dec->w;
    long long T[AVAE_MAX_STAGES + 1];
    if (stage_lengths(c, frames, T))
        return fail(AVAE_ESHAPE, "avae_bigvgan_decode: length overflow");
    const size_t slot = decode_slot_bytes(c, B, T);
    if (slot == 0) return fail(AVAE_ESHAPE, "avae_bigvgan_decode: workspace size overflows");
    const size_t need = decode_slots(dec) * slot;
    if (!workspace || ws_bytes < need)
        return fail(AVAE_EWORKSPACE, "avae_bigvgan_decode: workspace %zu bytes < %zu needed",
                    ws_bytes, need);
    char* ws = (char*)workspace;
    float* M = (float*)(ws + 0 * slot);   // stage input/output (MRF accumulator)
    float* X = (float*)(ws + 1 * slot);   // ConvT output: every AMP block's input
    float* cur = (float*)(ws + 2 * slot);
    float* t1 = (float*)(ws + 3 * slot);
    float* t2 = (float*)(ws + 4 * slot);

    const int F = frames;
    const float* h = latent;
    int cin = c.c_in;
    avae::prof_set_phase(avae::kPhaseDecIn);
    if (c.has_latent_affine) {
        AVAE_TRY(avae::launch_channel_affine(h, X, w.latent_std, w.latent_mean, B, c.c_in, F, s),
                 "latent affine");
        h = X;
    }
    if (c.dec_in_ch) {
        ConvEpilogue e{w.dec_in_b, nullptr, 1.0f, 0};
        AVAE_TRY(avae::launch_conv1d(h, cur, w.dec_in_w, B, cin, c.dec_in_ch, F, F, 1, 1, 0, e, s),
                 "dec_in");
        h = cur;
        cin = c.dec_in_ch;
    }
    avae::prof_set_phase(avae::kPhaseConvPre);
    {
        ConvEpilogue e{w.conv_pre_b, nullptr, 1.0f, 0};
        AVAE_TRY(avae::launch_conv1d(h, M, w.conv_pre_w, B, cin, c.ch[0], F, F, c.k_pre, 1,
                                     (c.k_pre - 1) / 2, e, s),
                 "conv_pre");
    }
    if (stage_out && stage_out[0])
        AVAE_TRY(hipMemcpyAsync(stage_out[0], M, (size_t)B * c.ch[0] * F * sizeof(float),
                                hipMemcpyDeviceToDevice, s),
                 "trace copy");
    const float inv_nk = 1.0f / (float)c.n_kernels;
    for (int i = 0; i < c.n_stages; ++i) {
        const int ci = c.ch[i], co = c.ch[i + 1];
        const int Ti = (int)T[i], To = (int)T[i + 1];
        const int pad = (c.up_k[i] - c.rates[i]) / 2;
        avae::prof_set_phase(avae::kPhaseUpsamples);
        AVAE_TRY(avae::launch_convtr1d(M, X, w.up_w[i], w.up_b[i], B, ci, co, Ti, To, c.up_k[i],
                                       c.rates[i], pad, s),
                 "ConvTranspose1d");
        avae::prof_set_phase(avae::kPhaseResblocks);
        if (dec->concurrent) {
            std::lock_guard<std::mutex> lk(dec->mu);
            // fork: every block waits for the ConvT output X
            AVAE_TRY(hipEventRecord(dec->fork, s), "fork event");
            for (int k = 1; k < c.n_kernels; ++k)
                AVAE_TRY(hipStreamWaitEvent(dec->side[k - 1], dec->fork, 0), "fork wait");
            // block 0 writes M; block k >= 1 its own slot after the scratch slots
            float* outs[AVAE_MAX_KERNELS] = {M};
            for (int k = 1; k < c.n_kernels; ++k)
                outs[k] = (float*)(ws + (size_t)(1 + 3 * c.n_kernels + k) * slot);
            // enqueued one dilation step of every block at a time, so that no
            // stream waits for the host to finish enqueuing the blocks before it
            for (int q = 0; q < c.n_dil; ++q)
                for (int k = 0; k < c.n_kernels; ++k) {
                    hipStream_t sk = k == 0 ? s : dec->side[k - 1];
                    float* sc = (float*)(ws + (size_t)(2 + 3 * k) * slot);
                    float* s1 = (float*)(ws + (size_t)(3 + 3 * k) * slot);
                    float* s2 = (float*)(ws + (size_t)(4 + 3 * k) * slot);
                    const bool fused = dec->pw1[i][k][0] != nullptr;
                    int rc = run_amp(X, outs[k], B, co, To, c.rb_k[k], c.n_dil, c.rb_d[k],
                                     w.w1[i][k], w.b1[i][k], w.w2[i][k], w.b2[i][k],
                                     w.act_la[i][k], w.act_lb[i][k],
                                     fused ? dec->pw1[i][k] : nullptr,
                                     fused ? dec->pw2[i][k] : nullptr, dec->fw1[i][k],
                                     dec->fw2[i][k], inv_nk, 0, sc, s1, s2, dec->taps, sk, nullptr,
                                     q, q + 1);
                    if (rc) return rc;
                }
            // join, then M = block 0 + the others (each already scaled by 1/nk)
            for (int k = 1; k < c.n_kernels; ++k) {
                AVAE_TRY(hipEventRecord(dec->join[k - 1], dec->side[k - 1]), "join event");
                AVAE_TRY(hipStreamWaitEvent(s, dec->join[k - 1], 0), "join wait");
            }
            AVAE_TRY(avae::launch_sum_into(M, outs + 1, c.n_kernels - 1, (size_t)B * co * To, s),
                     "MRF sum");
        } else {
            for (int j = 0; j < c.n_kernels; ++j) {
                const bool fused = dec->pw1[i][j][0] != nullptr;
                int rc = run_amp(X, M, B, co, To, c.rb_k[j], c.n_dil, c.rb_d[j], w.w1[i][j],
                                 w.b1[i][j], w.w2[i][j], w.b2[i][j], w.act_la[i][j],
                                 w.act_lb[i][j], fused ? dec->pw1[i][j] : nullptr,
                                 fused ? dec->pw2[i][j] : nullptr, dec->fw1[i][j],
                                 dec->fw2[i][j], inv_nk, j > 0 ? 1 : 0, cur, t1, t2, dec->taps,
                                 s);
                if (rc) return rc;
            }
        }
        if (stage_out && stage_out[1 + i])
            AVAE_TRY(hipMemcpyAsync(stage_out[1 + i], M, (size_t)B * co * To * sizeof(float),
                                    hipMemcpyDeviceToDevice, s),
                     "trace copy");
    }
    const int cl = c.ch[c.n_stages];
    const int TL = (int)T[c.n_stages];
    avae::prof_set_phase(avae::kPhaseActPost);
    AVAE_TRY(avae::launch_act1d(M, t1, B, cl, TL, w.post_la, w.post_lb, dec->taps, s),
             "act_post");
    avae::prof_set_phase(avae::kPhaseConvPost);
    float* pre = (stage_out && stage_out[c.n_stages + 1]) ? stage_out[c.n_stages + 1] : nullptr;
    AVAE_TRY(avae::launch_conv_out1(t1, wave, pre, w.conv_post_w, w.conv_post_b, B, cl, TL,
                                    c.k_post, c.final_act, 0, s),
             "conv_post");
    avae::prof_set_phase(avae::kPhaseNone);
    return AVAE_OK;
}

}  // namespace

extern "C" int avae_bigvgan_decode(const avae_decoder* dec, const float* latent, int B,
                                   int frames, float* wave, void* workspace, size_t ws_bytes,
                                   void* stream) {
    return decode_impl(dec, latent, B, frames, wave, workspace, ws_bytes, nullptr,
                       (hipStream_t)stream);
}

extern "C" int avae_bigvgan_decode_traced(const avae_decoder* dec, const float* latent, int B,
                                          int frames, float* wave, void* workspace,
                                          size_t ws_bytes, float* const* stage_out,
                                          void* stream) {
    return decode_impl(dec, latent, B, frames, wave, workspace, ws_bytes, stage_out,
                       (hipStream_t)stream);
}

// =========================================================================
// Streaming decode
// =========================================================================

namespace {

using avae::plan::hop_of;
using avae::plan::reach_frames;

bool stream_plan(const avae_decoder* dec, int B, int tile_frames, int halo,
                 avae::plan::StreamBytes* p) {
    return avae::plan::stream_bytes(dec->cfg, decode_slots(dec), B, tile_frames, halo, p);
}

}  // namespace

extern "C" int avae_decoder_reach_frames(const avae_decoder* dec, int* out_frames) {
    if (!dec || !out_frames) return fail(AVAE_EINVAL, "avae_decoder_reach_frames: null argument");
    *out_frames = reach_frames(dec->cfg);
    return AVAE_OK;
}

extern "C" size_t avae_decoder_streaming_workspace_bytes(const avae_decoder* dec, int B,
                                                         int tile_frames, int halo_frames) {
    if (!dec || B < 1 || tile_frames < 1) return 0;
    const int halo = halo_frames < 0 ? reach_frames(dec->cfg) : halo_frames;
    avae::plan::StreamBytes p;
    if (!stream_plan(dec, B, tile_frames, halo, &p)) return 0;
    return p.total();
}

extern "C" int avae_bigvgan_decode_streaming(const avae_decoder* dec, const float* latent, int B,
                                             int frames, float* wave, int tile_frames,
                                             int halo_frames, void* workspace, size_t ws_bytes,
                                             void* stream) {
    if (!dec || !latent || !wave)
        return fail(AVAE_EINVAL, "avae_bigvgan_decode_streaming: null argument");
    if (B < 1 || frames < 1 || tile_frames < 1)
        return fail(AVAE_EINVAL, "avae_bigvgan_decode_streaming: B, frames, tile_frames must be >= 1");
    const avae_config& c = dec->cfg;
    const long long hop = hop_of(c);
    long long T[AVAE_MAX_STAGES + 1];
    if (stage_lengths(c, frames, T) || T[c.n_stages] != frames * hop ||
        stage_lengths(c, 1, T) || T[c.n_stages] != hop)
        return fail(AVAE_ESHAPE,
                    "avae_bigvgan_decode_streaming: output length is not frames x hop for this config");
    const int halo = halo_frames < 0 ? reach_frames(c) : halo_frames;
    const avae::plan::TileGrid g = avae::plan::tile_grid(frames, tile_frames, halo);
    avae::plan::StreamBytes plan;
    if (!stream_plan(dec, B, g.tf, halo, &plan))
        return fail(AVAE_ESHAPE, "avae_bigvgan_decode_streaming: tile too long");
    if (!workspace || ws_bytes < plan.total())
        return fail(AVAE_EWORKSPACE, "avae_bigvgan_decode_streaming: workspace %zu bytes < %zu",
                    ws_bytes, plan.total());
    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    float* crop = (float*)ws;
    float* twave = (float*)(ws + plan.crop_bytes);
    void* dws = ws + plan.crop_bytes + plan.wave_bytes;
    const size_t rows = (size_t)B * c.c_in;
    // One batched decode per group of tiles with equal crop lengths.
    return avae::plan::for_each_tile_group(g, [&](const int* group, int ng, int glen) -> int {
        for (int k = 0; k < ng; ++k) {
            int c0, len;
            g.crop(group[k], &c0, &len);
            AVAE_TRY(hipMemcpy2DAsync(crop + (size_t)k * rows * len, (size_t)len * sizeof(float),
                                      latent + c0, (size_t)frames * sizeof(float),
                                      (size_t)len * sizeof(float), rows, hipMemcpyDeviceToDevice,
                                      s),
                     "streaming crop copy");
        }
        int rc = decode_impl(dec, crop, B * ng, glen, twave, dws, plan.dec_bytes, nullptr, s);
        if (rc) return rc;
        const size_t lcrop = (size_t)glen * hop;
        for (int k = 0; k < ng; ++k) {
            int c0, len, f0, f1;
            g.crop(group[k], &c0, &len);
            g.kept(group[k], &f0, &f1);
            AVAE_TRY(hipMemcpy2DAsync(wave + (size_t)f0 * hop, (size_t)frames * hop * sizeof(float),
                                      twave + (size_t)k * B * lcrop + (size_t)(f0 - c0) * hop,
                                      lcrop * sizeof(float), (size_t)(f1 - f0) * hop * sizeof(float),
                                      (size_t)B, hipMemcpyDeviceToDevice, s),
                     "streaming tile copy");
        }
        return AVAE_OK;
    });
}

// =========================================================================
// Plain Snake and the Music-3 DAV decoder
// =========================================================================

extern "C" int avae_probe_mfma(int chains, int blocks, int iters, float* sink, void* stream) {
    if (!sink) return fail(AVAE_EINVAL, "avae_probe_mfma: sink is null");
    if ((chains != 8 && chains != 16) || blocks < 1 || iters < 1)
        return fail(AVAE_EINVAL, "avae_probe_mfma: chains must be 8 or 16, blocks and iters >= 1 "
                                 "(got %d, %d, %d)", chains, blocks, iters);
    avae::prof_set_phase(avae::kPhaseNone);
    AVAE_TRY(avae::launch_mfma_probe(chains, blocks, iters, sink, (hipStream_t)stream),
             "avae_probe_mfma launch");
    return AVAE_OK;
}

extern "C" int avae_probe_copy(const float* x, float* y, long long n, void* stream) {
    if (!x || !y) return fail(AVAE_EINVAL, "avae_probe_copy: null pointer");
    if (n < 4 || n % 4 != 0 || n / 4 > 0x7fffffffLL * 256)
        return fail(AVAE_EINVAL, "avae_probe_copy: n must be a positive multiple of 4 (got %lld)", n);
    if ((((uintptr_t)x) | ((uintptr_t)y)) & 15)
        return fail(AVAE_EINVAL, "avae_probe_copy: x and y must be 16-byte aligned");
    avae::prof_set_phase(avae::kPhaseNone);
    AVAE_TRY(avae::launch_stream_copy(x, y, n / 4, (hipStream_t)stream), "avae_probe_copy launch");
    return AVAE_OK;
}

extern "C" int avae_snake(const float* x, float* y, int B, int C, int T, const float* alpha,
                          void* stream) {
    if (!x || !y || !alpha) return fail(AVAE_EINVAL, "avae_snake: null pointer");
    if (B < 1 || C < 1 || T < 1)
        return fail(AVAE_EINVAL, "avae_snake: B, C, T must be >= 1 (got %d, %d, %d)", B, C, T);
    avae::prof_set_phase(avae::kPhaseNone);
    AVAE_TRY(avae::launch_snake(x, y, B, C, T, alpha, (hipStream_t)stream), "avae_snake launch");
    return AVAE_OK;
}

struct avae_dav {
    avae_dav_config cfg;
    avae_dav_weights w;  // pointers into `blob`
    void* blob = nullptr;
    // frequency-domain weights of the units' first (dilated) convolutions
    // that plan::fft_amp_pack selects (else null)
    const float* fw1[AVAE_MAX_STAGES][AVAE_MAX_DIL] = {};
    void* fblob = nullptr;
    int device = 0;
};

namespace {

int check_dav_config(const avae_dav_config* c) {
    if (c->c_side < 1 || c->dec_in_ch < 1) return fail(AVAE_EINVAL, "dav config: c_side/dec_in_ch < 1");
    if (c->k_pre < 1 || c->k_pre % 2 == 0 || c->k_pre > AVAE_MAX_TAPS || c->k_post < 1 ||
        c->k_post % 2 == 0 || c->k_post > AVAE_MAX_TAPS)
        return fail(AVAE_ESHAPE, "dav config: k_pre/k_post must be odd and <= %d", AVAE_MAX_TAPS);
    if (c->n_stages < 1 || c->n_stages > AVAE_MAX_STAGES)
        return fail(AVAE_ESHAPE, "dav config: n_stages must be in [1, %d]", AVAE_MAX_STAGES);
    if (c->unit_k < 1 || c->unit_k % 2 == 0 || c->unit_k > AVAE_MAX_TAPS)
        return fail(AVAE_ESHAPE, "dav config: unit_k must be odd and <= %d", AVAE_MAX_TAPS);
    if (c->n_units < 1 || c->n_units > AVAE_MAX_DIL)
        return fail(AVAE_ESHAPE, "dav config: n_units must be in [1, %d]", AVAE_MAX_DIL);
    for (int u = 0; u < c->n_units; ++u)
        if (c->unit_dil[u] < 1 || (long long)(c->unit_k - 1) * c->unit_dil[u] > 4096)
            return fail(AVAE_ESHAPE, "dav config: bad unit_dil[%d]", u);
    for (int i = 0; i <= c->n_stages; ++i)
        if (c->ch[i] < 1) return fail(AVAE_EINVAL, "dav config: ch[%d] < 1", i);
    if (c->ch[c->n_stages] > 1024)
        return fail(AVAE_ESHAPE, "dav config: last width %d too wide for conv_post", c->ch[c->n_stages]);
    for (int i = 0; i < c->n_stages; ++i)
        if (c->strides[i] < 1 || c->up_k[i] < c->strides[i] || c->up_k[i] > AVAE_MAX_TAPS)
            return fail(AVAE_ESHAPE, "dav config: stage %d needs 1 <= stride <= up_k <= %d", i,
                        AVAE_MAX_TAPS);
    return AVAE_OK;
}

int dav_lengths(const avae_dav_config& c, int frames, long long* T) {
    T[0] = frames;
    for (int i = 0; i < c.n_stages; ++i) {
        const int p = (c.up_k[i] - c.strides[i]) / 2;
        T[i + 1] = (T[i] - 1) * c.strides[i] + c.up_k[i] - 2LL * p;
        if (T[i + 1] < 1 || T[i + 1] > 0x7fffffffLL) return 1;
    }
    return 0;
}

// One workspace slot: the largest [2B, C, T] activation of the 2 B side
// passes, or the largest spectrum of a unit convolution run in the
// frequency domain (0 if a size overflows).
size_t dav_slot_bytes(const avae_dav_config& c, int B, const long long* T) {
    const long long B2 = 2LL * B;
    size_t m = avae::plan::tensor_bytes(B2, std::max(c.dec_in_ch, c.ch[0]), T[0]);
    bool over = m == 0 || B2 > 0x3fffffffLL;
    for (int i = 0; i < c.n_stages && !over; ++i) {
        const size_t a = avae::plan::tensor_bytes(B2, c.ch[i], T[i]);
        const size_t b = avae::plan::tensor_bytes(B2, c.ch[i + 1], T[i + 1]);
        over = over || a == 0 || b == 0;
        m = std::max(m, std::max(a, b));
        for (int u = 0; u < c.n_units; ++u)
            if (avae::plan::fft_amp_use((int)B2, c.ch[i + 1], (int)T[i + 1], c.unit_k,
                                        c.unit_dil[u])) {
                const size_t f = avae::plan::fft_spectrum_bytes((int)B2, c.ch[i + 1],
                                                                (int)T[i + 1], c.unit_k,
                                                                c.unit_dil[u]);
                over = over || f == 0;
                m = std::max(m, f);
            }
    }
    return over ? 0 : m;
}

int dav_decode_impl(const avae_dav* dav, const float* latent, int B, int frames, float* wave,
                    void* workspace, size_t ws_bytes, float* const* trace, hipStream_t s) {
    if (!dav || !latent || !wave) return fail(AVAE_EINVAL, "avae_dav_decode: null argument");
    if (B < 1 || frames < 1) return fail(AVAE_EINVAL, "avae_dav_decode: B, frames must be >= 1");
    const avae_dav_config& c = dav->cfg;
    const avae_dav_weights& w = dav->w;
    long long T[AVAE_MAX_STAGES + 1];
    if (dav_lengths(c, frames, T)) return fail(AVAE_ESHAPE, "avae_dav_decode: length overflow");
    if ((long long)2 * B * T[c.n_stages] > 0x7fffffffLL)
        return fail(AVAE_ESHAPE, "avae_dav_decode: output too long");
    const size_t slot = dav_slot_bytes(c, B, T);
    if (slot == 0) return fail(AVAE_ESHAPE, "avae_dav_decode: workspace size overflows");
    if (!workspace || ws_bytes < 3 * slot)
        return fail(AVAE_EWORKSPACE, "avae_dav_decode: workspace %zu bytes < %zu needed", ws_bytes,
                    3 * slot);
    char* ws = (char*)workspace;
    float* P0 = (float*)ws;             // the running activation
    float* P1 = (float*)(ws + slot);    // dec_in output / transposed-conv output
    float* P2 = (float*)(ws + 2 * slot);  // a unit's first conv output
    const int B2 = 2 * B;  // row 2b + side: the latent's channel halves are the sides
    const int F = frames;
    avae::prof_set_phase(avae::kPhaseDecIn);
    {
        ConvEpilogue e{w.dec_in_b, nullptr, 1.0f, 0, nullptr, nullptr};
        AVAE_TRY(avae::launch_conv1d(latent, P1, w.dec_in_w, B2, c.c_side, c.dec_in_ch, F, F, 1, 1,
                                     0, e, s),
                 "dav dec_in");
    }
    avae::prof_set_phase(avae::kPhaseConvPre);
    {
        ConvEpilogue e{w.conv_pre_b, nullptr, 1.0f, 0, nullptr, nullptr};
        AVAE_TRY(avae::launch_conv1d(P1, P0, w.conv_pre_w, B2, c.dec_in_ch, c.ch[0], F, F, c.k_pre,
                                     1, (c.k_pre - 1) / 2, e, s),
                 "dav conv_pre");
    }
    if (trace && trace[0])
        AVAE_TRY(hipMemcpyAsync(trace[0], P0, (size_t)B2 * c.ch[0] * F * sizeof(float),
                                hipMemcpyDeviceToDevice, s),
                 "trace copy");
    for (int i = 0; i < c.n_stages; ++i) {
        const int ci = c.ch[i], co = c.ch[i + 1];
        const int Ti = (int)T[i], To = (int)T[i + 1];
        avae::prof_set_phase(avae::kPhaseUpsamples);
        // the stage's Snake is applied as the transposed conv stages its input
        AVAE_TRY(avae::launch_convtr1d(P0, P1, w.up_w[i], w.up_b[i], B2, ci, co, Ti, To, c.up_k[i],
                                       c.strides[i], (c.up_k[i] - c.strides[i]) / 2, s,
                                       w.stage_alpha[i]),
                 "dav ConvTranspose1d");
        std::swap(P0, P1);
        avae::prof_set_phase(avae::kPhaseResblocks);
        for (int u = 0; u < c.n_units; ++u) {
            const int d = c.unit_dil[u];
            // c1: the first Snake on its input, the second in its epilogue
            ConvEpilogue e1{w.b1[i][u], nullptr, 1.0f, 0, w.a2[i][u], w.a1[i][u]};
            float* h = P2;  // c1's output
            if (dav->fw1[i][u] && avae::plan::fft_amp_use(B2, co, To, c.unit_k, d)) {
                // frequency domain: spectrum in P1, product in P2, output in P1
                AVAE_TRY(avae::launch_conv1d_fft(P0, P1, dav->fw1[i][u], B2, co, co, To,
                                                 c.unit_k, d, e1, P1, P2, s),
                         "dav unit conv_fft");
                h = P1;
            } else {
                AVAE_TRY(avae::launch_conv1d(P0, P2, w.w1[i][u], B2, co, co, To, To, c.unit_k, d,
                                             (c.unit_k - 1) / 2 * d, e1, s),
                         "dav unit conv");
            }
            // c2 (one tap) plus the residual, in place on the running activation
            ConvEpilogue e2{w.b2[i][u], P0, 1.0f, 0, nullptr, nullptr};
            AVAE_TRY(avae::launch_conv1d(h, P0, w.w2[i][u], B2, co, co, To, To, 1, 1, 0, e2, s),
                     "dav unit 1-tap conv");
        }
        if (trace && trace[1 + i])
            AVAE_TRY(hipMemcpyAsync(trace[1 + i], P0, (size_t)B2 * co * To * sizeof(float),
                                    hipMemcpyDeviceToDevice, s),
                     "trace copy");
    }
    const int cl = c.ch[c.n_stages];
    const int TL = (int)T[c.n_stages];
    avae::prof_set_phase(avae::kPhaseConvPost);
    float* pre = (trace && trace[c.n_stages + 1]) ? trace[c.n_stages + 1] : nullptr;
    // the final Snake is applied as conv_post stages its input
    AVAE_TRY(avae::launch_conv_out1(P0, wave, pre, w.conv_post_w, w.conv_post_b, B2, cl, TL,
                                    c.k_post, AVAE_FINAL_TANH, 1, s, w.post_alpha),
             "dav conv_post");
    avae::prof_set_phase(avae::kPhaseNone);
    return AVAE_OK;
}

}  // namespace

extern "C" int avae_dav_create(const avae_dav_config* cfg, const avae_dav_weights* w,
                               avae_dav** out) {
    if (!cfg || !w || !out) return fail(AVAE_EINVAL, "avae_dav_create: null argument");
    *out = nullptr;
    int rc = check_dav_config(cfg);
    if (rc) return rc;
    const avae_dav_config& c = *cfg;
    if (!w->dec_in_w || !w->conv_pre_w || !w->post_alpha || !w->conv_post_w)
        return fail(AVAE_EINVAL, "avae_dav_create: missing dec_in/conv_pre/post weights");
    for (int i = 0; i < c.n_stages; ++i) {
        if (!w->stage_alpha[i] || !w->up_w[i])
            return fail(AVAE_EINVAL, "avae_dav_create: missing stage %d snake/upsampler", i);
        for (int u = 0; u < c.n_units; ++u)
            if (!w->a1[i][u] || !w->w1[i][u] || !w->a2[i][u] || !w->w2[i][u])
                return fail(AVAE_EINVAL, "avae_dav_create: missing unit [%d][%d]", i, u);
    }
    avae_dav* d = new (std::nothrow) avae_dav();
    if (!d) return fail(AVAE_ENOMEM, "avae_dav_create: host allocation failed");
    d->cfg = c;
    std::memset(&d->w, 0, sizeof(d->w));
    BlobPlan plan;
    plan.add(&d->w.dec_in_w, w->dec_in_w, (size_t)c.dec_in_ch * c.c_side);
    plan.add(&d->w.dec_in_b, w->dec_in_b, c.dec_in_ch);
    plan.add(&d->w.conv_pre_w, w->conv_pre_w, (size_t)c.ch[0] * c.dec_in_ch * c.k_pre);
    plan.add(&d->w.conv_pre_b, w->conv_pre_b, c.ch[0]);
    for (int i = 0; i < c.n_stages; ++i) {
        const size_t ci = c.ch[i], co = c.ch[i + 1];
        plan.add(&d->w.stage_alpha[i], w->stage_alpha[i], ci);
        plan.add(&d->w.up_w[i], w->up_w[i], ci * co * c.up_k[i]);
        plan.add(&d->w.up_b[i], w->up_b[i], co);
        for (int u = 0; u < c.n_units; ++u) {
            plan.add(&d->w.a1[i][u], w->a1[i][u], co);
            plan.add(&d->w.w1[i][u], w->w1[i][u], co * co * c.unit_k);
            plan.add(&d->w.b1[i][u], w->b1[i][u], co);
            plan.add(&d->w.a2[i][u], w->a2[i][u], co);
            plan.add(&d->w.w2[i][u], w->w2[i][u], co * co);
            plan.add(&d->w.b2[i][u], w->b2[i][u], co);
        }
    }
    const size_t cl = c.ch[c.n_stages];
    plan.add(&d->w.post_alpha, w->post_alpha, cl);
    plan.add(&d->w.conv_post_w, w->conv_post_w, cl * c.k_post);
    plan.add(&d->w.conv_post_b, w->conv_post_b, 1);
    hipError_t e = hipGetDevice(&d->device);
    if (e != hipSuccess) {
        delete d;
        return hip_fail(e, "avae_dav_create: hipGetDevice");
    }
    e = hipMalloc(&d->blob, plan.total);
    if (e != hipSuccess) {
        delete d;
        return fail(AVAE_ENOMEM, "avae_dav_create: hipMalloc(%zu): %s", plan.total,
                    hipGetErrorString(e));
    }
    char* p = (char*)d->blob;
    for (auto& it : plan.items) {
        const size_t n = it.second.second;
        e = hipMemcpy(p, it.second.first, n * sizeof(float), hipMemcpyDefault);
        if (e != hipSuccess) {
            (void)hipFree(d->blob);
            delete d;
            return hip_fail(e, "avae_dav_create: weight copy");
        }
        *it.first = (const float*)p;
        p += round_up(n * sizeof(float), 256);
    }
    // frequency-domain copies of the units' dilated convolutions
    size_t fbytes = 0;
    for (int i = 0; i < c.n_stages; ++i)
        for (int u = 0; u < c.n_units; ++u)
            if (avae::plan::fft_amp_pack(c.ch[i + 1], c.unit_k, c.unit_dil[u]))
                fbytes += round_up(
                    avae::fft_conv_weight_floats(c.ch[i + 1], c.ch[i + 1]) * sizeof(float), 256);
    if (fbytes) {
        e = hipMalloc(&d->fblob, fbytes);
        if (e != hipSuccess) {
            (void)hipFree(d->blob);
            delete d;
            return fail(AVAE_ENOMEM, "avae_dav_create: hipMalloc(%zu): %s", fbytes,
                        hipGetErrorString(e));
        }
        char* fp = (char*)d->fblob;
        for (int i = 0; i < c.n_stages && e == hipSuccess; ++i)
            for (int u = 0; u < c.n_units && e == hipSuccess; ++u) {
                const int co = c.ch[i + 1];
                if (!avae::plan::fft_amp_pack(co, c.unit_k, c.unit_dil[u])) continue;
                e = avae::launch_fft_pack(d->w.w1[i][u], (float*)fp, co, co, c.unit_k,
                                          c.unit_dil[u], nullptr);
                d->fw1[i][u] = (const float*)fp;
                fp += round_up(avae::fft_conv_weight_floats(co, co) * sizeof(float), 256);
            }
        if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
        if (e != hipSuccess) {
            (void)hipFree(d->fblob);
            (void)hipFree(d->blob);
            delete d;
            return hip_fail(e, "avae_dav_create: frequency-domain weights");
        }
    }
    *out = d;
    return AVAE_OK;
}

extern "C" void avae_dav_destroy(avae_dav* dav) {
    if (!dav) return;
    if (dav->blob || dav->fblob) {
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(dav->device);
        if (dav->blob) (void)hipFree(dav->blob);
        if (dav->fblob) (void)hipFree(dav->fblob);
        (void)hipSetDevice(cur);
    }
    delete dav;
}

extern "C" int avae_dav_output_length(const avae_dav* dav, int frames, int* out_len) {
    if (!dav || !out_len) return fail(AVAE_EINVAL, "avae_dav_output_length: null argument");
    if (frames < 1) return fail(AVAE_EINVAL, "avae_dav_output_length: frames < 1");
    long long T[AVAE_MAX_STAGES + 1];
    if (dav_lengths(dav->cfg, frames, T))
        return fail(AVAE_ESHAPE, "avae_dav_output_length: length overflow");
    *out_len = (int)T[dav->cfg.n_stages];
    return AVAE_OK;
}

extern "C" size_t avae_dav_workspace_bytes(const avae_dav* dav, int B, int frames) {
    if (!dav || B < 1 || frames < 1) return 0;
    long long T[AVAE_MAX_STAGES + 1];
    if (dav_lengths(dav->cfg, frames, T)) return 0;
    return 3 * dav_slot_bytes(dav->cfg, B, T);
}

extern "C" int avae_dav_decode(const avae_dav* dav, const float* latent, int B, int frames,
                               float* wave, void* workspace, size_t ws_bytes, void* stream) {
    return dav_decode_impl(dav, latent, B, frames, wave, workspace, ws_bytes, nullptr,
                           (hipStream_t)stream);
}

extern "C" int avae_dav_decode_traced(const avae_dav* dav, const float* latent, int B, int frames,
                                      float* wave, void* workspace, size_t ws_bytes,
                                      float* const* stage_out, void* stream) {
    return dav_decode_impl(dav, latent, B, frames, wave, workspace, ws_bytes, stage_out,
                           (hipStream_t)stream);
}

// =========================================================================
// LTX bandwidth-extension tail
// =========================================================================

namespace {

constexpr double kHannRolloff = 0.99;  // [LTX] hann_sinc_upsample
constexpr double kHannZeros = 6.0;

int check_mel_shape(int n_freqs, int filter_len, int hop, int n_mels) {
    if (n_freqs < 1 || filter_len < 1 || hop < 1 || n_mels < 1)
        return fail(AVAE_EINVAL, "mel: sizes must be >= 1");
    if (filter_len < hop || filter_len % 32 != 0 || n_freqs > 384 || filter_len > 4096)
        return fail(AVAE_ESHAPE, "mel: need filter_len >= hop, filter_len %% 32 == 0, "
                                 "n_freqs <= 384, filter_len <= 4096");
    return AVAE_OK;
}

std::vector<float> hann_taps(int ratio) {
    const int k = avae::design_hann_sinc(ratio, kHannRolloff, kHannZeros, nullptr);
    std::vector<double> d(k);
    avae::design_hann_sinc(ratio, kHannRolloff, kHannZeros, d.data());
    std::vector<float> f(k);
    for (int i = 0; i < k; ++i) f[i] = (float)d[i];  // the page rounds its taps to float32
    return f;
}

}  // namespace

extern "C" int avae_mel_stft(const float* x, float* out, int B, int T, const float* forward_basis,
                             int n_freqs, int filter_len, int hop, const float* mel_basis,
                             int n_mels, void* stream) {
    if (!x || !out || !forward_basis || !mel_basis)
        return fail(AVAE_EINVAL, "avae_mel_stft: null pointer");
    if (B < 1 || T < 1) return fail(AVAE_EINVAL, "avae_mel_stft: B, T must be >= 1");
    int rc = check_mel_shape(n_freqs, filter_len, hop, n_mels);
    if (rc) return rc;
    const int frames = T / hop;
    if (frames < 1) return fail(AVAE_ESHAPE, "avae_mel_stft: T < hop gives no frame");
    avae::prof_set_phase(avae::kPhaseNone);
    AVAE_TRY(avae::launch_mel_stft(x, out, B, T, frames, forward_basis, n_freqs, filter_len, hop,
                                   mel_basis, n_mels, (hipStream_t)stream),
             "avae_mel_stft launch");
    return AVAE_OK;
}

extern "C" int avae_hann_sinc_upsample(const float* x, float* y, int B, int T, int ratio,
                                       void* stream) {
    if (!x || !y) return fail(AVAE_EINVAL, "avae_hann_sinc_upsample: null pointer");
    if (B < 1 || T < 1 || ratio < 1 || ratio > 4)
        return fail(AVAE_EINVAL, "avae_hann_sinc_upsample: B, T >= 1 and ratio in [1, 4]");
    if ((long long)T * ratio > 0x7fffffffLL)
        return fail(AVAE_ESHAPE, "avae_hann_sinc_upsample: output too long");
    const std::vector<float> taps = hann_taps(ratio);
    avae::prof_set_phase(avae::kPhaseNone);
    AVAE_TRY(avae::launch_bwe_combine(x, nullptr, y, B, T, T, 0, T * ratio, ratio, taps.data(),
                                      (int)taps.size(), 0, (hipStream_t)stream),
             "avae_hann_sinc_upsample launch");
    return AVAE_OK;
}

struct avae_bwe {
    avae_bwe_config cfg;
    avae_decoder* gen = nullptr;
    void* blob = nullptr;  // forward_basis, mel_basis
    const float* basis = nullptr;
    const float* mel = nullptr;
    std::vector<float> taps;
    int device = 0;
};

namespace {

struct BwePlan {
    int frames, Tp;
    long long Lres;
    size_t mel_bytes, res_bytes, gen_bytes;
    size_t total() const { return mel_bytes + res_bytes + gen_bytes; }
};

bool bwe_plan(const avae_bwe* bwe, int B, int T, BwePlan* p) {
    const avae_bwe_config& c = bwe->cfg;
    p->frames = (T + c.hop - 1) / c.hop;
    p->Tp = p->frames * c.hop;
    p->Lres = (long long)p->Tp * c.ratio;
    if (p->Lres > 0x7fffffffLL) return false;
    p->mel_bytes = round_up((size_t)B * c.n_mels * p->frames * sizeof(float), 256);
    p->res_bytes = round_up((size_t)B * (size_t)p->Lres * sizeof(float), 256);
    p->gen_bytes = avae_decoder_workspace_bytes(bwe->gen, B, p->frames);
    return p->gen_bytes > 0;
}

int bwe_decode_impl(const avae_bwe* bwe, const float* low, int B, int T, float* out,
                    void* workspace, size_t ws_bytes, float* mel_out, float* resid_out,
                    hipStream_t s) {
    if (!bwe || !low || !out) return fail(AVAE_EINVAL, "avae_bwe_decode: null argument");
    if (B < 1 || T < 1) return fail(AVAE_EINVAL, "avae_bwe_decode: B, T must be >= 1");
    const avae_bwe_config& c = bwe->cfg;
    BwePlan p;
    if (!bwe_plan(bwe, B, T, &p) || (long long)T * c.ratio > 0x7fffffffLL)
        return fail(AVAE_ESHAPE, "avae_bwe_decode: length overflow");
    if (!workspace || ws_bytes < p.total())
        return fail(AVAE_EWORKSPACE, "avae_bwe_decode: workspace %zu bytes < %zu needed", ws_bytes,
                    p.total());
    char* ws = (char*)workspace;
    float* mel = (float*)ws;
    float* res = (float*)(ws + p.mel_bytes);
    void* gws = ws + p.mel_bytes + p.res_bytes;
    avae::prof_set_phase(avae::kPhaseNone);
    AVAE_TRY(avae::launch_mel_stft(low, mel, B, T, p.frames, bwe->basis, c.n_freqs, c.filter_len,
                                   c.hop, bwe->mel, c.n_mels, s),
             "bwe mel");
    if (mel_out)
        AVAE_TRY(hipMemcpyAsync(mel_out, mel, (size_t)B * c.n_mels * p.frames * sizeof(float),
                                hipMemcpyDeviceToDevice, s),
                 "trace copy");
    int rc = decode_impl(bwe->gen, mel, B, p.frames, res, gws, p.gen_bytes, nullptr, s);
    if (rc) return rc;
    if (resid_out)
        AVAE_TRY(hipMemcpyAsync(resid_out, res, (size_t)B * p.Lres * sizeof(float),
                                hipMemcpyDeviceToDevice, s),
                 "trace copy");
    avae::prof_set_phase(avae::kPhaseNone);
    AVAE_TRY(avae::launch_bwe_combine(low, res, out, B, T, p.Tp, (int)p.Lres, T * c.ratio, c.ratio,
                                      bwe->taps.data(), (int)bwe->taps.size(), 1, s),
             "bwe combine");
    return AVAE_OK;
}

}  // namespace

extern "C" int avae_bwe_create(const avae_bwe_config* cfg, const avae_bwe_weights* w,
                               avae_bwe** out) {
    if (!cfg || !w || !out) return fail(AVAE_EINVAL, "avae_bwe_create: null argument");
    *out = nullptr;
    const avae_bwe_config& c = *cfg;
    int rc = check_mel_shape(c.n_freqs, c.filter_len, c.hop, c.n_mels);
    if (rc) return rc;
    if (c.ratio < 1 || c.ratio > 4) return fail(AVAE_EINVAL, "avae_bwe_create: ratio in [1, 4]");
    if (!w->forward_basis || !w->mel_basis)
        return fail(AVAE_EINVAL, "avae_bwe_create: missing STFT or mel basis");
    if (c.gen.c_in != c.n_mels || c.gen.dec_in_ch != 0 || c.gen.has_latent_affine)
        return fail(AVAE_ESHAPE, "avae_bwe_create: the generator reads the n_mels log-mel directly");
    rc = check_config(&c.gen);
    if (rc) return rc;
    long long T[AVAE_MAX_STAGES + 1];
    if (stage_lengths(c.gen, 1, T) || T[c.gen.n_stages] != (long long)c.hop * c.ratio ||
        stage_lengths(c.gen, 2, T) || T[c.gen.n_stages] != 2LL * c.hop * c.ratio)
        return fail(AVAE_ESHAPE, "avae_bwe_create: the generator must give hop * ratio samples a frame");
    avae_bwe* b = new (std::nothrow) avae_bwe();
    if (!b) return fail(AVAE_ENOMEM, "avae_bwe_create: host allocation failed");
    b->cfg = c;
    b->taps = hann_taps(c.ratio);
    rc = avae_decoder_create(&c.gen, &w->gen, &b->gen);
    if (rc) {
        delete b;
        return rc;
    }
    const size_t nb = (size_t)2 * c.n_freqs * c.filter_len, nm = (size_t)c.n_mels * c.n_freqs;
    const size_t bb = round_up(nb * sizeof(float), 256);
    hipError_t e = hipGetDevice(&b->device);
    if (e == hipSuccess) e = hipMalloc(&b->blob, bb + nm * sizeof(float));
    if (e == hipSuccess) e = hipMemcpy(b->blob, w->forward_basis, nb * sizeof(float), hipMemcpyDefault);
    if (e == hipSuccess)
        e = hipMemcpy((char*)b->blob + bb, w->mel_basis, nm * sizeof(float), hipMemcpyDefault);
    if (e != hipSuccess) {
        if (b->blob) (void)hipFree(b->blob);
        avae_decoder_destroy(b->gen);
        delete b;
        return hip_fail(e, "avae_bwe_create: basis copy");
    }
    b->basis = (const float*)b->blob;
    b->mel = (const float*)((char*)b->blob + bb);
    *out = b;
    return AVAE_OK;
}

extern "C" void avae_bwe_destroy(avae_bwe* bwe) {
    if (!bwe) return;
    avae_decoder_destroy(bwe->gen);
    if (bwe->blob) {
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(bwe->device);
        (void)hipFree(bwe->blob);
        (void)hipSetDevice(cur);
    }
    delete bwe;
}

extern "C" size_t avae_bwe_workspace_bytes(const avae_bwe* bwe, int B, int T) {
    if (!bwe || B < 1 || T < 1) return 0;
    BwePlan p;
    if (!bwe_plan(bwe, B, T, &p)) return 0;
    return p.total();
}

extern "C" int avae_bwe_decode(const avae_bwe* bwe, const float* low, int B, int T, float* out,
                               void* workspace, size_t ws_bytes, void* stream) {
    return bwe_decode_impl(bwe, low, B, T, out, workspace, ws_bytes, nullptr, nullptr,
                           (hipStream_t)stream);
}

extern "C" int avae_bwe_decode_traced(const avae_bwe* bwe, const float* low, int B, int T,
                                      float* out, void* workspace, size_t ws_bytes,
                                      float* mel_out, float* resid_out, void* stream) {
    return bwe_decode_impl(bwe, low, B, T, out, workspace, ws_bytes, mel_out, resid_out,
                           (hipStream_t)stream);
}
