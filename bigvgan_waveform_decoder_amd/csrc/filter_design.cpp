// Host float64 design of the Kaiser-windowed sinc resampling filter.
//
// [H3] = docs.rs page of cortiq_engine/audiovae.rs, items kaiser_sinc,
// bessel_i0, sinc: lowpass at `cutoff` cycles/sample with transition
// `half_width`; attenuation A = 2.285 (n/2 - 1) pi (4 half_width) + 7.95 and
// Kaiser's beta for it; taps at the half-integers of an even-length filter;
// normalised to unit sum.
#include <cmath>

#include "avae_internal.h"

namespace avae {
namespace {

// I0 by its power series: sum_k ((x/2)^k / k!)^2, summed until the terms
// stop mattering in float64.
double i0_series(double x) {
    const double h = 0.5 * x;
    double term = 1.0, sum = 1.0;
    for (int k = 1; k < 64; ++k) {
        const double f = h / k;
        term *= f * f;
        sum += term;
        if (term <= sum * 1e-18) break;
    }
    return sum;
}

double kaiser_beta_for(double atten) {
    if (atten > 50.0) return 0.1102 * (atten - 8.7);
    if (atten >= 21.0) return 0.5842 * std::pow(atten - 21.0, 0.4) + 0.07886 * (atten - 21.0);
    return 0.0;
}

}  // namespace

void design_kaiser_sinc(double cutoff, double half_width, int taps, double* out) {
    const double pi = 3.14159265358979323846;
    const int half = taps / 2;
    const double atten = 2.285 * (half - 1) * pi * (4.0 * half_width) + 7.95;
    const double beta = kaiser_beta_for(atten);
    const double i0b = i0_series(beta);
    double total = 0.0;
    for (int i = 0; i < taps; ++i) {
        const double r = 2.0 * i / (taps - 1) - 1.0;
        const double win = i0_series(beta * std::sqrt(std::fmax(0.0, 1.0 - r * r))) / i0b;
        const double t = (i - half) + 0.5;  // half-integer tap position
        const double arg = 2.0 * cutoff * t;
        const double sinc = (arg == 0.0) ? 1.0 : std::sin(pi * arg) / (pi * arg);
        out[i] = 2.0 * cutoff * win * sinc;
        total += out[i];
    }
    for (int i = 0; i < taps; ++i) out[i] /= total;
}

// The x`ratio` Hann-windowed sinc interpolator of the LTX bandwidth
// extension ([LTX] hann_sinc_upsample): w = ceil(lpw / rolloff) input samples
// each side, k = 2 w ratio + 1 taps; tap i sits at t = (i/ratio - w) rolloff
// and is sinc(t) cos^2(pi clamp(t, -lpw, lpw) / (2 lpw)) rolloff / ratio.
// Returns k (out must hold it).
int design_hann_sinc(int ratio, double rolloff, double lpw, double* out) {
    const double pi = 3.14159265358979323846;
    const int w = (int)std::ceil(lpw / rolloff);
    const int k = 2 * w * ratio + 1;
    if (!out) return k;
    for (int i = 0; i < k; ++i) {
        const double t = ((double)i / ratio - w) * rolloff;
        const double tc = std::fmin(std::fmax(t, -lpw), lpw);
        const double c = std::cos(tc * pi / lpw / 2.0);
        const double sinc = (t == 0.0) ? 1.0 : std::sin(pi * t) / (pi * t);
        out[i] = sinc * c * c * rolloff / ratio;
    }
    return k;
}

}  // namespace avae
