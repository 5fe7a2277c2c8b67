// Host-side planning arithmetic of the C-ABI: stage lengths, workspace slot
// sizes, the receptive-field reach and the tile grid of the streaming
// decode.  Plain C++ (no HIP), so that it also builds into a host-only check
// program under the address and undefined-behaviour sanitizers.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstddef>

#include "avae.h"

namespace avae {
namespace plan {

inline size_t round_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

// Bytes of a float32 tensor [a, b, c] (non-negative sizes), rounded up to
// 256 bytes; 0 when the size exceeds 2^60 bytes (no wrap-around).
inline size_t tensor_bytes(long long a, long long b, long long c) {
    if (a < 0 || b < 0 || c < 0) return 0;
    const long double v = (long double)a * (long double)b * (long double)c * 4.0L;
    if (v > (long double)(1ULL << 60)) return 0;
    return round_up((size_t)a * (size_t)b * (size_t)c * sizeof(float), 256);
}

// Per-stage lengths for `frames` frames: T[0] = frames, T[i+1] after stage i
// ([H3] ConvT1d::apply: Tout = (Tin - 1) s + k - 2 pad, pad = (k - s) / 2).
// Returns -1 if a length leaves [1, 2^31).
inline int stage_lengths(const avae_config& c, int frames, long long* T) {
    T[0] = frames;
    if (frames < 1) return -1;
    for (int i = 0; i < c.n_stages; ++i) {
        const int p = (c.up_k[i] - c.rates[i]) / 2;
        T[i + 1] = (T[i] - 1) * c.rates[i] + c.up_k[i] - 2LL * p;
        if (T[i + 1] < 1 || T[i + 1] > 0x7fffffffLL) return -1;
    }
    return 0;
}

// Overlap-save Conv1d (fftconv.hip): 256-point transforms, 128 frequency
// slots.  A row of T outputs is cut into nb blocks of L = 256 - (K-1) d; the
// B nb columns are split into ntiles tiles of 16 NJ columns (NJ <= 8), NP
// columns in all.
constexpr int kFftN = 256;
constexpr int kFftSlots = 128;

struct FftShape {
    int L = 0, nb = 0, NB = 0, NJ = 0, ntiles = 0, NP = 0;
};

inline bool fft_supported(int Cin, int Cout, int K, int d) {
    return Cin >= 16 && Cin % 16 == 0 && Cout >= 16 && Cout % 16 == 0 && K >= 1 && K % 2 == 1 &&
           d >= 1 && (long long)(K - 1) * d <= kFftN / 2;
}

// B, T >= 1 and a supported (K, d); ntiles = 0 if B nb overflows an int.
inline FftShape fft_shape(int B, int T, int K, int d) {
    FftShape s;
    s.L = kFftN - (K - 1) * d;
    s.nb = (int)(((long long)T + s.L - 1) / s.L);
    const long long nbt = (long long)B * s.nb;
    if (nbt > 0x3fffffffLL) return s;
    s.NB = (int)nbt;
    s.ntiles = (s.NB + 127) / 128;
    const int per = (s.NB + s.ntiles - 1) / s.ntiles;
    s.NJ = (per + 15) / 16;
    s.NP = s.ntiles * 16 * s.NJ;
    return s;
}

// Bytes of one spectrum (128 slots x C rows x NP complex float columns),
// rounded up to 256; 0 on overflow.
inline size_t fft_spectrum_bytes(int B, int C, int T, int K, int d) {
    const FftShape s = fft_shape(B, T, K, d);
    if (s.ntiles == 0) return 0;
    return tensor_bytes((long long)kFftSlots * 2, C, s.NP);
}

// The decoders' AMP convolutions whose frequency-domain weights are kept:
// 7 or more taps from 48 channels up (the transform form needs ~2
// multiply-adds per output and channel pair against K, and with the
// activation inside the forward transforms it also saves the activation's
// own pass), and 3 taps from 192 to 512 channels (there the saving is 3
// against 2 and the fused activation's; wider, the frequency-domain weights
// of one convolution pass 270 MB).
inline bool fft_amp_pack(int C, int K, int d) {
    if (!fft_supported(C, C, K, d)) return false;
    return K >= 7 ? C >= 48 : (K >= 3 && C >= 192 && C <= 512);
}

// Whether a kept convolution runs in the frequency domain for B rows of T
// samples: always with 7 or more taps; with 3 only when there are at least
// 64 columns (blocks x rows), below which the product streams its weights
// faster than it can use them and the direct form wins.
inline bool fft_amp_use(int B, int C, int T, int K, int d) {
    if (!fft_amp_pack(C, K, d)) return false;
    if (K >= 7) return true;
    const FftShape s = fft_shape(B, T, K, d);
    return s.ntiles > 0 && s.NB >= 64;
}

// Bytes of one decode workspace slot: the largest activation of the decode
// (B passes) and the largest spectrum of a frequency-domain AMP convolution,
// rounded up to 256 bytes; 0 if it does not fit a size_t.
inline size_t decode_slot_bytes(const avae_config& c, int B, const long long* T) {
    size_t m = 0;
    bool over = false;
    auto keep = [&](size_t b) {
        if (b == 0) over = true;
        if (b > m) m = b;
    };
    auto upd = [&](long long ch, long long t) { keep(tensor_bytes(B, ch, t)); };
    upd(c.c_in, T[0]);
    if (c.dec_in_ch) upd(c.dec_in_ch, T[0]);
    upd(c.ch[0], T[0]);
    for (int i = 0; i < c.n_stages; ++i) {
        const int co = c.ch[i + 1];
        upd(co, T[i + 1]);
        for (int j = 0; j < c.n_kernels; ++j) {
            const int K = c.rb_k[j];
            const int t = (int)T[i + 1];
            if (fft_amp_use(B, co, t, K, 1)) keep(fft_spectrum_bytes(B, co, t, K, 1));
            for (int q = 0; q < c.n_dil; ++q)
                if (fft_amp_use(B, co, t, K, c.rb_d[j][q]))
                    keep(fft_spectrum_bytes(B, co, t, K, c.rb_d[j][q]));
        }
    }
    return over ? 0 : m;
}

// Receptive-field reach in latent frames (per layer, in that layer's input
// samples: Activation1d +-5, a "same" conv (k-1)d/2, a ConvTranspose1d
// ceil(k/s)+1; each divided by the upsampling already applied), rounded up,
// plus one frame of slack.
inline int reach_frames(const avae_config& c) {
    double reach = (c.k_pre - 1) / 2.0;
    double rate = 1.0;
    for (int i = 0; i < c.n_stages; ++i) {
        reach += ((c.up_k[i] + c.rates[i] - 1) / c.rates[i] + 1) / rate;
        rate *= c.rates[i];
        double mrf = 0.0;
        for (int j = 0; j < c.n_kernels; ++j) {
            double r = 0.0;
            for (int q = 0; q < c.n_dil; ++q)
                r += 5.0 + (c.rb_k[j] - 1) * c.rb_d[j][q] / 2.0 + 5.0 + (c.rb_k[j] - 1) / 2.0;
            mrf = r > mrf ? r : mrf;
        }
        reach += mrf / rate;
    }
    reach += (5.0 + (c.k_post - 1) / 2.0) / rate;
    return (int)std::ceil(reach) + 1;
}

inline long long hop_of(const avae_config& c) {
    long long h = 1;
    for (int i = 0; i < c.n_stages; ++i) h *= c.rates[i];
    return h;
}

// Tiles decoded together in one batched pass of the streaming decode (their
// crops stacked along the batch axis); the streaming workspace covers this
// many tiles.
constexpr int kTileBatch = 4;

// The streaming decode's tiles.  Tile i keeps frames [i tf, min((i+1) tf,
// frames)).  Its crop: the first tile [0, tf + halo), the last tile the
// final tf + halo frames, an inner tile tf + 2 halo frames centred on it
// (slid inward when the halo reaches past an end), every length clipped to
// the sequence; each kept frame has at least `halo` frames of context on
// every side that is not a true end.  So there are at most two crop lengths.
struct TileGrid {
    int frames = 0, tf = 0, halo = 0, ntiles = 0, len_edge = 0, len_mid = 0;

    void crop(int i, int* c0, int* len) const {
        if (ntiles == 1) {
            *c0 = 0;
            *len = frames;
        } else if (i == 0) {
            *c0 = 0;
            *len = len_edge;
        } else if (i == ntiles - 1) {
            *c0 = frames - len_edge;
            *len = len_edge;
        } else {
            *c0 = std::max(0, std::min(i * tf - halo, frames - len_mid));
            *len = len_mid;
        }
    }
    void kept(int i, int* f0, int* f1) const {
        *f0 = i * tf;
        *f1 = std::min(*f0 + tf, frames);
    }
};

// frames >= 1, tile_frames >= 1, halo >= 0.
inline TileGrid tile_grid(int frames, int tile_frames, int halo) {
    TileGrid g;
    g.frames = frames;
    g.tf = tile_frames < frames ? tile_frames : frames;
    g.halo = halo;
    g.ntiles = (int)(((long long)frames + g.tf - 1) / g.tf);
    g.len_edge = (int)std::min<long long>((long long)g.tf + halo, frames);
    g.len_mid = (int)std::min<long long>((long long)g.tf + 2LL * halo, frames);
    return g;
}

// Calls fn(tiles, n, len) for each batched pass: first the end tiles (and a
// single whole-sequence tile), then the inner ones, in tile order, up to
// kTileBatch tiles of one crop length per call.  Stops at, and returns, the
// first non-zero return of fn.
template <class F>
int for_each_tile_group(const TileGrid& g, F&& fn) {
    for (int pass = 0; pass < 2; ++pass) {
        int group[kTileBatch];
        int ng = 0, glen = 0;
        for (int i = 0; i < g.ntiles; ++i) {
            const bool end_tile = (i == 0 || i == g.ntiles - 1);
            if (end_tile != (pass == 0)) continue;
            int c0, len;
            g.crop(i, &c0, &len);
            if (ng == kTileBatch || (ng > 0 && len != glen)) {
                const int rc = fn(group, ng, glen);
                if (rc) return rc;
                ng = 0;
            }
            glen = len;
            group[ng++] = i;
        }
        if (ng > 0) {
            const int rc = fn(group, ng, glen);
            if (rc) return rc;
        }
    }
    return 0;
}

// Workspace of the streaming decode: latent crops, tile waveforms and the
// decode workspace (n_slots slots) for kTileBatch tiles of B passes.
struct StreamBytes {
    size_t crop_bytes = 0, wave_bytes = 0, dec_bytes = 0;
    size_t total() const { return crop_bytes + wave_bytes + dec_bytes; }
};

inline bool stream_bytes(const avae_config& c, int n_slots, int B, int tile_frames, int halo,
                         StreamBytes* p) {
    const long long cf = (long long)tile_frames + 2LL * halo;
    if (B < 1 || tile_frames < 1 || halo < 0 || cf > 0x3fffffffLL) return false;
    if ((long long)B * kTileBatch > 0x7fffffffLL / 2) return false;
    const int rows = B * kTileBatch;
    long long T[AVAE_MAX_STAGES + 1];
    if (stage_lengths(c, (int)cf, T)) return false;
    const size_t slot = decode_slot_bytes(c, rows, T);
    if (slot == 0) return false;
    p->crop_bytes = tensor_bytes(rows, c.c_in, cf);
    p->wave_bytes = tensor_bytes(rows, 1, T[c.n_stages]);
    p->dec_bytes = (size_t)n_slots * slot;
    return p->crop_bytes > 0 && p->wave_bytes > 0;
}

}  // namespace plan
}  // namespace avae
