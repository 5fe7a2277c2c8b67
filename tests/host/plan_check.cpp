// Host-only check of the C-ABI's planning arithmetic (csrc/plan.h): decoder
// stage lengths and workspace sizes, the receptive-field reach and the tile
// grid of the streaming decode.  Built and run by tests/test_host_sanitized.py
// with the address and undefined-behaviour sanitizers; prints "plan_check ok"
// and exits 0 when every check holds.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "plan.h"

using namespace avae::plan;

static int g_fail = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);             \
            std::fprintf(stderr, "\n");                    \
            if (++g_fail > 20) std::exit(1);               \
        }                                                  \
    } while (0)

static avae_config bigvgan(int c_in, int c0, std::vector<int> rates, std::vector<int> up_k) {
    avae_config c{};
    c.c_in = c_in;
    c.k_pre = c.k_post = 7;
    c.n_stages = (int)rates.size();
    c.ch[0] = c0;
    for (int i = 0; i < c.n_stages; ++i) {
        c.rates[i] = rates[i];
        c.up_k[i] = up_k[i];
        c.ch[i + 1] = c.ch[i] / 2;
    }
    c.n_kernels = 3;
    const int ks[3] = {3, 7, 11};
    c.n_dil = 3;
    for (int j = 0; j < 3; ++j) {
        c.rb_k[j] = ks[j];
        c.rb_d[j][0] = 1;
        c.rb_d[j][1] = 3;
        c.rb_d[j][2] = 5;
    }
    return c;
}

// Every frame kept exactly once, kept frames inside their crop, crops inside
// the sequence with enough context, at most two crop lengths, every tile in
// exactly one batched group of equal crop lengths and at most kTileBatch.
static void check_grid(int frames, int tile, int halo) {
    const TileGrid g = tile_grid(frames, tile, halo);
    CHECK(g.tf >= 1 && g.tf <= frames, "tf %d frames %d", g.tf, frames);
    std::vector<int> kept(frames, 0);
    std::set<int> lens;
    for (int i = 0; i < g.ntiles; ++i) {
        int c0, len, f0, f1;
        g.crop(i, &c0, &len);
        g.kept(i, &f0, &f1);
        CHECK(f0 < f1, "empty tile %d", i);
        CHECK(c0 >= 0 && len >= 1 && c0 + len <= frames, "crop [%d,+%d) of %d", c0, len, frames);
        CHECK(c0 <= f0 && f1 <= c0 + len, "tile [%d,%d) outside crop [%d,+%d)", f0, f1, c0, len);
        const int left = f0 - c0, right = c0 + len - f1;
        CHECK(left >= halo || c0 == 0, "left context %d < halo %d", left, halo);
        CHECK(right >= halo || c0 + len == frames, "right context %d < halo %d", right, halo);
        for (int f = f0; f < f1; ++f) kept[f]++;
        lens.insert(len);
    }
    for (int f = 0; f < frames; ++f) CHECK(kept[f] == 1, "frame %d kept %d times", f, kept[f]);
    CHECK(lens.size() <= 2, "%zu crop lengths", lens.size());
    std::vector<int> seen(g.ntiles, 0);
    const int rc = for_each_tile_group(g, [&](const int* t, int n, int len) -> int {
        CHECK(n >= 1 && n <= kTileBatch, "group of %d", n);
        for (int k = 0; k < n; ++k) {
            CHECK(t[k] >= 0 && t[k] < g.ntiles, "tile index %d", t[k]);
            int c0, l;
            g.crop(t[k], &c0, &l);
            CHECK(l == len, "group length %d vs crop %d", len, l);
            seen[t[k]]++;
        }
        return 0;
    });
    CHECK(rc == 0, "rc %d", rc);
    for (int i = 0; i < g.ntiles; ++i) CHECK(seen[i] == 1, "tile %d decoded %d times", i, seen[i]);
}

int main() {
    // H3-shaped and LTX-shaped decoders: frames x hop output, the reach.
    const avae_config h3 = bigvgan(32, 1536, {5, 5, 2, 2, 2, 2, 2}, {11, 11, 4, 4, 4, 4, 4});
    const avae_config ltx = bigvgan(64, 1024, {5, 2, 2, 2, 2, 2}, {11, 4, 4, 4, 4, 4});
    long long T[AVAE_MAX_STAGES + 1];
    for (int f : {1, 2, 7, 400, 2000, 100000}) {
        CHECK(stage_lengths(h3, f, T) == 0 && T[7] == 800LL * f, "h3 %d -> %lld", f, T[7]);
        CHECK(stage_lengths(ltx, f, T) == 0 && T[6] == 160LL * f, "ltx %d -> %lld", f, T[6]);
    }
    CHECK(hop_of(h3) == 800 && hop_of(ltx) == 160, "hops");
    CHECK(reach_frames(h3) == 35, "h3 reach %d", reach_frames(h3));
    CHECK(reach_frames(ltx) == 45, "ltx reach %d", reach_frames(ltx));
    // lengths past 2^31 are rejected, not wrapped
    CHECK(stage_lengths(h3, 3000000, T) != 0, "h3 overflow accepted");
    CHECK(stage_lengths(h3, 0, T) != 0, "zero frames accepted");
    // workspace slots, workload 4: the largest activation is 30.72 MB ([2, 24,
    // 160000] and its equals), the largest spectrum 44.04 MB: the 384-channel
    // stage at 11 taps, dilation 5 (blocks of 206 outputs: 49 per row, 98
    // columns padded to 112) and the 192-channel stage (98 per row, 196
    // columns in two tiles of 112), 128 slots of complex floats.
    CHECK(stage_lengths(h3, 400, T) == 0, "h3 400");
    CHECK(decode_slot_bytes(h3, 2, T) == 128ULL * 2 * 384 * 112 * 4,
          "h3 slot %zu", decode_slot_bytes(h3, 2, T));
    {
        const FftShape a = fft_shape(2, 10000, 11, 5), b = fft_shape(2, 20000, 11, 5);
        CHECK(a.L == 206 && a.nb == 49 && a.NB == 98 && a.ntiles == 1 && a.NJ == 7 && a.NP == 112,
              "fft shape 384");
        CHECK(b.nb == 98 && b.NB == 196 && b.ntiles == 2 && b.NJ == 7 && b.NP == 224,
              "fft shape 192");
        CHECK(fft_amp_pack(384, 11, 5) && fft_amp_pack(192, 7, 1) && fft_amp_pack(96, 11, 5) &&
                  fft_amp_pack(48, 11, 5) && !fft_amp_pack(32, 11, 5) &&
                  fft_amp_pack(384, 3, 1) && !fft_amp_pack(768, 3, 1) &&
                  !fft_amp_pack(96, 3, 1) && !fft_amp_pack(100, 7, 1) &&
                  !fft_amp_pack(384, 11, 13),
              "fft selection");
        // 3 taps: the 384-channel stage (2 x 40 columns) yes, 2 x 8 columns no
        CHECK(fft_amp_use(2, 384, 10000, 3, 1) && !fft_amp_use(2, 384, 2000, 3, 1) &&
                  fft_amp_use(2, 384, 2000, 11, 5),
              "fft use");
    }
    // the column plan over many sizes: every column covered, at most 8 MFMA
    // tiles of 16 per workgroup, fewer than 16 padding columns per tile
    for (int B : {1, 2, 3, 8})
        for (int T = 1; T <= 70000; T = T * 3 + 1)
            for (int K : {3, 7, 11})
                for (int d : {1, 3, 5, 12}) {
                    if (!fft_supported(16, 64, K, d)) continue;
                    const FftShape f = fft_shape(B, T, K, d);
                    CHECK(f.ntiles >= 1 && f.NJ >= 1 && f.NJ <= 8 && f.NP >= f.NB &&
                              (long long)f.nb * f.L >= T && (long long)(f.nb - 1) * f.L < T &&
                              f.NP - f.NB < 16 * f.ntiles,
                          "fft shape B=%d T=%d K=%d d=%d", B, T, K, d);
                    CHECK(fft_spectrum_bytes(B, 64, T, K, d) == 128ULL * 2 * 64 * f.NP * 4,
                          "fft spectrum bytes");
                }
    // sizes that would wrap a 64-bit product give 0
    CHECK(tensor_bytes(0x7fffffff, 0x7fffffff, 0x7fffffff) == 0, "tensor_bytes wrap");
    CHECK(tensor_bytes(1, 1, 1) == 256, "tensor_bytes small");
    CHECK(tensor_bytes(-1, 1, 1) == 0, "tensor_bytes negative");
    CHECK(decode_slot_bytes(h3, 0x7fffffff, T) == 0 || decode_slot_bytes(h3, 0x7fffffff, T) >
          (size_t)0x7fffffff, "huge batch");
    StreamBytes sb;
    CHECK(stream_bytes(h3, 13, 2, 100, 35, &sb) && sb.total() > 0, "h3 streaming bytes");
    CHECK(!stream_bytes(h3, 13, 2, 0x3fffffff, 35, &sb), "huge tile accepted");
    CHECK(!stream_bytes(h3, 13, 0x7fffffff, 100, 35, &sb), "huge batch accepted");
    CHECK(!stream_bytes(h3, 13, 2, 100, -1, &sb), "negative halo accepted");
    // the tile grid, exhaustively over small sizes, then a few long ones
    for (int frames = 1; frames <= 160; ++frames)
        for (int tile = 1; tile <= frames + 3; ++tile)
            for (int halo : {0, 1, 2, 5, 17, 35, 45, 200}) check_grid(frames, tile, halo);
    for (int frames : {400, 1999, 2000, 100003})
        for (int tile : {1, 25, 100, 399, 4096})
            for (int halo : {0, 35, 45}) check_grid(frames, tile, halo);
    if (g_fail) {
        std::fprintf(stderr, "plan_check: %d failures\n", g_fail);
        return 1;
    }
    std::printf("plan_check ok\n");
    return 0;
}
