// Launch profiler: while a profiled region is open (avae_profile_begin ..
// avae_profile_end), every kernel launch is bracketed by two hipEvents
// recorded on its stream, and each launch is tagged with its kernel name, the
// decode phase it belongs to, and its algorithmic flops and bytes.  The
// events are created when the region opens, so the compute calls still
// allocate nothing on the device.  The region is process-wide: one at a
// time, from one host thread.
//
// Phases follow the audio decoder's own phase report ([H3] = docs.rs page of
// cortiq_engine/audiovae.rs, AVAE_TIME / avae_time_report): dec_in,
// conv_pre, upsamples, resblocks, act_post, conv_post.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "avae.h"
#include "avae_internal.h"

namespace avae {
namespace {

struct Rec {
    const char* name;
    int phase;
    double flops, bytes;
    size_t ev;
};

struct Agg {
    std::string name;
    long long launches = 0;
    double ms = 0, flops = 0, bytes = 0;
};

std::mutex g_mu;
bool g_on = false;
bool g_pending = false;
int g_phase = -1;
size_t g_next = 0;
long long g_dropped = 0;
std::vector<hipEvent_t> g_events;
std::vector<Rec> g_recs;
std::vector<Agg> g_aggs;
double g_phase_ms[6] = {0, 0, 0, 0, 0, 0};

}  // namespace

void prof_set_phase(int phase) { g_phase = phase; }

void prof_pre(hipStream_t s) {
    if (!g_on) return;
    g_pending = false;
    if (g_next + 2 > g_events.size()) {
        ++g_dropped;
        return;
    }
    if (hipEventRecord(g_events[g_next], s) == hipSuccess) g_pending = true;
}

void prof_post(hipStream_t s, const char* name, double flops, double bytes) {
    if (!g_on || !g_pending) return;
    g_pending = false;
    if (hipEventRecord(g_events[g_next + 1], s) != hipSuccess) return;
    g_recs.push_back(Rec{name, g_phase, flops, bytes, g_next});
    g_next += 2;
}

}  // namespace avae

using namespace avae;

extern "C" int avae_profile_begin(int max_launches) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (max_launches < 1) return AVAE_EINVAL;
    const size_t need = 2 * (size_t)max_launches;
    while (g_events.size() < need) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return AVAE_EHIP;
        g_events.push_back(e);
    }
    g_recs.clear();
    g_recs.reserve(max_launches);
    g_aggs.clear();
    g_next = 0;
    g_dropped = 0;
    g_phase = -1;
    std::memset(g_phase_ms, 0, sizeof(g_phase_ms));
    g_on = true;
    return AVAE_OK;
}

extern "C" int avae_profile_end(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return AVAE_EINVAL;
    g_on = false;
    if (!g_recs.empty() && hipEventSynchronize(g_events[g_recs.back().ev + 1]) != hipSuccess)
        return AVAE_EHIP;
    std::map<std::string, size_t> idx;
    for (const Rec& r : g_recs) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_events[r.ev], g_events[r.ev + 1]) != hipSuccess)
            return AVAE_EHIP;
        auto it = idx.find(r.name);
        if (it == idx.end()) {
            it = idx.emplace(r.name, g_aggs.size()).first;
            g_aggs.push_back(Agg{r.name});
        }
        Agg& a = g_aggs[it->second];
        a.launches += 1;
        a.ms += ms;
        a.flops += r.flops;
        a.bytes += r.bytes;
        if (r.phase >= 0 && r.phase < 6) g_phase_ms[r.phase] += ms;
    }
    return g_dropped ? AVAE_ESHAPE : AVAE_OK;
}

extern "C" int avae_profile_count(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    return (int)g_aggs.size();
}

extern "C" int avae_profile_entry(int i, char* name, int name_len, long long* launches,
                                  double* total_ms, double* flops, double* bytes) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (i < 0 || i >= (int)g_aggs.size()) return AVAE_EINVAL;
    const Agg& a = g_aggs[i];
    if (name && name_len > 0) {
        std::strncpy(name, a.name.c_str(), name_len - 1);
        name[name_len - 1] = 0;
    }
    if (launches) *launches = a.launches;
    if (total_ms) *total_ms = a.ms;
    if (flops) *flops = a.flops;
    if (bytes) *bytes = a.bytes;
    return AVAE_OK;
}

extern "C" int avae_profile_phases(double* ms6) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!ms6) return AVAE_EINVAL;
    for (int i = 0; i < 6; ++i) ms6[i] = g_phase_ms[i];
    return AVAE_OK;
}
