// Per-kernel timing: when enabled, every kernel the library launches carries a
// start/stop event pair stamped by its own dispatch (hipExtLaunchKernel), and
// the elapsed times are accumulated per kernel name when read.  Off by
// default; meant for eager runs (not for graph capture).
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"

namespace moe {

namespace {

struct Pending {
    int id;
    hipEvent_t start, stop;
};

struct Stat {
    std::string name;
    long long count = 0;
    double total_ms = 0.0;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Stat> g_stats;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

int stat_id(const char *name) {
    for (size_t i = 0; i < g_stats.size(); ++i)
        if (g_stats[i].name == name) return (int)i;
    g_stats.push_back(Stat{name});
    return (int)g_stats.size() - 1;
}

}  // namespace

bool prof_events(const char *name, hipEvent_t *start, hipEvent_t *stop) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return false;
    hipEvent_t a = take_event();
    hipEvent_t b = a ? take_event() : nullptr;
    if (!a || !b) {
        if (a) g_pool.push_back(a);
        return false;
    }
    g_pending.push_back(Pending{stat_id(name), a, b});
    *start = a;
    *stop = b;
    return true;
}

}  // namespace moe

extern "C" {

moe_status moe_profile_enable(int32_t on) {
    std::lock_guard<std::mutex> lk(moe::g_mu);
    moe::g_on = on != 0;
    return MOE_OK;
}

moe_status moe_profile_reset(void) {
    std::lock_guard<std::mutex> lk(moe::g_mu);
    for (auto &p : moe::g_pending) {
        (void)hipEventSynchronize(p.stop);
        moe::g_pool.push_back(p.start);
        moe::g_pool.push_back(p.stop);
    }
    moe::g_pending.clear();
    moe::g_stats.clear();
    return MOE_OK;
}

moe_status moe_profile_read(int32_t index, const char **name, int64_t *count, double *total_ms) {
    std::lock_guard<std::mutex> lk(moe::g_mu);
    for (auto &p : moe::g_pending) {
        float ms = 0.f;
        if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
            moe::g_stats[p.id].count += 1;
            moe::g_stats[p.id].total_ms += ms;
        }
        moe::g_pool.push_back(p.start);
        moe::g_pool.push_back(p.stop);
    }
    moe::g_pending.clear();
    if (index < 0 || index >= (int)moe::g_stats.size()) return MOE_ERR_INVALID_ARG;
    if (name) *name = moe::g_stats[index].name.c_str();
    if (count) *count = moe::g_stats[index].count;
    if (total_ms) *total_ms = moe::g_stats[index].total_ms;
    return MOE_OK;
}

}  // extern "C"
