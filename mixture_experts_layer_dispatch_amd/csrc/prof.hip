// Per-kernel timing for measurement tools: while enabled, every launch made by
// the library is bracketed by two HIP events recorded on the launch's own stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"

namespace moe {

std::atomic<int> g_prof_on{0};

namespace {
struct Rec {
    const char *name;
    hipEvent_t a, b;
};
std::mutex g_mu;
std::vector<Rec> g_recs;
thread_local hipEvent_t t_begin = nullptr;
}  // namespace

void prof_begin(hipStream_t st) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return;
    hipEvent_t a;
    if (hipEventCreate(&a) != hipSuccess) { t_begin = nullptr; return; }
    (void)hipEventRecord(a, st);
    t_begin = a;
}

void prof_end(const char *name, hipStream_t st) {
    if (!g_prof_on.load(std::memory_order_relaxed) || !t_begin) return;
    hipEvent_t b;
    if (hipEventCreate(&b) != hipSuccess) return;
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_mu);
    g_recs.push_back({name, t_begin, b});
    t_begin = nullptr;
}

int prof_report(char *buf, size_t n) {
    std::vector<Rec> recs;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        recs.swap(g_recs);
    }
    std::map<std::string, std::pair<long, double>> acc;
    std::vector<std::string> order;
    for (auto &r : recs) {
        (void)hipEventSynchronize(r.b);
        float ms = 0.0f;
        (void)hipEventElapsedTime(&ms, r.a, r.b);
        auto it = acc.find(r.name);
        if (it == acc.end()) {
            order.push_back(r.name);
            acc[r.name] = {1, ms};
        } else {
            it->second.first += 1;
            it->second.second += ms;
        }
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    std::string out;
    for (auto &nm : order) {
        char line[256];
        std::snprintf(line, sizeof(line), "%s %ld %.6f\n", nm.c_str(), acc[nm].first, acc[nm].second);
        out += line;
    }
    if (buf && n) {
        size_t m = out.size() < n - 1 ? out.size() : n - 1;
        out.copy(buf, m);
        buf[m] = 0;
        return (int)m;
    }
    return (int)out.size();
}

}  // namespace moe
