// Status strings, HIP error plumbing and the optional kernel-timing hooks of
// the CSA2 C ABI (include/csa2.h).
#include <string.h>

#include <vector>

#include "internal.hpp"

namespace csa2 {

static thread_local int g_last_hip = 0;

void set_last_hip_error(hipError_t e) { g_last_hip = (int)e; }

int check_launch() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        set_last_hip_error(e);
        return CSA2_ERR_HIP;
    }
    return CSA2_OK;
}

// ------------------------------------------------------------ profiling

namespace {
struct Rec {
    const char* name;
    hipEvent_t a, b;
};
struct Prof {
    bool on = false;
    std::vector<Rec> pending;       // recorded, not yet read
    std::vector<hipEvent_t> pool;   // spare events
    struct Sum {
        const char* name;
        int n;
        double ms;
    };
    std::vector<Sum> sums;
    hipEvent_t take() {
        if (!pool.empty()) {
            hipEvent_t e = pool.back();
            pool.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
    void drain() {
        for (auto& r : pending) {
            float ms = 0.f;
            if (r.a && r.b && hipEventSynchronize(r.b) == hipSuccess &&
                hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
                bool found = false;
                for (auto& s : sums)
                    if (strcmp(s.name, r.name) == 0) { s.n++; s.ms += ms; found = true; }
                if (!found) sums.push_back({r.name, 1, (double)ms});
            }
            if (r.a) pool.push_back(r.a);
            if (r.b) pool.push_back(r.b);
        }
        pending.clear();
    }
};
Prof g_prof;
}  // namespace

void prof_begin(const char* name, hipStream_t s) {
    if (!g_prof.on) return;
    Rec r{name, g_prof.take(), nullptr};
    if (r.a) (void)hipEventRecord(r.a, s);
    g_prof.pending.push_back(r);
}

void prof_end(hipStream_t s) {
    if (!g_prof.on || g_prof.pending.empty()) return;
    Rec& r = g_prof.pending.back();
    r.b = g_prof.take();
    if (r.b) (void)hipEventRecord(r.b, s);
}

}  // namespace csa2

extern "C" {

const char* csa2_status_str(int status) {
    switch (status) {
        case CSA2_OK: return "CSA2_OK";
        case CSA2_ERR_NULL: return "CSA2_ERR_NULL: a required pointer is NULL";
        case CSA2_ERR_SHAPE: return "CSA2_ERR_SHAPE: a size is negative or inconsistent";
        case CSA2_ERR_UNSUPPORTED: return "CSA2_ERR_UNSUPPORTED: shape outside the kernels' range";
        case CSA2_ERR_WORKSPACE: return "CSA2_ERR_WORKSPACE: workspace too small";
        case CSA2_ERR_HIP: return "CSA2_ERR_HIP: a HIP launch failed";
        default: return "CSA2: unknown status";
    }
}

int csa2_last_hip_error(void) { return csa2::g_last_hip; }

int csa2_profile_enable(int enable) {
    csa2::g_prof.on = enable != 0;
    return CSA2_OK;
}

int csa2_profile_reset(void) {
    csa2::g_prof.drain();
    csa2::g_prof.sums.clear();
    return CSA2_OK;
}

int csa2_profile_read(int slot, const char** name, int* launches, double* total_ms) {
    csa2::g_prof.drain();
    if (slot < 0 || slot >= (int)csa2::g_prof.sums.size()) return CSA2_ERR_SHAPE;
    if (name) *name = csa2::g_prof.sums[slot].name;
    if (launches) *launches = csa2::g_prof.sums[slot].n;
    if (total_ms) *total_ms = csa2::g_prof.sums[slot].ms;
    return CSA2_OK;
}

}  // extern "C"
