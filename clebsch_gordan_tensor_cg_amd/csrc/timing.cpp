// Opt-in per-launch timing: when enabled, every kernel the library launches
// is bracketed by two HIP events recorded on its launch stream, so a caller
// can read the duration of each kernel (not only of each API call).
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace cgtp {
namespace {
struct Rec {
    std::string name;
    hipEvent_t a = nullptr, b = nullptr;
    bool ok = true;   // both events recorded
};
std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
}  // namespace

TimedLaunch::TimedLaunch(const char *name, hipStream_t s) : s_(s) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return;
    Rec r;
    r.name = name;
    if (hipEventCreate(&r.a) != hipSuccess) return;
    if (hipEventCreate(&r.b) != hipSuccess || hipEventRecord(r.a, s) != hipSuccess) {
        (void)hipEventDestroy(r.a);
        if (r.b) (void)hipEventDestroy(r.b);
        return;
    }
    g_recs.push_back(r);
    idx_ = (long)g_recs.size() - 1;
}

TimedLaunch::~TimedLaunch() {
    if (idx_ < 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (idx_ < (long)g_recs.size() && hipEventRecord(g_recs[idx_].b, s_) != hipSuccess) g_recs[idx_].ok = false;
}

}  // namespace cgtp

using namespace cgtp;

extern "C" {

int cgtp_timing_enable(int enable) {
    clear_error();
    std::lock_guard<std::mutex> lk(g_mu);
    g_on = enable != 0;
    return CGTP_OK;
}

int cgtp_timing_collect(char (*names)[64], float *ms, int32_t cap, int32_t *n) {
    clear_error();
    if (cap < 0 || (cap > 0 && (!names || !ms)) || !n)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_timing_collect: bad argument");
    std::vector<Rec> recs;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        recs.swap(g_recs);
    }
    int32_t k = 0;
    int rc = CGTP_OK;
    for (Rec &r : recs) {
        float t = -1.0f;
        if (!r.ok || hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
            rc = set_error(CGTP_ERR_HIP, "cgtp_timing_collect: event query failed");
        if (k < cap) {
            std::strncpy(names[k], r.name.c_str(), 63);
            names[k][63] = 0;
            ms[k] = t;
            ++k;
        }
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    *n = k;
    return rc;
}

}  // extern "C"
