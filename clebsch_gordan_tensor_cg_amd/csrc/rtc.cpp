// Runtime compilation of generated kernels (hipRTC, loaded on first use)
// and an on-disk code-object cache keyed by a hash of the source and the
// compile options.  The cache can be filled ahead of time on a machine
// without a GPU (CGTP_PLAN_NO_LOAD): compilation needs no device, only
// loading the module does.
#include <dlfcn.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstdio>
#include <cstdlib>
#include <fstream>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "internal.h"

namespace cgtp {
namespace {

// The few hipRTC entry points used, resolved with dlsym so the library has
// no link-time dependency on the runtime compiler.
typedef int (*fn_create)(void **, const char *, const char *, int, const char **, const char **);
typedef int (*fn_compile)(void *, int, const char **);
typedef int (*fn_logsize)(void *, size_t *);
typedef int (*fn_log)(void *, char *);
typedef int (*fn_codesize)(void *, size_t *);
typedef int (*fn_code)(void *, char *);
typedef int (*fn_destroy)(void **);

struct Rtc {
    bool ok = false;
    std::string why;
    fn_create create;
    fn_compile compile;
    fn_logsize logsize;
    fn_log log;
    fn_codesize codesize;
    fn_code code;
    fn_destroy destroy;
};

Rtc &rtc() {
    static Rtc r;
    static std::once_flag once;
    std::call_once(once, [] {
        const char *names[] = {"libhiprtc.so.7", "libhiprtc.so", "/opt/rocm/lib/libhiprtc.so"};
        void *h = nullptr;
        for (const char *n : names)
            if ((h = dlopen(n, RTLD_NOW | RTLD_GLOBAL))) break;
        if (!h) {
            r.why = std::string("cannot load hipRTC: ") + dlerror();
            return;
        }
        r.create = (fn_create)dlsym(h, "hiprtcCreateProgram");
        r.compile = (fn_compile)dlsym(h, "hiprtcCompileProgram");
        r.logsize = (fn_logsize)dlsym(h, "hiprtcGetProgramLogSize");
        r.log = (fn_log)dlsym(h, "hiprtcGetProgramLog");
        r.codesize = (fn_codesize)dlsym(h, "hiprtcGetCodeSize");
        r.code = (fn_code)dlsym(h, "hiprtcGetCode");
        r.destroy = (fn_destroy)dlsym(h, "hiprtcDestroyProgram");
        r.ok = r.create && r.compile && r.logsize && r.log && r.codesize && r.code && r.destroy;
        if (!r.ok) r.why = "hipRTC library lacks an expected symbol";
    });
    return r;
}

const std::vector<std::string> &options() {
    static const std::vector<std::string> o = {
        "--offload-arch=gfx950", "-O3", "-std=c++17",
        // packed FP32 instructions stay off on this target
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"};
    return o;
}

uint64_t fnv1a(const std::string &s, uint64_t h = 1469598103934665603ull) {
    for (unsigned char c : s) {
        h ^= c;
        h *= 1099511628211ull;
    }
    return h;
}

std::string cache_dir() {
    if (const char *e = std::getenv("CGTP_CACHE_DIR")) return e;
    Dl_info info;
    if (dladdr((void *)&cache_dir, &info) && info.dli_fname) {
        std::string p = info.dli_fname;
        auto slash = p.rfind('/');
        if (slash != std::string::npos) return p.substr(0, slash) + "/_kcache";
    }
    return "_kcache";
}

bool read_file(const std::string &path, std::vector<char> &out) {
    std::ifstream f(path, std::ios::binary);
    if (!f) return false;
    out.assign(std::istreambuf_iterator<char>(f), std::istreambuf_iterator<char>());
    return !out.empty();
}

void write_file_atomic(const std::string &dir, const std::string &path, const std::vector<char> &data) {
    mkdir(dir.c_str(), 0755);
    std::string tmp = path + ".tmp" + std::to_string(getpid());
    {
        std::ofstream f(tmp, std::ios::binary);
        if (!f) return;
        f.write(data.data(), (std::streamsize)data.size());
    }
    std::rename(tmp.c_str(), path.c_str());
}

std::mutex g_compile_mutex;

}  // namespace

int compile_and_load(Plan &p, bool load, std::string &err) {
    std::string opts;
    for (auto &o : options()) opts += o + " ";
    char key[32];
    std::snprintf(key, sizeof key, "%016llx", (unsigned long long)fnv1a(p.source + "|" + opts));
    p.cache_key = key;
    const std::string dir = cache_dir();
    const std::string path = dir + "/" + p.cache_key + ".hsaco";

    std::vector<char> code;
    p.cached = read_file(path, code);
    if (!p.cached) {
        std::lock_guard<std::mutex> lk(g_compile_mutex);
        Rtc &r = rtc();
        if (!r.ok) {
            err = r.why;
            return CGTP_ERR_COMPILE;
        }
        if (std::getenv("CGTP_FAULT") && std::string(std::getenv("CGTP_FAULT")) == "compile") {
            err = "compilation failure injected by CGTP_FAULT=compile";
            return CGTP_ERR_COMPILE;
        }
        void *prog = nullptr;
        if (r.create(&prog, p.source.c_str(), "cgtp_generated.hip", 0, nullptr, nullptr) != 0) {
            err = "hiprtcCreateProgram failed";
            return CGTP_ERR_COMPILE;
        }
        std::vector<const char *> ov;
        for (auto &o : options()) ov.push_back(o.c_str());
        int rc = r.compile(prog, (int)ov.size(), ov.data());
        size_t ls = 0;
        r.logsize(prog, &ls);
        std::string log(ls + 1, '\0');
        if (ls) r.log(prog, &log[0]);
        if (rc != 0) {
            err = "hipRTC compilation failed:\n" + log;
            r.destroy(&prog);
            return CGTP_ERR_COMPILE;
        }
        size_t cs = 0;
        r.codesize(prog, &cs);
        code.resize(cs);
        r.code(prog, code.data());
        r.destroy(&prog);
        write_file_atomic(dir, path, code);
    }
    p.n_kernels = (p.mode == CGTP_UVU) ? 7 : 1;
    if (!load) return CGTP_OK;

    hipError_t e = hipGetDevice(&p.device);
    if (e == hipSuccess) e = hipModuleLoadData(&p.module, code.data());
    if (e == hipSuccess) e = hipModuleGetFunction(&p.k_fwd, p.module, "cgtp_fwd");
    if (e == hipSuccess && p.n_kernels > 1) e = hipModuleGetFunction(&p.k_bwd, p.module, "cgtp_bwd");
    if (e == hipSuccess && p.n_kernels > 2) e = hipModuleGetFunction(&p.k_dbl, p.module, "cgtp_dbl");
    if (e == hipSuccess && p.n_kernels > 3) e = hipModuleGetFunction(&p.k_bwd_full, p.module, "cgtp_bwd_full");
    if (e == hipSuccess && p.n_kernels > 4) e = hipModuleGetFunction(&p.k_dbl_full, p.module, "cgtp_dbl_full");
    if (e == hipSuccess && p.n_kernels > 5) e = hipModuleGetFunction(&p.k_fb, p.module, "cgtp_fb");
    if (e == hipSuccess && p.n_kernels > 6) e = hipModuleGetFunction(&p.k_fb_full, p.module, "cgtp_fb_full");
    if (e == hipSuccess && p.uvw_pf) e = hipModuleGetFunction(&p.k_uvw_pf, p.module, "cgtp_uvw_pf");
    if (e != hipSuccess) {
        err = std::string("loading generated code object: ") + hipGetErrorString(e);
        return CGTP_ERR_HIP;
    }
    p.loaded = true;
    return CGTP_OK;
}

}  // namespace cgtp
