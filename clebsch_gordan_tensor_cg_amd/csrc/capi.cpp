// C ABI: plan construction and the execution calls that launch the
// generated kernels.  See include/cgtp.h for the contract of every call.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <functional>
#include <new>
#include <string>

#include "internal.h"

namespace cgtp {

int launch_zero(cgtp_dtype dt, void *p, int64_t n, hipStream_t s);

namespace {
thread_local std::string g_error;

size_t elem_bytes(cgtp_dtype d) { return d == CGTP_F64 ? 8 : (d == CGTP_BF16_F32ACC ? 2 : 4); }
size_t out_bytes(cgtp_dtype d) { return d == CGTP_F64 ? 8 : 4; }

bool path_ok(const Irrep &a, const Irrep &b, const Irrep &c) {
    if (c.l < std::abs(a.l - b.l) || c.l > a.l + b.l) return false;
    if (a.parity && b.parity && c.parity && a.parity * b.parity != c.parity) return false;
    return true;
}

std::vector<int64_t> offsets(const std::vector<Irrep> &v) {
    std::vector<int64_t> o;
    int64_t acc = 0;
    for (auto &ir : v) {
        o.push_back(acc);
        acc += (int64_t)ir.mul * ir.dim();
    }
    o.push_back(acc);
    return o;
}

int check_loaded(cgtp_plan_t plan) {
    if (!plan) return set_error(CGTP_ERR_INVALID_ARGUMENT, "plan is NULL");
    if (!plan->p.loaded)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "plan was created with CGTP_PLAN_NO_LOAD or has no kernels");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != plan->p.device)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "plan was loaded on another device");
    return CGTP_OK;
}

int launch(hipFunction_t f, const char *name, int64_t blocks, hipStream_t s, void **args, unsigned threads = 64) {
    if (blocks <= 0) return CGTP_OK;
    if (blocks > 0x7fffffffLL) return set_error(CGTP_ERR_INVALID_ARGUMENT, "grid too large");
    TimedLaunch tl(name, s);
    hipError_t e = hipModuleLaunchKernel(f, (unsigned)blocks, 1, 1, threads, 1, 1, 0, s, args, nullptr);
    if (e != hipSuccess) return set_error(CGTP_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    return CGTP_OK;
}

bool blocks_covered(const std::vector<Irrep> &irreps, const std::vector<Path> &paths, bool out_side) {
    std::vector<char> cov(irreps.size(), 0);
    for (auto &P : paths) cov[out_side ? P.i3 : P.i1] = 1;
    for (char c : cov)
        if (!c) return false;
    return true;
}

// forward launch with an explicit operand set (used by the forward and by
// the double backward's substituted calls)
// vec/vperm: edge vectors from which the kernels compute the SH rows
// themselves (y unused), or NULL
int run_fwd(const Plan &p, const void *x, const void *y, const void *w, const int32_t *src,
            const int32_t *row_ptr, const int32_t *order, int64_t n_items, int graph, void *out, int accumulate,
            hipStream_t s, const void *vec = nullptr, const int32_t *vperm = nullptr) {
    if (!accumulate && !blocks_covered(p.out, p.paths, true)) {
        int rc = launch_zero(p.dtype == CGTP_F64 ? CGTP_F64 : CGTP_F32, out, n_items * p.dim3, s);
        if (rc) return rc;
        accumulate = 1;
    }
    long long n = n_items;
    void *args[] = {(void *)&x, (void *)&y, (void *)&w, (void *)&src, (void *)&row_ptr, (void *)&order,
                    (void *)&vec, (void *)&vperm, (void *)&out, &n, &graph, &accumulate};
    const int64_t ipw = p.fwd.items_per_wave;
    return launch(p.k_fwd, "cgtp_fwd", (n_items + ipw - 1) / ipw * p.fwd.n_units, s, args);
}

struct BwdOut {
    void *g_w = nullptr;  // per-edge weight gradient
    bool acc_w = false;
    bool want_m = false;  // per-edge x-messages into the workspace
    bool acc_m = false;
    void *g_y = nullptr;  // per-edge y gradient
    bool acc_y = false;
    void *fwd = nullptr;  // fused forward of the same operands (double backward, or with fb)
    bool acc_fwd = false;
    bool fb = false;      // forward and backward of one operand set (fwd = f(x, y, w))
    bool keep_parts = false;  // leave the per-unit y-gradient partials in the workspace
    void *m_out = nullptr;    // x-messages straight into this array instead of the workspace
                              // (independent items: message t is item t's x-gradient)
    int graph = 1;            // 0: independent items (item t is its own one-edge segment)
};

// workspace layout of the backward calls: x-messages [E][dim1] in the edges'
// (destination) order, gathered through src_perm by the segment sums;
// SH-gradient parts [units][E][dim2]; per-edge force vectors [E][3]
int parts_units(const Plan &p) { return std::max(1, std::max(p.bwd.n_units, p.fb.n_units)); }
char *ws_parts(const Plan &p, char *ws, int64_t n_edges) {
    return ws + align256((size_t)n_edges * p.dim1 * out_bytes(p.dtype));
}
// per-edge force vectors [E][3] of the backward with forces
char *ws_force(const Plan &p, char *ws, int64_t n_edges) {
    return ws_parts(p, ws, n_edges) + align256((size_t)parts_units(p) * n_edges * p.dim2 * out_bytes(p.dtype));
}

int run_bwd(const Plan &p, const void *x, const void *y, const void *w, const int32_t *src,
            const int32_t *row_ptr, const int32_t *order, const void *g_out, int64_t n_nodes, int64_t n_edges,
            BwdOut o, char *ws, hipStream_t s, const void *vec = nullptr, const int32_t *vperm = nullptr) {
    void *m = o.m_out ? o.m_out : (void *)ws;
    char *parts = ws_parts(p, ws, n_edges);
    const bool fused = o.fwd != nullptr && !o.fb;   // the double backward's y term
    const bool fb = o.fb;
    const KernelShape &ks = fused ? p.dbl : fb ? p.fb : p.bwd;
    const bool use_parts = !fused && o.g_y && ks.n_units > 1;
    int flags = 0;
    if (o.g_w) flags |= 1 | (o.acc_w ? 8 : 0);
    if (o.want_m) flags |= 2 | (o.acc_m ? 16 : 0);
    if (o.g_y) flags |= 4 | (use_parts ? 64 : (o.acc_y ? 32 : 0));
    if ((fused || fb) && o.acc_fwd) flags |= 256;
    if (!flags && !fused && !fb) return CGTP_OK;
    if (o.want_m && !o.acc_m && !blocks_covered(p.in1, p.paths, false)) {
        int rc = launch_zero(p.dtype, m, n_edges * p.dim1, s);
        if (rc) return rc;
        flags |= 16;
    }
    if ((fused || fb) && !o.acc_fwd && !blocks_covered(p.out, p.paths, true)) {
        int rc = launch_zero(p.dtype, o.fwd, n_nodes * p.dim3, s);
        if (rc) return rc;
        flags |= 256;
    }
    void *third = fused ? o.fwd : (use_parts ? (void *)parts : o.g_y);
    void *fourth = o.fwd;
    void *gw = o.g_w;
    long long n = n_nodes, ne = n_edges;
    int graph = o.graph;
    void *args[] = {(void *)&x, (void *)&y, (void *)&w, (void *)&src, (void *)&row_ptr, (void *)&order,
                    (void *)&vec, (void *)&vperm, (void *)&g_out, &gw, &m, &third, &n, &ne, &graph, &flags};
    void *args_fb[] = {(void *)&x, (void *)&y, (void *)&w, (void *)&src, (void *)&row_ptr, (void *)&order,
                       (void *)&vec, (void *)&vperm, (void *)&g_out, &gw, &m, &third, &fourth, &n, &ne, &graph,
                       &flags};
    const int64_t ipw = ks.items_per_wave;
    const bool full = fused ? ((p.tune.full & 2) && flags == dbl_full_flags(p))
                      : fb  ? ((p.tune.full & 4) && flags == fb_full_flags(p))
                            : ((p.tune.full & 1) && flags == bwd_full_flags(p));
    hipFunction_t f = fused ? (full ? p.k_dbl_full : p.k_dbl)
                      : fb  ? (full ? p.k_fb_full : p.k_fb)
                            : (full ? p.k_bwd_full : p.k_bwd);
    const char *name = fused ? (full ? "cgtp_dbl_full" : "cgtp_dbl")
                       : fb  ? (full ? "cgtp_fb_full" : "cgtp_fb")
                             : (full ? "cgtp_bwd_full" : "cgtp_bwd");
    int rc = launch(f, name, (n_nodes + ipw - 1) / ipw * ks.n_units, s, fb ? args_fb : args);
    if (rc) return rc;
    if (use_parts && !o.keep_parts) rc = launch_sum_parts(p.dtype, parts, ks.n_units, n_edges * p.dim2, o.g_y, o.acc_y, s);
    return rc;
}

}  // namespace

int set_error(int code, const std::string &msg) {
    g_error = msg;
    return code;
}
void clear_error() { g_error.clear(); }

}  // namespace cgtp

using namespace cgtp;

extern "C" {

const char *cgtp_last_error(void) { return g_error.c_str(); }
const char *cgtp_version(void) { return "cgtp 0.1 (gfx950)"; }

int cgtp_plan(const char *irreps_in1, const char *irreps_in2, const char *irreps_out, const cgtp_path *paths,
              int32_t n_paths, cgtp_mode mode, cgtp_dtype dtype, uint32_t flags, cgtp_plan_t *out) {
    clear_error();
    if (!out) return set_error(CGTP_ERR_INVALID_ARGUMENT, "out is NULL");
    *out = nullptr;
    if (mode != CGTP_UVU && mode != CGTP_UVW) return set_error(CGTP_ERR_INVALID_ARGUMENT, "unknown mode");
    if (dtype != CGTP_F32 && dtype != CGTP_F64 && dtype != CGTP_BF16_F32ACC)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "unknown dtype");
    if (flags & ~(uint32_t)(CGTP_SHARED_WEIGHTS | CGTP_PLAN_NO_LOAD | CGTP_BF16_WEIGHTS | CGTP_RADIAL_HIDDEN(255)))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "unknown flag bits");
    const int radial_h = (int)((flags >> 16) & 255u);
    if (radial_h > 0 && (mode != CGTP_UVW || dtype != CGTP_BF16_F32ACC || !(flags & CGTP_SHARED_WEIGHTS) ||
                         radial_h > 64))
        return set_error(CGTP_ERR_UNSUPPORTED,
                         "radial weights: uvw, bf16 inputs, CGTP_SHARED_WEIGHTS and a hidden width of 1..64");
    if (n_paths < 0 || (n_paths > 0 && !paths)) return set_error(CGTP_ERR_INVALID_ARGUMENT, "bad path list");
    try {
        cgtp_plan_t h = new cgtp_plan_s;
        Plan &p = h->p;
        std::string err;
        auto fail = [&](int code, const std::string &msg) {
            delete h;
            return set_error(code, msg);
        };
        int rc;
        if ((rc = parse_irreps(irreps_in1, p.in1, err)) || (rc = parse_irreps(irreps_in2, p.in2, err)) ||
            (rc = parse_irreps(irreps_out, p.out, err)))
            return fail(rc, err);
        if (p.in1.empty() || p.in2.empty() || p.out.empty()) return fail(CGTP_ERR_INVALID_ARGUMENT, "empty irreps");
        for (auto *v : {&p.in1, &p.in2, &p.out})
            for (auto &ir : *v)
                if (ir.l > kMaxL) return fail(CGTP_ERR_UNSUPPORTED, "degree above 6 is not supported");
        p.mode = mode;
        p.dtype = dtype;
        p.flags = flags;
        p.radial_h = (int)((flags >> 16) & 255u);
        p.tune = tuning_from_env();
        auto o1 = offsets(p.in1), o2 = offsets(p.in2), o3 = offsets(p.out);
        p.dim1 = o1.back();
        p.dim2 = o2.back();
        p.dim3 = o3.back();
        p.off1.assign(o1.begin(), o1.end() - 1);
        p.off2.assign(o2.begin(), o2.end() - 1);
        p.off3.assign(o3.begin(), o3.end() - 1);
        for (auto &ir : p.in2) p.lmax2 = std::max(p.lmax2, ir.l);
        {
            // input 2 laid out as one SH row (1x0 + 1x1 + ... + 1xL, parity
            // absent or (-1)^l): the SH can be computed inside the kernels
            bool sh = p.in2.size() <= 7;
            for (size_t l = 0; l < p.in2.size() && sh; ++l) {
                const Irrep &ir = p.in2[l];
                sh = ir.mul == 1 && ir.l == (int)l && (ir.parity == 0 || ir.parity == ((l & 1) ? -1 : 1));
            }
            p.sh_lmax = sh ? (int)p.in2.size() - 1 : -1;
        }
        if (p.radial_h > 0 && p.sh_lmax < 0)
            return fail(CGTP_ERR_UNSUPPORTED, "radial weights need input 2 = one SH row (computed from edge vectors)");

        std::vector<cgtp_path> list;
        if (n_paths > 0) {
            list.assign(paths, paths + n_paths);
        } else {
            for (int a = 0; a < (int)p.in1.size(); ++a)
                for (int b = 0; b < (int)p.in2.size(); ++b)
                    for (int c = 0; c < (int)p.out.size(); ++c) {
                        if (!path_ok(p.in1[a], p.in2[b], p.out[c])) continue;
                        if (mode == CGTP_UVU && p.out[c].mul != p.in1[a].mul) continue;
                        list.push_back({a, b, c});
                    }
        }
        if (list.empty()) return fail(CGTP_ERR_INVALID_ARGUMENT, "no allowed path");
        int64_t woff = 0;
        for (auto &cp : list) {
            if (cp.i_in1 < 0 || cp.i_in1 >= (int)p.in1.size() || cp.i_in2 < 0 || cp.i_in2 >= (int)p.in2.size() ||
                cp.i_out < 0 || cp.i_out >= (int)p.out.size())
                return fail(CGTP_ERR_INVALID_ARGUMENT, "path index out of range");
            const Irrep &a = p.in1[cp.i_in1], &b = p.in2[cp.i_in2], &c = p.out[cp.i_out];
            if (!path_ok(a, b, c))
                return fail(CGTP_ERR_INVALID_ARGUMENT, "path (" + std::to_string(cp.i_in1) + "," +
                                                           std::to_string(cp.i_in2) + "," + std::to_string(cp.i_out) +
                                                           ") violates the selection rule");
            if (mode == CGTP_UVU && c.mul != a.mul)
                return fail(CGTP_ERR_INVALID_ARGUMENT, "uvu path needs mul_out == mul_in1");
            Path P;
            P.i1 = cp.i_in1;
            P.i2 = cp.i_in2;
            P.i3 = cp.i_out;
            P.l1 = a.l;
            P.l2 = b.l;
            P.l3 = c.l;
            P.mul1 = a.mul;
            P.mul2 = b.mul;
            P.mul3 = c.mul;
            P.off1 = p.off1[P.i1];
            P.off2 = p.off2[P.i2];
            P.off3 = p.off3[P.i3];
            P.woff = woff;
            P.wnum = (int64_t)a.mul * b.mul * (mode == CGTP_UVW ? c.mul : 1);
            woff += P.wnum;
            if ((rc = real_coupling(P.l1, P.l2, P.l3, P.R, err))) return fail(rc, err);
            const int d2 = 2 * P.l2 + 1, d3 = 2 * P.l3 + 1;
            for (int i = 0; i < 2 * P.l1 + 1; ++i)
                for (int j = 0; j < d2; ++j)
                    for (int k = 0; k < d3; ++k) {
                        double c2 = P.R[((size_t)i * d2 + j) * d3 + k];
                        if (std::fabs(c2) > 1e-14) P.nz.push_back({i, j, k, c2});
                    }
            p.paths.push_back(std::move(P));
        }
        p.wnumel = woff;
        if (mode == CGTP_UVU && dtype == CGTP_BF16_F32ACC)
            return fail(CGTP_ERR_UNSUPPORTED, "bf16 inputs are provided for uvw plans only");
        if ((flags & CGTP_BF16_WEIGHTS) && (mode != CGTP_UVU || dtype != CGTP_F32))
            return fail(CGTP_ERR_UNSUPPORTED, "bf16 weight storage is provided for uvu float plans only");
        if (mode == CGTP_UVW && (dtype != CGTP_BF16_F32ACC || !(flags & CGTP_SHARED_WEIGHTS))) {
            // uvw kernels exist for bf16 operands with one shared weight set
            // (channel mixing on the matrix cores); other uvw plans serve
            // coupling queries only
            *out = h;
            return CGTP_OK;
        }
        choose_shapes(p);
        p.source = generate_source(p);
        if ((rc = compile_and_load(p, !(flags & CGTP_PLAN_NO_LOAD), err))) return fail(rc, err);
        if (std::getenv("CGTP_DEBUG")) dump_plan(p);
        *out = h;
        return CGTP_OK;
    } catch (const std::bad_alloc &) {
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "out of host memory while planning");
    } catch (const std::exception &e) {
        return set_error(CGTP_ERR_INVALID_ARGUMENT, std::string("planning failed: ") + e.what());
    }
}

int cgtp_plan_info(cgtp_plan_t plan, cgtp_plan_dims *d) {
    clear_error();
    if (!plan || !d) return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL argument");
    const Plan &p = plan->p;
    d->dim_in1 = p.dim1;
    d->dim_in2 = p.dim2;
    d->dim_out = p.dim3;
    d->weight_numel = p.wnumel;
    d->n_paths = (int32_t)p.paths.size();
    d->lmax_in2 = p.lmax2;
    d->n_kernels = p.n_kernels;
    d->cached = p.cached ? 1 : 0;
    return CGTP_OK;
}

int cgtp_plan_paths(cgtp_plan_t plan, cgtp_path *paths, int32_t cap) {
    clear_error();
    if (!plan || (cap > 0 && !paths)) return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL argument");
    const Plan &p = plan->p;
    for (int32_t a = 0; a < cap && a < (int32_t)p.paths.size(); ++a)
        paths[a] = {p.paths[a].i1, p.paths[a].i2, p.paths[a].i3};
    return CGTP_OK;
}

int cgtp_plan_coupling(cgtp_plan_t plan, int32_t pidx, double *R, int64_t cap) {
    clear_error();
    if (!plan || !R) return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL argument");
    const Plan &p = plan->p;
    if (pidx < 0 || pidx >= (int32_t)p.paths.size()) return set_error(CGTP_ERR_INVALID_ARGUMENT, "path index");
    const auto &v = p.paths[pidx].R;
    if (cap < (int64_t)v.size()) return set_error(CGTP_ERR_INVALID_ARGUMENT, "capacity too small");
    std::memcpy(R, v.data(), v.size() * sizeof(double));
    return CGTP_OK;
}

int cgtp_plan_source(cgtp_plan_t plan, char *buf, int64_t cap, int64_t *len) {
    clear_error();
    if (!plan) return set_error(CGTP_ERR_INVALID_ARGUMENT, "plan is NULL");
    const std::string &s = plan->p.source;
    if (len) *len = (int64_t)s.size();
    if (buf && cap > 0) {
        int64_t n = std::min<int64_t>(cap - 1, (int64_t)s.size());
        std::memcpy(buf, s.data(), (size_t)n);
        buf[n] = 0;
    }
    return CGTP_OK;
}

void cgtp_plan_destroy(cgtp_plan_t plan) {
    if (!plan) return;
    if (plan->p.module) (void)hipModuleUnload(plan->p.module);
    delete plan;
}

// scratch of the forward calls: uvw path tensors T (bf16) and the partial
// tiles of split mixing contractions; uvu forwards take none
static size_t fwd_ws_bytes(const Plan &p, int64_t n_items) {
    if (p.mode != CGTP_UVW) return 0;
    return align256((size_t)n_items * p.t_per_item * 2) + align256(mix_part_bytes(p, n_items));
}

// scratch of the backward calls (layout above ws_parts / ws_force)
static size_t graph_ws_bytes(const Plan &p, int64_t n_nodes, int64_t n_edges) {
    (void)n_nodes;
    const size_t eb = out_bytes(p.dtype);
    return align256((size_t)n_edges * p.dim1 * eb) + align256((size_t)parts_units(p) * n_edges * p.dim2 * eb) +
           align256((size_t)n_edges * 3 * eb) + 256;
}

static int run_uvw(const Plan &p, const void *x, const void *y, const void *w, const int32_t *src,
                   const int32_t *row_ptr, const int32_t *order, int64_t n_items, int graph, void *out, void *ws,
                   size_t ws_bytes, hipStream_t s, const void *vec = nullptr, const int32_t *vperm = nullptr,
                   const float *radial = nullptr) {
    const size_t need = fwd_ws_bytes(p, n_items);
    if (ws_bytes < need || (!ws && need)) return set_error(CGTP_ERR_INVALID_ARGUMENT, "workspace too small");
    void *part = (char *)ws + align256((size_t)n_items * p.t_per_item * 2);
    if (((uintptr_t)ws) & 255) return set_error(CGTP_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    long long n = n_items;
    void *args[] = {(void *)&x, (void *)&y, (void *)&src, (void *)&row_ptr, (void *)&order, (void *)&vec,
                    (void *)&vperm, (void *)&radial, &ws, &n, &graph};
    const int64_t ipw = p.fwd.items_per_wave;
    // graph calls: the per-pair matrix-core form where the plan has it (one
    // workgroup per pair of nodes); else the per-edge kernel, or the
    // per-node matrix-core form (one workgroup of four wavefronts per item and
    // input-1 block)
    // (its x segments, and with the mixing inside the weight rows, are read
    // in 16-byte groups: they must be 16-byte aligned)
    const bool pf = graph && p.uvw_pf && ((uintptr_t)x & 15) == 0 && (!p.uvw_pf_mix || ((uintptr_t)w & 15) == 0);
    if (pf) {
        // the pair kernel; with the mixing inside it writes out directly
        void *pargs[] = {(void *)&x, (void *)&y, (void *)&src, (void *)&row_ptr, (void *)&order, (void *)&vec,
                         (void *)&vperm, (void *)&radial, &ws, &n, &graph, (void *)&w, &out};
        int rc = launch(p.k_uvw_pf, "cgtp_uvw_pf", (n_items + 1) / 2, s, pargs, 64 * p.uvw_pf_waves);
        if (rc || p.uvw_pf_mix) return rc;
    }
    int rc = pf          ? CGTP_OK
             : p.uvw_mma ? launch(p.k_fwd, "cgtp_fwd", n_items * p.uvw_mma_groups, s, args, 256)
                         : launch(p.k_fwd, "cgtp_fwd", (n_items + ipw - 1) / ipw * p.fwd.n_units, s, args);
    if (rc) return rc;
    int acc = 0;
    if (!blocks_covered(p.out, p.paths, true)) {
        if ((rc = launch_zero(CGTP_F32, out, n_items * p.dim3, s))) return rc;
        acc = 1;
    }
    if ((rc = launch_uvw_mix(p, ws, w, n_items, out, acc, part, s))) return rc;
    return CGTP_OK;
}

int cgtp_forward(cgtp_plan_t plan, const void *x, const void *y, const void *w, int64_t batch, void *out,
                 void *workspace, size_t workspace_bytes, cgtp_stream_t stream) {
    clear_error();
    int rc = check_loaded(plan);
    if (rc) return rc;
    if (batch < 0 || batch > 0x7fffffffLL) return set_error(CGTP_ERR_INVALID_ARGUMENT, "batch out of range");
    if (batch == 0) return CGTP_OK;
    if (!x || !y || !w || !out) return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL buffer");
    if (plan->p.radial_h > 0)
        return set_error(CGTP_ERR_UNSUPPORTED, "radial plans run through cgtp_conv_forward_radial");
    if (plan->p.mode == CGTP_UVW)
        return run_uvw(plan->p, x, y, w, nullptr, nullptr, nullptr, batch, 0, out, workspace, workspace_bytes,
                       (hipStream_t)stream);
    return run_fwd(plan->p, x, y, w, nullptr, nullptr, nullptr, batch, 0, out, 0, (hipStream_t)stream);
}

static int conv_forward_impl(cgtp_plan_t plan, const void *x, const void *sh, const void *vec, const int32_t *vperm,
                             const void *w, const int32_t *src, const int32_t *dst_row_ptr, const int32_t *node_order,
                             int64_t n_nodes, int64_t n_edges, void *out, void *workspace, size_t workspace_bytes,
                             cgtp_stream_t stream, bool radial_call = false, const float *radial = nullptr) {
    int rc = check_loaded(plan);
    if (rc) return rc;
    if ((plan->p.radial_h > 0) && !radial_call)
        return set_error(CGTP_ERR_UNSUPPORTED, "radial plans run through cgtp_conv_forward_radial");
    if (n_nodes < 0 || n_edges < 0 || n_edges > 0x7fffffffLL || n_nodes > 0x7fffffffLL)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "sizes out of range");
    if (n_nodes == 0) return CGTP_OK;
    if (!dst_row_ptr || !out || (n_edges > 0 && (!x || !(sh || vec) || !w || !src)))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL buffer");
    if (plan->p.mode == CGTP_UVW)
        return run_uvw(plan->p, x, sh, w, src, dst_row_ptr, node_order, n_nodes, 1, out, workspace,
                       workspace_bytes, (hipStream_t)stream, vec, vperm, radial);
    return run_fwd(plan->p, x, sh, w, src, dst_row_ptr, node_order, n_nodes, 1, out, 0, (hipStream_t)stream, vec, vperm);
}

static int check_vec_plan(cgtp_plan_t plan) {
    if (plan && (plan->p.sh_lmax < 0 || plan->p.tune.stage <= 0))
        return set_error(CGTP_ERR_UNSUPPORTED,
                         "SH from edge vectors needs input 2 = 1x0+1x1+...+1xL (one SH row) and LDS staging");
    return CGTP_OK;
}

int cgtp_conv_forward(cgtp_plan_t plan, const void *x, const void *sh, const void *w, const int32_t *src,
                      const int32_t *dst_row_ptr, const int32_t *node_order, int64_t n_nodes, int64_t n_edges,
                      void *out, void *workspace, size_t workspace_bytes, cgtp_stream_t stream) {
    clear_error();
    return conv_forward_impl(plan, x, sh, nullptr, nullptr, w, src, dst_row_ptr, node_order, n_nodes, n_edges, out,
                             workspace, workspace_bytes, stream);
}

int cgtp_conv_forward_radial(cgtp_plan_t plan, const void *x, const void *vec, const int32_t *vec_perm,
                             const float *radial, const void *w, const int32_t *src, const int32_t *dst_row_ptr,
                             const int32_t *node_order, int64_t n_nodes, int64_t n_edges, void *out, void *workspace,
                             size_t workspace_bytes, cgtp_stream_t stream) {
    clear_error();
    int rc = check_vec_plan(plan);
    if (rc) return rc;
    if (plan->p.radial_h <= 0)
        return set_error(CGTP_ERR_UNSUPPORTED, "cgtp_conv_forward_radial needs a plan with CGTP_RADIAL_HIDDEN(H)");
    if (n_edges > 0 && (!vec || !radial)) return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL buffer");
    return conv_forward_impl(plan, x, nullptr, vec, vec_perm, w, src, dst_row_ptr, node_order, n_nodes, n_edges, out,
                             workspace, workspace_bytes, stream, true, radial);
}

int cgtp_conv_forward_vec(cgtp_plan_t plan, const void *x, const void *vec, const int32_t *vec_perm, const void *w,
                          const int32_t *src, const int32_t *dst_row_ptr, const int32_t *node_order, int64_t n_nodes,
                          int64_t n_edges, void *out, void *workspace, size_t workspace_bytes, cgtp_stream_t stream) {
    clear_error();
    int rc = check_vec_plan(plan);
    if (rc) return rc;
    if (n_edges > 0 && !vec) return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL buffer");
    return conv_forward_impl(plan, x, nullptr, vec, vec_perm, w, src, dst_row_ptr, node_order, n_nodes, n_edges, out,
                             workspace, workspace_bytes, stream);
}

int cgtp_workspace_bytes(cgtp_plan_t plan, int64_t n_items, int64_t n_edges, size_t *bytes) {
    clear_error();
    if (!plan || !bytes || n_items < 0 || n_edges < 0) return set_error(CGTP_ERR_INVALID_ARGUMENT, "bad argument");
    const Plan &p = plan->p;
    // the single product's backward counts each item as a one-edge segment
    *bytes = std::max(fwd_ws_bytes(p, n_items), graph_ws_bytes(p, n_items, std::max(n_edges, n_items)));
    return CGTP_OK;
}

static int check_graph_args(cgtp_plan_t plan, int64_t n_nodes, int64_t n_edges, void *ws, size_t ws_bytes) {
    int rc = check_loaded(plan);
    if (rc) return rc;
    if (plan->p.mode != CGTP_UVU || !plan->p.k_bwd)
        return set_error(CGTP_ERR_UNSUPPORTED, "backward kernels are provided for uvu fp32/fp64 plans");
    if (plan->p.flags & CGTP_SHARED_WEIGHTS)
        return set_error(CGTP_ERR_UNSUPPORTED, "backward with shared weights is not provided");
    if (n_nodes < 0 || n_edges < 0 || n_edges > 0x7fffffffLL || n_nodes > 0x7fffffffLL)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "sizes out of range");
    const size_t need = graph_ws_bytes(plan->p, n_nodes, n_edges);
    if (ws_bytes < need || (!ws && need)) return set_error(CGTP_ERR_INVALID_ARGUMENT, "workspace too small");
    if (((uintptr_t)ws) & 255) return set_error(CGTP_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    return CGTP_OK;
}

static int conv_backward_impl(cgtp_plan_t plan, const void *x, const void *sh, const void *vec,
                              const int32_t *vperm, const void *w, const int32_t *src, const int32_t *dst_row_ptr,
                              const int32_t *node_order, const int32_t *src_row_ptr, const int32_t *src_perm,
                              const void *g_out, int64_t n_nodes, int64_t n_edges, void *g_x, void *g_sh, void *g_w,
                              void *F, void *workspace, size_t workspace_bytes, cgtp_stream_t stream,
                              void *out = nullptr) {
    int rc = check_graph_args(plan, n_nodes, n_edges, workspace, workspace_bytes);
    if (rc) return rc;
    const Plan &p = plan->p;
    hipStream_t s = (hipStream_t)stream;
    if (n_nodes == 0) return CGTP_OK;
    if (!dst_row_ptr || ((g_x || F) && (!src_row_ptr || (n_edges > 0 && !src_perm))) ||
        (n_edges > 0 && (!x || !(sh || vec) || !w || !src || !g_out)))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL buffer");
    if (n_edges == 0) {
        if (out && (rc = launch_zero(p.dtype, out, n_nodes * p.dim3, s))) return rc;
        if (g_x && (rc = launch_zero(p.dtype, g_x, n_nodes * p.dim1, s))) return rc;
        if (F) return launch_zero(p.dtype, F, n_nodes * 3, s);
        return CGTP_OK;
    }
    // FP64 plans: forward and backward as two launches.  The one-pass kernel
    // is used for FP32 only: its FP64 form took a device memory fault on a
    // 128-channel plan with the SH computed from edge vectors, with no cause
    // found in the generated code, so it is switched off.
    if (out && p.dtype == CGTP_F64) {
        if ((rc = run_fwd(p, x, sh, w, src, dst_row_ptr, node_order, n_nodes, 1, out, 0, s, vec, vperm))) return rc;
        out = nullptr;
    }
    char *ws = (char *)workspace;
    BwdOut o;
    o.fwd = out;
    o.fb = out != nullptr;
    o.g_w = g_w;
    o.want_m = g_x != nullptr;
    o.g_y = g_sh;
    // forces without g_sh: the y-gradient stays as per-unit partials in the
    // workspace and the force kernel sums them
    const bool parts_force = F && !g_sh;
    if (parts_force) {
        o.g_y = ws_parts(p, ws, n_edges);
        o.keep_parts = true;
    }
    rc = run_bwd(p, x, sh, w, src, dst_row_ptr, node_order, g_out, n_nodes, n_edges, o, ws, s, vec, vperm);
    if (rc) return rc;
    if (g_x && (rc = launch_segment_sum_rows(p.dtype, workspace, src_row_ptr, src_perm, n_nodes, p.dim1, g_x, 0, s)))
        return rc;
    if (F) {
        const int units = (out ? p.fb : p.bwd).n_units;
        const int n_parts = parts_force && units > 1 ? units : 1;
        rc = launch_sh_forces(p.sh_lmax, p.dtype, vec, vperm, parts_force ? o.g_y : g_sh, n_parts, n_edges * p.dim2,
                              dst_row_ptr, src_row_ptr, src_perm, n_nodes, n_edges, F, ws_force(p, ws, n_edges), s);
    }
    return rc;
}

int cgtp_backward(cgtp_plan_t plan, const void *x, const void *sh, const void *w, const int32_t *src,
                  const int32_t *dst_row_ptr, const int32_t *node_order, const int32_t *src_row_ptr,
                  const int32_t *src_perm, const void *g_out, int64_t n_nodes, int64_t n_edges, void *g_x, void *g_sh,
                  void *g_w, void *workspace, size_t workspace_bytes, cgtp_stream_t stream) {
    clear_error();
    return conv_backward_impl(plan, x, sh, nullptr, nullptr, w, src, dst_row_ptr, node_order, src_row_ptr, src_perm,
                              g_out, n_nodes, n_edges, g_x, g_sh, g_w, nullptr, workspace, workspace_bytes, stream);
}

int cgtp_tp_backward(cgtp_plan_t plan, const void *x, const void *y, const void *w, int64_t batch, const void *g_out,
                     void *g_x, void *g_y, void *g_w, void *workspace, size_t workspace_bytes, cgtp_stream_t stream) {
    clear_error();
    // each item is its own one-edge segment: the graph calls' workspace for
    // batch nodes and batch edges, and no source reduction (message t is
    // item t's x-gradient, written straight into g_x)
    int rc = check_graph_args(plan, batch, batch, workspace, workspace_bytes);
    if (rc) return rc;
    if (batch == 0) return CGTP_OK;
    if (!x || !y || !w || !g_out) return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL buffer");
    const Plan &p = plan->p;
    BwdOut o;
    o.graph = 0;
    o.g_w = g_w;
    o.want_m = g_x != nullptr;
    o.m_out = g_x;
    o.g_y = g_y;
    return run_bwd(p, x, y, w, nullptr, nullptr, nullptr, g_out, batch, batch, o, (char *)workspace,
                   (hipStream_t)stream);
}

int cgtp_conv_backward_vec(cgtp_plan_t plan, const void *x, const void *vec, const int32_t *vec_perm, const void *w,
                           const int32_t *src, const int32_t *dst_row_ptr, const int32_t *node_order,
                           const int32_t *src_row_ptr, const int32_t *src_perm, const void *g_out, int64_t n_nodes,
                           int64_t n_edges, void *g_x, void *g_sh, void *g_w, void *F, void *workspace,
                           size_t workspace_bytes, cgtp_stream_t stream) {
    clear_error();
    int rc = check_vec_plan(plan);
    if (rc) return rc;
    if (n_edges > 0 && !vec) return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL buffer");
    return conv_backward_impl(plan, x, nullptr, vec, vec_perm, w, src, dst_row_ptr, node_order, src_row_ptr, src_perm,
                              g_out, n_nodes, n_edges, g_x, g_sh, g_w, F, workspace, workspace_bytes, stream);
}

int cgtp_conv_forward_backward(cgtp_plan_t plan, const void *x, const void *sh, const void *w, const int32_t *src,
                               const int32_t *dst_row_ptr, const int32_t *node_order, const int32_t *src_row_ptr,
                               const int32_t *src_perm, const void *g_out, int64_t n_nodes, int64_t n_edges, void *out,
                               void *g_x, void *g_sh, void *g_w, void *workspace, size_t workspace_bytes,
                               cgtp_stream_t stream) {
    clear_error();
    if (!out) return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_conv_forward_backward: out is NULL");
    return conv_backward_impl(plan, x, sh, nullptr, nullptr, w, src, dst_row_ptr, node_order, src_row_ptr, src_perm,
                              g_out, n_nodes, n_edges, g_x, g_sh, g_w, nullptr, workspace, workspace_bytes, stream, out);
}

int cgtp_conv_forward_backward_vec(cgtp_plan_t plan, const void *x, const void *vec, const int32_t *vec_perm,
                                   const void *w, const int32_t *src, const int32_t *dst_row_ptr,
                                   const int32_t *node_order, const int32_t *src_row_ptr, const int32_t *src_perm,
                                   const void *g_out, int64_t n_nodes, int64_t n_edges, void *out, void *g_x,
                                   void *g_sh, void *g_w, void *F, void *workspace, size_t workspace_bytes,
                                   cgtp_stream_t stream) {
    clear_error();
    int rc = check_vec_plan(plan);
    if (rc) return rc;
    if (!out) return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_conv_forward_backward_vec: out is NULL");
    if (n_edges > 0 && !vec) return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL buffer");
    return conv_backward_impl(plan, x, nullptr, vec, vec_perm, w, src, dst_row_ptr, node_order, src_row_ptr, src_perm,
                              g_out, n_nodes, n_edges, g_x, g_sh, g_w, F, workspace, workspace_bytes, stream, out);
}

int cgtp_double_backward(cgtp_plan_t plan, const void *x, const void *sh, const void *w, const void *g_out,
                         const void *gg_x, const void *gg_sh, const void *gg_w, const int32_t *src,
                         const int32_t *dst_row_ptr, const int32_t *node_order, const int32_t *src_row_ptr,
                         const int32_t *src_perm, int64_t n_nodes, int64_t n_edges, void *d_g_out, void *d_x,
                         void *d_sh, void *d_w, void *workspace, size_t workspace_bytes, cgtp_stream_t stream) {
    clear_error();
    int rc = check_graph_args(plan, n_nodes, n_edges, workspace, workspace_bytes);
    if (rc) return rc;
    const Plan &p = plan->p;
    hipStream_t s = (hipStream_t)stream;
    if (n_nodes == 0) return CGTP_OK;
    if (!dst_row_ptr || (d_x && (!src_row_ptr || (n_edges > 0 && !src_perm))) ||
        (n_edges > 0 && (!x || !w || !src || !g_out || ((gg_x || gg_w) && !sh))))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "NULL buffer");
    const int64_t E = n_edges;
    bool wrote_g = false, wrote_sh = false, wrote_w = false, wrote_m = false;
    if (E > 0) {
        // y term, one pass: d_g_out += f(x, gg_sh, w), d_x += fx*(g; gg_sh, w),
        // d_w += fw*(g; x, gg_sh)
        if (gg_sh && (d_g_out || d_x || d_w)) {
            BwdOut o;
            o.fwd = d_g_out;
            o.acc_fwd = wrote_g;
            o.want_m = d_x != nullptr;
            o.acc_m = wrote_m;
            o.g_w = d_w;
            o.acc_w = wrote_w;
            if ((rc = run_bwd(p, x, gg_sh, w, src, dst_row_ptr, node_order, g_out, n_nodes, E, o, (char *)workspace,
                              s)))
                return rc;
            wrote_g |= d_g_out != nullptr;
            wrote_m |= d_x != nullptr;
            wrote_w |= d_w != nullptr;
        }
        // x term: d_g_out += f(gg_x, sh, w), d_sh += fsh*(g; gg_x, w), d_w += fw*(g; gg_x, sh)
        if (gg_x) {
            if (d_g_out) {
                if ((rc = run_fwd(p, gg_x, sh, w, src, dst_row_ptr, node_order, n_nodes, 1, d_g_out, wrote_g, s)))
                    return rc;
                wrote_g = true;
            }
            if (d_sh || d_w) {
                BwdOut o;
                o.g_y = d_sh;
                o.acc_y = wrote_sh;
                o.g_w = d_w;
                o.acc_w = wrote_w;
                if ((rc = run_bwd(p, gg_x, sh, w, src, dst_row_ptr, node_order, g_out, n_nodes, E, o,
                                  (char *)workspace, s)))
                    return rc;
                wrote_sh |= d_sh != nullptr;
                wrote_w |= d_w != nullptr;
            }
        }
        // w term: d_g_out += f(x, sh, gg_w), d_x += fx*(g; sh, gg_w), d_sh += fsh*(g; x, gg_w)
        if (gg_w) {
            if (d_g_out) {
                if ((rc = run_fwd(p, x, sh, gg_w, src, dst_row_ptr, node_order, n_nodes, 1, d_g_out, wrote_g, s)))
                    return rc;
                wrote_g = true;
            }
            if (d_x || d_sh) {
                BwdOut o;
                o.want_m = d_x != nullptr;
                o.acc_m = wrote_m;
                o.g_y = d_sh;
                o.acc_y = wrote_sh;
                if ((rc = run_bwd(p, x, sh, gg_w, src, dst_row_ptr, node_order, g_out, n_nodes, E, o,
                                  (char *)workspace, s)))
                    return rc;
                wrote_m |= d_x != nullptr;
                wrote_sh |= d_sh != nullptr;
            }
        }
    }
    if (d_g_out && !wrote_g && (rc = launch_zero(p.dtype, d_g_out, n_nodes * p.dim3, s))) return rc;
    if (d_x) {
        if (wrote_m) rc = launch_segment_sum_rows(p.dtype, workspace, src_row_ptr, src_perm, n_nodes, p.dim1, d_x, 0, s);
        else rc = launch_zero(p.dtype, d_x, n_nodes * p.dim1, s);
        if (rc) return rc;
    }
    if (d_sh && !wrote_sh && (rc = launch_zero(p.dtype, d_sh, E * p.dim2, s))) return rc;
    if (d_w && !wrote_w && (rc = launch_zero(p.dtype, d_w, E * p.wnumel, s))) return rc;
    return CGTP_OK;
}

}  // extern "C"
