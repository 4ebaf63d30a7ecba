// Planner: irreps parsing, path enumeration and validation, real coupling
// tensors, and the split of the work into wavefront units.
//
// "An Efficient Sparse Kernel Generator for O(3)-Equivariant Deep
// Networks" (abstract) does the tensor product's analysis once, at model
// compile time, and emits kernels specialised to it; this file is that
// analysis.  The coupling tensors follow the textbook construction
// (Clebsch-Gordan coefficients by the Racah formula, then a change of every
// index to the real spherical-harmonic basis).
#include <cmath>
#include <complex>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <algorithm>
#include <functional>
#include <numeric>
#include <string>

#include "internal.h"

namespace cgtp {

// ---------------------------------------------------------------------------
// Irreps grammar: term ('+' term)*, term = MUL 'x' L [e|o]
// ---------------------------------------------------------------------------
int parse_irreps(const char *s, std::vector<Irrep> &out, std::string &err) {
    out.clear();
    if (!s) {
        err = "irreps string is NULL";
        return CGTP_ERR_INVALID_ARGUMENT;
    }
    const char *c = s;
    auto skip = [&]() {
        while (*c == ' ' || *c == '\t') ++c;
    };
    auto number = [&](long &v) -> bool {
        skip();
        if (*c < '0' || *c > '9') return false;
        v = 0;
        while (*c >= '0' && *c <= '9') {
            v = v * 10 + (*c - '0');
            if (v > (1L << 30)) return false;
            ++c;
        }
        return true;
    };
    int labelled = -1;
    for (;;) {
        Irrep ir;
        long mul, l;
        if (!number(mul)) break;
        skip();
        if (*c != 'x') break;
        ++c;
        if (!number(l)) break;
        skip();
        int par = 0;
        if (*c == 'e') par = 1, ++c;
        else if (*c == 'o') par = -1, ++c;
        int lab = par != 0;
        if (labelled >= 0 && lab != labelled) {
            err = std::string("mixed parity-labelled and unlabelled irreps in '") + s + "'";
            return CGTP_ERR_INVALID_ARGUMENT;
        }
        labelled = lab;
        if (mul <= 0) {
            err = std::string("multiplicity must be positive in '") + s + "'";
            return CGTP_ERR_INVALID_ARGUMENT;
        }
        ir.mul = (int)mul;
        ir.l = (int)l;
        ir.parity = par;
        out.push_back(ir);
        skip();
        if (*c == '+') {
            ++c;
            continue;
        }
        if (*c == 0) return CGTP_OK;
        break;
    }
    err = std::string("cannot parse irreps '") + s + "' near offset " + std::to_string(c - s);
    return CGTP_ERR_INVALID_ARGUMENT;
}

// ---------------------------------------------------------------------------
// Real coupling tensors
// ---------------------------------------------------------------------------
namespace {

using cld = std::complex<long double>;

long double factorial_ld(int n) {
    static long double tab[64];
    static std::once_flag once;
    std::call_once(once, [] {
        tab[0] = 1.0L;
        for (int i = 1; i < 64; ++i) tab[i] = tab[i - 1] * (long double)i;
    });
    return tab[n];
}

// <l1 m1 l2 m2 | l3 m3>, Condon-Shortley convention (Racah's closed form).
long double clebsch_gordan(int l1, int m1, int l2, int m2, int l3, int m3) {
    if (m1 + m2 != m3) return 0.0L;
    if (std::abs(m1) > l1 || std::abs(m2) > l2 || std::abs(m3) > l3) return 0.0L;
    if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) return 0.0L;
    const long double tri = factorial_ld(l1 + l2 - l3) * factorial_ld(l1 - l2 + l3) *
                            factorial_ld(-l1 + l2 + l3) / factorial_ld(l1 + l2 + l3 + 1);
    const long double mfac = factorial_ld(l1 + m1) * factorial_ld(l1 - m1) *
                             factorial_ld(l2 + m2) * factorial_ld(l2 - m2) *
                             factorial_ld(l3 + m3) * factorial_ld(l3 - m3);
    // summation index z runs where every factorial argument is >= 0
    const int zmin = std::max({0, l2 - l3 - m1, l1 - l3 + m2});
    const int zmax = std::min({l1 + l2 - l3, l1 - m1, l2 + m2});
    long double sum = 0.0L;
    for (int z = zmin; z <= zmax; ++z) {
        long double den = factorial_ld(z) * factorial_ld(l1 + l2 - l3 - z) *
                          factorial_ld(l1 - m1 - z) * factorial_ld(l2 + m2 - z) *
                          factorial_ld(l3 - l2 + m1 + z) * factorial_ld(l3 - l1 - m2 + z);
        sum += ((z & 1) ? -1.0L : 1.0L) / den;
    }
    return std::sqrt((2.0L * l3 + 1.0L) * tri * mfac) * sum;
}

// Real harmonic of order m (degree l) as a combination of complex ones:
// up to two (mu, coefficient) terms.
struct Term {
    int mu;
    cld a;
};
int real_from_complex(int m, Term out[2]) {
    const long double h = 1.0L / std::sqrt(2.0L);
    const long double sgn = (std::abs(m) & 1) ? -1.0L : 1.0L;
    if (m == 0) {
        out[0] = {0, cld(1.0L, 0.0L)};
        return 1;
    }
    if (m > 0) {
        out[0] = {-m, cld(h, 0.0L)};
        out[1] = {m, cld(sgn * h, 0.0L)};
        return 2;
    }
    out[0] = {m, cld(0.0L, h)};
    out[1] = {-m, cld(0.0L, -sgn * h)};
    return 2;
}

}  // namespace

int real_coupling(int l1, int l2, int l3, std::vector<double> &R, std::string &err) {
    if (l1 < 0 || l2 < 0 || l3 < 0 || l1 > kMaxL || l2 > kMaxL || l3 > kMaxL) {
        err = "degree above 6 is not supported";
        return CGTP_ERR_UNSUPPORTED;
    }
    if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) {
        err = "degrees violate the triangle rule";
        return CGTP_ERR_INVALID_ARGUMENT;
    }
    const int d1 = 2 * l1 + 1, d2 = 2 * l2 + 1, d3 = 2 * l3 + 1;
    const bool odd = ((l1 + l2 + l3) & 1) != 0;
    R.assign((size_t)d1 * d2 * d3, 0.0);
    for (int m1 = -l1; m1 <= l1; ++m1) {
        Term t1[2];
        const int n1 = real_from_complex(m1, t1);
        for (int m2 = -l2; m2 <= l2; ++m2) {
            Term t2[2];
            const int n2 = real_from_complex(m2, t2);
            for (int m3 = -l3; m3 <= l3; ++m3) {
                Term t3[2];
                const int n3 = real_from_complex(m3, t3);
                cld acc(0.0L, 0.0L);
                for (int a = 0; a < n1; ++a)
                    for (int b = 0; b < n2; ++b)
                        for (int c = 0; c < n3; ++c) {
                            if (t1[a].mu + t2[b].mu != t3[c].mu) continue;
                            const long double cg =
                                clebsch_gordan(l1, t1[a].mu, l2, t2[b].mu, l3, t3[c].mu);
                            acc += t3[c].a * std::conj(t1[a].a) * std::conj(t2[b].a) * cg;
                        }
                R[((size_t)(m1 + l1) * d2 + (m2 + l2)) * d3 + (m3 + l3)] =
                    (double)(odd ? acc.imag() : acc.real());
            }
        }
    }
    return CGTP_OK;
}

// ---------------------------------------------------------------------------
// Work split.  Each wavefront evaluates one group of paths for one item
// (node or sample) over a slice of channels.  Groups are the connected
// components of "shares an input-1 block or an output block", so every
// output block and every input-1 block is owned by exactly one group: the
// forward writes each output block once, and the backward's per-edge
// input-1 messages are written by exactly one wavefront.
// ---------------------------------------------------------------------------
namespace {

int next_pow2(int v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// kind: 0 forward, 1 backward, 2 fused double backward, 3 forward and backward in one pass
void split(Plan &p, KernelShape &ks, int kind) {
    const int np = (int)p.paths.size();
    std::vector<int> parent(np);
    std::iota(parent.begin(), parent.end(), 0);
    std::function<int(int)> find = [&](int a) { return parent[a] == a ? a : parent[a] = find(parent[a]); };
    for (int a = 0; a < np; ++a)
        for (int b = a + 1; b < np; ++b)
            if (p.paths[a].i1 == p.paths[b].i1 || p.paths[a].i3 == p.paths[b].i3)
                parent[find(a)] = find(b);
    ks.groups.clear();
    std::vector<int> gid(np, -1);
    for (int a = 0; a < np; ++a) {
        int r = find(a);
        if (gid[r] < 0) {
            gid[r] = (int)ks.groups.size();
            ks.groups.emplace_back();
        }
        Group &g = ks.groups[gid[r]];
        g.paths.push_back(a);
        auto add = [](std::vector<int> &v, int x) {
            for (int y : v)
                if (y == x) return;
            v.push_back(x);
        };
        add(g.in1_blocks, p.paths[a].i1);
        add(g.out_blocks, p.paths[a].i3);
        g.max_mul = std::max(g.max_mul, std::max(p.paths[a].mul1, p.paths[a].mul3));
    }
    int max_mul = 0;
    for (auto &g : ks.groups) max_mul = std::max(max_mul, g.max_mul);
    ks.lanes_per_item = max_mul >= 64 ? 64 : next_pow2(std::max(1, max_mul));
    ks.items_per_wave = 64 / ks.lanes_per_item;
    const int wide = (p.dtype == CGTP_F64) ? 2 : 1;
    ks.n_units = 0;
    for (auto &g : ks.groups) {
        // registers per channel held across the edge loop: accumulators (or
        // the cotangent row), operands of the current and the prefetched
        // edge, and the backward's message accumulators
        int acc = 0, xin = 0, wts = 0;
        for (int b : g.out_blocks) acc += p.out[b].dim();
        for (int b : g.in1_blocks) xin += p.in1[b].dim();
        for (int a : g.paths) wts += p.paths[a].mul2;
        int per_ch = acc + (1 + std::max(1, kind == 0 ? p.tune.depth : p.tune.depth_bwd)) * (xin + wts);
        if (kind >= 1) per_ch += xin;  // message accumulators
        if (kind >= 2) per_ch += acc;  // fused forward accumulators
        per_ch *= wide;
        g.cpl = 1;
        if (ks.lanes_per_item == 64 && g.max_mul > 64 && per_ch * 2 <= p.tune.budget) g.cpl = 2;
        if (p.tune.cpl[kind] > 0 && ks.lanes_per_item == 64) g.cpl = p.tune.cpl[kind];
        g.slices = (g.max_mul + ks.lanes_per_item * g.cpl - 1) / (ks.lanes_per_item * g.cpl);
        ks.n_units += g.slices;
    }
}

}  // namespace

Tuning tuning_from_env() {
    Tuning t;
    const char *e = std::getenv("CGTP_TUNE");
    if (!e) return t;
    std::string s = e;
    size_t pos = 0;
    while (pos < s.size()) {
        size_t comma = s.find(',', pos);
        if (comma == std::string::npos) comma = s.size();
        std::string kv = s.substr(pos, comma - pos);
        size_t eq = kv.find('=');
        if (eq != std::string::npos) {
            std::string k = kv.substr(0, eq);
            int v = std::atoi(kv.c_str() + eq + 1);
            if (k == "cpl_fwd") t.cpl[0] = v;
            else if (k == "cpl_bwd") t.cpl[1] = v;
            else if (k == "cpl_dbl") t.cpl[2] = v;
            else if (k == "cpl_fb") t.cpl[3] = v;
            else if (k == "budget") t.budget = v;
            else if (k == "yvec") t.y_vector = v != 0;
            else if (k == "ntw") t.nt_w = v < 0 ? -1 : (v != 0);
            else if (k == "pf") t.prefetch = v != 0;
            else if (k == "stage") t.stage = v < 0 ? 0 : (v > 256 ? 256 : v);
            else if (k == "cypath") t.cy_path = v;
            else if (k == "depth") t.depth = v < 1 ? 1 : (v > 4 ? 4 : v);
            else if (k == "depth_bwd") t.depth_bwd = v < 1 ? 1 : (v > 4 ? 4 : v);
            else if (k == "bgy") t.bgy = v != 0;
            else if (k == "gy64") t.gy64 = v != 0;
            else if (k == "redx") t.redx = v != 0;
            else if (k == "stnt") t.stnt = v & 15;
            else if (k == "full") t.full = v & 7;
            else if (k == "ubudget") t.ubudget = v < 1 ? 0 : v;
            else if (k == "ucpl") t.ucpl = v < 1 ? 0 : (v > 8 ? 8 : v);
            else if (k == "umma") t.umma = v != 0;
            else if (k == "pform") t.pform = v;
            else if (k == "pfw") t.pfw = v;
            else if (k == "pfuse") t.pfuse = v;
            else if (k == "pfocc") t.pfocc = v;
            else if (k == "pfma") t.pfma = v;
            else if (k == "mix3") t.mix3 = v;
            else if (k == "pfml") t.pfml = v;
            else if (k == "cstage") t.cstage = v != 0;
            else if (k == "mix2") t.mix2 = v < 0 ? -1 : (v != 0);
        }
        pos = comma + 1;
    }
    return t;
}

// uvw: every path writes its own slice of T, so groups are the input-1
// blocks, split further into units of at most `budget` accumulators per
// channel.
void split_uvw(Plan &p, KernelShape &ks) {
    ks.groups.clear();
    int max_mul = 0;
    for (auto &P : p.paths) max_mul = std::max(max_mul, P.mul1);
    // cpl channels per lane share each edge's uniform products
    const int cpl = p.tune.ucpl > 0 ? p.tune.ucpl : 1;
    const int lanes = (max_mul + cpl - 1) / cpl;
    ks.lanes_per_item = lanes >= 64 ? 64 : next_pow2(std::max(1, lanes));
    ks.items_per_wave = 64 / ks.lanes_per_item;
    // accumulators per lane: one per (path, v, k) and channel slot, times H+1
    // with radial weights; defaults from sweeps of the 44-path l <= 6 layer
    // (100 x 18 atoms)
    const int budget = (p.tune.ubudget > 0 ? p.tune.ubudget : (p.radial_h > 0 ? 144 : 32)) / cpl;
    for (int b = 0; b < (int)p.in1.size(); ++b) {
        Group cur;
        int acc = 0;
        for (int a = 0; a < (int)p.paths.size(); ++a) {
            const Path &P = p.paths[a];
            if (P.i1 != b) continue;
            const int need = P.mul2 * (2 * P.l3 + 1) * (p.radial_h + 1);
            if (!cur.paths.empty() && acc + need > budget) {
                ks.groups.push_back(cur);
                cur = Group();
                acc = 0;
            }
            cur.paths.push_back(a);
            if (cur.in1_blocks.empty()) cur.in1_blocks.push_back(b);
            cur.max_mul = std::max(cur.max_mul, P.mul1);
            acc += need;
        }
        if (!cur.paths.empty()) ks.groups.push_back(cur);
    }
    ks.n_units = 0;
    for (auto &g : ks.groups) {
        g.cpl = cpl;
        g.slices = (g.max_mul + ks.lanes_per_item * cpl - 1) / (ks.lanes_per_item * cpl);
        ks.n_units += g.slices;
    }
}

void mix_tables(Plan &p) {
    p.mix.clear();
    p.mix_of_path.assign(p.paths.size(), -1);
    int64_t off = 0;
    for (int b3 = 0; b3 < (int)p.out.size(); ++b3) {
        MixBlock mb;
        mb.b3 = b3;
        mb.d3 = p.out[b3].dim();
        mb.mul3 = p.out[b3].mul;
        for (int a = 0; a < (int)p.paths.size(); ++a)
            if (p.paths[a].i3 == b3) {
                mb.koff.push_back(mb.K);
                mb.K += (int64_t)p.paths[a].mul1 * p.paths[a].mul2;
                mb.paths.push_back(a);
                p.mix_of_path[a] = (int)p.mix.size();
            }
        if (mb.paths.empty()) continue;
        // radial: columns (h, path, u, v), h = 0..H, each h a full copy of the paths
        mb.Kr = mb.K * (p.radial_h + 1);
        mb.t_off_per_item = off;
        off += mb.d3 * mb.Kr;
        p.mix.push_back(mb);
    }
    p.t_per_item = off;
}

void choose_shapes(Plan &p) {
    // uniform products per path where registers are tight: FP64 (two VGPRs
    // each) and the bf16 uvw layers (SH rows up to l = 6); per edge otherwise
    if (p.tune.cy_path < 0) p.tune.cy_path = (p.dtype == CGTP_F64 || p.dtype == CGTP_BF16_F32ACC) ? 1 : 0;
    // uvw layers without radial weights: shorter chunks (a quarter of the LDS
    // per wavefront) and two edges in flight measured faster (sweep of the
    // 100 x 18 atom layer: 47 against 50 us); the radial form keeps 64 and 3
    const bool uvw_plain = p.mode == CGTP_UVW && p.radial_h == 0;
    if (p.tune.stage < 0) p.tune.stage = uvw_plain ? 32 : 64;
    if (p.tune.depth <= 0) p.tune.depth = uvw_plain ? 2 : 3;
    // the backward kinds: two edges in flight (C4 one-pass and double backward
    // 583.5 against 586.5 us with three; the forward is faster with three)
    if (p.tune.depth_bwd <= 0) p.tune.depth_bwd = 2;
    // the uniform products of an edge made once into LDS (one lane per edge)
    // instead of by every lane: measured slower on the 100 x 18 atom layer
    // (66 against 49 us; radial 211 against 148 us: 174 VGPRs, half the
    // occupancy), so off unless asked for
    if (p.tune.cstage < 0) p.tune.cstage = 0;
    if (p.mode == CGTP_UVW) {
        mix_tables(p);
        split_uvw(p, p.fwd);
        const size_t lds = uvw_mma_lds_bytes(p);
        p.uvw_mma = p.tune.umma && lds > 0 && lds <= kUvwMmaMaxLds;
        p.uvw_mma_groups = p.uvw_mma ? uvw_mma_group_count(p) : 0;
        // the per-pair matrix-core form unless switched off, or the per-node
        // one asked for instead
        p.uvw_pf = (p.tune.pform > 0 || (p.tune.pform < 0 && !p.uvw_mma)) && uvw_pf_eligible(p);
        p.uvw_pf_waves = p.uvw_pf ? uvw_pf_wave_count(p) : 0;
        p.uvw_pf_mix = p.uvw_pf && uvw_pf_mixes(p);
        return;
    }
    split(p, p.fwd, 0);
    split(p, p.bwd, 1);
    split(p, p.dbl, 2);
    split(p, p.fb, 3);
}


// Plan dump (CGTP_DEBUG set in the environment): the paths with their
// nonzero counts, each kernel kind's work split and the tuning in force,
// one plan per block on stderr.
void dump_plan(const Plan &p) {
    auto irs = [](const std::vector<Irrep> &v) {
        std::string o;
        for (const Irrep &ir : v) {
            if (!o.empty()) o += "+";
            o += std::to_string(ir.mul) + "x" + std::to_string(ir.l) +
                 (ir.parity > 0 ? "e" : ir.parity < 0 ? "o" : "");
        }
        return o;
    };
    auto list = [](const std::vector<int> &v) {
        std::string o;
        for (int x : v) o += (o.empty() ? "" : " ") + std::to_string(x);
        return o;
    };
    const char *dt = p.dtype == CGTP_F64 ? "f64" : p.dtype == CGTP_F32 ? "f32" : "bf16-f32acc";
    std::fprintf(stderr, "cgtp plan: %s (dim %lld) x %s (dim %lld) -> %s (dim %lld), %s, %s, flags 0x%x\n",
                 irs(p.in1).c_str(), (long long)p.dim1, irs(p.in2).c_str(), (long long)p.dim2, irs(p.out).c_str(),
                 (long long)p.dim3, p.mode == CGTP_UVW ? "uvw" : "uvu", dt, p.flags);
    size_t nnz = 0;
    for (size_t a = 0; a < p.paths.size(); ++a) {
        const Path &P = p.paths[a];
        nnz += P.nz.size();
        std::fprintf(stderr, "  path %zu: blocks (%d, %d, %d), l (%d x %d -> %d), mul %d x %d -> %d, %zu nonzeros, "
                             "weights at %lld\n",
                     a, P.i1, P.i2, P.i3, P.l1, P.l2, P.l3, P.mul1, P.mul2, P.mul3, P.nz.size(), (long long)P.woff);
    }
    std::fprintf(stderr, "  %zu paths, %zu nonzeros, %lld weights per item, SH degree in the kernels %d\n",
                 p.paths.size(), nnz, (long long)p.wnumel, p.sh_lmax);
    const char *names[] = {"forward", "backward", "double backward", "forward+backward"};
    const KernelShape *shapes[] = {&p.fwd, &p.bwd, &p.dbl, &p.fb};
    for (int k = 0; k < 4; ++k) {
        const KernelShape &ks = *shapes[k];
        if (ks.groups.empty()) continue;
        std::fprintf(stderr, "  %s: %d lanes per item, %d items per wavefront, %d units\n", names[k],
                     ks.lanes_per_item, ks.items_per_wave, ks.n_units);
        for (size_t gi = 0; gi < ks.groups.size(); ++gi) {
            const Group &g = ks.groups[gi];
            std::fprintf(stderr, "    group %zu: paths [%s], input-1 blocks [%s], output blocks [%s], %d channels, "
                                 "%d per lane, %d slices\n",
                         gi, list(g.paths).c_str(), list(g.in1_blocks).c_str(), list(g.out_blocks).c_str(), g.max_mul,
                         g.cpl, g.slices);
        }
    }
    const Tuning &t = p.tune;
    std::fprintf(stderr, "  tuning: depth %d, depth_bwd %d, stage %d, budget %d, gy64 %d, redx %d, stnt %d, full %d, "
                         "bgy %d, pform %d, pfuse %d\n",
                 t.depth, t.depth_bwd, t.stage, t.budget, (int)t.gy64, (int)t.redx, t.stnt, t.full, (int)t.bgy,
                 t.pform, t.pfuse);
    std::fprintf(stderr, "  generated source: %zu bytes, %d kernels, code object %s\n", p.source.size(), p.n_kernels,
                 p.cached ? "from the cache" : "compiled");
}

}  // namespace cgtp
