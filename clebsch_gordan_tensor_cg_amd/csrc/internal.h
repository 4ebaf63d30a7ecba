// Internal declarations of the cgtp library (planner, code generator,
// runtime compiler and launchers).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/cgtp.h"

namespace cgtp {

constexpr int kMaxL = 6;

struct Irrep {
    int mul = 0;
    int l = 0;
    int parity = 0;  // +1 even, -1 odd, 0 unlabelled
    int dim() const { return 2 * l + 1; }
};

// One nonzero of a real coupling tensor: R[i][j][k] = c.
struct Nonzero {
    int i, j, k;
    double c;
};

struct Path {
    int i1, i2, i3;
    int l1, l2, l3;
    int mul1, mul2, mul3;
    int64_t off1, off2, off3;  // element offsets of the blocks in their rows
    int64_t woff;              // offset of the path's weights in a weight row
    int64_t wnum;              // number of weights of the path
    std::vector<double> R;     // dense [d1][d2][d3]
    std::vector<Nonzero> nz;   // nonzeros of R (|c| > 1e-14), i-major order
};

// A kernel "unit": the paths one wavefront evaluates for one item, and the
// channel slice it covers.  Units of a group share code.
struct Group {
    std::vector<int> paths;     // indices into Plan::paths
    std::vector<int> in1_blocks;
    std::vector<int> out_blocks;
    int max_mul = 0;            // channel range the group covers
    int cpl = 1;                // channels per lane
    int slices = 1;             // ceil(max_mul / (lanes_per_item * cpl))
};

struct KernelShape {
    int lanes_per_item = 64;    // LPI: lanes that share one item
    int items_per_wave = 1;     // 64 / LPI
    std::vector<Group> groups;
    int n_units = 0;            // sum of slices over groups
};

// Generator options.  Defaults are the tuned values; CGTP_TUNE (comma list
// of key=value: cpl_fwd, cpl_bwd, cpl_dbl, cpl_fb, yvec, ntw, pf, budget, stage, cypath, depth, bgy, gy64, redx, stnt, full,
// ubudget, ucpl, umma, cstage, mix2, mix3, depth_bwd, pform, pfw, pfuse, pfocc, pfma, pfml)
// overrides
// them for experiments.
struct Tuning {
    int cpl[4] = {0, 0, 0, 0};  // channels per lane per kernel kind (0 = by budget)
    int budget = 112;        // VGPR estimate allowed for two channels per lane
    bool y_vector = true;    // load the y row with vector (not scalar) loads
    int nt_w = -1;           // non-temporal loads of the per-edge weights: -1 where one item fills a
                             // wavefront (plain where items share one), 0 never, 1 always
    bool prefetch = true;    // load edge t+1 while edge t is computed
    int stage = -1;          // edges per LDS chunk of src and y rows (0 = off; -1: 64, or 32 for uvw
                             // layers without radial weights)
    int cy_path = -1;        // uniform products per path (1) or per edge (0); -1: by dtype
    int depth = 0;           // edges of prefetch in flight (staged loop; 0: 3, or 2 for uvw layers
                             // without radial weights)
    int depth_bwd = 0;       // the same for the backward, double backward and one-pass kernels (0: 2)
    bool bgy = false;        // backward via B_ij = sum_k R_ijk g_k (fewer FMAs, more VGPRs)
    bool gy64 = true;        // SH-gradient rows summed across lanes in FP64 (float plans)
    int stnt = 4;            // rows written by non-temporal stores, by kind (bit set): 1 the forward's output
                             // rows, 2 the output rows of the one-pass and double-backward kernels, 4 weight
                             // gradients, 8 x-messages; the rest by plain stores
    bool redx = true;        // cross-lane sums by VALU lane exchanges (permlane swaps, DPP) instead of
                             // shuffles through the LDS crossbar
    int full = 7;            // dispatch to the folded-flag kernels: bit 0 backward, bit 1 double backward, bit 2 fused forward+backward
    int ubudget = 0;         // uvw accumulators per lane and unit (0: 32, or 144 with radial weights)
    int ucpl = 0;            // uvw channels per lane (0: 1)
    int cstage = -1;         // uvw: each chunk's uniform CG x SH products computed once per edge into LDS
                             // (1) or by every lane of the wavefront (0); -1: 0 (measured slower)
    int mix2 = -1;           // uvw mixing: the whole contraction span staged at once, 16x16x32 MFMA (1), or
                             // 256-row steps with 16x16x16 MFMA (0); -1: the first where every block's
                             // contraction fits one span of 512 rows (C5 mixing 20.3 -> 18.1 us)
    int mix3 = -1;           // uvw mixing: the streaming form over the whole contraction (1, or -1: wherever a
                             // block's contraction is longer than one span of the second form), or never (0)
    int umma = 0;            // uvw path tensors as per-node products on the matrix cores where they fit
                             // (measured slower on the 100 x 18 atom layer: off by default)
    int pform = -1;          // uvw path tensors of graph calls from per-chunk products P_i = sum_e y_e x_e,i
                             // on the matrix cores, two nodes per wavefront (1), or the per-edge kernel
                             // (0); -1: the first wherever the plan allows it
    int pfw = 0;             // wavefronts per node pair in that kernel (0: 4)
    int pfuse = 1;           // that kernel also does the channel mixing where the plan allows it
    int pfocc = 0;           // its wavefronts per SIMD asked of the compiler (0: 4)
    int pfma = 0;            // its mixing: products whose weight rows are loaded ahead (0: 6)
    int pfml = 0;            // and whose fragments are read from LDS ahead (0: 2)
};
Tuning tuning_from_env();

// uvw plans: the paths into output block b3, concatenated along the
// contraction dimension K of the channel-mixing product T_b3 . W_b3.
struct MixBlock {
    int b3 = 0;
    int d3 = 1, mul3 = 0;
    int64_t K = 0;                 // sum over its paths of mul1 * mul2 (one copy of the paths)
    int64_t Kr = 0;                // contraction length: K times (radial hidden width + 1)
    int64_t t_off_per_item = 0;    // offset of its T region / n_items
    std::vector<int> paths;        // in path order
    std::vector<int64_t> koff;     // row offset of each path inside K
};

struct Plan {
    Tuning tune;
    std::vector<Irrep> in1, in2, out;
    std::vector<int64_t> off1, off2, off3;
    cgtp_mode mode = CGTP_UVU;
    cgtp_dtype dtype = CGTP_F32;
    uint32_t flags = 0;
    int64_t dim1 = 0, dim2 = 0, dim3 = 0, wnumel = 0;
    int lmax2 = 0;
    int sh_lmax = -1;  // input 2 is the SH row of degrees 0..sh_lmax (one copy each), else -1
    int radial_h = 0;  // uvw with per-edge weights from a radial network of this hidden width (0: none)
    std::vector<Path> paths;

    KernelShape fwd, bwd, dbl, fb;   // fb: forward and backward in one pass
    std::vector<MixBlock> mix;     // uvw only
    std::vector<int> mix_of_path;  // uvw: index into mix for each path
    int64_t t_per_item = 0;        // uvw: T elements per item
    bool uvw_mma = false;          // uvw: path tensors by the matrix-core kernel
    int uvw_mma_groups = 0;        // its workgroups per item (input-1 blocks with paths), 256 threads each
    bool uvw_pf = false;           // uvw: graph calls take the path tensors from cgtp_uvw_pf
    int uvw_pf_waves = 0;          // its wavefronts per workgroup (one workgroup per pair of nodes)
    bool uvw_pf_mix = false;       // and it does the channel mixing too (writes out, not T)
    std::string source;
    std::string cache_key;
    bool cached = false;
    bool loaded = false;
    int n_kernels = 0;

    hipModule_t module = nullptr;
    hipFunction_t k_fwd = nullptr;
    hipFunction_t k_bwd = nullptr;
    hipFunction_t k_dbl = nullptr;
    hipFunction_t k_bwd_full = nullptr;  // k_bwd with bwd_full_flags folded in
    hipFunction_t k_dbl_full = nullptr;  // k_dbl with dbl_full_flags folded in
    hipFunction_t k_fb = nullptr;        // forward + backward of the same edges in one pass
    hipFunction_t k_fb_full = nullptr;   // k_fb with fb_full_flags folded in
    hipFunction_t k_uvw_pf = nullptr;    // uvw path tensors of graph calls, per pair of nodes
    int device = -1;
};

// workspace sub-buffers start on 256-byte boundaries
inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Flags of the full, non-accumulating backward (g_w, messages, SH gradient,
// per-unit parts when there are several units) and fused double backward
// (d_w and messages); the code object holds a copy of each kernel with
// these folded in at compile time.
inline int bwd_full_flags(const Plan &p) { return 1 | 2 | 4 | (p.bwd.n_units > 1 ? 64 : 0); }
inline int dbl_full_flags(const Plan &) { return 1 | 2; }
inline int fb_full_flags(const Plan &p) { return 1 | 2 | 4 | (p.fb.n_units > 1 ? 64 : 0); }

// uvw path tensors on the matrix cores: LDS bytes of one workgroup (0 when
// the plan has no such kernel: radial weights, or no path)
size_t uvw_mma_lds_bytes(const Plan &p);
int uvw_mma_group_count(const Plan &p);
// uvw path tensors per pair of nodes on the matrix cores: whether the plan
// allows them, and the wavefronts of each pair's workgroup
bool uvw_pf_eligible(const Plan &p);
int uvw_pf_wave_count(const Plan &p);
bool uvw_pf_mixes(const Plan &p);   // that kernel also does the channel mixing (no T in memory)
constexpr size_t kUvwMmaMaxLds = 64 * 1024;   // static LDS of one workgroup

// planner
int parse_irreps(const char *s, std::vector<Irrep> &out, std::string &err);
int real_coupling(int l1, int l2, int l3, std::vector<double> &R, std::string &err);
void choose_shapes(Plan &p);
// the plan's paths, work split and tuning on stderr (CGTP_DEBUG)
void dump_plan(const Plan &p);

// code generation
std::string generate_source(const Plan &p);

// runtime compilation and cache
int compile_and_load(Plan &p, bool load, std::string &err);

// opt-in per-launch timing (timing.cpp): records HIP events around a launch
class TimedLaunch {
  public:
    TimedLaunch(const char *name, hipStream_t s);
    ~TimedLaunch();
    TimedLaunch(const TimedLaunch &) = delete;
    TimedLaunch &operator=(const TimedLaunch &) = delete;

  private:
    hipStream_t s_;
    long idx_ = -1;
};
#define CGTP_LAUNCH(name, stream, ...)               \
    do {                                             \
        ::cgtp::TimedLaunch cgtp_tl_(name, stream);  \
        hipLaunchKernelGGL(__VA_ARGS__);             \
    } while (0)

// error state
int set_error(int code, const std::string &msg);
void clear_error();

// launch helpers for the fixed kernels (kernels.hip)
int launch_segment_sum_rows(cgtp_dtype dt, const void *rows, const int32_t *row_ptr,
                            const int32_t *perm, int64_t n_seg, int64_t width, void *out,
                            int accumulate, hipStream_t s);
int launch_sum_parts(cgtp_dtype dt, const void *parts, int n_parts, int64_t n, void *out,
                     int accumulate, hipStream_t s);
int launch_zero(cgtp_dtype dt, void *p, int64_t n, hipStream_t s);
// inv[perm[k]] = k for k < n
// forces from (a sum of n_parts partial) SH gradients, v: n_edges x 3 scratch
int launch_sh_forces(int lmax, cgtp_dtype dt, const void *vec, const int32_t *perm, const void *g_sh, int n_parts,
                     int64_t part_stride, const int32_t *dst_row_ptr, const int32_t *src_row_ptr,
                     const int32_t *src_perm, int64_t n_nodes, int64_t n_edges, void *F, void *v, hipStream_t s);
// out[item][off3 + w*d3 + k] (=|+=) sum_K T[(item*d3 + k)*K + kk] W_b3[kk][w]
// channel mixing of every output block of a uvw layer (T: path tensors)
int launch_uvw_mix(const Plan &p, const void *T, const void *w, int64_t n_items, void *out, int accumulate,
                   void *part, hipStream_t s);
// bytes of partial tiles the mixing of n_items rows needs (split contraction)
size_t mix_part_bytes(const Plan &p, int64_t n_items);

}  // namespace cgtp

struct cgtp_plan_s {
    cgtp::Plan p;
};
