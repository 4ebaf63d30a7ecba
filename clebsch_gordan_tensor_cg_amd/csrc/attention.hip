// Graph sparse attention on the matrix cores ("Fused3S: Fast Sparse
// Attention on Tensor Cores", abstract): the three sparse steps -- sampled
// dense-dense product (SDDMM), row softmax and sparse-dense product (SpMM)
// -- fused in one kernel, so the scores never leave the chip.
//
//   s_e = scale <q[i][h], k[j][h]>  for every edge e = (j -> i) of the CSR
//   out[i][h] = sum_e softmax_i(s)_e v[j][h]
//
// MI355X design: rows are taken in windows of 16 consecutive destination
// rows (the M/N size of the 16x16x16 bf16 MFMA).  A first kernel compacts
// each window's edges in LDS: keys (column, row) are sorted, and each
// distinct column becomes one column of the window with a 16-bit mask of
// the rows that hold it.  A second kernel takes one (window, head) per
// workgroup and processes the distinct columns 16 at a time:
//   S^T = K_cols Q^T          one MFMA per 16 of the head dimension
//   online softmax per row    (running max and sum, masked entries = 0)
//   O  += P V_cols            P rounded to bf16, FP32 accumulation
// Computing S transposed leaves each lane with four scores of one row, which
// is exactly the A-operand layout that the P V product needs, so P never
// goes through LDS.  Windows with more edges than fit in LDS are compacted
// in batches whose entries follow one another.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <string>

#include "internal.h"

namespace cgtp {
namespace {

constexpr int kWin = 16;         // destination rows per window
constexpr int kCap = 2048;       // window edges compacted per batch
constexpr int kThreads = 256;    // four wavefronts, one head each
constexpr int kMaxChunks = 8;    // head dimension up to 128
constexpr int kDepth = 2;        // tiles loaded ahead of the one computed

typedef short a_s4 __attribute__((ext_vector_type(4)));
typedef float a_f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ short to_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7fffu + ((u >> 16) & 1u);   // round to nearest even
    return (short)(u >> 16);
}

// Window compaction: the edges of 16 consecutive rows, taken kCap at a time,
// sorted by (column, row); each distinct column of a batch becomes one entry
// (column, 16-bit mask of the rows holding it).  The entries of window w go
// to [row_ptr[16 w] + 16 w, ...), padded with empty entries to a multiple of
// 16; win_n[w] = their padded count.  Batches of a window with more than kCap
// edges follow one another (a column may then appear once per batch, each
// time with its own rows).
__global__ void __launch_bounds__(kThreads) k_attention_compact(const int32_t *__restrict__ col,
                                                                 const int32_t *__restrict__ row_ptr, int64_t n_rows,
                                                                 int64_t n_cols, int32_t *__restrict__ ucol,
                                                                 uint16_t *__restrict__ umask,
                                                                 int32_t *__restrict__ win_n) {
    __shared__ uint32_t key[kCap];
    __shared__ int32_t rp[kWin + 1];
    __shared__ int32_t part[kThreads];
    __shared__ int32_t n_unique;
    const int64_t w = blockIdx.x, r0 = w * kWin;
    const int nrw = (int)std::min<int64_t>(kWin, n_rows - r0);
    if (threadIdx.x <= kWin) rp[threadIdx.x] = row_ptr[r0 + std::min<int>(threadIdx.x, nrw)];
    __syncthreads();
    const int e_beg = rp[0], e_end = rp[nrw];
    const int64_t base = (int64_t)e_beg + kWin * w;   // first entry of the window
    int written = 0;                                  // entries of the window so far
    for (int b0 = e_beg; b0 < e_end; b0 += kCap) {
        const int nb = std::min(kCap, e_end - b0);
        int np2 = 1;
        while (np2 < nb) np2 <<= 1;
        // keys of the batch; edges whose column is out of range are dropped
        for (int t = threadIdx.x; t < np2; t += kThreads) {
            uint32_t kv = 0xffffffffu;
            if (t < nb) {
                const int e = b0 + t;
                int r = 0;
                while (r + 1 < nrw && rp[r + 1] <= e) ++r;
                const int32_t c = col[e];
                if (c >= 0 && c < n_cols) kv = ((uint32_t)c << 4) | (uint32_t)r;
            }
            key[t] = kv;
        }
        __syncthreads();
        // bitonic sort of key[0, np2)
        for (int size = 2; size <= np2; size <<= 1)
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int t = threadIdx.x; t < np2 / 2; t += kThreads) {
                    const int lo = 2 * t - (t & (stride - 1)), hi = lo + stride;
                    const uint32_t a = key[lo], b = key[hi];
                    if ((a > b) == ((lo & size) == 0)) {
                        key[lo] = b;
                        key[hi] = a;
                    }
                }
                __syncthreads();
            }
        // each thread owns a run of sorted keys: count the run heads, scan,
        // then write its distinct columns and their row masks
        const int per = (nb + kThreads - 1) / kThreads;
        const int t0 = threadIdx.x * per, t1 = std::min(nb, t0 + per);
        int heads = 0;
        for (int t = t0; t < t1; ++t) {
            const uint32_t kv = key[t];
            if (kv != 0xffffffffu && (t == 0 || (key[t - 1] >> 4) != (kv >> 4))) ++heads;
        }
        part[threadIdx.x] = heads;
        __syncthreads();
        if (threadIdx.x == 0) {
            int run = 0;
            for (int i = 0; i < kThreads; ++i) {
                const int c = part[i];
                part[i] = run;
                run += c;
            }
            n_unique = run;
        }
        __syncthreads();
        int u = written + part[threadIdx.x];
        for (int t = t0; t < t1; ++t) {
            const uint32_t kv = key[t];
            if (kv == 0xffffffffu || (t > 0 && (key[t - 1] >> 4) == (kv >> 4))) continue;
            uint32_t m = 0;
            for (int t2 = t; t2 < nb && key[t2] != 0xffffffffu && (key[t2] >> 4) == (kv >> 4); ++t2)
                m |= 1u << (key[t2] & 15u);
            ucol[base + u] = (int32_t)(kv >> 4);
            umask[base + u] = (uint16_t)m;
            ++u;
        }
        written += n_unique;
        __syncthreads();   // key, part and n_unique are reused by the next batch
    }
    const int padded = (written + 15) & ~15;
    for (int t = written + threadIdx.x; t < padded; t += kThreads) {
        ucol[base + t] = -1;
        umask[base + t] = 0;
    }
    if (threadIdx.x == 0) win_n[w] = padded;
}

// Layout of the compacted windows inside the caller's buffer.
struct AttnLayout {
    int32_t *ucol;
    uint16_t *umask;
    int32_t *win_n;
    size_t bytes;
    AttnLayout(void *p, int64_t n_rows, int64_t n_edges) {
        const size_t n_win = (size_t)((n_rows + kWin - 1) / kWin);
        const size_t cap = (size_t)n_edges + kWin * n_win;
        ucol = (int32_t *)p;
        umask = (uint16_t *)((char *)p + align256(cap * sizeof(int32_t)));
        win_n = (int32_t *)((char *)umask + align256(cap * sizeof(uint16_t)));
        bytes = align256(cap * sizeof(int32_t)) + align256(cap * sizeof(uint16_t)) + align256(n_win * sizeof(int32_t));
    }
};

// One workgroup per (window, head); its four wavefronts take every fourth
// 16-column tile of the window and keep their own running softmax, merged
// through LDS at the end.  The next tile's K and V operands are loaded
// before the current tile is computed.
template <int NC>   // head dimension = 16 NC
__global__ void __launch_bounds__(kThreads) k_sparse_attention_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ ucol, const uint16_t *__restrict__ umask,
    const int32_t *__restrict__ win_n, int64_t n_rows, int H, float scale, float *__restrict__ out) {
    constexpr int kWaves = kThreads / 64;
    constexpr int kMaxChunks = NC, nchunk = NC, D = 16 * NC;
    __shared__ float s_m[kWaves][kWin], s_l[kWaves][kWin];
    __shared__ float s_o[kWaves][kWin][D];
    const int64_t w = blockIdx.x, r0 = w * kWin;
    const int h = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rq = lane & 15, quad = lane >> 4;
    const int nrw = (int)std::min<int64_t>(kWin, n_rows - r0);
    const int64_t base = (int64_t)row_ptr[r0] + kWin * w;
    const int ntile = win_n[w] / 16;

    // Q^T fragments (B operand: B[kk][r] = q[r0 + r][h][kk]); lane holds row
    // rq, head-dimension entries 4 quad..+3 of each chunk of 16
    a_s4 qf[kMaxChunks];
    a_f4 acc[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        qf[c] = a_s4{0, 0, 0, 0};
        acc[c] = a_f4{0.f, 0.f, 0.f, 0.f};
        if (c < nchunk && rq < nrw) qf[c] = *(const a_s4 *)(q + ((r0 + rq) * H + h) * (int64_t)D + c * 16 + 4 * quad);
    }
    float m_run = -INFINITY, l_run = 0.f;   // softmax state of row rq

    // operands of one tile: K rows (A operand), V entries (B operand) and
    // the row masks; kDepth tiles are in flight ahead of the one computed
    struct Tile {
        a_s4 ka[kMaxChunks], vb[kMaxChunks];
        uint32_t mk[4];
    };
    auto load_tile = [&](int tile, Tile &T) {
        if (tile >= ntile) return;
        const int64_t e0 = base + 16 * (int64_t)tile;
        const int ca = ucol[e0 + rq];
        int cv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            cv[i] = ucol[e0 + 4 * quad + i];
            T.mk[i] = umask[e0 + 4 * quad + i];
        }
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            if (c >= nchunk) break;
            T.ka[c] = ca >= 0 ? *(const a_s4 *)(k + ((int64_t)ca * H + h) * D + c * 16 + 4 * quad) : a_s4{0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                T.vb[c][i] = cv[i] >= 0 ? (short)v[((int64_t)cv[i] * H + h) * D + c * 16 + rq] : (short)0;
        }
    };
    Tile ring[kDepth + 1];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) load_tile(wave + d * kWaves, ring[d]);
    for (int tile = wave; tile < ntile; tile += kWaves) {
        load_tile(tile + kDepth * kWaves, ring[kDepth]);
        const Tile &T = ring[0];
        // S^T[c][r] = <k[col c], q[r]>; lane holds S[row rq][columns 4 quad + i]
        a_f4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            if (c >= nchunk) break;
            st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(T.ka[c], qf[c], st, 0, 0, 0);
        }
        float s[4], p[4];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[i] = ((T.mk[i] >> rq) & 1u) ? st[i] * scale : -INFINITY;
            tmax = fmaxf(tmax, s[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float corr = m_new == -INFINITY ? 1.f : __expf(m_run - m_new);
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = s[i] == -INFINITY ? 0.f : __expf(s[i] - m_new);
            psum += p[i];
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l_run = l_run * corr + psum;
        m_run = m_new;
        // the accumulator rows are 4 quad + i: their corrections
        float co[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) co[i] = __shfl(corr, 4 * quad + i, 64);
        // P is already in the A-operand layout: lane holds P[row rq][4 quad + i]
        const a_s4 pa = {to_bf16(p[0]), to_bf16(p[1]), to_bf16(p[2]), to_bf16(p[3])};
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c) {
            if (c >= nchunk) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[c][i] *= co[i];
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, T.vb[c], acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int d = 0; d < kDepth; ++d) ring[d] = ring[d + 1];
    }
    // merge the wavefronts' states: O = sum_w O_w e^(m_w - M) / sum_w l_w e^(m_w - M)
    if (quad == 0) {
        s_m[wave][rq] = m_run;
        s_l[wave][rq] = l_run;
    }
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        if (c >= nchunk) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[wave][4 * quad + i][16 * c + rq] = acc[c][i];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < nrw * D; idx += kThreads) {
        const int r = idx / D, dd = idx % D;
        float M = -INFINITY;
        for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, s_m[wv][r]);
        float num = 0.f, den = 0.f;
        if (M != -INFINITY)
            for (int wv = 0; wv < kWaves; ++wv) {
                const float f = s_m[wv][r] == -INFINITY ? 0.f : __expf(s_m[wv][r] - M);
                num += s_o[wv][r][dd] * f;
                den += s_l[wv][r] * f;
            }
        out[((r0 + r) * H + h) * D + dd] = den > 0.f ? num / den : 0.f;
    }
}

int hip_ok(hipError_t e, const char *what) {
    if (e == hipSuccess) return CGTP_OK;
    return set_error(CGTP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Row form: one group of D/4 lanes per (row, head), four head dimensions per
// lane (one 8-byte load of k and of v per edge), the row's edges walked in
// order with an online softmax in FP32.  For graphs whose 16-row windows
// share few columns (random numbering: about one row per distinct column),
// the window kernel's 16 x 16 tiles are nearly empty; here every lane does
// useful work, k and v rows are read once per edge from the caches, and no
// layout is needed.  P is not rounded (FP32 throughout after the bf16 loads).
// LPH: lanes per head (D / 4, a power of two).  A wavefront holds 64 / LPH
// (row, head) slots: several heads of one row, or several rows when the
// heads do not fill it.
// Sum over each aligned group of LPH lanes, every lane receiving the sum:
// DPP lane moves (quad permutes, then the half-row and row mirrors) instead
// of LDS permutes; only the step across 16-lane rows (LPH = 32) shuffles.
__device__ __forceinline__ float dpp_add(float x, int ctrl_tag) {
    int v = __float_as_int(x);
    switch (ctrl_tag) {   // the control must be a constant of the instruction
        case 0: v = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true); break;    // quad_perm [1,0,3,2]
        case 1: v = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true); break;    // quad_perm [2,3,0,1]
        case 2: v = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true); break;   // row_half_mirror
        default: v = __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true); break;  // row_mirror
    }
    return x + __int_as_float(v);
}
template <int LPH>
__device__ __forceinline__ float head_sum(float s) {
    s = dpp_add(s, 0);
    s = dpp_add(s, 1);
    if constexpr (LPH >= 8) s = dpp_add(s, 2);
    if constexpr (LPH >= 16) s = dpp_add(s, 3);
    if constexpr (LPH >= 32) s += __shfl_xor(s, 16, 64);
    return s;
}

template <int LPH>
__global__ void __launch_bounds__(256) k_sparse_attention_rows_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ col, const int32_t *__restrict__ row_ptr, int64_t n_rows, int64_t n_cols, int H,
    float scale, float *__restrict__ out) {
    constexpr int D = 4 * LPH, SLOTS = 64 / LPH;
    const int lane = threadIdx.x & 63;
    const int64_t wave = blockIdx.x * (int64_t)(blockDim.x / 64) + (threadIdx.x >> 6);
    const int slot = lane / LPH, sub = lane % LPH;
    int64_t row;
    int head;
    if (H >= SLOTS) {   // several wavefronts per row
        const int64_t wpr = (H + SLOTS - 1) / SLOTS;
        row = wave / wpr;
        head = (int)(wave % wpr) * SLOTS + slot;
    } else {            // several rows per wavefront
        const int rpw = SLOTS / H;
        const int r = slot / H;
        row = wave * rpw + r;
        head = slot % H;
        if (r >= rpw) row = n_rows;   // slots past the last whole row stay idle
    }
    const bool active = row < n_rows && head < H;
    int beg = 0, end = 0;
    if (active) {
        beg = row_ptr[row];
        end = row_ptr[row + 1];
    }
    // the wavefront walks as many edges as its longest row
    int len = end - beg;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) len = max(len, __shfl_xor(len, off, 64));
    float qv[4] = {0.f, 0.f, 0.f, 0.f};
    if (active) {
        const uint2 qq = *(const uint2 *)(q + (row * H + head) * (int64_t)D + 4 * sub);
        qv[0] = __uint_as_float(qq.x << 16) * scale;
        qv[1] = __uint_as_float(qq.x & 0xffff0000u) * scale;
        qv[2] = __uint_as_float(qq.y << 16) * scale;
        qv[3] = __uint_as_float(qq.y & 0xffff0000u) * scale;
    }
    float m = -INFINITY, l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
    constexpr int U = 4;   // edges whose operands are loaded together
    for (int t0 = 0; t0 < len; t0 += U) {
        uint2 kk[U], vv[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = beg + t0 + u;
            const int c = t < end ? col[t] : -1;
            ok[u] = c >= 0 && c < n_cols;
            const int64_t at = ((int64_t)(ok[u] ? c : 0) * H + (active ? head : 0)) * D + 4 * sub;
            kk[u] = ok[u] ? *(const uint2 *)(k + at) : make_uint2(0u, 0u);
            vv[u] = ok[u] ? *(const uint2 *)(v + at) : make_uint2(0u, 0u);
        }
        // the batch's scores, then one running-max update and one rescale for
        // the whole batch (invalid edges score -inf and weigh 0)
        float sc[U];
        float mb = m;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float s = qv[0] * __uint_as_float(kk[u].x << 16) + qv[1] * __uint_as_float(kk[u].x & 0xffff0000u) +
                      qv[2] * __uint_as_float(kk[u].y << 16) + qv[3] * __uint_as_float(kk[u].y & 0xffff0000u);
            s = head_sum<LPH>(s);
            sc[u] = ok[u] ? s : -INFINITY;   // the whole head group agrees on ok
            mb = fmaxf(mb, sc[u]);
        }
        if (mb == -INFINITY) continue;   // no valid edge yet in this head group
        const float corr = __expf(m - mb);
        l *= corr;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] *= corr;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float p = __expf(sc[u] - mb);   // 0 for an invalid edge
            l += p;
            acc[0] += p * __uint_as_float(vv[u].x << 16);
            acc[1] += p * __uint_as_float(vv[u].x & 0xffff0000u);
            acc[2] += p * __uint_as_float(vv[u].y << 16);
            acc[3] += p * __uint_as_float(vv[u].y & 0xffff0000u);
        }
        m = mb;
    }
    if (!active) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float4 o = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    *(float4 *)(out + (row * H + head) * (int64_t)D + 4 * sub) = o;
}

}  // namespace
}  // namespace cgtp

using namespace cgtp;

extern "C" {

int cgtp_sparse_attention_layout_bytes(int64_t n_rows, int64_t n_edges, size_t *bytes) {
    clear_error();
    if (!bytes || n_rows < 0 || n_edges < 0)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention_layout_bytes: bad argument");
    *bytes = AttnLayout(nullptr, n_rows, n_edges).bytes;
    return CGTP_OK;
}

int cgtp_sparse_attention_prepare(const int32_t *col, const int32_t *row_ptr, int64_t n_rows, int64_t n_cols,
                                  int64_t n_edges, void *layout, size_t layout_bytes, cgtp_stream_t stream) {
    clear_error();
    if (n_rows < 0 || n_cols < 0 || n_edges < 0 || n_rows > 0x7fffffffLL || n_edges > 0x7fffffffLL ||
        n_cols >= (1LL << 28) - 1)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention_prepare: sizes out of range");
    if (n_rows == 0) return CGTP_OK;
    const AttnLayout L(layout, n_rows, n_edges);
    if (!row_ptr || !layout || layout_bytes < L.bytes || (n_edges > 0 && !col))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention_prepare: NULL buffer or layout too small");
    if (((uintptr_t)layout) & 255)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention_prepare: layout must be 256-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const int64_t n_win = (n_rows + kWin - 1) / kWin;
    CGTP_LAUNCH("k_attention_compact", s, k_attention_compact, dim3((unsigned)n_win), dim3(kThreads), 0, s, col, row_ptr,
                n_rows, n_cols, L.ucol, L.umask, L.win_n);
    return hip_ok(hipGetLastError(), "sparse attention prepare launch");
}

int cgtp_sparse_attention(cgtp_dtype dtype, int32_t n_heads, int32_t head_dim, float scale, const void *q,
                          const void *k, const void *v, const int32_t *row_ptr, int64_t n_rows, int64_t n_edges,
                          const void *layout, size_t layout_bytes, void *out, cgtp_stream_t stream) {
    clear_error();
    if (dtype != CGTP_BF16_F32ACC)
        return set_error(CGTP_ERR_UNSUPPORTED, "cgtp_sparse_attention: bf16 inputs (CGTP_BF16_F32ACC) only");
    if (n_heads < 1 || n_heads > 65535 || head_dim < 16 || head_dim > 16 * kMaxChunks || head_dim % 16 != 0)
        return set_error(CGTP_ERR_INVALID_ARGUMENT,
                         "cgtp_sparse_attention: head_dim must be 16..128, a multiple of 16; n_heads 1..65535");
    if (n_rows < 0 || n_edges < 0 || n_rows > 0x7fffffffLL || n_edges > 0x7fffffffLL)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention: sizes out of range");
    if (n_rows == 0) return CGTP_OK;
    const AttnLayout L(const_cast<void *>(layout), n_rows, n_edges);
    if (!row_ptr || !out || !layout || layout_bytes < L.bytes || (n_edges > 0 && (!q || !k || !v)))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention: NULL buffer or layout too small");
    if ((((uintptr_t)q) | ((uintptr_t)k)) & 7)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention: q and k must be 8-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)((n_rows + kWin - 1) / kWin), (unsigned)n_heads);
    switch (head_dim / 16) {
#define CGTP_ATTN_CASE(NC)                                                                                          \
    case NC:                                                                                                         \
        CGTP_LAUNCH("k_sparse_attention_bf16", s, k_sparse_attention_bf16<NC>, grid, dim3(kThreads), 0, s,           \
                    (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, row_ptr, L.ucol, L.umask, L.win_n, \
                    n_rows, (int)n_heads, scale, (float *)out);                                                      \
        break;
        CGTP_ATTN_CASE(1)
        CGTP_ATTN_CASE(2)
        CGTP_ATTN_CASE(3)
        CGTP_ATTN_CASE(4)
        CGTP_ATTN_CASE(5)
        CGTP_ATTN_CASE(6)
        CGTP_ATTN_CASE(7)
        CGTP_ATTN_CASE(8)
#undef CGTP_ATTN_CASE
    }
    return hip_ok(hipGetLastError(), "sparse attention launch");
}


int cgtp_sparse_attention_rows(cgtp_dtype dtype, int32_t n_heads, int32_t head_dim, float scale, const void *q,
                               const void *k, const void *v, const int32_t *col, const int32_t *row_ptr,
                               int64_t n_rows, int64_t n_cols, int64_t n_edges, void *out, cgtp_stream_t stream) {
    clear_error();
    if (dtype != CGTP_BF16_F32ACC)
        return set_error(CGTP_ERR_UNSUPPORTED, "cgtp_sparse_attention_rows: bf16 inputs (CGTP_BF16_F32ACC) only");
    if (n_heads < 1 || n_heads > 65535 ||
        (head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128))
        return set_error(CGTP_ERR_INVALID_ARGUMENT,
                         "cgtp_sparse_attention_rows: head_dim must be 16, 32, 64 or 128; n_heads 1..65535");
    if (n_rows < 0 || n_cols < 0 || n_edges < 0 || n_rows > 0x7fffffffLL || n_edges > 0x7fffffffLL ||
        n_cols > 0x7fffffffLL)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention_rows: sizes out of range");
    if (n_rows == 0) return CGTP_OK;
    if (!row_ptr || !out || (n_edges > 0 && (!q || !k || !v || !col)))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention_rows: NULL buffer");
    if ((((uintptr_t)q) | ((uintptr_t)k) | ((uintptr_t)v)) & 7 || ((uintptr_t)out) & 15)
        return set_error(CGTP_ERR_INVALID_ARGUMENT,
                         "cgtp_sparse_attention_rows: q, k, v must be 8-byte and out 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const int lph = head_dim / 4, slots = 64 / lph;
    const int64_t waves = n_heads >= slots ? n_rows * ((n_heads + slots - 1) / slots)
                                           : (n_rows + slots / n_heads - 1) / (slots / n_heads);
    const int64_t blocks = (waves + 3) / 4;
    if (blocks > 0x7fffffffLL) return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention_rows: grid too large");
    switch (lph) {
#define CGTP_ROWS_CASE(L)                                                                                         \
    case L:                                                                                                        \
        CGTP_LAUNCH("k_sparse_attention_rows_bf16", s, k_sparse_attention_rows_bf16<L>, dim3((unsigned)blocks),     \
                    dim3(256), 0, s, (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, col, row_ptr,    \
                    n_rows, n_cols, (int)n_heads, scale, (float *)out);                                            \
        break;
        CGTP_ROWS_CASE(4)
        CGTP_ROWS_CASE(8)
        CGTP_ROWS_CASE(16)
        CGTP_ROWS_CASE(32)
#undef CGTP_ROWS_CASE
    }
    return hip_ok(hipGetLastError(), "sparse attention (rows) launch");
}

}  // extern "C"
