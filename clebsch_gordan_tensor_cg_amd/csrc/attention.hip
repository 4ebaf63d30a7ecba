// Graph sparse attention on the matrix cores ("Fused3S: Fast Sparse
// Attention on Tensor Cores", abstract): the three sparse steps -- sampled
// dense-dense product (SDDMM), row softmax and sparse-dense product (SpMM)
// -- fused in one kernel, so the scores never leave the chip.
//
//   s_e = scale <q[i][h], k[j][h]>  for every edge e = (j -> i) of the CSR
//   out[i][h] = sum_e softmax_i(s)_e v[j][h]
//
// MI355X design: a workgroup takes a window of 16 consecutive destination
// rows (the M/N size of the 16x16x16 bf16 MFMA) and one group of four heads
// (one wavefront per head).  The window's edges are compacted in LDS: keys
// (column, row) are sorted, each distinct column becomes one column of the
// window with a 16-bit mask of the rows that hold it, and the distinct
// columns are processed 16 at a time:
//   S^T = K_cols Q^T          one MFMA per 16 of the head dimension
//   online softmax per row    (running max and sum, masked entries = 0)
//   O  += P V_cols            P rounded to bf16, FP32 accumulation
// Computing S transposed leaves each lane with four scores of one row, which
// is exactly the A-operand layout that the P V product needs, so P never
// goes through LDS.  Windows with more edges than fit in LDS are taken in
// batches that continue the same running softmax.
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

typedef short a_s4 __attribute__((ext_vector_type(4)));
typedef float a_f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ short to_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7fffu + ((u >> 16) & 1u);   // round to nearest even
    return (short)(u >> 16);
}

__global__ void __launch_bounds__(kThreads) k_sparse_attention_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ col, const int32_t *__restrict__ row_ptr, int64_t n_rows, int64_t n_cols, int H,
    int D, float scale, float *__restrict__ out) {
    __shared__ uint32_t key[kCap];       // (column << 4) | row in window, sorted
    __shared__ int32_t ucol[kCap];       // distinct columns of the batch, padded with -1
    __shared__ uint16_t umask[kCap];     // rows of the window holding each distinct column
    __shared__ int32_t rp[kWin + 1];
    __shared__ int32_t part[kThreads];
    __shared__ int32_t n_unique;

    const int64_t r0 = (int64_t)blockIdx.x * kWin;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int h = blockIdx.y * (kThreads / 64) + wave;
    const bool head_live = h < H;
    const int nrw = (int)std::min<int64_t>(kWin, n_rows - r0);
    const int nchunk = D / 16;
    if (threadIdx.x <= kWin) rp[threadIdx.x] = row_ptr[r0 + std::min<int>(threadIdx.x, nrw)];
    __syncthreads();
    const int e_beg = rp[0], e_end = rp[nrw];

    // Q^T fragments of the window (B operand: B[kk][r] = q[r0 + r][h][kk]);
    // lane holds row lane%16, head-dim entries 4(lane/16)..+3 of each chunk
    a_s4 qf[kMaxChunks];
    a_f4 acc[kMaxChunks];
    const int rq = lane & 15, quad = lane >> 4;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        qf[c] = a_s4{0, 0, 0, 0};
        acc[c] = a_f4{0.f, 0.f, 0.f, 0.f};
        if (c < nchunk && head_live && rq < nrw)
            qf[c] = *(const a_s4 *)(q + ((r0 + rq) * H + h) * (int64_t)D + c * 16 + 4 * quad);
    }
    float m_run = -INFINITY, l_run = 0.f;   // softmax state of row lane%16

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
        // distinct columns: each thread owns a run of sorted keys, counts the
        // run heads, and after an exclusive scan writes its columns and masks
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
        int u = part[threadIdx.x];
        for (int t = t0; t < t1; ++t) {
            const uint32_t kv = key[t];
            if (kv == 0xffffffffu || (t > 0 && (key[t - 1] >> 4) == (kv >> 4))) continue;
            uint32_t m = 0;
            for (int t2 = t; t2 < nb && (key[t2] >> 4) == (kv >> 4) && key[t2] != 0xffffffffu; ++t2)
                m |= 1u << (key[t2] & 15u);
            ucol[u] = (int32_t)(kv >> 4);
            umask[u] = (uint16_t)m;
            ++u;
        }
        __syncthreads();
        const int nu = n_unique;
        const int nu16 = (nu + 15) & ~15;
        for (int t = nu + threadIdx.x; t < nu16; t += kThreads) {
            ucol[t] = -1;
            umask[t] = 0;
        }
        __syncthreads();

        if (head_live) {
            for (int cb = 0; cb < nu16; cb += 16) {
                // S^T[c][r] = <k[col c], q[r]>: A = K rows of the 16 columns
                const int ca = ucol[cb + rq];
                a_f4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < kMaxChunks; ++c) {
                    if (c >= nchunk) break;
                    a_s4 a = {0, 0, 0, 0};
                    if (ca >= 0) a = *(const a_s4 *)(k + ((int64_t)ca * H + h) * D + c * 16 + 4 * quad);
                    st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, qf[c], st, 0, 0, 0);
                }
                // lane holds S[row rq][columns cb + 4 quad + i]
                float s[4], p[4];
                float tmax = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool on = (umask[cb + 4 * quad + i] >> rq) & 1u;
                    s[i] = on ? st[i] * scale : -INFINITY;
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
                const a_s4 pa = {to_bf16(p[0]), to_bf16(p[1]), to_bf16(p[2]), to_bf16(p[3])};
                int cv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) cv[i] = ucol[cb + 4 * quad + i];
#pragma unroll
                for (int c = 0; c < kMaxChunks; ++c) {
                    if (c >= nchunk) break;
                    // B[kk][dd] = v[col kk][h][16 c + dd]: lane holds rows 4 quad + i, column rq
                    a_s4 vb;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        vb[i] = cv[i] >= 0 ? (short)v[((int64_t)cv[i] * H + h) * D + c * 16 + rq] : (short)0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[c][i] *= co[i];
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, acc[c], 0, 0, 0);
                }
            }
        }
        __syncthreads();   // LDS is rewritten by the next batch
    }
    if (!head_live) return;
    // out[r][h][16 c + rq] = O[r][.] / l[r] for the rows 4 quad + i
    float lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) lo[i] = __shfl(l_run, 4 * quad + i, 64);
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        if (c >= nchunk) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * quad + i;
            if (r < nrw) out[((r0 + r) * H + h) * D + c * 16 + rq] = lo[i] > 0.f ? acc[c][i] / lo[i] : 0.f;
        }
    }
}

int hip_ok(hipError_t e, const char *what) {
    if (e == hipSuccess) return CGTP_OK;
    return set_error(CGTP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace
}  // namespace cgtp

using namespace cgtp;

extern "C" {

int cgtp_sparse_attention(cgtp_dtype dtype, int32_t n_heads, int32_t head_dim, float scale, const void *q,
                          const void *k, const void *v, const int32_t *col, const int32_t *row_ptr, int64_t n_rows,
                          int64_t n_cols, int64_t n_edges, void *out, cgtp_stream_t stream) {
    clear_error();
    if (dtype != CGTP_BF16_F32ACC)
        return set_error(CGTP_ERR_UNSUPPORTED, "cgtp_sparse_attention: bf16 inputs (CGTP_BF16_F32ACC) only");
    if (n_heads < 1 || head_dim < 16 || head_dim > 16 * kMaxChunks || head_dim % 16 != 0)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention: head_dim must be 16..128, a multiple of 16");
    if (n_rows < 0 || n_cols < 0 || n_edges < 0 || n_rows > 0x7fffffffLL || n_edges > 0x7fffffffLL ||
        n_cols >= (1LL << 28) - 1)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention: sizes out of range");
    if (n_rows == 0) return CGTP_OK;
    if (!row_ptr || !out || (n_edges > 0 && (!q || !k || !v || !col)))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention: NULL buffer");
    if ((((uintptr_t)q) | ((uintptr_t)k)) & 7)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sparse_attention: q and k must be 8-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)((n_rows + kWin - 1) / kWin), (unsigned)((n_heads + 3) / 4));
    CGTP_LAUNCH("k_sparse_attention_bf16", s, k_sparse_attention_bf16, grid, dim3(kThreads), 0, s,
                (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, col, row_ptr, n_rows, n_cols,
                (int)n_heads, (int)head_dim, scale, (float *)out);
    return hip_ok(hipGetLastError(), "sparse attention launch");
}

}  // extern "C"
