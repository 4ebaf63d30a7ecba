// Fixed HIP kernels for gfx950 and their C ABI entry points: CSR build
// (counting sort with a per-segment rank so the order is exactly the stable
// order), CSR validation, real spherical harmonics of edge vectors, the
// force reduction and the force-loss cotangent, segment sums of rows and
// sums of partial buffers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <string>

#include "internal.h"

namespace cgtp {
namespace {

constexpr int kBlock = 256;

inline unsigned grid_for(int64_t n, int per_block = kBlock) {
    int64_t g = (n + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 0x7fffffff) g = 0x7fffffff;
    return (unsigned)g;
}

int hip_check(hipError_t e, const char *what) {
    if (e == hipSuccess) return CGTP_OK;
    return set_error(CGTP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// Generic fills, row segment sums, part sums
// ---------------------------------------------------------------------------
template <class T>
__global__ void k_fill(T *p, int64_t n, T v) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// out[s][c] (=|+=) sum_{k in [row_ptr[s], row_ptr[s+1])} rows[perm[k]][c]
// One workgroup per segment (blockIdx.y splits wide rows); each thread owns
// a 16-byte column chunk and keeps four source rows in flight.  Rows are
// summed in segment order.
template <class T>
struct Vec16;
template <>
struct Vec16<float> {
    typedef float V __attribute__((ext_vector_type(4)));
    static constexpr int N = 4;
    __device__ static V zero() { return V{0.f, 0.f, 0.f, 0.f}; }
    __device__ static void add(V &a, const V &b) { a += b; }
};
template <>
struct Vec16<double> {
    typedef double V __attribute__((ext_vector_type(2)));
    static constexpr int N = 2;
    __device__ static V zero() { return V{0.0, 0.0}; }
    __device__ static void add(V &a, const V &b) { a += b; }
};

template <class T, bool kPerm>
__global__ void __launch_bounds__(256) k_segment_sum_rows(const T *__restrict__ rows, const int32_t *__restrict__ row_ptr,
                                                          const int32_t *__restrict__ perm, int64_t n_seg,
                                                          int64_t width, T *__restrict__ out, int accumulate) {
    using VT = Vec16<T>;
    using V = typename VT::V;
    const bool vec_ok = (width % VT::N) == 0 && (((uintptr_t)rows | (uintptr_t)out) & 15) == 0;
    const int64_t step = (int64_t)gridDim.y * blockDim.x * VT::N;
    // persistent workgroups: each walks over segments, so the loads of one
    // segment overlap the tail of the previous one
    for (int64_t s = blockIdx.x; s < n_seg; s += gridDim.x) {
    const int beg = row_ptr[s], end = row_ptr[s + 1];
    for (int64_t c = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * VT::N; c < width; c += step) {
        if (vec_ok) {
            V acc = VT::zero();
            // sixteen source rows in flight per thread; the segment's last
            // rows in the same batch, masked (rows still summed in order)
            for (int k = beg; k < end; k += 16) {
                V a[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    // past the segment's end (the same for the whole
                    // workgroup): no row load, the index read clamped in range
                    const bool ok = k + u < end;
                    const int kk = ok ? k + u : beg;
                    const int64_t r = kPerm ? perm[kk] : kk;
                    // each row is read once: stream it past the caches
                    a[u] = ok ? __builtin_nontemporal_load((const V *)(rows + r * width + c)) : VT::zero();
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) VT::add(acc, a[u]);
            }
            V *o = (V *)(out + s * width + c);
            if (accumulate) {
                V prev = *o;
                VT::add(prev, acc);
                *o = prev;
            } else {
                *o = acc;
            }
        } else {
            for (int64_t cc = c; cc < c + VT::N && cc < width; ++cc) {
                T acc = 0;
                for (int k = beg; k < end; ++k) acc += rows[(int64_t)(kPerm ? perm[k] : k) * width + cc];
                T *o = out + s * width + cc;
                *o = accumulate ? *o + acc : acc;
            }
        }
    }
    }
}

template <class T>
__global__ void k_sum_parts(const T *__restrict__ parts, int n_parts, int64_t n, T *__restrict__ out,
                            int accumulate) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        // the unit partials of an SH-gradient row, summed in FP64 (as the
        // lanes of each unit were)
        double acc = 0;
        for (int p = 0; p < n_parts; ++p) acc += (double)parts[p * n + i];
        out[i] = (T)(accumulate ? (double)out[i] + acc : acc);
    }
}

// ---------------------------------------------------------------------------
// CSR build
// ---------------------------------------------------------------------------
// Keys are counted in LDS: a workgroup takes a contiguous run of edges and
// one range of at most kCsrBins keys, counts its keys there and publishes
// only its nonzero bins, so the device-wide atomics number about
// (#workgroups x #bins) rather than one per edge.  Keys outside
// [0, n_keys) are skipped.
constexpr int kCsrBins = 16384;  // 64 KiB of LDS counters per workgroup
// Node processing order: nodes by decreasing segment length (longest
// first, so the long segments do not form the tail of a launch).  Buckets
// are kOrderBuckets-1-min(len, kOrderBuckets-1); the order within a bucket
// is whatever the atomics give, which changes no result (each node is
// computed by one wavefront in its fixed edge order).
constexpr int kOrderBuckets = 1024;
constexpr int64_t kOrderSmallMax = 65536;   // rows ordered by one workgroup
__device__ __forceinline__ int lpt_bucket(int len) {
    return kOrderBuckets - 1 - (len < kOrderBuckets - 1 ? (len < 0 ? 0 : len) : kOrderBuckets - 1);
}
__device__ __forceinline__ int order_bucket(const int32_t *__restrict__ rp, int64_t i) {
    return lpt_bucket(rp[i + 1] - rp[i]);
}

// Turns the kOrderBuckets counts in h into exclusive starts.  Called by all
// 1024 threads of a workgroup (one bucket each) after the counts are in
// place; wsum: 16 words of LDS.  Ends with a barrier.
__device__ __forceinline__ void lpt_bucket_starts(int32_t *h, int32_t *wsum) {
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int32_t own = h[t];
    int32_t incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    if (wid == 0) {
        int32_t ws = lane < 16 ? wsum[lane] : 0;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const int32_t v = __shfl_up(ws, off, 64);
            if (lane >= off) ws += v;
        }
        if (lane < 16) wsum[lane] = ws;
    }
    __syncthreads();
    h[t] = (wid ? wsum[wid - 1] : 0) + incl - own;
    __syncthreads();
}

constexpr int kCsrThreads = 1024;

// Visits the keys of edges [e0, e1) owned by this thread, eight loads in
// flight at a time; a slot past e1 sees key -1 (skipped by every caller).
template <class F>
__device__ __forceinline__ void for_block_keys(const int32_t *__restrict__ key, int64_t e0, int64_t e1, F f) {
    constexpr int U = 8;
    for (int64_t base = e0 + threadIdx.x; base < e1; base += (int64_t)U * blockDim.x) {
        int32_t k[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = base + (int64_t)u * blockDim.x;
            k[u] = e < e1 ? key[e] : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) f(base + (int64_t)u * blockDim.x, k[u]);
    }
}

__global__ void __launch_bounds__(kCsrThreads) k_count(const int32_t *__restrict__ key, int64_t n, int64_t n_keys,
                                                       int64_t per, int32_t *__restrict__ cnt) {
    extern __shared__ int32_t h[];
    const int64_t k0 = (int64_t)blockIdx.y * kCsrBins;
    const int kb = (int)std::min<int64_t>(kCsrBins, n_keys - k0);
    const int64_t e0 = (int64_t)blockIdx.x * per, e1 = std::min<int64_t>(n, e0 + per);
    for (int i = threadIdx.x; i < kb; i += blockDim.x) h[i] = 0;
    __syncthreads();
    for_block_keys(key, e0, e1, [&](int64_t, int32_t kk) {
        const int64_t k = kk - k0;
        if (kk >= 0 && k >= 0 && k < kb) atomicAdd(&h[k], 1);
    });
    __syncthreads();
    for (int i = threadIdx.x; i < kb; i += blockDim.x)
        if (h[i]) atomicAdd(&cnt[k0 + i], h[i]);
}

// Same partition as k_count.  Each workgroup reserves, per nonzero bin, a
// run of slots inside that key's segment with one device atomic, then
// hands the slots out to its edges with LDS atomics.  The order inside a
// segment is therefore arbitrary; k_rank_segments makes it canonical.
__global__ void __launch_bounds__(kCsrThreads) k_scatter(const int32_t *__restrict__ key, int64_t n, int64_t n_keys,
                                                         int64_t per, const int32_t *__restrict__ row_ptr,
                                                         int32_t *__restrict__ cursor, int32_t *__restrict__ tmp) {
    extern __shared__ int32_t h[];
    const int64_t k0 = (int64_t)blockIdx.y * kCsrBins;
    const int kb = (int)std::min<int64_t>(kCsrBins, n_keys - k0);
    const int64_t e0 = (int64_t)blockIdx.x * per, e1 = std::min<int64_t>(n, e0 + per);
    for (int i = threadIdx.x; i < kb; i += blockDim.x) h[i] = 0;
    __syncthreads();
    for_block_keys(key, e0, e1, [&](int64_t, int32_t kk) {
        const int64_t k = kk - k0;
        if (kk >= 0 && k >= 0 && k < kb) atomicAdd(&h[k], 1);
    });
    __syncthreads();
    // reservations: up to four device atomics of a thread in flight together
    for (int i0 = threadIdx.x; i0 < kb; i0 += 4 * blockDim.x) {
        int c[4], r[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * (int)blockDim.x;
            c[u] = i < kb ? h[i] : 0;
            b[u] = c[u] ? row_ptr[k0 + i] : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = c[u] ? atomicAdd(&cursor[k0 + i0 + u * (int)blockDim.x], c[u]) : 0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (c[u]) h[i0 + u * (int)blockDim.x] = b[u] + r[u];
    }
    __syncthreads();
    for_block_keys(key, e0, e1, [&](int64_t e, int32_t kk) {
        const int64_t k = kk - k0;
        if (kk >= 0 && k >= 0 && k < kb) tmp[atomicAdd(&h[k], 1)] = (int32_t)e;
    });
}

// Key spaces too wide for a few LDS ranges: one device atomic per edge.
__global__ void k_count_global(const int32_t *__restrict__ key, int64_t n, int64_t n_keys, int32_t *__restrict__ cnt) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
        const int32_t k = key[e];
        if (k >= 0 && k < n_keys) atomicAdd(&cnt[k], 1);
    }
}

__global__ void k_scatter_global(const int32_t *__restrict__ key, int64_t n, int64_t n_keys,
                                 const int32_t *__restrict__ row_ptr, int32_t *__restrict__ cursor,
                                 int32_t *__restrict__ tmp) {
    for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
        const int32_t k = key[e];
        if (k >= 0 && k < n_keys) tmp[row_ptr[k] + atomicAdd(&cursor[k], 1)] = (int32_t)e;
    }
}

// Small key arrays (at most 65,535 edges and 2,048 keys) in one launch, with
// no device atomics and no communication between workgroups.  The edges are
// cut into runs of a power-of-two length (at least 64, at most
// kSmallCsrMaxRuns runs).  Workgroup r counts the keys of the whole array in
// LDS -- each key's total in the low half of a word, its count in the runs
// before r in the high half (a run or the array holds at most 65,535 edges,
// so no carry) -- scans the totals into each key's first slot and so knows
// where its own run's edges of each key go.  Its first wavefront then walks
// the run in edge order, 64 edges at a time: one ballot per key bit finds
// the lanes holding the same key, which ranks each edge among the chunk's
// equal keys and elects the highest such lane to advance the key's next
// slot.  The placement is therefore stable (edge order inside every segment)
// without a sort.  Workgroup 0 also writes row_ptr and, with order non-NULL,
// the longest-first node order (as k_order_small) from the totals.  Each
// workgroup rereads the key array (at most 256 KiB) from L2.  The run count
// trades that redundant counting against the length of the one-wavefront
// walk: on 100 molecules of 18 atoms (25,710 edges) 51 runs of 512 edges took
// 14.7 us, 101 of 256 12.8 us, 201 of 128 11.7 us and 402 of 64 15.9 us.
constexpr int kSmallCsrMaxRuns = 256;
constexpr int64_t kSmallCsrMaxKeys = 2048;
constexpr int64_t kSmallCsrMaxEdges = 65535;
constexpr int kSmallCsrChunks = 4;           // 64-edge chunks of one run (a run holds at most 256 edges)
static_assert(kSmallCsrMaxKeys == 2048, "the key-match ballots cover 11 bits");
static_assert(kSmallCsrMaxEdges <= (int64_t)kSmallCsrMaxRuns * 64 * kSmallCsrChunks, "runs of at most 256 edges");
constexpr int kSmallCsrKeysPerThread = 32;   // keys per thread and round of the counting
__host__ __device__ constexpr bool small_csr(int64_t n_edges, int64_t n_keys) {
    return n_edges > 0 && n_keys > 0 && n_edges <= kSmallCsrMaxEdges && n_keys <= kSmallCsrMaxKeys;
}
// runs of 2^s edges: the smallest power of two, at least 64, with at most
// kSmallCsrMaxRuns runs covering n
__host__ __device__ constexpr int small_csr_run_shift(int64_t n) {
    int sh = 6;
    while ((int64_t(kSmallCsrMaxRuns) << sh) < n) ++sh;
    return sh;
}
__host__ __device__ constexpr int64_t small_csr_runs(int64_t n) {
    return (n + (int64_t(1) << small_csr_run_shift(n)) - 1) >> small_csr_run_shift(n);
}

// lanes of this wavefront whose key equals this lane's key (valid lanes
// only); keys lie in [0, 2^nbits)
__device__ __forceinline__ uint64_t same_key_lanes(int32_t k, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
    for (int b = 0; b < nbits; ++b) {   // nbits <= 11
        const uint32_t mine = (uint32_t)(((int32_t)((uint32_t)k << (31 - b))) >> 31);   // 0 or ~0
        const uint64_t bb = __ballot(mine != 0u);
        lo &= ~((uint32_t)bb ^ mine);
        hi &= ~((uint32_t)(bb >> 32) ^ mine);
    }
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__global__ void __launch_bounds__(1024) k_csr_small(const int32_t *__restrict__ key, const int32_t *__restrict__ val,
                                                    int64_t n, int64_t n_keys, int nbits, int32_t *__restrict__ row_ptr,
                                                    int32_t *__restrict__ perm, int32_t *__restrict__ sorted_key,
                                                    int32_t *__restrict__ sorted_val, int32_t *__restrict__ order) {
    __shared__ uint32_t cnt[kSmallCsrMaxKeys];   // counts (total | before << 16), then each key's next slot
    __shared__ int32_t wsum[16];
    __shared__ int32_t hb[kOrderBuckets];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int nk = (int)n_keys;
    const int rsh = small_csr_run_shift(n);
    const int64_t r0 = (int64_t)blockIdx.x << rsh;
    const int64_t r1 = r0 + (int64_t(1) << rsh) < n ? r0 + (int64_t(1) << rsh) : n;
    const bool lead = blockIdx.x == 0;
    for (int i = t; i < nk; i += blockDim.x) cnt[i] = 0u;
    if (order && lead) hb[t] = 0;
    __syncthreads();
    // 32 keys of a thread in flight at once: one round for up to 32,768 edges
    for (int h = 0; h * kSmallCsrKeysPerThread * 1024 < n; ++h) {
        int32_t kr[kSmallCsrKeysPerThread];
#pragma unroll
        for (int u = 0; u < kSmallCsrKeysPerThread; ++u) {
            const int64_t e = t + (int64_t)(h * kSmallCsrKeysPerThread + u) * 1024;
            const int32_t kv = key[e < n ? e : n - 1];   // clamped: no branch around the load
            kr[u] = e < n ? kv : -1;
        }
#pragma unroll
        for (int u = 0; u < kSmallCsrKeysPerThread; ++u) {
            const int k = kr[u];
            const int64_t e = t + (int64_t)(h * kSmallCsrKeysPerThread + u) * 1024;
            if (k >= 0 && k < nk) atomicAdd(&cnt[k], e < r0 ? 0x10001u : 1u);
        }
    }
    __syncthreads();
    // two consecutive keys per thread: totals, scan, row_ptr, this run's first slots
    int tot[2], bef[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int k = 2 * t + q;
        const uint32_t c = k < nk ? cnt[k] : 0u;
        tot[q] = (int)(c & 0xffffu);
        bef[q] = (int)(c >> 16);
    }
    const int own = tot[0] + tot[1];
    int incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int v = __shfl_up(incl, off, 64);
        if (lane >= off) incl += v;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();   // also: every count is read before any is overwritten below
    int before = 0;
    for (int w = 0; w < wv; ++w) before += wsum[w];
    const int first = before + incl - own;
    if (2 * t < nk) {
        if (lead) {
            row_ptr[2 * t] = first;
            if (2 * t + 1 < nk) row_ptr[2 * t + 1] = first + tot[0];
        }
        cnt[2 * t] = (uint32_t)(first + bef[0]);
        if (2 * t + 1 < nk) cnt[2 * t + 1] = (uint32_t)(first + tot[0] + bef[1]);
    }
    if (lead && t == (int)blockDim.x - 1) row_ptr[nk] = before + incl;   // every valid key counted
    if (order && lead) {   // uniform: the whole workgroup takes this branch or none of it
#pragma unroll
        for (int q = 0; q < 2; ++q)
            if (2 * t + q < nk) atomicAdd(&hb[lpt_bucket(tot[q])], 1);
        __syncthreads();   // also orders the reads of wsum above before its reuse
        lpt_bucket_starts(hb, wsum);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            if (2 * t + q < nk) order[atomicAdd(&hb[lpt_bucket(tot[q])], 1)] = 2 * t + q;
    }
    __syncthreads();
    if (wv != 0) return;
    // the first wavefront walks the run; every chunk's keys and values in flight at once
    int32_t kb[kSmallCsrChunks], vb[kSmallCsrChunks] = {};
#pragma unroll
    for (int u = 0; u < kSmallCsrChunks; ++u) {
        const int64_t e = r0 + 64 * u + lane;
        const int64_t ec = e < r1 ? e : r1 - 1;   // clamped: no branch around the loads
        const int32_t kv = key[ec];
        kb[u] = e < r1 ? kv : -1;
        if (sorted_val) vb[u] = val[ec];
    }
#pragma unroll
    for (int u = 0; u < kSmallCsrChunks; ++u) {
        if (r0 + 64 * u >= r1) break;   // uniform across the wavefront
        const int64_t e = r0 + 64 * u + lane;
        const int32_t k = kb[u];
        const bool valid = k >= 0 && k < nk;
        const uint64_t m = same_key_lanes(k, valid, nbits);
        const int base = valid ? (int)cnt[k] : 0;   // read by every lane before the update
        if (valid) {
            const int slot = base + lanes_below(m);
            perm[slot] = (int32_t)e;
            if (sorted_key) sorted_key[slot] = k;
            if (sorted_val) sorted_val[slot] = vb[u];
        }
        if (valid && ((m >> lane) >> 1) == 0) cnt[k] = (uint32_t)(base + __popcll(m));
    }
}


// The whole order in one workgroup (small graphs): count, scan and place
// in LDS.
__global__ void __launch_bounds__(1024) k_order_small(const int32_t *__restrict__ rp, int64_t n,
                                                       int32_t *__restrict__ order) {
    __shared__ int32_t h[kOrderBuckets];
    __shared__ int32_t wsum[16];
    const int t = threadIdx.x;
    h[t] = 0;
    __syncthreads();
    for (int64_t i = t; i < n; i += 1024) atomicAdd(&h[order_bucket(rp, i)], 1);
    __syncthreads();
    lpt_bucket_starts(h, wsum);
    for (int64_t i = t; i < n; i += 1024) order[atomicAdd(&h[order_bucket(rp, i)], 1)] = (int32_t)i;
}

__global__ void __launch_bounds__(1024) k_order_count(const int32_t *__restrict__ rp, int64_t n,
                                                       int32_t *__restrict__ cnt) {
    __shared__ int32_t h[kOrderBuckets];
    for (int i = threadIdx.x; i < kOrderBuckets; i += blockDim.x) h[i] = 0;
    __syncthreads();
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        atomicAdd(&h[order_bucket(rp, i)], 1);
    __syncthreads();
    for (int i = threadIdx.x; i < kOrderBuckets; i += blockDim.x)
        if (h[i]) atomicAdd(&cnt[i], h[i]);
}

__global__ void __launch_bounds__(1024) k_order_scatter(const int32_t *__restrict__ rp, int64_t n,
                                                         const int32_t *__restrict__ start,
                                                         int32_t *__restrict__ cursor, int32_t *__restrict__ order) {
    __shared__ int32_t h[kOrderBuckets];
    for (int i = threadIdx.x; i < kOrderBuckets; i += blockDim.x) h[i] = 0;
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    for (int64_t i = i0; i < n; i += stride) atomicAdd(&h[order_bucket(rp, i)], 1);
    __syncthreads();
    for (int i = threadIdx.x; i < kOrderBuckets; i += blockDim.x) {
        const int c = h[i];
        if (c) h[i] = start[i] + atomicAdd(&cursor[i], c);
    }
    __syncthreads();
    for (int64_t i = i0; i < n; i += stride) order[atomicAdd(&h[order_bucket(rp, i)], 1)] = (int32_t)i;
}

// Exclusive scan of cnt[0..n) into row_ptr[0..n]; one workgroup, four
// consecutive counts per thread, wavefront scans by shuffles.
// With order non-NULL (n at most 65536 rows) it then writes the longest-first
// node order of the rows whose lengths cnt holds, as k_order_small does.
// With max_out non-NULL it also stores the largest count there.
__global__ void __launch_bounds__(1024) k_scan(const int32_t *__restrict__ cnt, int64_t n,
                                                int32_t *__restrict__ row_ptr, int32_t *__restrict__ order,
                                                int32_t *__restrict__ max_out) {
    __shared__ int32_t wsum[16];
    __shared__ int32_t hb[kOrderBuckets];
    __shared__ int32_t wmax[16];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int32_t carry = 0, vmax = 0;
    for (int64_t base = 0; base < n; base += 4096) {
        const int64_t i0 = base + 4 * (int64_t)threadIdx.x;
        int32_t v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = i0 + q < n ? cnt[i0 + q] : 0;
        vmax = max(vmax, max(max(v[0], v[1]), max(v[2], v[3])));
        const int32_t own = v[0] + v[1] + v[2] + v[3];
        int32_t incl = own;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t t = __shfl_up(incl, off, 64);
            if (lane >= off) incl += t;
        }
        if (lane == 63) wsum[wid] = incl;
        __syncthreads();
        if (wid == 0) {
            int32_t ws = lane < 16 ? wsum[lane] : 0;
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                const int32_t t = __shfl_up(ws, off, 64);
                if (lane >= off) ws += t;
            }
            if (lane < 16) wsum[lane] = ws;
        }
        __syncthreads();
        int32_t run = carry + (wid ? wsum[wid - 1] : 0) + incl - own;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (i0 + q < n) row_ptr[i0 + q] = run;
            run += v[q];
        }
        carry += wsum[15];
        __syncthreads();
    }
    if (threadIdx.x == 0) row_ptr[n] = carry;
    if (max_out) {   // uniform across the workgroup
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) vmax = max(vmax, __shfl_xor(vmax, off, 64));
        if (lane == 0) wmax[wid] = vmax;
        __syncthreads();
        if (threadIdx.x == 0) {
            int32_t m = 0;
            for (int w = 0; w < 16; ++w) m = max(m, wmax[w]);
            *max_out = m;
        }
    }
    if (order) {   // uniform across the workgroup
        const int t = threadIdx.x;
        hb[t] = 0;
        __syncthreads();
        for (int64_t i = t; i < n; i += 1024) atomicAdd(&hb[lpt_bucket(cnt[i])], 1);
        __syncthreads();
        lpt_bucket_starts(hb, wsum);
        for (int64_t i = t; i < n; i += 1024) order[atomicAdd(&hb[lpt_bucket(cnt[i])], 1)] = (int32_t)i;
    }
}

// One wavefront per segment: each element's final slot is the number of
// smaller edge ids in its segment, which reproduces the stable order no
// matter in which order the scatter's atomics landed.  The segment is staged
// in LDS.  Segments longer than kRankLds (hubs) are left to the trailing
// workgroups of the same launch (blockIdx.x >= n_keys), which do nothing
// unless *max_deg exceeds kRankLds.  They take the CSR slots 64 at a time;
// each lane finds its slot's segment by binary search in row_ptr, and the
// lanes of one hub rank their elements together against the whole segment,
// staged through LDS kRankLds ids at a time: O(deg^2 / 64) LDS reads per hub
// spread over the trailing workgroups instead of one wavefront's global loads.
constexpr int kRankLds = 2048;
constexpr int kRankHubGroups = 1024;   // trailing workgroups of k_rank_segments (fewer for small edge counts)

__device__ __forceinline__ void rank_emit(int32_t me, int slot, const int32_t *__restrict__ key,
                                          const int32_t *__restrict__ val, int32_t *__restrict__ perm,
                                          int32_t *__restrict__ sorted_key, int32_t *__restrict__ sorted_val) {
    perm[slot] = me;
    if (sorted_key) sorted_key[slot] = key[me];
    if (sorted_val) sorted_val[slot] = val[me];
}

__global__ void __launch_bounds__(64) k_rank_segments(const int32_t *__restrict__ row_ptr, int64_t n_keys,
                                                      const int32_t *__restrict__ tmp,
                                                      const int32_t *__restrict__ key,
                                                      const int32_t *__restrict__ val,
                                                      const int32_t *__restrict__ max_deg,
                                                      int32_t *__restrict__ perm,
                                                      int32_t *__restrict__ sorted_key,
                                                      int32_t *__restrict__ sorted_val) {
    __shared__ int32_t seg[kRankLds];
    const int lane = threadIdx.x;
    if ((int64_t)blockIdx.x < n_keys) {
        const int64_t s = blockIdx.x;
        const int beg = row_ptr[s], end = row_ptr[s + 1];
        const int deg = end - beg;
        if (deg > kRankLds) return;   // a hub: the trailing workgroups rank it
        for (int i = lane; i < deg; i += 64) seg[i] = tmp[beg + i];
        __syncthreads();
        for (int i = lane; i < deg; i += 64) {
            const int32_t me = seg[i];
            int rank = 0;
            for (int j = 0; j < deg; ++j) rank += seg[j] < me;
            rank_emit(me, beg + rank, key, val, perm, sorted_key, sorted_val);
        }
        return;
    }
    if (*max_deg <= kRankLds) return;   // no hub: the common case ends here
    const int64_t g = (int64_t)blockIdx.x - n_keys, n_groups = (int64_t)gridDim.x - n_keys;
    const int64_t n_slots = row_ptr[n_keys];
    for (int64_t c = g; c * 64 < n_slots; c += n_groups) {   // uniform across the workgroup
        const int64_t p = c * 64 + lane;
        // segment of slot p: the last s with row_ptr[s] <= p (a slot lies in
        // a nonempty segment, so the search ends on it)
        int64_t lo = 0, hi = n_keys;   // row_ptr[lo] <= p < row_ptr[hi]
        if (p < n_slots)
            while (hi - lo > 1) {
                const int64_t mid = (lo + hi) >> 1;
                if (row_ptr[mid] <= p) lo = mid;
                else hi = mid;
            }
        const int beg = p < n_slots ? row_ptr[lo] : 0;
        const int end = p < n_slots ? row_ptr[lo + 1] : 0;
        bool todo = p < n_slots && end - beg > kRankLds;
        const int32_t me = todo ? tmp[p] : 0;
        // the hubs among these 64 slots, one at a time (at most two: each
        // is longer than the chunk)
        while (__any(todo)) {
            const int lead = __builtin_ctzll(__ballot(todo));
            const int hb = __shfl(beg, lead, 64), he = __shfl(end, lead, 64);
            const bool mine = todo && beg == hb;
            int rank = 0;
            for (int t0 = hb; t0 < he; t0 += kRankLds) {
                const int len = min(kRankLds, he - t0);
                for (int i = lane; i < len; i += 64) seg[i] = tmp[t0 + i];
                __syncthreads();
                if (mine)
                    for (int j = 0; j < len; ++j) rank += seg[j] < me;
                __syncthreads();
            }
            if (mine) rank_emit(me, hb + rank, key, val, perm, sorted_key, sorted_val);
            todo = todo && !mine;
        }
    }
}

__global__ void k_validate(const int32_t *__restrict__ row_ptr, int64_t n_rows, int64_t n_edges,
                           const int32_t *__restrict__ idx, int64_t range, int32_t *__restrict__ bad) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t t0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    for (int64_t r = t0; r < n_rows; r += stride)
        if (row_ptr[r] > row_ptr[r + 1]) bad[0] = 1;
    if (t0 == 0 && (row_ptr[0] != 0 || row_ptr[n_rows] != n_edges)) bad[0] = 1;
    if (idx)
        for (int64_t e = t0; e < n_edges; e += stride)
            if (idx[e] < 0 || idx[e] >= range) bad[0] = 1;
}

// Transpose CSR of a canonical edge list (sorted by source, ties by
// destination) from its destination CSR.  perm[t] is the canonical id of the
// edge at destination-sorted position t.  The edges of source s are the
// canonical run [first index with src >= s, first index with src >= s+1),
// ordered by destination and therefore by destination-sorted position, which
// is the stable order by source of the destination-sorted edges: the
// transpose's entry for canonical edge e is the position t with perm[t] = e,
// and its row pointers are those run boundaries.  Row pointer s is the first
// canonical index whose source is at least s: position t (0..E) opens rows
// (src[t-1], src[t]], with src[-1] = -1 and src[E] = n_keys, sources clamped
// to [-1, n_keys] (every write in bounds whatever src holds; for a sorted
// list this equals a binary search for each s).
__global__ void k_csr_transpose_canonical(const int32_t *__restrict__ src, const int32_t *__restrict__ perm,
                                          int64_t n_edges, int64_t n_keys, int32_t *__restrict__ src_perm,
                                          int32_t *__restrict__ src_row_ptr) {
    auto clamp_key = [n_keys](int64_t v) { return v < -1 ? (int64_t)-1 : (v > n_keys ? n_keys : v); };
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t <= n_edges;
         t += (int64_t)gridDim.x * blockDim.x) {
        if (t < n_edges) {
            const int32_t e = perm[t];
            if (e >= 0 && e < n_edges) src_perm[e] = (int32_t)t;   // in bounds whatever perm holds
        }
        const int64_t prev = t == 0 ? -1 : clamp_key(src[t - 1]);
        const int64_t cur = t == n_edges ? n_keys : clamp_key(src[t]);
        for (int64_t k = prev + 1; k <= cur; ++k) src_row_ptr[k] = (int32_t)t;
    }
}

// ---------------------------------------------------------------------------
// Real spherical harmonics, component normalisation.
// On the unit sphere, with u = r/|r| and (u_x + i u_y)^m = A_m + i B_m:
//   Y_{l,0}  = N_l0 Q_l^0(u_z)
//   Y_{l,m}  = N_lm Q_l^m(u_z) A_m,  Y_{l,-m} = N_lm Q_l^m(u_z) B_m  (m > 0)
// where Q_l^m = d^m P_l / dz^m obeys the associated-Legendre recurrence
// (Q_m^m = (2m-1)!!, Q_{m+1}^m = (2m+1) z Q_m^m, then the three-term rule),
// N_l0 = sqrt(2l+1), N_lm = sqrt(2(2l+1)(l-m)!/(l+m)!).
// These polynomials extend Y off the sphere; the gradient with respect to r
// is (I - u u^T) grad_u / |r|, independent of the extension, with
// dQ_l^m/dz = Q_l^{m+1}, d(A_m,B_m)/dx = m (A_{m-1}, B_{m-1}),
// d(A_m,B_m)/dy = m (-B_{m-1}, A_{m-1}).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr double fact_d(int n) { return n <= 1 ? 1.0 : n * fact_d(n - 1); }

template <int L>
struct ShNorm {
    double v[(L + 1) * (L + 1)];
    constexpr ShNorm() : v() {
        for (int l = 0; l <= L; ++l)
            for (int m = 0; m <= l; ++m) {
                double s = (2.0 * l + 1.0) * (m == 0 ? 1.0 : 2.0 * fact_d(l - m) / fact_d(l + m));
                // constexpr square root by Newton's method
                double r = s > 1 ? s : 1.0;
                for (int it = 0; it < 64; ++it) r = 0.5 * (r + s / r);
                v[l * l + l + m] = r;
            }
    }
};

template <class T, int L>
struct ShPoly {
    T Q[L + 2][L + 2];  // Q[l][m], with Q[l][l+1] = 0
    T A[L + 1], B[L + 1];
    __device__ void eval(T ux, T uy, T uz) {
        for (int l = 0; l <= L; ++l)
            for (int m = 0; m <= L + 1; ++m) Q[l][m] = 0;
        T dfm = 1;  // (2m-1)!!
        for (int m = 0; m <= L; ++m) {
            if (m > 0) dfm *= (T)(2 * m - 1);
            Q[m][m] = dfm;
            if (m + 1 <= L) Q[m + 1][m] = (T)(2 * m + 1) * uz * dfm;
            for (int l = m + 2; l <= L; ++l)
                Q[l][m] = ((T)(2 * l - 1) * uz * Q[l - 1][m] - (T)(l + m - 1) * Q[l - 2][m]) / (T)(l - m);
        }
        A[0] = 1;
        B[0] = 0;
        for (int m = 1; m <= L; ++m) {
            A[m] = ux * A[m - 1] - uy * B[m - 1];
            B[m] = ux * B[m - 1] + uy * A[m - 1];
        }
    }
};

template <class T>
__device__ inline void store_sh(T *p, T v) { *p = v; }
__device__ inline void store_sh(uint16_t *p, float v) {
    // round to nearest even bf16
    uint32_t u = __float_as_uint(v);
    u += 0x7fffu + ((u >> 16) & 1u);
    *p = (uint16_t)(u >> 16);
}

template <class T, class S, int L>
__global__ void k_sh(const T *__restrict__ vec, const int32_t *__restrict__ perm, int64_t n,
                     S *__restrict__ sh) {
    constexpr ShNorm<L> N{};
    constexpr int NS = (L + 1) * (L + 1);
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = perm ? perm[t] : t;
        T rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
        const T inv = (T)1 / sqrt(rx * rx + ry * ry + rz * rz);
        ShPoly<T, L> P;
        P.eval(rx * inv, ry * inv, rz * inv);
        S *o = sh + t * NS;
#pragma unroll
        for (int l = 0; l <= L; ++l) {
            store_sh(o + l * l + l, (T)N.v[l * l + l] * P.Q[l][0]);
#pragma unroll
            for (int m = 1; m <= l; ++m) {
                const T nq = (T)N.v[l * l + l + m] * P.Q[l][m];
                store_sh(o + l * l + l + m, nq * P.A[m]);
                store_sh(o + l * l + l - m, nq * P.B[m]);
            }
        }
    }
}

// grad_u of every Y_k contracted with a per-k weight: G = sum_k c_k grad_u Y_k
template <class T, int L>
__device__ inline void sh_grad_contract(const ShPoly<T, L> &P, const T *c, T G[3]) {
    constexpr ShNorm<L> N{};
    G[0] = G[1] = G[2] = 0;
#pragma unroll
    for (int l = 0; l <= L; ++l) {
        // m = 0
        G[2] += c[l * l + l] * (T)N.v[l * l + l] * P.Q[l][1];
#pragma unroll
        for (int m = 1; m <= l; ++m) {
            const T nm = (T)N.v[l * l + l + m];
            const T cp = c[l * l + l + m], cn = c[l * l + l - m];
            const T q = P.Q[l][m], dq = P.Q[l][m + 1];
            // Y+ = nm q A_m ; Y- = nm q B_m
            G[0] += nm * q * (T)m * (cp * P.A[m - 1] + cn * P.B[m - 1]);
            G[1] += nm * q * (T)m * (-cp * P.B[m - 1] + cn * P.A[m - 1]);
            G[2] += nm * dq * (cp * P.A[m] + cn * P.B[m]);
        }
    }
}

// The force path runs in FP64 whatever the storage type.  Its last step,
// the force-loss cotangent -J (F[dst] - F[src]), multiplies force errors by
// the SH Jacobian, which grows as 1/|r| on the shortest edges, so FP32
// roundoff in F (sums of about a hundred edge vectors per atom) would reach
// the second derivatives ten to twenty times amplified.  The three kernels
// below load and store the storage type and compute in double.

// per-edge force vector v_t = J_t^T g_t = (I - u u^T) G / |r|; g_t is the
// sum of n_parts partial rows part_stride elements apart
template <class T, int L>
__global__ void k_edge_force(const T *__restrict__ vec, const int32_t *__restrict__ perm,
                             const T *__restrict__ g_sh, int n_parts, int64_t part_stride, int64_t n,
                             T *__restrict__ v) {
    constexpr int NS = (L + 1) * (L + 1);
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = perm ? perm[t] : t;
        const double rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
        const double rn = sqrt(rx * rx + ry * ry + rz * rz), inv = 1.0 / rn;
        const double u[3] = {rx * inv, ry * inv, rz * inv};
        ShPoly<double, L> P;
        P.eval(u[0], u[1], u[2]);
        double c[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) c[k] = g_sh[t * NS + k];
        for (int q = 1; q < n_parts; ++q)
#pragma unroll
            for (int k = 0; k < NS; ++k) c[k] += g_sh[q * part_stride + t * NS + k];
        double G[3];
        sh_grad_contract<double, L>(P, c, G);
        const double ug = u[0] * G[0] + u[1] * G[1] + u[2] * G[2];
#pragma unroll
        for (int a = 0; a < 3; ++a) v[3 * t + a] = (T)((G[a] - u[a] * ug) * inv);
    }
}

// F[a] = -sum_{t in dst seg a} v_t + sum_{k in src seg a} v_{src_perm[k]}
// One wavefront per atom: lanes stride over the atom's edges, then a
// butterfly sum over the wavefront.
template <class T>
__global__ void __launch_bounds__(64) k_node_force(const T *__restrict__ v, const int32_t *__restrict__ dst_row_ptr,
                                                   const int32_t *__restrict__ src_row_ptr,
                                                   const int32_t *__restrict__ src_perm, int64_t n_nodes,
                                                   T *__restrict__ F) {
    const int64_t a = blockIdx.x;
    const int lane = threadIdx.x;
    double f0 = 0, f1 = 0, f2 = 0;
    for (int t = dst_row_ptr[a] + lane; t < dst_row_ptr[a + 1]; t += 64) {
        f0 -= v[3 * (int64_t)t];
        f1 -= v[3 * (int64_t)t + 1];
        f2 -= v[3 * (int64_t)t + 2];
    }
    for (int k = src_row_ptr[a] + lane; k < src_row_ptr[a + 1]; k += 64) {
        const int64_t t = src_perm[k];
        f0 += v[3 * t];
        f1 += v[3 * t + 1];
        f2 += v[3 * t + 2];
    }
    for (int off = 32; off >= 1; off >>= 1) {
        f0 += __shfl_xor(f0, off, 64);
        f1 += __shfl_xor(f1, off, 64);
        f2 += __shfl_xor(f2, off, 64);
    }
    if (lane == 0) {
        F[3 * a] = (T)f0;
        F[3 * a + 1] = (T)f1;
        F[3 * a + 2] = (T)f2;
    }
}

// gg_sh[t] = -J_t d,  d = F[dst t] - F[src t];  J_t d = grad_u Y . d_perp / |r|
template <class T, int L>
__global__ void k_force_cotangent(const T *__restrict__ vec, const int32_t *__restrict__ perm,
                                  const int32_t *__restrict__ src, const int32_t *__restrict__ dst,
                                  const T *__restrict__ F, int64_t n, T *__restrict__ gg) {
    constexpr ShNorm<L> N{};
    constexpr int NS = (L + 1) * (L + 1);
    for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = perm ? perm[t] : t;
        const double rx = vec[3 * e], ry = vec[3 * e + 1], rz = vec[3 * e + 2];
        const double rn = sqrt(rx * rx + ry * ry + rz * rz), inv = 1.0 / rn;
        const double u[3] = {rx * inv, ry * inv, rz * inv};
        const int64_t a = dst[t], b = src[t];
        double d[3] = {(double)F[3 * a] - (double)F[3 * b], (double)F[3 * a + 1] - (double)F[3 * b + 1],
                       (double)F[3 * a + 2] - (double)F[3 * b + 2]};
        const double ud = u[0] * d[0] + u[1] * d[1] + u[2] * d[2];
#pragma unroll
        for (int c = 0; c < 3; ++c) d[c] = (d[c] - u[c] * ud) * inv;
        ShPoly<double, L> P;
        P.eval(u[0], u[1], u[2]);
        T *o = gg + t * NS;
#pragma unroll
        for (int l = 0; l <= L; ++l) {
            o[l * l + l] = (T)(-N.v[l * l + l] * P.Q[l][1] * d[2]);
#pragma unroll
            for (int m = 1; m <= l; ++m) {
                const double nm = N.v[l * l + l + m];
                const double q = P.Q[l][m], dq = P.Q[l][m + 1];
                const double gp0 = nm * q * m * P.A[m - 1], gp1 = -nm * q * m * P.B[m - 1], gp2 = nm * dq * P.A[m];
                const double gn0 = nm * q * m * P.B[m - 1], gn1 = nm * q * m * P.A[m - 1], gn2 = nm * dq * P.B[m];
                o[l * l + l + m] = (T)(-(gp0 * d[0] + gp1 * d[1] + gp2 * d[2]));
                o[l * l + l - m] = (T)(-(gn0 * d[0] + gn1 * d[1] + gn2 * d[2]));
            }
        }
    }
}

template <template <int> class F, class... A>
int dispatch_l(int lmax, A... a) {
    switch (lmax) {
        case 0: return F<0>::run(a...);
        case 1: return F<1>::run(a...);
        case 2: return F<2>::run(a...);
        case 3: return F<3>::run(a...);
        case 4: return F<4>::run(a...);
        case 5: return F<5>::run(a...);
        case 6: return F<6>::run(a...);
    }
    return set_error(CGTP_ERR_UNSUPPORTED, "lmax must be in [0, 6]");
}

template <int L>
struct ShLaunch {
    static int run(cgtp_dtype dt, const void *vec, const int32_t *perm, int64_t n, void *sh, hipStream_t s) {
        unsigned g = grid_for(n);
        if (dt == CGTP_F32)
            CGTP_LAUNCH("k_sh", s, (k_sh<float, float, L>), dim3(g), dim3(kBlock), 0, s, (const float *)vec, perm, n, (float *)sh);
        else if (dt == CGTP_F64)
            CGTP_LAUNCH("k_sh", s, (k_sh<double, double, L>), dim3(g), dim3(kBlock), 0, s, (const double *)vec, perm, n, (double *)sh);
        else
            CGTP_LAUNCH("k_sh", s, (k_sh<float, uint16_t, L>), dim3(g), dim3(kBlock), 0, s, (const float *)vec, perm, n, (uint16_t *)sh);
        return hip_check(hipGetLastError(), "spherical harmonics launch");
    }
};

template <int L>
struct ForceLaunch {
    static int run(cgtp_dtype dt, const void *vec, const int32_t *perm, const void *g_sh, int n_parts,
                   int64_t part_stride, int64_t n, void *v, hipStream_t s) {
        unsigned g = grid_for(n);
        if (dt == CGTP_F32)
            CGTP_LAUNCH("k_edge_force", s, (k_edge_force<float, L>), dim3(g), dim3(kBlock), 0, s, (const float *)vec, perm,
                        (const float *)g_sh, n_parts, part_stride, n, (float *)v);
        else
            CGTP_LAUNCH("k_edge_force", s, (k_edge_force<double, L>), dim3(g), dim3(kBlock), 0, s, (const double *)vec, perm,
                        (const double *)g_sh, n_parts, part_stride, n, (double *)v);
        return hip_check(hipGetLastError(), "edge force launch");
    }
};

template <int L>
struct CotLaunch {
    static int run(cgtp_dtype dt, const void *vec, const int32_t *perm, const int32_t *src, const int32_t *dst,
                   const void *F, int64_t n, void *gg, hipStream_t s) {
        unsigned g = grid_for(n);
        if (dt == CGTP_F32)
            CGTP_LAUNCH("k_force_cotangent", s, (k_force_cotangent<float, L>), dim3(g), dim3(kBlock), 0, s, (const float *)vec, perm,
                               src, dst, (const float *)F, n, (float *)gg);
        else
            CGTP_LAUNCH("k_force_cotangent", s, (k_force_cotangent<double, L>), dim3(g), dim3(kBlock), 0, s, (const double *)vec,
                               perm, src, dst, (const double *)F, n, (double *)gg);
        return hip_check(hipGetLastError(), "force cotangent launch");
    }
};


// ---------------------------------------------------------------------------
// uvw channel mixing on the matrix cores:
//   out[item][off3 + w*d3 + k] (=|+=) sum_kk T[(item*d3 + k)*K + kk] * Wb[kk][w]
// T and W are bf16 (raw 16-bit), accumulation in FP32.  Row kk of Wb is row
// (kk - kstart[p]) of path p's weight block [mul1*mul2][mul3] at woff[p].
// A workgroup of four wavefronts stages a chunk of Wb (kMixKC rows x 64
// columns) in LDS; each wavefront computes 16 rows x 64 columns with
// v_mfma_f32_16x16x16_bf16: lane l supplies A[l%16][4(l/16)+0..3] and
// B[4(l/16)+0..3][l%16], and receives D[4(l/16)+i][l%16], i = 0..3.
// ---------------------------------------------------------------------------
constexpr int kMixMaxPaths = 64;
constexpr int kMixKC = 256;   // contraction rows staged per step (32 KiB of bf16 at 64 columns)
constexpr int kMixMaxBlocks = 4;   // output blocks mixed by one launch
// one output block of a mixing launch
struct MixBlockArgs {
    int32_t np, d3, mul3, n_split;
    int32_t rows_uniform;          // rows of every path (mul1 * mul2) when equal, else 0
    int64_t M, K, Kb, off3, t_off, part_off, kspan, wg_start;
    int32_t kstart[kMixMaxPaths + 1];
    int32_t woff[kMixMaxPaths];
};
struct MixArgs {
    int32_t nb;
    MixBlockArgs b[kMixMaxBlocks];
};

typedef short cgtp_s4 __attribute__((ext_vector_type(4)));
typedef float cgtp_f4 __attribute__((ext_vector_type(4)));

// out[item][off3 + w*d3 + k] (=|+=) sum_r T[item*d3 + k][r] W'[r][w]: the
// channel mixing of one output block on the matrix cores.  Contraction row
// r = h*Kb + kk (h < n_rep, kk < Kb) reads weight row
// h*wstride + woff_p + (kk - kstart_p)*mul3 of the path p holding kk (n_rep
// copies of the paths: the rows of a radial network's output layer).  A
// workgroup owns 64 rows of T (16 per wavefront) and 64 output columns and
// stages the weights in LDS kMixKC rows at a time, rows interleaved in groups
// of four: element (r, c) of a chunk sits at ((r/4)*64 + c)*4 + r%4 (before
// the chunk swizzle below), so a lane's B fragment (four consecutive rows of
// one column) is one 8-byte read.
// Per step the A fragments and the weight tiles are loaded together (one
// round trip), the tiles are transposed in registers and written to LDS.
// Split contraction: with n_split > 1, workgroup (g, s) sums only the
// contraction rows [s*kspan, (s+1)*kspan) of row group g and writes its
// partial tile to part[s][row][column]; k_uvw_mix_reduce adds the parts.
// All output blocks of a layer in one launch: workgroups
// [wg_start_b, wg_start_{b+1}) serve block b.
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
// 16-byte chunk j of row group q is stored at chunk j ^ mix_swizzle(q) of that
// group (bits 3 and 1..0 of the chunk index): the tile writes of a wavefront
// then spread over all sixteen 16-byte bank groups, and the B-fragment reads
// touch each group twice at most
__device__ __forceinline__ int mix_swizzle(int q) { return ((q & 1) << 3) | ((q >> 1) & 3); }
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// kFast: every contraction length a multiple of 16, full 64-column weight
// rows in 16-byte segments and 8-byte aligned path tensors, so loads need no
// guards (the general variant checks every element).
template <bool kFast>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) k_uvw_mix(const uint16_t *__restrict__ T0, const uint16_t *__restrict__ W,
                                                 int64_t wstride, MixArgs args, float *__restrict__ out, int64_t dim3,
                                                 int accumulate, float *__restrict__ part0) {
    __shared__ __attribute__((aligned(16))) uint16_t Ws[kMixKC * 64];
    __shared__ int64_t wrow[kMixKC];
    __shared__ int32_t s_kstart[kMixMaxPaths + 1];
    __shared__ int64_t s_woff[kMixMaxPaths];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // this workgroup's block; its fields are read with constant indices
    int bsel = 0;
#pragma unroll
    for (int i = 1; i < kMixMaxBlocks; ++i)
        if (i < args.nb && (int64_t)blockIdx.x >= args.b[i].wg_start) bsel = i;
    int np = 0, d3 = 1, mul3 = 0, n_split = 1;
    int64_t M = 0, K = 0, Kb = 1, off3 = 0, t_off = 0, part_off = 0, kspan = 0, wg_start = 0;
#pragma unroll
    for (int i = 0; i < kMixMaxBlocks; ++i)
        if (i == bsel) {
            np = args.b[i].np, d3 = args.b[i].d3, mul3 = args.b[i].mul3, n_split = args.b[i].n_split;
            M = args.b[i].M, K = args.b[i].K, Kb = args.b[i].Kb, off3 = args.b[i].off3, t_off = args.b[i].t_off;
            part_off = args.b[i].part_off, kspan = args.b[i].kspan, wg_start = args.b[i].wg_start;
            // the path table is indexed by runtime values: keep it in LDS
            if (tid <= np) s_kstart[tid] = args.b[i].kstart[tid];
            if (tid < np) s_woff[tid] = args.b[i].woff[tid];
        }
    __syncthreads();
    const uint16_t *__restrict__ T = T0 + t_off;
    float *__restrict__ part = part0 + part_off;
    const int64_t wg = blockIdx.x - wg_start;
    const int64_t wg_count = (bsel + 1 < args.nb ? args.b[bsel + 1 < kMixMaxBlocks ? bsel + 1 : 0].wg_start
                                                  : (int64_t)gridDim.x) - wg_start;
    const int r_a = lane & 15;
    const int kq = 4 * (lane >> 4);
    const int64_t n_groups = (M + 63) / 64;
    const int split = (int)(wg % n_split);
    const int64_t k_begin = split * kspan, k_end = std::min<int64_t>(K, k_begin + kspan);
    const bool vec_ok = (K % 4) == 0 && (((uintptr_t)T) & 7) == 0;
    // whole 16-byte weight segments: 8-aligned rows and offsets, full columns
    bool wvec = (mul3 % 64) == 0 && (((uintptr_t)W) & 15) == 0 && (wstride % 8) == 0;
    for (int p = 0; p < np; ++p) wvec = wvec && (s_woff[p] % 8) == 0;
    for (int cb = 0; cb < mul3; cb += 64) {
        const int ncol = mul3 - cb < 64 ? mul3 - cb : 64;
        for (int64_t grp = wg / n_split; grp < n_groups; grp += wg_count / n_split) {
            const int64_t row0 = grp * 64 + wv * 16;
            const int64_t arow = row0 + r_a < M ? row0 + r_a : M - 1;
            const uint16_t *__restrict__ Trow = T + arow * K;
            cgtp_f4 acc[4];
            for (int ct = 0; ct < 4; ++ct) acc[ct] = (cgtp_f4){0.f, 0.f, 0.f, 0.f};
            for (int64_t k0 = k_begin; k0 < k_end; k0 += kMixKC) {
                const int kc = (int)(k_end - k0 < kMixKC ? k_end - k0 : kMixKC);
                __syncthreads();   // the previous step's weights and row table are no longer read
                for (int kr = tid; kr < kc; kr += 256) {
                    const int r = (int)(k0 + kr), h = r / (int)Kb, kk = r - h * (int)Kb;
                    int p = 0;
                    while (p + 1 < np && kk >= s_kstart[p + 1]) ++p;
                    wrow[kr] = h * wstride + s_woff[p] + (int64_t)(kk - s_kstart[p]) * mul3 + cb;
                }
                __syncthreads();
                // this lane's A fragments for the whole step, issued with the weight loads
                const int n_st = (kc + 15) / 16;
                const uint16_t *__restrict__ Tk = Trow + k0 + kq;
                // A fragments in two halves: the first is loaded with the weight
                // tiles, the second after the staging barrier, under the first
                // half's matrix operations
                constexpr int kHalf = kMixKC / 32;
                cgtp_s4 af[2][kHalf];
                auto load_a = [&](int hf) {
#pragma unroll
                    for (int j = 0; j < kHalf; ++j) {
                        const int st = hf * kHalf + j;
                        if constexpr (kFast) {
                            // whole 16-row steps; a step past the chunk rereads its last
                            // step (its weight rows are zero)
                            af[hf][j] = *(const cgtp_s4 *)(Tk + 16 * (st < n_st ? st : n_st - 1));
                        } else if (vec_ok && st * 16 + 16 <= kc) {   // uniform: the whole step is inside
                            af[hf][j] = *(const cgtp_s4 *)(Tk + st * 16);
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                af[hf][j][i] = st * 16 + kq + i < kc ? (short)Tk[st * 16 + i] : (short)0;
                        }
                    }
                };
                load_a(0);
                // weight tiles of 4 rows x 8 columns: tile t covers rows 4(t/8)..+3 and
                // columns 8(t%8)..+7; four tiles per thread
#pragma unroll
                for (int j = 0; j < kMixKC * 64 / 32 / 256; ++j) {
                    const int ti = tid + 256 * j, q = ti >> 3, c8 = (ti & 7) * 8;
                    uint4 v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kr = 4 * q + i;
                        if constexpr (kFast) {   // clamped row, zero past the chunk
                            const uint4 t = *(const uint4 *)(W + wrow[kr < kc ? kr : kc - 1] + c8);
                            v[i] = kr < kc ? t : make_uint4(0, 0, 0, 0);
                            continue;
                        }
                        v[i] = make_uint4(0, 0, 0, 0);
                        if (kr >= kc || c8 >= ncol) continue;
                        const uint16_t *__restrict__ src = W + wrow[kr] + c8;
                        if (wvec) {
                            v[i] = *(const uint4 *)src;
                        } else {
                            uint32_t e[8];
#pragma unroll
                            for (int c = 0; c < 8; ++c) e[c] = c8 + c < ncol ? src[c] : 0u;
                            v[i] = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                                              e[6] | (e[7] << 16));
                        }
                    }
                    const uint32_t w0[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
                    const uint32_t w1[4] = {v[1].x, v[1].y, v[1].z, v[1].w};
                    const uint32_t w2[4] = {v[2].x, v[2].y, v[2].z, v[2].w};
                    const uint32_t w3[4] = {v[3].x, v[3].y, v[3].z, v[3].w};
                    uint4 *dst = (uint4 *)Ws + q * 32;
                    const int fq = mix_swizzle(q);
#pragma unroll
                    for (int h = 0; h < 4; ++h)   // columns c8+2h and c8+2h+1
                        dst[((c8 >> 1) + h) ^ fq] = make_uint4(lo_halves(w0[h], w1[h]), lo_halves(w2[h], w3[h]),
                                                               hi_halves(w0[h], w1[h]), hi_halves(w2[h], w3[h]));
                }
                __syncthreads();
                if (row0 >= M) continue;   // this wavefront has no rows (it still joined the barriers)
                if (n_st > kHalf) load_a(1);
                // blocks of eight steps; the steps of the last block past the chunk
                // meet zero weight rows
#pragma unroll
                for (int c = 0; c < kMixKC / 128; ++c) {
                    if (c * 8 >= n_st) break;   // uniform
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int st = c * 8 + j;
                        const int q = 4 * st + (lane >> 4), fq = mix_swizzle(q);
                        const cgtp_s4 *bq = (const cgtp_s4 *)Ws + q * 64 + (r_a & 1);
#pragma unroll
                        for (int ct = 0; ct < 4; ++ct)
                            acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                                af[st / kHalf][st % kHalf], bq[2 * ((8 * ct + (r_a >> 1)) ^ fq)], acc[ct], 0, 0, 0);
                    }
                }
            }
            if (row0 >= M) continue;
            // rows row0+kq+i, i = 0..3: (item, k) of the first by one division, then stepped
            const int64_t rq = row0 + kq;
            const int64_t item_q = rq / d3;
            const int k_q = (int)(rq - item_q * d3);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int col = cb + ct * 16 + r_a;
                if (col >= mul3) continue;
                int64_t item = item_q;
                int k = k_q;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (rq + i < M) {
                        if (n_split > 1) {
                            part[((int64_t)split * M + rq + i) * mul3 + col] = acc[ct][i];
                        } else {
                            float *o = out + item * dim3 + off3 + (int64_t)col * d3 + k;
                            *o = accumulate ? *o + acc[ct][i] : acc[ct][i];
                        }
                    }
                    if (++k == d3) k = 0, ++item;
                }
            }
        }
    }
}

// Second form of the mixing, for blocks whose contraction rows come in whole
// 32-row steps, whose paths hold whole 8-row groups and whose columns come in
// 64-column tiles with 16-byte aligned weights and path tensors (the TFN
// layers).  A workgroup of four wavefronts still owns 64 rows of T (16 per
// wavefront) and 64 output columns, but stages its whole contraction span
// (at most kMix2MaxK rows, 64 KiB) at once and issues every A fragment
// together with the weight loads: one global round trip, one barrier, then
// the products on v_mfma_f32_16x16x32_bf16.  The weight rows of a 32-row step
// are stored interleaved in groups of eight: element (r, c) of the span at
// mix2_slot(r/8, c)*8 + r%8, so a lane's B fragment (eight consecutive rows
// of one column) is one 16-byte read.  Lane l supplies A[l%16][8(l/16)+j] and
// B[8(l/16)+j][l%16], j = 0..7, and receives D[4(l/16)+i][l%16], i = 0..3.
// The row of path p's weight block for contraction row r = h*Kb + kk is
// found once per 8-row group: p = kk / rows when every path has the same
// number of rows, else by a search of the path table.
constexpr int kMix2MaxK = 512;
typedef __bf16 cgtp_bf16x8 __attribute__((ext_vector_type(8)));
// 16-byte slot of column c in 8-row group q: the low three bits of c are
// XORed with ((c >> 3) + q) mod 8, so the staging writes (eight column
// groups of two row groups per 16 lanes) and the fragment reads (16
// consecutive columns) of 16 lanes fall in 16 distinct slots modulo 256 bytes
__device__ __forceinline__ int mix2_slot(int q, int c) { return q * 64 + (c ^ (((c >> 3) + q) & 7)); }

__global__ void __launch_bounds__(256) k_uvw_mix2(const uint16_t *__restrict__ T0, const uint16_t *__restrict__ W,
                                                  int64_t wstride, MixArgs args, float *__restrict__ out,
                                                  int64_t dim3, int accumulate, float *__restrict__ part0) {
    __shared__ __attribute__((aligned(16))) uint16_t Ws[kMix2MaxK * 64];
    __shared__ int32_t s_kstart[kMixMaxPaths + 1];
    __shared__ int64_t s_woff[kMixMaxPaths];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int bsel = 0;
#pragma unroll
    for (int i = 1; i < kMixMaxBlocks; ++i)
        if (i < args.nb && (int64_t)blockIdx.x >= args.b[i].wg_start) bsel = i;
    int np = 0, d3 = 1, mul3 = 0, n_split = 1, rows_u = 0;
    int64_t M = 0, K = 0, Kb = 1, off3 = 0, t_off = 0, part_off = 0, kspan = 0, wg_start = 0;
#pragma unroll
    for (int i = 0; i < kMixMaxBlocks; ++i)
        if (i == bsel) {
            np = args.b[i].np, d3 = args.b[i].d3, mul3 = args.b[i].mul3, n_split = args.b[i].n_split;
            rows_u = args.b[i].rows_uniform;
            M = args.b[i].M, K = args.b[i].K, Kb = args.b[i].Kb, off3 = args.b[i].off3, t_off = args.b[i].t_off;
            part_off = args.b[i].part_off, kspan = args.b[i].kspan, wg_start = args.b[i].wg_start;
            if (tid <= np) s_kstart[tid] = args.b[i].kstart[tid];
            if (tid < np) s_woff[tid] = args.b[i].woff[tid];
        }
    __syncthreads();
    const uint16_t *__restrict__ T = T0 + t_off;
    float *__restrict__ part = part0 + part_off;
    const int64_t wg = blockIdx.x - wg_start;
    const int64_t wg_count = (bsel + 1 < args.nb ? args.b[bsel + 1 < kMixMaxBlocks ? bsel + 1 : 0].wg_start
                                                  : (int64_t)gridDim.x) - wg_start;
    const int r_a = lane & 15, g = lane >> 4;
    const int64_t n_groups = (M + 63) / 64;
    const int split = (int)(wg % n_split);
    const int64_t k_begin = split * kspan, k_end = std::min<int64_t>(K, k_begin + kspan);
    const int kc = (int)(k_end - k_begin);   // a multiple of 32, at most kMix2MaxK
    const int ns = kc / 32;
    for (int cb = 0; cb < mul3; cb += 64) {
        for (int64_t grp = wg / n_split; grp < n_groups; grp += wg_count / n_split) {
            const int64_t row0 = grp * 64 + wv * 16;
            const int64_t arow = row0 + r_a < M ? row0 + r_a : M - 1;
            const cgtp_bf16x8 *__restrict__ Ta = (const cgtp_bf16x8 *)(T + arow * K + k_begin) + g;
            __syncthreads();   // the previous group's weights are no longer read
            // every A fragment of the span, in flight with the weight loads
            cgtp_bf16x8 af[kMix2MaxK / 32];
#pragma unroll
            for (int st = 0; st < kMix2MaxK / 32; ++st)
                af[st] = Ta[4 * (st < ns ? st : 0)];   // clamped: every fragment is a register
            // weight tiles of 8 rows x 8 columns: tile t covers rows 8(t/8)..+7
            // and columns 8(t%8)..+7 of the span
#pragma unroll
            for (int j = 0; j < kMix2MaxK * 64 / 64 / 256; ++j) {
                const int ti = tid + 256 * j, q = ti >> 3, c8 = (ti & 7) * 8;
                if (8 * q >= kc) continue;
                const int64_t r = k_begin + 8 * q;
                const int h = (int)(r / Kb), kk = (int)(r - h * Kb);
                int p;
                if (rows_u > 0) {
                    p = kk / rows_u;
                } else {
                    p = 0;
                    while (p + 1 < np && kk >= s_kstart[p + 1]) ++p;
                }
                const uint16_t *__restrict__ src =
                    W + h * wstride + s_woff[p] + (int64_t)(kk - s_kstart[p]) * mul3 + cb + c8;
                uint4 v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = *(const uint4 *)(src + (int64_t)i * mul3);
                const uint32_t w[8][4] = {{v[0].x, v[0].y, v[0].z, v[0].w}, {v[1].x, v[1].y, v[1].z, v[1].w},
                                          {v[2].x, v[2].y, v[2].z, v[2].w}, {v[3].x, v[3].y, v[3].z, v[3].w},
                                          {v[4].x, v[4].y, v[4].z, v[4].w}, {v[5].x, v[5].y, v[5].z, v[5].w},
                                          {v[6].x, v[6].y, v[6].z, v[6].w}, {v[7].x, v[7].y, v[7].z, v[7].w}};
                uint4 *ws4 = (uint4 *)Ws;
#pragma unroll
                for (int d = 0; d < 4; ++d) {   // columns c8+2d (low halves) and c8+2d+1 (high halves)
                    ws4[mix2_slot(q, c8 + 2 * d)] = make_uint4(lo_halves(w[0][d], w[1][d]), lo_halves(w[2][d], w[3][d]),
                                                               lo_halves(w[4][d], w[5][d]), lo_halves(w[6][d], w[7][d]));
                    ws4[mix2_slot(q, c8 + 2 * d + 1)] =
                        make_uint4(hi_halves(w[0][d], w[1][d]), hi_halves(w[2][d], w[3][d]), hi_halves(w[4][d], w[5][d]),
                                   hi_halves(w[6][d], w[7][d]));
                }
            }
            __syncthreads();
            if (row0 >= M) continue;   // no rows for this wavefront (it still joined the barriers)
            cgtp_f4 acc[4];
            for (int ct = 0; ct < 4; ++ct) acc[ct] = (cgtp_f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < kMix2MaxK / 32; ++st) {
                if (st < ns) {   // uniform
                    const cgtp_bf16x8 *bq = (const cgtp_bf16x8 *)Ws;
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[st], bq[mix2_slot(4 * st + g, r_a + 16 * ct)],
                                                                          acc[ct], 0, 0, 0);
                }
            }
            const int64_t rq = row0 + 4 * g;
            const int64_t item_q = rq / d3;
            const int k_q = (int)(rq - item_q * d3);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int col = cb + ct * 16 + r_a;
                int64_t item = item_q;
                int k = k_q;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (rq + i < M) {
                        if (n_split > 1) {
                            part[((int64_t)split * M + rq + i) * mul3 + col] = acc[ct][i];
                        } else {
                            float *o = out + item * dim3 + off3 + (int64_t)col * d3 + k;
                            *o = accumulate ? *o + acc[ct][i] : acc[ct][i];
                        }
                    }
                    if (++k == d3) k = 0, ++item;
                }
            }
        }
    }
}

// The streaming form, for contractions longer than one span (a radial
// network's (H+1)-fold rows): a workgroup owns 64 rows of T (16 per
// wavefront) and 64 output columns and walks the whole contraction in
// stages of kMix3Stage 32-row steps, so no partial tiles and no reduction.
// Each stage's A fragments (16 bytes per lane and step, straight from T) and
// weight rows (16 bytes per thread and step: row tid/8, columns
// 8 (tid%8) .. + 7) are loaded kMix3Ahead stages before the stage is
// multiplied; the weight rows go to one of two LDS buffers, one barrier per
// stage, and the B fragments come back by two transposed reads (in each
// 16-lane quarter, lane 4 q + r receives element r of the 8-byte reads of
// lanes q, q + 4, q + 8 and q + 12: lane 4 j + q reads row 8 kg + 4 h + j,
// columns 16 ct + 4 q .. + 3, and lane n receives rows 8 kg + 4 h .. + 3 of
// column 16 ct + n).  The weight offset of every 8-row group of the
// contraction is computed once per workgroup into an LDS table.
// 16-byte chunk j of a stored weight row r sits at chunk j ^ mix3_swz(r): the
// 8 rows x 2 chunks of a 32-lane transposed read then fill all 16 bank groups.
constexpr int kMix3Stage = 4;
constexpr int kMix3Ahead = 3;
constexpr int kMix3MaxSteps = 512;   // contraction rows of one block at most 32 x this
__device__ __forceinline__ int mix3_swz(int r) { return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2); }
typedef __attribute__((address_space(3))) cgtp_s4 cgtp_lds_s4;
typedef __bf16 cgtp_bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t cgtp_u32x4 __attribute__((ext_vector_type(4)));   // (a plain vector: kept in registers)

__global__ void __launch_bounds__(256) k_uvw_mix3(const uint16_t *__restrict__ T0, const uint16_t *__restrict__ W,
                                                  int64_t wstride, MixArgs args, float *__restrict__ out,
                                                  int64_t dim3, int accumulate) {
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][kMix3Stage * 32 * 64];
    __shared__ int64_t wtab[kMix3MaxSteps * 4];
    __shared__ int32_t s_kstart[kMixMaxPaths + 1];
    __shared__ int64_t s_woff[kMixMaxPaths];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int bsel = 0;
#pragma unroll
    for (int i = 1; i < kMixMaxBlocks; ++i)
        if (i < args.nb && (int64_t)blockIdx.x >= args.b[i].wg_start) bsel = i;
    int np = 0, d3 = 1, mul3 = 0, rows_u = 0;
    int64_t M = 0, K = 0, Kb = 1, off3 = 0, t_off = 0, wg_start = 0;
#pragma unroll
    for (int i = 0; i < kMixMaxBlocks; ++i)
        if (i == bsel) {
            np = args.b[i].np, d3 = args.b[i].d3, mul3 = args.b[i].mul3, rows_u = args.b[i].rows_uniform;
            M = args.b[i].M, K = args.b[i].K, Kb = args.b[i].Kb, off3 = args.b[i].off3, t_off = args.b[i].t_off;
            wg_start = args.b[i].wg_start;
            if (tid <= np) s_kstart[tid] = args.b[i].kstart[tid];
            if (tid < np) s_woff[tid] = args.b[i].woff[tid];
        }
    __syncthreads();
    const int nsteps = (int)(K / 32);   // K a multiple of 32, at most 32 kMix3MaxSteps
    // weight offset of contraction row 8 i (its 8-row group inside one path)
    for (int i = tid; i < 4 * nsteps; i += 256) {
        const int r = 8 * i, kbi = (int)Kb;
        const int h = r / kbi, kk = r - h * kbi;
        int p = 0;
        if (rows_u > 0)
            p = kk / rows_u;
        else
            while (p + 1 < np && kk >= s_kstart[p + 1]) ++p;
        wtab[i] = h * wstride + s_woff[p] + (int64_t)(kk - s_kstart[p]) * mul3;
    }
    __syncthreads();
    const uint16_t *__restrict__ T = T0 + t_off;
    const int64_t wg = blockIdx.x - wg_start;
    const int64_t wg_count = (bsel + 1 < args.nb ? args.b[bsel + 1 < kMixMaxBlocks ? bsel + 1 : 0].wg_start
                                                  : (int64_t)gridDim.x) - wg_start;
    const int r_a = lane & 15, g = lane >> 4;
    const int64_t n_groups = (M + 63) / 64;
    const int nst = (nsteps + kMix3Stage - 1) / kMix3Stage;
    const int wr = tid >> 3, wc = tid & 7;   // this thread's weight row in a step and its 16-byte chunk
    const int wrow = (wr & 7) * mul3 + 8 * wc;   // its offset inside the row's 8-row group
    const int wsw = 8 * (wc ^ mix3_swz(wr));     // its chunk's place in a stored row
    for (int cb = 0; cb < mul3; cb += 64) {
        for (int64_t grp = wg; grp < n_groups; grp += wg_count) {
            const int64_t row0 = grp * 64 + wv * 16;
            const int64_t arow = row0 + r_a < M ? row0 + r_a : M - 1;
            const cgtp_bf16x8 *__restrict__ Ta = (const cgtp_bf16x8 *)(T + arow * K) + g;
            const uint16_t *__restrict__ Wc = W + cb + wrow;
            // ring slot u holds stage st = u (mod 4) in registers: fragments
            // a<u>[q] and weight rows w<u>[q], q < kMix3Stage
            static_assert(kMix3Ahead == 3, "the ring below is written out for 4 slots");
            cgtp_bf16x8 a0[kMix3Stage], a1[kMix3Stage], a2[kMix3Stage], a3[kMix3Stage];
            cgtp_u32x4 w0[kMix3Stage], w1[kMix3Stage], w2[kMix3Stage], w3[kMix3Stage];
            // loads of stage st; a step past the end reads the last step again
            // (an L2 hit) and its products are skipped.  No load sits in a
            // branch: at a join the compiler would wait for every load in flight.
#define CGTP_MIX3_LOAD(u, st)                                                            \
    {                                                                                    \
        _Pragma("unroll") for (int q = 0; q < kMix3Stage; ++q) {                         \
            const int step_ = (st) * kMix3Stage + q;                                     \
            const int sc_ = step_ < nsteps ? step_ : nsteps - 1;                         \
            a##u[q] = Ta[4 * sc_];                                                       \
            w##u[q] = *(const cgtp_u32x4 *)(Wc + wtab[4 * sc_ + (wr >> 3)]);             \
        }                                                                                \
    }
            // stage st from slot u (loading stage st + 3 into slot un first):
            // weight rows to LDS, barrier, products
#define CGTP_MIX3_STAGE(u, un, st)                                                                            \
    {                                                                                                         \
        CGTP_MIX3_LOAD(un, (st) + kMix3Ahead)                                                                 \
        uint16_t *__restrict__ buf = Ws[(st) & 1];                                                            \
        {                                                                                                     \
            _Pragma("unroll") for (int q = 0; q < kMix3Stage; ++q)                                            \
                *(cgtp_u32x4 *)(buf + (q * 32 + wr) * 64 + wsw) = w##u[q];                                    \
        }                                                                                                     \
        __syncthreads();                                                                                      \
        _Pragma("unroll") for (int q = 0; q < kMix3Stage; ++q) {                                              \
            if ((st) * kMix3Stage + q >= nsteps) break; /* uniform; no load in this branch */                 \
            _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) {                                                \
                cgtp_s4 t2_[2];                                                                               \
                _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                               \
                    const int r = 8 * g + 4 * h + ((lane >> 2) & 3);                                          \
                    const int chunk = (2 * ct + ((lane & 3) >> 1)) ^ mix3_swz(r);                             \
                    t2_[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                         \
                        (cgtp_lds_s4 *)(buf + (q * 32 + r) * 64 + 8 * chunk + 4 * (lane & 1)));               \
                }                                                                                             \
                const cgtp_bf16x8 b_ = __builtin_shufflevector(__builtin_bit_cast(cgtp_bf16x4, t2_[0]),       \
                                                               __builtin_bit_cast(cgtp_bf16x4, t2_[1]), 0, 1, \
                                                               2, 3, 4, 5, 6, 7);                             \
                acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a##u[q], b_, acc[ct], 0, 0, 0);             \
            }                                                                                                 \
        }                                                                                                     \
    }
            CGTP_MIX3_LOAD(0, 0)
            CGTP_MIX3_LOAD(1, 1)
            CGTP_MIX3_LOAD(2, 2)
#pragma unroll
            for (int q = 0; q < kMix3Stage; ++q) a3[q] = a0[q], w3[q] = w0[q];   // defined before slot 3's first use
            cgtp_f4 acc[4];
            for (int ct = 0; ct < 4; ++ct) acc[ct] = (cgtp_f4){0.f, 0.f, 0.f, 0.f};
            // four stages per iteration, the last ones past the end without
            // products; every wavefront runs the same stages (the barriers match)
            for (int st0 = 0; st0 < nst; st0 += 4) {
                CGTP_MIX3_STAGE(0, 3, st0)
                CGTP_MIX3_STAGE(1, 0, st0 + 1)
                CGTP_MIX3_STAGE(2, 1, st0 + 2)
                CGTP_MIX3_STAGE(3, 2, st0 + 3)
            }
#undef CGTP_MIX3_STAGE
#undef CGTP_MIX3_LOAD
            __syncthreads();   // every wavefront is done with both buffers before the next group writes them
            if (row0 >= M) continue;
            const int64_t rq = row0 + 4 * g;
            const int64_t item_q = rq / d3;
            const int k_q = (int)(rq - item_q * d3);
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                const int col = cb + ct * 16 + r_a;
                int64_t item = item_q;
                int k = k_q;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (rq + i < M) {
                        float *o = out + item * dim3 + off3 + (int64_t)col * d3 + k;
                        *o = accumulate ? *o + acc[ct][i] : acc[ct][i];
                    }
                    if (++k == d3) k = 0, ++item;
                }
            }
        }
    }
}

// out[item][off3 + col*d3 + k] (=|+=) sum_s part[s][item*d3 + k][col] for
// every split block of the launch (elements enumerated block after block).
// I: the index type of the element arithmetic (32-bit divisions whenever
// every block's M * mul3 fits).
template <class I>
__global__ void k_uvw_mix_reduce(const float *__restrict__ part0, MixArgs args, int64_t total, float *__restrict__ out,
                                 int64_t dim3, int accumulate) {
    for (int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i0 < total;
         i0 += (int64_t)gridDim.x * blockDim.x) {
        int64_t i = i0;
        int d3 = 1, mul3 = 1, n_split = 1;
        int64_t M = 0, off3 = 0, part_off = 0;
#pragma unroll
        for (int b = 0, done = 0; b < kMixMaxBlocks; ++b) {
            if (done || b >= args.nb || args.b[b].n_split < 2) continue;
            const int64_t cnt = args.b[b].M * args.b[b].mul3;
            if (i < cnt) {
                d3 = args.b[b].d3, mul3 = args.b[b].mul3, n_split = args.b[b].n_split;
                M = args.b[b].M, off3 = args.b[b].off3, part_off = args.b[b].part_off;
                done = 1;
            } else {
                i -= cnt;
            }
        }
        const float *__restrict__ part = part0 + part_off;
        const I ii = (I)i, r = ii / (I)mul3, col = ii - r * (I)mul3;
        float acc = 0.f;
        for (int sp = 0; sp < n_split; ++sp) acc += part[(int64_t)sp * M * mul3 + i];
        const I item = r / (I)d3, k = r - item * (I)d3;
        float *o = out + (int64_t)item * dim3 + off3 + (int64_t)col * d3 + k;
        *o = accumulate ? *o + acc : acc;
    }
}

}  // namespace

// contraction splits of a mixing block: enough workgroups to fill the chip
// (about 512), each split a whole number of staging steps
int mix_splits(const MixBlock &mb, int64_t n_items) {
    const int64_t groups = (n_items * mb.d3 + 63) / 64;
    const int64_t steps = (mb.Kr + kMixKC - 1) / kMixKC;
    // a short contraction is not worth the extra reduction launch
    if (steps <= 2) return 1;
    int64_t sp = (512 + groups - 1) / groups;
    return (int)std::max<int64_t>(1, std::min<int64_t>(sp, steps));
}

// splits of the second mixing form: each span at most kMix2MaxK rows
int mix2_splits(const MixBlock &mb, int64_t n_items) {
    return std::max<int>(mix_splits(mb, n_items), (int)((mb.Kr + kMix2MaxK - 1) / kMix2MaxK));
}

size_t mix_part_bytes(const Plan &p, int64_t n_items) {
    size_t b = 0;   // every split block has its own partial tiles (blocks run together)
    for (const MixBlock &mb : p.mix) {
        // enough for either mixing form
        const int sp = std::max(mix_splits(mb, n_items), mix2_splits(mb, n_items));
        if (sp > 1) b += (size_t)sp * n_items * mb.d3 * mb.mul3;
    }
    return b * sizeof(float);
}

int launch_uvw_mix(const Plan &p, const void *T, const void *w, int64_t n_items, void *out, int accumulate,
                   void *part, hipStream_t s) {
    if (n_items <= 0) return CGTP_OK;
    int64_t part_off = 0;
    for (size_t b0 = 0; b0 < p.mix.size(); b0 += kMixMaxBlocks) {
        MixArgs args{};
        args.nb = (int)std::min<size_t>(kMixMaxBlocks, p.mix.size() - b0);
        int64_t wg = 0, red = 0, red_max = 0;
        // unguarded loads: 16-row contraction steps, whole 16-byte weight
        // segments, 8-byte aligned path-tensor rows
        bool fast = (((uintptr_t)T) & 7) == 0 && (((uintptr_t)w) & 15) == 0 && p.wnumel % 8 == 0;
        // the second form: whole 32-row steps, paths of whole 8-row groups,
        // 16-byte aligned path-tensor rows
        // (by default only where every block's contraction fits one span:
        // more spans than the first form's splits grow the partial sums and
        // their reduction, which measured no net gain on the radial layer)
        bool v2 = p.tune.mix2 != 0 && (((uintptr_t)T) & 15) == 0 && (((uintptr_t)w) & 15) == 0 && p.wnumel % 8 == 0;
        // the streaming form (by default wherever a block's contraction is
        // longer than one span of the second form): the same alignment, whole
        // 32-row steps and 64-column tiles
        bool v3 = p.tune.mix3 != 0 && (((uintptr_t)T) & 15) == 0 && (((uintptr_t)w) & 15) == 0 && p.wnumel % 8 == 0;
        bool v3_wanted = p.tune.mix3 > 0;
        for (int i = 0; i < args.nb; ++i) {
            const MixBlock &mb = p.mix[b0 + i];
            v2 = v2 && mb.K % 32 == 0 && mb.mul3 % 64 == 0 && (n_items * mb.t_off_per_item) % 8 == 0 &&
                 (int)mb.paths.size() <= kMixMaxPaths && (p.tune.mix2 > 0 || mb.Kr <= kMix2MaxK);
            for (int pi : mb.paths)
                v2 = v2 && p.paths[pi].woff % 8 == 0 && ((int64_t)p.paths[pi].mul1 * p.paths[pi].mul2) % 8 == 0;
            v3 = v3 && mb.Kr % 32 == 0 && mb.Kr <= 32 * kMix3MaxSteps && mb.mul3 % 64 == 0 &&
                 (n_items * mb.t_off_per_item) % 8 == 0 && (int)mb.paths.size() <= kMixMaxPaths;
            for (int pi : mb.paths)
                v3 = v3 && p.paths[pi].woff % 8 == 0 && ((int64_t)p.paths[pi].mul1 * p.paths[pi].mul2) % 8 == 0;
            v3_wanted = v3_wanted || mb.Kr > kMix2MaxK;
        }
        v3 = v3 && v3_wanted;
        if (v3) v2 = false;
        for (int i = 0; i < args.nb; ++i) {
            const MixBlock &mb = p.mix[b0 + i];
            fast = fast && mb.Kr % 16 == 0 && mb.mul3 % 64 == 0 && (n_items * mb.t_off_per_item) % 4 == 0;
            for (int pi : mb.paths) fast = fast && p.paths[pi].woff % 8 == 0;
            if ((int)mb.paths.size() > kMixMaxPaths)
                return set_error(CGTP_ERR_UNSUPPORTED, "more than 64 paths into one output block");
            MixBlockArgs &a = args.b[i];
            a.np = (int)mb.paths.size();
            for (int j = 0; j < a.np; ++j) {
                a.kstart[j] = (int32_t)mb.koff[j];
                a.woff[j] = (int32_t)p.paths[mb.paths[j]].woff;
            }
            a.kstart[a.np] = (int32_t)mb.K;
            a.d3 = mb.d3;
            a.mul3 = mb.mul3;
            a.M = n_items * mb.d3;
            a.K = mb.Kr;
            a.Kb = mb.K;
            a.off3 = p.off3[mb.b3];
            a.t_off = n_items * mb.t_off_per_item;
            a.rows_uniform = (int32_t)((int64_t)p.paths[mb.paths[0]].mul1 * p.paths[mb.paths[0]].mul2);
            for (int pi : mb.paths)
                if ((int64_t)p.paths[pi].mul1 * p.paths[pi].mul2 != a.rows_uniform) a.rows_uniform = 0;
            if (v3) {
                a.n_split = 1;
                a.kspan = mb.Kr;
            } else if (v2) {
                a.n_split = mix2_splits(mb, n_items);
                const int64_t steps = mb.Kr / 32;
                a.kspan = (steps + a.n_split - 1) / a.n_split * 32;
            } else {
                a.n_split = mix_splits(mb, n_items);
                const int64_t steps = (mb.Kr + kMixKC - 1) / kMixKC;
                a.kspan = (steps + a.n_split - 1) / a.n_split * kMixKC;
            }
            a.part_off = part_off;
            if (a.n_split > 1) {
                part_off += (int64_t)a.n_split * a.M * a.mul3;
                red += a.M * a.mul3;
                red_max = std::max<int64_t>(red_max, a.M * a.mul3);
            }
            int64_t groups = (a.M + 63) / 64;
            if (groups * a.n_split > 4096) groups = std::max<int64_t>(1, 4096 / a.n_split);
            a.wg_start = wg;
            wg += groups * a.n_split;
        }
        if (v3)
            CGTP_LAUNCH("k_uvw_mix3", s, k_uvw_mix3, dim3((unsigned)wg), dim3(256), 0, s, (const uint16_t *)T,
                        (const uint16_t *)w, p.wnumel, args, (float *)out, p.dim3, accumulate);
        else if (v2)
            CGTP_LAUNCH("k_uvw_mix2", s, k_uvw_mix2, dim3((unsigned)wg), dim3(256), 0, s, (const uint16_t *)T,
                        (const uint16_t *)w, p.wnumel, args, (float *)out, p.dim3, accumulate, (float *)part);
        else if (fast)
            CGTP_LAUNCH("k_uvw_mix", s, k_uvw_mix<true>, dim3((unsigned)wg), dim3(256), 0, s, (const uint16_t *)T,
                        (const uint16_t *)w, p.wnumel, args, (float *)out, p.dim3, accumulate, (float *)part);
        else
            CGTP_LAUNCH("k_uvw_mix", s, k_uvw_mix<false>, dim3((unsigned)wg), dim3(256), 0, s, (const uint16_t *)T,
                        (const uint16_t *)w, p.wnumel, args, (float *)out, p.dim3, accumulate, (float *)part);
        if (red > 0) {
            unsigned g = grid_for(red);
            if (g > 8192) g = 8192;
            if (red_max < (int64_t(1) << 31))
                CGTP_LAUNCH("k_uvw_mix_reduce", s, k_uvw_mix_reduce<uint32_t>, dim3(g), dim3(kBlock), 0, s,
                            (const float *)part, args, red, (float *)out, p.dim3, accumulate);
            else
                CGTP_LAUNCH("k_uvw_mix_reduce", s, k_uvw_mix_reduce<int64_t>, dim3(g), dim3(kBlock), 0, s,
                            (const float *)part, args, red, (float *)out, p.dim3, accumulate);
        }
    }
    return hip_check(hipGetLastError(), "uvw mix launch");
}

// ---------------------------------------------------------------------------
// internal launchers used by the generated-kernel paths
// ---------------------------------------------------------------------------
int launch_segment_sum_rows(cgtp_dtype dt, const void *rows, const int32_t *row_ptr, const int32_t *perm,
                            int64_t n_seg, int64_t width, void *out, int accumulate, hipStream_t s) {
    if (n_seg <= 0 || width <= 0) return CGTP_OK;
    const int per = dt == CGTP_F64 ? 2 : 4;  // elements per thread chunk
    // just enough threads (a multiple of 64, at most 256) for one row
    int64_t chunks = (width + per - 1) / per;
    int threads = (int)std::min<int64_t>(kBlock, (chunks + 63) / 64 * 64);
    int64_t gy = (chunks + threads - 1) / threads;
    if (gy > 65535) gy = 65535;
    // about sixteen workgroups per compute unit, each walking over segments
    // (4096 measured 3 % faster than 2048 on 4096 rows of 512 floats)
    const int64_t gx = std::min<int64_t>(n_seg, 4096);
    dim3 grid((unsigned)gx, (unsigned)gy);
    if (dt == CGTP_F64) {
        if (perm)
            CGTP_LAUNCH("k_segment_sum_rows", s, (k_segment_sum_rows<double, true>), grid, dim3(threads), 0, s,
                        (const double *)rows, row_ptr, perm, n_seg, width, (double *)out, accumulate);
        else
            CGTP_LAUNCH("k_segment_sum_rows", s, (k_segment_sum_rows<double, false>), grid, dim3(threads), 0, s,
                        (const double *)rows, row_ptr, perm, n_seg, width, (double *)out, accumulate);
    } else {
        if (perm)
            CGTP_LAUNCH("k_segment_sum_rows", s, (k_segment_sum_rows<float, true>), grid, dim3(threads), 0, s,
                        (const float *)rows, row_ptr, perm, n_seg, width, (float *)out, accumulate);
        else
            CGTP_LAUNCH("k_segment_sum_rows", s, (k_segment_sum_rows<float, false>), grid, dim3(threads), 0, s,
                        (const float *)rows, row_ptr, perm, n_seg, width, (float *)out, accumulate);
    }
    return hip_check(hipGetLastError(), "segment sum launch");
}

int launch_sum_parts(cgtp_dtype dt, const void *parts, int n_parts, int64_t n, void *out, int accumulate,
                     hipStream_t s) {
    if (n <= 0) return CGTP_OK;
    unsigned g = grid_for(n);
    if (g > 65536) g = 65536;
    if (dt == CGTP_F64)
        CGTP_LAUNCH("k_sum_parts", s, k_sum_parts<double>, dim3(g), dim3(kBlock), 0, s, (const double *)parts, n_parts, n,
                           (double *)out, accumulate);
    else
        CGTP_LAUNCH("k_sum_parts", s, k_sum_parts<float>, dim3(g), dim3(kBlock), 0, s, (const float *)parts, n_parts, n,
                           (float *)out, accumulate);
    return hip_check(hipGetLastError(), "part sum launch");
}

int launch_sh_forces(int lmax, cgtp_dtype dt, const void *vec, const int32_t *perm, const void *g_sh, int n_parts,
                     int64_t part_stride, const int32_t *dst_row_ptr, const int32_t *src_row_ptr,
                     const int32_t *src_perm, int64_t n_nodes, int64_t n_edges, void *F, void *v, hipStream_t s) {
    if (n_edges > 0) {
        int rc = dispatch_l<ForceLaunch>(lmax, dt, vec, perm, g_sh, n_parts, part_stride, n_edges, v, s);
        if (rc) return rc;
    }
    if (n_nodes == 0 || !F) return CGTP_OK;
    unsigned g = (unsigned)n_nodes;
    if (dt == CGTP_F32)
        CGTP_LAUNCH("k_node_force", s, k_node_force<float>, dim3(g), dim3(64), 0, s, (const float *)v, dst_row_ptr,
                    src_row_ptr, src_perm, n_nodes, (float *)F);
    else
        CGTP_LAUNCH("k_node_force", s, k_node_force<double>, dim3(g), dim3(64), 0, s, (const double *)v, dst_row_ptr,
                    src_row_ptr, src_perm, n_nodes, (double *)F);
    return hip_check(hipGetLastError(), "node force launch");
}


int launch_zero(cgtp_dtype dt, void *p, int64_t n, hipStream_t s) {
    if (n <= 0) return CGTP_OK;
    unsigned g = grid_for(n);
    if (g > 65536) g = 65536;
    if (dt == CGTP_F64)
        CGTP_LAUNCH("k_fill", s, k_fill<double>, dim3(g), dim3(kBlock), 0, s, (double *)p, n, 0.0);
    else
        CGTP_LAUNCH("k_fill", s, k_fill<float>, dim3(g), dim3(kBlock), 0, s, (float *)p, n, 0.0f);
    return hip_check(hipGetLastError(), "fill launch");
}

}  // namespace cgtp

using namespace cgtp;

extern "C" {

int cgtp_csr_workspace_bytes(int64_t n_edges, int64_t n_keys, size_t *bytes) {
    clear_error();
    if (!bytes || n_edges < 0 || n_keys < 0)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_csr_workspace_bytes: bad argument");
    *bytes = align256(sizeof(int32_t) * (size_t)(n_keys + 1)) * 2 + align256(sizeof(int32_t) * (size_t)(n_edges + 1));
    return CGTP_OK;
}

int cgtp_build_csr(const int32_t *key, const int32_t *val, int64_t n_edges, int64_t n_keys, int32_t *perm,
                   int32_t *row_ptr, int32_t *sorted_key, int32_t *sorted_val, void *workspace,
                   size_t workspace_bytes, cgtp_stream_t stream) {
    return cgtp_build_csr_order(key, val, n_edges, n_keys, perm, row_ptr, sorted_key, sorted_val, nullptr,
                                workspace, workspace_bytes, stream);
}

int cgtp_build_csr_order(const int32_t *key, const int32_t *val, int64_t n_edges, int64_t n_keys, int32_t *perm,
                         int32_t *row_ptr, int32_t *sorted_key, int32_t *sorted_val, int32_t *order,
                         void *workspace, size_t workspace_bytes, cgtp_stream_t stream) {
    clear_error();
    hipStream_t s = (hipStream_t)stream;
    size_t need = 0;
    cgtp_csr_workspace_bytes(n_edges, n_keys, &need);
    if (n_edges < 0 || n_keys < 0 || n_edges > 0x7fffffff || n_keys > 0x7ffffffe)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_build_csr: sizes out of range");
    if (!row_ptr || (n_edges > 0 && (!key || !perm || (sorted_val && !val))) || !workspace ||
        workspace_bytes < need)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_build_csr: NULL pointer or workspace too small");
    if (order && n_keys == 0) order = nullptr;   // nothing to order
    if (small_csr(n_edges, n_keys)) {
        int nbits = 0;
        while ((int64_t(1) << nbits) < n_keys) ++nbits;
        CGTP_LAUNCH("k_csr_small", s, k_csr_small, dim3((unsigned)small_csr_runs(n_edges)), dim3(1024), 0, s, key, val,
                    n_edges, n_keys, nbits, row_ptr, perm, sorted_key, sorted_val, order);
        return hip_check(hipGetLastError(), "cgtp_build_csr launch");
    }
    char *ws = (char *)workspace;
    int32_t *cnt = (int32_t *)ws;
    int32_t *cursor = (int32_t *)(ws + align256(sizeof(int32_t) * (size_t)(n_keys + 1)));
    int32_t *tmp = (int32_t *)(ws + 2 * align256(sizeof(int32_t) * (size_t)(n_keys + 1)));
    // cnt and cursor are adjacent: one fill clears both
    const int64_t n_clear = (int64_t)(cursor - cnt) + n_keys + 1;
    CGTP_LAUNCH("k_fill", s, k_fill<int32_t>, dim3(grid_for(n_clear)), dim3(kBlock), 0, s, cnt, n_clear, 0);
    if (n_edges > 0 && n_keys > 0) {
        const int64_t bins = std::min<int64_t>(n_keys, kCsrBins);
        const int64_t ranges = (n_keys + kCsrBins - 1) / kCsrBins;
        // runs of at least one edge per counter keep the device atomics (one
        // per nonzero counter of a run) at most one per edge; runs of 4096
        // edges spread the 213,738-edge box over 53 workgroups (16,384:
        // k_scatter 17 us, 4,096: 10 us)
        int64_t per = std::max<int64_t>(4096, bins);
        int64_t splits = (n_edges + per - 1) / per;
        if (splits > 65535) {
            splits = 65535;
            per = (n_edges + splits - 1) / splits;
        }
        const dim3 grid((unsigned)splits, (unsigned)ranges);
        const size_t lds = sizeof(int32_t) * (size_t)bins;
        // each LDS range rereads the keys, so wide key spaces go to device atomics
        const bool lds_path = ranges <= 8;
        const unsigned ge = std::min<unsigned>(grid_for(n_edges), 65536u);
        if (lds_path)
            CGTP_LAUNCH("k_count", s, k_count, grid, dim3(kCsrThreads), lds, s, key, n_edges, n_keys, per, cnt);
        else
            CGTP_LAUNCH("k_count_global", s, k_count_global, dim3(ge), dim3(kBlock), 0, s, key, n_edges, n_keys, cnt);
        int32_t *fold = n_keys <= kOrderSmallMax ? order : nullptr;   // order from the counts, same launch
        CGTP_LAUNCH("k_scan", s, k_scan, dim3(1), dim3(1024), 0, s, cnt, n_keys, row_ptr, fold, cnt + n_keys);
        if (fold) order = nullptr;
        if (lds_path)
            CGTP_LAUNCH("k_scatter", s, k_scatter, grid, dim3(kCsrThreads), lds, s, key, n_edges, n_keys, per, row_ptr,
                        cursor, tmp);
        else
            CGTP_LAUNCH("k_scatter_global", s, k_scatter_global, dim3(ge), dim3(kBlock), 0, s, key, n_edges, n_keys,
                        row_ptr, cursor, tmp);
        // trailing workgroups for hub segments: one per 64 edges, at most
        // kRankHubGroups, within the grid's 2^31 - 1 limit
        const int64_t hub_groups =
            std::max<int64_t>(1, std::min<int64_t>({(n_edges + 63) / 64, kRankHubGroups, 0x7fffffff - n_keys}));
        CGTP_LAUNCH("k_rank_segments", s, k_rank_segments, dim3((unsigned)(n_keys + hub_groups)), dim3(64), 0, s,
                    row_ptr, n_keys, tmp, key, val, cnt + n_keys, perm, sorted_key, sorted_val);
    } else {
        CGTP_LAUNCH("k_fill", s, k_fill<int32_t>, dim3(grid_for(n_keys + 1)), dim3(kBlock), 0, s, row_ptr, n_keys + 1, 0);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_check(e, "cgtp_build_csr launch");
    if (!order) return CGTP_OK;
    // not folded into the counting launches (no edges, or more rows than one
    // workgroup orders): the separate order launches; a wide key space leaves
    // the CSR's workspace, free again in stream order, larger than they need
    if (n_keys <= kOrderSmallMax) {
        CGTP_LAUNCH("k_order_small", s, k_order_small, dim3(1), dim3(1024), 0, s, row_ptr, n_keys, order);
        return hip_check(hipGetLastError(), "cgtp_build_csr order launch");
    }
    return cgtp_node_order(row_ptr, n_keys, order, workspace, workspace_bytes, stream);
}

int cgtp_build_csr_transpose_canonical(const int32_t *src, const int32_t *perm, int64_t n_edges, int64_t n_keys,
                                       int32_t *src_perm, int32_t *src_row_ptr, cgtp_stream_t stream) {
    clear_error();
    if (n_edges < 0 || n_keys < 0 || n_edges > 0x7fffffff || n_keys > 0x7ffffffe)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_build_csr_transpose_canonical: sizes out of range");
    if (!src_row_ptr || (n_edges > 0 && (!src || !perm || !src_perm)))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_build_csr_transpose_canonical: NULL pointer");
    hipStream_t s = (hipStream_t)stream;
    const unsigned g = (unsigned)std::min<int64_t>(grid_for(n_edges + 1), 65536);   // positions 0..E
    CGTP_LAUNCH("k_csr_transpose_canonical", s, k_csr_transpose_canonical, dim3(g), dim3(kBlock), 0, s, src, perm,
                n_edges, n_keys, src_perm, src_row_ptr);
    return hip_check(hipGetLastError(), "cgtp_build_csr_transpose_canonical launch");
}

}  // extern "C"

// Scratch of cgtp_build_csr_order_noalloc: a fixed array in the library's
// device code, one copy per device, held until the process ends.  Host code
// uses it only through the address hipGetSymbolAddress returns on each
// device (the array's name in host code is not a device address).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// the scratch array's address on the current device, looked up once per device
int noalloc_scratch(void **ptr) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_check(e, "cgtp_build_csr_order_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return set_error(CGTP_ERR_UNSUPPORTED, "cgtp_build_csr_order_noalloc: device id");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r != hipSuccess || !p) return hip_check(r != hipSuccess ? r : hipErrorInvalidSymbol,
                                                    "cgtp_build_csr_order_noalloc: scratch address");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return CGTP_OK;
}
}  // namespace

extern "C" {

int cgtp_build_csr_order_noalloc(const int32_t *key, const int32_t *val, int64_t n_edges, int64_t n_keys,
                                 int32_t *perm, int32_t *row_ptr, int32_t *sorted_key, int32_t *sorted_val,
                                 int32_t *order, cgtp_stream_t stream) {
    clear_error();
    if (n_edges < 0 || n_keys < 0 || n_edges > 0x7fffffff || n_keys > 0x7ffffffe)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_build_csr_order_noalloc: sizes out of range");
    size_t need = 0, need_order = 0;
    cgtp_csr_workspace_bytes(n_edges, n_keys, &need);
    cgtp_node_order_workspace_bytes(n_keys, &need_order);
    if (std::max(need, need_order) > kNoallocScratchBytes)
        return set_error(CGTP_ERR_INVALID_ARGUMENT,
                         "cgtp_build_csr_order_noalloc: the graph needs " + std::to_string(std::max(need, need_order)) +
                             " bytes of scratch, more than the library's fixed " +
                             std::to_string(kNoallocScratchBytes) + "; use cgtp_build_csr_order with a workspace");
    void *ws = nullptr;
    const int rc = noalloc_scratch(&ws);
    if (rc) return rc;
    return cgtp_build_csr_order(key, val, n_edges, n_keys, perm, row_ptr, sorted_key, sorted_val, order, ws,
                                kNoallocScratchBytes, stream);
}

int cgtp_node_order_workspace_bytes(int64_t n_nodes, size_t *bytes) {
    clear_error();
    if (!bytes || n_nodes < 0) return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_node_order_workspace_bytes: bad argument");
    *bytes = 3 * align256(sizeof(int32_t) * (kOrderBuckets + 1));
    return CGTP_OK;
}

int cgtp_node_order(const int32_t *row_ptr, int64_t n_nodes, int32_t *order, void *workspace, size_t workspace_bytes,
                    cgtp_stream_t stream) {
    clear_error();
    hipStream_t s = (hipStream_t)stream;
    size_t need = 0;
    cgtp_node_order_workspace_bytes(n_nodes, &need);
    if (n_nodes < 0 || n_nodes > 0x7ffffffe) return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_node_order: n_nodes out of range");
    if (n_nodes == 0) return CGTP_OK;
    if (!row_ptr || !order || !workspace || workspace_bytes < need)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_node_order: NULL pointer or workspace too small");
    if (n_nodes <= kOrderSmallMax) {
        CGTP_LAUNCH("k_order_small", s, k_order_small, dim3(1), dim3(1024), 0, s, row_ptr, n_nodes, order);
        return hip_check(hipGetLastError(), "cgtp_node_order launch");
    }
    const size_t part = align256(sizeof(int32_t) * (kOrderBuckets + 1));
    int32_t *cnt = (int32_t *)workspace;
    int32_t *cursor = (int32_t *)((char *)workspace + part);
    int32_t *start = (int32_t *)((char *)workspace + 2 * part);
    const int64_t n_clear = 2 * (int64_t)(part / sizeof(int32_t));
    CGTP_LAUNCH("k_fill", s, k_fill<int32_t>, dim3(grid_for(n_clear)), dim3(kBlock), 0, s, cnt, n_clear, 0);
    // a few workgroups: each publishes at most kOrderBuckets counts
    const unsigned g = (unsigned)std::min<int64_t>(64, (n_nodes + 4095) / 4096);
    CGTP_LAUNCH("k_order_count", s, k_order_count, dim3(g), dim3(1024), 0, s, row_ptr, n_nodes, cnt);
    CGTP_LAUNCH("k_scan", s, k_scan, dim3(1), dim3(1024), 0, s, cnt, (int64_t)kOrderBuckets, start, nullptr, nullptr);
    CGTP_LAUNCH("k_order_scatter", s, k_order_scatter, dim3(g), dim3(1024), 0, s, row_ptr, n_nodes, start, cursor,
                order);
    return hip_check(hipGetLastError(), "cgtp_node_order launch");
}

int cgtp_validate_csr(const int32_t *row_ptr, int64_t n_rows, int64_t n_edges, const int32_t *idx,
                      int64_t n_idx_range, void *workspace, cgtp_stream_t stream) {
    clear_error();
    hipStream_t s = (hipStream_t)stream;
    if (!row_ptr || !workspace || n_rows < 0 || n_edges < 0)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_validate_csr: bad argument");
    int32_t *bad = (int32_t *)workspace;
    CGTP_LAUNCH("k_fill", s, k_fill<int32_t>, dim3(1), dim3(64), 0, s, bad, 1, 0);
    unsigned g = grid_for(std::max(n_rows, n_edges));
    if (g > 4096) g = 4096;
    CGTP_LAUNCH("k_validate", s, k_validate, dim3(g), dim3(kBlock), 0, s, row_ptr, n_rows, n_edges, idx, n_idx_range, bad);
    int32_t h = 0;
    int rc = hip_check(hipMemcpyAsync(&h, bad, sizeof h, hipMemcpyDeviceToHost, s), "validate copy");
    if (rc) return rc;
    rc = hip_check(hipStreamSynchronize(s), "validate sync");
    if (rc) return rc;
    if (h) return set_error(CGTP_ERR_GRAPH, "CSR validation failed: row_ptr not monotone, wrong ends, or index out of range");
    return CGTP_OK;
}

int cgtp_sh(int32_t lmax, cgtp_dtype dtype, const void *vec, const int32_t *perm, int64_t n, void *sh,
            cgtp_stream_t stream) {
    clear_error();
    if (n < 0 || (n > 0 && (!vec || !sh))) return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sh: bad argument");
    if (dtype != CGTP_F32 && dtype != CGTP_F64 && dtype != CGTP_BF16_F32ACC)
        return set_error(CGTP_ERR_UNSUPPORTED, "cgtp_sh: dtype");
    if (n == 0) return CGTP_OK;
    return dispatch_l<ShLaunch>(lmax, dtype, vec, perm, n, sh, (hipStream_t)stream);
}

int cgtp_sh_vjp_forces(int32_t lmax, cgtp_dtype dtype, const void *vec, const int32_t *perm, const void *g_sh,
                       const int32_t *dst_row_ptr, const int32_t *src_row_ptr, const int32_t *src_perm, int64_t n_nodes,
                       int64_t n_edges, void *g_vec, void *F, void *workspace, size_t workspace_bytes,
                       cgtp_stream_t stream) {
    clear_error();
    hipStream_t s = (hipStream_t)stream;
    if (dtype != CGTP_F32 && dtype != CGTP_F64) return set_error(CGTP_ERR_UNSUPPORTED, "cgtp_sh_vjp_forces: dtype");
    if (n_nodes < 0 || n_edges < 0 || n_edges > 0x7fffffffLL || n_nodes > 0x7fffffffLL)
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sh_vjp_forces: sizes out of range");
    // the per-edge vectors go to g_vec when given, else to the workspace
    const size_t need = g_vec ? 0 : (size_t)n_edges * 3 * (dtype == CGTP_F64 ? 8 : 4);
    if ((F && n_nodes > 0 && (!dst_row_ptr || !src_row_ptr || (n_edges > 0 && !src_perm))) ||
        (n_edges > 0 && (!vec || !g_sh)) || ((F || g_vec) && need > 0 && (!workspace || workspace_bytes < need)))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_sh_vjp_forces: NULL buffer or workspace too small");
    if (!F && !g_vec) return CGTP_OK;
    if (!F) n_nodes = 0;   // the vectors only
    return launch_sh_forces(lmax, dtype, vec, perm, g_sh, 1, 0, dst_row_ptr, src_row_ptr, src_perm, n_nodes, n_edges,
                            F, g_vec ? g_vec : workspace, s);
}

int cgtp_force_loss_sh_cotangent(int32_t lmax, cgtp_dtype dtype, const void *vec, const int32_t *perm,
                                 const int32_t *src, const int32_t *dst, const void *F, int64_t n_edges,
                                 void *gg_sh, cgtp_stream_t stream) {
    clear_error();
    if (dtype != CGTP_F32 && dtype != CGTP_F64)
        return set_error(CGTP_ERR_UNSUPPORTED, "cgtp_force_loss_sh_cotangent: dtype");
    if (n_edges < 0 || (n_edges > 0 && (!vec || !src || !dst || !F || !gg_sh)))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_force_loss_sh_cotangent: bad argument");
    if (n_edges == 0) return CGTP_OK;
    return dispatch_l<CotLaunch>(lmax, dtype, vec, perm, src, dst, F, n_edges, gg_sh, (hipStream_t)stream);
}

}  // extern "C"

// Streaming bandwidth probe (a measurement aid, not part of the hot path):
// every lane moves 16-byte vectors with non-temporal loads and stores over a
// grid-stride loop.  KIND 0 reads src and folds it into one value that is
// stored only if it equals a value no finite input sum reaches (so the loads
// cannot be removed), 1 writes dst, 2 copies src to dst.
template <int KIND>
__global__ void __launch_bounds__(256) k_stream_probe(const float *__restrict__ src, float *__restrict__ dst,
                                                      int64_t n_vec) {
    typedef float V __attribute__((ext_vector_type(4)));
    const V *a = (const V *)src;
    V *b = (V *)dst;
    const int64_t st = (int64_t)gridDim.x * blockDim.x;
    V acc = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n_vec; i += st) {
        if (KIND == 1) {
            const V v = {1.f, 2.f, 3.f, (float)(i & 1023)};
            __builtin_nontemporal_store(v, b + i);
        } else {
            const V v = __builtin_nontemporal_load(a + i);
            if (KIND == 2) __builtin_nontemporal_store(v, b + i);
            else acc += v;
        }
    }
    if (KIND == 0 && acc.x + acc.y + acc.z + acc.w == __builtin_inff()) dst[0] = acc.x;
}

extern "C" int cgtp_stream_probe(int32_t kind, const void *src, void *dst, size_t bytes, cgtp_stream_t stream) {
    clear_error();
    if (kind < 0 || kind > 2 || bytes % 16 || (kind != 1 && !src) || !dst ||
        (((uintptr_t)src | (uintptr_t)dst) & 15))
        return set_error(CGTP_ERR_INVALID_ARGUMENT, "cgtp_stream_probe: bad argument");
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return CGTP_OK;
    hipStream_t s = (hipStream_t)stream;
    // grids measured best on MI355X for each stream kind (1 GiB buffers):
    // reads 2048 workgroups, writes and copies 1024
    const unsigned g = (unsigned)std::min<int64_t>(kind == 0 ? 2048 : 1024, (n + 255) / 256);
    const float *a = (const float *)src;
    float *b = (float *)dst;
    if (kind == 0) CGTP_LAUNCH("k_stream_probe_read", s, k_stream_probe<0>, dim3(g), dim3(256), 0, s, a, b, n);
    else if (kind == 1) CGTP_LAUNCH("k_stream_probe_write", s, k_stream_probe<1>, dim3(g), dim3(256), 0, s, a, b, n);
    else CGTP_LAUNCH("k_stream_probe_copy", s, k_stream_probe<2>, dim3(g), dim3(256), 0, s, a, b, n);
    return hip_check(hipGetLastError(), "stream probe launch");
}
