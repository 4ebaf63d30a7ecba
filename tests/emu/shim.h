// Host emulation of the HIP subset that the generated convolution kernels
// use, for running them on the CPU under AddressSanitizer.  The 64 lanes of
// a wavefront are fibers (ucontext) on one host thread; a barrier --
// __syncthreads, a wavefront sync, each half of a cross-lane shuffle --
// switches to the next lane, round robin, so every lane reaches a barrier
// before any lane passes it (the kernels reach their barriers uniformly).
// Workgroups (one wavefront each) run one after another; LDS arrays become
// function statics shared by the lanes.  Stack switches are announced to
// AddressSanitizer through its fiber interface.  Test infrastructure only.
#pragma once
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <csetjmp>
#include <ucontext.h>
#include <sanitizer/common_interface_defs.h>

struct emu_dim3 {
    unsigned x = 0, y = 0, z = 0;
};
extern emu_dim3 threadIdx, blockIdx, blockDim, gridDim;

struct EmuLane {
    ucontext_t ctx;        // the lane's first entry
    jmp_buf jb;            // where it waits at its current barrier
    bool started = false;
    char *stack = nullptr;
};
constexpr size_t kEmuStack = size_t(4) << 20;
extern EmuLane emu_lane[64];
extern ucontext_t emu_main_ctx;
extern jmp_buf emu_main_jb;
extern int emu_done;

// switch from the running lane to lane `to` (to < 0: back to the host once
// the workgroup has finished).  A lane is entered the first time through
// its context and afterwards by a jump to its barrier (no system call).
inline void emu_switch(int to) {
    const int from = (int)threadIdx.x;
    void *fake = nullptr;
    if (_setjmp(emu_lane[from].jb) == 0) {
        if (to < 0) {
            __sanitizer_start_switch_fiber(nullptr, nullptr, 0);
            _longjmp(emu_main_jb, 1);
        }
        __sanitizer_start_switch_fiber(&fake, emu_lane[to].stack, kEmuStack);
        threadIdx.x = (unsigned)to;
        if (!emu_lane[to].started) {
            emu_lane[to].started = true;
            setcontext(&emu_lane[to].ctx);
        }
        _longjmp(emu_lane[to].jb, 1);
    }
    __sanitizer_finish_switch_fiber(fake, nullptr, nullptr);
}
inline void emu_barrier() { emu_switch(((int)threadIdx.x + 1) & 63); }

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static
#define __syncthreads() emu_barrier()
#define __builtin_amdgcn_fence(...) ((void)0)
#define __builtin_amdgcn_wave_barrier() emu_barrier()

using std::fma;
using std::sqrt;

template <class T>
inline T __shfl_xor(T v, int mask, int width = 64) {
    static T buf[64];
    const int lane = (int)threadIdx.x;
    buf[lane] = v;
    emu_barrier();
    const T r = buf[(lane ^ mask) & (width - 1)];
    emu_barrier();
    return r;
}
inline float __uint_as_float(unsigned u) {
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}
inline unsigned __float_as_uint(float f) {
    unsigned u;
    std::memcpy(&u, &f, 4);
    return u;
}
inline float __expf(float v) { return std::exp(v); }
inline float __int_as_float(int u) {
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}
inline int __float_as_int(float f) {
    int u;
    std::memcpy(&u, &f, 4);
    return u;
}
inline long long __double_as_longlong(double d) {
    long long u;
    std::memcpy(&u, &d, 8);
    return u;
}
inline double __longlong_as_double(long long u) {
    double d;
    std::memcpy(&d, &u, 8);
    return d;
}

// Cross-lane moves of the gfx950 instruction set, as documented: the pair
// returned by a swap is (new first operand, new second operand).
struct emu_u2 {
    unsigned v[2];
    unsigned operator[](int i) const { return v[i]; }
};
// lanes 32-63 of a trade places with lanes 0-31 of b
inline emu_u2 __builtin_amdgcn_permlane32_swap(unsigned a, unsigned b, bool, bool) {
    static unsigned ba[64], bb[64];
    const int lane = (int)threadIdx.x;
    ba[lane] = a;
    bb[lane] = b;
    emu_barrier();
    emu_u2 r;
    r.v[0] = lane < 32 ? ba[lane] : bb[lane - 32];
    r.v[1] = lane < 32 ? ba[lane + 32] : bb[lane];
    emu_barrier();
    return r;
}
// odd rows (16 lanes) of a trade places with the even rows of b below them
inline emu_u2 __builtin_amdgcn_permlane16_swap(unsigned a, unsigned b, bool, bool) {
    static unsigned ba[64], bb[64];
    const int lane = (int)threadIdx.x;
    const bool odd = (lane >> 4) & 1;
    ba[lane] = a;
    bb[lane] = b;
    emu_barrier();
    emu_u2 r;
    r.v[0] = odd ? bb[lane - 16] : ba[lane];
    r.v[1] = odd ? bb[lane] : ba[lane + 16];
    emu_barrier();
    return r;
}
// data-parallel-primitive moves within rows of 16 lanes: row mirror, half-row
// mirror and quad permutations (the controls the kernels use)
inline int __builtin_amdgcn_mov_dpp(int v, int ctrl, int, int, bool) {
    static int buf[64];
    const int lane = (int)threadIdx.x;
    buf[lane] = v;
    emu_barrier();
    const int base = lane & ~15, l = lane & 15;
    int src;
    if (ctrl == 0x140) src = base + (15 - l);
    else if (ctrl == 0x141) src = base + (l & 8) + (7 - (l & 7));
    else if (ctrl >= 0 && ctrl < 0x100) src = (lane & ~3) + ((ctrl >> (2 * (lane & 3))) & 3);
    else std::abort();
    const int r = buf[src];
    emu_barrier();
    return r;
}

// Runs one workgroup of 64 lanes: lane l runs body() with threadIdx.x == l.
template <class F>
struct EmuGroup {
    static F *body;
    static void entry() {
        __sanitizer_finish_switch_fiber(nullptr, nullptr, nullptr);
        (*body)();
        // every lane finishes in the same round; the last one returns to the host
        if (++emu_done == 64) emu_switch(-1);
        else emu_switch(((int)threadIdx.x + 1) & 63);
    }
};
template <class F>
F *EmuGroup<F>::body = nullptr;

template <class F>
void emu_run_group(F &f) {
    EmuGroup<F>::body = &f;
    emu_done = 0;
    for (int l = 0; l < 64; ++l) {
        if (!emu_lane[l].stack) emu_lane[l].stack = (char *)std::malloc(kEmuStack);
        getcontext(&emu_lane[l].ctx);
        emu_lane[l].ctx.uc_stack.ss_sp = emu_lane[l].stack;
        emu_lane[l].ctx.uc_stack.ss_size = kEmuStack;
        emu_lane[l].ctx.uc_link = nullptr;
        emu_lane[l].started = false;
        makecontext(&emu_lane[l].ctx, (void (*)())EmuGroup<F>::entry, 0);
    }
    void *fake = nullptr;
    if (_setjmp(emu_main_jb) == 0) {
        threadIdx.x = 0;
        emu_lane[0].started = true;
        __sanitizer_start_switch_fiber(&fake, emu_lane[0].stack, kEmuStack);
        setcontext(&emu_lane[0].ctx);
    }
    __sanitizer_finish_switch_fiber(fake, nullptr, nullptr);
}
