// Runs the one-pass forward+backward kernels (cgtp_fb with run-time flags,
// or cgtp_fb_full with the folded ones) of a generated plan source on the
// CPU through tests/emu/shim.h (64 lane fibers per workgroup).  Every buffer is allocated at its exact size,
// so AddressSanitizer reports any access outside it.  Inputs and outputs are
// raw little-endian files in the working directory.  Test infrastructure.
//
// usage: run_fb FULL N E dim1 dim2 dim3 wnumel units ipw flags vec(0/1)
#include "shim.h"

#include <cstdio>
#include <cstdlib>

emu_dim3 threadIdx, blockIdx, blockDim, gridDim;
EmuLane emu_lane[64];
ucontext_t emu_main_ctx;
jmp_buf emu_main_jb;
int emu_done;

#include "kernel.inc"

typedef REAL T;

template <class U>
static U *load(const char *name, size_t n) {
    U *p = (U *)malloc(n * sizeof(U));
    FILE *f = fopen(name, "rb");
    if (!f || fread(p, sizeof(U), n, f) != n) {
        fprintf(stderr, "cannot read %s\n", name);
        exit(2);
    }
    fclose(f);
    return p;
}
template <class U>
static void save(const char *name, const U *p, size_t n) {
    FILE *f = fopen(name, "wb");
    fwrite(p, sizeof(U), n, f);
    fclose(f);
}

int main(int argc, char **argv) {
    if (argc != 12) {
        fprintf(stderr, "usage: run_fb FULL N E dim1 dim2 dim3 wnumel units ipw flags vec\n");
        return 2;
    }
    const int full = atoi(argv[1]);
    const long long N = atoll(argv[2]), E = atoll(argv[3]);
    const long long d1 = atoll(argv[4]), d2 = atoll(argv[5]), d3 = atoll(argv[6]), wn = atoll(argv[7]);
    const int units = atoi(argv[8]), ipw = atoi(argv[9]), flags = atoi(argv[10]), with_vec = atoi(argv[11]);
    T *x = load<T>("x.bin", N * d1);
    T *w = load<T>("w.bin", E * wn);
    T *g = load<T>("g.bin", N * d3);
    int *src = load<int>("src.bin", E);
    int *rp = load<int>("rp.bin", N + 1);
    T *vec = with_vec ? load<T>("vec.bin", E * 3) : nullptr;
    int *vperm = with_vec ? load<int>("vperm.bin", E) : nullptr;
    T *y = with_vec ? nullptr : load<T>("y.bin", E * d2);
    // outputs, zeroed like the host code zeroes them for blocks no path covers
    T *gw = (flags & 1) ? (T *)calloc(E * wn, sizeof(T)) : nullptr;
    T *m = (flags & 2) ? (T *)calloc(E * d1, sizeof(T)) : nullptr;
    const long long third_n = (flags & 64) ? (long long)units * E * d2 : E * d2;
    T *third = (flags & 4) ? (T *)calloc(third_n, sizeof(T)) : nullptr;
    T *out = (T *)calloc(N * d3, sizeof(T));
    const long long n_blocks = (N + ipw - 1) / ipw * units;
    blockDim.x = 64;
    gridDim.x = (unsigned)n_blocks;
    auto lane_body = [&] {
        if (full)
            cgtp_fb_full(x, y, w, src, rp, nullptr, vec, vperm, g, gw, m, third, out, N, E, 1, flags);
        else
            cgtp_fb(x, y, w, src, rp, nullptr, vec, vperm, g, gw, m, third, out, N, E, 1, flags);
    };
    for (long long b = 0; b < n_blocks; ++b) {
        blockIdx.x = (unsigned)b;
        emu_run_group(lane_body);
    }
    save("out_emu.bin", out, N * d3);
    if (gw) save("gw_emu.bin", gw, E * wn);
    if (m) save("m_emu.bin", m, E * d1);
    if (third) save("third_emu.bin", third, third_n);
    printf("emulated %lld workgroups\n", n_blocks);
    free(x); free(w); free(g); free(src); free(rp); free(vec); free(vperm); free(y);
    free(gw); free(m); free(third); free(out);
    return 0;
}
