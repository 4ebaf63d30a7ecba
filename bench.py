"""Benchmark of the fused CG tensor-product convolution hot path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload c4|c2|c3|c1|c5] [--no-cpu-baseline]
                    [--separate-sh] [--bf16-weights] [--all-parity] [--morton]
                    [--natural-order] [--nominal-e] [--unfused] [--graph]

Default workload "c4" (one step = the whole hot path on the 4096-atom
periodic water-density box, cutoff 5 A, node 128x0e+128x1o, SH l<=3, uvu,
fp32): CSR of the edges by destination (carrying the source index), the
transpose CSR by source and the longest-row-first processing order; the
convolution forward and backward in one pass over the edges (out, g_x, g_w,
and the forces of E = sum of the 0e output blocks through the SH Jacobian;
E is linear in out, so g_out = dE/dout is known before the forward), with
the spherical harmonics of the edge vectors computed inside the kernel; the
force-loss cotangent on the SH; and the double backward (d/dx, d/dw,
d/dg_out) driven by that cotangent.  --unfused runs the forward and the
backward as separate calls.  --separate-sh runs the SH and the forces as
kernels of their own with SH and SH-gradient arrays in memory.  Other workloads time the
forward path alone: c2 (same graph), c3 (16384 atoms, fp64, node
128x0e+128x1o+128x2e), c1 (1000 independent products), c5 (100 molecules of
18 atoms, uvw bf16 with matrix-core mixing).  Inputs are resident in HBM
before timing starts.  --graph times replays of the step captured once into
a HIP graph instead of the calls as Python issues them.  Prints one JSON
line.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "edges/sec fused CG-TP conv (fwd, fwd+bwd) + achieved HBM GB/s vs peak, 1 GPU"
HBM_PEAK_GBS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 78.6   # non-packed FMA rate: 256 CU x 2.4 GHz x 64 lanes x 2
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core rate (published, without sparsity)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4", choices=["c4", "c2", "c3", "c1", "c5", "c5r", "attn", "attn_mol"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe-copy", action="store_true",
                    help="kept for old command lines: the 512 MiB device copy now always runs first")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--batch", type=int, default=None,
                    help="c1: items of the single product (default 1000; 1000000 gives a bandwidth figure)")
    ap.add_argument("--bf16-weights", action="store_true",
                    help="c2/c4: per-edge weights stored as bf16 (float arithmetic)")
    ap.add_argument("--all-parity", action="store_true",
                    help="c2/c3/c4: every output parity for l3 <= 3 (13 / 24 paths, one block per path)")
    ap.add_argument("--morton", action="store_true",
                    help="c2/c3/c4: atoms numbered along a Z-order curve of their positions")
    ap.add_argument("--separate-sh", action="store_true",
                    help="SH by their own kernel into an [E][dim2] array read by the convolution, forces from "
                         "a g_sh array (default: SH computed inside the convolution kernels from the edge "
                         "vectors, forces from the backward's SH-gradient partials)")
    ap.add_argument("--natural-order", action="store_true",
                    help="hand destination rows to the device in node-id order (no longest-first order; "
                         "the FP64 c3 layer always uses node-id order)")
    ap.add_argument("--attn-form", default=None, choices=["windows", "rows"],
                    help="attention workloads: 16-row windows on the matrix cores (prepared layout) or the "
                         "row form on the VALU straight from the CSR (default: the faster one measured for the "
                         "graph -- rows for the randomly numbered water box, windows for Morton numbering and "
                         "for the molecule batch)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured once into a HIP graph (default: the library calls as "
                         "Python issues them; graph replay measured slower for these steps)")
    ap.add_argument("--unfused", action="store_true",
                    help="c4: forward and backward as separate calls (default: one pass over the edges)")
    ap.add_argument("--nominal-e", action="store_true",
                    help="c2/c3/c4 graph with cutoff 4.153 A (about 30 neighbours, the nominal edge count)")
    return ap.parse_args()


NOMINAL_CUTOFF = 4.153   # 0.1 / A^3 x (4/3) pi r^3 = 30 neighbours


def time_steps(torch, args, step):
    """args.warmup untimed steps, then args.steps timed steps between HIP
    events (synchronized before and after), with nothing recorded between
    the calls of a step.  With --graph the step is captured once into a HIP
    graph (torch.cuda.CUDAGraph is a hipGraph on ROCm) and replayed: every
    kernel of the step runs on each replay.  Returns (mean ms per step,
    per-step ms, launch mode, graph)."""
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run, graph = step, None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
        run()
        torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    # Python's garbage collector stays off while the steps are issued (as in
    # timeit): a collection pause on the host would leave the GPU idle
    gc_on = gc.isenabled()
    gc.disable()
    try:
        marks[0].record()
        for i in range(args.steps):
            run()
            marks[i + 1].record()
        torch.cuda.synchronize()
    finally:
        if gc_on:
            gc.enable()
    per_step = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    mode = "eager" if graph is None else "hip graph of the step (captured once, replayed)"
    return marks[0].elapsed_time(marks[-1]) / args.steps, per_step, mode, graph


class Timer:
    """Per-kernel durations from HIP events recorded on the launch stream
    (torch's current stream, which every cgtp call launches on)."""

    def __init__(self, torch):
        self.t = torch
        self.pairs = {}

    def run(self, name, fn):
        s = self.t.cuda.Event(enable_timing=True)
        e = self.t.cuda.Event(enable_timing=True)
        s.record()
        r = fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))
        return r

    def ms(self):
        return {k: float(np.mean([s.elapsed_time(e) for s, e in v])) for k, v in self.pairs.items()}


# ---------------------------------------------------------------------------
# algorithmic bytes: each array counted once at its storage size; gathers of
# source-node rows that hit in cache are not counted
# ---------------------------------------------------------------------------
# shb: bytes per edge of the SH operand -- the SH row (dim2 elements), or,
# with the SH computed in the kernel, the edge vector and its index
def alg_bytes_conv_fwd(N, E, d1, d3, wn, eb, ob, wb, shb):
    return N * d1 * eb + N * d3 * ob + E * shb + E * wn * wb + E * 4 + (N + 1) * 4


def alg_bytes_conv_bwd(N, E, d1, d2, d3, wn, eb, wb, shb):
    # reads x, g_out, the SH operand, w, src, row_ptr; writes g_x, g_sh (or
    # its partials), g_w (at the arithmetic width)
    return N * (2 * d1 + d3) * eb + E * (shb + d2 * eb) + E * wn * (wb + eb) + E * 4 + (N + 1) * 4


def alg_bytes_conv_fb(N, E, d1, d2, d3, wn, eb, ob, wb, shb):
    # the backward's arrays plus the forward's output rows
    return alg_bytes_conv_bwd(N, E, d1, d2, d3, wn, eb, wb, shb) + N * d3 * ob


def alg_bytes_conv_dbl(N, E, d1, d2, d3, wn, eb, wb):
    # reads x, g_out, gg_sh, w, src, row_ptr; writes d_g_out, d_x, d_w
    return N * (2 * d1 + 2 * d3) * eb + E * d2 * eb + E * wn * (wb + eb) + E * 4 + (N + 1) * 4


def parse_irreps(s):
    out = []
    for term in s.split("+"):
        mul, rest = term.strip().split("x")
        out.append((int(mul), int(rest[:-1] if rest[-1] in "eo" else rest), rest))
    return out


def zero_e_columns(irreps: str):
    """Columns of the 0e blocks of an irreps row (the energy read-out)."""
    cols, off = [], 0
    for mul, l, name in parse_irreps(irreps):
        if name == "0e":
            cols.extend(range(off, off + mul))
        off += mul * (2 * l + 1)
    return np.array(cols, dtype=np.int64)


def tp_flops(cfg, plan):
    """2 flops per CG nonzero per (u, v) channel pair, from the plan's own
    coupling tensors."""
    a, b, c = parse_irreps(cfg.irreps_in1), parse_irreps(cfg.irreps_in2), parse_irreps(cfg.irreps_out)
    tot = 0
    for p, (i1, i2, i3) in enumerate(plan.paths()):
        R = plan.coupling(p, (2 * a[i1][1] + 1, 2 * b[i2][1] + 1, 2 * c[i3][1] + 1))
        tot += 2 * int((np.abs(R) > 1e-14).sum()) * a[i1][0] * b[i2][0]
    return tot


def counted_traffic_rw(workload, kernel, source):
    """(read, written) bytes per launch leaving L2 toward memory (from the
    per-size request counters; Infinity-Cache hits included, so an upper
    bound on HBM bytes), measured with rocprofv3 for exactly this workload
    (its full description) and generated source (profiles/hbm_traffic__*.json),
    else None."""
    import glob
    import hashlib
    sha = hashlib.sha1(source.encode()).hexdigest()
    for path in glob.glob(os.path.join(ROOT, "profiles", "hbm_traffic__*.json")):
        for r in json.load(open(path))["records"]:
            if r["workload"] == workload and r["kernel"] == kernel and r["source_sha1"] == sha:
                return int(r["read_bytes"]), int(r["write_bytes"])
    return None


def counted_traffic(workload, kernel, source):
    """Counted bytes per launch (reads + writes, see counted_traffic_rw), else None."""
    rw = counted_traffic_rw(workload, kernel, source)
    return None if rw is None else rw[0] + rw[1]


def copy_probe(torch):
    n = 512 * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e)
    return {"bytes_read": 4 * n, "bytes_written": 4 * n, "ms": ms, "GB_per_s": 8 * n / (ms * 1e-3) / 1e9}


def stream_probe(torch, B, nbytes=1 << 30, reps=5):
    """Plain streams on this device through the library's probe kernel
    (16-byte non-temporal loads and stores): 1 GiB read, 1 GiB written,
    1 GiB copied (read + written), each the best of `reps` launches after
    one warm-up.  Buffers four times the Infinity Cache, so the bytes are
    HBM bytes."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    res = {"bytes": nbytes}
    for kind in ("read", "write", "copy"):
        B.cgtp_stream_probe(kind, a, b)
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            s = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            s.record()
            B.cgtp_stream_probe(kind, a, b)
            e.record()
            torch.cuda.synchronize()
            ms = s.elapsed_time(e)
            best = ms if best is None else min(best, ms)
        moved = nbytes * (2 if kind == "copy" else 1)
        res[f"{kind}_GB_per_s"] = round(moved / (best * 1e-3) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return res


def against_streams(roof, sp):
    """The kernel's rate next to the measured plain streams; with counted
    (read, written) bytes, the time those bytes take at the measured read
    and write rates (a serial model that the copy stream follows) and the
    fraction of it the kernel reaches."""
    rw = roof.pop("_rw", None)
    if roof.get("unit") != "GB/s":
        return
    roof["frac_of_measured_read"] = round(roof["achieved"] / sp["read_GB_per_s"], 4)
    if rw is not None:
        model_ms = (rw[0] / (sp["read_GB_per_s"] * 1e9) + rw[1] / (sp["write_GB_per_s"] * 1e9)) * 1e3
        roof["traffic_rw"] = [rw[0], rw[1]]
        roof["traffic_model_ms"] = round(model_ms, 4)
        roof["frac_of_traffic_model"] = round(model_ms / roof["avg_ms"], 4)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands on a bounded sample
# ---------------------------------------------------------------------------
def cpu_baseline_conv(cfg, g, x_np, w_np, full_step: bool, frac: float):
    import oracle
    from clebsch_gordan_tensor_cg_amd import workloads as W
    prob = oracle.Problem(cfg.irreps_in1, cfg.irreps_in2, cfg.irreps_out, cfg.mode, cfg.paths,
                          cfg.shared_weights)
    n_s = max(1, int(g.n_nodes * frac))
    mask = g.dst < n_s
    src, dst, vec = g.src[mask], g.dst[mask], g.vec[mask]
    w = w_np if cfg.shared_weights else w_np[mask]
    E_s = int(mask.sum())
    vec = vec.astype(np.float64 if cfg.dtype == "f64" else np.float32)
    lmax = cfg.extra["lmax"]
    t0 = time.perf_counter()
    sh = oracle.spherical_harmonics(lmax, vec)
    if cfg.dtype == "bf16":
        sh = W.round_to(sh, "bf16")
    perm, rp = oracle.csr(dst, g.n_nodes)
    if full_step:
        oracle.csr(src[perm], g.n_nodes)
    out = prob.conv_forward(x_np, sh, w, src, dst, g.n_nodes)
    if full_step:
        G = np.zeros_like(out)
        G[:, zero_e_columns(cfg.irreps_out)] = 1.0
        gx, gsh, gw = prob.conv_backward(x_np, sh, w, src, dst, G)
        F = oracle.forces(lmax, g.n_nodes, src, dst, vec, gsh)
        gg = oracle.force_loss_cotangent(lmax, g.n_nodes, src, dst, vec, F)
        prob.conv_double_backward(x_np, sh, w, src, dst, G, None, gg, None)
    dt_s = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    what = "csr+sh+fwd+bwd+forces+force_cotangent+double_bwd" if full_step else "csr+sh+fwd"
    return {"value": E_s / dt_s, "unit": "edges/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} over the {E_s} edges into the first {n_s} of {g.n_nodes} nodes "
                      f"(all nodes as sources), {dt_s:.1f} s, OpenMP threads={threads}"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_single_thread(g, x_c2, w_c2, seed: int):
    """The oracle on one thread: the C2 forward on the edges into the first
    2 % of the nodes, and the C1 single product (1000 samples, repeated for
    3 s).  Thread count set through the oracle's OpenMP runtime, restored
    afterwards."""
    import oracle
    from clebsch_gordan_tensor_cg_amd import workloads as W
    c2 = W.config("c2")
    prob = oracle.Problem(c2.irreps_in1, c2.irreps_in2, c2.irreps_out, c2.mode, c2.paths)
    n_s = max(1, g.n_nodes // 50)
    mask = g.dst < n_s
    E_s = int(mask.sum())
    src, dst = g.src[mask], g.dst[mask]
    vec = g.vec[mask].astype(np.float32)
    w = w_c2[mask]
    before = oracle.set_threads(0)
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        sh = oracle.spherical_harmonics(3, vec)
        oracle.csr(dst, g.n_nodes)
        prob.conv_forward(x_c2, sh, w, src, dst, g.n_nodes)
        dt2 = time.perf_counter() - t0
        c1 = W.config("c1")
        p1 = oracle.Problem(c1.irreps_in1, c1.irreps_in2, c1.irreps_out, c1.mode, c1.paths)
        rng = np.random.default_rng(seed)
        n = c1.extra["batch"]
        x = W.normal(rng, (n, p1.dim1), "f32")
        y = W.normal(rng, (n, p1.dim2), "f32")
        wc = W.normal(rng, (n, p1.weight_numel), "f32")
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 3.0:
            p1.tp_forward(x, y, wc)
            reps += 1
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(before)
    return {"cores": 1,
            "c2_fwd": {"value": E_s / dt2, "unit": "edges/s",
                       "sample": f"csr+sh+fwd over the {E_s} edges into the first {n_s} of {g.n_nodes} nodes, "
                                 f"{dt2:.1f} s"},
            "c1": {"value": reps * n / dt1, "unit": "samples/s",
                   "sample": f"{reps} repetitions of the {n}-sample forward, {dt1:.1f} s"}}


def cpu_baseline_single(cfg, x, y, w):
    import oracle
    prob = oracle.Problem(cfg.irreps_in1, cfg.irreps_in2, cfg.irreps_out, cfg.mode, cfg.paths,
                          cfg.shared_weights)
    n = min(x.shape[0], 100000)   # a bounded sample of a large batch
    x, y, w = x[:n], y[:n], w[:n]
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < 5.0:
        prob.tp_forward(x, y, w)
        reps += 1
    dt_s = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": reps * n / dt_s, "unit": "samples/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} repetitions of the {n}-sample forward, {dt_s:.1f} s, OpenMP threads={threads}"}


# ---------------------------------------------------------------------------
# convolution workloads
# ---------------------------------------------------------------------------
def bench_conv(args, torch, B, W):
    name = args.workload
    base = "c2" if name in ("c4", "c2") else name
    if (args.all_parity or args.morton) and name not in ("c2", "c3", "c4"):
        raise SystemExit("--all-parity and --morton apply to the c2, c3 and c4 workloads")
    cfg = W.config(base + ("a" if args.all_parity else ""))
    full = name == "c4"
    if args.unfused and not full:
        raise SystemExit("--unfused applies to the c4 workload")
    fused = full and not args.unfused
    dtype = cfg.dtype
    rng = np.random.default_rng(args.seed)
    if name == "c5":
        g = W.molecule_batch(cfg.extra["n_graphs"], cfg.extra["n_atoms"], cutoff=cfg.extra["cutoff"], rng=rng)
    else:
        cut = NOMINAL_CUTOFF if args.nominal_e else cfg.extra["cutoff"]
        g = W.periodic_graph(cfg.extra["n_atoms"], cutoff=cut, rng=rng, morton=args.morton)
    bf16w = bool(args.bf16_weights)
    sh_in_conv = not args.separate_sh
    if bf16w and name not in ("c2", "c4"):
        raise SystemExit("--bf16-weights applies to the c2 and c4 workloads")
    plan = B.Plan(cfg.irreps_in1, cfg.irreps_in2, cfg.irreps_out, cfg.paths, cfg.mode, dtype,
                  cfg.shared_weights, bf16_weights=bf16w)
    lmax = cfg.extra["lmax"]
    x_np = W.normal(rng, (g.n_nodes, plan.dim_in1), dtype)
    w_np = W.normal(rng, (plan.weight_numel,) if cfg.shared_weights else (g.n_edges, plan.weight_numel), dtype)
    if bf16w:
        w_np = W.round_to(w_np, "bf16")
    N, E = g.n_nodes, g.n_edges
    dev = "cuda"
    td = B.TORCH_DTYPES[dtype]
    od = plan.out_dtype
    eb = {"f64": 8, "f32": 4, "bf16": 2}[dtype]
    wb = 2 if bf16w else eb
    ob = 8 if dtype == "f64" else 4
    # inputs resident in HBM: canonical edge list and vectors, node features,
    # per-edge weights already in CSR (destination-sorted) order
    src_c = torch.from_numpy(g.src).to(dev)
    dst_c = torch.from_numpy(g.dst).to(dev)
    vec = torch.from_numpy(g.vec.astype(np.float64 if dtype == "f64" else np.float32)).to(dev)
    x = torch.from_numpy(x_np).to(dev).to(td)
    if cfg.shared_weights:
        w = torch.from_numpy(w_np).to(dev).to(plan.weight_dtype)
    else:
        w = torch.from_numpy(w_np[np.argsort(g.dst, kind="stable")]).to(dev).to(plan.weight_dtype)
    perm = torch.empty(E, dtype=torch.int32, device=dev)
    rp = torch.empty(N + 1, dtype=torch.int32, device=dev)
    dst_s = torch.empty(E, dtype=torch.int32, device=dev)
    src_s = torch.empty(E, dtype=torch.int32, device=dev)
    src_perm = torch.empty(E, dtype=torch.int32, device=dev)
    src_rp = torch.empty(N + 1, dtype=torch.int32, device=dev)
    csr_ws = B.workspace(B.cgtp_csr_workspace_bytes(E, N), dev)
    order = torch.empty(N, dtype=torch.int32, device=dev)
    # longest rows first, except on the FP64 layer (16,384 rows of even
    # degree), where node-id order measured 2 % faster
    natural = args.natural_order or name == "c3"
    node_order = None if natural else order
    sh = torch.empty(E, plan.dim_in2, dtype=td, device=dev)
    out = torch.empty(N, plan.dim_out, dtype=od, device=dev)
    nb_f = B.cgtp_workspace_bytes(plan, N) if plan.mode == "uvw" else 0
    f_ws = B.workspace(nb_f, dev) if nb_f else None
    timer = Timer(torch)
    if full:
        g_out = torch.zeros(N, plan.dim_out, dtype=td, device=dev)
        g_out[:, torch.from_numpy(zero_e_columns(cfg.irreps_out)).to(dev)] = 1.0
        ws = B.workspace(B.cgtp_workspace_bytes(plan, N, E), dev)
        fo_ws = B.workspace(E * 3 * (8 if dtype == "f64" else 4), dev)
        g_x = torch.empty(N, plan.dim_in1, dtype=td, device=dev)
        g_sh = torch.empty(E, plan.dim_in2, dtype=td, device=dev)
        g_w = torch.empty(E, plan.weight_numel, dtype=td, device=dev)
        F = torch.empty(N, 3, dtype=td, device=dev)
        gg = torch.empty(E, plan.dim_in2, dtype=td, device=dev)
        d_g = torch.empty(N, plan.dim_out, dtype=td, device=dev)
        d_x = torch.empty(N, plan.dim_in1, dtype=td, device=dev)
        d_w = torch.empty(E, plan.weight_numel, dtype=td, device=dev)

    def step(timed: bool):
        run = timer.run if timed else (lambda name_, fn: fn())
        # the transpose CSR (by source) serves only the backward passes; the
        # edge list is canonical (sorted by source, then destination), so it
        # follows from the destination CSR's perm in one launch.  The node
        # order comes out of the destination CSR's own launches
        run("csr", lambda: (B.cgtp_build_csr(dst_c, N, val=src_c, ws=csr_ws, out=(perm, rp, dst_s, src_s))
                            if natural else
                            B.cgtp_build_csr_order(dst_c, N, val=src_c, ws=csr_ws, out=(perm, rp, dst_s, src_s),
                                                   order=order),
                            B.cgtp_build_csr_transpose_canonical(src_c, perm, N, out=(src_perm, src_rp))
                            if full else None))
        if sh_in_conv and fused:
            # one pass: out, g_x, g_w and the forces (from the per-unit
            # SH-gradient partials), SH computed inside the kernel
            run("conv_fb", lambda: B.cgtp_conv_forward_backward_vec(
                plan, x, vec, perm, w, src_s, rp, src_rp, src_perm, g_out, ws=ws, out=(out, g_x, None, g_w, F),
                node_order=node_order))
        elif sh_in_conv:
            # SH computed inside the convolution kernels; forces straight from
            # the backward's per-unit SH-gradient partials
            run("conv_fwd", lambda: B.cgtp_conv_forward_vec(plan, x, vec, perm, w, src_s, rp, out=out, ws=f_ws,
                                                            node_order=node_order))
            if not full:
                return
            run("conv_bwd", lambda: B.cgtp_conv_backward_vec(plan, x, vec, perm, w, src_s, rp, src_rp, src_perm,
                                                             g_out, ws=ws, out=(g_x, None, g_w, F),
                                                             node_order=node_order))
        elif fused:
            run("sh", lambda: B.cgtp_sh(lmax, vec, perm, dtype, out=sh))
            run("conv_fb", lambda: B.cgtp_conv_forward_backward(plan, x, sh, w, src_s, rp, src_rp, src_perm, g_out,
                                                                ws=ws, out=(out, g_x, g_sh, g_w),
                                                                node_order=node_order))
            run("forces", lambda: B.cgtp_sh_vjp_forces(lmax, vec, perm, g_sh, rp, src_rp, src_perm, dtype, ws=fo_ws,
                                                       out=(None, F)))
        else:
            run("sh", lambda: B.cgtp_sh(lmax, vec, perm, dtype, out=sh))
            run("conv_fwd", lambda: B.cgtp_conv_forward(plan, x, sh, w, src_s, rp, out=out, ws=f_ws,
                                                        node_order=node_order))
            if not full:
                return
            run("conv_bwd", lambda: B.cgtp_backward(plan, x, sh, w, src_s, rp, src_rp, src_perm, g_out,
                                                    ws=ws, out=(g_x, g_sh, g_w), node_order=node_order))
            run("forces", lambda: B.cgtp_sh_vjp_forces(lmax, vec, perm, g_sh, rp, src_rp, src_perm, dtype, ws=fo_ws,
                                                       out=(None, F)))
        run("force_cot", lambda: B.cgtp_force_loss_sh_cotangent(lmax, vec, perm, src_s, dst_s, F, dtype, out=gg))
        run("double_bwd", lambda: B.cgtp_double_backward(plan, x, None if sh_in_conv else sh, w, g_out, None, gg,
                                                         None, src_s, rp, src_rp, src_perm, ws=ws,
                                                         out=(d_g, d_x, None, d_w), node_order=node_order))

    ms, per_step, launch_mode, graph = time_steps(torch, args, lambda: step(False))
    # per-call durations: an eager pass with events between the calls
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record()
    for i in range(args.steps):
        step(True)
        marks[i + 1].record()
    torch.cuda.synchronize()
    eager_ms = marks[0].elapsed_time(marks[-1]) / args.steps
    kms = timer.ms()
    # per-kernel durations: one more pass with the library's per-launch
    # events (recorded on the launch stream) enabled
    B.cgtp_timing_enable(True)
    for _ in range(args.steps):
        step(False)
    torch.cuda.synchronize()
    B.cgtp_timing_enable(False)
    per_kernel = {}
    for kname, kms_ in B.cgtp_timing_collect():
        per_kernel.setdefault(kname, []).append(kms_)
    launches = {k: {"calls_per_step": len(v) / args.steps, "avg_ms": float(np.mean(v)),
                    "ms_per_step": float(np.sum(v)) / args.steps} for k, v in per_kernel.items()}

    d1, d2, d3, wn = plan.dim_in1, plan.dim_in2, plan.dim_out, plan.weight_numel
    # algorithmic bytes per launch of the generated kernels (each array once
    # at its storage size; the backward's per-edge x-messages are an
    # intermediate and not counted)
    alg = {}
    vb = 8 if dtype == "f64" else 4
    shb = 3 * vb + 4 if sh_in_conv else d2 * eb
    # the uvw path tensors: the per-pair matrix-core kernel where the plan has it
    pt = "cgtp_uvw_pf" if "cgtp_uvw_pf" in launches else "cgtp_fwd"
    if name == "c5":
        alg[pt] = N * d1 * eb + E * shb + E * 4 + (N + 1) * 4   # path tensors (bf16) stay in cache
    else:
        alg["cgtp_fwd"] = alg_bytes_conv_fwd(N, E, d1, d3, wn, eb, ob, wb, shb)
    if full:
        # the kernels' own traffic: no x-row writes, node rows counted once
        alg["cgtp_bwd"] = N * (d1 + d3) * eb + E * (shb + d2 * eb) + E * wn * (wb + eb) + E * 4 + (N + 1) * 4
        alg["cgtp_dbl"] = N * (d1 + 2 * d3) * eb + E * d2 * eb + E * wn * (wb + eb) + E * 4 + (N + 1) * 4
        # the same kernels with the full call's flags folded in
        alg["cgtp_fb"] = alg["cgtp_bwd"] + N * d3 * ob   # plus the forward's output rows
        alg["cgtp_bwd_full"], alg["cgtp_dbl_full"], alg["cgtp_fb_full"] = alg["cgtp_bwd"], alg["cgtp_dbl"], alg["cgtp_fb"]
    kern = {}
    for k, v in launches.items():
        kern[k] = dict(v)
        if k in alg:
            gbs = alg[k] / (v["avg_ms"] * 1e-3) / 1e9
            kern[k].update({"alg_bytes": int(alg[k]), "GB_per_s": round(gbs, 1),
                            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
    calls = {}
    if "conv_fwd" in kms:
        calls["conv_fwd"] = {"ms": kms["conv_fwd"], "GB_per_s": round(
            alg_bytes_conv_fwd(N, E, d1, d3, wn, eb, ob, wb, shb) / (kms["conv_fwd"] * 1e-3) / 1e9, 1)}
    if "conv_fb" in kms:
        calls["conv_fb"] = {"ms": kms["conv_fb"], "GB_per_s": round(
            alg_bytes_conv_fb(N, E, d1, d2, d3, wn, eb, ob, wb, shb) / (kms["conv_fb"] * 1e-3) / 1e9, 1)}
    if full and "conv_bwd" in kms:
        calls["conv_bwd"] = {"ms": kms["conv_bwd"], "GB_per_s": round(
            alg_bytes_conv_bwd(N, E, d1, d2, d3, wn, eb, wb, shb) / (kms["conv_bwd"] * 1e-3) / 1e9, 1)}
    if full:
        calls["double_bwd"] = {"ms": kms["double_bwd"], "GB_per_s": round(
            alg_bytes_conv_dbl(N, E, d1, d2, d3, wn, eb, wb) / (kms["double_bwd"] * 1e-3) / 1e9, 1)}
    workload = ((W.config("c4").name if full else cfg.name) +
                (f", cutoff {NOMINAL_CUTOFF} A" if args.nominal_e and name != "c5" else "") +
                (", bf16 weight storage" if bf16w else "") +
                (", all output parities" if args.all_parity and full else "") +
                (", Morton node order" if args.morton else "") +
                (", rows in node-id order" if args.natural_order and name != "c3" else "") +
                (", forward and backward as separate calls" if full and not fused else "") +
                (", SH by a separate kernel" if not sh_in_conv else ""))
    # dominant kernel: largest share of the step
    dom = max((k for k in kern if k in alg), key=lambda k: kern[k]["ms_per_step"])
    roof = {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["GB_per_s"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": kern[dom]["frac_hbm_peak"],
            "traffic": counted_traffic(workload, dom, plan.source()),
            "_rw": counted_traffic_rw(workload, dom, plan.source()),
            "alg_bytes_per_launch": kern[dom]["alg_bytes"], "avg_ms": round(kern[dom]["avg_ms"], 4)}
    if name == "c5":
        # the path tensors (and, where they run in the same kernel, the channel
        # mixing) dominate; algorithmic flops: the CG terms of every edge's
        # product and the mixing's multiply-adds
        flop = tp_flops(cfg, plan) * E
        mixes = pt == "cgtp_uvw_pf" and not any(k.startswith("k_uvw_mix") for k in kern)
        if mixes:   # the channel mixing runs inside the same kernel: its flops too
            a_ir, c_ir = parse_irreps(cfg.irreps_in1), parse_irreps(cfg.irreps_out)
            flop += sum(2 * N * (2 * c_ir[b][1] + 1) * c_ir[b][0] *
                        sum(a_ir[i1][0] for (i1, _, i3) in plan.paths() if i3 == b) for b in range(len(c_ir)))
        t_ms = kern[pt]["avg_ms"]
        tf = flop / (t_ms * 1e-3) / 1e12
        # the pair kernel runs its products (and the mixing) on the matrix
        # cores: bf16 MFMA peak; the per-edge kernel on the FP32 VALU
        peak = BF16_MFMA_PEAK_TFLOPS if pt == "cgtp_uvw_pf" else FP32_VECTOR_PEAK_TFLOPS
        roof = {"bound": "mfma" if pt == "cgtp_uvw_pf" else "alu", "kernel": pt, "achieved": round(tf, 3),
                "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 4),
                "traffic": None, "alg_flop_per_launch": int(flop), "avg_ms": round(t_ms, 4)}
        if pt == "cgtp_uvw_pf":
            roof["flop_count"] = ("the CG terms of every edge's product" + (" plus the channel mixing (done in the "
                                  "same kernel)" if mixes else "") + "; the kernel forms each 16-edge chunk's "
                                  "products on the matrix cores and applies the CG terms once per chunk; it is "
                                  "bound by the latency of each node pair's loads, far below this peak")
    res = {
        "metric": METRIC,
        "value": E / (ms * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": float(np.min(per_step)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": workload, "n_atoms": N, "n_edges": E,
                   "irreps_node": cfg.irreps_in1, "irreps_sh": cfg.irreps_in2, "irreps_out": cfg.irreps_out,
                   "n_paths": plan.n_paths,
                   "step": (("csr+sh+fwd+bwd+forces+force_cotangent+double_bwd" +
                             (" (forward and backward in one pass: g_out = dE/dout does not depend on out)"
                              if fused else "")) if full
                            else "csr (by destination) + node order + sh + fwd")},
        "roofline": roof,
        "launch": launch_mode,
        "ms_per_step_with_call_events": round(eager_ms, 4),
        "fwd_edges_per_s": E / (kms["conv_fwd"] * 1e-3) if "conv_fwd" in kms else None,
        "calls": calls,
        "kernels": kern,
        "call_ms": {k: round(v, 4) for k, v in kms.items()},
    }
    if full and fused and sh_in_conv:
        # the forward half of the metric on the same graph, inputs and CSR:
        # the convolution forward alone (SH computed in the kernel), timed
        # over its own K calls, with its own roofline
        res["fwd"] = forward_leg(args, torch, B, plan, x, vec, perm, w, src_s, rp, out, node_order, N, E,
                                 alg_bytes_conv_fwd(N, E, d1, d3, wn, eb, ob, wb, shb),
                                 W.config("c2").name + (", bf16 weight storage" if bf16w else "") +
                                 (", Morton node order" if args.morton else ""))
        res["fwd_edges_per_s"] = res["fwd"]["value"]
    if not args.no_cpu_baseline:
        frac = {"c4": 0.25, "c2": 0.5, "c3": 0.02, "c5": 0.03}[name]
        res["cpu_baseline"] = cpu_baseline_conv(cfg, g, x_np, w_np, full, frac)
        res["cpu_baseline"]["cpu_model"] = cpu_model()
        res["cpu_baseline"]["host_cpus"] = os.cpu_count()
        if "fwd" in res:
            res["fwd"]["cpu_baseline"] = cpu_baseline_conv(cfg, g, x_np, w_np, False, 0.5)
        if name in ("c4", "c2") and not bf16w and not args.all_parity:
            res["cpu_baseline"]["single_thread"] = cpu_single_thread(g, x_np, w_np, args.seed)
    return res


def forward_leg(args, torch, B, plan, x, vec, perm, w, src_s, rp, out, node_order, N, E, alg_bytes, workload):
    """K forward calls (after W untimed ones) between HIP events, then the
    per-launch durations of the forward kernel from the library's events."""
    call = lambda: B.cgtp_conv_forward_vec(plan, x, vec, perm, w, src_s, rp, out=out, node_order=node_order)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record()
    for i in range(args.steps):
        call()
        marks[i + 1].record()
    torch.cuda.synchronize()
    per = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    ms = marks[0].elapsed_time(marks[-1]) / args.steps
    B.cgtp_timing_enable(True)
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    B.cgtp_timing_enable(False)
    kt = [m for k, m in B.cgtp_timing_collect() if k == "cgtp_fwd"]
    k_ms = float(np.mean(kt))
    gbs = alg_bytes / (k_ms * 1e-3) / 1e9
    return {"value": E / (ms * 1e-3), "unit": "edges/s", "ms_per_call": ms, "ms_per_call_median": float(np.median(per)),
            "ms_per_call_min": float(np.min(per)), "calls": args.steps,
            "config": {"workload": workload, "n_atoms": N, "n_edges": E,
                       "step": "conv forward (SH from the edge vectors inside the kernel), CSR and node order "
                               "built beforehand"},
            "roofline": {"bound": "hbm", "kernel": "cgtp_fwd", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": counted_traffic(workload, "cgtp_fwd", plan.source()),
                         "_rw": counted_traffic_rw(workload, "cgtp_fwd", plan.source()),
                         "alg_bytes_per_launch": int(alg_bytes), "avg_ms": round(k_ms, 4)}}


def bench_single(args, torch, B, W):
    cfg = W.config("c1")
    rng = np.random.default_rng(args.seed)
    n = args.batch or cfg.extra["batch"]
    plan = B.Plan(cfg.irreps_in1, cfg.irreps_in2, cfg.irreps_out, cfg.paths, cfg.mode, cfg.dtype)
    x_np = W.normal(rng, (n, plan.dim_in1), "f32")
    y_np = W.normal(rng, (n, plan.dim_in2), "f32")
    w_np = W.normal(rng, (n, plan.weight_numel), "f32")
    x, y, w = (torch.from_numpy(a).cuda() for a in (x_np, y_np, w_np))
    out = torch.empty(n, plan.dim_out, device="cuda")
    ms, per_step, launch_mode, graph = time_steps(torch, args, lambda: B.cgtp_forward(plan, x, y, w, out=out))
    # the kernel alone, from the library's per-launch events
    B.cgtp_timing_enable(True)
    for _ in range(args.steps):
        B.cgtp_forward(plan, x, y, w, out=out)
    torch.cuda.synchronize()
    B.cgtp_timing_enable(False)
    k_ms = float(np.mean([m for k_, m in B.cgtp_timing_collect() if k_ == "cgtp_fwd"]))
    nbytes = n * (plan.dim_in1 + plan.dim_in2 + plan.weight_numel + plan.dim_out) * 4
    gbs = nbytes / (k_ms * 1e-3) / 1e9
    res = {"metric": METRIC, "value": n / (ms * 1e-3), "unit": "samples/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "ms_per_step_median": float(np.median(per_step)),
           "ms_per_step_min": float(np.min(per_step)), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic", "launch": launch_mode,
           "config": {"workload": cfg.name if n == cfg.extra["batch"] else cfg.name.replace(
                          "batch 1000", f"batch {n}"), "batch": n, "n_paths": plan.n_paths},
           "roofline": {"bound": "hbm", "kernel": "cgtp_fwd", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 5), "traffic": None,
                        "alg_bytes_per_launch": nbytes, "avg_ms": round(k_ms, 5)}}
    if nbytes < (64 << 20):
        res["roofline"]["note"] = (f"{nbytes / 1e3:.0f} KB per launch: launch latency, not bandwidth, bounds "
                                   "this size (--batch 1000000 for a bandwidth figure)")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_single(cfg, x_np, y_np, w_np)
    return res


# ---------------------------------------------------------------------------
# TFN layer with per-edge radial weights (uvw, bf16 in, FP32 accumulation)
# ---------------------------------------------------------------------------
RADIAL_HIDDEN = 8


def bench_radial(args, torch, B, W):
    cfg = W.config("c5")
    H = RADIAL_HIDDEN
    rng = np.random.default_rng(args.seed)
    g = W.molecule_batch(cfg.extra["n_graphs"], cfg.extra["n_atoms"], cutoff=cfg.extra["cutoff"], rng=rng)
    plan = B.Plan(cfg.irreps_in1, cfg.irreps_in2, cfg.irreps_out, cfg.paths, "uvw", "bf16", True, radial_hidden=H)
    N, E = g.n_nodes, g.n_edges
    x_np = W.normal(rng, (N, plan.dim_in1), "bf16")
    w_np = W.normal(rng, (H + 1, plan.weight_numel), "bf16") * np.float32(0.5)
    radial_np = np.stack([rng.uniform(-1.0, 1.0, H), rng.uniform(-1.0, 1.0, H)]).astype(np.float32)
    dev = "cuda"
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(torch.bfloat16)
    x, w = bf(x_np), bf(w_np)
    radial = torch.from_numpy(radial_np).to(dev)
    src_c, dst_c = torch.from_numpy(g.src).to(dev), torch.from_numpy(g.dst).to(dev)
    vec = torch.from_numpy(g.vec.astype(np.float32)).to(dev)
    perm = torch.empty(E, dtype=torch.int32, device=dev)
    rp = torch.empty(N + 1, dtype=torch.int32, device=dev)
    dst_s = torch.empty(E, dtype=torch.int32, device=dev)
    src_s = torch.empty(E, dtype=torch.int32, device=dev)
    order = torch.empty(N, dtype=torch.int32, device=dev)
    csr_ws = B.workspace(B.cgtp_csr_workspace_bytes(E, N), dev)
    out = torch.empty(N, plan.dim_out, dtype=torch.float32, device=dev)
    f_ws = B.workspace(B.cgtp_workspace_bytes(plan, N), dev)

    def step():
        B.cgtp_build_csr_order(dst_c, N, val=src_c, ws=csr_ws, out=(perm, rp, dst_s, src_s), order=order)
        B.cgtp_conv_forward_radial(plan, x, vec, perm, radial, w, src_s, rp, out=out, ws=f_ws, node_order=order)

    ms, per_step, launch_mode, graph = time_steps(torch, args, step)
    B.cgtp_timing_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    B.cgtp_timing_enable(False)
    per_kernel = {}
    for kname, kms_ in B.cgtp_timing_collect():
        per_kernel.setdefault(kname, []).append(kms_)
    kern = {k: {"calls_per_step": len(v) / args.steps, "avg_ms": float(np.mean(v)),
                "ms_per_step": float(np.sum(v)) / args.steps} for k, v in per_kernel.items()}
    # path-tensor kernel: the CG products (as in the shared-weight layer) plus
    # one FMA per radial row for every (path, u, v, k) of every edge
    a_ir, c_ir = parse_irreps(cfg.irreps_in1), parse_irreps(cfg.irreps_out)
    outer = sum(2 * H * a_ir[i1][0] * (2 * c_ir[i3][1] + 1) for (i1, _, i3) in plan.paths())
    flop = (tp_flops(cfg, plan) + outer) * E
    t_ms = kern["cgtp_fwd"]["avg_ms"]
    tf = flop / (t_ms * 1e-3) / 1e12
    mix_flop = sum(2 * N * (2 * c_ir[b][1] + 1) * c_ir[b][0] * (H + 1) *
                   sum(a_ir[i1][0] for (i1, _, i3) in plan.paths() if i3 == b) for b in range(len(c_ir)))
    mix_k = next(k for k in ("k_uvw_mix3", "k_uvw_mix2", "k_uvw_mix") if k in kern)
    # the mixing with its partial-tile reduction, if the form has one
    mix_ms = kern[mix_k]["ms_per_step"] + kern.get("k_uvw_mix_reduce", {"ms_per_step": 0.0})["ms_per_step"]
    # the (H+1)-fold path tensors the mixing reads (bf16), every output block
    t_bytes = sum(2 * N * (2 * c_ir[b][1] + 1) * (H + 1) *
                  sum(a_ir[i1][0] for (i1, _, i3) in plan.paths() if i3 == b) for b in range(len(c_ir)))
    res = {"metric": METRIC, "value": E / (ms * 1e-3), "unit": "edges/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "ms_per_step_median": float(np.median(per_step)),
           "ms_per_step_min": float(np.min(per_step)), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "launch": launch_mode,
           "config": {"workload": cfg.name + f", per-edge radial weights (hidden width {H})", "n_atoms": N,
                      "n_edges": E, "n_paths": plan.n_paths,
                      "step": "csr + node order + radial uvw conv (SH and radial network in the kernel)"},
           "roofline": {"bound": "alu", "kernel": "cgtp_fwd", "achieved": round(tf, 3),
                        "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / FP32_VECTOR_PEAK_TFLOPS, 4), "traffic": None,
                        "alg_flop_per_launch": int(flop), "avg_ms": round(t_ms, 4)},
           "mixing": {"kernel": mix_k, "ms_per_step": round(mix_ms, 4),
                      "TFLOP_per_s": round(mix_flop / (mix_ms * 1e-3) / 1e12, 3), "peak_bf16_mfma": 2500.0,
                      "path_tensor_bytes": int(t_bytes), "GB_per_s": round(t_bytes / (mix_ms * 1e-3) / 1e9, 1)},
           "kernels": kern}
    if not args.no_cpu_baseline:
        import oracle
        prob = oracle.Problem(cfg.irreps_in1, cfg.irreps_in2, cfg.irreps_out, "uvw", cfg.paths, shared_weights=False)
        n_s = max(1, N // 100)
        mask = g.dst < n_s
        v64 = g.vec[mask].astype(np.float32).astype(np.float64)
        t0 = time.perf_counter()
        sh = oracle.spherical_harmonics(6, v64)
        oracle.conv_forward_radial(prob, x_np, sh, np.linalg.norm(v64, axis=1), radial_np, w_np, g.src[mask],
                                   g.dst[mask], N)
        dt = time.perf_counter() - t0
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        res["cpu_baseline"] = {"value": int(mask.sum()) / dt, "unit": "edges/s", "cores": threads, "kind": "oracle",
                               "sample": f"radial network + SH + conv over the {int(mask.sum())} edges into the first "
                                         f"{n_s} of {N} nodes, {dt:.1f} s, OpenMP threads={threads}"}
    return res


# ---------------------------------------------------------------------------
# fused graph sparse attention (SDDMM, softmax, SpMM on the matrix cores)
# ---------------------------------------------------------------------------
MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_attention(args, torch, B, W):
    rng = np.random.default_rng(args.seed)
    if args.workload == "attn":
        g = W.periodic_graph(4096, cutoff=5.0, rng=rng, morton=args.morton)
        H, D, what = 8, 32, "graph attention on the 4096-atom water box (cutoff 5 A), 8 heads x 32"
    else:
        g = W.molecule_batch(100, 18, cutoff=5.0, rng=rng)
        H, D, what = 8, 16, "graph attention on 100 molecules x 18 atoms (cutoff 5 A), 8 heads x 16"
    if args.morton:
        what += ", Morton node order"
    N, E = g.n_nodes, g.n_edges
    q_np, k_np, v_np = (W.normal(rng, (N, H, D), "bf16") for _ in range(3))
    perm = np.argsort(g.dst, kind="stable")
    rp_np = np.concatenate([[0], np.cumsum(np.bincount(g.dst, minlength=N))]).astype(np.int32)
    bf = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    q, k, v = bf(q_np), bf(k_np), bf(v_np)
    col = torch.from_numpy(g.src[perm].astype(np.int32)).cuda()
    rp = torch.from_numpy(rp_np).cuda()
    out = torch.empty(N, H, D, dtype=torch.float32, device="cuda")
    form = args.attn_form or ("rows" if args.workload == "attn" and not args.morton else "windows")
    rows_form = form == "rows"
    if rows_form:
        # straight from the CSR: nothing is prepared
        prepare_ms = 0.0
        kname = "k_sparse_attention_rows_bf16"
        call = lambda: B.cgtp_sparse_attention_rows(q, k, v, col, rp, out=out)
    else:
        # the graph is compacted once (it serves every head, layer and call);
        # its cost is reported beside the step
        layout = B.cgtp_sparse_attention_prepare(col, rp, N)
        torch.cuda.synchronize()
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        p0.record()
        B.cgtp_sparse_attention_prepare(col, rp, N, out=layout)
        p1.record()
        torch.cuda.synchronize()
        prepare_ms = p0.elapsed_time(p1)
        kname = "k_sparse_attention_bf16"
        call = lambda: B.cgtp_sparse_attention(q, k, v, rp, E, layout, out=out)
    ms, per_step, launch_mode, graph = time_steps(torch, args, call)
    B.cgtp_timing_enable(True)
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    B.cgtp_timing_enable(False)
    kt = [m for n_, m in B.cgtp_timing_collect() if n_ == kname]
    k_ms = float(np.mean(kt))
    flop = 4.0 * E * H * D          # two products of length D per edge and head
    tf = flop / (k_ms * 1e-3) / 1e12
    peak = FP32_VECTOR_PEAK_TFLOPS if rows_form else MFMA_BF16_PEAK_TFLOPS
    nbytes = 3 * N * H * D * 2 + N * H * D * 4 + E * 4 + (N + 1) * 4
    res = {"metric": METRIC, "value": E / (ms * 1e-3), "unit": "edges/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "ms_per_step_median": float(np.median(per_step)),
           "ms_per_step_min": float(np.min(per_step)), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "launch": launch_mode,
           "config": {"workload": what, "n_nodes": N, "n_edges": E, "heads": H, "head_dim": D,
                      "step": ("fused SDDMM + softmax + SpMM, row form from the CSR (CSR built once, outside the step)"
                               if rows_form else
                               "fused SDDMM + softmax + SpMM (CSR and window compaction built once, outside the step)"),
                      "prepare_ms": round(prepare_ms, 4)},
           "roofline": {"bound": "alu" if rows_form else "mfma", "kernel": kname, "achieved": round(tf, 3),
                        "peak": peak, "unit": "TFLOP/s", "frac": round(tf / peak, 5),
                        "traffic": None, "alg_flop_per_launch": int(flop), "alg_bytes_per_launch": int(nbytes),
                        "avg_ms": round(k_ms, 4),
                        "note": "useful products only (4 E H D); operands are cache-resident at this size"}}
    if not args.no_cpu_baseline:
        import oracle
        n_s = N // 4
        mask = g.dst < n_s
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 5.0:
            oracle.sparse_attention(q_np, k_np, v_np, g.src[mask], g.dst[mask], n_s)
            reps += 1
        dt = time.perf_counter() - t0
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        res["cpu_baseline"] = {"value": reps * int(mask.sum()) / dt, "unit": "edges/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"{reps} repetitions over the {int(mask.sum())} edges into the first {n_s} "
                                         f"of {N} rows, {dt:.1f} s, OpenMP threads={threads}"}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "one GPU only: --gpus must be 1 (no path across GPUs is built)",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    from clebsch_gordan_tensor_cg_amd import workloads as W
    from clebsch_gordan_tensor_cg_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        from clebsch_gordan_tensor_cg_amd import build as b
        b.build(verbose=False)
    torch.cuda.set_device(0)
    probe = copy_probe(torch)
    sprobe = stream_probe(torch, B)
    if args.workload == "c1":
        res = bench_single(args, torch, B, W)
    elif args.workload == "c5r":
        res = bench_radial(args, torch, B, W)
    elif args.workload in ("attn", "attn_mol"):
        res = bench_attention(args, torch, B, W)
    else:
        res = bench_conv(args, torch, B, W)
    # context: the dominant kernel against a measured device-copy stream
    # (512 MiB read + 512 MiB written), next to the datasheet peak
    res["copy_probe"] = probe
    res["stream_probe"] = sprobe
    roof = res["roofline"]
    if roof["unit"] == "GB/s":
        roof["frac_of_measured_copy"] = round(roof["achieved"] / probe["GB_per_s"], 4)
    against_streams(roof, sprobe)
    if "fwd" in res:
        against_streams(res["fwd"]["roofline"], sprobe)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
