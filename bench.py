"""Benchmark of the fused CG tensor-product convolution hot path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4|c2|c3|c1|c5]
                    [--no-cpu-baseline]

Default workload (one step = the whole hot path on the 4096-atom periodic
water-density box, cutoff 5 A, node 128x0e+128x1o, SH l<=3, uvu, fp32):
  CSR of the edges by destination (carrying the source index) and the
  transpose CSR by source, spherical harmonics of the edge vectors, fused
  convolution forward, backward (g_x, g_sh, g_w for E = sum of the 0e output
  blocks), forces from g_sh, the force-loss cotangent on the SH, and the
  double backward (d/dx, d/dw, d/dg_out) driven by that cotangent.
Inputs (edge vectors, node features, per-edge weights in CSR order) are
resident in HBM before timing starts.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "edges/sec fused CG-TP conv (fwd, fwd+bwd) + achieved HBM GB/s vs peak, 1 GPU"
HBM_PEAK_GBS = 8000.0
FP64_PEAK_TFLOPS = 78.6


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4", choices=["c4", "c2", "c3", "c1"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    return ap.parse_args()


class Timer:
    """Per-kernel durations from HIP events recorded on the launch stream."""

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


def conv_workload(args, torch, B, W, cfg_name):
    cfg = W.config("c2" if cfg_name in ("c4", "c2") else cfg_name)
    dtype = cfg.dtype
    rng = np.random.default_rng(args.seed)
    g = W.periodic_graph(cfg.extra["n_atoms"], cutoff=cfg.extra["cutoff"], rng=rng)
    plan = B.Plan(cfg.irreps_in1, cfg.irreps_in2, cfg.irreps_out, cfg.paths, cfg.mode, dtype)
    x_np = W.normal(rng, (g.n_nodes, plan.dim_in1), dtype)
    w_np = W.normal(rng, (g.n_edges, plan.weight_numel), dtype)
    return cfg, g, plan, x_np, w_np


def alg_bytes_fwd(N, E, plan, eb):
    # each node array once, each per-edge array once (x gathers from cache
    # not counted): x, out rows; sh, w rows; src; row_ptr
    return (N * (plan.dim_in1 + plan.dim_out) * eb + E * (plan.dim_in2 + plan.weight_numel) * eb
            + E * 4 + (N + 1) * 4)


def alg_bytes_bwd(N, E, plan, eb):
    # reads x, g_out, sh, w, src, row_ptr; writes g_x, g_sh, g_w
    return (N * (2 * plan.dim_in1 + plan.dim_out) * eb + E * 2 * (plan.dim_in2 + plan.weight_numel) * eb
            + E * 4 + (N + 1) * 4)


def cpu_baseline_conv(cfg, g, x_np, w_np, full_step: bool):
    """The oracle as it stands on a bounded sample: the edges into the first
    quarter of the nodes (all nodes kept as sources)."""
    import oracle
    prob = oracle.Problem(cfg.irreps_in1, cfg.irreps_in2, cfg.irreps_out, cfg.mode, cfg.paths)
    n_s = g.n_nodes // 4 if full_step else g.n_nodes // 2
    mask = g.dst < n_s
    src, dst, vec, w = g.src[mask], g.dst[mask], g.vec[mask], w_np[mask]
    E_s = int(mask.sum())
    dt = np.float64 if cfg.dtype == "f64" else np.float32
    vec = vec.astype(dt)
    t0 = time.perf_counter()
    sh = oracle.spherical_harmonics(3, vec)
    perm, rp = oracle.csr(dst, g.n_nodes)
    perm2, rp2 = oracle.csr(src[perm], g.n_nodes)
    out = prob.conv_forward(x_np, sh, w, src, dst, g.n_nodes)
    if full_step:
        G = np.zeros_like(out)
        G[:, zero_e_columns(cfg.irreps_out)] = 1.0
        gx, gsh, gw = prob.conv_backward(x_np, sh, w, src, dst, G)
        F = oracle.forces(3, g.n_nodes, src, dst, vec, gsh)
        gg = oracle.force_loss_cotangent(3, g.n_nodes, src, dst, vec, F)
        prob.conv_double_backward(x_np, sh, w, src, dst, G, None, gg, None)
    dt_s = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    what = "fwd+bwd+forces+double-bwd" if full_step else "fwd"
    return {"value": E_s / dt_s, "unit": "edges/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} over the {E_s} edges into the first {n_s} of {g.n_nodes} nodes "
                      f"(all nodes as sources), {dt_s:.1f} s, OpenMP threads={threads}"}


def zero_e_columns(irreps: str):
    """Columns of the 0e blocks of an irreps row (the energy read-out)."""
    cols, off = [], 0
    for term in irreps.split("+"):
        mul, rest = term.strip().split("x")
        mul, l = int(mul), int(rest[:-1] if rest[-1] in "eo" else rest)
        if rest == "0e":
            cols.extend(range(off, off + mul))
        off += mul * (2 * l + 1)
    return np.array(cols, dtype=np.int64)


def bench_conv(args, torch, B, W):
    cfg, g, plan, x_np, w_np = conv_workload(args, torch, B, W, args.workload)
    dtype = cfg.dtype
    full = args.workload == "c4"
    N, E = g.n_nodes, g.n_edges
    dev = "cuda"
    td = B.TORCH_DTYPES[dtype]
    eb = 8 if dtype == "f64" else 4
    # inputs resident in HBM: canonical edge list and vectors, node features,
    # per-edge weights in CSR (destination-sorted) order
    src_c = torch.from_numpy(g.src).to(dev)
    dst_c = torch.from_numpy(g.dst).to(dev)
    vec = torch.from_numpy(g.vec.astype(np.float64 if dtype == "f64" else np.float32)).to(dev)
    x = torch.from_numpy(x_np).to(dev)
    perm_np = np.argsort(g.dst, kind="stable")
    w = torch.from_numpy(w_np[perm_np]).to(dev)
    # outputs and workspaces preallocated
    perm = torch.empty(E, dtype=torch.int32, device=dev)
    rp = torch.empty(N + 1, dtype=torch.int32, device=dev)
    dst_s = torch.empty(E, dtype=torch.int32, device=dev)
    src_s = torch.empty(E, dtype=torch.int32, device=dev)
    src_perm = torch.empty(E, dtype=torch.int32, device=dev)
    src_rp = torch.empty(N + 1, dtype=torch.int32, device=dev)
    csr_ws = B.workspace(B.cgtp_csr_workspace_bytes(E, N), dev)
    sh = torch.empty(E, plan.dim_in2, dtype=td, device=dev)
    out = torch.empty(N, plan.dim_out, dtype=td, device=dev)
    timer = Timer(torch)
    if full:
        g_out = torch.zeros(N, plan.dim_out, dtype=td, device=dev)
        g_out[:, torch.from_numpy(zero_e_columns(cfg.irreps_out)).to(dev)] = 1.0
        ws = B.workspace(B.cgtp_conv_workspace_bytes(plan, N, E), dev)
        f_ws = B.workspace(B.cgtp_forces_workspace_bytes(E, dtype), dev)
        g_x = torch.empty(N, plan.dim_in1, dtype=td, device=dev)
        g_sh = torch.empty(E, plan.dim_in2, dtype=td, device=dev)
        g_w = torch.empty(E, plan.weight_numel, dtype=td, device=dev)
        F = torch.empty(N, 3, dtype=td, device=dev)
        gg = torch.empty(E, plan.dim_in2, dtype=td, device=dev)
        d_g = torch.empty(N, plan.dim_out, dtype=td, device=dev)
        d_x = torch.empty(N, plan.dim_in1, dtype=td, device=dev)
        d_w = torch.empty(E, plan.weight_numel, dtype=td, device=dev)

    def step(timed: bool):
        run = timer.run if timed else (lambda name, fn: fn())
        run("csr", lambda: (B.cgtp_build_csr(dst_c, N, val=src_c, ws=csr_ws, out=(perm, rp, dst_s, src_s)),
                            B.cgtp_build_csr(src_s, N, sorted_key=False, ws=csr_ws,
                                             out=(src_perm, src_rp, None, None))))
        run("sh", lambda: B.cgtp_spherical_harmonics(3, vec, perm, dtype, out=sh))
        run("conv_fwd", lambda: B.cgtp_conv_forward(plan, x, sh, w, src_s, rp, out=out))
        if not full:
            return
        run("conv_bwd", lambda: B.cgtp_conv_backward(plan, x, sh, w, src_s, dst_s, rp, src_rp, src_perm, g_out,
                                                     ws=ws, out=(g_x, g_sh, g_w)))
        run("forces", lambda: B.cgtp_sh_forces(3, vec, perm, g_sh, rp, src_rp, src_perm, dtype, ws=f_ws, out=F))
        run("force_cot", lambda: B.cgtp_force_loss_sh_cotangent(3, vec, perm, src_s, dst_s, F, dtype, out=gg))
        run("double_bwd", lambda: B.cgtp_conv_double_backward(plan, x, sh, w, src_s, dst_s, rp, src_rp, src_perm,
                                                              g_out, None, gg, None, ws=ws,
                                                              out=(d_g, d_x, None, d_w)))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        step(True)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms = total_ms / args.steps
    kms = timer.ms()
    # dominant kernel and its roofline (algorithmic bytes / measured time)
    ab = {"conv_fwd": alg_bytes_fwd(N, E, plan, eb)}
    if full:
        ab["conv_bwd"] = alg_bytes_bwd(N, E, plan, eb)
    dom = max(ab, key=lambda k: kms[k])
    achieved = ab[dom] / (kms[dom] * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": {"conv_fwd": "cgtp_fwd", "conv_bwd": "cgtp_bwd (+ segment sum)"}[dom],
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "alg_bytes_per_launch": int(ab[dom]), "avg_ms": round(kms[dom], 4)}
    fwd_gbs = ab["conv_fwd"] / (kms["conv_fwd"] * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": E / (ms * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name if not full else W.config("c4").name, "n_atoms": N, "n_edges": E,
                   "irreps_node": cfg.irreps_in1, "irreps_sh": cfg.irreps_in2, "n_paths": plan.n_paths,
                   "step": ("csr+sh+fwd+bwd+forces+force_cotangent+double_bwd" if full else "csr+sh+fwd")},
        "roofline": roof,
        "fwd": {"edges_per_s": E / (kms["conv_fwd"] * 1e-3), "ms": kms["conv_fwd"],
                "GB_per_s": round(fwd_gbs, 1), "frac_hbm_peak": round(fwd_gbs / HBM_PEAK_GBS, 4)},
        "kernel_ms": {k: round(v, 4) for k, v in kms.items()},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_conv(cfg, g, x_np, w_np, full)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    from clebsch_gordan_tensor_cg_amd import workloads as W
    from clebsch_gordan_tensor_cg_amd import binding as B
    if not os.path.exists(B.LIB_PATH):
        from clebsch_gordan_tensor_cg_amd import build as b
        b.build(verbose=False)
    torch.cuda.set_device(0)
    res = bench_conv(args, torch, B, W)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
