"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This module only draws inputs: atom positions, neighbour lists, node
features and per-edge weights.  It holds none of the tensor-product
arithmetic (no CG, no spherical harmonics, no contraction), so the oracle
and the HIP path can both take their inputs from it.

Recipes (the pages name the workloads but publish no inputs):
  * MACE-like periodic boxes at water atom density (about 0.1 atoms per
    cubic angstrom), cutoff 5 angstrom, as in the low-precision MACE page
    (NVT/NPT water simulations).  Directed edges are ordered pairs i != j
    with minimum-image distance strictly below the cutoff; no self loops.
  * Molecule batches for the TFN / SE(3)-Transformer layer: 100 graphs of
    18 atoms, QM9-sized, all pairs within 5 angstrom (the QM9 dataset is not
    available; these stand in for its shape only).
  * Node features and radial weights ~ N(0, 1) drawn in float64 with
    numpy's PCG64 generator, then rounded to the workload dtype.

Draw order for a seed: positions, then node features, then per-edge
weights (edges in canonical (src, dst) lexicographic order).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WATER_DENSITY = 0.1  # atoms / A^3


@dataclass
class Graph:
    n_nodes: int
    pos: np.ndarray          # [N, 3] float64
    src: np.ndarray          # [E] int32, canonical (src, dst) lexicographic order
    dst: np.ndarray          # [E] int32
    vec: np.ndarray          # [E, 3] float64, pos[dst] - pos[src] (minimum image)
    box: float | None = None

    @property
    def n_edges(self) -> int:
        return int(self.src.shape[0])


def _canonical(src, dst, vec):
    order = np.lexsort((dst, src))
    return (src[order].astype(np.int32), dst[order].astype(np.int32), vec[order])


def morton_order(pos: np.ndarray, box: float, bits: int = 10) -> np.ndarray:
    """Permutation of the atoms along a Z-order (Morton) curve of their
    positions in a cube of side `box`: interleaved bits of the quantised
    x, y, z coordinates, ties by atom index."""
    q = np.clip((pos / box * (1 << bits)).astype(np.int64), 0, (1 << bits) - 1)
    code = np.zeros(len(pos), dtype=np.int64)
    for b in range(bits):
        for axis in range(3):
            code |= ((q[:, axis] >> b) & 1) << (3 * b + axis)
    return np.lexsort((np.arange(len(pos)), code))


def periodic_graph(n_atoms: int, density: float = WATER_DENSITY, cutoff: float = 5.0,
                   seed: int = 0, rng: np.random.Generator | None = None, morton: bool = False) -> Graph:
    """Atoms uniform in a periodic cube; directed minimum-image pairs < cutoff.
    morton=True numbers the atoms along a Z-order curve of their positions
    (same draws, same pairs; only the node ids change)."""
    from scipy.spatial import cKDTree

    rng = np.random.default_rng(seed) if rng is None else rng
    L = (n_atoms / density) ** (1.0 / 3.0)
    pos = rng.uniform(0.0, L, size=(n_atoms, 3))
    if morton:
        pos = pos[morton_order(pos, L)]
    if cutoff >= L / 2:
        raise ValueError("cutoff must be below half the box for minimum image")
    tree = cKDTree(pos, boxsize=L)
    pairs = tree.query_pairs(cutoff * (1 + 1e-9), output_type="ndarray")
    i, j = pairs[:, 0], pairs[:, 1]
    d = pos[j] - pos[i]
    d -= L * np.round(d / L)
    keep = np.einsum("ij,ij->i", d, d) < cutoff * cutoff
    i, j, d = i[keep], j[keep], d[keep]
    src = np.concatenate([i, j])
    dst = np.concatenate([j, i])
    vec = np.concatenate([d, -d])      # pos[dst] - pos[src]
    src, dst, vec = _canonical(src, dst, vec)
    return Graph(n_atoms, pos, src, dst, vec, box=L)


def molecule_batch(n_graphs: int = 100, n_atoms: int = 18, density: float = WATER_DENSITY,
                   cutoff: float = 5.0, seed: int = 0,
                   rng: np.random.Generator | None = None) -> Graph:
    """Each molecule: atoms uniform in a ball holding n_atoms at `density`
    (rejection from the enclosing cube); all directed pairs < cutoff inside
    each molecule.  Node id = graph * n_atoms + atom."""
    rng = np.random.default_rng(seed) if rng is None else rng
    R = (3.0 * n_atoms / (4.0 * np.pi * density)) ** (1.0 / 3.0)
    pos = np.empty((n_graphs * n_atoms, 3))
    k = 0
    while k < n_graphs * n_atoms:
        p = rng.uniform(-R, R, size=3)
        if p @ p < R * R:
            pos[k] = p
            k += 1
    srcs, dsts, vecs = [], [], []
    for g in range(n_graphs):
        base = g * n_atoms
        P = pos[base:base + n_atoms]
        d = P[None, :, :] - P[:, None, :]            # d[i, j] = P[j] - P[i]
        dist2 = np.einsum("ijk,ijk->ij", d, d)
        ii, jj = np.nonzero((dist2 < cutoff * cutoff) & ~np.eye(n_atoms, dtype=bool))
        srcs.append(ii + base)
        dsts.append(jj + base)
        vecs.append(d[ii, jj])
    src, dst, vec = _canonical(np.concatenate(srcs), np.concatenate(dsts), np.concatenate(vecs))
    return Graph(n_graphs * n_atoms, pos, src, dst, vec)


def normal(rng: np.random.Generator, shape, dtype) -> np.ndarray:
    """N(0,1) drawn in float64, rounded to `dtype` ('f32', 'f64' or 'bf16').

    bf16 values are returned as float32 arrays holding exactly representable
    bf16 numbers (round to nearest even)."""
    a = rng.standard_normal(size=shape)
    return round_to(a, dtype)


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f64":
        return np.ascontiguousarray(a, dtype=np.float64)
    f = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return f
    if dtype == "bf16":
        u = f.view(np.uint32).astype(np.uint64)
        rnd = ((u >> 16) & 1) + 0x7FFF
        u = ((u + rnd) >> 16) << 16
        return u.astype(np.uint32).view(np.float32)
    raise ValueError(dtype)


def bf16_bits(a_f32: np.ndarray) -> np.ndarray:
    """uint16 storage of float32 values that are exact bf16 numbers."""
    return (np.ascontiguousarray(a_f32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# Irreps of the workloads
# ---------------------------------------------------------------------------

def sh_irreps(lmax: int, parity: bool = True) -> str:
    return "+".join(f"1x{l}{('e' if l % 2 == 0 else 'o') if parity else ''}"
                    for l in range(lmax + 1))


def _parse(s):
    out = []
    for t in s.split("+"):
        mul, rest = t.strip().split("x")
        out.append((int(mul), int(rest[:-1] if rest[-1] in "eo" else rest),
                    {"e": 1, "o": -1}.get(rest[-1], 0)))
    return out


def one_block_per_path(irreps_in1: str, irreps_in2: str, targets: list[str]):
    """Output irreps with one block per (i1, i2, target) triple that the
    selection rule allows, in i1-major, i2, target order; uvu multiplicity
    (mul_out = mul_in1).  Returns (irreps_out, paths)."""
    a_list, b_list = _parse(irreps_in1), _parse(irreps_in2)
    tl = []
    for t in targets:
        l = int(t[:-1]) if t[-1] in "eo" else int(t)
        tl.append((l, {"e": 1, "o": -1}.get(t[-1], 0), t))
    blocks, paths = [], []
    for i1, (m1, l1, p1) in enumerate(a_list):
        for i2, (_, l2, p2) in enumerate(b_list):
            for (l3, p3, name) in tl:
                if not abs(l1 - l2) <= l3 <= l1 + l2:
                    continue
                if p1 and p2 and p3 and p1 * p2 != p3:
                    continue
                paths.append((i1, i2, len(blocks)))
                blocks.append(f"{m1}x{name}")
    return "+".join(blocks), paths


@dataclass
class TPConfig:
    name: str
    irreps_in1: str
    irreps_in2: str
    irreps_out: str
    mode: str
    dtype: str
    paths: list | None = None          # None: all allowed paths
    shared_weights: bool = False
    extra: dict = field(default_factory=dict)


ALL_PARITY_TARGETS = ["0e", "0o", "1e", "1o", "2e", "2o", "3e", "3o"]


def config(name: str) -> TPConfig:
    """The five workloads; sizes and inputs are drawn by `make_*` below."""
    mace_targets = ["0e", "1o", "2e", "3o"]
    if name == "c1":
        return TPConfig("single CG TP 8x0e+8x1o (x) 0e+1o+2e, batch 1000, fp32",
                        "8x0e+8x1o", "1x0e+1x1o+1x2e", "8x0e+8x1o+8x2e", "uvu", "f32",
                        extra=dict(batch=1000))
    if name in ("c2", "c4"):
        x = "128x0e+128x1o"
        out, paths = one_block_per_path(x, sh_irreps(3), mace_targets)
        title = ("MACE-like fused conv fwd fp32, 4096 atoms" if name == "c2"
                 else "MACE-like conv fwd+bwd+forces+double-bwd fp32, 4096 atoms")
        return TPConfig(title, x, sh_irreps(3), out, "uvu", "f32", paths,
                        extra=dict(n_atoms=4096, cutoff=5.0, lmax=3))
    if name == "c3":
        x = "128x0e+128x1o+128x2e"
        out, paths = one_block_per_path(x, sh_irreps(3), mace_targets)
        return TPConfig("MACE-like fused conv fwd fp64, 16384 atoms", x, sh_irreps(3), out,
                        "uvu", "f64", paths, extra=dict(n_atoms=16384, cutoff=5.0, lmax=3))
    if name in ("c2a", "c3a"):
        # every output parity for l3 <= 3: 13 paths (c2a, dim 7040) and 24
        # paths (c3a), one 128-channel block per path
        base = config(name[:2])
        out, paths = one_block_per_path(base.irreps_in1, base.irreps_in2, ALL_PARITY_TARGETS)
        return TPConfig(base.name + ", all output parities", base.irreps_in1, base.irreps_in2, out, "uvu",
                        base.dtype, paths, extra=dict(base.extra))
    if name == "c5":
        return TPConfig("TFN-like uvw conv bf16-in fp32-acc, 100 x 18-atom graphs",
                        "32x0+32x1+32x2+32x3", sh_irreps(6, parity=False),
                        "64x0+64x1+64x2+64x3", "uvw", "bf16", None, shared_weights=True,
                        extra=dict(n_graphs=100, n_atoms=18, cutoff=5.0, lmax=6))
    raise KeyError(name)


def irreps_dim(s: str) -> int:
    return sum(m * (2 * l + 1) for (m, l, _) in _parse(s))


def weight_numel(cfg: TPConfig, paths) -> int:
    a, b, c = _parse(cfg.irreps_in1), _parse(cfg.irreps_in2), _parse(cfg.irreps_out)
    n = 0
    for (i1, i2, i3) in paths:
        n += a[i1][0] * b[i2][0] * (c[i3][0] if cfg.mode == "uvw" else 1)
    return n


@dataclass
class ConvInputs:
    graph: Graph
    x: np.ndarray       # [N, dim1] in the workload dtype (bf16 held as f32)
    w: np.ndarray       # [E, wnumel] (or [wnumel] shared), canonical edge order


def make_conv_inputs(graph: Graph, dim1: int, wnumel: int, dtype: str,
                     rng: np.random.Generator, shared: bool = False) -> ConvInputs:
    x = normal(rng, (graph.n_nodes, dim1), dtype)
    w = normal(rng, (wnumel,) if shared else (graph.n_edges, wnumel), dtype)
    return ConvInputs(graph, x, w)
