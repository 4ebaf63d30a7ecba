"""Test-only dense torch (CPU, float64) formulation of the tensor product.

Built from the oracle's per-path coupling tensors (pinned separately) with
torch.einsum, so autograd gives independent gradients and second
derivatives to pin the oracle's hand-written adjoint loops against.
"""
import numpy as np
import torch

import oracle


class DenseTP:
    def __init__(self, prob: "oracle.Problem"):
        self.prob = prob
        self.R = [torch.from_numpy(oracle.real_cg(int(r["l1"]), int(r["l2"]), int(r["l3"])))
                  for r in prob.table]

    def forward(self, x, y, w):
        """x [B, dim1], y [B, dim2], w [B, wnumel] or [wnumel] (shared)."""
        p = self.prob
        B = x.shape[0]
        out = torch.zeros(B, p.dim3, dtype=x.dtype)
        outs = [out]
        for R, r in zip(self.R, p.table):
            l1, l2, l3 = int(r["l1"]), int(r["l2"]), int(r["l3"])
            m1, m2, m3 = int(r["mul1"]), int(r["mul2"]), int(r["mul3"])
            d1, d2, d3 = 2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1
            o1, o2, o3, wo = int(r["off1"]), int(r["off2"]), int(r["off3"]), int(r["woff"])
            xb = x[:, o1:o1 + m1 * d1].reshape(B, m1, d1)
            yb = y[:, o2:o2 + m2 * d2].reshape(B, m2, d2)
            if p.mode == "uvu":
                n = m1 * m2
                wb = (w[wo:wo + n].reshape(m1, m2) if p.shared_weights
                      else w[:, wo:wo + n].reshape(B, m1, m2))
                eq = "ijk,bui,bvj,uv->buk" if p.shared_weights else "ijk,bui,bvj,buv->buk"
                blk = torch.einsum(eq, R, xb, yb, wb)
            else:
                n = m1 * m2 * m3
                wb = (w[wo:wo + n].reshape(m1, m2, m3) if p.shared_weights
                      else w[:, wo:wo + n].reshape(B, m1, m2, m3))
                eq = "ijk,bui,bvj,uvo->bok" if p.shared_weights else "ijk,bui,bvj,buvo->bok"
                blk = torch.einsum(eq, R, xb, yb, wb)
            pad = torch.zeros(B, p.dim3, dtype=x.dtype)
            pad[:, o3:o3 + m3 * d3] = blk.reshape(B, m3 * d3)
            outs.append(pad)
        return sum(outs)

    def conv(self, x, y, w, src, dst, n_nodes):
        src_t = torch.as_tensor(np.asarray(src, np.int64))
        dst_t = torch.as_tensor(np.asarray(dst, np.int64))
        msg = self.forward(x[src_t], y, w)
        out = torch.zeros(n_nodes, self.prob.dim3, dtype=x.dtype)
        return out.index_add(0, dst_t, msg)
