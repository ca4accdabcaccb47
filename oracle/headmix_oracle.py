"""Oracle for the offline calibration of the head mix W by least squares.

TEST INFRASTRUCTURE ONLY.  Only the test suite and the bench's CPU-baseline
leg may import this module.  It shares no code with the HIP library.

The MapFlow page (163.com article "跨模型上下文交接还要重算KV?北大提出MapFlow",
section "从内部表示,走向 token 之间的依赖关系") maps the sender's attention
maps onto the receiver's heads with a learned linear combination of heads.
Only those mapping weights are trained, with both models frozen, once by
offline calibration.  The page names no objective.  The reading used here:
for each mapped layer, W minimises the squared Frobenius distance between the
receiver's own block maps and the mixed sender maps over every block of the
sender's kept union, plus a ridge term:

    J(W) = sum_r sum_(i, j) || A_r[i, j] - sum_h W[r, h] Pt_h[i, j] ||_F^2
           + lam * ||W||_F^2

where, for query row-block i and column block j of the union of the sender
heads' kept sets,
    Pt_h[i, j] = sender head h's kept block (its probabilities), or 0 when h
                 does not keep j: exactly the operand the fused step mixes;
    A_r[i, j]  = receiver head r's block from its own compressed map, or 0
                 when r does not keep j.
Blocks outside the union add a constant to J and are left out.  Setting the
gradient to zero gives, row by row, the normal equations

    (G + lam I) w_r = b_r,   G[h, h'] = sum <Pt_h, Pt_h'>,   b_r[h] = sum <A_r, Pt_h>,

(inner products over the B x B entries of a block).  They are solved by a
Cholesky factorisation of G + lam I that drops head k when its pivot falls to
at most 1e-12 of its diagonal (a head that keeps nothing, or whose maps lie
in the span of earlier heads): a dropped head gets weight 0 and the others
are the fit without it.

Inputs are CSRs as the compression writes them: row (l * H + h) * R + i for
layer l, head h and row-block i of R, values key-major B x B per entry (the
inner product does not depend on the element order, as long as both maps use
the same one).  Everything is float64 numpy; matrix products use numpy's
matmul as a library primitive.
"""
from __future__ import annotations

import math
from typing import Dict, Sequence, Tuple

import numpy as np

DROP_TOL = 1e-12


def kept_blocks(row_ptr: np.ndarray, col_idx: np.ndarray, values: np.ndarray, layer: int, head: int,
                H: int, R: int, i: int) -> Dict[int, np.ndarray]:
    """Column block -> flattened fp64 block of CSR row (layer, head, i)."""
    row = (layer * H + head) * R + i
    e0, e1 = int(row_ptr[row]), int(row_ptr[row + 1])
    return {int(col_idx[e]): np.asarray(values[e], dtype=np.float64).ravel() for e in range(e0, e1)}


def gram_and_cross(sender: Tuple[np.ndarray, np.ndarray, np.ndarray], receiver: Tuple[np.ndarray, np.ndarray, np.ndarray],
                   layer_map: Sequence[int], H_s: int, H_r: int, R: int, B: int) -> Tuple[np.ndarray, np.ndarray]:
    """G [L, H_s, H_s] and b [L, H_r, H_s] of the normal equations, one pair
    per receiver layer l (sender CSR layer layer_map[l], receiver CSR layer l)."""
    L = len(layer_map)
    G = np.zeros((L, H_s, H_s))
    b = np.zeros((L, H_r, H_s))
    for l in range(L):
        s = int(layer_map[l])
        for i in range(R):
            sk = [kept_blocks(*sender, s, h, H_s, R, i) for h in range(H_s)]
            rk = [kept_blocks(*receiver, l, r, H_r, R, i) for r in range(H_r)]
            union = sorted(set().union(*[set(m) for m in sk]))
            for j in union:
                X = np.zeros((H_s, B * B))
                for h in range(H_s):
                    if j in sk[h]:
                        X[h] = sk[h][j]
                A = np.zeros((H_r, B * B))
                for r in range(H_r):
                    if j in rk[r]:
                        A[r] = rk[r][j]
                G[l] += X @ X.T
                b[l] += A @ X.T
    return G, b


def solve_headmix(G: np.ndarray, b: np.ndarray, lam: float) -> Tuple[np.ndarray, np.ndarray]:
    """W [H_r, H_s] from one layer's normal equations, and the dropped-head
    mask.  Column-by-column Cholesky of M = G + lam I with the drop rule, then
    a forward and a back substitution per receiver head."""
    H = G.shape[0]
    M = G + lam * np.eye(H)
    Lf = np.zeros((H, H))
    dropped = np.zeros(H, dtype=bool)
    for k in range(H):
        piv = M[k, k] - sum(Lf[k, p] * Lf[k, p] for p in range(k))
        if not (M[k, k] > 0.0) or piv <= DROP_TOL * M[k, k]:
            dropped[k] = True
            continue
        Lf[k, k] = math.sqrt(piv)
        for i in range(k + 1, H):
            Lf[i, k] = (M[i, k] - sum(Lf[i, p] * Lf[k, p] for p in range(k))) / Lf[k, k]
    W = np.zeros((b.shape[0], H))
    for r in range(b.shape[0]):
        y = np.zeros(H)
        for k in range(H):
            if not dropped[k]:
                y[k] = (b[r, k] - sum(Lf[k, p] * y[p] for p in range(k))) / Lf[k, k]
        w = np.zeros(H)
        for k in reversed(range(H)):
            if not dropped[k]:
                w[k] = (y[k] - sum(Lf[p, k] * w[p] for p in range(k + 1, H))) / Lf[k, k]
        W[r] = w
    return W, dropped


def fit_headmix(sender, receiver, layer_map: Sequence[int], H_s: int, H_r: int, R: int, B: int,
                lam: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """(W [L, H_r, H_s], dropped [L, H_s], G, b)."""
    G, b = gram_and_cross(sender, receiver, layer_map, H_s, H_r, R, B)
    Ws, drops = zip(*[solve_headmix(G[l], b[l], lam) for l in range(len(layer_map))])
    return np.stack(Ws), np.stack(drops), G, b


def objective(sender, receiver, layer: int, sender_layer: int, W: np.ndarray, H_s: int, H_r: int, R: int,
              B: int, lam: float) -> float:
    """J of one layer by explicit sums over every entry (for small cases)."""
    J = lam * float(np.sum(W * W))
    for i in range(R):
        sk = [kept_blocks(*sender, sender_layer, h, H_s, R, i) for h in range(H_s)]
        rk = [kept_blocks(*receiver, layer, r, H_r, R, i) for r in range(H_r)]
        union = sorted(set().union(*[set(m) for m in sk]))
        for j in union:
            for r in range(H_r):
                for e in range(B * B):
                    mix = 0.0
                    for h in range(H_s):
                        if j in sk[h]:
                            mix += W[r, h] * sk[h][j][e]
                    a = rk[r][j][e] if j in rk[r] else 0.0
                    J += (a - mix) ** 2
    return J
