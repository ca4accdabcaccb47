"""Plain fp64 CPU oracle for MapFlow's data-parallel hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
the bench's CPU-baseline leg may import this module.  It shares no code with
the HIP library and must never be used as a fallback for it.

What it computes, in the order the MapFlow page describes it (163.com article
"跨模型上下文交接还要重算KV?北大提出MapFlow", sections "从内部表示,走向 token
之间的依赖关系" and "让复用真正省时,还需要解决存储和执行问题"):

1. the sender's attention map of one head, P = softmax(Q K^T / sqrt(d)) over
   the causal columns (the token-to-token dependency map that is reused);
2. block-level statistics of that map on a regular 2-D grid of B x B blocks:
   the attention probability mass of each block (first stage of the staged
   compression, paragraph "第一");
3. per query row-block, the blocks kept by cumulative attention probability:
   the shortest prefix of blocks, in order of decreasing mass, whose summed
   mass reaches tau (paragraph "第一");
4. extraction of the kept blocks' probabilities (second stage, paragraph
   "第一"), stored unchanged;
5. the receiver's output: for each receiver head r, a learned linear
   combination over sender heads of the kept maps, multiplied by the
   receiver's own values (paragraph "第三"; the head mapping is a learned
   linear combination, section "从内部表示…").

Readings where the pages are silent (each one is listed in the design notes):
block statistic = summed probability divided by the number of valid rows of
the row-block (so the masses of a row-block sum to 1); selection per (layer,
sender head, row-block); ties in mass go to the lower column-block index; no
forced blocks; kept values are not renormalised; the mixed map is purely
linear (no bias, no re-softmax); tau >= 1 keeps every causal block; GQA maps
query head h to key head h // (H / H_kv).

Everything is float64 numpy.  Matrix products use numpy's matmul as a
library primitive; there is no blocking, fusion or reordering beyond the
definitions above.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# Row-block bookkeeping for packed (varlen, chunked) batches
# ----------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class RowBlock:
    """Query row-block `local` of packed sequence `seq` (global index `index`)."""

    index: int          # global row-block index (sequence order)
    seq: int            # packed sequence entry
    local: int          # row-block number inside the chunk
    q0: int             # first packed query row of the block
    rows: int           # valid rows R_i
    pos0: int           # absolute position of the block's first row
    k0: int             # first packed key row of the sequence
    klen: int           # keys of the sequence (prefix length)

    @property
    def last_pos(self) -> int:
        return self.pos0 + self.rows - 1


def enumerate_rowblocks(cu_q: Sequence[int], cu_k: Sequence[int],
                        q_pos0: Optional[Sequence[int]], B: int) -> List[RowBlock]:
    """Row-blocks of a packed batch.  The block grid restarts in every sequence
    and is aligned to absolute positions (a chunk starts on a block edge)."""
    out: List[RowBlock] = []
    S = len(cu_q) - 1
    for s in range(S):
        qlen = int(cu_q[s + 1]) - int(cu_q[s])
        klen = int(cu_k[s + 1]) - int(cu_k[s])
        p0 = 0 if q_pos0 is None else int(q_pos0[s])
        assert p0 % B == 0, "chunk start must be a multiple of the block size"
        assert klen >= p0 + qlen, "keys must cover the chunk's causal prefix"
        nrb = (qlen + B - 1) // B
        for i in range(nrb):
            rows = min(B, qlen - i * B)
            out.append(RowBlock(len(out), s, i, int(cu_q[s]) + i * B, rows,
                                p0 + i * B, int(cu_k[s]), klen))
    return out


def num_candidates(rb: RowBlock, B: int) -> int:
    """Causal column blocks of a row-block: 0 .. floor(last_pos / B)."""
    return rb.last_pos // B + 1


# ----------------------------------------------------------------------------
# 1. the sender's causal attention map (one head, one strip of query rows)
# ----------------------------------------------------------------------------


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def kv_head(h: int, H: int, H_kv: int) -> int:
    """Grouped heads: query head h reads key/value head h // (H / H_kv)."""
    return h // (H // H_kv)


def causal_probs(q_rows: np.ndarray, k_keys: np.ndarray, pos_rows: np.ndarray,
                 scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """P[r, c] = softmax_c(scale * q_r . k_c) over c <= pos_rows[r].

    q_rows [R, d], k_keys [n, d] (keys 0..n-1 of the sequence), pos_rows [R]
    absolute positions.  Returns (P [R, n] with zeros on masked entries,
    lse [R] = log sum_c exp(scale * q_r . k_c))."""
    S = (q_rows @ k_keys.T) * scale
    n = k_keys.shape[0]
    allowed = np.arange(n)[None, :] <= pos_rows[:, None]
    S = np.where(allowed, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    e = np.exp(S - m)
    z = e.sum(axis=1, keepdims=True)
    P = e / z
    lse = (m + np.log(z))[:, 0]
    return P, lse


# ----------------------------------------------------------------------------
# 2. block statistics
# ----------------------------------------------------------------------------


def block_masses(P: np.ndarray, B: int, ncand: int) -> np.ndarray:
    """Normalised mass of each column block of a row-block strip.

    P [R, n] is the strip of R valid rows; m[j] = sum over the block's entries
    of P, divided by R, for j = 0 .. ncand-1 (so sum_j m[j] = 1)."""
    R, n = P.shape
    m = np.zeros(ncand)
    for j in range(ncand):
        m[j] = P[:, j * B: min(n, (j + 1) * B)].sum() / R
    return m


# ----------------------------------------------------------------------------
# 3. selection by cumulative attention probability
# ----------------------------------------------------------------------------


@dataclasses.dataclass
class Selection:
    masses: np.ndarray      # [ncand] normalised masses
    order: np.ndarray       # candidates by (mass desc, index asc)
    cum: np.ndarray         # cum[k] = summed mass of the first k in `order` (cum[0] = 0)
    kstar: int              # number kept
    tau: float

    @property
    def kept(self) -> np.ndarray:
        return np.sort(self.order[: self.kstar])


def selection_order(m: np.ndarray) -> np.ndarray:
    """Candidates sorted by decreasing mass; equal masses by increasing index."""
    idx = np.arange(m.shape[0])
    return np.lexsort((idx, -m))


def select_blocks(m: np.ndarray, tau: float) -> Selection:
    """Keep the shortest prefix of the mass order whose cumulative mass reaches
    tau.  tau >= 1 keeps every candidate; so does a cumulative sum that never
    reaches tau through rounding."""
    order = selection_order(m)
    cum = np.concatenate([[0.0], np.cumsum(m[order])])
    n = m.shape[0]
    if tau >= 1.0:
        kstar = n
    else:
        reach = np.nonzero(cum[1:] >= tau)[0]
        kstar = int(reach[0]) + 1 if reach.size else n
    return Selection(m, order, cum, kstar, tau)


def accept_set(sel: Selection, other: Iterable[int], eps: float = 1e-6) -> Tuple[bool, int, List[int]]:
    """Is `other` an acceptable kept set for this row-block?

    Another implementation's arithmetic may move the cut by rounding.  A block
    the other set keeps in excess (oracle rank >= k*) is accepted when the
    oracle's cumulative mass before it is still below tau + eps; a block it
    drops (oracle rank < k*) is accepted when the oracle's cumulative mass
    before it already reaches tau - eps.  A swap across the cut is accepted
    when the excess and the dropped block differ in mass by at most eps.
    Returns (ok, number of differing blocks, offending blocks)."""
    mine = set(int(x) for x in sel.kept)
    theirs = set(int(x) for x in other)
    extra, missing = theirs - mine, mine - theirs
    if not extra and not missing:
        return True, 0, []
    n = sel.order.shape[0]
    rank = np.empty(n, dtype=np.int64)
    rank[sel.order] = np.arange(n)
    bad = [j for j in extra | missing if j < 0 or j >= n]
    if bad:
        return False, len(extra) + len(missing), sorted(bad)
    m = sel.masses
    for x in extra:
        swap = any(abs(m[x] - m[y]) <= eps for y in missing)
        if not (sel.cum[rank[x]] < sel.tau + eps or swap):
            bad.append(x)
    for y in missing:
        swap = any(abs(m[x] - m[y]) <= eps for x in extra)
        if not (sel.cum[rank[y]] >= sel.tau - eps or swap):
            bad.append(y)
    return (not bad), len(extra) + len(missing), sorted(bad)


# ----------------------------------------------------------------------------
# 4. extraction
# ----------------------------------------------------------------------------


def extract_blocks(P: np.ndarray, kept: np.ndarray, B: int) -> np.ndarray:
    """Kept blocks of a strip, unchanged: vals[t] = P[:, j*B:(j+1)*B] for
    j = kept[t], padded with zeros to B x B past the last row or key."""
    R, n = P.shape
    out = np.zeros((len(kept), B, B))
    for t, j in enumerate(kept):
        c1 = min(n, (j + 1) * B)
        out[t, :R, : c1 - j * B] = P[:, j * B: c1]
    return out


# ----------------------------------------------------------------------------
# Staged compression of one layer (steps 1-4), all or some row-blocks
# ----------------------------------------------------------------------------


@dataclasses.dataclass
class UnitResult:
    """Steps 1-4 for one (sender head, row-block)."""

    lse: np.ndarray                   # [R]
    sel: Selection
    values: np.ndarray                # [k*, B, B]
    strip: Optional[np.ndarray] = None  # P [R, n], kept only on request

    def block(self, j: int, B: int) -> np.ndarray:
        """Values of column block j (kept or not) from the remembered strip."""
        if self.strip is None:
            raise KeyError(f"block {j} is not kept; compress with keep_strips=True")
        return extract_blocks(self.strip, np.asarray([j]), B)[0]


def compress_unit(q: np.ndarray, k: np.ndarray, rb: RowBlock, h: int, B: int,
                  tau: float, scale: float, keep_strip: bool = False, extract: bool = True) -> UnitResult:
    """Steps 1-4 for one unit; extract=False stops after the selection (step
    3) and leaves values empty."""
    H, H_kv = q.shape[1], k.shape[1]
    qr = q[rb.q0: rb.q0 + rb.rows, h, :]
    kk = k[rb.k0: rb.k0 + rb.klen, kv_head(h, H, H_kv), :]
    ncand = num_candidates(rb, B)
    keys = kk[: min(rb.klen, ncand * B)]
    pos = rb.pos0 + np.arange(rb.rows)
    P, lse = causal_probs(qr, keys, pos, scale)
    m = block_masses(P, B, ncand)
    sel = select_blocks(m, tau)
    vals = extract_blocks(P, sel.kept, B) if extract else np.zeros((0, B, B))
    return UnitResult(lse, sel, vals, P if keep_strip else None)


@dataclasses.dataclass
class LayerCompression:
    rowblocks: List[RowBlock]
    units: Dict[Tuple[int, int], UnitResult]   # (h, rb.index) -> result

    def kept(self, h: int, rb: int) -> np.ndarray:
        return self.units[(h, rb)].sel.kept


def compress_layer(q: np.ndarray, k: np.ndarray, cu_q, cu_k, q_pos0, B: int,
                   tau: float, scale: Optional[float] = None,
                   heads: Optional[Iterable[int]] = None,
                   rowblocks: Optional[Iterable[int]] = None,
                   keep_strips: bool = False, extract: bool = True) -> LayerCompression:
    """q [Tq, H_s, d], k [Tk, H_kv, d] float64 packed; returns steps 1-4 for the
    requested heads and row-blocks (default: all); extract=False stops each
    unit after its selection."""
    scale = default_scale(q.shape[2]) if scale is None else scale
    rbs = enumerate_rowblocks(cu_q, cu_k, q_pos0, B)
    hs = range(q.shape[1]) if heads is None else heads
    which = range(len(rbs)) if rowblocks is None else rowblocks
    units = {}
    for i in which:
        for h in hs:
            units[(h, i)] = compress_unit(q, k, rbs[i], h, B, tau, scale, keep_strips, extract)
    return LayerCompression(rbs, units)


def csr_of(lc: LayerCompression, H_s: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Block-sparse CSR of one fully compressed layer: row (h, rb) in head-major
    order; columns ascending; values [nnz, B, B]."""
    nrb = len(lc.rowblocks)
    row_ptr = np.zeros(H_s * nrb + 1, dtype=np.int64)
    cols, vals = [], []
    for h in range(H_s):
        for i in range(nrb):
            u = lc.units[(h, i)]
            row_ptr[h * nrb + i + 1] = row_ptr[h * nrb + i] + u.sel.kstar
            cols.append(u.sel.kept)
            vals.append(u.values)
    col_idx = np.concatenate(cols) if cols else np.zeros(0, np.int64)
    values = np.concatenate(vals) if vals else np.zeros((0,))
    return row_ptr, col_idx, values


# ----------------------------------------------------------------------------
# 5. mapped attention . V for the receiver
# ----------------------------------------------------------------------------


def gather_paged(pool: np.ndarray, block_table: np.ndarray, cu_k, page_size: int) -> np.ndarray:
    """Contiguous packed values from a paged pool: token t of sequence s lives in
    page block_table[s, t // page_size] at slot t % page_size."""
    S = len(cu_k) - 1
    out = np.zeros((int(cu_k[-1]),) + pool.shape[2:])
    for s in range(S):
        n = int(cu_k[s + 1]) - int(cu_k[s])
        for t in range(n):
            out[int(cu_k[s]) + t] = pool[block_table[s, t // page_size], t % page_size]
    return out


def mapped_rowblock(kept_vals: Sequence[Tuple[np.ndarray, np.ndarray]], W: np.ndarray,
                    v: np.ndarray, rb: RowBlock, B: int) -> np.ndarray:
    """O[r] for one row-block: sum over sender heads h of W[r, h] times head h's
    map restricted to its kept blocks, times the receiver's values V_g(r).

    kept_vals[h] = (kept column blocks, their [k, B, B] values); v [Tk, H_kv_r, d]
    packed.  Returns O [rows, H_r, d]."""
    H_r, H_s = W.shape
    H_kv = v.shape[1]
    d = v.shape[2]
    ncols = num_candidates(rb, B) * B
    vseq = np.zeros((ncols, H_kv, d))
    n = min(rb.klen, ncols)
    vseq[:n] = v[rb.k0: rb.k0 + n]
    # each head's kept map as a dense strip (zeros outside kept blocks)
    Pt = np.zeros((H_s, B, ncols))
    for h in range(H_s):
        kept, vals = kept_vals[h]
        for t, j in enumerate(kept):
            Pt[h, :, j * B:(j + 1) * B] = vals[t]
    O = np.zeros((rb.rows, H_r, d))
    for r in range(H_r):
        A = np.tensordot(W[r], Pt, axes=(0, 0))        # mixed map [B, ncols]
        O[:, r, :] = (A @ vseq[:, kv_head(r, H_r, H_kv), :])[: rb.rows]
    return O


def mapped_layer(lc: LayerCompression, W: np.ndarray, v: np.ndarray, Tq: int,
                 B: int, rowblocks: Optional[Iterable[int]] = None,
                 kept_override: Optional[Dict[Tuple[int, int], np.ndarray]] = None) -> np.ndarray:
    """O [Tq, H_r, d] of one receiver layer from a compressed sender layer (rows
    of row-blocks not requested are NaN).  `kept_override[(h, rb)]` replaces a
    kept set by another set the caller has already accepted with `accept_set`;
    its values come from the oracle's own map (needs keep_strips=True)."""
    H_r, H_s = W.shape
    O = np.full((Tq, H_r, v.shape[2]), np.nan)
    which = range(len(lc.rowblocks)) if rowblocks is None else rowblocks
    for i in which:
        rb = lc.rowblocks[i]
        kv = []
        for h in range(H_s):
            u = lc.units[(h, i)]
            kept = u.sel.kept
            vals = u.values
            if kept_override is not None and (h, i) in kept_override:
                kept = np.asarray(sorted(kept_override[(h, i)]), dtype=np.int64)
                vals = np.stack([u.block(int(j), B) for j in kept]) if len(kept) else np.zeros((0, B, B))
            kv.append((kept, vals))
        O[rb.q0: rb.q0 + rb.rows] = mapped_rowblock(kv, W, v, rb, B)
    return O


# ----------------------------------------------------------------------------
# Dense helpers for tiny cases
# ----------------------------------------------------------------------------


def dense_map(q: np.ndarray, k: np.ndarray, h: int, scale: Optional[float] = None,
              pos0: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Whole causal map of one head of one sequence: P [Rq, n], lse [Rq]."""
    scale = default_scale(q.shape[2]) if scale is None else scale
    H, H_kv = q.shape[1], k.shape[1]
    pos = pos0 + np.arange(q.shape[0])
    return causal_probs(q[:, h, :], k[:, kv_head(h, H, H_kv), :], pos, scale)
