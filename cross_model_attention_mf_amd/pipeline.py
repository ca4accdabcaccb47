"""The hot path as one call sequence over device tensors.

sender side:   block statistics -> selection + extraction (staged compression)
receiver side: fused mapped attention . V over the resident compressed state

Only allocation and call order live here; all arithmetic is in libmapflow.so.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import torch

from . import mapflow as mf


@dataclasses.dataclass
class SenderState:
    """Compressed sender maps resident in HBM (one CSR over all layers)."""

    desc: mf.SenderDesc
    batch: mf.Batch
    row_lse: torch.Tensor      # [L, H_s, Tq] fp32
    block_mass: torch.Tensor   # [L, H_s, total_rb, max_cb] fp32
    row_ptr: torch.Tensor      # [L*H_s*total_rb + 1] int32
    col_idx: torch.Tensor      # [capacity] int32
    values: torch.Tensor       # [capacity, B, B]
    nnz: Optional[int]
    workspace: torch.Tensor
    stats_workspace: Optional[torch.Tensor] = None

    @property
    def B(self) -> int:
        return self.desc.B


def alloc_sender(batch: mf.Batch, q: torch.Tensor, k: torch.Tensor, B: int, capacity: int,
                 sm_scale: float = 0.0) -> SenderState:
    if q.dim() == 3:
        q, k = q[None], k[None]
    desc = mf.sender_desc(q, k, B, sm_scale)
    L, H = desc.num_layers, desc.H_s
    dev = q.device
    row_lse = torch.empty((L, H, batch.info.total_q), dtype=torch.float32, device=dev)
    block_mass = torch.empty((L, H, batch.total_rowblocks, max(batch.max_colblocks, 1)),
                             dtype=torch.float32, device=dev)
    row_ptr = torch.empty(L * H * batch.total_rowblocks + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
    values = torch.empty((max(capacity, 1), B, B), dtype=q.dtype, device=dev)
    ws = torch.empty(max(mf.compress_workspace_size(desc, batch), 1), dtype=torch.uint8, device=dev)
    n_sws = mf.block_stats_workspace_size(desc, batch)
    sws = torch.empty(n_sws, dtype=torch.uint8, device=dev) if n_sws else None
    return SenderState(desc, batch, row_lse, block_mass, row_ptr, col_idx, values, None, ws, sws)


def count_capacity(batch: mf.Batch, q, k, B: int, tau: float, sm_scale: float = 0.0) -> int:
    """Kept-block count for (q, k, tau): stats + selection with no values (syncs once)."""
    st = alloc_sender(batch, q, k, B, 0, sm_scale)
    qq, kk = (q[None], k[None]) if q.dim() == 3 else (q, k)
    mf.block_stats(st.desc, batch, qq, kk, st.row_lse, st.block_mass, st.stats_workspace)
    return mf.compress_blocks(st.desc, batch, qq, kk, st.row_lse, st.block_mass, tau, st.row_ptr,
                              None, None, 0, st.workspace, sync_count=True)


def compress(st: SenderState, q, k, tau: float, sync_count: bool = True, stream=None) -> SenderState:
    qq, kk = (q[None], k[None]) if q.dim() == 3 else (q, k)
    mf.block_stats(st.desc, st.batch, qq, kk, st.row_lse, st.block_mass, st.stats_workspace, stream)
    st.nnz = mf.compress_blocks(st.desc, st.batch, qq, kk, st.row_lse, st.block_mass, tau,
                                st.row_ptr, st.col_idx, st.values, st.col_idx.numel(),
                                st.workspace, sync_count, stream)
    return st


def mapped(st: SenderState, W: torch.Tensor, v: torch.Tensor, layer_map: Sequence[int],
           out: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
           page_size: int = 0, stream=None, split: bool = False,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W [L_r, H_r, H_s] fp32; v [L_r, Tk, H_kv_r, d] (or a paged pool
    [L_r, pages, page_size, H_kv_r, d] with block_table [S, max_pages]).
    Returns O [L_r, Tq, H_r, d].  split=True takes mf_mapped_attn_v_split,
    with `workspace` (allocated here when None and one is needed)."""
    if W.dim() == 2:
        W = W[None]
    if v.dim() == (4 if block_table is not None else 3):
        v = v[None]
    L_r, H_r, H_s = W.shape
    d = v.shape[-1]
    Tq = st.batch.info.total_q
    if out is None:
        out = torch.empty((L_r, Tq, H_r, d), dtype=v.dtype, device=v.device)
    desc = mf.receiver_desc(v, H_s, H_r, d, st.B, layer_map, st.desc.num_layers, out[0].numel(),
                            st.col_idx.numel(), block_table, page_size)
    if split:
        if workspace is None:
            workspace = split_workspace(desc, st.batch, v.device)
        mf.mapped_attn_v_split(desc, st.batch, st.row_ptr, st.col_idx, st.values, W, v, out, workspace, stream)
    else:
        mf.mapped_attn_v(desc, st.batch, st.row_ptr, st.col_idx, st.values, W, v, out, stream)
    return out


def split_workspace(desc, batch, device) -> Optional[torch.Tensor]:
    """Workspace of mf_mapped_attn_v_split for this receiver and batch (None
    when no split applies); torch's allocations are 256-byte aligned."""
    n = mf.mapped_split_workspace_size(desc, batch)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def mapped_multi(st: SenderState, receivers: Sequence[tuple], layer_map: Sequence[int], stream=None):
    """Several receivers of one sender state in one call.  receivers: (W, v) or
    (W, v, block_table, page_size) per receiver, shaped as for `mapped`.
    Returns the list of O tensors."""
    descs, Ws, vs, outs = [], [], [], []
    for rcv in receivers:
        W, v = rcv[0], rcv[1]
        block_table = rcv[2] if len(rcv) > 2 else None
        page_size = rcv[3] if len(rcv) > 3 else 0
        if W.dim() == 2:
            W = W[None]
        if v.dim() == (4 if block_table is not None else 3):
            v = v[None]
        L_r, H_r, H_s = W.shape
        d = v.shape[-1]
        out = torch.empty((L_r, st.batch.info.total_q, H_r, d), dtype=v.dtype, device=v.device)
        descs.append(mf.receiver_desc(v, H_s, H_r, d, st.B, layer_map, st.desc.num_layers, out[0].numel(),
                                      st.col_idx.numel(), block_table, page_size))
        Ws.append(W); vs.append(v); outs.append(out)
    mf.mapped_attn_v_multi(descs, st.batch, st.row_ptr, st.col_idx, st.values, Ws, vs, outs, stream)
    return outs


def fetch_overlapped(cache: mf.MapCache, keys, m: int, n_blocks: int, suffix: Optional[SenderState],
                     row_ptr_out: torch.Tensor, col_idx_out: torch.Tensor, values_out: torch.Tensor,
                     recompute, fetch_stream) -> int:
    """Fetch the cached rows of a sequence (the splice of its first m
    row-blocks with the suffix's) on `fetch_stream` while `recompute()` runs
    its work on the current stream; the current stream then waits for the
    fetch.  The recompute is launched first, so its kernels take their
    compute units before the copy fills the rest.  Returns the spliced entry
    count."""
    cur = torch.cuda.current_stream()
    ready = torch.cuda.Event()
    ready.record(cur)
    suffix_rp = suffix.row_ptr.cpu().numpy() if suffix is not None else None
    recompute()
    fetch_stream.wait_event(ready)
    for t in (row_ptr_out, col_idx_out, values_out):
        t.record_stream(fetch_stream)
    if suffix is not None:
        for t in (suffix.col_idx, suffix.values):
            t.record_stream(fetch_stream)
    with torch.cuda.stream(fetch_stream):
        if suffix is None:
            nnz = cache.splice(keys[:m], m, n_blocks, None, 0, 0, None, None, row_ptr_out, col_idx_out,
                               values_out, stream=fetch_stream)
        else:
            nnz = cache.splice(keys[:m], m, n_blocks, suffix_rp, suffix.batch.total_rowblocks, 0,
                               suffix.col_idx, suffix.values, row_ptr_out, col_idx_out, values_out,
                               stream=fetch_stream)
    cur.wait_stream(fetch_stream)
    return nnz


class LayerGroupPipeline:
    """The whole path over groups of layers, with the fused step of group g
    on a second stream while block statistics and compression of group g + 1
    run on the current one.  Receiver layer l reads sender layer l.

    Each group owns its compressed state; the kept-block capacity of every
    group is counted once at construction (a host sync), so a step issues
    none.  The kernels and their inputs are those of the sequential order,
    so the outputs are the same bit for bit; only the overlap changes.  The
    statistics kernel is bound by MFMA and VALU work, the fused kernel by its
    copy pipeline, so the two share the chip better than either alone."""

    def __init__(self, batch: mf.Batch, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 W: torch.Tensor, out: torch.Tensor, B: int, tau: float, H_r: int, groups: int,
                 map_stream: Optional[torch.cuda.Stream] = None):
        L = q.shape[0]
        if not 1 <= groups <= L:
            raise ValueError(f"groups must lie in [1, {L}], got {groups}")
        self.batch, self.tau = batch, tau
        self.map_stream = map_stream if map_stream is not None else torch.cuda.Stream()
        self.groups = []
        for g in range(groups):
            l0, l1 = g * L // groups, (g + 1) * L // groups
            qg, kg = q[l0:l1], k[l0:l1]
            cap = count_capacity(batch, qg, kg, B, tau)
            st = alloc_sender(batch, qg, kg, B, cap)
            og = out[l0:l1]
            desc = mf.receiver_desc(v[l0:l1], st.desc.H_s, H_r, st.desc.d, B, list(range(l1 - l0)), l1 - l0,
                                    og[0].numel(), st.col_idx.numel())
            self.groups.append((qg, kg, cap, st, desc, W[l0:l1], v[l0:l1], og))

    @property
    def capacity(self) -> int:
        return sum(g[2] for g in self.groups)

    def step(self, pipelined: bool = True) -> None:
        cur = torch.cuda.current_stream()
        # the previous step's fused launches read the states this step rewrites
        cur.wait_stream(self.map_stream)
        for qg, kg, cap, st, desc, Wg, vg, og in self.groups:
            mf.block_stats(st.desc, self.batch, qg, kg, st.row_lse, st.block_mass, st.stats_workspace, cur)
            mf.compress_blocks(st.desc, self.batch, qg, kg, st.row_lse, st.block_mass, self.tau, st.row_ptr,
                               st.col_idx, st.values, cap, st.workspace, sync_count=False, stream=cur)
            if pipelined:
                self.map_stream.wait_stream(cur)
                # the caching allocator must not hand these out again while the
                # second stream may still read or write them
                for t in (st.row_ptr, st.col_idx, st.values, Wg, vg, og):
                    t.record_stream(self.map_stream)
                mf.mapped_attn_v(desc, self.batch, st.row_ptr, st.col_idx, st.values, Wg, vg, og,
                                 stream=self.map_stream)
            else:
                mf.mapped_attn_v(desc, self.batch, st.row_ptr, st.col_idx, st.values, Wg, vg, og, stream=cur)
        if pipelined:
            cur.wait_stream(self.map_stream)


def fit_headmix(sender: SenderState, receiver: SenderState, layer_map: Sequence[int], lam: float = 0.0,
                stream=None):
    """Least-squares head mix from a sender's and a receiver's compressed maps
    of one batch.  Returns (W [L_r, H_r, H_s] fp32, dropped [L_r, H_s] int32,
    G [L_r, H_s, H_s] fp64, b [L_r, H_r, H_s] fp64)."""
    L_r, H_s, H_r = len(layer_map), sender.desc.H_s, receiver.desc.H_s
    dev = sender.row_ptr.device
    desc = mf.headmix_desc(sender.values.dtype, sender.B, layer_map, sender.desc.num_layers, H_s, H_r,
                           sender.col_idx.numel(), receiver.col_idx.numel())
    G = torch.empty((L_r, H_s, H_s), dtype=torch.float64, device=dev)
    b = torch.empty((L_r, H_r, H_s), dtype=torch.float64, device=dev)
    ws = torch.empty(max(mf.headmix_workspace_size(desc, sender.batch), 1), dtype=torch.uint8, device=dev)
    mf.headmix_gram(desc, sender.batch, sender.row_ptr, sender.col_idx, sender.values, receiver.row_ptr,
                    receiver.col_idx, receiver.values, G, b, ws, stream)
    W = torch.empty((L_r, H_r, H_s), dtype=torch.float32, device=dev)
    dropped = torch.empty((L_r, H_s), dtype=torch.int32, device=dev)
    mf.headmix_solve(desc, G, b, lam, W, dropped, stream)
    return W, dropped, G, b
