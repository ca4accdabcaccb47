"""Seeded synthetic inputs shaped like long-context prefill workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scores, softmax, block masses, selection or mixing).
Both the CPU oracle and the HIP path consume exactly the arrays produced here.

Structure of the sender's Q/K (used by every workload except the tiny one):
the caller-visible API takes only Q and K, so the attention pattern the pages
describe for real maps (a few heavy key positions, a local band, a sink at the
start of the context; MapFlow page, section on importance-based block
sparsity) is encoded into Q and K:

* column bias (exact): the last head dimension carries q = d**0.25 and
  k = d**0.25 * beta_c, which adds beta_c to every logit of key column c
  after the 1/sqrt(d) scale: beta = 6 on the first block of each sequence
  (the sink), +3 on 8 heavy key columns drawn per (layer, sequence), else 0;
* local band: dimensions 0..31 carry a shared AR(1) process z_t with
  rho = exp(-1/128); q_t = k_t = g * z_t with g = sqrt(10 * sqrt(d) / 32),
  so the expected extra logit between positions r and c is 10 * rho**|r-c|;
* heads of one layer share sink, band and heavy columns and differ only in
  the N(0, 1) noise of the remaining dimensions.

Random streams: numpy PCG64 seeded with SeedSequence([seed, workload_id,
layer, tensor_id, sequence]).  bf16 rounding is round-to-nearest-even via
torch's CPU cast.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

# tensor ids inside the seed sequence
_T_Q, _T_K, _T_V, _T_W, _T_BAND, _T_HEAVY, _T_PAGES, _T_LENS = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes and distributions of one synthetic workload."""

    name: str
    workload_id: int
    dtype: str                      # "f32" or "bf16"
    H_s: int                        # sender query heads
    H_r: int                        # receiver heads
    d: int                          # head dim (sender and receiver)
    B: int                          # block size
    taus: tuple                     # thresholds exercised (first one is the default)
    seqlens: tuple                  # full sequence lengths (keys)
    num_layers: int = 1             # mapped layers
    sender_layers: Optional[tuple] = None    # sender layer id per mapped layer
    receiver_layers: Optional[tuple] = None  # receiver layer id per mapped layer
    H_kv_s: Optional[int] = None    # sender key heads (None = H_s)
    H_kv_r: Optional[int] = None    # receiver value heads (None = H_r)
    structured: bool = True
    w_var: float = 1.0 / 32.0
    chunk: Optional[int] = None     # query rows per prefill chunk (None = whole)
    paged: bool = False
    page_size: int = 16
    seed: int = 0
    extra_receivers: tuple = ()     # ((H_r, w_var), ...) for one-sender / many-receiver

    @property
    def hkv_s(self) -> int:
        return self.H_kv_s or self.H_s

    @property
    def hkv_r(self) -> int:
        return self.H_kv_r or self.H_r

    @property
    def tau(self) -> float:
        return self.taus[0]

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def lognormal_lengths(n: int, mu: float, sigma: float, lo: int, hi: int,
                      seed: int, workload_id: int) -> tuple:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [seed, workload_id, 0, _T_LENS, 0])))
    x = np.round(rng.lognormal(mu, sigma, size=n)).astype(np.int64)
    return tuple(int(v) for v in np.clip(x, lo, hi))


def standard_workloads(seed: int = 0) -> List[Workload]:
    """The five workloads: tiny fp32, 4K single layer, 8K x 16 layers (tau sweep),
    varlen chunked paged prefill, 32K one-sender/two-receivers."""
    w1 = Workload("tiny_fp32_n256", 1, "f32", H_s=4, H_r=2, d=64, B=32,
                  taus=(0.95,), seqlens=(256,), structured=False, w_var=0.5,
                  seed=seed)
    w2 = Workload("bf16_4k_8b_to_3b", 2, "bf16", H_s=32, H_r=24, d=128, B=64,
                  taus=(0.95,), seqlens=(4096,), seed=seed)
    w3 = Workload("bf16_8k_16layers", 3, "bf16", H_s=32, H_r=24, d=128, B=64,
                  taus=(0.95, 0.90, 0.99), seqlens=(8192,), num_layers=16,
                  sender_layers=tuple(range(16, 32)),
                  receiver_layers=tuple(range(8, 24)), seed=seed)
    lens4 = lognormal_lengths(32, 7.5, 0.8, 256, 16384, seed, 4)
    w4 = Workload("bf16_varlen_chunked_paged", 4, "bf16", H_s=32, H_r=24, d=128,
                  B=64, taus=(0.95,), seqlens=lens4, num_layers=16,
                  sender_layers=tuple(range(16, 32)),
                  receiver_layers=tuple(range(8, 24)), chunk=2048, paged=True,
                  seed=seed)
    w5 = Workload("bf16_32k_14b_to_8b_3b", 5, "bf16", H_s=40, H_r=32, d=128,
                  B=128, taus=(0.95,), seqlens=(32768,), w_var=1.0 / 40.0,
                  extra_receivers=((24, 1.0 / 40.0),), seed=seed)
    return [w1, w2, w3, w4, w5]


def workload_by_id(wid: int, seed: int = 0) -> Workload:
    return standard_workloads(seed)[wid - 1]


def _rng(wl: Workload, layer: int, tensor: int, seq: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [wl.seed, wl.workload_id, layer, tensor, seq])))


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Round a float array to the workload dtype (RNE for bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _sender_qk_one_seq(wl: Workload, layer: int, seq: int, n: int):
    """Q [n, H_s, d], K [n, H_kv_s, d] float32 for one full sequence."""
    d = wl.d
    q = _rng(wl, layer, _T_Q, seq).standard_normal((n, wl.H_s, d), dtype=np.float32)
    k = _rng(wl, layer, _T_K, seq).standard_normal((n, wl.hkv_s, d), dtype=np.float32)
    if not wl.structured:
        return q, k
    # local band: shared AR(1) process on dims 0..31
    rb = _rng(wl, layer, _T_BAND, seq)
    rho = math.exp(-1.0 / 128.0)
    eps = rb.standard_normal((n, 32))
    z = np.empty((n, 32))
    z[0] = eps[0]
    s = math.sqrt(1.0 - rho * rho)
    for t in range(1, n):
        z[t] = rho * z[t - 1] + s * eps[t]
    g = math.sqrt(10.0 * math.sqrt(d) / 32.0)
    band = (g * z).astype(np.float32)
    q[:, :, :32] = band[:, None, :]
    k[:, :, :32] = band[:, None, :]
    # column bias on the last dimension
    beta = np.zeros(n, dtype=np.float64)
    beta[: min(wl.B, n)] = 6.0
    if n > wl.B:
        rh = _rng(wl, layer, _T_HEAVY, seq)
        cand = np.arange(wl.B, n)
        heavy = rh.choice(cand, size=min(8, cand.size), replace=False)
        beta[heavy] += 3.0
    r4 = d ** 0.25
    q[:, :, d - 1] = np.float32(r4)
    k[:, :, d - 1] = (r4 * beta).astype(np.float32)[:, None]
    return q, k


@dataclasses.dataclass
class LayerInputs:
    """One mapped layer of a batch, host arrays in the workload dtype.

    q      [Tq, H_s, d]      packed query rows (chunks)
    k      [Tk, H_kv_s, d]   packed keys (full prefixes)
    v      [Tk, H_kv_r, d]   packed receiver values (contiguous layout)
    w      [H_r, H_s] float32 head-mix matrix
    """

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    w: torch.Tensor
    extra_w: tuple = ()
    extra_v: tuple = ()


@dataclasses.dataclass
class BatchLayout:
    """Packing of a batch: query chunk rows and key prefixes per sequence."""

    cu_seqlens_q: np.ndarray   # int32 [S+1]
    cu_seqlens_k: np.ndarray   # int32 [S+1]
    q_pos0: np.ndarray         # int32 [S] absolute position of each chunk's first row
    seq_ids: np.ndarray        # int32 [S] which workload sequence each entry is

    @property
    def num_seqs(self) -> int:
        return int(self.q_pos0.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def total_k(self) -> int:
        return int(self.cu_seqlens_k[-1])


def num_chunk_steps(wl: Workload) -> int:
    if wl.chunk is None:
        return 1
    return max(math.ceil(n / wl.chunk) for n in wl.seqlens)


def batch_layout(wl: Workload, step: int = 0) -> BatchLayout:
    """Step t of chunked prefill: chunk t of every sequence still active; keys
    are each active sequence's prefix up to the chunk end.  Without chunking,
    one step holds every sequence whole."""
    qs, ks, p0, ids = [], [], [], []
    for sid, n in enumerate(wl.seqlens):
        if wl.chunk is None:
            a, b = 0, n
        else:
            a = step * wl.chunk
            if a >= n:
                continue
            b = min(n, a + wl.chunk)
        qs.append(b - a)
        ks.append(b)
        p0.append(a)
        ids.append(sid)
    cu_q = np.zeros(len(qs) + 1, dtype=np.int32)
    cu_k = np.zeros(len(qs) + 1, dtype=np.int32)
    cu_q[1:] = np.cumsum(qs)
    cu_k[1:] = np.cumsum(ks)
    return BatchLayout(cu_q, cu_k, np.asarray(p0, dtype=np.int32),
                       np.asarray(ids, dtype=np.int32))


def _head_mix(wl: Workload, layer: int, H_r: int, var: float, which: int) -> torch.Tensor:
    w = _rng(wl, layer, _T_W, which).standard_normal((H_r, wl.H_s)) * math.sqrt(var)
    return torch.from_numpy(w.astype(np.float32))


def layer_inputs(wl: Workload, layer: int, step: int = 0,
                 layout: Optional[BatchLayout] = None) -> LayerInputs:
    """Inputs of mapped layer `layer` (0-based) for chunk step `step`."""
    lay = layout or batch_layout(wl, step)
    qs, ks, vs = [], [], []
    extra_v = [[] for _ in wl.extra_receivers]
    for e in range(lay.num_seqs):
        sid = int(lay.seq_ids[e])
        n_full = wl.seqlens[sid]
        q_full, k_full = _sender_qk_one_seq(wl, layer, sid, n_full)
        a = int(lay.q_pos0[e])
        qlen = int(lay.cu_seqlens_q[e + 1] - lay.cu_seqlens_q[e])
        klen = int(lay.cu_seqlens_k[e + 1] - lay.cu_seqlens_k[e])
        qs.append(q_full[a:a + qlen])
        ks.append(k_full[:klen])
        v_full = _rng(wl, layer, _T_V, sid).standard_normal(
            (n_full, wl.hkv_r, wl.d), dtype=np.float32)
        vs.append(v_full[:klen])
        for x, (hr, _) in enumerate(wl.extra_receivers):
            vx = _rng(wl, layer, _T_V, 1000 * (x + 1) + sid).standard_normal(
                (n_full, hr, wl.d), dtype=np.float32)
            extra_v[x].append(vx[:klen])
    q = to_dtype(np.concatenate(qs, 0), wl.dtype)
    k = to_dtype(np.concatenate(ks, 0), wl.dtype)
    v = to_dtype(np.concatenate(vs, 0), wl.dtype)
    w = _head_mix(wl, layer, wl.H_r, wl.w_var, 0)
    ew = tuple(_head_mix(wl, layer, hr, var, x + 1)
               for x, (hr, var) in enumerate(wl.extra_receivers))
    ev = tuple(to_dtype(np.concatenate(xs, 0), wl.dtype) for xs in extra_v)
    return LayerInputs(q, k, v, w, ew, ev)


@dataclasses.dataclass
class PagedV:
    """Paged value cache: pool [num_pages, page_size, H_kv, d] and per-sequence
    page tables [S, max_pages] (int32, -1 = unused)."""

    pool: torch.Tensor
    block_table: np.ndarray
    page_size: int


def page_values(v: torch.Tensor, layout: BatchLayout, page_size: int,
                seed_rng: np.random.Generator) -> PagedV:
    """Scatter packed values into randomly permuted pages of `page_size` tokens."""
    S = layout.num_seqs
    klens = np.diff(layout.cu_seqlens_k)
    npages = [int(math.ceil(int(n) / page_size)) for n in klens]
    total = int(sum(npages))
    perm = seed_rng.permutation(total)
    max_pages = max(npages) if npages else 0
    table = np.full((S, max(max_pages, 1)), -1, dtype=np.int32)
    H, d = v.shape[1], v.shape[2]
    pool = torch.zeros((max(total, 1), page_size, H, d), dtype=v.dtype)
    nxt = 0
    for s in range(S):
        k0 = int(layout.cu_seqlens_k[s])
        for p in range(npages[s]):
            phys = int(perm[nxt]); nxt += 1
            table[s, p] = phys
            a = p * page_size
            b = min(int(klens[s]), a + page_size)
            pool[phys, : b - a] = v[k0 + a: k0 + b]
    return PagedV(pool, table, page_size)


def page_rng(wl: Workload, layer: int) -> np.random.Generator:
    return _rng(wl, layer, _T_PAGES, 0)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a workload-dtype tensor to float64 (for the oracle)."""
    return t.to(torch.float64).numpy()
