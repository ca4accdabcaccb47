"""Parity harness: run the HIP path through the C ABI and compare with the oracle.

Tolerances (written here once, used by every parity test):
  block masses   |gpu - oracle| <= MASS_TOL                (normalised mass)
  row LSE        |gpu - oracle| <= LSE_TOL
  index sets     bit-exact, except blocks at the cut accepted by
                 oracle.accept_set with eps = SET_EPS
  values         fp32: rtol 1e-4 (see VAL_RTOL_F32); bf16: one bf16 ulp (rtol 2**-8)
  output O       fp32: max-abs <= 1e-5; bf16: max-abs <= 2e-2 * ||O_oracle||_inf,
                 O_oracle evaluated on the accepted index sets
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
import sys
import time
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np
import torch

from cross_model_attention_mf_amd import mapflow as mf
from cross_model_attention_mf_amd import pipeline, synth
from oracle import mapflow_oracle as orc

MASS_TOL = 1e-6
LSE_TOL = 1e-4
SET_EPS = 1e-6
O_TOL_F32 = 1e-5
O_REL_BF16 = 2e-2
# fp32 values: P = exp(s - lse) inherits the rounding of an fp32 dot product of
# length d (|error| <~ d * 2**-24 * |s|) plus that of lse; with |s| <= 20 and
# d = 64 this is ~8e-5 relative, so stored fp32 values are held to 1e-4.
VAL_RTOL_F32 = 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class GpuRun:
    wl: synth.Workload
    tau: float
    layout: synth.BatchLayout
    inputs: List[synth.LayerInputs]
    state: pipeline.SenderState
    outs: List[torch.Tensor]            # one O [L, Tq, H_r, d] per receiver
    block_table: Optional[np.ndarray]
    layer_map: List[int]
    split_ws: Optional[torch.Tensor] = None   # workspace of the split launch (split=True)


def run_gpu(wl: synth.Workload, tau: float, layers: Sequence[int], step: int = 0,
            layer_map: Optional[Sequence[int]] = None, streams: bool = False,
            multi: bool = False, split: bool = False,
            edit: Optional[Callable[[List[synth.LayerInputs]], None]] = None) -> GpuRun:
    """streams: one launch per receiver, each on its own stream; multi: every
    receiver in one mf_mapped_attn_v_multi call; split: the first receiver
    through mf_mapped_attn_v_split (its workspace is kept on the run); edit:
    changes the host inputs in place before they are uploaded (the oracle
    checks then see the edited ones)."""
    lay = synth.batch_layout(wl, step)
    inputs = [synth.layer_inputs(wl, l, step, lay) for l in layers]
    if edit is not None:
        edit(inputs)
    dev = torch.device("cuda")
    q = torch.stack([x.q for x in inputs]).to(dev)
    k = torch.stack([x.k for x in inputs]).to(dev)
    chunked = wl.chunk is not None
    batch = mf.Batch(lay.cu_seqlens_q, lay.cu_seqlens_k, lay.q_pos0 if chunked else None, wl.B)
    log(f"[parity] {wl.name} tau={tau} layers={list(layers)} step={step} "
        f"Tq={lay.total_q} rowblocks={batch.total_rowblocks}")
    cap = pipeline.count_capacity(batch, q, k, wl.B, tau)
    st = pipeline.alloc_sender(batch, q, k, wl.B, cap)
    pipeline.compress(st, q, k, tau)
    assert st.nnz == cap
    lm = list(range(len(layers))) if layer_map is None else list(layer_map)
    receivers = [(wl.H_r, [x.w for x in inputs], [x.v for x in inputs])]
    for e, (hr, _) in enumerate(wl.extra_receivers):
        receivers.append((hr, [x.extra_w[e] for x in inputs], [x.extra_v[e] for x in inputs]))
    outs, table = [], None
    launches = []
    for hr, ws, vs in receivers:
        W = torch.stack([ws[l] for l in range(len(lm))]).to(dev)
        if wl.paged:
            pvs = [synth.page_values(vs[l], lay, wl.page_size, synth.page_rng(wl, 0)) for l in range(len(lm))]
            table = pvs[0].block_table
            pool = torch.stack([p.pool for p in pvs]).to(dev)
            bt = torch.from_numpy(table).to(dev)
            launches.append((W, pool, bt))
        else:
            launches.append((W, torch.stack(vs).to(dev), None))
    if multi:
        outs = pipeline.mapped_multi(st, [(W, v, bt, wl.page_size) for W, v, bt in launches], lm)
    elif streams and len(launches) > 1:
        ss = [torch.cuda.Stream() for _ in launches]
        cur = torch.cuda.current_stream()
        for s in ss:
            s.wait_stream(cur)
        for (W, v, bt), s in zip(launches, ss):
            with torch.cuda.stream(s):
                outs.append(pipeline.mapped(st, W, v, lm, block_table=bt, page_size=wl.page_size, stream=s))
        for s in ss:
            cur.wait_stream(s)
    elif split:
        W, v, bt = launches[0]
        L_r, H_r = W.shape[0], W.shape[1]
        out = torch.empty((L_r, lay.total_q, H_r, wl.d), dtype=v.dtype, device=dev)
        desc = mf.receiver_desc(v, wl.H_s, H_r, wl.d, wl.B, lm, st.desc.num_layers, out[0].numel(),
                                st.col_idx.numel(), bt, wl.page_size if bt is not None else 0)
        ws = pipeline.split_workspace(desc, batch, dev)
        if ws is not None:
            ws.fill_(0xA5)   # stale bytes: the launch must not depend on the workspace's contents
        outs.append(pipeline.mapped(st, W, v, lm, out=out, block_table=bt, page_size=wl.page_size, split=True,
                                    workspace=ws))
        torch.cuda.synchronize()
        return GpuRun(wl, tau, lay, inputs, st, outs, table, lm, ws)
    else:
        for W, v, bt in launches:
            outs.append(pipeline.mapped(st, W, v, lm, block_table=bt, page_size=wl.page_size))
    torch.cuda.synchronize()
    return GpuRun(wl, tau, lay, inputs, st, outs, table, lm)


@dataclasses.dataclass
class Report:
    max_mass_err: float = 0.0
    max_lse_err: float = 0.0
    max_val_err: float = 0.0
    max_o_err: float = 0.0
    o_inf: float = 0.0
    units: int = 0
    borderline: int = 0
    kept_gpu: int = 0
    kept_oracle: int = 0


def sample_rowblocks(n: int, k: int, seed: int = 0) -> List[int]:
    """First, last and k-2 spread row-blocks (always includes the ragged tail)."""
    if n <= k:
        return list(range(n))
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, n - 1), size=k - 2, replace=False)
    return sorted({0, n - 1, *[int(x) for x in mid]})


def oracle_layer(q64, k64, cu_q, cu_k, p0, B: int, tau: float, heads=None, rowblocks=None,
                 workers: int = 1, extract: bool = True) -> orc.LayerCompression:
    """orc.compress_layer, one call per sender head on a thread pool when
    workers > 1 (numpy releases the GIL in its products and exponentials);
    the units are merged unchanged."""
    hs = list(range(q64.shape[1])) if heads is None else list(heads)
    if workers <= 1 or len(hs) == 1:
        return orc.compress_layer(q64, k64, cu_q, cu_k, p0, B, tau, heads=hs, rowblocks=rowblocks,
                                  extract=extract)
    with concurrent.futures.ThreadPoolExecutor(min(workers, len(hs))) as ex:
        parts = list(ex.map(lambda h: orc.compress_layer(q64, k64, cu_q, cu_k, p0, B, tau, heads=[h],
                                                         rowblocks=rowblocks, extract=extract), hs))
    units = {}
    for part in parts:
        units.update(part.units)
    return orc.LayerCompression(parts[0].rowblocks, units)


def host_workers() -> int:
    """CPU threads for the oracle: the cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def check_layer(run: GpuRun, li: int, rowblocks: Optional[Sequence[int]] = None,
                heads: Optional[Sequence[int]] = None, check_output: bool = True,
                rep: Optional[Report] = None, check_values: bool = True, workers: int = 1,
                lse_tol: float = LSE_TOL) -> Report:
    """Compare layer index li of a GPU run with the oracle on the given
    row-blocks (all by default) and sender heads (all by default): block
    masses, row LSE and index sets always; stored values when check_values;
    the receivers' output when check_output (all heads only)."""
    wl, tau, lay = run.wl, run.tau, run.layout
    rep = rep or Report()
    B = wl.B
    q64 = synth.to_f64(run.inputs[li].q)
    k64 = synth.to_f64(run.inputs[li].k)
    chunked = wl.chunk is not None
    p0 = lay.q_pos0 if chunked else None
    t0 = time.time()
    lc = oracle_layer(q64, k64, lay.cu_seqlens_q, lay.cu_seqlens_k, p0, B, tau, heads=heads,
                      rowblocks=rowblocks, workers=workers, extract=check_values or check_output)
    st = run.state
    H = wl.H_s
    nrb = st.batch.total_rowblocks
    rbs = list(range(nrb)) if rowblocks is None else list(rowblocks)
    hs = list(range(H)) if heads is None else list(heads)
    row_ptr = st.row_ptr.cpu().numpy().astype(np.int64)
    lse_g = st.row_lse[li].cpu().numpy()
    mass_g = st.block_mass[li].cpu().numpy()
    is_bf16 = wl.dtype == "bf16"
    override: Dict = {}
    for i in rbs:
        rb = lc.rowblocks[i]
        for h in hs:
            u = lc.units[(h, i)]
            rep.units += 1
            ncand = len(u.sel.masses)
            mg = mass_g[h, i]
            rep.max_mass_err = max(rep.max_mass_err, float(np.max(np.abs(mg[:ncand] - u.sel.masses))))
            assert np.all(mg[ncand:] == 0), "masses past the causal range must be 0"
            lg = lse_g[h, rb.q0: rb.q0 + rb.rows]
            rep.max_lse_err = max(rep.max_lse_err, float(np.max(np.abs(lg - u.lse))))
            row = (li * H + h) * nrb + i
            e0, e1 = int(row_ptr[row]), int(row_ptr[row + 1])
            cols = st.col_idx[e0:e1].cpu().numpy()
            assert np.all(np.diff(cols) > 0), "col_idx must ascend within a row"
            ok, ndiff, bad = orc.accept_set(u.sel, cols, SET_EPS)
            assert ok, (f"layer {li} head {h} rowblock {i}: index set differs beyond the cut window; "
                        f"gpu {cols.tolist()} oracle {u.sel.kept.tolist()} bad {bad}")
            rep.borderline += ndiff
            rep.kept_gpu += len(cols)
            rep.kept_oracle += u.sel.kstar
            if ndiff:
                override[(h, i)] = cols
                u = orc.compress_unit(q64, k64, rb, h, B, tau, orc.default_scale(wl.d), keep_strip=True)
                lc.units[(h, i)] = u
            if not check_values:
                continue
            # stored key-major: [e][key][query]
            vals_g = st.values[e0:e1].to(torch.float64).cpu().numpy().transpose(0, 2, 1)
            for t, j in enumerate(cols):
                want = u.block(int(j), B) if ndiff else u.values[list(u.sel.kept).index(j)]
                err = np.abs(vals_g[t] - want)
                rep.max_val_err = max(rep.max_val_err, float(err.max()))
                tol = (2.0 ** -8 * np.abs(want) + 1e-30) if is_bf16 else (VAL_RTOL_F32 * np.abs(want) + 1e-9)
                if not np.all(err <= tol):
                    r, c = np.unravel_index(np.argmax(err - tol), err.shape)
                    raise AssertionError(
                        f"values of layer {li} head {h} rowblock {i} block {j}: at ({r},{c}) got "
                        f"{vals_g[t][r, c]!r} want {want[r, c]!r}; max rel err "
                        f"{float(np.max(err / (np.abs(want) + 1e-30))):.3e}")
    assert rep.max_mass_err <= MASS_TOL, f"block mass error {rep.max_mass_err:.3e}"
    assert rep.max_lse_err <= lse_tol, f"row lse error {rep.max_lse_err:.3e}"
    if check_output and heads is None:
        for e, out in enumerate(run.outs):
            # every receiver layer that reads CSR layer li
            for lr, sl in enumerate(run.layer_map):
                if sl != li:
                    continue
                Wl = (run.inputs[lr].w if e == 0 else run.inputs[lr].extra_w[e - 1]).double().numpy()
                vl = synth.to_f64(run.inputs[lr].v if e == 0 else run.inputs[lr].extra_v[e - 1])
                O_ref = orc.mapped_layer(lc, Wl, vl, lay.total_q, B, rowblocks=rbs, kept_override=override)
                O_g = out[lr].to(torch.float64).cpu().numpy()
                rows = np.concatenate([np.arange(lc.rowblocks[i].q0, lc.rowblocks[i].q0 + lc.rowblocks[i].rows)
                                       for i in rbs])
                err = float(np.max(np.abs(O_g[rows] - O_ref[rows])))
                oinf = float(np.max(np.abs(O_ref[rows])))
                rep.max_o_err = max(rep.max_o_err, err)
                rep.o_inf = max(rep.o_inf, oinf)
                if is_bf16:
                    assert err <= O_REL_BF16 * oinf, f"O error {err:.3e} vs {O_REL_BF16} * {oinf:.3e}"
                else:
                    assert err <= O_TOL_F32, f"O error {err:.3e}"
    log(f"[parity] layer {li}: units={rep.units} mass_err={rep.max_mass_err:.2e} "
        f"lse_err={rep.max_lse_err:.2e} val_err={rep.max_val_err:.2e} O_err={rep.max_o_err:.2e} "
        f"(|O|inf {rep.o_inf:.2e}) borderline={rep.borderline} kept={rep.kept_gpu}/{rep.kept_oracle} "
        f"oracle {time.time() - t0:.1f}s")
    return rep


def check_csr(q_layers: Sequence[torch.Tensor], k_layers: Sequence[torch.Tensor], cu_q, cu_k, q_pos0,
              B: int, tau: float, row_ptr: torch.Tensor, col_idx: torch.Tensor, values: torch.Tensor) -> int:
    """Compare a compressed CSR (every layer, head and row-block, as
    mf_compress_blocks numbers its rows) with the oracle run on the host
    inputs q_layers[l] [Tq, H, d], k_layers[l] [Tk, H_kv, d].  Index sets must
    pass accept_set; values the per-dtype tolerance of check_layer.  Returns
    the number of borderline blocks."""
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy()
    is_bf16 = values.dtype == torch.bfloat16
    H = q_layers[0].shape[1]
    border = 0
    for li, (ql, kl) in enumerate(zip(q_layers, k_layers)):
        q64, k64 = synth.to_f64(ql), synth.to_f64(kl)
        lc = orc.compress_layer(q64, k64, cu_q, cu_k, q_pos0, B, tau)
        nrb = len(lc.rowblocks)
        for h in range(H):
            for i in range(nrb):
                row = (li * H + h) * nrb + i
                e0, e1 = int(rp[row]), int(rp[row + 1])
                cols = ci[e0:e1]
                u = lc.units[(h, i)]
                ok, ndiff, bad = orc.accept_set(u.sel, cols, SET_EPS)
                assert ok, f"layer {li} head {h} rowblock {i}: gpu {cols.tolist()} oracle {u.sel.kept.tolist()}"
                border += ndiff
                if ndiff:
                    u = orc.compress_unit(q64, k64, lc.rowblocks[i], h, B, tau, orc.default_scale(q64.shape[2]),
                                          keep_strip=True)
                got = values[e0:e1].to(torch.float64).cpu().numpy().transpose(0, 2, 1)
                for t, j in enumerate(cols):
                    want = u.block(int(j), B) if ndiff else u.values[list(u.sel.kept).index(j)]
                    tol = (2.0 ** -8 * np.abs(want) + 1e-30) if is_bf16 else (VAL_RTOL_F32 * np.abs(want) + 1e-9)
                    assert np.all(np.abs(got[t] - want) <= tol), f"values of layer {li} head {h} rowblock {i} block {j}"
    assert int(rp[0]) == 0 and int(rp[-1]) == ci.shape[0], "row_ptr must run from 0 to the entry count"
    return border


def check_masses(q: torch.Tensor, k: torch.Tensor, cu_q, cu_k, B: int, block_mass: torch.Tensor,
                 rowblocks: Sequence[int]) -> float:
    """Block masses of one layer (q [Tq, H, d], k host tensors) on the given
    row-blocks against the oracle; returns the largest error."""
    q64, k64 = synth.to_f64(q), synth.to_f64(k)
    lc = orc.compress_layer(q64, k64, cu_q, cu_k, None, B, 1.0, rowblocks=rowblocks)
    got = block_mass.cpu().numpy()
    err = 0.0
    for (h, i), u in lc.units.items():
        n = len(u.sel.masses)
        err = max(err, float(np.max(np.abs(got[h, i, :n] - u.sel.masses))))
    assert err <= MASS_TOL, f"block mass error {err:.3e}"
    return err
