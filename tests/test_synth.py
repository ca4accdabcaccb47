"""Seeded synthetic inputs: determinism, shapes and packing (CPU only)."""
import numpy as np
import torch

from cross_model_attention_mf_amd import synth


def test_deterministic_per_seed():
    wl = synth.workload_by_id(2).replace(seqlens=(300,))
    a, b = synth.layer_inputs(wl, 0), synth.layer_inputs(wl, 0)
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.w, b.w)]:
        assert torch.equal(x, y)
    c = synth.layer_inputs(wl, 1)
    assert not torch.equal(a.q, c.q)
    d = synth.layer_inputs(wl.replace(seed=1), 0)
    assert not torch.equal(a.q, d.q)


def test_shapes_and_dtypes():
    for wl in synth.standard_workloads():
        small = wl.replace(seqlens=tuple(min(n, 700) for n in wl.seqlens[:3]),
                           chunk=256 if wl.chunk else None)
        lay = synth.batch_layout(small, 0)
        li = synth.layer_inputs(small, 0, layout=lay)
        want = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        assert li.q.dtype == want and li.k.dtype == want and li.v.dtype == want
        assert li.q.shape == (lay.total_q, wl.H_s, wl.d)
        assert li.k.shape == (lay.total_k, wl.hkv_s, wl.d)
        assert li.v.shape == (lay.total_k, wl.hkv_r, wl.d)
        assert li.w.shape == (wl.H_r, wl.H_s) and li.w.dtype == torch.float32
        assert len(li.extra_w) == len(wl.extra_receivers)


def test_chunked_layout_steps():
    wl = synth.workload_by_id(4).replace(seqlens=(100, 300, 513), chunk=128)
    assert synth.num_chunk_steps(wl) == 5
    lay = synth.batch_layout(wl, 2)
    # step 2: chunk [256, 384) of sequences long enough
    assert list(lay.seq_ids) == [1, 2]
    assert list(lay.q_pos0) == [256, 256]
    assert list(np.diff(lay.cu_seqlens_q)) == [44, 128]
    assert list(np.diff(lay.cu_seqlens_k)) == [300, 384]
    li = synth.layer_inputs(wl, 0, 2)
    full = synth.layer_inputs(wl.replace(chunk=None), 0)
    lay_full = synth.batch_layout(wl.replace(chunk=None))
    # chunk rows equal the same rows of the unchunked sequence
    a = int(lay_full.cu_seqlens_q[1]) + 256
    assert torch.equal(li.q[:44], full.q[a:a + 44])


def test_varlen_lengths_distribution():
    lens = synth.workload_by_id(4).seqlens
    assert len(lens) == 32 and min(lens) >= 256 and max(lens) <= 16384


def test_paging_roundtrip():
    wl = synth.workload_by_id(4).replace(seqlens=(40, 17), chunk=None)
    lay = synth.batch_layout(wl)
    li = synth.layer_inputs(wl, 0)
    pv = synth.page_values(li.v, lay, 16, synth.page_rng(wl, 0))
    for s in range(2):
        n = int(lay.cu_seqlens_k[s + 1] - lay.cu_seqlens_k[s])
        for t in range(n):
            page = pv.block_table[s, t // 16]
            assert torch.equal(pv.pool[page, t % 16], li.v[int(lay.cu_seqlens_k[s]) + t])
