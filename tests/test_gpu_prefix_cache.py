"""Prefix cache of compressed maps on the GPU, through the C ABI.

A sequence's compressed rows for its first m blocks come from the cache, the
rest from compressing the sequence as a chunk that starts at row m * B; the
spliced CSR must equal, bit for bit, what compressing the whole sequence
writes (causality: a row's kept blocks and values see only keys up to the
row).  The whole-sequence compression itself is checked against the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

from cross_model_attention_mf_amd import mapflow as mf
from cross_model_attention_mf_amd import pipeline, synth
import parity

pytestmark = pytest.mark.gpu


def seq_workload(dtype, B, d, T, wid=21, H_s=4, L=2):
    return synth.Workload(name="prefix_seq", workload_id=wid, dtype=dtype, H_s=H_s, H_r=3, d=d, B=B,
                          taus=(0.9,), seqlens=(T,), num_layers=L, structured=True, w_var=0.5)


def seq_qk(wl):
    xs = [synth.layer_inputs(wl, l) for l in range(wl.num_layers)]
    return torch.stack([x.q for x in xs]).cuda(), torch.stack([x.k for x in xs]).cuda()


def compress_rows(q, k, B, tau, q0=0, cu=None):
    """Compress q rows [q0, T) of one sequence (or a whole batch given cu)."""
    T = k.shape[1]
    if cu is None:
        batch = mf.Batch([0, T - q0], [0, T], [q0] if q0 else None, B)
    else:
        batch = mf.Batch(cu, cu, None, B)
    qs = q[:, q0:].contiguous()
    cap = pipeline.count_capacity(batch, qs, k, B, tau)
    st = pipeline.alloc_sender(batch, qs, k, B, cap)
    pipeline.compress(st, qs, k, tau)
    return st


def tokens_of(T, seed):
    return np.random.default_rng(seed).integers(0, 50000, T, dtype=np.int32)


def splice(cache, keys, m, n_blocks, suf, like, cap=None):
    L, H, B = like.desc.num_layers, like.desc.H_s, like.B
    cap = like.col_idx.numel() if cap is None else cap
    rp = torch.full((L * H * n_blocks + 1,), -1, dtype=torch.int32, device="cuda")
    ci = torch.full((max(cap, 1),), -1, dtype=torch.int32, device="cuda")
    vals = torch.zeros((max(cap, 1), B, B), dtype=like.values.dtype, device="cuda")
    if suf is None:
        nnz = cache.splice(keys[:m], m, n_blocks, None, 0, 0, None, None, rp, ci, vals)
    else:
        nnz = cache.splice(keys[:m], m, n_blocks, suf.row_ptr.cpu().numpy(), suf.batch.total_rowblocks, 0,
                           suf.col_idx, suf.values, rp, ci, vals)
    torch.cuda.synchronize()
    return nnz, rp, ci, vals


def assert_same_csr(got, full):
    nnz, rp, ci, vals = got
    assert nnz == full.nnz
    assert torch.equal(rp, full.row_ptr)
    assert torch.equal(ci[:nnz], full.col_idx[:nnz])
    assert torch.equal(vals[:nnz], full.values[:nnz])


@pytest.mark.parametrize("dtype,B,d", [("bf16", 64, 128), ("bf16", 32, 64), ("f32", 32, 64), ("bf16", 128, 64)])
def test_splice_equals_whole_sequence_compression(dtype, B, d):
    T = 7 * B + 19
    wl = seq_workload(dtype, B, d, T)
    tau = 0.9
    run = parity.run_gpu(wl, tau, [0, 1])
    for l in range(2):
        parity.check_layer(run, l)
    full = run.state
    n_blocks = full.batch.total_rowblocks
    q, k = seq_qk(wl)
    keys = mf.prefix_block_hashes(tokens_of(T, 5), B)
    assert len(keys) == 7 and n_blocks == 8
    cache = mf.MapCache(q.dtype, 2, wl.H_s, B, 64 << 20)
    cache.insert(keys, full.row_ptr.cpu().numpy(), n_blocks, 0, full.col_idx, full.values)
    for m in (0, 1, 4, 7):
        if m:
            assert cache.lookup(keys[:m]) == m
        suf = compress_rows(q, k, B, tau, m * B)
        got = splice(cache, keys, m, n_blocks, suf, full)
        assert_same_csr(got, full)
        if m:
            cache.release(keys[:m], m)
        if m == 4:
            # the spliced map drives the fused kernel to the same outputs
            nnz, rp, ci, vals = got
            st2 = dataclasses.replace(full, row_ptr=rp, col_idx=ci, values=vals, nnz=nnz)
            W = torch.stack([x.w for x in run.inputs]).cuda()
            v = torch.stack([x.v for x in run.inputs]).cuda()
            assert torch.equal(pipeline.mapped(st2, W, v, [0, 1]), run.outs[0])
    s = cache.stats()
    assert s["entries"] == 1 and s["pinned_entries"] == 0
    assert s["blocks_hit"] == 1 + 4 + 7
    cache.close()


def test_whole_sequence_from_cache_and_divergent_sequences():
    B, d, tau = 64, 128, 0.9
    T = 6 * B
    wl = seq_workload("bf16", B, d, T, wid=22)
    q, k = seq_qk(wl)
    full = compress_rows(q, k, B, tau)
    toks = tokens_of(T, 7)
    keys = mf.prefix_block_hashes(toks, B)
    cache = mf.MapCache(q.dtype, 2, wl.H_s, B, 64 << 20)
    cache.insert(keys, full.row_ptr.cpu().numpy(), 6, 0, full.col_idx, full.values)
    # every block cached: no suffix at all
    assert cache.lookup(keys) == 6
    assert_same_csr(splice(cache, keys, 6, 6, None, full), full)
    cache.release(keys, 6)
    # a second sequence that shares the first 3 blocks (tokens, q and k) and
    # then diverges, longer than the cached one
    T2 = 9 * B + 5
    wl2 = seq_workload("bf16", B, d, T2, wid=23)
    q2, k2 = seq_qk(wl2)
    q2[:, : 3 * B] = q[:, : 3 * B]
    k2[:, : 3 * B] = k[:, : 3 * B]
    toks2 = np.concatenate([toks[: 3 * B], tokens_of(T2 - 3 * B, 8)])
    keys2 = mf.prefix_block_hashes(toks2, B)
    assert np.array_equal(keys2[:3], keys[:3]) and keys2[3] != keys[3]
    full2 = compress_rows(q2, k2, B, tau)
    m = cache.lookup(keys2)
    assert m == 3
    suf2 = compress_rows(q2, k2, B, tau, m * B)
    assert_same_csr(splice(cache, keys2, m, 10, suf2, full2), full2)
    cache.release(keys2, m)
    # a splice past the output capacity writes nothing and reports the count
    m = cache.lookup(keys2)
    with pytest.raises(mf.MapflowError) as e:
        splice(cache, keys2, m, 10, suf2, full2, cap=full2.nnz - 1)
    assert e.value.status == mf.MF_ERR_CAPACITY
    cache.release(keys2, m)
    cache.close()


def test_rows_of_a_batched_compression_are_cached_per_sequence():
    """Insert a sequence's rows out of a two-sequence batch (rb_first > 0)."""
    B, d, tau = 64, 128, 0.85
    TX, TA = 3 * B + 40, 5 * B + 11
    qx, kx = seq_qk(seq_workload("bf16", B, d, TX, wid=24))
    qa, ka = seq_qk(seq_workload("bf16", B, d, TA, wid=25))
    batch_st = compress_rows(torch.cat([qx, qa], 1), torch.cat([kx, ka], 1), B, tau, cu=[0, TX, TX + TA])
    full_a = compress_rows(qa, ka, B, tau)
    keys = mf.prefix_block_hashes(tokens_of(TA, 9), B)
    cache = mf.MapCache(qa.dtype, 2, 4, B, 64 << 20)
    R = batch_st.batch.total_rowblocks
    cache.insert(keys, batch_st.row_ptr.cpu().numpy(), R, 4, batch_st.col_idx, batch_st.values)
    m = cache.lookup(keys)
    assert m == 5
    suf = compress_rows(qa, ka, B, tau, m * B)
    assert_same_csr(splice(cache, keys, m, 6, suf, full_a), full_a)
    cache.release(keys, m)
    cache.close()


def test_eviction_is_lru_and_skips_pinned_entries():
    B, d, tau = 64, 64, 0.9
    T = 4 * B
    seqs = []
    for i, wid in enumerate((26, 27, 28)):
        wl = seq_workload("bf16", B, d, T, wid=wid)
        q, k = seq_qk(wl)
        st = compress_rows(q, k, B, tau)
        seqs.append((st, mf.prefix_block_hashes(tokens_of(T, 30 + i), B)))
    # entry sizes from a roomy cache
    big = mf.MapCache(torch.bfloat16, 2, 4, B, 64 << 20)
    sizes = []
    for st, keys in seqs:
        before = big.stats()["bytes_used"]
        big.insert(keys, st.row_ptr.cpu().numpy(), 4, 0, st.col_idx, st.values)
        sizes.append(big.stats()["bytes_used"] - before)
    table = (64 << 20) - big.stats()["bytes_capacity"]
    big.close()
    sa, sb, sc = sizes
    (a, ka), (b, kb), (c, kc) = seqs
    cache = mf.MapCache(torch.bfloat16, 2, 4, B, table + sa + max(sb, sc))
    ins = lambda st, keys: cache.insert(keys, st.row_ptr.cpu().numpy(), 4, 0, st.col_idx, st.values)
    ins(a, ka)
    ins(b, kb)
    assert cache.stats()["bytes_used"] == sa + sb
    assert cache.lookup(ka) == 4          # pins A, the least recently used
    assert cache.lookup(kb) == 4
    cache.release(kb, 4)
    ins(c, kc)                            # evicts B: A is pinned
    s = cache.stats()
    assert s["evictions"] == 1 and s["entries"] == 2 and s["pinned_entries"] == 1
    assert cache.lookup(kb) == 0
    assert_same_csr(splice(cache, ka, 4, 4, None, a), a)
    # with A and C both pinned, B no longer fits
    assert cache.lookup(kc) == 4
    with pytest.raises(mf.MapflowError) as e:
        ins(b, kb)
    assert e.value.status == mf.MF_ERR_CAPACITY
    cache.release(kc, 4)
    cache.release(ka, 4)
    # A was used before C: it goes first, and C too if B does not fit in A's room
    ins(b, kb)
    s = cache.stats()
    assert s["evictions"] in (2, 3) and s["entries"] == 4 - s["evictions"]
    assert cache.lookup(ka) == 0
    assert cache.lookup(kc) == (4 if s["evictions"] == 2 else 0)
    assert cache.lookup(kb) == 4
    assert_same_csr(splice(cache, kb, 4, 4, None, b), b)
    cache.close()


def test_fetch_overlapped_with_other_work_is_exact():
    """Splices run stream-ordered on a side stream while other kernels run on
    the current stream; back-to-back calls reuse the staging area.  The
    spliced CSR is checked against the oracle, and so are the masses of the
    work that ran beside the fetch."""
    B, d, tau = 64, 128, 0.9
    T = 7 * B + 19
    wl = seq_workload("bf16", B, d, T, wid=29)
    q, k = seq_qk(wl)
    q_host, k_host = q.cpu(), k.cpu()
    full = compress_rows(q, k, B, tau)
    keys = mf.prefix_block_hashes(tokens_of(T, 11), B)
    cache = mf.MapCache(q.dtype, 2, wl.H_s, B, 64 << 20)
    cache.insert(keys, full.row_ptr.cpu().numpy(), 8, 0, full.col_idx, full.values)
    # other work: block statistics of another model's Q/K
    oq, ok = seq_qk(seq_workload("bf16", B, d, 4 * T, wid=30, H_s=6))
    ob = mf.Batch([0, 4 * T], [0, 4 * T], None, B)
    ost = pipeline.alloc_sender(ob, oq, ok, B, 0)

    def other():
        mf.block_stats(ost.desc, ob, oq, ok, ost.row_lse, ost.block_mass, ost.stats_workspace)

    other()
    torch.cuda.synchronize()
    ref_mass = ost.block_mass.clone()
    nrb_o = ob.total_rowblocks
    parity.check_masses(oq[0].cpu(), ok[0].cpu(), [0, 4 * T], [0, 4 * T], B, ref_mass[0],
                        [0, nrb_o // 2, nrb_o - 1])
    side = torch.cuda.Stream()
    for m in (4, 7, 7):
        assert cache.lookup(keys[:m]) == m
        suf = compress_rows(q, k, B, tau, m * B)
        rp = torch.full_like(full.row_ptr, -1)
        ci = torch.full_like(full.col_idx, -1)
        vals = torch.zeros_like(full.values)
        ost.block_mass.zero_()
        nnz = pipeline.fetch_overlapped(cache, keys, m, 8, suf, rp, ci, vals, other, side)
        torch.cuda.synchronize()
        cache.release(keys[:m], m)
        assert_same_csr((nnz, rp, ci, vals), full)
        assert torch.equal(ost.block_mass, ref_mass)
        if m == 4:
            parity.check_csr(list(q_host), list(k_host), [0, T], [0, T], None, B, tau, rp, ci[:nnz], vals[:nnz])
    cache.close()
