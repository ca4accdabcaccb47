"""HIP path vs the fp64 oracle through the C ABI (needs an MI355X).

Small cases compare every output; full-size workloads run in the launch
configuration the bench times and compare sampled row-blocks (all heads),
always including the first and the ragged last row-block."""
import ctypes

import numpy as np
import pytest
import torch

from cross_model_attention_mf_amd import mapflow as mf
from cross_model_attention_mf_amd import pipeline, synth
import parity

pytestmark = pytest.mark.gpu

W1, W2, W3, W4, W5 = synth.standard_workloads()


def tiny_structured(dtype="f32", **kw):
    base = dict(name="tiny_structured", workload_id=11, dtype=dtype, H_s=4, H_r=2, d=64, B=32,
                taus=(0.95,), seqlens=(256,), structured=True, w_var=0.5)
    base.update(kw)
    return synth.Workload(**base)


def test_tiny_fp32_workload_full():
    run = parity.run_gpu(W1, W1.tau, [0])
    rep = parity.check_layer(run, 0)
    assert rep.units == 4 * 8


@pytest.mark.parametrize("tau", [0.3, 0.5, 0.8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tiny_structured_tau_variants(tau, dtype):
    wl = tiny_structured(dtype)
    run = parity.run_gpu(wl, tau, [0])
    rep = parity.check_layer(run, 0)
    assert rep.kept_gpu < rep.units * 5  # selection really drops blocks


@pytest.mark.parametrize("B,d", [(32, 128), (64, 64), (128, 64), (64, 128)])
def test_block_and_head_dims(B, d):
    wl = tiny_structured("bf16", B=B, d=d, seqlens=(3 * B + 17,), H_s=3, H_r=5)
    run = parity.run_gpu(wl, 0.9, [0])
    parity.check_layer(run, 0)


def test_identity_mapping_tau_one_equals_dense_attention():
    wl = tiny_structured("f32", H_r=4, seqlens=(200,))
    run = parity.run_gpu(wl, 1.0, [0])
    rep = parity.check_layer(run, 0)
    # tau = 1 keeps every causal block
    nrb = run.state.batch.total_rowblocks
    assert rep.kept_gpu == sum((min(200, (i + 1) * 32) - 1) // 32 + 1 for i in range(nrb)) * 4
    # with W = I the output is dense causal attention of the sender heads
    q = synth.to_f64(run.inputs[0].q); k = synth.to_f64(run.inputs[0].k); v = synth.to_f64(run.inputs[0].v)
    st = run.state
    W = torch.eye(4, dtype=torch.float32, device="cuda")[None]
    o = pipeline.mapped(st, W, run.inputs[0].v[None].cuda(), [0])
    ref = np.zeros((200, 4, 64))
    for h in range(4):
        P, _ = __import__("oracle.mapflow_oracle", fromlist=["x"]).dense_map(q, k, h)
        ref[:, h] = P @ v[:, h]
    assert np.max(np.abs(o[0].double().cpu().numpy() - ref)) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_varlen_chunked_paged_gqa(dtype):
    wl = tiny_structured(dtype, workload_id=12, H_s=4, H_kv_s=2, H_r=6, H_kv_r=3, d=64, B=32,
                         seqlens=(1000, 77, 300, 33), chunk=256, paged=True, num_layers=2)
    for step in range(synth.num_chunk_steps(wl)):
        run = parity.run_gpu(wl, 0.9, [0, 1], step=step, layer_map=[1, 0])
        parity.check_layer(run, 0)
        parity.check_layer(run, 1)


def test_bf16_4k_workload_sampled():
    run = parity.run_gpu(W2, W2.tau, [0])
    n = run.state.batch.total_rowblocks
    rep = parity.check_layer(run, 0, rowblocks=parity.sample_rowblocks(n, 6))
    frac = rep.kept_gpu / sum(i + 1 for i in parity.sample_rowblocks(n, 6)) / W2.H_s
    parity.log(f"[parity] kept fraction on sampled row-blocks {frac:.3f}")


def split_counts(run) -> np.ndarray:
    """The splits each (unit, head group) of a split launch took, from the
    head of its workspace."""
    wl = run.wl
    ug = run.state.batch.total_rowblocks * (wl.B // 64) * len(run.layer_map) * ((wl.H_r + 7) // 8)
    return run.split_ws[: 4 * ug].view(torch.int32).cpu().numpy()


def test_bf16_4k_workload_split_union_walk():
    """The 4K single layer through the split launch: its longest unions are
    cut into column ranges; the row-blocks with the most splits and a sample
    are checked whole against the oracle."""
    run = parity.run_gpu(W2, W2.tau, [0], split=True)
    n = run.state.batch.total_rowblocks
    counts = split_counts(run).reshape(n, -1)
    assert counts.max() > 1, "the 4K layer should take union splits"
    longest = [int(i) for i in np.argsort(-counts.max(axis=1))[:3]]
    rbs = sorted(set(longest) | set(parity.sample_rowblocks(n, 3, seed=7)))
    parity.log(f"[parity] splits per row-block (max over groups): {counts.max(axis=1).tolist()}")
    parity.check_layer(run, 0, rowblocks=rbs)


@pytest.mark.parametrize("B,d,Hs,Hr,Hkv,seqlens,paged", [
    (64, 128, 32, 24, None, (64 * 21 + 17,), False),           # one ragged sequence
    (64, 64, 12, 9, None, (64 * 13 + 5, 200, 64 * 6), False),    # varlen, a partial head group
    (128, 128, 40, 16, None, (128 * 9 + 33,), False),          # 128-row blocks: both parts split
    (64, 128, 32, 24, 8, (64 * 11 + 3, 300), True),            # paged grouped-query values
])
def test_split_union_walk_matches_oracle(B, d, Hs, Hr, Hkv, seqlens, paged):
    wl = tiny_structured("bf16", workload_id=15, B=B, d=d, H_s=Hs, H_r=Hr, H_kv_r=Hkv, seqlens=seqlens,
                         num_layers=1, paged=paged)
    # tau = 0.99 keeps enough blocks per row-block (up to 5-13 here) for splits
    run = parity.run_gpu(wl, 0.99, [0], split=True)
    assert split_counts(run).max() > 1
    parity.check_layer(run, 0)
    # the unsplit launch: the same sums in another order
    plain = parity.run_gpu(wl, 0.99, [0])
    o_s, o_p = run.outs[0].float(), plain.outs[0].float()
    assert torch.allclose(o_s, o_p, rtol=2e-2, atol=2e-2 * float(o_p.abs().max()))
    # partials are summed in range order: repeated calls give the same bits
    again = parity.run_gpu(wl, 0.99, [0], split=True)
    assert torch.equal(run.outs[0], again.outs[0])


def test_split_union_walk_several_layers_and_a_layer_map():
    """Splits over two receiver layers that read the sender's layers in
    reverse order: each (row-block, layer, head group) has its own splits and
    partials."""
    wl = tiny_structured("bf16", workload_id=17, B=64, d=128, H_s=32, H_r=20, seqlens=(64 * 17 + 40, 64 * 5),
                         num_layers=2)
    run = parity.run_gpu(wl, 0.99, [0, 1], layer_map=[1, 0], split=True)
    assert split_counts(run).max() > 1
    for li in (0, 1):
        parity.check_layer(run, li)
    plain = parity.run_gpu(wl, 0.99, [0, 1], layer_map=[1, 0])
    o_s, o_p = run.outs[0].float(), plain.outs[0].float()
    assert torch.allclose(o_s, o_p, rtol=2e-2, atol=2e-2 * float(o_p.abs().max()))


def test_split_launch_checks_its_workspace():
    """A split launch refuses a missing, short or misaligned workspace before
    launching anything."""
    wl = tiny_structured("bf16", workload_id=15, B=64, d=128, H_s=32, H_r=24, seqlens=(64 * 21 + 17,),
                         num_layers=1)
    run = parity.run_gpu(wl, 0.99, [0], split=True)
    ws = run.split_ws
    assert ws is not None
    st, dev = run.state, ws.device
    W = run.inputs[0].w[None].to(dev)
    v = run.inputs[0].v[None].to(dev)
    out = torch.zeros_like(run.outs[0])
    desc = mf.receiver_desc(v, wl.H_s, wl.H_r, wl.d, wl.B, [0], 1, out[0].numel(), st.col_idx.numel())
    need = mf.mapped_split_workspace_size(desc, st.batch)
    assert need == ws.numel() > 0

    def call(ptr, nbytes):
        return mf.lib().mf_mapped_attn_v_split(ctypes.byref(desc), ctypes.byref(st.batch.c), st.row_ptr.data_ptr(),
                                               st.col_idx.data_ptr(), st.values.data_ptr(), W.data_ptr(),
                                               v.data_ptr(), out.data_ptr(), ptr, nbytes,
                                               torch.cuda.current_stream().cuda_stream)
    assert call(None, 0) == mf.MF_ERR_WORKSPACE
    assert call(ws.data_ptr(), need - 1) == mf.MF_ERR_WORKSPACE
    big = torch.empty(need + 256, dtype=torch.uint8, device=dev)
    assert call(big.data_ptr() + 16, need) == mf.MF_ERR_INVALID
    torch.cuda.synchronize()
    assert not out.any(), "a refused call must launch nothing"
    assert call(big.data_ptr(), need) == mf.MF_OK
    torch.cuda.synchronize()
    assert torch.equal(out, run.outs[0])


def test_split_launch_without_splits_is_the_plain_launch():
    """A launch large enough to fill the chip takes no splits and needs no
    workspace: its output is mf_mapped_attn_v's bit for bit."""
    wl = tiny_structured("bf16", workload_id=16, B=64, d=128, H_s=32, H_r=24, seqlens=(64 * 40,), num_layers=12)
    run = parity.run_gpu(wl, 0.95, list(range(12)), split=True)
    assert run.split_ws is None
    plain = parity.run_gpu(wl, 0.95, list(range(12)))
    assert torch.equal(run.outs[0], plain.outs[0])
    parity.check_layer(run, 11, rowblocks=[0, 39])


@pytest.mark.timeout(600)
@pytest.mark.parametrize("tau,full_layer", [(0.95, 8), (0.90, 3), (0.99, 12)])
def test_bf16_8k_16_layers(tau, full_layer):
    """All 16 layers in one launch per stage (the bench's configuration);
    sampled row-blocks of the first and last layer, and one whole layer (all
    128 row-blocks x 32 sender heads: masses, LSE, index sets, values, O)."""
    run = parity.run_gpu(W3, tau, list(range(W3.num_layers)))
    n = run.state.batch.total_rowblocks
    for li in (0, 15):
        parity.check_layer(run, li, rowblocks=parity.sample_rowblocks(n, 3, seed=li))
    rep = parity.check_layer(run, full_layer, workers=parity.host_workers())
    assert rep.units == n * W3.H_s


def test_varlen_chunked_paged_16_layers_sampled():
    steps = synth.num_chunk_steps(W4)
    for step in (0, steps - 1):
        run = parity.run_gpu(W4, W4.tau, list(range(W4.num_layers)), step=step)
        n = run.state.batch.total_rowblocks
        parity.check_layer(run, 3, rowblocks=parity.sample_rowblocks(n, 4, seed=step))


@pytest.mark.timeout(900)
def test_32k_one_sender_two_receivers_two_streams():
    run = parity.run_gpu(W5, W5.tau, [0], streams=True)
    n = run.state.batch.total_rowblocks
    parity.check_layer(run, 0, rowblocks=[0, n // 2, n - 1])
    # every row-block and sender head: masses, LSE and index sets
    rep = parity.check_layer(run, 0, check_output=False, check_values=False, workers=parity.host_workers())
    assert rep.units == n * W5.H_s
    # the two concurrent launches equal the same launches run one after another
    seq = parity.run_gpu(W5.replace(seqlens=(4096,)), W5.tau, [0], streams=False)
    par = parity.run_gpu(W5.replace(seqlens=(4096,)), W5.tau, [0], streams=True)
    for a, b in zip(seq.outs, par.outs):
        assert torch.equal(a, b)


def test_several_receivers_in_one_launch():
    # one sender (40 heads, B = 128) feeding receivers of 32 and 24 heads in one
    # call: oracle parity, and the same outputs as one launch per receiver
    wl = W5.replace(seqlens=(4096,))
    multi = parity.run_gpu(wl, wl.tau, [0], multi=True)
    n = multi.state.batch.total_rowblocks
    parity.check_layer(multi, 0, rowblocks=[0, n // 2, n - 1])
    sep = parity.run_gpu(wl, wl.tau, [0])
    for a, b in zip(multi.outs, sep.outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("B,d", [(64, 64), (64, 128), (32, 64), (128, 128)])
def test_several_receivers_varlen_paged_gqa(B, d):
    # grouped-query first receiver (6 heads over 3 value heads) and a 9-head
    # second one, paged values, varlen chunked batch, two layers
    wl = tiny_structured("bf16", workload_id=16, B=B, d=d, H_s=12, H_r=6, H_kv_r=3,
                         extra_receivers=((9, 0.5),), paged=True, page_size=16,
                         seqlens=(3 * B + 17, B + 5, 2 * B), chunk=2 * B, num_layers=2)
    multi = parity.run_gpu(wl, 0.9, [0, 1], step=1, multi=True)
    for li in range(2):
        parity.check_layer(multi, li)
    sep = parity.run_gpu(wl, 0.9, [0, 1], step=1)
    for a, b in zip(multi.outs, sep.outs):
        assert torch.equal(a, b)


def test_capacity_sync_and_async():
    wl = tiny_structured("bf16", seqlens=(512,))
    run = parity.run_gpu(wl, 0.8, [0])
    st = run.state
    nnz = st.nnz
    q = run.inputs[0].q[None].cuda(); k = run.inputs[0].k[None].cuda()
    small = pipeline.alloc_sender(st.batch, q, k, wl.B, nnz - 3)
    mf.block_stats(small.desc, small.batch, q, k, small.row_lse, small.block_mass, small.stats_workspace)
    with pytest.raises(mf.MapflowError) as e:
        mf.compress_blocks(small.desc, small.batch, q, k, small.row_lse, small.block_mass, 0.8,
                           small.row_ptr, small.col_idx, small.values, nnz - 3, small.workspace)
    assert e.value.status == mf.MF_ERR_CAPACITY
    assert torch.equal(small.row_ptr, st.row_ptr)
    # asynchronous: entries past capacity are dropped, row_ptr[last] still holds the count
    small.col_idx.fill_(-7)
    mf.compress_blocks(small.desc, small.batch, q, k, small.row_lse, small.block_mass, 0.8,
                       small.row_ptr, small.col_idx, small.values, nnz - 3, small.workspace,
                       sync_count=False)
    torch.cuda.synchronize()
    assert int(small.row_ptr[-1]) == nnz
    assert torch.equal(small.col_idx, st.col_idx[: nnz - 3])
    assert torch.equal(small.values, st.values[: nnz - 3])


def test_empty_and_degenerate_batches():
    # zero sequences: every call is a no-op that succeeds
    b = mf.Batch([0], [0], None, 64)
    q = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16, device="cuda")
    st = pipeline.alloc_sender(b, q, q, 64, 1)
    pipeline.compress(st, q, q, 0.9)
    assert st.nnz == 0 and int(st.row_ptr[0]) == 0
    # a zero-length chunk between sequences and single-token sequences
    wl = tiny_structured("f32", workload_id=13, seqlens=(1, 40, 1, 65))
    run = parity.run_gpu(wl, 0.7, [0])
    parity.check_layer(run, 0)


def test_repeat_calls_are_deterministic():
    wl = tiny_structured("bf16", seqlens=(700,))
    a = parity.run_gpu(wl, 0.9, [0])
    b = parity.run_gpu(wl, 0.9, [0])
    assert torch.equal(a.state.block_mass, b.state.block_mass)
    assert torch.equal(a.state.col_idx[: a.state.nnz], b.state.col_idx[: b.state.nnz])
    assert torch.equal(a.outs[0], b.outs[0])


@pytest.mark.parametrize("B,d,Hs,Hr,Hkv", [(64, 128, 32, 24, None), (128, 128, 40, 16, None), (32, 64, 5, 6, None),
                                            (64, 64, 12, 9, None), (64, 64, 24, 8, None), (64, 64, 32, 8, None),
                                            (64, 64, 40, 8, None), (128, 64, 16, 8, None), (64, 128, 12, 8, None),
                                            (64, 128, 8, 8, None), (128, 128, 20, 24, None),
                                            # half-stage ring: a head pair with one head past H_s;
                                            # 128-row blocks at d = 128
                                            (64, 128, 31, 8, None), (128, 128, 32, 16, None),
                                            # grouped-query receivers: V staged per value head
                                            (64, 128, 32, 24, 8), (128, 128, 40, 32, 8), (64, 64, 24, 12, 4),
                                            (64, 128, 16, 16, 2), (128, 64, 8, 20, 5), (64, 128, 48, 16, 4),
                                            # 33-64 sender heads: two K chunks of 32, or 32 + 16
                                            (64, 64, 64, 8, None), (64, 128, 56, 8, 2), (128, 128, 48, 24, None),
                                            (128, 64, 36, 16, 8)])
def test_portable_and_mfma_mapped_kernels_agree_with_oracle(B, d, Hs, Hr, Hkv):
    wl = tiny_structured("bf16", workload_id=14, B=B, d=d, H_s=Hs, H_r=Hr, H_kv_r=Hkv,
                         seqlens=(4 * B + 9, B + 3), num_layers=1)
    runs = []
    for stages in (("mapped",), ()):
        with mf.force_portable(*stages):
            run = parity.run_gpu(wl, 0.9, [0])
        parity.check_layer(run, 0)
        runs.append(run.outs[0].float())
    # both kernels compute the same sums in a different order
    assert torch.allclose(runs[0], runs[1], rtol=2e-2, atol=2e-2 * float(runs[0].abs().max()))


@pytest.mark.parametrize("B,d", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_portable_and_mfma_block_stats_agree_with_oracle(B, d):
    # varlen chunked batch: groups of four row-blocks cut short by sequence
    # ends, a one-row tail block, a sequence shorter than one block, several
    # (layer, head) pairs per XCD queue, and chunk rows starting past 0; at
    # B = 128 also last row-blocks whose second 64-row half is empty (1, 17,
    # 60 and 64 rows) or partial (100 rows)
    seqlens = ((64 * 9 + 17, 64 * 2 + 1, 63, 64 * 5, 700) if B == 64 else
               (128 * 5 + 17, 128 + 1, 63, 128 * 3 + 64, 700, 128 * 2 + 100))
    wl = tiny_structured("bf16", workload_id=15, B=B, d=d, H_s=12, H_r=4, num_layers=2,
                         seqlens=seqlens, chunk=256)
    results = []
    for stages in (("stats",), ()):
        with mf.force_portable(*stages):
            run = parity.run_gpu(wl, 0.9, [0, 1], step=1)
        for li in range(2):
            parity.check_layer(run, li)
        results.append((run.state.row_lse.clone(), run.state.block_mass.clone()))
    (lse_p, mass_p), (lse_f, mass_f) = results
    assert torch.allclose(lse_p, lse_f, rtol=0, atol=1e-4)
    assert float((mass_p - mass_f).abs().max()) <= 2e-6


@pytest.mark.parametrize("B,d", [(64, 64), (64, 128), (128, 128)])
def test_block_stats_scores_far_above_the_diagonal_block(B, d):
    """Keys whose scores lie far above the diagonal block's maximum move the
    row's exponent reference mid-row: from a first 32-key half, from a second
    half after the first was summed against the old reference, and where
    exp2 against the old reference overflows fp32 (block 0).  MFMA and
    portable kernels against the oracle."""
    # natural-log logits planted on every row that sees the key, walking down
    # from the diagonal (64-key blocks): block 4 (about 29 log2 units above
    # the diagonal's maximum, where an fp32 log mass against the diagonal's
    # reference would lose the mass's sixth digit), block 3 (first half),
    # block 2 (second half), block 1 (second half, within the reference's
    # range), block 0 (first half, exp2 against the old reference overflows)
    plants = ((4 * 64 + 20, 20.0), (3 * 64 + 8, 75.0), (2 * 64 + 40, 135.0), (64 + 40, 150.0), (10, 250.0))

    def plant(inputs):
        x = inputs[0]
        x.q[:, :, 0] = 4.0
        for pos, logit in plants:
            x.k[pos, :, 0] = logit * d ** 0.5 / 4.0

    wl = tiny_structured("bf16", workload_id=17, B=B, d=d, H_s=4, H_r=2, num_layers=1,
                         seqlens=(6 * 64 + 5 if B == 64 else 3 * 128 + 70, 2 * B + 7))
    masses = []
    for stages in (("stats",), ()):
        with mf.force_portable(*stages):
            run = parity.run_gpu(wl, 0.9, [0], edit=plant)
        # a score near 250 comes from a d-term fp32 dot product of that size:
        # its rounding is bounded by d 2^-24 |score|, above the usual 1e-4
        rep = parity.check_layer(run, 0, lse_tol=parity.LSE_TOL + d * 2.0 ** -24 * 260.0)
        parity.log(f"[parity] planted scores: mass err {rep.max_mass_err:.2e} lse err {rep.max_lse_err:.2e}")
        masses.append(run.state.block_mass.clone())
    assert float((masses[0] - masses[1]).abs().max()) <= 2e-6


@pytest.mark.parametrize("B,seqlens", [(64, (64 * 9 + 17, 63, 700)),          # up to 64 candidates per row
                                       (32, (32 * 120 + 5, 40)),              # up to 128
                                       (32, (32 * 250 + 31, 32 * 3))])         # up to 256
def test_wave_and_workgroup_selection_agree(B, seqlens):
    """The one-wave-per-row selection and the workgroup sort give the same
    CSR; the run is also checked against the oracle."""
    wl = tiny_structured("bf16", workload_id=16, B=B, d=64, H_s=6, H_r=4, seqlens=seqlens)
    runs = []
    for stages in (("select",), ()):
        with mf.force_portable(*stages):
            for tau in (0.5, 0.95):
                runs.append(parity.run_gpu(wl, tau, [0]))
    nrb = runs[-1].state.batch.total_rowblocks
    parity.check_layer(runs[-1], 0, rowblocks=parity.sample_rowblocks(nrb, 12))
    for a, b in zip(runs[:2], runs[2:]):
        assert a.state.nnz == b.state.nnz
        assert torch.equal(a.state.row_ptr, b.state.row_ptr)
        assert torch.equal(a.state.col_idx, b.state.col_idx)
        assert torch.equal(a.state.values, b.state.values)


@pytest.mark.parametrize("B,d", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_portable_and_mfma_extraction_agree_with_oracle(B, d):
    """bf16: the MFMA extraction and its portable twin write the same CSR;
    their values (each rounded to bf16 from its own fp32 scores) agree to a
    bf16 rounding step, and both match the oracle."""
    wl = tiny_structured("bf16", workload_id=17, B=B, d=d, H_s=6, H_r=4,
                         seqlens=(B * 5 + 9, B * 2, 33, B + 70), chunk=None)
    runs = []
    for stages in (("extract",), ()):
        with mf.force_portable(*stages):
            run = parity.run_gpu(wl, 0.9, [0])
        parity.check_layer(run, 0)
        runs.append(run.state)
    a, b = runs
    assert a.nnz == b.nnz
    assert torch.equal(a.row_ptr, b.row_ptr) and torch.equal(a.col_idx, b.col_idx)
    diff = (a.values[: a.nnz].float() - b.values[: b.nnz].float()).abs().max().item()
    assert diff <= 2.0 ** -8, diff


@pytest.mark.parametrize("groups", [2, 3])
def test_layer_group_pipeline_equals_one_pass(groups):
    # each layer group's fused step on a second stream, overlapping the next
    # group's statistics: the same O bit for bit as one pass over all layers,
    # which itself matches the oracle
    wl = tiny_structured("bf16", workload_id=18, B=64, d=128, H_s=32, H_r=24, seqlens=(5 * 64 + 9,),
                         num_layers=4)
    run = parity.run_gpu(wl, 0.9, list(range(4)))
    parity.check_layer(run, 3)
    dev = torch.device("cuda")
    q = torch.stack([x.q for x in run.inputs]).to(dev)
    k = torch.stack([x.k for x in run.inputs]).to(dev)
    v = torch.stack([x.v for x in run.inputs]).to(dev)
    W = torch.stack([x.w for x in run.inputs]).to(dev)
    batch = mf.Batch(run.layout.cu_seqlens_q, run.layout.cu_seqlens_k, None, wl.B)
    out = torch.empty_like(run.outs[0])
    pipe = pipeline.LayerGroupPipeline(batch, q, k, v, W, out, wl.B, 0.9, wl.H_r, groups)
    assert pipe.capacity == run.state.nnz
    for overlap in (True, False, True):
        out.zero_()
        pipe.step(overlap)
        torch.cuda.synchronize()
        assert torch.equal(out, run.outs[0])


def test_compress_with_row_ptr_not_16_byte_aligned():
    # a row_ptr that is only 4-byte aligned takes the scan's element-wise
    # path: the same CSR as the vector path
    wl = tiny_structured("bf16", workload_id=19, B=64, d=64, H_s=6, H_r=4, seqlens=(9 * 64 + 5, 300),
                         num_layers=2)
    run = parity.run_gpu(wl, 0.9, [0, 1])
    parity.check_layer(run, 1)
    st = run.state
    dev = torch.device("cuda")
    q = torch.stack([x.q for x in run.inputs]).to(dev)
    k = torch.stack([x.k for x in run.inputs]).to(dev)
    big = torch.full((st.row_ptr.numel() + 1,), -1, dtype=torch.int32, device=dev)
    rp = big[1:]
    assert rp.data_ptr() % 16 != 0
    col = torch.empty_like(st.col_idx)
    vals = torch.empty_like(st.values)
    nnz = mf.compress_blocks(st.desc, st.batch, q, k, st.row_lse, st.block_mass, 0.9, rp, col, vals,
                             col.numel(), st.workspace, sync_count=True)
    assert nnz == st.nnz
    assert torch.equal(rp, st.row_ptr)
    assert torch.equal(col[:nnz], st.col_idx[:nnz]) and torch.equal(vals[:nnz], st.values[:nnz])


def test_mfma_probe_runs_and_writes_every_output():
    out = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    for vec in (False, True):
        mf.mfma_probe(out, 4, 16, vec)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
