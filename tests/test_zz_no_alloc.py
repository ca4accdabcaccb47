"""The no-allocation compression entry point against the workspace one
(needs an MI355X).  Two calls in a row, the second on a smaller batch, so the
static scratch the first call left behind must not leak into the second."""
import pytest
import torch

from cross_model_attention_mf_amd import mapflow as mf
from cross_model_attention_mf_amd import pipeline, synth
import parity

pytestmark = pytest.mark.gpu


def _inputs(seqlens, layers):
    wl = synth.Workload(name="noalloc", workload_id=41, dtype="bf16", H_s=8, H_r=4, d=128, B=64,
                        taus=(0.9,), seqlens=seqlens, structured=True, num_layers=layers)
    lay = synth.batch_layout(wl)
    ins = [synth.layer_inputs(wl, l, layout=lay) for l in range(layers)]
    q = torch.stack([x.q for x in ins]).cuda()
    k = torch.stack([x.k for x in ins]).cuda()
    batch = mf.Batch(lay.cu_seqlens_q, lay.cu_seqlens_k, None, wl.B)
    return wl, lay, ins, q, k, batch


def test_noalloc_compression_equals_workspace_compression():
    for seqlens, layers in (((2000, 700, 129), 2), ((300,), 1)):
        wl, lay, ins, q, k, batch = _inputs(seqlens, layers)
        tau = 0.9
        cap = pipeline.count_capacity(batch, q, k, wl.B, tau)
        ref = pipeline.compress(pipeline.alloc_sender(batch, q, k, wl.B, cap), q, k, tau)
        got = pipeline.alloc_sender(batch, q, k, wl.B, cap)
        mf.block_stats(got.desc, batch, q, k, got.row_lse, got.block_mass, got.stats_workspace)
        # scratch garbage from a previous call must not matter: the new entry
        # point's buffers start filled with junk
        got.row_ptr.fill_(-7)
        got.col_idx.fill_(-7)
        got.values.fill_(3.0)
        nnz = mf.compress_blocks_noalloc(got.desc, batch, q, k, got.row_lse, got.block_mass, tau, got.row_ptr,
                                         got.col_idx, got.values, cap, sync_count=True)
        torch.cuda.synchronize()
        assert nnz == ref.nnz == cap
        assert torch.equal(got.row_ptr, ref.row_ptr)
        assert torch.equal(got.col_idx[:cap], ref.col_idx[:cap])
        assert torch.equal(got.values[:cap], ref.values[:cap])
        # and against the oracle on every unit of the first layer
        run = parity.GpuRun(wl, tau, lay, ins, got, [], None, list(range(layers)))
        parity.check_layer(run, 0, check_output=False)


def test_noalloc_rejects_batches_beyond_its_scratch():
    # 64 layers x 64 heads x 512 row-blocks x (16 bit words + a count) > 16 MiB;
    # the call fails on the host before touching any tensor
    H, L, T, d = 64, 64, 32768, 128
    batch = mf.Batch([0, T], [0, T], None, 64)
    desc = mf.SenderDesc(mf.dtype_code(torch.bfloat16), L, H, H, d, 64, 0.0, T * H * d, T * H * d)
    assert mf.compress_workspace_size(desc, batch) > mf.STATIC_SCRATCH_BYTES
    x = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    rp = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(mf.MapflowError) as e:
        mf.compress_blocks_noalloc(desc, batch, x, x, rp, rp, 0.9, rp, None, None, 0)
    assert "static scratch" in str(e.value)
