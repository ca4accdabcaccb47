"""Least-squares head-mix fit on the GPU vs the fp64 oracle, through the C ABI.

G and b are sums of exact fp64 products taken in another order than the
oracle's, so they agree to a few ulps of the largest entry (checked at
1e-10 relative).  W is fp32 from an fp64 solve: it is compared with the
oracle's W at a tolerance that grows with the conditioning of G + lambda I,
and through the oracle's normal equations."""
import numpy as np
import pytest
import torch

from cross_model_attention_mf_amd import mapflow as mf
from cross_model_attention_mf_amd import pipeline, synth
from oracle import headmix_oracle as hm

pytestmark = pytest.mark.gpu


def compress(wl, tau, layers):
    lay = synth.batch_layout(wl)
    xs = [synth.layer_inputs(wl, l, layout=lay) for l in layers]
    q = torch.stack([x.q for x in xs]).cuda()
    k = torch.stack([x.k for x in xs]).cuda()
    chunked = wl.chunk is not None
    batch = mf.Batch(lay.cu_seqlens_q, lay.cu_seqlens_k, lay.q_pos0 if chunked else None, wl.B)
    cap = pipeline.count_capacity(batch, q, k, wl.B, tau)
    return pipeline.compress(pipeline.alloc_sender(batch, q, k, wl.B, cap), q, k, tau)


def host_csr(st):
    return (st.row_ptr.cpu().numpy().astype(np.int64), st.col_idx[: st.nnz].cpu().numpy().astype(np.int64),
            st.values[: st.nnz].float().cpu().numpy().astype(np.float64))


def check_fit(sender, receiver, layer_map, lam, sender_host=None, receiver_host=None, state_like=None):
    W, dropped, G, b = pipeline.fit_headmix(sender, receiver, layer_map, lam)
    torch.cuda.synchronize()
    H_s, H_r = sender.desc.H_s, receiver.desc.H_s
    R, B = sender.batch.total_rowblocks, sender.B
    sh = sender_host or host_csr(sender)
    rh = receiver_host or host_csr(receiver)
    Wo, do, Go, bo = hm.fit_headmix(sh, rh, layer_map, H_s, H_r, R, B, lam)
    Gg, bg = G.cpu().numpy(), b.cpu().numpy()
    assert np.allclose(Gg, Go, rtol=0, atol=1e-10 * np.abs(Go).max())
    assert np.allclose(bg, bo, rtol=0, atol=1e-10 * max(np.abs(bo).max(), 1e-300))
    assert np.array_equal(dropped.cpu().numpy().astype(bool), do)
    Wg = W.cpu().numpy().astype(np.float64)
    for l in range(len(layer_map)):
        keep = ~do[l]
        M = Go[l][np.ix_(keep, keep)] + lam * np.eye(int(keep.sum()))
        cond = np.linalg.cond(M) if keep.any() else 1.0
        tol = max(1e-6, cond * 1e-13) * max(np.abs(Wo[l]).max(), 1e-30)
        assert np.abs(Wg[l] - Wo[l]).max() <= tol, (l, cond, np.abs(Wg[l] - Wo[l]).max(), tol)
        res = (Go[l] + lam * np.eye(H_s)) @ Wg[l].T - bo[l].T
        # fp32 rounding of W (6e-8 relative) moves the residual by at most ~cond times that
        assert np.abs(res[keep]).max() <= 1e-6 * max(1.0, cond) * max(np.abs(bo[l]).max(), 1e-30)
    return W, dropped


@pytest.mark.parametrize("dtype,B,d", [("f32", 32, 64), ("bf16", 64, 128), ("bf16", 128, 64)])
def test_fit_on_compressed_maps_matches_oracle(dtype, B, d):
    seqlens = (3 * B + 17, B + 5, 2 * B)
    sw = synth.Workload(name="hm_sender", workload_id=41, dtype=dtype, H_s=6, H_r=5, d=d, B=B, taus=(0.9,),
                        seqlens=seqlens, num_layers=2, w_var=0.5)
    rw = synth.Workload(name="hm_receiver", workload_id=42, dtype=dtype, H_s=5, H_r=5, d=d, B=B, taus=(0.9,),
                        seqlens=seqlens, num_layers=3, w_var=0.5)
    sender = compress(sw, 0.9, [0, 1])
    receiver = compress(rw, 0.95, [0, 1, 2])
    for lam in (0.0, 1e-3):
        check_fit(sender, receiver, [1, 0, 1], lam)


def test_fit_on_varlen_chunked_batch():
    wl = synth.Workload(name="hm_chunked", workload_id=43, dtype="bf16", H_s=8, H_r=4, d=64, B=64, taus=(0.9,),
                        seqlens=(700, 130, 64 * 9 + 1), num_layers=1, chunk=256, w_var=0.5)
    rwl = wl.replace(workload_id=44, H_s=4)
    lay = synth.batch_layout(wl, 1)
    def comp(w, tau):
        xs = [synth.layer_inputs(w, 0, 1, lay)]
        q = torch.stack([x.q for x in xs]).cuda(); k = torch.stack([x.k for x in xs]).cuda()
        batch = mf.Batch(lay.cu_seqlens_q, lay.cu_seqlens_k, lay.q_pos0, w.B)
        cap = pipeline.count_capacity(batch, q, k, w.B, tau)
        return pipeline.compress(pipeline.alloc_sender(batch, q, k, w.B, cap), q, k, tau)
    check_fit(comp(wl, 0.9), comp(rwl, 0.8), [0], 0.0)


def to_state(like, csr, H, L, values_dtype):
    """A SenderState-shaped holder of a host CSR on the device (batch of `like`)."""
    import dataclasses
    rp, ci, vals = csr
    dev = torch.device("cuda")
    st = dataclasses.replace(like, row_ptr=torch.from_numpy(rp.astype(np.int32)).to(dev),
                             col_idx=torch.from_numpy(ci.astype(np.int32)).to(dev),
                             values=torch.from_numpy(vals).to(values_dtype).to(dev), nnz=len(ci))
    st.desc = type(like.desc)(*[getattr(like.desc, f) for f, _ in like.desc._fields_])
    st.desc.H_s = H
    st.desc.num_layers = L
    return st


def random_causal_csr(rng, L, H, R, B, keep, empty=(), copy_of=None):
    row_ptr, cols, vals, store = [0], [], [], {}
    for l in range(L):
        for h in range(H):
            for i in range(R):
                if copy_of and h in copy_of:
                    kc, kv = store[(l, copy_of[h], i)]
                elif h in empty:
                    kc, kv = [], []
                else:
                    kc = [j for j in range(i + 1) if rng.random() < keep] or [i]
                    kv = [rng.random((B, B)).astype(np.float32).astype(np.float64) for _ in kc]
                store[(l, h, i)] = (kc, kv)
                cols += kc
                vals += kv
                row_ptr.append(len(cols))
    return np.asarray(row_ptr), np.asarray(cols), np.stack(vals)


def test_planted_mix_is_recovered_and_degenerate_heads_dropped():
    rng = np.random.default_rng(7)
    B, R, H_s, H_r = 32, 6, 7, 4
    batch = mf.Batch([0, R * B], [0, R * B], None, B)
    q = torch.zeros((1, R * B, H_s, 64), dtype=torch.float32, device="cuda")
    like = pipeline.alloc_sender(batch, q, q, B, 1)
    # head 3 keeps nothing, head 6 repeats head 2
    sender = random_causal_csr(rng, 2, H_s, R, B, 0.6, empty=(3,), copy_of={6: 2})
    Wstar = rng.standard_normal((2, H_r, H_s))
    Wstar[:, :, [3, 6]] = 0.0
    # receiver maps: the planted mix of the sender maps on the union, in fp32
    rp, cols, vals = [0], [], []
    for l in range(2):
        for r in range(H_r):
            for i in range(R):
                sk = [hm.kept_blocks(*sender, l, h, H_s, R, i) for h in range(H_s)]
                for j in sorted(set().union(*[set(m) for m in sk])):
                    v = sum(Wstar[l, r, h] * sk[h][j] for h in range(H_s) if j in sk[h])
                    cols.append(j)
                    vals.append(np.asarray(v, dtype=np.float32).astype(np.float64).reshape(B, B))
                rp.append(len(cols))
    receiver = (np.asarray(rp), np.asarray(cols), np.stack(vals))
    s_st = to_state(like, sender, H_s, 2, torch.float32)
    r_st = to_state(like, receiver, H_r, 2, torch.float32)
    W, dropped = check_fit(s_st, r_st, [0, 1], 0.0, sender, receiver)
    assert dropped.cpu().numpy().tolist() == [[0, 0, 0, 1, 0, 0, 1]] * 2
    Wg = W.cpu().numpy()
    assert np.all(Wg[:, :, [3, 6]] == 0.0)
    # head 6 duplicates head 2: the fit puts their combined weight on head 2
    want = Wstar.copy()
    want[:, :, 2] += Wstar[:, :, 6]
    assert np.allclose(Wg, want, rtol=1e-4, atol=1e-4)


def test_full_size_two_layers_of_the_8k_workload():
    W3 = synth.standard_workloads()[2]
    sender = compress(W3, 0.95, [0, 1])
    rwl = W3.replace(workload_id=45, H_s=W3.H_r)
    receiver = compress(rwl, 0.95, [0, 1])
    check_fit(sender, receiver, [0, 1], 1e-6)


def test_repeat_calls_are_bit_identical():
    sw = synth.Workload(name="hm_rep", workload_id=46, dtype="bf16", H_s=12, H_r=8, d=64, B=64, taus=(0.9,),
                        seqlens=(900,), num_layers=1, w_var=0.5)
    s = compress(sw, 0.9, [0])
    r = compress(sw.replace(workload_id=47, H_s=8), 0.9, [0])
    a = pipeline.fit_headmix(s, r, [0], 0.0)
    b = pipeline.fit_headmix(s, r, [0], 0.0)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("H_s,H_r", [(40, 24), (64, 64), (1, 1)])
def test_fit_with_wide_and_single_heads(H_s, H_r):
    """Several 16 x 16 output tiles per wave (up to 8 for 64 + 64 heads) and
    the one-head extreme."""
    seqlens = (5 * 32 + 7, 40)
    sw = synth.Workload(name="hm_wide_s", workload_id=48, dtype="bf16", H_s=H_s, H_r=4, d=64, B=32,
                        taus=(0.9,), seqlens=seqlens, num_layers=1, w_var=0.5)
    rw = sw.replace(workload_id=49, H_s=H_r)
    sender = compress(sw, 0.9, [0])
    receiver = compress(rw, 0.9, [0])
    check_fit(sender, receiver, [0], 1e-4)
