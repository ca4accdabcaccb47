"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or the mathematics
fix: library routines (scipy softmax/logsumexp, torch SDPA in float64),
closed-form identities (tau = 1 and W = I gives dense causal attention),
invariants (masses sum to 1, linearity in W, head permutation), brute force
over every subset on tiny inputs, and hand-derived golden cases.  The
`test_planted_*` tests plant a plausible mistake into the oracle and check
that at least one pin catches it.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import mapflow_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "selection_cases.json")


def rand_qkv(rng, T, H, Hkv, d, Hr=None, Hkv_r=None, scale_bias=0.0):
    q = rng.standard_normal((T, H, d))
    k = rng.standard_normal((T, Hkv, d))
    if scale_bias:
        # give some structure so the maps are far from uniform
        q[:, :, 0] = scale_bias
        k[:, :, 0] = rng.standard_normal(T)[:, None] * scale_bias
    v = rng.standard_normal((T, Hkv_r or Hr or H, d))
    return q, k, v


def sdpa_reference(q, k, v, cu_q, cu_k, q_pos0, Hr_map=None):
    """Dense causal attention per sequence via torch's SDPA in float64 (CPU).
    q [Tq,H,d], k [Tk,Hkv,d], v [Tk,Hkv_v,d]; head h uses k head h//(H/Hkv) and
    v head h//(H/Hkv_v)."""
    H, d = q.shape[1], q.shape[2]
    out = np.zeros((q.shape[0], H, v.shape[2]))
    for s in range(len(cu_q) - 1):
        a, b = cu_q[s], cu_q[s + 1]
        ka, kb = cu_k[s], cu_k[s + 1]
        p0 = 0 if q_pos0 is None else q_pos0[s]
        qq = torch.from_numpy(q[a:b]).permute(1, 0, 2)[None]
        kk = torch.from_numpy(np.repeat(k[ka:kb], H // k.shape[1], axis=1)).permute(1, 0, 2)[None]
        vv = torch.from_numpy(np.repeat(v[ka:kb], H // v.shape[1], axis=1)).permute(1, 0, 2)[None]
        pos = p0 + torch.arange(b - a)
        mask = torch.arange(kb - ka)[None, :] <= pos[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        out[a:b] = o[0].permute(1, 0, 2).numpy()
    return out


def run_oracle(q, k, v, W, cu_q, cu_k, q_pos0, B, tau):
    lc = orc.compress_layer(q, k, cu_q, cu_k, q_pos0, B, tau)
    return lc, orc.mapped_layer(lc, W, v, q.shape[0], B)


# ---------------------------------------------------------------- pins: softmax

def check_softmax_vs_scipy(seed=0):
    rng = np.random.default_rng(seed)
    R, n, d = 7, 40, 16
    q = rng.standard_normal((R, d)) * 2
    k = rng.standard_normal((n, d))
    pos = np.array([3, 10, 11, 20, 33, 38, 39])
    P, lse = orc.causal_probs(q, k, pos, orc.default_scale(d))
    ok = True
    for r in range(R):
        s = (q[r] @ k[: pos[r] + 1].T) / math.sqrt(d)
        ok &= np.allclose(P[r, : pos[r] + 1], scipy.special.softmax(s), rtol=1e-12, atol=1e-15)
        ok &= np.all(P[r, pos[r] + 1:] == 0)
        ok &= abs(lse[r] - scipy.special.logsumexp(s)) < 1e-12
    return ok


def test_softmax_matches_scipy():
    assert check_softmax_vs_scipy()


def test_rows_sum_to_one():
    rng = np.random.default_rng(1)
    q, k, _ = rand_qkv(rng, 50, 2, 2, 8, scale_bias=3.0)
    P, _ = orc.dense_map(q, k, 1)
    assert np.allclose(P.sum(1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.triu(P, 1) == 0)


# ------------------------------------------------------------ pins: block mass

def check_block_mass_bruteforce(seed=2, B=4):
    rng = np.random.default_rng(seed)
    n = 18
    q, k, _ = rand_qkv(rng, n, 1, 1, 6, scale_bias=2.0)
    P_full = np.zeros((n, n))
    for r in range(n):  # library softmax row by row
        P_full[r, : r + 1] = scipy.special.softmax(q[r, 0] @ k[: r + 1, 0].T / math.sqrt(6))
    lc = orc.compress_layer(q, k, [0, n], [0, n], None, B, 1.0)
    ok = True
    for rb in lc.rowblocks:
        m = lc.units[(0, rb.index)].sel.masses
        ok &= m.shape[0] == rb.last_pos // B + 1
        for j in range(m.shape[0]):
            tot = 0.0
            for r in range(rb.pos0, rb.pos0 + rb.rows):
                for c in range(j * B, min(n, (j + 1) * B)):
                    tot += P_full[r, c]
            ok &= abs(m[j] - tot / rb.rows) < 1e-14
        ok &= abs(m.sum() - 1.0) < 1e-14
    return ok


def test_block_mass_bruteforce():
    assert check_block_mass_bruteforce()


def test_masses_sum_to_one_structured():
    rng = np.random.default_rng(3)
    q, k, _ = rand_qkv(rng, 300, 3, 1, 16, scale_bias=4.0)
    lc = orc.compress_layer(q, k, [0, 300], [0, 300], None, 32, 0.9)
    for u in lc.units.values():
        assert abs(u.sel.masses.sum() - 1.0) < 1e-13


# ------------------------------------------------------------- pins: selection

def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def check_golden():
    for c in load_golden():
        sel = orc.select_blocks(np.asarray(c["masses"], dtype=np.float64), c["tau"])
        if list(sel.kept) != c["kept"]:
            return False
    return True


def test_selection_golden():
    for c in load_golden():
        sel = orc.select_blocks(np.asarray(c["masses"], dtype=np.float64), c["tau"])
        assert list(sel.kept) == c["kept"], c["name"]


def check_selection_bruteforce(seed=4, trials=60):
    """The kept set has the minimum size among all subsets reaching tau, and
    among those the maximum mass (greedy by mass is optimal for this)."""
    rng = np.random.default_rng(seed)
    for t in range(trials):
        n = int(rng.integers(1, 11))
        m = rng.dirichlet(np.full(n, 0.4))
        tau = float(rng.choice([0.3, 0.5, 0.8, 0.9, 0.95, 0.99]))
        sel = orc.select_blocks(m, tau)
        best_size, best_mass = None, -1.0
        for size in range(1, n + 1):
            masses = [sum(m[list(c)]) for c in itertools.combinations(range(n), size)]
            reach = [x for x in masses if x >= tau]
            if reach:
                best_size, best_mass = size, max(reach)
                break
        if best_size is None:
            best_size, best_mass = n, m.sum()
        if len(sel.kept) != best_size or abs(m[sel.kept].sum() - best_mass) > 1e-12:
            return False
    return True


def test_selection_bruteforce():
    assert check_selection_bruteforce()


def test_tau_nesting_and_tau_one():
    rng = np.random.default_rng(5)
    q, k, _ = rand_qkv(rng, 256, 2, 2, 16, scale_bias=3.0)
    taus = [0.3, 0.6, 0.9, 0.99, 1.0]
    lcs = [orc.compress_layer(q, k, [0, 256], [0, 256], None, 32, t) for t in taus]
    for key in lcs[0].units:
        sets = [set(lc.units[key].sel.kept.tolist()) for lc in lcs]
        for a, b in zip(sets, sets[1:]):
            assert a <= b
        rb = lcs[0].rowblocks[key[1]]
        assert sets[-1] == set(range(rb.last_pos // 32 + 1))


def test_accept_set_window():
    m = np.array([0.5, 0.3, 0.2 - 5e-7, 5e-7])
    sel = orc.select_blocks(m, 0.8)
    assert list(sel.kept) == [0, 1]
    ok, n, bad = orc.accept_set(sel, [0, 1, 2], eps=1e-6)   # cumulative 0.8 == tau: cut ambiguous
    assert ok and n == 1
    ok, n, bad = orc.accept_set(sel, [0], eps=1e-6)
    assert not ok and bad == [1]
    # swap of two near-equal masses across the cut
    m2 = np.array([0.4, 0.3, 0.15 + 4e-7, 0.15 - 4e-7])
    sel2 = orc.select_blocks(m2, 0.8)
    assert list(sel2.kept) == [0, 1, 2]
    assert orc.accept_set(sel2, [0, 1, 3])[0]
    assert not orc.accept_set(sel2, [0, 2, 3])[0]


# ---------------------------------------------------- pins: mapped output, SDPA

def check_sdpa_identity(seed=6, gqa=False, chunked=False):
    rng = np.random.default_rng(seed)
    H, Hkv, d, B = 4, (2 if gqa else 4), 16, 16
    lens = [70, 33, 128]
    if chunked:
        # second chunk of each sequence: rows [32, len)
        p0 = [32, 0, 64]
    else:
        p0 = [0, 0, 0]
    qs, ks, vs, cu_q, cu_k = [], [], [], [0], [0]
    for n, a in zip(lens, p0):
        q, k, v = rand_qkv(rng, n, H, Hkv, d, Hkv_r=Hkv, scale_bias=2.5)
        qs.append(q[a:]); ks.append(k); vs.append(v)
        cu_q.append(cu_q[-1] + n - a); cu_k.append(cu_k[-1] + n)
    q, k, v = np.concatenate(qs), np.concatenate(ks), np.concatenate(vs)
    W = np.eye(H)
    _, O = run_oracle(q, k, v, W, cu_q, cu_k, p0, B, 1.0)
    ref = sdpa_reference(q, k, v, cu_q, cu_k, p0)
    return np.allclose(O, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("gqa,chunked", [(False, False), (True, False), (False, True), (True, True)])
def test_tau1_identity_equals_sdpa(gqa, chunked):
    assert check_sdpa_identity(gqa=gqa, chunked=chunked)


def test_linear_in_W_and_onehot_and_permutation():
    rng = np.random.default_rng(7)
    Hs, Hr, d, B, T = 4, 3, 16, 16, 96
    q, k, _ = rand_qkv(rng, T, Hs, Hs, d, scale_bias=3.0)
    v = rng.standard_normal((T, Hr, d))
    W1 = rng.standard_normal((Hr, Hs)); W2 = rng.standard_normal((Hr, Hs))
    lc = orc.compress_layer(q, k, [0, T], [0, T], None, B, 0.8)
    O = lambda W, lc=lc: orc.mapped_layer(lc, W, v, T, B)
    assert np.allclose(O(W1 + 0.7 * W2), O(W1) + 0.7 * O(W2), atol=1e-12)
    # one-hot row: O_r = (P restricted to head h's kept blocks) V_r
    Wh = np.zeros((Hr, Hs)); Wh[1, 2] = 1.0
    Oh = O(Wh)
    P, _ = orc.dense_map(q, k, 2)
    Pk = np.zeros_like(P)
    for rb in lc.rowblocks:
        for j in lc.units[(2, rb.index)].sel.kept:
            rows = slice(rb.pos0, rb.pos0 + rb.rows)
            Pk[rows, j * B:(j + 1) * B] = P[rows, j * B:(j + 1) * B]
    assert np.allclose(Oh[:, 1, :], Pk @ v[:, 1, :], atol=1e-12)
    assert np.all(Oh[:, [0, 2], :] == 0)
    # permuting sender heads together with W's columns changes nothing
    perm = np.array([2, 0, 3, 1])
    lcp = orc.compress_layer(q[:, perm], k[:, perm], [0, T], [0, T], None, B, 0.8)
    assert np.allclose(orc.mapped_layer(lcp, W1[:, perm], v, T, B), O(W1), atol=1e-12)


def test_values_equal_dense_entries():
    rng = np.random.default_rng(8)
    q, k, _ = rand_qkv(rng, 200, 2, 2, 16, scale_bias=3.0)
    B = 32
    lc = orc.compress_layer(q, k, [0, 200], [0, 200], None, B, 0.7)
    for h in range(2):
        P, lse = orc.dense_map(q, k, h)
        for rb in lc.rowblocks:
            u = lc.units[(h, rb.index)]
            assert np.allclose(u.lse, lse[rb.pos0: rb.pos0 + rb.rows], atol=1e-13)
            for t, j in enumerate(u.sel.kept):
                blk = np.zeros((B, B))
                part = P[rb.pos0: rb.pos0 + rb.rows, j * B:(j + 1) * B]
                blk[: part.shape[0], : part.shape[1]] = part
                assert np.allclose(u.values[t], blk, rtol=1e-12, atol=1e-16)


# ------------------------------------------------------- pins: layout variants

def test_varlen_equals_per_sequence_and_chunked_equals_whole():
    rng = np.random.default_rng(9)
    H, d, B = 2, 16, 16
    lens = [45, 100, 64]
    seqs = [rand_qkv(rng, n, H, H, d, scale_bias=3.0) for n in lens]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = np.concatenate([s[0] for s in seqs]); k = np.concatenate([s[1] for s in seqs])
    v = np.concatenate([s[2] for s in seqs])
    W = rng.standard_normal((H, H))
    _, Opacked = run_oracle(q, k, v, W, cu, cu, None, B, 0.85)
    for s, n in enumerate(lens):
        _, Os = run_oracle(seqs[s][0], seqs[s][1], seqs[s][2], W, [0, n], [0, n], None, B, 0.85)
        assert np.allclose(Opacked[cu[s]:cu[s + 1]], Os, atol=1e-13)
    # chunked: rows [48, 100) of sequence 1 against its full prefix
    q1, k1, v1 = seqs[1]
    lc_whole = orc.compress_layer(q1, k1, [0, 100], [0, 100], None, B, 0.85)
    _, Ow = run_oracle(q1, k1, v1, W, [0, 100], [0, 100], None, B, 0.85)
    lc_chunk = orc.compress_layer(q1[48:], k1, [0, 52], [0, 100], [48], B, 0.85)
    _, Oc = run_oracle(q1[48:], k1, v1, W, [0, 52], [0, 100], [48], B, 0.85)
    assert np.allclose(Oc, Ow[48:], atol=1e-13)
    for rb in lc_chunk.rowblocks:
        whole_index = rb.local + 3
        for h in range(H):
            assert np.array_equal(lc_chunk.kept(h, rb.index), lc_whole.kept(h, whole_index))


def test_paged_gather_equals_contiguous():
    rng = np.random.default_rng(10)
    lens = [37, 16, 50]
    cu = np.concatenate([[0], np.cumsum(lens)])
    v = rng.standard_normal((cu[-1], 2, 4))
    ps = 16
    npages = [math.ceil(n / ps) for n in lens]
    perm = rng.permutation(sum(npages))
    pool = np.zeros((sum(npages), ps, 2, 4))
    table = np.full((3, max(npages)), -1)
    nxt = 0
    for s, n in enumerate(lens):
        for p in range(npages[s]):
            table[s, p] = perm[nxt]; nxt += 1
            seg = v[cu[s] + p * ps: cu[s] + min(n, (p + 1) * ps)]
            pool[table[s, p], : seg.shape[0]] = seg
    assert np.array_equal(orc.gather_paged(pool, table, cu, ps), v)


# ------------------------------------------ planted mistakes must fail a pin

def _with(monkeypatch, name, fn):
    monkeypatch.setattr(orc, name, fn)


def test_planted_wrong_scale(monkeypatch):
    _with(monkeypatch, "default_scale", lambda d: 1.0 / d)
    assert not check_sdpa_identity()


def test_planted_causal_off_by_one(monkeypatch):
    real = orc.causal_probs

    def bad(q_rows, k_keys, pos_rows, scale):
        return real(q_rows, k_keys, np.maximum(pos_rows - 1, 0), scale)
    _with(monkeypatch, "causal_probs", bad)
    assert not check_sdpa_identity()


def test_planted_reversed_keys(monkeypatch):
    real = orc.causal_probs
    _with(monkeypatch, "causal_probs",
          lambda q_rows, k_keys, pos_rows, scale: real(q_rows, k_keys[::-1].copy(), pos_rows, scale))
    assert not (check_softmax_vs_scipy() and check_sdpa_identity())


def test_planted_unnormalised_mass(monkeypatch):
    real = orc.block_masses
    _with(monkeypatch, "block_masses", lambda P, B, n: real(P, B, n) * P.shape[0])
    assert not check_block_mass_bruteforce()


def test_planted_tie_order(monkeypatch):
    _with(monkeypatch, "selection_order",
          lambda m: np.lexsort((-np.arange(m.shape[0]), -m)))
    assert not check_golden()


def test_planted_strict_cut(monkeypatch):
    def bad(m, tau):
        order = orc.selection_order(m)
        cum = np.concatenate([[0.0], np.cumsum(m[order])])
        reach = np.nonzero(cum[1:] > tau)[0]
        kstar = int(reach[0]) + 1 if reach.size else m.shape[0]
        return orc.Selection(m, order, cum, kstar, tau)
    _with(monkeypatch, "select_blocks", bad)
    assert not check_golden()


def test_planted_ascending_mass_order(monkeypatch):
    _with(monkeypatch, "selection_order", lambda m: np.lexsort((np.arange(m.shape[0]), m)))
    assert not (check_golden() and check_selection_bruteforce())


def test_planted_wrong_kv_group(monkeypatch):
    _with(monkeypatch, "kv_head", lambda h, H, Hkv: h % Hkv)
    assert not check_sdpa_identity(gqa=True)


def check_dense_mix(seed=11):
    """tau = 1 keeps every causal block, so O_r = (sum_h W[r,h] P_h) V_r with
    the dense maps P_h (computed here with scipy's softmax)."""
    rng = np.random.default_rng(seed)
    T, H, d = 64, 3, 8
    q, k, v = rand_qkv(rng, T, H, H, d, scale_bias=2.0)
    W = rng.standard_normal((H, H))
    lc = orc.compress_layer(q, k, [0, T], [0, T], None, 16, 1.0)
    O = orc.mapped_layer(lc, W, v, T, 16)
    Ps = []
    for h in range(H):
        P = np.zeros((T, T))
        for r in range(T):
            P[r, : r + 1] = scipy.special.softmax(q[r, h] @ k[: r + 1, h].T / math.sqrt(d))
        Ps.append(P)
    ref = np.zeros_like(O)
    for r in range(H):
        ref[:, r] = sum(W[r, h] * Ps[h] for h in range(H)) @ v[:, r]
    return np.allclose(O, ref, rtol=1e-11, atol=1e-12)


def test_tau1_general_W_equals_dense_mix():
    assert check_dense_mix()


def test_planted_transposed_W(monkeypatch):
    real = orc.mapped_rowblock
    _with(monkeypatch, "mapped_rowblock",
          lambda kept_vals, W, v, rb, B: real(kept_vals, W.T.copy(), v, rb, B))
    assert not check_dense_mix()


def test_planted_renormalised_values(monkeypatch):
    real = orc.extract_blocks

    def bad(P, kept, B):
        vals = real(P, kept, B)
        tot = vals.sum(axis=(0, 2), keepdims=True)
        return np.where(tot > 0, vals / np.where(tot > 0, tot, 1), 0)
    _with(monkeypatch, "extract_blocks", bad)
    with pytest.raises(AssertionError):
        test_values_equal_dense_entries()


# ---- block keys of the prefix cache (FNV-1a 64, chained per block)

def test_fnv1a_64_published_vectors():
    # test vectors published with the FNV reference description
    from oracle import prefix_hash_oracle as ph
    assert ph.fnv1a_64(b"") == 0xCBF29CE484222325
    assert ph.fnv1a_64(b"a") == 0xAF63DC4C8601EC8C
    assert ph.fnv1a_64(b"foobar") == 0x85944171F73967E8


def test_prefix_block_keys_depend_on_the_prefix_only():
    from oracle import prefix_hash_oracle as ph
    rng = np.random.default_rng(3)
    toks = rng.integers(0, 50000, size=8 * 16).tolist()
    keys = ph.prefix_block_keys(toks, 16)
    assert len(keys) == 8 and len(set(keys)) == 8
    # a token changed in block 5 changes keys 5.. and no earlier one
    t2 = list(toks)
    t2[5 * 16 + 3] += 1
    k2 = ph.prefix_block_keys(t2, 16)
    assert k2[:5] == keys[:5] and all(a != b for a, b in zip(k2[5:], keys[5:]))
    # the first key is FNV-1a of eight zero bytes and the block's tokens
    data = (0).to_bytes(8, "little") + b"".join(int(t).to_bytes(4, "little") for t in toks[:16])
    assert keys[0] == ph.fnv1a_64(data)
    # a trailing partial block gets no key
    assert len(ph.prefix_block_keys(toks[:16 * 3 + 5], 16)) == 3


# ------------------------------------------------ pins: CSR order of a layer

def _hand_layer():
    """Two sender heads x three row-blocks of 32 rows with kept sets chosen by
    hand; every value of block t of (head h, row-block i) is 100 h + 10 i + t,
    so the position of each block in the CSR shows which unit it came from."""
    B = 32
    kept = {(0, 0): [0], (0, 1): [0, 1], (0, 2): [0, 2],
            (1, 0): [0], (1, 1): [1], (1, 2): [0, 1, 2]}
    rbs = orc.enumerate_rowblocks([0, 96], [0, 96], None, B)
    units = {}
    for (h, i), ks in kept.items():
        n = i + 1
        rest = [j for j in range(n) if j not in ks]
        sel = orc.Selection(np.zeros(n), np.asarray(ks + rest), np.zeros(n + 1), len(ks), 0.5)
        vals = np.stack([np.full((B, B), 100.0 * h + 10 * i + t) for t in range(len(ks))])
        units[(h, i)] = orc.UnitResult(np.zeros(B), sel, vals)
    return orc.LayerCompression(rbs, units)


# The library numbers CSR row (layer l, head h, row-block i) as
# (l * H_s + h) * total_rowblocks + i: head-major, row-blocks fastest.  For the
# hand layer above that order is (0,0) (0,1) (0,2) (1,0) (1,1) (1,2).
HAND_ROW_PTR = [0, 1, 3, 5, 6, 7, 10]
HAND_COL_IDX = [0, 0, 1, 0, 2, 0, 1, 0, 1, 2]
HAND_MARKERS = [0, 10, 11, 20, 21, 100, 110, 120, 121, 122]


def check_csr_order():
    row_ptr, col_idx, values = orc.csr_of(_hand_layer(), 2)
    return (row_ptr.tolist() == HAND_ROW_PTR and col_idx.tolist() == HAND_COL_IDX
            and values[:, 0, 0].tolist() == HAND_MARKERS
            and bool(np.all(values == values[:, :1, :1])))


def test_csr_of_is_head_major_with_ascending_columns():
    assert check_csr_order()


def test_planted_rowblock_major_csr(monkeypatch):
    def bad(lc, H_s):
        nrb = len(lc.rowblocks)
        row_ptr = np.zeros(H_s * nrb + 1, dtype=np.int64)
        cols, vals = [], []
        r = 0
        for i in range(nrb):
            for h in range(H_s):
                u = lc.units[(h, i)]
                row_ptr[r + 1] = row_ptr[r] + u.sel.kstar
                r += 1
                cols.append(u.sel.kept)
                vals.append(u.values)
        return row_ptr, np.concatenate(cols), np.concatenate(vals)
    _with(monkeypatch, "csr_of", bad)
    assert not check_csr_order()
