"""Pins of the head-mix calibration oracle to facts outside itself (CPU only).

The least-squares fit of W is checked against numpy's own least-squares and
linear solvers on the explicit design matrix, against a planted exact
solution, against brute-force evaluation of the objective, and on the
degenerate heads its drop rule handles.  `test_planted_*` plant a plausible
mistake into the oracle and check that a pin catches it.
"""
import numpy as np
import pytest

from oracle import headmix_oracle as hm


def random_csr(rng, L, H, R, B, keep, force_empty=(), copy_of=None, base=None):
    """CSR over L layers x H heads x R causal row-blocks with random kept
    sets (probability `keep` per causal block) and random non-negative values.
    force_empty: heads that keep nothing.  copy_of {h: g}: head h copies head
    g's kept blocks and values."""
    row_ptr, cols, vals = [0], [], []
    store = {}
    for l in range(L):
        for h in range(H):
            for i in range(R):
                if copy_of and h in copy_of:
                    kc, kv = store[(l, copy_of[h], i)]
                elif h in force_empty:
                    kc, kv = [], []
                else:
                    kc = [j for j in range(i + 1) if rng.random() < keep]
                    kv = [rng.random((B, B)) for _ in kc]
                store[(l, h, i)] = (kc, kv)
                cols += kc
                vals += kv
                row_ptr.append(len(cols))
    values = np.stack(vals) if vals else np.zeros((0, B, B))
    return np.asarray(row_ptr), np.asarray(cols, dtype=np.int64), values


def design(sender, receiver, l, s, H_s, H_r, R, B):
    """Explicit least-squares design of one layer: one row per entry of every
    (row-block, column block) pair either side keeps, one column per sender
    head; right-hand sides per receiver head."""
    X_rows, Y_rows = [], []
    for i in range(R):
        sk = [hm.kept_blocks(*sender, s, h, H_s, R, i) for h in range(H_s)]
        rk = [hm.kept_blocks(*receiver, l, r, H_r, R, i) for r in range(H_r)]
        cols = sorted(set().union(*[set(m) for m in sk + rk]))
        for j in cols:
            X_rows.append(np.stack([sk[h].get(j, np.zeros(B * B)) for h in range(H_s)], 1))
            Y_rows.append(np.stack([rk[r].get(j, np.zeros(B * B)) for r in range(H_r)], 1))
    return np.concatenate(X_rows), np.concatenate(Y_rows)


def mixed_receiver(sender, Wstar, layer_map, H_s, H_r, R, B):
    """Receiver CSR that keeps the sender union, with values sum_h W*[r,h] Pt_h."""
    row_ptr, cols, vals = [0], [], []
    for l in range(len(layer_map)):
        for r in range(H_r):
            for i in range(R):
                sk = [hm.kept_blocks(*sender, layer_map[l], h, H_s, R, i) for h in range(H_s)]
                for j in sorted(set().union(*[set(m) for m in sk])):
                    v = sum(Wstar[l, r, h] * sk[h][j] for h in range(H_s) if j in sk[h])
                    cols.append(j)
                    vals.append(np.asarray(v).reshape(B, B))
                row_ptr.append(len(cols))
    return np.asarray(row_ptr), np.asarray(cols, dtype=np.int64), np.stack(vals)


def check_planted(seed=0):
    rng = np.random.default_rng(seed)
    H_s, H_r, R, B = 5, 3, 4, 4
    sender = random_csr(rng, 2, H_s, R, B, 0.7)
    Wstar = rng.standard_normal((2, H_r, H_s))
    receiver = mixed_receiver(sender, Wstar, [1, 0], H_s, H_r, R, B)
    W, dropped, _, _ = hm.fit_headmix(sender, receiver, [1, 0], H_s, H_r, R, B, 0.0)
    return not dropped.any() and np.allclose(W, Wstar, rtol=1e-9, atol=1e-9)


def check_lstsq(seed=1, lam=0.0):
    rng = np.random.default_rng(seed)
    H_s, H_r, R, B = 4, 3, 5, 3
    sender = random_csr(rng, 1, H_s, R, B, 0.6)
    receiver = random_csr(rng, 1, H_r, R, B, 0.6)   # keeps blocks outside the union too
    W, _, G, b = hm.fit_headmix(sender, receiver, [0], H_s, H_r, R, B, lam)
    X, Y = design(sender, receiver, 0, 0, H_s, H_r, R, B)
    if lam:
        X = np.concatenate([X, np.sqrt(lam) * np.eye(H_s)])
        Y = np.concatenate([Y, np.zeros((H_s, H_r))])
    ref = np.linalg.lstsq(X, Y, rcond=None)[0].T
    ok = np.allclose(W[0], ref, rtol=1e-9, atol=1e-10)
    if lam:
        ok = ok and np.allclose(W[0], np.linalg.solve(G[0] + lam * np.eye(H_s), b[0].T).T, rtol=1e-9, atol=1e-10)
    return ok


def test_planted_solution_is_recovered():
    assert check_planted()


@pytest.mark.parametrize("lam", [0.0, 0.3])
def test_fit_equals_numpy_least_squares(lam):
    assert check_lstsq(lam=lam)


def test_gram_is_the_design_products():
    rng = np.random.default_rng(2)
    H_s, H_r, R, B = 3, 2, 4, 2
    sender = random_csr(rng, 1, H_s, R, B, 0.8)
    receiver = random_csr(rng, 1, H_r, R, B, 0.8)
    G, b = hm.gram_and_cross(sender, receiver, [0], H_s, H_r, R, B)
    X, Y = design(sender, receiver, 0, 0, H_s, H_r, R, B)
    assert np.allclose(G[0], X.T @ X, rtol=1e-12) and np.allclose(b[0], Y.T @ X, rtol=1e-12)


def test_empty_and_duplicate_heads_are_dropped():
    rng = np.random.default_rng(3)
    H_s, H_r, R, B = 5, 2, 4, 3
    sender = random_csr(rng, 1, H_s, R, B, 0.7, force_empty=(2,), copy_of={4: 1})
    receiver = random_csr(rng, 1, H_r, R, B, 0.7)
    W, dropped, _, _ = hm.fit_headmix(sender, receiver, [0], H_s, H_r, R, B, 0.0)
    assert dropped[0].tolist() == [False, False, True, False, True]
    assert np.all(W[0][:, [2, 4]] == 0.0)
    X, Y = design(sender, receiver, 0, 0, H_s, H_r, R, B)
    keep = [0, 1, 3]
    ref = np.linalg.lstsq(X[:, keep], Y, rcond=None)[0].T
    assert np.allclose(W[0][:, keep], ref, rtol=1e-8, atol=1e-10)


def test_objective_is_minimal_by_brute_force():
    rng = np.random.default_rng(4)
    H_s, H_r, R, B = 3, 2, 3, 2
    sender = random_csr(rng, 1, H_s, R, B, 0.8)
    receiver = random_csr(rng, 1, H_r, R, B, 0.8)
    lam = 0.05
    W, _, _, _ = hm.fit_headmix(sender, receiver, [0], H_s, H_r, R, B, lam)
    J0 = hm.objective(sender, receiver, 0, 0, W[0], H_s, H_r, R, B, lam)
    for _ in range(20):
        d = rng.standard_normal(W[0].shape) * 1e-3
        assert hm.objective(sender, receiver, 0, 0, W[0] + d, H_s, H_r, R, B, lam) > J0
    # zero gradient: central differences of the brute-force objective
    eps = 1e-5
    for r in range(H_r):
        for h in range(H_s):
            E = np.zeros_like(W[0])
            E[r, h] = eps
            g = (hm.objective(sender, receiver, 0, 0, W[0] + E, H_s, H_r, R, B, lam)
                 - hm.objective(sender, receiver, 0, 0, W[0] - E, H_s, H_r, R, B, lam)) / (2 * eps)
            assert abs(g) < 1e-6


# ------------------------------------------ planted mistakes must fail a pin

def test_planted_ridge_on_every_entry(monkeypatch):
    real = hm.solve_headmix
    monkeypatch.setattr(hm, "solve_headmix", lambda G, b, lam: real(G + lam * (np.ones_like(G) - np.eye(G.shape[0])), b, lam))
    assert not check_lstsq(lam=0.3)


def test_planted_cross_term_of_the_wrong_receiver_head(monkeypatch):
    real = hm.gram_and_cross

    def bad(*a, **k):
        G, b = real(*a, **k)
        return G, np.roll(b, 1, axis=1)
    monkeypatch.setattr(hm, "gram_and_cross", bad)
    assert not check_planted()


def test_planted_per_head_scale_slip(monkeypatch):
    real = hm.solve_headmix

    def bad(G, b, lam):
        W, d = real(G, b, lam)
        return W * (1.0 + 1e-3 * np.arange(W.shape[1])), d   # a per-head scale slip
    monkeypatch.setattr(hm, "solve_headmix", bad)
    assert not check_lstsq()
