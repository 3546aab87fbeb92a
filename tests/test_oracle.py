"""Pins for the CPU oracle: each check ties it to something other than itself.

Sources: POET-X summary page (arXiv 2603.05500 digest), Method §1 (eq. 3,
input-centric chain), §2 (permutation merge), §3 (block-diagonal products),
§4 (Cayley-Neumann parameterization, eq. 9, packed upper triangle), §5 (the
intermediates a, b, z), §6 (POET-XQ, dequantize inside the product); the
background section (W_RP = R W0 P keeps the singular values of W0).

What pins what:
  * CNP forward: Q = 0 gives I; the page's product form (I+Q)(I+sum Q^i) equals
    eq. 9; closed form G^T G = (I - Q^4)^2; G = Cayley(Q)(I - Q^4) with the
    Cayley transform from a LAPACK solve; hand-worked b = 2 fixture.
  * CNP backward: hand-worked b = 2 fixture; central differences; the
    directional-derivative identity; Q = 0 closed form.
  * merge + layer forward: an independently assembled dense P^T W R^T with
    explicit permutation matrices (unmerged, four permutations); theta = 0
    reduces to a plain linear layer checked against a library matmul.
  * layer backward: central differences on theta_R, theta_P and X; theta = 0
    closed forms.
  * int8: merge is exact; theta = 0 equals X (diag(s) q)^T.
  * spectrum: singular values of the effective weight match W's to O(|Q|^4).
  * phase-end fold: X W_eff^T equals the dense unmerged layer; with theta = 0 the
    fold undoes the merge exactly.
  * optimizer on packed theta: the closed-form first Adam step and three steps of
    the library optimizer (torch.optim.Adam).
  * blocks of unequal size (ceil(d/b) blocks, the last one smaller): the dense
    unmerged layer built with the library's block_diag from blocks that the test
    slices out of the flat theta itself; central differences on theta and X;
    divisible widths reduce exactly to the [n][p] layout.
  * a mutation test plants plausible mistakes in a copy of the oracle and
    checks that some pin above fails for each.
"""

import os

import numpy as np
import pytest
import scipy.linalg as sla

from oracle import poetx_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def rand_theta(n, b, std, rng=RNG):
    return rng.standard_normal((n, O.packed_size(b))) * std


def perm_matrix(perm):
    """Psi with (Psi x)[i] = x[perm[i]]."""
    d = len(perm)
    M = np.zeros((d, d))
    M[np.arange(d), perm] = 1.0
    return M


# ---------------------------------------------------------------- packing ----

def test_packed_count_and_skew():
    for b in (2, 3, 8, 32, 256):
        assert O.packed_size(b) == b * (b - 1) // 2
    th = rand_theta(3, 6, 1.0)
    Q = O.skew_from_packed(th, 6)
    np.testing.assert_array_equal(Q, -np.swapaxes(Q, 1, 2))
    assert np.all(np.diagonal(Q, axis1=1, axis2=2) == 0)
    # row-major strict upper triangle (a convention the page leaves open)
    k = 0
    for i in range(6):
        for j in range(i + 1, 6):
            assert Q[1, i, j] == th[1, k]
            k += 1


# ------------------------------------------------------------ CNP forward ----

def _check_cnp_forward(cnp_forward):
    """All forward pins; returns None or raises AssertionError."""
    b = 16
    # Q = 0 -> identity, bit for bit
    G0 = cnp_forward(np.zeros((2, O.packed_size(b))), b)
    assert np.array_equal(G0, np.broadcast_to(np.eye(b), (2, b, b)))
    th = rand_theta(4, b, 0.05)
    Q = O.skew_from_packed(th, b)
    G = cnp_forward(th, b)
    I = np.eye(b)
    # the page's product form (I + Q)(I + Q + Q^2 + Q^3)
    prod = np.stack([(I + q) @ (I + q + q @ q + q @ q @ q) for q in Q])
    np.testing.assert_allclose(G, prod, rtol=0, atol=1e-13)
    # closed form G^T G = (I - Q^4)^2
    for g, q in zip(G, Q):
        q4 = np.linalg.matrix_power(q, 4)
        np.testing.assert_allclose(g.T @ g, (I - q4) @ (I - q4), rtol=0, atol=1e-13)
        # Cayley transform by a LAPACK solve: C = (I + Q)(I - Q)^-1, G = C (I - Q^4)
        C = np.linalg.solve((I - q).T, (I + q).T).T
        np.testing.assert_allclose(g, C @ (I - q4), rtol=0, atol=1e-13)
    # b = 2 hand-worked fixture
    rows = np.loadtxt(os.path.join(GOLDEN, "cnp_b2.txt"))
    for r in rows:
        g = cnp_forward(np.array([[r[0]]]), 2)[0]
        np.testing.assert_allclose(g.ravel(), r[1:5], rtol=0, atol=1e-15)


def test_cnp_forward_pins():
    _check_cnp_forward(O.cnp_forward)


def test_cnp_orthogonality_error_shrinks_with_q():
    """|G^T G - I| = |Q^8 - 2Q^4|: halving Q cuts it about 16x (Method §4: G is only
    approximately orthogonal; the error is governed by the dropped series terms)."""
    b = 64
    th = rand_theta(3, b, 0.02)
    errs = []
    for s in (1.0, 0.5, 0.25):
        G = O.cnp_forward(th * s, b)
        errs.append(max(np.linalg.norm(g.T @ g - np.eye(b)) for g in G))
    assert errs[0] > errs[1] > errs[2]
    assert 10.0 < errs[0] / errs[1] < 20.0
    assert 10.0 < errs[1] / errs[2] < 20.0


# ----------------------------------------------------------- CNP backward ----

def _check_cnp_backward(cnp_forward, cnp_backward):
    # hand-worked b = 2
    rows = np.loadtxt(os.path.join(GOLDEN, "cnp_b2.txt"))
    for r in rows:
        d = cnp_backward(np.array([[r[0]]]), r[5:9].reshape(1, 2, 2), 2)
        np.testing.assert_allclose(d[0, 0], r[9], rtol=0, atol=1e-13)
    b = 8
    rng = np.random.default_rng(7)
    th = rand_theta(2, b, 0.2, rng)
    Gbar = rng.standard_normal((2, b, b))
    d = cnp_backward(th, Gbar, b)
    # central differences of L(theta) = <Gbar, G(theta)>
    h = 1e-6
    fd = np.zeros_like(th)
    for n in range(th.shape[0]):
        for k in range(th.shape[1]):
            tp = th.copy(); tp[n, k] += h
            tm = th.copy(); tm[n, k] -= h
            fd[n, k] = (np.sum(Gbar[n] * cnp_forward(tp, b)[n]) - np.sum(Gbar[n] * cnp_forward(tm, b)[n])) / (2 * h)
    np.testing.assert_allclose(d, fd, rtol=0, atol=1e-8)
    # directional identity <Gbar, DG(Q)[E]> = sum_k dtheta_k e_k with E skew from packed e
    e = rng.standard_normal(th.shape)
    E = O.skew_from_packed(e, b)
    Q = O.skew_from_packed(th, b)
    for n in range(2):
        q, E_ = Q[n], E[n]
        q2, q3 = q @ q, q @ q @ q
        DG = 2 * E_ + 2 * (q @ E_ + E_ @ q) + 2 * (q2 @ E_ + q @ E_ @ q + E_ @ q2) \
            + (q3 @ E_ + q2 @ E_ @ q + q @ E_ @ q2 + E_ @ q3)
        np.testing.assert_allclose(np.sum(Gbar[n] * DG), np.dot(d[n], e[n]), rtol=1e-12, atol=1e-12)
    # Q = 0: dtheta = 2 (Gbar_ij - Gbar_ji)
    d0 = cnp_backward(np.zeros_like(th), Gbar, b)
    ii, jj = np.triu_indices(b, 1)
    np.testing.assert_allclose(d0, 2 * (Gbar[:, ii, jj] - Gbar[:, jj, ii]), rtol=0, atol=1e-14)


def test_cnp_backward_pins():
    _check_cnp_backward(O.cnp_forward, O.cnp_backward)


# ------------------------------------------------------------ layer forward ----

def _small_layer(rng, n=5, d_in=12, d_out=8, b=4, std=0.1, perms=True):
    W = rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)
    th_r = rand_theta(d_in // b, b, std, rng)
    th_p = rand_theta(d_out // b, b, std, rng)
    X = rng.standard_normal((n, d_in))
    dZ = rng.standard_normal((n, d_out))
    pin = rng.permutation(d_in) if perms else None
    pout = rng.permutation(d_out) if perms else None
    return W, th_r, th_p, X, dZ, pin, pout, b


def dense_reference(W, G_R, G_P, X, pin, pout):
    """Unmerged, dense, column-form eq. 3: z = P^T (W (R^T x)) with
    R = Psi_in^T Diag(G_R) Psi_in and P = Psi_out^T Diag(G_P) Psi_out (Method §1-§2)."""
    d_out, d_in = W.shape
    Pi = perm_matrix(pin if pin is not None else np.arange(d_in))
    Po = perm_matrix(pout if pout is not None else np.arange(d_out))
    R = Pi.T @ sla.block_diag(*G_R) @ Pi
    P = Po.T @ sla.block_diag(*G_P) @ Po
    return (P.T @ (W @ (R.T @ X.T))).T


def _check_layer_forward(layer_forward, merge_perm, cnp_forward):
    rng = np.random.default_rng(11)
    for perms in (True, False):
        W, th_r, th_p, X, dZ, pin, pout, b = _small_layer(rng, perms=perms)
        G_R, G_P = cnp_forward(th_r, b), cnp_forward(th_p, b)
        Wm = merge_perm(W, pout, pin)
        Z = layer_forward(X, Wm, G_R, G_P, pin, pout)
        np.testing.assert_allclose(Z, dense_reference(W, G_R, G_P, X, pin, pout), rtol=0, atol=1e-13)
        # merge = Psi_out W Psi_in^T with dense permutation matrices, exactly
        if perms:
            assert np.array_equal(Wm, perm_matrix(pout) @ W @ perm_matrix(pin).T)
        # theta = 0: a plain linear layer, X W^T (library matmul), perms or not
        I_r = np.broadcast_to(np.eye(b), G_R.shape)
        I_p = np.broadcast_to(np.eye(b), G_P.shape)
        Z0 = layer_forward(X, Wm, cnp_forward(0 * th_r, b), cnp_forward(0 * th_p, b), pin, pout)
        np.testing.assert_allclose(Z0, np.matmul(X, W.T), rtol=0, atol=1e-13)
        np.testing.assert_allclose(layer_forward(X, Wm, I_r, I_p, None, None), np.matmul(X, Wm.T),
                                   rtol=0, atol=1e-13)


def test_layer_forward_pins():
    _check_layer_forward(O.layer_forward, O.merge_perm, O.cnp_forward)


def _check_fold(fold, merge_perm, cnp_forward):
    rng = np.random.default_rng(21)
    for perms in (True, False):
        W, th_r, th_p, X, dZ, pin, pout, b = _small_layer(rng, perms=perms)
        G_R, G_P = cnp_forward(th_r, b), cnp_forward(th_p, b)
        Wm = merge_perm(W, pout, pin)
        Weff = fold(Wm, G_R, G_P, pin, pout)
        # the folded weight reproduces the dense, unmerged layer (eq. 3 with R and P)
        np.testing.assert_allclose(X @ Weff.T, dense_reference(W, G_R, G_P, X, pin, pout), rtol=0, atol=1e-12)
        # theta = 0 (G = I): the fold undoes the merge exactly
        I_r = np.broadcast_to(np.eye(b), G_R.shape)
        I_p = np.broadcast_to(np.eye(b), G_P.shape)
        assert np.array_equal(fold(Wm, I_r, I_p, pin, pout), W)
    # blocks of unequal size (ceil(d/b) blocks, the last one smaller)
    for d_in, d_out, b in RAGGED:
        W, th_r, th_p, X, dZ, pin, pout = _ragged_layer(rng, d_in, d_out, b)
        G_R, G_P = _blocks_from_flat(th_r, d_in, b), _blocks_from_flat(th_p, d_out, b)
        Weff = fold(merge_perm(W, pout, pin), G_R, G_P, pin, pout)
        np.testing.assert_allclose(X @ Weff.T, dense_reference(W, G_R, G_P, X, pin, pout), rtol=0, atol=1e-12)


def test_fold_pins():
    _check_fold(O.fold_weights, O.merge_perm, O.cnp_forward)


def _check_adam(adam_step):
    import torch
    rng = np.random.default_rng(31)
    th0 = rng.standard_normal(300) * 0.01
    g = [rng.standard_normal(300) for _ in range(3)]
    lr, b1, b2, eps, gamma = 1e-3, 0.9, 0.999, 1e-8, 0.5
    # closed form of the first step from zero state: theta - gamma lr g / (|g| + eps)
    th1, m1, v1 = adam_step(th0, g[0], np.zeros(300), np.zeros(300), lr, b1, b2, eps, 1, gamma)
    np.testing.assert_allclose(th1, th0 - gamma * lr * g[0] / (np.abs(g[0]) + eps), rtol=1e-12, atol=1e-15)
    # three steps against the library optimizer (torch.optim.Adam, float64, lr = gamma lr)
    p = torch.nn.Parameter(torch.tensor(th0, dtype=torch.float64))
    opt = torch.optim.Adam([p], lr=gamma * lr, betas=(b1, b2), eps=eps)
    th, m, v = th0, np.zeros(300), np.zeros(300)
    for t in range(1, 4):
        p.grad = torch.tensor(g[t - 1], dtype=torch.float64)
        opt.step()
        th, m, v = adam_step(th, g[t - 1], m, v, lr, b1, b2, eps, t, gamma)
    np.testing.assert_allclose(th, p.detach().numpy(), rtol=0, atol=1e-15)


def test_adam_pins():
    _check_adam(O.adam_step)


def test_layer_empty_tokens():
    rng = np.random.default_rng(3)
    W, th_r, th_p, X, dZ, pin, pout, b = _small_layer(rng, n=0)
    r = O.poetx_step(X, dZ, O.merge_perm(W, pout, pin), th_r, th_p, b, pin, pout)
    assert r["Z"].shape == (0, 8) and r["dX"].shape == (0, 12)
    assert np.all(r["dtheta_R"] == 0) and np.all(r["dtheta_P"] == 0)


# ----------------------------------------------------------- layer backward ----

def _check_layer_backward(poetx_step, merge_perm):
    rng = np.random.default_rng(5)
    W, th_r, th_p, X, dZ, pin, pout, b = _small_layer(rng, n=3, d_in=8, d_out=12, b=4, std=0.15)
    Wm = merge_perm(W, pout, pin)
    r = poetx_step(X, dZ, Wm, th_r, th_p, b, pin, pout)

    def loss(tr, tp, x):
        # independent dense evaluation (unmerged, explicit R and P)
        Z = dense_reference(W, O.cnp_forward(tr, b), O.cnp_forward(tp, b), x, pin, pout)
        return np.sum(Z * dZ)

    h = 1e-6
    for name, arr, key in (("R", th_r, "dtheta_R"), ("P", th_p, "dtheta_P"), ("X", X, "dX")):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap = arr.copy(); ap[idx] += h
            am = arr.copy(); am[idx] -= h
            args_p = [th_r, th_p, X]
            args_m = [th_r, th_p, X]
            slot = {"R": 0, "P": 1, "X": 2}[name]
            args_p[slot] = ap
            args_m[slot] = am
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(r[key], fd, rtol=0, atol=2e-8, err_msg=name)
    # theta = 0 closed forms: dX = dZ W; dtheta_P from dG_P = B~^T dZ~ with B~ = X~ W'^T
    r0 = poetx_step(X, dZ, Wm, 0 * th_r, 0 * th_p, b, pin, pout)
    np.testing.assert_allclose(r0["dX"], dZ @ W, rtol=0, atol=1e-13)
    Bt = X[:, pin] @ Wm.T
    dZt = dZ[:, pout]
    dGp = np.stack([Bt[:, j * b:(j + 1) * b].T @ dZt[:, j * b:(j + 1) * b] for j in range(Wm.shape[0] // b)])
    ii, jj = np.triu_indices(b, 1)
    np.testing.assert_allclose(r0["dtheta_P"], 2 * (dGp[:, ii, jj] - dGp[:, jj, ii]), rtol=0, atol=1e-13)


def test_layer_backward_pins():
    _check_layer_backward(O.poetx_step, O.merge_perm)


# ------------------------------------------------------------ ragged blocks ----

def _blocks_from_flat(theta, d, b):
    """Test-side reading of the flat layout: floor(d/b) packed vectors of size
    b(b-1)/2, then the last block's, each turned into G by cnp_forward."""
    full, last = divmod(d, b)
    p = b * (b - 1) // 2
    Gs = list(O.cnp_forward(theta[:full * p].reshape(full, p), b)) if full else []
    if last:
        Gs.append(O.cnp_forward(theta[full * p:][None], last)[0])
    return Gs


RAGGED = [(10, 7, 4), (9, 12, 4), (5, 6, 8)]  # last blocks 2 | 3, 1 | none, whole side < b


def _ragged_layer(rng, d_in, d_out, b, n=3, std=0.15):
    W = rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)
    pr = sum(s * (s - 1) // 2 for s in O.block_sizes(d_in, b))
    pp = sum(s * (s - 1) // 2 for s in O.block_sizes(d_out, b))
    th_r = rng.standard_normal(pr) * std
    th_p = rng.standard_normal(pp) * std
    X = rng.standard_normal((n, d_in))
    dZ = rng.standard_normal((n, d_out))
    return W, th_r, th_p, X, dZ, rng.permutation(d_in), rng.permutation(d_out)


def _check_ragged(poetx_step):
    assert O.block_sizes(10, 4) == [4, 4, 2] and O.block_sizes(7, 4) == [4, 3]
    assert O.block_sizes(8, 4) == [4, 4] and O.block_sizes(9, 4) == [4, 4, 1] and O.block_sizes(3, 4) == [3]
    rng = np.random.default_rng(41)
    for d_in, d_out, b in RAGGED:
        W, th_r, th_p, X, dZ, pin, pout = _ragged_layer(rng, d_in, d_out, b)
        Wm = O.merge_perm(W, pout, pin)
        r = poetx_step(X, dZ, Wm, th_r, th_p, b, pin, pout)
        G_R, G_P = _blocks_from_flat(th_r, d_in, b), _blocks_from_flat(th_p, d_out, b)
        np.testing.assert_allclose(r["Z"], dense_reference(W, G_R, G_P, X, pin, pout), rtol=0, atol=1e-13)

        def loss(tr, tp, x):
            Z = dense_reference(W, _blocks_from_flat(tr, d_in, b), _blocks_from_flat(tp, d_out, b), x, pin, pout)
            return np.sum(Z * dZ)

        h = 1e-6
        for slot, key in ((0, "dtheta_R"), (1, "dtheta_P"), (2, "dX")):
            base = [th_r, th_p, X]
            fd = np.zeros_like(base[slot])
            for idx in np.ndindex(fd.shape):
                ap, am = [a.copy() for a in base], [a.copy() for a in base]
                ap[slot][idx] += h
                am[slot][idx] -= h
                fd[idx] = (loss(*ap) - loss(*am)) / (2 * h)
            np.testing.assert_allclose(r[key], fd, rtol=0, atol=2e-8, err_msg=f"{key} at {(d_in, d_out, b)}")
    # divisible widths: the flat layout is the [n][p] layout, block after block
    W, th_r, th_p, X, dZ, pin, pout = _ragged_layer(rng, 8, 12, 4)
    Wm = O.merge_perm(W, pout, pin)
    rf = poetx_step(X, dZ, Wm, th_r, th_p, 4, pin, pout)
    ru = O.poetx_step(X, dZ, Wm, th_r.reshape(2, 6), th_p.reshape(3, 6), 4, pin, pout)
    assert np.array_equal(rf["Z"], ru["Z"]) and np.array_equal(rf["dX"], ru["dX"])
    assert np.array_equal(rf["dtheta_R"], ru["dtheta_R"].ravel())
    assert np.array_equal(rf["dtheta_P"], ru["dtheta_P"].ravel())


def test_ragged_blocks_pins():
    _check_ragged(O.poetx_step)


# -------------------------------------------------------------------- int8 ----

def test_int8_merge_and_dequant():
    rng = np.random.default_rng(9)
    d_out, d_in, b = 8, 12, 4
    q = rng.integers(-127, 128, size=(d_out, d_in)).astype(np.int8)
    s = (rng.random(d_out) * 0.01 + 1e-3).astype(np.float32)
    pin, pout = rng.permutation(d_in), rng.permutation(d_out)
    qm, sm = O.merge_perm_int8(q, s, pout, pin)
    assert qm.dtype == np.int8
    assert np.array_equal(qm, q[pout][:, pin]) and np.array_equal(sm, s[pout])
    X = rng.standard_normal((6, d_in))
    W = s.astype(np.float64)[:, None] * q.astype(np.float64)
    I_r = np.broadcast_to(np.eye(b), (d_in // b, b, b))
    I_p = np.broadcast_to(np.eye(b), (d_out // b, b, b))
    Z = O.layer_forward(X, O.dequantize_rows(qm, sm), I_r, I_p, pin, pout)
    np.testing.assert_allclose(Z, np.matmul(X, W.T), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- spectrum ----

def test_spectrum_preserved_to_q4():
    """Background section: orthogonal R, P leave the singular values of W unchanged;
    CNP's G is orthogonal up to O(|Q|^4), so the effective weight's spectrum moves by O(|Q|^4)."""
    rng = np.random.default_rng(21)
    W, th_r, th_p, X, dZ, pin, pout, b = _small_layer(rng, d_in=16, d_out=16, b=8, std=0.05)
    sv_w = np.linalg.svd(W, compute_uv=False)
    devs = []
    for s in (1.0, 0.5):
        G_R, G_P = O.cnp_forward(th_r * s, b), O.cnp_forward(th_p * s, b)
        Weff = O.layer_forward(np.eye(16), O.merge_perm(W, pout, pin), G_R, G_P, pin, pout).T
        devs.append(np.max(np.abs(np.linalg.svd(Weff, compute_uv=False) - sv_w)) / sv_w[0])
    assert devs[0] < 1e-3
    assert devs[0] / max(devs[1], 1e-300) > 8.0


# ------------------------------------------------------------------ mutants ----

def _mutants():
    """Plausible mistakes, each planted in a copy of one oracle function."""
    def fwd_drop_q3(th, b, return_q2=False):
        Q = O.skew_from_packed(th, b); Q2 = Q @ Q
        return np.eye(b)[None] + 2 * (Q + Q2) + Q2 @ Q2

    def fwd_sign(th, b, return_q2=False):
        Q = O.skew_from_packed(th, b); Q2 = Q @ Q
        return np.eye(b)[None] + 2 * (-Q + Q2 - Q2 @ Q) + Q2 @ Q2

    def fwd_half(th, b, return_q2=False):
        Q = O.skew_from_packed(th, b); Q2 = Q @ Q
        return np.eye(b)[None] + (Q + Q2 + Q2 @ Q) + Q2 @ Q2

    def bwd_no_transpose(th, dG, b):
        Q = O.skew_from_packed(th, b)
        n = Q.shape[0]
        pw = [np.broadcast_to(np.eye(b), (n, b, b)), Q, Q @ Q, Q @ Q @ Q]
        Qbar = np.zeros_like(dG, dtype=np.float64)
        for m, c in enumerate((2.0, 2.0, 2.0, 1.0), start=1):
            for a in range(m):
                Qbar += c * (pw[a] @ dG @ pw[m - 1 - a])
        return O.packed_from_matrix(Qbar)

    def bwd_drop_cross(th, dG, b):
        Q = O.skew_from_packed(th, b)
        Qt = np.swapaxes(Q, 1, 2)
        Qbar = 2 * dG + 2 * (Qt @ dG + dG @ Qt)
        return O.packed_from_matrix(Qbar)

    def bwd_pack_sum(th, dG, b):
        d = O.cnp_backward(th, dG, b)
        ii, jj = O.triu_pairs(b)
        return d + 2 * np.asarray(dG)[:, jj, ii]  # Qbar_ij + Qbar_ji-like slip

    def merge_swapped(W, pout, pin):
        # uses the inverse of perm_in on the columns
        return np.asarray(W)[np.asarray(pout)][:, np.argsort(pin)]

    def fwd_layer_transposed(X, Wm, G_R, G_P, pin=None, pout=None, keep=False):
        return O.layer_forward(X, Wm, np.swapaxes(G_R, 1, 2), G_P, pin, pout)

    def fwd_layer_no_scatter(X, Wm, G_R, G_P, pin=None, pout=None, keep=False):
        Z = O.layer_forward(X, Wm, G_R, G_P, pin, None)
        return Z if pout is None else Z  # forgets the output permutation

    def step_wrong_dgp(X, dZ, Wm, tr, tp, b, pin=None, pout=None):
        r = O.poetx_step(X, dZ, Wm, tr, tp, b, pin, pout)
        r["dtheta_P"] = O.cnp_backward(tp, np.swapaxes(r["dG_P"], 1, 2), b)
        return r

    def step_no_dx_scatter(X, dZ, Wm, tr, tp, b, pin=None, pout=None):
        r = O.poetx_step(X, dZ, Wm, tr, tp, b, None if pin is None else pin, pout)
        if pin is not None:
            r["dX"] = r["dX"][:, pin]
        return r

    def fold_untransposed(Wm, G_R, G_P, pin=None, pout=None):
        return O.fold_weights(Wm, np.swapaxes(G_R, 1, 2), G_P, pin, pout)

    def fold_gathers(Wm, G_R, G_P, pin=None, pout=None):
        # gathers with the permutations where the fold must scatter
        W = O.fold_weights(Wm, G_R, G_P, None, None)
        return W if pin is None else W[np.asarray(pout)][:, np.asarray(pin)]

    def adam_no_bias_correction(theta, g, m, v, lr, b1, b2, eps, t, gamma=1.0):
        m = b1 * np.asarray(m) + (1 - b1) * np.asarray(g)
        v = b2 * np.asarray(v) + (1 - b2) * np.asarray(g) ** 2
        return np.asarray(theta) - gamma * lr * m / (np.sqrt(v) + eps), m, v

    def step_ragged_tail_ignored(X, dZ, Wm, tr, tp, b, pin=None, pout=None):
        # the smaller last input block stays the identity (its parameters unused)
        d_in = np.shape(Wm)[1]
        full = d_in // b
        tr = np.array(tr, dtype=np.float64)
        if d_in % b:
            tr[full * (b * (b - 1) // 2):] = 0.0
        return O.poetx_step(X, dZ, Wm, tr, tp, b, pin, pout)

    def step_ragged_tail_grad_dropped(X, dZ, Wm, tr, tp, b, pin=None, pout=None):
        r = O.poetx_step(X, dZ, Wm, tr, tp, b, pin, pout)
        d_out = np.shape(Wm)[0]
        if d_out % b:
            r["dtheta_P"][(d_out // b) * (b * (b - 1) // 2):] = 0.0
        return r

    return [
        ("ragged last block ignored", lambda: _check_ragged(step_ragged_tail_ignored)),
        ("ragged last block gradient dropped", lambda: _check_ragged(step_ragged_tail_grad_dropped)),
        ("adam without bias correction", lambda: _check_adam(adam_no_bias_correction)),
        ("fold keeps G_R untransposed", lambda: _check_fold(fold_untransposed, O.merge_perm, O.cnp_forward)),
        ("fold gathers instead of scattering", lambda: _check_fold(fold_gathers, O.merge_perm, O.cnp_forward)),
        ("fwd drops Q^3", lambda: _check_cnp_forward(fwd_drop_q3)),
        ("fwd sign slip", lambda: _check_cnp_forward(fwd_sign)),
        ("fwd missing factor 2", lambda: _check_cnp_forward(fwd_half)),
        ("bwd without transposes", lambda: _check_cnp_backward(O.cnp_forward, bwd_no_transpose)),
        ("bwd drops higher terms", lambda: _check_cnp_backward(O.cnp_forward, bwd_drop_cross)),
        ("bwd packing slip", lambda: _check_cnp_backward(O.cnp_forward, bwd_pack_sum)),
        ("merge uses inverse perm", lambda: _check_layer_forward(O.layer_forward, merge_swapped, O.cnp_forward)),
        ("block apply transposed", lambda: _check_layer_forward(fwd_layer_transposed, O.merge_perm, O.cnp_forward)),
        ("output scatter dropped", lambda: _check_layer_forward(fwd_layer_no_scatter, O.merge_perm, O.cnp_forward)),
        ("dG_P transposed", lambda: _check_layer_backward(step_wrong_dgp, O.merge_perm)),
        ("dX scatter slip", lambda: _check_layer_backward(step_no_dx_scatter, O.merge_perm)),
    ]


@pytest.mark.parametrize("name,check", _mutants(), ids=[m[0] for m in _mutants()])
def test_pins_catch_planted_mistakes(name, check):
    with pytest.raises(AssertionError):
        check()
