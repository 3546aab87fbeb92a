"""Plain fp64 CPU oracle for the POET-X linear layer (forward, backward, CNP, merge).

TEST INFRASTRUCTURE ONLY.  This module is the oracle that the HIP path is
compared against.  Only the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the
``orthogonal_reparameterized_amd`` package and its C-ABI library) never imports,
links or calls anything in here, and nothing in here imports the product.

Source: the POET-X summary page "POET-X: Memory-efficient LLM Training by
Scaling Orthogonal Transformation" (arXiv 2603.05500 digest), section
"core method and technical details" (subsections 1-6, eq. 3 and eq. 9).
Every function below names the subsection it follows.  Everything is computed
in float64 with plain NumPy steps; the only library primitive used is the
matrix product (``@``).  No blocking, fusion or reordering is applied beyond
what the formulas state.

Conventions (readings of the page where it is silent or ambiguous):
  * activations are token-major rows: X[N][d_in], Z[N][d_out]; the frozen
    weight is W[d_out][d_in] (the map "W" of eq. 3 takes the input to the
    output).
  * G_R acts on the input side (d_in/b blocks), G_P on the output side
    (d_out/b blocks).
  * permutations are index arrays; gather X~[t][i] = X[t][perm_in[i]], scatter
    Z[t][perm_out[i]] = Z~[t][i]; a missing (None) permutation is the identity.
  * packed skew storage: theta[k] is Q[i][j] (i < j) with k running row-major
    over the strict upper triangle, Q[j][i] = -theta[k].
  * a side of width d with block size b has ceil(d/b) diagonal blocks: floor(d/b)
    of size b, then one of size d - b*floor(d/b) when that is not zero (Method
    §3).  Block sets are sequences of square arrays (an array [n][b][b] when all
    sizes agree); a flat theta holds the blocks' packed vectors one after another.

Parity status: every function here is pinned by tests/test_oracle.py against
closed forms, library routines, an independent dense assembly and finite
differences.  The packing order and sign of theta are a convention the page
does not fix (it gives only the count b(b-1)/2); they are shared by
specification, i.e. "parity unpinned" for the order itself.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "packed_size",
    "triu_pairs",
    "skew_from_packed",
    "packed_from_matrix",
    "cnp_forward",
    "cnp_backward",
    "merge_perm",
    "merge_perm_int8",
    "dequantize_rows",
    "block_sizes",
    "split_packed",
    "cnp_forward_blocks",
    "cnp_backward_blocks",
    "layer_forward",
    "layer_backward",
    "poetx_step",
]


# ---------------------------------------------------------------------------
# Packed skew-symmetric storage (Method §4: only the upper triangle of Q is
# stored, b(b-1)/2 numbers per block instead of b^2).
# ---------------------------------------------------------------------------

def packed_size(b: int) -> int:
    """Number of free parameters of one b x b skew block (Method §4)."""
    return b * (b - 1) // 2


def triu_pairs(b: int):
    """(i, j) index arrays of the strict upper triangle, row-major order."""
    ii, jj = [], []
    for i in range(b):
        for j in range(i + 1, b):
            ii.append(i)
            jj.append(j)
    return np.array(ii, dtype=np.int64), np.array(jj, dtype=np.int64)


def skew_from_packed(theta: np.ndarray, b: int) -> np.ndarray:
    """Unpack theta[n][p] into skew matrices Q[n][b][b] (Method §4).

    Q[i][j] = theta[k], Q[j][i] = -theta[k] for i < j, zero diagonal.
    """
    theta = np.asarray(theta, dtype=np.float64)
    n = theta.shape[0]
    assert theta.shape == (n, packed_size(b))
    ii, jj = triu_pairs(b)
    Q = np.zeros((n, b, b), dtype=np.float64)
    Q[:, ii, jj] = theta
    Q[:, jj, ii] = -theta
    return Q


def packed_from_matrix(M: np.ndarray) -> np.ndarray:
    """Gradient of a loss w.r.t. packed theta, given its gradient M = dL/dQ.

    theta[k] enters Q at (i, j) with +1 and at (j, i) with -1, so
    dL/dtheta[k] = M[i][j] - M[j][i].
    """
    M = np.asarray(M, dtype=np.float64)
    b = M.shape[-1]
    ii, jj = triu_pairs(b)
    return M[:, ii, jj] - M[:, jj, ii]


# ---------------------------------------------------------------------------
# Cayley-Neumann parameterization (Method §4, eq. 9).
# ---------------------------------------------------------------------------

# Coefficients of the truncated series G = I + 2Q + 2Q^2 + 2Q^3 + Q^4, i.e.
# eq. 9: G = 2(Q + Q^2 + Q^2.Q) + Q^2.Q^2 + I.
_CNP_COEF = (2.0, 2.0, 2.0, 1.0)  # coefficients of Q^1, Q^2, Q^3, Q^4


def cnp_forward(theta: np.ndarray, b: int, return_q2: bool = False):
    """G[n][b][b] from packed theta[n][p], literally eq. 9 (Method §4).

    Q2 = Q.Q ; G = I + 2 (Q + Q2 + Q2.Q) + Q2.Q2
    """
    Q = skew_from_packed(theta, b)
    Q2 = Q @ Q
    Q3 = Q2 @ Q
    Q4 = Q2 @ Q2
    eye = np.eye(b, dtype=np.float64)[None]
    G = eye + 2.0 * (Q + Q2 + Q3) + Q4
    if return_q2:
        return G, Q2
    return G


def cnp_backward(theta: np.ndarray, dG: np.ndarray, b: int) -> np.ndarray:
    """dL/dtheta[n][p] from dL/dG[n][b][b] (Method §4, the backward of eq. 9).

    The page says the fused backward uses only Q and Q^2 but does not print
    its formula (eq. 10).  This is the exact adjoint of eq. 9, written out
    from the product rule: the directional derivative of Q^m along E is
    sum_{a=0}^{m-1} Q^a E Q^(m-1-a), whose adjoint applied to Gbar is
    sum_a (Q^a)^T Gbar (Q^(m-1-a))^T.  Summing over m with the eq. 9
    coefficients gives Qbar = dL/dQ; the packed gradient then follows from
    ``packed_from_matrix``.
    """
    Q = skew_from_packed(theta, b)
    Gbar = np.asarray(dG, dtype=np.float64)
    n = Q.shape[0]
    eye = np.broadcast_to(np.eye(b, dtype=np.float64), (n, b, b))
    powers = [eye, Q, Q @ Q, Q @ Q @ Q]  # Q^0 .. Q^3
    powT = [np.swapaxes(P, -1, -2) for P in powers]
    Qbar = np.zeros_like(Gbar)
    for m, c in enumerate(_CNP_COEF, start=1):
        for a in range(m):
            Qbar += c * (powT[a] @ Gbar @ powT[m - 1 - a])
    return packed_from_matrix(Qbar)


# ---------------------------------------------------------------------------
# Blocks of unequal size: the ceil(d/b) blocks of Method §3, the last one holding
# the d - b*floor(d/b) remaining coordinates.
# ---------------------------------------------------------------------------

def block_sizes(d: int, b: int):
    """Sizes of the diagonal blocks of a side of width d with block size b."""
    full, last = divmod(int(d), int(b))
    return [int(b)] * full + ([last] if last else [])


def split_packed(theta, sizes):
    """The per-block packed vectors of a flat theta (blocks one after another)."""
    theta = np.asarray(theta, dtype=np.float64)
    out, o = [], 0
    for s in sizes:
        p = packed_size(s)
        out.append(theta[o:o + p])
        o += p
    assert o == theta.shape[0], "flat theta length does not match the block sizes"
    return out


def cnp_forward_blocks(theta, sizes):
    """G of every block (eq. 9 per block, each at its own size), from a flat theta."""
    return [cnp_forward(t[None], s)[0] for t, s in zip(split_packed(theta, sizes), sizes)]


def cnp_backward_blocks(theta, dG, sizes):
    """Flat dL/dtheta from the blocks' dL/dG (the adjoint of eq. 9 per block)."""
    parts = [cnp_backward(t[None], np.asarray(g, dtype=np.float64)[None], s)[0]
             for t, g, s in zip(split_packed(theta, sizes), dG, sizes)]
    return np.concatenate(parts) if parts else np.zeros(0)


# ---------------------------------------------------------------------------
# Permutation merge (Method §2: W is fixed during the inner phase, so the two
# weight-side permutations are folded into it once: W' = Psi_out W Psi_in^T).
# ---------------------------------------------------------------------------

def merge_perm(W: np.ndarray, perm_out, perm_in) -> np.ndarray:
    """W'[i][k] = W[perm_out[i]][perm_in[k]] (Method §2)."""
    W = np.asarray(W)
    rows = np.arange(W.shape[0]) if perm_out is None else np.asarray(perm_out, dtype=np.int64)
    cols = np.arange(W.shape[1]) if perm_in is None else np.asarray(perm_in, dtype=np.int64)
    return W[rows][:, cols]


def merge_perm_int8(q: np.ndarray, scale: np.ndarray, perm_out, perm_in):
    """Int8 weight with one scale per output row: q' as merge_perm, s'[i] = s[perm_out[i]].

    A per-row scale rides along with its row, so this is exact (Method §6:
    the low-bit W is what is stored; it is only dequantized inside the product).
    """
    qm = merge_perm(q, perm_out, perm_in)
    rows = np.arange(q.shape[0]) if perm_out is None else np.asarray(perm_out, dtype=np.int64)
    return qm, np.asarray(scale)[rows]


def dequantize_rows(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """W[i][k] = s[i] * q[i][k] in float64 (Method §6, dequantize then multiply)."""
    return np.asarray(scale, dtype=np.float64)[:, None] * np.asarray(q, dtype=np.float64)


# ---------------------------------------------------------------------------
# Layer forward / backward (Method §1 eq. 3, §3 block-diagonal products,
# §5 the intermediates a, b, z).
# ---------------------------------------------------------------------------

def _gather_cols(M, perm):
    return M if perm is None else M[:, np.asarray(perm, dtype=np.int64)]


def _scatter_cols(M, perm):
    if perm is None:
        return M
    out = np.empty_like(M)
    out[:, np.asarray(perm, dtype=np.int64)] = M
    return out


def _blocks(G):
    """A block set as a list of float64 square arrays."""
    return [np.asarray(g, dtype=np.float64) for g in G]


def _stack_if_uniform(blocks):
    """An array [n][b][b] when all blocks share one size, else the list itself."""
    if len({g.shape[0] for g in blocks}) <= 1 and blocks:
        return np.stack(blocks)
    return blocks


def _block_right(M, G):
    """Row-wise block-diagonal product: the columns of block j (offset o, size s) are
    out[:, o:o+s] = M[:, o:o+s] @ G[j]."""
    G = _blocks(G)
    out = np.empty((M.shape[0], sum(g.shape[0] for g in G)), dtype=np.float64)
    o = 0
    for g in G:
        s = g.shape[0]
        out[:, o:o + s] = M[:, o:o + s] @ g
        o += s
    return out


def _block_right_t(M, G):
    """out[:, o:o+s] = M[:, o:o+s] @ G[j]^T (adjoint of _block_right in M)."""
    G = _blocks(G)
    out = np.empty((M.shape[0], sum(g.shape[0] for g in G)), dtype=np.float64)
    o = 0
    for g in G:
        s = g.shape[0]
        out[:, o:o + s] = M[:, o:o + s] @ g.T
        o += s
    return out


def _block_grad(L, R, sizes):
    """dG[j] = L[:, o:o+s]^T @ R[:, o:o+s] over the blocks' column ranges (sum over tokens)."""
    out, o = [], 0
    for s in sizes:
        out.append(L[:, o:o + s].T @ R[:, o:o + s])
        o += s
    return _stack_if_uniform(out)


def layer_forward(X, Wm, G_R, G_P, perm_in=None, perm_out=None, keep=False):
    """Z from X with the merged weight W' (Method §1 eq. 3 and §2).

    Token-major form of z = P^T (W (R^T x)) with the weight-side permutations
    merged into W' = Psi_out W Psi_in^T:
        X~ = gather(X, perm_in)           (remaining input permutation)
        A  = X~ . Diag(G_R)               (a = G_R^T x, per block, Method §3)
        B  = A . W'^T                     (b = W' a)
        Z~ = B . Diag(G_P)                (z~ = G_P^T b, per block)
        Z  = scatter(Z~, perm_out)        (remaining output permutation)
    """
    X = np.asarray(X, dtype=np.float64)
    Wm = np.asarray(Wm, dtype=np.float64)
    Xt = _gather_cols(X, perm_in)
    A = _block_right(Xt, G_R)
    B = A @ Wm.T
    Zt = _block_right(B, G_P)
    Z = _scatter_cols(Zt, perm_out)
    if keep:
        return Z, dict(Xt=Xt, A=A, B=B, Zt=Zt)
    return Z


def layer_backward(X, dZ, Wm, G_R, G_P, perm_in=None, perm_out=None):
    """Chain rule through layer_forward; W' gets no gradient (Method §1).

    Returns dX, dG_R, dG_P and the recomputed intermediate B.
        dZ~  = gather(dZ, perm_out)
        dB   = dZ~ . Diag(G_P)^T,        dG_P[j] = B_j^T dZ~_j
        dA   = dB . W'
        dX~  = dA . Diag(G_R)^T,         dG_R[j] = X~_j^T dA_j
        dX   = scatter(dX~, perm_in)
    """
    X = np.asarray(X, dtype=np.float64)
    dZ = np.asarray(dZ, dtype=np.float64)
    Wm = np.asarray(Wm, dtype=np.float64)
    G_R, G_P = _blocks(G_R), _blocks(G_P)
    Xt = _gather_cols(X, perm_in)
    A = _block_right(Xt, G_R)
    B = A @ Wm.T
    dZt = _gather_cols(dZ, perm_out)
    dB = _block_right_t(dZt, G_P)
    dG_P = _block_grad(B, dZt, [g.shape[0] for g in G_P])
    dA = dB @ Wm
    dXt = _block_right_t(dA, G_R)
    dG_R = _block_grad(Xt, dA, [g.shape[0] for g in G_R])
    dX = _scatter_cols(dXt, perm_in)
    return dX, dG_R, dG_P, B


# ---------------------------------------------------------------------------
# Phase-end fold: the consolidation step of merge-then-reinitialize (the POET
# recipe's periodic merge of the learned transforms into the frozen weight, on the
# "Poet Orthogonal LLM Training" skill page; with POET-X's merged permutations,
# Method §2).  The next phase then starts from theta = 0 and new permutations.
# ---------------------------------------------------------------------------

def _block_diag(G):
    G = _blocks(G)
    d = sum(g.shape[0] for g in G)
    D = np.zeros((d, d), dtype=np.float64)
    o = 0
    for g in G:
        s = g.shape[0]
        D[o:o + s, o:o + s] = g
        o += s
    return D


def fold_weights(Wm, G_R, G_P, perm_in=None, perm_out=None):
    """The layer's effective weight in original coordinates.

    With M = Diag(G_P)^T . W' . Diag(G_R)^T (dense block-diagonal assembly),
        W[perm_out[i]][perm_in[k]] = M[i][k],
    so that X . W^T equals layer_forward(X, W', G_R, G_P, perm_in, perm_out).
    """
    Wm = np.asarray(Wm, dtype=np.float64)
    M = _block_diag(G_P).T @ Wm @ _block_diag(G_R).T
    d_out, d_in = M.shape
    rows = np.arange(d_out) if perm_out is None else np.asarray(perm_out, dtype=np.int64)
    cols = np.arange(d_in) if perm_in is None else np.asarray(perm_in, dtype=np.int64)
    W = np.empty_like(M)
    W[np.ix_(rows, cols)] = M
    return W


# ---------------------------------------------------------------------------
# Optimizer on packed theta: the state lives on the b(b-1)/2 packed parameters per
# block (Method §4, which halves optimizer state and gradients); gamma scales the
# learning rate (practical advice 3, 0.5 for POET-XQ).  Adam as published by Kingma
# and Ba (2015); the pages fix no other hyperparameter.
# ---------------------------------------------------------------------------

def adam_step(theta, g, m, v, lr, beta1, beta2, eps, t, gamma=1.0):
    """One Adam step; returns the new (theta, m, v)."""
    theta, g = np.asarray(theta, dtype=np.float64), np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    return theta - gamma * lr * m_hat / (np.sqrt(v_hat) + eps), m, v


def poetx_step(X, dZ, Wm, theta_R, theta_P, b, perm_in=None, perm_out=None):
    """One full step of the layer: CNP forward, forward, backward, CNP backward.

    theta_* are [n][p] when b divides the side's width; a flat theta (one
    dimension) holds the ceil(d/b) blocks of block_sizes(d, b), the last one
    possibly smaller, and its gradient comes back flat too.
    Returns a dict with G_R, G_P, Z, dX, dG_R, dG_P, dtheta_R, dtheta_P, B.
    """
    d_out, d_in = np.shape(Wm)

    def fwd(theta, d):
        if np.ndim(theta) == 1:
            return cnp_forward_blocks(theta, block_sizes(d, b))
        return cnp_forward(theta, b)

    def bwd(theta, dG, d):
        if np.ndim(theta) == 1:
            return cnp_backward_blocks(theta, dG, block_sizes(d, b))
        return cnp_backward(theta, dG, b)

    G_R, G_P = fwd(theta_R, d_in), fwd(theta_P, d_out)
    Z = layer_forward(X, Wm, G_R, G_P, perm_in, perm_out)
    dX, dG_R, dG_P, B = layer_backward(X, dZ, Wm, G_R, G_P, perm_in, perm_out)
    return dict(
        G_R=G_R, G_P=G_P, Z=Z, dX=dX, dG_R=dG_R, dG_P=dG_P, B=B,
        dtheta_R=bwd(theta_R, dG_R, d_in),
        dtheta_P=bwd(theta_P, dG_P, d_out),
    )
