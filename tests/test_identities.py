"""Algebraic identities the HIP kernels rely on, checked in float64 against the oracle.

These do not test the oracle; they check that a regrouping a kernel computes is the same
function as the oracle's definition (so a kernel that follows it faithfully must agree).
"""
import numpy as np
import pytest

from oracle import poetx_oracle as O


def _skew(theta, b):
    q = np.zeros((b, b))
    iu = np.triu_indices(b, 1)
    q[iu] = theta
    return q - q.T


@pytest.mark.parametrize("b,std", [(8, 0.3), (16, 0.1), (32, 0.05)])
def test_fused_cnp_backward_regrouping(b, std):
    """The fused CNP backward (one row panel of Qbar^T per workgroup): with U_j = Q^j[C,:]
    and W_0 = Gb^T[C,:], W_j = W_{j-1} Q + U_j Gb^T (j = 1..3) and
    Qbar^T[C,:] = W_3 + 2 (W_0 + W_1 + W_2); dtheta = (Qbar - Qbar^T) on the strict upper
    triangle.  Computed here on row panels of 4 rows, against the oracle's eq. 9 adjoint."""
    rng = np.random.default_rng(b)
    p = b * (b - 1) // 2
    theta = rng.standard_normal((1, p)) * std
    gb = rng.standard_normal((1, b, b))
    q = _skew(theta[0], b)
    qbar_t = np.zeros((b, b))
    for r0 in range(0, b, 4):
        rows = slice(r0, r0 + 4)
        u = q[rows].copy()                    # U_1
        w = gb[0].T[rows].copy()              # W_0
        run = 2 * w
        for j in range(1, 4):
            w, u = w @ q + u @ gb[0].T, u @ q  # W_j, U_{j+1}
            if j < 3:
                run += 2 * w
        qbar_t[rows] = w + run
    qbar = qbar_t.T
    iu = np.triu_indices(b, 1)
    got = (qbar - qbar.T)[iu]
    ref = O.cnp_backward(theta, gb, b)[0]
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_fused_regrouping_detects_a_wrong_term():
    """The check above is sensitive: dropping the U_j Gb^T terms changes the result."""
    b = 16
    rng = np.random.default_rng(0)
    theta = rng.standard_normal((1, b * (b - 1) // 2)) * 0.1
    gb = rng.standard_normal((1, b, b))
    q = _skew(theta[0], b)
    w = gb[0].T.copy()
    run = 2 * w
    for j in range(1, 4):
        w = w @ q                             # U_j Gb^T dropped
        if j < 3:
            run += 2 * w
    qbar = (w + run).T
    iu = np.triu_indices(b, 1)
    ref = O.cnp_backward(theta, gb, b)[0]
    assert np.max(np.abs((qbar - qbar.T)[iu] - ref)) > 1e-3 * np.max(np.abs(ref))
