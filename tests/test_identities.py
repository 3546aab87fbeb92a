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


def _five_product_e(q, gb, rows_per_panel=4):
    """E of the five-product CNP backward, one row panel C at a time as the kernel runs it:
    1a Q[C] H and Q[C] K, 1b H[C] Q, J[C] = 2K[C] - H[C]Q - Q[C]H, F[C] = -2H[C] + Q[C]K +
    J[C]Q, E[C] = K[C] + F[C]Q, with K = Gb - Gb^T and H = Gb + Gb^T."""
    b = q.shape[0]
    k, h = gb - gb.T, gb + gb.T
    e = np.zeros((b, b))
    for r0 in range(0, b, rows_per_panel):
        c = slice(r0, r0 + rows_per_panel)
        qh, qk = q[c] @ h, q[c] @ k          # 1a
        hq = h[c] @ q                         # 1b
        j = 2 * k[c] - hq - qh
        f = -2 * h[c] + qk + j @ q            # 2
        e[c] = k[c] + f @ q                   # 3
    return e


@pytest.mark.parametrize("b,std", [(8, 0.3), (16, 0.1), (32, 0.05)])
def test_five_product_cnp_backward(b, std):
    """The CNP backward's five products: E - E^T on the strict upper triangle is dtheta, the
    skew part of the adjoint of eq. 9 (Qbar - Qbar^T), against the oracle's adjoint."""
    rng = np.random.default_rng(b)
    p = b * (b - 1) // 2
    theta = rng.standard_normal((1, p)) * std
    gb = rng.standard_normal((1, b, b))
    e = _five_product_e(_skew(theta[0], b), gb[0])
    iu = np.triu_indices(b, 1)
    got = (e - e.T)[iu]
    ref = O.cnp_backward(theta, gb, b)[0]
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("drop", ["qk", "jq", "sign_k"])
def test_five_product_form_detects_a_wrong_term(drop):
    """The check above is sensitive: a dropped product or a transposed K changes dtheta."""
    b = 16
    rng = np.random.default_rng(0)
    theta = rng.standard_normal((1, b * (b - 1) // 2)) * 0.1
    gb = rng.standard_normal((1, b, b))
    q = _skew(theta[0], b)
    k, h = gb[0] - gb[0].T, gb[0] + gb[0].T
    if drop == "sign_k":
        k = -k
    j = 2 * k - h @ q - q @ h
    f = -2 * h + (0 if drop == "qk" else q @ k) + (0 if drop == "jq" else j @ q)
    e = k + f @ q
    iu = np.triu_indices(b, 1)
    ref = O.cnp_backward(theta, gb, b)[0]
    assert np.max(np.abs((e - e.T)[iu] - ref)) > 1e-3 * np.max(np.abs(ref))
