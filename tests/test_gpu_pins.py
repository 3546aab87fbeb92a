"""GPU half of the theta = 0 pins: with every Q = 0 the CNP gives G = I exactly, and the
POET-X layer reduces to a plain linear layer (POET-X summary page, Method §1, eq. 3: the
orthogonal factors are identities; Method §2: the merged permutations cancel; Method §6:
an int8 weight with row scales is the dequantized weight).  So, checked against a library
matmul in float64 (not against the oracle):

  * Z = X W^T, with and without the activation permutations (bf16 and int8 weights);
  * dX = dZ W;
  * dG_P = B~^T dZ~ per block with B~ = X~ W'^T, and the CNP backward's closed form at
    Q = 0: dtheta[k(i, j)] = 2 (dG[i][j] - dG[j][i]).

The kernels round to bf16 once per stored intermediate.  At G = I the block products are
exact (a product with 1 and zeros, accumulated in float32), so Z carries exactly one
rounding, of the W' product's float32 sum: |Z - ref| <= ulp_bf16(ref) / 2 plus the
float32 accumulation error, bounded here by 2^-16 sum_k |x_k| |w_k| (the typical error of
a 4096-term float32 sum is about 64 x 2^-24 of that).  dX of an int8 layer carries a
second rounding (of dB' = dZ~ diag(s'), the row scales folded into the W' product's left
operand, each element within 2^-8 of itself): 2^-8 sum_k |dz_k s_k| |q_k| more.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from orthogonal_reparameterized_amd import workloads as WL  # noqa: E402
from tests.helpers import bf16_ulp, norm_max_err, to_host_f64  # noqa: E402


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from orthogonal_reparameterized_amd import binding
    return binding


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _zero_theta(inp):
    out = dict(inp)
    out["theta_r"] = np.zeros_like(inp["theta_r"])
    out["theta_p"] = np.zeros_like(inp["theta_p"])
    return out


def _weight(wl, inp):
    """The layer's weight in original coordinates, float64 (int8: q times its row scale)."""
    if wl.w == "i8":
        return inp["w_q"].astype(np.float64) * inp["w_s"].astype(np.float64)[:, None]
    return WL.to_f64(inp["w"], wl.w)


def _rows(n, count=384):
    """Sampled token rows: spread over the whole batch, the first and the last included."""
    r = np.unique(np.concatenate([np.linspace(0, n - 1, count).astype(np.int64), [0, n - 1]]))
    return r


CASES = [
    # (workload key, activation permutations)
    (3, True), (3, False), (5, True), (5, False),
]


@pytest.mark.parametrize("key,perms", CASES)
def test_theta_zero_layer_is_linear(B, key, perms):
    """Full-size workloads 3 (bf16) and 5 (int8) at theta = 0: Z = X W^T and dX = dZ W on
    sampled token rows, element by element, within one bf16 rounding (two for the int8 dX)."""
    from orthogonal_reparameterized_amd.step import LayerStep
    wl = WL.WORKLOADS[key]
    inp = _zero_theta(WL.make_layer_inputs(wl, perms=perms))
    variant = "mem" if wl.w == "i8" else "fast"
    _say(f"theta = 0 pin: workload {key} perms={perms} {variant}")
    st = LayerStep(wl, inp, variant, perms=perms)
    out = st.step(want_dg=True)
    torch.cuda.synchronize()
    # G = I bitwise (the CNP at Q = 0)
    eye = torch.eye(wl.b, dtype=torch.float32)
    for g in (st.g_r, st.g_p):
        assert torch.equal(g.float().cpu(), eye.expand(g.shape[0], wl.b, wl.b))
    rows = _rows(wl.n_tokens)
    sel = torch.from_numpy(rows).cuda()
    w = _weight(wl, inp)
    x = WL.to_f64(inp["x"], wl.act)[rows]
    dz = WL.to_f64(inp["dz"], wl.act)[rows]
    z_ref = x @ w.T
    dx_ref = dz @ w
    z = to_host_f64(st.z[sel])
    dx = to_host_f64(out["dx"][sel])
    z_bound = 0.5 * bf16_ulp(z_ref) + 2.0 ** -16 * (np.abs(x) @ np.abs(w).T)
    if wl.w == "i8":
        q, s = inp["w_q"].astype(np.float64), inp["w_s"].astype(np.float64)
        dx_bound = (bf16_ulp(dx_ref) + 2.0 ** -16 * (np.abs(dz) @ np.abs(w))
                    + 2.0 ** -8 * ((np.abs(dz) * s[None, :]) @ np.abs(q)))
    else:
        dx_bound = 0.5 * bf16_ulp(dx_ref) + 2.0 ** -16 * (np.abs(dz) @ np.abs(w))
    zerr, dxerr = np.abs(z - z_ref), np.abs(dx - dx_ref)
    _say(f"  Z: max |err|/bound {np.max(zerr / z_bound):.3f}, dX: {np.max(dxerr / dx_bound):.3f}")
    assert np.all(zerr <= z_bound)
    assert np.all(dxerr <= dx_bound)


@pytest.mark.parametrize("w_dtype,perms", [("bf16", True), ("bf16", False), ("i8", True)])
def test_theta_zero_gradients_closed_form(B, w_dtype, perms):
    """257 tokens, 512 -> 768, b = 256 at theta = 0: Z, dX, dG_P, dG_R and both dtheta against
    the closed forms built from library matmuls (2e-2 layer bar for the gradients, whose
    inputs B~ and dA carry a bf16 rounding each)."""
    from orthogonal_reparameterized_amd.step import LayerStep
    variants = ("mem",) if w_dtype == "i8" else ("fast", "mem")
    wl = WL.Workload(88, "pin small", 257, 512, 768, 256, "bf16", w_dtype, "bf16", 0.01, 512,
                     perms=perms, variants=variants)
    inp = _zero_theta(WL.make_layer_inputs(wl))
    w = _weight(wl, inp)
    x = WL.to_f64(inp["x"], "bf16")
    dz = WL.to_f64(inp["dz"], "bf16")
    pin = inp["perm_in"] if perms else np.arange(wl.d_in)
    pout = inp["perm_out"] if perms else np.arange(wl.d_out)
    wm = w[np.ix_(pout, pin)]                       # W' = Psi_out W Psi_in^T
    xg, dzg = x[:, pin], dz[:, pout]                # X~, dZ~
    bt = xg @ wm.T                                  # B~ = X~ W'^T
    da = dzg @ wm                                   # dA = dZ~ W'
    b = wl.b

    def blockgrad(left, right, d):
        return np.stack([left[:, j * b:(j + 1) * b].T @ right[:, j * b:(j + 1) * b] for j in range(d // b)])

    def dtheta(dg):
        iu = np.triu_indices(b, 1)
        return np.stack([2.0 * (g[iu] - g.T[iu]) for g in dg])

    ref = {"Z": x @ w.T, "dX": dz @ w, "dG_P": blockgrad(bt, dzg, wl.d_out), "dG_R": blockgrad(xg, da, wl.d_in)}
    ref["dtheta_P"], ref["dtheta_R"] = dtheta(ref["dG_P"]), dtheta(ref["dG_R"])
    for variant in variants:
        st = LayerStep(wl, inp, variant, perms=perms)
        out = st.step(want_dg=True)
        torch.cuda.synchronize()
        got = {"Z": st.z, "dX": out["dx"], "dG_P": out["dg_p"], "dG_R": out["dg_r"],
               "dtheta_P": out["dtheta_p"], "dtheta_R": out["dtheta_r"]}
        errs = {k: norm_max_err(to_host_f64(got[k]), ref[k]) for k in ref}
        _say(f"theta = 0 closed forms {w_dtype} perms={perms} {variant}: {errs}")
        for k, e in errs.items():
            assert e <= 2e-2, (variant, k, e)
        # Z has exactly one rounding here too
        assert np.all(np.abs(to_host_f64(st.z) - ref["Z"])
                      <= 0.5 * bf16_ulp(ref["Z"]) + 2.0 ** -16 * (np.abs(x) @ np.abs(w).T))
