"""GPU parity of the packed-parameter options: theta stored in bf16 (the CNP widens it
exactly and computes in float32), and the Adam update fused into the CNP backward's last
pass (poetx_backward_adam), each against the fp64 oracle (POET-X summary page, Method §4:
packed theta and optimizer state on the b(b-1)/2 parameters; practical advice 3: the
learning-rate scale gamma).

Bars: fp32 CNP outputs 1e-5 relative Frobenius per block; bf16 G within one bf16 ulp; bf16
layer outputs and gradients 2e-2 normalized max; Adam state to rtol 1e-5 (float32
arithmetic); a bf16 theta within one bf16 ulp of the oracle's exact update of the same
starting values (the update is computed in float32, then rounded once).
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from oracle import poetx_oracle as O  # noqa: E402
from orthogonal_reparameterized_amd import workloads as WL  # noqa: E402
from tests.helpers import (bf16_ulp, flat, norm_max_err, oracle_layer, rel_fro_per_block,  # noqa: E402
                           to_host_f64)

TOL_BF16 = 2e-2
TOL_CNP_F32 = 1e-5


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from orthogonal_reparameterized_amd import binding
    return binding


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf16_theta(inp):
    """The inputs with theta rounded to bf16 (bit patterns), and the exact values as fp32."""
    out = dict(inp)
    for k in ("theta_r", "theta_p"):
        bits = WL.f32_to_bf16_bits(inp[k])
        out[k] = bits
        out[k + "_f32"] = WL.bf16_bits_to_f32(bits)
    return out


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("n,b", [(11, 64), (5, 256), (2, 512), (6, 48), (3, 160)])
def test_cnp_bf16_theta(B, n, b):
    """CNP forward (fp32 and bf16 G) and backward from a bf16 theta: the oracle on the same
    (exactly widened) values."""
    theta, dg = WL.make_cnp_inputs(n, b, 0.02, seed=500 + b)
    bits = WL.f32_to_bf16_bits(theta)
    exact = WL.bf16_bits_to_f32(bits).astype(np.float64)
    th = _bf16_dev(bits)
    g32 = B.poetx_cnp(B.POETX_CNP_FWD, th, b, g_dtype=torch.float32)
    g16 = B.poetx_cnp(B.POETX_CNP_FWD, th, b, g_dtype=torch.bfloat16)
    d = B.poetx_cnp(B.POETX_CNP_BWD, th, b, dg=torch.from_numpy(dg).cuda())
    torch.cuda.synchronize()
    assert d.dtype == torch.float32
    ref = O.cnp_forward(exact, b)
    assert rel_fro_per_block(to_host_f64(g32), ref) <= TOL_CNP_F32
    assert np.all(np.abs(to_host_f64(g16) - ref) <= np.maximum(bf16_ulp(ref), 2.0 ** -20))
    ref_d = O.cnp_backward(exact, dg.astype(np.float64), b)
    assert rel_fro_per_block(to_host_f64(d), ref_d) <= TOL_CNP_F32


@pytest.mark.parametrize("n,b", [(600, 256), (1100, 64), (40, 128)])
def test_cnp_bf16_theta_many_blocks(B, n, b):
    """bf16 theta where the row-panel kernels take many blocks (600 of 256 and 1100 of 64:
    64- and 32-row panels) and few (40 of 128: 32-row panels).  With bf16 theta the
    kernels drop Q's lo plane and its MFMA pass (Q is exact in bf16); sampled blocks against
    the oracle, and the saved-Q backward bitwise equal to the one that unpacks theta."""
    theta, dg = WL.make_cnp_inputs(n, b, 0.02, seed=700 + b)
    bits = WL.f32_to_bf16_bits(theta)
    exact = WL.bf16_bits_to_f32(bits).astype(np.float64)
    th = _bf16_dev(bits)
    dgt = torch.from_numpy(dg).cuda()
    q = B.qsave_like(th, b)
    g32 = B.poetx_cnp(B.POETX_CNP_FWD, th, b, g_dtype=torch.float32, qsave=q)
    d0 = B.poetx_cnp(B.POETX_CNP_BWD, th, b, dg=dgt)
    d1 = B.poetx_cnp(B.POETX_CNP_BWD, th, b, dg=dgt, qsave=q)
    torch.cuda.synchronize()
    _say(f"cnp bf16 theta n={n} b={b}")
    assert torch.equal(d0.view(torch.int32), d1.view(torch.int32))
    idx = np.array([0, 1, n // 2, n - 1])
    sel = torch.from_numpy(idx).cuda()
    assert rel_fro_per_block(to_host_f64(g32[sel]), O.cnp_forward(exact[idx], b)) <= TOL_CNP_F32
    ref_d = O.cnp_backward(exact[idx], dg[idx].astype(np.float64), b)
    assert rel_fro_per_block(to_host_f64(d1[sel]), ref_d) <= TOL_CNP_F32


LAYERS = [
    # (n_tokens, d_in, d_out, b): the chains and the MFMA block kernels; smaller last blocks
    (257, 512, 768, 256),
    (130, 640, 896, 256),
]


@pytest.mark.parametrize("n,d_in,d_out,b", LAYERS)
@pytest.mark.parametrize("variant", ["fast", "mem"])
def test_layer_bf16_theta(B, n, d_in, d_out, b, variant):
    from orthogonal_reparameterized_amd.step import LayerStep
    wl = WL.Workload(87, "bf16 theta", n, d_in, d_out, b, "bf16", "bf16", "bf16", 0.02, d_in)
    inp = _bf16_theta(WL.make_layer_inputs(wl))
    ref = oracle_layer(dict(inp, theta_r=inp["theta_r_f32"], theta_p=inp["theta_p_f32"]), wl)
    st = LayerStep(wl, inp, variant, theta_dtype="bf16")
    out = st.step(want_dg=True)
    torch.cuda.synchronize()
    assert st.theta_r.dtype == torch.bfloat16 and out["dtheta_r"].dtype == torch.float32
    errs = {k: norm_max_err(flat(to_host_f64(v)), flat(ref[r])) for k, v, r in
            (("Z", st.z, "Z"), ("dX", out["dx"], "dX"), ("dtheta_R", out["dtheta_r"], "dtheta_R"),
             ("dtheta_P", out["dtheta_p"], "dtheta_P"), ("G_R", st.g_r, "G_R"))}
    _say(f"bf16 theta {d_in}->{d_out} b={b} {variant}: {errs}")
    for k, e in errs.items():
        assert e <= TOL_BF16, (k, e)


def test_layer_bf16_theta_workload3(B):
    """Workload 3 at full size with a bf16 theta, fast variant, every output element."""
    from orthogonal_reparameterized_amd.step import LayerStep
    wl = WL.WORKLOADS[3]
    inp = _bf16_theta(WL.make_layer_inputs(wl))
    _say("bf16 theta workload 3: oracle ...")
    ref = oracle_layer(dict(inp, theta_r=inp["theta_r_f32"], theta_p=inp["theta_p_f32"]), wl)
    st = LayerStep(wl, inp, "fast", theta_dtype="bf16", transposed_weight=True)
    out = st.step()
    torch.cuda.synchronize()
    for k, v, r in (("Z", st.z, "Z"), ("dX", out["dx"], "dX"), ("dtheta_R", out["dtheta_r"], "dtheta_R"),
                    ("dtheta_P", out["dtheta_p"], "dtheta_P")):
        e = norm_max_err(flat(to_host_f64(v)), flat(ref[r]))
        _say(f"  {k}: {e:.2e}")
        assert e <= TOL_BF16, (k, e)


HP = dict(lr=1e-3, betas=(0.9, 0.999), eps=1e-8, gamma=0.5)


def _f32(x):
    return float(np.float32(x))


def _oracle_adam(theta, g, m, v, t):
    """The oracle's Adam step on the kernel's own float32 hyperparameter values."""
    return O.adam_step(theta, g, m, v, _f32(HP["lr"]), _f32(HP["betas"][0]), _f32(HP["betas"][1]), _f32(HP["eps"]),
                       t, _f32(HP["gamma"]))


def _close_state(got, ref):
    """Adam state from float32 arithmetic: each element within 1e-5 of itself, or within
    2^-20 of the largest (m = b1 m + (1 - b1) g cancels to near zero for some elements,
    where float32 rounding of the operands, 2^-24 of their size, dominates)."""
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=2.0 ** -20 * float(np.max(np.abs(ref))))


@pytest.mark.parametrize("n", [5, 4096 + 3])
def test_adam_step_bf16_theta(B, n):
    """poetx_adam_step on a bf16 theta, three steps: each step's new theta within one bf16
    ulp of the oracle's exact update of the step's starting values; m, v to rtol 1e-5."""
    rng = np.random.default_rng(61)
    th = _bf16_dev(WL.f32_to_bf16_bits((rng.standard_normal(n) * 0.01).astype(np.float32)))
    m, v = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    for t in range(1, 4):
        g = (rng.standard_normal(n) * 0.1).astype(np.float32)
        th0, m0, v0 = to_host_f64(th), to_host_f64(m), to_host_f64(v)
        B.poetx_adam_step(th, torch.from_numpy(g).cuda(), m, v, lr=HP["lr"], step=t, betas=HP["betas"],
                          eps=HP["eps"], gamma=HP["gamma"])
        torch.cuda.synchronize()
        rt, rm, rv = _oracle_adam(th0, g, m0, v0, t)
        assert np.all(np.abs(to_host_f64(th) - rt) <= bf16_ulp(rt)), t
        _close_state(to_host_f64(m), rm)
        _close_state(to_host_f64(v), rv)


FUSED = [
    # (workload / shape, theta dtype): the chains (b = 256), smaller last blocks, the
    # float32 vector-ALU layer (workload 1, b = 32)
    ((257, 512, 768, 256, "bf16"), "f32"),
    ((257, 512, 768, 256, "bf16"), "bf16"),
    ((130, 640, 896, 256, "bf16"), "f32"),
    # last blocks of 232 and 248 (padded CNP blocks; the update as its own pass)
    ((200, 1000, 2040, 256, "bf16"), "f32"),
    ((200, 1000, 2040, 256, "bf16"), "bf16"),
    ((64, 256, 256, 32, "f32"), "f32"),
]


@pytest.mark.parametrize("shape,tdt", FUSED)
@pytest.mark.parametrize("variant", ["fast", "mem"])
def test_backward_adam_fused(B, shape, tdt, variant):
    """poetx_backward_adam over three steps: the layer's dX and dtheta against the oracle's
    step on the current theta, and theta, m, v against the oracle's Adam of that dtheta
    applied to the same starting values (a bf16 theta within one bf16 ulp)."""
    from orthogonal_reparameterized_amd.step import LayerStep
    n, d_in, d_out, b, act = shape
    wl = WL.Workload(86, "fused adam", n, d_in, d_out, b, act, act, act, 0.02, d_in)
    inp = WL.make_layer_inputs(wl)
    if tdt == "bf16":
        inp = _bf16_theta(inp)
    st = LayerStep(wl, inp, variant, theta_dtype=tdt)
    tol = TOL_BF16 if act == "bf16" else 1e-4
    for t in range(1, 4):
        th_r0, th_p0 = to_host_f64(st.theta_r), to_host_f64(st.theta_p)
        state0 = [to_host_f64(getattr(st.adam, k)) if st.adam else np.zeros(th.size)
                  for k, th in (("m_r", th_r0), ("v_r", th_r0), ("m_p", th_p0), ("v_p", th_p0))]
        out = st.step_adam(keep_dtheta=True, **HP)
        torch.cuda.synchronize()
        shp_r, shp_p = np.shape(inp["theta_r"]), np.shape(inp["theta_p"])
        ref = oracle_layer(dict(inp, theta_r=th_r0.reshape(shp_r).astype(np.float32),
                                theta_p=th_p0.reshape(shp_p).astype(np.float32)), wl)
        e = {"dX": norm_max_err(to_host_f64(out["dx"]), ref["dX"]),
             "dtheta_R": norm_max_err(flat(to_host_f64(out["dtheta_r"])), flat(ref["dtheta_R"])),
             "dtheta_P": norm_max_err(flat(to_host_f64(out["dtheta_p"])), flat(ref["dtheta_P"]))}
        _say(f"fused adam {d_in}->{d_out} b={b} theta {tdt} {variant} step {t}: {e}")
        for k, v in e.items():
            assert v <= tol, (t, k, v)
        # the update of the kernel's own gradient, element by element
        for side, th0, mi, vi in (("r", th_r0, 0, 1), ("p", th_p0, 2, 3)):
            g = to_host_f64(getattr(st, "dtheta_" + side)).ravel()
            rt, rm, rv = _oracle_adam(th0.ravel(), g, state0[mi].ravel(), state0[vi].ravel(), t)
            got_t = to_host_f64(getattr(st, "theta_" + side)).ravel()
            if tdt == "bf16":
                assert np.all(np.abs(got_t - rt) <= bf16_ulp(rt)), (t, side)
            else:
                np.testing.assert_allclose(got_t, rt, rtol=1e-5, atol=1e-7)
            _close_state(to_host_f64(getattr(st.adam, "m_" + side)).ravel(), rm)
            _close_state(to_host_f64(getattr(st.adam, "v_" + side)).ravel(), rv)


def test_backward_adam_matches_separate_pass(B):
    """Workload 3 at full size: the fused update equals poetx_backward followed by
    poetx_adam_step on the same dtheta (the same float32 operations), at step 1 and, from
    the step-1 state of the separate pass copied into both, at step 2."""
    from orthogonal_reparameterized_amd.step import LayerStep
    wl = WL.WORKLOADS[3]
    inp = WL.make_layer_inputs(wl)
    fused = LayerStep(wl, inp, "fast", transposed_weight=True)
    sep = LayerStep(wl, inp, "fast", transposed_weight=True)
    st_sep = B.AdamState.zeros_like(sep.layer)
    for t in range(1, 3):
        fused.step_adam(keep_dtheta=True, **HP)
        out = sep.step()
        for side in ("r", "p"):
            B.poetx_adam_step(getattr(sep, "theta_" + side), out["dtheta_" + side], getattr(st_sep, "m_" + side),
                              getattr(st_sep, "v_" + side), lr=HP["lr"], step=t, betas=HP["betas"], eps=HP["eps"],
                              gamma=HP["gamma"])
        torch.cuda.synchronize()
        for side in ("r", "p"):
            # the same theta in: the same kernels give the same gradient
            assert torch.equal(fused.dtheta_r if side == "r" else fused.dtheta_p, out["dtheta_" + side])
            a, c = getattr(fused, "theta_" + side), getattr(sep, "theta_" + side)
            assert torch.allclose(a, c, rtol=1e-6, atol=1e-9), (t, side, (a - c).abs().max().item())
            for k in ("m_", "v_"):
                x, y = getattr(fused.adam, k + side), getattr(st_sep, k + side)
                assert torch.allclose(x, y, rtol=1e-6, atol=1e-6 * y.abs().max().item()), (t, k + side)
            # both continue from the same state
            a.copy_(c)
            getattr(fused.adam, "m_" + side).copy_(getattr(st_sep, "m_" + side))
            getattr(fused.adam, "v_" + side).copy_(getattr(st_sep, "v_" + side))
    _say("fused Adam = separate pass at workload 3")
