"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Tolerances (from the arithmetic: float32 products accumulate to about 1e-6 relative, and one
bf16 rounding of an operand or result costs up to 2^-9 = 2e-3 relative, a few of them per step):
  * float32 CNP outputs (G in fp32, dtheta from an identical dG): max over blocks
    of the relative Frobenius error <= 1e-5.
  * bf16 G: every element within one bf16 ulp of the oracle's value (absolute
    floor 2^-20 for entries near zero).
  * bf16 layer outputs and gradients: ||got - ref||_inf / ||ref||_inf <= 2e-2.
  * float32 layer (workload 1): the same metric <= 1e-4.
  * integer / byte work (the permutation merge): bit-exact.
"""

import functools
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from oracle import poetx_oracle as O  # noqa: E402
from orthogonal_reparameterized_amd import workloads as WL  # noqa: E402
from tests.helpers import (bf16_ulp, flat, norm_max_err, oracle_layer, rel_fro,  # noqa: E402
                           rel_fro_per_block, split_g, to_host_f64)

TOL_BF16 = 2e-2
TOL_F32_LAYER = 1e-4
TOL_CNP_F32 = 1e-5


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from orthogonal_reparameterized_amd import binding
    return binding


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ------------------------------------------------------------------- CNP ----

# b = 64..512 run the row-panel kernels (the forward chain, the five-product backward;
# n = 11 and 19 also cover the blocks past the last full group of 8 in the workgroup order),
# b = 192 the per-product MFMA path, b = 100, 200 and 300 the row-panel kernels on blocks
# padded to 128, 256 and 512, b = 32 and 48 the float32 vector-ALU path
CNP_CASES = [(8, 32, 0.02), (11, 64, 0.03), (19, 128, 0.02), (3, 192, 0.01), (3, 256, 0.01),
             (2, 512, 0.01), (2, 1024, 0.005),
             # enough blocks for the 64-row panels (4 workgroups per CU): 517 = 8 * 64 + 5
             # also leaves blocks past the last full group of 8
             (517, 128, 0.02), (256, 256, 0.01),
             # more blocks of 256 and 512 (several rounds of workgroups)
             (600, 256, 0.01), (40, 512, 0.01),
             # block sizes without kernels of their own (padded blocks)
             (3, 100, 0.02), (9, 200, 0.01), (2, 300, 0.01)]


@pytest.mark.parametrize("n,b,std", CNP_CASES + [(5, 48, 0.05)])
def test_cnp_forward_f32(B, n, b, std):
    _say(f"cnp fwd f32 n={n} b={b}")
    theta, _ = WL.make_cnp_inputs(n, b, std, seed=100 + b)
    g = B.poetx_cnp(B.POETX_CNP_FWD, torch.from_numpy(theta).cuda(), b, g_dtype=torch.float32)
    ref = O.cnp_forward(theta.astype(np.float64), b)
    assert rel_fro_per_block(to_host_f64(g), ref) <= TOL_CNP_F32


@pytest.mark.parametrize("n,b", [(9, 64), (4, 128), (4, 256), (2, 512), (3, 160)])
def test_cnp_forward_bf16_ulp(B, n, b):
    _say(f"cnp fwd bf16 n={n} b={b}")
    theta, _ = WL.make_cnp_inputs(n, b, 0.01, seed=200 + b)
    g = B.poetx_cnp(B.POETX_CNP_FWD, torch.from_numpy(theta).cuda(), b, g_dtype=torch.bfloat16)
    ref = O.cnp_forward(theta.astype(np.float64), b)
    got = to_host_f64(g)
    bound = np.maximum(bf16_ulp(ref), 2.0 ** -20)
    assert np.all(np.abs(got - ref) <= bound)


def test_cnp_size_one_blocks(B):
    """Blocks of size 1 have no parameters: G = [1] in either dtype, no gradient entries."""
    th = torch.zeros((5, 0), device="cuda")
    for dt in (torch.float32, torch.bfloat16):
        g = B.poetx_cnp(B.POETX_CNP_FWD, th, 1, g_dtype=dt)
        assert torch.equal(g.float().cpu(), torch.ones(5, 1, 1))
    d = B.poetx_cnp(B.POETX_CNP_BWD, th, 1, dg=torch.ones((5, 1, 1), device="cuda"))
    assert d.shape == (5, 0)


def test_cnp_zero_is_identity(B):
    b = 256
    th = torch.zeros((3, b * (b - 1) // 2), device="cuda")
    for dt in (torch.float32, torch.bfloat16):
        g = B.poetx_cnp(B.POETX_CNP_FWD, th, b, g_dtype=dt)
        assert torch.equal(g.float().cpu(), torch.eye(b).expand(3, b, b))


@pytest.mark.parametrize("n,b,std", CNP_CASES)
def test_cnp_backward_f32(B, n, b, std):
    _say(f"cnp bwd f32 n={n} b={b}")
    theta, dg = WL.make_cnp_inputs(n, b, std, seed=300 + b)
    d = B.poetx_cnp(B.POETX_CNP_BWD, torch.from_numpy(theta).cuda(), b, dg=torch.from_numpy(dg).cuda())
    ref = O.cnp_backward(theta.astype(np.float64), dg.astype(np.float64), b)
    assert rel_fro_per_block(to_host_f64(d), ref) <= TOL_CNP_F32


def test_cnp_workload2_sampled(B):
    """Workload 2 at full size (4096 blocks, b=256): G and dtheta on sampled blocks."""
    wl = WL.WORKLOADS[2]
    _say("cnp workload 2 full size")
    theta, dg = WL.make_cnp_inputs(wl.nblocks, wl.b, wl.theta_std, seed=WL.BASE_SEED + 2)
    th_d = torch.from_numpy(theta).cuda()
    g = B.poetx_cnp(B.POETX_CNP_FWD, th_d, wl.b, g_dtype=torch.bfloat16)
    d = B.poetx_cnp(B.POETX_CNP_BWD, th_d, wl.b, dg=torch.from_numpy(dg).cuda())
    torch.cuda.synchronize()
    idx = np.array([0, 1, 777, 2048, 4095])
    ref_g = O.cnp_forward(theta[idx].astype(np.float64), wl.b)
    got_g = to_host_f64(g[torch.from_numpy(idx).cuda()])
    assert np.all(np.abs(got_g - ref_g) <= np.maximum(bf16_ulp(ref_g), 2.0 ** -20))
    ref_d = O.cnp_backward(theta[idx].astype(np.float64), dg[idx].astype(np.float64), wl.b)
    assert rel_fro_per_block(to_host_f64(d[torch.from_numpy(idx).cuda()]), ref_d) <= TOL_CNP_F32


def test_layer_cnp_backward_two_sides_one_launch(B):
    """A layer wide enough (32768 -> 32768, b = 256: 128 + 128 blocks) that its CNP backward
    runs the five-product kernel over both sides in one launch of 64-row panels.  The layer's dtheta on sampled
    blocks of each side against the oracle's CNP backward of the dG the layer itself
    reports; W, x and dz are drawn on the GPU (their values do not enter the check)."""
    torch.manual_seed(11)
    d, b, n = 32768, 256, 64
    nb = d // b
    p = b * (b - 1) // 2
    rng = np.random.default_rng(12)
    th_r = (rng.standard_normal((nb, p)) * 0.01).astype(np.float32)
    th_p = (rng.standard_normal((nb, p)) * 0.01).astype(np.float32)
    tr, tp = torch.from_numpy(th_r).cuda(), torch.from_numpy(th_p).cuda()
    w = (torch.randn(d, d, device="cuda", dtype=torch.bfloat16) * d ** -0.5)
    g_r = B.poetx_cnp(B.POETX_CNP_FWD, tr, b, g_dtype=torch.bfloat16)
    g_p = B.poetx_cnp(B.POETX_CNP_FWD, tp, b, g_dtype=torch.bfloat16)
    L = B.Layer(w, tr, tp, g_r, g_p, b, act_dtype=torch.bfloat16, variant=B.POETX_FAST)
    x = torch.randn(n, d, device="cuda", dtype=torch.bfloat16)
    dz = torch.randn(n, d, device="cuda", dtype=torch.bfloat16)
    _say("cnp backward, two sides in one launch: layer 32768 -> 32768")
    _, sb = B.poetx_forward(L, x)
    torch.cuda.synchronize()
    B.prof_read()
    B.prof_enable(True)
    out = B.poetx_backward(L, x, dz, sb, want_dg=True)
    torch.cuda.synchronize()
    B.prof_enable(False)
    assert "cnp_bwd5" in B.prof_read()  # the launch this test is for
    idx = np.array([0, 1, 77, nb - 1])
    for th, key_g, key_t in ((th_r, "dg_r", "dtheta_r"), (th_p, "dg_p", "dtheta_p")):
        dg = out[key_g][torch.from_numpy(idx).cuda()].double().cpu().numpy()
        ref = O.cnp_backward(th[idx].astype(np.float64), dg, b)
        got = out[key_t][torch.from_numpy(idx).cuda()].double().cpu().numpy()
        assert rel_fro_per_block(got, ref) <= TOL_CNP_F32, key_t


@pytest.mark.parametrize("n,b", [(40, 256), (600, 256), (70, 64), (24, 512), (3, 96), (5, 48)])
def test_cnp_saved_q_is_transparent(B, n, b):
    """poetx_cnp's qsave (Q's planes kept by the forward, read by the backward instead of
    unpacking theta again) changes nothing: G and dtheta are bitwise those of calls without
    it, on the row-panel paths (40 blocks of 256: 32-row panels; 600: 64-row panels;
    b = 64, 512), and where qsave is ignored (b = 96 and 48, which take the padded
    row-panel and the vector-ALU paths)."""
    _say(f"cnp saved Q n={n} b={b}")
    theta, dg = WL.make_cnp_inputs(n, b, 0.01, seed=900 + b)
    th = torch.from_numpy(theta).cuda()
    dgt = torch.from_numpy(dg).cuda()
    q = B.qsave_like(th, b)
    g0 = B.poetx_cnp(B.POETX_CNP_FWD, th, b, g_dtype=torch.bfloat16)
    g1 = B.poetx_cnp(B.POETX_CNP_FWD, th, b, g_dtype=torch.bfloat16, qsave=q)
    d0 = B.poetx_cnp(B.POETX_CNP_BWD, th, b, dg=dgt)
    d1 = B.poetx_cnp(B.POETX_CNP_BWD, th, b, dg=dgt, qsave=q)
    torch.cuda.synchronize()
    assert torch.equal(g0.view(torch.int16), g1.view(torch.int16))
    assert torch.equal(d0.view(torch.int32), d1.view(torch.int32))
    # and the backward with qsave matches the oracle
    idx = np.array([0, n - 1])
    ref = O.cnp_backward(theta[idx].astype(np.float64), dg[idx].astype(np.float64), b)
    assert rel_fro_per_block(to_host_f64(d1[torch.from_numpy(idx).cuda()]), ref) <= TOL_CNP_F32


def test_layer_saved_q_is_transparent(B):
    """A layer step whose CNP forward keeps Q's planes for the backward (the layer's q_r /
    q_p) gives bitwise the results of one that unpacks theta again, fast and mem."""
    from orthogonal_reparameterized_amd.step import LayerStep
    wl = WL.Workload(89, "saved q", 300, 512, 768, 256, "bf16", "bf16", "bf16", 0.01, 512)
    inp = WL.make_layer_inputs(wl)
    for variant in ("fast", "mem"):
        outs = []
        for save_q in (False, True):
            st = LayerStep(wl, inp, variant, save_q=save_q)
            out = st.step(want_dg=True)
            torch.cuda.synchronize()
            outs.append({"z": st.z.clone(), "dx": out["dx"].clone(), "dtheta_r": out["dtheta_r"].clone(),
                         "dtheta_p": out["dtheta_p"].clone()})
        _say(f"layer saved Q {variant}")
        for k in outs[0]:
            a, c = outs[0][k], outs[1][k]
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               c.view(torch.int16) if c.dtype == torch.bfloat16 else c.view(torch.int32)), (variant, k)


@pytest.mark.parametrize("b", [2, 32, 64])
def test_cnp_many_blocks(B, b):
    """More blocks than a grid's y or z dimension holds (65535): the vector-ALU path (b = 2,
    32) and the chains (b = 64), forward and backward, on sampled blocks either side of it."""
    n = 66000
    _say(f"cnp many blocks n={n} b={b}")
    theta, dg = WL.make_cnp_inputs(n, b, 0.02, seed=400 + b)
    th_d = torch.from_numpy(theta).cuda()
    g = B.poetx_cnp(B.POETX_CNP_FWD, th_d, b, g_dtype=torch.float32)
    d = B.poetx_cnp(B.POETX_CNP_BWD, th_d, b, dg=torch.from_numpy(dg).cuda())
    torch.cuda.synchronize()
    idx = np.array([0, 1, 65534, 65535, 65536, n - 1])
    sel = torch.from_numpy(idx).cuda()
    ref_g = O.cnp_forward(theta[idx].astype(np.float64), b)
    assert rel_fro_per_block(to_host_f64(g[sel]), ref_g) <= TOL_CNP_F32
    ref_d = O.cnp_backward(theta[idx].astype(np.float64), dg[idx].astype(np.float64), b)
    assert rel_fro_per_block(to_host_f64(d[sel]), ref_d) <= TOL_CNP_F32


# ----------------------------------------------------------------- merge ----

@pytest.mark.parametrize("dt", ["f32", "bf16", "i8"])
def test_merge_bit_exact(B, dt):
    rng = np.random.default_rng(5)
    d_out, d_in = 384, 640
    pin, pout = rng.permutation(d_in).astype(np.int32), rng.permutation(d_out).astype(np.int32)
    if dt == "i8":
        w = rng.integers(-127, 128, size=(d_out, d_in)).astype(np.int8)
        s = rng.random(d_out).astype(np.float32)
        wm, sm = B.poetx_merge_perm(torch.from_numpy(w).cuda(), torch.from_numpy(pout).cuda(),
                                    torch.from_numpy(pin).cuda(), torch.from_numpy(s).cuda())
        qr, sr = O.merge_perm_int8(w, s, pout, pin)
        assert np.array_equal(wm.cpu().numpy(), qr) and np.array_equal(sm.cpu().numpy(), sr)
        # the 1-byte transpose (the backward's W'^T of an int8 layer): 16-byte chunk path, and
        # a width that is not a multiple of 16 (element path)
        for rows, cols in ((384, 640), (40, 72)):
            q = rng.integers(-127, 128, size=(rows, cols)).astype(np.int8)
            q_t = torch.empty((cols, rows), dtype=torch.int8, device="cuda")
            B.poetx_merge_perm(torch.from_numpy(q).cuda(), None, None,
                               torch.ones(rows, dtype=torch.float32, device="cuda"), out_t=q_t)
            assert np.array_equal(q_t.cpu().numpy(), q.T)
        return
    w = rng.standard_normal((d_out, d_in)).astype(np.float32)
    if dt == "bf16":
        bits = WL.f32_to_bf16_bits(w)
        wt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        ref = O.merge_perm(bits, pout, pin)
        w_t = torch.empty((d_in, d_out), dtype=torch.bfloat16, device="cuda")
        wm, _ = B.poetx_merge_perm(wt, torch.from_numpy(pout).cuda(), torch.from_numpy(pin).cuda(), out_t=w_t)
        assert np.array_equal(wm.view(torch.int16).cpu().numpy().view(np.uint16), ref)
        assert np.array_equal(w_t.view(torch.int16).cpu().numpy().view(np.uint16), ref.T)
    else:
        wt = torch.empty((d_in, d_out), dtype=torch.float32, device="cuda")
        wm, _ = B.poetx_merge_perm(torch.from_numpy(w).cuda(), torch.from_numpy(pout).cuda(),
                                   torch.from_numpy(pin).cuda(), out_t=wt)
        ref = O.merge_perm(w, pout, pin)
        assert np.array_equal(wm.cpu().numpy(), ref)
        assert np.array_equal(wt.cpu().numpy(), ref.T)


# ----------------------------------------------------------------- layer ----

def _run_step(wl, inp, variant, perms=True, transposed_weight=False, keep_x=True):
    from orthogonal_reparameterized_amd.step import LayerStep
    st = LayerStep(wl, inp, variant, perms=perms, transposed_weight=transposed_weight, keep_x=keep_x)
    out = st.step(want_dg=True)
    torch.cuda.synchronize()
    return st, out


def _compare(st, out, ref, tol, label):
    # blocks of unequal size come back from the oracle as lists: compare flattened
    def e(got, key):
        return norm_max_err(flat(to_host_f64(got)), flat(ref[key]))
    errs = {
        "G_R": e(st.g_r, "G_R"),
        "G_P": e(st.g_p, "G_P"),
        "Z": e(st.z, "Z"),
        "dX": e(out["dx"], "dX"),
        "dG_R": e(out["dg_r"], "dG_R"),
        "dG_P": e(out["dg_p"], "dG_P"),
        "dtheta_R": e(out["dtheta_r"], "dtheta_R"),
        "dtheta_P": e(out["dtheta_p"], "dtheta_P"),
    }
    fro = {k: rel_fro(flat(to_host_f64(v)), flat(ref[r])) for k, v, r in
           (("Z", st.z, "Z"), ("dX", out["dx"], "dX"), ("dtheta_R", out["dtheta_r"], "dtheta_R"))}
    _say(f"{label}: normalized max errors {errs} rel-fro {fro}")
    for k, e in errs.items():
        assert e <= tol, f"{label} {k}: {e} > {tol}"


@pytest.mark.parametrize("variant", ["fast", "mem"])
def test_layer_workload1_f32(B, variant):
    wl = WL.WORKLOADS[1]
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    st, out = _run_step(wl, inp, variant)
    _compare(st, out, ref, TOL_F32_LAYER, f"workload1 {variant}")


@pytest.mark.parametrize("n,d_in,d_out,b", [(257, 512, 768, 256), (8192, 4096, 4096, 256)])
def test_layer_kept_x_matches_regather(B, n, d_in, d_out, b):
    """The fast variant's kept X~ (saved_x) must give bit-identical results to gathering x
    again in the backward: the same kernels read the same values."""
    wl = WL.Workload(91, "kept x", n, d_in, d_out, b, "bf16", "bf16", "bf16", 0.01, d_in)
    inp = WL.make_layer_inputs(wl)
    st0, out0 = _run_step(wl, inp, "fast", keep_x=False)
    st1, out1 = _run_step(wl, inp, "fast", keep_x=True)
    assert st0.saved_x is None and st1.saved_x is not None
    # the kept copy is the gathered input itself
    xg = st1.x[:, st1.perm_in.long()]
    assert torch.equal(st1.saved_x, xg)
    assert torch.equal(st0.z, st1.z)
    for k in ("dx", "dtheta_r", "dtheta_p", "dg_r", "dg_p"):
        assert torch.equal(out0[k], out1[k]), k
    _say(f"kept x {n}x{d_in}->{d_out}: identical to the re-gather")


def test_layer_f32_over_four_million_tokens(B):
    """fp32 layer (float32 vector-ALU products) past 65535 x 64 = 4194240 tokens, the rows one
    launch of those products covers: 61 oracle tokens tiled 68760 times.  Z and dX repeat the
    oracle's per-token values; dG and dtheta are 68760 times the oracle's (sums over tokens).
    Tolerance for the sums, relative to their largest magnitude: 1024-token chunks summed in
    float32, then 4096 partials summed in order, (1024 + 4096 / 2) x 2^-24 = 1.8e-4; the
    test allows 3e-4 (measured about 1e-5)."""
    n0, k = 61, 68760
    wl = WL.Workload(92, "tiled f32", n0, 64, 64, 32, "f32", "f32", "f32", 0.02, 64)
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    big = dict(inp, x=np.tile(inp["x"], (k, 1)), dz=np.tile(inp["dz"], (k, 1)))
    _say(f"tiled f32 layer: {n0 * k} tokens")
    for variant in ("fast", "mem"):
        st, out = _run_step(wl, big, variant)
        z = st.z.view(k, n0, wl.d_out).double()
        dx = out["dx"].view(k, n0, wl.d_in).double()
        for name, got, r in (("Z", z, ref["Z"]), ("dX", dx, ref["dX"])):
            rt = torch.from_numpy(np.asarray(r, dtype=np.float64)).cuda()
            err = ((got - rt).abs().max() / rt.abs().max()).item()
            assert err <= TOL_F32_LAYER, f"{variant} {name}: {err}"
        errs, scale = {}, {}
        for key, rkey in (("dtheta_r", "dtheta_R"), ("dtheta_p", "dtheta_P"), ("dg_r", "dG_R"), ("dg_p", "dG_P")):
            got, want = flat(to_host_f64(out[key])), k * flat(ref[rkey])
            errs[key] = float(np.max(np.abs(got - want)))
            scale[key] = float(np.max(np.abs(want)))
        _say(f"tiled f32 layer {variant}: max abs errors {errs} max abs values {scale}")
        for key in errs:
            assert errs[key] <= 3e-4 * scale[key], f"{variant} {key}: {errs[key] / scale[key]}"
        _say(f"tiled f32 layer {variant}: ok")
        del st, out
        torch.cuda.empty_cache()


def test_layer_bf16_long_token_sums(B):
    """bf16 layer at 4096 -> 4096, b = 256, 268800 tokens (64 oracle tokens tiled 4200 times):
    past 4 partitions x 65536 tokens, so the streaming block gradient splits its token sums
    into more partials.  Z and dX repeat the oracle's per-token values; dG and dtheta are
    4200 times the oracle's, within the bf16 layer bar."""
    n0, k = 64, 4200
    wl = WL.Workload(93, "tiled bf16", n0, 4096, 4096, 256, "bf16", "bf16", "bf16", 0.01, 4096)
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    big = dict(inp, x=np.tile(inp["x"], (k, 1)), dz=np.tile(inp["dz"], (k, 1)))
    _say(f"tiled bf16 layer: {n0 * k} tokens")
    st, out = _run_step(wl, big, "fast")
    for name, got, r in (("Z", st.z, ref["Z"]), ("dX", out["dx"], ref["dX"])):
        g = got.view(k, n0, -1).float()
        rt = torch.from_numpy(np.asarray(r, dtype=np.float32)).cuda()
        err = ((g - rt).abs().max() / rt.abs().max()).item()
        assert err <= TOL_BF16, f"{name}: {err}"
    for key, rkey in (("dtheta_r", "dtheta_R"), ("dtheta_p", "dtheta_P"), ("dg_r", "dG_R"), ("dg_p", "dG_P")):
        err = norm_max_err(flat(to_host_f64(out[key])), k * flat(ref[rkey]))
        assert err <= TOL_BF16, f"{key}: {err}"
    _say("tiled bf16 layer: ok")


SMALL_BF16 = [
    # (n_tokens, d_in, d_out, b, perms) -- several 128-wide tiles and ragged token tails
    (257, 512, 768, 256, True),
    (130, 1024, 512, 512, True),
    (64, 256, 256, 128, False),
    (1, 384, 256, 128, True),
    # b = 64: streaming block kernels at 64 columns, W' products on MFMA (at 576 and 320 on
    # the tail form of the NT kernel)
    (257, 512, 768, 64, True),
    (130, 576, 320, 64, True),
    (33, 256, 256, 64, False),
]


@pytest.mark.parametrize("n,d_in,d_out,b,perms", SMALL_BF16)
@pytest.mark.parametrize("variant", ["fast", "mem"])
def test_layer_bf16_small(B, n, d_in, d_out, b, perms, variant):
    wl = WL.Workload(90, "small bf16", n, d_in, d_out, b, "bf16", "bf16", "bf16", 0.01, d_in, perms=perms)
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    st, out = _run_step(wl, inp, variant)
    _compare(st, out, ref, TOL_BF16, f"small n={n} {d_in}->{d_out} b={b} perms={perms} {variant}")


@pytest.mark.parametrize("n,d_in,d_out,b", [(257, 512, 768, 256), (130, 1024, 512, 512)])
def test_layer_bf16_transposed_weight(B, n, d_in, d_out, b):
    """With W'^T kept from the merge the backward reads it k-contiguous; same results."""
    wl = WL.Workload(97, "small bf16 wt", n, d_in, d_out, b, "bf16", "bf16", "bf16", 0.01, d_in)
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    st, out = _run_step(wl, inp, "fast", transposed_weight=True)
    _compare(st, out, ref, TOL_BF16, f"W'^T n={n} {d_in}->{d_out} b={b}")


def test_layer_bf16_generic_block(B):
    """b = 48 (not a multiple of 128): vector-ALU block products and CNP; the W' products
    (96 and 144 wide) on the NT kernel's tail form."""
    wl = WL.Workload(91, "small bf16 b48", 70, 96, 144, 48, "bf16", "bf16", "bf16", 0.02, 96)
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    st, out = _run_step(wl, inp, "fast")
    _compare(st, out, ref, TOL_BF16, "b=48 generic")


RAGGED = [
    # (n_tokens, d_in, d_out, b, dtype): ceil(d/b) blocks, the last one smaller
    (257, 640, 896, 256, "bf16"),   # last blocks 128 | 128 on the MFMA kernels
    (100, 384, 640, 512, "bf16"),   # input side narrower than b (one block of 384)
    (70, 576, 320, 256, "bf16"),    # 128 does not divide d_in: the W' products on the NT
                                    # kernel's tail form; the 256-blocks and the last blocks of
                                    # 64 on the MFMA block kernels
    (777, 1000, 2040, 256, "bf16"), # neither width tiles: a k tail (40, 56) and a partial
                                    # n tile in both W' products; last blocks 232 | 248
    (300, 1288, 776, 64, "bf16"),   # b = 64 with last blocks of 8
    (513, 4000, 3000, 256, "bf16"), # many tiles with k and n tails; last blocks 160 | 184
    (64, 200, 150, 32, "f32"),      # last blocks 8 | 22
    (33, 97, 70, 32, "f32"),        # a last block of size 1 (no parameters) | 6
]


@pytest.mark.parametrize("n,d_in,d_out,b,dt", RAGGED)
@pytest.mark.parametrize("variant", ["fast", "mem"])
def test_layer_ragged_blocks(B, n, d_in, d_out, b, dt, variant):
    wl = WL.Workload(96, "ragged", n, d_in, d_out, b, dt, dt, dt, 0.02, d_in)
    assert wl.ragged
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    _say(f"ragged n={n} {d_in}->{d_out} b={b} {dt} {variant}")
    st, out = _run_step(wl, inp, variant)
    _compare(st, out, ref, TOL_BF16 if dt == "bf16" else TOL_F32_LAYER, f"ragged {d_in}->{d_out} b={b} {variant}")


@pytest.mark.parametrize("d_in,d_out", [(32768, 256), (256, 32768)])
def test_layer_widest_rows(B, d_in, d_out):
    """64 KB activation rows (the widest the library takes), a few tokens: the element-wise
    permutation path, a W' product of one tile split along k, 128-block CNP calls."""
    wl = WL.Workload(99, "widest", 3, d_in, d_out, 256, "bf16", "bf16", "bf16", 0.01, d_in)
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    _say(f"widest rows {d_in}->{d_out}")
    for variant in ("fast", "mem"):
        st, out = _run_step(wl, inp, variant)
        _compare(st, out, ref, TOL_BF16, f"widest {d_in}->{d_out} {variant}")


@pytest.mark.parametrize("variant", ["fast", "mem"])
def test_layer_b1024(B, variant):
    """b = 1024: CNP on the per-product MFMA path, block products on the MFMA engines."""
    wl = WL.Workload(98, "b1024", 130, 2048, 1024, 1024, "bf16", "bf16", "bf16", 0.005, 2048)
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    _say(f"b=1024 {variant}")
    st, out = _run_step(wl, inp, variant)
    _compare(st, out, ref, TOL_BF16, f"b=1024 {variant}")


@pytest.mark.parametrize("d_in,d_out,b", [(512, 768, 256), (1024, 1536, 512)])
def test_layer_int8_small(B, d_in, d_out, b):
    """int8 W' with per-row scales (mem).  The scales enter the backward's P-side block
    product as per-column factors; at b = 512 that is the streaming half-block kernel (3
    blocks: 42 of its 48 workgroups busy, a ragged last token tile)."""
    wl = WL.Workload(92, "small int8", 200, d_in, d_out, b, "bf16", "i8", "bf16", 0.01, d_in, variants=("mem",))
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    st, out = _run_step(wl, inp, "mem")
    _compare(st, out, ref, TOL_BF16, f"int8 small b={b}")


def test_int8_fast_rejected(B):
    wl = WL.Workload(93, "int8 fast", 16, 256, 256, 128, "bf16", "i8", "bf16", 0.01, 256)
    inp = WL.make_layer_inputs(wl)
    from orthogonal_reparameterized_amd.step import LayerStep
    st = LayerStep(wl, inp, "mem")
    st.layer.variant = B.POETX_FAST
    with pytest.raises(B.PoetxError) as e:
        B.poetx_forward(st.layer, st.x, st.z, torch.empty_like(st.z))
    assert e.value.status == B.POETX_ERR_UNSUPPORTED


# ------------------------------------------------------------ phase-end fold ----

FOLD_CASES = [
    # (d_in, d_out, b, dtype, perms): fp32 vector-ALU path, and the bf16 block kernels
    (256, 256, 32, "f32", True),
    (512, 768, 256, "bf16", True),
    (256, 384, 128, "bf16", False),
    (1024, 512, 512, "bf16", True),
    (640, 896, 256, "bf16", True),   # a smaller last block on each side
    (200, 150, 32, "f32", True),
]


def _fold_layer(wl, inp):
    from orthogonal_reparameterized_amd.step import LayerStep
    st = LayerStep(wl, inp, "mem")
    st.cnp()
    return st


@pytest.mark.parametrize("d_in,d_out,b,dt,perms", FOLD_CASES)
def test_fold(B, d_in, d_out, b, dt, perms):
    """poetx_fold against the oracle's fold of the same W', G_R, G_P and permutations."""
    _say(f"fold {d_in}x{d_out} b={b} {dt} perms={perms}")
    wl = WL.Workload(95, "fold", 16, d_in, d_out, b, dt, dt, dt, 0.02, d_in, perms=perms)
    inp = WL.make_layer_inputs(wl)
    st = _fold_layer(wl, inp)
    w_eff = B.poetx_fold(st.layer)
    ref = O.fold_weights(to_host_f64(st.w_merged), split_g(to_host_f64(st.g_r), d_in, b),
                         split_g(to_host_f64(st.g_p), d_out, b), inp["perm_in"], inp["perm_out"])
    tol = TOL_CNP_F32 if dt == "f32" else TOL_BF16
    assert norm_max_err(to_host_f64(w_eff), ref) <= tol


def test_fold_phase_identity(B):
    """The next phase starts from the folded weight, theta = 0 and new permutations, and
    computes the same layer: its forward matches the old phase's forward."""
    wl = WL.Workload(96, "fold phase", 130, 512, 768, 256, "bf16", "bf16", "bf16", 0.02, 512)
    inp = WL.make_layer_inputs(wl)
    st = _fold_layer(wl, inp)
    z_old, _ = B.poetx_forward(st.layer, st.x)
    w_eff = B.poetx_fold(st.layer)
    rng = np.random.default_rng(7)
    pin = torch.from_numpy(rng.permutation(wl.d_in).astype(np.int32)).cuda()
    pout = torch.from_numpy(rng.permutation(wl.d_out).astype(np.int32)).cuda()
    w_new, _ = B.poetx_merge_perm(w_eff, pout, pin)
    th_r, th_p = torch.zeros_like(st.theta_r), torch.zeros_like(st.theta_p)
    g_r = B.poetx_cnp(B.POETX_CNP_FWD, th_r, wl.b)
    g_p = B.poetx_cnp(B.POETX_CNP_FWD, th_p, wl.b)
    layer = B.Layer(w_new, th_r, th_p, g_r, g_p, wl.b, act_dtype=torch.bfloat16, variant=B.POETX_MEM,
                    perm_in=pin, perm_out=pout)
    z_new, _ = B.poetx_forward(layer, st.x)
    assert torch.equal(g_r.float().cpu(), torch.eye(wl.b).expand_as(g_r.float().cpu()))
    assert norm_max_err(to_host_f64(z_new), to_host_f64(z_old)) <= TOL_BF16


@pytest.mark.parametrize("key", [3, 4])
def test_fold_full_size_sampled(B, key):
    """Workloads 3 and 4 at full size: sampled (P-block, R-block) pairs of the folded
    weight against the oracle's fold of that block pair."""
    wl = WL.WORKLOADS[key]
    _say(f"fold workload {key}")
    inp = WL.make_layer_inputs(wl, n_tokens=64)
    st = _fold_layer(wl, inp)
    w_eff = to_host_f64(B.poetx_fold(st.layer))
    wm = to_host_f64(st.w_merged)
    g_r, g_p = to_host_f64(st.g_r), to_host_f64(st.g_p)
    pin, pout = np.asarray(inp["perm_in"], np.int64), np.asarray(inp["perm_out"], np.int64)
    b, n_r, n_p = wl.b, wl.d_in // wl.b, wl.d_out // wl.b
    for jp, jr in [(0, 0), (n_p - 1, n_r - 1), (n_p // 2, 1), (1, n_r // 2)]:
        rows, cols = slice(jp * b, (jp + 1) * b), slice(jr * b, (jr + 1) * b)
        ref = O.fold_weights(wm[rows, cols], g_r[jr:jr + 1], g_p[jp:jp + 1])
        got = w_eff[np.ix_(pout[rows], pin[cols])]
        assert norm_max_err(got, ref) <= TOL_BF16, (jp, jr)


# ------------------------------------------------------------ optimizer ----

@pytest.mark.parametrize("n", [4, 1023, 32 * 32640])
def test_adam_step(B, n):
    """poetx_adam_step over several steps against the oracle's Adam, float32 state."""
    rng = np.random.default_rng(41)
    th = (rng.standard_normal(n) * 0.01).astype(np.float32)
    th_d = torch.from_numpy(th).cuda()
    m_d, v_d = torch.zeros_like(th_d), torch.zeros_like(th_d)
    ref_t, ref_m, ref_v = th.astype(np.float64), np.zeros(n), np.zeros(n)
    # the kernel takes its hyperparameters as float32: the oracle gets the same values
    lr, b1, b2, eps, gamma = (float(np.float32(x)) for x in (1e-3, 0.9, 0.999, 1e-8, 0.5))
    for t in range(1, 4):
        g = rng.standard_normal(n).astype(np.float32)
        B.poetx_adam_step(th_d, torch.from_numpy(g).cuda(), m_d, v_d, lr=1e-3, step=t, gamma=0.5)
        ref_t, ref_m, ref_v = O.adam_step(ref_t, g, ref_m, ref_v, lr, b1, b2, eps, t, gamma)
    torch.cuda.synchronize()
    # float32 arithmetic: state to a few ulp; theta moves by ~1e-3 per step
    np.testing.assert_allclose(m_d.cpu().numpy(), ref_m, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(v_d.cpu().numpy(), ref_v, rtol=1e-5, atol=1e-9)
    np.testing.assert_allclose(th_d.cpu().numpy(), ref_t, rtol=1e-5, atol=1e-7)


@functools.lru_cache(maxsize=None)
def _full(key):
    wl = WL.WORKLOADS[key]
    inp = WL.make_layer_inputs(wl)
    _say(f"oracle for workload {key} ...")
    ref = oracle_layer(inp, wl)
    _say(f"oracle for workload {key} done")
    return wl, inp, ref


@pytest.mark.parametrize("key,variant,wt", [(3, "fast", False), (3, "fast", True), (3, "mem", False),
                                             (4, "fast", True), (4, "mem", False), (5, "mem", False),
                                             (6, "fast", True), (6, "mem", False)])
def test_layer_full_size(B, key, variant, wt):
    wl, inp, ref = _full(key)
    _say(f"workload {key} {variant} (W'^T kept: {wt}) on GPU")
    st, out = _run_step(wl, inp, variant, transposed_weight=wt)
    _compare(st, out, ref, TOL_BF16, f"workload{key} {variant}")


@pytest.mark.parametrize("b", [256, 512])
def test_layer_many_tiles_ragged(B, b):
    """12289 tokens at 2048 -> 2048: 49 row tiles of 256, the last one holding a single
    token.  The W' products take 392 whole tiles in two rounds (the leftover round is too
    full to split along k) and, at b = 512, the batched block products 4 x 49 x 2 tiles."""
    wl = WL.Workload(98, "many tiles ragged", 12289, 2048, 2048, b, "bf16", "bf16", "bf16", 0.01, 2048)
    inp = WL.make_layer_inputs(wl)
    ref = oracle_layer(inp, wl)
    for variant in ("fast", "mem"):
        st, out = _run_step(wl, inp, variant)
        _compare(st, out, ref, TOL_BF16, f"many tiles ragged b={b} {variant}")
        del st, out


def test_fast_mem_identical_and_deterministic(B):
    wl = WL.Workload(94, "det", 300, 512, 512, 256, "bf16", "bf16", "bf16", 0.01, 512)
    inp = WL.make_layer_inputs(wl)
    st_f, out_f = _run_step(wl, inp, "fast")
    z1, dx1, r1, p1 = st_f.z.clone(), out_f["dx"].clone(), out_f["dtheta_r"].clone(), out_f["dtheta_p"].clone()
    out_f2 = st_f.step()
    torch.cuda.synchronize()
    assert torch.equal(st_f.z, z1) and torch.equal(out_f2["dx"], dx1)
    assert torch.equal(out_f2["dtheta_r"], r1) and torch.equal(out_f2["dtheta_p"], p1)
    st_m, out_m = _run_step(wl, inp, "mem")
    assert torch.equal(st_m.z, z1) and torch.equal(out_m["dx"], dx1)
    assert torch.equal(out_m["dtheta_r"], r1) and torch.equal(out_m["dtheta_p"], p1)


def test_null_perm_equals_identity_perm(B):
    wl = WL.Workload(95, "idperm", 100, 256, 512, 128, "bf16", "bf16", "bf16", 0.01, 256)
    inp = WL.make_layer_inputs(wl, perms=False)
    st0, out0 = _run_step(wl, inp, "fast", perms=False)
    inp_id = dict(inp)
    inp_id["perm_in"] = np.arange(wl.d_in, dtype=np.int32)
    inp_id["perm_out"] = np.arange(wl.d_out, dtype=np.int32)
    st1, out1 = _run_step(wl, inp_id, "fast", perms=True)
    assert torch.equal(st0.z, st1.z) and torch.equal(out0["dx"], out1["dx"])
    assert torch.equal(out0["dtheta_r"], out1["dtheta_r"])


def test_zero_tokens(B):
    wl = WL.Workload(96, "empty", 0, 256, 256, 128, "bf16", "bf16", "bf16", 0.01, 256)
    inp = WL.make_layer_inputs(wl)
    st, out = _run_step(wl, inp, "fast")
    assert st.z.shape == (0, 256)
    assert torch.count_nonzero(out["dtheta_r"]) == 0 and torch.count_nonzero(out["dtheta_p"]) == 0
