"""poetx_cnp_noalloc (the CNP with its workspace in the library's static device array)
through the C ABI against poetx_cnp with a caller-allocated workspace: the same kernels,
so the results must be bitwise equal.  Two calls in a row, the second with a smaller input
(the array keeps the first call's contents), forward and backward; and a call whose
workspace exceeds the array is refused before any launch."""

import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from orthogonal_reparameterized_amd import workloads as WL  # noqa: E402


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from orthogonal_reparameterized_amd import binding
    return binding


def _noalloc(B, direction, theta, b, g=None, dg=None, dtheta=None):
    st = B.raw.poetx_cnp_noalloc(direction, theta.shape[0], b, ctypes.c_void_p(theta.data_ptr()), B.POETX_F32,
                                 ctypes.c_void_p(g.data_ptr()) if g is not None else None,
                                 B.POETX_BF16 if g is not None and g.dtype == torch.bfloat16 else B.POETX_F32,
                                 ctypes.c_void_p(dg.data_ptr()) if dg is not None else None, B.POETX_F32,
                                 ctypes.c_void_p(dtheta.data_ptr()) if dtheta is not None else None,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("g_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_call(B, g_dtype):
    for n, b, seed in ((32, 256, 1), (5, 128, 2)):  # second call smaller
        theta, dg = WL.make_cnp_inputs(n, b, 0.01, seed=700 + seed)
        th = torch.from_numpy(theta).cuda()
        dgt = torch.from_numpy(dg).cuda()
        g_ref = B.poetx_cnp(B.POETX_CNP_FWD, th, b, g_dtype=g_dtype)
        d_ref = B.poetx_cnp(B.POETX_CNP_BWD, th, b, dg=dgt)
        g = torch.full((n, b, b), 7.0, dtype=g_dtype, device="cuda")
        d = torch.full_like(th, 7.0)
        assert _noalloc(B, B.POETX_CNP_FWD, th, b, g=g) == B.POETX_OK
        assert _noalloc(B, B.POETX_CNP_BWD, th, b, dg=dgt, dtheta=d) == B.POETX_OK
        torch.cuda.synchronize()
        assert torch.equal(g, g_ref), (n, b)
        assert torch.equal(d, d_ref), (n, b)


def test_noalloc_rejects_oversize(B):
    # 4096 blocks of b = 256: the backward's workspace is far above the static array
    n, b = 4096, 256
    th = torch.zeros((1, b * (b - 1) // 2), device="cuda")
    st = B.raw.poetx_cnp_noalloc(B.POETX_CNP_BWD, n, b, ctypes.c_void_p(th.data_ptr()), B.POETX_F32, None,
                                 B.POETX_F32, ctypes.c_void_p(th.data_ptr()), B.POETX_F32,
                                 ctypes.c_void_p(th.data_ptr()), None)
    assert st == B.POETX_ERR_WORKSPACE
    torch.cuda.synchronize()
