"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, answers workspace queries, and rejects bad arguments on the
host with the documented status codes before launching anything."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "poetx.h")


@pytest.fixture(scope="module")
def B():
    from orthogonal_reparameterized_amd import binding
    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(poetx_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported(B):
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    lib = ctypes.CDLL(B.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(B):
    assert re.match(r"\d+\.\d+\.\d+", B.version())
    for code, name in ((0, "POETX_OK"), (-1, "POETX_ERR_INVALID_ARG"), (-2, "POETX_ERR_SHAPE"),
                       (-3, "POETX_ERR_UNSUPPORTED"), (-4, "POETX_ERR_WORKSPACE"), (-5, "POETX_ERR_HIP")):
        assert B.raw.poetx_status_string(code).decode() == name


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def layer(B, **kw):
    c = B.PoetxLayerC()
    c.d_in, c.d_out, c.b = kw.get("d_in", 512), kw.get("d_out", 768), kw.get("b", 256)
    c.act_dtype = kw.get("act", B.POETX_BF16)
    c.w_dtype = kw.get("w", B.POETX_BF16)
    c.g_dtype = kw.get("g", B.POETX_BF16)
    c.variant = kw.get("variant", B.POETX_FAST)
    for f in ("w_merged", "theta_r", "theta_p", "g_r", "g_p"):
        setattr(c, f, kw.get(f, FAKE))
    c.w_scale = kw.get("w_scale", None)
    c.perm_in = kw.get("perm_in", None)
    c.perm_out = kw.get("perm_out", None)
    return c


def fwd(B, c, n=64, ws=None, ws_bytes=0, x=FAKE, z=FAKE, saved=FAKE, saved_x=None):
    nb = ctypes.c_size_t(ws_bytes)
    st = B.raw.poetx_forward(ctypes.byref(c), n, x, z, saved, saved_x, ws, ctypes.byref(nb), None)
    return st, nb.value


def bwd(B, c, n=64, ws=None, ws_bytes=0, saved=FAKE, dtr=FAKE, dtp=FAKE, saved_x=None):
    nb = ctypes.c_size_t(ws_bytes)
    st = B.raw.poetx_backward(ctypes.byref(c), n, FAKE, FAKE, saved, saved_x, FAKE, dtr, dtp, None, None, ws,
                              ctypes.byref(nb), None)
    return st, nb.value


def test_workspace_queries(B):
    st, need_fast = fwd(B, layer(B))
    assert st == B.POETX_OK and need_fast > 0
    st, need_mem = fwd(B, layer(B, variant=B.POETX_MEM), saved=None)
    assert st == B.POETX_OK and need_mem > need_fast  # mem keeps B in the workspace
    st, need_b = bwd(B, layer(B))
    assert st == B.POETX_OK and need_b > 0
    # a kept X~ (fast, with an input permutation) replaces the workspace copy: N x d_in bf16 less
    perm = layer(B, perm_in=FAKE)
    st, ws_gather = fwd(B, perm)
    st2, ws_kept = fwd(B, perm, saved_x=FAKE)
    assert st == st2 == B.POETX_OK and ws_gather - ws_kept == 64 * 512 * 2
    st, ws_gather = bwd(B, perm)
    st2, ws_kept = bwd(B, perm, saved_x=FAKE)
    assert st == st2 == B.POETX_OK and ws_gather - ws_kept == 64 * 512 * 2
    # without an input permutation there is nothing to keep
    assert fwd(B, layer(B), saved_x=FAKE)[1] == need_fast
    nb = ctypes.c_size_t(0)
    assert B.raw.poetx_cnp(B.POETX_CNP_FWD, 16, 256, None, B.POETX_F32, None, B.POETX_BF16, None, None, B.POETX_F32,
                           None, None, ctypes.byref(nb), None) == B.POETX_OK
    assert nb.value >= 16 * 256 * 256 * 4


def test_validation_codes(B):
    ok = layer(B)
    # shape errors
    assert fwd(B, layer(B, b=1))[0] == B.POETX_ERR_SHAPE
    assert fwd(B, layer(B, b=2048, d_in=4096, d_out=4096))[0] == B.POETX_ERR_SHAPE  # above 1024
    # ceil(d/b) blocks: b need not divide the widths (512 = 5 * 100 + 12); b = 1024 is supported
    assert fwd(B, layer(B, b=100))[0] == B.POETX_OK
    assert bwd(B, layer(B, b=100))[0] == B.POETX_OK
    assert fwd(B, layer(B, b=1024, d_in=2048, d_out=2048))[0] == B.POETX_OK
    # widest rows: 64 KB of activations per token (32768 bf16), one step past that is refused
    assert fwd(B, layer(B, d_in=32768, d_out=256))[0] == B.POETX_OK
    assert fwd(B, layer(B, d_in=256, d_out=32768))[0] == B.POETX_OK
    assert fwd(B, layer(B, d_in=32768 + 256, d_out=256))[0] == B.POETX_ERR_UNSUPPORTED
    assert bwd(B, layer(B, d_in=256, d_out=32768 + 256))[0] == B.POETX_ERR_UNSUPPORTED
    # invalid arguments
    assert fwd(B, layer(B, act=7))[0] == B.POETX_ERR_INVALID_ARG
    assert fwd(B, layer(B, variant=5))[0] == B.POETX_ERR_INVALID_ARG
    assert fwd(B, ok, n=-1)[0] == B.POETX_ERR_INVALID_ARG
    assert fwd(B, layer(B, w_merged=None), ws=FAKE, ws_bytes=1 << 40)[0] == B.POETX_ERR_INVALID_ARG
    assert fwd(B, ok, ws=FAKE, ws_bytes=1 << 40, x=None)[0] == B.POETX_ERR_INVALID_ARG
    assert fwd(B, ok, ws=FAKE, ws_bytes=1 << 40, saved=None)[0] == B.POETX_ERR_INVALID_ARG
    assert fwd(B, layer(B, variant=B.POETX_MEM))[0] == B.POETX_ERR_INVALID_ARG  # mem with saved_b
    mem = layer(B, variant=B.POETX_MEM, perm_in=FAKE)
    assert fwd(B, mem, saved=None, saved_x=FAKE)[0] == B.POETX_ERR_INVALID_ARG  # mem keeps nothing
    assert bwd(B, mem, saved=None, saved_x=FAKE)[0] == B.POETX_ERR_INVALID_ARG
    assert bwd(B, ok, ws=FAKE, ws_bytes=1 << 40, dtr=None)[0] == B.POETX_ERR_INVALID_ARG
    # unsupported combinations: int8 weight with the fast variant (POET-XQ needs recompute)
    assert fwd(B, layer(B, w=B.POETX_I8, w_scale=FAKE))[0] == B.POETX_ERR_UNSUPPORTED
    assert fwd(B, layer(B, w=B.POETX_F32))[0] == B.POETX_ERR_UNSUPPORTED    # mixed fp32 weight, bf16 act
    assert fwd(B, layer(B, g=B.POETX_F32))[0] == B.POETX_ERR_UNSUPPORTED
    # workspace too small
    st, need = fwd(B, ok)
    assert fwd(B, ok, ws=FAKE, ws_bytes=need - 1)[0] == B.POETX_ERR_WORKSPACE
    st, need = bwd(B, ok)
    assert bwd(B, ok, ws=FAKE, ws_bytes=need - 1)[0] == B.POETX_ERR_WORKSPACE
    # CNP
    nb = ctypes.c_size_t(1 << 40)
    for bad_b in (0, 2048):
        assert B.raw.poetx_cnp(B.POETX_CNP_FWD, 4, bad_b, FAKE, B.POETX_F32, FAKE, B.POETX_BF16, None, None, 0, None, FAKE,
                               ctypes.byref(nb), None) == B.POETX_ERR_SHAPE
    q = ctypes.c_size_t(0)  # blocks of size 1 (no parameters) are accepted
    assert B.raw.poetx_cnp(B.POETX_CNP_FWD, 4, 1, None, B.POETX_F32, None, B.POETX_BF16, None, None, 0, None, None,
                           ctypes.byref(q), None) == B.POETX_OK
    assert B.raw.poetx_cnp(9, 4, 64, FAKE, B.POETX_F32, FAKE, B.POETX_BF16, None, None, 0, None, FAKE,
                           ctypes.byref(nb), None) == B.POETX_ERR_INVALID_ARG
    assert B.raw.poetx_cnp(B.POETX_CNP_BWD, 4, 64, FAKE, B.POETX_F32, None, 0, None, None, B.POETX_F32, FAKE, FAKE,
                           ctypes.byref(nb), None) == B.POETX_ERR_INVALID_ARG   # dg missing
    small = ctypes.c_size_t(16)
    assert B.raw.poetx_cnp(B.POETX_CNP_FWD, 4, 64, FAKE, B.POETX_F32, FAKE, B.POETX_BF16, None, None, 0, None, FAKE,
                           ctypes.byref(small), None) == B.POETX_ERR_WORKSPACE
    # a saved-Q buffer must be 16-byte aligned
    assert B.raw.poetx_cnp(B.POETX_CNP_FWD, 4, 64, FAKE, B.POETX_F32, FAKE, B.POETX_BF16, FAKE + 8, None, 0, None,
                           FAKE, ctypes.byref(nb), None) == B.POETX_ERR_INVALID_ARG
    # merge
    assert B.raw.poetx_merge_perm(None, None, B.POETX_BF16, 4, 4, None, None, FAKE, None, None, None) == B.POETX_ERR_INVALID_ARG
    assert B.raw.poetx_merge_perm(FAKE, None, B.POETX_I8, 4, 4, None, None, FAKE, None, None, None) == B.POETX_ERR_INVALID_ARG
    assert B.raw.poetx_merge_perm(FAKE, None, B.POETX_BF16, 4, 4, None, None, FAKE, None, FAKE, None) == B.POETX_ERR_INVALID_ARG
    # rows of W past 64 KB are refused before any launch
    assert B.raw.poetx_merge_perm(FAKE, None, B.POETX_BF16, 4, 32768 + 8, None, None, FAKE, None, None,
                                  None) == B.POETX_ERR_UNSUPPORTED


FAKE_OUT = 0x20000  # a second never-dereferenced address (distinct from the layer's W')


def fold(B, c, w_out=FAKE_OUT, ws=None, ws_bytes=0):
    nb = ctypes.c_size_t(ws_bytes)
    st = B.raw.poetx_fold(ctypes.byref(c), w_out, ws, ctypes.byref(nb), None)
    return st, nb.value


def test_fold_validation(B):
    st, need = fold(B, layer(B))
    assert st == B.POETX_OK and need >= 3 * 512 * 768 * 2  # three [d_out][d_in] bf16 buffers
    assert fold(B, layer(B), ws=FAKE, ws_bytes=need - 1)[0] == B.POETX_ERR_WORKSPACE
    assert fold(B, layer(B), w_out=None, ws=FAKE, ws_bytes=need)[0] == B.POETX_ERR_INVALID_ARG
    assert fold(B, layer(B), w_out=FAKE, ws=FAKE, ws_bytes=need)[0] == B.POETX_ERR_INVALID_ARG  # aliases W'
    assert fold(B, layer(B, w=B.POETX_I8, w_scale=FAKE, variant=B.POETX_MEM))[0] == B.POETX_ERR_UNSUPPORTED
    assert fold(B, layer(B, b=2048, d_in=4096, d_out=4096))[0] == B.POETX_ERR_SHAPE
    assert fold(B, layer(B, b=100))[0] == B.POETX_OK  # a smaller last block on each side


def test_adam_validation(B):
    f = B.raw.poetx_adam_step
    assert f(0, None, B.POETX_F32, None, None, None, 1e-3, 0.9, 0.999, 1e-8, 1, 1.0, None) == B.POETX_OK  # empty: no-op
    assert f(8, FAKE, B.POETX_F32, FAKE, FAKE, FAKE, 1e-3, 0.9, 0.999, 1e-8, 0, 1.0, None) == B.POETX_ERR_INVALID_ARG
    assert f(8, FAKE, B.POETX_F32, FAKE, FAKE, FAKE, 1e-3, 1.0, 0.999, 1e-8, 1, 1.0, None) == B.POETX_ERR_INVALID_ARG
    assert f(8, FAKE, B.POETX_F32, FAKE, FAKE, FAKE, 1e-3, 0.9, 0.999, 0.0, 1, 1.0, None) == B.POETX_ERR_INVALID_ARG
    assert f(8, FAKE, B.POETX_F32, None, FAKE, FAKE, 1e-3, 0.9, 0.999, 1e-8, 1, 1.0, None) == B.POETX_ERR_INVALID_ARG
    assert f(8, FAKE + 4, B.POETX_F32, FAKE, FAKE, FAKE, 1e-3, 0.9, 0.999, 1e-8, 1, 1.0, None) == B.POETX_ERR_INVALID_ARG


def _c_params(name):
    """Parameter type strings of `name` as declared in poetx.h."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    body = m.group(1).strip()
    if body in ("", "void"):
        return []
    return [" ".join(p.split()) for p in body.split(",")]


def _ctype_of(decl):
    """ctypes class a binding must use for one C parameter declaration."""
    d = decl.replace("const ", "")
    if "size_t *" in d or "size_t*" in d:
        return "size_t_ptr"
    if "poetx_layer *" in d:
        return "layer_ptr"
    if "poetx_adam *" in d:
        return "adam_ptr"
    if "char *" in d:
        return (ctypes.c_char_p, ctypes.c_void_p)
    if "*" in d:
        return ctypes.c_void_p
    base = d.split()[0]
    return {"int64_t": ctypes.c_int64, "int32_t": ctypes.c_int32, "int": ctypes.c_int,
            "float": ctypes.c_float, "size_t": ctypes.c_size_t}[base]


def test_header_signatures_match_binding(B):
    """Every entry point's parameter list in poetx.h (count and types) is what the binding
    declares, and the poetx_layer struct has the binding's field order and types."""
    for name in declared_functions():
        want = [_ctype_of(p) for p in _c_params(name)]
        got = list(getattr(B.raw, name).argtypes or [])
        assert len(got) == len(want), (name, len(got), len(want))
        for w, g in zip(want, got):
            if w == "size_t_ptr":
                assert g is ctypes.POINTER(ctypes.c_size_t), name
            elif w == "layer_ptr":
                assert g is ctypes.POINTER(B.PoetxLayerC), name
            elif w == "adam_ptr":
                assert g is ctypes.POINTER(B.PoetxAdamC), name
            elif w is ctypes.c_int:
                assert g in (ctypes.c_int, ctypes.c_int32), name
            elif isinstance(w, tuple):
                assert g in w, (name, w, g)
            else:
                assert g is w, (name, w, g)
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} poetx_layer;", text, flags=re.S).group(1)
    fields = []
    for decl in body.split(";"):
        decl = " ".join(decl.split())
        if not decl:
            continue
        typ = "ptr" if "*" in decl else decl.split()[0]
        for nm in decl.replace("*", " ").split()[1 if typ != "ptr" else 0:]:
            nm = nm.strip(",")
            if nm and nm not in ("const", "void", "float", "int32_t", "int64_t"):
                fields.append((nm, typ))
    cmap = {"int64_t": ctypes.c_int64, "int32_t": ctypes.c_int32, "ptr": ctypes.c_void_p, "float": ctypes.c_float}
    assert [(n, cmap[t]) for n, t in fields] == list(B.PoetxLayerC._fields_)
    body = re.search(r"typedef struct \{([^{}]*)\} poetx_adam;", text).group(1)
    fields = []
    for decl in body.split(";"):
        decl = " ".join(decl.split())
        if not decl:
            continue
        typ = "ptr" if "*" in decl else decl.split()[0]
        for nm in decl.replace("*", " ").split()[1:]:
            nm = nm.strip(",")
            if nm:
                fields.append((nm, typ))
    assert [(n, cmap[t]) for n, t in fields] == list(B.PoetxAdamC._fields_)


def test_int8_with_transposed_weight_refused(B):
    """A kept W'^T is a BF16-only option: an I8 layer that sets it is refused on the host."""
    c = layer(B, w=B.POETX_I8, w_scale=FAKE, variant=B.POETX_MEM)
    assert fwd(B, c, saved=None)[0] == B.POETX_OK
    c.w_merged_t = FAKE_OUT
    assert fwd(B, c, saved=None)[0] == B.POETX_ERR_INVALID_ARG
    assert bwd(B, c, saved=None)[0] == B.POETX_ERR_INVALID_ARG


def test_backward_adam_validation(B):
    """poetx_backward_adam: same workspace as poetx_backward; optimizer arguments checked on the
    host (NULL opt or buffers, step < 1, beta outside [0, 1), eps <= 0)."""
    c = layer(B)
    st, need = bwd(B, c)
    nb = ctypes.c_size_t(0)
    o = B.PoetxAdamC()
    o.lr, o.beta1, o.beta2, o.eps, o.gamma, o.step = 1e-3, 0.9, 0.999, 1e-8, 1.0, 1
    o.m_r = o.v_r = o.m_p = o.v_p = FAKE
    o.theta_r_out = o.theta_p_out = FAKE

    def call(opt, ws=None, ws_bytes=0, dtr=None, dtp=None):
        nb = ctypes.c_size_t(ws_bytes)
        st = B.raw.poetx_backward_adam(ctypes.byref(c), 64, FAKE, FAKE, FAKE, None, FAKE, dtr, dtp,
                                       ctypes.byref(opt) if opt is not None else None, ws, ctypes.byref(nb), None)
        return st, nb.value
    st, need_a = call(o)
    assert st == B.POETX_OK and need_a == need
    assert call(None)[0] == B.POETX_ERR_INVALID_ARG
    assert call(o, ws=FAKE, ws_bytes=need - 1)[0] == B.POETX_ERR_WORKSPACE
    for field, bad in (("step", 0), ("beta1", 1.0), ("beta2", -0.1), ("eps", 0.0), ("m_p", None),
                       ("theta_r_out", None)):
        o2 = B.PoetxAdamC.from_buffer_copy(o)
        setattr(o2, field, bad)
        assert call(o2, ws=FAKE, ws_bytes=need)[0] == B.POETX_ERR_INVALID_ARG, field
    # theta dtype of the layer: F32 or BF16
    bad = layer(B)
    bad.theta_dtype = 7
    assert fwd(B, bad)[0] == B.POETX_ERR_INVALID_ARG
    bad.theta_dtype = B.POETX_BF16
    assert fwd(B, bad)[0] == B.POETX_OK


def test_binding_rejects_mismatched_buffers(B):
    """The binding checks every buffer the library reads or writes through a raw pointer
    (dtype, element count, contiguity) before any device call: a bf16 dtheta for the
    float32 gradient, a short G or a short saved-Q buffer raise ValueError."""
    import torch
    b, n = 64, 3
    p = b * (b - 1) // 2
    th32 = torch.zeros(n, p)
    th16 = th32.to(torch.bfloat16)
    dg = torch.zeros(n, b, b)
    with pytest.raises(ValueError):
        B.poetx_cnp(B.POETX_CNP_BWD, th16, b, dg=dg, dtheta=torch.empty_like(th16))
    with pytest.raises(ValueError):
        B.poetx_cnp(B.POETX_CNP_FWD, th32, b, g=torch.empty(n, b, b - 1))
    with pytest.raises(ValueError):
        B.poetx_cnp(B.POETX_CNP_FWD, th32, b, qsave=torch.empty(n - 1, b, b))
    with pytest.raises(ValueError):
        B.poetx_cnp(B.POETX_CNP_BWD, th32, b, dg=dg.to(torch.bfloat16))
    with pytest.raises(ValueError):
        B.poetx_cnp(B.POETX_CNP_FWD, th32[:, :p - 1], b)
