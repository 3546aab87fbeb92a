"""Thin ctypes binding over libpoetx (include/poetx.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory (its caching allocator) and the
current HIP stream.  A nonzero status from the library raises ``PoetxError``.
If the shared library is missing this module raises at import: there is no
fallback path.

Python names mirror the C entry points:
    poetx_merge_perm, poetx_cnp, poetx_forward, poetx_backward
plus ``Layer`` (the poetx_layer descriptor) and the measurement hooks.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpoetx.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build it with `python -m orthogonal_reparameterized_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

POETX_OK, POETX_ERR_INVALID_ARG, POETX_ERR_SHAPE = 0, -1, -2
POETX_ERR_UNSUPPORTED, POETX_ERR_WORKSPACE, POETX_ERR_HIP = -3, -4, -5
POETX_F32, POETX_BF16, POETX_I8 = 0, 1, 2
POETX_FAST, POETX_MEM = 0, 1
POETX_CNP_FWD, POETX_CNP_BWD = 0, 1

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t


class PoetxLayerC(ctypes.Structure):
    _fields_ = [
        ("d_in", _i64), ("d_out", _i64), ("b", _i64),
        ("act_dtype", _i32), ("w_dtype", _i32), ("g_dtype", _i32), ("variant", _i32),
        ("w_merged", _vp), ("w_merged_t", _vp), ("w_scale", _vp), ("perm_in", _vp), ("perm_out", _vp),
        ("theta_r", _vp), ("theta_p", _vp), ("g_r", _vp), ("g_p", _vp), ("theta_dtype", _i32),
        ("q_r", _vp), ("q_p", _vp),
    ]


class PoetxAdamC(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("eps", ctypes.c_float),
        ("gamma", ctypes.c_float), ("step", _i64),
        ("m_r", _vp), ("v_r", _vp), ("m_p", _vp), ("v_p", _vp), ("theta_r_out", _vp), ("theta_p_out", _vp),
    ]


_lib.poetx_merge_perm.argtypes = [_vp, _vp, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.poetx_cnp.argtypes = [_i32, _i64, _i64, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _vp, _vp,
                           ctypes.POINTER(_sz), _vp]
_lib.poetx_forward.argtypes = [ctypes.POINTER(PoetxLayerC), _i64, _vp, _vp, _vp, _vp, _vp,
                               ctypes.POINTER(_sz), _vp]
_lib.poetx_backward.argtypes = [ctypes.POINTER(PoetxLayerC), _i64, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _vp, ctypes.POINTER(_sz), _vp]
_lib.poetx_cnp_noalloc.argtypes = [_i32, _i64, _i64, _vp, _i32, _vp, _i32, _vp, _i32, _vp, _vp]
_lib.poetx_backward_adam.argtypes = [ctypes.POINTER(PoetxLayerC), _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                     ctypes.POINTER(PoetxAdamC), _vp, ctypes.POINTER(_sz), _vp]
_lib.poetx_fold.argtypes = [ctypes.POINTER(PoetxLayerC), _vp, _vp, ctypes.POINTER(_sz), _vp]
_lib.poetx_adam_step.argtypes = [_i64, _vp, _i32, _vp, _vp, _vp, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                 ctypes.c_float, _i64, ctypes.c_float, _vp]
_lib.poetx_status_string.argtypes = [ctypes.c_int]
_lib.poetx_status_string.restype = ctypes.c_char_p
_lib.poetx_version.restype = ctypes.c_char_p
_lib.poetx_prof_enable.argtypes = [_i32]
_lib.poetx_prof_read.argtypes = [ctypes.c_char_p, _sz]
_lib.poetx_prof_only.argtypes = [ctypes.c_char_p]
for _f in ("poetx_merge_perm", "poetx_cnp", "poetx_cnp_noalloc", "poetx_forward", "poetx_backward", "poetx_backward_adam", "poetx_fold",
           "poetx_adam_step",
           "poetx_prof_enable", "poetx_prof_only", "poetx_prof_read"):
    getattr(_lib, _f).restype = ctypes.c_int

EXPORTED = ("poetx_merge_perm", "poetx_cnp", "poetx_cnp_noalloc", "poetx_forward", "poetx_backward", "poetx_backward_adam", "poetx_fold",
            "poetx_adam_step",
            "poetx_status_string", "poetx_version", "poetx_prof_enable", "poetx_prof_only", "poetx_prof_read")


class PoetxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.poetx_status_string(status).decode()} ({status})")


def _check(st: int, where: str):
    if st != POETX_OK:
        raise PoetxError(st, where)


def library_path() -> str:
    return _LIB_PATH


def version() -> str:
    return _lib.poetx_version().decode()


_DT = {torch.float32: POETX_F32, torch.bfloat16: POETX_BF16, torch.int8: POETX_I8}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _ptr(t: Optional[torch.Tensor], align: int = 16):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if t.data_ptr() % align:
        raise ValueError(f"tensor must be {align}-byte aligned")
    return ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


# Scratch tensors keyed by (device, stream): each is allocated while its stream is the
# current one and only ever used by calls on that stream, so the caching allocator's
# stream ordering makes both the reuse between calls and the release of an outgrown
# buffer safe.  Layers driven on different streams get different workspaces.
_ws_cache: dict = {}


def _workspace(dev: torch.device, nbytes: int) -> torch.Tensor:
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    key = (idx, torch.cuda.current_stream(idx).cuda_stream)
    t = _ws_cache.get(key)
    if t is None or t.numel() < nbytes:
        with torch.cuda.device(idx):
            t = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=f"cuda:{idx}")
        _ws_cache[key] = t
    return t


def release_workspace():
    _ws_cache.clear()


# --------------------------------------------------------------------------
def poetx_merge_perm(w: torch.Tensor, perm_out=None, perm_in=None, w_scale=None,
                     out: Optional[torch.Tensor] = None, out_scale: Optional[torch.Tensor] = None,
                     out_t: Optional[torch.Tensor] = None):
    """W'[i][k] = W[perm_out[i]][perm_in[k]] (and s'[i] = s[perm_out[i]] for int8).

    If out_t is given it also receives W'^T ([d_in][d_out]).
    """
    d_out, d_in = w.shape
    out = torch.empty_like(w) if out is None else out
    if w.dtype == torch.int8 and out_scale is None:
        out_scale = torch.empty_like(w_scale)
    st = _lib.poetx_merge_perm(_ptr(w), _ptr(w_scale), _dt(w), d_out, d_in, _ptr(perm_out),
                               _ptr(perm_in), _ptr(out), _ptr(out_scale) if w.dtype == torch.int8 else None,
                               _ptr(out_t), _stream(w.device))
    _check(st, "poetx_merge_perm")
    return out, (out_scale if w.dtype == torch.int8 else None)


def _need(t: Optional[torch.Tensor], name: str, numel: int, dtypes) -> None:
    """A buffer the library reads or writes through a raw pointer: contiguous, of one of the
    expected dtypes and with exactly the elements the call touches."""
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    if t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def qsave_like(theta: torch.Tensor, b: int) -> torch.Tensor:
    """A buffer for poetx_cnp's qsave (n * b * b * 4 bytes, 16-byte aligned)."""
    return torch.empty((theta.shape[0], b, b), dtype=torch.float32, device=theta.device)


def poetx_cnp(direction: int, theta: torch.Tensor, b: int, *, g: Optional[torch.Tensor] = None,
              g_dtype: torch.dtype = torch.bfloat16, dg: Optional[torch.Tensor] = None,
              dtheta: Optional[torch.Tensor] = None, qsave: Optional[torch.Tensor] = None):
    """FWD: returns G [n][b][b] in g_dtype; BWD: returns dtheta [n][b(b-1)/2] from dg.
    qsave (optional, from qsave_like): FWD fills it, BWD on the same theta reads Q from it."""
    n = theta.shape[0]
    dev = theta.device
    p = b * (b - 1) // 2
    # the library writes through raw pointers: every buffer's dtype and size is checked here
    _need(theta, "theta", n * p, (torch.float32, torch.bfloat16))
    if direction == POETX_CNP_FWD:
        g = torch.empty((n, b, b), dtype=g_dtype, device=dev) if g is None else g
        _need(g, "g", n * b * b, (torch.float32, torch.bfloat16))
        gdt, dgdt = _dt(g), POETX_F32
    else:
        dtheta = torch.empty(theta.shape, dtype=torch.float32, device=dev) if dtheta is None else dtheta
        _need(dg, "dg", n * b * b, (torch.float32,))
        _need(dtheta, "dtheta", n * p, (torch.float32,))
        gdt, dgdt = POETX_F32, _dt(dg)
    if qsave is not None:
        _need(qsave, "qsave", n * b * b, (torch.float32,))
    tdt = _dt(theta)
    nbytes = _sz(0)
    _check(_lib.poetx_cnp(direction, n, b, None, tdt, None, gdt, None, None, dgdt, None, None,
                          ctypes.byref(nbytes), None), "poetx_cnp(size)")
    ws = _workspace(dev, nbytes.value)
    nb = _sz(ws.numel())
    # poetx_cnp takes element-aligned theta, G and dG (a smaller last block of a side
    # sits at an offset of whole blocks, which need not be a multiple of 16 bytes)
    def ep(t):
        return None if t is None else _ptr(t, t.element_size())
    st = _lib.poetx_cnp(direction, n, b, ep(theta), tdt, ep(g), gdt, _ptr(qsave), ep(dg), dgdt, ep(dtheta),
                        _ptr(ws), ctypes.byref(nb), _stream(dev))
    _check(st, "poetx_cnp")
    return g if direction == POETX_CNP_FWD else dtheta


@dataclass
class Layer:
    """Python view of poetx_layer: the tensors stay owned by the caller."""
    w_merged: torch.Tensor
    theta_r: torch.Tensor
    theta_p: torch.Tensor
    g_r: torch.Tensor
    g_p: torch.Tensor
    b: int
    act_dtype: torch.dtype = torch.bfloat16
    variant: int = POETX_FAST
    w_scale: Optional[torch.Tensor] = None
    perm_in: Optional[torch.Tensor] = None
    perm_out: Optional[torch.Tensor] = None
    w_merged_t: Optional[torch.Tensor] = None
    q_r: Optional[torch.Tensor] = None    # qsave buffers the CNP forward filled (full blocks)
    q_p: Optional[torch.Tensor] = None

    @property
    def d_out(self):
        return self.w_merged.shape[0]

    @property
    def d_in(self):
        return self.w_merged.shape[1]

    def to_c(self) -> PoetxLayerC:
        c = PoetxLayerC()
        c.d_in, c.d_out, c.b = self.d_in, self.d_out, self.b
        c.act_dtype = _DT[self.act_dtype]
        c.w_dtype = _dt(self.w_merged)
        c.g_dtype = _dt(self.g_r)
        c.variant = self.variant
        c.theta_dtype = _dt(self.theta_r)
        for q, d in ((self.q_r, self.d_in), (self.q_p, self.d_out)):
            if q is not None:
                _need(q, "q_r / q_p", (d // self.b) * self.b * self.b, (torch.float32,))
        for name in ("w_merged", "w_merged_t", "w_scale", "perm_in", "perm_out", "theta_r", "theta_p",
                     "g_r", "g_p", "q_r", "q_p"):
            p = _ptr(getattr(self, name))
            setattr(c, name, p.value if p is not None else None)
        return c


def poetx_forward(layer: Layer, x: torch.Tensor, z: Optional[torch.Tensor] = None,
                  saved_b: Optional[torch.Tensor] = None, saved_x: Optional[torch.Tensor] = None):
    """Returns (z, saved_b); saved_b is None for the mem variant.  saved_x (fast variant,
    optional, [N][d_in]) receives the gathered input for poetx_backward."""
    L = layer.to_c()
    n = x.shape[0]
    dev = x.device
    z = torch.empty((n, layer.d_out), dtype=layer.act_dtype, device=dev) if z is None else z
    if layer.variant == POETX_FAST and saved_b is None:
        saved_b = torch.empty((n, layer.d_out), dtype=layer.act_dtype, device=dev)
    if layer.variant == POETX_MEM:
        saved_b = None
    nbytes = _sz(0)
    _check(_lib.poetx_forward(ctypes.byref(L), n, None, None, None, _ptr(saved_x), None, ctypes.byref(nbytes),
                              None), "poetx_forward(size)")
    ws = _workspace(dev, nbytes.value)
    nb = _sz(ws.numel())
    st = _lib.poetx_forward(ctypes.byref(L), n, _ptr(x), _ptr(z), _ptr(saved_b), _ptr(saved_x), _ptr(ws),
                            ctypes.byref(nb), _stream(dev))
    _check(st, "poetx_forward")
    return z, saved_b


def poetx_backward(layer: Layer, x: torch.Tensor, dz: torch.Tensor,
                   saved_b: Optional[torch.Tensor] = None, *, saved_x=None, dx=None, dtheta_r=None,
                   dtheta_p=None, want_dg: bool = False):
    """Returns dict(dx, dtheta_r, dtheta_p[, dg_r, dg_p]).  saved_x: what poetx_forward wrote
    into its saved_x, or None."""
    L = layer.to_c()
    n = x.shape[0]
    dev = x.device
    dx = torch.empty((n, layer.d_in), dtype=layer.act_dtype, device=dev) if dx is None else dx
    dtheta_r = torch.empty(layer.theta_r.shape, dtype=torch.float32, device=dev) if dtheta_r is None else dtheta_r
    dtheta_p = torch.empty(layer.theta_p.shape, dtype=torch.float32, device=dev) if dtheta_p is None else dtheta_p
    _need(dx, "dx", n * layer.d_in, (layer.act_dtype,))
    _need(dtheta_r, "dtheta_r", layer.theta_r.numel(), (torch.float32,))
    _need(dtheta_p, "dtheta_p", layer.theta_p.numel(), (torch.float32,))
    dg_r = dg_p = None
    if want_dg:
        b = layer.b
        if layer.d_in % b or layer.d_out % b:  # flat: full blocks, then the smaller last block
            dg_r = torch.empty((layer.d_in // b) * b * b + (layer.d_in % b) ** 2, dtype=torch.float32, device=dev)
            dg_p = torch.empty((layer.d_out // b) * b * b + (layer.d_out % b) ** 2, dtype=torch.float32,
                               device=dev)
        else:
            dg_r = torch.empty((layer.d_in // b, b, b), dtype=torch.float32, device=dev)
            dg_p = torch.empty((layer.d_out // b, b, b), dtype=torch.float32, device=dev)
    nbytes = _sz(0)
    _check(_lib.poetx_backward(ctypes.byref(L), n, None, None, None, _ptr(saved_x), None, None, None,
                               _ptr(dg_r), _ptr(dg_p), None, ctypes.byref(nbytes), None), "poetx_backward(size)")
    ws = _workspace(dev, nbytes.value)
    nb = _sz(ws.numel())
    st = _lib.poetx_backward(ctypes.byref(L), n, _ptr(x), _ptr(dz), _ptr(saved_b), _ptr(saved_x), _ptr(dx),
                             _ptr(dtheta_r), _ptr(dtheta_p), _ptr(dg_r), _ptr(dg_p), _ptr(ws),
                             ctypes.byref(nb), _stream(dev))
    _check(st, "poetx_backward")
    out = dict(dx=dx, dtheta_r=dtheta_r, dtheta_p=dtheta_p)
    if want_dg:
        out.update(dg_r=dg_r, dg_p=dg_p)
    return out


def poetx_fold(layer: Layer, w_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The layer's effective weight [d_out][d_in] in original coordinates (see poetx.h)."""
    L = layer.to_c()
    dev = layer.w_merged.device
    if w_out is None:
        w_out = torch.empty((layer.d_out, layer.d_in), dtype=layer.w_merged.dtype, device=dev)
    nbytes = _sz(0)
    _check(_lib.poetx_fold(ctypes.byref(L), None, None, ctypes.byref(nbytes), None), "poetx_fold(size)")
    ws = _workspace(dev, nbytes.value)
    nb = _sz(ws.numel())
    _check(_lib.poetx_fold(ctypes.byref(L), _ptr(w_out), _ptr(ws), ctypes.byref(nb), _stream(dev)),
           "poetx_fold")
    return w_out


def poetx_adam_step(theta: torch.Tensor, grad: torch.Tensor, m: torch.Tensor, v: torch.Tensor, *, lr: float,
                    step: int, betas=(0.9, 0.999), eps: float = 1e-8, gamma: float = 1.0):
    """In-place Adam update of packed theta (float32 or bf16) and its float32 state m, v
    from grad = dtheta."""
    _need(theta, "theta", theta.numel(), (torch.float32, torch.bfloat16))
    for t, nm in ((grad, "grad"), (m, "m"), (v, "v")):
        _need(t, nm, theta.numel(), (torch.float32,))
    _check(_lib.poetx_adam_step(theta.numel(), _ptr(theta), _dt(theta), _ptr(grad), _ptr(m), _ptr(v), lr,
                                betas[0], betas[1], eps, step, gamma, _stream(theta.device)), "poetx_adam_step")
    return theta


@dataclass
class AdamState:
    """Adam state of a layer's two packed thetas (float32, theta's layout) and its step."""
    m_r: torch.Tensor
    v_r: torch.Tensor
    m_p: torch.Tensor
    v_p: torch.Tensor
    step: int = 0

    @staticmethod
    def zeros_like(layer: "Layer") -> "AdamState":
        z = [torch.zeros(t.shape, dtype=torch.float32, device=t.device)
             for t in (layer.theta_r, layer.theta_r, layer.theta_p, layer.theta_p)]
        return AdamState(*z)


def poetx_backward_adam(layer: Layer, x: torch.Tensor, dz: torch.Tensor, state: AdamState,
                        saved_b: Optional[torch.Tensor] = None, *, lr: float, betas=(0.9, 0.999),
                        eps: float = 1e-8, gamma: float = 1.0, saved_x=None, dx=None, dtheta_r=None,
                        dtheta_p=None):
    """The backward with one Adam step of layer.theta_r / layer.theta_p (in place) fused into
    the CNP backward's last pass; state.step advances by one.  Returns dict(dx[, dtheta_*])."""
    L = layer.to_c()
    n = x.shape[0]
    dev = x.device
    dx = torch.empty((n, layer.d_in), dtype=layer.act_dtype, device=dev) if dx is None else dx
    _need(dx, "dx", n * layer.d_in, (layer.act_dtype,))
    for t, th, nm in ((state.m_r, layer.theta_r, "m_r"), (state.v_r, layer.theta_r, "v_r"),
                      (state.m_p, layer.theta_p, "m_p"), (state.v_p, layer.theta_p, "v_p")):
        _need(t, nm, th.numel(), (torch.float32,))
    for t, th, nm in ((dtheta_r, layer.theta_r, "dtheta_r"), (dtheta_p, layer.theta_p, "dtheta_p")):
        if t is not None:
            _need(t, nm, th.numel(), (torch.float32,))
    state.step += 1
    opt = PoetxAdamC()
    opt.lr, opt.beta1, opt.beta2, opt.eps, opt.gamma, opt.step = lr, betas[0], betas[1], eps, gamma, state.step
    for name in ("m_r", "v_r", "m_p", "v_p"):
        setattr(opt, name, _ptr(getattr(state, name)).value)
    opt.theta_r_out, opt.theta_p_out = _ptr(layer.theta_r).value, _ptr(layer.theta_p).value
    nbytes = _sz(0)
    _check(_lib.poetx_backward_adam(ctypes.byref(L), n, None, None, None, _ptr(saved_x), None, None, None,
                                    ctypes.byref(opt), None, ctypes.byref(nbytes), None), "poetx_backward_adam(size)")
    ws = _workspace(dev, nbytes.value)
    nb = _sz(ws.numel())
    st = _lib.poetx_backward_adam(ctypes.byref(L), n, _ptr(x), _ptr(dz), _ptr(saved_b), _ptr(saved_x), _ptr(dx),
                                  _ptr(dtheta_r), _ptr(dtheta_p), ctypes.byref(opt), _ptr(ws), ctypes.byref(nb),
                                  _stream(dev))
    _check(st, "poetx_backward_adam")
    out = dict(dx=dx)
    if dtheta_r is not None:
        out.update(dtheta_r=dtheta_r, dtheta_p=dtheta_p)
    return out


def prof_enable(on: bool = True):
    _check(_lib.poetx_prof_enable(1 if on else 0), "poetx_prof_enable")


def prof_only(label: Optional[str] = None):
    """Record only the launches labelled `label` (None: every launch)."""
    _check(_lib.poetx_prof_only(label.encode() if label else None), "poetx_prof_only")


def prof_read() -> dict:
    """{kernel label: (launches, total_ms, min_ms, max_ms)} recorded by this thread since
    the last read."""
    buf = ctypes.create_string_buffer(1 << 16)
    _check(_lib.poetx_prof_read(buf, len(buf)), "poetx_prof_read")
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms, mn, mx = line.split()
        out[name] = (int(n), float(ms), float(mn), float(mx))
    return out


# Raw handle for tests of the host-side validation (calls that fail before any launch).
raw = _lib
