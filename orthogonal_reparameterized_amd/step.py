"""One POET-X layer step on the GPU through the C ABI: CNP forward (both sides),
layer forward, layer backward (which ends with the CNP backward).

Holds the device tensors of one layer (merged weight, packed thetas, G's,
activations and gradient buffers) so that steps can be repeated without
re-uploading.  Marshalling only; the arithmetic is in libpoetx.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def upload(arr, dtype: str, device="cuda"):
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


class LayerStep:
    def __init__(self, wl, inputs: dict, variant: str = "fast", device="cuda", perms: bool = True,
                 transposed_weight: bool = False, keep_x: bool = True, theta_dtype: str = "f32",
                 save_q: bool = True):
        """theta_dtype "bf16": inputs["theta_r"], inputs["theta_p"] hold bf16 bit patterns and
        theta is stored in bf16 (dtheta and the optimizer state stay float32).  save_q: the CNP
        forward keeps Q's planes of the full blocks (poetx_cnp's qsave) for the backward."""
        self.wl = wl
        self.variant = B.POETX_FAST if variant == "fast" else B.POETX_MEM
        act = _TORCH[wl.act]
        self.act = act
        dev = torch.device(device)
        self.dev = dev
        self.perm_in = upload(inputs["perm_in"], "i32", dev) if perms and inputs["perm_in"] is not None else None
        self.perm_out = upload(inputs["perm_out"], "i32", dev) if perms and inputs["perm_out"] is not None else None
        if wl.w == "i8":
            w = upload(inputs["w_q"], "i8", dev)
            s = upload(inputs["w_s"], "f32", dev)
        else:
            w = upload(inputs["w"], wl.w, dev)
            s = None
        # phase start: merge the weight-side permutations into W once (Method §2); optionally
        # also keep W'^T so that the backward product reads it k-contiguous
        self.w_merged_t = (torch.empty((wl.d_in, wl.d_out), dtype=w.dtype, device=dev)
                           if transposed_weight else None)
        self.w_merged, self.w_scale = B.poetx_merge_perm(w, self.perm_out, self.perm_in, s,
                                                         out_t=self.w_merged_t)
        del w
        # theta_R and theta_P (and G_R, G_P) live in one buffer each, so that the CNP
        # forward of both sides is a single poetx_cnp call over n_R + n_P blocks.  With a
        # smaller last block on a side (b not dividing its width) the side's theta and G
        # are flat: full blocks first, then the last block.
        self.n_r, self.n_p = wl.d_in // wl.b, wl.d_out // wl.b
        self.l_r, self.l_p = wl.d_in % wl.b, wl.d_out % wl.b
        self.ragged = bool(self.l_r or self.l_p)
        self.x = upload(inputs["x"], wl.act, dev)
        self.dz = upload(inputs["dz"], wl.act, dev)
        n, b = self.x.shape[0], wl.b
        if not self.ragged:
            self.theta = upload(np.concatenate([inputs["theta_r"], inputs["theta_p"]]), theta_dtype, dev)
            self.theta_r, self.theta_p = self.theta[:self.n_r], self.theta[self.n_r:]
            self.g = torch.empty((self.n_r + self.n_p, b, b), dtype=act, device=dev)
            self.g_r, self.g_p = self.g[:self.n_r], self.g[self.n_r:]
            self.q = B.qsave_like(self.theta, b) if save_q else None
            self.q_r, self.q_p = (self.q[:self.n_r], self.q[self.n_r:]) if save_q else (None, None)
        else:
            # one allocation per side, so that each side's buffer starts 16-byte aligned
            self.theta = None
            self.theta_r = upload(np.ravel(inputs["theta_r"]), theta_dtype, dev)
            self.theta_p = upload(np.ravel(inputs["theta_p"]), theta_dtype, dev)
            self.g = None
            self.g_r = torch.empty(self.n_r * b * b + self.l_r ** 2, dtype=act, device=dev)
            self.g_p = torch.empty(self.n_p * b * b + self.l_p ** 2, dtype=act, device=dev)
            self.q = None
            self.q_r = torch.empty((self.n_r, b, b), dtype=torch.float32, device=dev) if save_q and self.n_r else None
            self.q_p = torch.empty((self.n_p, b, b), dtype=torch.float32, device=dev) if save_q and self.n_p else None
        self.z = torch.empty((n, wl.d_out), dtype=act, device=dev)
        self.saved_b = torch.empty((n, wl.d_out), dtype=act, device=dev) if self.variant == B.POETX_FAST else None
        # fast: also keep the gathered input X~ for the backward (no second gather of x)
        self.saved_x = (torch.empty((n, wl.d_in), dtype=act, device=dev)
                        if self.variant == B.POETX_FAST and keep_x and self.perm_in is not None else None)
        self.dx = torch.empty((n, wl.d_in), dtype=act, device=dev)
        self.dtheta_r = torch.empty(self.theta_r.shape, dtype=torch.float32, device=dev)
        self.dtheta_p = torch.empty(self.theta_p.shape, dtype=torch.float32, device=dev)
        self.adam = None  # Adam state of the fused update (step_adam)
        self.layer = B.Layer(self.w_merged, self.theta_r, self.theta_p, self.g_r, self.g_p, b,
                             act_dtype=act, variant=self.variant, w_scale=self.w_scale,
                             perm_in=self.perm_in, perm_out=self.perm_out, w_merged_t=self.w_merged_t,
                             q_r=self.q_r, q_p=self.q_p)

    def cnp(self):
        b = self.wl.b
        if not self.ragged:
            # both sides share b: one call over the n_R + n_P blocks of the shared buffer
            B.poetx_cnp(B.POETX_CNP_FWD, self.theta, b, g=self.g, qsave=self.q)
            return
        p = b * (b - 1) // 2
        for theta, g, n, last, q in ((self.theta_r, self.g_r, self.n_r, self.l_r, self.q_r),
                                     (self.theta_p, self.g_p, self.n_p, self.l_p, self.q_p)):
            if n:
                B.poetx_cnp(B.POETX_CNP_FWD, theta[:n * p].view(n, p), b, g=g[:n * b * b].view(n, b, b), qsave=q)
            if last:
                B.poetx_cnp(B.POETX_CNP_FWD, theta[n * p:].view(1, last * (last - 1) // 2), last,
                            g=g[n * b * b:].view(1, last, last))

    def forward(self):
        B.poetx_forward(self.layer, self.x, self.z, self.saved_b, self.saved_x)

    def backward(self, want_dg=False):
        return B.poetx_backward(self.layer, self.x, self.dz, self.saved_b, saved_x=self.saved_x, dx=self.dx,
                                dtheta_r=self.dtheta_r, dtheta_p=self.dtheta_p, want_dg=want_dg)

    def step(self, want_dg=False):
        self.cnp()
        self.forward()
        return self.backward(want_dg)

    def step_adam(self, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, gamma=1.0, keep_dtheta=False):
        """A training step with the Adam update of theta fused into the backward's CNP pass
        (theta updated in place; dtheta also written when keep_dtheta)."""
        if self.adam is None:
            self.adam = B.AdamState.zeros_like(self.layer)
        self.cnp()
        self.forward()
        return B.poetx_backward_adam(self.layer, self.x, self.dz, self.adam, self.saved_b, lr=lr, betas=betas,
                                     eps=eps, gamma=gamma, saved_x=self.saved_x, dx=self.dx,
                                     dtheta_r=self.dtheta_r if keep_dtheta else None,
                                     dtheta_p=self.dtheta_p if keep_dtheta else None)
