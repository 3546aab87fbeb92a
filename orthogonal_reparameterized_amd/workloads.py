"""Seeded synthetic inputs for the POET-X layer workloads.

This module only draws random numbers and converts dtypes.  It holds none of
the layer's arithmetic, so both the CPU oracle (through the tests) and the HIP
path can be fed from it.  Random numbers are drawn in float64 with NumPy's
PCG64 and rounded once to the storage dtype (float32 round-to-nearest-even,
then bfloat16 round-to-nearest-even where the workload is bf16).

Workloads (the summary page measures single layers at Llama-8B-like shapes and
quantized training at 13B-like shapes; the shapes below stand in for those):

  1  fp32 layer, N=64 tokens, 256 -> 256, b=32
  2  CNP alone: 4096 independent b=256 blocks
  3  Llama-8B-like attention projection: N=8192, 4096 -> 4096, b=256 (bf16)
  4  Llama-8B-like MLP up-projection: N=8192, 4096 -> 14336, b=512 (bf16)
  5  POET-XQ 13B-like MLP: N=4096, 5120 -> 13824, b=256, int8 weight with
     per-output-row fp32 scales (mem variant only)
  6  workload 3 at block size b=64
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20260305


@dataclass(frozen=True)
class Workload:
    key: int
    name: str
    n_tokens: int = 0
    d_in: int = 0
    d_out: int = 0
    b: int = 0
    act: str = "bf16"        # activation dtype: "f32" | "bf16"
    w: str = "bf16"          # weight dtype: "f32" | "bf16" | "i8"
    g: str = "bf16"          # dtype G is produced in
    theta_std: float = 0.01
    w_var_den: int = 1       # W ~ N(0, 1/w_var_den)
    variants: tuple = ("fast", "mem")
    nblocks: int = 0         # CNP-only workload
    perms: bool = True

    @property
    def n_r(self):  # full b x b blocks of the input side
        return self.d_in // self.b

    @property
    def n_p(self):
        return self.d_out // self.b

    @property
    def l_r(self):  # size of the input side's last, smaller block (0: none)
        return self.d_in % self.b

    @property
    def l_p(self):
        return self.d_out % self.b

    @property
    def ragged(self):
        return bool(self.l_r or self.l_p)

    @property
    def p(self):
        return self.b * (self.b - 1) // 2

    def theta_len(self, side: str) -> int:
        n, last = (self.n_r, self.l_r) if side == "r" else (self.n_p, self.l_p)
        return n * self.p + last * (last - 1) // 2


WORKLOADS = {
    1: Workload(1, "fp32 layer 256->256 b=32 N=64", 64, 256, 256, 32, "f32", "f32", "f32",
                0.02, 256),
    2: Workload(2, "CNP 4096 blocks b=256", b=256, g="bf16", theta_std=0.01, nblocks=4096,
                variants=()),
    3: Workload(3, "attn-proj 4096->4096 b=256 N=8192", 8192, 4096, 4096, 256, "bf16", "bf16",
                "bf16", 0.01, 4096),
    4: Workload(4, "mlp-up 4096->14336 b=512 N=8192", 8192, 4096, 14336, 512, "bf16", "bf16",
                "bf16", 0.01, 4096),
    5: Workload(5, "xq-mlp 5120->13824 b=256 N=4096 int8", 4096, 5120, 13824, 256, "bf16", "i8",
                "bf16", 0.01, 5120, variants=("mem",)),
    # workload 3's shapes at the smaller block size b = 64 (64 + 64 blocks)
    6: Workload(6, "attn-proj 4096->4096 b=64 N=8192", 8192, 4096, 4096, 64, "bf16", "bf16",
                "bf16", 0.01, 4096),
}


# ---------------------------------------------------------------------------
# dtype helpers (bit-level; no layer arithmetic)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(arr, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array ("bf16" arrays are uint16 bit patterns)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def store(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 draws to the storage dtype (f32 RNE, then bf16 RNE)."""
    x32 = np.asarray(x64, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "f32":
        return x32
    raise ValueError(dtype)


def quantize_rows_int8(w64: np.ndarray):
    """Symmetric per-row absmax int8 quantizer used only to make int8 inputs.

    s[i] = max_k |W[i][k]| / 127 (stored as float32); q = clamp(rne(W / s), -127, 127).
    The page says only "low-bit W"; the oracle consumes (q, s) as given.
    """
    amax = np.abs(w64).max(axis=1)
    s = (np.where(amax > 0, amax, 1.0) / 127.0).astype(np.float32)
    q = np.clip(np.rint(w64 / s.astype(np.float64)[:, None]), -127, 127).astype(np.int8)
    return q, s


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------

def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(7)]


def make_layer_inputs(wl: Workload, n_tokens: int | None = None, seed: int | None = None,
                      perms: bool | None = None, theta_scale: float = 1.0):
    """Draw perm_in, perm_out, W, theta_R, theta_P, X, dZ for a layer workload.

    Returns a dict of host arrays in storage dtypes: bf16 arrays are uint16 bit
    patterns; W is (q int8, s float32) for the int8 workload.
    """
    n = wl.n_tokens if n_tokens is None else n_tokens
    seed = BASE_SEED + wl.key if seed is None else seed
    use_perm = wl.perms if perms is None else perms
    g_pin, g_pout, g_w, g_tr, g_tp, g_x, g_dz = _streams(seed)
    out = {}
    out["perm_in"] = g_pin.permutation(wl.d_in).astype(np.int32) if use_perm else None
    out["perm_out"] = g_pout.permutation(wl.d_out).astype(np.int32) if use_perm else None
    w64 = g_w.standard_normal((wl.d_out, wl.d_in)) / np.sqrt(wl.w_var_den)
    if wl.w == "i8":
        out["w_q"], out["w_s"] = quantize_rows_int8(w64)
    else:
        out["w"] = store(w64, wl.w)
    del w64
    # [n][p] when b divides both widths; otherwise flat, the blocks' packed vectors one
    # after another (the last block of a side is the smaller one)
    shp_r = (wl.n_r, wl.p) if not wl.ragged else (wl.theta_len("r"),)
    shp_p = (wl.n_p, wl.p) if not wl.ragged else (wl.theta_len("p"),)
    out["theta_r"] = (g_tr.standard_normal(shp_r) * wl.theta_std * theta_scale).astype(np.float32)
    out["theta_p"] = (g_tp.standard_normal(shp_p) * wl.theta_std * theta_scale).astype(np.float32)
    out["x"] = store(g_x.standard_normal((n, wl.d_in)), wl.act)
    out["dz"] = store(g_dz.standard_normal((n, wl.d_out)), wl.act)
    return out


def make_cnp_inputs(nblocks: int, b: int, theta_std: float, seed: int):
    """theta[n][p] ~ N(0, theta_std^2) (float32) and dG[n][b][b] ~ N(0, 1) (float32)."""
    g_t, g_d = [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(2)]
    p = b * (b - 1) // 2
    theta = (g_t.standard_normal((nblocks, p)) * theta_std).astype(np.float32)
    dg = g_d.standard_normal((nblocks, b, b)).astype(np.float32)
    return theta, dg
