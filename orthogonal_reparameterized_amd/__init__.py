"""POET-X linear layer on AMD MI355X (gfx950): HIP kernels behind a C ABI.

The compute path lives in ``libpoetx.so`` (built from ``csrc/``); the Python
binding in :mod:`orthogonal_reparameterized_amd.binding` only marshals
arguments.  Import the binding explicitly; importing the package itself does not
load the shared library.
"""

__all__ = ["binding", "workloads"]
