"""recurrent_cell_amd: a CfC K-loop (forward + full BPTT) for MI355X (gfx950).

The compute lives in ``libcfc.so`` (hand-written HIP kernels behind a C ABI,
declared in include/cfc.h).  ``recurrent_cell_amd.cfc`` is the thin Python
binding with the same names; importing this package loads nothing, the
library is opened on first use and an error is raised if it is missing.
"""
__all__ = ["cfc", "inputs"]
