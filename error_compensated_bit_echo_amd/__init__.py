"""Echo rank pipeline for MI355X (gfx950): error-compensated 4-bit all-reduce,
per-rank compute path.

`binding` wraps the C-ABI library libecho (HIP kernels); `inputs` draws the
seeded synthetic workloads.  Importing this package loads nothing: the
library is loaded on first use of `binding`.
"""
__all__ = ["binding", "inputs"]
