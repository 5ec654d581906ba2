"""HHR sparse-attention decode for MI355X (gfx950): a C-ABI library of HIP kernels.

Importing the package loads nothing; `long_context_decode_gkr_amd.binding` loads the built
library (libhhr.so) and fails loudly if it is missing.
"""
