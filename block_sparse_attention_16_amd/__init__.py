"""MI355X (gfx950) dynamic block-sparse attention for video DiTs.

Block-importance estimation (mean-pooled scores, row softmax, Top-p) and a
sparse FlashAttention-style forward/backward with exact per-block attention
mass, implemented as hand-written HIP kernels behind a C ABI (libbsa.so,
declared in include/bsa.h).  This package is a thin torch binding of it.
"""
from .api import (Csr, bsa_backward, bsa_estimate_mask, bsa_forward, bsa_last_error, bsa_permute_tokens,
                  bsa_select_from_mass, bsa_select_from_mass_noalloc,
                  bsa_status_string, bsa_structured_mask, bsa_version, bsa_workspace_size, csr_from_host, make_shape,
                  num_rows)
from ._lib import BsaError, LIB_PATH, load

__all__ = ["Csr", "bsa_backward", "bsa_estimate_mask", "bsa_forward", "bsa_last_error", "bsa_permute_tokens",
           "bsa_select_from_mass", "bsa_select_from_mass_noalloc",
           "bsa_status_string", "bsa_structured_mask",
           "bsa_version", "bsa_workspace_size", "csr_from_host", "make_shape", "num_rows", "BsaError", "LIB_PATH",
           "load"]
