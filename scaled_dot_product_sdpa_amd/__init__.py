"""Scaled dot-product attention for MI355X (gfx950): hand-written HIP kernels behind a
small C ABI (include/sdpa.h), with this package as the thin Python binding.

    o, lse = sdpa_forward(q, k, v, mask=None, scale=None, is_causal=False,
                          seq_lens_q=None, seq_lens_kv=None)
    # is_causal: False, True (top-left diagonal) or CAUSAL_BOTTOM_RIGHT (2)
    dq, dk, dv = sdpa_backward(q, k, v, o, dO, lse, mask=None, scale=None, is_causal=False,
                               seq_lens_q=None, seq_lens_kv=None)

Importing the package does not load the library; the first call does, and fails if it
has not been built (``python -m scaled_dot_product_sdpa_amd.build``).
"""

from .api import (BACKWARD_STAGES, CAUSAL_BOTTOM_RIGHT, CAUSAL_TOP_LEFT, EXPORTS, LIB_PATH,
                  BackwardCall, ForwardCall, PagedDecode, PagedDecodeCall, Problem, SdpaError,
                  load_library, sdpa_backward, sdpa_decode_paged, sdpa_forward,
                  sdpa_forward_noalloc)

__all__ = ["sdpa_forward", "sdpa_forward_noalloc", "sdpa_backward", "sdpa_decode_paged", "ForwardCall", "BackwardCall",
           "PagedDecodeCall", "PagedDecode", "BACKWARD_STAGES",
           "CAUSAL_TOP_LEFT", "CAUSAL_BOTTOM_RIGHT", "load_library", "LIB_PATH", "EXPORTS",
           "Problem", "SdpaError"]
