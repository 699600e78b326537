"""MI355X (gfx950) GatedDeltaNet gated delta-rule: chunked varlen prefill and
pooled decode behind the C ABI in include/gdn.h.

The functions below are thin ctypes wrappers with the C names; the work runs
in the HIP kernels of libgdn.so (built by ``python -m
gateddeltanet_chunked_delta_amd.build``).  They raise if the library is
missing; there is no CPU fallback.
"""
from .binding import (GDN_BF16, GDN_F32, GdnError, GdnProblem, gdn_decode_multi,  # noqa: F401
                      gdn_decode_step,
                      gdn_prefill_varlen, gdn_prefill_varlen_noalloc, gdn_prefill_varlen_pooled,
                      gdn_prefill_workspace_bytes, load,
                      make_problem, status_string)
