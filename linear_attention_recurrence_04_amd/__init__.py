"""Gated DeltaNet (gated delta rule) layer core for MI355X (gfx950).

``gdn_chunk_prefill`` and ``gdn_decode_step`` call the C ABI of libgdn.so
(include/gdn.h).  The library is loaded on first use, so the seeded input
generator (``.inputs``) imports on machines without a GPU; a call without the
built library raises.
"""
from .binding import (GDN_DTYPE_BF16, GDN_DTYPE_F32, GdnError, GdnProblem,  # noqa: F401
                      gdn_abi_version, gdn_calib_copy, gdn_calib_mfma_loop, gdn_causal_conv1d,
                      gdn_gated_rmsnorm,
                      gdn_chunk_prefill, gdn_chunk_prefill_ckpt,
                      gdn_chunk_prefill_gated, gdn_decode_step_gated, gdn_decode_multi,
                      gdn_chunk_prefill_varlen, gdn_chunk_prefill_onchip,
                      gdn_chunk_prefill_workspace_bytes,
                      gdn_chunk_prefill_variant, gdn_decode_step, gdn_status_string,
                      make_problem, selected_prefill_kernel)
