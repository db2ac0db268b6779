"""prefill_gemm_amd — packed-weight products for MI355X (gfx950).

The hot path is hand-written HIP in ``csrc/`` behind the C ABI of
``include/pg.h`` (built into ``libpg.so``); this package is its thin Python
binding plus the layer-frame orchestration.  Importing it loads libpg and
fails loudly if the library has not been built: there is no CPU fallback.
"""
from ._lib import (PG_EINVAL, PG_ELAUNCH, PG_ETIMEOUT, PG_EUNSUPPORTED, PG_EWORKSPACE, PG_OK, PGError,
                   Q4TPWeight, Q82Weight, Q8Weight, argmax_rows, attn_kv_append, attn_prefill, expert_bank_q82, expert_bank_q4tp, gemv_q4tp, moe_route_sigmoid, add_rmsnorm, decode_frame_q8, decode_frame_q8_workspace, decode_frame_q8_status,
                   decode_frame_q8_workspace_bytes, decode_frame_timeouts, gemv_f16, gemv_q8, gemv_q82, gemv_q8_addnorm, gemv_q8_normed,
                   gemv_q8_residual, lib, moe_grouped, norm_parts,
                   moe_grouped_workspace_bytes, prefill_frame_q8, prefill_frame_q8_meta, prefill_frame_q8_workspace_bytes,
                   prefill_gemm_q8, prefill_gemm_q8_noalloc, prefill_gemm_q82, prefill_gemm_q4tp, prefill_gemm_q8_addnorm,
                   prefill_gemm_q8_workspace_bytes,
                   stream_read, strerror, version)
from .frame import PB_MAX, Frame, Prompt

lib()

__all__ = ["PG_OK", "PG_EINVAL", "PG_EUNSUPPORTED", "PG_ELAUNCH", "PG_EWORKSPACE", "PG_ETIMEOUT", "PGError",
           "Q8Weight", "Q82Weight", "Q4TPWeight", "gemv_q4tp", "argmax_rows", "moe_route_sigmoid", "attn_kv_append", "attn_prefill", "expert_bank_q82", "expert_bank_q4tp", "gemv_q82", "decode_frame_q8", "decode_frame_q8_workspace", "decode_frame_q8_status", "decode_frame_q8_workspace_bytes",
           "decode_frame_timeouts", "gemv_q8", "gemv_q8_addnorm", "gemv_q8_residual", "gemv_q8_normed",
           "norm_parts", "gemv_f16", "prefill_frame_q8", "prefill_frame_q8_meta", "prefill_frame_q8_workspace_bytes",
           "prefill_gemm_q8", "prefill_gemm_q8_noalloc", "prefill_gemm_q82", "prefill_gemm_q4tp", "prefill_gemm_q8_addnorm",
           "prefill_gemm_q8_workspace_bytes",
           "add_rmsnorm", "moe_grouped", "moe_grouped_workspace_bytes", "stream_read", "strerror", "version",
           "lib", "Frame", "Prompt", "PB_MAX"]
