"""MI355X-native small-q GQA decode attention: gfx950 HIP kernels behind a C ABI
(include/fr_decode_attn.h), with a thin ctypes binding of the same names."""
from .binding import (  # noqa: F401
    FR_ERR_CAPTURE, FR_ERR_HIP, FR_ERR_INVALID, FR_ERR_UNSUPPORTED, FR_ERR_WORKSPACE, FR_OK,
    FR_MAX_COPIES, FR_MAX_HEADS, FR_NOALLOC_SCRATCH_BYTES, FR_MAX_TOKENS, FR_MAX_TOKENS_UNMASKED,
    FR_PLAN_UNMASKED, FR_Q_F16, FR_Q_F32, FR_Q_ROUND_F16, FR_VARIANT_DECOMPOSED, FR_VARIANT_FUSED,
    FrError,
    fr_abi_version, fr_decode_attn, fr_decode_attn_batched, fr_decode_attn_ex, fr_decode_attn_gqa,
    fr_decode_attn_gqa_noalloc,
    fr_decode_attn_plan, fr_decode_attn_profile_events, fr_decode_attn_q16, fr_decode_attn_reserve,
    fr_decode_attn_workspace_query, fr_decode_attn_workspace_release,
    fr_decode_attn_workspace_size, fr_f16_copy_batch, fr_qkv_post, fr_status_str)
