"""gqa_split_kv_amd -- split-KV grouped-query-attention decode for MI355X (gfx950).

The work runs in hand-written HIP kernels inside libgqa_decode.so, behind the C
ABI declared in include/gqa_decode.h (decode, multi-token decode) and
include/gqa_prefill.h (causal prefill).  This package holds that library's
sources (csrc/), its build script (build.py), the ctypes binding (binding.py)
and the seeded synthetic workloads (inputs.py).
"""
from .binding import (  # noqa: F401
    EXPORTS, GQA_DTYPE_BF16, GQA_DTYPE_F16, GQA_DTYPE_F32, GqaArgs, GqaError, GqaPlan, GqaPrefillArgs, decode,
    gqa_decode, gqa_decode_ex, gqa_decode_f16, gqa_decode_noalloc, gqa_decode_f32, gqa_decode_make_plan, gqa_decode_validate,
    gqa_decode_workspace_bytes, gqa_last_error_message, gqa_prefill, gqa_prefill_ex, gqa_prefill_f16,
    gqa_prefill_validate, gqa_prefill_workspace_bytes, gqa_probe_copy, gqa_probe_read, gqa_release, gqa_status_str, lib, make_args,
    make_prefill_args, prefill)
