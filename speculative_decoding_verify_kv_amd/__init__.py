"""MI355X (gfx950) speculative-decoding verify attention.

The computation lives in libverify_attn.so (hand-written HIP kernels behind a
C ABI, include/verify_attn.h).  This package only marshals arguments:
`_binding` mirrors the C entry points one to one, and `device` moves host
arrays into torch device tensors (torch supplies device memory and streams).
"""

from ._binding import (  # noqa: F401
    DTYPE_CODES,
    EXPORTED,
    LIB_PATH,
    VA_EHIP,
    VA_EINVAL,
    VA_EUNSUPPORTED,
    VA_EWORKSPACE,
    VA_FLAG_BAD_CTX,
    VA_FLAG_BAD_PAGE,
    VA_FLAG_BAD_PARENT,
    VA_FLAG_BAD_PATH,
    VA_FLAG_BAD_ROWS,
    VA_OK,
    Plan,
    VaPlanInfo,
    VaProblem,
    VerifyAttnError,
    load,
    make_problem,
    verify_attn_plan,
    verify_attn_plan_for_cus,
    verify_attn_plan_get_info,
    verify_attn_append_kv,
    verify_attn_promote_kv,
    verify_attn_promote_workspace_bytes,
    verify_attn_read_flags,
    verify_attn_run,
    verify_attn_run_merge,
    verify_attn_run_noalloc,
    verify_attn_run_partial,
    verify_attn_run_ragged,
    verify_attn_status_string,
)
