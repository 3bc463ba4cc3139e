"""ctypes binding of libverify_attn.so (include/verify_attn.h).

Argument marshalling only: every step of verify attention runs in the HIP
kernels of the shared library.  Device buffers are passed as raw pointers
(torch tensors' data_ptr()), streams as hipStream_t handles.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# VERIFY_ATTN_LIB names another build of the same library (the host-sanitizer
# build of tests/run_sanitized.py); the default is the in-tree build.
LIB_PATH = os.environ.get("VERIFY_ATTN_LIB") or os.path.join(HERE, "libverify_attn.so")

VA_OK, VA_EINVAL, VA_EUNSUPPORTED, VA_EWORKSPACE, VA_EHIP = 0, -1, -2, -3, -4
VA_F32, VA_F16, VA_BF16, VA_Q8_0 = 0, 1, 2, 3
VA_FLAG_BAD_CTX, VA_FLAG_BAD_PAGE, VA_FLAG_BAD_PARENT, VA_FLAG_BAD_PATH, VA_FLAG_BAD_ROWS = 0x1, 0x2, 0x4, 0x8, 0x10

DTYPE_CODES = {"f32": VA_F32, "f16": VA_F16, "bf16": VA_BF16, "q8_0": VA_Q8_0}


class VaProblem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("rows_per_seq", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("max_ctx", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("has_parent", ctypes.c_int32),
        ("max_total_rows", ctypes.c_int32),
    ]


class VaPlanInfo(ctypes.Structure):
    _fields_ = [
        ("num_splits", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("row_groups", ctypes.c_int32),
        ("rows_per_group", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("pages_per_split", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class VerifyAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {verify_attn_status_string(status)} ({status})")


_lib = None
EXPORTED = (
    "verify_attn_plan", "verify_attn_plan_for_cus", "verify_attn_plan_get_info", "verify_attn_plan_destroy",
    "verify_attn_run", "verify_attn_run_ragged", "verify_attn_run_partial", "verify_attn_run_merge",
    "verify_attn_run_noalloc", "verify_attn_append_kv",
    "verify_attn_promote_kv", "verify_attn_promote_workspace_bytes", "verify_attn_read_flags",
    "verify_attn_status_string",
)


def load(path: Optional[str] = None):
    """Load the shared library (raises if it is not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run speculative_decoding_verify_kv_amd.build.build()")
    lib = ctypes.CDLL(p)
    vp = ctypes.c_void_p
    i32 = ctypes.c_int32
    plan_pp = ctypes.POINTER(vp)
    lib.verify_attn_plan.argtypes = [ctypes.POINTER(VaProblem), i32, i32, plan_pp, ctypes.POINTER(ctypes.c_size_t)]
    lib.verify_attn_plan_for_cus.argtypes = [ctypes.POINTER(VaProblem), i32, i32, plan_pp,
                                             ctypes.POINTER(ctypes.c_size_t)]
    lib.verify_attn_plan_get_info.argtypes = [vp, ctypes.POINTER(VaPlanInfo)]
    lib.verify_attn_plan_destroy.argtypes = [vp]
    lib.verify_attn_plan_destroy.restype = None
    run_args = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.verify_attn_run.argtypes = run_args
    lib.verify_attn_run_ragged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, ctypes.c_size_t,
                                           vp]
    lib.verify_attn_run_partial.argtypes = run_args
    lib.verify_attn_run_merge.argtypes = [vp, i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.verify_attn_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
    lib.verify_attn_append_kv.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.verify_attn_promote_kv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.verify_attn_promote_workspace_bytes.argtypes = [vp]
    lib.verify_attn_promote_workspace_bytes.restype = ctypes.c_size_t
    lib.verify_attn_read_flags.argtypes = [vp, vp, vp, ctypes.POINTER(ctypes.c_uint32)]
    lib.verify_attn_status_string.argtypes = [i32]
    lib.verify_attn_status_string.restype = ctypes.c_char_p
    for n in ("verify_attn_plan", "verify_attn_plan_for_cus", "verify_attn_plan_get_info", "verify_attn_run",
              "verify_attn_run_ragged",
              "verify_attn_run_partial", "verify_attn_run_merge", "verify_attn_run_noalloc", "verify_attn_append_kv",
              "verify_attn_promote_kv",
              "verify_attn_read_flags"):
        getattr(lib, n).restype = i32
    if path is None:
        _lib = lib
    return lib


def verify_attn_status_string(status: int) -> str:
    return load().verify_attn_status_string(int(status)).decode()


def _check(st: int, what: str):
    if st != VA_OK:
        raise VerifyAttnError(st, what)


def make_problem(*, num_seqs, rows_per_seq, num_q_heads, num_kv_heads, head_dim, num_pages, max_pages_per_seq,
                 max_ctx, q_dtype="bf16", kv_dtype="q8_0", out_dtype="f16", scale=0.0, has_parent=False,
                 page_size=16, max_total_rows=0) -> VaProblem:
    return VaProblem(num_seqs=num_seqs, rows_per_seq=rows_per_seq, num_q_heads=num_q_heads,
                     num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size, num_pages=num_pages,
                     max_pages_per_seq=max_pages_per_seq, max_ctx=max_ctx, q_dtype=DTYPE_CODES[q_dtype],
                     kv_dtype=DTYPE_CODES[kv_dtype], out_dtype=DTYPE_CODES[out_dtype], scale=float(scale),
                     has_parent=int(bool(has_parent)), max_total_rows=int(max_total_rows))


class Plan:
    """Owns a va_plan*; destroyed with the object."""

    def __init__(self, handle: ctypes.c_void_p, workspace_bytes: int, problem: VaProblem):
        self.handle = handle
        self.workspace_bytes = int(workspace_bytes)
        self.problem = problem

    def info(self) -> VaPlanInfo:
        return verify_attn_plan_get_info(self)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.verify_attn_plan_destroy(h)
            self.handle = None


def verify_attn_plan(problem: VaProblem, num_splits: int = 0, device_ordinal: int = 0) -> Plan:
    lib = load()
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    _check(lib.verify_attn_plan(ctypes.byref(problem), int(num_splits), int(device_ordinal), ctypes.byref(h),
                                ctypes.byref(ws)), "verify_attn_plan")
    return Plan(h, ws.value, problem)


def verify_attn_plan_for_cus(problem: VaProblem, num_splits: int, num_cus: int) -> Plan:
    lib = load()
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    _check(lib.verify_attn_plan_for_cus(ctypes.byref(problem), int(num_splits), int(num_cus), ctypes.byref(h),
                                        ctypes.byref(ws)), "verify_attn_plan_for_cus")
    return Plan(h, ws.value, problem)


def verify_attn_plan_get_info(plan: Plan) -> VaPlanInfo:
    info = VaPlanInfo()
    _check(load().verify_attn_plan_get_info(plan.handle, ctypes.byref(info)), "verify_attn_plan_get_info")
    return info


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream


def verify_attn_run(plan: Plan, q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent, num_splits,
                    out, lse, workspace, workspace_bytes=None, stream=None, *, raise_on_error=True) -> int:
    wsb = plan.workspace_bytes if workspace_bytes is None else int(workspace_bytes)
    st = load().verify_attn_run(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                                _ptr(block_table), _ptr(ctx_lens), _ptr(parent), int(num_splits), _ptr(out),
                                _ptr(lse), _ptr(workspace), wsb, _stream(stream))
    if raise_on_error:
        _check(st, "verify_attn_run")
    return st


def verify_attn_run_ragged(plan: Plan, q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, cu_rows, parent,
                           num_splits, out, lse, workspace, workspace_bytes=None, stream=None, *,
                           raise_on_error=True) -> int:
    wsb = plan.workspace_bytes if workspace_bytes is None else int(workspace_bytes)
    st = load().verify_attn_run_ragged(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                       _ptr(v_scale), _ptr(block_table), _ptr(ctx_lens), _ptr(cu_rows), _ptr(parent),
                                       int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), wsb, _stream(stream))
    if raise_on_error:
        _check(st, "verify_attn_run_ragged")
    return st


def verify_attn_run_partial(plan: Plan, q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent,
                            num_splits, out, lse, workspace, workspace_bytes=None, stream=None,
                            *, raise_on_error=True) -> int:
    wsb = plan.workspace_bytes if workspace_bytes is None else int(workspace_bytes)
    st = load().verify_attn_run_partial(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                        _ptr(v_scale), _ptr(block_table), _ptr(ctx_lens), _ptr(parent),
                                        int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), wsb, _stream(stream))
    if raise_on_error:
        _check(st, "verify_attn_run_partial")
    return st


def verify_attn_run_merge(plan: Plan, num_splits, out, lse, workspace, workspace_bytes=None, stream=None,
                          *, raise_on_error=True) -> int:
    wsb = plan.workspace_bytes if workspace_bytes is None else int(workspace_bytes)
    st = load().verify_attn_run_merge(plan.handle, int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), wsb,
                                      _stream(stream))
    if raise_on_error:
        _check(st, "verify_attn_run_merge")
    return st


def verify_attn_run_noalloc(plan: Plan, q, k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent,
                            num_splits, out, lse, flags, stream=None, *, raise_on_error=True) -> int:
    st = load().verify_attn_run_noalloc(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                        _ptr(v_scale), _ptr(block_table), _ptr(ctx_lens), _ptr(parent),
                                        int(num_splits), _ptr(out), _ptr(lse), _ptr(flags), _stream(stream))
    if raise_on_error:
        _check(st, "verify_attn_run_noalloc")
    return st


def verify_attn_append_kv(plan: Plan, k_new, v_new, new_dtype: str, k_pool, v_pool, k_scale, v_scale, block_table,
                          ctx_lens, workspace, workspace_bytes=None, stream=None, *, raise_on_error=True) -> int:
    wsb = plan.workspace_bytes if workspace_bytes is None else int(workspace_bytes)
    st = load().verify_attn_append_kv(plan.handle, _ptr(k_new), _ptr(v_new), DTYPE_CODES[new_dtype], _ptr(k_pool),
                                      _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(ctx_lens),
                                      _ptr(workspace), wsb, _stream(stream))
    if raise_on_error:
        _check(st, "verify_attn_append_kv")
    return st


def verify_attn_promote_workspace_bytes(plan: Plan) -> int:
    return int(load().verify_attn_promote_workspace_bytes(plan.handle))


def verify_attn_promote_kv(plan: Plan, accepted, n_accepted, parent, k_pool, v_pool, k_scale, v_scale, block_table,
                           ctx_lens, new_ctx, workspace, workspace_bytes=None, stream=None, *,
                           raise_on_error=True) -> int:
    wsb = verify_attn_promote_workspace_bytes(plan) if workspace_bytes is None else int(workspace_bytes)
    st = load().verify_attn_promote_kv(plan.handle, _ptr(accepted), _ptr(n_accepted), _ptr(parent), _ptr(k_pool),
                                       _ptr(v_pool), _ptr(k_scale), _ptr(v_scale), _ptr(block_table),
                                       _ptr(ctx_lens), _ptr(new_ctx), _ptr(workspace), wsb, _stream(stream))
    if raise_on_error:
        _check(st, "verify_attn_promote_kv")
    return st


def verify_attn_read_flags(plan: Plan, workspace, stream=None) -> int:
    flags = ctypes.c_uint32()
    _check(load().verify_attn_read_flags(plan.handle, _ptr(workspace), _stream(stream), ctypes.byref(flags)),
           "verify_attn_read_flags")
    return flags.value
