"""ctypes front end of the fp64 verify-attention oracle (oracle.c).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  It shares no code with the HIP
library and never calls it.

The functions accept any object that carries the workload attributes
(num_seqs, B, H, KVH, D, num_pages, max_pages, q_dtype, kv_dtype, scale, q,
k_pool, v_pool, k_scale, v_scale, block_table, ctx_lens, parent) with the
layouts documented in oracle.h.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIB names another build of oracle.c (the sanitizer build of
# tests/run_sanitized.py), which is loaded as it is and never rebuilt.
_LIB_ENV = os.environ.get("ORACLE_LIB")
_LIB_PATH = _LIB_ENV or os.path.join(_HERE, "liboracle.so")
_lib = None

_DT = {"f32": 0, "f16": 1, "bf16": 2, "q8_0": 3}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (portable x86-64, -O2)."""
    if _LIB_ENV:
        if not os.path.exists(_LIB_ENV):
            raise RuntimeError(f"ORACLE_LIB={_LIB_ENV} does not exist")
        return _LIB_ENV
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lpthread", "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("num_seqs", "B", "H", "KVH", "D", "num_pages", "max_pages", "q_dtype", "kv_dtype")] + [
        ("scale", ctypes.c_double)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, dp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        sp = ctypes.POINTER(_Shape)
        lib.orc_attention.argtypes = [sp, vp, vp, vp, vp, vp, ip, ip, ip, ip, dp, dp, ctypes.c_int]
        lib.orc_attention_items.argtypes = [sp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ctypes.c_int32, ip, dp, dp,
                                            ctypes.c_int]
        lib.orc_split_partials.argtypes = [sp, vp, vp, vp, vp, vp, ip, ip, ip, ip, ctypes.c_int32, ip, dp, dp,
                                           dp, ctypes.c_int]
        lib.orc_merge.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, dp, dp, dp, dp, dp]
        lib.orc_f32_to_f16.argtypes = [ctypes.c_int64, vp, vp]
        lib.orc_decode_f16.argtypes = [ctypes.c_int64, vp, vp]
        lib.orc_decode_bf16.argtypes = [ctypes.c_int64, vp, vp]
        lib.orc_quantize_blocks.argtypes = [ctypes.c_int64, vp, vp, vp]
        lib.orc_append_kv.argtypes = [sp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, ip, ip]
        lib.orc_promote_kv.argtypes = [sp, ip, ip, ip, vp, vp, vp, vp, ip, ip, ip]
        for f in (lib.orc_attention, lib.orc_attention_items, lib.orc_split_partials, lib.orc_merge,
                  lib.orc_f32_to_f16, lib.orc_quantize_blocks, lib.orc_append_kv, lib.orc_promote_kv,
                  lib.orc_decode_f16, lib.orc_decode_bf16):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


class OracleError(ValueError):
    pass


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _prep(w):
    shape = _Shape(num_seqs=w.num_seqs, B=w.B, H=w.H, KVH=w.KVH, D=w.D, num_pages=w.num_pages,
                   max_pages=w.max_pages, q_dtype=_DT[w.q_dtype], kv_dtype=_DT[w.kv_dtype],
                   scale=float(np.float32(w.scale)))
    arrs = dict(
        q=np.ascontiguousarray(w.q), k=np.ascontiguousarray(w.k_pool), v=np.ascontiguousarray(w.v_pool),
        ks=None if w.k_scale is None else np.ascontiguousarray(w.k_scale).view(np.uint16),
        vs=None if w.v_scale is None else np.ascontiguousarray(w.v_scale).view(np.uint16),
        bt=np.ascontiguousarray(w.block_table, dtype=np.int32),
        ctx=np.ascontiguousarray(w.ctx_lens, dtype=np.int32),
        par=None if w.parent is None else np.ascontiguousarray(w.parent, dtype=np.int32),
        cu=None if getattr(w, "cu_rows", None) is None else np.ascontiguousarray(w.cu_rows, dtype=np.int32),
    )
    if w.q_dtype in ("f16", "bf16"):
        arrs["q"] = arrs["q"].view(np.uint16)
    return shape, arrs


def _common(a):
    return (_ptr(a["q"]), _ptr(a["k"]), _ptr(a["v"]), _ptr(a["ks"]), _ptr(a["vs"]), _ptr(a["bt"]),
            _ptr(a["ctx"]), _ptr(a["par"]), _ptr(a["cu"]))


def total_rows(w) -> int:
    """Packed query rows of a workload: num_seqs*B, or cu_rows[-1] when ragged."""
    cu = getattr(w, "cu_rows", None)
    return w.num_seqs * w.B if cu is None else int(cu[-1])


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def attention(w, nthreads: Optional[int] = None):
    """Definition evaluated in fp64 -> (out [rows, H, D], lse [rows, H])."""
    lib = _load()
    shape, a = _prep(w)
    out = np.zeros((total_rows(w), w.H, w.D), np.float64)
    lse = np.zeros((total_rows(w), w.H), np.float64)
    rc = lib.orc_attention(ctypes.byref(shape), *_common(a), _ptr(out), _ptr(lse),
                           nthreads or default_threads())
    if rc != 0:
        raise OracleError("oracle rejected the inputs (rc=%d)" % rc)
    return out, lse


def attention_items(w, items: Sequence[Sequence[int]], nthreads: Optional[int] = None):
    """Definition for chosen (seq, sequence-local row, head) triples -> (out [n, D], lse [n])."""
    lib = _load()
    shape, a = _prep(w)
    it = np.ascontiguousarray(np.asarray(items, np.int32).reshape(-1, 3))
    out = np.zeros((it.shape[0], w.D), np.float64)
    lse = np.zeros((it.shape[0],), np.float64)
    rc = lib.orc_attention_items(ctypes.byref(shape), *_common(a), it.shape[0], _ptr(it), _ptr(out), _ptr(lse),
                                 nthreads or default_threads())
    if rc != 0:
        raise OracleError("oracle rejected the inputs (rc=%d)" % rc)
    return out, lse


def split_partials(w, bounds: np.ndarray, nthreads: Optional[int] = None):
    """Split partials for a token partition bounds [nseq, S+1] -> (m, l, o)."""
    lib = _load()
    shape, a = _prep(w)
    b = np.ascontiguousarray(bounds, np.int32)
    S = b.shape[1] - 1
    nrows = total_rows(w) * w.H
    m = np.zeros((S, nrows), np.float64)
    l = np.zeros((S, nrows), np.float64)
    o = np.zeros((S, nrows, w.D), np.float64)
    rc = lib.orc_split_partials(ctypes.byref(shape), *_common(a), S, _ptr(b), _ptr(m), _ptr(l), _ptr(o),
                                nthreads or default_threads())
    if rc != 0:
        raise OracleError("oracle rejected the inputs (rc=%d)" % rc)
    return m, l, o


def merge(m: np.ndarray, l: np.ndarray, o: np.ndarray):
    """Log-sum-exp merge of split partials -> (out [nrows, D], lse [nrows])."""
    lib = _load()
    m = np.ascontiguousarray(m, np.float64)
    l = np.ascontiguousarray(l, np.float64)
    o = np.ascontiguousarray(o, np.float64)
    S, nrows = m.shape
    D = o.shape[-1]
    out = np.zeros((nrows, D), np.float64)
    lse = np.zeros((nrows,), np.float64)
    rc = lib.orc_merge(S, nrows, D, _ptr(m), _ptr(l), _ptr(o), _ptr(out), _ptr(lse))
    if rc != 0:
        raise OracleError("merge rejected the inputs (rc=%d)" % rc)
    return out, lse


def decode_f16(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> float64, by the oracle's decoder."""
    lib = _load()
    bits = np.ascontiguousarray(bits, np.uint16)
    out = np.zeros(bits.shape, np.float64)
    lib.orc_decode_f16(bits.size, _ptr(bits), _ptr(out))
    return out


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, by the oracle's decoder."""
    lib = _load()
    bits = np.ascontiguousarray(bits, np.uint16)
    out = np.zeros(bits.shape, np.float64)
    lib.orc_decode_bf16(bits.size, _ptr(bits), _ptr(out))
    return out


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """fp32 values -> IEEE binary16 bit patterns (uint16), round to nearest even."""
    lib = _load()
    x = np.ascontiguousarray(x, np.float32)
    out = np.zeros(x.shape, np.uint16)
    lib.orc_f32_to_f16(x.size, _ptr(x), _ptr(out))
    return out


def quantize_blocks(x: np.ndarray):
    """x [..., 32k] fp32 -> (q int8 same shape, d fp16 bits [..., k]) per 32-entry block."""
    lib = _load()
    x = np.ascontiguousarray(x, np.float32)
    assert x.shape[-1] % 32 == 0
    q = np.zeros(x.shape, np.int8)
    d = np.zeros(x.shape[:-1] + (x.shape[-1] // 32,), np.uint16)
    lib.orc_quantize_blocks(x.size // 32, _ptr(x), _ptr(q), _ptr(d))
    return q, d


def append_kv(w, k_new: np.ndarray, v_new: np.ndarray, new_dtype: str):
    """Write the drafted rows' K/V (k_new, v_new [nseq*B, KVH, D]; new_dtype
    "f32" | "f16" | "bf16", 16-bit inputs as raw bits) into copies of w's pools.
    Returns (k_pool, v_pool, k_scale, v_scale) with scales as fp16 arrays (or None)."""
    lib = _load()
    if getattr(w, "cu_rows", None) is not None:
        raise OracleError("KV append / promotion take B rows per sequence, not ragged rows")
    shape, a = _prep(w)
    k = a["k"].copy()
    v = a["v"].copy()
    ks = None if a["ks"] is None else a["ks"].copy()
    vs = None if a["vs"] is None else a["vs"].copy()
    kn = np.ascontiguousarray(k_new)
    vn = np.ascontiguousarray(v_new)
    if new_dtype in ("f16", "bf16"):
        kn, vn = kn.view(np.uint16), vn.view(np.uint16)
    rc = lib.orc_append_kv(ctypes.byref(shape), _DT[new_dtype], _ptr(kn), _ptr(vn), _ptr(k), _ptr(v), _ptr(ks),
                           _ptr(vs), _ptr(a["bt"]), _ptr(a["ctx"]))
    if rc != 0:
        raise OracleError("oracle rejected the append (rc=%d)" % rc)
    return (k.view(w.k_pool.dtype), v.view(w.v_pool.dtype), None if ks is None else ks.view(np.float16),
            None if vs is None else vs.view(np.float16))


def promote_kv(w, accepted: np.ndarray, n_accepted: np.ndarray):
    """Accepted-path promotion on copies of w's pools.  accepted [nseq, B]
    (root-first drafted-row indices, entries past n_accepted ignored),
    n_accepted [nseq].  Returns (k_pool, v_pool, k_scale, v_scale, new_ctx)."""
    lib = _load()
    if getattr(w, "cu_rows", None) is not None:
        raise OracleError("KV append / promotion take B rows per sequence, not ragged rows")
    shape, a = _prep(w)
    k = a["k"].copy()
    v = a["v"].copy()
    ks = None if a["ks"] is None else a["ks"].copy()
    vs = None if a["vs"] is None else a["vs"].copy()
    acc = np.ascontiguousarray(accepted, np.int32).reshape(w.num_seqs, w.B)
    n = np.ascontiguousarray(n_accepted, np.int32).reshape(w.num_seqs)
    new_ctx = np.zeros(w.num_seqs, np.int32)
    rc = lib.orc_promote_kv(ctypes.byref(shape), _ptr(acc), _ptr(n), _ptr(a["par"]), _ptr(k), _ptr(v), _ptr(ks),
                            _ptr(vs), _ptr(a["bt"]), _ptr(a["ctx"]), _ptr(new_ctx))
    if rc != 0:
        raise OracleError("oracle rejected the promotion (rc=%d)" % rc)
    return (k.view(w.k_pool.dtype), v.view(w.v_pool.dtype), None if ks is None else ks.view(np.float16),
            None if vs is None else vs.view(np.float16), new_ctx)
