"""Move host arrays to torch device tensors and describe them to the C ABI.

Marshalling only (no attention arithmetic): torch provides device memory and
streams; the kernels in libverify_attn.so do the work.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from ._binding import VaProblem, make_problem


def _torch():
    import torch

    return torch


def to_device(w, device="cuda") -> Dict[str, object]:
    """Device copies of a workload's arrays (layouts unchanged)."""
    torch = _torch()

    def t(a: Optional[np.ndarray]):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if not a.flags.writeable:
            a = a.copy()
        if a.dtype == np.uint16:  # bf16 bits
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(a).to(device)

    return dict(
        q=t(w.q), k_pool=t(w.k_pool), v_pool=t(w.v_pool), k_scale=t(w.k_scale), v_scale=t(w.v_scale),
        block_table=t(np.asarray(w.block_table, np.int32)), ctx_lens=t(np.asarray(w.ctx_lens, np.int32)),
        parent=None if w.parent is None else t(np.asarray(w.parent, np.int32)),
        cu_rows=None if getattr(w, "cu_rows", None) is None else t(np.asarray(w.cu_rows, np.int32)),
    )


def _rows(w) -> int:
    cu = getattr(w, "cu_rows", None)
    return w.num_seqs * w.B if cu is None else int(cu[-1])


def problem_for(w, *, out_dtype: Optional[str] = None, max_ctx: Optional[int] = None,
                scale: Optional[float] = None, max_total_rows: Optional[int] = None) -> VaProblem:
    """Problem of a workload; a ragged one (cu_rows) gets max_total_rows (default: its row count)."""
    if max_total_rows is None:
        max_total_rows = 0 if getattr(w, "cu_rows", None) is None else max(_rows(w), 1)
    return make_problem(
        num_seqs=w.num_seqs, rows_per_seq=w.B, num_q_heads=w.H, num_kv_heads=w.KVH, head_dim=w.D,
        num_pages=w.num_pages, max_pages_per_seq=w.max_pages,
        max_ctx=int(max_ctx if max_ctx is not None else w.max_ctx),
        q_dtype=w.q_dtype, kv_dtype=w.kv_dtype, out_dtype=out_dtype or w.out_dtype,
        scale=float(w.scale if scale is None else scale), has_parent=w.parent is not None,
        max_total_rows=max_total_rows)


def empty_out(w, out_dtype: str, device="cuda"):
    torch = _torch()
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[out_dtype]
    out = torch.empty((max(_rows(w), 1), w.H, w.D), dtype=dt, device=device)
    lse = torch.empty((max(_rows(w), 1), w.H), dtype=torch.float32, device=device)
    return out, lse


def workspace(plan, device="cuda"):
    """A zeroed workspace of the plan's size (flag word cleared)."""
    torch = _torch()
    return torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=device)
