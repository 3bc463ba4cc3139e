"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
compare with the fp64 oracle."""

from __future__ import annotations

import sys

import numpy as np

import oracle
import speculative_decoding_verify_kv_amd as va
from speculative_decoding_verify_kv_amd import device as vdev

REL_L2 = 1e-3
MAX_ABS = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ensure_lib():
    import os

    if not os.path.exists(va.LIB_PATH):
        raise RuntimeError("libverify_attn.so is not built")
    va.load()


def run_gpu(w, num_splits=0, out_dtype="f16", dev=None, plan_splits=None, entry="run", max_ctx=None):
    """Run verify attention on the GPU; returns (out fp64, lse fp64, flags, plan info)."""
    import torch

    dev = dev if dev is not None else vdev.to_device(w)
    prob = vdev.problem_for(w, out_dtype=out_dtype, max_ctx=max_ctx)
    plan = va.verify_attn_plan(prob, num_splits if plan_splits is None else plan_splits, 0)
    ws = vdev.workspace(plan)
    out, lse = vdev.empty_out(w, out_dtype)
    args = (plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"], dev["block_table"],
            dev["ctx_lens"], dev["parent"], num_splits, out, lse, ws)
    if entry == "run":
        va.verify_attn_run(*args)
    else:
        va.verify_attn_run_partial(*args)
        S = num_splits or plan.info().num_splits
        if S > 1:
            va.verify_attn_run_merge(plan, num_splits, out, lse, ws)
    torch.cuda.synchronize()
    flags = va.verify_attn_read_flags(plan, ws)
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy(), flags, plan.info()


def errors(got, ref):
    d = got - ref
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    return rel, float(np.abs(d).max())


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (for normal values)."""
    ax = np.abs(x).astype(np.float64)
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_parity(got, ref, out_dtype, what=""):
    rel, mx = errors(got, ref)
    say(f"  parity {what}: rel_l2={rel:.3e} max_abs={mx:.3e} ({out_dtype})")
    assert np.all(np.isfinite(got)), what
    assert mx <= MAX_ABS, (what, mx)
    if out_dtype == "bf16":
        # bf16 rounding alone is ~1.7e-3 relative L2 on these values, so the
        # relative gate cannot apply as such.  Gate: each element within one
        # bf16 ulp of the fp64 oracle, plus an absolute allowance of 1e-3 of the
        # tensor's rms for the fp32 pipeline error (it dominates for elements
        # near zero, whose ulp is tiny); relative L2 within 4e-3.
        rms = float(np.sqrt(np.mean(ref * ref)))
        assert np.all(np.abs(got - ref) <= bf16_ulp(ref) + 1e-3 * rms), what
        assert rel <= 4e-3, (what, rel)
    else:
        assert rel <= REL_L2, (what, rel)
    return rel, mx


class OracleCache:
    def __init__(self):
        self.c = {}

    def get(self, w):
        key = id(w)
        if key not in self.c:
            self.c[key] = oracle.attention(w)
        return self.c[key]
