"""verify_attn_run_noalloc (the entry point for callers that cannot allocate:
its split partials live in the library's own per-GPU device array) against
verify_attn_run on the same inputs and plan: two calls in a row, the second
with a smaller input, outputs and lse bit for bit equal, and both at the
oracle's gate.  Also: device-side metadata errors reach the caller's flag
word."""

import copy

import numpy as np
import pytest

import oracle
import speculative_decoding_verify_kv_amd as va
import synthetic as S
from speculative_decoding_verify_kv_amd import device as vdev

from .gpu_util import check_parity, ensure_lib, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def both(w, num_splits):
    """(run out, run lse, noalloc out, noalloc lse, noalloc flags, plan info)."""
    import torch

    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f16"), num_splits, 0)
    ws = vdev.workspace(plan)
    out_a, lse_a = vdev.empty_out(w, "f16")
    out_b, lse_b = vdev.empty_out(w, "f16")
    out_b.fill_(float("nan"))
    lse_b.fill_(float("nan"))
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"], dev["block_table"],
            dev["ctx_lens"], dev["parent"], 0)
    va.verify_attn_run(*args, out_a, lse_a, ws)
    va.verify_attn_run_noalloc(*args, out_b, lse_b, flags)
    torch.cuda.synchronize()
    assert va.verify_attn_read_flags(plan, ws) == 0
    f = lambda t: t.float().cpu().double().numpy()
    return f(out_a), f(lse_a), f(out_b), f(lse_b), int(flags.item()), plan.info()


def test_noalloc_matches_run_twice_then_smaller():
    big = S.q8_long(ctx=8192)
    small = S.tree_mixed(ctx=2000)
    for w, sp in ((big, 0), (small, 4)):
        say(f"[case] noalloc {w.name} S={sp or 'plan'}")
        oa, la, ob, lb, fl, info = both(w, sp)
        assert fl == 0
        assert info.num_splits > 1
        assert np.array_equal(oa, ob), w.name
        assert np.array_equal(la, lb), w.name
        ref, lref = oracle.attention(w)
        check_parity(ob, ref, "f16", f"noalloc {w.name} S={info.num_splits}")


def test_noalloc_direct_and_flags():
    import torch

    w = S.tree_mixed(ctx=700)
    say("[case] noalloc direct path and a bad page id")
    oa, la, ob, lb, fl, info = both(w, 1)
    assert fl == 0 and np.array_equal(oa, ob) and np.array_equal(la, lb)
    bad = copy.deepcopy(w)
    bad.block_table = bad.block_table.copy()
    bad.block_table[0, 2] = w.num_pages + 3
    dev = vdev.to_device(bad)
    plan = va.verify_attn_plan(vdev.problem_for(bad, out_dtype="f16"), 0, 0)
    out, lse = vdev.empty_out(bad, "f16")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    va.verify_attn_run_noalloc(plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                               dev["block_table"], dev["ctx_lens"], dev["parent"], 0, out, lse, flags)
    torch.cuda.synchronize()
    assert int(flags.item()) & va.VA_FLAG_BAD_PAGE
    assert np.all(np.isnan(out.float().cpu().numpy()))
