"""One workspace carried through calls on different inputs, plans and split
counts, as a serving loop reuses its buffer from step to step.

The workspace starts with every byte 0xFF (NaN partials, -1 counters and
list entries) apart from its zeroed flag header.  Each call must equal, bit
for bit, the same call on a fresh zeroed workspace, and the first call on
each input must meet the oracle's gate: no call may read what an earlier
call left behind (partials of more splits, rows of a longer batch, the
previous work list).  The workspace is caller-owned and part of admission
(page "perf(gfx1100): speed up long-context DFlash verify 13.4% with FA2
split-KV and retain HipGraph/Redline PM4", Maintainer-review follow-up).
"""

import numpy as np
import pytest

import oracle
import synthetic as S
import speculative_decoding_verify_kv_amd as va
from speculative_decoding_verify_kv_amd import device as vdev

from .gpu_util import check_parity, ensure_lib, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _dirty_workspace(nbytes):
    import torch

    ws = torch.full((max(nbytes, 256),), 0xFF, dtype=torch.uint8, device="cuda")
    ws[:256].zero_()
    return ws


def _outputs(w, out_dtype, ragged):
    import torch

    rows = w.total_rows if ragged else w.num_seqs * w.B
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[out_dtype]
    out = torch.full((rows, w.H, w.D), float("nan"), dtype=dt, device="cuda")
    lse = torch.full((rows, w.H), float("nan"), dtype=torch.float32, device="cuda")
    return out, lse


def _launch(plan, dev, ws, num_splits, out, lse, ragged, stream=None):
    args = (dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"], dev["block_table"],
            dev["ctx_lens"])
    if ragged:
        va.verify_attn_run_ragged(plan, *args, dev["cu_rows"], dev["parent"], num_splits, out, lse, ws,
                                  stream=stream)
    else:
        va.verify_attn_run(plan, *args, dev["parent"], num_splits, out, lse, ws, stream=stream)


def _call(w, plan, dev, ws, num_splits, out_dtype, ragged):
    import torch

    out, lse = _outputs(w, out_dtype, ragged)
    _launch(plan, dev, ws, num_splits, out, lse, ragged)
    torch.cuda.synchronize()
    flags = va.verify_attn_read_flags(plan, ws)
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy(), flags


def _run_sequence(items, calls, out_dtype, ragged):
    """items: name -> workload; calls: [(name, num_splits)] in order, all on one workspace."""
    plans = {k: va.verify_attn_plan(vdev.problem_for(w, out_dtype=out_dtype), 0, 0) for k, w in items.items()}
    devs = {k: vdev.to_device(w) for k, w in items.items()}
    ws = _dirty_workspace(max(p.workspace_bytes for p in plans.values()))
    refs, seen = {}, set()
    for name, s in calls:
        w, plan = items[name], plans[name]
        S_eff = s or plan.info().num_splits
        say(f"[case] {'ragged' if ragged else 'uniform'} {name} S={S_eff} on the shared workspace")
        got, lse, flags = _call(w, plan, devs[name], ws, s, out_dtype, ragged)
        assert flags == 0
        fresh_ws = vdev.workspace(plan)
        fresh, flse, fflags = _call(w, plan, devs[name], fresh_ws, s, out_dtype, ragged)
        assert fflags == 0
        assert np.array_equal(got, fresh), f"{name} S={S_eff}: shared workspace differs from a fresh one"
        assert np.array_equal(lse, flse)
        if name not in refs:
            refs[name] = oracle.attention(w)
        if (name, S_eff) not in seen:
            seen.add((name, S_eff))
            check_parity(got, refs[name][0], out_dtype, f"{name} S={S_eff}")


def test_uniform_calls_share_one_workspace():
    """A one-sequence 8-bit call and a two-sequence call with other contexts,
    row count and heads, alternating with split counts from the plan, 5 and 1
    (direct, no partials), then the first again."""
    items = {
        "a": S.make_workload("ws_a", ctx_lens=[3000], B=16, H=24, KVH=4, D=256, q_dtype="bf16",
                             kv_dtype="q8_0", seed=71, permute=True, spare_pages=3, poison=True),
        "b": S.make_workload("ws_b", ctx_lens=[1900, 2600], B=8, H=16, KVH=2, D=128, q_dtype="f16",
                             kv_dtype="q8_0", seed=72, permute=True, spare_pages=2, poison=True),
    }
    _run_sequence(items, [("a", 0), ("b", 0), ("a", 5), ("b", 1), ("a", 0), ("b", 3)], "f32", ragged=False)


def test_ragged_calls_share_one_workspace():
    """The mixed lowering (prefill, decoders, tree) and a smaller ragged batch
    with fewer sequences, alternating, with the plan's split count and a
    small one: the second call's work list is shorter than the first's."""
    small = S.mixed_lowering(seed=9, prefill=(40,), prefill_ctx=(700,), direct_ctx=(3000,), tree_ctx=5000,
                             n_direct=1, n_tree=5)
    items = {"mixed": S.mixed_lowering(), "small": small}
    _run_sequence(items, [("mixed", 0), ("small", 0), ("mixed", 4), ("small", 2), ("mixed", 0)], "f16",
                  ragged=True)


def test_concurrent_streams_distinct_workspaces():
    """Three calls (two uniform plans and a ragged one) issued round-robin on
    three streams, 6 times each with no synchronisation in between, each call
    with its own workspace: the calls may overlap on the device, and each
    stream's last result equals the same call run alone, bit for bit
    (concurrent calls need distinct workspaces, nothing else)."""
    import torch

    items = [
        (S.make_workload("cs_a", ctx_lens=[6000], B=16, H=24, KVH=4, D=256, q_dtype="bf16", kv_dtype="q8_0",
                         seed=81, permute=True), False),
        (S.make_workload("cs_b", ctx_lens=[2500, 900, 4100], B=4, H=8, KVH=1, D=64, q_dtype="f32",
                         kv_dtype="f16", seed=82, permute=True), False),
        (S.mixed_lowering(seed=83, prefill=(24,), prefill_ctx=(800,), direct_ctx=(5000, 1500), tree_ctx=3000,
                          n_direct=2, n_tree=4), True),
    ]
    runs = []
    for w, ragged in items:
        plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f32"), 0, 0)
        dev = vdev.to_device(w)
        alone = _call(w, plan, dev, vdev.workspace(plan), 0, "f32", ragged)
        assert alone[2] == 0
        out, lse = _outputs(w, "f32", ragged)
        runs.append((w, ragged, plan, dev, vdev.workspace(plan), out, lse, alone, torch.cuda.Stream()))
    torch.cuda.synchronize()
    say(f"[case] {len(runs)} streams x 6 calls, no sync in between")
    for _ in range(6):
        for w, ragged, plan, dev, ws, out, lse, alone, st in runs:
            _launch(plan, dev, ws, 0, out, lse, ragged, stream=st)
    torch.cuda.synchronize()
    for w, ragged, plan, dev, ws, out, lse, alone, st in runs:
        assert va.verify_attn_read_flags(plan, ws) == 0
        assert np.array_equal(out.float().cpu().double().numpy(), alone[0]), w.name
        assert np.array_equal(lse.cpu().double().numpy(), alone[1]), w.name
