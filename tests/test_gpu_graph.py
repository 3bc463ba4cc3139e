"""Graph capture of the verify step (KV append + verify attention).

The grid of every launch is fixed by the plan, ctx / block table / parent are
read on the device, and nothing in verify_attn_append_kv or verify_attn_run
allocates, synchronises or memsets, so one captured graph serves any live
context up to max_ctx (the retained fixed-grid route of the page
"perf(gfx1100): speed up long-context DFlash verify 13.4% with FA2 split-KV
and retain HipGraph/Redline PM4", Summary and Default and admission policy).
Each replay runs after eager work on the same stream and is checked against
the oracle and against the same call made eagerly."""

import copy

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verify_kv_amd as va
import synthetic as S
from speculative_decoding_verify_kv_amd import device as vdev

from .gpu_util import check_parity, ensure_lib, errors, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _to_dev_rows(a):
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def _copy_rows(dst, a):
    a = np.ascontiguousarray(a)
    dst.copy_(torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a))


@pytest.mark.parametrize("tree", [False, True])
def test_graph_replay_follows_live_context(tree):
    say(f"[case] graph replay tree={tree}")
    max_ctx = 6000
    B = 10 if tree else 16
    par = S.tree_parent(2, 8, np.random.default_rng(5)) if tree else None
    w = S.make_workload("graph", ctx_lens=[max_ctx], B=B, H=24, KVH=4, D=256, q_dtype="bf16", kv_dtype="q8_0",
                        seed=61, permute=True, spare_pages=4, poison=True, parent=par)
    dev = vdev.to_device(w)
    base_pools = {k: dev[k].clone() for k in ("k_pool", "v_pool", "k_scale", "v_scale")}
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f32", max_ctx=max_ctx), 0, 0)
    ws = vdev.workspace(plan)
    out, lse = vdev.empty_out(w, "f32")
    k_new, v_new = S.new_kv_rows(w, "bf16", seed=1)
    kn, vn = _to_dev_rows(k_new), _to_dev_rows(v_new)

    def step():
        va.verify_attn_append_kv(plan, kn, vn, "bf16", dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                                 dev["block_table"], dev["ctx_lens"], ws, stream=torch.cuda.current_stream())
        va.verify_attn_run(plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                           dev["block_table"], dev["ctx_lens"], dev["parent"], 0, out, lse, ws,
                           stream=torch.cuda.current_stream())

    # warm up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(77)
    for rep, ctx in enumerate([max_ctx, 3001, 1033, 257, max_ctx - 5]):
        # live inputs for this replay: context, new rows, Q; pools reset to the base
        for k in base_pools:
            dev[k].copy_(base_pools[k])
        wq = copy.deepcopy(w)
        wq.ctx_lens = np.array([ctx], np.int32)
        wq.q = S.bf16_bits_from_f32(rng.standard_normal(w.q.shape, dtype=np.float32))
        k_new, v_new = S.new_kv_rows(w, "bf16", seed=100 + rep)
        dev["ctx_lens"].copy_(torch.from_numpy(wq.ctx_lens))
        _copy_rows(dev["q"].view(torch.int16), wq.q)
        _copy_rows(kn, k_new)
        _copy_rows(vn, v_new)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        got_lse = lse.cpu().double().numpy()
        assert va.verify_attn_read_flags(plan, ws) == 0
        # reference: the oracle on the oracle-appended pools for this context
        rk, rv, rks, rvs = oracle.append_kv(wq, k_new, v_new, "bf16")
        wa = copy.copy(wq)
        wa.k_pool, wa.v_pool, wa.k_scale, wa.v_scale = rk, rv, rks, rvs
        ref, ref_lse = oracle.attention(wa)
        check_parity(got, ref, "f32", f"replay {rep} ctx={ctx}")
        assert np.abs(got_lse - ref_lse).max() <= 2e-3
        # the same step made eagerly gives the same bits
        for k in base_pools:
            dev[k].copy_(base_pools[k])
        step()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().double().numpy(), got)


def test_graph_replay_time_is_close_to_eager():
    """Report replay vs eager time for the headline shape (no bound asserted
    beyond a sanity factor: replay must not be slower than 1.5x eager)."""
    say("[case] graph timing")
    w = S.q8_long(ctx=32768)
    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f16"), 0, 0)
    ws = vdev.workspace(plan)
    out, lse = vdev.empty_out(w, "f16")

    def step():
        va.verify_attn_run(plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                           dev["block_table"], dev["ctx_lens"], None, 0, out, lse, ws,
                           stream=torch.cuda.current_stream())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    eager_ref = out.clone()

    def timed(fn, n=20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    t_eager = timed(step)
    t_graph = timed(g.replay)
    say(f"  eager {t_eager:.1f} us/call, graph replay {t_graph:.1f} us/call")
    assert torch.equal(out, eager_ref)
    assert t_graph <= 1.5 * t_eager


def test_graph_replay_ragged_follows_live_rows():
    """A captured ragged call (the work-list pass, the partial and the merge
    kernels) replayed with the row counts (cu_rows), contexts and Q changed on
    the device between replays: the work list is rebuilt on the device each
    time, so every replay matches the oracle for its own batch and, bit for
    bit, the same call made eagerly (capture-friendly fixed grids: page
    "perf(gfx1100): speed up long-context DFlash verify 13.4% with FA2
    split-KV and retain HipGraph/Redline PM4", Summary)."""
    say("[case] ragged graph replay")
    ctx_cap = [800, 3200, 1600, 5000]
    w = S.make_workload("graph_ragged", ctx_lens=ctx_cap, rows=[24, 1, 6, 3], H=8, KVH=2, D=128, q_dtype="bf16",
                        kv_dtype="q8_0", seed=63, permute=True, spare_pages=3, poison=True)
    cap = w.total_rows
    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f32"), 0, 0)
    ws = vdev.workspace(plan)
    q_buf = torch.zeros((cap, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    q_buf.view(torch.int16).copy_(torch.from_numpy(np.ascontiguousarray(w.q).view(np.int16)))
    out = torch.full((cap, w.H, w.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((cap, w.H), float("nan"), dtype=torch.float32, device="cuda")

    def step():
        va.verify_attn_run_ragged(plan, q_buf, dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                                  dev["block_table"], dev["ctx_lens"], dev["cu_rows"], None, 0, out, lse, ws,
                                  stream=torch.cuda.current_stream())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(79)
    cases = [([24, 1, 6, 3], [800, 3200, 1600, 5000]),
             ([0, 1, 24, 5], [700, 3100, 1500, 4000]),
             ([10, 10, 10, 4], [300, 2000, 1600, 4900]),
             ([1, 0, 0, 1], [33, 1, 1, 17])]
    for rep, (rows, ctx) in enumerate(cases):
        cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
        n = int(cu[-1])
        assert n <= cap and max(rows) <= w.B and all(c <= m for c, m in zip(ctx, ctx_cap))
        qn = S.bf16_bits_from_f32(rng.standard_normal((n, w.H, w.D), dtype=np.float32))
        dev["cu_rows"].copy_(torch.from_numpy(cu))
        dev["ctx_lens"].copy_(torch.from_numpy(np.asarray(ctx, np.int32)))
        q_buf[:n].view(torch.int16).copy_(torch.from_numpy(np.ascontiguousarray(qn).view(np.int16)))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out[:n].cpu().double().numpy()
        got_lse = lse[:n].cpu().double().numpy()
        assert va.verify_attn_read_flags(plan, ws) == 0
        wq = copy.copy(w)
        wq.cu_rows, wq.ctx_lens, wq.q = cu, np.asarray(ctx, np.int32), qn
        ref, ref_lse = oracle.attention(wq)
        check_parity(got, ref, "f32", f"ragged replay {rep} rows={rows} ctx={ctx}")
        assert np.abs(got_lse - ref_lse).max() <= 2e-3
        step()
        torch.cuda.synchronize()
        assert np.array_equal(out[:n].cpu().double().numpy(), got)
        assert np.array_equal(lse[:n].cpu().double().numpy(), got_lse)


def test_graph_replay_noalloc_entry():
    """The entry point for callers that cannot allocate, captured once and
    replayed with the context changed on the device: each replay equals, bit
    for bit, verify_attn_run on the same inputs."""
    say("[case] no-allocation entry graph replay")
    max_ctx = 9000
    w = S.make_workload("graph_noalloc", ctx_lens=[max_ctx, 4000], B=16, H=24, KVH=4, D=256, q_dtype="bf16",
                        kv_dtype="q8_0", seed=65, permute=True, spare_pages=2)
    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f16", max_ctx=max_ctx), 0, 0)
    ws = vdev.workspace(plan)
    out, lse = vdev.empty_out(w, "f16")
    out_r, lse_r = vdev.empty_out(w, "f16")
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"], dev["block_table"],
            dev["ctx_lens"], None, 0)

    def step():
        va.verify_attn_run_noalloc(*args, out, lse, flags, stream=torch.cuda.current_stream())

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep, ctx in enumerate([[max_ctx, 4000], [5000, 3999], [17, 8191], [max_ctx, 16]]):
        dev["ctx_lens"].copy_(torch.from_numpy(np.asarray(ctx, np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        va.verify_attn_run(*args, out_r, lse_r, ws)
        torch.cuda.synchronize()
        assert int(flags.item()) == 0 and va.verify_attn_read_flags(plan, ws) == 0
        say(f"  replay {rep} ctx={ctx}")
        assert torch.equal(out, out_r) and torch.equal(lse, lse_r)
