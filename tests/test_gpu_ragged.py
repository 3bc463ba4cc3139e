"""GPU parity of ragged rows (verify_attn_run_ragged): paged prefill segments,
direct rows and a draft tree in one call, against the fp64 oracle.

Source: the page "perf(qwen35): retain speculation during paged prefill",
Mechanism (one step lowers [prefill segments][direct rows][tree rows]) and
Correctness failure found during qualification (rows of one sequence changed
when a tree suffix joined the launch at the 1,024-token boundary).  Every
call goes through the C ABI; expected values come from the oracle only.
"""

import copy

import numpy as np
import pytest

import oracle
import synthetic as S
import speculative_decoding_verify_kv_amd as va
from speculative_decoding_verify_kv_amd import device as vdev

from .gpu_util import check_parity, ensure_lib, errors, say
from .test_oracle_ragged import tiny_ragged

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def run_ragged(w, num_splits=0, out_dtype="f16", *, plan=None, dev=None, cu_rows=None, q=None, parent=None):
    """verify_attn_run_ragged on w (cu_rows / q / parent override the workload's);
    returns (out fp64 [rows], lse fp64 [rows], flags, plan)."""
    import torch

    dev = dev if dev is not None else vdev.to_device(w)
    if plan is None:
        plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype=out_dtype), num_splits, 0)
    cap = plan.problem.max_total_rows
    ws = vdev.workspace(plan)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[out_dtype]
    out = torch.full((cap, w.H, w.D), float("nan"), dtype=dt, device="cuda")
    lse = torch.full((cap, w.H), float("nan"), dtype=torch.float32, device="cuda")
    cu = dev["cu_rows"] if cu_rows is None else torch.from_numpy(np.asarray(cu_rows, np.int32)).cuda()
    qq = dev["q"] if q is None else q
    par = dev["parent"] if parent is None else parent
    va.verify_attn_run_ragged(plan, qq, dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                              dev["block_table"], dev["ctx_lens"], cu, par, num_splits, out, lse, ws)
    torch.cuda.synchronize()
    flags = va.verify_attn_read_flags(plan, ws)
    return out.float().cpu().double().numpy(), lse.cpu().double().numpy(), flags, plan


_cache = {}


def mixed():
    if "mixed" not in _cache:
        w = S.mixed_lowering()
        say(f"[oracle] {w.name} rows={w.cu_rows.tolist()} ctx={w.ctx_lens.tolist()}")
        o, l = oracle.attention(w)
        _cache["mixed"] = (w, o, l)
    return _cache["mixed"]


@pytest.mark.parametrize("S_", [1, 8, 0])
def test_mixed_lowering(S_):
    w, ref, lref = mixed()
    say(f"[case] mixed lowering S={S_}")
    got, lse, flags, plan = run_ragged(w, S_, "f16")
    n = w.total_rows
    assert flags == 0
    check_parity(got[:n], ref, "f16", f"mixed S={plan.info().num_splits if S_ == 0 else S_}")
    assert np.abs(lse[:n] - lref).max() <= 2e-3
    assert np.all(np.isnan(got[n:]))  # nothing past the packed rows is written


@pytest.mark.parametrize("kv,S_", [("f16", 1), ("f16", 3), ("q8_0", 1), ("q8_0", 4)])
def test_tiny_ragged(kv, S_):
    # an empty sequence, one direct row, a 70-row chain (past the 64-row
    # ancestry window) and a tree; D=64, 4 query heads over 2 KV heads
    w = tiny_ragged(kv)
    say(f"[case] tiny ragged kv={kv} S={S_} rows={np.diff(w.cu_rows).tolist()}")
    ref, lref = oracle.attention(w)
    got, lse, flags, _ = run_ragged(w, S_, "f32")
    assert flags == 0
    check_parity(got[:w.total_rows], ref, "f32", f"tiny ragged {kv} S={S_}")
    assert np.abs(lse[:w.total_rows] - lref).max() <= 2e-3


@pytest.mark.parametrize("S_", [1, 8, 0])
def test_long_prefill_segment(S_):
    # 300 prefill rows ending at ctx 1500 plus one direct row: many row groups,
    # each cut at its last visible key
    if "prefill" not in _cache:
        w = S.make_workload("prefill300", ctx_lens=[1500, 2100], rows=[300, 1], H=24, KVH=4, D=256,
                            q_dtype="bf16", kv_dtype="q8_0", seed=51, permute=True, spare_pages=7, poison=True)
        say("[oracle] prefill300")
        _cache["prefill"] = (w, oracle.attention(w)[0])
    w, ref = _cache["prefill"]
    say(f"[case] long prefill S={S_}")
    got, _, flags, plan = run_ragged(w, S_, "f16")
    assert flags == 0
    say(f"  plan: S={plan.info().num_splits} row_groups={plan.info().row_groups}")
    check_parity(got[:w.total_rows], ref, "f16", f"prefill300 S={S_}")


@pytest.mark.parametrize("S_,ctxs", [(1, (4096, 4112, 5000, 6000)), (8, (4096, 4112, 5000, 6000)),
                                     (16, (8192, 8200, 12000, 16000))])
def test_uniform_rows_through_ragged_entry_bitwise(S_, ctxs):
    # B rows per sequence written as cu_rows = [0, B, 2B, ...]: the same plan
    # shape and split count must give the same bits as verify_attn_run.  The
    # contexts are long enough (>= S splits of 32 pages) that the ragged rule
    # (a sequence's splits hold at least 32 pages) cuts the same splits as
    # the uniform one; shorter sequences take fewer, longer splits there.
    # At S = 8 the ragged merge takes each row with one wave (at most 8
    # splits), at S = 16 with a workgroup, as the uniform merge always does.
    import torch

    w = S.paged_ragged(ctxs=ctxs)
    wr = copy.deepcopy(w)
    wr.cu_rows = np.arange(0, w.num_seqs * w.B + 1, w.B, dtype=np.int32)
    say(f"[case] uniform via ragged S={S_}")
    dev = vdev.to_device(wr)
    plan_u = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f32"), S_, 0)
    ws = vdev.workspace(plan_u)
    out_u, lse_u = vdev.empty_out(w, "f32")
    va.verify_attn_run(plan_u, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                       dev["block_table"], dev["ctx_lens"], None, S_, out_u, lse_u, ws)
    torch.cuda.synchronize()
    got, lse, flags, plan_r = run_ragged(wr, S_, "f32", dev=dev)
    assert plan_r.info().rows_per_group == plan_u.info().rows_per_group
    assert flags == 0
    np.testing.assert_array_equal(got, out_u.double().cpu().numpy())
    np.testing.assert_array_equal(lse, lse_u.double().cpu().numpy())


@pytest.mark.parametrize("S_", [8, 0])
def test_rows_joining_do_not_change_other_rows_bitwise(S_):
    """The tree sequence joining the call, or the prefill segments leaving it,
    leaves every other sequence's rows bit for bit unchanged (one plan)."""
    import torch

    w, ref, _ = mixed()
    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f16"), S_, 0)
    full, _, flags, _ = run_ragged(w, S_, "f16", plan=plan, dev=dev)
    assert flags == 0
    cu = w.cu_rows
    # 1) the tree sequence with no rows
    no_tree = cu.copy()
    no_tree[-1] = no_tree[-2]
    a, _, flags, _ = run_ragged(w, S_, "f16", plan=plan, dev=dev, cu_rows=no_tree)
    assert flags == 0
    np.testing.assert_array_equal(a[:cu[-2]], full[:cu[-2]])
    # 2) the prefill segments with no rows: the direct and tree rows move to the
    #    front of the packed layout and keep their bits
    keep = cu[2]
    cu2 = np.concatenate([[0, 0, 0], cu[3:] - keep]).astype(np.int32)
    q2 = dev["q"][keep:].contiguous()
    par2 = dev["parent"][keep:].contiguous()
    b, _, flags, _ = run_ragged(w, S_, "f16", plan=plan, dev=dev, cu_rows=cu2, q=q2, parent=par2)
    assert flags == 0
    np.testing.assert_array_equal(b[:cu2[-1]], full[keep:cu[-1]])
    del torch


def test_bad_rows_and_long_non_chain_flagged():
    w, ref, _ = mixed()
    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f16"), 8, 0)
    cu = w.cu_rows
    # the last sequence claims rows past the packed capacity: flagged, nothing
    # of it written, the others intact
    bad = cu.copy()
    bad[-1] = cu[-1] + 5
    say("[case] cu_rows past capacity")
    got, _, flags, _ = run_ragged(w, 8, "f16", plan=plan, dev=dev, cu_rows=bad)
    assert flags & va.VA_FLAG_BAD_ROWS
    check_parity(got[:cu[-2]], ref[:cu[-2]], "f16", "others beside a bad cu_rows entry")
    # a decreasing entry
    bad = cu.copy()
    bad[3] = cu[2] - 1
    got, _, flags, _ = run_ragged(w, 8, "f16", plan=plan, dev=dev, cu_rows=bad)
    assert flags & va.VA_FLAG_BAD_ROWS
    check_parity(got[:cu[2] - 1], ref[:cu[2] - 1], "f16", "sequences before a decreasing cu_rows entry")
    # the 100-row prefill segment with a parent that is not a chain: its rows NaN
    wb = copy.deepcopy(w)
    wb.parent = w.parent.copy()
    wb.parent[77] = 10
    say("[case] long segment with a non-chain parent")
    got, _, flags, _ = run_ragged(wb, 8, "f16", plan=plan)
    assert flags & va.VA_FLAG_BAD_PARENT
    assert np.all(np.isnan(got[:100]))
    check_parity(got[100:cu[-1]], ref[100:], "f16", "others beside a bad long parent")


def test_ragged_graph_replay_with_live_rows():
    """Capture one ragged call, then change cu_rows / ctx on the device and
    replay: every replay matches the oracle for the rows it was given."""
    import torch

    w, ref, _ = mixed()
    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f16"), 8, 0)
    ws = vdev.workspace(plan)
    cap = plan.problem.max_total_rows
    out = torch.empty((cap, w.H, w.D), dtype=torch.float16, device="cuda")
    lse = torch.empty((cap, w.H), dtype=torch.float32, device="cuda")
    cu_live = dev["cu_rows"].clone()
    s = torch.cuda.Stream()
    args = lambda: (plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                    dev["block_table"], dev["ctx_lens"], cu_live, dev["parent"], 8, out, lse, ws)
    with torch.cuda.stream(s):
        va.verify_attn_run_ragged(*args(), stream=s)  # warm up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        va.verify_attn_run_ragged(*args(), stream=s)
    torch.cuda.synchronize()
    cu = w.cu_rows
    no_tree = cu.copy()
    no_tree[-1] = no_tree[-2]
    for rep, c in enumerate([cu, no_tree, cu]):
        cu_live.copy_(torch.from_numpy(c.astype(np.int32)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().double().numpy()
        n = int(c[-1])
        check_parity(got[:n], ref[:n], "f16", f"graph replay {rep} rows={n}")


@pytest.mark.parametrize("S_", [1, 0])
def test_longest_prefill_segment(S_):
    """A 4,096-row prefill segment (the largest ragged row count) beside a
    5-row direct chain, 4 query heads over 2 KV heads, D 64."""
    if "r4096" not in _cache:
        w = S.make_workload("r4096", ctx_lens=[4200, 300], rows=[4096, 5], H=4, KVH=2, D=64, q_dtype="bf16",
                            kv_dtype="q8_0", seed=4, permute=True,
                            parent=np.concatenate([S.chain_parent(4096), S.chain_parent(5)]))
        say("[oracle] r4096")
        _cache["r4096"] = (w,) + oracle.attention(w)
    w, ref, lref = _cache["r4096"]
    say(f"[case] 4096-row segment S={S_}")
    got, lse, flags, plan = run_ragged(w, S_, "f32")
    assert flags == 0
    n = w.total_rows
    check_parity(got[:n], ref, "f32", f"4096-row segment S={S_}")
    assert np.abs(lse[:n] - lref).max() <= 2e-3


@pytest.mark.parametrize("S_", [64, 256])
def test_short_sequences_leave_their_extra_splits(S_):
    """Ragged calls split each sequence by its own context into splits of at
    least 32 pages: contexts of 17, 130 and 4,000 tokens fill 1, 1 and 8 of
    the S splits, and the workgroups of the other splits write nothing.  The
    partial area of the workspace is filled with NaN bytes first, so the
    merge reading any split that was not written would show."""
    import torch

    w = S.make_workload("short_splits", ctx_lens=[17, 130, 4000, 64], rows=[5, 12, 16, 0], H=24, KVH=4, D=256,
                        q_dtype="bf16", kv_dtype="q8_0", seed=67, permute=True, spare_pages=3, poison=True)
    say(f"[case] short sequences S={S_} ctx={w.ctx_lens.tolist()} rows={np.diff(w.cu_rows).tolist()}")
    ref, lref = oracle.attention(w)
    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f32"), S_, 0)
    ws = vdev.workspace(plan)
    ws[256:] = 0xFF  # NaN in every fp32 partial slot (the flag header stays zero)
    cap = plan.problem.max_total_rows
    out = torch.full((cap, w.H, w.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((cap, w.H), float("nan"), dtype=torch.float32, device="cuda")
    va.verify_attn_run_ragged(plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                              dev["block_table"], dev["ctx_lens"], dev["cu_rows"], dev["parent"], S_, out, lse, ws)
    torch.cuda.synchronize()
    assert va.verify_attn_read_flags(plan, ws) == 0
    n = w.total_rows
    got = out.cpu().double().numpy()[:n]
    check_parity(got, ref, "f32", f"short sequences S={S_}")
    assert np.abs(lse.cpu().double().numpy()[:n] - lref).max() <= 2e-3


def test_largest_split_count_in_row_entries():
    """At S = 256 a 131,072-token sequence fills every split (32 pages each),
    so its rows' entries in the merge's list carry 255 (splits - 1) in bits
    23-30; a 600-token sequence beside it fills two (38 pages).  The partial area
    is filled with NaN bytes first, so a split read past a row's own count
    would show.  The list read back equals its rule, and the outputs match
    the oracle."""
    import torch

    w = S.make_workload("split256", ctx_lens=[131072, 600], rows=[3, 2], H=8, KVH=2, D=64, q_dtype="bf16",
                        kv_dtype="q8_0", seed=71, permute=True, spare_pages=3, poison=True)
    say(f"[case] split counts at S=256 ctx={w.ctx_lens.tolist()} rows={np.diff(w.cu_rows).tolist()}")
    ref, lref = oracle.attention(w)
    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f32"), 256, 0)
    ws = vdev.workspace(plan)
    ws[256:] = 0xFF
    cap = plan.problem.max_total_rows
    out = torch.full((cap, w.H, w.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((cap, w.H), float("nan"), dtype=torch.float32, device="cuda")
    va.verify_attn_run_ragged(plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                              dev["block_table"], dev["ctx_lens"], dev["cu_rows"], dev["parent"], 256, out, lse, ws)
    torch.cuda.synchronize()
    assert va.verify_attn_read_flags(plan, ws) == 0
    n_items, n_rows, n_heavy, it, mrows = _read_work_list(ws, w, plan)
    want_items, want_rows, want_heavy = _work_list_model(w, w.cu_rows, 256, plan)
    assert (mrows >> 23).tolist() == [255, 255, 255, 1, 1]
    assert n_items == len(want_items) and n_rows == len(want_rows) and n_heavy == want_heavy == 3
    assert mrows.tolist() == want_rows
    assert [tuple(x) for x in it.tolist()] == want_items
    n = w.total_rows
    check_parity(out.cpu().double().numpy()[:n], ref, "f32", "split counts at S=256")
    assert np.abs(lse.cpu().double().numpy()[:n] - lref).max() <= 2e-3


@pytest.mark.parametrize("kv,S_", [("q8_0", 0), ("f16", 3)])
@pytest.mark.parametrize("nseq", [150, 64, 65])
def test_many_sequences(kv, S_, nseq):
    # 150 (and 64, 65) sequences of 0-4 rows, empty ones among them: the work
    # list orders them by size and numbers their row groups (up to 64
    # sequences by the one-wave pass, a lane each; 65 and more by the
    # one-workgroup pass)
    rng = np.random.default_rng(29)
    rows = rng.integers(0, 5, 150)
    rows[[0, 63, 64, 127, 128, 149]] = [0, 0, 3, 0, 2, 0]
    ctxs = rows + rng.integers(1, 150, 150)
    rows, ctxs = rows[:nseq], ctxs[:nseq]
    w = tiny_ragged(kv, seed=29, rows=tuple(int(r) for r in rows), ctxs=tuple(int(c) for c in ctxs), tree=False)
    say(f"[case] {len(rows)} ragged sequences, {int(rows.sum())} rows, kv={kv} S={S_}")
    ref, lref = oracle.attention(w)
    got, lse, flags, plan = run_ragged(w, S_, "f16")
    n = w.total_rows
    assert flags == 0
    check_parity(got[:n], ref, "f16", f"150 sequences kv={kv} S={plan.info().num_splits if S_ == 0 else S_}")
    assert np.abs(lse[:n] - lref).max() <= 2e-3


def _item_cap(w, plan, S):
    """Entries the grid holds: S * groups * KVH, groups bounding the row groups
    of sequences whose rows fill the packed capacity."""
    info = plan.info()
    G = w.H // w.KVH
    qr = info.rows_per_group
    cap_rows = plan.problem.max_total_rows
    bound = (cap_rows * G + w.num_seqs * (qr - 1)) // qr
    groups = max(1, min(bound, w.num_seqs * info.row_groups))
    return S * groups * w.KVH


def _work_list_model(w, cu, S, plan, ctx_lens=None):
    """The work list a ragged call should hold, written out from its rule: each
    sequence's row groups (ceil(rows * G / rows_per_group); none for a bad
    cu_rows entry), pages per split (at least 32) and splits from its own
    context (one split for a bad context); sequences taken in index order
    while their rows fit the packed capacity and their entries the grid;
    those ordered by split count, then pages per split, descending (ties by
    index); each sequence's entries by split, row group, KV head; then its
    packed rows for the merge, and how many of those rows have more than 8
    splits.  An entry's first word is the sequence, with bit 30 set for a
    sequence of at most 32 (row, head) pairs when the plan's row groups are
    larger."""
    info = plan.info()
    G = w.H // w.KVH
    cap_rows = plan.problem.max_total_rows
    B = plan.problem.rows_per_seq
    max_ctx = plan.problem.max_ctx
    max_pages = plan.problem.max_pages_per_seq
    cap = _item_cap(w, plan, S)
    ctx_lens = w.ctx_lens if ctx_lens is None else ctx_lens
    seqs = []
    ib = rb = 0
    for s in range(w.num_seqs):
        a, e = int(cu[s]), int(cu[s + 1])
        bad = a < 0 or e < a or e > cap_rows or e - a > B
        rows = 0 if bad else e - a
        groups = -(-rows * G // info.rows_per_group)
        ctx = int(ctx_lens[s])
        ctx_bad = ctx < rows or ctx > max_ctx or ctx > max_pages * 16
        np_ = 0 if ctx_bad else -(-ctx // 16)
        pp = max(-(-np_ // S), 32)
        splits = max(1, -(-np_ // pp))
        items = groups * splits * w.KVH
        ib += items
        rb += rows
        fits = ib <= cap and rb <= cap_rows
        key = (splits << 21) + min(pp, (1 << 21) - 1) if (fits and items) else 0
        seqs.append((key, s, a, rows, groups, splits, items))
    seqs = [t if t[0] else (0, t[1], t[2], 0, t[4], t[5], 0) for t in seqs]
    order = sorted(seqs, key=lambda t: (-t[0], t[1]))
    items, merge_rows, heavy = [], [], 0
    for key, s, a, rows, groups, splits, n in order:
        if not n:  # not taken, or nothing to do
            continue
        # a sequence of at most 32 (row, head) pairs runs the 32-row body
        thin = info.rows_per_group > 32 and rows * G <= 32
        word = s | (0x40000000 if thin else 0)
        for sp in range(splits):
            for g in range(groups):
                for kvh in range(w.KVH):
                    items.append((word, (g << 16) | (sp << 8) | kvh))
        # each row entry carries its sequence's split count less one from bit 23
        merge_rows.extend(r | ((splits - 1) << 23) for r in range(a, a + rows))
        heavy += rows if splits > 8 else 0
    return items, merge_rows, heavy


def _read_work_list(ws, w, plan):
    info = plan.info()
    nrows = plan.problem.max_total_rows * w.H
    smax = info.max_splits
    off = 256
    if smax > 1:
        off = -(-(256 + smax * nrows * (w.D + 2) * 4) // 256) * 256
    raw = ws.cpu().numpy()
    cnt = raw[off:off + 12].view(np.int32)
    mr_bytes = -(-plan.problem.max_total_rows * 4 // 16) * 16
    mrows = raw[off + 16:off + 16 + 4 * int(cnt[1])].view(np.int32)
    it = raw[off + 16 + mr_bytes:off + 16 + mr_bytes + 8 * int(cnt[0])].view(np.int32).reshape(-1, 2)
    return int(cnt[0]), int(cnt[1]), int(cnt[2]), it, mrows


@pytest.mark.parametrize("name", ["mixed", "paged4", "many"])
def test_work_list_matches_its_rule(name):
    """The work list, read back from the workspace, equals the list its rule
    gives, entry for entry (integer work: bit-exact): the counts, the
    entries and the merge's row order, from the one-wave pass (up to 64
    sequences) and from the one-workgroup pass (150 sequences)."""
    import torch

    if name == "mixed":
        w = S.mixed_lowering()
        cu = w.cu_rows
    elif name == "paged4":
        w = copy.deepcopy(S.paged_ragged())
        w.parent = None
        cu = np.arange(0, 65, 16, dtype=np.int32)
        w.cu_rows = cu
    else:
        rng = np.random.default_rng(41)
        counts = rng.integers(0, 5, size=150)
        ctxs = rng.integers(8, 3000, size=150)
        w = S.make_workload("sched_many", ctx_lens=list(ctxs), rows=list(counts), H=8, KVH=2, D=64,
                            q_dtype="bf16", kv_dtype="q8_0", seed=41, permute=True)
        cu = w.cu_rows
    say(f"[case] work list {name}")
    dev = vdev.to_device(w)
    for S_ in (0, 8):
        plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f16"), S_, 0)
        Sc = S_ or plan.info().num_splits
        ws = vdev.workspace(plan)
        cap = plan.problem.max_total_rows
        out = torch.empty((cap, w.H, w.D), dtype=torch.float16, device="cuda")
        lse = torch.empty((cap, w.H), dtype=torch.float32, device="cuda")
        cu_d = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
        va.verify_attn_run_ragged(plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                                  dev["block_table"], dev["ctx_lens"], cu_d, dev["parent"], S_, out, lse, ws)
        torch.cuda.synchronize()
        n_items, n_rows, n_heavy, it, mrows = _read_work_list(ws, w, plan)
        want_items, want_rows, want_heavy = _work_list_model(w, cu, Sc, plan)
        say(f"  S={Sc}: {n_items} entries, {n_rows} rows, {n_heavy} merged by workgroup")
        assert n_items == len(want_items) and n_rows == len(want_rows) and n_heavy == want_heavy
        assert mrows.tolist() == want_rows
        assert [tuple(x) for x in it.tolist()] == want_items


@pytest.mark.parametrize("seed", range(24))
def test_work_list_random_batches(seed):
    """Random batches (1 to 150 sequences, 0 to 9 rows, contexts up to 3,000,
    the plan's S or a random one), some with bad cu_rows entries or contexts:
    the list read back equals its rule, entry for entry, and the bad entries
    are flagged."""
    import torch

    rng = np.random.default_rng(900 + seed)
    n = int(rng.choice([1, 2, 5, 17, 63, 64, 65, 150]))
    rows = rng.integers(0, 10, n)
    ctxs = rows + rng.integers(1, 3000, n)
    w = S.make_workload(f"sched_rand{seed}", ctx_lens=list(ctxs), rows=list(rows), H=8, KVH=2, D=64,
                        q_dtype="bf16", kv_dtype="q8_0", seed=900 + seed, permute=True)
    dev = vdev.to_device(w)
    S_ = int(rng.choice([0, 0, 1, 3, 8, 40]))
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f16"), S_, 0)
    Sc = S_ or plan.info().num_splits
    cu = w.cu_rows.copy()
    ctx_live = w.ctx_lens.copy()
    if seed % 3 == 1 and n > 2:  # a decreasing entry (its sequence and the next change)
        k = int(rng.integers(1, n))
        cu[k] = max(0, int(cu[k - 1]) - 1)
    cap_rows, B = plan.problem.max_total_rows, plan.problem.rows_per_seq
    expect_bad_rows = any(cu[s] < 0 or cu[s + 1] < cu[s] or cu[s + 1] > cap_rows or cu[s + 1] - cu[s] > B
                          for s in range(n))
    if seed % 3 == 2:  # a context past max_ctx: that sequence keeps one split
        ctx_live[int(rng.integers(0, n))] = plan.problem.max_ctx + 1
    say(f"[case] work list random seed={seed} n={n} rows={int(rows.sum())} S={Sc}")
    ws = vdev.workspace(plan)
    cap = plan.problem.max_total_rows
    out = torch.empty((cap, w.H, w.D), dtype=torch.float16, device="cuda")
    lse = torch.empty((cap, w.H), dtype=torch.float32, device="cuda")
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    ctx_d = torch.from_numpy(np.asarray(ctx_live, np.int32)).cuda()
    va.verify_attn_run_ragged(plan, dev["q"], dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                              dev["block_table"], ctx_d, cu_d, None, S_, out, lse, ws)
    torch.cuda.synchronize()
    n_items, n_rows, n_heavy, it, mrows = _read_work_list(ws, w, plan)
    want_items, want_rows, want_heavy = _work_list_model(w, cu, Sc, plan, ctx_live)
    assert (n_items, n_rows, n_heavy) == (len(want_items), len(want_rows), want_heavy)
    assert mrows.tolist() == want_rows
    assert [tuple(x) for x in it.tolist()] == want_items
    flags = va.verify_attn_read_flags(plan, ws)
    assert bool(flags & va.VA_FLAG_BAD_ROWS) == expect_bad_rows


def _thin_mix(seed):
    """A ragged batch of one sequence with many rows (so the plan's row groups
    hold 64 or 96 rows) beside 2-5 sequences of 0-8 rows, in a seeded head
    layout, head_dim and KV type."""
    rng = np.random.default_rng(7000 + seed)
    H, KVH = [(24, 4), (8, 2), (16, 2), (4, 1)][seed % 4]
    G = H // KVH
    D = [64, 128, 256][seed % 3]
    kv = ["q8_0", "f16"][(seed // 3) % 2]
    n_small = int(rng.integers(2, 6))
    big = int(rng.integers(33 // G + 2, 80 // G + 12))
    rows = [big] + [int(x) for x in rng.integers(0, 9, size=n_small)]
    order = rng.permutation(len(rows))
    rows = [rows[i] for i in order]
    ctx = [int(max(r, rng.integers(40, 3000))) for r in rows]
    w = S.make_workload(f"thin_mix{seed}", ctx_lens=ctx, rows=rows, H=H, KVH=KVH, D=D, q_dtype="bf16",
                        kv_dtype=kv, seed=7100 + seed, permute=True, spare_pages=3, poison=True)
    return w


@pytest.mark.parametrize("seed", range(10))
def test_thin_entries_in_mixed_batches(seed):
    """Sequences of at most 32 (row, head) pairs beside a long one run the
    32-row partial body (the work-list pass marks their entries): every row
    meets the oracle's gate, and every sequence's rows equal, bit for bit,
    the same sequence run alone on the same plan (which body runs follows
    from the sequence's own rows and the plan only)."""
    import torch

    w = _thin_mix(seed)
    G = w.H // w.KVH
    rows = np.diff(w.cu_rows).tolist()
    plan = va.verify_attn_plan(vdev.problem_for(w, out_dtype="f32"), 0, 0)
    qr = plan.info().rows_per_group
    thin = [r for r in rows if 0 < r and r * G <= 32 and qr > 32]
    say(f"[case] thin mix seed={seed} H={w.H}/{w.KVH} D={w.D} kv={w.kv_dtype} rows={rows} "
        f"ctx={w.ctx_lens.tolist()} group={qr} thin={len(thin)}")
    assert qr > 32 and thin  # the batch exercises both bodies
    got, lse, flags, _ = run_ragged(w, 0, "f32", plan=plan)
    assert flags == 0
    n = w.total_rows
    ref, lref = oracle.attention(w)
    check_parity(got[:n], ref, "f32", f"thin mix {seed}")
    assert np.abs(lse[:n] - lref).max() <= 2e-3
    dev = vdev.to_device(w)
    for s, r in enumerate(rows):
        if r == 0:
            continue
        # sequence s alone: the other sequences get no rows
        a = int(w.cu_rows[s])
        cu = np.zeros(w.num_seqs + 1, np.int32)
        cu[s + 1:] = r
        q_alone = torch.zeros_like(dev["q"])
        q_alone[:r] = dev["q"][a:a + r]
        alone, alone_lse, aflags, _ = run_ragged(w, 0, "f32", plan=plan, dev=dev, cu_rows=cu, q=q_alone)
        assert aflags == 0
        assert np.array_equal(alone[:r], got[a:a + r]), f"sequence {s} ({r} rows) changed with the batch"
        assert np.array_equal(alone_lse[:r], lse[a:a + r])
