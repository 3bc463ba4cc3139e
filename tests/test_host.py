"""Host-only tests of libverify_attn.so: exports, plan validation, the split
heuristic and workspace sizing, and run-time argument checks that fail
before anything is launched (no GPU needed)."""

import ctypes
import os
import re

import pytest

import speculative_decoding_verify_kv_amd as va

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(va.LIB_PATH):
        from speculative_decoding_verify_kv_amd import build

        build.build()
    return va.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "verify_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(verify_attn_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(va.EXPORTED)


def qwen(**kw):
    base = dict(num_seqs=1, rows_per_seq=16, num_q_heads=24, num_kv_heads=4, head_dim=256, num_pages=2048,
                max_pages_per_seq=2048, max_ctx=32768, q_dtype="bf16", kv_dtype="q8_0", out_dtype="f16")
    base.update(kw)
    return va.make_problem(**base)


def plan_status(problem, splits=0, cus=256):
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    st = va.load().verify_attn_plan_for_cus(ctypes.byref(problem) if problem is not None else None, splits, cus,
                                            ctypes.byref(h), ctypes.byref(ws))
    if st == 0:
        va.load().verify_attn_plan_destroy(h)
    else:
        assert not h.value  # nothing handed out on error
    return st


def test_headline_plan_and_workspace(lib):
    p = va.verify_attn_plan_for_cus(qwen(), 0, 256)
    info = p.info()
    # one workgroup per (split, KV head) covers all 96 rows of the GQA group,
    # so 64 splits x 4 KV heads fill the 256 CUs once
    assert info.row_groups == 1 and info.rows_per_group == 96
    assert info.num_splits == 64 and info.max_splits == 64
    assert info.pages_per_split == 32
    nrows = 1 * 16 * 24
    # flag header, then fp32 O, m and l per split and row
    assert info.workspace_bytes == 256 + 64 * nrows * (256 + 2) * 4
    assert p.workspace_bytes == info.workspace_bytes


@pytest.mark.parametrize("cus", [1, 8, 64, 256, 304])
def test_heuristic_bounds(lib, cus):
    p = va.verify_attn_plan_for_cus(qwen(), 0, cus)
    info = p.info()
    units = 4 * info.row_groups
    assert 1 <= info.num_splits <= 256
    # whole 64-token tiles, at least two, per split
    assert info.pages_per_split >= 8 and info.pages_per_split % 4 == 0
    tiles = info.pages_per_split // 4
    # one round of workgroups at most ...
    assert info.num_splits * units <= max(cus, units)
    # ... and no fewer tiles per split would still fit in it
    if tiles > 2 and cus >= units:
        assert -(-2048 // (4 * (tiles - 1))) * units > cus
    # the fewest splits with that many tiles
    assert -(-2048 // info.pages_per_split) == info.num_splits


def test_explicit_splits_and_direct(lib):
    p = va.verify_attn_plan_for_cus(qwen(), 8, 256)
    assert p.info().num_splits == 8 and p.info().max_splits == 8
    p1 = va.verify_attn_plan_for_cus(qwen(), 1, 256)
    assert p1.info().workspace_bytes == 256  # direct path needs only the flag header


@pytest.mark.parametrize("B,G,D,nt,rg", [(16, 6, 256, 6, 1), (10, 6, 256, 4, 1), (32, 6, 256, 6, 2),
                                         (4, 6, 256, 2, 1), (16, 6, 128, 6, 1), (4, 2, 64, 2, 1),
                                         (64, 6, 256, 6, 4), (1, 1, 64, 2, 1), (7, 6, 256, 4, 1),
                                         (20, 6, 256, 4, 2), (33, 6, 128, 6, 3)])
def test_row_tiling(lib, B, G, D, nt, rg):
    prob = qwen(rows_per_seq=B, num_q_heads=4 * G, head_dim=D)
    info = va.verify_attn_plan_for_cus(prob, 0, 256).info()
    assert info.rows_per_group == 16 * nt and info.row_groups == rg
    assert info.rows_per_group * info.row_groups >= B * G


def test_small_context_caps_splits(lib):
    # two tiles (8 pages) per split at least: 16 pages give 2 splits
    prob = qwen(rows_per_seq=1, num_q_heads=4, head_dim=64, max_ctx=256, max_pages_per_seq=16, num_pages=16)
    assert va.verify_attn_plan_for_cus(prob, 0, 256).info().num_splits == 2
    prob = qwen(max_ctx=256, max_pages_per_seq=16, num_pages=16)
    assert va.verify_attn_plan_for_cus(prob, 0, 256).info().num_splits == 2
    # 2,048 tokens: 128 pages, 16 splits of 2 tiles
    prob = qwen(max_ctx=2048, max_pages_per_seq=128, num_pages=128)
    assert va.verify_attn_plan_for_cus(prob, 0, 256).info().num_splits == 16
    # 20,676 tokens: 1,293 pages; 64 splits would need 6 tiles each anyway, so 54
    prob = qwen(max_ctx=20676, max_pages_per_seq=1293, num_pages=1293)
    info = va.verify_attn_plan_for_cus(prob, 0, 256).info()
    assert info.num_splits == 54 and info.pages_per_split == 24


def test_many_sequences_fill_the_cus_once(lib):
    # 32 sequences x 4 KV heads = 128 units: 2 splits of 64 tiles each, one
    # round of 256 workgroups
    prob = qwen(num_seqs=32, max_ctx=8192, max_pages_per_seq=512, num_pages=32 * 512)
    info = va.verify_attn_plan_for_cus(prob, 0, 256).info()
    assert info.num_splits == 2 and info.pages_per_split == 256
    # 6 KV heads: floor(256 / 6) = 42 splits, never a 43rd that would spill
    # two workgroups into a second round
    prob = qwen(num_q_heads=24, num_kv_heads=6)
    info = va.verify_attn_plan_for_cus(prob, 0, 256).info()
    assert info.num_splits * 6 * info.row_groups <= 256


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=25), va.VA_EINVAL),
    (dict(head_dim=96), va.VA_EUNSUPPORTED),
    (dict(rows_per_seq=65), va.VA_EUNSUPPORTED),
    (dict(page_size=32), va.VA_EUNSUPPORTED),
    (dict(kv_dtype="f32"), va.VA_EUNSUPPORTED),
    (dict(kv_dtype="bf16"), va.VA_EUNSUPPORTED),
    (dict(q_dtype="q8_0"), va.VA_EUNSUPPORTED),
    (dict(out_dtype="q8_0"), va.VA_EUNSUPPORTED),
    (dict(max_ctx=32769), va.VA_EINVAL),          # beyond the block table
    (dict(max_ctx=8), va.VA_EINVAL),              # fewer tokens than drafted rows
    (dict(scale=-1.0), va.VA_EINVAL),
    (dict(num_seqs=0), va.VA_EINVAL),
])
def test_plan_rejects(lib, kw, status):
    assert plan_status(qwen(**kw)) == status


def test_plan_rejects_null_and_bad_splits(lib):
    assert plan_status(None) == va.VA_EINVAL
    assert plan_status(qwen(), splits=257) == va.VA_EINVAL
    assert plan_status(qwen(), splits=-1) == va.VA_EINVAL
    assert plan_status(qwen(), cus=0) == va.VA_EINVAL


# ---- run-time checks: all fail before any HIP call, so they run without a GPU ----

FAKE = 1 << 20  # 16-byte aligned, never dereferenced on these paths


def run_status(plan, **over):
    a = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, k_scale=FAKE, v_scale=FAKE, block_table=FAKE, ctx_lens=FAKE,
             parent=None, num_splits=0, out=FAKE, lse=None, workspace=FAKE, workspace_bytes=plan.workspace_bytes)
    a.update(over)
    return va.verify_attn_run(plan, a["q"], a["k_pool"], a["v_pool"], a["k_scale"], a["v_scale"],
                              a["block_table"], a["ctx_lens"], a["parent"], a["num_splits"], a["out"], a["lse"],
                              a["workspace"], a["workspace_bytes"], None, raise_on_error=False)


def test_run_rejects_bad_arguments(lib):
    plan = va.verify_attn_plan_for_cus(qwen(), 8, 256)
    assert run_status(plan, workspace_bytes=plan.workspace_bytes - 1) == va.VA_EWORKSPACE
    assert run_status(plan, num_splits=9) == va.VA_EWORKSPACE
    assert run_status(plan, num_splits=-2) == va.VA_EINVAL
    assert run_status(plan, q=None) == va.VA_EINVAL
    assert run_status(plan, out=None) == va.VA_EINVAL
    assert run_status(plan, workspace=None) == va.VA_EINVAL
    assert run_status(plan, k_scale=None) == va.VA_EINVAL        # Q8 needs scales
    assert run_status(plan, q=FAKE + 8) == va.VA_EINVAL          # misaligned
    assert run_status(plan, workspace=FAKE + 16) == va.VA_EINVAL
    assert run_status(plan, parent=FAKE) == va.VA_EINVAL         # has_parent == 0
    assert run_status(plan, block_table=FAKE + 2) == va.VA_EINVAL
    plan_p = va.verify_attn_plan_for_cus(qwen(has_parent=True), 8, 256)
    assert run_status(plan_p) == va.VA_EINVAL                    # parent required
    plan_f16 = va.verify_attn_plan_for_cus(qwen(kv_dtype="f16"), 8, 256)
    assert run_status(plan_f16) == va.VA_EINVAL                  # fp16 KV takes no scales


def test_merge_entry_checks(lib):
    plan = va.verify_attn_plan_for_cus(qwen(), 8, 256)
    f = va.verify_attn_run_merge
    assert f(plan, 1, FAKE, None, FAKE, plan.workspace_bytes, None, raise_on_error=False) == va.VA_EINVAL
    assert f(plan, 9, FAKE, None, FAKE, plan.workspace_bytes, None, raise_on_error=False) == va.VA_EWORKSPACE
    assert f(plan, 8, FAKE, None, FAKE, 100, None, raise_on_error=False) == va.VA_EWORKSPACE


def append_status(plan, **over):
    a = dict(k_new=FAKE, v_new=FAKE, new_dtype="f32", k_pool=FAKE, v_pool=FAKE, k_scale=FAKE, v_scale=FAKE,
             block_table=FAKE, ctx_lens=FAKE, workspace=FAKE, workspace_bytes=256)
    a.update(over)
    return va.verify_attn_append_kv(plan, a["k_new"], a["v_new"], a["new_dtype"], a["k_pool"], a["v_pool"],
                                    a["k_scale"], a["v_scale"], a["block_table"], a["ctx_lens"], a["workspace"],
                                    a["workspace_bytes"], None, raise_on_error=False)


def test_append_rejects_bad_arguments(lib):
    plan = va.verify_attn_plan_for_cus(qwen(), 8, 256)
    assert append_status(plan, new_dtype="q8_0") == va.VA_EINVAL    # inputs are f32 / f16 / bf16
    assert append_status(plan, k_new=None) == va.VA_EINVAL
    assert append_status(plan, v_pool=None) == va.VA_EINVAL
    assert append_status(plan, k_scale=None) == va.VA_EINVAL        # 8-bit pools need their scales
    assert append_status(plan, k_new=FAKE + 4) == va.VA_EINVAL      # misaligned
    assert append_status(plan, ctx_lens=FAKE + 2) == va.VA_EINVAL
    assert append_status(plan, workspace=FAKE + 64) == va.VA_EINVAL
    assert append_status(plan, workspace_bytes=255) == va.VA_EWORKSPACE
    plan_f16 = va.verify_attn_plan_for_cus(qwen(kv_dtype="f16"), 8, 256)
    assert append_status(plan_f16) == va.VA_EINVAL                  # fp16 pools take no scales
    assert va.load().verify_attn_append_kv(None, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                           256, None) == va.VA_EINVAL


def promote_status(plan, **over):
    a = dict(accepted=FAKE, n_accepted=FAKE, parent=None, k_pool=FAKE, v_pool=FAKE, k_scale=FAKE, v_scale=FAKE,
             block_table=FAKE, ctx_lens=FAKE, new_ctx=None, workspace=FAKE,
             workspace_bytes=va.verify_attn_promote_workspace_bytes(plan))
    a.update(over)
    return va.verify_attn_promote_kv(plan, a["accepted"], a["n_accepted"], a["parent"], a["k_pool"], a["v_pool"],
                                     a["k_scale"], a["v_scale"], a["block_table"], a["ctx_lens"], a["new_ctx"],
                                     a["workspace"], a["workspace_bytes"], None, raise_on_error=False)


def test_promote_workspace_and_rejections(lib):
    plan = va.verify_attn_plan_for_cus(qwen(), 8, 256)
    # 256-byte header + per (row, KV head, K or V) one staged row: D int8 + D/32 fp16 scales, 16-byte rounded
    assert va.verify_attn_promote_workspace_bytes(plan) == 256 + 1 * 16 * 4 * 2 * 272
    assert promote_status(plan, workspace_bytes=va.verify_attn_promote_workspace_bytes(plan) - 1) == va.VA_EWORKSPACE
    assert promote_status(plan, accepted=None) == va.VA_EINVAL
    assert promote_status(plan, parent=FAKE) == va.VA_EINVAL          # has_parent == 0
    assert promote_status(plan, k_scale=None) == va.VA_EINVAL
    assert promote_status(plan, new_ctx=FAKE + 2) == va.VA_EINVAL
    assert promote_status(plan, new_ctx=FAKE + 64, ctx_lens=FAKE + 64) == va.VA_EINVAL  # new_ctx is ctx_lens
    assert promote_status(plan, workspace=FAKE + 128) == va.VA_EINVAL
    plan_p = va.verify_attn_plan_for_cus(qwen(has_parent=True), 8, 256)
    assert promote_status(plan_p) == va.VA_EINVAL                     # parent required
    plan_f16 = va.verify_attn_plan_for_cus(qwen(kv_dtype="f16"), 8, 256)
    assert va.verify_attn_promote_workspace_bytes(plan_f16) == 256 + 1 * 16 * 4 * 2 * 512
    assert promote_status(plan_f16) == va.VA_EINVAL                   # fp16 pools take no scales
    assert va.load().verify_attn_promote_workspace_bytes(None) == 0


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4):
        assert va.verify_attn_status_string(st)
    assert va.verify_attn_status_string(-99) == "unknown status"


# ---------------------------------------------------------------------------
# ragged plans (verify_attn_run_ragged)
# ---------------------------------------------------------------------------

def ragged_status(plan, **over):
    a = dict(q=FAKE, k_pool=FAKE, v_pool=FAKE, k_scale=FAKE, v_scale=FAKE, block_table=FAKE, ctx_lens=FAKE,
             cu_rows=FAKE, parent=None, num_splits=0, out=FAKE, lse=None, workspace=FAKE,
             workspace_bytes=plan.workspace_bytes)
    a.update(over)
    return va.verify_attn_run_ragged(plan, a["q"], a["k_pool"], a["v_pool"], a["k_scale"], a["v_scale"],
                                     a["block_table"], a["ctx_lens"], a["cu_rows"], a["parent"], a["num_splits"],
                                     a["out"], a["lse"], a["workspace"], a["workspace_bytes"], None,
                                     raise_on_error=False)


def test_ragged_plan_sizes_by_packed_rows(lib):
    # 5 sequences, at most 100 rows each, 149 packed rows: the workspace and the
    # row tiling follow the packed capacity and the largest count
    prob = qwen(num_seqs=5, rows_per_seq=100, max_total_rows=149, max_ctx=40000, max_pages_per_seq=2500,
                num_pages=8192)
    plan = va.verify_attn_plan_for_cus(prob, 8, 256)
    info = plan.info()
    assert info.rows_per_group == 96 and info.row_groups == 7  # 600 rows -> 38 tiles -> 7 groups of 6
    # header, fp32 partials of 8 splits, then (256-byte aligned) the work list: 2 counts in 16 bytes, the 149 packed
    # rows (padded to 16 bytes) and 8 splits x 14 row groups x 4 KV heads
    # entries of 8 bytes (14 = (149 * 6 + 5 * 95) // 96 groups at most)
    parts = 256 + 8 * 149 * 24 * 258 * 4
    assert info.workspace_bytes == -(-parts // 256) * 256 + 16 + 608 + 8 * 14 * 4 * 8
    # the plan's own split count is sized for one long decode sequence (one
    # row group per KV head) filling the CUs that two minimum-size splits per
    # KV head of each of the 4 other sequences leave (256 - 32 = 224, 56 per
    # KV head): 2,500 pages in 53 splits of 12 tiles; the shorter sequences of
    # the call keep to fewer splits themselves
    info = va.verify_attn_plan_for_cus(prob, 0, 256).info()
    assert info.num_splits == 53 and info.pages_per_split == 48
    # one sequence keeps every CU; many keep at least half of them
    one = qwen(num_seqs=1, rows_per_seq=100, max_total_rows=100, max_ctx=40000, max_pages_per_seq=2500,
               num_pages=8192)
    assert va.verify_attn_plan_for_cus(one, 0, 256).info().num_splits == 63
    many = qwen(num_seqs=40, rows_per_seq=4, max_total_rows=160, max_ctx=40000, max_pages_per_seq=2500,
                num_pages=8192)
    assert va.verify_attn_plan_for_cus(many, 0, 256).info().num_splits == 32  # 128 CUs: 32 per KV head, 20 tiles
    # long prefill segments are allowed only in ragged plans
    assert plan_status(qwen(rows_per_seq=65)) == va.VA_EUNSUPPORTED
    assert plan_status(qwen(rows_per_seq=4096, max_total_rows=4096, max_ctx=32768)) == va.VA_OK
    assert plan_status(qwen(rows_per_seq=4097, max_total_rows=4097, max_ctx=32768)) == va.VA_EUNSUPPORTED
    # the work list holds at most 2,048 sequences and 256 KV heads
    assert plan_status(qwen(num_seqs=2048, rows_per_seq=1, max_total_rows=2048)) == va.VA_OK
    assert plan_status(qwen(num_seqs=2049, rows_per_seq=1, max_total_rows=2049)) == va.VA_EUNSUPPORTED
    assert plan_status(qwen(num_seqs=2049, rows_per_seq=1)) == va.VA_OK  # uniform plans have no such list
    # one split's partials (rows x heads x head_dim floats) must stay below 2^31 bytes
    assert plan_status(qwen(num_seqs=1365, rows_per_seq=64, max_ctx=64)) == va.VA_OK       # 2,096,640 row-heads
    assert plan_status(qwen(num_seqs=1366, rows_per_seq=64, max_ctx=64)) == va.VA_EUNSUPPORTED  # 2,098,176
    # capacity above num_seqs * rows_per_seq, or negative
    assert plan_status(qwen(num_seqs=2, rows_per_seq=10, max_total_rows=21)) == va.VA_EINVAL
    assert plan_status(qwen(max_total_rows=-1)) == va.VA_EINVAL


def test_ragged_entry_checks(lib):
    ragged = va.verify_attn_plan_for_cus(qwen(num_seqs=3, rows_per_seq=40, max_total_rows=50), 4, 256)
    uniform = va.verify_attn_plan_for_cus(qwen(), 4, 256)
    assert ragged_status(uniform) == va.VA_EINVAL                 # uniform plans take verify_attn_run
    assert ragged_status(ragged, cu_rows=None) == va.VA_EINVAL
    assert ragged_status(ragged, cu_rows=FAKE + 2) == va.VA_EINVAL
    assert ragged_status(ragged, parent=FAKE) == va.VA_EINVAL     # has_parent == 0
    assert ragged_status(ragged, num_splits=5) == va.VA_EWORKSPACE
    assert ragged_status(ragged, workspace_bytes=ragged.workspace_bytes - 1) == va.VA_EWORKSPACE
    assert ragged_status(ragged, q=FAKE + 8) == va.VA_EINVAL
    # the ragged plan is refused by every entry point that assumes B rows per sequence
    assert run_status(ragged) == va.VA_EINVAL
    f = va.verify_attn_run_merge
    assert f(ragged, 4, FAKE, None, FAKE, ragged.workspace_bytes, None, raise_on_error=False) == va.VA_EINVAL
    assert append_status(ragged) == va.VA_EINVAL
    assert promote_status(ragged) == va.VA_EINVAL
    assert va.load().verify_attn_run_ragged(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE,
                                            None, FAKE, 1 << 30, None) == va.VA_EINVAL


def test_noalloc_host_rejections(lib):
    """verify_attn_run_noalloc refuses, before any device call: a NULL flag
    word, a ragged plan, and partials beyond its 64 MiB device array."""
    import ctypes

    fake = 1 << 20  # aligned non-NULL stand-ins (nothing is dereferenced on the host)
    big = va.make_problem(num_seqs=64, rows_per_seq=16, num_q_heads=24, num_kv_heads=4, head_dim=256,
                          num_pages=2048 * 64, max_pages_per_seq=2048, max_ctx=32768)
    plan = va.verify_attn_plan_for_cus(big, 64, 256)
    args = [plan.handle] + [fake] * 8 + [0, fake, fake]
    assert lib.verify_attn_run_noalloc(*args, None, None) == va.VA_EINVAL  # no flag word
    # 64 * 16 * 24 rows x 258 floats x 64 splits = 1.6 GB of partials
    assert lib.verify_attn_run_noalloc(*args, fake, None) == va.VA_EWORKSPACE
    # the direct path (S = 1) needs no partials at all, but still a device; a
    # ragged plan is refused outright
    rag = va.make_problem(num_seqs=2, rows_per_seq=8, num_q_heads=4, num_kv_heads=2, head_dim=64,
                          num_pages=64, max_pages_per_seq=32, max_ctx=512, max_total_rows=10)
    rplan = va.verify_attn_plan_for_cus(rag, 4, 256)
    assert lib.verify_attn_run_noalloc(rplan.handle, *([fake] * 8), 0, fake, fake, fake, None) == va.VA_EINVAL
