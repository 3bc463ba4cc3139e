"""GPU KV append (verify_attn_append_kv) against the oracle's append.

Integer codes, fp16 scales and fp16 pool values are compared bit for bit over
the whole pools (untouched slots included); then the verify attention run on
the GPU-appended pools is checked against the oracle attention of the
oracle-appended workload."""

import copy

import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verify_kv_amd as va
import synthetic as S
from speculative_decoding_verify_kv_amd import device as vdev

from .gpu_util import check_parity, ensure_lib, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _rows_to_device(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def gpu_append(w, k_new, v_new, new_dtype):
    """Append on the GPU into device copies of w's pools; returns (dev, flags)."""
    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w), 1, 0)
    ws = vdev.workspace(plan)
    kn, vn = _rows_to_device(k_new), _rows_to_device(v_new)
    va.verify_attn_append_kv(plan, kn, vn, new_dtype, dev["k_pool"], dev["v_pool"], dev["k_scale"], dev["v_scale"],
                             dev["block_table"], dev["ctx_lens"], ws)
    torch.cuda.synchronize()
    return dev, va.verify_attn_read_flags(plan, ws)


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


def case(kv_dtype, D=256, seed=51, ctxs=(40, 17, 300, 1033), B=16):
    return S.make_workload(f"append_{kv_dtype}_{D}", ctx_lens=list(ctxs), B=B, H=24, KVH=4, D=D, q_dtype="bf16",
                           kv_dtype=kv_dtype, seed=seed, permute=True, spare_pages=6, poison=True)


@pytest.mark.parametrize("kv_dtype", ["q8_0", "f16"])
@pytest.mark.parametrize("new_dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [256, 128, 64])
def test_append_bitwise(kv_dtype, new_dtype, D):
    say(f"[case] append kv={kv_dtype} new={new_dtype} D={D}")
    w = case(kv_dtype, D=D)
    k_new, v_new = S.new_kv_rows(w, new_dtype, seed=7)
    rk, rv, rks, rvs = oracle.append_kv(w, k_new, v_new, new_dtype)
    dev, flags = gpu_append(w, k_new, v_new, new_dtype)
    assert flags == 0
    assert np.array_equal(_bytes(dev["k_pool"]), rk.view(np.uint8).reshape(-1))
    assert np.array_equal(_bytes(dev["v_pool"]), rv.view(np.uint8).reshape(-1))
    if kv_dtype == "q8_0":
        assert np.array_equal(_bytes(dev["k_scale"]), rks.view(np.uint8).reshape(-1))
        assert np.array_equal(_bytes(dev["v_scale"]), rvs.view(np.uint8).reshape(-1))


@pytest.mark.parametrize("seed", range(12))
def test_append_random_bitwise(seed):
    """Seeded random batches: head_dim 64/128/256, 8-bit or fp16 pools, 4
    head layouts, B 1-32, 1-20 sequences with contexts from B to 3,000 (the
    drafted slots often straddle a page), f32 / f16 / bf16 rows.  Pools and
    scales bit for bit against the oracle's append, untouched slots
    included."""
    rng = np.random.default_rng(8000 + seed)
    D = int(rng.choice([64, 128, 256]))
    H, KVH = [(4, 2), (8, 1), (24, 4), (6, 6)][int(rng.integers(0, 4))]
    kv = str(rng.choice(["q8_0", "f16"]))
    new_dtype = str(rng.choice(["f32", "f16", "bf16"]))
    B = int(rng.integers(1, 33))
    nseq = int(rng.integers(1, 21))
    ctxs = [int(rng.integers(B, 3001)) for _ in range(nseq)]
    w = S.make_workload(f"append_rand{seed}", ctx_lens=ctxs, B=B, H=H, KVH=KVH, D=D, q_dtype="bf16", kv_dtype=kv,
                        seed=8000 + seed, permute=True, spare_pages=4, poison=True)
    say(f"[case] append random seed={seed} D={D} H={H}/{KVH} kv={kv} new={new_dtype} B={B} nseq={nseq}")
    k_new, v_new = S.new_kv_rows(w, new_dtype, seed=seed)
    rk, rv, rks, rvs = oracle.append_kv(w, k_new, v_new, new_dtype)
    dev, flags = gpu_append(w, k_new, v_new, new_dtype)
    assert flags == 0
    assert np.array_equal(_bytes(dev["k_pool"]), rk.view(np.uint8).reshape(-1))
    assert np.array_equal(_bytes(dev["v_pool"]), rv.view(np.uint8).reshape(-1))
    if kv == "q8_0":
        assert np.array_equal(_bytes(dev["k_scale"]), rks.view(np.uint8).reshape(-1))
        assert np.array_equal(_bytes(dev["v_scale"]), rvs.view(np.uint8).reshape(-1))


def test_append_extreme_blocks_bitwise():
    """Zero blocks, tiny and huge magnitudes, exact ties and NaN entries."""
    say("[case] append extreme blocks")
    w = case("q8_0", D=256, ctxs=(64, 200), B=8)
    k_new, v_new = S.new_kv_rows(w, "f32", seed=9)
    k_new = k_new.copy()
    v_new = v_new.copy()
    k_new[0, 0, :32] = 0.0                                  # all-zero block
    k_new[0, 1, :32] *= np.float32(1e-6)                    # tiny scale (fp16 subnormal)
    k_new[1, 0, 32:64] *= np.float32(3e4)                    # large values
    k_new[2, 2, :32] = 0.0
    k_new[2, 2, 0] = np.float32(127 / 8)
    k_new[2, 2, 1:8] = np.float32([2.5, -2.5, 0.5, -0.5, 1.5, 126.5, -3.5]) / 8  # exact ties
    v_new[3, 3, 64] = np.nan
    rk, rv, rks, rvs = oracle.append_kv(w, k_new, v_new, "f32")
    dev, flags = gpu_append(w, k_new, v_new, "f32")
    assert flags == 0
    for name, ref in (("k_pool", rk), ("v_pool", rv), ("k_scale", rks), ("v_scale", rvs)):
        assert np.array_equal(_bytes(dev[name]), ref.view(np.uint8).reshape(-1)), name


@pytest.mark.parametrize("S_", [1, 0])
def test_append_then_verify(S_):
    """Append the drafted rows on the GPU, then verify over the same pools."""
    say(f"[case] append then verify S={S_}")
    w = case("q8_0", D=256, ctxs=(1032, 5000), B=16)
    k_new, v_new = S.new_kv_rows(w, "bf16", seed=11)
    rk, rv, rks, rvs = oracle.append_kv(w, k_new, v_new, "bf16")
    wa = copy.copy(w)
    wa.k_pool, wa.v_pool, wa.k_scale, wa.v_scale = rk, rv, rks, rvs
    ref, _ = oracle.attention(wa)
    dev, flags = gpu_append(w, k_new, v_new, "bf16")
    assert flags == 0
    got = run_gpu(w, S_, "f32", dev=dev)[0]
    check_parity(got, ref, "f32", f"append+verify S={S_}")


def test_append_bad_metadata_flags_and_writes_nothing_else():
    say("[case] append bad metadata")
    w = case("q8_0", D=128, ctxs=(64, 200), B=8)
    k_new, v_new = S.new_kv_rows(w, "f32", seed=13)
    bad = copy.deepcopy(w)
    bad.block_table = bad.block_table.copy()
    t = int(w.ctx_lens[1]) - w.B          # first drafted slot of sequence 1
    bad.block_table[1, t // 16] = w.num_pages + 3
    dev, flags = gpu_append(bad, k_new, v_new, "f32")
    assert flags & va.VA_FLAG_BAD_PAGE
    # sequence 0 is written as the oracle writes it; sequence 1's rows in the bad
    # page are skipped, so its other rows still match an append of sequence 1
    # with only those rows
    good = copy.deepcopy(w)
    good.num_seqs, good.ctx_lens, good.block_table = 1, w.ctx_lens[:1].copy(), w.block_table[:1].copy()
    rk, rv, rks, rvs = oracle.append_kv(good, k_new[:w.B], v_new[:w.B], "f32")
    kp = dev["k_pool"].cpu().numpy()
    for i in range(w.B):
        tt = int(w.ctx_lens[0]) - w.B + i
        pg, sl = int(w.block_table[0, tt // 16]), tt % 16
        assert np.array_equal(kp[pg, :, sl], rk[pg, :, sl])
    bad2 = copy.deepcopy(w)
    bad2.ctx_lens = np.array([w.B - 1, 200], np.int32)
    dev2, flags2 = gpu_append(bad2, k_new, v_new, "f32")
    assert flags2 & va.VA_FLAG_BAD_CTX
