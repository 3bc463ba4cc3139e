"""Pins for the fp64 oracle: it is checked against things other than itself.

- an independent numpy brute force (explicit ancestor sets, dense mask),
- torch's fp64 scaled_dot_product_attention with a boolean mask,
- hand-derived closed forms (tests/golden/), exact special cases,
- invariants the definition fixes: split/merge partition independence,
  causal and tree visibility, block-table permutation, GQA replication.
"""

import copy
import json
import math
import os

import numpy as np
import pytest

import oracle
import synthetic as S

from . import _brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _relerr(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


# --------------------------------------------------------------------------
# workloads small enough for the brute force
# --------------------------------------------------------------------------

def w_dense():
    return S.tiny_dense()  # fp32 K/V, the shape of the tiny dense verify case


def w_dense_f16():
    return S.tiny_dense(kv_dtype="f16")


def w_paged_q8():
    return S.make_workload("pin_paged_q8", ctx_lens=[5, 37, 70], B=5, H=4, KVH=2, D=64, q_dtype="bf16",
                           kv_dtype="q8_0", seed=11, permute=True, spare_pages=3, poison=True)


def w_paged_f16_q16():
    return S.make_workload("pin_paged_f16", ctx_lens=[33, 16], B=3, H=6, KVH=2, D=64, q_dtype="f16",
                           kv_dtype="f16", seed=12, permute=True, spare_pages=2, poison=True)


def w_tree():
    rng = np.random.default_rng(99)
    par = np.stack([S.tree_parent(2, 6, rng), S.tree_parent(2, 6, rng)])
    return S.make_workload("pin_tree", ctx_lens=[45, 8], B=8, H=4, KVH=2, D=32, q_dtype="bf16",
                           kv_dtype="q8_0", seed=13, permute=True, spare_pages=1, poison=True, parent=par)


ALL = [w_dense, w_dense_f16, w_paged_q8, w_paged_f16_q16, w_tree]


@pytest.mark.parametrize("make", ALL, ids=lambda f: f.__name__)
def test_oracle_matches_bruteforce(make):
    w = make()
    o, l = oracle.attention(w)
    bo, bl = _brute.attention(w)
    assert np.all(np.isfinite(o))
    assert _relerr(o, bo) <= 1e-12
    assert np.abs(l - bl).max() <= 1e-12 * max(1.0, np.abs(bl).max())


@pytest.mark.parametrize("make", [w_dense, w_paged_q8, w_tree], ids=lambda f: f.__name__)
def test_oracle_matches_torch_sdpa(make):
    torch = pytest.importorskip("torch")
    w = make()
    o, _ = oracle.attention(w)
    Q = _brute.decode_q(w).reshape(w.num_seqs, w.B, w.H, w.D)
    G = w.H // w.KVH
    for s in range(w.num_seqs):
        K, V = _brute.gather_kv(w, s)
        vis = _brute.visibility(w, s)
        q = torch.from_numpy(np.ascontiguousarray(Q[s].transpose(1, 0, 2)))           # [H, B, D]
        k = torch.from_numpy(np.ascontiguousarray(np.repeat(K.transpose(1, 0, 2), G, 0)))  # [H, ctx, D]
        v = torch.from_numpy(np.ascontiguousarray(np.repeat(V.transpose(1, 0, 2), G, 0)))
        mask = torch.from_numpy(vis)[None].expand(w.H, -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=w.scale)
        got = o.reshape(w.num_seqs, w.B, w.H, w.D)[s].transpose(1, 0, 2)
        assert _relerr(got, ref.numpy()) <= 1e-12


# --------------------------------------------------------------------------
# split form + merge
# --------------------------------------------------------------------------

def _random_bounds(w, S_, rng):
    b = np.zeros((w.num_seqs, S_ + 1), np.int32)
    for s in range(w.num_seqs):
        ctx = int(w.ctx_lens[s])
        cuts = np.sort(rng.integers(0, ctx + 1, S_ - 1))
        b[s, 1:S_] = cuts
        b[s, S_] = ctx
    return b


@pytest.mark.parametrize("make", [w_dense, w_paged_q8, w_tree], ids=lambda f: f.__name__)
@pytest.mark.parametrize("S_", [1, 2, 5, 16])
def test_merge_of_any_partition_equals_direct(make, S_):
    w = make()
    o, l = oracle.attention(w)
    rng = np.random.default_rng(S_)
    for trial in range(3):
        b = _random_bounds(w, S_, rng)
        m, ll, oo = oracle.split_partials(w, b)
        mo, ml = oracle.merge(m, ll, oo)
        if S_ == 1:
            # one split is the direct path itself: weight exp(0) = 1, the same
            # sums in the same order, so the merge reproduces it bit for bit
            assert np.array_equal(mo.reshape(o.shape), o)
            assert np.array_equal(ml.reshape(l.shape), l)
        assert _relerr(mo.reshape(o.shape), o) <= 1e-12
        assert np.abs(ml.reshape(l.shape) - l).max() <= 1e-12 * max(1.0, np.abs(l).max())


def test_partition_with_empty_and_one_key_splits():
    w = w_dense()
    ctx = int(w.ctx_lens[0])
    b = np.array([[0, 0, 1, 1, 2, 100, 100, ctx, ctx]], np.int32)  # empty, 1-key, empty, 1-key, ... splits
    m, ll, oo = oracle.split_partials(w, b)
    assert np.all(ll[0] == 0) and np.all(np.isneginf(m[0]))  # empty split: m=-inf, l=0
    mo, _ = oracle.merge(m, ll, oo)
    o, _ = oracle.attention(w)
    assert _relerr(mo.reshape(o.shape), o) <= 1e-12


def test_every_key_its_own_split():
    w = w_paged_f16_q16()
    S_ = int(w.ctx_lens.max())
    b = np.zeros((w.num_seqs, S_ + 1), np.int32)
    for s in range(w.num_seqs):
        c = int(w.ctx_lens[s])
        b[s, : c + 1] = np.arange(c + 1)
        b[s, c + 1:] = c
    m, ll, oo = oracle.split_partials(w, b)
    mo, _ = oracle.merge(m, ll, oo)
    o, _ = oracle.attention(w)
    assert _relerr(mo.reshape(o.shape), o) <= 1e-12


# --------------------------------------------------------------------------
# visibility invariants
# --------------------------------------------------------------------------

def _token_loc(w, s, j):
    return int(w.block_table[s, j // S.PAGE]), j % S.PAGE


def _perturb_token(w, s, j, rng):
    w = copy.deepcopy(w)
    page, slot = _token_loc(w, s, j)
    if w.kv_dtype == "q8_0":
        w.k_pool[page, :, slot, :] = rng.integers(-127, 128, w.k_pool[page, :, slot, :].shape)
        w.v_pool[page, :, :, slot] = rng.integers(-127, 128, w.v_pool[page, :, :, slot].shape)
        w.k_scale[page, :, slot, :] = np.float16(3.0)
        w.v_scale[page, :, :, slot] = np.float16(-2.0)
    else:
        w.k_pool[page, :, slot, :] = rng.standard_normal(w.k_pool[page, :, slot, :].shape) * 5
        w.v_pool[page, :, :, slot] = rng.standard_normal(w.v_pool[page, :, :, slot].shape) * 5
    return w


@pytest.mark.parametrize("make", [w_dense, w_paged_q8], ids=lambda f: f.__name__)
def test_causal_rows_ignore_later_keys(make):
    w = make()
    rng = np.random.default_rng(5)
    o, _ = oracle.attention(w)
    o = o.reshape(w.num_seqs, w.B, w.H, w.D)
    for s in range(w.num_seqs):
        base = int(w.ctx_lens[s]) - w.B
        for k in range(w.B):  # perturb the slot of drafted row k
            w2 = _perturb_token(w, s, base + k, rng)
            o2, _ = oracle.attention(w2)
            o2 = o2.reshape(o.shape)
            assert np.array_equal(o2[s, :k], o[s, :k])          # earlier rows: bitwise unchanged
            assert not np.array_equal(o2[s, k:], o[s, k:])      # the row itself and later rows see it
            others = [t for t in range(w.num_seqs) if t != s]
            assert np.array_equal(o2[others], o[others])


def test_chain_parent_equals_null_bitwise():
    w = w_paged_q8()
    w2 = copy.deepcopy(w)
    w2.parent = np.tile(np.arange(-1, w.B - 1, dtype=np.int32), (w.num_seqs, 1))
    assert np.array_equal(oracle.attention(w)[0], oracle.attention(w2)[0])


def test_tree_rows_ignore_non_ancestors():
    w = w_tree()
    rng = np.random.default_rng(6)
    o, _ = oracle.attention(w)
    o = o.reshape(w.num_seqs, w.B, w.H, w.D)
    for s in range(w.num_seqs):
        base = int(w.ctx_lens[s]) - w.B
        anc = _brute.ancestor_sets(w.parent[s], w.B)
        for a in range(w.B):
            w2 = _perturb_token(w, s, base + a, rng)
            o2 = oracle.attention(w2)[0].reshape(o.shape)
            for i in range(w.B):
                same = np.array_equal(o2[s, i], o[s, i])
                assert same == (a not in anc[i]), (s, a, i)


def test_all_roots_see_prefix_and_self():
    w = w_tree()
    w.parent = np.full((w.num_seqs, w.B), -1, np.int32)
    o, _ = oracle.attention(w)
    # brute force with the explicit prefix-plus-self mask
    bo, _ = _brute.attention(w)
    assert _relerr(o, bo) <= 1e-12
    vis = _brute.visibility(w, 0)
    base = int(w.ctx_lens[0]) - w.B
    assert np.array_equal(vis[:, base:], np.eye(w.B, dtype=bool))


# --------------------------------------------------------------------------
# paging and GQA
# --------------------------------------------------------------------------

def _repage(w, perm):
    """Move physical page p to perm[p]; the logical content is unchanged."""
    w2 = copy.deepcopy(w)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm))
    w2.k_pool = w.k_pool[inv]
    w2.v_pool = w.v_pool[inv]
    if w.k_scale is not None:
        w2.k_scale = w.k_scale[inv]
        w2.v_scale = w.v_scale[inv]
    w2.block_table = perm[w.block_table].astype(np.int32)
    return w2


@pytest.mark.parametrize("make", [w_paged_q8, w_paged_f16_q16, w_tree], ids=lambda f: f.__name__)
def test_block_table_permutation_invariance_bitwise(make):
    w = make()
    perm = np.random.default_rng(7).permutation(w.num_pages).astype(np.int32)
    o, l = oracle.attention(w)
    o2, l2 = oracle.attention(_repage(w, perm))
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_identity_table_equals_contiguous_gather():
    w = w_dense()
    K, V = _brute.gather_kv(w, 0)
    # contiguous pool: page p holds tokens 16p..16p+15 in order
    assert np.array_equal(w.block_table[0, : w.num_pages], np.arange(w.num_pages))
    Kc = w.k_pool.transpose(0, 2, 1, 3).reshape(-1, w.KVH, w.D)
    assert np.array_equal(K, Kc.astype(np.float64))


def test_gqa_replication_equals_mha_bitwise():
    w = w_paged_q8()
    G = w.H // w.KVH
    w2 = copy.deepcopy(w)
    rep = np.repeat(np.arange(w.KVH), G)
    w2.KVH = w.H
    w2.k_pool = np.ascontiguousarray(w.k_pool[:, rep])
    w2.v_pool = np.ascontiguousarray(w.v_pool[:, rep])
    w2.k_scale = np.ascontiguousarray(w.k_scale[:, rep])
    w2.v_scale = np.ascontiguousarray(w.v_scale[:, rep])
    assert np.array_equal(oracle.attention(w)[0], oracle.attention(w2)[0])


# --------------------------------------------------------------------------
# closed forms and golden fixtures
# --------------------------------------------------------------------------

def _single_page_f32(D, ctx, B, q, K, V, scale=1.0):
    w = S.make_workload("closed", ctx_lens=[ctx], B=B, H=1, KVH=1, D=D, q_dtype="f32", kv_dtype="f32",
                        seed=0, scale=scale)
    w.q[...] = np.asarray(q, np.float32).reshape(w.q.shape)
    for j in range(ctx):
        page, slot = _token_loc(w, 0, j)
        w.k_pool[page, 0, slot, :] = K[j]
        w.v_pool[page, 0, :, slot] = V[j]
    return w


def test_golden_q8_single_key():
    g = json.load(open(os.path.join(GOLD, "q8_single_key.json")))
    D = g["D"]
    w = S.make_workload("gold_q8", ctx_lens=[1], B=1, H=1, KVH=1, D=D, q_dtype="f32", kv_dtype="q8_0",
                        seed=0, scale=g["softmax_scale"])
    w.q[...] = 1.0
    w.k_pool[0, 0, 0, :] = np.asarray(g["k_int8"], np.int8)
    w.v_pool[0, 0, :, 0] = np.asarray(g["v_int8"], np.int8)
    w.k_scale[0, 0, 0, :] = np.uint16(g["scale_f16_bits"]).view(np.float16)
    w.v_scale[0, 0, :, 0] = np.uint16(g["scale_f16_bits"]).view(np.float16)
    o, l = oracle.attention(w)
    assert np.array_equal(o[0, 0], np.asarray(g["expected_out"]))
    assert l[0, 0] == g["expected_lse"]


def test_golden_two_key_logistic():
    g = json.load(open(os.path.join(GOLD, "two_key_logistic.json")))
    D = g["D"]
    e = np.eye(D)
    w = _single_page_f32(D, 2, 1, g["a"] * e[0], [e[0], np.zeros(D)], [e[0], e[1]], scale=g["softmax_scale"])
    o, l = oracle.attention(w)
    assert abs(o[0, 0, 0] - g["expected_out_dim0"]) <= 1e-15
    assert abs(o[0, 0, 1] - g["expected_out_dim1"]) <= 1e-15
    assert np.all(o[0, 0, 2:] == 0)
    assert abs(l[0, 0] - g["expected_lse"]) <= 1e-15


def test_zero_query_gives_mean_of_visible_values():
    w = w_tree()
    w.q[...] = 0  # bf16 bits 0 == +0.0
    o, l = oracle.attention(w)
    o = o.reshape(w.num_seqs, w.B, w.H, w.D)
    G = w.H // w.KVH
    for s in range(w.num_seqs):
        _, V = _brute.gather_kv(w, s)
        vis = _brute.visibility(w, s)
        for i in range(w.B):
            for h in range(w.H):
                mean = V[vis[i], h // G, :].mean(axis=0)
                assert np.abs(o[s, i, h] - mean).max() <= 1e-13
                assert abs(l.reshape(w.num_seqs, w.B, w.H)[s, i, h] - math.log(vis[i].sum())) <= 1e-13


def test_constant_values_give_that_constant():
    w = w_dense()
    w.v_pool[...] = np.float32(0.375)
    o, _ = oracle.attention(w)
    assert np.abs(o - 0.375).max() <= 1e-15


def test_dominant_key_selects_its_value():
    D = 32
    rng = np.random.default_rng(8)
    K = rng.standard_normal((20, D))
    V = rng.standard_normal((20, D))
    K[7] = 0
    K[7, 0] = 200.0  # score 200 vs O(5) for the rest
    q = np.zeros(D)
    q[0] = 1.0
    w = _single_page_f32(D, 20, 4, np.tile(q, 4), K, V)
    o, _ = oracle.attention(w)
    assert np.abs(o[:, 0, :] - V[7].astype(np.float32)).max() <= 1e-12


def test_single_visible_key_returns_it():
    D = 64
    rng = np.random.default_rng(9)
    K = rng.standard_normal((1, D))
    V = rng.standard_normal((1, D))
    w = _single_page_f32(D, 1, 1, rng.standard_normal(D), K, V, scale=0.125)
    o, l = oracle.attention(w)
    assert np.array_equal(o[0, 0], V[0].astype(np.float32).astype(np.float64))
    z = 0.125 * np.dot(w.q[0, 0].astype(np.float64), K[0].astype(np.float32).astype(np.float64))
    assert abs(l[0, 0] - z) <= 1e-13


# --------------------------------------------------------------------------
# the oracle rejects malformed metadata
# --------------------------------------------------------------------------

def test_rejects_bad_metadata():
    w = w_tree()
    bad = copy.deepcopy(w)
    bad.ctx_lens = bad.ctx_lens.copy()
    bad.ctx_lens[1] = w.B - 1
    with pytest.raises(oracle.OracleError):
        oracle.attention(bad)
    bad = copy.deepcopy(w)
    bad.parent[0, 3] = 3
    with pytest.raises(oracle.OracleError):
        oracle.attention(bad)
    bad = copy.deepcopy(w)
    bad.block_table[0, 0] = w.num_pages
    with pytest.raises(oracle.OracleError):
        oracle.attention(bad)


# --------------------------------------------------------------------------
# generator sanity (the inputs both sides read)
# --------------------------------------------------------------------------

def test_generator_q8_roundtrip_and_tables():
    w = S.make_workload("gen", ctx_lens=[300, 17], B=4, H=4, KVH=2, D=64, kv_dtype="q8_0", seed=3,
                        permute=True, spare_pages=4)
    rng = np.random.default_rng(3)
    # block table: a bijection onto distinct physical pages
    used = np.concatenate([w.block_table[s, : (int(c) + 15) // 16] for s, c in enumerate(w.ctx_lens)])
    assert len(set(used.tolist())) == len(used)
    assert used.min() >= 0 and used.max() < w.num_pages
    # regenerate the float values the generator drew and check |x - d*q| <= d/2
    rng.standard_normal((w.num_seqs * w.B, w.H, w.D), dtype=np.float32)
    rng.permutation(w.num_pages)
    for s in range(w.num_seqs):
        c = int(w.ctx_lens[s])
        kf = rng.standard_normal((c, w.KVH, w.D), dtype=np.float32)
        rng.standard_normal((c, w.KVH, w.D), dtype=np.float32)
        K, _ = _brute.gather_kv(w, s)
        kd = np.repeat(w.k_scale[w.block_table[s][np.arange(c) // 16], :, np.arange(c) % 16, :]
                       .astype(np.float64), 32, -1)
        assert np.all(np.abs(kf - K) <= kd / 2 + 1e-12 * np.abs(kf))
    par = S.tree_parent(2, 8, np.random.default_rng(1))
    assert all(-1 <= par[i] < i for i in range(len(par)))


# --------------------------------------------------------------------------
# 16-bit decoders (every fp16 Q value, fp16 K/V value and 8-bit block scale
# passes through the oracle's fp16 decoder; bf16 Q through its bf16 decoder)
# --------------------------------------------------------------------------

def test_fp16_decode_every_bit_pattern():
    """All 65,536 binary16 patterns against numpy's float16 -> float64
    conversion: zeros of both signs, every subnormal, normals, infinities
    and NaNs."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_f16(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))  # -0.0 stays -0.0
    # the subnormal range in closed form: pattern m (1 <= m < 1024) is m * 2^-24
    m = np.arange(1, 1024)
    assert np.array_equal(got[m], m * 2.0 ** -24)
    assert np.array_equal(got[0x8000 + m], -m * 2.0 ** -24)
    assert got[0x7C00] == np.inf and got[0xFC00] == -np.inf


def test_bf16_decode_every_bit_pattern():
    """All 65,536 bfloat16 patterns against torch's bfloat16 -> float64
    conversion."""
    torch = pytest.importorskip("torch")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_q8_decode_with_subnormal_and_extreme_scales():
    """A one-key 8-bit context whose block scales are fp16 subnormals, the
    smallest normal and the largest finite value: with Q = e_d (a one-hot
    query) the attention output is that key's V, and the one-key score is
    the decoded K element; both must equal scale * code in closed form."""
    scales = np.array([1, 0x3FF, 0x400, 0x7BFF, 0x0001, 0x3C00, 0x8001, 0x5BFF], np.uint16)  # fp16 bit patterns
    codes = np.array([127, -127, 1, -1, 64, -128, 3, 100], np.int8)
    D = 256
    w = S.make_workload("one_key", ctx_lens=[1], B=1, H=1, KVH=1, D=D, q_dtype="f32", kv_dtype="q8_0", seed=0)
    w.k_pool[...] = 0
    w.v_pool[...] = 0
    w.k_scale[...] = np.float16(0)
    for b in range(D // 32):
        w.k_pool[0, 0, 0, 32 * b] = codes[b]
        w.k_scale[0, 0, 0, b] = scales[b:b + 1].view(np.float16)[0]
        w.v_pool[0, 0, 32 * b + 5, 0] = codes[b]
        w.v_scale[0, 0, b, 0] = scales[b:b + 1].view(np.float16)[0]
    exact = scales.view(np.float16).astype(np.float64) * codes.astype(np.float64)
    o, lse = oracle.attention(w)
    # one visible key: weight 1, output = V of that key
    v = np.zeros(D)
    v[32 * np.arange(D // 32) + 5] = exact
    assert np.array_equal(o.reshape(D), v)
    # the score of the single key is the lse: scale * sum_d q_d k_d, q one-hot on dim 32 b
    for b in range(D // 32):
        w.q[...] = 0
        w.q[0, 0, 32 * b] = 1.0
        o, lse = oracle.attention(w)
        assert lse.reshape(())[()] == np.float64(np.float32(w.scale)) * exact[b]
