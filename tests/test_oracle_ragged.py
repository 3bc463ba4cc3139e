"""Pins of the oracle's ragged-row form (one call mixing paged prefill
segments, direct rows and a draft tree).

Source: the page "perf(qwen35): retain speculation during paged prefill",
Mechanism (a step lowers ragged prefill segments, ordinary direct rows and
fixed-width tree rows together; prefill and direct rows are positioned causal
reads, parent metadata covers only the tree) and Correctness failure found
during qualification (direct rows must not change when other rows join the
launch).  Each pin ties the ragged oracle to something other than itself:
the independent numpy brute force, the uniform-row oracle on re-packed or
truncated inputs, or an invariant the definition fixes.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest

import oracle
import synthetic as S
from tests import _brute


def tiny_ragged(kv_dtype="f32", seed=11, rows=(3, 0, 1, 70, 9), ctxs=(100, 50, 33, 200, 150), tree=True,
                **kw):
    """Tiny ragged batch: a chain of 3, an empty sequence, one direct row, a
    70-row prefill chain (past the 64-row ancestry window) and 2 direct rows +
    a 7-node tree; D=64, 4 query heads over 2 KV heads."""
    rng = np.random.default_rng(seed)
    par = [S.chain_parent(n) for n in rows]
    if tree:
        par[-1] = S.tree_parent(2, rows[-1] - 2, rng)
    return S.make_workload("tiny_ragged", ctx_lens=list(ctxs), rows=list(rows), H=4, KVH=2, D=64,
                           q_dtype="f32", kv_dtype=kv_dtype, seed=seed, permute=True, spare_pages=3,
                           parent=np.concatenate(par), **kw)


@pytest.mark.parametrize("kv_dtype", ["f32", "f16", "q8_0"])
def test_ragged_matches_brute_force(kv_dtype):
    w = tiny_ragged(kv_dtype)
    out, lse = oracle.attention(w)
    bo, bl = _brute.attention(w)
    assert out.shape == (w.total_rows, w.H, w.D)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_ragged_without_parent_is_causal():
    # parent == NULL on a ragged call: every sequence is a chain
    w = tiny_ragged(tree=False)
    w_nopar = dataclasses.replace(w, parent=None)
    a, la = oracle.attention(w)
    b, lb = oracle.attention(w_nopar)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)
    bo, _ = _brute.attention(w_nopar)
    np.testing.assert_allclose(b, bo, rtol=0, atol=1e-12)


def test_equal_counts_match_uniform_layout():
    # n_s = B for every s: packed row cu[s] + i is uniform row s*B + i
    w = S.make_workload("u", ctx_lens=[90, 130, 64], B=5, H=4, KVH=2, D=64, q_dtype="f32", kv_dtype="q8_0",
                        seed=4, permute=True, parent=S.tree_parent(1, 4, np.random.default_rng(1)))
    r = dataclasses.replace(w, cu_rows=np.array([0, 5, 10, 15], np.int32), parent=w.parent.reshape(-1).copy())
    a, la = oracle.attention(w)
    b, lb = oracle.attention(r)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def _single_sequence(w, s):
    """Sequence s of a ragged workload alone, as a uniform B = n_s workload."""
    r0, n = w.seq_rows(s)
    par = None if w.parent is None else w.parent[r0:r0 + n][None, :].copy()
    return dataclasses.replace(w, num_seqs=1, B=n, q=w.q[r0:r0 + n].copy(), block_table=w.block_table[s:s + 1].copy(),
                               ctx_lens=w.ctx_lens[s:s + 1].copy(), parent=par, cu_rows=None)


def test_sequences_are_independent():
    # a sequence's rows come out the same whether it runs alone or in the mix
    w = tiny_ragged("q8_0")
    out, lse = oracle.attention(w)
    for s in range(w.num_seqs):
        r0, n = w.seq_rows(s)
        if n == 0:
            continue
        o1, l1 = oracle.attention(_single_sequence(w, s))
        np.testing.assert_array_equal(out[r0:r0 + n], o1)
        np.testing.assert_array_equal(lse[r0:r0 + n], l1)


def test_prefill_row_is_a_decode_row_at_its_position():
    # chain row i of a segment sits at slot p = ctx - n + i and sees [0, p]:
    # exactly a single direct row of the same sequence truncated to p + 1 tokens
    w = tiny_ragged("f16")
    out, lse = oracle.attention(w)
    s = 3
    r0, n = w.seq_rows(s)
    ctx = int(w.ctx_lens[s])
    for i in (0, 1, 37, 63, 64, 65, n - 1):
        p = ctx - n + i
        one = dataclasses.replace(w, num_seqs=1, B=1, q=w.q[r0 + i:r0 + i + 1].copy(),
                                  block_table=w.block_table[s:s + 1].copy(),
                                  ctx_lens=np.array([p + 1], np.int32), parent=None, cu_rows=None)
        o1, l1 = oracle.attention(one)
        np.testing.assert_array_equal(out[r0 + i], o1[0])
        np.testing.assert_array_equal(lse[r0 + i], l1[0])


def test_future_keys_do_not_matter():
    # overwrite K/V of the prefill segment's last 30 slots: rows before them are unchanged
    w = tiny_ragged("f32")
    out, _ = oracle.attention(w)
    s = 3
    r0, n = w.seq_rows(s)
    ctx = int(w.ctx_lens[s])
    k, v = w.k_pool.copy(), w.v_pool.copy()
    for t in range(ctx - 30, ctx):
        pg, sl = w.block_table[s, t // 16], t % 16
        k[pg, :, sl, :] = 1e3
        v[pg, :, :, sl] = -7.0
    out2, _ = oracle.attention(dataclasses.replace(w, k_pool=k, v_pool=v))
    keep = n - 30  # rows at slots < ctx - 30
    np.testing.assert_array_equal(out[r0:r0 + keep], out2[r0:r0 + keep])
    assert not np.allclose(out[r0 + keep:r0 + n], out2[r0 + keep:r0 + n])


@pytest.mark.parametrize("nsplit", [1, 3, 8])
def test_ragged_split_merge_equals_direct(nsplit):
    w = tiny_ragged("q8_0")
    rng = np.random.default_rng(nsplit)
    bounds = np.zeros((w.num_seqs, nsplit + 1), np.int32)
    for s in range(w.num_seqs):
        cuts = np.sort(rng.integers(0, int(w.ctx_lens[s]) + 1, nsplit - 1))
        bounds[s] = np.concatenate([[0], cuts, [w.ctx_lens[s]]])
    m, l, o = oracle.split_partials(w, bounds)
    assert m.shape == (nsplit, w.total_rows * w.H)
    mo, ml = oracle.merge(m, l, o)
    out, lse = oracle.attention(w)
    np.testing.assert_allclose(mo.reshape(out.shape), out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml.reshape(lse.shape), lse, rtol=0, atol=1e-12)


def test_items_address_sequence_local_rows():
    w = tiny_ragged("f32")
    out, lse = oracle.attention(w)
    items = [(3, 69, 3), (4, 8, 0), (2, 0, 1), (0, 2, 2)]
    o, l = oracle.attention_items(w, items)
    for t, (s, i, h) in enumerate(items):
        r0, _ = w.seq_rows(s)
        np.testing.assert_array_equal(o[t], out[r0 + i, h])
        assert l[t] == lse[r0 + i, h]


@pytest.mark.parametrize("bad", ["cu_start", "cu_order", "ctx_short", "parent", "item_row"])
def test_ragged_rejections(bad):
    w = tiny_ragged("f32")
    if bad == "cu_start":
        w = dataclasses.replace(w, cu_rows=w.cu_rows + 1)
    elif bad == "cu_order":
        cu = w.cu_rows.copy()
        cu[2] = cu[1] - 1
        w = dataclasses.replace(w, cu_rows=cu)
    elif bad == "ctx_short":
        c = w.ctx_lens.copy()
        c[3] = 69  # holds fewer than its 70 rows
        w = dataclasses.replace(w, ctx_lens=c)
    elif bad == "parent":
        par = w.parent.copy()
        par[w.cu_rows[4] + 3] = 3  # a row cannot be its own parent
        w = dataclasses.replace(w, parent=par)
    if bad == "item_row":
        with pytest.raises(oracle.OracleError):
            oracle.attention_items(w, [(2, 1, 0)])  # sequence 2 has one row
        return
    with pytest.raises(oracle.OracleError):
        oracle.attention(w)
