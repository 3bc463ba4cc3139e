"""Pins for the oracle's accepted-path KV promotion: the accepted rows' bytes
land, in path order, in the slots right after the path's anchor; nothing else
changes; a chain prefix is a no-op; a bad path changes nothing at all."""

from __future__ import annotations

import copy

import numpy as np
import pytest

import oracle
import synthetic as S


def tree_case(kv_dtype="q8_0", seed=31):
    rng = np.random.default_rng(seed)
    par = np.stack([S.tree_parent(2, 8, rng) for _ in range(3)])
    w = S.make_workload("promote", ctx_lens=[40, 300, 1033], B=10, H=8, KVH=2, D=64, q_dtype="bf16",
                        kv_dtype=kv_dtype, seed=seed, permute=True, spare_pages=4, poison=True, parent=par)
    return w


def path_to(par_s, node):
    """Root-first tree path ending at `node` (drafted rows >= 2 are tree rows)."""
    p = [node]
    while par_s[p[-1]] >= 2:
        p.append(int(par_s[p[-1]]))
    return p[::-1]


def slot_bytes(w, k, v, ks, vs, s, t):
    page, slot = int(w.block_table[s, t // 16]), t % 16
    c = np.ascontiguousarray
    parts = [c(k[page, :, slot]).view(np.uint8), c(v[page, :, :, slot]).view(np.uint8)]
    if ks is not None:
        parts += [c(ks[page, :, slot]).view(np.uint8), c(vs[page, :, :, slot]).view(np.uint8)]
    return np.concatenate([x.reshape(-1) for x in parts])


@pytest.mark.parametrize("kv_dtype", ["q8_0", "f16"])
def test_promotion_moves_the_accepted_path(kv_dtype):
    w = tree_case(kv_dtype)
    acc = np.full((w.num_seqs, w.B), -1, np.int32)
    n = np.zeros(w.num_seqs, np.int32)
    for s in range(w.num_seqs):
        path = path_to(w.parent[s], w.B - 1 - s)  # a path to a deep-ish node
        acc[s, :len(path)] = path
        n[s] = len(path)
    k, v, ks, vs, new_ctx = oracle.promote_kv(w, acc, n)
    for s in range(w.num_seqs):
        base = int(w.ctx_lens[s]) - w.B
        dst = base + int(w.parent[s][acc[s, 0]]) + 1
        assert new_ctx[s] == dst + n[s]
        moved = set(range(dst, dst + n[s]))
        for j in range(n[s]):
            src = base + int(acc[s, j])
            assert np.array_equal(slot_bytes(w, k, v, ks, vs, s, dst + j),
                                  slot_bytes(w, w.k_pool, w.v_pool, w.k_scale, w.v_scale, s, src))
        for t in range(int(w.ctx_lens[s])):
            if t not in moved:
                assert np.array_equal(slot_bytes(w, k, v, ks, vs, s, t),
                                      slot_bytes(w, w.k_pool, w.v_pool, w.k_scale, w.v_scale, s, t))


def test_chain_prefix_is_a_no_op():
    w = S.make_workload("promote_chain", ctx_lens=[77, 500], B=6, H=8, KVH=2, D=64, q_dtype="bf16",
                        kv_dtype="q8_0", seed=5, permute=True)
    acc = np.tile(np.arange(6, dtype=np.int32), (2, 1))
    k, v, ks, vs, new_ctx = oracle.promote_kv(w, acc, np.array([4, 6], np.int32))
    assert np.array_equal(k, w.k_pool) and np.array_equal(v, w.v_pool)
    assert np.array_equal(ks.view(np.uint16), w.k_scale.view(np.uint16))
    assert new_ctx.tolist() == [77 - 6 + 4, 500]


def test_overlapping_source_and_destination():
    # direct rows 0, 1; tree rows 2..7 with 3 -> 5 -> 6 a path under row 1
    par = np.array([[-1, 0, 1, 1, 2, 3, 5, 4]], np.int32)
    w = S.make_workload("promote_overlap", ctx_lens=[50], B=8, H=8, KVH=2, D=64, q_dtype="bf16",
                        kv_dtype="q8_0", seed=9, parent=par)
    k, v, ks, vs, new_ctx = oracle.promote_kv(w, np.array([[3, 5, 6, 0, 0, 0, 0, 0]], np.int32),
                                              np.array([3], np.int32))
    base = 50 - 8
    for j, r in enumerate([3, 5, 6]):
        assert np.array_equal(slot_bytes(w, k, v, ks, vs, 0, base + 2 + j),
                              slot_bytes(w, w.k_pool, w.v_pool, w.k_scale, w.v_scale, 0, base + r))
    assert new_ctx[0] == base + 5


def test_bad_path_writes_nothing():
    w = tree_case()
    acc = np.zeros((w.num_seqs, w.B), np.int32)
    n = np.zeros(w.num_seqs, np.int32)
    good = path_to(w.parent[0], w.B - 1)
    acc[0, :len(good)] = good
    n[0] = len(good)
    # sequence 1: two siblings / a non-child step
    acc[1, :2] = [2, 2]
    n[1] = 2
    with pytest.raises(oracle.OracleError):
        oracle.promote_kv(w, acc, n)
    bad = acc.copy()
    bad[1, :2] = [2, w.B]  # out of range
    with pytest.raises(oracle.OracleError):
        oracle.promote_kv(w, bad, n)
