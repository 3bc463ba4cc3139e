"""Pins for the oracle's KV append and 8-bit block quantiser.

The quantiser decides integers, so it is pinned by exact properties of the
format (on-grid values come back exactly, the half-ulp error bound, the code
of the largest entry, sign symmetry, power-of-two scaling, zero and NaN
blocks), by a hand-derived block under tests/golden/, and its fp32 -> fp16
rounding by numpy's own conversion.  The append is pinned by what must and
must not change in the pools."""

from __future__ import annotations

import copy
import json
import os

import numpy as np
import pytest

import oracle
import synthetic as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_f32_to_f16_matches_numpy_rounding():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, size=400_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    # ties and near-ties around every fp16 spacing, subnormals, overflow edge
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    with np.errstate(over="ignore"):
        nxt = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float32)
    mid = (h.astype(np.float64) + nxt.astype(np.float64)) / 2
    extra = np.concatenate([mid.astype(np.float32), np.nextafter(mid.astype(np.float32), 0),
                            np.nextafter(mid.astype(np.float32), np.inf),
                            np.float32([65504, 65519.99, 65520, 1e-8, 2.98e-8, 5.96e-8, 0.0, -0.0, np.inf])])
    x = np.concatenate([x, extra, -extra])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16(x), ref)
    assert np.isnan(oracle.f32_to_f16(np.float32([np.nan])).view(np.float16)[0])


def test_quantise_golden_block():
    g = json.load(open(os.path.join(GOLD, "q8_quantize_block.json")))
    q, d = oracle.quantize_blocks(np.float32(g["x"])[None, :])
    assert int(d[0, 0]) == g["scale_bits"]
    assert q[0].tolist() == g["q"]


def test_quantise_on_grid_values_round_trip_exactly():
    rng = np.random.default_rng(12)
    for _ in range(200):
        e = int(rng.integers(-12, 5))
        d16 = np.float16(np.float32(rng.uniform(1, 2)) * np.float32(2.0 ** e))
        q = rng.integers(-127, 128, size=32)
        q[int(rng.integers(0, 32))] = 127 * (1 if rng.random() < 0.5 else -1)
        x = (np.float32(d16) * q.astype(np.float32)).astype(np.float32)  # exact: 11 x 8 bits
        qq, dd = oracle.quantize_blocks(x[None, :])
        assert dd[0, 0] == np.float16(d16).view(np.uint16)
        assert np.array_equal(qq[0], q.astype(np.int8))


def test_quantise_ties_round_away_from_zero():
    # scale exactly 1/8: the block's largest magnitude is 127/8
    x = np.zeros(32, np.float32)
    x[0] = 127 / 8
    ties = [2.5, -2.5, 0.5, -0.5, 1.5, 126.5, -3.5]
    for j, t in enumerate(ties):
        x[1 + j] = t / 8
    q, d = oracle.quantize_blocks(x[None])
    assert d[0, 0] == np.float16(0.125).view(np.uint16)
    assert q[0, 1:1 + len(ties)].tolist() == [3, -3, 1, -1, 2, 127, -4]


def test_quantise_error_bound_and_largest_code():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((4000, 32)) * rng.uniform(0.01, 20, size=(4000, 1))).astype(np.float32)
    q, d = oracle.quantize_blocks(x)
    dd = d.view(np.float16).astype(np.float64)[:, 0:1]
    err = np.abs(x.astype(np.float64) - dd * q.astype(np.float64))
    assert np.all(err <= 0.5 * dd * (1 + 2.0 ** -10) + 1e-30)
    imax = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(len(x)), imax]) == 127)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)


def test_quantise_sign_symmetry_scaling_zero_and_nan():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((500, 32)).astype(np.float32)
    q, d = oracle.quantize_blocks(x)
    qn, dn = oracle.quantize_blocks(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d)
    for k in (-3, -1, 2, 4):
        qs, ds = oracle.quantize_blocks(x * np.float32(2.0 ** k))
        assert np.array_equal(qs, q)
        assert np.array_equal(ds.view(np.float16).astype(np.float64), d.view(np.float16).astype(np.float64) * 2.0 ** k)
    q0, d0 = oracle.quantize_blocks(np.zeros((1, 32), np.float32))
    assert d0[0, 0] == 0 and not q0.any()
    xn = x[:1].copy()
    xn[0, 5] = np.nan
    qn, dn = oracle.quantize_blocks(xn)
    assert qn[0, 5] == 0
    ref_q, ref_d = oracle.quantize_blocks(np.where(np.isnan(xn), np.float32(0), xn))
    assert dn[0, 0] == ref_d[0, 0] and np.array_equal(np.delete(qn, 5), np.delete(ref_q, 5))


def _append_case(kv_dtype, new_dtype, seed=21):
    w = S.make_workload(f"append_{kv_dtype}", ctx_lens=[40, 17, 300], B=5, H=8, KVH=2, D=64, q_dtype="bf16",
                        kv_dtype=kv_dtype, seed=seed, permute=True, spare_pages=4, poison=True)
    k_new, v_new = S.new_kv_rows(w, new_dtype, seed=seed + 1)
    return w, k_new, v_new


def _rows_f32(a, dtype):
    if dtype == "f32":
        return a.astype(np.float32)
    if dtype == "f16":
        return a.view(np.float16).astype(np.float32)
    return S.bf16_bits_to_f32(a)


def _slot_index(w, s, i):
    t = int(w.ctx_lens[s]) - w.B + i
    return int(w.block_table[s, t // 16]), t % 16


@pytest.mark.parametrize("kv_dtype", ["q8_0", "f16"])
@pytest.mark.parametrize("new_dtype", ["f32", "f16", "bf16"])
def test_append_writes_exactly_the_drafted_slots(kv_dtype, new_dtype):
    w, k_new, v_new = _append_case(kv_dtype, new_dtype)
    k, v, ks, vs = oracle.append_kv(w, k_new, v_new, new_dtype)
    touched = np.zeros((w.num_pages, w.KVH, 16), bool)
    kf, vf = _rows_f32(k_new, new_dtype), _rows_f32(v_new, new_dtype)
    for s in range(w.num_seqs):
        for i in range(w.B):
            page, slot = _slot_index(w, s, i)
            touched[page, :, slot] = True
            for g in range(w.KVH):
                r = s * w.B + i
                if kv_dtype == "f16":
                    assert np.array_equal(k[page, g, slot].view(np.uint16), kf[r, g].astype(np.float16).view(np.uint16))
                    assert np.array_equal(v[page, g, :, slot].view(np.uint16), vf[r, g].astype(np.float16).view(np.uint16))
                else:
                    qk, dk = oracle.quantize_blocks(kf[r, g][None])
                    qv, dv = oracle.quantize_blocks(vf[r, g][None])
                    assert np.array_equal(k[page, g, slot], qk[0]) and np.array_equal(ks[page, g, slot].view(np.uint16), dk[0])
                    assert np.array_equal(v[page, g, :, slot], qv[0]) and np.array_equal(vs[page, g, :, slot].view(np.uint16), dv[0])
                    # dequantised rows stay within half a step of the new values
                    rec = ks[page, g, slot].astype(np.float64).repeat(32) * k[page, g, slot].astype(np.float64)
                    assert np.all(np.abs(rec - kf[r, g]) <= 0.5 * ks[page, g, slot].astype(np.float64).repeat(32) * 1.001 + 1e-30)
    # everything else is bitwise unchanged (poisoned tails and spare pages included)
    keep = ~touched
    assert np.array_equal(k.view(np.uint8).reshape(w.num_pages, w.KVH, 16, -1)[keep],
                          w.k_pool.view(np.uint8).reshape(w.num_pages, w.KVH, 16, -1)[keep])
    vt = v.view(np.uint8).reshape(w.num_pages, w.KVH, w.D, 16, -1).transpose(0, 1, 3, 2, 4)
    vt0 = w.v_pool.view(np.uint8).reshape(w.num_pages, w.KVH, w.D, 16, -1).transpose(0, 1, 3, 2, 4)
    assert np.array_equal(vt[keep], vt0[keep])
    if kv_dtype == "q8_0":
        assert np.array_equal(ks.view(np.uint16)[keep], w.k_scale.view(np.uint16)[keep])
        assert np.array_equal(vs.view(np.uint16).transpose(0, 1, 3, 2)[keep], w.v_scale.view(np.uint16).transpose(0, 1, 3, 2)[keep])


def test_append_rejects_bad_metadata():
    w, k_new, v_new = _append_case("q8_0", "f32")
    bad = copy.deepcopy(w)
    bad.block_table = bad.block_table.copy()
    bad.block_table[0, 1] = w.num_pages
    with pytest.raises(oracle.OracleError):
        oracle.append_kv(bad, k_new, v_new, "f32")
    bad = copy.deepcopy(w)
    bad.ctx_lens = np.array([4, 17, 300], np.int32)
    with pytest.raises(oracle.OracleError):
        oracle.append_kv(bad, k_new, v_new, "f32")
