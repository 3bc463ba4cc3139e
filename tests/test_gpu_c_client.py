"""The C ABI from plain C: tests/c_abi/verify_c_client (built by
__graft_entry__.build()) plans, allocates, runs verify_attn_run and the
partial + merge pair, reads the flag word and checks two admission errors
through include/verify_attn.h alone, on inputs this test writes from the
seeded generator.  Its output must meet the oracle's gate and equal, bit for
bit, the same call made through the Python binding."""

import os
import struct
import subprocess

import numpy as np
import pytest

import oracle
import speculative_decoding_verify_kv_amd as va
import synthetic as S
from speculative_decoding_verify_kv_amd import device as vdev

from .gpu_util import check_parity, ensure_lib, run_gpu, say

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "verify_c_client")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()
    if not os.path.exists(CLIENT):
        raise RuntimeError("tests/c_abi/verify_c_client is not built (__graft_entry__.build() builds it)")


def _arrays(w):
    def raw(a):
        return b"" if a is None else np.ascontiguousarray(a).tobytes()
    return [raw(w.q), raw(w.k_pool), raw(w.v_pool), raw(w.k_scale), raw(w.v_scale),
            raw(np.asarray(w.block_table, np.int32)), raw(np.asarray(w.ctx_lens, np.int32)),
            raw(None if w.parent is None else np.asarray(w.parent, np.int32))]


@pytest.mark.parametrize("case", ["tree_q8_f16out", "chain_f16kv_f32out", "headline_shape_q8"])
def test_c_client_matches_binding_and_oracle(case, tmp_path):
    if case == "tree_q8_f16out":
        par = S.tree_parent(2, 8, np.random.default_rng(3))
        w = S.make_workload("c_tree", ctx_lens=[1500, 640], B=10, H=24, KVH=4, D=256, q_dtype="bf16",
                            kv_dtype="q8_0", seed=91, permute=True, spare_pages=3, poison=True, parent=par)
        out_dtype, splits = "f16", 0
    elif case == "chain_f16kv_f32out":
        w = S.make_workload("c_chain", ctx_lens=[900, 2100, 333], B=4, H=8, KVH=2, D=128, q_dtype="f32",
                            kv_dtype="f16", seed=92, permute=True)
        out_dtype, splits = "f32", 3
    else:
        w = S.q8_long(ctx=8192, seed=93, permute=True)
        out_dtype, splits = "f16", 0
    say(f"[case] C client {case}")
    prob = vdev.problem_for(w, out_dtype=out_dtype)
    inp = tmp_path / "in.bin"
    outp = tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(b"VACLIENT")
        f.write(bytes(prob))
        f.write(struct.pack("<i", splits))
        for a in _arrays(w):
            f.write(struct.pack("<q", len(a)))
            f.write(a)
    r = subprocess.run([CLIENT, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    data = outp.read_bytes()
    n = struct.unpack_from("<i", data, 0)[0]
    rec = struct.unpack_from(f"<{n}i", data, 4)
    (st_plan, st_info, plan_S, st_short, st_null, st_run, st_flags, flags, st_part, st_merge, st_flags2, flags2,
     msg_len) = rec
    assert st_plan == va.VA_OK and st_info == va.VA_OK and st_run == va.VA_OK
    assert st_short == va.VA_EWORKSPACE and st_null == va.VA_EINVAL
    assert st_part == va.VA_OK and st_merge == va.VA_OK and st_flags == va.VA_OK and st_flags2 == va.VA_OK
    assert flags == 0 and flags2 == 0 and msg_len > 0
    rows = w.num_seqs * w.B
    esz = 4 if out_dtype == "f32" else 2
    ob, lb = rows * w.H * w.D * esz, rows * w.H * 4
    off = 4 + 4 * n
    o1, l1 = data[off:off + ob], data[off + ob:off + ob + lb]
    o2, l2 = data[off + ob + lb:off + 2 * ob + lb], data[off + 2 * ob + lb:off + 2 * ob + 2 * lb]
    assert len(l2) == lb
    ndt = np.float32 if out_dtype == "f32" else np.float16
    got = np.frombuffer(o1, ndt).astype(np.float64).reshape(rows, w.H, w.D)
    got_lse = np.frombuffer(l1, np.float32).astype(np.float64).reshape(rows, w.H)
    # the two-launch form equals the one-call form, bit for bit
    assert o1 == o2 and l1 == l2
    # the same call through the Python binding gives the same bits
    ref_b, ref_b_lse, bflags, info = run_gpu(w, splits, out_dtype)
    assert info.num_splits == plan_S and bflags == 0
    assert np.array_equal(got, ref_b) and np.array_equal(got_lse, ref_b_lse)
    ref, ref_lse = oracle.attention(w)
    check_parity(got, ref, out_dtype, f"C client {case} S={splits or plan_S}")
    assert np.abs(got_lse - ref_lse).max() <= 2e-3
