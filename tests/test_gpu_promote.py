"""GPU accepted-path promotion (verify_attn_promote_kv) against the oracle:
pools compared bit for bit (every slot), new_ctx equal, whole-batch rejection
of a bad path, and a verify over the promoted prefix."""

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


def tree_case(kv_dtype="q8_0", D=256, seed=71, ctxs=(40, 300, 1033, 5000)):
    rng = np.random.default_rng(seed)
    par = np.stack([S.tree_parent(2, 8, rng) for _ in ctxs])
    return S.make_workload("promote", ctx_lens=list(ctxs), B=10, H=24, KVH=4, D=D, q_dtype="bf16",
                           kv_dtype=kv_dtype, seed=seed, permute=True, spare_pages=5, poison=True, parent=par)


def path_to(par_s, node):
    p = [node]
    while par_s[p[-1]] >= 2:
        p.append(int(par_s[p[-1]]))
    return p[::-1]


def paths(w, pick):
    acc = np.zeros((w.num_seqs, w.B), np.int32)
    n = np.zeros(w.num_seqs, np.int32)
    for s in range(w.num_seqs):
        pth = pick(s)
        acc[s, :len(pth)] = pth
        n[s] = len(pth)
    return acc, n


def gpu_promote(w, acc, n, ws_out=None):
    dev = vdev.to_device(w)
    plan = va.verify_attn_plan(vdev.problem_for(w), 1, 0)
    wsb = va.verify_attn_promote_workspace_bytes(plan)
    ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
    if ws_out is not None:
        ws_out.append(ws)
    acc_d = torch.from_numpy(np.ascontiguousarray(acc)).cuda()
    n_d = torch.from_numpy(np.ascontiguousarray(n)).cuda()
    new_ctx = torch.full((w.num_seqs,), -7, dtype=torch.int32, device="cuda")
    va.verify_attn_promote_kv(plan, acc_d, n_d, dev["parent"], dev["k_pool"], dev["v_pool"], dev["k_scale"],
                              dev["v_scale"], dev["block_table"], dev["ctx_lens"], new_ctx, ws, wsb)
    torch.cuda.synchronize()
    return dev, new_ctx.cpu().numpy(), va.verify_attn_read_flags(plan, ws)


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy().reshape(-1)


def _same_pools(dev, k, v, ks, vs):
    ok = np.array_equal(_bytes(dev["k_pool"]), k.view(np.uint8).reshape(-1))
    ok &= np.array_equal(_bytes(dev["v_pool"]), v.view(np.uint8).reshape(-1))
    if ks is not None:
        ok &= np.array_equal(_bytes(dev["k_scale"]), ks.view(np.uint8).reshape(-1))
        ok &= np.array_equal(_bytes(dev["v_scale"]), vs.view(np.uint8).reshape(-1))
    return ok


@pytest.mark.parametrize("kv_dtype", ["q8_0", "f16"])
@pytest.mark.parametrize("D", [256, 64])
def test_promote_bitwise(kv_dtype, D):
    say(f"[case] promote kv={kv_dtype} D={D}")
    w = tree_case(kv_dtype, D)
    acc, n = paths(w, lambda s: path_to(w.parent[s], w.B - 1 - (s % 4)))
    k, v, ks, vs, new_ctx = oracle.promote_kv(w, acc, n)
    dev, got_ctx, flags = gpu_promote(w, acc, n)
    assert flags == 0
    assert np.array_equal(got_ctx, new_ctx)
    assert _same_pools(dev, k, v, ks, vs)


def test_promote_empty_and_single_paths():
    say("[case] promote empty / single-node paths")
    w = tree_case("q8_0", 128, seed=3, ctxs=(64, 99))
    acc = np.zeros((2, w.B), np.int32)
    n = np.array([0, 1], np.int32)
    acc[1, 0] = int(np.nonzero(w.parent[1] == 1)[0][0])  # a tree root hanging on the last direct row
    k, v, ks, vs, new_ctx = oracle.promote_kv(w, acc, n)
    dev, got_ctx, flags = gpu_promote(w, acc, n)
    assert flags == 0 and np.array_equal(got_ctx, new_ctx)
    assert _same_pools(dev, k, v, ks, vs)


def test_promote_bad_path_writes_nothing():
    say("[case] promote bad path")
    w = tree_case("q8_0", 128, seed=4, ctxs=(64, 300))
    acc, n = paths(w, lambda s: path_to(w.parent[s], w.B - 1))
    if len(path_to(w.parent[1], w.B - 1)) >= 2:
        acc[1, 1] = acc[1, 0]   # a node repeated: not a parent chain
    else:
        acc[1, 0] = w.B         # out of range
    dev, got_ctx, flags = gpu_promote(w, acc, n)
    assert flags & va.VA_FLAG_BAD_PATH
    assert np.array_equal(got_ctx, w.ctx_lens)
    assert _same_pools(dev, w.k_pool, w.v_pool, w.k_scale, w.v_scale)


def test_promote_then_verify_over_the_promoted_prefix():
    """After promotion the durable prefix [0, new_ctx) holds the accepted
    tokens; a causal verify of its last 4 tokens matches the oracle run on the
    oracle-promoted pools."""
    say("[case] promote then verify")
    w = tree_case("q8_0", 256, seed=8, ctxs=(1033, 5000))
    acc, n = paths(w, lambda s: path_to(w.parent[s], w.B - 1 - s))
    k, v, ks, vs, new_ctx = oracle.promote_kv(w, acc, n)
    dev, got_ctx, flags = gpu_promote(w, acc, n)
    assert flags == 0 and np.array_equal(got_ctx, new_ctx)
    wv = copy.deepcopy(w)
    wv.B, wv.parent = 4, None
    wv.ctx_lens = new_ctx.astype(np.int32)
    wv.q = np.ascontiguousarray(w.q.reshape(w.num_seqs, w.B, w.H, w.D)[:, :4].reshape(-1, w.H, w.D))
    wv.k_pool, wv.v_pool, wv.k_scale, wv.v_scale = k, v, ks, vs
    ref, _ = oracle.attention(wv)
    dv = vdev.to_device(wv)
    for name in ("k_pool", "v_pool", "k_scale", "v_scale"):
        dv[name] = dev[name]
    got = run_gpu(wv, 0, "f32", dev=dv)[0]
    check_parity(got, ref, "f32", "verify after promotion")


# A batch of at most 256 (sequence, path slot) pairs is one launch; a larger
# one is three launches, whose status word (workspace bytes 4..7) records a
# failed check.
ONE_LAUNCH_PAIRS = 256


@pytest.mark.parametrize("nseq", [6, 26])
def test_promote_one_and_three_launch_forms(nseq):
    ctxs = [40 + 37 * i for i in range(nseq)]
    w = tree_case("q8_0", 256, seed=12, ctxs=ctxs)
    one = nseq * w.B <= ONE_LAUNCH_PAIRS
    assert one == (nseq == 6)
    say(f"[case] promote {nseq} sequences, {nseq * w.B} path slots ({'one launch' if one else 'three launches'})")
    acc, n = paths(w, lambda s: path_to(w.parent[s], w.B - 1 - (s % 5)))
    n[3] = 0  # one sequence accepts nothing
    k, v, ks, vs, new_ctx = oracle.promote_kv(w, acc, n)
    dev, got_ctx, flags = gpu_promote(w, acc, n)
    assert flags == 0
    assert np.array_equal(got_ctx, new_ctx)
    assert _same_pools(dev, k, v, ks, vs)
    # a bad path in the last sequence: nothing is written in either form
    acc_bad = acc.copy()
    acc_bad[nseq - 1, 0] = w.B
    wss = []
    dev, got_ctx, flags = gpu_promote(w, acc_bad, n, wss)
    assert flags & va.VA_FLAG_BAD_PATH
    assert np.array_equal(got_ctx, w.ctx_lens)
    assert _same_pools(dev, w.k_pool, w.v_pool, w.k_scale, w.v_scale)
    status = int(wss[0][4:8].cpu().numpy().view(np.uint32)[0])
    assert status == (0 if one else int(va.VA_FLAG_BAD_PATH))


@pytest.mark.parametrize("seed", range(16))
def test_promote_random(seed):
    """Seeded random batches: head_dim 64/128/256, 8-bit or fp16 KV, 4 head
    layouts, B 2-32 rows of direct chain plus draft tree, 1-29 sequences (so
    both the one-launch form, up to 256 (sequence, slot) pairs, and the
    three-launch form run), and per sequence an empty path or the path from
    a random ancestor down to a random row.  Pools bit for bit and new_ctx
    against the oracle."""
    rng = np.random.default_rng(7000 + seed)
    D = int(rng.choice([64, 128, 256]))
    H, KVH = [(4, 2), (8, 1), (24, 4), (6, 6)][int(rng.integers(0, 4))]
    kv = str(rng.choice(["q8_0", "f16"]))
    B = int(rng.integers(2, 33))
    nseq = int(rng.integers(1, 30))
    n_direct = int(rng.integers(0, B))
    ctxs = [int(rng.integers(B, 3000)) for _ in range(nseq)]
    par = np.stack([S.tree_parent(n_direct, B - n_direct, rng) for _ in range(nseq)])
    w = S.make_workload(f"promote_rand{seed}", ctx_lens=ctxs, B=B, H=H, KVH=KVH, D=D, q_dtype="bf16",
                        kv_dtype=kv, seed=7000 + seed, permute=True, spare_pages=3, poison=True, parent=par)
    acc = np.zeros((nseq, B), np.int32)
    n = np.zeros(nseq, np.int32)
    for s in range(nseq):
        if rng.random() < 0.15:
            continue
        chain = [int(rng.integers(0, B))]
        while par[s][chain[-1]] >= 0:
            chain.append(int(par[s][chain[-1]]))
        pth = chain[::-1][int(rng.integers(0, len(chain))):]
        acc[s, :len(pth)] = pth
        n[s] = len(pth)
    say(f"[case] promote random seed={seed} D={D} H={H}/{KVH} kv={kv} B={B} nseq={nseq} pairs={nseq * B} "
        f"n={n.tolist()}")
    k, v, ks, vs, new_ctx = oracle.promote_kv(w, acc, n)
    dev, got_ctx, flags = gpu_promote(w, acc, n)
    assert flags == 0
    assert np.array_equal(got_ctx, new_ctx)
    assert _same_pools(dev, k, v, ks, vs)
