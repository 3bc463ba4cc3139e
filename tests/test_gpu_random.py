"""Seeded random sweep of GPU parity against the fp64 oracle.

Each case draws a shape (head_dim, query / KV heads, rows per sequence,
sequences, contexts), the dtypes (Q, KV, output), the mask (chain, tree or
none), a permuted page table with spare and poisoned pages, uniform or ragged
rows (ragged: empty sequences and prefill segments past 64 rows included) and
the split count (plan's choice, direct, or 2..40).  The definition they are
checked against is the one on the page "perf(gfx1100): speed up long-context
DFlash verify 13.4% with FA2 split-KV and retain HipGraph/Redline PM4"
(Performance, batch-16 kernel screen: partials merged by log-sum-exp) and the
tree / positional rules of "perf(qwen35): retain speculation during paged
prefill" (Mechanism); expected values come from the oracle only.
"""

import numpy as np
import pytest

import oracle
import synthetic as S

from .gpu_util import check_bf16_twin, check_parity, ensure_lib, run_gpu, say
from .test_gpu_ragged import run_ragged

pytestmark = pytest.mark.gpu

N_CASES = 96


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def draw_case(seed):
    rng = np.random.default_rng(9000 + seed)
    D = int(rng.choice([64, 128, 256]))
    H, KVH = [(4, 2), (8, 1), (24, 4), (6, 6), (12, 4)][int(rng.integers(0, 5))]
    kv = str(rng.choice(["f16", "q8_0"]))
    q = str(rng.choice(["f32", "bf16", "f16"]))
    out = str(rng.choice(["f16", "bf16", "f32"]))
    nseq = int(rng.integers(1, 4))
    ragged = rng.random() < 0.3
    kw = dict(H=H, KVH=KVH, D=D, q_dtype=q, kv_dtype=kv, out_dtype=out, seed=seed, permute=True,
              spare_pages=int(rng.integers(0, 5)), poison=bool(rng.random() < 0.5))
    if ragged:
        rows = [int(rng.choice([0, int(rng.integers(1, 9)), int(rng.integers(9, 100))])) for _ in range(nseq)]
        ctx = [int(rng.integers(max(r, 1), 2500)) for r in rows]
        par = [S.chain_parent(r) for r in rows]
        # a tree on one short sequence
        for s, r in enumerate(rows):
            if 3 <= r <= 64 and rng.random() < 0.5:
                par[s] = S.tree_parent(1, r - 1, rng)
                break
        w = S.make_workload(f"rand{seed}", ctx_lens=ctx, rows=rows, parent=np.concatenate(par), **kw)
    else:
        B = int(rng.integers(1, 33))
        ctx = [int(rng.integers(B, 2500)) for _ in range(nseq)]
        mask = rng.integers(0, 3)
        parent = None if mask == 0 else S.chain_parent(B) if mask == 1 else S.tree_parent(min(B, 2), B - min(B, 2), rng)
        w = S.make_workload(f"rand{seed}", ctx_lens=ctx, B=B, parent=parent, **kw)
    splits = int(rng.choice([0, 1, int(rng.integers(2, 41))]))
    return w, splits, ragged


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_case(seed):
    w, splits, ragged = draw_case(seed)
    rows = w.cu_rows.tolist() if ragged else [w.B] * w.num_seqs
    say(f"[case] seed={seed} D={w.D} H={w.H}/{w.KVH} q={w.q_dtype} kv={w.kv_dtype} out={w.out_dtype} "
        f"rows={rows} ctx={w.ctx_lens.tolist()} parent={'none' if w.parent is None else 'given'} S={splits}")
    ref, lref = oracle.attention(w)
    if ragged and w.total_rows == 0:
        # every sequence empty: the buffers still have the plan's capacity
        # (one row; the host cannot see the device's row counts)
        import torch

        qdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.q_dtype]
        q1 = torch.zeros((1, w.H, w.D), dtype=qdt, device="cuda")
        par1 = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        got, lse, flags, _ = run_ragged(w, splits, w.out_dtype, q=q1, parent=par1)
        got, lse = got[:0], lse[:0]
    elif ragged:
        got, lse, flags, _ = run_ragged(w, splits, w.out_dtype)
        n = w.total_rows
        got, lse = got[:n], lse[:n]
    else:
        got, lse, flags, _ = run_gpu(w, splits, w.out_dtype)
    assert flags == 0
    if got.size == 0:
        return  # no rows in the batch: nothing to compare, and no flag raised
    if w.out_dtype == "bf16":
        # the same call with fp32 output: it passes the gate, and the bf16
        # output is its round-to-nearest-even
        if ragged:
            twin = run_ragged(w, splits, "f32")[0][:w.total_rows]
        else:
            twin = run_gpu(w, splits, "f32")[0]
        check_bf16_twin(got, twin, ref, f"random seed {seed}")
    else:
        check_parity(got, ref, w.out_dtype, f"random seed {seed}")
    assert np.abs(lse - lref).max() <= 2e-3
