"""Seeded workload builders for verify attention.

Every array here is synthetic: N(0,1) values drawn from numpy's PCG64 stream
for a given seed, shaped like the pages' verify workloads (Qwen-style GQA
with 24 query heads over 4 KV heads of width 256, B drafted rows per
sequence, 16-token pages, contexts from 256 to 40,000 tokens).  The pages
measure on real long-context prompts; these arrays stand in for them and
take only their shapes.

Memory layouts produced (all C-contiguous):

  q         [num_seqs*B, H, D]            float32 | float16 | bf16 bits (uint16)
                                          ([total_rows, H, D] with ragged rows)
  k_pool    [num_pages, KVH, 16, D]       token-major rows
  v_pool    [num_pages, KVH, D, 16]       dim-major (the 16 tokens of a page are
                                          contiguous for each dimension)
  k_scale   [num_pages, KVH, 16, D/32]    float16, 8-bit pools only
  v_scale   [num_pages, KVH, D/32, 16]    float16, 8-bit pools only
  block_table [num_seqs, max_pages]       int32
  ctx_lens  [num_seqs]                    int32, counts every valid token,
                                          including the B drafted rows
  parent    [num_seqs, B] int32 or None   -1 <= parent[i] < i
                                          ([total_rows] with ragged rows)
  cu_rows   [num_seqs + 1] int32 or None  ragged rows: sequence s owns packed
                                          rows cu_rows[s] .. cu_rows[s+1] - 1,
                                          the last tokens of its context; B is
                                          then the largest per-sequence count

An 8-bit pool stores x ~= d * q with one float16 scale d per 32 consecutive
head_dim indices of one (token, KV head): d = max|x| / 127 (computed in
float32, stored as float16 round-to-nearest-even), q = clamp(round half away
from zero (x / d), -127, 127).  This only prepares inputs; consumers read the
stored (q, d) pairs and never re-quantise.
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

PAGE = 16


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest-even); return the raw bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[np.isnan(x)] = 0x7FC0
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _quantize_blocks(x: np.ndarray):
    """x [..., D] float32 -> (q int8 [..., D], d float16 [..., D/32])."""
    D = x.shape[-1]
    xb = x.reshape(*x.shape[:-1], D // 32, 32).astype(np.float32)
    amax = np.abs(xb).max(axis=-1)
    d16 = (amax / np.float32(127.0)).astype(np.float32).astype(np.float16)
    dd = d16.astype(np.float32)[..., None]
    safe = np.where(dd > 0, dd, np.float32(1.0))
    r = np.where(dd > 0, xb / safe, np.float32(0.0))
    q = np.sign(r) * np.floor(np.abs(r) + np.float32(0.5))
    q = np.clip(q, -127, 127).astype(np.int8)
    return q.reshape(x.shape), d16


@dataclasses.dataclass
class Workload:
    name: str
    num_seqs: int
    B: int
    H: int
    KVH: int
    D: int
    num_pages: int
    max_pages: int
    q_dtype: str           # "f32" | "f16" | "bf16"
    kv_dtype: str          # "f32" | "f16" | "q8_0"
    out_dtype: str         # "f16" | "bf16" | "f32"
    scale: float           # softmax scale as an fp32 value
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    k_scale: Optional[np.ndarray]
    v_scale: Optional[np.ndarray]
    block_table: np.ndarray
    ctx_lens: np.ndarray
    parent: Optional[np.ndarray]
    seed: int = 0
    cu_rows: Optional[np.ndarray] = None

    @property
    def total_rows(self) -> int:
        return self.num_seqs * self.B if self.cu_rows is None else int(self.cu_rows[-1])

    def seq_rows(self, s: int):
        """(first packed row, row count) of sequence s."""
        if self.cu_rows is None:
            return s * self.B, self.B
        return int(self.cu_rows[s]), int(self.cu_rows[s + 1] - self.cu_rows[s])

    @property
    def max_ctx(self) -> int:
        return int(self.ctx_lens.max())

    def kv_bytes_valid(self) -> int:
        """Bytes of K and V (and scales) for every valid token."""
        per_tok_head = 2 * self.D * (1 if self.kv_dtype == "q8_0" else 2 if self.kv_dtype == "f16" else 4)
        if self.kv_dtype == "q8_0":
            per_tok_head += 2 * 2 * (self.D // 32)
        return int(self.ctx_lens.sum()) * self.KVH * per_tok_head


def tree_parent(n_direct: int, n_tree: int, rng: np.random.Generator) -> np.ndarray:
    """Parent array for `n_direct` chained direct rows followed by a draft tree.

    Tree node t draws its in-tree parent uniformly from {-1, ..., t-1}; -1 hangs
    the node on the last direct row, so every tree row sees the whole causal
    prefix including the direct rows.
    """
    B = n_direct + n_tree
    par = np.empty(B, np.int32)
    for i in range(n_direct):
        par[i] = i - 1
    for t in range(n_tree):
        p = int(rng.integers(-1, t)) if t > 0 else -1
        par[n_direct + t] = (n_direct - 1) if p < 0 else (n_direct + p)
    return par


def make_workload(
    name: str,
    *,
    ctx_lens: Sequence[int],
    B: int = 0,
    H: int,
    KVH: int,
    D: int,
    q_dtype: str = "bf16",
    kv_dtype: str = "q8_0",
    out_dtype: str = "f16",
    seed: int = 0,
    permute: bool = False,
    spare_pages: int = 0,
    poison: bool = False,
    parent: Optional[np.ndarray] = None,
    q_gain: float = 1.0,
    scale: Optional[float] = None,
    max_pages: Optional[int] = None,
    rows: Optional[Sequence[int]] = None,
) -> Workload:
    """rows: per-sequence query-row counts (ragged); then B is their maximum
    and parent, when given, is packed per row."""
    rng = np.random.default_rng(seed)
    nseq = len(ctx_lens)
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    cu_rows = None
    if rows is not None:
        n = np.asarray(rows, dtype=np.int32)
        if n.shape != (nseq,) or np.any(n < 0):
            raise ValueError("rows needs one non-negative count per sequence")
        cu_rows = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        B = max(int(n.max()), 1)
        need = n
    else:
        need = np.full(nseq, B)
    if B < 1:
        raise ValueError("B must be at least 1")
    if np.any(ctx < need):
        raise ValueError("every context must hold its query rows")
    if D % 32:
        raise ValueError("head_dim must be a multiple of 32")
    total = nseq * B if cu_rows is None else int(cu_rows[-1])

    qf = (rng.standard_normal((total, H, D), dtype=np.float32) * np.float32(q_gain)).astype(np.float32)
    if q_dtype == "f32":
        q = qf
    elif q_dtype == "f16":
        q = qf.astype(np.float16)
    elif q_dtype == "bf16":
        q = bf16_bits_from_f32(qf)
    else:
        raise ValueError(q_dtype)

    npages_seq = [(int(c) + PAGE - 1) // PAGE for c in ctx]
    used = sum(npages_seq)
    num_pages = used + spare_pages
    if max_pages is None:
        max_pages = max(npages_seq)
    order = rng.permutation(num_pages).astype(np.int32) if permute else np.arange(num_pages, dtype=np.int32)
    block_table = np.zeros((nseq, max_pages), np.int32)
    off = 0
    for s in range(nseq):
        block_table[s, : npages_seq[s]] = order[off : off + npages_seq[s]]
        off += npages_seq[s]

    q8 = kv_dtype == "q8_0"
    if q8:
        k_pool = np.zeros((num_pages, KVH, PAGE, D), np.int8)
        v_pool = np.zeros((num_pages, KVH, D, PAGE), np.int8)
        k_scale = np.zeros((num_pages, KVH, PAGE, D // 32), np.float16)
        v_scale = np.zeros((num_pages, KVH, D // 32, PAGE), np.float16)
    else:
        npdt = {"f16": np.float16, "f32": np.float32}[kv_dtype]
        k_pool = np.zeros((num_pages, KVH, PAGE, D), npdt)
        v_pool = np.zeros((num_pages, KVH, D, PAGE), npdt)
        k_scale = v_scale = None

    if poison:
        # Fill everything with garbage bytes and NaN scales / values first; the
        # valid tokens are written over it below, so only slots that hold no
        # token (page tails, spare pages) keep the poison.
        if q8:
            k_pool[...] = rng.integers(-127, 128, k_pool.shape, dtype=np.int8)
            v_pool[...] = rng.integers(-127, 128, v_pool.shape, dtype=np.int8)
            k_scale[...] = np.float16(np.nan)
            v_scale[...] = np.float16(np.nan)
        else:
            k_pool[...] = np.nan
            v_pool[...] = np.nan

    for s in range(nseq):
        c = int(ctx[s])
        kf = rng.standard_normal((c, KVH, D), dtype=np.float32)
        vf = rng.standard_normal((c, KVH, D), dtype=np.float32)
        tok = np.arange(c)
        pg = block_table[s, tok // PAGE]
        sl = tok % PAGE
        if q8:
            kq, kd = _quantize_blocks(kf)
            vq, vd = _quantize_blocks(vf)
            k_pool[pg, :, sl, :] = kq
            k_scale[pg, :, sl, :] = kd
            # dim-major V page: [page, kvh, dim, slot]
            v_pool[pg[:, None], np.arange(KVH)[None, :], :, sl[:, None]] = vq
            v_scale[pg[:, None], np.arange(KVH)[None, :], :, sl[:, None]] = vd
        else:
            npdt = k_pool.dtype
            k_pool[pg, :, sl, :] = kf.astype(npdt)
            v_pool[pg[:, None], np.arange(KVH)[None, :], :, sl[:, None]] = vf.astype(npdt)

    if parent is not None:
        if cu_rows is None:
            parent = np.ascontiguousarray(np.broadcast_to(np.asarray(parent, np.int32), (nseq, B)))
        else:
            parent = np.ascontiguousarray(np.asarray(parent, np.int32).reshape(total))
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    return Workload(
        name=name, num_seqs=nseq, B=B, H=H, KVH=KVH, D=D, num_pages=num_pages,
        max_pages=max_pages, q_dtype=q_dtype, kv_dtype=kv_dtype, out_dtype=out_dtype,
        scale=float(np.float32(scale)), q=q, k_pool=k_pool, v_pool=v_pool,
        k_scale=k_scale, v_scale=v_scale, block_table=block_table, ctx_lens=ctx,
        parent=parent, seed=seed, cu_rows=cu_rows,
    )


# ---------------------------------------------------------------------------
# Named workloads (shapes of the pages' verify traffic)
# ---------------------------------------------------------------------------

def tiny_dense(kv_dtype: str = "f32", seed: int = 0, **kw) -> Workload:
    """1 sequence, B=4 rows at ctx-4..ctx-1, 2 query heads over 1 KV head,
    head_dim 64, ctx 256, fp32 Q, causal, contiguous pages."""
    return make_workload("tiny_dense_b4_h2_kv1_d64_ctx256", ctx_lens=[256], B=4, H=2, KVH=1, D=64,
                         q_dtype="f32", kv_dtype=kv_dtype, seed=seed, **kw)


def qwen_dense(ctx: int = 8192, D: int = 256, seed: int = 1, **kw) -> Workload:
    """1 sequence, B=16, 24/4 heads, bf16 Q, fp16 K/V, contiguous pages."""
    return make_workload(f"qwen_dense_b16_h24_kv4_d{D}_f16kv_ctx{ctx}", ctx_lens=[ctx], B=16, H=24, KVH=4,
                         D=D, q_dtype="bf16", kv_dtype="f16", seed=seed, **kw)


def q8_long(ctx: int = 32768, seed: int = 2, permute: bool = False, **kw) -> Workload:
    """1 sequence, B=16, 24/4 heads, D=256, bf16 Q, 8-bit K/V."""
    tag = "_perm" if permute else ""
    return make_workload(f"q8_b16_h24_kv4_d256_ctx{ctx}{tag}", ctx_lens=[ctx], B=16, H=24, KVH=4, D=256,
                         q_dtype="bf16", kv_dtype="q8_0", seed=seed, permute=permute, **kw)


def paged_ragged(ctxs: Sequence[int] = (1016, 1024, 1032, 40000), seed: int = 3, **kw) -> Workload:
    """4 sequences x B=16 in one shared, permuted pool of 16-token pages with
    NaN-poisoned tail slots and spare pages."""
    kw.setdefault("spare_pages", 37)
    kw.setdefault("poison", True)
    return make_workload("paged_ragged_b16_h24_kv4_d256_q8_" + "_".join(map(str, ctxs)), ctx_lens=list(ctxs),
                         B=16, H=24, KVH=4, D=256, q_dtype="bf16", kv_dtype="q8_0", seed=seed,
                         permute=True, **kw)


def tree_mixed(ctx: int = 20676, seed: int = 4, n_direct: int = 2, n_tree: int = 8, **kw) -> Workload:
    """1 sequence: 2 direct causal rows + a width-8 draft tree (seeded parents),
    24/4 heads, D=256, 8-bit paged permuted pool."""
    rng = np.random.default_rng(seed + 1000)
    par = tree_parent(n_direct, n_tree, rng)
    kw.setdefault("poison", True)
    kw.setdefault("spare_pages", 5)
    return make_workload(f"tree_mixed_{n_direct}d{n_tree}t_h24_kv4_d256_q8_ctx{ctx}", ctx_lens=[ctx],
                         B=n_direct + n_tree, H=24, KVH=4, D=256, q_dtype="bf16", kv_dtype="q8_0",
                         seed=seed, permute=True, parent=par, **kw)


def chain(B: int, ctx: int = 20676, seed: int = 4, **kw) -> Workload:
    """1 sequence of B sequential (chain) draft rows, 24/4 heads, D=256, 8-bit paged permuted pool."""
    kw.setdefault("poison", True)
    return make_workload(f"chain_b{B}_h24_kv4_d256_q8_ctx{ctx}", ctx_lens=[ctx], B=B, H=24, KVH=4, D=256,
                         q_dtype="bf16", kv_dtype="q8_0", seed=seed, permute=True, **kw)


def chain_parent(n: int) -> np.ndarray:
    """Parent array of n positioned causal rows (prefill segment or direct rows)."""
    return np.arange(-1, n - 1, dtype=np.int32)


def mixed_lowering(seed: int = 5, prefill=(100, 37), prefill_ctx=(1016, 1032),
                   direct_ctx=(1024, 40000), tree_ctx: int = 20676, n_direct: int = 2, n_tree: int = 8,
                   **kw) -> Workload:
    """One call holding the three row kinds of a mixed step, in order:
    paged ragged prefill segments (chains of `prefill` rows ending at their
    contexts), established decoders with one direct row each, and one
    sequence of n_direct direct rows plus a width-n_tree draft tree.  Contexts
    straddle the 1,024-token (64-page) boundary.  24/4 heads, D=256, 8-bit
    paged KV in one permuted, NaN-poisoned pool; parent packed per row."""
    rng = np.random.default_rng(seed + 2000)
    rows = list(prefill) + [1] * len(direct_ctx) + [n_direct + n_tree]
    ctxs = list(prefill_ctx) + list(direct_ctx) + [tree_ctx]
    par = [chain_parent(n) for n in rows[:-1]] + [tree_parent(n_direct, n_tree, rng)]
    kw.setdefault("poison", True)
    kw.setdefault("spare_pages", 11)
    name = "mixed_prefill{}_direct{}_tree{}+{}_h24_kv4_d256_q8".format(
        "-".join(map(str, prefill)), len(direct_ctx), n_direct, n_tree)
    return make_workload(name, ctx_lens=ctxs, rows=rows, H=24, KVH=4, D=256, q_dtype="bf16",
                         kv_dtype="q8_0", seed=seed, permute=True, parent=np.concatenate(par), **kw)


def _bf16_const(x: float) -> np.uint16:
    return bf16_bits_from_f32(np.array([x], np.float32))[0]


def _set_k_block(w: Workload, tok: np.ndarray, blk: int, dim: int, code: np.ndarray, d: float) -> None:
    """Overwrite 8-bit K block `blk` of the tokens `tok` (positions in
    sequence 0, every KV head): all codes 0 except `dim` (= code) and the
    block scale d (an fp16 value)."""
    pg = w.block_table[0, tok // PAGE]
    sl = tok % PAGE
    lo = 32 * blk
    w.k_pool[pg, :, sl, lo:lo + 32] = 0
    w.k_pool[pg, :, sl, dim] = np.asarray(code, np.int8)[:, None]
    w.k_scale[pg, :, sl, blk] = np.float16(d)


def peaked(ctx: int = 32768, gain: float = 4.0, seed: int = 2, **kw) -> Workload:
    """The 8-bit headline shape with Q scaled by `gain`: scores of standard
    deviation ~gain nats, so a few keys dominate each row and the running max
    of the online softmax is raised throughout the context."""
    return make_workload(f"peaked_g{gain:g}_q8_b16_h24_kv4_d256_ctx{ctx}", ctx_lens=[ctx], B=16, H=24, KVH=4,
                         D=256, q_dtype="bf16", kv_dtype="q8_0", seed=seed, q_gain=gain, **kw)


def rising_max(ctx: int = 32768, slope_log2: float = 0.375, seed: int = 21, **kw) -> Workload:
    """8-bit headline shape whose scores rise along the context by `slope_log2`
    (base-2 units) per token, the same for every row and query head: each
    64-key tile lifts the running max by 64 * slope_log2 (24 at the default),
    so the online softmax rescales its running sum and output over and over,
    with the earlier keys still weighing in.

    Construction (exact in the stored format): every query row has 16 in dims
    0, 32 and 64 and small noise (0.05 N(0,1)) elsewhere; key j gets the
    target score z_j = ln2 * slope_log2 * (j - ctx/2) nats split as
    128 q0 + q1 + q2 / 128 over dims 0, 32, 64 of K blocks 0, 1, 2 with block
    scales 128, 1 and 1/128 (every other code of those blocks is 0), so that
    scale * q.k = z_j + noise.  Blocks 3.. and V are the usual N(0,1) data."""
    w = make_workload(f"rising_max_s{slope_log2:g}_q8_b16_h24_kv4_d256_ctx{ctx}", ctx_lens=[ctx], B=16, H=24,
                      KVH=4, D=256, q_dtype="bf16", kv_dtype="q8_0", seed=seed, permute=True, q_gain=0.05, **kw)
    w.q[:, :, 0] = w.q[:, :, 32] = w.q[:, :, 64] = _bf16_const(16.0)
    j = np.arange(ctx)
    z = math.log(2.0) * slope_log2 * (j - ctx / 2)
    q0 = np.floor(z / 128.0)
    r = z - 128.0 * q0
    q1 = np.floor(r)
    q2 = np.floor((r - q1) * 128.0)
    if np.abs(q0).max() > 127:
        raise ValueError("slope too steep for the 8-bit construction at this context")
    _set_k_block(w, j, 0, 0, q0.astype(np.int8), 128.0)
    _set_k_block(w, j, 1, 32, q1.astype(np.int8), 1.0)
    _set_k_block(w, j, 2, 64, q2.astype(np.int8), 1.0 / 128.0)
    return w


def late_dominant(ctx: int = 32768, margin: float = 13.0, seed: int = 23, **kw) -> Workload:
    """8-bit headline shape with one key near the end of the context (56
    tokens before the drafted rows, so in the last split of any split count
    and visible to every row) whose score exceeds the others by about
    `margin` nats for every row: every query row has 16 in dim 0, and that
    key's K block 0 is zero but for code 127 in dim 0 with scale
    margin / 127 (fp16).  It takes most of each row's weight, and the merge
    must weigh the last split against all earlier ones."""
    w = make_workload(f"late_dominant_q8_b16_h24_kv4_d256_ctx{ctx}", ctx_lens=[ctx], B=16, H=24, KVH=4, D=256,
                      q_dtype="bf16", kv_dtype="q8_0", seed=seed, permute=True, **kw)
    w.q[:, :, 0] = _bf16_const(16.0)
    jd = np.array([ctx - w.B - 40])
    _set_k_block(w, jd, 0, 0, np.array([127], np.int8), float(np.float16(margin / 127.0)))
    return w


def new_kv_rows(w: Workload, dtype: str = "f32", seed: int = 0):
    """K and V vectors for the B drafted rows of every sequence, as a KV append
    receives them: two arrays [num_seqs*B, KVH, D] of N(0,1) values in `dtype`
    ("f32" float32, "f16" float16, "bf16" raw bfloat16 bits as uint16)."""
    rng = np.random.default_rng(seed)
    shape = (w.num_seqs * w.B, w.KVH, w.D)
    out = []
    for _ in range(2):
        x = rng.standard_normal(shape, dtype=np.float32)
        if dtype == "f16":
            x = x.astype(np.float16)
        elif dtype == "bf16":
            x = bf16_bits_from_f32(x)
        out.append(np.ascontiguousarray(x))
    return out[0], out[1]
