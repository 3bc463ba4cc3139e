"""Brute-force fp64 verify attention in numpy, written independently of the oracle.

It decodes the paged pools with numpy fancy indexing (not per-element loops),
materialises a boolean [rows x ctx] visibility matrix from explicitly
collected ancestor *sets*, and runs a dense masked softmax.  Used only to pin
the oracle on tiny inputs.
"""

from __future__ import annotations

import numpy as np

PAGE = 16


def decode_q(w) -> np.ndarray:
    if w.q_dtype == "bf16":
        return (np.asarray(w.q, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(w.q).astype(np.float64)


def gather_kv(w, s: int):
    """Contiguous fp64 K, V for sequence s: [ctx, KVH, D] each."""
    ctx = int(w.ctx_lens[s])
    tok = np.arange(ctx)
    pages = w.block_table[s][tok // PAGE]
    slots = tok % PAGE
    if w.kv_dtype == "q8_0":
        kq = w.k_pool[pages, :, slots, :].astype(np.float64)                      # [ctx, KVH, D]
        kd = w.k_scale[pages, :, slots, :].astype(np.float64)                     # [ctx, KVH, D/32]
        K = kq * np.repeat(kd, 32, axis=-1)
        vq = w.v_pool[pages, :, :, slots].astype(np.float64)                      # [ctx, KVH, D]
        vd = w.v_scale[pages, :, :, slots].astype(np.float64)                     # [ctx, KVH, D/32]
        V = vq * np.repeat(vd, 32, axis=-1)
    else:
        K = w.k_pool[pages, :, slots, :].astype(np.float64)
        V = w.v_pool[pages, :, :, slots].astype(np.float64)
    return K, V


def ancestor_sets(parent_row, B):
    sets = []
    for i in range(B):
        s = {i}
        a = i
        while True:
            a = (a - 1) if parent_row is None else int(parent_row[a])
            if a < 0:
                break
            s.add(a)
        sets.append(s)
    return sets


def rows_of(w, s: int):
    """(first packed row, count) of sequence s, uniform or ragged."""
    cu = getattr(w, "cu_rows", None)
    if cu is None:
        return s * w.B, w.B
    return int(cu[s]), int(cu[s + 1]) - int(cu[s])


def parent_slice(w, s: int):
    if w.parent is None:
        return None
    r0, n = rows_of(w, s)
    return w.parent[s] if getattr(w, "cu_rows", None) is None else w.parent[r0:r0 + n]


def visibility(w, s: int) -> np.ndarray:
    ctx = int(w.ctx_lens[s])
    _, n = rows_of(w, s)
    base = ctx - n
    anc = ancestor_sets(parent_slice(w, s), n)
    vis = np.zeros((n, ctx), bool)
    vis[:, :base] = True
    for i in range(n):
        for a in anc[i]:
            vis[i, base + a] = True
    return vis


def attention(w):
    Q = decode_q(w).reshape(-1, w.H, w.D)
    G = w.H // w.KVH
    out = np.zeros((Q.shape[0], w.H, w.D))
    lse = np.zeros((Q.shape[0], w.H))
    for s in range(w.num_seqs):
        r0, n = rows_of(w, s)
        if n == 0:
            continue
        K, V = gather_kv(w, s)
        vis = visibility(w, s)
        for h in range(w.H):
            g = h // G
            z = w.scale * (Q[r0:r0 + n, h, :] @ K[:, g, :].T)     # [n, ctx]
            z = np.where(vis, z, -np.inf)
            M = z.max(axis=1, keepdims=True)
            e = np.exp(z - M)
            L = e.sum(axis=1, keepdims=True)
            out[r0:r0 + n, h, :] = (e @ V[:, g, :]) / L
            lse[r0:r0 + n, h] = (M + np.log(L))[:, 0]
    return out, lse
