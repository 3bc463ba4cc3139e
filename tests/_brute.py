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


def visibility(w, s: int) -> np.ndarray:
    ctx = int(w.ctx_lens[s])
    base = ctx - w.B
    anc = ancestor_sets(None if w.parent is None else w.parent[s], w.B)
    vis = np.zeros((w.B, ctx), bool)
    vis[:, :base] = True
    for i in range(w.B):
        for a in anc[i]:
            vis[i, base + a] = True
    return vis


def attention(w):
    Q = decode_q(w).reshape(w.num_seqs, w.B, w.H, w.D)
    G = w.H // w.KVH
    out = np.zeros((w.num_seqs, w.B, w.H, w.D))
    lse = np.zeros((w.num_seqs, w.B, w.H))
    for s in range(w.num_seqs):
        K, V = gather_kv(w, s)
        vis = visibility(w, s)
        for h in range(w.H):
            g = h // G
            z = w.scale * (Q[s, :, h, :] @ K[:, g, :].T)          # [B, ctx]
            z = np.where(vis, z, -np.inf)
            M = z.max(axis=1, keepdims=True)
            e = np.exp(z - M)
            L = e.sum(axis=1, keepdims=True)
            out[s, :, h, :] = (e @ V[:, g, :]) / L
            lse[s, :, h] = (M + np.log(L))[:, 0]
    return out.reshape(w.num_seqs * w.B, w.H, w.D), lse.reshape(w.num_seqs * w.B, w.H)
