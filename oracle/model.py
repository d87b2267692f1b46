"""Target-model forward over the verify window, fp64 NumPy.  Test infrastructure.

What it computes (CS349E Lecture 6, "Optimizing Autoregressive Decode"):
  * section 6.2 (Leviathan's Algorithm 1, step 2): one target forward yields
    p_1 .. p_{gamma+1}; row i of the window [pending, x_1 .. x_gamma] is fed the
    prefix up to x_i and its logits give the distribution of the next token;
  * section 6.2 (KV handling): the cache holds the confirmed sequence minus its
    last token, so the window sits at positions kv_len .. kv_len + gamma;
  * section 4.2 (selective batching): all sequences' rows are flattened for
    the per-token layers, attention is done per sequence over its own cache;
  * section 10.3 (tree verification): with a token tree each node attends to
    itself and its ancestors only.

Model (a Llama-style dense decoder, the shape the workloads name):
    x = E[token]
    per layer: h = RMSNorm(x) * g1; q, k, v = h Wq^T, h Wk^T, h Wv^T;
               rotary embedding on q and k at the row's absolute position;
               o = softmax(q K^T / sqrt(D) + mask) V over cached rows < kv_len
                   and the allowed suffix rows; query head h reads KV head
                   floor(h / (Hq / Hkv));
               x += o Wo^T;  h = RMSNorm(x) * g2;
               x += (silu(h Wg^T) * (h Wu^T)) Wd^T
    z = RMSNorm(x) * g_f  W_lm^T

Readings where the pages say nothing (each listed in the design notes):
  * RMSNorm eps 1e-5; rotary embedding in rotate-half form pairing dims i and
    i + D/2 with frequency theta^(-2i/D);
  * tree rows sit at position kv_len + depth(node);
  * the suffix's own K/V are used unrounded within the step (the GPU keeps them
    in fp32 scratch); what is committed to the cache is their bf16 rounding.
"""
from __future__ import annotations

import numpy as np

from .numerics import as_f64, bf16_bits_to_f64, f64_to_bf16_bits


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding.  x [..., D]; pos broadcasts to x[..., 0]."""
    D = x.shape[-1]
    half = D // 2
    inv_freq = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / D)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, allowed: np.ndarray,
           scale: float) -> np.ndarray:
    """softmax(q keys^T * scale, masked to `allowed`) vals.
    q [nq, D], keys / vals [nk, D], allowed [nq, nk] bool."""
    s = (q @ keys.T) * scale
    s = np.where(allowed, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=1, keepdims=True)) @ vals


def check_tree(parent_row) -> None:
    """A valid tree: node 0 is the root (parent -1), every other parent precedes
    its child."""
    p = np.asarray(parent_row)
    if p[0] != -1:
        raise ValueError("tree root must have parent -1")
    for i in range(1, len(p)):
        if not (0 <= p[i] < i):
            raise ValueError(f"node {i}: parent {p[i]} must be in [0, {i})")


def tree_depths(parent_row) -> np.ndarray:
    check_tree(parent_row)
    p = np.asarray(parent_row)
    d = np.zeros(len(p), dtype=np.int64)
    for i in range(1, len(p)):
        d[i] = d[p[i]] + 1
    return d


def visibility(T: int, parent_row=None) -> np.ndarray:
    """vis[i, j]: may suffix row i attend to suffix row j?  Chain: j <= i.
    Tree: j is i or one of its ancestors."""
    if parent_row is None:
        return np.tril(np.ones((T, T), dtype=bool))
    check_tree(parent_row)
    p = np.asarray(parent_row)
    vis = np.zeros((T, T), dtype=bool)
    for i in range(T):
        j = i
        while j >= 0:
            vis[i, j] = True
            j = p[j]
    return vis


class Weights:
    """Name -> fp64 array view over the raw weight list (bf16 bit patterns or
    floats), decoded on each access so an 8B-shaped model is converted one
    matrix at a time."""

    def __init__(self, names, arrays):
        self._w = dict(zip(names, arrays))

    def __getitem__(self, name) -> np.ndarray:
        return as_f64(self._w[name])

    def rows(self, name, idx) -> np.ndarray:
        return as_f64(self._w[name][np.asarray(idx)])


def _decode_cache(a):
    a = np.asarray(a)
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def forward(shape, W: Weights, tokens, kv_len, k_cache, v_cache, tree_parent=None):
    """Verify-window forward.

    tokens      [B, T] ints: row 0 is the pending token, rows 1.. the drafts
                (tree: node ids in an order where parents precede children)
    kv_len      [B] committed cache length per sequence
    k_cache     [L, B, Hkv, max_ctx, D] (bf16 bits or floats), rows < kv_len[b]
    v_cache     [L, B, Hkv, D, max_ctx] (values stored transposed)
    tree_parent None for a chain, else [B, T] parent ids (root -1)

    Returns logits [B, T, V] and the suffix's rotated keys / values
    k_new, v_new [L, B, T, Hkv, D] (fp64, unrounded).
    """
    tokens = np.asarray(tokens)
    kv_len = np.asarray(kv_len)
    B, T = tokens.shape
    L, d = shape.n_layers, shape.d_model
    Hq, Hkv, D, F = shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.d_ffn
    G = Hq // Hkv
    eps, theta = shape.rms_eps, shape.rope_theta

    if tree_parent is None:
        pos = kv_len[:, None] + np.arange(T)[None, :]
        vis = [visibility(T)] * B
    else:
        tp = np.asarray(tree_parent)
        pos = np.stack([kv_len[b] + tree_depths(tp[b]) for b in range(B)])
        vis = [visibility(T, tp[b]) for b in range(B)]

    x = W.rows("embed", tokens.reshape(-1)).reshape(B, T, d)
    k_new = np.zeros((L, B, T, Hkv, D))
    v_new = np.zeros((L, B, T, Hkv, D))
    scale = 1.0 / np.sqrt(D)

    for l in range(L):
        h = rms_norm(x, W[f"l{l}.attn_norm"], eps)
        qkv = h @ W[f"l{l}.w_qkv"].T
        q = qkv[..., : Hq * D].reshape(B, T, Hq, D)
        k = qkv[..., Hq * D: (Hq + Hkv) * D].reshape(B, T, Hkv, D)
        v = qkv[..., (Hq + Hkv) * D:].reshape(B, T, Hkv, D)
        q = rope(q, pos[:, :, None], theta)
        k = rope(k, pos[:, :, None], theta)
        k_new[l], v_new[l] = k, v

        o = np.zeros((B, T, Hq, D))
        for b in range(B):
            n = int(kv_len[b])
            for kh in range(Hkv):
                kc = _decode_cache(k_cache[l, b, kh, :n, :])          # [n, D]
                vc = _decode_cache(v_cache[l, b, kh, :, :n]).T        # [n, D]
                keys = np.concatenate([kc, k[b, :, kh, :]], axis=0)   # [n+T, D]
                vals = np.concatenate([vc, v[b, :, kh, :]], axis=0)
                allowed = np.concatenate([np.ones((T, n), dtype=bool), vis[b]], axis=1)  # [T, n+T]
                for g in range(G):
                    hq = kh * G + g
                    o[b, :, hq, :] = attend(q[b, :, hq, :], keys, vals, allowed, scale)
        x = x + o.reshape(B, T, Hq * D) @ W[f"l{l}.w_o"].T
        h = rms_norm(x, W[f"l{l}.ffn_norm"], eps)
        gu = h @ W[f"l{l}.w_gate_up"].T
        a = silu(gu[..., :F]) * gu[..., F:]
        x = x + a @ W[f"l{l}.w_down"].T

    hf = rms_norm(x, W["final_norm"], eps)
    logits = hf @ W["lm_head"].T
    return logits, k_new, v_new


def forward_ragged(shape, W: Weights, tokens_rows, cu, kv_len, k_cache, v_cache):
    """Compact ("ragged") verify, the DeepSeek-V4 analysis page, section 4:
    sequence b verifies its own chain of len_b = cu[b+1] - cu[b] rows, packed
    back to back in tokens_rows.  No row attends across sequences, so each
    sequence's rows are exactly the chain forward of that sequence alone with
    T = len_b.  Returns logits [cu[B], V] and per-sequence lists of the
    suffix keys / values [L, len_b, Hkv, D]."""
    tokens_rows = np.asarray(tokens_rows)
    cu = [int(c) for c in cu]
    logits, k_new, v_new = [], [], []
    for b in range(len(cu) - 1):
        toks = tokens_rows[cu[b]:cu[b + 1]][None, :]
        lg, kn, vn = forward(shape, W, toks, np.asarray(kv_len)[b:b + 1], k_cache[:, b:b + 1],
                             v_cache[:, b:b + 1])
        logits.append(lg[0])
        k_new.append(kn[:, 0])
        v_new.append(vn[:, 0])
    return np.concatenate(logits, axis=0), k_new, v_new


def page_slots(table_row, n_slots: int, page: int = 64):
    """Paged KV (PagedAttention, the CS349E lecture's reading list; 64-slot
    pages as on the ninfer sweep page): a block table maps a sequence's
    logically contiguous slots to scattered physical pages; slot s is offset
    s % page of page table_row[s // page].  Returns (page, offset) per slot."""
    s = np.arange(n_slots)
    return np.asarray(table_row)[s // page], s % page


def gather_pages(k_pool, v_pool, table, n_slots: int, page: int = 64):
    """Dense views of the sequences' first n_slots slots from a page pool:
    k_pool [L, pages, Hkv, page, D], v_pool [L, pages, Hkv, D, page], table
    [B, pages_per_seq] -> K [L, B, Hkv, n_slots, D], V [L, B, Hkv, D, n_slots]."""
    B = len(table)
    L, _, H, _, D = k_pool.shape
    k = np.zeros((L, B, H, n_slots, D), dtype=k_pool.dtype)
    v = np.zeros((L, B, H, D, n_slots), dtype=v_pool.dtype)
    for b in range(B):
        pg, off = page_slots(table[b], n_slots, page)
        k[:, b] = k_pool[:, pg, :, off, :].transpose(1, 2, 0, 3)
        v[:, b] = v_pool[:, pg, :, :, off].transpose(1, 2, 3, 0)
    return k, v


def scatter_pages(k_dense, v_dense, table, k_pool, v_pool, page: int = 64):
    """Inverse of gather_pages: write the dense slots into their pages."""
    B, n_slots = k_dense.shape[1], k_dense.shape[3]
    for b in range(B):
        pg, off = page_slots(table[b], n_slots, page)
        k_pool[:, pg, :, off, :] = k_dense[:, b].transpose(2, 0, 1, 3)
        v_pool[:, pg, :, :, off] = v_dense[:, b].transpose(3, 0, 1, 2)


def write_suffix(k_cache, v_cache, k_new, v_new, kv_len, rows=None):
    """Store the window's K/V (rounded to bf16) at slots kv_len[b] + i, as the
    verify step does for every row before acceptance is known.  Caches are
    uint16 bf16 bit arrays, modified in place."""
    L, B, T = k_new.shape[:3]
    rows = range(T) if rows is None else rows
    for b in range(B):
        for i in rows:
            s = int(kv_len[b]) + i
            k_cache[:, b, :, s, :] = f64_to_bf16_bits(k_new[:, b, i])
            v_cache[:, b, :, :, s] = f64_to_bf16_bits(v_new[:, b, i])


def commit_chain(kv_len, n_accepted):
    """Pending-token invariant: the pending token and the n accepted drafts are
    now confirmed and cached; the emitted extra token becomes the next pending
    token and is not cached (CS349E Lecture 6, section 6.2).  The rejected tail
    stays in the cache but lies beyond the length (the Kimi-K3 tuning page:
    a pure-attention cache is indexed by position, abandoning costs nothing)."""
    return np.asarray(kv_len) + np.asarray(n_accepted) + 1


def commit_tree(k_cache, v_cache, kv_len, paths):
    """Tree commit: the accepted path's nodes (root first) move to contiguous
    slots kv_len + 0 .. n.  Copies run in ascending path order, which never
    overwrites a slot that a later copy still has to read (path node j has
    id >= j).  Returns the new lengths."""
    new_len = np.array(kv_len, copy=True)
    for b, path in enumerate(paths):
        base = int(kv_len[b])
        for j, node in enumerate(path):
            if node != j:
                k_cache[:, b, :, base + j, :] = k_cache[:, b, :, base + node, :]
                v_cache[:, b, :, :, base + j] = v_cache[:, b, :, :, base + node]
        new_len[b] = base + len(path)
    return new_len
