"""Pins of the oracle's model forward: each component against a library routine
or an independent mathematical formulation, and the whole forward against
consistency properties the method fixes (prefill vs incremental decode, tree
rows vs their root-to-node chains, GQA vs duplicated heads)."""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

from oracle import model as M
from oracle.numerics import bf16_bits_to_f64


def _shape(L=2, d=32, Hq=4, Hkv=2, D=8, F=48, V=50, theta=10000.0):
    return SimpleNamespace(n_layers=L, d_model=d, n_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                           d_ffn=F, vocab=V, rms_eps=1e-5, rope_theta=theta)


def _weights(sh, seed=0, std=0.3):
    rng = np.random.default_rng(seed)
    d, F, V = sh.d_model, sh.d_ffn, sh.vocab
    qkv = (sh.n_heads + 2 * sh.n_kv_heads) * sh.head_dim
    names, arrs = ["embed"], [rng.normal(size=(V, d)) * std]
    for l in range(sh.n_layers):
        names += [f"l{l}.attn_norm", f"l{l}.w_qkv", f"l{l}.w_o", f"l{l}.ffn_norm",
                  f"l{l}.w_gate_up", f"l{l}.w_down"]
        arrs += [1 + 0.1 * rng.normal(size=d), rng.normal(size=(qkv, d)) * std,
                 rng.normal(size=(d, sh.n_heads * sh.head_dim)) * std, 1 + 0.1 * rng.normal(size=d),
                 rng.normal(size=(2 * F, d)) * std, rng.normal(size=(d, F)) * std]
    names += ["final_norm", "lm_head"]
    arrs += [1 + 0.1 * rng.normal(size=d), rng.normal(size=(V, d)) * std]
    return names, arrs


def _empty_cache(sh, B, ctx):
    k = np.zeros((sh.n_layers, B, sh.n_kv_heads, ctx, sh.head_dim))
    v = np.zeros((sh.n_layers, B, sh.n_kv_heads, sh.head_dim, ctx))
    return k, v


def _store(kc, vc, k_new, v_new, kv_len):
    """Store unrounded window K/V at slots kv_len + i (float caches)."""
    L, B, T = k_new.shape[:3]
    for b in range(B):
        for i in range(T):
            kc[:, b, :, kv_len[b] + i, :] = k_new[:, b, i]
            vc[:, b, :, :, kv_len[b] + i] = v_new[:, b, i]


def test_rms_norm_matches_torch():
    x = np.random.default_rng(0).normal(size=(5, 64)) * 3
    g = np.random.default_rng(1).normal(size=64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-5)
    assert np.allclose(M.rms_norm(x, g, 1e-5), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    assert np.allclose(M.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-13, atol=1e-15)


def test_rope_is_complex_rotation():
    """Rotate-half RoPE pairing (i, i + D/2) is multiplication of
    x_i + j x_{i+D/2} by exp(j pos theta^(-2i/D))."""
    rng = np.random.default_rng(2)
    D, theta = 16, 500000.0
    x = rng.normal(size=(7, D))
    pos = np.array([0, 1, 5, 100, 2047, 32767, 40000])
    got = M.rope(x, pos, theta)
    zc = x[:, : D // 2] + 1j * x[:, D // 2:]
    f = np.exp(1j * pos[:, None] * theta ** (-np.arange(0, D, 2) / D))
    want = zc * f
    assert np.allclose(got[:, : D // 2], want.real, atol=1e-12)
    assert np.allclose(got[:, D // 2:], want.imag, atol=1e-12)


def test_rope_relative_position_and_norm():
    rng = np.random.default_rng(3)
    q, k = rng.normal(size=32), rng.normal(size=32)
    d1 = M.rope(q, np.array(70), 10000.0) @ M.rope(k, np.array(30), 10000.0)
    d2 = M.rope(q, np.array(1040), 10000.0) @ M.rope(k, np.array(1000), 10000.0)
    assert abs(d1 - d2) < 1e-9
    assert abs(np.linalg.norm(M.rope(q, np.array(12345), 10000.0)) - np.linalg.norm(q)) < 1e-12


def test_attend_matches_torch_sdpa():
    rng = np.random.default_rng(4)
    nq, nk, D = 9, 23, 16
    q, k, v = rng.normal(size=(nq, D)), rng.normal(size=(nk, D)), rng.normal(size=(nk, D))
    allowed = rng.random((nq, nk)) < 0.6
    allowed[:, 0] = True
    got = M.attend(q, k, v, allowed, 1 / np.sqrt(D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(allowed)[None])[0].numpy()
    assert np.allclose(got, ref, atol=1e-12)


def test_chain_mask_is_causal_sdpa():
    rng = np.random.default_rng(5)
    T, D = 6, 8
    q, k, v = rng.normal(size=(T, D)), rng.normal(size=(T, D)), rng.normal(size=(T, D))
    got = M.attend(q, k, v, M.visibility(T), 1 / np.sqrt(D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=True)[0].numpy()
    assert np.allclose(got, ref, atol=1e-12)


def test_prefill_equals_incremental_decode():
    """Causal consistency: a forward over the whole window from an empty cache
    equals a forward over its first k rows, then (with those K/V cached) a
    forward over the rest at kv_len = k; and each verify row equals a T=1
    decode after feeding the rows before it."""
    sh = _shape()
    W = M.Weights(*_weights(sh))
    B, T = 2, 7
    toks = np.random.default_rng(6).integers(0, sh.vocab, size=(B, T))
    kc, vc = _empty_cache(sh, B, 16)
    full, _, _ = M.forward(sh, W, toks, np.zeros(B, int), kc, vc)
    for k in [1, 3, 6]:
        kc, vc = _empty_cache(sh, B, 16)
        z1, kn, vn = M.forward(sh, W, toks[:, :k], np.zeros(B, int), kc, vc)
        _store(kc, vc, kn, vn, np.zeros(B, int))
        z2, _, _ = M.forward(sh, W, toks[:, k:], np.full(B, k), kc, vc)
        assert np.allclose(np.concatenate([z1, z2], axis=1), full, atol=1e-10)
    # one row at a time
    kc, vc = _empty_cache(sh, B, 16)
    rows = []
    for i in range(T):
        z, kn, vn = M.forward(sh, W, toks[:, i:i + 1], np.full(B, i), kc, vc)
        _store(kc, vc, kn, vn, np.full(B, i))
        rows.append(z)
    assert np.allclose(np.concatenate(rows, axis=1), full, atol=1e-10)


def test_ragged_kv_len_per_sequence():
    """Rows are independent across sequences (selective batching): a batch with
    different cache lengths equals each sequence run alone."""
    sh = _shape()
    W = M.Weights(*_weights(sh, seed=1))
    rng = np.random.default_rng(7)
    B, T, ctx = 3, 4, 20
    kc = rng.normal(size=(sh.n_layers, B, sh.n_kv_heads, ctx, sh.head_dim))
    vc = rng.normal(size=(sh.n_layers, B, sh.n_kv_heads, sh.head_dim, ctx))
    kv_len = np.array([0, 5, 13])
    toks = rng.integers(0, sh.vocab, size=(B, T))
    z, _, _ = M.forward(sh, W, toks, kv_len, kc, vc)
    for b in range(B):
        zb, _, _ = M.forward(sh, W, toks[b:b + 1], kv_len[b:b + 1], kc[:, b:b + 1], vc[:, b:b + 1])
        assert np.allclose(z[b], zb[0], atol=1e-12)


def test_tree_rows_equal_root_to_node_chains():
    """Each tree node's logits equal the chain forward over its root-to-node
    path: the ancestor mask plus depth positions reproduce the chain."""
    sh = _shape()
    W = M.Weights(*_weights(sh, seed=2))
    rng = np.random.default_rng(8)
    ctx = 24
    kc = rng.normal(size=(sh.n_layers, 1, sh.n_kv_heads, ctx, sh.head_dim))
    vc = rng.normal(size=(sh.n_layers, 1, sh.n_kv_heads, sh.head_dim, ctx))
    parent = [-1, 0, 0, 0, 1, 1, 2, 4, 4, 6]
    T = len(parent)
    toks = rng.integers(0, sh.vocab, size=(1, T))
    kv_len = np.array([9])
    zt, _, _ = M.forward(sh, W, toks, kv_len, kc, vc, tree_parent=np.array([parent]))
    for i in range(T):
        path = []
        j = i
        while j >= 0:
            path.append(j)
            j = parent[j]
        path = path[::-1]
        zc, _, _ = M.forward(sh, W, toks[:, path], kv_len, kc, vc)
        assert np.allclose(zt[0, i], zc[0, -1], atol=1e-10)


def test_tree_all_ones_equals_chain_forward():
    sh = _shape()
    W = M.Weights(*_weights(sh, seed=3))
    rng = np.random.default_rng(9)
    kc, vc = _empty_cache(sh, 2, 12)
    toks = rng.integers(0, sh.vocab, size=(2, 5))
    parent = np.array([[-1, 0, 1, 2, 3]] * 2)
    a, _, _ = M.forward(sh, W, toks, np.zeros(2, int), kc, vc)
    b, _, _ = M.forward(sh, W, toks, np.zeros(2, int), kc, vc, tree_parent=parent)
    assert np.allclose(a, b, atol=1e-12)


def test_gqa_equals_mha_with_duplicated_kv_heads():
    """Query head h reads KV head floor(h / G): duplicating each KV head's
    weights G times into an MHA model gives the same logits."""
    g_sh = _shape(Hq=4, Hkv=2)
    m_sh = _shape(Hq=4, Hkv=4)
    names, arrs = _weights(g_sh, seed=4)
    D, Hq = g_sh.head_dim, g_sh.n_heads
    m_arrs = []
    for n, a in zip(names, arrs):
        if n.endswith("w_qkv"):
            q = a[: Hq * D]
            k = a[Hq * D: (Hq + 2) * D].reshape(2, D, -1)
            v = a[(Hq + 2) * D:].reshape(2, D, -1)
            k = np.repeat(k, 2, axis=0).reshape(4 * D, -1)
            v = np.repeat(v, 2, axis=0).reshape(4 * D, -1)
            a = np.concatenate([q, k, v])
        m_arrs.append(a)
    rng = np.random.default_rng(10)
    toks = rng.integers(0, g_sh.vocab, size=(1, 6))
    kc, vc = _empty_cache(g_sh, 1, 8)
    kc2, vc2 = _empty_cache(m_sh, 1, 8)
    a, _, _ = M.forward(g_sh, M.Weights(names, arrs), toks, np.zeros(1, int), kc, vc)
    b, _, _ = M.forward(m_sh, M.Weights(names, m_arrs), toks, np.zeros(1, int), kc2, vc2)
    assert np.allclose(a, b, atol=1e-12)


def test_commit_tree_compacts_path_in_place():
    sh = _shape(L=1)
    B, ctx = 1, 20
    kc = np.arange(sh.n_layers * B * sh.n_kv_heads * ctx * sh.head_dim, dtype=np.uint16).reshape(
        sh.n_layers, B, sh.n_kv_heads, ctx, sh.head_dim)
    vc = np.ascontiguousarray(np.swapaxes(kc, 3, 4)) + 7
    k0, v0 = kc.copy(), vc.copy()
    base = 5
    path = [0, 1, 3, 4, 9]     # node 1 stays, node 3 -> slot 2, 4 -> 3 (read after 3 moved), 9 -> 4
    new_len = M.commit_tree(kc, vc, np.array([base]), [path])
    assert new_len[0] == base + len(path)
    for j, node in enumerate(path):
        assert np.array_equal(kc[:, 0, :, base + j], k0[:, 0, :, base + node])
        assert np.array_equal(vc[:, 0, :, :, base + j], v0[:, 0, :, :, base + node])
    assert np.array_equal(kc[:, :, :, :base], k0[:, :, :, :base])


def test_write_suffix_rounds_to_bf16():
    sh = _shape(L=1)
    kc = np.zeros((1, 1, sh.n_kv_heads, 10, sh.head_dim), dtype=np.uint16)
    vc = np.zeros((1, 1, sh.n_kv_heads, sh.head_dim, 10), dtype=np.uint16)
    rng = np.random.default_rng(11)
    kn = rng.normal(size=(1, 1, 3, sh.n_kv_heads, sh.head_dim))
    vn = rng.normal(size=(1, 1, 3, sh.n_kv_heads, sh.head_dim))
    M.write_suffix(kc, vc, kn, vn, np.array([4]))
    got = bf16_bits_to_f64(kc[0, 0, :, 4:7, :])
    want = torch.from_numpy(kn[0, 0].transpose(1, 0, 2).astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(got, want)


def test_bad_tree_rejected():
    with pytest.raises(ValueError):
        M.check_tree([-1, 0, 2])
    with pytest.raises(ValueError):
        M.check_tree([0, 0])


def test_window_prefix_rows_do_not_depend_on_later_rows():
    """The property cap-accept rests on (DeepSeek-V4 analysis page, section 4):
    in a chain window the first L rows' logits do not depend on the rows after
    them, so a fixed-width forward capped at L rows gives the logits of an
    L-row (compact) forward."""
    sh = _shape()
    W = M.Weights(*_weights(sh, seed=3))
    rng = np.random.default_rng(8)
    B, T, ctx = 2, 6, 12
    kc = rng.normal(size=(sh.n_layers, B, sh.n_kv_heads, ctx + T, sh.head_dim))
    vc = rng.normal(size=(sh.n_layers, B, sh.n_kv_heads, sh.head_dim, ctx + T))
    kv_len = np.array([4, 11])
    toks = rng.integers(0, sh.vocab, size=(B, T))
    full, _, _ = M.forward(sh, W, toks, kv_len, kc, vc)
    for L in range(1, T):
        part, _, _ = M.forward(sh, W, toks[:, :L], kv_len, kc, vc)
        assert np.allclose(part, full[:, :L], atol=1e-12)
        # and the later rows do depend on a changed earlier token
    toks2 = toks.copy()
    toks2[:, 2] = (toks2[:, 2] + 1) % sh.vocab
    z2, _, _ = M.forward(sh, W, toks2, kv_len, kc, vc)
    assert np.allclose(z2[:, :2], full[:, :2], atol=1e-12)
    assert not np.allclose(z2[:, 3:], full[:, 3:], atol=1e-6)


def test_forward_ragged_packs_the_batched_forward():
    """Compact verify with equal lengths packs the batched chain forward row
    for row; with unequal lengths every sequence's rows are its own forward."""
    sh = _shape()
    W = M.Weights(*_weights(sh, seed=4))
    rng = np.random.default_rng(9)
    B, T, ctx = 3, 4, 10
    kc = rng.normal(size=(sh.n_layers, B, sh.n_kv_heads, ctx + T, sh.head_dim))
    vc = rng.normal(size=(sh.n_layers, B, sh.n_kv_heads, sh.head_dim, ctx + T))
    kv_len = np.array([2, 9, 5])
    toks = rng.integers(0, sh.vocab, size=(B, T))
    full, kn, vn = M.forward(sh, W, toks, kv_len, kc, vc)
    cu = [0, 4, 8, 12]
    zr, knr, vnr = M.forward_ragged(sh, W, toks.reshape(-1), cu, kv_len, kc, vc)
    assert np.allclose(zr, full.reshape(B * T, -1), atol=1e-12)
    for b in range(B):
        assert np.allclose(knr[b], kn[:, b], atol=1e-12) and np.allclose(vnr[b], vn[:, b], atol=1e-12)
    lens = [3, 1, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    rows = np.concatenate([toks[b, :lens[b]] for b in range(B)])
    zr, _, _ = M.forward_ragged(sh, W, rows, cu, kv_len, kc, vc)
    for b in range(B):
        assert np.allclose(zr[cu[b]:cu[b + 1]], full[b, :lens[b]], atol=1e-12)


def test_paged_gather_follows_the_block_table():
    """Paged KV: every slot s of sequence b is read from page table[b][s // 64]
    at offset s % 64 (pool values encode their own page and offset)."""
    L, H, D, page, npages = 2, 2, 3, 64, 10
    rng = np.random.default_rng(12)
    table = rng.permutation(npages)[:6].reshape(2, 3)
    code = np.arange(npages)[None, :, None, None, None] * 1000 + np.arange(page)[None, None, None, :, None]
    kp = np.broadcast_to(code, (L, npages, H, page, D)).astype(np.float64)
    vp = np.broadcast_to(code.transpose(0, 1, 2, 4, 3), (L, npages, H, D, page)).astype(np.float64)
    k, v = M.gather_pages(kp, vp, table, 3 * page)
    for b in range(2):
        for s in range(3 * page):
            want = table[b][s // page] * 1000 + s % page
            assert np.all(k[:, b, :, s, :] == want) and np.all(v[:, b, :, :, s] == want)
    # scatter is its inverse on the mapped slots
    kq, vq = np.zeros_like(kp), np.zeros_like(vp)
    M.scatter_pages(k, v, table, kq, vq)
    assert np.array_equal(M.gather_pages(kq, vq, table, 3 * page)[0], k)


def test_paged_placement_does_not_change_the_forward():
    """Two pools holding the same sequences on different physical pages give
    the same logits (the table only names where slots live)."""
    sh = _shape()
    W = M.Weights(*_weights(sh, seed=5))
    rng = np.random.default_rng(13)
    B, T, page, pps, npages = 2, 3, 64, 2, 7
    kd = rng.normal(size=(sh.n_layers, B, sh.n_kv_heads, pps * page, sh.head_dim))
    vd = rng.normal(size=(sh.n_layers, B, sh.n_kv_heads, sh.head_dim, pps * page))
    kv_len = np.array([70, 33])
    toks = rng.integers(0, sh.vocab, size=(B, T))
    outs = []
    for seed in (1, 2):
        table = np.random.default_rng(seed).permutation(npages)[:B * pps].reshape(B, pps)
        kp = np.zeros((sh.n_layers, npages, sh.n_kv_heads, page, sh.head_dim))
        vp = np.zeros((sh.n_layers, npages, sh.n_kv_heads, sh.head_dim, page))
        M.scatter_pages(kd, vd, table, kp, vp)
        kg, vg = M.gather_pages(kp, vp, table, pps * page)
        outs.append(M.forward(sh, W, toks, kv_len, kg, vg)[0])
    assert np.array_equal(outs[0], outs[1])
    assert np.allclose(outs[0], M.forward(sh, W, toks, kv_len, kd, vd)[0], atol=0)


def test_commit_chain_pending_token_convention():
    """After n accepted drafts the pending token and the n drafts are cached:
    kv_len grows by n + 1 (CS349E Lecture 6, section 6.2)."""
    assert list(M.commit_chain([10, 0, 5], [2, 0, 3])) == [13, 1, 9]


def test_speculative_greedy_rounds_with_commit_equal_plain_decoding():
    """Several verify rounds through the oracle's forward, greedy accept and
    chain commit produce the target's own greedy decoding token for token
    (CS349E Lecture 6, section 7.4), with the verify window's K/V written at
    kv_len + i before acceptance and kept only up to the committed length.  An
    off-by-one in the commit or the window's positions breaks the equality."""
    from oracle import accept as A
    sh = _shape(V=37)
    W = M.Weights(*_weights(sh, seed=12))
    rng = np.random.default_rng(13)
    P, n_out, ctx = 6, 24, 64
    prompt = rng.integers(0, sh.vocab, size=(1, P))

    def prefill():
        kc, vc = _empty_cache(sh, 1, ctx)
        z, kn, vn = M.forward(sh, W, prompt, np.zeros(1, int), kc, vc)
        _store(kc, vc, kn, vn, np.zeros(1, int))
        return kc, vc, int(np.argmax(z[0, -1]))

    # plain greedy decoding, one row per step
    kc, vc, pending = prefill()
    kv, plain = P, [pending]
    while len(plain) < n_out:
        z, kn, vn = M.forward(sh, W, np.array([[pending]]), np.array([kv]), kc, vc)
        _store(kc, vc, kn, vn, np.array([kv]))
        kv += 1
        pending = int(np.argmax(z[0, 0]))
        plain.append(pending)

    # speculative rounds: drafts right about 60% of the time
    kc, vc, pending = prefill()
    kv, spec = np.array([P]), [pending]
    while len(spec) < n_out:
        gamma = int(rng.integers(1, 5))
        drafts = []
        for i in range(gamma):
            k = len(spec) + i
            right = plain[k] if k < len(plain) else 0
            drafts.append(right if rng.random() < 0.6 else int(rng.integers(0, sh.vocab)))
        toks = np.array([[pending] + drafts])
        z, kn, vn = M.forward(sh, W, toks, kv, kc, vc)
        _store(kc, vc, kn, vn, kv)
        n, out, _ = A.accept_chain_one(z[0], None, toks[0], 0.0, None)
        kv = M.commit_chain(kv, [n])
        pending = out[-1]
        spec += out
    assert spec[:n_out] == plain
