"""Paged KV cache (PagedAttention pages of 64 slots, a block table per
sequence; CS349E Lecture 6: a paged rollback edits the table's length and
frees the surplus pages): the verify step, attention and tree commit through a
seeded random block table, against the oracle on the gathered dense cache."""
import numpy as np
import pytest
import torch

import synth
from oracle import accept as OA
from oracle import model as OM
from oracle import philox
from oracle.numerics import bf16_bits_to_f64
from speculative_decoding_verify_spec_amd.engine import VerifyEngine
from tests.gpu_util import bf16_close, DRAW_BAND_SHARED, compare_decisions, dev, logits_rel_err, oracle_weights

pytestmark = pytest.mark.gpu

PAGE = 64


def _paged_engine(sh, max_batch, max_ctx, max_rows, ctx_len, extra_pages=3):
    """Engine over a page pool holding the same synthetic context as a dense
    cache; pool pages no table entry names are NaN."""
    names, w = synth.make_weights(sh, device=dev())
    dense = synth.make_kv_cache(sh, max_batch, max_ctx, ctx_len, device=dev(), poison_tail=True)
    pps = max_ctx // PAGE
    npages = max_batch * pps + extra_pages
    table = synth.random_block_table(max_batch, pps, npages)
    kd, vd = synth.kv_views(dense, sh, max_batch, max_ctx)
    kd, vd = synth.to_numpy_raw(kd), synth.to_numpy_raw(vd)
    L, H, D = sh.n_layers, sh.n_kv_heads, sh.head_dim
    nan_bits = np.uint16(0x7FC0)
    kp = np.full((L, npages, H, PAGE, D), nan_bits, dtype=np.uint16)
    vp = np.full((L, npages, H, D, PAGE), nan_bits, dtype=np.uint16)
    OM.scatter_pages(kd, vd, table.numpy(), kp, vp)
    pool = torch.from_numpy(np.stack([kp.reshape(L, -1), vp.reshape(L, -1)], axis=1).reshape(-1).view(np.int16))
    pool = pool.view(torch.bfloat16).to(dev())
    eng = VerifyEngine(sh, w, pool, max_batch, max_ctx, max_rows, kv_pages=npages)
    tdev = table.to(dev())
    eng.set_block_table(tdev)
    return eng, names, w, pool, tdev, npages, (kd, vd)


def _gather(pool, sh, table, npages, max_ctx):
    L, H, D = sh.n_layers, sh.n_kv_heads, sh.head_dim
    raw = synth.to_numpy_raw(pool).reshape(L, 2, npages * H * PAGE * D)
    kp = raw[:, 0].reshape(L, npages, H, PAGE, D)
    vp = raw[:, 1].reshape(L, npages, H, D, PAGE)
    return OM.gather_pages(kp, vp, table.cpu().numpy(), max_ctx), (kp, vp)


@pytest.mark.parametrize("B,T,ctx,branching", [(3, 4, [300, 17, 700], None), (2, 8, [1000, 37], None),
                                               (2, 15, [129, 500], [2, 2, 2])])
def test_paged_step_matches_oracle(B, T, ctx, branching):
    sh = synth.MINI8B
    print(f"[paged] B={B} T={T} ctx={ctx} tree={branching}", flush=True)
    max_ctx = 1024
    eng, names, w, pool, table, npages, (kd, vd) = _paged_engine(sh, 4, max_ctx, 16, ctx + [0] * (4 - B))
    W = oracle_weights(names, w)
    (k0, v0), (kp0, vp0) = _gather(pool, sh, table, npages, max_ctx)
    assert np.array_equal(k0, kd) and np.array_equal(v0, vd)  # the pool holds the dense context
    tokens = synth.make_tokens(B, T, sh.vocab, seed=31 + T, device=dev())
    kv = torch.tensor(ctx, dtype=torch.int32, device=dev())
    parent = synth.random_tree(branching, B).to(dev()) if branching else None
    z = torch.full((B, T, sh.vocab), float("nan"), device=dev())
    eng.step(tokens, kv, z, parent)
    torch.cuda.synchronize()
    zo, kn, vn = OM.forward(sh, W, tokens.cpu().numpy(), np.array(ctx), kd[:, :B], vd[:, :B],
                            tree_parent=None if parent is None else parent.cpu().numpy())
    err = logits_rel_err(z.cpu().numpy(), zo)
    print(f"  logits rel err max {err.max():.2e}", flush=True)
    assert err.max() < 1e-3
    (kg, vg), (kp, vp) = _gather(pool, sh, table, npages, max_ctx)
    ko, vo = kd.copy(), vd.copy()
    OM.write_suffix(ko[:, :B], vo[:, :B], kn, vn, np.array(ctx))
    for b in range(B):
        s0, s1 = ctx[b], ctx[b] + T
        bf16_close(kg[:, b, :, s0:s1], ko[:, b, :, s0:s1])
        bf16_close(vg[:, b, :, :, s0:s1], vo[:, b, :, :, s0:s1])
        assert np.array_equal(kg[:, b, :, :s0], kd[:, b, :, :s0])
        assert np.array_equal(kg[:, b, :, s1:], kd[:, b, :, s1:])  # NaN tail untouched
    # pages no table row names are untouched
    named = set(table.cpu().numpy().reshape(-1).tolist())
    for pg in range(npages):
        if pg not in named:
            assert np.array_equal(kp[:, pg], kp0[:, pg]) and np.array_equal(vp[:, pg], vp0[:, pg])
    assert eng.device_errors() == 0


def test_paged_tree_commit_and_table_edit():
    """Tree accept commits the accepted path through the table; moving a
    sequence's page to a free pool page and editing the table in place leaves
    the next step's logits unchanged (recorded launches read the entries)."""
    sh = synth.MINI8B
    B, ctx, max_ctx = 2, [200, 90], 512
    eng, names, w, pool, table, npages, (kd, vd) = _paged_engine(sh, 2, max_ctx, 16, ctx, extra_pages=4)
    parent = synth.random_tree([2, 2, 2], B).to(dev())
    T = parent.shape[1]
    tokens = synth.make_tokens(B, T, sh.vocab, seed=41, device=dev())
    kv = torch.tensor(ctx, dtype=torch.int32, device=dev())
    z = torch.empty((B, T, sh.vocab), device=dev())
    for _ in range(2):  # direct, then recorded and replayed
        eng.step(tokens, kv, z, parent)
    torch.cuda.synchronize()
    z_ref = z.clone()
    (k_before, v_before), _ = _gather(pool, sh, table, npages, max_ctx)
    # accept greedily with tokens forced onto a known path: node tokens = argmax
    q, _ = synth.noisy_draft_dist(z, 0.5, 43, 1.0)
    out = torch.zeros((B, T), dtype=torch.int32, device=dev())
    nacc = torch.zeros((B,), dtype=torch.int32, device=dev())
    kv_out = torch.zeros((B,), dtype=torch.int32, device=dev())
    eng.accept(z, q, tokens, out, nacc, kv, kv_out, tree_parent=parent, temperature=0.0, seed=1, round_=0)
    torch.cuda.synchronize()
    orc = OA.accept(z.double().cpu().numpy(), None, tokens.cpu().numpy(), 0.0, philox.Uniforms(1, 0),
                    tree_parent=parent.cpu().numpy())
    compare_decisions(out.cpu().numpy(), nacc.cpu().numpy(), orc, "paged tree", draw_band=DRAW_BAND_SHARED)
    (k_after, v_after), _ = _gather(pool, sh, table, npages, max_ctx)
    for b in range(B):
        path = orc["paths"][b]
        for j, node in enumerate(path):
            assert np.array_equal(k_after[:, b, :, ctx[b] + j], k_before[:, b, :, ctx[b] + node])
            assert np.array_equal(v_after[:, b, :, :, ctx[b] + j], v_before[:, b, :, :, ctx[b] + node])
    # move sequence 1's page 1 to a free page and edit the table in place
    pool_k = pool.view(sh.n_layers, 2, npages, -1)
    free = sorted(set(range(npages)) - set(table.cpu().numpy().reshape(-1).tolist()))[0]
    old = int(table[1, 1])
    pool_k[:, :, free] = pool_k[:, :, old]
    pool_k[:, :, old] = float("nan")
    table[1, 1] = free
    torch.cuda.synchronize()
    z2 = torch.empty_like(z)
    eng.step(tokens, kv, z2, parent)
    torch.cuda.synchronize()
    # rows before kv_len are unchanged by the commit, and the window rows are
    # rewritten by the step itself, so the logits repeat
    assert torch.equal(z2, z_ref)
    assert eng.device_errors() == 0


def test_paged_needs_a_table():
    sh = synth.MINI8B
    names, w = synth.make_weights(sh, device=dev())
    npages = 8
    pool = torch.zeros((sh.n_layers * 2 * npages * sh.n_kv_heads * PAGE * sh.head_dim,), dtype=torch.bfloat16,
                       device=dev())
    eng = VerifyEngine(sh, w, pool, 2, 256, 4, kv_pages=npages)
    from speculative_decoding_verify_spec_amd import SPEC_ERR_STATE, SpecError
    z = torch.empty((1, 1, sh.vocab), device=dev())
    with pytest.raises(SpecError) as e:
        eng.step(torch.zeros((1, 1), dtype=torch.int32, device=dev()), torch.zeros(1, dtype=torch.int32, device=dev()), z)
    assert e.value.status == SPEC_ERR_STATE
