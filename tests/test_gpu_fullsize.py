"""Parity at the full Llama-3-8B shape (32 layers, d=4096, V=128256, bf16) in
the launch configurations of the benchmarked workload and the larger ones:

  * B=1, context 2048, chain gamma=3 (the benchmarked round): all rows;
  * B=8, context 1024, chain gamma=3 (M=32);
  * B=4, context 4096, token tree [4,4,2,2] (117 rows per sequence, M=468);
  * B=16, context 32768, chain gamma=7 (M=128, 68.7 GB of cache).

The GPU runs the whole batch; the oracle recomputes the sampled sequences
(rows of different sequences are independent), so its cost stays bounded.
Checks per sampled sequence: logits (per-row relative error at most 1e-3,
what the fp32-activation path achieves with room to spare; the contract
bound is 2e-2), the K/V
the step wrote, and the accept decisions on the oracle's own logits (near
ties counted).  The accept decisions of every sequence are also checked on
the GPU's logits (shared-logits tier)."""
import gc

import numpy as np
import pytest
import torch

import synth
from oracle import accept as OA
from oracle import model as OM
from oracle import philox
from speculative_decoding_verify_spec_amd.engine import VerifyEngine
from tests.gpu_util import (DRAW_BAND_SHARED, LOGIT_RTOL_FULL, bf16_close, compare_decisions, dev, logits_rel_err,
                            oracle_weights)

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]


@pytest.fixture(scope="module")
def model8b():
    sh = synth.LLAMA8B
    print("[8b] weights", flush=True)
    names, w = synth.make_weights(sh, device=dev())
    W = oracle_weights(names, w)
    yield sh, w, W
    del w, W
    gc.collect()
    torch.cuda.empty_cache()


def _chain_drafts(B, gamma, V, sigma, temp, seed):
    """Pending tokens and gamma drafts sampled from a synthetic draft
    distribution q = softmax(z' + eps) over random logits z' (independent of
    the path under test)."""
    pend = synth.make_tokens(B, 1, V, seed=seed, device=dev())
    if gamma == 0:
        return pend, None
    zd = synth.random_logits((B, gamma), V, seed=seed + 1, device=dev())
    q, zn = synth.noisy_draft_dist(zd, sigma, seed + 2, temp if temp > 0 else 1.0)
    if temp > 0:
        x = synth.sample_from(q, seed + 3)[..., 0]
    else:
        x = zn.argmax(-1).to(torch.int32)
    return torch.cat([pend, x], 1).contiguous(), q


def _tree_drafts(B, branching, V, sigma, seed):
    parent = synth.random_tree(branching, B).to(dev())
    T = parent.shape[1]
    zd = synth.random_logits((B, T), V, seed=seed, device=dev())
    q, _ = synth.noisy_draft_dist(zd, sigma, seed + 1)
    tok = synth.make_tokens(B, T, V, seed=seed + 2).clone()
    ch = synth.tree_children(parent[0].cpu().tolist())
    g = torch.Generator(device="cpu").manual_seed(seed + 3)
    for b in range(B):
        for v in range(T):
            if ch[v]:
                picks = torch.multinomial(q[b, v].double().cpu(), len(ch[v]), replacement=False, generator=g)
                for c, x in zip(ch[v], picks.tolist()):
                    tok[b, c] = x
    return tok.to(torch.int32).to(dev()), q, parent


def _round(model, B, ctx, T, tokens, q, sample, parent=None, temp=1.0, seed=7, prepare=None):
    """One verify + accept round on the GPU against the oracle.  `prepare`
    (engine, kv_len, tokens) -> tokens may run steps first to choose drafts."""
    sh, w, W = model
    max_ctx = ((max(ctx) + T + 63) // 64) * 64
    print(f"[8b] B={B} T={T} ctx={max(ctx)} tree={parent is not None} temp={temp}: cache", flush=True)
    cache = synth.make_kv_cache(sh, B, max_ctx, ctx, device=dev(), poison_tail=True)
    eng = VerifyEngine(sh, w, cache, B, max_ctx, T)
    kv = torch.tensor(ctx, dtype=torch.int32, device=dev())
    if prepare is not None:
        tokens = prepare(eng, kv, tokens)
    z = torch.full((B, T, sh.vocab), float("nan"), device=dev())
    eng.step(tokens, kv, z, tree_parent=parent)
    torch.cuda.synchronize()
    # the sampled sequences' cache as the step left it (a tree's accept then
    # moves the accepted path's K/V to the slots after the root)
    k, v = synth.kv_views(cache, sh, B, max_ctx)
    snap = {b: (synth.to_numpy_raw(k[:, b:b + 1]).copy(), synth.to_numpy_raw(v[:, b:b + 1]).copy())
            for b in sample}
    out = torch.full((B, T), -5, dtype=torch.int32, device=dev())
    nacc = torch.full((B,), -5, dtype=torch.int32, device=dev())
    kv_out = torch.zeros((B,), dtype=torch.int32, device=dev())
    eng.accept(z, q, tokens, out, nacc, kv, kv_out, tree_parent=parent, temperature=temp, seed=seed, round_=3)
    torch.cuda.synchronize()
    assert torch.isfinite(z).all()
    assert eng.device_errors() == 0
    tok_h = tokens.cpu().numpy()
    par_h = None if parent is None else parent.cpu().numpy()
    q_h = None if q is None else q.double().cpu().numpy()
    out_h, nacc_h = out.cpu().numpy(), nacc.cpu().numpy()
    uni = philox.Uniforms(seed, 3)

    # shared-logits tier: the oracle's accept on the GPU's logits, every sequence
    orc = OA.accept(z.double().cpu().numpy(), q_h, tok_h, temp, uni, tree_parent=par_h)
    near = compare_decisions(out_h, nacc_h, orc, "shared logits", draw_band=DRAW_BAND_SHARED, cap=max(1, B // 16))
    print(f"  shared-logits near-ties {near}/{B}", flush=True)

    for b in sample:
        print(f"  oracle forward, sequence {b}", flush=True)
        kc, vc = snap[b]
        sl = slice(b, b + 1)
        if parent is not None:
            # the commit copied path node j's K/V to slot kv_len + j, in place
            # (the views again: V is gathered into a copy when it is taken)
            k, v = synth.kv_views(cache, sh, B, max_ctx)
            ka = synth.to_numpy_raw(k[:, b:b + 1])
            va = synth.to_numpy_raw(v[:, b:b + 1])
            path = orc["paths"][b] if nacc_h[b] == orc["n_accepted"][b] else None
            if path is not None:
                for j, node in enumerate(path):
                    assert np.array_equal(ka[:, 0, :, ctx[b] + j], kc[:, 0, :, ctx[b] + node])
                    assert np.array_equal(va[:, 0, :, :, ctx[b] + j], vc[:, 0, :, :, ctx[b] + node])
        # the step has already written its rows' K/V: the oracle's context is
        # [0, ctx) only, so the written slots never enter its attention
        zo, kn, vn = OM.forward(sh, W, tok_h[sl], np.array(ctx[b:b + 1]), kc, vc,
                                tree_parent=None if par_h is None else par_h[sl])
        err = logits_rel_err(z[b:b + 1].cpu().numpy(), zo)
        print(f"    logits rel err max {err.max():.2e} median {np.median(err):.2e}", flush=True)
        assert err.max() < LOGIT_RTOL_FULL
        ko, vo = kc.copy(), vc.copy()
        OM.write_suffix(ko, vo, kn, vn, np.array(ctx[b:b + 1]))
        s0, s1 = ctx[b], ctx[b] + T
        # 32 layers of fp32-vs-fp64 noise: allow 5e-4 of the RMS before rounding
        # (the logits agree to ~5e-5; a wrong row would be off by the RMS)
        bf16_close(kc[:, 0, :, s0:s1], ko[:, 0, :, s0:s1], max_frac=4e-2, noise=5e-4)
        bf16_close(vc[:, 0, :, :, s0:s1], vo[:, 0, :, :, s0:s1], max_frac=4e-2, noise=5e-4)
        # end-to-end tier: decisions on the oracle's own logits
        orc_b = OA.accept(zo, None if q_h is None else q_h[sl], tok_h[sl], temp, _shifted(uni, b),
                          tree_parent=None if par_h is None else par_h[sl])
        nb = compare_decisions(out_h[sl], nacc_h[sl], orc_b, f"sequence {b}", cap=1)
        print(f"    end-to-end near-ties {nb}", flush=True)
    del eng, cache, z
    gc.collect()
    torch.cuda.empty_cache()
    return nacc_h


class _shifted:
    """Uniforms of sequence b presented as sequence 0 of a one-sequence batch."""

    def __init__(self, uni, b):
        self.uni, self.b = uni, b

    def __call__(self, bb, s):
        return self.uni(self.b + bb, s)


def test_benchmarked_round(model8b):
    """B=1, ctx 2048, chain gamma=3 at temperature 1: the bench's round."""
    V = synth.LLAMA8B.vocab
    tokens, q = _chain_drafts(1, 3, V, 1.0, 1.0, seed=101)
    _round(model8b, 1, [2048], 4, tokens, q, sample=[0])


def test_batch8_chain(model8b):
    V = synth.LLAMA8B.vocab
    tokens, q = _chain_drafts(8, 3, V, 1.0, 1.0, seed=202)
    _round(model8b, 8, [1024] * 8, 4, tokens, q, sample=[0, 7])


def test_tree_4_4_2_2(model8b):
    V = synth.LLAMA8B.vocab
    tokens, q, parent = _tree_drafts(4, [4, 4, 2, 2], V, 1.0, seed=303)
    assert parent.shape[1] == 117
    _round(model8b, 4, [4096] * 4, 117, tokens, q, sample=[2], parent=parent)


def test_long_context_gamma7(model8b):
    V = synth.LLAMA8B.vocab
    tokens, q = _chain_drafts(16, 7, V, 1.5, 0.0, seed=404)
    _round(model8b, 16, [32768] * 16, 8, tokens, None, sample=[5], temp=0.0)


def test_gamma1_b1(model8b):
    """B=1, ctx 2048, gamma=1 (two rows: the 2-row GEMM kernels at full width)."""
    V = synth.LLAMA8B.vocab
    tokens, q = _chain_drafts(1, 1, V, 1.0, 1.0, seed=111)
    _round(model8b, 1, [2048], 2, tokens, q, sample=[0])


def test_gamma7_b1(model8b):
    """B=1, ctx 2048, gamma=7 (eight rows), a close draft (sigma 0.5)."""
    V = synth.LLAMA8B.vocab
    tokens, q = _chain_drafts(1, 7, V, 0.5, 1.0, seed=121)
    _round(model8b, 1, [2048], 8, tokens, q, sample=[0])


def test_batch32_chain(model8b):
    """B=32, ctx 1024, gamma=3: 128 rows on the large-tile GEMMs."""
    V = synth.LLAMA8B.vocab
    tokens, q = _chain_drafts(32, 3, V, 1.0, 1.0, seed=505)
    _round(model8b, 32, [1024] * 32, 4, tokens, q, sample=[0, 31])


def test_batch128_chain(model8b):
    """B=128, ctx 1024, gamma=3: 512 rows, the largest chain workload; the
    shared-logits tier covers all 128 sequences, the oracle's forward two."""
    V = synth.LLAMA8B.vocab
    tokens, q = _chain_drafts(128, 3, V, 1.0, 1.0, seed=606)
    _round(model8b, 128, [1024] * 128, 4, tokens, q, sample=[5, 77])


def test_long_context_gamma7_sampled(model8b):
    """B=16, ctx 32768, gamma=7 at temperature 1 (the long-context workload
    is reported greedy and sampled)."""
    V = synth.LLAMA8B.vocab
    tokens, q = _chain_drafts(16, 7, V, 1.5, 1.0, seed=414)
    _round(model8b, 16, [32768] * 16, 8, tokens, q, sample=[9])


def test_tree_4_4_2_2_greedy(model8b):
    """B=4, ctx 4096, tree [4,4,2,2], greedy.  Each sequence's first child at
    every depth is set, depth by depth, to the target's argmax at its parent
    (a node's logits depend on its ancestors only), so the greedy walk goes
    down to a leaf instead of stopping at the root."""
    V = synth.LLAMA8B.vocab
    tokens, q, parent = _tree_drafts(4, [4, 4, 2, 2], V, 1.0, seed=707)
    ch = synth.tree_children(parent[0].cpu().tolist())

    def prepare(eng, kv, tok):
        tok = tok.clone()
        z = torch.empty((4, 117, V), device=dev())
        node = [0] * 4
        for _ in range(4):
            eng.step(tok, kv, z, tree_parent=parent)
            torch.cuda.synchronize()
            for b in range(4):
                first = ch[node[b]][0]
                tok[b, first] = int(z[b, node[b]].argmax())
                node[b] = first
        return tok

    n = _round(model8b, 4, [4096] * 4, 117, tokens, None, sample=[1], parent=parent, temp=0.0, prepare=prepare)
    # every first child is its parent's argmax: the walk reaches a leaf
    # (depth 4), unless an argmax gap is a near-tie the comparison excused
    assert (n == 4).sum() >= 3, n
