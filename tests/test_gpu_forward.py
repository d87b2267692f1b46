"""Parity of spec_verify_step (and a full verify round) with the oracle's
forward on the same seeded weights, cache and tokens.

Bars: logits per row max|dz| / max|z| <= 2e-2 (the target contract; the
fp32-activation path lands far below it); cache slots written by the step equal
the oracle's bf16 rounding of its own K/V except for rare one-ulp rounding
ties; accept decisions equal the oracle's apart from counted near-ties."""
import numpy as np
import pytest
import torch

import synth
from oracle import accept as OA
from oracle import model as OM
from oracle import philox
from oracle.numerics import bf16_bits_to_f64
from tests.gpu_util import LOGIT_RTOL, build_engine, compare_decisions, dev, logits_rel_err
from tests.gpu_util import bf16_close as _bf16_close
from tests.gpu_util import oracle_cache, oracle_weights

pytestmark = pytest.mark.gpu


def _run_step(eng, tokens, kv_len, parent=None):
    B, T = tokens.shape
    logits = torch.full((B, T, eng.shape.vocab), float("nan"), device=dev())
    eng.step(tokens, kv_len, logits, parent)
    torch.cuda.synchronize()
    return logits


def test_toy_prefill_and_verify_round():
    """Toy decoder (2 layers, d=256, fp32): each side prefills the 32-token
    prompt itself, then verifies a gamma=4 chain drafted by the noisy-target
    draft (sigma=1) from the oracle's own logits; temperature 1 and greedy."""
    sh = synth.TOY
    print("[toy] prefill 32 + verify gamma=4", flush=True)
    max_ctx, gamma = 128, 4
    eng, names, w, cache = build_engine(sh, 1, max_ctx, 32, ctx_len=0)
    W = oracle_weights(names, w)
    kc, vc = oracle_cache(cache, sh, 1, max_ctx)
    prompt = synth.make_tokens(1, 32, sh.vocab, seed=synth.SEED_PROMPT, device=dev())
    zero = torch.zeros(1, dtype=torch.int32, device=dev())
    zg = _run_step(eng, prompt, zero)
    zo, kn, vn = OM.forward(sh, W, prompt.cpu().numpy(), np.array([0]), kc, vc)
    err = logits_rel_err(zg.cpu().numpy(), zo)
    print(f"  prefill logits rel err max {err.max():.2e}", flush=True)
    assert err.max() < 1e-4
    OM.write_suffix(kc, vc, kn, vn, np.array([0]))
    # cache rows written by the GPU prefill vs the oracle's bf16 rounding
    kg, vg = oracle_cache(cache, sh, 1, max_ctx)
    _bf16_close(kg[:, :, :, :32], kc[:, :, :, :32])
    _bf16_close(vg[..., :32], vc[..., :32])

    for temp in (1.0, 0.0):
        y0 = int(np.argmax(zo[0, -1]))
        # draft from the oracle's logits, one position at a time
        kd, vd = kc.copy(), vc.copy()
        toks, zrows, qrows = [y0], [], []
        gq = torch.Generator().manual_seed(11 if temp else 12)
        for i in range(gamma):
            zi, kn1, vn1 = OM.forward(sh, W, np.array([[toks[-1]]]), np.array([32 + i]), kd, vd)
            OM.write_suffix(kd, vd, kn1, vn1, np.array([32 + i]))
            zt = torch.from_numpy(zi[0, 0]).float()
            q, zn = synth.noisy_draft_dist(zt[None], 1.0, 100 + i + (0 if temp else 50), 1.0)
            x = int(torch.multinomial(q[0].double(), 1, generator=gq)) if temp else int(zn[0].argmax())
            toks.append(x)
            qrows.append(q[0])
        tokens = torch.tensor([toks], dtype=torch.int32, device=dev())
        kv = torch.tensor([32], dtype=torch.int32, device=dev())
        zg = _run_step(eng, tokens, kv)
        zo, kn, vn = OM.forward(sh, W, tokens.cpu().numpy(), np.array([32]), kc, vc)
        err = logits_rel_err(zg.cpu().numpy(), zo)
        print(f"  verify T={temp} logits rel err max {err.max():.2e}", flush=True)
        assert err.max() < 1e-4
        q = torch.stack(qrows)[None].to(dev())
        out = torch.zeros((1, gamma + 1), dtype=torch.int32, device=dev())
        nacc = torch.zeros((1,), dtype=torch.int32, device=dev())
        kv_out = torch.zeros((1,), dtype=torch.int32, device=dev())
        eng.accept(zg, q, tokens, out, nacc, kv, kv_out, temperature=temp, seed=9, round_=1)
        torch.cuda.synchronize()
        orc = OA.accept(zo, q.double().cpu().numpy(), tokens.cpu().numpy(), temp, philox.Uniforms(9, 1))
        compare_decisions(out.cpu().numpy(), nacc.cpu().numpy(), orc, f"toy T={temp}")
        assert int(kv_out[0]) == 32 + int(nacc[0]) + 1
        print(f"  T={temp}: accepted {int(nacc[0])}, out {out.cpu().tolist()}", flush=True)
    assert eng.device_errors() == 0


GQA_CASES = [
    # B, T, ctx lengths, tree branching or None
    (1, 1, [300], None),
    (3, 4, [300, 1, 777], None),
    (2, 8, [1000, 64], None),
    # a 16-row chain: 64 queries per KV head, the widest chain of the LDS form
    (2, 16, [997, 33], None),
    (2, 15, [129, 500], [2, 2, 2]),
    (1, 7, [0], None),
    # a deep tree (a 71-node chain, then a fork): nodes with more than 64
    # ancestors, several batches of visible suffix rows per query
    (1, 74, [200], [1] * 71 + [2]),
    # one row at 5000 and 8000 keys: 40 and 60 context splits, so the combine
    # merges 41 and 61 partials, 8 per round of requests after the first
    (1, 1, [5000], None),
    (1, 1, [8000], None),
]


@pytest.mark.parametrize("B,T,ctx,branching", GQA_CASES)
def test_gqa_bf16_step_matches_oracle(B, T, ctx, branching):
    """8B-like layout (32 q / 8 kv heads of 128, d=4096, bf16) with two layers,
    a short FFN and vocab, synthetic bf16 cache of ragged lengths with a NaN
    poisoned tail: logits and written cache slots against the oracle."""
    _gqa_step_case(synth.MINI8B, B, T, ctx, branching)


# The same layout with 4 KV heads: 8 query heads per KV head, so a suffix
# wave's four queries (trees; chains of 128 or more (sequence, KV head)
# pairs) start at head 0 or head 4 of their row.
G8 = synth.ModelShape(n_layers=2, d_model=4096, n_heads=32, n_kv_heads=4, head_dim=128,
                      d_ffn=1024, vocab=8192, rms_eps=1e-5, rope_theta=500000.0, weight_dtype="bf16")
G8_CASES = [
    # B, T, ctx lengths, tree branching or None: trees and 32-sequence chains
    # on the register form (16 queries per KV head) and the LDS form (more)
    (1, 2, [400], [1]),
    (2, 15, [300, 57], [2, 2, 2]),
    (32, 2, [150] * 31 + [3], None),
    (32, 4, [200] * 31 + [3], None),
]


@pytest.mark.parametrize("B,T,ctx,branching", G8_CASES)
def test_gqa_group8_step_matches_oracle(B, T, ctx, branching):
    """8 query heads per KV head: logits and written cache slots against the
    oracle, on trees and on a chain batch of 128 (sequence, KV head) pairs."""
    _gqa_step_case(G8, B, T, ctx, branching)


def _gqa_step_case(sh, B, T, ctx, branching):
    print(f"[gqa] G={sh.n_heads // sh.n_kv_heads} B={B} T={T} ctx={ctx} tree={branching}", flush=True)
    max_ctx = max(1088, (max(ctx) + T + 63) // 64 * 64)
    nb = max(4, B)
    eng, names, w, cache = build_engine(sh, nb, max_ctx, max(16, T), ctx_len=ctx + [0] * (nb - B))
    W = oracle_weights(names, w)
    kc, vc = oracle_cache(cache, sh, nb, max_ctx)
    tokens = synth.make_tokens(B, T, sh.vocab, seed=77 + T, device=dev())
    kv = torch.tensor(ctx, dtype=torch.int32, device=dev())
    parent = synth.random_tree(branching, B).to(dev()) if branching else None
    assert parent is None or parent.shape[1] == T
    zg = _run_step(eng, tokens, kv, parent)
    assert torch.isfinite(zg).all()
    zo, kn, vn = OM.forward(sh, W, tokens.cpu().numpy(), np.array(ctx), kc[:, :B], vc[:, :B],
                            tree_parent=None if parent is None else parent.cpu().numpy())
    err = logits_rel_err(zg.cpu().numpy(), zo)
    print(f"  logits rel err max {err.max():.2e} median {np.median(err):.2e}", flush=True)
    assert err.max() < 1e-3
    # the step wrote every row's K/V at slot kv_len + i
    kg, vg = oracle_cache(cache, sh, nb, max_ctx)
    ko, vo = kc.copy(), vc.copy()
    OM.write_suffix(ko[:, :B], vo[:, :B], kn, vn, np.array(ctx))
    for b in range(B):
        s0, s1 = ctx[b], ctx[b] + T
        _bf16_close(kg[:, b, :, s0:s1], ko[:, b, :, s0:s1])
        _bf16_close(vg[:, b, :, :, s0:s1], vo[:, b, :, :, s0:s1])
        # nothing before the window changed
        assert np.array_equal(kg[:, b, :, :s0], kc[:, b, :, :s0])
    assert eng.device_errors() == 0


FFN_CASES = [
    # B, T, ctx lengths: M = 1, 2 (the 2-row k-stationary and streaming
    # kernels), 3 and 4 (split-K down whose sum the next QKV launch adds,
    # matrix-core gate/up), 6 and 8 (split-K down + reduce, tiled QKV), 12
    (1, 1, [700]),
    (1, 2, [700]),
    (1, 6, [700]),
    (1, 3, [700]),
    (1, 4, [700]),
    (2, 4, [700, 33]),
    (3, 4, [5, 700, 129]),
]


@pytest.mark.parametrize("B,T,ctx", FFN_CASES)
def test_full_width_ffn_step_matches_oracle(B, T, ctx):
    """The 8B layer at full width (FFN 14336, K = 14336 for the down
    projection) with two layers: every GEMM path the 8B model takes at these
    row counts, against the oracle's logits and cache."""
    sh = synth.FFN8B
    print(f"[ffn] B={B} T={T} ctx={ctx}", flush=True)
    max_ctx = 768
    eng, names, w, cache = build_engine(sh, 3, max_ctx, 8, ctx_len=ctx + [0] * (3 - B))
    W = oracle_weights(names, w)
    kc, vc = oracle_cache(cache, sh, 3, max_ctx)
    tokens = synth.make_tokens(B, T, sh.vocab, seed=91 + T, device=dev())
    kv = torch.tensor(ctx, dtype=torch.int32, device=dev())
    zg = _run_step(eng, tokens, kv)
    assert torch.isfinite(zg).all()
    zo, kn, vn = OM.forward(sh, W, tokens.cpu().numpy(), np.array(ctx), kc[:, :B], vc[:, :B])
    err = logits_rel_err(zg.cpu().numpy(), zo)
    print(f"  logits rel err max {err.max():.2e} median {np.median(err):.2e}", flush=True)
    assert err.max() < 1e-3
    kg, vg = oracle_cache(cache, sh, 3, max_ctx)
    ko, vo = kc.copy(), vc.copy()
    OM.write_suffix(ko[:, :B], vo[:, :B], kn, vn, np.array(ctx))
    for b in range(B):
        s0, s1 = ctx[b], ctx[b] + T
        _bf16_close(kg[:, b, :, s0:s1], ko[:, b, :, s0:s1])
        _bf16_close(vg[:, b, :, :, s0:s1], vo[:, b, :, :, s0:s1])
    assert eng.device_errors() == 0


def test_step_flags_bad_inputs_without_faulting():
    sh = synth.MINI8B
    max_ctx = 128
    eng, names, w, cache = build_engine(sh, 2, max_ctx, 8, ctx_len=[10, 10])
    tokens = synth.make_tokens(2, 4, sh.vocab, seed=3, device=dev())
    tokens[1, 2] = -3
    kv = torch.tensor([10, max_ctx - 2], dtype=torch.int32, device=dev())  # second overflows
    logits = torch.zeros((2, 4, sh.vocab), device=dev())
    eng.step(tokens, kv, logits)
    torch.cuda.synchronize()
    flags = eng.device_errors()
    assert flags & 1 and flags & 4
    bad_tree = torch.tensor([[-1, 0, 2, 1]] * 2, dtype=torch.int32, device=dev())
    kv = torch.tensor([10, 10], dtype=torch.int32, device=dev())
    tokens[1, 2] = 5
    eng.step(tokens, kv, logits, bad_tree)
    torch.cuda.synchronize()
    assert eng.device_errors() == 2
    assert eng.device_errors() == 0  # reading clears the word
