"""Multi-round invariants of speculative decoding run entirely on the HIP path
(prefill, draft decodes, verify, accept, commit; toy decoder, fp32 weights).
Rounds diverge from any other implementation at the first near-tie, so they
are judged by what the method guarantees over many rounds, not row by row:

  * per-position acceptance of the noisy-target draft (q = softmax(z + eps),
    eps ~ N(0, sigma^2)) against its closed form 2 Phi(-sigma/2), and the mean
    tokens per round against eq. (1), (1 - alpha^(gamma+1)) / (1 - alpha), at
    the measured alpha (CS349E Lecture 6, sections 8.1 and 8.3: independent
    positions);
  * speculative greedy decoding emits exactly the target's greedy decoding
    (section 7.4)."""
import math

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import build_engine, dev

pytestmark = pytest.mark.gpu

PROMPT = 32


def _prefill(eng, sh):
    prompt = synth.make_tokens(1, PROMPT, sh.vocab, seed=synth.SEED_PROMPT, device=dev())
    z = torch.empty((1, PROMPT, sh.vocab), device=dev())
    eng.step(prompt, torch.zeros(1, dtype=torch.int32, device=dev()), z)
    return int(z[0, -1].argmax())


def _draft(eng, sh, pending, kv, gamma, sigma, temperature, seed):
    """gamma sequential T=1 decodes of the target give z_i for each drafted
    prefix; the draft distribution is q_i = softmax(z_i + eps_i)."""
    toks, qs = [pending], []
    z1 = torch.empty((1, 1, sh.vocab), device=dev())
    for i in range(gamma):
        t = torch.tensor([[toks[-1]]], dtype=torch.int32, device=dev())
        eng.step(t, kv + i, z1)
        q, zn = synth.noisy_draft_dist(z1[:, 0], sigma, seed * 16 + i, temperature if temperature > 0 else 1.0)
        if temperature > 0:
            x = int(synth.sample_from(q, seed * 16 + 8 + i)[0, 0])
        else:
            x = int(zn[0].argmax())
        toks.append(x)
        qs.append(q)
    tokens = torch.tensor([toks], dtype=torch.int32, device=dev())
    q = torch.stack(qs, 1).contiguous() if temperature > 0 else None
    return tokens, q


def test_acceptance_and_tokens_per_round_closed_forms():
    """128 rounds at gamma = 4, sigma = 1, temperature 1."""
    sh = synth.TOY
    gamma, sigma, R = 4, 1.0, 128
    max_ctx = ((PROMPT + R * (gamma + 1) + gamma + 64) // 64) * 64
    eng, *_ = build_engine(sh, 1, max_ctx, PROMPT, ctx_len=[0], poison=False)
    pending = _prefill(eng, sh)
    kv = torch.tensor([PROMPT], dtype=torch.int32, device=dev())
    logits = torch.empty((1, gamma + 1, sh.vocab), device=dev())
    out = torch.empty((1, gamma + 1), dtype=torch.int32, device=dev())
    nacc = torch.empty((1,), dtype=torch.int32, device=dev())
    kv_out = torch.empty_like(kv)
    ns = []
    for r in range(R):
        tokens, q = _draft(eng, sh, pending, kv, gamma, sigma, 1.0, seed=1000 + r)
        eng.step(tokens, kv, logits)
        eng.accept(logits, q, tokens, out, nacc, kv, kv_out, temperature=1.0, seed=synth.SEED_ACCEPT, round_=r)
        torch.cuda.synchronize()
        n = int(nacc[0])
        assert 0 <= n <= gamma and int(kv_out[0]) == int(kv[0]) + n + 1
        ns.append(n)
        pending = int(out[0, n])
        kv = kv_out.clone()
    assert eng.device_errors() == 0
    ns = np.array(ns)
    passed = ns.sum()
    reached = np.minimum(ns + 1, gamma).sum()
    alpha = passed / reached
    beta = 2.0 * 0.5 * math.erfc((sigma / 2.0) / math.sqrt(2.0))  # 2 Phi(-sigma/2)
    se_a = math.sqrt(alpha * (1 - alpha) / reached)
    tpr = (ns + 1).mean()
    se_t = (ns + 1).std(ddof=1) / math.sqrt(R)
    e1 = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    print(f"  alpha {alpha:.4f} +- {se_a:.4f} (2 Phi(-sigma/2) = {beta:.4f}); tokens/round {tpr:.4f} +- {se_t:.4f} "
          f"(eq. 1 at alpha: {e1:.4f})", flush=True)
    assert abs(alpha - beta) < 3 * se_a
    assert abs(tpr - e1) < 3 * se_t


def test_speculative_greedy_equals_greedy_decoding():
    """64 tokens of speculative greedy decoding (gamma = 4, drafts the argmax
    of the noisy target) against 64 plain greedy T=1 decode steps from the
    same prefill, token for token.  Should the two ever part, it must be at a
    top-2 near-tie of the plain decode's logits (the two paths sum in
    different orders)."""
    sh = synth.TOY
    gamma, sigma, L = 4, 0.2, 64
    max_ctx = ((PROMPT + 2 * L + gamma + 64) // 64) * 64
    eng, *_ = build_engine(sh, 1, max_ctx, PROMPT, ctx_len=[0], poison=False)
    y0 = _prefill(eng, sh)

    kv = torch.tensor([PROMPT], dtype=torch.int32, device=dev())
    logits = torch.empty((1, gamma + 1, sh.vocab), device=dev())
    out = torch.empty((1, gamma + 1), dtype=torch.int32, device=dev())
    nacc = torch.empty((1,), dtype=torch.int32, device=dev())
    kv_out = torch.empty_like(kv)
    spec, pending, r, accepted = [y0], y0, 0, 0
    while len(spec) < L:
        tokens, _ = _draft(eng, sh, pending, kv, gamma, sigma, 0.0, seed=5000 + r)
        eng.step(tokens, kv, logits)
        eng.accept(logits, None, tokens, out, nacc, kv, kv_out, temperature=0.0, seed=1, round_=r)
        torch.cuda.synchronize()
        n = int(nacc[0])
        accepted += n
        spec += [int(t) for t in out[0, :n + 1].cpu()]
        pending = spec[-1]
        kv = kv_out.clone()
        r += 1
    assert accepted > 0, "the drafts were never right: the check would not exercise multi-token rounds"

    # plain greedy decoding from the same prefill (the cache rows < PROMPT are
    # untouched by the rounds above; every later row is rewritten before use)
    kv = torch.tensor([PROMPT], dtype=torch.int32, device=dev())
    z1 = torch.empty((1, 1, sh.vocab), device=dev())
    plain, gaps, pending = [y0], [], y0
    while len(plain) < L:
        eng.step(torch.tensor([[pending]], dtype=torch.int32, device=dev()), kv, z1)
        torch.cuda.synchronize()
        top = torch.topk(z1[0, 0].double(), 2).values
        gaps.append(float((top[0] - top[1]) / z1[0, 0].abs().max()))
        pending = int(z1[0, 0].argmax())
        plain.append(pending)
        kv = kv + 1
    assert eng.device_errors() == 0
    print(f"  {r} rounds, {accepted} drafts accepted; smallest top-2 gap {min(gaps):.2e}", flush=True)
    for i in range(L):
        if spec[i] != plain[i]:
            assert gaps[i - 1] < 1e-4, (i, spec[:i + 1], plain[:i + 1], gaps[i - 1])
            break


def test_live_rounds_match_the_oracle_end_to_end():
    """30 live rounds on the HIP path (the step's own prefill, gamma T=1
    draft decodes, verify, accept, commit; gamma = 4, sigma = 1) at
    temperature 1 and greedy, replayed by the oracle from its own prefill and
    its own commits with the same drafts, q and uniforms: every round agrees
    (a near tie, should one occur, ends the comparison and is counted; no
    mismatch is allowed), and the logits stay within 1e-4 of the oracle's."""
    import bench

    sh = synth.TOY
    R = 30
    print(f"[multiround] toy live rounds against the oracle, R={R}", flush=True)
    max_ctx = ((bench.TOY_PROMPT + R * (bench.TOY_GAMMA + 1) + bench.TOY_GAMMA + 64) // 64) * 64
    eng, names, w, _ = build_engine(sh, 1, max_ctx, bench.TOY_PROMPT, ctx_len=[0], poison=False)
    prompt = synth.make_tokens(1, bench.TOY_PROMPT, sh.vocab, seed=synth.SEED_PROMPT, device=dev())
    modes = {t: {"recs": bench.toy_live(eng, sh, prompt, R, t, 1.0, dev())[1]} for t in (1.0, 0.0)}
    assert eng.device_errors() == 0
    _, near = bench.toy_oracle(sh, names, w, prompt, modes)
    for key, rep in near["end_to_end"].items():
        print(f"  {key}: {rep}", flush=True)
        assert rep["mismatches"] == 0, rep
        assert rep["rounds_compared"] == R or rep["near_tie_differences"] == 1, rep
        assert rep["max_logits_rel_err"] < 1e-4, rep
