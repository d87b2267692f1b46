"""Parity of spec_accept with the oracle's accept on the same synthetic logits,
draft distributions, draft tokens and Philox uniforms.  Token ids and accept
counts must be bit-exact apart from counted near-ties (|u - min(1, p/q)| or
the CDF boundary distance below 1e-4, measured on the oracle's fp64 p, q)."""
import numpy as np
import pytest
import torch

import synth
from oracle import accept as OA
from oracle import philox
from tests.gpu_util import ADJUST_BAND, DRAW_BAND_SHARED, compare_decisions, dev

pytestmark = pytest.mark.gpu


def _accept_shape(V):
    return synth.ModelShape(n_layers=1, d_model=64, n_heads=1, n_kv_heads=1, head_dim=64, d_ffn=64,
                            vocab=V, rms_eps=1e-5, rope_theta=10000.0, weight_dtype="f32")


_engines = {}


def _engine(V, max_batch, max_rows, max_ctx=256):
    key = (V, max_batch, max_rows, max_ctx)
    if key not in _engines:
        from speculative_decoding_verify_spec_amd.engine import VerifyEngine
        sh = _accept_shape(V)
        _, w = synth.make_weights(sh, device=dev())
        cache = synth.make_kv_cache(sh, max_batch, max_ctx, max_ctx // 2, device=dev(), poison_tail=False)
        _engines[key] = VerifyEngine(sh, w, cache, max_batch, max_ctx, max_rows)
    return _engines[key]


def _chain_inputs(B, gamma, V, temperature, sigma, seed):
    T = gamma + 1
    z = synth.random_logits((B, T), V, seed=seed, device=dev())
    tokens = synth.make_tokens(B, T, V, seed=seed + 1, device=dev())
    if temperature > 0:
        q, _ = synth.noisy_draft_dist(z[:, :gamma], sigma, seed + 2, temperature)
        if gamma:
            tokens[:, 1:] = synth.sample_from(q, seed + 3)[..., 0]
    else:
        q = None
        _, zn = synth.noisy_draft_dist(z[:, :gamma], sigma, seed + 2, 0.0)
        if gamma:
            tokens[:, 1:] = zn.argmax(-1).to(torch.int32)
    return z, q, tokens


CHAIN_CASES = [
    # V, B, gamma, temperature, sigma
    (8, 4, 3, 1.0, 1.0),
    (8, 4, 1, 1.0, 3.0),
    (4099, 3, 4, 1.0, 1.0),
    (4099, 3, 7, 0.7, 0.5),
    (4099, 2, 0, 1.0, 1.0),
    (128256, 2, 3, 1.0, 1.0),
    (128256, 1, 7, 1.0, 0.5),
    (8, 4, 3, 0.0, 1.0),
    (4099, 3, 5, 0.0, 0.3),
    (128256, 2, 3, 0.0, 0.5),
    # the batch of the largest chain workload: 128 sequences, gamma = 3
    (128256, 128, 3, 1.0, 1.0),
    (128256, 128, 3, 0.0, 1.0),
]


@pytest.mark.parametrize("V,B,gamma,temp,sigma", CHAIN_CASES)
def test_chain_accept_matches_oracle(V, B, gamma, temp, sigma):
    print(f"[chain accept] V={V} B={B} gamma={gamma} T={temp} sigma={sigma}", flush=True)
    T = gamma + 1
    eng = _engine(V, max(4, B), 8)
    near, rounds, n_total = 0, 6 if B <= 8 else 2, 0
    for r in range(rounds):
        seed = 1000 * V % 9973 + 17 * r + gamma
        z, q, tokens = _chain_inputs(B, gamma, V, temp, sigma, seed)
        kv_len = torch.arange(5, 5 + B, dtype=torch.int32, device=dev())
        kv_out = torch.full((B,), -7, dtype=torch.int32, device=dev())
        out = torch.full((B, T), -5, dtype=torch.int32, device=dev())
        nacc = torch.full((B,), -5, dtype=torch.int32, device=dev())
        qq = q if q is not None else None
        eng.accept(z, qq, tokens, out, nacc, kv_len, kv_out, temperature=temp, seed=42 + r, round_=r)
        torch.cuda.synchronize()
        zn = z.double().cpu().numpy()
        qn = q.double().cpu().numpy() if q is not None else None
        orc = OA.accept(zn, qn, tokens.cpu().numpy(), temp, philox.Uniforms(42 + r, r))
        near += compare_decisions(out.cpu().numpy(), nacc.cpu().numpy(), orc, f"round {r}", draw_band=DRAW_BAND_SHARED)
        assert np.array_equal(kv_out.cpu().numpy(), kv_len.cpu().numpy() + nacc.cpu().numpy() + 1)
        n_total += B
        assert eng.device_errors() == 0
    print(f"  near-ties {near}/{n_total}", flush=True)
    assert near <= max(1, n_total // 20)


def _tree_inputs(B, branching, V, temperature, sigma, seed, replacement):
    parent = synth.random_tree(branching, B).to(dev())
    T = parent.shape[1]
    z = synth.random_logits((B, T), V, seed=seed, device=dev())
    tokens = synth.make_tokens(B, T, V, seed=seed + 1, device=dev())
    q, zn = synth.noisy_draft_dist(z, sigma, seed + 2, temperature if temperature > 0 else 1.0)
    ch = synth.tree_children(parent[0].cpu().tolist())
    g = torch.Generator(device="cpu").manual_seed(seed + 3)
    tok = tokens.cpu()
    for b in range(B):
        for v in range(T):
            kids = ch[v]
            if not kids:
                continue
            if temperature > 0:
                picks = torch.multinomial(q[b, v].double().cpu(), len(kids), replacement=replacement, generator=g)
            else:
                picks = torch.topk(zn[b, v].cpu(), len(kids)).indices
            for c, x in zip(kids, picks.tolist()):
                tok[b, c] = x
    return z, q, tok.to(torch.int32).to(dev()), parent


TREE_CASES = [
    # V, B, branching, temperature, replacement
    (16, 3, [2, 2], 1.0, False),
    (4099, 2, [4, 2, 2], 1.0, False),
    (4099, 2, [3, 2], 1.0, True),
    (128256, 1, [4, 4, 2, 2], 1.0, False),
    (4099, 2, [4, 2, 2], 0.0, False),
    (128256, 2, [2, 2, 1], 0.0, False),
]


@pytest.mark.parametrize("V,B,branching,temp,repl", TREE_CASES)
def test_tree_accept_matches_oracle(V, B, branching, temp, repl):
    print(f"[tree accept] V={V} B={B} branching={branching} T={temp} replacement={repl}", flush=True)
    max_rows = 1 + sum(int(np.prod(branching[:i + 1])) for i in range(len(branching)))
    eng = _engine(V, 4, 128, max_ctx=512)
    near, n_total = 0, 0
    for r in range(4):
        seed = 31 * V % 7919 + 13 * r
        z, q, tokens, parent = _tree_inputs(B, branching, V, temp, 0.8, seed, repl)
        T = parent.shape[1]
        assert T == max_rows
        kv_len = torch.full((B,), 100, dtype=torch.int32, device=dev())
        # odd rounds update the lengths in place (kv_len_out may alias kv_len)
        kv_out = kv_len if r % 2 else torch.zeros((B,), dtype=torch.int32, device=dev())
        out = torch.full((B, T), -5, dtype=torch.int32, device=dev())
        nacc = torch.full((B,), -5, dtype=torch.int32, device=dev())
        k_before, v_before = synth.kv_views(eng.kv_cache.clone(), _accept_shape(V), 4, 512)
        eng.accept(z, q if temp > 0 else None, tokens, out, nacc, kv_len, kv_out, tree_parent=parent,
                   temperature=temp, seed=7 + r, round_=r, replacement=repl)
        torch.cuda.synchronize()
        orc = OA.accept(z.double().cpu().numpy(), q.double().cpu().numpy() if temp > 0 else None,
                        tokens.cpu().numpy(), temp, philox.Uniforms(7 + r, r),
                        tree_parent=parent.cpu().numpy(), replacement=repl)
        near += compare_decisions(out.cpu().numpy(), nacc.cpu().numpy(), orc, f"round {r}", draw_band=DRAW_BAND_SHARED)
        n_total += B
        assert eng.device_errors() == 0
        # commit: the accepted path's K/V now sit at slots kv_len + 0..n
        k_after, v_after = synth.kv_views(eng.kv_cache, _accept_shape(V), 4, 512)
        n = nacc.cpu().numpy()
        assert np.array_equal(kv_out.cpu().numpy(), 100 + n + 1)
        for b in range(B):
            path = orc["paths"][b]
            if int(n[b]) != len(path) - 1:
                continue  # a near-tie took another path
            for j, node in enumerate(path):
                assert torch.equal(k_after[:, b, :, 100 + j], k_before[:, b, :, 100 + node])
                assert torch.equal(v_after[:, b, :, :, 100 + j], v_before[:, b, :, :, 100 + node])
    print(f"  near-ties {near}/{n_total}", flush=True)
    assert near <= max(1, n_total // 10)


def test_tree_walk_longer_than_its_step_launches():
    """A root with 16 children drafted from a far-off draft (sigma 4: each is
    accepted with probability ~2 Phi(-2) ~ 0.05) needs up to 16 rejection
    passes plus the draw, more than the step launches the walk gets: the pick
    kernel finishes those walks in one workgroup, against the same oracle."""
    V, B, branching = 4099, 4, [16, 1]
    eng = _engine(V, 4, 128, max_ctx=512)
    near, n_total, long_walks = 0, 0, 0
    for r in range(3):
        seed = 977 + r
        z, q, tokens, parent = _tree_inputs(B, branching, V, 1.0, 4.0, seed, False)
        T = parent.shape[1]
        print(f"[tree walk] V={V} B={B} branching={branching} round {r}", flush=True)
        kv_len = torch.full((B,), 100, dtype=torch.int32, device=dev())
        out = torch.full((B, T), -5, dtype=torch.int32, device=dev())
        nacc = torch.full((B,), -5, dtype=torch.int32, device=dev())
        eng.accept(z, q, tokens, out, nacc, kv_len, None, tree_parent=parent, temperature=1.0, seed=11 + r,
                   round_=r, replacement=False)
        torch.cuda.synchronize()
        orc = OA.accept(z.double().cpu().numpy(), q.double().cpu().numpy(), tokens.cpu().numpy(), 1.0,
                        philox.Uniforms(11 + r, r), tree_parent=parent.cpu().numpy(), replacement=False)
        near += compare_decisions(out.cpu().numpy(), nacc.cpu().numpy(), orc, f"round {r}", draw_band=DRAW_BAND_SHARED)
        n_total += B
        assert eng.device_errors() == 0
        # rejections at the root (children are tested in id order): with the
        # draw pass, 12 or more take more passes than the 12 step launches
        for b in range(B):
            path = orc["paths"][b]
            rejected = path[1] - 1 if len(path) > 1 else 16
            long_walks += rejected >= 12
    print(f"  near-ties {near}/{n_total}, walks past 12 rejections {long_walks}", flush=True)
    assert long_walks > 0, "no walk needed the one-workgroup finish"
    assert near <= max(1, n_total // 10)


def test_accept_flags_bad_draft_token():
    V, B, gamma = 4099, 2, 3
    eng = _engine(V, 4, 8)
    z, q, tokens = _chain_inputs(B, gamma, V, 1.0, 1.0, 5)
    tokens[0, 2] = V + 5
    kv_len = torch.zeros((B,), dtype=torch.int32, device=dev())
    out = torch.zeros((B, gamma + 1), dtype=torch.int32, device=dev())
    nacc = torch.zeros((B,), dtype=torch.int32, device=dev())
    eng.accept(z, q, tokens, out, nacc, kv_len, None, temperature=1.0, seed=1, round_=0)
    torch.cuda.synchronize()
    flags = eng.device_errors()
    assert flags & 1
    assert int(nacc[0]) <= 1  # the bad draft is never accepted


# ----------------------------------------------------------------------------
# top-k / top-p adjusted target (CS349E Lecture 6, section 7.3)
# ----------------------------------------------------------------------------

def _adjusted_rows(zn, temperature, top_k, top_p):
    """The draft side applies the same adjustment to its own logits (oracle
    arithmetic on the host; the drafted tokens are then sampled from it)."""
    zz = zn.double().cpu().numpy()
    flat = zz.reshape(-1, zz.shape[-1])
    q = np.stack([OA.adjust(r, temperature, top_k, top_p)[0] for r in flat]).reshape(zz.shape)
    q = torch.from_numpy(q).float()
    return (q / q.sum(dim=-1, keepdim=True)).to(dev())


def _logits(rows_shape, V, seed, scale, ties):
    z = synth.random_logits(rows_shape, V, seed=seed, device=dev(), scale=scale)
    if ties:
        z = torch.round(z * 2.0) / 2.0  # about V / 64 tokens share each logit value
    return z


ADJ_CHAIN_CASES = [
    # V, B, gamma, temperature, sigma, top_k, top_p, logit scale, ties
    (8, 4, 3, 1.0, 1.0, 3, 1.0, 1.28, False),
    (8, 4, 3, 1.0, 1.0, 0, 0.6, 1.28, False),
    (4099, 3, 4, 1.0, 1.0, 20, 1.0, 4.0, False),
    (4099, 3, 3, 0.7, 0.5, 0, 0.9, 4.0, False),
    (4099, 2, 3, 1.0, 1.0, 30, 0.8, 4.0, True),
    (4099, 2, 2, 1.0, 1.0, 0, 0.0, 4.0, True),
    (128256, 2, 3, 1.0, 1.0, 50, 0.9, 4.0, False),
    (128256, 1, 5, 1.0, 0.5, 0, 0.95, 4.0, False),
    (128256, 2, 3, 1.0, 1.0, 2000, 1.0, 1.28, False),
    # 160 logits rows: more than one batch of the selection passes (128 rows)
    (4099, 40, 3, 1.0, 1.0, 20, 0.9, 4.0, False),
]


@pytest.mark.parametrize("V,B,gamma,temp,sigma,top_k,top_p,scale,ties", ADJ_CHAIN_CASES)
def test_chain_accept_adjusted_matches_oracle(V, B, gamma, temp, sigma, top_k, top_p, scale, ties):
    print(f"[chain accept adjusted] V={V} B={B} gamma={gamma} T={temp} top_k={top_k} top_p={top_p} "
          f"scale={scale} ties={ties}", flush=True)
    T = gamma + 1
    eng = _engine(V, max(4, B), 8)
    near, n_total = 0, 0
    for r in range(6):
        seed = 777 * V % 9973 + 29 * r + gamma
        z = _logits((B, T), V, seed, scale, ties)
        tokens = synth.make_tokens(B, T, V, seed=seed + 1, device=dev())
        _, zn = synth.noisy_draft_dist(z[:, :gamma], sigma, seed + 2, temp)
        q = _adjusted_rows(zn, temp, top_k, top_p)
        if gamma:
            tokens[:, 1:] = synth.sample_from(q, seed + 3)[..., 0]
        kv_len = torch.arange(5, 5 + B, dtype=torch.int32, device=dev())
        kv_out = torch.full((B,), -7, dtype=torch.int32, device=dev())
        out = torch.full((B, T), -5, dtype=torch.int32, device=dev())
        nacc = torch.full((B,), -5, dtype=torch.int32, device=dev())
        eng.accept(z, q, tokens, out, nacc, kv_len, kv_out, temperature=temp, seed=42 + r, round_=r,
                   top_k=top_k, top_p=top_p)
        torch.cuda.synchronize()
        orc = OA.accept(z.double().cpu().numpy(), q.double().cpu().numpy(), tokens.cpu().numpy(), temp,
                        philox.Uniforms(42 + r, r), top_k=top_k, top_p=top_p)
        near += compare_decisions(out.cpu().numpy(), nacc.cpu().numpy(), orc, f"round {r}", draw_band=DRAW_BAND_SHARED)
        # the extra token lies in the adjusted support of its row (unless that
        # row's nucleus cut is itself a near-tie)
        for b in range(B):
            n = int(nacc[b])
            p_row, am = OA.adjust(z[b, n].double().cpu().numpy(), temp, top_k, top_p)
            assert p_row[int(out[b, n])] > 0.0 or am < ADJUST_BAND, (b, n, int(out[b, n]))
        assert np.array_equal(kv_out.cpu().numpy(), kv_len.cpu().numpy() + nacc.cpu().numpy() + 1)
        n_total += B
        assert eng.device_errors() == 0
    print(f"  near-ties {near}/{n_total}", flush=True)
    assert near <= max(1, n_total // 20)


ADJ_TREE_CASES = [
    # V, B, branching, top_k, top_p, adjust the draft too
    (4099, 2, [4, 2, 2], 10, 1.0, True),
    (4099, 2, [3, 2], 0, 0.9, False),
    (128256, 1, [4, 4, 2, 2], 40, 0.95, False),
]


@pytest.mark.parametrize("V,B,branching,top_k,top_p,adjust_q", ADJ_TREE_CASES)
def test_tree_accept_adjusted_matches_oracle(V, B, branching, top_k, top_p, adjust_q):
    print(f"[tree accept adjusted] V={V} B={B} branching={branching} top_k={top_k} top_p={top_p} "
          f"adjust_q={adjust_q}", flush=True)
    eng = _engine(V, 4, 128, max_ctx=512)
    near, n_total = 0, 0
    for r in range(4):
        seed = 53 * V % 7919 + 11 * r
        parent = synth.random_tree(branching, B).to(dev())
        T = parent.shape[1]
        z = _logits((B, T), V, seed, 4.0, False)
        tokens = synth.make_tokens(B, T, V, seed=seed + 1, device=dev())
        q, zn = synth.noisy_draft_dist(z, 0.8, seed + 2, 1.0)
        if adjust_q:
            q = _adjusted_rows(zn, 1.0, top_k, top_p)
        ch = synth.tree_children(parent[0].cpu().tolist())
        g = torch.Generator(device="cpu").manual_seed(seed + 3)
        tok = tokens.cpu()
        for b in range(B):
            for v in range(T):
                if ch[v]:
                    picks = torch.multinomial(q[b, v].double().cpu(), len(ch[v]), replacement=False, generator=g)
                    for c, x in zip(ch[v], picks.tolist()):
                        tok[b, c] = x
        tokens = tok.to(torch.int32).to(dev())
        kv_len = torch.full((B,), 100, dtype=torch.int32, device=dev())
        kv_out = torch.zeros((B,), dtype=torch.int32, device=dev())
        out = torch.full((B, T), -5, dtype=torch.int32, device=dev())
        nacc = torch.full((B,), -5, dtype=torch.int32, device=dev())
        eng.accept(z, q, tokens, out, nacc, kv_len, kv_out, tree_parent=parent, temperature=1.0, seed=7 + r,
                   round_=r, top_k=top_k, top_p=top_p)
        torch.cuda.synchronize()
        orc = OA.accept(z.double().cpu().numpy(), q.double().cpu().numpy(), tokens.cpu().numpy(), 1.0,
                        philox.Uniforms(7 + r, r), tree_parent=parent.cpu().numpy(), top_k=top_k, top_p=top_p)
        near += compare_decisions(out.cpu().numpy(), nacc.cpu().numpy(), orc, f"round {r}", draw_band=DRAW_BAND_SHARED)
        n_total += B
        assert eng.device_errors() == 0
    print(f"  near-ties {near}/{n_total}", flush=True)
    assert near <= max(1, n_total // 10)


DEGENERATE = ["q_zero_at_draft", "q_equals_p", "q_twice_p", "one_hot_residual"]


@pytest.mark.parametrize("case", DEGENERATE)
def test_chain_accept_degenerate_probabilities(case):
    """Edge cases of the rule with probabilities both sides hold exactly
    (uniform logits over V = 4096: p = 2^-12 in fp32 and fp64), so every
    decision must agree bit for bit, with no near-tie excuse:
      q_zero_at_draft  q(x) = 0 at every draft: u * 0 < p(x), always accepted,
                       then the bonus from p;
      q_equals_p       q = p: u < 1 always accepts;
      q_twice_p        q = 2p (unnormalised): accepted iff u < 1/2; after a
                       rejection max(0, p - q) has no mass and the draw falls
                       back to p (the reading for a zero-mass residual);
      one_hot_residual q moves 2^-12 from token y to the draft x: accepted iff
                       u < 1/2, and a rejection must resample y."""
    V, B, gamma = 4096, 16, 3
    T = gamma + 1
    eng = _engine(V, B, 8)
    g = torch.Generator().manual_seed(DEGENERATE.index(case))
    z = torch.zeros((B, T, V), device=dev())
    tokens = torch.randint(0, V, (B, T), generator=g).to(torch.int32)
    p = torch.full((B, gamma, V), 1.0 / V)
    if case == "q_zero_at_draft":
        q = p.clone()
        for b in range(B):
            for i in range(gamma):
                q[b, i, tokens[b, i + 1]] = 0.0
    elif case == "q_equals_p":
        q = p.clone()
    elif case == "q_twice_p":
        q = 2.0 * p
    else:
        q = p.clone()
        for b in range(B):
            for i in range(gamma):
                x = int(tokens[b, i + 1])
                y = (x + 1 + int(torch.randint(0, V - 1, (1,), generator=g))) % V
                q[b, i, x] = 2.0 / V
                q[b, i, y] = 0.0
    q, tokens = q.to(dev()), tokens.to(dev())
    total = np.zeros(T, dtype=int)
    for r in range(4):
        kv_len = torch.full((B,), 50, dtype=torch.int32, device=dev())
        kv_out = torch.zeros_like(kv_len)
        out = torch.full((B, T), -5, dtype=torch.int32, device=dev())
        nacc = torch.full((B,), -5, dtype=torch.int32, device=dev())
        eng.accept(z, q, tokens, out, nacc, kv_len, kv_out, temperature=1.0, seed=99, round_=r)
        torch.cuda.synchronize()
        orc = OA.accept(z.double().cpu().numpy(), q.double().cpu().numpy(), tokens.cpu().numpy(), 1.0,
                        philox.Uniforms(99, r))
        n = nacc.cpu().numpy()
        assert np.array_equal(n, orc["n_accepted"]), (case, n, orc["n_accepted"])
        for b in range(B):
            assert np.array_equal(out.cpu().numpy()[b, :n[b] + 1], orc["out_tokens"][b, :n[b] + 1]), (case, b)
        if case in ("q_zero_at_draft", "q_equals_p"):
            assert np.all(n == gamma)
        if case == "one_hot_residual":
            for b in range(B):
                if n[b] < gamma:  # the resampled token is the one q gave up
                    assert q[b, n[b], int(out[b, n[b]])] == 0.0
        np.add.at(total, n, 1)
        assert eng.device_errors() == 0
    if case in ("q_twice_p", "one_hot_residual"):
        assert total[:gamma].sum() > 0 and total.sum() == 4 * B  # rejections happened


def test_accept_rejects_bad_adjustment():
    V, B, gamma = 4099, 1, 2
    eng = _engine(V, 4, 8)
    z, q, tokens = _chain_inputs(B, gamma, V, 1.0, 1.0, 9)
    out = torch.zeros((B, gamma + 1), dtype=torch.int32, device=dev())
    nacc = torch.zeros((B,), dtype=torch.int32, device=dev())
    from speculative_decoding_verify_spec_amd import SpecError
    for kw in (dict(top_k=-1), dict(top_p=1.5), dict(top_p=float("nan"))):
        with pytest.raises(SpecError):
            eng.accept(z, q, tokens, out, nacc, None, None, temperature=1.0, **kw)
