"""Pins of the CPU oracle's accept rule, uniforms and closed forms against what
the pages and the mathematics fix (never against the oracle itself)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import accept as acc
from oracle import metrics, philox
from oracle.numerics import bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_examples.json")))


# ----------------------------------------------------------------------------
# exact output distribution of one chain round by enumeration
# ----------------------------------------------------------------------------

def _random_dist(rng, V, zeros=0):
    w = rng.gamma(0.7, size=V)
    if zeros:
        w[rng.choice(V, zeros, replace=False)] = 0.0
    return w / w.sum()


class _Tables:
    """A toy target p(.|prefix) and draft q(.|prefix), one random distribution per
    prefix of drafted tokens (tuples), so conditionals are exact by construction."""

    def __init__(self, V, depth, seed):
        rng = np.random.default_rng(seed)
        self.V = V
        self.p, self.q = {}, {}
        for d in range(depth + 1):
            for pre in itertools.product(range(V), repeat=d):
                self.p[pre] = _random_dist(rng, V)
                # some drafts put zero mass where p does not, and vice versa
                self.q[pre] = _random_dist(rng, V, zeros=1 if (len(pre) % 2) else 0)


def _enumerate_chain(tab, gamma, variant="residual"):
    """Exact distribution of the oracle's emitted tokens, extended to gamma+1
    tokens with the target's own conditionals.  Draft tuples are enumerated
    with weight prod q; every uniform's range is split at the decision
    boundaries implied by the pages' rule (accept iff u < p/q; inverse CDF of
    the residual) and the oracle is called at each cell's midpoint."""
    V = tab.V
    joint = {}
    for xs in itertools.product(range(V), repeat=gamma):
        w_draft = 1.0
        for i in range(gamma):
            w_draft *= tab.q[xs[:i]][xs[i]]
        if w_draft == 0.0:
            continue
        z = np.stack([np.log(np.maximum(tab.p[xs[:i]], 1e-300)) for i in range(gamma + 1)])
        qrows = np.stack([tab.q[xs[:i]] for i in range(gamma)])
        tokens = [0] + list(xs)
        # walk the accept cells: n accepted, then the final draw
        prefix_w = 1.0
        for n in range(gamma + 1):
            # cell in which drafts 1..n are accepted and draft n+1 (if any) rejected
            acc_u, w = [], prefix_w
            if n < gamma:
                p, qq = tab.p[xs[:n]], tab.q[xs[:n]]
                t = min(1.0, p[xs[n]] / qq[xs[n]])
                w *= (1.0 - t)
                rej_mid = (t + 1.0) / 2.0
            if w == 0.0:
                if n < gamma:
                    p, qq = tab.p[xs[:n]], tab.q[xs[:n]]
                    prefix_w *= min(1.0, p[xs[n]] / qq[xs[n]])
                continue
            # accept uniforms for drafts 1..n at their accept-cell midpoints
            us = {}
            for i in range(n):
                p, qq = tab.p[xs[:i]], tab.q[xs[:i]]
                us[i] = min(1.0, p[xs[i]] / qq[xs[i]]) / 2.0
            if n < gamma:
                us[n] = rej_mid
            pn = tab.p[xs[:n]]
            if n < gamma and variant == "residual":
                r = np.maximum(0.0, pn - tab.q[xs[:n]])
                if r.sum() <= 0:
                    r = pn
            else:
                r = pn
            R = r.sum()
            c = np.cumsum(r)
            for y in range(V):
                if r[y] <= 0:
                    continue
                lo = c[y - 1] if y else 0.0
                us[gamma] = (lo + r[y] / 2.0) / R
                ny, out, _ = acc.accept_chain_one(z, qrows, tokens, 1.0, lambda s: us[s], _variant=variant)
                cell_w = w_draft * w * r[y] / R
                key = tuple(out)
                joint[key] = joint.get(key, 0.0) + cell_w
            if n < gamma:
                p, qq = tab.p[xs[:n]], tab.q[xs[:n]]
                prefix_w *= min(1.0, p[xs[n]] / qq[xs[n]])
    # extend each emitted prefix to gamma+1 tokens with the target's conditionals
    full = np.zeros((V,) * (gamma + 1))
    for out, w in joint.items():
        k = len(out)
        for rest in itertools.product(range(V), repeat=gamma + 1 - k):
            seq = out + rest
            pr = w
            for j in range(k, gamma + 1):
                pr *= tab.p[seq[:j]][seq[j]]
            full[seq] += pr
    return full


def _target_joint(tab, gamma):
    V = tab.V
    full = np.zeros((V,) * (gamma + 1))
    for seq in itertools.product(range(V), repeat=gamma + 1):
        pr = 1.0
        for j in range(gamma + 1):
            pr *= tab.p[seq[:j]][seq[j]]
        full[seq] = pr
    return full


@pytest.mark.parametrize("gamma", [1, 2, 3])
def test_chain_enumeration_output_is_p(gamma):
    """The speculative round's output distribution is exactly the target's
    (CS349E Lecture 6, section 7.1; the lecture's demo 1 checks the same by
    computing output probabilities instead of sampling)."""
    tab = _Tables(V=8, depth=gamma, seed=10 + gamma)
    got = _enumerate_chain(tab, gamma)
    want = _target_joint(tab, gamma)
    assert abs(got.sum() - 1.0) < 1e-12
    assert np.abs(got - want).max() < 1e-12


@pytest.mark.parametrize("variant", ["resample_from_p", "deterministic"])
def test_chain_enumeration_wrong_variants_fail(variant):
    """Both wrong implementations of section 7.5 change the output distribution."""
    tab = _Tables(V=8, depth=2, seed=3)
    got = _enumerate_chain(tab, 2, variant=variant)
    want = _target_joint(tab, 2)
    assert 0.5 * np.abs(got - want).sum() > 1e-3


def _single_step_dist(p, q, variant="residual"):
    tab = _Tables(V=len(p), depth=1, seed=0)
    tab.p[()] = np.asarray(p, float)
    tab.q[()] = np.asarray(q, float)
    full = _enumerate_chain(tab, 1, variant=variant)
    return full.sum(axis=1)  # marginal of the first emitted token


def test_exercise3_worked_example():
    g = GOLDEN["ex3_single_step"]
    p, q = np.array(g["p"]), np.array(g["q"])
    assert metrics.beta(p, q) == pytest.approx(g["beta"], abs=1e-12)
    assert 1 - metrics.total_variation(p, q) == pytest.approx(g["beta"], abs=1e-12)
    r = np.maximum(0, p - q)
    assert np.allclose(r / r.sum(), g["residual_normalised"])
    assert np.allclose(_single_step_dist(p, q), g["output"], atol=1e-12)


def test_exercise4_resample_from_p_bias():
    g3, g4 = GOLDEN["ex3_single_step"], GOLDEN["ex4_resample_from_p"]
    out = _single_step_dist(g3["p"], g3["q"], variant="resample_from_p")
    assert np.allclose(out, g4["output"], atol=1e-12)
    assert metrics.total_variation(out, g3["p"]) == pytest.approx(g4["tv"], abs=1e-12)


def test_beta_equals_one_minus_tv():
    """Section 7.2: beta = sum min(p, q) = 1 - TV(p, q) to rounding."""
    rng = np.random.default_rng(0)
    for _ in range(200):
        V = int(rng.integers(2, 5000))
        p, q = _random_dist(rng, V), _random_dist(rng, V)
        assert abs(metrics.beta(p, q) - (1 - metrics.total_variation(p, q))) < 1e-12


def test_acceptance_probability_is_beta_by_sampling():
    """One-position acceptance rate over many drafts equals beta (section 7.2)."""
    rng = np.random.default_rng(1)
    V = 16
    p, q = _random_dist(rng, V), _random_dist(rng, V)
    z = np.log(np.stack([p, p]))
    n_acc, N = 0, 40000
    xs = rng.choice(V, size=N, p=q)
    us = rng.random(N)
    for x, u in zip(xs, us):
        n, _, _ = acc.accept_chain_one(z, q[None], [0, x], 1.0, lambda s: u if s == 0 else 0.5)
        n_acc += n
    b = metrics.beta(p, q)
    se = np.sqrt(b * (1 - b) / N)
    assert abs(n_acc / N - b) < 4 * se


# ----------------------------------------------------------------------------
# greedy
# ----------------------------------------------------------------------------

def test_greedy_is_argmax_prefix():
    """Section 7.4 and the Kimi-K3 tuning page: greedy acceptance is the longest
    prefix where draft == target argmax; the extra token is the argmax at the
    break."""
    rng = np.random.default_rng(2)
    for _ in range(300):
        gamma, V = int(rng.integers(1, 8)), 12
        z = rng.normal(size=(gamma + 1, V))
        am = z.argmax(axis=1)
        drafts = am[:gamma].copy()
        k = int(rng.integers(0, gamma + 1))
        if k < gamma:
            drafts[k] = (drafts[k] + 1 + rng.integers(0, V - 1)) % V
        n, out, _ = acc.accept_chain_one(z, None, [0] + list(drafts), 0.0, None)
        assert n == k
        assert out == list(drafts[:k]) + [int(am[k])]


def test_greedy_speculative_equals_greedy_decoding():
    """Speculative greedy output equals the target's own greedy output token for
    token (section 7.4), with a deterministic toy target p(.|prefix)."""
    V, L = 9, 40

    def target_logits(prefix):
        h = np.random.default_rng(hash(tuple(prefix)) % (2 ** 32))
        return h.normal(size=V)

    plain = []
    for _ in range(L):
        plain.append(int(np.argmax(target_logits(plain))))
    rng = np.random.default_rng(5)
    spec = []
    while len(spec) < L:
        gamma = int(rng.integers(1, 5))
        drafts = []
        for i in range(gamma):  # a draft that is right about half the time
            zt = target_logits(spec + drafts)
            drafts.append(int(np.argmax(zt)) if rng.random() < 0.6 else int(rng.integers(0, V)))
        z = np.stack([target_logits(spec + drafts[:i]) for i in range(gamma + 1)])
        n, out, _ = acc.accept_chain_one(z, None, [0] + drafts, 0.0, None)
        spec += out
    assert spec[:L] == plain


def test_greedy_ties_lowest_id():
    z = np.array([[0.0, 3.0, 3.0, 1.0], [0.0, 0.0, 0.0, 0.0]])
    n, out, _ = acc.accept_chain_one(z, None, [0, 2], 0.0, None)
    assert n == 0 and out == [1]


# ----------------------------------------------------------------------------
# token tree
# ----------------------------------------------------------------------------

def test_tree_all_ones_is_chain():
    """A tree whose branching is all ones consumes the chain's uniforms and
    makes the chain's decisions (sampled and greedy)."""
    rng = np.random.default_rng(7)
    for trial in range(300):
        gamma, V = int(rng.integers(1, 7)), 50
        z = rng.normal(size=(gamma + 1, V)) * 1.5
        q = np.stack([_random_dist(rng, V) for _ in range(gamma + 1)])
        drafts = [int(rng.choice(V, p=q[i])) for i in range(gamma)]
        us = rng.random(gamma + 1)
        temp = 0.0 if trial % 3 == 0 else 1.0
        if temp == 0.0:
            am = z.argmax(1)
            for i in range(gamma):
                if rng.random() < 0.7:
                    drafts[i] = int(am[i])
        tokens = [0] + drafts
        parent = [-1] + list(range(gamma))
        n, out_c, _ = acc.accept_chain_one(z, q[:gamma], tokens, temp, lambda s: us[s])
        path, out_t, _ = acc.accept_tree_one(z, q, tokens, parent, temp, lambda s: us[s])
        assert path == list(range(n + 1))
        assert out_t == out_c


def _tree_round_sample(rng, tab, branching, replacement, variant="residual"):
    """Draw one token tree from the draft tables (children of a node drawn from
    q(.|path) with or without replacement), run the oracle's tree accept with
    fresh uniforms, return the first two emitted tokens."""
    V = tab.V
    parents, toks, ctx = [-1], [0], [()]
    level = [0]
    for k in branching:
        nxt = []
        for v in level:
            qv = tab.q[ctx[v]].copy()
            chosen = []
            for _ in range(k):
                x = int(rng.choice(V, p=qv / qv.sum()))
                chosen.append(x)
                if not replacement:
                    qv[x] = 0.0
            for x in chosen:
                parents.append(v)
                toks.append(x)
                ctx.append(ctx[v] + (x,))
                nxt.append(len(parents) - 1)
        level = nxt
    T = len(parents)
    z = np.stack([np.log(np.maximum(tab.p[c], 1e-300)) if c in tab.p else np.zeros(V) for c in ctx])
    q = np.stack([tab.q[c] if c in tab.q else np.full(V, 1.0 / V) for c in ctx])
    us = rng.random(T)
    path, out, _ = acc.accept_tree_one(z, q, toks, parents, 1.0, lambda s: us[s],
                                       replacement=replacement, _variant=variant)
    # continue with the target's own conditionals if only one token came out
    if len(out) < 2:
        out = out + [int(rng.choice(V, p=tab.p[tuple(out)]))]
    return tuple(out[:2])


def _chi2(counts, exp):
    """Pearson chi-square with cells of expectation < 5 pooled into one."""
    counts, exp = counts.ravel(), exp.ravel()
    big = exp >= 5
    c = list(counts[big]) + [counts[~big].sum()]
    e = list(exp[big]) + [exp[~big].sum()]
    c, e = np.array(c), np.array(e)
    keep = e > 0
    return float(((c[keep] - e[keep]) ** 2 / e[keep]).sum()), int(keep.sum() - 1)


@pytest.mark.parametrize("replacement", [False, True])
def test_tree_sampled_output_is_p(replacement):
    """Sampled tree walk: the joint of the first two emitted tokens matches the
    target's p(y1) p(y2|y1) within sampling error (chi-square)."""
    V, branching, N = 4, [2, 2], 40000
    tab = _Tables(V=V, depth=3, seed=21)
    rng = np.random.default_rng(22)
    counts = np.zeros((V, V))
    for _ in range(N):
        y = _tree_round_sample(rng, tab, branching, replacement)
        counts[y] += 1
    want = np.array([[tab.p[()][a] * tab.p[(a,)][b] for b in range(V)] for a in range(V)])
    chi2, dof = _chi2(counts, want * N)
    # P(chi2_15 > 50) ~ 1e-5
    assert chi2 < 50 + 2.5 * (dof - 15), (chi2, dof)


def test_tree_wrong_variant_detected():
    """Negative control: resampling from p after rejected siblings is biased and
    the same statistic sees it."""
    V, branching, N = 4, [2, 2], 40000
    tab = _Tables(V=V, depth=3, seed=21)
    rng = np.random.default_rng(23)
    counts = np.zeros((V, V))
    for _ in range(N):
        counts[_tree_round_sample(rng, tab, branching, False, variant="resample_from_p")] += 1
    want = np.array([[tab.p[()][a] * tab.p[(a,)][b] for b in range(V)] for a in range(V)])
    chi2, dof = _chi2(counts, want * N)
    assert chi2 > 200, (chi2, dof)


def test_tree_greedy_walk():
    """Greedy tree: descend while a child carries the argmax token."""
    z = np.full((7, 5), -1.0)
    # root -> children 1,2 ; node 1 -> 3,4 ; node 2 -> 5,6
    parent = [-1, 0, 0, 1, 1, 2, 2]
    tokens = [0, 3, 1, 2, 4, 0, 1]
    z[0, 1] = 5.0   # argmax at root = token 1 -> node 2
    z[2, 1] = 5.0   # argmax at node 2 = token 1 -> node 6
    z[6, 3] = 5.0   # leaf: emit argmax 3
    path, out, _ = acc.accept_tree_one(z, None, tokens, parent, 0.0, None)
    assert path == [0, 2, 6] and out == [1, 1, 3]


# ----------------------------------------------------------------------------
# closed forms printed on the pages
# ----------------------------------------------------------------------------

def test_expected_tokens_examples():
    g = GOLDEN["ex5_expected_tokens"]
    e = metrics.expected_tokens(g["alpha"], g["gamma"])
    assert round(e, 2) == g["expected_tokens"]
    c = (e / g["measured_speedup"] - 1) / g["gamma"]
    assert round(c, 3) == g["implied_c"]
    for a, lim in GOLDEN["sec8_1_limits"]["cases"]:
        assert metrics.expected_tokens(a, 10000) == pytest.approx(lim, rel=1e-9)
    g7 = GOLDEN["ex7_compute_increase"]
    assert round(metrics.expected_tokens(g7["alpha"], g7["gamma"]), 3) == g7["expected_tokens"]
    for c_hat, inc in g7["cases"]:
        assert round(metrics.compute_increase(g7["alpha"], g7["gamma"], c_hat), 2) == inc


def test_expected_tokens_by_simulation():
    """Eq. (1) holds for independent per-position acceptance with unequal beta
    (section 8.3): simulate rounds with per-position acceptance probabilities."""
    rng = np.random.default_rng(4)
    gamma, N = 5, 200000
    betas = rng.uniform(0.3, 0.9, size=gamma)
    acc_mat = rng.random((N, gamma)) < betas
    n = np.argmin(np.concatenate([acc_mat, np.zeros((N, 1), bool)], axis=1), axis=1)
    want = 1 + sum(np.prod(betas[:i + 1]) for i in range(gamma))
    assert abs((n + 1).mean() - want) < 4 * (n + 1).std() / np.sqrt(N)
    assert metrics.expected_tokens(0.6, gamma) == pytest.approx(1 + sum(0.6 ** (i + 1) for i in range(gamma)))


def test_speedup_examples():
    g = GOLDEN["ex6_speedup"]
    for gamma, s in g["cases"]:
        assert round(metrics.walltime_speedup(g["alpha"], gamma, g["c"]), 2) == s


def test_tree_counting_example():
    g = GOLDEN["ex9_tree"]
    assert metrics.tree_draft_nodes(g["branching"]) == g["draft_nodes"]
    hit = {int(k): v for k, v in g["topk_hit"].items()}
    assert round(metrics.tree_tau_independent(g["branching"], hit), 2) == g["tau"]


def test_weight_read_fraction():
    g = GOLDEN["ex11_weight_reads"]
    assert round(1.0 / g["tokens_per_forward"], 2) == g["fraction"]


def test_accept_metric_definitions():
    g = GOLDEN["accept_metrics"]
    assert metrics.strict_accept_rate(g["correct_drafts"], g["verify_ct"], g["num_draft_tokens"]) == \
        pytest.approx(g["strict_accept_rate"])
    assert metrics.accept_length(g["completion_tokens"], g["verify_ct"]) == pytest.approx(g["accept_length"])


def test_division_and_break_even():
    g = GOLDEN["division"]
    tok_per_ms = (1 + g["p"]) / (g["t_verify_ms"] + g["t_draft_ms"])
    assert round(tok_per_ms, 3) == g["tok_per_ms"]
    assert abs(tok_per_ms * 1000 - g["measured_tok_s"]) / g["measured_tok_s"] < 0.03
    be = metrics.break_even_verify(g["p"], g["t_decode_ms"], g["t_draft_ms"])
    assert round(be, 1) == g["break_even_ms"]
    assert round(be / g["t_decode_ms"], 2) == g["break_even_ratio"]
    # verify at twice decode never wins with one draft (section 2.1)
    for p in np.linspace(0, 1, 11):
        assert metrics.division_speedup(p, 1.0, 2.0, 0.0) <= 1.0


# ----------------------------------------------------------------------------
# Philox4x64-10 and bf16
# ----------------------------------------------------------------------------

def test_philox_matches_numpy():
    """numpy.random.Philox is an independent Philox4x64-10; random_raw() returns
    the words of the block at counter + 1, word 0 first."""
    rng = np.random.default_rng(9)
    cases = [((0, 0, 0, 0), (0, 0)), ((7, 0, 0, 0), (12345, 0))]
    for _ in range(3000):
        c = tuple(int(x) for x in rng.integers(0, 2 ** 63, size=4, dtype=np.int64))
        k = tuple(int(x) for x in rng.integers(0, 2 ** 63, size=2, dtype=np.int64))
        cases.append((c, k))
    cases.append(((2 ** 64 - 2, 5, 0, 0), (1, 2)))
    for c, k in cases:
        g = np.random.Philox(counter=np.array(c, dtype=np.uint64), key=np.array(k, dtype=np.uint64))
        ref = [g.random_raw() for _ in range(4)]
        c1 = list(c)
        # numpy pre-increments the 256-bit counter
        carry = 1
        for i in range(4):
            s = c1[i] + carry
            c1[i], carry = s & philox.MASK64, s >> 64
        assert list(philox.philox4x64(c1, k)) == [int(x) for x in ref]


def test_uniform_range_and_resolution():
    us = np.array([philox.uniform(42, 3, b, s) for b in range(20) for s in range(50)])
    assert us.min() >= 0.0 and us.max() < 1.0
    assert np.all((us * 2 ** 24) == np.floor(us * 2 ** 24))
    assert abs(us.mean() - 0.5) < 0.05


def test_bf16_round_nearest_even():
    import torch
    rng = np.random.default_rng(11)
    x32 = (rng.normal(size=20000) * rng.choice([1e-3, 1.0, 1e3], size=20000)).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(round_to_bf16(x32.astype(np.float64)), ref)
    # exact ties go to even
    assert round_to_bf16(np.array([1.0 + 2 ** -8]))[0] == 1.0
    assert round_to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    bits = f64_to_bf16_bits(np.array([1.5, -2.0, 0.0]))
    assert np.array_equal(bf16_bits_to_f64(bits), [1.5, -2.0, 0.0])
