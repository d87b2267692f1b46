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


class _NotConstant(Exception):
    """The oracle's output changes inside a cell of the rule's partition."""


def _constant_on_cell(cells, run):
    """The oracle's output for uniforms in the box `cells` (slot -> [lo, hi)).
    It is evaluated at the box's midpoint and just inside its lower and upper
    corners; each decision is monotone in its uniform (a threshold test, or
    an inverse CDF), so equal outputs at the three points mean the oracle's
    own decision boundaries are the rule's: no boundary of the oracle lies
    inside a cell, and the midpoint's output holds for the whole cell.
    Raises _NotConstant otherwise."""
    def at(f):
        return {s: lo + (hi - lo) * f for s, (lo, hi) in cells.items()}
    mid = tuple(run(at(0.5)))
    for f in (1e-9, 1.0 - 1e-9):
        if tuple(run(at(f))) != mid:
            raise _NotConstant(cells)
    return mid


def _enumerate_chain(tab, gamma, variant="residual", ztab=None, temperature=1.0, adj=None):
    """Exact distribution of the oracle's emitted tokens, extended to gamma+1
    tokens with the target's own conditionals.  Draft tuples are enumerated
    with weight prod q; every uniform's range is split at the decision
    boundaries implied by the pages' rule (accept iff u < p/q; inverse CDF of
    the residual) and the oracle's output is taken on each cell after
    checking that it is constant there (`_constant_on_cell`).

    With `ztab` the oracle receives log ztab.p as logits, with `temperature`
    and the sampling adjustments `adj`, while the cells come from tab.p: the
    adjusted target the oracle should be sampling."""
    V = tab.V
    ztab = tab if ztab is None else ztab
    adj = adj or {}
    joint = {}
    for xs in itertools.product(range(V), repeat=gamma):
        w_draft = 1.0
        for i in range(gamma):
            w_draft *= tab.q[xs[:i]][xs[i]]
        if w_draft == 0.0:
            continue
        z = np.stack([np.log(np.maximum(ztab.p[xs[:i]], 1e-300)) for i in range(gamma + 1)])
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
            # accept uniforms for drafts 1..n in their accept cells [0, t)
            cells = {}
            for i in range(n):
                p, qq = tab.p[xs[:i]], tab.q[xs[:i]]
                cells[i] = (0.0, min(1.0, p[xs[i]] / qq[xs[i]]))
            if n < gamma:
                cells[n] = (2.0 * rej_mid - 1.0, 1.0)
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
                cy = dict(cells)
                cy[gamma] = (lo / R, c[y] / R)
                out = _constant_on_cell(
                    cy, lambda u: acc.accept_chain_one(z, qrows, tokens, temperature, lambda s: u[s],
                                                       _variant=variant, **adj)[1])
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
    try:
        got = _enumerate_chain(tab, 2, variant=variant)
    except _NotConstant:
        return
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


def _tree_configs(tab, branching, replacement):
    """Every token tree the draft can produce with the given branching (BFS node
    order, root = node 0 with an empty prefix), with its probability: a
    node's children are drawn one after another from q(.|prefix), without
    replacement (each draw renormalised over the tokens not yet drawn) or
    with it."""
    V = tab.V

    def child_lists(qv, k):
        out = []
        for xs in itertools.product(range(V), repeat=k):
            if not replacement and len(set(xs)) < k:
                continue
            w, left = 1.0, 1.0
            for x in xs:
                w *= qv[x] / left
                if not replacement:
                    left -= qv[x]
            if w > 0.0:
                out.append((xs, w))
        return out

    trees = [([-1], [0], [()], 1.0)]
    level = 1
    for k in branching:
        nxt = []
        for parents, toks, ctx, w in trees:
            frontier = [v for v in range(len(parents)) if len(ctx[v]) == level - 1]
            partial = [(parents, toks, ctx, w)]
            for v in frontier:
                grown = []
                for pa, tk, cx, wt in partial:
                    for xs, wx in child_lists(tab.q[cx[v]], k):
                        grown.append((pa + [v] * k, tk + list(xs), cx + [cx[v] + (x,) for x in xs], wt * wx))
                partial = grown
            nxt += partial
        trees = nxt
        level += 1
    return trees


def _enumerate_tree(tab, branching, replacement, variant="residual", ztab=None, adj=None,
                    oracle_replacement=None):
    """Exact distribution of the tokens the oracle's tree walk emits, extended to
    depth+1 tokens with the target's own conditionals.  Every tree the draft
    can produce is enumerated with its probability; within a tree, every
    uniform's range is split at the boundaries the rule implies (child c,
    slot c - 1: accept iff u < r(x)/q'(x), with r and q' updated after each
    rejected sibling as the residual rule says; the final draw, slot T - 1:
    inverse CDF of r) and the oracle's output is taken on each cell after
    checking that it is constant there (`_constant_on_cell`).
    `ztab` / `adj` as in _enumerate_chain; `oracle_replacement` hands the
    oracle a different replacement flag than the one the trees were drawn
    with (a negative control)."""
    V = tab.V
    ztab = tab if ztab is None else ztab
    adj = adj or {}
    orep = replacement if oracle_replacement is None else oracle_replacement
    depth = len(branching)
    joint = {}
    for parents, toks, ctx, w_tree in _tree_configs(tab, branching, replacement):
        T = len(parents)
        kids = [[c for c in range(1, T) if parents[c] == v] for v in range(T)]
        z = np.stack([np.log(np.maximum(ztab.p[c], 1e-300)) for c in ctx])
        q = np.stack([tab.q[c] if c in tab.q else np.full(V, 1.0 / V) for c in ctx])

        def draw(r, us, w):
            R = r.sum()
            c = np.cumsum(r)
            for y in range(V):
                if r[y] <= 0:
                    continue
                lo = c[y - 1] if y else 0.0
                cy = dict(us)
                cy[T - 1] = (lo / R, c[y] / R)
                key = _constant_on_cell(
                    cy, lambda u: acc.accept_tree_one(z, q, toks, parents, 1.0, lambda s: u.get(s, 0.5),
                                                      replacement=orep, _variant=variant, **adj)[1])
                joint[key] = joint.get(key, 0.0) + w_tree * w * r[y] / R

        def visit(v, us, w):
            r = tab.p[ctx[v]].copy()
            if not kids[v]:
                draw(r, us, w)
                return
            qp = tab.q[ctx[v]].copy()
            for c in kids[v]:
                x = toks[c]
                t = 1.0 if qp[x] <= 0 else min(1.0, r[x] / qp[x])
                if t > 0.0:
                    visit(c, {**us, c - 1: (0.0, t)}, w * t)
                if t >= 1.0:
                    return
                us = {**us, c - 1: (t, 1.0)}
                w = w * (1.0 - t)
                res = np.maximum(0.0, r - qp)
                if res.sum() > 0.0:
                    r = res / res.sum()
                if not replacement:
                    qp[x] = 0.0
                    qp = qp / qp.sum()
            draw(r, us, w)

        visit(0, {}, 1.0)
    full = np.zeros((V,) * (depth + 1))
    for out, w in joint.items():
        k = len(out)
        for rest in itertools.product(range(V), repeat=depth + 1 - k):
            seq = out + rest
            pr = w
            for j in range(k, depth + 1):
                pr *= tab.p[seq[:j]][seq[j]]
            full[seq] += pr
    return full


TREE_CASES = [(4, [2, 2], False, 21), (4, [2, 2], True, 21), (5, [3, 1], False, 26)]


@pytest.mark.parametrize("V,branching,replacement,seed", TREE_CASES)
def test_tree_enumeration_output_is_p(V, branching, replacement, seed):
    """Sampled tree walk, exact: over every tree the draft can produce with the
    branching and every cell of the uniforms, the joint of the three tokens
    the round yields (accepted path and extra token, continued with the
    target's conditionals) is the target's p(y1) p(y2|y1) p(y3|y1,y2) to
    1e-12, for children drawn with and without replacement, with two and
    three siblings per node (CS349E Lecture 6, section 7.1, applied per node;
    section 10.3 for the tree)."""
    tab = _Tables(V=V, depth=2, seed=seed)
    got = _enumerate_tree(tab, branching, replacement)
    want = _target_joint(tab, 2)
    assert abs(got.sum() - 1.0) < 1e-12
    assert np.abs(got - want).max() < 1e-12


@pytest.mark.parametrize("variant,oracle_replacement", [
    ("resample_from_p", None), ("no_renorm", None), ("residual", True)])
@pytest.mark.parametrize("V,branching,seed", [(4, [2, 2], 21), (5, [3, 1], 26)])
def test_tree_enumeration_wrong_walks_fail(variant, oracle_replacement, V, branching, seed):
    """Negative controls on the same enumeration: keeping r = p after rejected
    siblings, removing a rejected child from q' without renormalising, and
    never updating q' for children drawn without replacement each either put
    a decision boundary inside a cell of the rule's partition or move the
    output distribution away from p."""
    tab = _Tables(V=V, depth=2, seed=seed)
    try:
        got = _enumerate_tree(tab, branching, False, variant=variant,
                              oracle_replacement=oracle_replacement)
    except _NotConstant:
        return
    want = _target_joint(tab, 2)
    assert 0.5 * np.abs(got - want).sum() > 1e-3


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


# ----------------------------------------------------------------------------
# sampling adjustments: temperature, top-k, top-p (CS349E Lecture 6, section 7.3)
# ----------------------------------------------------------------------------

def _brute_adjust(p, temperature=1.0, top_k=0, top_p=1.0):
    """Independent statement of the adjusted distribution for tiny V: tempered
    p ~ p^(1/T); top-k keeps the tokens with fewer than k tokens ranked above
    them (higher probability, or equal probability and lower id); the nucleus
    is, among all subsets of the kept tokens whose renormalised mass reaches
    top_p, one of minimum size, and of those the heaviest."""
    p = np.asarray(p, dtype=np.float64) ** (1.0 / temperature)
    p = p / p.sum()
    V = p.size
    keep = np.ones(V, bool)
    if 0 < top_k < V:
        for x in range(V):
            above = sum(1 for y in range(V) if p[y] > p[x] or (p[y] == p[x] and y < x))
            keep[x] = above < top_k
    if top_p < 1.0:
        cand = [x for x in range(V) if keep[x]]
        mass = p[cand].sum()
        best = None
        for size in range(1, len(cand) + 1):
            for sub in itertools.combinations(cand, size):
                m = p[list(sub)].sum() / mass
                if m >= top_p and (best is None or m > best[0]):
                    best = (m, sub)
            if best is not None:
                break
        keep[:] = False
        keep[list(best[1])] = True
    r = np.where(keep, p, 0.0)
    return r / r.sum()


ADJ_CASES = [(1.0, 3, 1.0), (1.0, 0, 0.7), (0.7, 5, 0.85), (1.3, 2, 0.95), (1.0, 1, 1.0), (1.0, 0, 0.05)]


@pytest.mark.parametrize("temperature,top_k,top_p", ADJ_CASES)
def test_adjust_matches_subset_brute_force(temperature, top_k, top_p):
    """The oracle's top-k / nucleus agree with the subset definition on random
    distributions (V = 8)."""
    rng = np.random.default_rng(int(100 * temperature) + 7 * top_k + int(100 * top_p))
    for _ in range(200):
        p = _random_dist(rng, 8)
        got, _ = acc.adjust(np.log(p), temperature, top_k, top_p)
        want = _brute_adjust(p, temperature, top_k, top_p)
        assert np.abs(got - want).max() < 1e-14, (p, got, want)


def test_adjust_special_cases():
    z = np.array([0.3, 2.0, -1.0, 2.0, 0.5])
    # top-k = 1 and a tiny nucleus are the greedy one-hot; equal logits go to the lower id
    for p, _ in (acc.adjust(z, 1.0, top_k=1), acc.adjust(z, 1.0, top_p=1e-6)):
        assert np.array_equal(p, np.eye(5)[1])
    # switched off: plain softmax
    p, m = acc.adjust(z, 0.8, top_k=0, top_p=1.0)
    e = np.exp(z / 0.8 - (z / 0.8).max())
    assert np.abs(p - e / e.sum()).max() < 1e-15 and m == np.inf
    p, _ = acc.adjust(z, 1.0, top_k=5)
    assert np.abs(p - acc.softmax(z, 1.0)).max() < 1e-15
    # top-k = 2 keeps the two tied maxima; top-k = 3 adds logit 0.5 (id 4)
    assert np.array_equal(acc.adjust(z, 1.0, top_k=2)[0] > 0, [False, True, False, True, False])
    assert np.array_equal(acc.adjust(z, 1.0, top_k=3)[0] > 0, [False, True, False, True, True])
    # a nucleus that must split the tie keeps the lower id
    y = np.log(np.array([0.1, 0.3, 0.3, 0.3]))
    assert np.array_equal(acc.adjust(y, 1.0, top_p=0.5)[0] > 0, [False, True, True, False])
    # the margin is the distance of the cumulative mass to top_p at the cut
    p4 = np.array([0.4, 0.3, 0.2, 0.1])
    _, m = acc.adjust(np.log(p4), 1.0, top_p=0.65)
    assert abs(m - 0.05) < 1e-12


@pytest.mark.parametrize("temperature,top_k,top_p,adjust_q", [
    (1.0, 3, 1.0, True), (1.0, 0, 0.75, True), (0.7, 5, 0.8, True), (1.0, 4, 0.9, False)])
def test_chain_enumeration_adjusted_output(temperature, top_k, top_p, adjust_q):
    """With the adjustments the round's output is exactly the adjusted target,
    whether the draft was adjusted the same way or not (section 7.3: the rule
    holds for any q, an unadjusted draft is only accepted less often)."""
    gamma = 2
    raw = _Tables(V=8, depth=gamma, seed=40 + top_k)
    tab = _Tables(V=8, depth=0, seed=0)
    tab.p = {k: _brute_adjust(v, temperature, top_k, top_p) for k, v in raw.p.items()}
    tab.q = {k: (_brute_adjust(v, temperature, top_k, top_p) if adjust_q else v) for k, v in raw.q.items()}
    got = _enumerate_chain(tab, gamma, ztab=raw, temperature=temperature,
                           adj=dict(top_k=top_k, top_p=top_p))
    want = _target_joint(tab, gamma)
    assert abs(got.sum() - 1.0) < 1e-12
    assert np.abs(got - want).max() < 1e-12
    # and it is not the unadjusted target
    assert 0.5 * np.abs(got - _target_joint(raw, gamma)).sum() > 1e-2


def test_tree_enumeration_adjusted_output():
    """Tree walk with top-k and top-p on both sides, exact: the round's output
    is the adjusted target (section 7.3), and not the unadjusted one."""
    V = 5
    raw = _Tables(V=V, depth=2, seed=24)
    adj = dict(top_k=4, top_p=0.8)
    tab = _Tables(V=V, depth=0, seed=0)
    tab.p = {k: _brute_adjust(v, 1.0, **adj) for k, v in raw.p.items()}
    tab.q = {k: _brute_adjust(v, 1.0, **adj) for k, v in raw.q.items()}
    got = _enumerate_tree(tab, [2, 1], False, ztab=raw, adj=adj)
    want = _target_joint(tab, 2)
    assert abs(got.sum() - 1.0) < 1e-12
    assert np.abs(got - want).max() < 1e-12
    assert 0.5 * np.abs(got - _target_joint(raw, 2)).sum() > 1e-2


# ----------------------------------------------------------------------------
# ragged chains (DeepSeek-V4 analysis page, section 4)
# ----------------------------------------------------------------------------

def test_accept_ragged_equal_lengths_is_the_chain_accept():
    rng = np.random.default_rng(31)
    B, T, V = 3, 4, 16
    z = rng.normal(size=(B, T, V)) * 2
    q = np.stack([[_random_dist(rng, V) for _ in range(T - 1)] for _ in range(B)])
    toks = rng.integers(0, V, size=(B, T))
    U = philox.Uniforms(5, 2)
    want = acc.accept(z, q, toks, 1.0, U)
    got = acc.accept_ragged(z.reshape(B * T, V), q.reshape(B * (T - 1), V), toks.reshape(-1),
                            [b * T for b in range(B)], [T] * B, [b * (T - 1) for b in range(B)], 1.0, U)
    assert np.array_equal(got["n_accepted"], want["n_accepted"])
    assert np.array_equal(got["out_tokens"], want["out_tokens"])


def test_accept_ragged_caps_and_packing_agree():
    """Cap-accept on a fixed-width window and compact accept on the packed
    rows decide the same: sequence b's first len_b rows are the same rows, and
    it is accepted as a chain of len_b - 1 drafts either way; at most len_b - 1
    drafts are accepted."""
    rng = np.random.default_rng(32)
    B, T, V = 4, 5, 12
    z = rng.normal(size=(B, T, V)) * 2
    q = np.stack([[_random_dist(rng, V) for _ in range(T - 1)] for _ in range(B)])
    toks = rng.integers(0, V, size=(B, T))
    lens = [5, 1, 3, 2]
    U = philox.Uniforms(9, 4)
    cap = acc.accept_ragged(z.reshape(B * T, V), q.reshape(B * (T - 1), V), toks.reshape(-1),
                            [b * T for b in range(B)], lens, [b * (T - 1) for b in range(B)], 1.0, U, max_len=T)
    cu = np.concatenate([[0], np.cumsum(lens)])
    zp = np.concatenate([z[b, :lens[b]] for b in range(B)])
    qp = np.concatenate([q[b, :lens[b] - 1] for b in range(B)])
    tp = np.concatenate([toks[b, :lens[b]] for b in range(B)])
    cmp_ = acc.accept_ragged(zp, qp, tp, cu[:-1], lens, cu[:-1] - np.arange(B), 1.0, U, max_len=T)
    assert np.array_equal(cap["out_tokens"], cmp_["out_tokens"])
    assert np.all(cap["n_accepted"] <= np.array(lens) - 1)
    # a length-1 sequence has no draft: its one token is a draw from p of its row
    p1 = acc.softmax(z[1, 0], 1.0)
    x, _ = acc.inverse_cdf(p1, U(1, 0))
    assert cap["n_accepted"][1] == 0 and cap["out_tokens"][1, 0] == x


# ----------------------------------------------------------------------------
# margins of the decisions (they decide which GPU/oracle differences are
# near-ties), against hand-computed cases
# ----------------------------------------------------------------------------

def test_top2_margin_hand_cases():
    # gap between the two largest logits over the largest magnitude
    assert acc.top2_margin(np.array([1.0, 3.0, 2.0])) == pytest.approx(1.0 / 3.0, abs=1e-15)
    assert acc.top2_margin(np.array([-4.0, 0.5, 0.25])) == pytest.approx(0.25 / 4.0, abs=1e-15)
    # a tie at the top has margin 0; a single entry has nothing to flip to
    assert acc.top2_margin(np.array([2.0, 2.0, -1.0])) == 0.0
    assert acc.top2_margin(np.array([7.0])) == np.inf


def test_inverse_cdf_margin_hand_cases():
    # r = (0.2, 0.3, 0.5), u = 0.45: cumsum (0.2, 0.5, 1.0), u R = 0.45 falls in
    # token 1's interval [0.2, 0.5); distance to the nearer edge 0.05
    x, m = acc.inverse_cdf(np.array([0.2, 0.3, 0.5]), 0.45)
    assert x == 1 and m == pytest.approx(0.05, abs=1e-15)
    # unnormalised r = (1, 1, 2), R = 4, u = 0.3: u R = 1.2 in [1, 2) -> token 1,
    # distances 0.2 and 0.8, margin 0.2 / R = 0.05
    x, m = acc.inverse_cdf(np.array([1.0, 1.0, 2.0]), 0.3)
    assert x == 1 and m == pytest.approx(0.05, abs=1e-15)
    # zero-mass entries are never drawn; u = 0 takes the first positive entry
    x, m = acc.inverse_cdf(np.array([0.0, 0.0, 3.0, 1.0]), 0.0)
    assert x == 2 and m == 0.0
    # the strict test: u R exactly on a boundary goes to the next token
    x, _ = acc.inverse_cdf(np.array([0.25, 0.25, 0.5]), 0.5)
    assert x == 2


def test_accept_margin_hand_case():
    # p(x) / q(x) = 0.3 / 0.5 = 0.6, u = 0.65: rejected, margin |0.65 - 0.6|
    z = np.log(np.array([[0.3, 0.7], [0.5, 0.5]]))
    q = np.array([[0.5, 0.5]])
    n, out, m = acc.accept_chain_one(z, q, [1, 0], 1.0, lambda s: 0.65 if s == 0 else 0.1)
    assert n == 0 and m[0] == pytest.approx(0.05, abs=1e-12)
    # the residual max(0, p - q) = (0, 0.2) leaves token 1 only
    assert out == [1]
