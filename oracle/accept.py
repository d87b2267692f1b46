"""Speculative-sampling accept / resample / bonus, fp64.  Test infrastructure.

Chain (CS349E Lecture 6, "Optimizing Autoregressive Decode", section 6.2,
Leviathan et al.'s Algorithm 1, steps 3-5):
  for i = 1 .. gamma: accept x_i when u_i < p_i(x_i) / q_i(x_i), else stop;
  n = number accepted; if n < gamma draw the extra token from
  norm(max(0, p_{n+1} - q_{n+1})), otherwise take a bonus token from p_{gamma+1};
  emit x_1 .. x_n and the extra token.
The test u < p/q is evaluated as u * q < p (the Kimi-K3 tuning page, "What
SGLang actually runs": a uniform times the draft probability under the target
probability), which avoids the division.

Sampling settings (section 7.3): every setting is sampling from an adjusted
distribution, and speculative sampling on the adjusted p and q yields the
adjusted p.  p_i = softmax(z_i / T), then top-k keeps the k most likely tokens
(the rest set to zero, as logits of -inf) and renormalises, then top-p keeps
the nucleus (the shortest run of most likely tokens whose renormalised mass
reaches top_p) and renormalises (see `adjust`).  q arrives already adjusted by
the draft side, the same way.  Greedy (section 7.4, T = 0): accept x_i iff it
equals argmax z_i; the extra token is argmax z_{n+1}, the only positive term of
the residual of two one-hot distributions.

Token tree (section 10.3 gives only greedy trees; the sampled walk is the
reading taken here, exact for any draft distribution by section 7.3's remark
that the proof holds whatever q is): at node v with target r = p_v and the
distribution q' its children were drawn from, test the children in their
order; a rejected child replaces r by norm(max(0, r - q')) and, for children
drawn without replacement, removes that token from q' and renormalises.  All
children rejected: draw from r.  Reached a leaf: bonus from p_leaf.  Greedy:
descend into the child whose token is argmax p_v, else emit that argmax.

Readings where the pages say nothing:
  * inverse-CDF sampling in token-id order with a strict test,
    token = min{x : sum_{y<=x} r(y) > u * sum(r)};
  * greedy ties resolve to the lowest token id;
  * a residual whose mass is zero in floating point falls back to the
    distribution it was taken from (p for the chain);
  * uniforms come from Philox4x64-10 (see philox.py for slot assignment);
  * "most likely" orders tokens by logit, largest first, equal logits by
    lower id; top-k is applied before top-p (the order an engine's verify
    calls its two renormalisations in, Kimi-K3 tuning page); the nucleus
    is the shortest such prefix with cumulative mass >= top_p; top_k = 0
    and top_p = 1 switch them off; greedy ignores both (the argmax is
    always kept).

Each function also returns a trace of the margins of the decisions it took, so
a test can tell a genuine mismatch from a near-tie: accept tests record
|u - min(1, p/q)|, draws record the distance of u * R to the nearest CDF
boundary divided by R, argmax decisions the top-2 gap over max |z|.  The
nucleus cuts' margins (distance of the cumulative mass to top_p) are kept
apart, in `adjust_margins`: they are masses, compared against a different
band.
"""
from __future__ import annotations

import numpy as np


def softmax(z: np.ndarray, temperature: float) -> np.ndarray:
    s = np.asarray(z, dtype=np.float64) / temperature
    s = s - s.max()
    e = np.exp(s)
    return e / e.sum()


def likelihood_order(z: np.ndarray) -> np.ndarray:
    """Token ids from most to least likely: descending logit, equal logits by
    ascending id."""
    z = np.asarray(z, dtype=np.float64)
    return np.lexsort((np.arange(z.size), -z))


def adjust(z: np.ndarray, temperature: float, top_k: int = 0, top_p: float = 1.0):
    """Adjusted target distribution (section 7.3): softmax(z / T) restricted to
    the top-k tokens, renormalised, then to the top-p nucleus, renormalised.
    Returns (p, margin): margin is the distance of the nucleus' cumulative
    mass to top_p at the cut (how far the boundary decision is from flipping),
    inf when top-p is off."""
    p = softmax(z, temperature)
    V = p.size
    margin = np.inf
    if not (0 < top_k < V) and not (top_p < 1.0):
        return p, margin
    order = likelihood_order(z)
    kept = order[:top_k] if 0 < top_k < V else order
    if top_p < 1.0:
        pk = p[kept] / p[kept].sum()
        c = np.cumsum(pk)
        hit = np.nonzero(c >= top_p)[0]
        n = int(hit[0]) if hit.size else kept.size - 1
        margin = float(c[n] - top_p) if hit.size else np.inf
        if n > 0:
            margin = min(margin, float(top_p - c[n - 1]))
        kept = kept[:n + 1]
    r = np.zeros(V)
    r[kept] = p[kept]
    return r / r.sum(), margin


def argmax_lowest(z: np.ndarray) -> int:
    """Index of the maximum; ties go to the lowest index."""
    return int(np.argmax(np.asarray(z)))


def top2_margin(z: np.ndarray) -> float:
    z = np.asarray(z, dtype=np.float64)
    if z.size < 2:
        return np.inf
    part = np.partition(z, -2)
    scale = max(np.abs(z).max(), 1e-300)
    return float((part[-1] - part[-2]) / scale)


def inverse_cdf(r: np.ndarray, u: float):
    """Smallest x with cumsum(r)[x] > u * R, R = cumsum(r)[-1].  Returns
    (token, margin)."""
    c = np.cumsum(np.asarray(r, dtype=np.float64))
    R = c[-1]
    t = u * R
    x = int(np.argmax(c > t))
    lo = c[x - 1] if x > 0 else 0.0
    margin = min(t - lo, c[x] - t) / R
    return x, float(margin)


def accept_chain_one(z, q, tokens, temperature, u, _variant="residual", top_k=0, top_p=1.0,
                     adjust_margins=None, trace=None):
    """One sequence.  z [gamma+1, V] target logits for the window rows;
    q [gamma, V] draft probabilities (row j: distribution draft j+1 came from);
    tokens [gamma+1] = [pending, x_1 .. x_gamma]; u(slot) -> uniform;
    top_k / top_p adjust the target (see `adjust`); the nucleus cuts'
    margins are appended to `adjust_margins` when given.
    Returns (n_accepted, emitted tokens [n+1], margins).

    _variant plants one of the two wrong implementations of section 7.5 for
    negative-control tests only: "resample_from_p" draws the extra token from p
    after a rejection; "deterministic" rejects whenever q > p.

    With `trace` (a dict) the decisions' positions are recorded for aligning
    another implementation's output with this one: trace["depths"][k] is the
    emitted position decision k (margins[k]) decides, and trace["draw"] is
    (u * R, cumsum(r)) of the final inverse-CDF draw (sampled mode)."""
    gamma = len(tokens) - 1
    margins = []
    depths = [] if trace is None else trace.setdefault("depths", [])
    adjust_margins = [] if adjust_margins is None else adjust_margins
    if temperature == 0.0:
        n = 0
        while n < gamma:
            am = argmax_lowest(z[n])
            margins.append(top2_margin(z[n]))
            depths.append(n)
            if int(tokens[n + 1]) != am:
                break
            n += 1
        margins.append(top2_margin(z[n]))
        depths.append(n)
        extra = argmax_lowest(z[n])
        return n, [int(t) for t in tokens[1:n + 1]] + [extra], margins

    n = 0
    for i in range(gamma):
        p, am = adjust(z[i], temperature, top_k, top_p)
        adjust_margins.append(am)
        x = int(tokens[i + 1])
        ui = u(i)
        margins.append(abs(ui - min(1.0, p[x] / q[i][x])) if q[i][x] > 0 else np.inf)
        depths.append(i)
        ok = (q[i][x] <= p[x]) if _variant == "deterministic" else (ui * q[i][x] < p[x])
        if ok:
            n += 1
        else:
            break
    p, am = adjust(z[n], temperature, top_k, top_p)
    adjust_margins.append(am)
    if n < gamma and _variant != "resample_from_p":
        r = np.maximum(0.0, p - np.asarray(q[n], dtype=np.float64))
        if not (r.sum() > 0.0):
            r = p
    else:
        r = p
    extra, m = inverse_cdf(r, u(gamma))
    margins.append(m)
    depths.append(n)
    if trace is not None:
        c = np.cumsum(np.asarray(r, dtype=np.float64))
        trace["draw"] = (u(gamma) * c[-1], c)
    return n, [int(t) for t in tokens[1:n + 1]] + [extra], margins


def accept_tree_one(z, q, tokens, parent, temperature, u, replacement=False, _variant="residual",
                    top_k=0, top_p=1.0, adjust_margins=None, trace=None):
    """One sequence with a token tree.  z [T, V] logits per node; q [T, V] the
    draft distribution each node's children were drawn from; tokens [T] node
    tokens (node 0 = pending token); parent [T] (root -1).  u(slot) -> uniform.
    Returns (path node ids from the root, emitted tokens, margins).

    _variant plants a wrong walk for negative-control tests only:
    "resample_from_p" keeps r = p_v after rejected siblings; "no_renorm"
    removes a rejected child from q' without renormalising q'."""
    T = len(tokens)
    children = [[] for _ in range(T)]
    for c in range(1, T):
        children[int(parent[c])].append(c)
    margins = []
    depths = [] if trace is None else trace.setdefault("depths", [])
    adjust_margins = [] if adjust_margins is None else adjust_margins
    v = 0
    path = [0]

    def final_draw(r):
        extra, m = inverse_cdf(r, u(T - 1))
        margins.append(m)
        depths.append(len(path) - 1)
        if trace is not None:
            c = np.cumsum(np.asarray(r, dtype=np.float64))
            trace["draw"] = (u(T - 1) * c[-1], c)
        return extra

    if temperature == 0.0:
        while True:
            am = argmax_lowest(z[v])
            margins.append(top2_margin(z[v]))
            depths.append(len(path) - 1)
            nxt = [c for c in children[v] if int(tokens[c]) == am]
            if not nxt:
                return path, [int(tokens[c]) for c in path[1:]] + [am], margins
            v = nxt[0]
            path.append(v)

    while True:
        r, am = adjust(z[v], temperature, top_k, top_p)
        adjust_margins.append(am)
        if not children[v]:
            extra = final_draw(r)
            return path, [int(tokens[c]) for c in path[1:]] + [extra], margins
        qp = np.asarray(q[v], dtype=np.float64).copy()
        accepted = None
        for c in children[v]:
            x = int(tokens[c])
            uc = u(c - 1)
            margins.append(abs(uc - min(1.0, r[x] / qp[x])) if qp[x] > 0 else np.inf)
            depths.append(len(path) - 1)
            if uc * qp[x] < r[x]:
                accepted = c
                break
            if _variant == "resample_from_p":
                continue
            res = np.maximum(0.0, r - qp)
            if res.sum() > 0.0:
                r = res / res.sum()
            if not replacement:
                qp[x] = 0.0
                s = qp.sum()
                if s > 0.0 and _variant != "no_renorm":
                    qp = qp / s
        if accepted is None:
            extra = final_draw(r)
            return path, [int(tokens[c]) for c in path[1:]] + [extra], margins
        v = accepted
        path.append(v)


def accept(logits, q, tokens, temperature, uniforms, tree_parent=None, replacement=False,
           _variant="residual", top_k=0, top_p=1.0):
    """Batch driver.  logits [B, T, V]; q [B, T-1, V] (chain) or [B, T, V] (tree);
    tokens [B, T]; uniforms(b, slot) -> float; top_k / top_p as in `adjust`.
    Returns dict with n_accepted [B], out_tokens [B, T] (-1 padded), paths,
    margins and adjust_margins (lists per sequence), and traces (per sequence:
    the emitted position of each margin's decision, and the final draw's
    u * R and CDF, see accept_chain_one)."""
    logits = np.asarray(logits)
    B, T = np.asarray(tokens).shape
    n_acc = np.zeros(B, dtype=np.int64)
    out = np.full((B, T), -1, dtype=np.int64)
    paths, margins, adj_margins, traces = [], [], [], []
    for b in range(B):
        ub = (lambda s, b=b: uniforms(b, s))
        am = []
        tr = {}
        if tree_parent is None:
            n, toks, m = accept_chain_one(logits[b], None if q is None else q[b], tokens[b],
                                          temperature, ub, _variant, top_k, top_p, am, tr)
            path = list(range(n + 1))
        else:
            path, toks, m = accept_tree_one(logits[b], None if q is None else q[b], tokens[b],
                                            tree_parent[b], temperature, ub, replacement, _variant,
                                            top_k, top_p, am, tr)
            n = len(path) - 1
        traces.append(tr)
        n_acc[b] = n
        out[b, : len(toks)] = toks
        paths.append(path)
        margins.append(m)
        adj_margins.append(am)
    return {"n_accepted": n_acc, "out_tokens": out, "paths": paths, "margins": margins,
            "adjust_margins": adj_margins, "traces": traces}


def accept_ragged(logits_rows, q_rows, tokens_rows, row_start, lens, q_start, temperature, uniforms,
                  max_len=None, top_k=0, top_p=1.0):
    """Ragged chains (the DeepSeek-V4 analysis page, section 4): sequence b is
    a chain of gamma_b = lens[b] - 1 drafts whose window rows start at
    row_start[b] of logits_rows / tokens_rows and whose draft distributions
    start at q_start[b] of q_rows.  Each sequence is accepted exactly as a
    chain of its own length (same uniforms' slots 0 .. gamma_b).  Compact
    mode packs the rows; cap-accept keeps a fixed width T and caps the
    length.  Returns the same dict as `accept`, out_tokens [B, max_len]."""
    B = len(lens)
    max_len = int(max(lens)) if max_len is None else int(max_len)
    n_acc = np.zeros(B, dtype=np.int64)
    out = np.full((B, max_len), -1, dtype=np.int64)
    margins, adj_margins, paths, traces = [], [], [], []
    for b in range(B):
        r0, n_b = int(row_start[b]), int(lens[b])
        z = np.asarray(logits_rows)[r0:r0 + n_b]
        q = None if q_rows is None else np.asarray(q_rows)[int(q_start[b]):int(q_start[b]) + n_b - 1]
        toks = np.asarray(tokens_rows)[r0:r0 + n_b]
        am = []
        tr = {}
        n, em, m = accept_chain_one(z, q, toks, temperature, (lambda s, b=b: uniforms(b, s)),
                                    top_k=top_k, top_p=top_p, adjust_margins=am, trace=tr)
        traces.append(tr)
        n_acc[b] = n
        out[b, :len(em)] = em
        margins.append(m)
        adj_margins.append(am)
        paths.append(list(range(n + 1)))
    return {"n_accepted": n_acc, "out_tokens": out, "paths": paths, "margins": margins,
            "adjust_margins": adj_margins, "traces": traces}
