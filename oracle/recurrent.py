"""Recurrent-state verify, fp64.  Test infrastructure only.

What the pages fix (Kimi-K3 tuning page, "Verification on a recurrent layer
is not a cache write", and the list of hot-path operators in "Why it
retargets to ROCm without being ported"):
  * a recurrent layer carries a state that is a value, not a table indexed by
    position; verifying T = gamma + 1 speculated positions advances it
    serially through all of them;
  * the state that survives acceptance is the one after the last committed
    position, so every candidate must still be recoverable when acceptance
    has run (the engines on that page keep gamma + 1 states per request and
    scatter the survivor afterwards);
  * the layer's verify path holds a short causal convolution, the
    recurrence itself (named KDA there) and the post-verify state scatter.

The pages name the recurrence but do not write it out.  The reading taken
here is the gated delta rule that name refers to, per head h with key and
value width D, state S in R^{D x D} (rows: key channels i, columns: value
channels j):

    raw channels of position t:  x~_t = [q~ | k~ | v~]  (3 H D values)
    causal conv over positions:  c_t[ch] = sum_{w < W} cw[ch][w] * x~_{t-W+1+w}[ch]
                                 (positions before the window come from the
                                 conv state: the W-1 raw inputs that precede it)
    activation:                  x_t = silu(c_t)
    per-head q, k:               q^ = q / sqrt(|q|^2 + 1e-6) * D^-1/2,
                                 k^ = k / sqrt(|k|^2 + 1e-6)
    decay:                       S <- Diag(exp(g_t)) S        (g_t in R^D, <= 0)
    delta write:                 S <- S + beta_t k^ (v - S^T k^)^T
    output:                      o_t = S^T q^

With the pending-token convention of the chain commit (the window's first
input is the last committed token), n accepted drafts commit window positions
0 .. n, so the survivor is the state after position n and the new conv state
is the W-1 raw inputs ending at position n.

Pins (tests/test_oracle_recurrent.py): the delta write stores v under k^
exactly; it is one gradient step of 0.5 |S^T k - v|^2 with step beta
(checked against finite differences); orthonormal keys reduce it to the
outer-product memory sum_t k_t v_t^T; beta = 0 reduces it to a pure decay;
the convolution equals numpy's convolve over the concatenated sequence; a
window committed and continued equals one longer window.
"""
from __future__ import annotations

import numpy as np

L2_EPS = 1e-6


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def conv_window(x: np.ndarray, conv_w: np.ndarray, conv_state: np.ndarray) -> np.ndarray:
    """Causal depthwise convolution of one sequence's window, then SiLU.

    x [T][C] raw inputs, conv_w [C][W] taps, conv_state [W-1][C] the raw
    inputs of the W-1 positions before the window (oldest first).
    Returns [T][C]: silu(sum_w conv_w[c][w] * raw[t - (W-1) + w][c])."""
    x = np.asarray(x, dtype=np.float64)
    cw = np.asarray(conv_w, dtype=np.float64)
    st = np.asarray(conv_state, dtype=np.float64).reshape(-1, x.shape[1])
    T, C = x.shape
    W = cw.shape[1]
    out = np.zeros((T, C))
    for t in range(T):
        acc = np.zeros(C)
        for w in range(W):
            p = t - (W - 1) + w  # window position of this tap's input
            raw = x[p] if p >= 0 else st[W - 1 + p]
            acc += cw[:, w] * raw
        out[t] = silu(acc)
    return out


def l2norm(v: np.ndarray) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v / np.sqrt(np.sum(v * v) + L2_EPS)


def delta_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, decay: np.ndarray,
               beta: float) -> tuple[np.ndarray, np.ndarray]:
    """One position of the gated delta rule on normalised q, k.
    S [D][D] (key rows, value columns), decay = exp(g) [D].  Returns (S', o)."""
    S = np.asarray(decay, dtype=np.float64)[:, None] * np.asarray(S, dtype=np.float64)
    u = S.T @ k  # what the state currently returns for key k
    S = S + beta * np.outer(k, v - u)
    return S, S.T @ q


def _split_heads(xc: np.ndarray, H: int, D: int):
    q = xc[: H * D].reshape(H, D)
    k = xc[H * D: 2 * H * D].reshape(H, D)
    v = xc[2 * H * D:].reshape(H, D)
    return q, k, v


def verify(x, gate, beta, conv_w, conv_state, state, slots=None):
    """Verify window of B sequences.

    x [B][T][3HD], gate [B][T][H][D] (log decay), beta [B][T][H],
    conv_w [3HD][W], conv_state [S][W-1][3HD], state [S][H][D][D], slots [B]
    (pool slot of each sequence; None = b).
    Returns (out [B][T][H][D], snapshots [B][T][H][D][D])."""
    x = np.asarray(x, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    B, T, _ = x.shape
    H, D = gate.shape[2], gate.shape[3]
    out = np.zeros((B, T, H, D))
    snaps = np.zeros((B, T, H, D, D))
    for b in range(B):
        s = b if slots is None else int(slots[b])
        xc = conv_window(x[b], conv_w, conv_state[s])
        for h in range(H):
            S = np.asarray(state[s][h], dtype=np.float64)
            for t in range(T):
                q, k, v = _split_heads(xc[t], H, D)
                qh = l2norm(q[h]) / np.sqrt(D)
                kh = l2norm(k[h])
                S, o = delta_step(S, qh, kh, v[h], np.exp(gate[b, t, h]), beta[b, t, h])
                out[b, t, h] = o
                snaps[b, t, h] = S
    return out, snaps


def commit(x, num_accepted, conv_state, state, snapshots, slots=None):
    """Post-verify state scatter.  With n = num_accepted[b] clamped into
    [0, T-1], the sequence's pool slot receives the state after window
    position n and the conv state of the W-1 raw inputs ending at position n.
    Returns new (conv_state, state) arrays; the inputs are not modified."""
    x = np.asarray(x, dtype=np.float64)
    cs = np.array(conv_state, dtype=np.float64, copy=True)
    st = np.array(state, dtype=np.float64, copy=True)
    B, T, _ = x.shape
    Wm1 = cs.shape[1]
    for b in range(B):
        s = b if slots is None else int(slots[b])
        n = min(max(int(num_accepted[b]), 0), T - 1)
        st[s] = snapshots[b][n]
        old = np.array(cs[s], copy=True)
        for w in range(Wm1):
            p = n - (Wm1 - 1) + w  # window position of the kept raw input
            cs[s][w] = x[b][p] if p >= 0 else old[Wm1 + p]
    return cs, st
