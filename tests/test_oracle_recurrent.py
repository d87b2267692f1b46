"""Pins of the recurrent-state verify oracle (oracle/recurrent.py) against
closed forms, a library routine and brute force -- never against itself."""
import numpy as np
import pytest

from oracle import recurrent as rec
import synth


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# the delta write
# ----------------------------------------------------------------------------

def test_delta_write_stores_v_under_its_key():
    """With no decay and beta = 1, the updated state returns exactly v for the
    (unit) key it was written under, whatever it held before."""
    r = _rng(1)
    D = 16
    S = r.normal(size=(D, D))
    k = r.normal(size=D)
    k /= np.linalg.norm(k)
    v = r.normal(size=D)
    S2, _ = rec.delta_step(S, np.zeros(D), k, v, np.ones(D), 1.0)
    np.testing.assert_allclose(S2.T @ k, v, rtol=0, atol=1e-12)
    # directions orthogonal to k are untouched
    w = r.normal(size=D)
    w -= (w @ k) * k
    np.testing.assert_allclose(S2.T @ w, S.T @ w, rtol=0, atol=1e-12)


def test_delta_write_is_one_gradient_step():
    """The write is one step of size beta down the gradient of the regression
    loss 0.5 |S^T k - v|^2, taken after the decay; the gradient here comes from
    central finite differences of the loss, entry by entry."""
    r = _rng(2)
    D = 5
    S0 = r.normal(size=(D, D))
    k = r.normal(size=D)
    v = r.normal(size=D)
    decay = np.exp(-r.uniform(0, 0.5, size=D))
    beta = 0.37
    Sd = decay[:, None] * S0

    def loss(S):
        e = S.T @ k - v
        return 0.5 * float(e @ e)

    grad = np.zeros((D, D))
    h = 1e-6
    for i in range(D):
        for j in range(D):
            Sp, Sm = Sd.copy(), Sd.copy()
            Sp[i, j] += h
            Sm[i, j] -= h
            grad[i, j] = (loss(Sp) - loss(Sm)) / (2 * h)
    S1, _ = rec.delta_step(S0, np.zeros(D), k, v, decay, beta)
    np.testing.assert_allclose(S1, Sd - beta * grad, rtol=0, atol=1e-8)


def test_orthonormal_keys_give_the_outer_product_memory():
    """From a zero state with no decay and beta = 1, orthonormal keys store
    sum_t k_t v_t^T, and querying with k_s reads back v_s."""
    r = _rng(3)
    D, T = 12, 7
    Q, _ = np.linalg.qr(r.normal(size=(D, D)))
    keys = Q[:, :T].T  # T orthonormal rows
    vals = r.normal(size=(T, D))
    S = np.zeros((D, D))
    for t in range(T):
        S, o = rec.delta_step(S, keys[t], keys[t], vals[t], np.ones(D), 1.0)
        np.testing.assert_allclose(o, vals[t], atol=1e-12)
    np.testing.assert_allclose(S, keys.T @ vals, atol=1e-12)
    for s in range(T):
        np.testing.assert_allclose(S.T @ keys[s], vals[s], atol=1e-12)


# ----------------------------------------------------------------------------
# convolution and normalisation
# ----------------------------------------------------------------------------

def _numpy_conv(x, cw, cs):
    """np.convolve over each channel's concatenated sequence (state, window):
    the valid part of the correlation with the taps."""
    T, C = x.shape
    W = cw.shape[1]
    out = np.zeros((T, C))
    for c in range(C):
        z = np.concatenate([cs[:, c], x[:, c]]) if W > 1 else x[:, c]
        out[:, c] = np.convolve(z, cw[c][::-1], mode="valid")
    return out


@pytest.mark.parametrize("W", [1, 2, 4])
def test_conv_window_matches_numpy_convolve(W):
    r = _rng(4 + W)
    T, C = 5, 9
    x = r.normal(size=(T, C))
    cw = r.normal(size=(C, W))
    cs = r.normal(size=(W - 1, C))
    pre = _numpy_conv(x, cw, cs)
    np.testing.assert_allclose(rec.conv_window(x, cw, cs), pre / (1 + np.exp(-pre)), atol=1e-13)


def test_conv_special_taps():
    r = _rng(9)
    T, C, W = 4, 6, 4
    x = r.normal(size=(T, C))
    cs = r.normal(size=(W - 1, C))
    last = np.zeros((C, W))
    last[:, W - 1] = 1.0
    np.testing.assert_allclose(rec.conv_window(x, last, cs), x / (1 + np.exp(-x)), atol=1e-14)
    first = np.zeros((C, W))
    first[:, 0] = 1.0  # reads the input W-1 positions back: the state, then x
    z = np.concatenate([cs, x])[:T]
    np.testing.assert_allclose(rec.conv_window(x, first, cs), z / (1 + np.exp(-z)), atol=1e-14)


def test_l2norm():
    r = _rng(10)
    v = 100.0 * r.normal(size=64)
    assert abs(np.linalg.norm(rec.l2norm(v)) - 1.0) < 1e-9
    np.testing.assert_array_equal(rec.l2norm(np.zeros(8)), np.zeros(8))


# ----------------------------------------------------------------------------
# the whole window
# ----------------------------------------------------------------------------

def _inputs(B, T, H, D, W, slots, seed):
    inp = synth.make_recurrent_inputs(synth.RecurrentShape(H, D, W), B, T, slots, seed=seed)
    return {k: v.double().numpy() for k, v in inp.items()}


def test_zero_write_is_pure_decay():
    """beta = 0: the state only decays, S_t = Diag(exp(g_1 + .. + g_t)) S_0, and
    o_t = S_t^T q^_t with q^ from the numpy convolution."""
    B, T, H, D, W = 2, 4, 2, 8, 3
    a = _inputs(B, T, H, D, W, B, 11)
    a["beta"][:] = 0.0
    out, snaps = rec.verify(a["x"], a["gate"], a["beta"], a["conv_w"], a["conv_state"], a["state"])
    for b in range(B):
        pre = _numpy_conv(a["x"][b], a["conv_w"], a["conv_state"][b])
        xc = pre / (1 + np.exp(-pre))
        for h in range(H):
            cum = np.zeros(D)
            for t in range(T):
                cum += a["gate"][b, t, h]
                S = np.exp(cum)[:, None] * a["state"][b, h]
                np.testing.assert_allclose(snaps[b, t, h], S, rtol=1e-12, atol=1e-14)
                q = xc[t, h * D:(h + 1) * D]
                q = q / np.sqrt(q @ q + 1e-6) / np.sqrt(D)
                np.testing.assert_allclose(out[b, t, h], S.T @ q, rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("n", [0, 1, 3])
def test_commit_then_continue_equals_one_long_window(n):
    """Window 1 (T1 positions) committed after n accepted drafts, then window 2
    from the survivor, equals one window over positions 0..n of window 1
    followed by window 2: the survivor index and the conv-state update agree
    with the causal definition."""
    B, T1, T2, H, D, W = 2, 4, 3, 2, 8, 4
    a = _inputs(B, T1, H, D, W, B, 20)
    b2 = _inputs(B, T2, H, D, W, B, 21)
    out1, snaps1 = rec.verify(a["x"], a["gate"], a["beta"], a["conv_w"], a["conv_state"], a["state"])
    nacc = np.full(B, n)
    cs, st = rec.commit(a["x"], nacc, a["conv_state"], a["state"], snaps1)
    out2, snaps2 = rec.verify(b2["x"], b2["gate"], b2["beta"], a["conv_w"], cs, st)

    keep = n + 1
    xl = np.concatenate([a["x"][:, :keep], b2["x"]], axis=1)
    gl = np.concatenate([a["gate"][:, :keep], b2["gate"]], axis=1)
    bl = np.concatenate([a["beta"][:, :keep], b2["beta"]], axis=1)
    outl, snapsl = rec.verify(xl, gl, bl, a["conv_w"], a["conv_state"], a["state"])
    np.testing.assert_allclose(out1[:, :keep], outl[:, :keep], rtol=0, atol=0)
    np.testing.assert_allclose(out2, outl[:, keep:], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(snaps2, snapsl[:, keep:], rtol=1e-12, atol=1e-14)


def test_commit_clamps_and_follows_slots():
    B, T, H, D, W, NS = 3, 3, 1, 4, 2, 5
    a = _inputs(B, T, H, D, W, NS, 30)
    slots = np.array([4, 0, 2])
    out, snaps = rec.verify(a["x"], a["gate"], a["beta"], a["conv_w"], a["conv_state"], a["state"], slots)
    # the same sequences with their pool rows moved to b
    out_b, _ = rec.verify(a["x"], a["gate"], a["beta"], a["conv_w"], a["conv_state"][slots], a["state"][slots])
    np.testing.assert_array_equal(out, out_b)
    cs, st = rec.commit(a["x"], [-5, 99, 1], a["conv_state"], a["state"], snaps, slots)
    np.testing.assert_array_equal(st[4], snaps[0, 0])
    np.testing.assert_array_equal(st[0], snaps[1, T - 1])
    np.testing.assert_array_equal(st[2], snaps[2, 1])
    for untouched in (1, 3):
        np.testing.assert_array_equal(st[untouched], a["state"][untouched])
        np.testing.assert_array_equal(cs[untouched], a["conv_state"][untouched])
    np.testing.assert_array_equal(cs[0][0], a["x"][1, T - 1])  # W-1 = 1 raw input kept
    np.testing.assert_array_equal(cs[4][0], a["x"][0, 0])
