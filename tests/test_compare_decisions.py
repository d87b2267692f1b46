"""The GPU tests' decision comparison (tests/gpu_util.compare_decisions),
pinned on hand-made oracle traces: it may excuse a differing result only by
the near-tie of the first decision on which the results differ."""
import numpy as np
import pytest

from oracle import accept as OA
from tests.gpu_util import DRAW_BAND_SHARED, compare_decisions


def _oracle(z, q, tokens, u):
    return OA.accept(z[None], None if q is None else q[None], np.asarray([tokens]), 1.0 if q is not None else 0.0,
                     lambda b, s: u[s])


def _flat_case(V=4096, seed=0):
    rng = np.random.default_rng(seed)
    z = rng.normal(size=(3, V))
    q = np.exp(z[:2] + rng.normal(size=(2, V)))
    q /= q.sum(1, keepdims=True)
    return z, q


def test_identical_results_need_no_excuse():
    z, q = _flat_case()
    orc = _oracle(z, q, [5, 7, 9], [0.99, 0.99, 0.5])
    n, out = orc["n_accepted"], orc["out_tokens"]
    assert compare_decisions(out, n, orc) == 0


def test_a_far_final_draw_is_a_mismatch():
    """At V = 4096 every final draw's own margin is below 1e-4; a token far
    from u * R on the CDF must still fail."""
    z, q = _flat_case()
    orc = _oracle(z, q, [5, 7, 9], [0.99, 0.99, 0.5])
    n, out = orc["n_accepted"].copy(), orc["out_tokens"].copy()
    k = int(n[0])
    out[0, k] = (out[0, k] + 500) % 4096
    with pytest.raises(AssertionError):
        compare_decisions(out, n, orc)


def test_a_neighbouring_draw_across_a_close_boundary_is_excused():
    """u * R just below the upper boundary of the oracle's token x: a GPU that
    drew the next positive-mass token sits 1e-9 of R away, inside the band."""
    z, q = _flat_case()
    orc = _oracle(z, q, [5, 7, 9], [0.99, 0.99, 0.5])
    t, c = orc["traces"][0]["draw"]
    x = int(orc["out_tokens"][0, int(orc["n_accepted"][0])])
    orc2 = _oracle(z, q, [5, 7, 9], [0.99, 0.99, c[x] / c[-1] - 1e-9])
    k2 = int(orc2["n_accepted"][0])
    assert int(orc2["out_tokens"][0, k2]) == x
    y = x + 1
    while c[y] - c[y - 1] <= 0:
        y += 1
    out2 = orc2["out_tokens"].copy()
    out2[0, k2] = y
    assert compare_decisions(out2, orc2["n_accepted"], orc2, draw_band=DRAW_BAND_SHARED) == 1
    # two tokens further on, the same GPU token is a mismatch
    out2[0, k2] = y + 2
    with pytest.raises(AssertionError):
        compare_decisions(out2, orc2["n_accepted"], orc2, draw_band=DRAW_BAND_SHARED)


def test_a_wrong_accept_count_is_not_hidden_by_the_draw_margin():
    """The draw margin is tiny at large V; a differing accept count is judged
    on its own test's margin only."""
    z, q = _flat_case()
    p0 = np.exp(z[0] - z[0].max())
    p0 /= p0.sum()
    x0 = int(np.argmax(q[0] / p0))              # a draft the target all but rules out
    orc = _oracle(z, q, [5, x0, 9], [0.999, 0.999, 0.5])
    n, out = orc["n_accepted"].copy(), orc["out_tokens"].copy()
    assert n[0] == 0 and orc["margins"][0][0] > 0.5
    n[0] = 1
    out[0, :2] = [x0, 3]
    with pytest.raises(AssertionError):
        compare_decisions(out, n, orc)


def test_greedy_near_tie_is_excused_only_at_its_row():
    V = 50
    z = np.zeros((3, V))
    z[0, 3] = 2.0
    z[0, 4] = 2.0 - 1e-6       # row 0: a top-2 near-tie (3 vs 4)
    z[1, 8] = 5.0              # row 1: clear argmax 8
    orc = _oracle(z, None, [1, 3, 8], [0, 0, 0])
    assert orc["n_accepted"][0] == 2
    out = np.array([[4, 0, 0]])  # GPU took 4 at row 0: excused by row 0's gap
    assert compare_decisions(out, np.array([0]), orc) == 1
    out = np.array([[3, 9, 0]])  # GPU disagrees at row 1, whose gap is large
    with pytest.raises(AssertionError):
        compare_decisions(out, np.array([1]), orc)


def test_cap_on_excused_sequences():
    V = 50
    z = np.zeros((2, V))
    z[0, 3] = 2.0
    z[0, 4] = 2.0 - 1e-6
    orc = OA.accept(np.stack([z, z]), None, np.array([[1, 3], [1, 3]]), 0.0, lambda b, s: 0.0)
    out = np.array([[4, 0], [4, 0]])
    with pytest.raises(AssertionError):
        compare_decisions(out, np.array([0, 0]), orc, cap=1)
