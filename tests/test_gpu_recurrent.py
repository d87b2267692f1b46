"""Recurrent-state verify on the GPU (spec_recurrent_verify / _commit) against
the fp64 oracle (oracle/recurrent.py): window outputs, the per-position state
snapshots, both commit modes, chained rounds and the full-size shape.

Tolerance: the kernels compute in fp32.  Every reduction is a sum of at most
D = 128 products, a window has at most 16 positions and the decay keeps the
state bounded, so the rounding error stays within a few 1e-6 of the
magnitudes involved; REC_RTOL = 1e-4 of the largest magnitude of each
compared (sequence, head) block leaves room for that and still fails any
dropped term, wrong index or transposed operand (errors of order 1)."""
import numpy as np
import pytest
import torch

import speculative_decoding_verify_spec_amd as S
import synth
from oracle import recurrent as OR
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

REC_RTOL = 1e-4


def _close(gpu, orc, what, axes):
    """max |gpu - orc| over each block (the trailing `axes` dims) within
    REC_RTOL of that block's largest |orc|."""
    g = np.asarray(gpu, np.float64)
    o = np.asarray(orc, np.float64)
    red = tuple(range(o.ndim - axes, o.ndim))
    err = np.abs(g - o).max(axis=red)
    scale = np.maximum(np.abs(o).max(axis=red), 1e-30)
    worst = float((err / scale).max()) if err.size else 0.0
    assert worst <= REC_RTOL, f"{what}: relative error {worst:.3e}"
    return worst


class _Pool:
    def __init__(self, rs, B, T, n_slots, seed):
        self.rs, self.B, self.T = rs, B, T
        self.inp = synth.make_recurrent_inputs(rs, B, T, n_slots, seed=seed)
        self.d = {k: v.to(dev()).contiguous() for k, v in self.inp.items()}
        self.dims = S.spec_recurrent_dims(rs.n_heads, rs.head_dim, rs.conv_width, n_slots)

    def host(self, k):
        return self.inp[k].double().numpy()


def _verify(p, slot, snapshots=True, stream=None):
    rs, B, T = p.rs, p.B, p.T
    H, D = rs.n_heads, rs.head_dim
    out = torch.full((B, T, H, D), 7.0, device=dev())
    snaps = torch.full((B, T, H, D, D), 7.0, device=dev()) if snapshots else None
    S.spec_recurrent_verify(p.dims, B, T, p.d["x"], p.d["gate"], p.d["beta"], p.d["conv_w"], slot,
                            p.d["conv_state"], p.d["state"], out, snaps)
    return out, snaps


def _commit(p, slot, nacc, snaps, conv_state, state):
    S.spec_recurrent_commit(p.dims, p.B, p.T, p.d["x"], p.d["gate"], p.d["beta"], p.d["conv_w"], slot, nacc,
                            snaps, conv_state, state)


CASES = [
    # B, T, H, D, W, n_slots, slots (None = identity)
    (3, 4, 4, 128, 4, 3, None),
    (2, 1, 2, 64, 1, 2, None),
    (2, 16, 2, 64, 8, 2, None),
    (5, 3, 3, 128, 2, 7, [6, 0, 3, -1, 2]),  # a permuted pool, one sequence skipped
]


@pytest.mark.parametrize("B,T,H,D,W,NS,slots", CASES)
def test_verify_and_both_commits_match_oracle(B, T, H, D, W, NS, slots):
    print(f"recurrent parity B={B} T={T} H={H} D={D} W={W} slots={slots}", flush=True)
    rs = synth.RecurrentShape(H, D, W)
    p = _Pool(rs, B, T, NS, seed=100 + B * 7 + T)
    slot_d = torch.tensor(slots, dtype=torch.int32, device=dev()) if slots is not None else None
    out, snaps = _verify(p, slot_d)
    out_ns, _ = _verify(p, slot_d, snapshots=False)
    torch.cuda.synchronize()
    # keeping snapshots does not change the outputs
    assert torch.equal(out, out_ns)

    live = [b for b in range(B) if slots is None or slots[b] >= 0]
    ol = None if slots is None else [slots[b] for b in live]
    o_out, o_snaps = OR.verify(p.host("x")[live], p.host("gate")[live], p.host("beta")[live], p.host("conv_w"),
                               p.host("conv_state"), p.host("state"), ol)
    out_h, snaps_h = out.cpu().numpy(), snaps.cpu().numpy()
    _close(out_h[live], o_out, "outputs", 1)
    _close(snaps_h[live], o_snaps, "snapshots", 2)
    for b in range(B):
        if b not in live:  # skipped sequence: nothing written
            assert (out_h[b] == 7.0).all() and (snaps_h[b] == 7.0).all()

    # accepted counts, two of them outside [0, T-1] (clamped)
    nacc = [(b * 5 + 1) % (T + 2) - 1 for b in range(B)]
    nacc_d = torch.tensor(nacc, dtype=torch.int32, device=dev())
    cs_a, st_a = p.d["conv_state"].clone(), p.d["state"].clone()
    cs_b, st_b = p.d["conv_state"].clone(), p.d["state"].clone()
    _commit(p, slot_d, nacc_d, snaps, cs_a, st_a)   # scatter the survivor snapshot
    _commit(p, slot_d, nacc_d, None, cs_b, st_b)    # replay the committed positions
    torch.cuda.synchronize()
    assert torch.equal(st_a, st_b), "replay and scatter commits differ"
    assert torch.equal(cs_a, cs_b)
    o_cs, o_st = OR.commit(p.host("x")[live], [nacc[b] for b in live], p.host("conv_state"), p.host("state"),
                           o_snaps, ol)
    _close(st_a.cpu().numpy(), o_st, "committed state", 2)
    # the conv state holds copied inputs: exact
    np.testing.assert_array_equal(cs_a.cpu().double().numpy(), o_cs)


def test_chained_rounds_match_oracle():
    """Three verify -> accept -> commit rounds on one pool (replay commits),
    each round's window drawn afresh; the pool after every round and every
    round's outputs follow the oracle's rounds."""
    rs = synth.RecurrentShape(4, 128, 4)
    B, T = 4, 4
    dims = S.spec_recurrent_dims(4, 128, 4, B)
    base = synth.make_recurrent_inputs(rs, B, T, B, seed=7)
    cs_d, st_d = base["conv_state"].to(dev()), base["state"].to(dev())
    cs_o, st_o = base["conv_state"].double().numpy(), base["state"].double().numpy()
    for rnd in range(3):
        print(f"recurrent chained round {rnd}", flush=True)
        w = synth.make_recurrent_inputs(rs, B, T, B, seed=1000 + rnd)
        wd = {k: w[k].to(dev()) for k in ("x", "gate", "beta")}
        conv_w = base["conv_w"].to(dev())
        out = torch.empty((B, T, 4, 128), device=dev())
        S.spec_recurrent_verify(dims, B, T, wd["x"], wd["gate"], wd["beta"], conv_w, None, cs_d, st_d, out, None)
        nacc = [(rnd + b) % T for b in range(B)]
        S.spec_recurrent_commit(dims, B, T, wd["x"], wd["gate"], wd["beta"], conv_w, None,
                                torch.tensor(nacc, dtype=torch.int32, device=dev()), None, cs_d, st_d)
        torch.cuda.synchronize()
        h = {k: w[k].double().numpy() for k in ("x", "gate", "beta")}
        o_out, o_snaps = OR.verify(h["x"], h["gate"], h["beta"], base["conv_w"].double().numpy(), cs_o, st_o)
        cs_o, st_o = OR.commit(h["x"], nacc, cs_o, st_o, o_snaps)
        _close(out.cpu().numpy(), o_out, f"round {rnd} outputs", 1)
        _close(st_d.cpu().numpy(), st_o, f"round {rnd} state", 2)
        np.testing.assert_array_equal(cs_d.cpu().double().numpy(), cs_o)


def test_full_size_sampled():
    """48 sequences, a 4-position window, 32 heads of width 128, 4 taps (the
    shape bench.py --recurrent 48 times): all outputs checked, snapshots and
    committed states of a sample of sequences."""
    rs = synth.RECURRENT_8B
    B, T = 48, 4
    print("recurrent full size B=48 T=4", flush=True)
    p = _Pool(rs, B, T, B, seed=4242)
    out, snaps = _verify(p, None)
    nacc = torch.tensor([b % T for b in range(B)], dtype=torch.int32, device=dev())
    st_a = p.d["state"].clone()
    cs_a = p.d["conv_state"].clone()
    _commit(p, None, nacc, None, cs_a, st_a)
    torch.cuda.synchronize()
    o_out, _ = OR.verify(p.host("x"), p.host("gate"), p.host("beta"), p.host("conv_w"), p.host("conv_state"),
                         p.host("state"))
    _close(out.cpu().numpy(), o_out, "outputs", 1)
    sample = [0, 17, 46, 47]
    o_out_s, o_snaps = OR.verify(p.host("x")[sample], p.host("gate")[sample], p.host("beta")[sample],
                                 p.host("conv_w"), p.host("conv_state")[sample], p.host("state")[sample])
    _close(snaps[sample].cpu().numpy(), o_snaps, "snapshots", 2)
    _, o_st = OR.commit(p.host("x")[sample], nacc.cpu().numpy()[sample], p.host("conv_state")[sample],
                        p.host("state")[sample], o_snaps)
    _close(st_a[sample].cpu().numpy(), o_st, "committed state", 2)


def test_empty_batch_is_a_no_op():
    dims = S.spec_recurrent_dims(2, 64, 4, 2)
    z = torch.zeros(16, device=dev())
    assert S.spec_recurrent_verify(dims, 0, 4, z, z, z, z, None, z, z, z, None, check=False) == S.SPEC_OK
    assert S.spec_recurrent_commit(dims, 0, 4, z, z, z, z, None, z, None, z, z, check=False) == S.SPEC_OK


def test_commit_verify_equals_separate_calls():
    """Three rounds as fused calls (commit of the previous window + verify of
    the new one) against the same rounds as verify + replay commit: the
    outputs of every round and the final pool are bit-identical, and follow
    the oracle."""
    rs = synth.RecurrentShape(4, 128, 4)
    B, T = 3, 4
    dims = S.spec_recurrent_dims(4, 128, 4, B)
    base = synth.make_recurrent_inputs(rs, B, T, B, seed=11)
    conv_w = base["conv_w"].to(dev())
    cs_a, st_a = base["conv_state"].to(dev()), base["state"].to(dev())
    cs_b, st_b = cs_a.clone(), st_a.clone()
    cs_o, st_o = base["conv_state"].double().numpy(), base["state"].double().numpy()
    prev = None
    for rnd in range(3):
        print(f"recurrent fused round {rnd}", flush=True)
        w = synth.make_recurrent_inputs(rs, B, T, B, seed=2000 + rnd)
        wd = {k: w[k].to(dev()) for k in ("x", "gate", "beta")}
        nacc = torch.tensor([(rnd * 2 + b) % (T + 1) - (b == 2) for b in range(B)], dtype=torch.int32, device=dev())
        out_a = torch.empty((B, T, 4, 128), device=dev())
        S.spec_recurrent_verify(dims, B, T, wd["x"], wd["gate"], wd["beta"], conv_w, None, cs_a, st_a, out_a, None)
        S.spec_recurrent_commit(dims, B, T, wd["x"], wd["gate"], wd["beta"], conv_w, None, nacc, None, cs_a, st_a)
        out_b = torch.empty_like(out_a)
        if prev is None:
            S.spec_recurrent_commit_verify(dims, B, 0, None, None, None, None, T, wd["x"], wd["gate"], wd["beta"],
                                           conv_w, None, cs_b, st_b, out_b)
        else:
            S.spec_recurrent_commit_verify(dims, B, T, prev[0]["x"], prev[0]["gate"], prev[0]["beta"], prev[1], T,
                                           wd["x"], wd["gate"], wd["beta"], conv_w, None, cs_b, st_b, out_b)
        torch.cuda.synchronize()
        assert torch.equal(out_a, out_b), f"round {rnd}: fused outputs differ"
        h = {k: w[k].double().numpy() for k in ("x", "gate", "beta")}
        o_out, o_snaps = OR.verify(h["x"], h["gate"], h["beta"], base["conv_w"].double().numpy(), cs_o, st_o)
        cs_o, st_o = OR.commit(h["x"], nacc.cpu().numpy(), cs_o, st_o, o_snaps)
        _close(out_b.cpu().numpy(), o_out, f"round {rnd} outputs", 1)
        prev = (wd, nacc)
    # the fused pool is one window behind: commit the last window
    S.spec_recurrent_commit(dims, B, T, prev[0]["x"], prev[0]["gate"], prev[0]["beta"], conv_w, None, prev[1], None,
                            cs_b, st_b)
    torch.cuda.synchronize()
    assert torch.equal(st_a, st_b) and torch.equal(cs_a, cs_b)
    _close(st_b.cpu().numpy(), st_o, "final state", 2)
