"""Ragged verify (the DeepSeek-V4 analysis page, section 4): compact forward of
packed per-sequence chains with padding rows up to an execution tier, and the
accept of ragged chains in compact and cap-accept layouts, against the
oracle's per-sequence forward and accept."""
import numpy as np
import pytest
import torch

import synth
from oracle import accept as OA
from oracle import model as OM
from oracle import philox
from tests.gpu_util import (bf16_close, build_engine, DRAW_BAND_SHARED, compare_decisions, dev, logits_rel_err, oracle_cache,
                            oracle_weights)

pytestmark = pytest.mark.gpu


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


RAGGED_CASES = [
    # shape, lens, padding rows, context lengths
    ("MINI8B", [4, 1, 3], 2, [300, 17, 700]),
    ("MINI8B", [8, 2], 0, [1000, 64]),
    ("MINI8B", [1, 1, 1, 1], 4, [5, 100, 200, 0]),
    ("MINI8B", [3, 5, 2, 6], 3, [129, 40, 600, 8]),
    ("FFN8B", [4, 2], 2, [500, 31]),
]


@pytest.mark.parametrize("shape,lens,pad,ctx", RAGGED_CASES)
def test_ragged_forward_matches_oracle(shape, lens, pad, ctx):
    sh = getattr(synth, shape)
    B = len(lens)
    cu = _cu(lens)
    rows = int(cu[-1]) + pad
    print(f"[ragged fwd] {shape} lens={lens} rows={rows} ctx={ctx}", flush=True)
    max_ctx = 1088 if shape == "MINI8B" else 576
    eng, names, w, cache = build_engine(sh, 4, max_ctx, 8, ctx_len=ctx + [0] * (4 - B))
    W = oracle_weights(names, w)
    kc, vc = oracle_cache(cache, sh, 4, max_ctx)
    toks = synth.make_tokens(1, rows, sh.vocab, seed=91 + rows, device=dev())[0]
    cu_d = torch.from_numpy(cu).to(dev())
    kv = torch.tensor(ctx, dtype=torch.int32, device=dev())
    z = torch.full((rows, sh.vocab), float("nan"), device=dev())
    eng.step_ragged(cu_d, max(lens), toks, kv, z)
    torch.cuda.synchronize()
    zo, kn, vn = OM.forward_ragged(sh, W, toks.cpu().numpy()[:cu[-1]], cu, np.array(ctx), kc[:, :B], vc[:, :B])
    zg = z[:cu[-1]].cpu().numpy()
    assert np.isfinite(zg).all()
    err = logits_rel_err(zg, zo)
    print(f"  logits rel err max {err.max():.2e}", flush=True)
    assert err.max() < 1e-3
    # each sequence wrote exactly its own rows' K/V at kv_len + i
    kg, vg = oracle_cache(cache, sh, 4, max_ctx)
    for b in range(B):
        ko, vo = kc[:, b:b + 1].copy(), vc[:, b:b + 1].copy()
        OM.write_suffix(ko, vo, kn[b][:, None], vn[b][:, None], np.array([ctx[b]]))
        s0, s1 = ctx[b], ctx[b] + lens[b]
        bf16_close(kg[:, b, :, s0:s1], ko[:, 0, :, s0:s1])
        bf16_close(vg[:, b, :, :, s0:s1], vo[:, 0, :, :, s0:s1])
        assert np.array_equal(kg[:, b, :, :s0], kc[:, b, :, :s0])
        # the poisoned tail past the sequence's rows is untouched (padding rows write nothing)
        assert np.array_equal(kg[:, b, :, s1:], kc[:, b, :, s1:])
        assert np.array_equal(vg[:, b, :, :, s1:], vc[:, b, :, :, s1:])
    for b in range(B, 4):
        assert np.array_equal(kg[:, b], kc[:, b]) and np.array_equal(vg[:, b], vc[:, b])
    assert eng.device_errors() == 0


def test_ragged_replay_matches_direct_launches():
    sh = synth.MINI8B
    lens, pad, ctx = [3, 1, 4], 4, [200, 50, 9]
    cu = torch.from_numpy(_cu(lens)).to(dev())
    rows = sum(lens) + pad
    eng, names, w, cache = build_engine(sh, 4, 512, 8, ctx_len=ctx + [0])
    toks = synth.make_tokens(1, rows, sh.vocab, seed=5, device=dev())[0]
    kv = torch.tensor(ctx, dtype=torch.int32, device=dev())

    def run():
        z = torch.full((rows, sh.vocab), float("nan"), device=dev())
        eng.step_ragged(cu, max(lens), toks, kv, z)
        torch.cuda.synchronize()
        return z[:sum(lens)].clone()

    eng.graphs(False)
    ref = run()
    eng.graphs(True)
    for rep in range(3):
        print(f"[ragged replay] {rep}", flush=True)
        assert torch.equal(run(), ref)
        # a static shape in between: the recordings are kept apart
        zs = torch.empty((2, 4, sh.vocab), device=dev())
        eng.step(toks[:8].view(2, 4).contiguous(), kv[:2].contiguous(), zs)
        torch.cuda.synchronize()
    assert eng.device_errors() == 0


def _accept_engine(V):
    sh = synth.ModelShape(n_layers=1, d_model=64, n_heads=1, n_kv_heads=1, head_dim=64, d_ffn=64,
                          vocab=V, rms_eps=1e-5, rope_theta=10000.0, weight_dtype="f32")
    from speculative_decoding_verify_spec_amd.engine import VerifyEngine
    _, w = synth.make_weights(sh, device=dev())
    cache = synth.make_kv_cache(sh, 8, 128, 64, device=dev(), poison_tail=False)
    return VerifyEngine(sh, w, cache, 8, 128, 8)


ACC_CASES = [
    # V, lens, max_len, temperature, top_k, top_p
    (4099, [4, 1, 3, 2], 4, 1.0, 0, 1.0),
    (4099, [5, 5, 1], 5, 0.0, 0, 1.0),
    (128256, [4, 2, 1], 4, 1.0, 0, 1.0),
    (128256, [6, 3], 6, 0.8, 40, 0.9),
]


@pytest.mark.parametrize("V,lens,max_len,temp,top_k,top_p", ACC_CASES)
@pytest.mark.parametrize("layout", ["compact", "cap"])
def test_ragged_accept_matches_oracle(V, lens, max_len, temp, top_k, top_p, layout):
    print(f"[ragged accept] {layout} V={V} lens={lens} T={temp} top_k={top_k} top_p={top_p}", flush=True)
    eng = _accept_engine(V)
    B = len(lens)
    near = 0
    for r in range(4):
        seed = 7 * V % 997 + 31 * r + len(lens)
        # a fixed-width window of max_len rows per sequence
        z = synth.random_logits((B, max_len), V, seed=seed, device=dev(), scale=2.0)
        toks = synth.make_tokens(B, max_len, V, seed=seed + 1, device=dev())
        q, zn = synth.noisy_draft_dist(z[:, :max_len - 1], 1.0, seed + 2, temp if temp > 0 else 1.0)
        if max_len > 1:
            toks[:, 1:] = synth.sample_from(q, seed + 3)[..., 0] if temp > 0 else zn.argmax(-1).to(torch.int32)
        if layout == "cap":
            zr, qr, tr = z.reshape(B * max_len, V), q.reshape(B * (max_len - 1), V), toks.reshape(-1)
            rstart = np.arange(B) * max_len
            qstart = np.arange(B) * (max_len - 1)
        else:
            cu = _cu(lens)
            pad = 3  # padding rows of the execution tier, never read
            zr = torch.cat([z[b, :lens[b]] for b in range(B)] + [z[0, :1].expand(pad, V)])
            qr = torch.cat([q[b, :lens[b] - 1] for b in range(B)] + [q[0, :1]])
            tr = torch.cat([toks[b, :lens[b]] for b in range(B)] + [toks[0, :1].expand(pad)]).contiguous()
            rstart = cu[:-1]
            qstart = cu[:-1] - np.arange(B)
        zr, qr = zr.contiguous(), qr.contiguous()
        rs_d = torch.tensor(rstart, dtype=torch.int32, device=dev())
        ln_d = torch.tensor(lens, dtype=torch.int32, device=dev())
        qs_d = torch.tensor(qstart, dtype=torch.int32, device=dev())
        kv = torch.arange(10, 10 + B, dtype=torch.int32, device=dev())
        kv_out = torch.full((B,), -3, dtype=torch.int32, device=dev())
        out = torch.full((B, max_len), -5, dtype=torch.int32, device=dev())
        nacc = torch.full((B,), -5, dtype=torch.int32, device=dev())
        eng.accept_ragged(rs_d, ln_d, qs_d, max_len, zr, qr, tr, out, nacc, kv, kv_out, temperature=temp,
                          seed=3 + r, round_=r, top_k=top_k, top_p=top_p)
        torch.cuda.synchronize()
        orc = OA.accept_ragged(zr.double().cpu().numpy(), qr.double().cpu().numpy(), tr.cpu().numpy(), rstart, lens,
                               qstart, temp, philox.Uniforms(3 + r, r), max_len=max_len, top_k=top_k, top_p=top_p)
        near += compare_decisions(out.cpu().numpy(), nacc.cpu().numpy(), orc, f"round {r}", draw_band=DRAW_BAND_SHARED)
        n = nacc.cpu().numpy()
        assert np.all(n <= np.array(lens) - 1)
        assert np.array_equal(kv_out.cpu().numpy(), kv.cpu().numpy() + n + 1)
        assert eng.device_errors() == 0
    assert near <= 1


def test_ragged_bad_layout_is_flagged():
    """Offsets that go backwards are clamped and flagged; the kernels stay in
    bounds and the call completes."""
    sh = synth.MINI8B
    eng, names, w, cache = build_engine(sh, 4, 256, 8, ctx_len=[10, 10, 10, 10], poison=False)
    cu = torch.tensor([0, 5, 3, 6], dtype=torch.int32, device=dev())
    toks = synth.make_tokens(1, 8, sh.vocab, seed=2, device=dev())[0]
    kv = torch.tensor([10, 10, 10], dtype=torch.int32, device=dev())
    z = torch.zeros((8, sh.vocab), device=dev())
    eng.step_ragged(cu, 4, toks, kv, z)
    torch.cuda.synchronize()
    from speculative_decoding_verify_spec_amd import SPEC_FLAG_LAYOUT
    assert eng.device_errors() & SPEC_FLAG_LAYOUT
