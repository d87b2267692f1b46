"""Replay of the recorded per-layer launch sequence against direct launches.

spec_verify_step records the per-layer kernels of each (B, T, chain/tree)
shape once as a HIP graph and replays it.  Replays must give bit-identical
logits and cache bytes to direct launches of the same kernels, on every
replay, with unrelated eager work and synchronisations between replays and
with several recorded shapes alive at once."""
import pytest
import torch

import synth
from gpu_util import build_engine, dev

pytestmark = pytest.mark.gpu


def _step(eng, tokens, kv, parent=None):
    B, T = tokens.shape
    z = torch.full((B, T, eng.shape.vocab), float("nan"), device=dev())
    eng.step(tokens, kv, z, tree_parent=parent)
    torch.cuda.synchronize()
    return z


def _written(cache, sh, tokens, kv, max_ctx):
    """The cache slots a step over `tokens` writes: [kv_len, kv_len + T) per sequence."""
    k, v = synth.kv_views(cache, sh, 4, max_ctx)
    T = tokens.shape[1]
    out = []
    for b, L in enumerate(kv.tolist()):
        out.append(k[:, b, :, L:L + T].clone())
        out.append(v[:, b, :, :, L:L + T].clone())
    return out


def test_graph_replay_matches_direct_launches():
    sh = synth.MINI8B
    max_ctx = 512
    eng, names, w, cache = build_engine(sh, 4, max_ctx, 16, ctx_len=[200, 31, 0, 77])
    shapes = [
        (synth.make_tokens(2, 4, sh.vocab, seed=11, device=dev()),
         torch.tensor([200, 31], dtype=torch.int32, device=dev()), None),
        (synth.make_tokens(1, 1, sh.vocab, seed=12, device=dev()),
         torch.tensor([200], dtype=torch.int32, device=dev()), None),
        (synth.make_tokens(3, 7, sh.vocab, seed=13, device=dev()),
         torch.tensor([200, 31, 0], dtype=torch.int32, device=dev()),
         synth.random_tree([2, 2], 3).to(dev())),
        # 64 rows: the library GEMM path inside the recording
        (synth.make_tokens(4, 16, sh.vocab, seed=14, device=dev()),
         torch.tensor([200, 31, 0, 77], dtype=torch.int32, device=dev()), None),
    ]
    # direct launches first: the reference logits and cache bytes per shape
    eng.graphs(False)
    ref = []
    for tokens, kv, parent in shapes:
        print(f"[graph] direct B={tokens.shape[0]} T={tokens.shape[1]} tree={parent is not None}", flush=True)
        z = _step(eng, tokens, kv, parent)
        ref.append((z.clone(), _written(cache, sh, tokens, kv, max_ctx)))
    eng.graphs(True)
    junk = torch.randn(1 << 20, device=dev())
    for rep in range(4):
        for i, (tokens, kv, parent) in enumerate(shapes):
            print(f"[graph] replay {rep} shape {i}", flush=True)
            z = _step(eng, tokens, kv, parent)
            assert torch.equal(z, ref[i][0]), f"replay {rep} shape {i}: logits differ"
            # the same rows rewrite the same cache slots with the same bytes
            got = _written(cache, sh, tokens, kv, max_ctx)
            assert all(torch.equal(a, b) for a, b in zip(got, ref[i][1])), f"replay {rep} shape {i}: cache"
            # unrelated eager work and a host sync between replays
            junk.mul_(1.0001).add_(0.5)
            torch.cuda.synchronize()
    # switching back to direct launches still matches
    eng.graphs(False)
    for i, (tokens, kv, parent) in enumerate(shapes):
        assert torch.equal(_step(eng, tokens, kv, parent), ref[i][0])
    assert eng.device_errors() == 0
