"""Parity of the tiled GEMM paths (9 or more rows) with the oracle: the
128-row x 256-weight-row tiles that serve 64 or more rows (with their K
slices when the tiles do not fill the chip; 8 waves, and the 4-wave form)
and the 32-row tiles below, each forced onto row counts of the other through
spec_gemm_route, and the weight-streaming kernels at 6 and 8 rows, on the 8B layer
layout (d = 4096, 32 / 8 heads of 128, bf16) with a short and a full-width
FFN.  Row counts span several tiles and ragged tails (136 = 128 + 8 rows,
468 = 3 tiles + 84 rows).  Bars: logits per row max|dz| / max|z| <= 1e-3
(the path keeps fp32 activations through bf16 hi/lo planes); the step's
cache slots equal the oracle's bf16 rounding apart from rounding ties."""
import numpy as np
import pytest
import torch

import speculative_decoding_verify_spec_amd as S
import synth
from oracle import model as OM
from tests.gpu_util import bf16_close, build_engine, dev, logits_rel_err, oracle_cache, oracle_weights

pytestmark = pytest.mark.gpu

CASES = [
    # shape, B, T, tree branching, route (0 automatic, 1 32-row tiles, 2 large
    # tiles, 3 large tiles in the 4-wave form)
    ("MINI8B", 16, 4, None, 0),     # M = 64: one row tile
    ("MINI8B", 32, 4, None, 0),     # M = 128
    ("MINI8B", 17, 8, None, 0),     # M = 136: a second row tile of 8 rows
    ("MINI8B", 4, 117, [4, 4, 2, 2], 0),  # M = 468: token trees
    ("MINI8B", 128, 4, None, 0),    # M = 512
    ("MINI8B", 10, 4, None, 2),     # M = 40 on the large tiles (one padded row tile)
    ("MINI8B", 3, 3, None, 2),      # M = 9 on the large tiles
    ("MINI8B", 32, 4, None, 1),     # M = 128 on the 32-row tiles
    ("FFN8B", 32, 4, None, 0),      # full-width FFN, K = 14336 for the down projection
    ("FFN8B", 20, 7, None, 0),      # M = 140
    ("MINI8B", 32, 4, None, 3),     # M = 128, 4-wave large tiles
    ("MINI8B", 17, 8, None, 3),     # M = 136, 4-wave large tiles, ragged row tile
    ("MINI8B", 1, 6, None, 0),      # M = 6: the weight-streaming kernels (no tiles up to 8 rows)
    ("MINI8B", 1, 8, None, 0),      # M = 8
]


@pytest.mark.parametrize("shape,B,T,branching,route", CASES)
def test_tiled_gemm_step_matches_oracle(shape, B, T, branching, route):
    sh = getattr(synth, shape)
    M = B * T
    print(f"[tiles] {shape} B={B} T={T} M={M} tree={branching} route={route}", flush=True)
    max_ctx = 256
    rng = np.random.default_rng(1000 + M)
    ctx = [int(c) for c in rng.integers(0, 120, size=B)]
    S.spec_gemm_route(route)
    try:
        eng, names, w, cache = build_engine(sh, B, max_ctx, T, ctx_len=ctx)
        W = oracle_weights(names, w)
        kc, vc = oracle_cache(cache, sh, B, max_ctx)
        tokens = synth.make_tokens(B, T, sh.vocab, seed=500 + M, device=dev())
        kv = torch.tensor(ctx, dtype=torch.int32, device=dev())
        parent = synth.random_tree(branching, B).to(dev()) if branching else None
        logits = torch.full((B, T, sh.vocab), float("nan"), device=dev())
        eng.step(tokens, kv, logits, parent)
        torch.cuda.synchronize()
    finally:
        S.spec_gemm_route(0)
    assert torch.isfinite(logits).all()
    zo, kn, vn = OM.forward(sh, W, tokens.cpu().numpy(), np.array(ctx), kc, vc,
                            tree_parent=None if parent is None else parent.cpu().numpy())
    err = logits_rel_err(logits.cpu().numpy(), zo)
    print(f"  logits rel err max {err.max():.2e} median {np.median(err):.2e}", flush=True)
    assert err.max() < 1e-3
    kg, vg = oracle_cache(cache, sh, B, max_ctx)
    ko, vo = kc.copy(), vc.copy()
    OM.write_suffix(ko, vo, kn, vn, np.array(ctx))
    for b in range(0, B, max(1, B // 8)):
        s0, s1 = ctx[b], ctx[b] + T
        bf16_close(kg[:, b, :, s0:s1], ko[:, b, :, s0:s1])
        bf16_close(vg[:, b, :, :, s0:s1], vo[:, b, :, :, s0:s1])
        assert np.array_equal(kg[:, b, :, :s0], kc[:, b, :, :s0])
    assert eng.device_errors() == 0
