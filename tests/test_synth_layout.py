"""The host views of the KV cache (synth.kv_views, kv_v_blocks) against the
layout the library addresses: K [L][2][B][Hkv][max_ctx][D] rows; V transposed
within 64-position blocks, element (b, h, dim, s) of a layer's V region at
(((b Hkv + h) (max_ctx / 64) + s / 64) D + dim) 64 + s % 64."""
import random

import torch

import synth


def test_kv_views_match_the_device_offsets():
    sh = synth.TOY
    L, H, D = sh.n_layers, sh.n_kv_heads, sh.head_dim
    rng = random.Random(7)
    for max_ctx, lens in ((64, [54, 5, 0]), (320, [310, 64, 65])):
        B = len(lens)
        cache = synth.make_kv_cache(sh, B, max_ctx, lens, poison_tail=True)
        k, v = synth.kv_views(cache, sh, B, max_ctx)
        flat = cache.view(L, 2, -1)
        for _ in range(500):
            l, b, h, d, s = (rng.randrange(L), rng.randrange(B), rng.randrange(H), rng.randrange(D),
                             rng.randrange(max_ctx))
            kk = flat[l, 0, ((b * H + h) * max_ctx + s) * D + d]
            vv = flat[l, 1, (((b * H + h) * (max_ctx // 64) + s // 64) * D + d) * 64 + s % 64]
            for view, ref in ((k[l, b, h, s, d], kk), (v[l, b, h, d, s], vv)):
                assert (torch.isnan(view) and torch.isnan(ref)) or view == ref
        # written positions are finite, the tail is the poison value
        for b, c in enumerate(lens):
            assert torch.isfinite(v[:, b, :, :, :c]).all() and torch.isnan(v[:, b, :, :, c:]).all()
            assert torch.isfinite(k[:, b, :, :c]).all() and torch.isnan(k[:, b, :, c:]).all()


def test_v_view_is_a_copy_and_blocks_write_through():
    sh = synth.TOY
    cache = synth.make_kv_cache(sh, 1, 128, [100], poison_tail=False)
    _, v = synth.kv_views(cache, sh, 1, 128)
    v.zero_()
    _, v2 = synth.kv_views(cache, sh, 1, 128)
    assert v2[:, :, :, :, :100].abs().sum() > 0  # the copy did not alias the cache
    vb = synth.kv_v_blocks(cache, sh, 1, 128)
    vb[0, 0, 0, 1, 3, 5] = 2.0
    _, v3 = synth.kv_views(cache, sh, 1, 128)
    assert v3[0, 0, 0, 3, 64 + 5] == 2.0
