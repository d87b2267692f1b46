"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, sizes buffers as documented and rejects bad arguments before
touching the device (all without a GPU)."""
import ctypes as C
import glob
import os
import re

import pytest

import speculative_decoding_verify_spec_amd as S
import synth

HEADERS = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                                        "*.h")))


def _declared():
    txt = "".join(open(h).read() for h in HEADERS)
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", txt)))


def test_header_declares_the_binding_names():
    assert set(_declared()) == set(S.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = S.lib()
    for name in _declared():
        assert hasattr(L, name), name
        assert C.cast(getattr(L, name), C.c_void_p).value


def test_status_strings():
    for st in range(0, -8, -1):
        assert S.spec_status_str(st)
    assert S.spec_status_str(0) == "ok"
    assert "unknown" in S.spec_status_str(-99)


def _cfg(**kw):
    base = dict(max_batch=2, max_ctx=128, max_rows_per_seq=8)
    base.update(kw)
    return S.make_config(synth.TOY, **base)


def test_kv_cache_bytes_formula():
    cfg = _cfg()
    sh = synth.TOY
    assert S.spec_kv_cache_bytes(cfg) == sh.n_layers * 2 * 2 * sh.n_kv_heads * 128 * sh.head_dim * 2
    assert S.spec_kv_cache_bytes(cfg) == synth.kv_cache_numel(sh, 2, 128) * 2


@pytest.mark.parametrize("field,value", [
    ("head_dim", 96), ("n_kv_heads", 3), ("max_ctx", 100), ("max_rows_per_seq", 129),
    ("weight_dtype", 7), ("d_model", 200), ("rms_eps", 0.0), ("max_batch", 0)])
def test_invalid_config_rejected(field, value):
    cfg = _cfg()
    setattr(cfg, field, value)
    assert S.spec_workspace_bytes(cfg) == 0
    assert S.spec_kv_cache_bytes(cfg) == 0
    st, h = S.spec_verify_init(cfg, [16] * synth.TOY.n_weights(), 16, 256, 1 << 30, None, check=False)
    assert st == S.SPEC_ERR_SHAPE and h is None


def test_workspace_grows_with_capacity():
    a = S.spec_workspace_bytes(_cfg())
    b = S.spec_workspace_bytes(_cfg(max_batch=8))
    c = S.spec_workspace_bytes(_cfg(max_ctx=1024))
    assert 0 < a < b and a < c
    assert a % 256 == 0


def test_init_argument_errors_without_device():
    cfg = _cfg()
    n = synth.TOY.n_weights()
    ws = S.spec_workspace_bytes(cfg)
    # null weights / cache / workspace
    assert S.spec_verify_init(cfg, [0] * n, 16, 256, ws, None, check=False)[0] == S.SPEC_ERR_INVALID_ARG
    assert S.spec_verify_init(cfg, [16] * n, 0, 256, ws, None, check=False)[0] == S.SPEC_ERR_INVALID_ARG
    # wrong weight count, misaligned weight, misaligned workspace
    assert S.spec_verify_init(cfg, [16] * (n - 1), 16, 256, ws, None, check=False)[0] == S.SPEC_ERR_INVALID_ARG
    assert S.spec_verify_init(cfg, [16] * (n - 1) + [18], 16, 256, ws, None, check=False)[0] == \
        S.SPEC_ERR_INVALID_ARG
    assert S.spec_verify_init(cfg, [16] * n, 16, 264, ws, None, check=False)[0] == S.SPEC_ERR_INVALID_ARG
    # workspace too small
    assert S.spec_verify_init(cfg, [16] * n, 16, 256, ws - 1, None, check=False)[0] == S.SPEC_ERR_CAPACITY


def test_calls_on_null_handle_are_rejected():
    smp = S.spec_sampling(1.0, 0, 1, 0, 0, 1.0)
    assert S.spec_verify_step(None, 1, 1, 16, 16, None, 16, None, check=False) == S.SPEC_ERR_INVALID_ARG
    assert S.spec_accept(None, 1, 2, 16, 16, 16, None, smp, 16, 16, 16, 16, None,
                         check=False) == S.SPEC_ERR_INVALID_ARG
    assert S.lib().spec_profile_enable(None, 1) == S.SPEC_ERR_INVALID_ARG
    assert S.lib().spec_profile_read(None, None, 0, 0) == -1
    S.spec_verify_destroy(None)


def test_recurrent_calls_reject_bad_arguments_without_device():
    dims = S.spec_recurrent_dims(4, 128, 4, 8)
    P = 256  # a fake, aligned address: nothing is launched on these paths
    ok = dict(x=P, gate=P, beta=P, conv_w=P, slot=None, conv_state=P, state=P, out=P)

    def ver(d=dims, B=2, T=4, **kw):
        a = dict(ok)
        a.update(kw)
        return S.spec_recurrent_verify(d, B, T, a["x"], a["gate"], a["beta"], a["conv_w"], a["slot"],
                                       a["conv_state"], a["state"], a["out"], None, None, check=False)

    def com(d=dims, B=2, T=4, snaps=None, **kw):
        a = dict(ok, nacc=P)
        a.update(kw)
        return S.spec_recurrent_commit(d, B, T, a["x"], a["gate"], a["beta"], a["conv_w"], a["slot"], a["nacc"],
                                       snaps, a["conv_state"], a["state"], None, check=False)

    assert ver(B=0) == S.SPEC_OK and com(B=0) == S.SPEC_OK  # empty batch: nothing to do
    for bad in (S.spec_recurrent_dims(0, 128, 4, 8), S.spec_recurrent_dims(4, 96, 4, 8),
                S.spec_recurrent_dims(4, 128, 0, 8), S.spec_recurrent_dims(4, 128, 9, 8),
                S.spec_recurrent_dims(4, 128, 4, 0)):
        assert ver(d=bad) == S.SPEC_ERR_SHAPE and com(d=bad) == S.SPEC_ERR_SHAPE
    assert ver(T=0) == S.SPEC_ERR_INVALID_ARG and ver(T=17) == S.SPEC_ERR_INVALID_ARG
    assert ver(B=-1) == S.SPEC_ERR_INVALID_ARG
    assert ver(B=9) == S.SPEC_ERR_INVALID_ARG  # more sequences than pool rows, no slot map
    assert ver(x=None) == S.SPEC_ERR_INVALID_ARG and ver(out=None) == S.SPEC_ERR_INVALID_ARG
    assert ver(conv_state=None) == S.SPEC_ERR_INVALID_ARG
    assert ver(state=P + 4) == S.SPEC_ERR_INVALID_ARG  # misaligned
    assert com(nacc=None) == S.SPEC_ERR_INVALID_ARG
    assert com(gate=None) == S.SPEC_ERR_INVALID_ARG  # replay needs the window inputs
    assert com(B=0, gate=None, snaps=P) == S.SPEC_OK  # the scatter does not
    assert com(x=None, snaps=P) == S.SPEC_ERR_INVALID_ARG  # conv state needs x when W > 1
    assert S.lib().spec_recurrent_verify(None, 1, 1, P, P, P, P, None, P, P, P, None, None) == \
        S.SPEC_ERR_INVALID_ARG

    def cv(d=dims, B=2, Tp=4, T=4, prev=P, **kw):
        a = dict(ok)
        a.update(kw)
        return S.spec_recurrent_commit_verify(d, B, Tp, prev, prev, prev, prev, T, a["x"], a["gate"], a["beta"],
                                              a["conv_w"], a["slot"], a["conv_state"], a["state"], a["out"],
                                              None, check=False)

    assert cv(B=0) == S.SPEC_OK and cv(B=0, Tp=0, prev=None) == S.SPEC_OK
    assert cv(Tp=-1) == S.SPEC_ERR_INVALID_ARG and cv(Tp=17) == S.SPEC_ERR_INVALID_ARG
    assert cv(prev=None) == S.SPEC_ERR_INVALID_ARG  # a previous window needs its inputs
    assert cv(T=0) == S.SPEC_ERR_INVALID_ARG and cv(out=None) == S.SPEC_ERR_INVALID_ARG
    assert cv(d=S.spec_recurrent_dims(4, 96, 4, 8)) == S.SPEC_ERR_SHAPE
    assert cv(prev=P + 8) == S.SPEC_ERR_INVALID_ARG  # misaligned


def test_gemm_route_argument_checked():
    L = S.lib()
    assert L.spec_gemm_route(4) == -1 and L.spec_gemm_route(-1) == -1
    assert L.spec_gemm_route(0) == 0


def test_static_accept_rejects_before_any_launch():
    """The allocation-free chain accept checks its arguments and its scratch
    capacity on the host: nothing is enqueued (no GPU needed here)."""
    L = S.lib()
    samp = S.spec_sampling(temperature=1.0, tree_replacement=0, seed=1, round=0, top_k=0, top_p=1.0)
    fake = C.c_void_p(256)  # never dereferenced: every call below fails its checks first
    args = lambda B, T, V: (B, T, V, fake, fake, fake, C.byref(samp), fake, fake, None, None, None, None)  # noqa: E731
    assert L.spec_accept_chain_static(*args(0, 4, 1000)) == -1
    assert L.spec_accept_chain_static(2, 4, 1000, None, fake, fake, C.byref(samp), fake, fake, None, None, None,
                                      None) == -1
    assert L.spec_accept_chain_static(*args(S.SPEC_STATIC_MAX_SEQS + 1, 1, 1000)) == -3
    assert L.spec_accept_chain_static(*args(64, 65, 1000)) == -3            # 4160 rows > 4096
    assert L.spec_accept_chain_static(*args(2, 129, 1000)) == -3            # T > 128
    assert L.spec_accept_chain_static(*args(2, 4, S.SPEC_STATIC_MAX_VOCAB + 1)) == -3
    samp.top_p = 0.9
    assert L.spec_accept_chain_static(*args(2, 4, 1000)) == -4              # top-p needs the handle's scratch


def test_stream_read_hook_rejects_before_any_launch():
    """The streaming-read measurement hook checks sizes and alignment on the
    host; an address that is never dereferenced stands in for device memory."""
    L = S.lib()
    us = C.c_double(0.0)
    fake = 1 << 40  # 4096-aligned, never touched: every call below is rejected first
    bad = [
        (None, 1 << 20, 4096, 1, 1, 4),          # null buffer
        (fake, 1 << 20, 4096, 1, 1, 5),          # unroll not 4 or 8
        (fake + 16, 1 << 20, 4096, 1, 1, 4),     # buffer not 4096-aligned
        (fake, 1 << 20, 4100, 1, 1, 4),          # read size not a multiple of 16
        (fake, (1 << 20) + 8, 4096, 1, 1, 4),    # buffer size not a multiple of 16
        (fake, 8192, 4096, 1, 1, 4),             # buffer below read + 8192
        (fake, 1 << 20, 4096, 0, 1, 4),          # iters < 1
        (fake, 1 << 20, 4096, 1, 0, 4),          # grid < 1
    ]
    for args in bad:
        assert L.spec_profile_stream_read(*args, None, C.byref(us)) == S.SPEC_ERR_INVALID_ARG, args
    assert L.spec_profile_stream_read(fake, 1 << 20, 4096, 1, 1, 4, None, None) == S.SPEC_ERR_INVALID_ARG
