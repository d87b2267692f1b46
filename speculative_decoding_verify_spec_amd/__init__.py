"""Python binding of the MI355X speculative verify step (C ABI in
include/spec_verify.h and include/spec_recurrent.h).

Argument marshalling only: every function below forwards to the symbol of the
same name in libspec_verify.so.  Device buffers may be passed as torch tensors
(their data_ptr() is used) or as raw integer addresses; streams as
torch.cuda.Stream or raw handles.  Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspec_verify.so")

SPEC_OK = 0
SPEC_ERR_INVALID_ARG = -1
SPEC_ERR_SHAPE = -2
SPEC_ERR_CAPACITY = -3
SPEC_ERR_UNSUPPORTED = -4
SPEC_ERR_DEVICE = -5
SPEC_ERR_STATE = -6
SPEC_ERR_DATA = -7

SPEC_DTYPE_F32 = 0
SPEC_DTYPE_BF16 = 1

SPEC_FLAG_TOKEN_RANGE = 1
SPEC_FLAG_TREE = 2
SPEC_FLAG_KV_OVERFLOW = 4
SPEC_FLAG_LAYOUT = 8

EXPORTED = [
    "spec_workspace_bytes", "spec_kv_cache_bytes", "spec_verify_init", "spec_verify_step",
    "spec_verify_step_ragged", "spec_accept", "spec_accept_ragged", "spec_device_errors", "spec_profile_enable", "spec_profile_read",
    "spec_profile_gemm", "spec_profile_stream_read", "spec_graph_enable", "spec_gemm_route", "spec_accept_chain_static", "spec_set_block_table", "spec_verify_destroy",
    "spec_status_str",
    "spec_recurrent_verify", "spec_recurrent_commit", "spec_recurrent_commit_verify",
]


class spec_config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ffn", C.c_int32),
                ("vocab", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_float),
                ("weight_dtype", C.c_int32), ("max_batch", C.c_int32), ("max_ctx", C.c_int32),
                ("max_rows_per_seq", C.c_int32), ("kv_page_size", C.c_int32), ("kv_pages", C.c_int32)]


class spec_sampling(C.Structure):
    _fields_ = [("temperature", C.c_float), ("tree_replacement", C.c_uint32),
                ("seed", C.c_uint64), ("round", C.c_uint64), ("top_k", C.c_int32), ("top_p", C.c_float)]


class spec_kernel_stat(C.Structure):
    _fields_ = [("name", C.c_char * 24), ("launches", C.c_int64), ("total_ms", C.c_double),
                ("algo_bytes", C.c_double)]


class spec_recurrent_dims(C.Structure):
    _fields_ = [("n_heads", C.c_int32), ("head_dim", C.c_int32), ("conv_width", C.c_int32),
                ("n_slots", C.c_int32)]


class SpecError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {status} ({spec_status_str(status)})")
        self.status = status


_lib = None


def lib():
    """Load libspec_verify.so (once).  Raises if it is missing: there is no
    fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} not built; run __graft_entry__.build() or "
                          "python -m speculative_decoding_verify_spec_amd.build")
    L = C.CDLL(LIB_PATH)
    vp, sz, i32 = C.c_void_p, C.c_size_t, C.c_int32
    L.spec_workspace_bytes.argtypes = [C.POINTER(spec_config)]
    L.spec_workspace_bytes.restype = sz
    L.spec_kv_cache_bytes.argtypes = [C.POINTER(spec_config)]
    L.spec_kv_cache_bytes.restype = sz
    L.spec_verify_init.argtypes = [C.POINTER(spec_config), C.POINTER(vp), sz, vp, vp, sz, vp,
                                   C.POINTER(vp)]
    L.spec_verify_init.restype = i32
    L.spec_verify_step.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp]
    L.spec_verify_step.restype = i32
    L.spec_verify_step_ragged.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp]
    L.spec_verify_step_ragged.restype = i32
    L.spec_accept.argtypes = [vp, i32, i32, vp, vp, vp, vp, C.POINTER(spec_sampling), vp, vp, vp, vp, vp]
    L.spec_accept.restype = i32
    L.spec_accept_ragged.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, C.POINTER(spec_sampling),
                                     vp, vp, vp, vp, vp]
    L.spec_accept_ragged.restype = i32
    L.spec_device_errors.argtypes = [vp, C.POINTER(C.c_uint32), vp]
    L.spec_device_errors.restype = i32
    L.spec_profile_enable.argtypes = [vp, i32]
    L.spec_profile_enable.restype = i32
    L.spec_profile_read.argtypes = [vp, C.POINTER(spec_kernel_stat), i32, i32]
    L.spec_profile_read.restype = i32
    L.spec_profile_gemm.argtypes = [vp, C.c_char_p, i32, i32, vp, C.POINTER(C.c_double),
                                    C.POINTER(C.c_double)]
    L.spec_profile_gemm.restype = i32
    L.spec_profile_stream_read.argtypes = [vp, C.c_size_t, C.c_size_t, i32, i32, i32, vp, C.POINTER(C.c_double)]
    L.spec_profile_stream_read.restype = i32
    L.spec_graph_enable.argtypes = [vp, i32]
    L.spec_graph_enable.restype = i32
    L.spec_gemm_route.argtypes = [i32]
    L.spec_gemm_route.restype = i32
    L.spec_accept_chain_static.argtypes = [i32, i32, i32, vp, vp, vp, C.POINTER(spec_sampling), vp, vp, vp, vp,
                                           vp, vp]
    L.spec_accept_chain_static.restype = i32
    L.spec_set_block_table.argtypes = [vp, vp, i32]
    L.spec_set_block_table.restype = i32
    L.spec_verify_destroy.argtypes = [vp]
    L.spec_verify_destroy.restype = None
    L.spec_status_str.argtypes = [i32]
    L.spec_status_str.restype = C.c_char_p
    L.spec_recurrent_verify.argtypes = [C.POINTER(spec_recurrent_dims), i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp]
    L.spec_recurrent_verify.restype = i32
    L.spec_recurrent_commit.argtypes = [C.POINTER(spec_recurrent_dims), i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp]
    L.spec_recurrent_commit.restype = i32
    L.spec_recurrent_commit_verify.argtypes = [C.POINTER(spec_recurrent_dims), i32, i32, vp, vp, vp, vp, i32, vp,
                                               vp, vp, vp, vp, vp, vp, vp, vp]
    L.spec_recurrent_commit_verify.restype = i32
    _lib = L
    return L


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn, st):
    if st != SPEC_OK:
        raise SpecError(fn, st)


KV_PAGE = 64  # slots per page of a paged cache
# capacity of spec_accept_chain_static's fixed scratch
SPEC_STATIC_MAX_ROWS = 4096
SPEC_STATIC_MAX_SEQS = 1024
SPEC_STATIC_MAX_VOCAB = 262144


def make_config(shape, max_batch, max_ctx, max_rows_per_seq, kv_pages: int = 0) -> spec_config:
    """spec_config from any object with the model-shape attributes; kv_pages > 0
    selects a paged cache of that many 64-slot pages."""
    return spec_config(shape.n_layers, shape.d_model, shape.n_heads, shape.n_kv_heads, shape.head_dim,
                       shape.d_ffn, shape.vocab, float(shape.rms_eps), float(shape.rope_theta),
                       SPEC_DTYPE_BF16 if shape.weight_dtype == "bf16" else SPEC_DTYPE_F32,
                       int(max_batch), int(max_ctx), int(max_rows_per_seq),
                       KV_PAGE if kv_pages else 0, int(kv_pages))


def spec_status_str(status: int) -> str:
    return lib().spec_status_str(int(status)).decode()


def spec_workspace_bytes(cfg: spec_config) -> int:
    return int(lib().spec_workspace_bytes(C.byref(cfg)))


def spec_kv_cache_bytes(cfg: spec_config) -> int:
    return int(lib().spec_kv_cache_bytes(C.byref(cfg)))


def spec_verify_init(cfg: spec_config, weights, kv_cache, workspace, workspace_bytes: int, stream=None,
                     check: bool = True):
    """Returns the handle (int), or (status, None) when check=False and it fails."""
    arr = (C.c_void_p * len(weights))(*[_ptr(w) for w in weights])
    h = C.c_void_p()
    st = lib().spec_verify_init(C.byref(cfg), arr, len(weights), _ptr(kv_cache), _ptr(workspace),
                                int(workspace_bytes), _stream(stream), C.byref(h))
    if check:
        _check("spec_verify_init", st)
        return h.value
    return st, h.value


def spec_verify_step(h, B, T, tokens, kv_len, tree_parent, logits, stream=None, check=True):
    st = lib().spec_verify_step(h, int(B), int(T), _ptr(tokens), _ptr(kv_len), _ptr(tree_parent),
                                _ptr(logits), _stream(stream))
    if check:
        _check("spec_verify_step", st)
    return st


def spec_verify_step_ragged(h, B, max_len, rows, cu_rows, tokens, kv_len, logits, stream=None, check=True):
    st = lib().spec_verify_step_ragged(h, int(B), int(max_len), int(rows), _ptr(cu_rows), _ptr(tokens),
                                       _ptr(kv_len), _ptr(logits), _stream(stream))
    if check:
        _check("spec_verify_step_ragged", st)
    return st


def spec_accept_ragged(h, B, max_len, rows, q_rows, row_start, lens, q_start, logits, q, tokens,
                       sampling: spec_sampling, out_tokens, num_accepted, kv_len, kv_len_out, stream=None,
                       check=True):
    st = lib().spec_accept_ragged(h, int(B), int(max_len), int(rows), int(q_rows), _ptr(row_start), _ptr(lens),
                                  _ptr(q_start), _ptr(logits), _ptr(q), _ptr(tokens), C.byref(sampling),
                                  _ptr(out_tokens), _ptr(num_accepted), _ptr(kv_len), _ptr(kv_len_out),
                                  _stream(stream))
    if check:
        _check("spec_accept_ragged", st)
    return st


def spec_accept(h, B, T, logits, q, tokens, tree_parent, sampling: spec_sampling, out_tokens,
                num_accepted, kv_len, kv_len_out, stream=None, check=True):
    st = lib().spec_accept(h, int(B), int(T), _ptr(logits), _ptr(q), _ptr(tokens), _ptr(tree_parent),
                           C.byref(sampling), _ptr(out_tokens), _ptr(num_accepted), _ptr(kv_len),
                           _ptr(kv_len_out), _stream(stream))
    if check:
        _check("spec_accept", st)
    return st


def spec_device_errors(h, stream=None) -> int:
    v = C.c_uint32(0)
    _check("spec_device_errors", lib().spec_device_errors(h, C.byref(v), _stream(stream)))
    return int(v.value)


def spec_profile_enable(h, enable: bool):
    _check("spec_profile_enable", lib().spec_profile_enable(h, 1 if enable else 0))


def spec_profile_read(h, reset: bool = True):
    arr = (spec_kernel_stat * 32)()
    n = lib().spec_profile_read(h, arr, 32, 1 if reset else 0)
    if n < 0:
        raise SpecError("spec_profile_read", SPEC_ERR_DEVICE)
    return {arr[i].name.decode(): {"launches": int(arr[i].launches), "total_ms": float(arr[i].total_ms),
                                   "algo_bytes": float(arr[i].algo_bytes)} for i in range(n)}


def spec_profile_gemm(h, cls: str, rows: int, iters: int, stream=None):
    """(milliseconds, algorithmic bytes) of `iters` back-to-back passes of one
    GEMM class over all layers."""
    ms, nbytes = C.c_double(0.0), C.c_double(0.0)
    _check("spec_profile_gemm", lib().spec_profile_gemm(h, cls.encode(), int(rows), int(iters),
                                                        _stream(stream), C.byref(ms), C.byref(nbytes)))
    return ms.value, nbytes.value


def spec_profile_stream_read(buf, read_bytes: int, iters: int, grid: int, unroll: int, stream=None):
    """Average launch-to-end microseconds of a plain streaming read of
    `read_bytes` from the device buffer `buf` (a tensor), windows rotating
    through it."""
    us = C.c_double(0.0)
    nbytes = buf.numel() * buf.element_size()
    _check("spec_profile_stream_read", lib().spec_profile_stream_read(
        _ptr(buf), nbytes, int(read_bytes), int(iters), int(grid), int(unroll), _stream(stream), C.byref(us)))
    return us.value


def spec_set_block_table(h, table, pages_per_seq: int):
    _check("spec_set_block_table", lib().spec_set_block_table(h, _ptr(table), int(pages_per_seq)))


def spec_graph_enable(h, enable: bool):
    _check("spec_graph_enable", lib().spec_graph_enable(h, 1 if enable else 0))


def spec_gemm_route(route: int):
    _check("spec_gemm_route", lib().spec_gemm_route(int(route)))


def spec_accept_chain_static(B, T, vocab, logits, q, tokens, sampling: spec_sampling, out_tokens, num_accepted,
                             kv_len=None, kv_len_out=None, flags=None, stream=None, check=True):
    st = lib().spec_accept_chain_static(int(B), int(T), int(vocab), _ptr(logits), _ptr(q), _ptr(tokens),
                                        C.byref(sampling), _ptr(out_tokens), _ptr(num_accepted), _ptr(kv_len),
                                        _ptr(kv_len_out), _ptr(flags), _stream(stream))
    if check:
        _check("spec_accept_chain_static", st)
    return st


def spec_verify_destroy(h):
    if h:
        lib().spec_verify_destroy(h)


def spec_recurrent_verify(dims: spec_recurrent_dims, B, T, x, gate, beta, conv_w, slot, conv_state, state, out,
                          snapshots=None, stream=None, check=True):
    st = lib().spec_recurrent_verify(C.byref(dims), int(B), int(T), _ptr(x), _ptr(gate), _ptr(beta),
                                     _ptr(conv_w), _ptr(slot), _ptr(conv_state), _ptr(state), _ptr(out),
                                     _ptr(snapshots), _stream(stream))
    if check:
        _check("spec_recurrent_verify", st)
    return st


def spec_recurrent_commit(dims: spec_recurrent_dims, B, T, x, gate, beta, conv_w, slot, num_accepted, snapshots,
                          conv_state, state, stream=None, check=True):
    st = lib().spec_recurrent_commit(C.byref(dims), int(B), int(T), _ptr(x), _ptr(gate), _ptr(beta),
                                     _ptr(conv_w), _ptr(slot), _ptr(num_accepted), _ptr(snapshots),
                                     _ptr(conv_state), _ptr(state), _stream(stream))
    if check:
        _check("spec_recurrent_commit", st)
    return st


def spec_recurrent_commit_verify(dims: spec_recurrent_dims, B, T_prev, prev_x, prev_gate, prev_beta, prev_accepted,
                                 T, x, gate, beta, conv_w, slot, conv_state, state, out, stream=None, check=True):
    st = lib().spec_recurrent_commit_verify(C.byref(dims), int(B), int(T_prev), _ptr(prev_x), _ptr(prev_gate),
                                            _ptr(prev_beta), _ptr(prev_accepted), int(T), _ptr(x), _ptr(gate),
                                            _ptr(beta), _ptr(conv_w), _ptr(slot), _ptr(conv_state), _ptr(state),
                                            _ptr(out), _stream(stream))
    if check:
        _check("spec_recurrent_commit_verify", st)
    return st
