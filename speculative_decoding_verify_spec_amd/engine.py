"""Buffer plumbing around the C ABI: allocates the workspace with torch, keeps
the weights and cache alive for the handle's lifetime and forwards calls.
No computation happens here."""
from __future__ import annotations

import torch

from . import (make_config, spec_accept, spec_accept_ragged, spec_device_errors, spec_graph_enable,
               spec_kv_cache_bytes, spec_profile_gemm, spec_sampling, spec_set_block_table, spec_verify_destroy,
               spec_verify_init, spec_verify_step, spec_verify_step_ragged, spec_workspace_bytes)


class VerifyEngine:
    def __init__(self, shape, weights, kv_cache: torch.Tensor, max_batch: int, max_ctx: int,
                 max_rows_per_seq: int, stream=None, kv_pages: int = 0):
        self.shape = shape
        self.cfg = make_config(shape, max_batch, max_ctx, max_rows_per_seq, kv_pages)
        self.weights = list(weights)
        self.kv_cache = kv_cache
        need = spec_kv_cache_bytes(self.cfg)
        have = kv_cache.numel() * kv_cache.element_size()
        if have < need:
            raise ValueError(f"kv cache has {have} bytes, needs {need}")
        self.ws_bytes = spec_workspace_bytes(self.cfg)
        dev = kv_cache.device
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
        self.handle = spec_verify_init(self.cfg, self.weights, self.kv_cache, self.workspace,
                                       self.ws_bytes, self.stream)

    def set_block_table(self, table):
        """Paged cache: table [max_batch, pages_per_seq] int32 on the device,
        read at every later step (edit it in place to grow or roll back)."""
        self.block_table = table
        spec_set_block_table(self.handle, table, table.shape[1])

    def step(self, tokens, kv_len, logits, tree_parent=None):
        B, T = tokens.shape
        return spec_verify_step(self.handle, B, T, tokens, kv_len, tree_parent, logits, self.stream)

    def step_ragged(self, cu_rows, max_len, tokens, kv_len, logits):
        """Compact verify: cu_rows [B+1] int32 row offsets; tokens [rows]; logits
        [rows, V] with rows >= cu_rows[B] (the padded execution tier)."""
        B = cu_rows.shape[0] - 1
        return spec_verify_step_ragged(self.handle, B, max_len, tokens.shape[0], cu_rows, tokens, kv_len, logits,
                                       self.stream)

    def accept_ragged(self, row_start, lens, q_start, max_len, logits, q, tokens, out_tokens, num_accepted,
                      kv_len, kv_len_out=None, temperature=1.0, seed=0, round_=0, top_k=0, top_p=1.0):
        """Ragged chain accept: sequence b has lens[b] rows from logits / token
        row row_start[b], its drafts' q rows from q_start[b]."""
        B = row_start.shape[0]
        smp = spec_sampling(float(temperature), 0, int(seed), int(round_), int(top_k), float(top_p))
        q_rows = 0 if q is None else q.reshape(-1, q.shape[-1]).shape[0]
        return spec_accept_ragged(self.handle, B, max_len, logits.reshape(-1, logits.shape[-1]).shape[0], q_rows,
                                  row_start, lens, q_start, logits, q, tokens, smp, out_tokens, num_accepted,
                                  kv_len, kv_len_out, self.stream)

    def accept(self, logits, q, tokens, out_tokens, num_accepted, kv_len, kv_len_out=None,
               tree_parent=None, temperature=1.0, seed=0, round_=0, replacement=False, top_k=0, top_p=1.0):
        B, T = tokens.shape
        smp = spec_sampling(float(temperature), 1 if replacement else 0, int(seed), int(round_), int(top_k),
                            float(top_p))
        return spec_accept(self.handle, B, T, logits, q, tokens, tree_parent, smp, out_tokens,
                           num_accepted, kv_len, kv_len_out, self.stream)

    def profile_gemm(self, cls: str, rows: int, iters: int):
        """(ms, algorithmic bytes) of `iters` back-to-back passes of one GEMM
        class over all layers; overwrites the workspace activations."""
        return spec_profile_gemm(self.handle, cls, rows, iters, self.stream)

    def graphs(self, enable: bool):
        """Replay the recorded per-layer launches (default) or launch directly."""
        spec_graph_enable(self.handle, enable)

    def device_errors(self) -> int:
        return spec_device_errors(self.handle, self.stream)

    def close(self):
        if self.handle:
            spec_verify_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
