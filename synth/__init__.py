"""Seeded synthetic inputs shared by the HIP path and the CPU oracle.

This module only draws random numbers and lays them out in the buffers the
C ABI expects.  It holds none of the verify method's arithmetic: no forward
pass, no accept rule, no residual, no commit.  Both sides read what it makes;
neither side's code lives here.

The model shapes follow the Llama-style decoder the workloads name:
RMSNorm, rotary position embedding, grouped-query attention, a SiLU-gated
feed-forward block and an untied output head.  All weight matrices (the
embedding included) are drawn from N(0, 0.02^2); the three norm gains are 1.

Weight order (one device pointer per entry, row-major [out, in]):
    embed [V, d]
    per layer: attn_norm [d] (fp32), w_qkv [(Hq + 2 Hkv) D, d] (q rows, then
               k rows, then v rows), w_o [d, Hq D], ffn_norm [d] (fp32),
               w_gate_up [2F, d] (gate rows, then up rows), w_down [d, F]
    final_norm [d] (fp32), lm_head [V, d]

KV cache: one bf16 buffer [L][2][max_batch][Hkv][max_ctx * D].  The K half
holds each head's keys row by row ([max_ctx][D]); the V half holds each
head's values transposed within blocks of 64 positions ([max_ctx/64][D][64],
the layout of a page of the paged cache).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, asdict

import torch

# ----------------------------------------------------------------------------
# model shapes
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    rms_eps: float
    rope_theta: float
    weight_dtype: str  # "f32" or "bf16"

    def as_dict(self):
        return asdict(self)

    @property
    def qkv_rows(self):
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def torch_dtype(self):
        return torch.float32 if self.weight_dtype == "f32" else torch.bfloat16

    def n_weights(self):
        return 1 + 6 * self.n_layers + 2

    def streamed_params(self):
        """Parameters one verify step reads (all matrices except the embedding
        table, of which only the gathered rows are touched)."""
        d, F = self.d_model, self.d_ffn
        per_layer = self.qkv_rows * d + d * self.n_heads * self.head_dim + 2 * F * d + d * F
        return self.n_layers * per_layer + self.vocab * d


# Toy dense decoder: 2 layers, d=256, 4 heads of 64, FFN 1024, vocab 4096, fp32.
TOY = ModelShape(n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
                 d_ffn=1024, vocab=4096, rms_eps=1e-5, rope_theta=10000.0,
                 weight_dtype="f32")

# Llama-3-8B shape: 32 layers, d=4096, 32 q / 8 kv heads of 128, FFN 14336,
# vocab 128256, bf16 weights.
LLAMA8B = ModelShape(n_layers=32, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128,
                     d_ffn=14336, vocab=128256, rms_eps=1e-5, rope_theta=500000.0,
                     weight_dtype="bf16")

# A reduced 8B-like shape (same head layout and GQA group, two layers, smaller
# FFN and vocab) used for parity at sizes the oracle finishes in seconds.
MINI8B = ModelShape(n_layers=2, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128,
                    d_ffn=1024, vocab=8192, rms_eps=1e-5, rope_theta=500000.0,
                    weight_dtype="bf16")

# The 8B layer at full width (FFN 14336) with two layers and a small vocab:
# exercises the long-K down projection at real size.
FFN8B = ModelShape(n_layers=2, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128,
                   d_ffn=14336, vocab=8192, rms_eps=1e-5, rope_theta=500000.0,
                   weight_dtype="bf16")

WEIGHT_STD = 0.02
# Synthetic cached K/V: the scale x.W has for unit-RMS x at d=4096.
KV_STD = WEIGHT_STD * math.sqrt(4096.0)

SEED_WEIGHTS, SEED_PROMPT, SEED_KV, SEED_NOISE, SEED_DRAFT, SEED_ACCEPT = 0, 1, 2, 3, 4, 5


def weight_names(shape: ModelShape):
    names = ["embed"]
    for l in range(shape.n_layers):
        names += [f"l{l}.attn_norm", f"l{l}.w_qkv", f"l{l}.w_o", f"l{l}.ffn_norm",
                  f"l{l}.w_gate_up", f"l{l}.w_down"]
    names += ["final_norm", "lm_head"]
    return names


def weight_shapes(shape: ModelShape):
    d, F, V = shape.d_model, shape.d_ffn, shape.vocab
    out = {"embed": (V, d)}
    for l in range(shape.n_layers):
        out[f"l{l}.attn_norm"] = (d,)
        out[f"l{l}.w_qkv"] = (shape.qkv_rows, d)
        out[f"l{l}.w_o"] = (d, shape.n_heads * shape.head_dim)
        out[f"l{l}.ffn_norm"] = (d,)
        out[f"l{l}.w_gate_up"] = (2 * F, d)
        out[f"l{l}.w_down"] = (d, F)
    out["final_norm"] = (d,)
    out["lm_head"] = (V, d)
    return out


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_weights(shape: ModelShape, seed: int = SEED_WEIGHTS, device="cpu"):
    """Return (names, tensors).  Matrices ~ N(0, 0.02^2) rounded to the weight
    dtype; norm gains are fp32 ones.  Each matrix has its own stream
    (seed * 1000003 + index) so tensors can be drawn one at a time."""
    names = weight_names(shape)
    shapes = weight_shapes(shape)
    out = []
    for i, n in enumerate(names):
        shp = shapes[n]
        if len(shp) == 1:
            out.append(torch.ones(shp, dtype=torch.float32, device=device))
            continue
        g = _gen(seed * 1000003 + i, device)
        # draw in row blocks to bound the fp32 temporary for the vocab matrices
        rows = shp[0]
        step = max(1, (1 << 26) // shp[1])
        res = torch.empty(shp, dtype=shape.torch_dtype, device=device)
        for r0 in range(0, rows, step):
            r1 = min(rows, r0 + step)
            blk = torch.randn((r1 - r0, shp[1]), generator=g, dtype=torch.float32, device=device)
            res[r0:r1] = (blk * WEIGHT_STD).to(shape.torch_dtype)
        out.append(res)
    return names, out


# ----------------------------------------------------------------------------
# KV cache
# ----------------------------------------------------------------------------


def kv_cache_numel(shape: ModelShape, max_batch: int, max_ctx: int) -> int:
    return shape.n_layers * 2 * max_batch * shape.n_kv_heads * max_ctx * shape.head_dim


KV_BLOCK = 64  # positions per V block (the page size)


def kv_v_blocks(cache: torch.Tensor, shape: ModelShape, max_batch: int, max_ctx: int):
    """The V half of the flat bf16 cache as stored: [L, B, Hkv, max_ctx/64, D, 64]
    (a view: writes go to the cache)."""
    L, H, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
    c = cache.view(L, 2, max_batch, H, max_ctx * D)
    return c[:, 1].view(L, max_batch, H, max_ctx // KV_BLOCK, D, KV_BLOCK)


def kv_views(cache: torch.Tensor, shape: ModelShape, max_batch: int, max_ctx: int, seqs: int = 0):
    """K view [L, B, Hkv, max_ctx, D] of the flat bf16 cache buffer, and V as
    [L, B, Hkv, D, max_ctx] (values transposed, positions in order).  K is a
    view of the buffer; V is a copy gathered from its 64-position blocks, for
    reading (write V through kv_v_blocks).  With seqs > 0 only the first seqs
    sequences (B = seqs)."""
    L, H, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
    nb = seqs if seqs > 0 else max_batch
    c = cache.view(L, 2, max_batch, H, max_ctx * D)
    k = c[:, 0].view(L, max_batch, H, max_ctx, D)[:, :nb]
    vb = kv_v_blocks(cache, shape, max_batch, max_ctx)[:, :nb]
    v = torch.empty((L, nb, H, D, max_ctx), dtype=cache.dtype, device=cache.device)
    v.view(L, nb, H, D, max_ctx // KV_BLOCK, KV_BLOCK).copy_(vb.permute(0, 1, 2, 4, 3, 5))
    return k, v


def make_kv_cache(shape: ModelShape, max_batch: int, max_ctx: int, ctx_len, seed: int = SEED_KV,
                  device="cpu", poison_tail: bool = True):
    """Allocate the cache and fill positions [0, ctx_len[b]) of every sequence
    with i.i.d. N(0, KV_STD^2) in bf16 (keys taken as already rotated).  The
    tail beyond ctx_len is NaN when poison_tail, so reads past the committed
    length show up as non-finite output."""
    n = kv_cache_numel(shape, max_batch, max_ctx)
    cache = torch.full((n,), float("nan") if poison_tail else 0.0, dtype=torch.bfloat16, device=device)
    k, _ = kv_views(cache, shape, max_batch, max_ctx)
    vb = kv_v_blocks(cache, shape, max_batch, max_ctx)
    g = _gen(seed, device)
    if isinstance(ctx_len, int):
        ctx_len = [ctx_len] * max_batch
    L, H, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
    for b, c in enumerate(ctx_len):
        if c <= 0:
            continue
        for l in range(L):
            kk = torch.randn((H, c, D), generator=g, device=device) * KV_STD
            vv = torch.randn((H, D, c), generator=g, device=device) * KV_STD
            k[l, b, :, :c, :] = kk.to(torch.bfloat16)
            # positions [0, c) of V into the 64-position blocks (block j holds
            # positions 64 j .. 64 j + 63 as [D][64])
            nb = (c + KV_BLOCK - 1) // KV_BLOCK
            vt = vb[l, b, :, :nb].permute(0, 2, 1, 3).reshape(H, D, nb * KV_BLOCK).clone()  # positions in order
            vt[:, :, :c] = vv.to(torch.bfloat16)
            vb[l, b, :, :nb] = vt.view(H, D, nb, KV_BLOCK).permute(0, 2, 1, 3)
    return cache


def paged_kv_views(pool: torch.Tensor, shape: ModelShape, kv_pages: int, page: int = 64):
    """K view [L, pages, Hkv, page, D] and V view [L, pages, Hkv, D, page] of a
    flat bf16 page pool."""
    L, H, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
    c = pool.view(L, 2, kv_pages, H, page * D)
    return c[:, 0].view(L, kv_pages, H, page, D), c[:, 1].view(L, kv_pages, H, D, page)


def make_kv_pool(shape: ModelShape, kv_pages: int, seed: int = SEED_KV, device="cpu", page: int = 64):
    """A page pool filled with i.i.d. N(0, KV_STD^2) bf16 (the synthetic
    context's distribution), for timing a paged cache."""
    L, H, D = shape.n_layers, shape.n_kv_heads, shape.head_dim
    g = _gen(seed, device)
    n = L * 2 * kv_pages * H * page * D
    return (torch.randn((n,), generator=g, device=device) * KV_STD).to(torch.bfloat16)


def random_block_table(max_batch: int, pages_per_seq: int, kv_pages: int, seed: int = SEED_KV):
    """A block table [max_batch, pages_per_seq] int32 naming distinct pool pages
    in a seeded random order (kv_pages >= max_batch * pages_per_seq)."""
    assert kv_pages >= max_batch * pages_per_seq
    g = torch.Generator(device="cpu").manual_seed(seed + 77)
    perm = torch.randperm(kv_pages, generator=g)[: max_batch * pages_per_seq]
    return perm.view(max_batch, pages_per_seq).to(torch.int32)


# ----------------------------------------------------------------------------
# tokens, logits and synthetic drafts
# ----------------------------------------------------------------------------


def make_tokens(B: int, T: int, vocab: int, seed: int = SEED_PROMPT, device="cpu"):
    g = _gen(seed, device)
    return torch.randint(0, vocab, (B, T), generator=g, dtype=torch.int32, device=device)


def random_logits(rows_shape, vocab: int, seed: int, scale: float = KV_STD, device="cpu"):
    """Flat random logits N(0, scale^2), the spread a random-init head gives."""
    g = _gen(seed, device)
    return torch.randn((*rows_shape, vocab), generator=g, dtype=torch.float32, device=device) * scale


def noisy_draft_dist(z: torch.Tensor, sigma: float, seed: int, temperature: float = 1.0):
    """Draft distribution of the noisy-target draft model: q = softmax((z + eps)/T),
    eps ~ N(0, sigma^2) i.i.d. per entry.  Returns (q fp32, noisy logits)."""
    g = _gen(seed, z.device)
    eps = torch.randn(z.shape, generator=g, dtype=torch.float32, device=z.device) * sigma
    zn = z.float() + eps
    if temperature == 0.0:
        return None, zn
    q = torch.softmax(zn.double() / temperature, dim=-1).float()
    # renormalise in fp32 so each row sums to 1 as stored
    q = q / q.sum(dim=-1, keepdim=True)
    return q, zn


def sample_from(q: torch.Tensor, seed: int, n: int = 1, replacement: bool = True):
    """Draw token ids from the rows of q (fp32 probabilities) with torch's own
    sampler; the draft side of the synthetic round."""
    g = _gen(seed, q.device)
    flat = q.reshape(-1, q.shape[-1]).double()
    ids = torch.multinomial(flat, n, replacement=replacement, generator=g)
    return ids.view(*q.shape[:-1], n).to(torch.int32)


def random_tree(branching, B: int = 1):
    """Full token tree with the given branching per depth, nodes in breadth-first
    order (every parent index precedes its children).  Node 0 is the root (the
    pending token).  Returns parent ids [B, T] int32 (root = -1)."""
    parents = [-1]
    level = [0]
    for k in branching:
        nxt = []
        for v in level:
            for _ in range(k):
                parents.append(v)
                nxt.append(len(parents) - 1)
        level = nxt
    t = torch.tensor(parents, dtype=torch.int32)
    return t.unsqueeze(0).repeat(B, 1)


def tree_children(parent_row):
    """children[v] = node ids whose parent is v, ascending."""
    T = len(parent_row)
    ch = [[] for _ in range(T)]
    for c in range(1, T):
        ch[int(parent_row[c])].append(c)
    return ch


# ----------------------------------------------------------------------------
# recurrent (linear-attention) layer inputs
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class RecurrentShape:
    n_heads: int     # H
    head_dim: int    # D, key and value width per head
    conv_width: int  # W, taps of the causal convolution

    @property
    def channels(self):
        return 3 * self.n_heads * self.head_dim


# 32 heads of width 128 with a 4-tap convolution: the mixer of a hybrid
# model's recurrent layers at the 8B width (d_model = 32 * 128)
RECURRENT_8B = RecurrentShape(n_heads=32, head_dim=128, conv_width=4)
SEED_RECURRENT = 4242


def make_recurrent_inputs(rs: RecurrentShape, B: int, T: int, n_slots: int, seed: int = SEED_RECURRENT,
                          device="cpu"):
    """Random inputs of one verify window of a recurrent layer, fp32:
      x          [B][T][3HD]     raw q|k|v channels, N(0, 1)
      gate       [B][T][H][D]    log decay, uniform in [-0.5, 0]
      beta       [B][T][H]       write strength, uniform in [0, 1]
      conv_w     [3HD][W]        taps, N(0, 1/W)
      conv_state [n_slots][W-1][3HD]  raw inputs before the window, N(0, 1)
      state      [n_slots][H][D][D]   recurrent states, N(0, 0.25)
    Each tensor has its own stream (seed * 1000003 + index)."""
    H, D, W, C = rs.n_heads, rs.head_dim, rs.conv_width, rs.channels

    def g(i):
        return _gen(seed * 1000003 + i, "cpu")

    out = {
        "x": torch.randn((B, T, C), generator=g(0)),
        "gate": -0.5 * torch.rand((B, T, H, D), generator=g(1)),
        "beta": torch.rand((B, T, H), generator=g(2)),
        "conv_w": torch.randn((C, W), generator=g(3)) / math.sqrt(W),
        "conv_state": torch.randn((n_slots, W - 1, C), generator=g(4)),
        "state": 0.5 * torch.randn((n_slots, H, D, D), generator=g(5)),
    }
    return {k: v.to(device) for k, v in out.items()}


# ----------------------------------------------------------------------------
# bf16 helpers for moving tensors to the oracle (bit reinterpretation only)
# ----------------------------------------------------------------------------


def to_numpy_raw(t: torch.Tensor):
    """Host copy as numpy: bf16 tensors come back as their uint16 bit patterns,
    everything else as is."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
