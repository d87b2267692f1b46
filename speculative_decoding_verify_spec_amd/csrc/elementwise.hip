// Per-step preparation and embedding gather.
#include "common.h"
#include "launch.h"

namespace sv {

// Slots a sequence may use: max_ctx, and with a paged cache also its table
// row's pages.  Paged: table entries for the pages of slots [0, n) must name
// pool pages (FLAG_LAYOUT otherwise; the addressing clamps them).
DEVI int seq_capacity(const PrepParams& p) {
  return p.kvm.table ? min(p.max_ctx, p.kvm.ppseq * KV_PAGE) : p.max_ctx;
}
DEVI void check_pages(const PrepParams& p, int b, int n) {
  if (!p.kvm.table) return;
  const int np = min(p.kvm.ppseq, (n + KV_PAGE - 1) / KV_PAGE);
  for (int i = 0; i < np; ++i) {
    const int pg = p.kvm.table[(size_t)b * p.kvm.ppseq + i];
    if (pg < 0 || pg >= p.kvm.npages) {
      atomicOr(p.flags, FLAG_LAYOUT);
      break;
    }
  }
}

// Workgroup (b, y) prepares rows PREP_ROWS*y .. of sequence b.  The first of
// a sequence copies kv_len into the workspace (the later kernels of the step
// read only the workspace, weights and cache, so their launch sequence can be
// recorded once and replayed) and validates cache room and the tree; every
// workgroup validates its rows' tokens, writes each row's clamped token,
// rotary position (kv_len + i for a chain, kv_len + depth for a tree node),
// cache slot (kv_len + i), for a tree the ancestor-or-self bitmask used by the
// attention mask, and gathers the rows' embeddings into the fp32 residual
// stream x.  A tree's depths and masks come from the whole parent array, which
// each workgroup reads (at most 128 entries).
constexpr int PREP_ROWS = 8;
template <typename WT>
__global__ __launch_bounds__(256) void prep_embed_kernel(PrepParams p) {
  const int b = blockIdx.x;
  const int T = p.T;
  const int r0 = blockIdx.y * PREP_ROWS, r1 = min(T, r0 + PREP_ROWS);
  const bool lead = blockIdx.y == 0;
  __shared__ int depth[128];
  __shared__ uint64_t anc_lo[128], anc_hi[128];
  __shared__ int stok[128];
  __shared__ int spar[128];
  const int kv = p.kv_len[b];
  const int cap = seq_capacity(p);
  if (lead && threadIdx.x == 0) {
    p.kv_copy[b] = kv;
    if (kv < 0 || kv > cap - T) atomicOr(p.flags, FLAG_KV_OVERFLOW);
    check_pages(p, b, min(cap, (kv < 0 ? 0 : kv) + T));
  }
  if (p.parent) {
    // a node's parent must precede it (the root's is -1); a bad link is
    // flagged and taken as a chain link, so every walk below ends at node 0
    const int32_t* par = p.parent + (size_t)b * T;
    bool bad = false;
    for (int i = threadIdx.x; i < T; i += blockDim.x) {
      int pi = par[i];
      if (i == 0 ? pi != -1 : (pi < 0 || pi >= i)) {
        bad = true;
        pi = i - 1;
      }
      spar[i] = pi;
    }
    if (bad && lead) atomicOr(p.flags, FLAG_TREE);
    __syncthreads();
    // each node walks to the root: its depth and its ancestor-or-self bits
    for (int i = r0 + threadIdx.x; i < r1; i += blockDim.x) {
      int d = 0;
      uint64_t lo = 0ull, hi = 0ull;
      for (int c = i;; c = spar[c], ++d) {
        if (c < 64) lo |= 1ull << c;
        else hi |= 1ull << (c - 64);
        if (c == 0) break;
      }
      depth[i] = d;
      anc_lo[i] = lo;
      anc_hi[i] = hi;
    }
  }
  __syncthreads();
  const int kvc = kv < 0 ? 0 : kv;
  for (int i = r0 + threadIdx.x; i < r1; i += blockDim.x) {
    const int m = b * T + i;
    int t = p.tokens[m];
    if (t < 0 || t >= p.vocab) {
      atomicOr(p.flags, FLAG_TOKEN_RANGE);
      t = t < 0 ? 0 : p.vocab - 1;
    }
    p.tok[m] = t;
    stok[i] = t;
    const int ps = kvc + (p.parent ? depth[i] : i);
    p.pos[m] = ps < p.max_ctx ? ps : p.max_ctx - 1;
    const int sl = kvc + i;
    p.slot[m] = (kv >= 0 && sl < cap) ? sl : -1;
    if (p.parent) {
      p.anc[2 * m] = anc_lo[i];
      p.anc[2 * m + 1] = anc_hi[i];
    }
  }
  __syncthreads();
  // embedding rows, 8 elements per thread per pass
  const WT* E = (const WT*)p.embed;
  const int per_row = p.d / 8;
  for (int e = threadIdx.x; e < (r1 - r0) * per_row; e += blockDim.x) {
    const int i = r0 + e / per_row, c = (e % per_row) * 8;
    const WT* src = E + (size_t)stok[i] * p.d + c;
    float* dst = p.x + ((size_t)(b * T + i)) * p.d + c;
    if constexpr (sizeof(WT) == 2) {
      const uint4 v = *(const uint4*)src;
      *(float4*)dst = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
      *(float4*)(dst + 4) = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
    } else {
      *(float4*)dst = *(const float4*)src;
      *(float4*)(dst + 4) = *(const float4*)(src + 4);
    }
  }
}

// Ragged (packed) chain rows, DeepSeek-V4 analysis page, section 4 (compact
// verify): sequence b owns rows cu[b] .. cu[b+1]-1 of the caller's token
// array, at positions and cache slots kv_len[b] + i; rows cu[B] .. rows-1 pad
// the launch up to its recorded size (token 0, no cache slot, sequence 0).
// Workgroup b < B prepares sequence b, workgroup B the padding rows.  An
// offset array that is not increasing, lengths outside [1, T] or offsets
// past `rows` set FLAG_LAYOUT; the values are clamped so every later access
// stays in bounds.
template <typename WT>
__global__ __launch_bounds__(256) void prep_ragged_kernel(PrepParams p) {
  const int b = blockIdx.x;
  __shared__ int s_start, s_len, s_kv;
  if (threadIdx.x == 0) {
    int start, len, kv = 0;
    if (b < p.B) {
      const int c0 = p.cu[b], c1 = p.cu[b + 1];
      start = c0 < 0 ? 0 : (c0 > p.rows ? p.rows : c0);
      len = c1 - c0;
      bool bad = c0 < 0 || c1 > p.rows || len < 1 || len > p.T || (b == 0 && c0 != 0);
      len = len < 0 ? 0 : (len > p.T ? p.T : len);
      if (start + len > p.rows) len = p.rows - start;
      if (bad) atomicOr(p.flags, FLAG_LAYOUT);
      kv = p.kv_len[b];
      p.kv_copy[b] = kv;
      p.rstart[b] = start;
      p.rlen[b] = len;
      if (kv < 0 || kv > seq_capacity(p) - len) atomicOr(p.flags, FLAG_KV_OVERFLOW);
      check_pages(p, b, min(seq_capacity(p), (kv < 0 ? 0 : kv) + len));
    } else {
      const int c = p.cu[p.B];
      start = c < 0 ? 0 : (c > p.rows ? p.rows : c);
      len = p.rows - start;
    }
    s_start = start;
    s_len = len;
    s_kv = kv;
  }
  __syncthreads();
  const int start = s_start, len = s_len, kv = s_kv;
  const bool pad = b == p.B;
  const int kvc = kv < 0 ? 0 : kv;
  for (int i = threadIdx.x; i < len; i += blockDim.x) {
    const int m = start + i;
    int t = pad ? 0 : p.tokens[m];
    if (t < 0 || t >= p.vocab) {
      atomicOr(p.flags, FLAG_TOKEN_RANGE);
      t = t < 0 ? 0 : p.vocab - 1;
    }
    p.tok[m] = t;
    const int ps = kvc + i;
    p.pos[m] = pad ? 0 : (ps < p.max_ctx ? ps : p.max_ctx - 1);
    p.slot[m] = (!pad && kv >= 0 && ps < seq_capacity(p)) ? ps : -1;
    p.seq[m] = pad ? 0 : b;
  }
  __syncthreads();
  const WT* E = (const WT*)p.embed;
  const int per_row = p.d / 8;
  for (int e = threadIdx.x; e < len * per_row; e += blockDim.x) {
    const int i = e / per_row, c = (e % per_row) * 8;
    const WT* src = E + (size_t)p.tok[start + i] * p.d + c;
    float* dst = p.x + ((size_t)(start + i)) * p.d + c;
    if constexpr (sizeof(WT) == 2) {
      const uint4 v = *(const uint4*)src;
      *(float4*)dst = make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
      *(float4*)(dst + 4) = make_float4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w));
    } else {
      *(float4*)dst = *(const float4*)src;
      *(float4*)(dst + 4) = *(const float4*)(src + 4);
    }
  }
}

hipError_t launch_prep(const PrepParams& p, hipStream_t s) {
  if (p.cu) {
    if (p.wdtype == 1)
      prep_ragged_kernel<uint16_t><<<p.B + 1, 256, 0, s>>>(p);
    else
      prep_ragged_kernel<float><<<p.B + 1, 256, 0, s>>>(p);
    return hipGetLastError();
  }
  const dim3 grid(p.B, (p.T + PREP_ROWS - 1) / PREP_ROWS);
  if (p.wdtype == 1)
    prep_embed_kernel<uint16_t><<<grid, 256, 0, s>>>(p);
  else
    prep_embed_kernel<float><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
