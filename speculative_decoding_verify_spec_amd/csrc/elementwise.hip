// Per-step preparation, embedding gather and RMSNorm.
#include "common.h"
#include "launch.h"

namespace sv {

// One workgroup per sequence.  Validates tokens, cache room and the tree;
// writes each row's clamped token, rotary position (kv_len + i for a chain,
// kv_len + depth for a tree node), cache slot (kv_len + i) and, for a tree,
// the ancestor-or-self bitmask used by the attention mask.
__global__ __launch_bounds__(128) void prep_kernel(PrepParams p) {
  const int b = blockIdx.x;
  const int T = p.T;
  __shared__ int depth[128];
  __shared__ uint64_t anc_lo[128], anc_hi[128];
  __shared__ int bad_tree;
  int kv = p.kv_len[b];
  if (threadIdx.x == 0) {
    bad_tree = 0;
    if (kv < 0 || kv > p.max_ctx - T) atomicOr(p.flags, FLAG_KV_OVERFLOW);
    if (p.parent) {
      const int32_t* par = p.parent + (size_t)b * T;
      depth[0] = 0;
      anc_lo[0] = 1ull;
      anc_hi[0] = 0ull;
      if (par[0] != -1) bad_tree = 1;
      for (int i = 1; i < T; ++i) {
        int pi = par[i];
        if (pi < 0 || pi >= i) {
          bad_tree = 1;
          pi = i - 1;  // treat as a chain link so later kernels stay in bounds
        }
        depth[i] = depth[pi] + 1;
        anc_lo[i] = anc_lo[pi] | (i < 64 ? (1ull << i) : 0ull);
        anc_hi[i] = anc_hi[pi] | (i >= 64 ? (1ull << (i - 64)) : 0ull);
      }
      if (bad_tree) atomicOr(p.flags, FLAG_TREE);
    }
  }
  __syncthreads();
  const int kvc = kv < 0 ? 0 : kv;
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    const int m = b * T + i;
    int t = p.tokens[m];
    if (t < 0 || t >= p.vocab) {
      atomicOr(p.flags, FLAG_TOKEN_RANGE);
      t = t < 0 ? 0 : p.vocab - 1;
    }
    p.tok[m] = t;
    int ps = kvc + (p.parent ? depth[i] : i);
    p.pos[m] = ps < p.max_ctx ? ps : p.max_ctx - 1;
    int sl = kvc + i;
    p.slot[m] = (kv >= 0 && sl < p.max_ctx) ? sl : -1;
    if (p.parent) {
      p.anc[2 * m] = anc_lo[i];
      p.anc[2 * m + 1] = anc_hi[i];
    }
  }
}

hipError_t launch_prep(const PrepParams& p, hipStream_t s) {
  prep_kernel<<<p.B, 128, 0, s>>>(p);
  return hipGetLastError();
}

// x[m][:] = E[tok[m]][:] in fp32.
template <typename WT>
__global__ __launch_bounds__(256) void embed_kernel(const WT* E, const int32_t* tok, float* x, int d) {
  const int m = blockIdx.x;
  const WT* row = E + (size_t)tok[m] * d;
  for (int k = threadIdx.x; k < d; k += 256) {
    if constexpr (sizeof(WT) == 2)
      x[(size_t)m * d + k] = bf16_to_f32(row[k]);
    else
      x[(size_t)m * d + k] = row[k];
  }
}

hipError_t launch_embed(const void* E, int wdtype, const int32_t* tok, float* x, int M, int d,
                        hipStream_t s) {
  if (wdtype == 1)
    embed_kernel<uint16_t><<<M, 256, 0, s>>>((const uint16_t*)E, tok, x, d);
  else
    embed_kernel<float><<<M, 256, 0, s>>>((const float*)E, tok, x, d);
  return hipGetLastError();
}

// One workgroup per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* x, const float* g, float* h, int d,
                                                      float eps) {
  const int m = blockIdx.x;
  const float* xr = x + (size_t)m * d;
  float ss = 0.f;
  for (int k = threadIdx.x; k < d; k += 256) ss += xr[k] * xr[k];
  ss = wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = part[0] + part[1] + part[2] + part[3];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
  for (int k = threadIdx.x; k < d; k += 256) h[(size_t)m * d + k] = xr[k] * inv * g[k];
}

hipError_t launch_rmsnorm(const float* x, const float* g, float* h, int M, int d, float eps,
                          hipStream_t s) {
  rmsnorm_kernel<<<M, 256, 0, s>>>(x, g, h, d, eps);
  return hipGetLastError();
}

}  // namespace sv
