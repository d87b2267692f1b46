// Device helpers shared by the verify-step kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define DEVI __device__ __forceinline__

// --- bf16 -----------------------------------------------------------------
// A dword holding two bf16 values: low half is element 0, high half element 1.
DEVI float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
DEVI float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
DEVI float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
DEVI uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): 16 significant bits,
// relative error <= 2^-17.  Used to feed fp32 activations to bf16 MFMA.
DEVI void split_bf16(float x, short& hi, short& lo) {
  uint32_t h = f32_to_bf16_rne(x);
  float r = x - __uint_as_float(h << 16);
  hi = (short)h;
  lo = (short)f32_to_bf16_rne(r);
}

// --- MFMA -----------------------------------------------------------------
// D(16x16, fp32) += A(16x16, bf16) * B(16x16, bf16).
// Lane l holds A[l%16][4(l/16) + e], B[4(l/16) + e][l%16] (e = 0..3) and
// D[4(l/16) + e][l%16].
DEVI floatx4 mfma16x16x16(shortx4 a, shortx4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16), the gfx950 form with
// twice the contraction per instruction: lane l holds A[l%16][8(l/16) + e],
// B[8(l/16) + e][l%16] (e = 0..7) and D as above.
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
DEVI floatx4 mfma16x16x32(shortx8 a, shortx8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16): lane l holds
// A[l%32][8(l/32) + e], B[8(l/32) + e][l%32] (e = 0..7) and D[8(i/4) +
// 4(l/32) + i%4][l%32] (i = 0..15).
typedef float floatx16 __attribute__((ext_vector_type(16)));
DEVI floatx16 mfma32x32x16(shortx8 a, shortx8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// --- wave reductions ------------------------------------------------------
DEVI float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DEVI float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// --- workgroup barrier for LDS traffic only -------------------------------
// __syncthreads() also orders global memory, which makes every wave wait for
// all of its outstanding global loads at the barrier.  Kernels that keep
// weight loads in flight across an LDS reduction use this barrier instead: it
// orders LDS accesses only, so the loads stay outstanding.
DEVI void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// --- Philox4x64-10 (Salmon et al., SC'11) -----------------------------------
// Key (seed, 0), counter (slot, sequence, round, 0); the accept uniform is
// u = (word0 >> 40) * 2^-24.
DEVI uint64_t philox4x64_word0(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t k0,
                               uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
    uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
    uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}
DEVI float philox_uniform(uint64_t seed, uint64_t round, int b, int slot) {
  uint64_t w = philox4x64_word0((uint64_t)slot, (uint64_t)b, round, 0ull, seed, 0ull);
  return (float)(w >> 40) * 0x1p-24f;
}

#define FLAG_TOKEN_RANGE 1u
#define FLAG_TREE 2u
#define FLAG_KV_OVERFLOW 4u
#define FLAG_LAYOUT 8u

// ---------------------------------------------------------------- KV addressing
// A layer's cache, dense or paged.  Dense: K region [maxB][Hkv][max_ctx][D],
// V region [maxB][Hkv][max_ctx / KV_PAGE][D][KV_PAGE]: V transposed within
// blocks of KV_PAGE slots, so that the key index (the contraction index of
// P V) is contiguous and a 32-key block's values are one 16 KB run with its
// neighbour (a plain [D][max_ctx] transpose read 64-byte pieces 64 KB apart:
// 3.0 TB/s against 7.0 for contiguous blocks, measured).  Paged
// (PagedAttention, pages of KV_PAGE slots): K region
// [npages][Hkv][KV_PAGE][D], V region [npages][Hkv][D][KV_PAGE]; slot s of
// sequence b lives in page table[b * ppseq + s / KV_PAGE] at offset
// s % KV_PAGE.  Page ids outside the pool are clamped (the prep kernel flags
// them), so no access leaves it.
constexpr int KV_PAGE = 64;
struct KvMap {
  const int32_t* table;  // [B][ppseq] page ids, or null: dense
  int ppseq;             // pages per sequence (table row length)
  int npages;            // pages in the pool
  int max_ctx;           // dense slot stride
};
// page holding slot s of sequence b (paged cache only), clamped into the pool
DEVI int kv_page(const KvMap& m, int b, int s) {
  int pi = s / KV_PAGE;
  pi = pi < 0 ? 0 : (pi >= m.ppseq ? m.ppseq - 1 : pi);
  const int pg = m.table[(size_t)b * m.ppseq + pi];
  return pg < 0 ? 0 : (pg >= m.npages ? m.npages - 1 : pg);
}
// first slot of slot s's run of contiguous slots (a page, or the whole
// sequence when dense), as an element offset of K row s and of V (dim 0, s);
// the _pg forms take the page of slot s already looked up (ignored when dense)
DEVI size_t kv_k_off_pg(const KvMap& m, int Hkv, int D, int b, int h, int s, int pg) {
  if (!m.table) return (((size_t)b * Hkv + h) * m.max_ctx + s) * D;
  return (((size_t)pg * Hkv + h) * KV_PAGE + (s % KV_PAGE)) * D;
}
DEVI size_t kv_k_off(const KvMap& m, int Hkv, int D, int b, int h, int s) {
  return kv_k_off_pg(m, Hkv, D, b, h, s, m.table ? kv_page(m, b, s) : 0);
}
// element offset of V (dim, slot s); the slots of one block of KV_PAGE
// (a page) are contiguous for a fixed dim, with this stride between dims
DEVI int kv_v_stride(const KvMap&) { return KV_PAGE; }
DEVI size_t kv_v_off_pg(const KvMap& m, int Hkv, int D, int b, int h, int dim, int s, int pg) {
  if (!m.table)
    return ((((size_t)b * Hkv + h) * (m.max_ctx / KV_PAGE) + s / KV_PAGE) * D + dim) * KV_PAGE + (s % KV_PAGE);
  return (((size_t)pg * Hkv + h) * D + dim) * KV_PAGE + (s % KV_PAGE);
}
DEVI size_t kv_v_off(const KvMap& m, int Hkv, int D, int b, int h, int dim, int s) {
  return kv_v_off_pg(m, Hkv, D, b, h, dim, s, m.table ? kv_page(m, b, s) : 0);
}
