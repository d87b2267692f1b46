// Attention of the verify rows over the KV cache plus the speculative suffix.
//
// Context part (attn_ctx_kernel).  Rows of one sequence that share a KV head
// (the GQA group of G query heads times T verify rows: nq = G*T query
// vectors) read that head's cached keys once, inside one wave, so the
// gamma+1 rows of a sequence share one KV read (CS349E Lecture 6, section 9.2).
// The context of a (sequence, KV head) is cut into `splits` workgroups of 4
// waves; each wave keeps its own online-softmax state (flash-decoding style),
// the four states are merged in LDS and the workgroup writes one partial
// (max, sum, unnormalised output) per query.  The
// products run on bf16 MFMA 16x16x16: S^T = K Q^T with K exact in bf16 and
// the fp32 queries split into bf16 hi + lo, then O^T += V^T P^T with the fp32
// probabilities split the same way; accumulation is fp32.  V is stored
// transposed in the cache so the key index (the contraction of P V) is
// contiguous.
//
// Combine part (attn_combine_kernel), one wave per (row, query head): merges
// the split partials, adds the suffix keys in fp32 (chain: rows 0..i; tree:
// the node and its ancestors) and normalises.  Keys beyond a wave's range are
// loaded as zeros and masked, so nothing past kv_len is ever used.
#include "common.h"
#include "launch.h"

namespace sv {

int attn_query_tiles_per_wave(int nq) { return nq > 16 ? 2 : 1; }
int attn_nsplit(int splits) { return splits; }

// Key index held in row r of key tile kt of the 32-key block at kb: rows
// 4g..4g+3 of both tiles cover keys kb + 8g .. kb + 8g + 7, so one 16-byte
// load of V^T feeds both tiles.
DEVI int blk_key(int kb, int kt, int r) { return kb + 8 * (r >> 2) + 4 * kt + (r & 3); }

template <int D, int QT>
__global__ __launch_bounds__(256) void attn_ctx_kernel(AttnParams p) {
  constexpr int DG = D / 4;   // dims per lane group
  constexpr int KSTEPS = D / 16;
  constexpr int DT = D / 16;  // output dim tiles
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int s = blockIdx.x;
  const int kvh = blockIdx.y % p.Hkv, qg = blockIdx.y / p.Hkv;
  const int b = blockIdx.z;
  const int G = p.Hq / p.Hkv;
  const int nq = G * p.T;

  int L = p.kv_len[b];
  L = L < 0 ? 0 : (L > p.max_ctx ? p.max_ctx : L);
  int chunk = (L + p.splits - 1) / p.splits;
  chunk = (chunk + 127) & ~127;
  const int kbeg = s * chunk;
  const int kend = min(L, kbeg + chunk);

  // ---- queries: B operand of S^T = K Q^T; lane (j, g) holds query j's dims
  // g*DG + 4*ks + e for k-step ks.
  shortx4 qhi[QT][KSTEPS], qlo[QT][KSTEPS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qi = (qg * QT + qt) * 16 + j;
    float qv[DG];
    if (qi < nq) {
      const int i = qi / G, gg = qi % G;
      const float* src = p.q + (((size_t)(b * p.T + i)) * p.Hq + kvh * G + gg) * D + g * DG;
#pragma unroll
      for (int e = 0; e < DG; e += 4) {
        float4 v = *(const float4*)(src + e);
        qv[e] = v.x * p.scale; qv[e + 1] = v.y * p.scale;
        qv[e + 2] = v.z * p.scale; qv[e + 3] = v.w * p.scale;
      }
    } else {
#pragma unroll
      for (int e = 0; e < DG; ++e) qv[e] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        short hi, lo;
        split_bf16(qv[4 * ks + e], hi, lo);
        qhi[qt][ks][e] = hi;
        qlo[qt][ks][e] = lo;
      }
    }
  }

  floatx4 o[QT][DT];
  float mrun[QT], lrun[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrun[qt] = -INFINITY;
    lrun[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[qt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const uint16_t* kbase = p.kc + ((size_t)b * p.Hkv + kvh) * (size_t)p.max_ctx * D;
  const uint16_t* vbase = p.vc + ((size_t)b * p.Hkv + kvh) * (size_t)D * p.max_ctx;

  for (int kb = kbeg + 32 * w; kb < kend; kb += 128) {
    // ---- K operand (A of S^T): lane row j of tile kt is key blk_key(kb, kt, j)
    shortx4 ka[2][KSTEPS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = blk_key(kb, kt, j);
      const bool ok = key < kend;
      const uint16_t* src = kbase + (size_t)key * D + g * DG;
#pragma unroll
      for (int e = 0; e < DG; e += 8) {
        uint4 v = ok ? *(const uint4*)(src + e) : make_uint4(0, 0, 0, 0);
        const int ks = e / 4;
        ka[kt][ks][0] = (short)(v.x & 0xffff); ka[kt][ks][1] = (short)(v.x >> 16);
        ka[kt][ks][2] = (short)(v.y & 0xffff); ka[kt][ks][3] = (short)(v.y >> 16);
        ka[kt][ks + 1][0] = (short)(v.z & 0xffff); ka[kt][ks + 1][1] = (short)(v.z >> 16);
        ka[kt][ks + 1][2] = (short)(v.w & 0xffff); ka[kt][ks + 1][3] = (short)(v.w >> 16);
      }
    }
    // ---- V^T operand (A of O^T += V^T P^T): lane row j of dim tile dt is
    // dim dt*16 + j; its k index 4g + e in key tile kt is key kb + 8g + 4kt + e.
    shortx4 va[DT][2];
    {
      const int k8 = kb + 8 * g;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint16_t* src = vbase + (size_t)(dt * 16 + j) * p.max_ctx + k8;
        uint4 v = (k8 < kend) ? *(const uint4*)src : make_uint4(0, 0, 0, 0);
        uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t h = (e & 1) ? (wv[e >> 1] >> 16) : (wv[e >> 1] & 0xffff);
          if (k8 + e >= kend) h = 0;  // never multiply a probability by data past the range
          va[dt][e >> 2][e & 3] = (short)h;
        }
      }
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      floatx4 st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          acc = mfma16x16x16(ka[kt][ks], qhi[qt][ks], acc);
          acc = mfma16x16x16(ka[kt][ks], qlo[qt][ks], acc);
        }
        st[kt] = acc;
      }
      // st[kt][e]: query j, key kb + 8g + 4kt + e
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (kb + 8 * g + 4 * kt + e >= kend) st[kt][e] = -INFINITY;
          bmax = fmaxf(bmax, st[kt][e]);
        }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
      const float mnew = fmaxf(mrun[qt], bmax);
      const float factor = __expf(mrun[qt] - mnew);
      mrun[qt] = mnew;
      float psum = 0.f;
      shortx4 phi[2], plo[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = __expf(st[kt][e] - mnew);
          psum += pe;
          short hi, lo;
          split_bf16(pe, hi, lo);
          phi[kt][e] = hi;
          plo[kt][e] = lo;
        }
      lrun[qt] = lrun[qt] * factor + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[qt][dt] *= factor;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          o[qt][dt] = mfma16x16x16(va[dt][kt], phi[kt], o[qt][dt]);
          o[qt][dt] = mfma16x16x16(va[dt][kt], plo[kt], o[qt][dt]);
        }
      }
    }
  }

  // ---- merge the four waves' states in LDS and write one partial per query
  constexpr int QN = QT * 16;
  constexpr int OS = D + 4;  // padded row stride of the staged outputs
  __shared__ float s_m[4][QN];
  __shared__ float s_l[4][QN];
  __shared__ float s_o[4][QN * OS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float l = lrun[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    lrun[qt] = l;
    if (g == 0) s_m[w][qt * 16 + j] = mrun[qt];
  }
  __syncthreads();
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qq = qt * 16 + j;
    const float mall = fmaxf(fmaxf(s_m[0][qq], s_m[1][qq]), fmaxf(s_m[2][qq], s_m[3][qq]));
    // a wave that saw no key has m = -inf and contributes nothing
    const float f = (mrun[qt] == -INFINITY) ? 0.f : __expf(mrun[qt] - mall);
    if (g == 0) s_l[w][qq] = lrun[qt] * f;
    float* dst = &s_o[w][qq * OS];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *(float4*)(dst + dt * 16 + 4 * g) =
          make_float4(o[qt][dt][0] * f, o[qt][dt][1] * f, o[qt][dt][2] * f, o[qt][dt][3] * f);
  }
  __syncthreads();
  const size_t pbase = (((size_t)s * p.B + b) * p.Hkv + kvh) * nq;
  for (int e = threadIdx.x; e < QN * D; e += 256) {
    const int qq = e / D, dd = e % D;
    const int qi = (qg * QT) * 16 + qq;
    if (qi >= nq) continue;
    const int o2 = qq * OS + dd;
    p.part_o[(pbase + qi) * D + dd] = s_o[0][o2] + s_o[1][o2] + s_o[2][o2] + s_o[3][o2];
  }
  if (threadIdx.x < QN) {
    const int qq = threadIdx.x;
    const int qi = (qg * QT) * 16 + qq;
    if (qi < nq) {
      const float mall = fmaxf(fmaxf(s_m[0][qq], s_m[1][qq]), fmaxf(s_m[2][qq], s_m[3][qq]));
      p.part_ml[2 * (pbase + qi)] = mall;
      p.part_ml[2 * (pbase + qi) + 1] = s_l[0][qq] + s_l[1][qq] + s_l[2][qq] + s_l[3][qq];
    }
  }
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  const int nq = (p.Hq / p.Hkv) * p.T;
  const int QT = attn_query_tiles_per_wave(nq);
  const int nqg = (nq + 16 * QT - 1) / (16 * QT);
  dim3 grid(p.splits, p.Hkv * nqg, p.B);
  if (p.D == 128) {
    if (QT == 1) attn_ctx_kernel<128, 1><<<grid, 256, 0, s>>>(p);
    else attn_ctx_kernel<128, 2><<<grid, 256, 0, s>>>(p);
  } else {
    if (QT == 1) attn_ctx_kernel<64, 1><<<grid, 256, 0, s>>>(p);
    else attn_ctx_kernel<64, 2><<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

// One workgroup per (row i, KV head, sequence); wave g handles query head
// kvh * G + g.  The split statistics are read by all lanes at once, the
// weighted sum of the split outputs keeps every load in flight, then the
// suffix keys (chain: rows 0..i; tree: the node and its ancestors) are added
// in fp32 and the result normalised.
template <int D>
__global__ __launch_bounds__(512) void attn_combine_kernel(CombineParams p) {
  constexpr int PL = D / 64;  // dims per lane
  constexpr int MAXS = 128;
  __shared__ float s_w[8][MAXS];
  const int i = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, gg = threadIdx.x >> 6;
  const int G = p.Hq / p.Hkv;
  const int hq = kvh * G + gg;
  const int nq = G * p.T;
  const int qi = i * G + gg;
  const int m = b * p.T + i;
  const int ns = p.nsplit;

  // split statistics: M = max over splits with mass, weights exp(m_s - M)
  float mloc = -INFINITY;
  for (int sp = lane; sp < ns; sp += 64) {
    const size_t base = (((size_t)sp * p.B + b) * p.Hkv + kvh) * nq + qi;
    if (p.part_ml[2 * base + 1] > 0.f) mloc = fmaxf(mloc, p.part_ml[2 * base]);
  }
  const float mstar = wave_max(mloc);
  float lloc = 0.f;
  for (int sp = lane; sp < ns; sp += 64) {
    const size_t base = (((size_t)sp * p.B + b) * p.Hkv + kvh) * nq + qi;
    const float ls = p.part_ml[2 * base + 1];
    const float wgt = (ls > 0.f) ? expf(p.part_ml[2 * base] - mstar) : 0.f;
    s_w[gg][sp] = wgt;
    lloc += wgt * ls;
  }
  float l = wave_sum(lloc);
  __syncthreads();
  float acc[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) acc[e] = 0.f;
  float mcur = mstar;
  if (l > 0.f) {
    int sp = 0;
    for (; sp + 8 <= ns; sp += 8) {
      float v[8][PL];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* src = p.part_o + ((((size_t)(sp + u) * p.B + b) * p.Hkv + kvh) * nq + qi) * D;
#pragma unroll
        for (int e = 0; e < PL; ++e) v[u][e] = src[lane + 64 * e];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < PL; ++e) acc[e] += s_w[gg][sp + u] * v[u][e];
    }
    for (; sp < ns; ++sp) {
      const float* src = p.part_o + ((((size_t)sp * p.B + b) * p.Hkv + kvh) * nq + qi) * D;
#pragma unroll
      for (int e = 0; e < PL; ++e) acc[e] += s_w[gg][sp] * src[lane + 64 * e];
    }
  } else {
    mcur = -INFINITY;
    l = 0.f;
  }
  // suffix keys in fp32
  float qv[PL];
  const float* qsrc = p.q + ((size_t)m * p.Hq + hq) * D;
#pragma unroll
  for (int e = 0; e < PL; ++e) qv[e] = qsrc[lane + 64 * e];
  for (int jj = 0; jj < p.T; ++jj) {
    bool vis;
    if (p.anc) {
      const uint64_t word = p.anc[2 * m + (jj >> 6)];
      vis = (word >> (jj & 63)) & 1ull;
    } else {
      vis = jj <= i;
    }
    if (!vis) continue;
    const int mj = b * p.T + jj;
    const float* ksp = p.k_suf + ((size_t)mj * p.Hkv + kvh) * D;
    float d = 0.f;
#pragma unroll
    for (int e = 0; e < PL; ++e) d += qv[e] * ksp[lane + 64 * e];
    const float sc = wave_sum(d) * p.scale;
    const float mnew = fmaxf(mcur, sc);
    const float f1 = expf(mcur - mnew), ee = expf(sc - mnew);
    const float* vsp = p.v_suf + ((size_t)mj * p.Hkv + kvh) * D;
#pragma unroll
    for (int e = 0; e < PL; ++e) acc[e] = acc[e] * f1 + ee * vsp[lane + 64 * e];
    l = l * f1 + ee;
    mcur = mnew;
  }
  float* dst = p.out + ((size_t)m * p.Hq + hq) * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < PL; ++e) dst[lane + 64 * e] = acc[e] * inv;
}

hipError_t launch_attn_combine(const CombineParams& p, hipStream_t s) {
  const int G = p.Hq / p.Hkv;
  if (G > 8 || p.nsplit > 128) return hipErrorInvalidValue;
  dim3 grid(p.T, p.Hkv, p.B);
  if (p.D == 128)
    attn_combine_kernel<128><<<grid, 64 * G, 0, s>>>(p);
  else
    attn_combine_kernel<64><<<grid, 64 * G, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
