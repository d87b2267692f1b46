// Skinny-M weight-streaming GEMM: Y[m][n] = sum_k X[m][k] * W[n][k] for a few
// activation rows m, every weight element read from HBM exactly once for all
// rows (CS349E Lecture 6, section 6.1: verifying gamma+1 positions reads the
// weights once, like one decode step).
//
// Layout of the work.  A workgroup owns YT output rows of W and all M
// activation rows.  Its KS waves interleave over K in 512-element steps; in a
// step each lane reads 16 bytes (8 bf16) of each of the YT weight rows, so one
// wave instruction reads a contiguous 1 KiB of a row.  Activations are fp32
// (read through the caches, shared by all waves of the GPU) and every product
// is accumulated in fp32.  At the end each wave folds its YT*M partial sums
// across the 64 lanes with a halving exchange (each stage sends half of the
// values it still holds), the waves add their results in LDS and the
// epilogue runs on the finished sums:
//   STORE  out[m][n] = y                      (LM head -> logits)
//   RESID  out[m][n] += y                     (O and down projections)
//   SWIGLU out[m][n] = silu(y_gate) * y_up    (gate/up: row pairs n, F + n)
//   QKV    rotary embedding on the (i, i + D/2) row pairs of each q/k head,
//          q -> rotated-query buffer, k/v -> fp32 suffix buffers and the bf16
//          cache slot of the row.
#include "common.h"
#include "launch.h"

namespace sv {

constexpr int YT = 8;        // weight rows per workgroup
constexpr int MAX_KS = 8;    // waves per workgroup splitting K

template <int MT>
struct MaxPow2 {
  static constexpr int v = (YT * MT <= 8) ? 8 : (YT * MT <= 16) ? 16 : (YT * MT <= 32) ? 32 : 64;
};

// Weight row handled by slot y of row group rg.
template <int EPI>
DEVI int gemm_row(const GemmParams& p, int rg, int y) {
  if (EPI == EPI_SWIGLU) {
    const int half = YT / 2;
    return y < half ? rg * half + y : p.F + rg * half + (y - half);
  }
  if (EPI == EPI_QKV) {
    const int half = YT / 2;
    const int gph = (p.D / 2) / half;  // row groups per head
    const int hh = rg / gph, i0 = (rg % gph) * half;
    return y < half ? hh * p.D + i0 + y : hh * p.D + p.D / 2 + i0 + (y - half);
  }
  return rg * YT + y;
}

// 8 consecutive weights of one row as fp32 (the address is always valid;
// `ok` only zeroes the values, so no load sits behind a branch).
template <typename WT>
DEVI void load_w8(const WT* __restrict__ W, size_t off, bool ok, float (&w)[8]);
template <>
DEVI void load_w8<uint16_t>(const uint16_t* __restrict__ W, size_t off, bool ok, float (&w)[8]) {
  uint4 v = *(const uint4*)(W + off);
  const uint32_t msk = ok ? 0xffffffffu : 0u;
  v.x &= msk; v.y &= msk; v.z &= msk; v.w &= msk;
  w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x);
  w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
  w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z);
  w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
}
template <>
DEVI void load_w8<float>(const float* __restrict__ W, size_t off, bool ok, float (&w)[8]) {
  float4 a = *(const float4*)(W + off);
  float4 b = *(const float4*)(W + off + 4);
  w[0] = ok ? a.x : 0.f; w[1] = ok ? a.y : 0.f; w[2] = ok ? a.z : 0.f; w[3] = ok ? a.w : 0.f;
  w[4] = ok ? b.x : 0.f; w[5] = ok ? b.y : 0.f; w[6] = ok ? b.z : 0.f; w[7] = ok ? b.w : 0.f;
}

// Halving exchange across the 64 lanes, unrolled at compile time: at offset
// O a lane keeps half of the CNT values it holds (the upper half when its bit
// O is set, else the lower half), adds the partner's copy of that half and
// sends the other half to the partner.  After log2(CNT) stages lane l holds
// the sum over the lanes of its group for value index l >> (6 - log2(CNT));
// the remaining stages add the group members' sums.
template <int CNT, int O>
DEVI void lane_fold(float* acc, int lane) {
  if constexpr (O >= 1) {
    if constexpr (CNT >= 2) {
      constexpr int H = CNT / 2;
      const bool upper = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = upper ? acc[i] : acc[i + H];
        const float keep = upper ? acc[i + H] : acc[i];
        acc[i] = keep + __shfl_xor(send, O, 64);
      }
      lane_fold<H, O / 2>(acc, lane);
    } else {
      acc[0] += __shfl_xor(acc[0], O, 64);
      lane_fold<1, O / 2>(acc, lane);
    }
  }
}

template <int MT, typename WT, int EPI>
__global__ __launch_bounds__(64 * MAX_KS) void gemm_valu_kernel(GemmParams p) {
  constexpr int NV = YT * MT;
  constexpr int NVP = MaxPow2<MT>::v;
  constexpr int U = MT <= 4 ? 2 : 1;  // K steps whose loads are issued together
  __shared__ float red[MAX_KS][NVP];
  __shared__ float tot[NVP];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int KS = blockDim.x >> 6;
  const int rg = blockIdx.x;
  const WT* __restrict__ W = (const WT*)p.W;
  const float* __restrict__ X = p.X;

  int rows[YT];
  bool rok[YT];
#pragma unroll
  for (int y = 0; y < YT; ++y) {
    rows[y] = gemm_row<EPI>(p, rg, y);
    rok[y] = rows[y] < p.N;
  }

  float acc[NVP];
#pragma unroll
  for (int i = 0; i < NVP; ++i) acc[i] = 0.f;

  const int nsteps = (p.K + 511) >> 9;
  // One K step: each lane loads 8 consecutive k of the YT weight rows and of
  // the MT activation rows.  Only the K tail (K not a multiple of 512) is
  // masked per lane; the address stays valid.
  auto load_step = [&](int s, float (&wv)[YT][8], float (&xv)[MT][8]) {
    const int kraw = s * 512 + lane * 8;
    const bool kok = kraw < p.K;
    const int k0 = kok ? kraw : 0;
#pragma unroll
    for (int y = 0; y < YT; ++y)
      load_w8<WT>(W, (size_t)(rok[y] ? rows[y] : 0) * p.K + k0, kok && rok[y], wv[y]);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const bool ok = kok && (m < p.M);
      const float* xs = X + (size_t)(m < p.M ? m : 0) * p.ldx + k0;
      const float4 a = *(const float4*)xs;
      const float4 b = *(const float4*)(xs + 4);
      xv[m][0] = ok ? a.x : 0.f; xv[m][1] = ok ? a.y : 0.f;
      xv[m][2] = ok ? a.z : 0.f; xv[m][3] = ok ? a.w : 0.f;
      xv[m][4] = ok ? b.x : 0.f; xv[m][5] = ok ? b.y : 0.f;
      xv[m][6] = ok ? b.z : 0.f; xv[m][7] = ok ? b.w : 0.f;
    }
  };
  auto fma_step = [&](const float (&wv)[YT][8], const float (&xv)[MT][8]) {
#pragma unroll
    for (int y = 0; y < YT; ++y)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float a = acc[y * MT + m];
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(wv[y][e], xv[m][e], a);
        acc[y * MT + m] = a;
      }
  };
  // Waves of the workgroup interleave over K steps; U steps' loads are issued
  // before their products so each wave keeps U*YT 16-byte loads in flight.
  int s = w;
  for (; s + (U - 1) * KS < nsteps; s += U * KS) {
    float wv[U][YT][8];
    float xv[U][MT][8];
#pragma unroll
    for (int u = 0; u < U; ++u) load_step(s + u * KS, wv[u], xv[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) fma_step(wv[u], xv[u]);
  }
  for (; s < nsteps; s += KS) {
    float wv[YT][8];
    float xv[MT][8];
    load_step(s, wv, xv);
    fma_step(wv, xv);
  }

  lane_fold<NVP, 32>(acc, lane);
  // lane l now holds value index l >> (6 - log2(NVP)); the lowest lane of each
  // group writes it.
  constexpr int SH = (NVP == 8) ? 3 : (NVP == 16) ? 2 : (NVP == 32) ? 1 : 0;
  if ((lane & ((1 << SH) - 1)) == 0) red[w][lane >> SH] = acc[0];
  __syncthreads();
  if (threadIdx.x < NV) {
    float t = 0.f;
    for (int i = 0; i < KS; ++i) t += red[i][threadIdx.x];
    tot[threadIdx.x] = t;
  }
  __syncthreads();

  // ---------------------------------------------------------------- epilogues
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    if (threadIdx.x < NV) {
      const int y = threadIdx.x / MT, m = threadIdx.x % MT;
      const int n = gemm_row<EPI>(p, rg, y);
      if (m < p.M && n < p.N) {
        float* o = p.out + (size_t)m * p.ldo + n;
        if constexpr (EPI == EPI_STORE)
          *o = tot[threadIdx.x];
        else
          *o += tot[threadIdx.x];
      }
    }
    return;
  } else {
  constexpr int NP = (YT / 2) * MT;  // (row pair, activation row) items
  if (threadIdx.x >= NP) return;
  const int yp = threadIdx.x / MT, m = threadIdx.x % MT;
  if (m >= p.M) return;
  const float a = tot[yp * MT + m];
  const float b = tot[(yp + YT / 2) * MT + m];
  if constexpr (EPI == EPI_SWIGLU) {
    const int n = gemm_row<EPI>(p, rg, yp);
    if (n < p.F) p.out[(size_t)m * p.ldo + n] = a / (1.0f + expf(-a)) * b;
    return;
  }
  // EPI_QKV
  const int r0 = gemm_row<EPI>(p, rg, yp);
  if (r0 >= p.N) return;
  const int D = p.D, half = D / 2;
  const int hh = r0 / D, i = r0 % D;  // i < D/2
  const int mg = p.m0 + m;            // global row
  const int bseq = mg / p.T;
  if (hh < p.Hq + p.Hkv) {
    const int ps = p.pos[mg];
    const float c = p.rope_cos[(size_t)ps * half + i], s = p.rope_sin[(size_t)ps * half + i];
    const float ra = a * c - b * s, rb = b * c + a * s;
    if (hh < p.Hq) {
      float* q = p.q_out + ((size_t)mg * p.Hq + hh) * D;
      q[i] = ra;
      q[i + half] = rb;
    } else {
      const int hk = hh - p.Hq;
      float* k = p.k_out + ((size_t)mg * p.Hkv + hk) * D;
      k[i] = ra;
      k[i + half] = rb;
      const int sl = p.slot[mg];
      if (sl >= 0) {
        uint16_t* kc = p.kcache + (((size_t)bseq * p.Hkv + hk) * p.max_ctx + sl) * D;
        kc[i] = (uint16_t)f32_to_bf16_rne(ra);
        kc[i + half] = (uint16_t)f32_to_bf16_rne(rb);
      }
    }
  } else {
    const int hv = hh - p.Hq - p.Hkv;
    float* v = p.v_out + ((size_t)mg * p.Hkv + hv) * D;
    v[i] = a;
    v[i + half] = b;
    const int sl = p.slot[mg];
    if (sl >= 0) {
      uint16_t* vc = p.vcache + ((size_t)bseq * p.Hkv + hv) * D * (size_t)p.max_ctx;
      vc[(size_t)i * p.max_ctx + sl] = (uint16_t)f32_to_bf16_rne(a);
      vc[(size_t)(i + half) * p.max_ctx + sl] = (uint16_t)f32_to_bf16_rne(b);
    }
  }
  }
}

template <int MT, int EPI>
static hipError_t launch_mte(const GemmParams& p, int groups, int ks, hipStream_t s) {
  if (p.wdtype == 1)
    gemm_valu_kernel<MT, uint16_t, EPI><<<groups, 64 * ks, 0, s>>>(p);
  else
    gemm_valu_kernel<MT, float, EPI><<<groups, 64 * ks, 0, s>>>(p);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_mt(const GemmParams& p, int groups, int ks, hipStream_t s) {
  switch (p.epi) {
    case EPI_STORE: return launch_mte<MT, EPI_STORE>(p, groups, ks, s);
    case EPI_RESID: return launch_mte<MT, EPI_RESID>(p, groups, ks, s);
    case EPI_SWIGLU: return launch_mte<MT, EPI_SWIGLU>(p, groups, ks, s);
    default: return launch_mte<MT, EPI_QKV>(p, groups, ks, s);
  }
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  int groups;
  if (p.epi == EPI_SWIGLU)
    groups = p.F / (YT / 2);
  else if (p.epi == EPI_QKV)
    groups = (p.Hq + 2 * p.Hkv) * ((p.D / 2) / (YT / 2));
  else
    groups = (p.N + YT - 1) / YT;
  // Enough waves to keep every CU streaming: split K across up to 8 waves
  // of a workgroup when there are few row groups.
  const int nsteps = (p.K + 511) / 512;
  int ks = 1;
  while (ks < MAX_KS && ks * 2 <= nsteps && groups * ks < 4096) ks *= 2;
  if (p.M <= 1) return launch_mt<1>(p, groups, ks, s);
  if (p.M <= 2) return launch_mt<2>(p, groups, ks, s);
  if (p.M <= 4) return launch_mt<4>(p, groups, ks, s);
  return launch_mt<8>(p, groups, ks, s);
}

}  // namespace sv
