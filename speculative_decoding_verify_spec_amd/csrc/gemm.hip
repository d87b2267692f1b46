// Skinny-M weight-streaming GEMM: Y[m][n] = sum_k X[m][k] * W[n][k] for a few
// activation rows m (M <= 8), every weight element read from HBM exactly once
// for all rows (CS349E Lecture 6, section 6.1: verifying gamma+1 positions
// reads the weights once, like one decode step).  Products are fp32 on the
// vector ALUs: bf16 weights widened to fp32, fp32 activations, fp32 sums.
//
// Work layout.  A K "step" is 512 consecutive k: each lane of a wave covers 8
// of them, so one wave instruction reads a contiguous 1 KiB of a weight row
// (non-temporal: weights are touched once per step and should not evict the
// activations from the caches).  A workgroup owns YT weight rows at a time
// and all M activation rows; its waves split the K steps between them.  Each
// wave folds its YT*M partial sums across its 64 lanes with a halving
// exchange, the waves add their results in LDS, and the epilogue runs on the
// finished sums.
//
// Two kernels:
//   * k-stationary (K <= 4 waves x 2 steps, i.e. K <= 4096): every wave keeps
//     its slice of the activation rows in registers for the whole kernel and
//     the workgroup loops over row groups.  Because the workgroup's waves
//     together hold entire activation rows, an RMSNorm in front of the GEMM is
//     fused here: the prologue sums x^2 over the rows, and scales each
//     register by g[k] / sqrt(mean + eps).
//   * streaming (longer K, the down projection at 1-2 rows): activations are
//     re-read through the caches with every step.
// (At 3-8 rows the down projection runs on the matrix-core kernel below, in
// K slices.)
//
// Epilogues:
//   STORE  out[m][n] = y                      (LM head -> logits)
//   RESID  out[m][n] += y                     (O and down projections)
//   SWIGLU out[m][n] = silu(y_gate) * y_up    (gate/up: row pairs n, F + n)
//   QKV    rotary embedding on the (i, i + D/2) row pairs of each q/k head,
//          q -> rotated-query buffer, k/v -> fp32 suffix buffers and the bf16
//          cache slot of the row.
#include "common.h"
#include "launch.h"

namespace sv {

constexpr int YT = 8;            // weight rows per row group
constexpr int KSTAT_WAVES = 4;   // waves per workgroup, k-stationary kernel
constexpr int KSTAT_SPW = 2;     // K steps per wave, k-stationary kernel
constexpr int STREAM_WAVES = 8;  // waves per workgroup, streaming kernel
constexpr int SPLIT_WAVES = 8;   // waves per workgroup, K-split matrix-core kernel

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

template <int EPI>
__host__ __device__ int gemm_groups(const GemmParams& p) {
  if (EPI == EPI_SWIGLU) return p.F / (YT / 2);
  if (EPI == EPI_QKV) return (p.Hq + 2 * p.Hkv) * ((p.D / 2) / (YT / 2));
  return (p.N + YT - 1) / YT;
}

// 8 consecutive weights of one row as fp32, loaded non-temporally.
template <typename WT>
DEVI void load_w8(const WT* __restrict__ W, size_t off, float (&w)[8]);
template <>
DEVI void load_w8<uint16_t>(const uint16_t* __restrict__ W, size_t off, float (&w)[8]) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)(W + off));
  w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x);
  w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
  w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z);
  w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
}
template <>
DEVI void load_w8<float>(const float* __restrict__ W, size_t off, float (&w)[8]) {
  const f32x4 a = __builtin_nontemporal_load((const f32x4*)(W + off));
  const f32x4 b = __builtin_nontemporal_load((const f32x4*)(W + off + 4));
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// Eight weights of one row as loaded, widened to fp32 only where they are
// used, so a prefetched row group costs 4 registers per 8 bf16 weights.
template <typename WT>
struct WRaw;
template <>
struct WRaw<uint16_t> {
  u32x4 v;
  DEVI void load(const uint16_t* __restrict__ W, size_t off) {
    v = __builtin_nontemporal_load((const u32x4*)(W + off));
  }
  DEVI void widen(float (&w)[8]) const {
    w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x);
    w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
    w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z);
    w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
  }
};
template <>
struct WRaw<float> {
  f32x4 a, b;
  DEVI void load(const float* __restrict__ W, size_t off) {
    a = __builtin_nontemporal_load((const f32x4*)(W + off));
    b = __builtin_nontemporal_load((const f32x4*)(W + off + 4));
  }
  DEVI void widen(float (&w)[8]) const {
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
};

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

template <int MT>
DEVI void fma_rows(float* acc, const float (&w)[8], const float (&x)[MT][8], int y) {
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    float a = acc[y * MT + m];
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaf(w[e], x[m][e], a);
    acc[y * MT + m] = a;
  }
}

// Fold one row group's partial sums over lanes and waves; returns with the
// YT*MT sums in tot[] (all threads synchronised).  With `ssq` (per-wave sums
// of x^2 of the activation rows, [nwaves][MT] in LDS) the sums are scaled by
// the rows' RMSNorm factor 1/sqrt(mean(x^2) + eps): the norm's gain was
// applied to the activations, its row factor is applied here.
template <int MT, bool LDS_ONLY = false>
DEVI void reduce_group(float* acc, int lane, int w, int nwaves, float (*red)[MaxPow2<MT>::v], float* tot,
                       const float (*ssq)[MT] = nullptr, float inv_k = 0.f, float eps = 0.f) {
  constexpr int NV = YT * MT;
  constexpr int NVP = MaxPow2<MT>::v;
  constexpr int SH = (NVP == 8) ? 3 : (NVP == 16) ? 2 : (NVP == 32) ? 1 : 0;
  lane_fold<NVP, 32>(acc, lane);
  if ((lane & ((1 << SH) - 1)) == 0) red[w][lane >> SH] = acc[0];
  if constexpr (LDS_ONLY) lds_barrier(); else __syncthreads();
  if (threadIdx.x < NV) {
    float t = 0.f;
    for (int i = 0; i < nwaves; ++i) t += red[i][threadIdx.x];
    if (ssq) {
      const int m = threadIdx.x % MT;
      float q = 0.f;
      for (int i = 0; i < nwaves; ++i) q += ssq[i][m];
      t *= 1.0f / sqrtf(q * inv_k + eps);
    }
    tot[threadIdx.x] = t;
  }
  if constexpr (LDS_ONLY) lds_barrier(); else __syncthreads();
}

// Per-row inputs of the QKV epilogue (cache slot, rotary cos/sin at the
// row's position), staged in LDS by the prologue so that the epilogue of
// every row group reads LDS instead of two dependent global loads.
template <int MT>
struct QkvStage {
  int slot[MT];
  float cs[MT][64];
  float sn[MT][64];
};

// The staging in three steps, for a prologue that must not wait on memory
// before its weight loads are out: the positions and slots are requested
// first (pos), the rotary values once the weights have been requested (rope;
// it waits only for the positions, the oldest loads), and the LDS stores
// come last (store).  Thread t of NT holds items t, t + NT, ...
template <int MT, int NT>
struct QkvPre {
  static constexpr int IT = (MT * 64 + NT - 1) / NT;
  int ps[IT], sl[IT];
  float c[IT], s[IT];
  DEVI void pos(const GemmParams& p) {
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int t = threadIdx.x + k * NT, m = t / 64;
      ps[k] = 0;
      sl[k] = 0;
      if (m < MT && m < p.M) {
        ps[k] = p.pos[p.m0 + m];
        if (t % 64 == 0) sl[k] = p.slot[p.m0 + m];
      }
    }
  }
  DEVI void rope(const GemmParams& p) {
    const int half = p.D / 2;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int t = threadIdx.x + k * NT, m = t / 64, i = t % 64;
      c[k] = s[k] = 0.f;
      if (m < MT && m < p.M && i < half) {
        c[k] = p.rope_cos[(size_t)ps[k] * half + i];
        s[k] = p.rope_sin[(size_t)ps[k] * half + i];
      }
    }
  }
  DEVI void store(const GemmParams& p, QkvStage<MT>* st) const {
    const int half = p.D / 2;
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int t = threadIdx.x + k * NT, m = t / 64, i = t % 64;
      if (m < MT && m < p.M) {
        if (i < half) {
          st->cs[m][i] = c[k];
          st->sn[m][i] = s[k];
        }
        if (i == 0) st->slot[m] = sl[k];
      }
    }
  }
};

// Epilogue for row group rg from the finished sums tot[y * MT + m].  `st`:
// the QKV stage in LDS, or null to read those inputs from global memory.
template <int MT, int EPI>
DEVI void epilogue(const GemmParams& p, int rg, const float* tot, const QkvStage<MT>* st = nullptr) {
  constexpr int NV = YT * MT;
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
    } else {
      // EPI_QKV
      const int r0 = gemm_row<EPI>(p, rg, yp);
      if (r0 >= p.N) return;
      const int D = p.D, half = D / 2;
      const int hh = r0 / D, i = r0 % D;  // i < D/2
      const int mg = p.m0 + m;            // global row
      const int bseq = p.seq ? p.seq[mg] : mg / p.T;
      const int sl = st ? st->slot[m] : p.slot[mg];
      if (hh < p.Hq + p.Hkv) {
        float c, s;
        if (st) {
          c = st->cs[m][i];
          s = st->sn[m][i];
        } else {
          const int ps = p.pos[mg];
          c = p.rope_cos[(size_t)ps * half + i];
          s = p.rope_sin[(size_t)ps * half + i];
        }
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
          if (sl >= 0) {
            uint16_t* kc = p.kcache + kv_k_off(p.kvm, p.Hkv, D, bseq, hk, sl);
            kc[i] = (uint16_t)f32_to_bf16_rne(ra);
            kc[i + half] = (uint16_t)f32_to_bf16_rne(rb);
          }
        }
      } else {
        const int hv = hh - p.Hq - p.Hkv;
        float* v = p.v_out + ((size_t)mg * p.Hkv + hv) * D;
        v[i] = a;
        v[i + half] = b;
        if (sl >= 0) {
          p.vcache[kv_v_off(p.kvm, p.Hkv, D, bseq, hv, i, sl)] = (uint16_t)f32_to_bf16_rne(a);
          p.vcache[kv_v_off(p.kvm, p.Hkv, D, bseq, hv, i + half, sl)] = (uint16_t)f32_to_bf16_rne(b);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- k-stationary
// XP: the launch completes its activation rows from deferred partial sums
// (GemmParams::xpart; QKV with the fused norm only).
template <int MT, typename WT, int EPI, bool NORM, int NW, bool XP = false>
__global__ __launch_bounds__(64 * NW) void gemm_kstat_kernel(GemmParams p) {
  constexpr int NVP = MaxPow2<MT>::v;
  constexpr int SPW = KSTAT_WAVES * KSTAT_SPW / NW;  // K steps per wave
  __shared__ float red[NW][NVP];
  __shared__ float tot[NVP];
  __shared__ float ssq[NW][MT];
  __shared__ QkvStage<(EPI == EPI_QKV) ? MT : 1> qst;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const WT* __restrict__ W = (const WT*)p.W;
  const int nsteps = (p.K + 511) >> 9;

  // ---- this wave's K steps.  A lane with no k in range loads from the start
  // of the row (always in bounds) and multiplies it by zero activations, so
  // the loads need no branches.
  int kofs[SPW];
  bool kok[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int s = w + i * NW;
    const int kraw = s * 512 + lane * 8;
    kok[i] = (s < nsteps) && (kraw < p.K);
    kofs[i] = kok[i] ? kraw : 0;
  }
  const int ngroups = gemm_groups<EPI>(p);
  WRaw<WT> wr[SPW][YT];
  auto load_group = [&](int g_) {
#pragma unroll
    for (int y = 0; y < YT; ++y) {
      int r = gemm_row<EPI>(p, g_, y);
      r = r < p.N ? r : 0;  // the LM head's last group may be short; those rows are never stored
#pragma unroll
      for (int i = 0; i < SPW; ++i) wr[i][y].load(W, (size_t)r * p.K + kofs[i]);
    }
  };
  int rg = blockIdx.x;

  // ---- prologue.  Everything the first row group needs is requested before
  // any of it is consumed: the rows' positions (QKV), this wave's activation
  // slice (with the deferred partial sums), the norm gain, then the first
  // group's weights, and the rotary values, which need the positions.  A
  // value consumed in between would make the wave wait for it, and for every
  // load requested before it, before the weights are even asked for.
  QkvPre<MT, 64 * NW> qpre;
  if constexpr (EPI == EPI_QKV) qpre.pos(p);
  float4 xa[SPW][MT][2];
#pragma unroll
  for (int i = 0; i < SPW; ++i)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float* xs = p.X + (size_t)(m < p.M ? m : 0) * p.ldx + kofs[i];
      xa[i][m][0] = *(const float4*)xs;
      xa[i][m][1] = *(const float4*)(xs + 4);
    }
  // the deferred reduce of the previous residual GEMM
  constexpr int NSL = XP ? GEMM_KSPLIT : 1;
  float4 pa[SPW][MT][NSL][2];
  if constexpr (XP) {
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
          const float* ps = p.xpart + ((size_t)(sl * 8 + (m < p.M ? m : 0))) * p.ldx + kofs[i];
          pa[i][m][sl][0] = *(const float4*)ps;
          pa[i][m][sl][1] = *(const float4*)(ps + 4);
        }
  }
  float4 ga[SPW][2];
  if constexpr (NORM) {
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      ga[i][0] = *(const float4*)(p.norm_g + kofs[i]);
      ga[i][1] = *(const float4*)(p.norm_g + kofs[i] + 4);
    }
  }
  // the first row group's weights (a workgroup without a group reads rows
  // clamped into range and never uses them)
  load_group(rg);
  if constexpr (EPI == EPI_QKV) qpre.rope(p);
  // nothing is scheduled across this point: left alone, the compiler adds the
  // partial sums (waiting for them) before the weight loads are issued
  __builtin_amdgcn_sched_barrier(0);

  // ---- this wave's activation slice, kept in registers
  float xr[SPW][MT][8];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const bool ok = kok[i] && (m < p.M);
      float4 a = xa[i][m][0], b = xa[i][m][1];
      if constexpr (XP) {
        // the partial sums in slice order, their sum added to the row
        float4 ta = make_float4(0.f, 0.f, 0.f, 0.f), tb = ta;
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) {
          const float4 qa = pa[i][m][sl][0], qb = pa[i][m][sl][1];
          ta.x += qa.x; ta.y += qa.y; ta.z += qa.z; ta.w += qa.w;
          tb.x += qb.x; tb.y += qb.y; tb.z += qb.z; tb.w += qb.w;
        }
        a.x += ta.x; a.y += ta.y; a.z += ta.z; a.w += ta.w;
        b.x += tb.x; b.y += tb.y; b.z += tb.z; b.w += tb.w;
        if (blockIdx.x == 0 && ok) {
          float* xo = p.xout + (size_t)m * p.ldx + kofs[i];
          *(float4*)xo = a;
          *(float4*)(xo + 4) = b;
        }
      }
      xr[i][m][0] = ok ? a.x : 0.f; xr[i][m][1] = ok ? a.y : 0.f;
      xr[i][m][2] = ok ? a.z : 0.f; xr[i][m][3] = ok ? a.w : 0.f;
      xr[i][m][4] = ok ? b.x : 0.f; xr[i][m][5] = ok ? b.y : 0.f;
      xr[i][m][6] = ok ? b.z : 0.f; xr[i][m][7] = ok ? b.w : 0.f;
    }
  }
  if constexpr (NORM) {
    // RMSNorm of the activation rows: the gain multiplies the registers now;
    // the row factor needs every wave's sum of squares and is applied to the
    // finished sums (reduce_group), so no barrier sits in front of the loop
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < SPW; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += xr[i][m][e] * xr[i][m][e];
      ss = wave_sum(ss);
      if (lane == 0) ssq[w][m] = ss;
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const float g[8] = {ga[i][0].x, ga[i][0].y, ga[i][0].z, ga[i][0].w,
                          ga[i][1].x, ga[i][1].y, ga[i][1].z, ga[i][1].w};
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) xr[i][m][e] *= g[e];
    }
  }
  // the rotary values reach LDS before the first group's reduction barrier
  if constexpr (EPI == EPI_QKV) qpre.store(p, &qst);

  for (; rg < ngroups; rg += gridDim.x) {
    // Each weight register is refilled with the next row group's weights as
    // soon as its current contents are consumed, so those loads are in flight
    // during the rest of this group's products, its reduction and epilogue.
    const int nx = rg + gridDim.x;
    const bool more = nx < ngroups;
    size_t rnext[YT];
#pragma unroll
    for (int y = 0; y < YT; ++y) {
      const int r = gemm_row<EPI>(p, more ? nx : rg, y);
      rnext[y] = (size_t)(r < p.N ? r : 0) * p.K;
    }
    // the residual values this group adds to, requested before the products
    // so that the epilogue does not wait for them (with the above: O at 4
    // rows 9.9 -> 9.3 us)
    float rpre = 0.f;
    if constexpr (EPI == EPI_RESID) {
      if (threadIdx.x < YT * MT) {
        const int y = threadIdx.x / MT, mm = threadIdx.x % MT;
        const int n = gemm_row<EPI>(p, rg, y);
        if (mm < p.M && n < p.N) rpre = p.out[(size_t)mm * p.ldo + n];
      }
    }
    float acc[NVP];
#pragma unroll
    for (int i = 0; i < NVP; ++i) acc[i] = 0.f;
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
      for (int y = 0; y < YT; ++y) {
        float wf[8];
        wr[i][y].widen(wf);
        if (more) wr[i][y].load(W, rnext[y] + kofs[i]);
        fma_rows<MT>(acc, wf, xr[i], y);
      }
    if constexpr (NORM)
      reduce_group<MT, true>(acc, lane, w, NW, red, tot, ssq, 1.0f / (float)p.K, p.eps);
    else
      reduce_group<MT, true>(acc, lane, w, NW, red, tot);
    if constexpr (EPI == EPI_RESID) {
      if (threadIdx.x < YT * MT) {
        const int y = threadIdx.x / MT, mm = threadIdx.x % MT;
        const int n = gemm_row<EPI>(p, rg, y);
        if (mm < p.M && n < p.N) p.out[(size_t)mm * p.ldo + n] = rpre + tot[threadIdx.x];
      }
      continue;
    }
    if constexpr (EPI == EPI_QKV) epilogue<MT, EPI>(p, rg, tot, &qst);
    else epilogue<MT, EPI>(p, rg, tot);
  }
}

// ---------------------------------------------------------------- matrix cores
// The same k-stationary scheme on the 4x4x4 bf16 matrix instruction with 16
// blocks (v_mfma_f32_4x4x4_16b_bf16).  Lane l = 4*blk + r: in each 128-k chunk,
// block blk covers k = 8*blk .. 8*blk+7.  For the weights (A operand) lane l
// holds row r of a 4-row set at those 8 k (one 16-byte load; a wave reads 4
// rows x 256 contiguous bytes); for the activations (B operand) it holds
// activation row r (4*mg + r for the second set of 4 rows) at the same k,
// split into bf16 hi + lo so the fp32 activations keep ~2^-16 relative
// accuracy.  Each instruction accumulates a 4x4 (weight row x activation row)
// tile per block; the 16 blocks' tiles are summed across lanes at the end of
// a row group.  Against the vector-ALU kernel this removes the widening of
// the weights and three quarters of the multiply-add issue, which is what
// makes the cost of a group grow with M there.
template <int MT, int EPI, bool NORM, int CPW, bool SPLIT, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void gemm_mfma_kernel(GemmParams p) {
  constexpr int MG = (MT + 3) / 4;  // sets of 4 activation rows
  constexpr int RG = YT / 4;        // sets of 4 weight rows per group
  constexpr int NV = YT * MT;
  static_assert(!SPLIT || (!NORM && EPI == EPI_RESID), "K is split only for residual GEMMs");
  __shared__ float red[NW][YT][4 * MG];
  __shared__ float tot[64];
  __shared__ float ssq[NW][4 * MG];
  __shared__ QkvStage<(EPI == EPI_QKV) ? MT : 1> qst;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 3, blk = lane >> 2;
  const uint16_t* __restrict__ W = (const uint16_t*)p.W;
  // SPLIT: workgroup row blockIdx.y takes K slice blockIdx.y of GEMM_KSPLIT
  // equal slices and writes its partial sums to p.part
  const int kext = SPLIT ? p.K / GEMM_KSPLIT : p.K;
  const int kbase = SPLIT ? (int)blockIdx.y * kext : 0;
  const int nch = kext >> 7;
  // chunks w, w+4, ... of 128 k; a chunk past the range is read at its first
  // chunk (in bounds) and multiplied by zero activations
  int kofs[CPW];
  bool cok[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int c = w + NW * i;
    cok[i] = c < nch;
    kofs[i] = kbase + (cok[i] ? c : 0) * 128 + 8 * blk;
  }
  const int ngroups = gemm_groups<EPI>(p);
  const int G = gridDim.x;
  auto row_off = [&](int g_, int a) {
    const int row = gemm_row<EPI>(p, g_, 4 * a + r);
    return (size_t)(row < p.N ? row : 0) * p.K;
  };
  // the first group's weights (requested after the activation loads below);
  // a workgroup with no group reads the head of row 0 and never uses it
  u32x4 wr[RG][CPW];
  int rg = blockIdx.x;
  auto first_group = [&]() {
#pragma unroll
    for (int a = 0; a < RG; ++a) {
      const size_t ro = rg < ngroups ? row_off(rg, a) : 0;
#pragma unroll
      for (int i = 0; i < CPW; ++i) wr[a][i] = __builtin_nontemporal_load((const u32x4*)(W + ro + kofs[i]));
    }
  };

  // the rows' positions first (QKV): the rotary loads that need them are
  // issued after the weights (see QkvPre)
  QkvPre<MT, 64 * NW> qpre;
  if constexpr (EPI == EPI_QKV) qpre.pos(p);
  // activations (times the norm gain), split into bf16 hi + lo
  shortx4 xh[CPW][MG][2], xl[CPW][MG][2];
  float ss[MG];
#pragma unroll
  for (int mg = 0; mg < MG; ++mg) ss[mg] = 0.f;
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    float g[8];
    if constexpr (NORM) {
      const float4 ga = *(const float4*)(p.norm_g + kofs[i]);
      const float4 gb = *(const float4*)(p.norm_g + kofs[i] + 4);
      g[0] = ga.x; g[1] = ga.y; g[2] = ga.z; g[3] = ga.w; g[4] = gb.x; g[5] = gb.y; g[6] = gb.z; g[7] = gb.w;
    }
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
      const int m = 4 * mg + r;
      const bool ok = cok[i] && m < p.M;
      const float* xs = p.X + (size_t)(m < p.M ? m : 0) * p.ldx + kofs[i];
      const float4 x0 = *(const float4*)xs, x1 = *(const float4*)(xs + 4);
      float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xv[e] = ok ? xv[e] : 0.f;
        if constexpr (NORM) {
          ss[mg] += xv[e] * xv[e];
          xv[e] *= g[e];
        }
        short hi, lo;
        split_bf16(xv[e], hi, lo);
        xh[i][mg][e >> 2][e & 3] = hi;
        xl[i][mg][e >> 2][e & 3] = lo;
      }
    }
  }
  // the first group's weights follow the activation loads, which would
  // otherwise queue behind them (gate/up at 4 rows: 38.5 -> 37.9 us)
  first_group();
  if constexpr (EPI == EPI_QKV) {
    qpre.rope(p);
    qpre.store(p, &qst);  // read after the first group's reduction barrier
  }
  if constexpr (NORM) {
    // per-wave sums of x^2 of each activation row (lanes with the same r)
#pragma unroll
    for (int mg = 0; mg < MG; ++mg) {
      float t = ss[mg];
      t += __shfl_xor(t, 4, 64);
      t += __shfl_xor(t, 8, 64);
      t += __shfl_xor(t, 16, 64);
      t += __shfl_xor(t, 32, 64);
      if (blk == 0) ssq[w][4 * mg + r] = t;
    }
  }

  for (; rg < ngroups; rg += G) {
    // the weight registers are refilled with the next group's rows as soon
    // as the products have read them; a workgroup without a next group reads
    // the head of row 0 again (in bounds, cached, never used)
    const int nx = rg + G;
    size_t rn[RG];
#pragma unroll
    for (int a = 0; a < RG; ++a) rn[a] = nx < ngroups ? row_off(nx, a) : 0;
    floatx4 acc[RG][MG];
#pragma unroll
    for (int a = 0; a < RG; ++a)
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) acc[a][mg] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int a = 0; a < RG; ++a)
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const u32x4 v = wr[a][i];
        const shortx4 w0 = __builtin_bit_cast(shortx4, u32x2{v.x, v.y});
        const shortx4 w1 = __builtin_bit_cast(shortx4, u32x2{v.z, v.w});
        wr[a][i] = __builtin_nontemporal_load((const u32x4*)(W + rn[a] + kofs[i]));
#pragma unroll
        for (int mg = 0; mg < MG; ++mg) {
          acc[a][mg] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(w0, xh[i][mg][0], acc[a][mg], 0, 0, 0);
          acc[a][mg] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(w0, xl[i][mg][0], acc[a][mg], 0, 0, 0);
          acc[a][mg] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(w1, xh[i][mg][1], acc[a][mg], 0, 0, 0);
          acc[a][mg] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(w1, xl[i][mg][1], acc[a][mg], 0, 0, 0);
        }
      }
    // lane (blk, r) holds rows 4a + v (v = 0..3) x activation row 4mg + r of
    // its block; sum the 16 blocks: halving over lane bits 5 and 4 (which
    // also spreads the 4 rows over the lanes), plain adds over bits 3 and 2
#pragma unroll
    for (int a = 0; a < RG; ++a)
#pragma unroll
      for (int mg = 0; mg < MG; ++mg) {
        const float v0 = acc[a][mg][0], v1 = acc[a][mg][1], v2 = acc[a][mg][2], v3 = acc[a][mg][3];
        const bool u5 = (lane & 32) != 0;
        float k0 = u5 ? v2 : v0, k1 = u5 ? v3 : v1;
        const float s0 = u5 ? v0 : v2, s1 = u5 ? v1 : v3;
        k0 += __shfl_xor(s0, 32, 64);
        k1 += __shfl_xor(s1, 32, 64);
        const bool u4 = (lane & 16) != 0;
        float kk = u4 ? k1 : k0;
        const float sk = u4 ? k0 : k1;
        kk += __shfl_xor(sk, 16, 64);
        kk += __shfl_xor(kk, 8, 64);
        kk += __shfl_xor(kk, 4, 64);
        if ((lane & 12) == 0) red[w][4 * a + ((lane >> 4) & 3)][4 * mg + r] = kk;
      }
    lds_barrier();
    if (threadIdx.x < NV) {
      const int y = threadIdx.x / MT, m = threadIdx.x % MT;
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) t += red[i][y][m];
      if constexpr (NORM) {
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) q += ssq[i][m];
        t *= 1.0f / sqrtf(q / (float)p.K + p.eps);
      }
      tot[threadIdx.x] = t;
    }
    lds_barrier();
    if constexpr (SPLIT) {
      if (threadIdx.x < NV) {
        const int y = threadIdx.x / MT, m = threadIdx.x % MT;
        const int n = gemm_row<EPI>(p, rg, y);
        if (m < p.M && n < p.N) p.part[((size_t)blockIdx.y * 8 + m) * p.ldo + n] = tot[threadIdx.x];
      }
    } else if constexpr (EPI == EPI_QKV) {
      epilogue<MT, EPI>(p, rg, tot, &qst);
    } else {
      epilogue<MT, EPI>(p, rg, tot);
    }
  }
}

// out[m][n] += sum over the K slices of the split partials, slice order fixed
__global__ __launch_bounds__(256) void gemm_split_reduce_kernel(GemmParams p) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= p.M * p.N) return;
  const int m = e / p.N, n = e % p.N;
  float t = 0.f;
#pragma unroll
  for (int sl = 0; sl < GEMM_KSPLIT; ++sl) t += p.part[((size_t)sl * 8 + m) * p.ldo + n];
  p.out[(size_t)m * p.ldo + n] += t;
}

// ---------------------------------------------------------------- streaming
template <int MT, typename WT, int EPI>
__global__ __launch_bounds__(64 * STREAM_WAVES) void gemm_stream_kernel(GemmParams p) {
  constexpr int NVP = MaxPow2<MT>::v;
  __shared__ float red[STREAM_WAVES][NVP];
  __shared__ float tot[NVP];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int rg = blockIdx.x;
  const WT* __restrict__ W = (const WT*)p.W;
  int rows[YT];
#pragma unroll
  for (int y = 0; y < YT; ++y) {
    const int r = gemm_row<EPI>(p, rg, y);
    rows[y] = r < p.N ? r : 0;
  }
  float acc[NVP];
#pragma unroll
  for (int i = 0; i < NVP; ++i) acc[i] = 0.f;
  const int nsteps = (p.K + 511) >> 9;
  for (int s = w; s < nsteps; s += STREAM_WAVES) {
    const int kraw = s * 512 + lane * 8;
    const bool kok = kraw < p.K;  // only the last step can be partial
    const int k0 = kok ? kraw : 0;
    float wv[YT][8];
#pragma unroll
    for (int y = 0; y < YT; ++y) load_w8<WT>(W, (size_t)rows[y] * p.K + k0, wv[y]);
    float xv[MT][8];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const bool ok = kok && (m < p.M);
      const float* xs = p.X + (size_t)(m < p.M ? m : 0) * p.ldx + k0;
      const float4 a = *(const float4*)xs;
      const float4 b = *(const float4*)(xs + 4);
      xv[m][0] = ok ? a.x : 0.f; xv[m][1] = ok ? a.y : 0.f;
      xv[m][2] = ok ? a.z : 0.f; xv[m][3] = ok ? a.w : 0.f;
      xv[m][4] = ok ? b.x : 0.f; xv[m][5] = ok ? b.y : 0.f;
      xv[m][6] = ok ? b.z : 0.f; xv[m][7] = ok ? b.w : 0.f;
    }
#pragma unroll
    for (int y = 0; y < YT; ++y) fma_rows<MT>(acc, wv[y], xv, y);
  }
  reduce_group<MT>(acc, lane, w, STREAM_WAVES, red, tot);
  epilogue<MT, EPI>(p, rg, tot);
}

// ---------------------------------------------------------------- launch
int device_cus() {
  static int ncu = 0;
  if (!ncu) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
      ncu = 256;
  }
  return ncu;
}

bool gemm_is_kstat(int K) { return K <= KSTAT_WAVES * KSTAT_SPW * 512; }

// Matrix cores or vector ALUs for an M-row launch.  Measured on the 8B layer
// shapes (back-to-back launches): the matrix-core kernel is flat in M (gate/up
// 38.9 / 39.4 / 41.0 us at M = 1 / 2 / 4, 63 us at M = 8 against 73 for the
// vector kernel) but slower on small matrices and at M <= 2 (QKV 18.8 vs
// 16.9 us and O 12.2 vs 10.7 us at M = 4), where its activation prologue is
// not amortised.  So: matrix cores from M = 5 on, and from M = 3 on for
// matrices of at least 64 Mi weights (gate/up, LM head).  At 5-8 rows they
// beat the 32-row tiles on every projection (6 rows: gate/up 45.3 against
// 53.6 us, LM head 182 against 194, QKV 20.5 against 24.5).
bool gemm_use_mfma(const GemmParams& p, int rows) {
  if (p.wdtype != 1 || (p.K & 127) || p.K > KSTAT_WAVES * 8 * 128) return false;
  const double elems = (double)(p.epi == EPI_SWIGLU ? 2 * p.F : p.N) * p.K;
  return rows >= 5 || (rows >= 3 && elems >= 64.0 * 1024 * 1024);
}

template <int MT, int EPI, int CPW, int NW>
static void launch_mfma_cpw(const GemmParams& p, int grid, hipStream_t s) {
  if (p.norm_g) gemm_mfma_kernel<MT, EPI, true, CPW, false, NW><<<grid, 64 * NW, 0, s>>>(p);
  else gemm_mfma_kernel<MT, EPI, false, CPW, false, NW><<<grid, 64 * NW, 0, s>>>(p);
}

// A residual GEMM over a long K (the down projection) at M >= 3: the
// streaming kernel re-reads the activation rows for every row group, and at
// 4 rows that traffic equals the weight traffic.  Instead GEMM_KSPLIT slices
// of K, each held in registers by the matrix-core kernel (8 waves of 7
// chunks of 128 for K = 14336), write partial sums, and their sum is added
// to the residual in slice order: by the small reduce kernel, or, with
// defer_reduce, by the prologue of the next GEMM that reads the residual
// rows (xpart).
bool gemm_use_split(const GemmParams& p) {
  if (!p.part || p.part_floats < (size_t)GEMM_KSPLIT * 8 * p.ldo || p.epi != EPI_RESID || p.norm_g || p.wdtype != 1 || p.M < 3) return false;
  if (p.K <= KSTAT_WAVES * 8 * 128 || p.K % (GEMM_KSPLIT * 128)) return false;
  return p.K / GEMM_KSPLIT <= SPLIT_WAVES * 8 * 128;
}

bool gemm_takes_xpart(const GemmParams& p) {
  // the k-stationary kernel with a fused norm, one launch of at most 4 rows
  return p.epi == EPI_QKV && p.norm_g && p.M >= 1 && p.M <= 4 && !gemm_tiled_ok(p) &&
         !gemm_use_mfma(p, p.M) && gemm_is_kstat(p.K) && p.K % 512 == 0;
}

template <int MT>
static hipError_t launch_split(const GemmParams& p, hipStream_t s) {
  const int groups = gemm_groups<EPI_RESID>(p);
  const int slots = device_cus() / GEMM_KSPLIT;  // one 8-wave workgroup per CU
  const int rounds = (groups + slots - 1) / slots;
  const dim3 grid((groups + rounds - 1) / rounds, GEMM_KSPLIT);
  const int cpw = ((p.K / GEMM_KSPLIT >> 7) + SPLIT_WAVES - 1) / SPLIT_WAVES;
  if (cpw <= 4) gemm_mfma_kernel<MT, EPI_RESID, false, 4, true, SPLIT_WAVES><<<grid, 64 * SPLIT_WAVES, 0, s>>>(p);
  else if (cpw <= 7) gemm_mfma_kernel<MT, EPI_RESID, false, 7, true, SPLIT_WAVES><<<grid, 64 * SPLIT_WAVES, 0, s>>>(p);
  else gemm_mfma_kernel<MT, EPI_RESID, false, 8, true, SPLIT_WAVES><<<grid, 64 * SPLIT_WAVES, 0, s>>>(p);
  if (!p.defer_reduce) gemm_split_reduce_kernel<<<(p.M * p.N + 255) / 256, 256, 0, s>>>(p);
  return hipGetLastError();
}

template <int MT, int EPI>
static hipError_t launch_mte(const GemmParams& p, hipStream_t s) {
  const int groups = gemm_groups<EPI>(p);
  // persistent workgroups, at most two per CU, each looping over row
  // groups; the grid is sized so that every workgroup gets the same number
  // of groups (up to one), which keeps the last round from running on a
  // fraction of the chip
  const int slots = 2 * device_cus();
  const int rounds = (groups + slots - 1) / slots;
  const int grid = (groups + rounds - 1) / rounds;
  if constexpr (EPI == EPI_RESID) {
    if (gemm_use_split(p)) return launch_split<MT>(p, s);
  }
  if (gemm_use_mfma(p, p.M)) {
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_STORE || EPI == EPI_QKV) {
      // the two largest weight streams take 8 waves of 4 chunks: gate/up
      // with one workgroup per CU (39.6 -> 38.2 us at 4 rows), the LM head
      // with three (171.6 -> 166 us); QKV (here from 5 rows on) like gate/up:
      // 20.5 us at 6 rows against 33.9 with 4 waves and 24.5 on the 32-row
      // tiles
      if (p.K <= 8 * 4 * 128) {
        const int slots8 = (EPI == EPI_STORE ? 3 : 1) * device_cus();
        const int rounds8 = (groups + slots8 - 1) / slots8;
        launch_mfma_cpw<MT, EPI, 4, 8>(p, (groups + rounds8 - 1) / rounds8, s);
        return hipGetLastError();
      }
    }
    const int cpw = ((p.K >> 7) + KSTAT_WAVES - 1) / KSTAT_WAVES;
    if (cpw <= 2) launch_mfma_cpw<MT, EPI, 2, KSTAT_WAVES>(p, grid, s);
    else if (cpw <= 4) launch_mfma_cpw<MT, EPI, 4, KSTAT_WAVES>(p, grid, s);
    else launch_mfma_cpw<MT, EPI, 8, KSTAT_WAVES>(p, grid, s);
  } else if (gemm_is_kstat(p.K)) {
    if constexpr (EPI == EPI_QKV || EPI == EPI_RESID) {
      // the smaller projections (QKV, O) ramp up faster with 8 waves of one K
      // step each: twice the workgroup's loads in flight from its start.
      // Measured on the 8B layers at 1-4 rows: QKV 16.8 -> 14.4 us with one
      // workgroup per CU, O 10.8 -> 9.8 us with two.
      const int slots = (EPI == EPI_QKV ? 1 : 2) * device_cus();
      const int rounds8 = (groups + slots - 1) / slots;
      const int grid8 = (groups + rounds8 - 1) / rounds8;
      const bool xp = EPI == EPI_QKV && p.xpart;
      if (p.wdtype == 1) {
        if (xp) gemm_kstat_kernel<MT, uint16_t, EPI, true, 8, EPI == EPI_QKV><<<grid8, 64 * 8, 0, s>>>(p);
        else if (p.norm_g) gemm_kstat_kernel<MT, uint16_t, EPI, true, 8><<<grid8, 64 * 8, 0, s>>>(p);
        else gemm_kstat_kernel<MT, uint16_t, EPI, false, 8><<<grid8, 64 * 8, 0, s>>>(p);
      } else {
        if (xp) gemm_kstat_kernel<MT, float, EPI, true, 8, EPI == EPI_QKV><<<grid8, 64 * 8, 0, s>>>(p);
        else if (p.norm_g) gemm_kstat_kernel<MT, float, EPI, true, 8><<<grid8, 64 * 8, 0, s>>>(p);
        else gemm_kstat_kernel<MT, float, EPI, false, 8><<<grid8, 64 * 8, 0, s>>>(p);
      }
    } else if (p.wdtype == 1) {
      if (p.norm_g) gemm_kstat_kernel<MT, uint16_t, EPI, true, KSTAT_WAVES><<<grid, 64 * KSTAT_WAVES, 0, s>>>(p);
      else gemm_kstat_kernel<MT, uint16_t, EPI, false, KSTAT_WAVES><<<grid, 64 * KSTAT_WAVES, 0, s>>>(p);
    } else {
      if (p.norm_g) gemm_kstat_kernel<MT, float, EPI, true, KSTAT_WAVES><<<grid, 64 * KSTAT_WAVES, 0, s>>>(p);
      else gemm_kstat_kernel<MT, float, EPI, false, KSTAT_WAVES><<<grid, 64 * KSTAT_WAVES, 0, s>>>(p);
    }
  } else {
    if (p.norm_g) return hipErrorInvalidValue;  // a fused norm needs whole rows per workgroup
    if (p.wdtype == 1)
      gemm_stream_kernel<MT, uint16_t, EPI><<<groups, 64 * STREAM_WAVES, 0, s>>>(p);
    else
      gemm_stream_kernel<MT, float, EPI><<<groups, 64 * STREAM_WAVES, 0, s>>>(p);
  }
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_mt(const GemmParams& p, hipStream_t s) {
  switch (p.epi) {
    case EPI_STORE: return launch_mte<MT, EPI_STORE>(p, s);
    case EPI_RESID: return launch_mte<MT, EPI_RESID>(p, s);
    case EPI_SWIGLU: return launch_mte<MT, EPI_SWIGLU>(p, s);
    default: return launch_mte<MT, EPI_QKV>(p, s);
  }
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  if (p.xpart && !gemm_takes_xpart(p)) return hipErrorInvalidValue;
  // planes written by the producer serve only the tiled kernels, and a fused
  // norm needs their sums of squares as well; a finish that prepares the next
  // launch's planes exists only for K-split residual launches
  if ((p.xs_ready && ((p.norm_g && !p.ssq_ready) || !gemm_tiled_ok(p))) ||
      (p.xs_out && (p.epi != EPI_SWIGLU || !gemm_tiled_ok(p))) ||
      (p.norm_next && (!p.xs_next || !gemm_finish_prepares(p))))
    return hipErrorInvalidValue;
  if (gemm_tiled_ok(p)) return launch_gemm_tiled(p, s);
  if (p.M <= 1) return launch_mt<1>(p, s);
  if (p.M <= 2) return launch_mt<2>(p, s);
  if (p.M <= 4) return launch_mt<4>(p, s);
  return launch_mt<8>(p, s);
}

}  // namespace sv
