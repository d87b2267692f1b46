// Tiled GEMM for many activation rows (5 or more for the QKV, gate/up and LM
// head projections, more than 8 for the residual ones):
// Y[m][n] = sum_k X[m][k] W[n][k]
// on the 16x16x32 bf16 matrix instruction, with the fp32 activations split
// into bf16 hi + lo (two products per tile) so they keep ~2^-16 relative
// accuracy, fp32 accumulation.  This is the regime where the skinny kernels
// run out of vector or matrix throughput, or stream the weights once per 8
// rows: the 32-row verify window of 8
// sequences, 117-row token trees, 128-row long-context batches.
//
// A first kernel splits the activation rows into bf16 hi and lo planes (times
// the RMSNorm gain, with each row's sum of squares); the tiled kernel then
// streams 64-k stages of weight rows and both planes through registers (three
// stages ahead of the products, no conversion inside the loop) into two LDS
// buffers.
//
// Output columns come in pairs (a, b) so that every epilogue has both of its
// operands in one lane:
//   STORE / RESID  tile t of NP pairs covers rows [2NP t, 2NP t + 2NP):
//                  a = 2NP t + j, b = a + NP
//   SWIGLU         pair f: a = gate row f, b = up row F + f
//   QKV            pair (head h, i < D/2): a = h D + i, b = a + D/2
//
// A workgroup (4 waves) owns BM = 32*MB activation rows and NP = 32 pairs
// (64 weight rows).  Wave w computes 32 rows x 16*PBW pairs over the k
// sub-steps kw, kw+KW, ... of every 64-k stage; the KW partial blocks are
// added in LDS at the end.  The RMSNorm row factor scales the finished sums.
//
// Few output tiles (the QKV, O and down projections at small M) would leave
// most of the chip idle; those launches split K over S workgroups, which
// write raw partial sums that a third kernel adds in a fixed order before
// applying the epilogue.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace sv {

namespace {

constexpr int TK = 64;       // k per stage
constexpr int NPAIR = 32;    // pairs per tile
constexpr int WROWS = 2 * NPAIR;

template <int EPI>
DEVI int pair_rows(const GemmParams& p, int j, int& rb) {
  if (EPI == EPI_SWIGLU) {
    rb = p.F + j;
    return j;
  }
  if (EPI == EPI_QKV) {
    const int half = p.D / 2;
    const int a = (j / half) * p.D + (j % half);
    rb = a + half;
    return a;
  }
  const int a = (j / NPAIR) * WROWS + (j % NPAIR);
  rb = a + NPAIR;
  return a;
}

template <int EPI>
__host__ __device__ int pair_count(const GemmParams& p) {
  if (EPI == EPI_SWIGLU) return p.F;
  if (EPI == EPI_QKV) return p.N / 2;
  return ((p.N + WROWS - 1) / WROWS) * NPAIR;
}

// Epilogue of one (row m, pair j) with its two finished sums.
template <int EPI>
DEVI void epilogue_pair(const GemmParams& p, int m, int j, float a, float b) {
  int rb;
  const int ra = pair_rows<EPI>(p, j, rb);
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    float* o = p.out + (size_t)m * p.ldo;
    if (EPI == EPI_STORE) {
      if (ra < p.N) o[ra] = a;
      if (rb < p.N) o[rb] = b;
    } else {
      if (ra < p.N) o[ra] += a;
      if (rb < p.N) o[rb] += b;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    p.out[(size_t)m * p.ldo + j] = a / (1.0f + expf(-a)) * b;
  } else {
    const int D = p.D, half = D / 2;
    const int hh = ra / D, i = ra % D;
    const int mg = p.m0 + m;
    const int bseq = p.seq ? p.seq[mg] : mg / p.T;
    const int sl = p.slot[mg];
    if (hh < p.Hq + p.Hkv) {
      const int ps = p.pos[mg];
      const float c = p.rope_cos[(size_t)ps * half + i], s = p.rope_sin[(size_t)ps * half + i];
      const float x0 = a * c - b * s, x1 = b * c + a * s;
      if (hh < p.Hq) {
        float* q = p.q_out + ((size_t)mg * p.Hq + hh) * D;
        q[i] = x0;
        q[i + half] = x1;
      } else {
        const int hk = hh - p.Hq;
        float* k = p.k_out + ((size_t)mg * p.Hkv + hk) * D;
        k[i] = x0;
        k[i + half] = x1;
        if (sl >= 0) {
          uint16_t* kc = p.kcache + kv_k_off(p.kvm, p.Hkv, D, bseq, hk, sl);
          kc[i] = (uint16_t)f32_to_bf16_rne(x0);
          kc[i + half] = (uint16_t)f32_to_bf16_rne(x1);
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

// Activations for the tiled kernel: X (fp32, times the RMSNorm gain when
// NORM) split into bf16 hi and lo planes [2][M][K], and each row's sum of
// squares in SSQ_BLK partial sums (one per 1024 k, added in a fixed order by
// row_factor).  One workgroup per (1024 k, row), one float4 per thread, so
// the whole pass costs one memory latency.
template <bool NORM>
__global__ __launch_bounds__(256) void gemm_split_x_kernel(GemmParams p) {
  const int blk = blockIdx.x, m = blockIdx.y;
  const float* x = p.X + (size_t)m * p.ldx;
  uint16_t* hi = p.xs + (size_t)m * p.K;
  uint16_t* lo = hi + (size_t)p.M * p.K;
  float ss = 0.f;
  const int k = blk * 1024 + 4 * threadIdx.x;
  if (k < p.K) {
    const float4 v = *(const float4*)(x + k);
    float xv[4] = {v.x, v.y, v.z, v.w};
    if (NORM) {
      const float4 g = *(const float4*)(p.norm_g + k);
      const float gv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        ss += xv[c] * xv[c];
        xv[c] *= gv[c];
      }
    }
    shortx4 h4, l4;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      short h, l;
      split_bf16(xv[c], h, l);
      h4[c] = h;
      l4[c] = l;
    }
    *(shortx4*)(hi + k) = h4;
    *(shortx4*)(lo + k) = l4;
  }
  if (NORM) {
    __shared__ float red[4];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) p.xs_ssq[m * SSQ_BLK + blk] = red[0] + red[1] + red[2] + red[3];
  }
}

// RMSNorm factor of activation row m from its partial sums of squares
DEVI float row_factor(const GemmParams& p, int m) {
  const int nblk = (p.K + 1023) / 1024;
  float q = 0.f;
  for (int b = 0; b < nblk; ++b) q += p.xs_ssq[m * SSQ_BLK + b];
  return 1.0f / sqrtf(q / (float)p.K + p.eps);
}

// LDS tile rows are 128 bytes (64 bf16 of k) in eight 16-byte chunks; chunk
// c of row r is stored in slot c ^ (r & 7), so the 16 rows one matrix
// operand read touches fall in different banks.
DEVI int swz(int r, int c) { return c ^ (r & 7); }

// MB row blocks of 32, KW k-groups; PBW pair blocks of 16 per wave.  Every
// thread moves a fixed set of 16-byte chunks of each stage (weight rows and
// both activation planes); a stage's chunks are requested R stages before
// they are multiplied, into a ring of R register sets, and written to one of
// two LDS buffers the stage before.
template <int MB, int KW, int R, int EPI, bool NORM, bool SPLIT>
__global__ __launch_bounds__(256, 1) void gemm_tiled_kernel(GemmParams p) {
  constexpr int NPB = NPAIR / 16;
  constexpr int PBW = MB * NPB * KW / 4;
  static_assert(PBW >= 1 && MB * (NPB / PBW) * KW == 4, "four waves");
  static_assert(KW == 1 || KW == 2, "a 64-k stage holds two 32-k steps");
  constexpr int BM = 32 * MB;
  constexpr int ROWS = WROWS + 2 * BM;  // tile rows per stage: W, X hi, X lo
  constexpr int CH = ROWS * 8 / 256;    // 16-byte chunks per thread per stage
  static_assert(CH * 256 == ROWS * 8, "chunks split evenly over the threads");
  static_assert(WROWS % 8 == 0 && BM % 8 == 0, "planes start on a swizzle period");
  static_assert(R == 3, "the loop below is unrolled for a ring of three");
  __shared__ __attribute__((aligned(16))) uint16_t s_t[2][ROWS * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int kw = w % KW, pbw = (w / KW) % (NPB / PBW), mb = w / (KW * (NPB / PBW));
  const int l16 = lane & 15, lg = lane >> 4;
  const int p0 = blockIdx.x * NPAIR;
  const int m0 = blockIdx.y * BM;
  const int npairs = pair_count<EPI>(p);
  const int kext = SPLIT ? p.K / (int)gridDim.z : p.K;
  const int kbeg = SPLIT ? (int)blockIdx.z * kext : 0;
  const int nst = kext / TK;

  // chunk i of this thread: stage row (tid + 256 i) / 8, 16-byte chunk
  // (tid + 256 i) % 8 of its 64 k; stored at slot swz(row, chunk)
  const uint16_t* src[CH];
  int dst[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int idx = tid + 256 * i;
    const int r = idx / 8, q = idx % 8;
    dst[i] = r * 64 + 8 * swz(r, q);
    if (r < WROWS) {
      const int j = p0 + (r % NPAIR);
      int rb;
      const int ra = pair_rows<EPI>(p, j < npairs ? j : 0, rb);
      int row = r < NPAIR ? ra : rb;
      row = (j < npairs && row < p.N) ? row : 0;
      src[i] = (const uint16_t*)p.W + (size_t)row * p.K + kbeg + 8 * q;
    } else {
      const int rx = r - WROWS;
      const int plane = rx / BM, ml = rx % BM;
      const int m = (m0 + ml < p.M) ? m0 + ml : p.M - 1;  // rows past M: any valid row, never stored
      src[i] = p.xs + ((size_t)plane * p.M + m) * p.K + kbeg + 8 * q;
    }
  }
  u32x4 ring[R][CH];
  auto fetch = [&](int st, auto sl) {
    constexpr int S = decltype(sl)::value;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const u32x4* g = (const u32x4*)(src[i] + st * TK);
      // the first WROWS*8 chunks of a stage are weights (streamed once,
      // non-temporal); the rest are the activation planes (re-read from L2)
      if (256 * i < WROWS * 8) ring[S][i] = __builtin_nontemporal_load(g);
      else ring[S][i] = *g;
    }
  };
  auto put = [&](auto sl, auto bf) {
    constexpr int S = decltype(sl)::value, B = decltype(bf)::value;
#pragma unroll
    for (int i = 0; i < CH; ++i) *(u32x4*)(&s_t[B][dst[i]]) = ring[S][i];
  };

  floatx4 acc[2][PBW][2];  // [row tile][pair block][a, b]
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int q = 0; q < PBW; ++q) acc[mt][q][0] = acc[mt][q][1] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto mult = [&](auto bf) {
    constexpr int B = decltype(bf)::value;
    const uint16_t* tw = s_t[B];
    const uint16_t* th = tw + WROWS * 64;
    const uint16_t* tl = th + BM * 64;
    // k-steps of 32 (the 16x16x32 instruction): lane group lg takes the
    // stage's 16-byte chunk 4 * step + lg of every row it reads
#pragma unroll
    for (int ss = 0; ss < 2 / KW; ++ss) {
      const int c = 4 * (kw + KW * ss) + lg;
      shortx8 ah[2], al[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int r = 32 * mb + 16 * mt + l16;
        ah[mt] = *(const shortx8*)(th + r * 64 + 8 * swz(r, c));
        al[mt] = *(const shortx8*)(tl + r * 64 + 8 * swz(r, c));
      }
#pragma unroll
      for (int q = 0; q < PBW; ++q) {
        const int ra = 16 * (pbw * PBW + q) + l16, rb = NPAIR + ra;
        const shortx8 ba = *(const shortx8*)(tw + ra * 64 + 8 * swz(ra, c));
        const shortx8 bb = *(const shortx8*)(tw + rb * 64 + 8 * swz(rb, c));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          acc[mt][q][0] = mfma16x16x32(ah[mt], ba, acc[mt][q][0]);
          acc[mt][q][0] = mfma16x16x32(al[mt], ba, acc[mt][q][0]);
          acc[mt][q][1] = mfma16x16x32(ah[mt], bb, acc[mt][q][1]);
          acc[mt][q][1] = mfma16x16x32(al[mt], bb, acc[mt][q][1]);
        }
      }
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  // stage st: ring slot st % 3, LDS buffer st % 2.  Step st requests stage
  // st + 3 into the slot stage st used, multiplies stage st, writes stage
  // st + 1 to the other buffer; one barrier per stage.  In the main loop the
  // steps are branch-free (a request past the last stage re-reads the last
  // stage, a write past it fills a buffer nobody reads), which lets the
  // compiler count the outstanding loads exactly.
  auto step = [&](int st, auto sl, auto bf, auto sl1, auto bf1) {
    fetch(min(st + R, nst - 1), sl);
    mult(bf);
    put(sl1, bf1);
    lds_barrier();  // orders LDS only: the ring's loads stay in flight
  };
  fetch(0, C0{});
  fetch(min(1, nst - 1), C1{});
  fetch(min(2, nst - 1), C2{});
  put(C0{}, C0{});
  lds_barrier();
  int st = 0;
  for (; st + 6 <= nst; st += 6) {
    step(st, C0{}, C0{}, C1{}, C1{});
    step(st + 1, C1{}, C1{}, C2{}, C0{});
    step(st + 2, C2{}, C0{}, C0{}, C1{});
    step(st + 3, C0{}, C1{}, C1{}, C0{});
    step(st + 4, C1{}, C0{}, C2{}, C1{});
    step(st + 5, C2{}, C1{}, C0{}, C0{});
  }
  if (st < nst) step(st, C0{}, C0{}, C1{}, C1{});
  if (st + 1 < nst) step(st + 1, C1{}, C1{}, C2{}, C0{});
  if (st + 2 < nst) step(st + 2, C2{}, C0{}, C0{}, C1{});
  if (st + 3 < nst) step(st + 3, C0{}, C1{}, C1{}, C0{});
  if (st + 4 < nst) step(st + 4, C1{}, C0{}, C2{}, C1{});

  // ---- add the KW partial blocks (the stage ring is free now)
  if constexpr (KW > 1) {
    constexpr int NA = 2 * PBW * 2 * 4;  // floats of acc per lane
    static_assert((KW - 1) * (4 / KW) * 64 * NA * 4 <= (int)sizeof(s_t), "reduction scratch");
    float* red = (float*)&s_t[0][0];
    const int blk = w / KW;
    __syncthreads();
    if (kw > 0) {
      float* dst = red + (((size_t)(kw - 1) * (4 / KW) + blk) * 64 + lane) * NA;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int q = 0; q < PBW; ++q)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) *(floatx4*)(dst + 4 * ((mt * PBW + q) * 2 + nt)) = acc[mt][q][nt];
    }
    __syncthreads();
    if (kw == 0) {
#pragma unroll
      for (int o = 1; o < KW; ++o) {
        const float* srcr = red + (((size_t)(o - 1) * (4 / KW) + blk) * 64 + lane) * NA;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int q = 0; q < PBW; ++q)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc[mt][q][nt] += *(const floatx4*)(srcr + 4 * ((mt * PBW + q) * 2 + nt));
      }
    }
  }
  if (kw != 0) return;
  // ---- epilogue: the lane holds rows 4*lg + e of each row tile, pair l16 of
  // each block; split launches store raw partial sums [z][m][pair][a, b]
#pragma unroll
  for (int q = 0; q < PBW; ++q) {
    const int j = p0 + 16 * (pbw * PBW + q) + l16;
    if (j >= npairs) continue;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 32 * mb + 16 * mt + 4 * lg + e;
        if (m >= p.M) continue;
        float a = acc[mt][q][0][e], b = acc[mt][q][1][e];
        if constexpr (SPLIT) {
          float* dst = p.part + (((size_t)blockIdx.z * p.M + m) * npairs + j) * 2;
          dst[0] = a;
          dst[1] = b;
        } else {
          if constexpr (NORM) {
            const float f = row_factor(p, m);
            a *= f;
            b *= f;
          }
          epilogue_pair<EPI>(p, m, j, a, b);
        }
      }
  }
}

// out = epilogue(sum over the K slices, in slice order)
template <int EPI, bool NORM>
__global__ __launch_bounds__(256) void gemm_tiled_finish_kernel(GemmParams p, int nsplit) {
  const int npairs = pair_count<EPI>(p);
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)p.M * npairs) return;
  const int m = (int)(e / npairs), j = (int)(e % npairs);
  float a = 0.f, b = 0.f;
  for (int z = 0; z < nsplit; ++z) {
    const float* src = p.part + (((size_t)z * p.M + m) * npairs + j) * 2;
    a += src[0];
    b += src[1];
  }
  if (NORM) {
    const float f = row_factor(p, m);
    a *= f;
    b *= f;
  }
  epilogue_pair<EPI>(p, m, j, a, b);
}

// Finish of a library GEMM over the stacked planes: d [2M][ldd] holds the
// products of the hi rows (0 .. M-1) and of the lo rows (M .. 2M-1) with
// every weight row.  Adds the two, applies the RMSNorm row factor and the
// epilogue.  One thread per (row, pair).
template <int EPI, bool NORM>
__global__ __launch_bounds__(256) void gemm_blas_finish_kernel(GemmParams p, const float* d, int ldd) {
  const int npairs = pair_count<EPI>(p);
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)p.M * npairs) return;
  const int m = (int)(e / npairs), j = (int)(e % npairs);
  int rb;
  const int ra = pair_rows<EPI>(p, j, rb);
  const float* hi = d + (size_t)m * ldd;
  const float* lo = d + (size_t)(p.M + m) * ldd;
  float a = ra < ldd ? hi[ra] + lo[ra] : 0.f;
  float b = rb < ldd ? hi[rb] + lo[rb] : 0.f;
  if (NORM) {
    const float f = row_factor(p, m);
    a *= f;
    b *= f;
  }
  epilogue_pair<EPI>(p, m, j, a, b);
}

template <int EPI>
static hipError_t launch_blas_finish_epi(const GemmParams& p, const float* d, int ldd, hipStream_t s) {
  const size_t n = (size_t)p.M * pair_count<EPI>(p);
  const int blocks = (int)((n + 255) / 256);
  if (p.norm_g) gemm_blas_finish_kernel<EPI, true><<<blocks, 256, 0, s>>>(p, d, ldd);
  else gemm_blas_finish_kernel<EPI, false><<<blocks, 256, 0, s>>>(p, d, ldd);
  return hipGetLastError();
}

template <int MB, int KW, int EPI>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  constexpr int R = 3;
  constexpr int BM = 32 * MB;
  const int tiles_n = (pair_count<EPI>(p) + NPAIR - 1) / NPAIR;
  const int tiles_m = (p.M + BM - 1) / BM;
  // split K while the tiles would not fill the chip, if scratch allows
  int nsplit = 1;
  while (p.part && tiles_n * tiles_m * nsplit < 384 && nsplit < 8 && (p.K / (2 * nsplit)) % TK == 0 &&
         (size_t)2 * nsplit * p.M * pair_count<EPI>(p) * 2 <= p.part_floats)
    nsplit *= 2;
  const bool norm = p.norm_g != nullptr;
  launch_split_x(p, s);
  const dim3 grid(tiles_n, tiles_m, nsplit);
  if (nsplit == 1) {
    if (norm) gemm_tiled_kernel<MB, KW, R, EPI, true, false><<<grid, 256, 0, s>>>(p);
    else gemm_tiled_kernel<MB, KW, R, EPI, false, false><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
  }
  gemm_tiled_kernel<MB, KW, R, EPI, false, true><<<grid, 256, 0, s>>>(p);
  const size_t n = (size_t)p.M * pair_count<EPI>(p);
  const int blocks = (int)((n + 255) / 256);
  if (norm) gemm_tiled_finish_kernel<EPI, true><<<blocks, 256, 0, s>>>(p, nsplit);
  else gemm_tiled_finish_kernel<EPI, false><<<blocks, 256, 0, s>>>(p, nsplit);
  return hipGetLastError();
}

// Row blocks by row count: up to 32 rows one block with the waves split over
// k; up to 64 rows two blocks; beyond, four (the weights are read once per
// 128 rows).
template <int EPI>
hipError_t launch_epi(const GemmParams& p, hipStream_t s) {
  if (p.M <= 32) return launch_cfg<1, 2, EPI>(p, s);
  if (p.M <= 64) return launch_cfg<2, 1, EPI>(p, s);
  return launch_cfg<4, 1, EPI>(p, s);
}

}  // namespace

// Measured on the 8B layer shapes (back-to-back launches): from 5 rows on the
// tiled kernel beats the skinny matrix-core kernel on the QKV, gate/up and LM
// head GEMMs (gate/up 48 vs 58 us at 5..8 rows); the residual GEMMs (O, down)
// gain only beyond 8 rows.
hipError_t launch_split_x(const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.K + 1023) / 1024, p.M);
  if (p.norm_g) gemm_split_x_kernel<true><<<grid, 256, 0, s>>>(p);
  else gemm_split_x_kernel<false><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_blas_finish(const GemmParams& p, const float* d, int ldd, hipStream_t s) {
  switch (p.epi) {
    case EPI_STORE: return launch_blas_finish_epi<EPI_STORE>(p, d, ldd, s);
    case EPI_RESID: return launch_blas_finish_epi<EPI_RESID>(p, d, ldd, s);
    case EPI_SWIGLU: return launch_blas_finish_epi<EPI_SWIGLU>(p, d, ldd, s);
    default: return launch_blas_finish_epi<EPI_QKV>(p, d, ldd, s);
  }
}

// Between 64 and 128 rows the library GEMM wins on the 4096-deep
// projections, but the tiled kernel wins on the 14336-deep down projection
// (128 rows: 69 against 80 us per layer), where the library's product
// scratch and finish pass cost the most.
bool gemm_tiled_preferred(const GemmParams& p) { return p.K > 8192 && p.M <= 128 && gemm_tiled_ok(p); }

bool gemm_tiled_ok(const GemmParams& p) {
  if (p.wdtype != 1 || p.K % TK || p.K > SSQ_BLK * 1024 || !p.xs || (size_t)2 * p.M * p.K > p.xs_elems) return false;
  return p.M > 8 || (p.M >= 5 && p.epi != EPI_RESID);
}

hipError_t launch_gemm_tiled(const GemmParams& p, hipStream_t s) {
  switch (p.epi) {
    case EPI_STORE: return launch_epi<EPI_STORE>(p, s);
    case EPI_RESID: return launch_epi<EPI_RESID>(p, s);
    case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(p, s);
    default: return launch_epi<EPI_QKV>(p, s);
  }
}

}  // namespace sv
