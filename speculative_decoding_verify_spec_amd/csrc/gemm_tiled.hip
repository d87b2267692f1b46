// Tiled GEMM for many activation rows (more than 8; up to 8 the
// weight-streaming kernels are faster on every 8B projection):
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

// Output pairs of a tile of NP pairs (2 NP weight rows); see the header.
template <int EPI, int NP>
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
  const int a = (j / NP) * (2 * NP) + (j % NP);
  rb = a + NP;
  return a;
}

template <int EPI, int NP>
__host__ __device__ int pair_count(const GemmParams& p) {
  if (EPI == EPI_SWIGLU) return p.F;
  if (EPI == EPI_QKV) return p.N / 2;
  return ((p.N + 2 * NP - 1) / (2 * NP)) * NP;
}

// Epilogue of one (row m, pair j) with its two finished sums.
template <int EPI, int NP>
DEVI void epilogue_pair(const GemmParams& p, int m, int j, float a, float b) {
  int rb;
  const int ra = pair_rows<EPI, NP>(p, j, rb);
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
    const float v = a / (1.0f + expf(-a)) * b;
    p.out[(size_t)m * p.ldo + j] = v;
    if (p.xs_out) {
      // the next GEMM's activation planes, as gemm_split_x_kernel writes them
      short h, l;
      split_bf16(v, h, l);
      p.xs_out[(size_t)m * p.ldo + j] = (uint16_t)h;
      p.xs_out[((size_t)p.M + m) * p.ldo + j] = (uint16_t)l;
    }
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
  const int npairs = pair_count<EPI, NPAIR>(p);
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
      const int ra = pair_rows<EPI, NPAIR>(p, j < npairs ? j : 0, rb);
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
          epilogue_pair<EPI, NPAIR>(p, m, j, a, b);
        }
      }
  }
}

// out = epilogue(sum over the K slices, in slice order)
template <int EPI, bool NORM, int NP>
__global__ __launch_bounds__(256) void gemm_tiled_finish_kernel(GemmParams p, int nsplit) {
  const int npairs = pair_count<EPI, NP>(p);
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
  epilogue_pair<EPI, NP>(p, m, j, a, b);
}

// Finish of a K-split residual GEMM that also prepares the next GEMM's
// activations (norm_next): out = out + (the slices' partial sums, in slice
// order, as gemm_tiled_finish_kernel adds them), then the bf16 hi/lo planes of
// out * norm_next into xs_next and the row's sum of squares over each 1024
// columns into xs_ssq, with the arithmetic of gemm_split_x_kernel.  One
// workgroup per (1024 columns, row): thread t takes pairs 512 blk + 2t and
// + 1, whose a and b columns (two adjacent pairs of columns) lie in that
// block since 1024 is a multiple of a tile's 2 NP columns.
template <int NP>
__global__ __launch_bounds__(256) void gemm_finish_norm_kernel(GemmParams p, int nsplit) {
  static_assert(1024 % (2 * NP) == 0 && NP % 2 == 0, "a workgroup's pairs fill whole tiles");
  const int blk = blockIdx.x, m = blockIdx.y;
  const int npairs = pair_count<EPI_RESID, NP>(p);
  const int j = blk * 512 + 2 * (int)threadIdx.x;
  float ss = 0.f;
  if (j < npairs) {
    float a0 = 0.f, b0 = 0.f, a1 = 0.f, b1 = 0.f;
    for (int z = 0; z < nsplit; ++z) {
      const float4 v = *(const float4*)(p.part + (((size_t)z * p.M + m) * npairs + j) * 2);
      a0 += v.x;
      b0 += v.y;
      a1 += v.z;
      b1 += v.w;
    }
    int rb;
    const int ra = pair_rows<EPI_RESID, NP>(p, j, rb);
    float* o = p.out + (size_t)m * p.ldo;
    uint16_t* hi = p.xs_next + (size_t)m * p.N;
    uint16_t* lo = hi + (size_t)p.M * p.N;
    // columns (ra, ra + 1) take a0, a1 and (rb, rb + 1) take b0, b1
    const int col[2] = {ra, rb};
    const float add[2][2] = {{a0, a1}, {b0, b1}};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = col[h];
      if (c + 2 > p.N) continue;  // a tile past the matrix (never for whole tiles)
      float2 y = *(float2*)(o + c);
      y.x += add[h][0];
      y.y += add[h][1];
      *(float2*)(o + c) = y;
      const float2 g = *(const float2*)(p.norm_next + c);
      ss += y.x * y.x;
      ss += y.y * y.y;
      short h0, l0, h1, l1;
      split_bf16(y.x * g.x, h0, l0);
      split_bf16(y.y * g.y, h1, l1);
      *(uint32_t*)(hi + c) = (uint32_t)(uint16_t)h0 | ((uint32_t)(uint16_t)h1 << 16);
      *(uint32_t*)(lo + c) = (uint32_t)(uint16_t)l0 | ((uint32_t)(uint16_t)l1 << 16);
    }
  }
  __shared__ float red[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) p.xs_ssq[m * SSQ_BLK + blk] = red[0] + red[1] + red[2] + red[3];
}

// The finish of a K-split launch: the plain one, or, for a residual GEMM
// with norm_next, the one that also writes the next GEMM's planes.
template <int EPI, int NP>
void launch_finish(const GemmParams& p, int nsplit, hipStream_t s) {
  if constexpr (EPI == EPI_RESID) {
    if (p.norm_next) {
      gemm_finish_norm_kernel<NP><<<dim3((p.N + 1023) / 1024, p.M), 256, 0, s>>>(p, nsplit);
      return;
    }
  }
  const size_t n = (size_t)p.M * pair_count<EPI, NP>(p);
  const int blocks = (int)((n + 255) / 256);
  if (p.norm_g) gemm_tiled_finish_kernel<EPI, true, NP><<<blocks, 256, 0, s>>>(p, nsplit);
  else gemm_tiled_finish_kernel<EPI, false, NP><<<blocks, 256, 0, s>>>(p, nsplit);
}

// K slices of a launch of the 32-row tiles: split while the tiles would not
// fill the chip, if the scratch allows, into at most 4 slices (a slice's
// pipeline of 64-k stages is mostly ramp below ~16 stages: on the 8B shape
// at 32 rows, 8 slices took the O projection 20.2 and the down projection
// 37.4 us per launch with their finish, 4 slices 18.5 and 34.6 us; B=8 step
// 5.07 -> 4.92 ms)
template <int MB, int EPI>
int cfg_splits(const GemmParams& p) {
  constexpr int BM = 32 * MB;
  const int tiles_n = (pair_count<EPI, NPAIR>(p) + NPAIR - 1) / NPAIR;
  const int tiles_m = (p.M + BM - 1) / BM;
  int nsplit = 1;
  while (p.part && tiles_n * tiles_m * nsplit < 384 && nsplit < 4 && (p.K / (2 * nsplit)) % TK == 0 &&
         (size_t)2 * nsplit * p.M * pair_count<EPI, NPAIR>(p) * 2 <= p.part_floats)
    nsplit *= 2;
  return nsplit;
}

template <int MB, int KW, int EPI>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  constexpr int R = 3;
  constexpr int BM = 32 * MB;
  const int tiles_n = (pair_count<EPI, NPAIR>(p) + NPAIR - 1) / NPAIR;
  const int tiles_m = (p.M + BM - 1) / BM;
  const int nsplit = cfg_splits<MB, EPI>(p);
  const bool norm = p.norm_g != nullptr;
  if (!p.xs_ready) launch_split_x(p, s);
  const dim3 grid(tiles_n, tiles_m, nsplit);
  if (nsplit == 1) {
    if (norm) gemm_tiled_kernel<MB, KW, R, EPI, true, false><<<grid, 256, 0, s>>>(p);
    else gemm_tiled_kernel<MB, KW, R, EPI, false, false><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
  }
  gemm_tiled_kernel<MB, KW, R, EPI, false, true><<<grid, 256, 0, s>>>(p);
  launch_finish<EPI, NPAIR>(p, nsplit, s);
  return hipGetLastError();
}

// ---------------------------------------------------------------- large tiles
// Many rows (64 or more: the windows of 16+ sequences, token trees, long
// verify windows of a batch): the contraction is dense enough that the
// matrix cores and the LDS, not the weight stream, bound it.  A workgroup
// owns BIG_BM = 128 activation rows and BIG_NP = 128 pairs (256 weight
// rows).  Its 8 waves (two per SIMD) form a 2 x 4 grid of 64 rows x 32
// pairs; per 16-k step a wave reads 2 + 2 activation fragments (hi, lo) and
// 2 weight fragments (a and b rows) from LDS and issues 8 32x32x16 products.
// (A 4-wave form, a 2 x 2 grid of 64 x 64 with one wave per SIMD, reads 8
// fragments per 16 products; it is kept as a measurement option and runs
// 4-7% slower.)
//
// Stages of 64 k (512 LDS rows of 128 bytes: 256 weight rows, then 128 hi
// and 128 lo activation rows) are requested two stages ahead into a ring of
// two register sets and written one stage ahead to one of two LDS buffers
// (128 KB).  The main loop is unrolled by two and branch-free, so every wait
// names exactly the loads it needs.
//
// What bounds it (8B gate/up at 512 rows, measured with parts of the step
// removed in a copy of this kernel): the products alone take 61% of the full
// time, and the loads alone hide completely behind them; the LDS traffic is
// the rest.  LDS moves about 144 bytes per clock per CU for 16-byte reads and
// about 73 for 16-byte writes, so a stage's 192 KB of operand reads and 64 KB
// of writes take about as long as its products (2048 clocks per SIMD).
//
// LDS rows are swizzled so that the 16 rows of one operand read hit distinct
// banks in groups of 8 lanes (32 banks) and of 16 lanes (64 banks): chunk c
// of row r sits in slot c ^ g(r), g(r) = (r & 7) ^ ((r >> 3) & 1).
//
// Tiles are numbered so that the hardware's round-robin dispatch over the 8
// XCDs gives each XCD a contiguous run of them, row tiles fastest: the row
// tiles of one weight tile run side by side on one XCD and share its weight
// stream through that XCD's L2.  Launches with fewer tiles than CUs split K
// into S slices of whole stages; the slices write raw partial sums that
// gemm_tiled_finish_kernel adds in slice order before the epilogue.
constexpr int BIG_BM = 128;
constexpr int BIG_NP = 128;
constexpr int BIG_WR = 2 * BIG_NP;
constexpr int BIG_ROWS = BIG_WR + 2 * BIG_BM;  // LDS rows per stage
constexpr int BIG_STAGE = BIG_ROWS * 64;       // bf16 elements per LDS stage

DEVI int big_g(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Instruction classes of the scheduler's group barriers, and 8 pairs of
// products each followed by one instruction of class A and one of class B.
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200;
template <int A, int B>
DEVI void sched_pairs8() {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    __builtin_amdgcn_sched_group_barrier(A, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    if constexpr (B != 0) __builtin_amdgcn_sched_group_barrier(B, 1, 0);
  }
}

// Buffer resource word 3 of the gfx9 family (raw buffer, 32-bit data format).
constexpr int BUF_WORD3 = 0x00020000;

// Per sub-step of a wave with 8 products: product k is followed by one
// instruction of class A while k < NA and one of class B while k < NB.
template <int NA, int A, int NB, int B>
DEVI void sched_mix8() {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    if constexpr (NA > 0) if (k < NA) __builtin_amdgcn_sched_group_barrier(A, 1, 0);
    if constexpr (NB > 0) if (k < NB) __builtin_amdgcn_sched_group_barrier(B, 1, 0);
  }
}

// NW = 8 (the default): a 2 x 4 grid of 64 rows x 32 pairs, two waves per
// SIMD, so that one wave's operand reads, requests and LDS writes run while
// the other's products keep the matrix core busy.  NW = 4: a 2 x 2 grid of
// 64 rows x 64 pairs, one wave per SIMD.
template <int EPI, bool NORM, bool SPLIT, int NW>
__global__ __launch_bounds__(64 * NW, 1) void gemm_big_kernel(GemmParams p, int tiles_m, int nsplit, int ntiles) {
  constexpr int NT = 64 * NW;                 // threads
  constexpr int RSTEP = NT / 8;               // stage rows between a thread's chunks
  constexpr int BIG_CH = BIG_ROWS * 8 / NT;   // 16-byte chunks per thread per stage
  constexpr int UB = NW == 4 ? 2 : 1;         // 32-pair blocks per wave
  // the two stage buffers are separate arrays, so the compiler can tell the
  // next stage's LDS writes from this stage's reads and interleave them
  __shared__ __attribute__((aligned(16))) uint16_t s_b0[BIG_STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t s_b1[BIG_STAGE];
  // ---- tile of this workgroup: each XCD takes a contiguous run
  const int per = (int)gridDim.x / 8;
  const int tl = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (tl >= ntiles) return;
  const int mt = tl % tiles_m;
  const int z = (tl / tiles_m) % nsplit;
  const int nt = tl / (tiles_m * nsplit);
  const int p0 = nt * BIG_NP;
  const int m0 = mt * BIG_BM;
  const int npairs = pair_count<EPI, BIG_NP>(p);
  const int nst_all = p.K / TK;
  const int sbeg = (int)((long long)nst_all * z / nsplit);
  const int nst = (int)((long long)nst_all * (z + 1) / nsplit) - sbeg;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int wm = w & 1, wp = w >> 1;

  // ---- the thread's chunks: stage row r = tid/8 + RSTEP i, chunk q = tid % 8;
  // byte offsets of the chunk's first k from the weight base (i < 8) or the
  // activation planes' base (i >= 8).  32-bit byte offsets let every load
  // take a scalar base plus a vector offset (weights up to 4 GB).
  uint32_t off[BIG_CH];
  const int q = tid & 7;
#pragma unroll
  for (int i = 0; i < BIG_CH; ++i) {
    const int r = (tid >> 3) + RSTEP * i;
    if (r < BIG_WR) {
      const int jl = r % BIG_NP;
      const int j = p0 + jl;
      int rb;
      const int ra = pair_rows<EPI, BIG_NP>(p, j < npairs ? j : 0, rb);
      int row = r < BIG_NP ? ra : rb;
      row = (j < npairs && row < p.N) ? row : 0;  // rows past the matrix load row 0, never stored
      off[i] = ((uint32_t)row * (uint32_t)p.K + 8 * q) * 2u;
    } else {
      const int rx = r - BIG_WR;
      const int plane = rx / BIG_BM, ml = rx % BIG_BM;
      const int m = (m0 + ml < p.M) ? m0 + ml : p.M - 1;  // rows past M: any valid row, never stored
      off[i] = (((uint32_t)plane * (uint32_t)p.M + (uint32_t)m) * (uint32_t)p.K + 8 * q) * 2u;
    }
  }
  // LDS byte offset of the thread's chunk 0; chunk i is 128 RSTEP i further
  // (g depends on r & 15 only, which is the same for every i)
  const int r0 = tid >> 3;
  const int dst0 = r0 * 128 + 16 * (q ^ big_g(r0));
  // buffer resources over the weight matrix and the two planes: a load is
  // base + (vector byte offset) + (scalar stage offset), and one outside the
  // resource's byte range returns zeros instead of faulting
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.W, (short)0, (int)((size_t)p.N * p.K * 2 < 0x7fffffffu ? (size_t)p.N * p.K * 2 : 0x7fffffffu),
      BUF_WORD3);
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.xs, (short)0, (int)((size_t)2 * p.M * p.K * 2), BUF_WORD3);

  constexpr int R = 2;  // register stages in flight (a third measured 5% slower)
  u32x4 ring[R][BIG_CH];
  auto fetch = [&](int st, auto sl) {
    constexpr int S = decltype(sl)::value;
    const int so = (sbeg + st) * TK * 2;
#pragma unroll
    for (int i = 0; i < BIG_CH; ++i) {
      // plain loads: a weight tile is read by the row tiles running beside it
      // on the same XCD (a non-temporal hint measured 5-15% slower), the
      // activation planes by every weight tile
      if (i < BIG_WR / RSTEP) ring[S][i] = __builtin_amdgcn_raw_buffer_load_b128(wres, off[i], so, 0);
      else ring[S][i] = __builtin_amdgcn_raw_buffer_load_b128(xres, off[i], so, 0);
    }
  };
  auto buf = [&](auto bf) -> char* {
    if constexpr (decltype(bf)::value == 0) return (char*)s_b0;
    else return (char*)s_b1;
  };
  auto put = [&](auto sl, auto bf) {
    constexpr int S = decltype(sl)::value;
    char* lds = buf(bf);
#pragma unroll
    for (int i = 0; i < BIG_CH; ++i) *(u32x4*)(lds + dst0 + 128 * RSTEP * i) = ring[S][i];
  };

  // 32x32x16 products: lane l holds operand row (or pair) l % 32 at k
  // 8 (l / 32) + e of each 16-k sub-step, and result column l % 32 at rows
  // 8 (i / 4) + 4 (l / 32) + i % 4.  Eight accumulators of 16 floats (rather
  // than 32 of 4) let the compiler keep every accumulator in place across
  // the loop.
  floatx16 acc[2][UB][2];  // [row tile of 32][pair block of 32][a, b]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < UB; ++b) acc[a][b][0] = acc[a][b][1] = floatx16{};
  const int pw = 32 * UB * wp;  // the wave's first pair in the tile

  const int l32 = lane & 31, lh = lane >> 5;
  const int gl = big_g(l32);
  auto mult = [&](auto bf) {
    const char* base = buf(bf) + l32 * 128;
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
      const char* cb = base + 16 * ((2 * ss + lh) ^ gl);
      shortx8 ah[2], al[2], ba[UB], bb[UB];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        ah[t] = *(const shortx8*)(cb + (BIG_WR + 64 * wm + 32 * t) * 128);
        al[t] = *(const shortx8*)(cb + (BIG_WR + BIG_BM + 64 * wm + 32 * t) * 128);
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        ba[u] = *(const shortx8*)(cb + (pw + 32 * u) * 128);
        bb[u] = *(const shortx8*)(cb + (BIG_NP + pw + 32 * u) * 128);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          acc[t][u][0] = mfma32x32x16(ah[t], ba[u], acc[t][u][0]);
          acc[t][u][1] = mfma32x32x16(ah[t], bb[u], acc[t][u][1]);
        }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < UB; ++u) {
          acc[t][u][0] = mfma32x32x16(al[t], ba[u], acc[t][u][0]);
          acc[t][u][1] = mfma32x32x16(al[t], bb[u], acc[t][u][1]);
        }
    }
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  // step st: request stage st + R into the ring slot stage st came from
  // (slot st % R), multiply stage st (LDS buffer st % 2), write stage st + 1
  // from its ring slot to the other buffer.  A request past the last stage
  // re-reads it and a write past it fills a buffer nobody reads, so the steps
  // are branch-free.
  //
  // With one wave per SIMD the matrix core idles whenever the wave issues
  // anything else between two products, so the step's 64 other instructions
  // (32 operand reads, 16 requests, 16 LDS writes) are placed one after each
  // product: the reads of sub-step s + 1 during sub-step s, the requests in
  // the first two sub-steps, the LDS writes (which wait for the requests of
  // the step before) in the last two.
  auto interleave = [&]() {
    if constexpr (NW == 4) {
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 8, 0);  // operand reads of sub-step 0
      sched_pairs8<SG_DS_READ, SG_VMEM_READ>();   // sub-step 0: reads of 1, requests
      sched_pairs8<SG_DS_READ, SG_VMEM_READ>();   // sub-step 1: reads of 2, requests
      sched_pairs8<SG_DS_READ, SG_DS_WRITE>();    // sub-step 2: reads of 3, LDS writes
      sched_pairs8<SG_DS_WRITE, 0>();             // sub-step 3: LDS writes
    } else {
      // 8 products, 6 operand reads per sub-step; 8 requests and 8 LDS writes
      // per step
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 6, 0);
      sched_mix8<6, SG_DS_READ, 4, SG_VMEM_READ>();
      sched_mix8<6, SG_DS_READ, 4, SG_VMEM_READ>();
      sched_mix8<6, SG_DS_READ, 4, SG_DS_WRITE>();
      sched_mix8<4, SG_DS_WRITE, 0, 0>();
    }
  };
  auto step = [&](int st, auto sl, auto bf, auto sl1, auto bf1) {
    fetch(min(st + R, nst - 1), sl);
    mult(bf);
    put(sl1, bf1);
    interleave();
    lds_barrier();  // orders LDS only: the ring's loads stay in flight
  };
  fetch(0, C0{});
  fetch(min(1, nst - 1), C1{});
  if constexpr (R == 3) fetch(min(2, nst - 1), C2{});
  put(C0{}, C0{});
  lds_barrier();
  int st = 0;
  if constexpr (R == 2) {
    for (; st + 2 <= nst; st += 2) {
      step(st, C0{}, C0{}, C1{}, C1{});
      step(st + 1, C1{}, C1{}, C0{}, C0{});
    }
    if (st < nst) step(st, C0{}, C0{}, C1{}, C1{});
  } else {
    // (slot, buffer) of stage st repeat every 6 stages
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
  }

  // ---- epilogue: lane l holds pair l % 32 of each pair block, rows
  // 8 (i / 4) + 4 (l / 32) + i % 4 of each row tile
  float fac[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + 64 * wm + 32 * t + 8 * (i >> 2) + 4 * lh + (i & 3);
      fac[t][i] = (NORM && !SPLIT && m < p.M) ? row_factor(p, m) : 1.0f;
    }
#pragma unroll
  for (int u = 0; u < UB; ++u) {
    const int j = p0 + pw + 32 * u + l32;
    if (j >= npairs) continue;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + 64 * wm + 32 * t + 8 * (i >> 2) + 4 * lh + (i & 3);
        if (m >= p.M) continue;
        const float a = acc[t][u][0][i], b = acc[t][u][1][i];
        if constexpr (SPLIT) {
          float* dst = p.part + (((size_t)z * p.M + m) * npairs + j) * 2;
          *(float2*)dst = make_float2(a, b);
        } else {
          epilogue_pair<EPI, BIG_NP>(p, m, j, a * fac[t][i], b * fac[t][i]);
        }
      }
  }
}

// K slices for a launch of `tiles` output tiles over `nst` stages.  Time of
// the slowest CU: rounds of resident workgroups x stages per slice x the time
// of a stage (~1.7 us: 8.4 MFLOP per tile stage at about half the CU's
// matrix-core peak), plus, for S > 1, writing and re-reading the partial sums
// (S x per_split_floats x 4 bytes each way, at ~5 TB/s).  Limited by the
// scratch.
int big_splits(int tiles, int nst, int cus, size_t per_split_floats, size_t part_floats) {
  int best = 1;
  double best_us = 1e300;
  for (int S = 1; S <= 8 && S <= nst; ++S) {
    if (S > 1 && (size_t)S * per_split_floats > part_floats) break;
    const double rounds = (double)((tiles * S + cus - 1) / cus);
    double us = rounds * ((nst + S - 1) / S) * 1.7;
    if (S > 1) us += 2.0 * S * (double)per_split_floats * 4.0 / 5.0e6;
    if (us < best_us - 1e-9) {
      best_us = us;
      best = S;
    }
  }
  return best;
}

template <int EPI, int NW>
hipError_t launch_big_nw(const GemmParams& p, hipStream_t s, bool norm, int nsplit, int tiles_m, int ntiles,
                         int grid) {
  if (nsplit == 1) {
    if (norm) gemm_big_kernel<EPI, true, false, NW><<<grid, 64 * NW, 0, s>>>(p, tiles_m, 1, ntiles);
    else gemm_big_kernel<EPI, false, false, NW><<<grid, 64 * NW, 0, s>>>(p, tiles_m, 1, ntiles);
    return hipGetLastError();
  }
  gemm_big_kernel<EPI, false, true, NW><<<grid, 64 * NW, 0, s>>>(p, tiles_m, nsplit, ntiles);
  launch_finish<EPI, BIG_NP>(p, nsplit, s);
  return hipGetLastError();
}

template <int EPI>
int big_nsplit(const GemmParams& p) {
  const int npairs = pair_count<EPI, BIG_NP>(p);
  const int tiles_n = (npairs + BIG_NP - 1) / BIG_NP;
  const int tiles_m = (p.M + BIG_BM - 1) / BIG_BM;
  return p.part ? big_splits(tiles_n * tiles_m, p.K / TK, device_cus(), (size_t)p.M * npairs * 2, p.part_floats)
                : 1;
}

template <int EPI>
hipError_t launch_big(const GemmParams& p, hipStream_t s) {
  const int npairs = pair_count<EPI, BIG_NP>(p);
  const int tiles_n = (npairs + BIG_NP - 1) / BIG_NP;
  const int tiles_m = (p.M + BIG_BM - 1) / BIG_BM;
  const int nsplit = big_nsplit<EPI>(p);
  const int ntiles = tiles_n * tiles_m * nsplit;
  const int grid = ((ntiles + 7) / 8) * 8;
  const bool norm = p.norm_g != nullptr;
  if (!p.xs_ready) launch_split_x(p, s);
  if (gemm_route == 3) return launch_big_nw<EPI, 4>(p, s, norm, nsplit, tiles_m, ntiles, grid);
  return launch_big_nw<EPI, 8>(p, s, norm, nsplit, tiles_m, ntiles, grid);
}

// Row blocks by row count: up to 32 rows one block with the waves split over
// k; up to 64 rows two blocks; beyond, four (the weights are read once per
// 128 rows).
template <int EPI>
hipError_t launch_epi(const GemmParams& p, hipStream_t s) {
  if (gemm_big_rows(p)) return launch_big<EPI>(p, s);
  if (p.M <= 32) return launch_cfg<1, 2, EPI>(p, s);
  if (p.M <= 64) return launch_cfg<2, 1, EPI>(p, s);
  return launch_cfg<4, 1, EPI>(p, s);
}

}  // namespace

hipError_t launch_split_x(const GemmParams& p, hipStream_t s) {
  const dim3 grid((p.K + 1023) / 1024, p.M);
  if (p.norm_g) gemm_split_x_kernel<true><<<grid, 256, 0, s>>>(p);
  else gemm_split_x_kernel<false><<<grid, 256, 0, s>>>(p);
  return hipGetLastError();
}

size_t gemm_big_part_floats(int M, size_t npairs, int K, int cus) {
  const int tiles = (int)((npairs + BIG_NP - 1) / BIG_NP) * ((M + BIG_BM - 1) / BIG_BM);
  const int S = big_splits(tiles, K / TK, cus, (size_t)M * npairs * 2, ~(size_t)0);
  return S > 1 ? (size_t)S * M * npairs * 2 : 0;
}

// Which tiles serve an M-row launch: the large tiles from 64 rows on, unless
// a measurement override is set (gemm_route: 1 = 32-row tiles, 2 = large
// tiles wherever the tiled kernels run, 3 = the large tiles' 4-wave form).
int gemm_route = 0;
bool gemm_big_rows(const GemmParams& p) {
  // buffer offsets are 32-bit: the weight matrix and the planes stay below 2 GB
  if ((size_t)p.N * p.K * 2 >= 0x7fffffffu || (size_t)4 * p.M * p.K >= 0x7fffffffu) return false;
  if (gemm_route == 1) return false;
  if (gemm_route == 2) return true;
  return p.M >= 64;
}

bool gemm_tiled_ok(const GemmParams& p) {
  if (p.wdtype != 1 || p.K % TK || p.K > SSQ_BLK * 1024 || !p.xs || (size_t)2 * p.M * p.K > p.xs_elems) return false;
  return p.M > 8;
}

bool gemm_finish_prepares(const GemmParams& p) {
  if (p.epi != EPI_RESID || !gemm_tiled_ok(p)) return false;
  if (gemm_big_rows(p)) return big_nsplit<EPI_RESID>(p) > 1;
  if (p.M <= 32) return cfg_splits<1, EPI_RESID>(p) > 1;
  if (p.M <= 64) return cfg_splits<2, EPI_RESID>(p) > 1;
  return cfg_splits<4, EPI_RESID>(p) > 1;
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
