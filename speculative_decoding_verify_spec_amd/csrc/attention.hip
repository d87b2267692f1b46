// Attention of the verify rows over the KV cache plus the speculative suffix.
//
// Context part (attn_ctx_kernel).  Rows of one sequence that share a KV head
// (the GQA group of G query heads times T verify rows: nq = G*T query
// vectors) read that head's cached keys once, inside one wave, so the
// gamma+1 rows of a sequence share one KV read (CS349E Lecture 6, section 9.2).
// The context of a (sequence, KV head) is cut into `splits` workgroups of 4
// waves; each wave keeps its own online-softmax state (flash-decoding style),
// the four states are merged in LDS and the workgroup writes one partial
// (max, sum, unnormalised output) per query.  The products run on the gfx950
// bf16 MFMA 16x16x32: S^T = K Q^T with K exact in bf16 and the fp32 queries
// split into bf16 hi + lo, then O^T += V^T P^T with the fp32 probabilities
// split the same way; accumulation is fp32.  V is stored transposed in the
// cache so the key index (the contraction of P V) is contiguous.  A wave's
// first key blocks (PFB of them) are requested before the queries are
// prepared, so the cache reads and the query reads overlap, and the block PFB
// further on is requested as soon as a block's registers are free.  More
// than 16 queries per KV head at D = 128 take attn_ctx_lds_kernel, which
// stages the key blocks in LDS instead.
//
// Suffix part: more workgroups per (sequence, KV head, query group) attend
// to the step's own keys in fp32 and write their partials in the slot after
// the context splits, so the suffix runs beside the context instead of after
// it.  Each wave walks only the rows its query sees (chain: rows 0..i; tree:
// the node and its ancestors), one query per wave for a small chain batch,
// four otherwise.
//
// Combine part (attn_combine_kernel), one wave per (row, query head): merges
// the nsplit partials of a query and normalises.  Keys at or beyond kv_len
// are loaded as zeros and masked, so nothing past kv_len is ever used.
#include "common.h"
#include "launch.h"

namespace sv {

// Shapes of the context workgroups, by the queries nq of a (sequence, KV
// head):
//   nq <= 16: one 16-query tile per wave, two workgroups per CU;
//   16 < nq <= 64 (chain windows of 5..16 rows): two 16-query tiles per
//     wave, so every wave's key block serves 32 queries.  At D = 128 the
//     blocks are staged in LDS (attn_ctx_lds_kernel below, two workgroups
//     per CU); at D = 64 two blocks are in flight per wave in registers
//     (PFB = 2), more than 256 registers per lane: one workgroup per CU;
//   nq > 64 (token trees): at D = 128 the LDS form as above, one 32-query
//     group per workgroup, the groups of a (sequence, KV head) placed on one
//     XCD so their key reads after the first hit its L2 (tree [4,4,2,2] at
//     B = 4: 133 against 269 us per layer); at D = 64 two 16-query groups
//     per workgroup walk the same key blocks in registers, two workgroups
//     per CU.
int attn_query_tiles(int nq, int D) { return (nq > 16 && (D == 128 || nq <= 64)) ? 2 : 1; }
int attn_groups_per_wg(int nq, int D) { return (D != 128 && nq > 64) ? 2 : 1; }
int attn_nsplit(int splits) { return splits + 1; }
// Suffix queries per wave: four for trees and for chains of 128 or more
// (sequence, KV head) pairs, one otherwise (a small batch's suffix must not
// outlast its context workgroups).  Measured at ctx 1024, T = 4: four per
// wave take B = 16 from 32.5 to 28.5 us per layer, but cost B = 4 and B = 8
// 2.5 and 1.1 us.
__host__ __device__ inline int attn_suffix_qpw(bool tree, int pairs) { return (tree || pairs >= 128) ? 4 : 1; }
// Suffix columns of a launch with `pairs` (sequence, KV head, query set)
// units: 4 * QT * QGW query tiles' worth, qpw queries per wave.
int attn_suffix_cols(bool tree, int pairs, int QT, int QGW) { return 4 * QT * QGW / attn_suffix_qpw(tree, pairs); }

// Key index held in row r of key tile kt of the 32-key block at kb: rows
// 4g..4g+3 of both tiles cover keys kb + 8g .. kb + 8g + 7, so one 16-byte
// load of V^T feeds both tiles.
DEVI int blk_key(int kb, int kt, int r) { return kb + 8 * (r >> 2) + 4 * kt + (r & 3); }

// One query of the suffix part (attn_suffix below).
template <int D>
DEVI void attn_suffix_query(const AttnParams& p, int kvh, int b, int qi) {
  constexpr int PL = D / 64;
  constexpr int SB = 8;  // visible rows whose loads are in flight at once
  const int lane = threadIdx.x & 63;
  const int G = p.Hq / p.Hkv;
  const int Tb = p.rlen ? p.rlen[b] : p.T;
  const int rs = p.rstart ? p.rstart[b] : b * p.T;
  const int nq = G * p.T;
  const int i = qi / G;
  float qv[PL];
  const float* qsrc = p.q + ((size_t)(rs + i) * p.Hq + kvh * G + qi % G) * D;
#pragma unroll
  for (int e = 0; e < PL; ++e) qv[e] = qsrc[lane + 64 * e] * p.scale;
  // visible rows: a tree row's ancestor-or-self bits, a chain row's rows
  // 0..i, below the sequence's row count
  uint64_t lo, hi;
  if (p.anc) {
    lo = p.anc[2 * (rs + i)];
    hi = p.anc[2 * (rs + i) + 1];
  } else {  // chain: rows 0..i
    lo = i >= 63 ? ~0ull : (2ull << i) - 1ull;
    hi = i < 64 ? 0ull : (i >= 127 ? ~0ull : (2ull << (i - 64)) - 1ull);
  }
  if (Tb < 64) lo &= (1ull << Tb) - 1ull;
  if (Tb <= 64) hi = 0;
  else if (Tb < 128) hi &= (1ull << (Tb - 64)) - 1ull;
  float m = -INFINITY, l = 0.f, o[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) o[e] = 0.f;
  while (lo | hi) {
    int js[SB];
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      int j = -1;
      if (lo) {
        j = __builtin_ctzll(lo);
        lo &= lo - 1ull;
      } else if (hi) {
        j = 64 + __builtin_ctzll(hi);
        hi &= hi - 1ull;
      }
      js[k] = j;
    }
    float kk[SB][PL], vv[SB][PL];
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      const size_t src = ((size_t)(rs + (js[k] < 0 ? 0 : js[k])) * p.Hkv + kvh) * D;
#pragma unroll
      for (int e = 0; e < PL; ++e) {
        kk[k][e] = js[k] >= 0 ? p.k_suf[src + lane + 64 * e] : 0.f;
        vv[k][e] = js[k] >= 0 ? p.v_suf[src + lane + 64 * e] : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      if (js[k] < 0) break;  // wave-uniform
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < PL; ++e) t += qv[e] * kk[k][e];
      const float sc = wave_sum(t);
      const float mn = fmaxf(m, sc);
      const float f = (m == -INFINITY) ? 0.f : __expf(m - mn);
      const float pe = __expf(sc - mn);
      l = l * f + pe;
      m = mn;
#pragma unroll
      for (int e = 0; e < PL; ++e) o[e] = o[e] * f + pe * vv[k][e];
    }
  }
  const size_t slot = (((size_t)p.splits * p.B + b) * p.Hkv + kvh) * nq;
#pragma unroll
  for (int e = 0; e < PL; ++e) p.part_o[(slot + qi) * D + lane + 64 * e] = o[e];
  if (lane == 0) {
    p.part_ml[2 * (slot + qi)] = m;
    p.part_ml[2 * (slot + qi) + 1] = l;
  }
}

// NQ consecutive queries qi0 .. qi0 + NQ - 1 of one suffix row (query heads
// of the same KV head): they see the same rows, so the visibility mask and
// each batch of keys and values are loaded once for all of them, and the
// wave waits for memory once per batch instead of once per query.  Each
// query keeps its own online softmax, in the per-query order above.
template <int D, int NQ>
DEVI void attn_suffix_row(const AttnParams& p, int kvh, int b, int qi0) {
  constexpr int PL = D / 64;
  constexpr int SB = 8;
  const int lane = threadIdx.x & 63;
  const int G = p.Hq / p.Hkv;
  const int Tb = p.rlen ? p.rlen[b] : p.T;
  const int rs = p.rstart ? p.rstart[b] : b * p.T;
  const int nq = G * p.T;
  const int i = qi0 / G;
  float qv[NQ][PL];
  const float* qsrc = p.q + ((size_t)(rs + i) * p.Hq + kvh * G + qi0 % G) * D;
#pragma unroll
  for (int n = 0; n < NQ; ++n)
#pragma unroll
    for (int e = 0; e < PL; ++e) qv[n][e] = qsrc[n * D + lane + 64 * e] * p.scale;
  uint64_t lo, hi;
  if (p.anc) {
    lo = p.anc[2 * (rs + i)];
    hi = p.anc[2 * (rs + i) + 1];
  } else {
    lo = i >= 63 ? ~0ull : (2ull << i) - 1ull;
    hi = i < 64 ? 0ull : (i >= 127 ? ~0ull : (2ull << (i - 64)) - 1ull);
  }
  if (Tb < 64) lo &= (1ull << Tb) - 1ull;
  if (Tb <= 64) hi = 0;
  else if (Tb < 128) hi &= (1ull << (Tb - 64)) - 1ull;
  float m[NQ], l[NQ], o[NQ][PL];
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
    m[n] = -INFINITY;
    l[n] = 0.f;
#pragma unroll
    for (int e = 0; e < PL; ++e) o[n][e] = 0.f;
  }
  while (lo | hi) {
    int js[SB];
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      int j = -1;
      if (lo) {
        j = __builtin_ctzll(lo);
        lo &= lo - 1ull;
      } else if (hi) {
        j = 64 + __builtin_ctzll(hi);
        hi &= hi - 1ull;
      }
      js[k] = j;
    }
    float kk[SB][PL], vv[SB][PL];
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      const size_t src = ((size_t)(rs + (js[k] < 0 ? 0 : js[k])) * p.Hkv + kvh) * D;
#pragma unroll
      for (int e = 0; e < PL; ++e) {
        kk[k][e] = js[k] >= 0 ? p.k_suf[src + lane + 64 * e] : 0.f;
        vv[k][e] = js[k] >= 0 ? p.v_suf[src + lane + 64 * e] : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      if (js[k] < 0) break;  // wave-uniform
#pragma unroll
      for (int n = 0; n < NQ; ++n) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < PL; ++e) t += qv[n][e] * kk[k][e];
        const float sc = wave_sum(t);
        const float mn = fmaxf(m[n], sc);
        const float f = (m[n] == -INFINITY) ? 0.f : __expf(m[n] - mn);
        const float pe = __expf(sc - mn);
        l[n] = l[n] * f + pe;
        m[n] = mn;
#pragma unroll
        for (int e = 0; e < PL; ++e) o[n][e] = o[n][e] * f + pe * vv[k][e];
      }
    }
  }
  const size_t slot = (((size_t)p.splits * p.B + b) * p.Hkv + kvh) * nq;
#pragma unroll
  for (int n = 0; n < NQ; ++n) {
#pragma unroll
    for (int e = 0; e < PL; ++e) p.part_o[(slot + qi0 + n) * D + lane + 64 * e] = o[n][e];
    if (lane == 0) {
      p.part_ml[2 * (slot + qi0 + n)] = m[n];
      p.part_ml[2 * (slot + qi0 + n) + 1] = l[n];
    }
  }
}

// The step's own keys, in fp32: a chain row i sees rows 0..i; a token-tree
// node sees itself and its ancestors only (CS349E Lecture 6, section 10.3),
// a handful of the tree's nodes.  Each wave walks the set bits of its
// query's visibility mask instead of every suffix row: the keys and values
// of up to SB visible rows are requested at once, straight from the fp32
// suffix buffers, then folded into an online softmax one key at a time
// (scores reduced over the wave).  No LDS, no barrier: waves of one
// workgroup are independent here.  Workgroup `sub` of a query group takes
// 4*qpw queries, qpw per wave.
template <int D, int QT>
DEVI void attn_suffix(const AttnParams& p, int kvh, int qg, int b, int sub, int qpw) {
  constexpr int QN = QT * 16;
  const int w = threadIdx.x >> 6;
  const int G = p.Hq / p.Hkv;
  const int Tb = p.rlen ? p.rlen[b] : p.T;
  const int qi0 = qg * QN + 4 * qpw * sub + qpw * w;
  if (qpw == 4 && G % 4 == 0) {
    // the wave's four queries (qi0 is a multiple of 4) are heads of one row
    if (qi0 < G * Tb) attn_suffix_row<D, 4>(p, kvh, b, qi0);
    return;
  }
  for (int k = 0; k < qpw; ++k) {
    const int qi = qi0 + k;
    if (qi >= G * Tb) break;  // wave-uniform
    attn_suffix_query<D>(p, kvh, b, qi);
  }
}

// Unit u of a launch with `splits` context columns and ncol - splits suffix
// columns per (KV head, sequence): every context unit comes before every
// suffix unit in dispatch order, so the short suffix workgroups fill the end
// of a launch that runs in several rounds of workgroups rather than
// stretching one of the rounds.
DEVI void attn_unit(int u, int splits, int ncol, int Hkv, int B, int& s, int& kvh, int& b) {
  const int nctx = splits * Hkv * B;
  if (u < nctx) {
    s = u % splits;
    kvh = (u / splits) % Hkv;
    b = u / (splits * Hkv);
  } else {
    const int v = u - nctx, nsuf = ncol - splits;
    s = splits + v % nsuf;
    kvh = (v / nsuf) % Hkv;
    b = v / (nsuf * Hkv);
  }
}

// PFB: key blocks each wave has in flight.  With PFB = 1 two workgroups fit
// on a CU; with more, one.
template <int D, int QT, int QGW, int PFB>
__global__ __launch_bounds__(256, PFB > 1 ? 1 : 2) void attn_ctx_kernel(AttnParams p) {
  constexpr int DG = D / 4;   // dims per lane group
  constexpr int KSTEPS = D / 32;  // 32-dim k-steps of the 16x16x32 products
  constexpr int DT = D / 16;  // output dim tiles
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int G = p.Hq / p.Hkv;
  const int nq = G * p.T;
  // Query groups of 16 * QT query vectors.  A context workgroup serves QGW
  // of them: its waves form QGW sets of WPG waves, set q holding group
  // QGW * qgw + q, and the sets walk the same key blocks, so each block is
  // fetched from HBM once per workgroup (the second set's reads hit the CU's
  // cache).
  constexpr int WPG = 4 / QGW;  // waves per query group
  const int nqg = (nq + 16 * QT - 1) / (16 * QT);
  const int nqw = (nqg + QGW - 1) / QGW;           // query-group sets
  // Workgroup placement.  Workgroups are dispatched round-robin over the 8
  // XCDs (each with its own L2), in launch order.  The query-group sets of
  // one (sequence, KV head, split) read the same keys and values, so they
  // are given ids that land on the same XCD one after another: unit u =
  // (split, kv head, sequence) goes to XCD u % 8, and its sets take
  // consecutive places in that XCD's sequence.
  // context splits + suffix workgroups (four queries each for a chain,
  // sixteen for a tree)
  const int qpw = attn_suffix_qpw(p.anc != nullptr, p.B * p.Hkv * nqw);
  const int ncol = p.splits + 4 * QT * QGW / qpw;
  const int units = ncol * p.Hkv * p.B;
  const int id = blockIdx.x;
  const int n = id / 8;
  const int u = (n / nqw) * 8 + id % 8;
  if (u >= units) return;  // padding of the last XCD round
  const int qgw = n % nqw;
  int s, kvh, b;
  attn_unit(u, p.splits, ncol, p.Hkv, p.B, s, kvh, b);

  constexpr int QN = QT * 16;
  constexpr int OS = D + 4;  // padded row stride of the staged outputs
  __shared__ float s_m[4][QN];
  __shared__ float s_l[4][QN];
  __shared__ float s_o[4][QN * OS];
  if (s >= p.splits) {  // the step's own keys
    const int sw = s - p.splits;
    const int per = 4 * QT / qpw;  // suffix workgroups per query group
    const int grp = qgw * QGW + sw / per;
    if (grp >= nqg) return;
    attn_suffix<D, QT>(p, kvh, grp, b, sw % per, qpw);
    return;
  }
  const int qsub = w / WPG, kw = w % WPG;
  const int qg = qgw * QGW + qsub;  // this wave's query group
  const int rs = p.rstart ? p.rstart[b] : b * p.T;
  const int nqb = G * (p.rlen ? p.rlen[b] : p.T);  // this sequence's queries
  int L = p.kv_len[b];
  const int cap = p.kvm.table ? min(p.max_ctx, p.kvm.ppseq * KV_PAGE) : p.max_ctx;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  int chunk = (L + p.splits - 1) / p.splits;
  chunk = (chunk + 127) & ~127;
  const int kbeg = s * chunk;
  const int kend = min(L, kbeg + chunk);

  // ---- raw cache loads of one 32-key block, issued before they are needed:
  // K rows of the block's two key tiles and the V^T columns of its keys;
  // keys at or past kend read as zeros.  A block's 32 slots are contiguous
  // (one page holds two blocks), so one lookup places the whole block.
  const int vstride = kv_v_stride(p.kvm);
  uint4 kraw[PFB][2][DG / 8];
  uint4 vraw[PFB][DT];
  auto load_block = [&](int kb, int sl) {
    const uint16_t* kblk = p.kc + kv_k_off(p.kvm, p.Hkv, D, b, kvh, kb);
    const uint16_t* vblk = p.vc + kv_v_off(p.kvm, p.Hkv, D, b, kvh, 0, kb);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = blk_key(kb, kt, j);
      const bool ok = key < kend;
      const uint16_t* src = kblk + (size_t)(ok ? key - kb : 0) * D + g * DG;
#pragma unroll
      for (int e = 0; e < DG / 8; ++e) kraw[sl][kt][e] = ok ? *(const uint4*)(src + 8 * e) : make_uint4(0, 0, 0, 0);
    }
    const int k8 = kb + 8 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* src = vblk + (size_t)(dt * 16 + j) * vstride + (k8 < kend ? 8 * g : 0);
      vraw[sl][dt] = (k8 < kend) ? *(const uint4*)src : make_uint4(0, 0, 0, 0);
    }
  };
  // ---- queries: B operand of S^T = K Q^T; lane (j, g) holds query j's dims
  // g*DG + 8*ks + e for k-step ks.  Their loads go out before the key block's:
  // behind it they arrived last and held up the first products (B=1, T=4,
  // ctx 2048: 8.6 -> 7.3 us with the queries taken out entirely).
  float4 qraw[QT][DG / 4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qi = (qg * QT + qt) * 16 + j;
    const int i = (qi < nqb ? qi : 0) / G, gg = (qi < nqb ? qi : 0) % G;
    const float* src = p.q + (((size_t)(rs + i)) * p.Hq + kvh * G + gg) * D + g * DG;
#pragma unroll
    for (int e = 0; e < DG; e += 4) qraw[qt][e / 4] = *(const float4*)(src + e);
  }
#pragma unroll
  for (int sl = 0; sl < PFB; ++sl) {
    const int kb0 = kbeg + 32 * kw + sl * 32 * WPG;
    if (kb0 < kend) load_block(kb0, sl);
  }

  shortx8 qhi[QT][KSTEPS], qlo[QT][KSTEPS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qi = (qg * QT + qt) * 16 + j;
    float qv[DG];
    const float sc = qi < nqb ? p.scale : 0.f;  // queries past the sequence's are zeros
#pragma unroll
    for (int e = 0; e < DG; e += 4) {
      const float4 v = qraw[qt][e / 4];
      qv[e] = v.x * sc; qv[e + 1] = v.y * sc;
      qv[e + 2] = v.z * sc; qv[e + 3] = v.w * sc;
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        short hi, lo;
        split_bf16(qv[8 * ks + e], hi, lo);
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

  for (int kbase = kbeg + 32 * kw; kbase < kend; kbase += 32 * WPG * PFB) {
#pragma unroll
  for (int sl = 0; sl < PFB; ++sl) {
    const int kb = kbase + sl * 32 * WPG;
    if (kb >= kend) break;
    // ---- K operand (A of S^T): lane row j of tile kt is key blk_key(kb, kt, j);
    // the raw 16 bytes of k-step ks are its dims g*DG + 8*ks .. + 7
    shortx8 ka[2][KSTEPS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) ka[kt][ks] = __builtin_bit_cast(shortx8, kraw[sl][kt][ks]);
    // ---- V^T operand (A of O^T += V^T P^T): lane row j of dim tile dt is
    // dim dt*16 + j; its k index 8g + e is key kb + 8g + e (the raw 16 bytes)
    shortx8 va[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) va[dt] = __builtin_bit_cast(shortx8, vraw[sl][dt]);
    if (kb + 32 > kend) {  // wave-uniform: the block that holds kend
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kb + 8 * g + e >= kend) va[dt][e] = 0;  // never multiply a probability by data past the range
    }
    // the block PFB further on takes this one's raw registers as soon as they
    // are converted, so its latency overlaps the products of the blocks in
    // between; with PFB = 1 two workgroups per CU still fit (240 VGPRs, no
    // spills), measured at 32K context: 440 -> 409 us at T = 1
    if (kb + 32 * WPG * PFB < kend) load_block(kb + 32 * WPG * PFB, sl);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      floatx4 st[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          acc = mfma16x16x32(ka[kt][ks], qhi[qt][ks], acc);
          acc = mfma16x16x32(ka[kt][ks], qlo[qt][ks], acc);
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
      // B operand of the PV product: query j's probabilities of keys
      // kb + 8g + e, where S^T left them (kt = e / 4)
      shortx8 phi, plo;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = __expf(st[kt][e] - mnew);
          psum += pe;
          short hi, lo;
          split_bf16(pe, hi, lo);
          phi[4 * kt + e] = hi;
          plo[4 * kt + e] = lo;
        }
      lrun[qt] = lrun[qt] * factor + psum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[qt][dt] *= factor;
        o[qt][dt] = mfma16x16x32(va[dt], phi, o[qt][dt]);
        o[qt][dt] = mfma16x16x32(va[dt], plo, o[qt][dt]);
      }
    }
  }

  }
  // ---- merge the waves of each query group in LDS and write one partial
  // per query
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float l = lrun[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    lrun[qt] = l;
    if (g == 0) s_m[w][qt * 16 + j] = mrun[qt];
  }
  __syncthreads();
  const int w0 = qsub * WPG;  // first wave of this wave's group
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qq = qt * 16 + j;
    float mall = -INFINITY;
#pragma unroll
    for (int i = 0; i < WPG; ++i) mall = fmaxf(mall, s_m[w0 + i][qq]);
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
  for (int e = threadIdx.x; e < QGW * QN * D; e += 256) {
    const int grp = e / (QN * D), r = e % (QN * D);
    const int qq = r / D, dd = r % D;
    const int qi = ((qgw * QGW + grp) * QT) * 16 + qq;
    if (qi >= nqb) continue;
    const int o2 = qq * OS + dd;
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < WPG; ++i) t += s_o[grp * WPG + i][o2];
    p.part_o[(pbase + qi) * D + dd] = t;
  }
  if (threadIdx.x < QGW * QN) {
    const int grp = threadIdx.x / QN, qq = threadIdx.x % QN;
    const int qi = ((qgw * QGW + grp) * QT) * 16 + qq;
    if (qi < nqb) {
      float mall = -INFINITY, lsum = 0.f;
#pragma unroll
      for (int i = 0; i < WPG; ++i) {
        mall = fmaxf(mall, s_m[grp * WPG + i][qq]);
        lsum += s_l[grp * WPG + i][qq];
      }
      p.part_ml[2 * (pbase + qi)] = mall;
      p.part_ml[2 * (pbase + qi) + 1] = lsum;
    }
  }
}

// Context attention with the key blocks staged in LDS (D = 128, chain
// windows of 5..16 rows: two 16-query tiles per wave).  The register form
// above holds two raw key blocks per wave in flight, which with the two
// query tiles' operands and accumulators exceeds the 256 registers of a
// lane: one wave per SIMD, values moving between the register files, and the
// loop bound by issue rather than HBM.  Here each wave streams its 32-key
// block (K rows and V^T columns, 16 KiB) straight from the cache into its
// own LDS buffer with direct global-to-LDS loads and takes the matrix
// operands from there, so no register holds raw cache data: two workgroups
// fit per CU (two waves per SIMD), and one wave's products cover the other's
// waits.  The next block is requested as soon as the current one has been
// read out of LDS.
//
// LDS layout of a wave's buffer (16-byte chunks; XOR swizzles keep the 16
// lanes of a read on distinct banks):
//   K: row R = 16*kt + j holds key blk_key(kb, kt, j); its chunk c (dims
//      8c..8c+7) sits at R*16 + (c ^ j);
//   V^T: row r = 16*dt + j holds dim r for the block's 32 keys; its chunk g
//      (keys 8g..8g+7) sits at 512 + r*4 + (g ^ (j >> 2)).
typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

template <int QT>
__global__ __launch_bounds__(256, 2) void attn_ctx_lds_kernel(AttnParams p) {
  constexpr int D = 128, DG = D / 4, KSTEPS = D / 32, DT = D / 16;
  constexpr int QN = QT * 16, OS = D + 4;
  __shared__ __attribute__((aligned(16))) uint4 s_kv[4][1024];
  __shared__ float s_m[4][QN];
  __shared__ float s_l[4][QN];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int G = p.Hq / p.Hkv;
  const int nq = G * p.T;
  // grid decode of attn_ctx_kernel with one query group per workgroup
  const int nqw = (nq + QN - 1) / QN;
  const int qpw = attn_suffix_qpw(p.anc != nullptr, p.B * p.Hkv * nqw);
  const int ncol = p.splits + 4 * QT / qpw;
  const int units = ncol * p.Hkv * p.B;
  const int id = blockIdx.x;
  const int n = id / 8;
  const int u = (n / nqw) * 8 + id % 8;
  if (u >= units) return;
  const int qg = n % nqw;
  int s, kvh, b;
  attn_unit(u, p.splits, ncol, p.Hkv, p.B, s, kvh, b);
  if (s >= p.splits) {  // the step's own keys: suffix workgroup s - splits of this query group
    attn_suffix<D, QT>(p, kvh, qg, b, s - p.splits, qpw);
    return;
  }
  const int rs = p.rstart ? p.rstart[b] : b * p.T;
  const int nqb = G * (p.rlen ? p.rlen[b] : p.T);
  int L = p.kv_len[b];
  const int cap = p.kvm.table ? min(p.max_ctx, p.kvm.ppseq * KV_PAGE) : p.max_ctx;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  int chunk = (L + p.splits - 1) / p.splits;
  chunk = (chunk + 127) & ~127;
  const int kbeg = s * chunk;
  const int kend = min(L, kbeg + chunk);

  // ---- a block's K rows and V^T columns into this wave's buffer.  All 32
  // slots of a block are inside the cache (blocks start at multiples of 32
  // below kend; a page holds two blocks); slots at or past kend may hold
  // anything and are masked after the read.
  const int vstride = kv_v_stride(p.kvm);
  uint4* kbuf = &s_kv[w][0];
  uint4* vbuf = &s_kv[w][512];
  auto issue_k = [&](int kb, int pg) {
    const uint16_t* kblk = p.kc + kv_k_off_pg(p.kvm, p.Hkv, D, b, kvh, kb, pg);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int R = 4 * i + (lane >> 4), jj = R & 15;
      const int key = 8 * (jj >> 2) + 4 * (R >> 4) + (jj & 3);
      const int c = (lane & 15) ^ jj;
      __builtin_amdgcn_global_load_lds((gptr_t)(kblk + (size_t)key * D + 8 * c), (lptr_t)(kbuf + 64 * i), 16, 0, 0);
    }
  };
  auto issue_v = [&](int kb, int pg) {
    const uint16_t* vblk = p.vc + kv_v_off_pg(p.kvm, p.Hkv, D, b, kvh, 0, kb, pg);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 16 * i + (lane >> 2);
      const int gl = (lane & 3) ^ ((r & 15) >> 2);
      __builtin_amdgcn_global_load_lds((gptr_t)(vblk + (size_t)r * vstride + 8 * gl), (lptr_t)(vbuf + 64 * i), 16, 0,
                                       0);
    }
  };
  // page of a block (paged cache), looked up a block ahead so that no wait
  // for it sits between a block's loads
  auto page_of = [&](int kb) { return p.kvm.table ? kv_page(p.kvm, b, kb) : 0; };
  int kb = kbeg + 32 * w;
  if (kb < kend) {
    const int pg = page_of(kb);
    issue_k(kb, pg);
    issue_v(kb, pg);
  }

  // ---- queries: B operand of S^T = K Q^T; lane (j, g) holds query j's
  // dims g*DG + 8*ks + e for k-step ks (32 dims per step)
  shortx8 qhi[QT][KSTEPS], qlo[QT][KSTEPS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qi = (qg * QT + qt) * 16 + j;
    float qv[DG];
    if (qi < nqb) {
      const int i = qi / G, gg = qi % G;
      const float* src = p.q + (((size_t)(rs + i)) * p.Hq + kvh * G + gg) * D + g * DG;
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
      for (int e = 0; e < 8; ++e) {
        short hi, lo;
        split_bf16(qv[8 * ks + e], hi, lo);
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

  const shortx8* kb8 = (const shortx8*)kbuf;
  const shortx8* vb8 = (const shortx8*)vbuf;
  for (; kb < kend; kb += 128) {
    const bool more = kb + 128 < kend;
    const int pgn = more ? page_of(kb + 128) : 0;
    // this block has landed in LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const bool tail = kb + 32 > kend;  // wave-uniform
    // ---- the block's operands out of LDS, then the buffer takes the next
    // block, whose load overlaps this block's products and softmax
    // lane row j of key tile kt, dims g*DG + 8*ks + e: chunk 4g + ks
    shortx8 ka[2][KSTEPS];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) ka[kt][ks] = kb8[(16 * kt + j) * 16 + ((4 * g + ks) ^ j)];
    // lane row j of dim tile dt, keys kb + 8g + e: chunk g of V^T row 16dt + j
    shortx8 va[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) va[dt] = vb8[(16 * dt + j) * 4 + (g ^ (j >> 2))];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (more) {
      issue_k(kb + 128, pgn);
      issue_v(kb + 128, pgn);
    }
    if (tail) {
      // never multiply a probability by data past the range
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (kb + 8 * g + e >= kend) va[dt][e] = 0;
    }
    // ---- S^T = K Q^T for both query tiles
    floatx4 st[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          acc = mfma16x16x32(ka[kt][ks], qhi[qt][ks], acc);
          acc = mfma16x16x32(ka[kt][ks], qlo[qt][ks], acc);
        }
        st[qt][kt] = acc;
      }
    // ---- online softmax; st[qt][kt][e] is query j, key kb + 8g + 4kt + e
    // B operand of O^T += V^T P^T: lane (j, g) holds query j's probabilities
    // of keys kb + 8g + e, which is where S^T left them (kt = e / 4)
    shortx8 phi[QT], plo[QT];
    float factor[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      if (tail) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (kb + 8 * g + 4 * kt + e >= kend) st[qt][kt][e] = -INFINITY;
      }
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) bmax = fmaxf(bmax, st[qt][kt][e]);
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
      const float mnew = fmaxf(mrun[qt], bmax);
      factor[qt] = __expf(mrun[qt] - mnew);
      mrun[qt] = mnew;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = __expf(st[qt][kt][e] - mnew);
          psum += pe;
          short hi, lo;
          split_bf16(pe, hi, lo);
          phi[qt][4 * kt + e] = hi;
          plo[qt][4 * kt + e] = lo;
        }
      lrun[qt] = lrun[qt] * factor[qt] + psum;
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        o[qt][dt] *= factor[qt];
        o[qt][dt] = mfma16x16x32(va[dt], phi[qt], o[qt][dt]);
        o[qt][dt] = mfma16x16x32(va[dt], plo[qt], o[qt][dt]);
      }
  }

  // ---- merge the four waves' states and write one partial per query; the
  // key buffers (no load is outstanding after the last block) hold the
  // staged outputs, one query tile at a time
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float l = lrun[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    lrun[qt] = l;
    if (g == 0) s_m[w][qt * 16 + j] = mrun[qt];
  }
  __syncthreads();
  float* s_o = (float*)&s_kv[0][0];
  const size_t pbase = (((size_t)s * p.B + b) * p.Hkv + kvh) * nq;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qq = qt * 16 + j;
    const float mall = fmaxf(fmaxf(s_m[0][qq], s_m[1][qq]), fmaxf(s_m[2][qq], s_m[3][qq]));
    // a wave that saw no key has m = -inf and contributes nothing
    const float f = (mrun[qt] == -INFINITY) ? 0.f : __expf(mrun[qt] - mall);
    if (g == 0) s_l[w][qq] = lrun[qt] * f;
    if (qt > 0) __syncthreads();  // the previous tile's sums have been read
    float* dst = s_o + (w * 16 + j) * OS;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *(float4*)(dst + dt * 16 + 4 * g) =
          make_float4(o[qt][dt][0] * f, o[qt][dt][1] * f, o[qt][dt][2] * f, o[qt][dt][3] * f);
    __syncthreads();
    for (int e = threadIdx.x; e < 16 * D; e += 256) {
      const int q16 = e / D, dd = e % D;
      const int qi = (qg * QT + qt) * 16 + q16;
      if (qi >= nqb) continue;
      const int o2 = q16 * OS + dd;
      p.part_o[(pbase + qi) * D + dd] = s_o[o2] + s_o[16 * OS + o2] + s_o[32 * OS + o2] + s_o[48 * OS + o2];
    }
  }
  if (threadIdx.x < QN) {
    const int qq = threadIdx.x;
    const int qi = qg * QN + qq;
    if (qi < nqb) {
      const float mall = fmaxf(fmaxf(s_m[0][qq], s_m[1][qq]), fmaxf(s_m[2][qq], s_m[3][qq]));
      p.part_ml[2 * (pbase + qi)] = mall;
      p.part_ml[2 * (pbase + qi) + 1] = s_l[0][qq] + s_l[1][qq] + s_l[2][qq] + s_l[3][qq];
    }
  }
}

hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  const int nq = (p.Hq / p.Hkv) * p.T;
  const int QT = attn_query_tiles(nq, p.D), QGW = attn_groups_per_wg(nq, p.D);
  const int nqg = (nq + 16 * QT - 1) / (16 * QT);
  const int nqw = (nqg + QGW - 1) / QGW;
  if (p.T > 128) return hipErrorInvalidValue;  // the suffix workgroup holds up to 128 keys
  // (context splits + suffix workgroups) per (kv head, sequence), each
  // repeated per set of QGW query groups, laid out XCD by XCD (see the
  // kernel)
  const int qpw = attn_suffix_qpw(p.anc != nullptr, p.B * p.Hkv * nqw);
  const int units = (p.splits + 4 * QT * QGW / qpw) * p.Hkv * p.B;
  const dim3 grid(((units + 7) / 8) * 8 * nqw);
  if (p.D == 128) {
    if (QT == 2) attn_ctx_lds_kernel<2><<<grid, 256, 0, s>>>(p);
    else attn_ctx_kernel<128, 1, 1, 1><<<grid, 256, 0, s>>>(p);
  } else {
    if (QT == 2) attn_ctx_kernel<64, 2, 1, 2><<<grid, 256, 0, s>>>(p);
    else if (QGW == 2) attn_ctx_kernel<64, 1, 2, 1><<<grid, 256, 0, s>>>(p);
    else attn_ctx_kernel<64, 1, 1, 1><<<grid, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

// One workgroup per (row i, KV head, sequence); wave gg handles query head
// kvh * G + gg.  Lanes read the split statistics in parallel (two splits per
// lane) and, in the same round of requests, the outputs of up to NF splits
// (all of them for NF >= nsplit), so the kernel waits for memory once; the
// weights reach the lanes by shuffles.  More splits than NF are added in
// further rounds of U.
template <int D, int NF>
__global__ __launch_bounds__(512) void attn_combine_kernel(CombineParams p) {
  constexpr int PL = D / 64;  // dims per lane
  constexpr int U = 8;        // splits per round beyond the first NF
  const int i = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, gg = threadIdx.x >> 6;
  const int G = p.Hq / p.Hkv;
  const int nq = G * p.T;
  if (p.rlen && i >= p.rlen[b]) return;  // ragged: past this sequence's rows
  const int qi = i * G + gg;
  const int m = (p.rstart ? p.rstart[b] : b * p.T) + i;
  const int ns = p.nsplit;
  const size_t stride = (size_t)p.B * p.Hkv * nq;  // between splits, in queries
  const size_t q0 = ((size_t)b * p.Hkv + kvh) * nq + qi;

  float ms[2], ls[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int sp = lane + 64 * c;
    ms[c] = -INFINITY;
    ls[c] = 0.f;
    if (sp < ns) {
      ms[c] = p.part_ml[2 * (sp * stride + q0)];
      ls[c] = p.part_ml[2 * (sp * stride + q0) + 1];
    }
  }
  // the first NF splits' outputs, requested with the statistics
  float v0[NF][PL];
#pragma unroll
  for (int u = 0; u < NF; ++u) {
    const int sp = u < ns ? u : ns - 1;
    const float* src = p.part_o + (sp * stride + q0) * D;
#pragma unroll
    for (int e = 0; e < PL; ++e) v0[u][e] = src[lane + 64 * e];
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int c = 0; c < 2; ++c)
    if (ls[c] > 0.f) mloc = fmaxf(mloc, ms[c]);
  const float mstar = wave_max(mloc);  // the suffix split always has mass
  float wt[2], lsum = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    wt[c] = (ls[c] > 0.f) ? __expf(ms[c] - mstar) : 0.f;
    lsum += wt[c] * ls[c];
  }
  const float l = wave_sum(lsum);

  float acc[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int u = 0; u < NF; ++u) {
    const float wsp = __shfl(u < 64 ? wt[0] : wt[1], u & 63, 64);
    if (u < ns) {
#pragma unroll
      for (int e = 0; e < PL; ++e) acc[e] += wsp * v0[u][e];
    }
  }
  for (int sp0 = NF; sp0 < ns; sp0 += U) {
    float v[U][PL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = sp0 + u < ns ? sp0 + u : ns - 1;
      const float* src = p.part_o + (sp * stride + q0) * D;
#pragma unroll
      for (int e = 0; e < PL; ++e) v[u][e] = src[lane + 64 * e];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = sp0 + u;
      const float wsp = __shfl(sp < 64 ? wt[0] : wt[1], sp & 63, 64);
      if (sp < ns) {
#pragma unroll
        for (int e = 0; e < PL; ++e) acc[e] += wsp * v[u][e];
      }
    }
  }
  float* dst = p.out + ((size_t)m * p.Hq + kvh * G + gg) * D;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < PL; ++e) {
    const float v = acc[e] * inv;
    dst[lane + 64 * e] = v;
    if (p.xs) {
      // the O projection's activation planes, as its split would write them
      const size_t K = (size_t)p.Hq * D, col = (size_t)(kvh * G + gg) * D + lane + 64 * e;
      short h, lo;
      split_bf16(v, h, lo);
      p.xs[(size_t)m * K + col] = (uint16_t)h;
      p.xs[((size_t)p.M + m) * K + col] = (uint16_t)lo;
    }
  }
}

hipError_t launch_attn_combine(const CombineParams& p, hipStream_t s) {
  const int G = p.Hq / p.Hkv;
  if (G > 8 || p.nsplit > 128) return hipErrorInvalidValue;
  dim3 grid(p.T, p.Hkv, p.B);
  // the splits' outputs all in one round of requests when they fit (32 x 2
  // floats per lane at D = 128), and no more requests than splits below 9
  // (requests past the last split re-read it)
  if (p.D == 128) {
    if (p.nsplit <= 4) attn_combine_kernel<128, 4><<<grid, 64 * G, 0, s>>>(p);
    else if (p.nsplit <= 8) attn_combine_kernel<128, 8><<<grid, 64 * G, 0, s>>>(p);
    else if (p.nsplit <= 16) attn_combine_kernel<128, 16><<<grid, 64 * G, 0, s>>>(p);
    else if (p.nsplit <= 24) attn_combine_kernel<128, 24><<<grid, 64 * G, 0, s>>>(p);
    else if (p.nsplit <= 32) attn_combine_kernel<128, 32><<<grid, 64 * G, 0, s>>>(p);
    else attn_combine_kernel<128, 8><<<grid, 64 * G, 0, s>>>(p);
  } else {
    if (p.nsplit <= 16) attn_combine_kernel<64, 16><<<grid, 64 * G, 0, s>>>(p);
    else if (p.nsplit <= 32) attn_combine_kernel<64, 32><<<grid, 64 * G, 0, s>>>(p);
    else attn_combine_kernel<64, 8><<<grid, 64 * G, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace sv
