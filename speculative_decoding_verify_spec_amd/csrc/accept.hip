// Speculative-sampling accept, residual resample, bonus token and KV commit.
//
// CS349E Lecture 6 ("Optimizing Autoregressive Decode"), section 6.2 steps
// 3-5: accept draft x_i when u_i < p_i(x_i)/q_i(x_i) (evaluated as
// u_i * q_i(x_i) < p_i(x_i), the form the Kimi-K3 tuning page describes), stop
// at the first rejection, then draw from norm(max(0, p_{n+1} - q_{n+1})) or,
// when every draft survived, a bonus token from p_{gamma+1}.  Greedy
// (section 7.4): longest prefix where draft == argmax, then that argmax.
// Token trees (section 10.3): walk from the root, testing each node's children
// in order against a running residual (see the sampled tree walk below).
//
// The vocabulary is cut into chunks of CH entries so a handful of rows still
// fills the GPU:
//   1. rowstats  (grid chunks x rows): per-chunk max and sum of exp (or argmax)
//   2. residual  (grid chunks x sequences): every workgroup combines the row
//      statistics, replays the accept tests (cheap: gamma lookups), and sums
//      the residual over its chunk
//   3. sample    (one workgroup per sequence): inverse CDF over chunk sums,
//      then a scan inside the chosen chunk; writes tokens and the commit.
// Sampling is inverse CDF in token-id order: the token is the smallest x with
// sum_{y<=x} r(y) > u * R.  Greedy ties go to the lowest id.  A residual with
// no mass in floating point falls back to p.
#include "common.h"
#include "launch.h"

namespace sv {

constexpr int CH = 4096;
int accept_chunks(int V) { return (V + CH - 1) / CH; }

// Block-wide sum / max for blockDim.x a multiple of 64 (<= 1024).
template <typename Tv>
DEVI Tv block_sum(Tv v, Tv* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  Tv t = 0;
  for (int i = 0; i < nw; ++i) t += sh[i];
  return t;
}
DEVI float block_max(float v, float* sh) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, sh[i]);
  return t;
}

DEVI bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// ---------------------------------------------------------------- pass 1
template <bool GREEDY>
__global__ __launch_bounds__(256) void accept_rowstats_kernel(AcceptParams p) {
  __shared__ float shf[16];
  __shared__ int shi[16];
  const int c = blockIdx.x, row = blockIdx.y;
  const float* z = p.logits + (size_t)row * p.V;
  const int y0 = c * CH, y1 = min(p.V, y0 + CH);
  float* out = p.rowstat + ((size_t)row * p.nch + c) * 2;
  // the thread's CH/256 entries are loaded at once (one memory latency), then
  // reduced from registers in ascending token order
  constexpr int PER = CH / 256;
  float zv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int y = y0 + threadIdx.x + 256 * e;
    zv[e] = y < y1 ? z[y] : 0.f;
  }
  if (GREEDY) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int y = y0 + threadIdx.x + 256 * e;
      if (y < y1 && better(zv[e], y, bv, bi)) { bv = zv[e]; bi = y; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((threadIdx.x & 63) == 0) { shf[threadIdx.x >> 6] = bv; shi[threadIdx.x >> 6] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
      float v0 = shf[0];
      int i0 = shi[0];
      for (int i = 1; i < 4; ++i)
        if (better(shf[i], shi[i], v0, i0)) { v0 = shf[i]; i0 = shi[i]; }
      out[0] = v0;
      out[1] = __int_as_float(i0);
    }
    return;
  }
  const float Tt = p.temperature;
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (y0 + (int)threadIdx.x + 256 * e < y1) mx = fmaxf(mx, zv[e] / Tt);
  mx = block_max(mx, shf);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (y0 + (int)threadIdx.x + 256 * e < y1) s += expf(zv[e] / Tt - mx);
  s = block_sum(s, shf);
  if (threadIdx.x == 0) { out[0] = mx; out[1] = s; }
}

// Combine the chunk statistics of one row: M = max, S = sum exp(z/T - M).
// The chunk loads are issued 16 at a time (one thread reads them all).
DEVI void row_ms(const AcceptParams& p, int row, float& M, float& S) {
  const float2* st = (const float2*)(p.rowstat + (size_t)row * p.nch * 2);
  M = -INFINITY;
  S = 0.f;
  for (int c0 = 0; c0 < p.nch; c0 += 16) {
    float2 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = c0 + i < p.nch ? st[c0 + i] : make_float2(-INFINITY, 0.f);
    float m = M;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, v[i].x);
    // rescale the running sum to the new maximum, then add this batch
    S = (M == -INFINITY) ? 0.f : S * expf(M - m);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (v[i].y != 0.f) S += v[i].y * expf(v[i].x - m);
    M = m;
  }
}
// Combine the chunk argmaxes of one row (loads issued 16 at a time).
DEVI void row_argmax(const AcceptParams& p, int row, int& idx) {
  const float2* st = (const float2*)(p.rowstat + (size_t)row * p.nch * 2);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int c0 = 0; c0 < p.nch; c0 += 16) {
    float2 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = c0 + i < p.nch ? st[c0 + i] : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (c0 + i >= p.nch) break;
      const int k = __float_as_int(v[i].y);
      if (better(v[i].x, k, bv, bi)) { bv = v[i].x; bi = k; }
    }
  }
  idx = bi;
}

DEVI int clamp_token(const AcceptParams& p, int x, bool& bad) {
  bad = (x < 0 || x >= p.V);
  if (bad) atomicOr(p.flags, FLAG_TOKEN_RANGE);
  return x < 0 ? 0 : (x >= p.V ? p.V - 1 : x);
}

// ---------------------------------------------------------------- top-k / top-p
// CS349E Lecture 6, section 7.3: the target is the adjusted distribution
// softmax(z / T), cut to the top-k tokens, renormalised, cut to the top-p
// nucleus, renormalised.  A row's kept set is a prefix of its tokens in
// likelihood order (larger logit first, equal logits by lower id), found by
// a radix selection over keys that order the logits, one 8-bit digit per
// pass from the top: every chunk workgroup counts the candidates of each
// digit value (tokens, and their mass exp(z/T - M) in fp64), the next pass
// merges the chunk counts and fixes the digit.  Top-k selects by count; the
// nucleus then selects by mass among the top-k tokens.  After the last digit
// the threshold key tau is exact; of the tokens whose key equals tau the
// first j by id are kept, j being what the count or the mass still needs.

// a larger float gets a larger key
DEVI uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
DEVI float key_float(uint32_t k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }
DEVI bool sel_keep(uint32_t tau, int cut, uint32_t key, int y) { return key > tau || (key == tau && y <= cut); }

// Keep rule of a row for the sampling kernels: everything when no
// adjustment applies.
struct RowRule {
  uint32_t tau;
  int cut;
};
DEVI RowRule row_rule(const AcceptParams& p, int row) {
  if (!p.fres) return RowRule{0u, 0x7fffffff};
  return RowRule{p.fres[row].tau, p.fres[row].cut};
}
// adjusted target probability of token y of a row with statistics (M, S)
DEVI float pval(const AcceptParams& p, const RowRule& r, float zy, int y, float M, float S) {
  const float v = expf(zy / p.temperature - M) / S;
  return sel_keep(r.tau, r.cut, order_key(zy), y) ? v : 0.f;
}

struct SelArgs {
  int row0;   // first row of this batch
  int phase;  // 0 top-k (by count), 1 top-p (by mass)
  int digit;  // 0..3: digit this pass counts; 4: finish
};

// Merge the previous digit's chunk counts of batch row rb and fix that digit.
// blockDim.x == 256: thread t sums bin t over the chunks, then suffix sums
// over the bins (from the top) locate the bin where the count or the mass
// from the top reaches what is still needed.  Leaves the state after the
// digit in *st, the digit in *bin, and the merged bins in s_cnt / s_mass;
// ends synchronised.
DEVI void sel_merge(const AcceptParams& p, const SelArgs& a, int rb, SelState* st, int* bin, uint32_t* s_cnt,
                    double* s_mass) {
  __shared__ uint32_t sc[256];
  __shared__ double sm[256];
  __shared__ int s_pick, s_low;
  const int t = threadIdx.x;
  const int pd = (a.digit - 1) & 1;
  const size_t hb = ((size_t)pd * SEL_ROWS + rb) * p.nch * 256;
  uint32_t cn = 0;
  double ms = 0.0;
#pragma unroll 8
  for (int c = 0; c < p.nch; ++c) {
    cn += p.fcnt[hb + (size_t)c * 256 + t];
    ms += p.fmass[hb + (size_t)c * 256 + t];
  }
  s_cnt[t] = cn;
  s_mass[t] = ms;
  sc[t] = cn;
  sm[t] = ms;
  if (t == 0) {
    s_pick = -1;
    s_low = 256;
  }
  __syncthreads();
  // inclusive suffix sums: sc[t] = sum of bins >= t
  for (int o = 1; o < 256; o <<= 1) {
    const uint32_t ac = t + o < 256 ? sc[t + o] : 0u;
    const double am = t + o < 256 ? sm[t + o] : 0.0;
    __syncthreads();
    sc[t] += ac;
    sm[t] += am;
    __syncthreads();
  }
  SelState s = p.fstate[pd * SEL_ROWS + rb];
  if (a.phase == 1 && s.rem < 0.0) s.rem = (double)p.top_p * sm[0];
  // the highest bin whose suffix reaches the target
  const bool hit = a.phase == 0 ? (sc[t] >= s.need) : (cn > 0 && sm[t] >= s.rem);
  if (hit) atomicMax(&s_pick, t);
  if (cn > 0) atomicMin(&s_low, t);
  __syncthreads();
  if (t == 0) {
    const int shift = 24 - 8 * (a.digit - 1);
    int b = s_pick;
    if (a.phase == 0) {
      if (b < 0) b = 0;
      const uint32_t cum = b < 255 ? sc[b + 1] : 0u;
      s.need -= cum;
      s.above += b < 255 ? sm[b + 1] : 0.0;
    } else if (b < 0) {
      // rounding left the total short of the target: the lowest occupied
      // bin, taken whole
      b = s_low < 256 ? s_low : 0;
      s.above += b < 255 ? sm[b + 1] : 0.0;
      s.rem = INFINITY;
    } else {
      const double cum = b < 255 ? sm[b + 1] : 0.0;
      s.rem -= cum;
      s.above += cum;
    }
    s.prefix |= (uint32_t)b << shift;
    *st = s;
    *bin = b;
  }
  __syncthreads();
}

// One digit of the selection over one chunk of one row.  Grid (nch, rows).
__global__ __launch_bounds__(256) void accept_select_kernel(AcceptParams p, SelArgs a) {
  __shared__ uint32_t s_cnt[256];
  __shared__ double s_mass[256];
  __shared__ SelState st;
  __shared__ int s_bin;
  const int c = blockIdx.x, rb = blockIdx.y, row = a.row0 + rb, t = threadIdx.x;
  if (a.digit == 0) {
    if (t == 0) st = SelState{0u, (uint32_t)p.top_k, -1.0, 0.0};
  } else {
    sel_merge(p, a, rb, &st, &s_bin, s_cnt, s_mass);
  }
  s_cnt[t] = 0;
  s_mass[t] = 0.0;
  __syncthreads();
  const SelState s = st;
  // phase 1 selects among the top-k set
  const uint32_t tk = a.phase == 1 ? p.fres[row].tau_k : 0u;
  const int ck = a.phase == 1 ? p.fres[row].cut_k : 0x7fffffff;
  float M, S;
  row_ms(p, row, M, S);
  const float Tt = p.temperature;
  const int shift = 24 - 8 * a.digit;
  const float* z = p.logits + (size_t)row * p.V;
  const int y1 = min(p.V, (c + 1) * CH);
  constexpr int PER = CH / 256;
  float zv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int y = c * CH + t + 256 * e;
    zv[e] = y < y1 ? z[y] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int y = c * CH + t + 256 * e;
    if (y >= y1) break;
    const float zy = zv[e];
    const uint32_t key = order_key(zy);
    if (a.digit > 0 && (key >> (shift + 8)) != (s.prefix >> (shift + 8))) continue;
    if (!sel_keep(tk, ck, key, y)) continue;
    const int bn = (key >> shift) & 255;
    atomicAdd(&s_cnt[bn], 1u);
    atomicAdd(&s_mass[bn], (double)expf(zy / Tt - M));
  }
  __syncthreads();
  const size_t hb = (((size_t)(a.digit & 1) * SEL_ROWS + rb) * p.nch + c) * 256;
  p.fcnt[hb + t] = s_cnt[t];
  p.fmass[hb + t] = s_mass[t];
  if (c == 0 && t == 0) p.fstate[(a.digit & 1) * SEL_ROWS + rb] = s;
}

// Fix the last digit, then find the j-th token (by id) whose key equals the
// threshold and write the row's rule.  Grid (rows), 256 threads.
__global__ __launch_bounds__(256) void accept_select_finish_kernel(AcceptParams p, SelArgs a) {
  constexpr int PER = CH / 256;
  __shared__ uint32_t s_cnt[256];
  __shared__ double s_mass[256];
  __shared__ SelState st;
  __shared__ int s_bin, s_chunk, s_rank, s_cut;
  __shared__ uint32_t scan[256];
  const int rb = blockIdx.x, row = a.row0 + rb, t = threadIdx.x;
  sel_merge(p, a, rb, &st, &s_bin, s_cnt, s_mass);
  const uint32_t tau = st.prefix;
  float M, S;
  row_ms(p, row, M, S);
  const float Tt = p.temperature;
  const uint32_t ties = s_cnt[s_bin];
  if (t == 0) {
    uint32_t j;
    if (a.phase == 0) {
      j = st.need;
    } else {
      const double e = (double)expf(key_float(tau) / Tt - M);
      const double need = st.rem / e;
      j = (need >= (double)ties) ? ties : (uint32_t)ceil(need);
    }
    j = j < 1 ? 1 : (j > ties ? ties : j);
    // chunk and rank of the j-th tie, from the last digit's chunk counts
    // (staged in scan[] by all threads below)
    s_rank = (int)j;
  }
  __syncthreads();
  {
    const size_t hb = ((size_t)1 * SEL_ROWS + rb) * p.nch * 256 + s_bin;
    for (int c = t; c < p.nch; c += 256) scan[c] = p.fcnt[hb + (size_t)c * 256];
  }
  __syncthreads();
  if (t == 0) {
    const uint32_t j = (uint32_t)s_rank;
    uint32_t cum = 0;
    int ch = p.nch - 1;
    for (int c = 0; c < p.nch; ++c) {
      const uint32_t k = scan[c];
      if (cum + k >= j) { ch = c; break; }
      cum += k;
    }
    s_chunk = ch;
    s_rank = (int)(j - cum);
    s_cut = ch * CH + CH - 1;
    const double mass = st.above + (double)j * (double)expf(key_float(tau) / Tt - M);
    if (a.phase == 0) p.fres[row].mass_k = mass;
  }
  __syncthreads();
  // in-chunk scan: thread t owns ids chunk*CH + PER*t .. + PER - 1
  const uint32_t tk = a.phase == 1 ? p.fres[row].tau_k : 0u;
  const int ck = a.phase == 1 ? p.fres[row].cut_k : 0x7fffffff;
  const float* z = p.logits + (size_t)row * p.V;
  const int y0 = s_chunk * CH + PER * t;
  uint32_t mine = 0;
  for (int e = 0; e < PER; ++e) {
    const int y = y0 + e;
    if (y < p.V) {
      const uint32_t key = order_key(z[y]);
      mine += (key == tau && sel_keep(tk, ck, key, y)) ? 1u : 0u;
    }
  }
  scan[t] = mine;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const uint32_t add = t >= o ? scan[t - o] : 0u;
    __syncthreads();
    scan[t] += add;
    __syncthreads();
  }
  const int excl = (int)(scan[t] - mine);
  if (excl < s_rank && s_rank <= excl + (int)mine) {
    int r = s_rank - excl;
    for (int e = 0; e < PER; ++e) {
      const int y = y0 + e;
      if (y >= p.V) break;
      const uint32_t key = order_key(z[y]);
      if (key == tau && sel_keep(tk, ck, key, y) && --r == 0) {
        s_cut = y;
        break;
      }
    }
  }
  __syncthreads();
  if (t == 0) {
    p.fres[row].tau = tau;
    p.fres[row].cut = s_cut;
    if (a.phase == 0) {
      p.fres[row].tau_k = tau;
      p.fres[row].cut_k = s_cut;
    }
  }
}

// Rows whose adjustment has no top-k step keep everything before top-p.
__global__ void accept_select_init_kernel(AcceptParams p, int row0, int nrows) {
  const int rb = blockIdx.x * blockDim.x + threadIdx.x;
  if (rb >= nrows) return;
  p.fres[row0 + rb] = SelRule{0u, 0x7fffffff, 0u, 0x7fffffff, 0.0};
}

// Replace each chunk's statistics by those of the kept tokens, relative to
// the row max (kept always: it is the first token in likelihood order), so
// that row_ms and the chunk sums describe the adjusted target.  Grid (nch,
// rows).  Other chunks' entries may be rewritten meanwhile: their maximum is
// M either way.
__global__ __launch_bounds__(256) void accept_select_apply_kernel(AcceptParams p, int row0) {
  __shared__ float shf[16];
  const int c = blockIdx.x, row = row0 + blockIdx.y;
  float M, S;
  row_ms(p, row, M, S);
  const RowRule r = row_rule(p, row);
  const float Tt = p.temperature;
  const float* z = p.logits + (size_t)row * p.V;
  const int y1 = min(p.V, (c + 1) * CH);
  constexpr int PER = CH / 256;
  float zv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int y = c * CH + threadIdx.x + 256 * e;
    zv[e] = y < y1 ? z[y] : 0.f;
  }
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int y = c * CH + threadIdx.x + 256 * e;
    if (y >= y1) break;
    if (sel_keep(r.tau, r.cut, order_key(zv[e]), y)) acc += expf(zv[e] / Tt - M);
  }
  acc = block_sum(acc, shf);
  if (threadIdx.x == 0) {
    p.rowstat[((size_t)row * p.nch + c) * 2] = M;
    p.rowstat[((size_t)row * p.nch + c) * 2 + 1] = acc;
  }
}

// ---------------------------------------------------------------- chain layout
// Sequence b of a chain has T rows from row b*T, and its drafts' q rows from
// b*(T-1); a ragged layout (DeepSeek-V4 analysis page, section 4) gives each
// sequence its own first row, length and first q row.  Lengths are clamped
// to [1, T] and rows to the buffers (FLAG_LAYOUT marks a clamp).
DEVI int chain_len(const AcceptParams& p, int b) {
  if (!p.rlen) return p.T;
  const int l = p.rlen[b];
  return l < 1 ? 1 : (l > p.T ? p.T : l);
}
DEVI int chain_row(const AcceptParams& p, int b, int i) {
  if (!p.rstart) return b * p.T + i;
  const int r = p.rstart[b] + i;
  return r < 0 ? 0 : (r >= p.rows ? p.rows - 1 : r);
}
DEVI int chain_qrow(const AcceptParams& p, int b, int i) {
  if (!p.qstart) return b * (p.T - 1) + i;
  const int r = p.qstart[b] + i;
  return r < 0 ? 0 : (r >= p.qrows ? p.qrows - 1 : r);
}
// FLAG_LAYOUT when sequence b's rows or q rows leave their buffers
DEVI void check_layout(const AcceptParams& p, int b) {
  if (!p.rstart) return;
  const int l = p.rlen[b], r = p.rstart[b], qr = p.qstart ? p.qstart[b] : 0;
  if (l < 1 || l > p.T || r < 0 || r + l > p.rows || (p.qstart && (qr < 0 || qr + l - 1 > p.qrows)))
    atomicOr(p.flags, FLAG_LAYOUT);
}

// ---------------------------------------------------------------- chain, pass 2
__global__ __launch_bounds__(256) void accept_chain_residual_kernel(AcceptParams p) {
  __shared__ float sM[128], sS[128];
  __shared__ float s_pz[128], s_qx[128], s_u[128];
  __shared__ int s_bad[128];
  __shared__ int sn;
  __shared__ float shf[16];
  const int c = blockIdx.x, b = blockIdx.y;
  const int T = chain_len(p, b), gamma = T - 1;
  // thread i: row i's statistics, then the inputs of draft i's accept test
  // (token, target and draft probability, uniform), all rows in parallel so
  // that the sequential decisions below read LDS only
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    float M, S;
    const int row = chain_row(p, b, i);
    row_ms(p, row, M, S);
    sM[i] = M;
    sS[i] = S;
    if (c == 0) { p.rowms[2 * row] = M; p.rowms[2 * row + 1] = S; }
    if (i < gamma) {
      const int xr = p.tokens[chain_row(p, b, i + 1)];
      const bool bad = xr < 0 || xr >= p.V;
      const int x = bad ? 0 : xr;
      s_pz[i] = pval(p, row_rule(p, row), p.logits[(size_t)row * p.V + x], x, M, S);
      s_qx[i] = p.q[(size_t)chain_qrow(p, b, i) * p.V + x];
      s_u[i] = philox_uniform(p.seed, p.round, b, i);
      s_bad[i] = bad;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (c == 0) check_layout(p, b);
    int n = 0;
    for (int i = 0; i < gamma; ++i) {
      if (s_bad[i]) {  // a token outside the vocabulary ends the chain
        atomicOr(p.flags, FLAG_TOKEN_RANGE);
        break;
      }
      if (s_u[i] * s_qx[i] < s_pz[i]) ++n;
      else break;
    }
    sn = n;
    if (c == 0) p.nacc[b] = n;
  }
  __syncthreads();
  const int n = sn;
  const float* z = p.logits + (size_t)chain_row(p, b, n) * p.V;
  const float* q = (n < gamma) ? p.q + (size_t)chain_qrow(p, b, n) * p.V : nullptr;
  const float M = sM[n], S = sS[n];
  const RowRule rr = row_rule(p, chain_row(p, b, n));
  const int y0 = c * CH, y1 = min(p.V, y0 + CH);
  // the chunk's logits (and draft probabilities) of this thread, loaded at
  // once, then summed in ascending token order
  constexpr int PER = CH / 256;
  float zv[PER], qv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int y = y0 + threadIdx.x + 256 * e;
    zv[e] = y < y1 ? z[y] : 0.f;
    qv[e] = (q && y < y1) ? q[y] : 0.f;
  }
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int y = y0 + threadIdx.x + 256 * e;
    if (y < y1) {
      const float pv = pval(p, rr, zv[e], y, M, S);
      acc += q ? fmaxf(0.f, pv - qv[e]) : pv;
    }
  }
  acc = block_sum(acc, shf);
  if (threadIdx.x == 0) p.rsum[(size_t)b * p.nch + c] = acc;
}

// Write the sequence's outputs: n accepted drafts, the extra token, -1 padding,
// and the chain commit kv_len + n + 1.
DEVI void write_chain_outputs(const AcceptParams& p, int b, int n, int extra) {
  const int T = p.T;
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    int v = -1;
    if (i < n) v = p.tokens[chain_row(p, b, i + 1)];
    else if (i == n) v = extra;
    p.out_tokens[b * T + i] = v;
  }
  if (threadIdx.x == 0) {
    p.num_accepted[b] = n;
    if (p.kv_len_out) p.kv_len_out[b] = p.kv_len[b] + n + 1;
  }
}

// ---------------------------------------------------------------- chain, pass 3
__global__ __launch_bounds__(256) void accept_chain_sample_kernel(AcceptParams p) {
  constexpr int PER = CH / 256;
  __shared__ double shd[16];
  __shared__ int s_c, s_deg, s_tok;
  __shared__ double s_base, s_t;
  const int b = blockIdx.x;
  const int T = chain_len(p, b), gamma = T - 1;
  const int n = p.nacc[b];
  const int row = chain_row(p, b, n);
  const float M = p.rowms[2 * row], S = p.rowms[2 * row + 1];
  if (threadIdx.x == 0) {
    double R = 0.0;
    for (int c = 0; c < p.nch; ++c) R += (double)p.rsum[(size_t)b * p.nch + c];
    int deg = !(R > 0.0);
    const float* st = p.rowstat + (size_t)row * p.nch * 2;
    if (deg) {
      R = 0.0;
      for (int c = 0; c < p.nch; ++c) R += (double)(st[2 * c + 1] * expf(st[2 * c] - M) / S);
    }
    const double t = (double)philox_uniform(p.seed, p.round, b, gamma) * R;
    double cum = 0.0;
    int cs = p.nch - 1;
    double base = 0.0;
    for (int c = 0; c < p.nch; ++c) {
      const double v = deg ? (double)(st[2 * c + 1] * expf(st[2 * c] - M) / S)
                           : (double)p.rsum[(size_t)b * p.nch + c];
      if (cum + v > t) { cs = c; base = cum; break; }
      cum += v;
      base = cum;
    }
    s_c = cs; s_deg = deg; s_base = base; s_t = t; s_tok = 0x7fffffff;
  }
  __syncthreads();
  const int c = s_c;
  const bool use_res = (n < gamma) && !s_deg;
  const float* z = p.logits + (size_t)row * p.V;
  const float* q = use_res ? p.q + (size_t)chain_qrow(p, b, n) * p.V : nullptr;
  const int y0 = c * CH + threadIdx.x * PER;
  const RowRule rr = row_rule(p, row);
  float r[PER];
  float loc = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int y = y0 + e;
    float v = 0.f;
    if (y < p.V) {
      const float pv = pval(p, rr, z[y], y, M, S);
      v = q ? fmaxf(0.f, pv - q[y]) : pv;
    }
    r[e] = v;
    loc += v;
  }
  // exclusive scan of the per-thread sums (double)
  __shared__ double scan[256];
  scan[threadIdx.x] = (double)loc;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    double add = threadIdx.x >= o ? scan[threadIdx.x - o] : 0.0;
    __syncthreads();
    scan[threadIdx.x] += add;
    __syncthreads();
  }
  const double excl = scan[threadIdx.x] - (double)loc;
  const double t = s_t;
  double run = s_base + excl;
  if (run <= t && run + (double)loc > t) {
    int found = -1;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      run += (double)r[e];
      if (found < 0 && run > t) found = y0 + e;
    }
    if (found >= 0) atomicMin(&s_tok, found);
  }
  __syncthreads();
  if (s_tok == 0x7fffffff) {
    // rounding left the crossing past the chunk's recomputed total: the last
    // token of the chunk with positive mass is the answer
    int last = -1;
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (r[e] > 0.f && y0 + e < p.V) last = y0 + e;
    __shared__ int s_last;
    if (threadIdx.x == 0) s_last = -1;
    __syncthreads();
    if (last >= 0) atomicMax(&s_last, last);
    __syncthreads();
    if (threadIdx.x == 0) s_tok = s_last >= 0 ? s_last : c * CH;
    __syncthreads();
  }
  write_chain_outputs(p, b, n, s_tok);
}

// ---------------------------------------------------------------- chain, greedy
__global__ __launch_bounds__(128) void accept_chain_greedy_kernel(AcceptParams p) {
  __shared__ int am[128], s_tok[128];
  __shared__ int s_n;
  const int b = blockIdx.x, T = chain_len(p, b), gamma = T - 1;
  // every row's argmax and every draft token in parallel; the sequential
  // comparisons below read LDS only
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    row_argmax(p, chain_row(p, b, i), am[i]);
    if (i < gamma) s_tok[i] = p.tokens[chain_row(p, b, i + 1)];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    check_layout(p, b);
    int n = 0;
    while (n < gamma) {
      const int x = s_tok[n];
      if (x < 0 || x >= p.V) {  // a token outside the vocabulary ends the chain
        atomicOr(p.flags, FLAG_TOKEN_RANGE);
        break;
      }
      if (x != am[n]) break;
      ++n;
    }
    s_n = n;
  }
  __syncthreads();
  write_chain_outputs(p, b, s_n, am[s_n]);
}

// ---------------------------------------------------------------- tree
// Validate the parent array and build child lists (children in ascending id).
// Called by every thread of the workgroup: the parent array is staged in LDS
// by all threads, then one thread links the children in ascending order.
DEVI void build_tree(const AcceptParams& p, int b, int* first_child, int* next_sib, int* spar) {
  const int T = p.T;
  const int32_t* par = p.parent + (size_t)b * T;
  for (int v = threadIdx.x; v < T; v += blockDim.x) {
    spar[v] = par[v];
    first_child[v] = -1;
    next_sib[v] = -1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    bool bad = spar[0] != -1;
    for (int c = T - 1; c >= 1; --c) {
      int pc = spar[c];
      if (pc < 0 || pc >= c) { bad = true; pc = c - 1; }
      next_sib[c] = first_child[pc];
      first_child[pc] = c;
    }
    if (bad) atomicOr(p.flags, FLAG_TREE);
  }
  __syncthreads();
}

// The accepted tree path for the commit kernel: the sequence's kv_len, the
// path length and the path, in the workspace.  Read here, before the commit
// kernel writes kv_len_out (which may alias kv_len).
DEVI void stash_tree_path(const AcceptParams& p, int b, const int* path, int plen) {
  if (!p.kv_len_out) return;
  int32_t* tp = p.tpath + (size_t)b * TPATH;
  if (threadIdx.x == 0) {
    tp[0] = p.kv_len[b];
    tp[1] = plen;
  }
  for (int i = threadIdx.x; i < plen; i += blockDim.x) tp[2 + i] = path[i];
}

// Tree commit: node path[j] of the accepted path moves to slot kv_len + j,
// for j in ascending order; node path[j] >= j, so no copy overwrites a slot
// a later copy still reads.  One workgroup per (layer, KV head) and
// sequence: the copies (a K row, and one V^T entry per dim, per node) spread
// over the chip instead of queueing in one CU.  Thread i keeps the same
// K chunk and V^T row for every j, so no barrier is needed.
__global__ __launch_bounds__(128) void accept_tree_commit_kernel(AcceptParams p) {
  const int lh = blockIdx.x, b = blockIdx.y;
  const int l = lh / p.Hkv, hk = lh % p.Hkv;
  const int32_t* tp = p.tpath + (size_t)b * TPATH;
  const int base = tp[0], plen = tp[1];
  if (lh == 0 && threadIdx.x == 0) p.kv_len_out[b] = base + plen;
  const int cap = p.kvm.table ? min(p.max_ctx, p.kvm.ppseq * KV_PAGE) : p.max_ctx;
  if (base < 0 || base + p.T > cap || plen < 1 || plen > p.T) return;
  // one K or V region: [maxB][Hkv][max_ctx][D] dense, [npages][Hkv][page][D] paged
  const size_t per = p.kvm.table ? (size_t)p.kvm.npages * p.Hkv * KV_PAGE * p.D
                                 : (size_t)p.maxB * p.Hkv * p.max_ctx * p.D;
  uint16_t* kreg = p.kv_cache + (size_t)(2 * l) * per;
  uint16_t* vreg = p.kv_cache + (size_t)(2 * l + 1) * per;
  const int t = threadIdx.x;
  for (int j = 1; j < plen; ++j) {
    const int src = tp[2 + j];
    if (src == j) continue;  // uniform
    if (t < p.D / 8) {
      const uint4 v = *(const uint4*)(kreg + kv_k_off(p.kvm, p.Hkv, p.D, b, hk, base + src) + 8 * t);
      *(uint4*)(kreg + kv_k_off(p.kvm, p.Hkv, p.D, b, hk, base + j) + 8 * t) = v;
    }
    if (t < p.D) {
      const uint16_t v = vreg[kv_v_off(p.kvm, p.Hkv, p.D, b, hk, t, base + src)];
      vreg[kv_v_off(p.kvm, p.Hkv, p.D, b, hk, t, base + j)] = v;
    }
  }
}

DEVI void write_tree_outputs(const AcceptParams& p, int b, const int* path, int plen, int extra) {
  const int T = p.T;
  for (int i = threadIdx.x; i < T; i += blockDim.x) {
    int v = -1;
    if (i < plen - 1) v = p.tokens[b * T + path[i + 1]];
    else if (i == plen - 1) v = extra;
    p.out_tokens[b * T + i] = v;
  }
  if (threadIdx.x == 0) p.num_accepted[b] = plen - 1;
}

__global__ __launch_bounds__(128) void accept_tree_greedy_kernel(AcceptParams p) {
  __shared__ int first_child[128], next_sib[128], path[128], am[128], spar[128];
  __shared__ int s_plen, s_extra;
  const int b = blockIdx.x, T = p.T;
  for (int i = threadIdx.x; i < T; i += blockDim.x) row_argmax(p, b * T + i, am[i]);
  build_tree(p, b, first_child, next_sib, spar);
  if (threadIdx.x == 0) {
    int v = 0, plen = 1;
    path[0] = 0;
    while (true) {
      int nxt = -1;
      for (int c = first_child[v]; c >= 0; c = next_sib[c]) {
        bool bad;
        const int x = clamp_token(p, p.tokens[b * T + c], bad);
        if (!bad && x == am[v]) { nxt = c; break; }
      }
      if (nxt < 0) break;
      v = nxt;
      path[plen++] = v;
    }
    s_plen = plen;
    s_extra = am[v];
  }
  __syncthreads();
  write_tree_outputs(p, b, path, s_plen, s_extra);
  stash_tree_path(p, b, path, s_plen);
}

// ---------------------------------------------------------------- sampled tree walk
// At node v the running target r starts as p_v and the running draft q' as
// q_v.  Child c (token x, uniform slot c - 1) is accepted when
// u * q'(x) < r(x).  A rejection replaces r by norm(max(0, r - q')) (kept as
// it was if that has no mass) and, without replacement, removes x from q'
// and renormalises it.  No child accepted: draw from r; a leaf reached:
// bonus from p_leaf (slot T - 1).
//
// The residual has a closed form.  With U_0 = p, N_0 = 1 and r_k = U_k / N_k,
// rejecting under q' = s_k q (s_k = 1, or 1 / the q mass of the tokens not
// yet removed; removed tokens have q' = 0) gives
//   U_k(y) = max(0, U_{k-1}(y) - N_{k-1} s_k q(y)),   N_k = sum_y U_k(y).
// Since max(0, max(0, a - b q) - c q) = max(0, a - (b + c) q) for q >= 0, a
// token not removed before step k has U_k(y) = max(0, p(y) - A_k q(y)) with
// A_k = A_{k-1} + N_{k-1} s_k, and a removed token keeps the value it had
// when it was removed.  So a rejection costs one reduction over the
// vocabulary, N_k, and nothing is written per token.  The walk runs as a
// short sequence of launches: each step launch has one workgroup per
// (vocabulary chunk, sequence); every workgroup first replays the decisions
// up to the next rejection (a few lookups, identical in all of them), then
// sums its chunk for that rejection's shift; the next launch combines the
// chunk sums.  The kernel boundary orders the sums before their use, and
// the state passes between launches in two alternating copies (chunk 0's
// workgroup writes the one the next launch reads).  A pick kernel draws the
// final token from the last pass's chunk sums and a scan of one chunk, and
// finishes, in one workgroup, a walk that needs more passes than launches.
constexpr int TW_N = 128;   // nodes per tree
constexpr int TW_STEPS = 12;  // step launches (a walk passes at most sum of children on its path + 1 times)
struct TwTree {
  int first_child[TW_N], next_sib[TW_N];
};
struct __align__(16) TwState {
  int v, plen, child;  // current node, path length, next child to test (-1: none left)
  int pend;            // 0 decisions to make, 1 rejection pass summed, 2 draw pass wanted, 3 draw pass summed
  int nrem, pend_x, draw_buf, pad;
  float M, S;          // softmax statistics of node v's row
  float A, An;         // residual shift, shift of the summed rejection pass
  double N, qtot;      // residual mass; q mass of node v's row (-1 until the first pass sums it)
  int path[TW_N];
  int rem_tok[TW_N];   // removed tokens (distinct), their p, q and kept residual value
  float rem_p[TW_N], rem_q[TW_N], rem_val[TW_N];
};
struct TwSeq {
  TwTree tree;
  TwState st[2];
};
// [B] TwSeq, then [2][B][nch] chunk sums (residual mass, q mass)
size_t tree_walk_bytes(int B, int nch) { return (size_t)B * sizeof(TwSeq) + (size_t)2 * B * nch * sizeof(double2); }
DEVI TwSeq* tw_seq(const AcceptParams& p, int b) { return (TwSeq*)p.twalk + b; }
DEVI double2* tw_sums(const AcceptParams& p, int buf, int b) {
  return (double2*)((char*)p.twalk + (size_t)p.B * sizeof(TwSeq)) + ((size_t)buf * p.B + b) * p.nch;
}
// copies of the state between global memory and LDS, 16 bytes per thread
DEVI void tw_copy(TwState* dst, const TwState* src) {
  static_assert(sizeof(TwState) % 16 == 0, "state copied in 16-byte words");
  for (int i = threadIdx.x; i < (int)(sizeof(TwState) / 16); i += blockDim.x) ((uint4*)dst)[i] = ((const uint4*)src)[i];
}

DEVI int tw_removed(const TwState& s, int x) {
  for (int i = 0; i < s.nrem; ++i)
    if (s.rem_tok[i] == x) return i;
  return -1;
}
// the running draft's scale: 1 / the q mass left (0 when none is)
DEVI float tw_qscale(const AcceptParams& p, const TwState& s) {
  if (p.replacement || s.nrem == 0) return 1.f;
  double qm = 0.0;
  for (int i = 0; i < s.nrem; ++i) qm += (double)s.rem_q[i];
  const double left = s.qtot - qm;
  return left > 0.0 ? (float)(1.0 / left) : 0.f;
}

// Combine the chunk sums of the rejection pass (shift An), then drop the
// rejected token from the draft.  One thread.
DEVI void tw_finalize(const AcceptParams& p, int b, TwState& s, const double2* part) {
  const int row = b * p.T + s.v;
  double tu = 0.0, tq = 0.0;
  for (int c0 = 0; c0 < p.nch; c0 += 16) {
    double2 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = c0 + i < p.nch ? part[c0 + i] : make_double2(0.0, 0.0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      tu += v[i].x;
      tq += v[i].y;
    }
  }
  if (s.qtot < 0.0) s.qtot = tq;
  // the removed tokens keep their values: take out what the pass counted
  for (int i = 0; i < s.nrem; ++i)
    tu += (double)s.rem_val[i] - (double)fmaxf(0.f, s.rem_p[i] - s.An * s.rem_q[i]);
  if (tu > 0.0) {
    s.A = s.An;
    s.N = tu;
  }
  const int x = s.pend_x;
  if (!p.replacement && tw_removed(s, x) < 0) {
    const float px = pval(p, row_rule(p, row), p.logits[(size_t)row * p.V + x], x, s.M, s.S);
    const float qx = p.q[(size_t)row * p.V + x];
    const int n = s.nrem;
    s.rem_tok[n] = x;
    s.rem_p[n] = px;
    s.rem_q[n] = qx;
    s.rem_val[n] = fmaxf(0.f, px - s.A * qx);
    s.nrem = n + 1;
  }
}

// Test children until a rejection needs a pass (pend 1 after its sum) or the
// walk ends (pend 2: the draw pass).  One thread.
DEVI void tw_decide(const AcceptParams& p, int b, TwState& s, const TwTree& tr) {
  while (s.pend == 0) {
    const int row = b * p.T + s.v;
    const int c = s.child;
    if (c < 0) {  // every child rejected: draw from the residual
      s.pend = 2;
      return;
    }
    bool bad;
    const int x = clamp_token(p, p.tokens[b * p.T + c], bad);
    const float u = philox_uniform(p.seed, p.round, b, c - 1);
    const float px = pval(p, row_rule(p, row), p.logits[(size_t)row * p.V + x], x, s.M, s.S);
    const float qraw = p.q[(size_t)row * p.V + x];
    const int ri = p.replacement ? -1 : tw_removed(s, x);
    const float rx = (float)((double)(ri >= 0 ? s.rem_val[ri] : fmaxf(0.f, px - s.A * qraw)) / s.N);
    const bool shrunk = !p.replacement && s.nrem > 0;
    const float qx = shrunk ? (ri >= 0 ? 0.f : qraw * tw_qscale(p, s)) : qraw;
    if (!bad && u * qx < rx) {
      // accepted: node c's own target and draft start afresh
      s.v = c;
      s.path[s.plen++] = c;
      s.A = 0.f;
      s.N = 1.0;
      s.nrem = 0;
      s.qtot = -1.0;
      float M, S;
      row_ms(p, b * p.T + c, M, S);
      s.M = M;
      s.S = S;
      s.child = tr.first_child[c];
      if (s.child < 0) {  // a leaf: bonus from its target
        s.pend = 2;
        return;
      }
      continue;
    }
    s.An = (float)((double)s.A + s.N * (double)(shrunk ? tw_qscale(p, s) : 1.f));
    s.pend_x = x;
    s.pend = 1;
  }
}

// Sum over tokens [y0, y1) of row `row` of max(0, p(y) - A q(y)) (p(y) itself
// for A = 0) and, with need_q, of q(y); all threads, ends synchronised.
DEVI double2 tw_chunk_sum(const AcceptParams& p, int row, float A, bool need_q, float M, float S, int y0, int y1,
                          double* shd) {
  const float* z = p.logits + (size_t)row * p.V;
  const float* qv = p.q + (size_t)row * p.V;
  const RowRule rr = row_rule(p, row);
  const bool useq = A != 0.f || need_q;
  double su = 0.0, sq = 0.0;
  constexpr int PER = CH / 256;
  for (int yb = y0; yb < y1; yb += 256 * PER) {
    float zr[PER], qr[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int y = yb + threadIdx.x + 256 * e;
      zr[e] = y < y1 ? z[y] : 0.f;
      qr[e] = (useq && y < y1) ? qv[y] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int y = yb + threadIdx.x + 256 * e;
      if (y < y1) {
        su += (double)fmaxf(0.f, pval(p, rr, zr[e], y, M, S) - A * qr[e]);
        sq += (double)qr[e];
      }
    }
  }
  su = block_sum(su, shd);
  sq = block_sum(sq, shd);
  __syncthreads();
  return make_double2(su, need_q ? sq : 0.0);
}

// Child lists and the walk's first state (one workgroup per sequence).
__global__ __launch_bounds__(128) void accept_tree_init_kernel(AcceptParams p) {
  __shared__ int first_child[TW_N], next_sib[TW_N], spar[TW_N];
  const int b = blockIdx.x;
  build_tree(p, b, first_child, next_sib, spar);
  TwSeq* sq = tw_seq(p, b);
  for (int i = threadIdx.x; i < p.T; i += blockDim.x) {
    sq->tree.first_child[i] = first_child[i];
    sq->tree.next_sib[i] = next_sib[i];
  }
  if (threadIdx.x == 0) {
    TwState& s = sq->st[0];
    s.v = 0;
    s.plen = 1;
    s.path[0] = 0;
    s.child = first_child[0];
    s.pend = s.child < 0 ? 2 : 0;
    s.nrem = 0;
    s.pend_x = 0;
    s.draw_buf = 0;
    s.A = 0.f;
    s.An = 0.f;
    s.N = 1.0;
    s.qtot = -1.0;
    float M, S;
    row_ms(p, b * p.T, M, S);
    s.M = M;
    s.S = S;
  }
}

// Step k of the walk: grid (chunks, sequences).
__global__ __launch_bounds__(256) void accept_tree_step_kernel(AcceptParams p, int k) {
  __shared__ TwState s;
  __shared__ double shd[16];
  const int c = blockIdx.x, b = blockIdx.y;
  TwSeq* sq = tw_seq(p, b);
  tw_copy(&s, &sq->st[k & 1]);
  __syncthreads();
  if (threadIdx.x == 0 && s.pend < 2) {
    if (s.pend == 1) {
      tw_finalize(p, b, s, tw_sums(p, (k - 1) & 1, b));
      s.child = sq->tree.next_sib[s.child];
      s.pend = 0;
    }
    tw_decide(p, b, s, sq->tree);
  }
  __syncthreads();
  const int pend = s.pend;
  if (pend == 1 || pend == 2) {
    const double2 r = tw_chunk_sum(p, b * p.T + s.v, pend == 1 ? s.An : s.A, pend == 1 && s.qtot < 0.0, s.M, s.S,
                                   c * CH, min(p.V, (c + 1) * CH), shd);
    if (threadIdx.x == 0) tw_sums(p, k & 1, b)[c] = r;
  }
  if (c == 0) {
    if (threadIdx.x == 0 && pend == 2) {
      s.pend = 3;
      s.draw_buf = k & 1;
    }
    __syncthreads();
    tw_copy(&sq->st[(k + 1) & 1], &s);
  }
}

// Final draw (one workgroup per sequence), after `nstep` step launches; walks
// that were not done by then are finished here, one chunk at a time.
__global__ __launch_bounds__(256) void accept_tree_pick_kernel(AcceptParams p, int nstep) {
  __shared__ TwState s;
  __shared__ double shd[16];
  __shared__ double2 part[64];
  __shared__ double csum[64];
  __shared__ double scan[256];
  __shared__ int s_chunk, s_tok;
  __shared__ double s_t;
  const int b = blockIdx.x, T = p.T, V = p.V;
  TwSeq* sq = tw_seq(p, b);
  tw_copy(&s, &sq->st[nstep & 1]);
  __syncthreads();
  const double2* src = tw_sums(p, (nstep - 1) & 1, b);
  while (s.pend != 3) {
    if (threadIdx.x == 0) {
      if (s.pend == 1) {
        tw_finalize(p, b, s, src);
        s.child = sq->tree.next_sib[s.child];
        s.pend = 0;
      }
      tw_decide(p, b, s, sq->tree);
    }
    __syncthreads();
    const int pend = s.pend;
    for (int c = 0; c < p.nch; ++c) {
      const double2 r = tw_chunk_sum(p, b * T + s.v, pend == 1 ? s.An : s.A, pend == 1 && s.qtot < 0.0, s.M, s.S,
                                     c * CH, min(V, (c + 1) * CH), shd);
      if (threadIdx.x == 0) part[c] = r;
    }
    src = part;
    if (threadIdx.x == 0 && pend == 2) {
      s.pend = 3;
      s.draw_buf = -1;
    }
    __syncthreads();
  }
  const double2* dsum = s.draw_buf >= 0 ? tw_sums(p, s.draw_buf, b) : part;
  const int row = b * T + s.v;
  const float* z = p.logits + (size_t)row * V;
  const float* qv = p.q + (size_t)row * V;
  const RowRule rr = row_rule(p, row);
  const float A = s.A;
  // value of token y in the final distribution (unnormalised)
  auto val = [&](float zy, float qy, int y) {
    for (int i = 0; i < s.nrem; ++i)
      if (s.rem_tok[i] == y) return s.rem_val[i];
    return fmaxf(0.f, pval(p, rr, zy, y, s.M, s.S) - A * qy);
  };
  if (threadIdx.x == 0) {
    for (int c = 0; c < p.nch; ++c) csum[c] = dsum[c].x;
    // the removed tokens keep their values
    for (int i = 0; i < s.nrem; ++i)
      csum[s.rem_tok[i] / CH] += (double)s.rem_val[i] - (double)fmaxf(0.f, s.rem_p[i] - A * s.rem_q[i]);
    double R = 0.0;
    for (int c = 0; c < p.nch; ++c) R += csum[c];
    const double t = (double)philox_uniform(p.seed, p.round, b, T - 1) * R;
    double cum = 0.0;
    int pick = -1, last = -1;
    for (int c = 0; c < p.nch; ++c) {
      if (csum[c] > 0.0) last = c;
      if (pick < 0 && cum + csum[c] > t) pick = c;
      if (pick < 0) cum += csum[c];
    }
    // rounding left t at or past the total: the last chunk with mass, whose
    // last token with mass is taken below
    s_chunk = pick >= 0 ? pick : (last >= 0 ? last : 0);
    s_t = pick >= 0 ? t - cum : INFINITY;
    s_tok = 0x7fffffff;
  }
  __syncthreads();
  // inverse CDF inside the chunk: thread i holds tokens y0 + 16 i .. + 15
  constexpr int PER = CH / 256;
  const int y0 = s_chunk * CH + PER * threadIdx.x, y1 = min(V, y0 + PER);
  float vr[PER];
  double loc = 0.0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int y = y0 + e;
    const float zy = y < y1 ? z[y] : 0.f;
    const float qy = (y < y1 && A != 0.f) ? qv[y] : 0.f;
    vr[e] = y < y1 ? val(zy, qy, y) : 0.f;
    loc += (double)vr[e];
  }
  scan[threadIdx.x] = loc;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const double add = threadIdx.x >= (unsigned)o ? scan[threadIdx.x - o] : 0.0;
    __syncthreads();
    scan[threadIdx.x] += add;
    __syncthreads();
  }
  const double t = s_t;
  double run = scan[threadIdx.x] - loc;
  if (run <= t && run + loc > t) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      run += (double)vr[e];
      if (run > t) {
        atomicMin(&s_tok, y0 + e);
        break;
      }
    }
  }
  __syncthreads();
  if (s_tok == 0x7fffffff) {
    int lastpos = -1;
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (vr[e] > 0.f) lastpos = y0 + e;
    __shared__ int s_last;
    if (threadIdx.x == 0) s_last = -1;
    __syncthreads();
    if (lastpos >= 0) atomicMax(&s_last, lastpos);
    __syncthreads();
    if (threadIdx.x == 0) s_tok = s_last >= 0 ? s_last : 0;
    __syncthreads();
  }
  write_tree_outputs(p, b, s.path, s.plen, s_tok);
  stash_tree_path(p, b, s.path, s.plen);
}

// Top-k / top-p selection for all rows, in batches of SEL_ROWS rows, then the
// chunk statistics of the kept tokens.
static hipError_t launch_select(const AcceptParams& p, hipStream_t s) {
  const int rows = p.rows;
  const bool topk = p.top_k > 0 && p.top_k < p.V, topp = p.top_p < 1.f;
  for (int row0 = 0; row0 < rows; row0 += SEL_ROWS) {
    const int nr = min(SEL_ROWS, rows - row0);
    accept_select_init_kernel<<<(nr + 63) / 64, 64, 0, s>>>(p, row0, nr);
    for (int phase = 0; phase < 2; ++phase) {
      if ((phase == 0 && !topk) || (phase == 1 && !topp)) continue;
      for (int d = 0; d < 4; ++d) accept_select_kernel<<<dim3(p.nch, nr), 256, 0, s>>>(p, SelArgs{row0, phase, d});
      accept_select_finish_kernel<<<nr, 256, 0, s>>>(p, SelArgs{row0, phase, 4});
    }
    accept_select_apply_kernel<<<dim3(p.nch, nr), 256, 0, s>>>(p, row0);
  }
  return hipGetLastError();
}

hipError_t launch_accept(const AcceptParams& pin, hipStream_t s) {
  const bool greedy = pin.temperature == 0.f;
  const bool adjust = !greedy && ((pin.top_k > 0 && pin.top_k < pin.V) || pin.top_p < 1.f);
  AcceptParams p = pin;
  if (!adjust) p.fres = nullptr;
  // the selection stages one count per chunk in a 256-entry LDS array
  if (adjust && (!p.fcnt || !p.fmass || !p.fstate || !p.fres || p.nch > 256)) return hipErrorInvalidValue;
  dim3 g1(p.nch, p.rows);
  if (greedy)
    accept_rowstats_kernel<true><<<g1, 256, 0, s>>>(p);
  else
    accept_rowstats_kernel<false><<<g1, 256, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (adjust && (e = launch_select(p, s)) != hipSuccess) return e;
  if (p.parent) {
    if (greedy) {
      accept_tree_greedy_kernel<<<p.B, 128, 0, s>>>(p);
    } else {
      if (p.T > TW_N || p.nch > 64 || !p.twalk) return hipErrorInvalidValue;
      accept_tree_init_kernel<<<p.B, 128, 0, s>>>(p);
      const int nstep = p.T < TW_STEPS ? p.T : TW_STEPS;
      for (int k = 0; k < nstep; ++k) accept_tree_step_kernel<<<dim3(p.nch, p.B), 256, 0, s>>>(p, k);
      accept_tree_pick_kernel<<<p.B, 256, 0, s>>>(p, nstep);
    }
    if (p.kv_len_out) {
      if (p.D > 128 || p.T > TPATH - 2 || !p.tpath) return hipErrorInvalidValue;
      accept_tree_commit_kernel<<<dim3(p.L * p.Hkv, p.B), 128, 0, s>>>(p);
    }
    return hipGetLastError();
  }
  if (greedy) {
    accept_chain_greedy_kernel<<<p.B, 128, 0, s>>>(p);
    return hipGetLastError();
  }
  accept_chain_residual_kernel<<<dim3(p.nch, p.B), 256, 0, s>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  accept_chain_sample_kernel<<<p.B, 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace sv
