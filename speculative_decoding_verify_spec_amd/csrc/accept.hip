// Speculative-sampling accept, residual resample, bonus token and KV commit.
//
// CS349E Lecture 6 ("Optimizing Autoregressive Decode"), section 6.2 steps
// 3-5: accept draft x_i when u_i < p_i(x_i)/q_i(x_i) (evaluated as
// u_i * q_i(x_i) < p_i(x_i), the form the Kimi-K3 tuning page describes), stop
// at the first rejection, then draw from norm(max(0, p_{n+1} - q_{n+1})) or,
// when every draft survived, a bonus token from p_{gamma+1}.  Greedy
// (section 7.4): longest prefix where draft == argmax, then that argmax.
// Token trees (section 10.3): walk from the root, testing each node's children
// in order against a running residual (see accept_tree_sampled_kernel).
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

// Sampled tree walk, one workgroup per sequence.  At node v the running target
// r starts as p_v and the draft q' as q_v.  Child c (token x, uniform slot
// c - 1) is accepted when u * q'(x) < r(x).  A rejection replaces r by
// norm(max(0, r - q')) (a pass over the vocabulary into one of two ping-pong
// buffers) and, without replacement, removes x from q' and renormalises.  No
// child accepted: draw from r; a leaf reached: bonus from p_leaf (slot T - 1).
__global__ __launch_bounds__(1024) void accept_tree_sampled_kernel(AcceptParams p) {
  __shared__ int first_child[128], next_sib[128], path[128], removed[128], spar[128];
  __shared__ double shd[16];
  __shared__ float s_M, s_S, s_Zr, s_qmass, s_qtot;
  __shared__ int s_cur, s_acc, s_nrem, s_tok;
  __shared__ double s_t;
  const int b = blockIdx.x, T = p.T, V = p.V;
  const float Tt = p.temperature;
  float* rb0 = p.rbuf + (size_t)b * V;
  float* rb1 = p.rbuf + ((size_t)p.B + b) * V;
  build_tree(p, b, first_child, next_sib, spar);
  int v = 0, plen = 1;
  if (threadIdx.x == 0) path[0] = 0;
  while (true) {
    const int row = b * T + v;
    const float* z = p.logits + (size_t)row * V;
    const float* qv = p.q + (size_t)row * V;
    if (threadIdx.x == 0) {
      float M, S;
      row_ms(p, row, M, S);
      s_M = M; s_S = S; s_cur = -1; s_Zr = 1.f; s_nrem = 0; s_qmass = 0.f; s_qtot = -1.f;
    }
    __syncthreads();
    int c = first_child[v];
    int accepted = -1;
    while (c >= 0) {
      if (threadIdx.x == 0) {
        bool bad;
        const int x = clamp_token(p, p.tokens[b * T + c], bad);
        const float u = philox_uniform(p.seed, p.round, b, c - 1);
        const float rx = (s_cur < 0) ? pval(p, row_rule(p, row), z[x], x, s_M, s_S) : (s_cur == 0 ? rb0 : rb1)[x] / s_Zr;
        float qx = qv[x];
        if (!p.replacement && s_nrem > 0) {
          bool gone = false;
          for (int i = 0; i < s_nrem; ++i) gone |= removed[i] == x;
          qx = gone ? 0.f : qx / (s_qtot - s_qmass);
        }
        s_acc = (!bad && u * qx < rx) ? 1 : 0;
        removed[s_nrem] = x;  // recorded now, counted only after a rejection
      }
      __syncthreads();
      if (s_acc) { accepted = c; break; }
      // rejection: r <- max(0, r - q') into the other buffer
      const int cur = s_cur;
      const float* src = cur == 1 ? rb1 : rb0;
      float* dst = cur == 0 ? rb1 : rb0;
      const float M = s_M, S = s_S, Zr = s_Zr;
      const int nrem = s_nrem;
      const float qscale = (!p.replacement && nrem > 0) ? 1.0f / (s_qtot - s_qmass) : 1.0f;
      const RowRule rr = row_rule(p, row);
      double zs = 0.0, qs = 0.0;
      // every token as if still in q'; the removed ones are fixed below.  A
      // thread's RU elements (a workgroup stride apart) are requested at once.
      constexpr int RU = 8;
      const float* rsrc = cur < 0 ? z : src;
      auto resid = [&](float zy, float qy, int y) {
        const float ry = cur < 0 ? pval(p, rr, zy, y, M, S) : zy / Zr;
        qs += (double)qy;
        const float d = fmaxf(0.f, ry - qy * qscale);
        zs += (double)d;
        return d;
      };
      if ((V & 3) == 0) {
        // rows are 16-byte aligned: four tokens per load
        const int V4 = V >> 2;
        for (int i0 = threadIdx.x; i0 < V4; i0 += RU * blockDim.x) {
          float4 zr[RU], qr[RU];
#pragma unroll
          for (int u = 0; u < RU; ++u) {
            const int i = min(i0 + u * (int)blockDim.x, V4 - 1);
            zr[u] = ((const float4*)rsrc)[i];
            qr[u] = ((const float4*)qv)[i];
          }
#pragma unroll
          for (int u = 0; u < RU; ++u) {
            const int i = i0 + u * blockDim.x;
            if (i < V4) {
              float4 d;
              d.x = resid(zr[u].x, qr[u].x, 4 * i);
              d.y = resid(zr[u].y, qr[u].y, 4 * i + 1);
              d.z = resid(zr[u].z, qr[u].z, 4 * i + 2);
              d.w = resid(zr[u].w, qr[u].w, 4 * i + 3);
              ((float4*)dst)[i] = d;
            }
          }
        }
      } else {
        for (int y0 = threadIdx.x; y0 < V; y0 += RU * blockDim.x) {
          float zr[RU], qr[RU];
#pragma unroll
          for (int u = 0; u < RU; ++u) {
            const int yc = min(y0 + u * (int)blockDim.x, V - 1);
            zr[u] = rsrc[yc];
            qr[u] = qv[yc];
          }
#pragma unroll
          for (int u = 0; u < RU; ++u) {
            const int y = y0 + u * blockDim.x;
            if (y < V) dst[y] = resid(zr[u], qr[u], y);
          }
        }
      }
      zs = block_sum(zs, shd);
      qs = block_sum(qs, shd);
      if (threadIdx.x == 0) {
        if (!p.replacement) {
          // a removed token has q' = 0: its residual is r itself (each
          // distinct token once; the pass above wrote r - q' there)
          for (int i = 0; i < nrem; ++i) {
            const int x = removed[i];
            bool seen = false;
            for (int k = 0; k < i; ++k) seen |= removed[k] == x;
            if (seen) continue;
            const float rx = cur < 0 ? pval(p, rr, z[x], x, M, S) : src[x] / Zr;
            const float dx = fmaxf(0.f, rx - qv[x] * qscale);
            zs += (double)rx - (double)dx;
            dst[x] = rx;
          }
        }
        if (zs > 0.0) { s_cur = (cur == 0) ? 1 : 0; s_Zr = (float)zs; }
        if (!p.replacement) {
          if (s_qtot < 0.f) s_qtot = (float)qs;
          s_qmass += qv[removed[s_nrem]];
          s_nrem = s_nrem + 1;
        }
      }
      __syncthreads();
      c = next_sib[c];
    }
    if (accepted < 0) break;
    v = accepted;
    if (threadIdx.x == 0) path[plen] = v;
    ++plen;
    if (first_child[v] < 0) {
      // leaf: bonus from p_leaf
      if (threadIdx.x == 0) {
        float M, S;
        row_ms(p, b * T + v, M, S);
        s_M = M; s_S = S; s_cur = -1; s_Zr = 1.f;
      }
      __syncthreads();
      break;
    }
  }
  // final draw from r (s_cur, s_Zr) or p_v (s_cur < 0) at node v, slot T - 1
  {
    const int row = b * T + v;
    const float* z = p.logits + (size_t)row * V;
    const int cur = s_cur;
    const float* src = cur == 1 ? rb1 : rb0;
    const float M = s_M, S = s_S;
    const RowRule rr = row_rule(p, row);
    const float* vsrc = cur < 0 ? z : src;
    auto val = [&](float x, int y) { return cur < 0 ? pval(p, rr, x, y, M, S) : x; };
    // thread chunks of a multiple of 4 tokens when rows are 16-byte aligned
    const bool vec = (V & 3) == 0;
    const int per = vec ? 4 * (((V >> 2) + blockDim.x - 1) / blockDim.x) : (V + blockDim.x - 1) / blockDim.x;
    const int y0 = min(V, (int)threadIdx.x * per), y1 = min(V, y0 + per);
    // the chunk's values in order, DB loads requested at once; f(y, value)
    // returns true to stop
    constexpr int DB = 8;
    auto walk = [&](auto f) {
      if (vec) {
        for (int yb = y0; yb < y1; yb += 4 * DB) {
          float4 c[DB];
#pragma unroll
          for (int u = 0; u < DB; ++u) {
            const int yy = yb + 4 * u;
            c[u] = yy < y1 ? *(const float4*)(vsrc + yy) : make_float4(0.f, 0.f, 0.f, 0.f);
          }
#pragma unroll
          for (int u = 0; u < DB; ++u) {
            const int yy = yb + 4 * u;
            if (yy < y1) {
              if (f(yy, val(c[u].x, yy))) return;
              if (f(yy + 1, val(c[u].y, yy + 1))) return;
              if (f(yy + 2, val(c[u].z, yy + 2))) return;
              if (f(yy + 3, val(c[u].w, yy + 3))) return;
            }
          }
        }
      } else {
        for (int yb = y0; yb < y1; yb += DB) {
          float c[DB];
#pragma unroll
          for (int u = 0; u < DB; ++u) c[u] = yb + u < y1 ? vsrc[yb + u] : 0.f;
#pragma unroll
          for (int u = 0; u < DB; ++u)
            if (yb + u < y1 && f(yb + u, val(c[u], yb + u))) return;
        }
      }
    };
    double loc = 0.0;
    walk([&](int, float v) {
      loc += (double)v;
      return false;
    });
    __shared__ double scan[1024];
    scan[threadIdx.x] = loc;
    if (threadIdx.x == 0) s_tok = 0x7fffffff;
    __syncthreads();
    for (int o = 1; o < (int)blockDim.x; o <<= 1) {
      double add = threadIdx.x >= o ? scan[threadIdx.x - o] : 0.0;
      __syncthreads();
      scan[threadIdx.x] += add;
      __syncthreads();
    }
    const double R = scan[blockDim.x - 1];
    if (threadIdx.x == 0) s_t = (double)philox_uniform(p.seed, p.round, b, T - 1) * R;
    __syncthreads();
    const double t = s_t;
    double run = scan[threadIdx.x] - loc;
    if (run <= t && run + loc > t) {
      walk([&](int y, float v) {
        run += (double)v;
        if (run > t) {
          atomicMin(&s_tok, y);
          return true;
        }
        return false;
      });
    }
    __syncthreads();
    if (s_tok == 0x7fffffff) {
      // rounding: take the last token with positive mass
      int last = -1;
      for (int y = y0; y < y1; ++y)
        if ((cur < 0 ? pval(p, rr, z[y], y, M, S) : src[y]) > 0.f) last = y;
      __shared__ int s_last;
      if (threadIdx.x == 0) s_last = -1;
      __syncthreads();
      if (last >= 0) atomicMax(&s_last, last);
      __syncthreads();
      if (threadIdx.x == 0) s_tok = s_last >= 0 ? s_last : 0;
      __syncthreads();
    }
  }
  write_tree_outputs(p, b, path, plen, s_tok);
  stash_tree_path(p, b, path, plen);
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
    if (greedy) accept_tree_greedy_kernel<<<p.B, 128, 0, s>>>(p);
    else accept_tree_sampled_kernel<<<p.B, 1024, 0, s>>>(p);
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
