// Verify on a recurrent (gated delta-rule) layer: the per-sequence state is
// advanced serially through the T window positions, and after acceptance the
// state of the last committed position becomes the sequence's pool state
// (Kimi-K3 tuning page, "Verification on a recurrent layer is not a cache
// write").  The layer's arithmetic is stated in spec_recurrent.h.
//
// One workgroup of 256 threads owns one (sequence, head): its D x D state
// lives in registers for the whole window.  Wave w covers the 64 value
// columns j = (w % (D/64)) * 64 + lane and a band of key rows; a thread holds
// the column segment S[i][j] for the RPT rows of its band, so every state
// load or store of a wave touches 256 contiguous bytes of one row.  A
// position costs two column reductions (S^T k^ before the write, S^T q^
// after it): per-thread partial sums over the band, then the bands' partials
// added in LDS in band order.
//
// HBM traffic per (sequence, head): the state read once, plus T snapshot
// writes when the caller keeps snapshots (non-temporal stores: at most one
// of them is read again), plus the small window inputs and outputs.  The
// replay commit reads and writes the state once more instead of writing T
// snapshots.
#include "common.h"
#include "spec_recurrent.h"

namespace sv {

constexpr int REC_THREADS = 256;
constexpr int REC_MAX_T = 16;
constexpr int REC_MAX_W = 8;
constexpr float REC_L2_EPS = 1e-6f;

struct RecParams {
  int B, T, H, W, n_slots;
  const float* x;       // [B][T][3HD]
  const float* gate;    // [B][T][H][D]
  const float* beta;    // [B][T][H]
  const float* conv_w;  // [3HD][W]
  const int32_t* slot;  // [B] or null
  const int32_t* nacc;  // [B] (commit)
  const float* snap_in; // [B][T][H][D][D] (scatter commit)
  float* conv_state;    // [n_slots][W-1][3HD]
  float* state;         // [n_slots][H][D][D]
  float* out;           // [B][T][H][D] (verify)
  float* snap;          // [B][T][H][D][D] (verify) or null
};

DEVI int rec_slot(const RecParams& p, int b) {
  const int s = p.slot ? p.slot[b] : b;
  return (s >= 0 && s < p.n_slots) ? s : -1;
}

DEVI int rec_committed(const RecParams& p, int b) {
  const int n = p.nacc[b];
  return n < 0 ? 0 : (n > p.T - 1 ? p.T - 1 : n);
}

// Rows of the per-position vectors are 16-byte aligned so a thread's
// consecutive key rows come in 4-wide LDS reads.
template <int D>
struct RecLds {
  alignas(16) float q[REC_MAX_T][D];    // q^ (normalised, scaled by D^-1/2)
  alignas(16) float k[REC_MAX_T][D];    // k^
  alignas(16) float v[REC_MAX_T][D];
  alignas(16) float dec[REC_MAX_T][D];  // exp(gate)
  float bet[REC_MAX_T];
  // S^T k^ partials by position parity: with one barrier per position (no
  // output reduction) a wave may write position t+1's partials while another
  // still reads position t's
  float red_u[2][4][D];
  float red_o[4][D];
};

// Window inputs of one workgroup, held in registers between the loads and
// the prologue arithmetic.  A thread owns whole channels (its raw inputs for
// every position, the W-1 before the window included, and its taps), so each
// raw input is loaded once and every load of the window is issued before the
// first is used.  Arrays are sized for the largest window and conv; entries
// past the actual ones are zero and never read.
template <int D>
struct RecIn {
  static constexpr int NCH = 3 * D;                                   // q, k, v channels of a head
  static constexpr int PER = (NCH + REC_THREADS - 1) / REC_THREADS;  // channels per thread
  static constexpr int NR = REC_MAX_T + REC_MAX_W - 1;               // raw inputs per channel
  static constexpr int NG = (REC_MAX_T * D + REC_THREADS - 1) / REC_THREADS;
  float raw[PER][NR];
  float cw[PER][REC_MAX_W];
  float g[NG];
  float bt;
};

template <int D>
DEVI void rec_issue(const RecParams& p, int b, int h, int s, int nt, RecIn<D>& in) {
  const int C = 3 * p.H * D, W = p.W;
#pragma unroll
  for (int c = 0; c < RecIn<D>::PER; ++c) {
    const int c3 = threadIdx.x + c * REC_THREADS;
    const bool ok = c3 < RecIn<D>::NCH;
    const int ch = ok ? (c3 / D) * p.H * D + h * D + c3 % D : 0;
#pragma unroll
    for (int w = 0; w < REC_MAX_W; ++w) in.cw[c][w] = (ok && w < W) ? p.conv_w[(size_t)ch * W + w] : 0.f;
#pragma unroll
    for (int r = 0; r < RecIn<D>::NR; ++r) {
      const int pos = r - (W - 1);  // window position of raw input r
      float v = 0.f;
      if (ok && pos < nt)
        v = pos >= 0 ? p.x[((size_t)b * p.T + pos) * C + ch]
                     : p.conv_state[((size_t)s * (W - 1) + r) * C + ch];
      in.raw[c][r] = v;
    }
  }
#pragma unroll
  for (int k = 0; k < RecIn<D>::NG; ++k) {
    const int idx = threadIdx.x + k * REC_THREADS;
    in.g[k] = idx < nt * D ? p.gate[(((size_t)b * p.T + idx / D) * p.H + h) * D + idx % D] : 0.f;
  }
  in.bt = (int)threadIdx.x < nt ? p.beta[((size_t)b * p.T + threadIdx.x) * p.H + h] : 0.f;
}

// Window prologue from the issued inputs: conv + SiLU of the head's q, k, v
// channels for positions 0 .. nt-1, decay factors and betas into LDS, then
// the per-position L2 normalisation of q and k.  Ends with the workgroup
// synchronised.
template <int D>
DEVI void rec_prologue(const RecParams& p, int nt, const RecIn<D>& in, RecLds<D>& L) {
  const int W = p.W;
#pragma unroll
  for (int c = 0; c < RecIn<D>::PER; ++c) {
    const int c3 = threadIdx.x + c * REC_THREADS;
    const int which = c3 / D, i = c3 % D;
    float* dst = which == 0 ? &L.q[0][i] : which == 1 ? &L.k[0][i] : &L.v[0][i];
#pragma unroll
    for (int t = 0; t < REC_MAX_T; ++t) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < REC_MAX_W; ++w)
        if (w < W) acc = fmaf(in.cw[c][w], in.raw[c][t + w], acc);
      if (c3 < RecIn<D>::NCH && t < nt) dst[t * D] = acc / (1.0f + expf(-acc));
    }
  }
#pragma unroll
  for (int k = 0; k < RecIn<D>::NG; ++k) {
    const int idx = threadIdx.x + k * REC_THREADS;
    if (idx < nt * D) L.dec[idx / D][idx % D] = expf(in.g[k]);
  }
  if ((int)threadIdx.x < nt) L.bet[threadIdx.x] = in.bt;
  __syncthreads();
  // one wave per (position, q or k) vector
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int item = w; item < 2 * nt; item += REC_THREADS / 64) {
    const int t = item >> 1;
    float* vec = (item & 1) ? L.k[t] : L.q[t];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) ss = fmaf(vec[lane + 64 * e], vec[lane + 64 * e], ss);
    ss = wave_sum(ss);
    float f = 1.0f / sqrtf(ss + REC_L2_EPS);
    if (!(item & 1)) f *= 1.0f / sqrtf((float)D);
#pragma unroll
    for (int e = 0; e < D / 64; ++e) vec[lane + 64 * e] *= f;
  }
  __syncthreads();
}

// Thread geometry of the state registers.
template <int D>
struct RecGeom {
  static constexpr int CB = D / 64;          // column blocks of 64
  static constexpr int RG = 4 / CB;          // row bands
  static constexpr int RPT = D / RG;         // rows per thread
  int j, band;
  DEVI RecGeom() {
    const int w = threadIdx.x >> 6;
    j = (w % CB) * 64 + (threadIdx.x & 63);
    band = w / CB;
  }
  DEVI int row(int r) const { return band * RPT + r; }
};

// One window position on the register state.  OUT: also reduce S^T q^ and
// return it (valid in band-0 threads).  Both commit modes and the verify run
// this same code, so the states they produce are identical.
template <int D, bool OUT>
DEVI float rec_step(float (&s)[RecGeom<D>::RPT], const RecGeom<D>& g, RecLds<D>& L, int t) {
  constexpr int RPT = RecGeom<D>::RPT, RG = RecGeom<D>::RG;
  float pu = 0.f;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    s[r] *= L.dec[t][g.row(r)];
    pu = fmaf(L.k[t][g.row(r)], s[r], pu);
  }
  L.red_u[t & 1][g.band][g.j] = pu;
  __syncthreads();
  float u = 0.f;
#pragma unroll
  for (int q = 0; q < RG; ++q) u += L.red_u[t & 1][q][g.j];
  const float delta = L.bet[t] * (L.v[t][g.j] - u);
  float po = 0.f;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    s[r] = fmaf(L.k[t][g.row(r)], delta, s[r]);
    if (OUT) po = fmaf(L.q[t][g.row(r)], s[r], po);
  }
  if (!OUT) return 0.f;
  L.red_o[g.band][g.j] = po;
  __syncthreads();
  float o = 0.f;
#pragma unroll
  for (int q = 0; q < RG; ++q) o += L.red_o[q][g.j];
  return o;
}

template <int D>
DEVI void rec_load_state(float (&s)[RecGeom<D>::RPT], const RecGeom<D>& g, const float* st) {
#pragma unroll
  for (int r = 0; r < RecGeom<D>::RPT; ++r) s[r] = st[(size_t)g.row(r) * D + g.j];
}

// New conv state of the head's channels: the W-1 raw inputs ending at window
// position n.  Every value is read before the workgroup barrier and written
// after it, because some of them come from the old conv state.
template <int D>
DEVI void rec_commit_conv(const RecParams& p, int b, int h, int s, int n) {
  const int Wm1 = p.W - 1;
  constexpr int MAXV = (3 * D * (REC_MAX_W - 1) + REC_THREADS - 1) / REC_THREADS;
  const int C = 3 * p.H * D, items = 3 * D * Wm1;
  float val[MAXV];
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int idx = threadIdx.x + k * REC_THREADS;
    if (idx < items) {
      const int wq = idx / (3 * D), c3 = idx % (3 * D);
      const int ch = (c3 / D) * p.H * D + h * D + c3 % D;
      const int pos = n - (Wm1 - 1) + wq;  // window position of the kept input
      val[k] = pos >= 0 ? p.x[((size_t)b * p.T + pos) * C + ch]
                        : p.conv_state[((size_t)s * Wm1 + (Wm1 + pos)) * C + ch];
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < MAXV; ++k) {
    const int idx = threadIdx.x + k * REC_THREADS;
    if (idx < items) {
      const int wq = idx / (3 * D), c3 = idx % (3 * D);
      const int ch = (c3 / D) * p.H * D + h * D + c3 % D;
      p.conv_state[((size_t)s * Wm1 + wq) * C + ch] = val[k];
    }
  }
}

// grid (H, B): verify window, outputs and optional snapshots
template <int D>
__global__ __launch_bounds__(REC_THREADS) void rec_verify_kernel(RecParams p) {
  __shared__ RecLds<D> L;
  const int h = blockIdx.x, b = blockIdx.y;
  const int s = rec_slot(p, b);
  if (s < 0) return;
  const RecGeom<D> g;
  RecIn<D> in;
  rec_issue<D>(p, b, h, s, p.T, in);
  float st[RecGeom<D>::RPT];
  rec_load_state<D>(st, g, p.state + ((size_t)s * p.H + h) * D * D);
  rec_prologue<D>(p, p.T, in, L);
  for (int t = 0; t < p.T; ++t) {
    const float o = rec_step<D, true>(st, g, L, t);
    if (g.band == 0) p.out[(((size_t)b * p.T + t) * p.H + h) * D + g.j] = o;
    if (p.snap) {
      float* sn = p.snap + (((size_t)b * p.T + t) * p.H + h) * D * D;
#pragma unroll
      for (int r = 0; r < RecGeom<D>::RPT; ++r) __builtin_nontemporal_store(st[r], &sn[(size_t)g.row(r) * D + g.j]);
    }
  }
}

// grid (H, B): replay commit, the pool state advanced through positions 0..n
template <int D>
__global__ __launch_bounds__(REC_THREADS) void rec_replay_kernel(RecParams p) {
  __shared__ RecLds<D> L;
  const int h = blockIdx.x, b = blockIdx.y;
  const int s = rec_slot(p, b);
  if (s < 0) return;
  const int n = rec_committed(p, b);
  const RecGeom<D> g;
  float* sp = p.state + ((size_t)s * p.H + h) * D * D;
  RecIn<D> in;
  rec_issue<D>(p, b, h, s, n + 1, in);
  float st[RecGeom<D>::RPT];
  rec_load_state<D>(st, g, sp);
  rec_prologue<D>(p, n + 1, in, L);
  for (int t = 0; t <= n; ++t) rec_step<D, false>(st, g, L, t);
#pragma unroll
  for (int r = 0; r < RecGeom<D>::RPT; ++r) sp[(size_t)g.row(r) * D + g.j] = st[r];
  if (p.W > 1) rec_commit_conv<D>(p, b, h, s, n);
}

// grid (H, B): the previous window's replay commit, then the verify of the
// new window from the committed state still in registers (one read and one
// write of the state per round instead of two reads and a write).  `pp`
// describes the previous window (pp.T == 0: nothing to commit), `p` the new
// one.  The same per-position code as the two separate kernels, so the
// results are identical to a replay commit followed by a verify.
template <int D>
__global__ __launch_bounds__(REC_THREADS) void rec_commit_verify_kernel(RecParams p, RecParams pp) {
  __shared__ RecLds<D> L;
  const int h = blockIdx.x, b = blockIdx.y;
  const int s = rec_slot(p, b);
  if (s < 0) return;
  const RecGeom<D> g;
  float* sp = p.state + ((size_t)s * p.H + h) * D * D;
  float st[RecGeom<D>::RPT];
  if (pp.T > 0) {
    const int n = rec_committed(pp, b);
    RecIn<D> in;
    rec_issue<D>(pp, b, h, s, n + 1, in);
    rec_load_state<D>(st, g, sp);
    rec_prologue<D>(pp, n + 1, in, L);
    for (int t = 0; t <= n; ++t) rec_step<D, false>(st, g, L, t);
#pragma unroll
    for (int r = 0; r < RecGeom<D>::RPT; ++r) sp[(size_t)g.row(r) * D + g.j] = st[r];
    if (p.W > 1) rec_commit_conv<D>(pp, b, h, s, n);
    // the new conv state is read back below by this workgroup, and the
    // window's LDS arrays are refilled
    __syncthreads();
  } else {
    rec_load_state<D>(st, g, sp);
  }
  RecIn<D> in;
  rec_issue<D>(p, b, h, s, p.T, in);
  rec_prologue<D>(p, p.T, in, L);
  for (int t = 0; t < p.T; ++t) {
    const float o = rec_step<D, true>(st, g, L, t);
    if (g.band == 0) p.out[(((size_t)b * p.T + t) * p.H + h) * D + g.j] = o;
  }
}

// grid (H, B): scatter commit, the survivor snapshot copied to the pool
template <int D>
__global__ __launch_bounds__(REC_THREADS) void rec_scatter_kernel(RecParams p) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int s = rec_slot(p, b);
  if (s < 0) return;
  const int n = rec_committed(p, b);
  const f32x4* src = (const f32x4*)(p.snap_in + (((size_t)b * p.T + n) * p.H + h) * D * D);
  f32x4* dst = (f32x4*)(p.state + ((size_t)s * p.H + h) * D * D);
#pragma unroll
  for (int k = 0; k < D * D / 4 / REC_THREADS; ++k) {
    const int e = threadIdx.x + k * REC_THREADS;
    dst[e] = src[e];
  }
  if (p.W > 1) rec_commit_conv<D>(p, b, h, s, n);
}

static spec_status rec_check(const spec_recurrent_dims* dims, int32_t B, int32_t T) {
  if (!dims) return SPEC_ERR_INVALID_ARG;
  if (dims->n_heads < 1 || (dims->head_dim != 64 && dims->head_dim != 128) || dims->conv_width < 1 ||
      dims->conv_width > REC_MAX_W || dims->n_slots < 1)
    return SPEC_ERR_SHAPE;
  if (B < 0 || B > 65535 || T < 1 || T > REC_MAX_T) return SPEC_ERR_INVALID_ARG;
  // the largest tensor, the snapshots, must index within size_t and the
  // channel index within int
  if ((int64_t)3 * dims->n_heads * dims->head_dim > (1 << 24)) return SPEC_ERR_SHAPE;
  return SPEC_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

template <int D>
static hipError_t rec_launch(int which, const RecParams& p, hipStream_t s) {
  const dim3 grid(p.H, p.B);
  if (which == 0) rec_verify_kernel<D><<<grid, REC_THREADS, 0, s>>>(p);
  else if (which == 1) rec_replay_kernel<D><<<grid, REC_THREADS, 0, s>>>(p);
  else rec_scatter_kernel<D><<<grid, REC_THREADS, 0, s>>>(p);
  return hipGetLastError();
}

static spec_status rec_run(int which, int D, const RecParams& p, hipStream_t s) {
  if (p.B == 0) return SPEC_OK;
  const hipError_t e = D == 64 ? rec_launch<64>(which, p, s) : rec_launch<128>(which, p, s);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_DEVICE;
}

}  // namespace sv

using namespace sv;

extern "C" {

spec_status spec_recurrent_verify(const spec_recurrent_dims* dims, int32_t B, int32_t T, const float* d_x,
                                  const float* d_gate, const float* d_beta, const float* d_conv_w,
                                  const int32_t* d_slot, const float* d_conv_state, const float* d_state,
                                  float* d_out, float* d_snapshots, void* stream) {
  const spec_status st = rec_check(dims, B, T);
  if (st != SPEC_OK) return st;
  if (!d_x || !d_gate || !d_beta || !d_conv_w || !d_state || !d_out) return SPEC_ERR_INVALID_ARG;
  if (dims->conv_width > 1 && !d_conv_state) return SPEC_ERR_INVALID_ARG;
  if (!d_slot && dims->n_slots < B) return SPEC_ERR_INVALID_ARG;
  const void* ptrs[] = {d_x, d_gate, d_beta, d_conv_w, d_slot, d_conv_state, d_state, d_out, d_snapshots};
  for (const void* q : ptrs)
    if (!aligned16(q)) return SPEC_ERR_INVALID_ARG;
  RecParams p{};
  p.B = B, p.T = T, p.H = dims->n_heads, p.W = dims->conv_width, p.n_slots = dims->n_slots;
  p.x = d_x, p.gate = d_gate, p.beta = d_beta, p.conv_w = d_conv_w, p.slot = d_slot;
  p.conv_state = const_cast<float*>(d_conv_state);  // read only in this kernel
  p.state = const_cast<float*>(d_state);            // read only in this kernel
  p.out = d_out, p.snap = d_snapshots;
  return rec_run(0, dims->head_dim, p, (hipStream_t)stream);
}

spec_status spec_recurrent_commit(const spec_recurrent_dims* dims, int32_t B, int32_t T, const float* d_x,
                                  const float* d_gate, const float* d_beta, const float* d_conv_w,
                                  const int32_t* d_slot, const int32_t* d_num_accepted,
                                  const float* d_snapshots, float* d_conv_state, float* d_state, void* stream) {
  const spec_status st = rec_check(dims, B, T);
  if (st != SPEC_OK) return st;
  if (!d_num_accepted || !d_state) return SPEC_ERR_INVALID_ARG;
  if (dims->conv_width > 1 && (!d_conv_state || !d_x)) return SPEC_ERR_INVALID_ARG;
  if (!d_snapshots && (!d_x || !d_gate || !d_beta || !d_conv_w)) return SPEC_ERR_INVALID_ARG;
  if (!d_slot && dims->n_slots < B) return SPEC_ERR_INVALID_ARG;
  const void* ptrs[] = {d_x, d_gate, d_beta, d_conv_w, d_slot, d_num_accepted, d_snapshots, d_conv_state, d_state};
  for (const void* q : ptrs)
    if (!aligned16(q)) return SPEC_ERR_INVALID_ARG;
  RecParams p{};
  p.B = B, p.T = T, p.H = dims->n_heads, p.W = dims->conv_width, p.n_slots = dims->n_slots;
  p.x = d_x, p.gate = d_gate, p.beta = d_beta, p.conv_w = d_conv_w, p.slot = d_slot;
  p.nacc = d_num_accepted, p.snap_in = d_snapshots, p.conv_state = d_conv_state, p.state = d_state;
  return rec_run(d_snapshots ? 2 : 1, dims->head_dim, p, (hipStream_t)stream);
}

}  // extern "C"

extern "C" {

spec_status spec_recurrent_commit_verify(const spec_recurrent_dims* dims, int32_t B, int32_t T_prev,
                                         const float* d_prev_x, const float* d_prev_gate, const float* d_prev_beta,
                                         const int32_t* d_prev_accepted, int32_t T, const float* d_x,
                                         const float* d_gate, const float* d_beta, const float* d_conv_w,
                                         const int32_t* d_slot, float* d_conv_state, float* d_state, float* d_out,
                                         void* stream) {
  const spec_status st = rec_check(dims, B, T);
  if (st != SPEC_OK) return st;
  if (T_prev < 0 || T_prev > REC_MAX_T) return SPEC_ERR_INVALID_ARG;
  if (!d_x || !d_gate || !d_beta || !d_conv_w || !d_state || !d_out) return SPEC_ERR_INVALID_ARG;
  if (dims->conv_width > 1 && !d_conv_state) return SPEC_ERR_INVALID_ARG;
  if (T_prev > 0 && (!d_prev_x || !d_prev_gate || !d_prev_beta || !d_prev_accepted)) return SPEC_ERR_INVALID_ARG;
  if (!d_slot && dims->n_slots < B) return SPEC_ERR_INVALID_ARG;
  const void* ptrs[] = {d_prev_x, d_prev_gate, d_prev_beta, d_prev_accepted, d_x, d_gate, d_beta, d_conv_w,
                        d_slot, d_conv_state, d_state, d_out};
  for (const void* q : ptrs)
    if (!aligned16(q)) return SPEC_ERR_INVALID_ARG;
  RecParams p{};
  p.B = B, p.T = T, p.H = dims->n_heads, p.W = dims->conv_width, p.n_slots = dims->n_slots;
  p.x = d_x, p.gate = d_gate, p.beta = d_beta, p.conv_w = d_conv_w, p.slot = d_slot;
  p.conv_state = d_conv_state, p.state = d_state, p.out = d_out;
  RecParams pp = p;
  pp.T = T_prev;
  pp.x = d_prev_x, pp.gate = d_prev_gate, pp.beta = d_prev_beta, pp.nacc = d_prev_accepted;
  if (B == 0) return SPEC_OK;
  const dim3 grid(p.H, p.B);
  hipStream_t s = (hipStream_t)stream;
  if (dims->head_dim == 64) rec_commit_verify_kernel<64><<<grid, REC_THREADS, 0, s>>>(p, pp);
  else rec_commit_verify_kernel<128><<<grid, REC_THREADS, 0, s>>>(p, pp);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_DEVICE;
}

}  // extern "C"
