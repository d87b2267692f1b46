// Host runtime behind the C ABI: validation, workspace carving, the launch
// sequence of one verify step, accept dispatch and per-kernel event timing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/spec_verify.h"
#include "launch.h"

using namespace sv;

namespace {

constexpr size_t ALIGN = 256;
size_t align_up(size_t v) { return (v + ALIGN - 1) & ~(ALIGN - 1); }

bool valid_config(const spec_config* c) {
  if (!c) return false;
  if (c->n_layers < 1 || c->d_model < 64 || c->n_heads < 1 || c->n_kv_heads < 1 || c->d_ffn < 64 ||
      c->vocab < 2)
    return false;
  if (c->n_heads % c->n_kv_heads) return false;
  if (c->head_dim != 64 && c->head_dim != 128) return false;
  if (c->d_model % 64 || c->d_ffn % 64 || (c->n_heads * c->head_dim) % 64) return false;
  if (c->weight_dtype != SPEC_DTYPE_F32 && c->weight_dtype != SPEC_DTYPE_BF16) return false;
  if (c->max_batch < 1 || c->max_rows_per_seq < 1 || c->max_rows_per_seq > 128) return false;
  if (c->max_ctx < 64 || c->max_ctx % 64 || c->max_ctx < c->max_rows_per_seq) return false;
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 1.f)) return false;
  if (c->kv_page_size != 0 && c->kv_page_size != KV_PAGE) return false;
  if (c->kv_page_size && c->kv_pages < 1) return false;
  return true;
}

// elements of one layer's K (or V) region
size_t kv_region_elems(const spec_config& c) {
  if (c.kv_page_size) return (size_t)c.kv_pages * c.n_kv_heads * KV_PAGE * c.head_dim;
  return (size_t)c.max_batch * c.n_kv_heads * c.max_ctx * c.head_dim;
}

// Context splits per (sequence, KV head, query group).  The larger of
//   * enough workgroups to fill the GPU: ~512 with the 16-query form (two
//     per CU), ~256 with the one-per-CU forms;
//   * splits of ~512 keys (1024 for 32-query tiles, whose waves do twice the
//     work per block), so a workgroup's fixed cost is spread over enough
//     blocks;
// bounded by splits of at least 128 keys, ~4096 context workgroups (16-query
// form) or ~2048 (the others), and a combine of at most 128 partials.
// Measured on the 8B shape: B=1, 2K context: 17 (the 128-key bound); B=16,
// 32K: 32 at T=1, 16 at T=8; B=128, 1K: 2 at T=4 (150 against 212 us for 4),
// 1 at T=8 (265 against 299 us for 2).
// The two forms with two workgroups per CU (16-query tiles, and 32-query
// tiles in LDS at head width 128) then take
//   * fewer splits where that makes their context and suffix workgroups one
//     round of the 512 resident ones (the suffix workgroups are dispatched
//     last, so a second round would hold only them) while a workgroup still
//     sees at most 2048 keys (4096 in the LDS form): at 1K context B=8 8 -> 4
//     splits, B=16 4 -> 3, B=32 2 -> 1 (attention 16.5 -> 15.2, 29.1 -> 25.3
//     and 43.0 -> 37.1 us per layer); tree [4,4,2,2] at B=1, 4K 4 -> 2
//     (43.6 -> 40.7 us);
//   * one split (LDS form) when its units alone number 256 or more and the
//     context is at most 8K: tree [4,4,2,2] at B=4, 4K (480 units) 1 split
//     against 4 from the rule above, 114 against 137 us per layer (2: 121,
//     3: 129, 6: 159).
int attn_splits(const spec_config& c, int B, int T, bool tree) {
  const int nq = (c.n_heads / c.n_kv_heads) * T;
  const int QT = attn_query_tiles(nq, c.head_dim), QGW = attn_groups_per_wg(nq, c.head_dim);
  const int nqg = (nq + 16 * QT - 1) / (16 * QT);
  const int units = B * c.n_kv_heads * ((nqg + QGW - 1) / QGW);
  const bool two_per_cu = QT == 1 && QGW == 1;
  const int fill = ((two_per_cu ? 512 : 256) + units - 1) / units;
  const int keys = std::max(1, c.max_ctx / (QT == 2 ? 1024 : 512));
  int s = std::max(fill, keys);
  s = std::min(s, (c.max_ctx + 127) / 128);
  const int cap = two_per_cu ? std::max(1, (4096 + units - 1) / units) : std::max(1, 2048 / units);
  s = std::min(s, cap);
  const bool lds_form = QT == 2 && c.head_dim == 128;
  if (two_per_cu || lds_form) {
    const int one = 512 / units - attn_suffix_cols(tree, units, QT, QGW);
    if (one >= 1 && (c.max_ctx + one - 1) / one <= (lds_form ? 4096 : 2048)) s = std::min(s, one);
  }
  if (lds_form && units >= 256 && c.max_ctx <= 8192) s = 1;
  return std::max(1, std::min(s, 127));
}

// Split-K scratch of the GEMMs: the skinny residual GEMM's [2][8][d], the
// 32-row tiled kernel's [S <= 8][M <= 64][pairs][2] partial sums (it splits
// only launches of at most 64 rows, and only while they fit) and the
// large-tile kernel's [S][M][pairs][2] for the slices it would choose on a
// 256-CU device at every row count from 64 to the largest.
size_t gemm_part_floats(const spec_config& c) {
  const size_t Mmax = (size_t)c.max_batch * c.max_rows_per_seq;
  const size_t qkv_pairs = (size_t)(c.n_heads + 2 * c.n_kv_heads) * c.head_dim / 2;
  const size_t pairs = std::max<size_t>(qkv_pairs, c.d_model);
  size_t need = std::max((size_t)GEMM_KSPLIT * 8 * c.d_model, 8 * std::min<size_t>(Mmax, 64) * pairs * 2);
  if (c.weight_dtype == SPEC_DTYPE_BF16) {
    const int d = c.d_model, F = c.d_ffn, HD = c.n_heads * c.head_dim;
    auto tile_pairs = [](int n) { return (size_t)((n + 255) / 256) * 128; };
    const size_t np[5] = {qkv_pairs, tile_pairs(d), (size_t)F, tile_pairs(d), tile_pairs(c.vocab)};
    const int K[5] = {d, HD, d, F, d};
    for (size_t M = 64; M <= Mmax; ++M)
      for (int g = 0; g < 5; ++g) need = std::max(need, gemm_big_part_floats((int)M, np[g], K[g], 256));
  }
  return need;
}

// bf16 hi/lo planes of the widest activation rows the tiled GEMM splits
size_t gemm_xs_elems(const spec_config& c) {
  const size_t Mmax = (size_t)c.max_batch * c.max_rows_per_seq;
  const size_t K = std::max<size_t>(std::max<size_t>(c.d_model, c.d_ffn), (size_t)c.n_heads * c.head_dim);
  return Mmax >= 5 ? 2 * Mmax * K : 0;
}

// Shape of one forward: B sequences, T rows each (ragged: at most T, M rows
// in all, padding included), a token tree or a chain.
struct StepShape {
  int B, T, M;
  bool tree, ragged;
  bool operator==(const StepShape& o) const {
    return B == o.B && T == o.T && M == o.M && tree == o.tree && ragged == o.ragged;
  }
};

struct Layout {
  size_t x, x2, q, ksuf, vsuf, attn, act, part_o, part_ml, rope_cos, rope_sin;
  size_t tok, pos, slot, anc, kvw, rstart, rlen, rseq, gpart, gxs, gssq, rowstat, rowms, rsum, nacc, twalk, tpath, gxs2, fcnt, fmass, fstate, fres,
      flags, total;
};

Layout plan(const spec_config& c) {
  Layout L{};
  const size_t Mmax = (size_t)c.max_batch * c.max_rows_per_seq;
  const size_t D = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads;
  size_t part = 0;
  for (int B = 1; B <= c.max_batch; ++B)
    for (int T = 1; T <= c.max_rows_per_seq; ++T)
      for (int tree = 0; tree < 2; ++tree) {
        const size_t n = (size_t)attn_nsplit(attn_splits(c, B, T, tree != 0)) * B * Hq * T;
        part = std::max(part, n);
      }
  const int nch = accept_chunks(c.vocab);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.x = take(Mmax * c.d_model * 4);
  L.x2 = take(Mmax * c.d_model * 4);  // residual rows, second buffer (deferred reduce)
  L.q = take(Mmax * Hq * D * 4);
  L.ksuf = take(Mmax * Hkv * D * 4);
  L.vsuf = take(Mmax * Hkv * D * 4);
  L.attn = take(Mmax * Hq * D * 4);
  L.act = take(Mmax * c.d_ffn * 4);
  L.part_o = take(part * D * 4);
  L.part_ml = take(part * 2 * 4);
  L.rope_cos = take((size_t)c.max_ctx * (D / 2) * 4);
  L.rope_sin = take((size_t)c.max_ctx * (D / 2) * 4);
  L.tok = take(Mmax * 4);
  L.pos = take(Mmax * 4);
  L.slot = take(Mmax * 4);
  L.anc = take(Mmax * 2 * 8);
  L.kvw = take((size_t)c.max_batch * 4);
  L.rstart = take((size_t)c.max_batch * 4);
  L.rlen = take((size_t)c.max_batch * 4);
  L.rseq = take(Mmax * 4);
  L.gpart = take(gemm_part_floats(c) * 4);
  L.gxs = take(gemm_xs_elems(c) * 2);
  L.gxs2 = take(gemm_xs_elems(c) * 2);  // the down projection's planes, written by gate/up
  L.gssq = take(Mmax * SSQ_BLK * 4);
  L.rowstat = take(Mmax * nch * 2 * 4);
  L.rowms = take(Mmax * 2 * 4);
  L.rsum = take((size_t)c.max_batch * nch * 4);
  L.nacc = take((size_t)c.max_batch * 4);
  L.twalk = take(tree_walk_bytes(c.max_batch, nch));
  L.tpath = take((size_t)c.max_batch * TPATH * 4);
  // top-k / top-p selection: histograms and state are indexed by a batch
  // row below SEL_ROWS in each of two alternating buffers
  L.fcnt = take((size_t)2 * SEL_ROWS * nch * 256 * 4);
  L.fmass = take((size_t)2 * SEL_ROWS * nch * 256 * 8);
  L.fstate = take((size_t)2 * SEL_ROWS * sizeof(SelState));
  L.fres = take(Mmax * sizeof(SelRule));
  L.flags = take(256);
  L.total = off;
  return L;
}

constexpr size_t kMaxGraphs = 32;  // recorded shapes kept per handle

const char* kClassNames[] = {"prep_embed", "gemm_qkv", "attention", "attn_combine", "gemm_o",
                             "gemm_gate_up", "gemm_down", "gemm_lm_head", "accept"};
enum KClass { K_PREP, K_QKV, K_ATTN, K_COMB, K_O, K_GU, K_DOWN, K_LM, K_ACC, K_N };

}  // namespace

struct spec_handle {
  spec_config cfg;
  int device = 0;
  std::vector<const void*> w;
  uint16_t* kv = nullptr;
  char* ws = nullptr;
  Layout lay{};
  // profiling
  bool prof = false;
  struct Rec {
    int cls;
    hipEvent_t a, b;
    double bytes;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  // recorded layer sequences, one per step shape, replayed as HIP graphs
  struct Graph {
    StepShape sh;
    hipGraphExec_t exec;
    uint64_t used;
    hipEvent_t done;  // recorded after each replay; null for a shape on direct launches
  };
  bool graphs = true;
  const int32_t* kv_table = nullptr;  // paged cache: [max_batch][kv_ppseq] page ids
  int kv_ppseq = 0;
  hipStream_t cap = nullptr;  // private stream used only to record
  std::vector<Graph> gcache;
  std::vector<Graph> retired;  // evicted recordings whose last replay may still run
  uint64_t gclock = 0;
  int64_t launches[K_N] = {};
  double ms[K_N] = {};
  double bytes[K_N] = {};

  template <typename P>
  P* at(size_t off) const { return (P*)(ws + off); }
  const void* W(size_t i) const { return w[i]; }
  size_t layer_w(int l, int k) const { return 1 + 6 * (size_t)l + k; }

  hipEvent_t ev() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

namespace {

// Bracket one launch with events when profiling is on.
template <typename F>
hipError_t timed(spec_handle* h, int cls, double bytes, hipStream_t s, F&& launch) {
  if (!h->prof) return launch();
  hipEvent_t a = h->ev(), b = h->ev();
  if (!a || !b) return hipErrorOutOfMemory;
  hipEventRecord(a, s);
  hipError_t e = launch();
  hipEventRecord(b, s);
  h->recs.push_back({cls, a, b, bytes});
  return e;
}

spec_status dev(hipError_t e) { return e == hipSuccess ? SPEC_OK : SPEC_ERR_DEVICE; }

// GEMM over M rows in launches of at most 8 activation rows.
// the cache addressing of the kernels: dense, or paged through the table
KvMap kv_map(const spec_handle* h) {
  const spec_config& c = h->cfg;
  if (!c.kv_page_size) return KvMap{nullptr, 0, 0, c.max_ctx};
  return KvMap{h->kv_table, h->kv_ppseq, c.kv_pages, c.max_ctx};
}

// the library's scratch buffers in a GEMM's parameters
void gemm_scratch(const spec_handle* h, GemmParams& p) {
  p.part = h->at<float>(h->lay.gpart);
  p.part_floats = gemm_part_floats(h->cfg);
  if (!p.xs_ready || !p.xs) p.xs = h->at<uint16_t>(h->lay.gxs);  // a producer's planes stay
  p.xs_elems = gemm_xs_elems(h->cfg);
  p.xs_ssq = h->at<float>(h->lay.gssq);
}

// The launch of p over M rows runs on the tiled kernels, which read the
// activation rows as bf16 hi/lo planes.
bool rows_tiled(const spec_handle* h, GemmParams p, int M) {
  gemm_scratch(h, p);
  p.M = M;
  return gemm_tiled_ok(p);
}

// The launch of p over M rows is a K-split residual GEMM on the tiled kernels
// whose finish can also write the next GEMM's planes (norm_next).
bool finish_prepares(const spec_handle* h, GemmParams p, int M) {
  gemm_scratch(h, p);
  p.M = M;
  return gemm_finish_prepares(p);
}

// The down projection of M rows prepares the next launch's activation planes
// (the next layer's QKV, or the LM head after the last layer) when its finish
// can and that launch runs on the tiled kernels too; both take the same
// activation width d_model.
bool down_prepares_next(const spec_handle* h, int M) {
  const spec_config& c = h->cfg;
  GemmParams gd{};
  gd.wdtype = c.weight_dtype; gd.N = c.d_model; gd.K = c.d_ffn; gd.epi = EPI_RESID;
  GemmParams nx{};
  nx.wdtype = c.weight_dtype; nx.K = c.d_model; nx.N = c.vocab; nx.epi = EPI_STORE;
  GemmParams nq{};
  nq.wdtype = c.weight_dtype; nq.K = c.d_model; nq.N = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim; nq.epi = EPI_QKV;
  return finish_prepares(h, gd, M) && rows_tiled(h, nx, M) && rows_tiled(h, nq, M);
}

hipError_t gemm_rows(spec_handle* h, int cls, GemmParams p, int M, hipStream_t s) {
  const size_t wbytes = h->cfg.weight_dtype == SPEC_DTYPE_BF16 ? 2 : 4;
  const size_t nrows = (p.epi == EPI_SWIGLU) ? (size_t)2 * p.F : (size_t)p.N;
  const size_t out_cols = (p.epi == EPI_SWIGLU) ? p.F : p.N;
  gemm_scratch(h, p);
  if (p.xpart && M > 8) return hipErrorInvalidValue;  // the partial sums are one launch's rows
  {
    GemmParams q = p;
    q.M = M;
    if (gemm_tiled_ok(q)) {
      // many rows: one tiled launch reads the weights once per 128 rows
      const double bytes = (double)nrows * p.K * wbytes + (double)M * p.K * 4 +
                           (double)M * out_cols * 4 * (p.epi == EPI_RESID ? 2 : 1);
      return timed(h, cls, bytes, s, [&] { return launch_gemm(q, s); });
    }
  }
  for (int m0 = 0; m0 < M; m0 += 8) {
    GemmParams q = p;
    q.M = std::min(8, M - m0);
    q.X = p.X + (size_t)m0 * p.ldx;
    q.m0 = m0;
    if (p.out) q.out = p.out + (size_t)m0 * p.ldo;
    double bytes = (double)q.M * p.K * 4 + (double)q.M * out_cols * 4 * (p.epi == EPI_RESID ? 2 : 1);
    if (m0 == 0) bytes += (double)nrows * p.K * wbytes;  // weights count once per GEMM
    hipError_t e = timed(h, cls, bytes, s, [&] { return launch_gemm(q, s); });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

namespace {

// At M rows the down projection runs as K slices and the next layer's QKV
// launch can finish their reduce in its prologue: then the reduce kernel of
// every layer but the last is left out.  The residual rows alternate between
// two buffers, because the QKV launch reads the old rows in every workgroup
// while its first workgroup writes the completed ones.
bool defer_down_reduce(const spec_handle* h, int M) {
  const spec_config& c = h->cfg;
  GemmParams gd{};
  gd.wdtype = c.weight_dtype; gd.ldx = c.d_ffn; gd.N = c.d_model; gd.K = c.d_ffn; gd.M = M;
  gd.epi = EPI_RESID; gd.ldo = c.d_model;
  gemm_scratch(h, gd);
  GemmParams gq{};
  gq.wdtype = c.weight_dtype; gq.ldx = c.d_model; gq.N = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  gq.K = c.d_model; gq.M = M; gq.epi = EPI_QKV;
  gq.norm_g = (const float*)h->W(h->layer_w(0, 0));
  gemm_scratch(h, gq);
  return c.n_layers > 1 && gemm_use_split(gd) && gemm_takes_xpart(gq);
}

// residual rows the LM head reads after the layers
float* final_residual(const spec_handle* h, int M) {
  const bool odd = defer_down_reduce(h, M) && (h->cfg.n_layers - 1) % 2 == 1;
  return h->at<float>(odd ? h->lay.x2 : h->lay.x);
}

// The per-layer kernels of a step.  They read only the weights, the cache and
// the workspace (kv_len through its copy made by the prep kernel), so for a
// given (B, T, chain/tree) the launch sequence is fixed and can be recorded.
hipError_t launch_layers(spec_handle* h, const StepShape& sh, hipStream_t s) {
  const spec_config& c = h->cfg;
  const Layout& L = h->lay;
  const int B = sh.B, T = sh.T;
  const bool tree = sh.tree;
  const int32_t* rstart = sh.ragged ? h->at<int32_t>(L.rstart) : nullptr;
  const int32_t* rlen = sh.ragged ? h->at<int32_t>(L.rlen) : nullptr;
  const int M = sh.M, d = c.d_model, D = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads, F = c.d_ffn;
  float* x = h->at<float>(L.x);
  float* q = h->at<float>(L.q);
  float* ks = h->at<float>(L.ksuf);
  float* vs = h->at<float>(L.vsuf);
  float* at = h->at<float>(L.attn);
  float* act = h->at<float>(L.act);
  int32_t* pos = h->at<int32_t>(L.pos);
  int32_t* slot = h->at<int32_t>(L.slot);
  uint64_t* anc = h->at<uint64_t>(L.anc);
  const int32_t* kvw = h->at<int32_t>(L.kvw);
  hipError_t e;
  const size_t per_region = kv_region_elems(c);  // elements of one K or V region
  const int splits = attn_splits(c, B, T, tree);
  const int nsplit = attn_nsplit(splits);
  const float scale = 1.0f / std::sqrt((float)D);
  const bool defer = defer_down_reduce(h, M);
  float* x2 = h->at<float>(L.x2);
  float* cur = x;  // residual rows entering the layer
  // the residual finishes write the next launch's planes and sums of squares
  // (no split launches in front of QKV, gate/up and the LM head)
  const bool down_next = down_prepares_next(h, M);

  for (int l = 0; l < c.n_layers; ++l) {
    const float* g1 = (const float*)h->W(h->layer_w(l, 0));
    const void* wqkv = h->W(h->layer_w(l, 1));
    const void* wo = h->W(h->layer_w(l, 2));
    const float* g2 = (const float*)h->W(h->layer_w(l, 3));
    const void* wgu = h->W(h->layer_w(l, 4));
    const void* wdn = h->W(h->layer_w(l, 5));
    uint16_t* kreg = h->kv + (size_t)(2 * l) * per_region;
    uint16_t* vreg = h->kv + (size_t)(2 * l + 1) * per_region;

    // with the previous layer's down reduce deferred, the QKV launch
    // completes the rows into the other buffer, which the layer then updates
    float* nxt = (defer && l > 0) ? (cur == x ? x2 : x) : cur;
    GemmParams gq{};
    gq.W = wqkv; gq.wdtype = c.weight_dtype; gq.X = cur; gq.ldx = d; gq.N = (Hq + 2 * Hkv) * D; gq.K = d;
    if (nxt != cur) {
      gq.xpart = h->at<float>(L.gpart);
      gq.xout = nxt;
    }
    gq.norm_g = g1; gq.eps = c.rms_eps;
    gq.xs_ready = gq.ssq_ready = down_next && l > 0;
    gq.epi = EPI_QKV; gq.pos = pos; gq.slot = slot;
    gq.rope_cos = h->at<float>(L.rope_cos); gq.rope_sin = h->at<float>(L.rope_sin);
    gq.q_out = q; gq.k_out = ks; gq.v_out = vs; gq.kcache = kreg; gq.vcache = vreg;
    gq.T = T; gq.Hq = Hq; gq.Hkv = Hkv; gq.D = D; gq.max_ctx = c.max_ctx;
    gq.seq = sh.ragged ? h->at<int32_t>(L.rseq) : nullptr;
    gq.kvm = kv_map(h);
    if ((e = gemm_rows(h, K_QKV, gq, M, s)) != hipSuccess) return e;

    AttnParams ap{q, kreg, vreg, kvw, ks, vs, tree ? anc : nullptr, h->at<float>(L.part_o),
                  h->at<float>(L.part_ml), B, T, Hq, Hkv, D, c.max_ctx, splits, scale, rstart, rlen, kv_map(h)};
    e = timed(h, K_ATTN, 0, s, [&] { return launch_attention(ap, s); });
    if (e != hipSuccess) return e;
    GemmParams go{};
    go.W = wo; go.wdtype = c.weight_dtype; go.X = at; go.ldx = Hq * D; go.N = d; go.K = Hq * D;
    go.epi = EPI_RESID; go.out = nxt; go.ldo = d;
    // on the tiled kernels the O projection reads its activation planes, which
    // the combine writes beside its fp32 output (no split launch)
    go.xs_ready = rows_tiled(h, go, M);
    CombineParams cp{h->at<float>(L.part_o), h->at<float>(L.part_ml), nsplit, at, B, T, Hq, Hkv, D, rstart, rlen,
                     go.xs_ready ? h->at<uint16_t>(L.gxs) : nullptr, M};
    e = timed(h, K_COMB, 0, s, [&] { return launch_attn_combine(cp, s); });
    if (e != hipSuccess) return e;
    GemmParams gg{};
    gg.W = wgu; gg.wdtype = c.weight_dtype; gg.X = nxt; gg.ldx = d; gg.N = 2 * F; gg.K = d;
    gg.norm_g = g2; gg.eps = c.rms_eps;
    gg.epi = EPI_SWIGLU; gg.out = act; gg.ldo = F; gg.F = F;
    if (go.xs_ready && rows_tiled(h, gg, M) && finish_prepares(h, go, M)) {
      // O's finish writes gate/up's planes (the O launch has read its own
      // from the same buffer before its finish runs)
      go.norm_next = g2;
      go.xs_next = h->at<uint16_t>(L.gxs);
      gg.xs_ready = gg.ssq_ready = true;
    }
    if ((e = gemm_rows(h, K_O, go, M, s)) != hipSuccess) return e;

    GemmParams gd{};
    gd.W = wdn; gd.wdtype = c.weight_dtype; gd.X = act; gd.ldx = F; gd.N = d; gd.K = F;
    gd.epi = EPI_RESID; gd.out = nxt; gd.ldo = d;
    gd.defer_reduce = defer && l + 1 < c.n_layers;
    if (rows_tiled(h, gg, M) && rows_tiled(h, gd, M)) {
      // the gate/up epilogue writes the down projection's planes into a second
      // buffer (gate/up is still reading its own from the first)
      gg.xs_out = h->at<uint16_t>(L.gxs2);
      gd.xs = gg.xs_out;
      gd.xs_ready = true;
    }
    if (down_next) {
      // the next layer's attention norm, or the final norm before the LM head
      gd.norm_next = (const float*)(l + 1 < c.n_layers ? h->W(h->layer_w(l + 1, 0)) : h->W(1 + 6 * (size_t)c.n_layers));
      gd.xs_next = h->at<uint16_t>(L.gxs);
    }
    if ((e = gemm_rows(h, K_GU, gg, M, s)) != hipSuccess) return e;
    if ((e = gemm_rows(h, K_DOWN, gd, M, s)) != hipSuccess) return e;
    cur = nxt;
  }
  return hipSuccess;
}

// Recordings that left the cache are destroyed once their last replay has
// finished (its event has completed), never by waiting for it.
void destroy_graph(spec_handle::Graph& g) {
  if (g.exec) hipGraphExecDestroy(g.exec);
  if (g.done) hipEventDestroy(g.done);
  g.exec = nullptr;
  g.done = nullptr;
}
void sweep_retired(spec_handle* h, bool wait) {
  for (size_t i = 0; i < h->retired.size();) {
    spec_handle::Graph& g = h->retired[i];
    const bool finished = !g.done || (wait ? hipEventSynchronize(g.done) == hipSuccess
                                           : hipEventQuery(g.done) == hipSuccess);
    if (!finished && !wait) {
      ++i;
      continue;
    }
    destroy_graph(g);
    h->retired.erase(h->retired.begin() + i);
  }
}
void retire_all(spec_handle* h) {
  for (auto& g : h->gcache) h->retired.push_back(g);
  h->gcache.clear();
}

// Replay of the recorded layer sequence for this shape, recorded on first use
// on the handle's private stream (recording runs nothing).  Returns null when
// recording or instantiation fails.
hipGraphExec_t layer_graph(spec_handle* h, const StepShape& sh) {
  if (!h->cap && hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking) != hipSuccess) {
    h->cap = nullptr;
    return nullptr;
  }
  if (hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal) != hipSuccess) return nullptr;
  const hipError_t le = launch_layers(h, sh, h->cap);
  hipGraph_t graph = nullptr;
  const hipError_t ce = hipStreamEndCapture(h->cap, &graph);
  if (le != hipSuccess || ce != hipSuccess || !graph) {
    if (graph) hipGraphDestroy(graph);
    return nullptr;
  }
  hipGraphExec_t ex = nullptr;
  const hipError_t ie = hipGraphInstantiate(&ex, graph, nullptr, nullptr, 0);
  hipGraphDestroy(graph);
  if (ie != hipSuccess) return nullptr;
  hipEvent_t done = nullptr;
  if (hipEventCreateWithFlags(&done, hipEventDisableTiming) != hipSuccess) {
    hipGraphExecDestroy(ex);
    return nullptr;
  }
  if (h->gcache.size() >= kMaxGraphs) {
    // the least recently used shape leaves the cache; it may still be running
    size_t old = 0;
    for (size_t i = 1; i < h->gcache.size(); ++i)
      if (h->gcache[i].used < h->gcache[old].used) old = i;
    h->retired.push_back(h->gcache[old]);
    h->gcache.erase(h->gcache.begin() + old);
  }
  h->gcache.push_back({sh, ex, ++h->gclock, done});
  return ex;
}

spec_status replay(spec_handle::Graph& g, hipStream_t s) {
  if (hipGraphLaunch(g.exec, s) != hipSuccess) return SPEC_ERR_DEVICE;
  return dev(hipEventRecord(g.done, s));
}

spec_status run_layers(spec_handle* h, const StepShape& sh, hipStream_t s) {
  sweep_retired(h, false);
  if (h->graphs && !h->prof) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return SPEC_ERR_DEVICE;
    if (cs == hipStreamCaptureStatusNone) {
      // the caller is not recording: replay our own recording of this shape
      for (auto& g : h->gcache)
        if (g.sh == sh) {
          g.used = ++h->gclock;
          // a shape whose recording failed stays on direct launches
          return g.exec ? replay(g, s) : dev(launch_layers(h, sh, s));
        }
      // first step of this shape: record its launch sequence (recording runs
      // nothing), then replay it
      const hipGraphExec_t ex = layer_graph(h, sh);
      if (!ex) {
        hipGetLastError();  // clear a capture error; this shape keeps direct launches
        h->gcache.push_back({sh, nullptr, ++h->gclock, nullptr});
        return dev(launch_layers(h, sh, s));
      }
      return replay(h->gcache.back(), s);
    }
  }
  return dev(launch_layers(h, sh, s));
}

}  // namespace

extern "C" {

const char* spec_status_str(spec_status s) {
  switch (s) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_INVALID_ARG: return "invalid argument";
    case SPEC_ERR_SHAPE: return "unsupported model shape";
    case SPEC_ERR_CAPACITY: return "beyond the capacity given at init";
    case SPEC_ERR_UNSUPPORTED: return "unsupported dtype or device";
    case SPEC_ERR_DEVICE: return "HIP runtime error";
    case SPEC_ERR_STATE: return "invalid handle state";
    case SPEC_ERR_DATA: return "device-side data error";
    default: return "unknown status";
  }
}

size_t spec_workspace_bytes(const spec_config* cfg) {
  if (!valid_config(cfg)) return 0;
  return plan(*cfg).total;
}

size_t spec_kv_cache_bytes(const spec_config* c) {
  if (!valid_config(c)) return 0;
  return (size_t)c->n_layers * 2 * kv_region_elems(*c) * 2;
}

spec_status spec_verify_init(const spec_config* cfg, const void* const* d_weights, size_t n_weights,
                             void* d_kv_cache, void* d_workspace, size_t workspace_bytes,
                             void* stream, spec_handle** out) {
  if (!cfg || !d_weights || !d_kv_cache || !d_workspace || !out) return SPEC_ERR_INVALID_ARG;
  *out = nullptr;
  if (!valid_config(cfg)) return SPEC_ERR_SHAPE;
  const size_t nw = 1 + 6 * (size_t)cfg->n_layers + 2;
  if (n_weights != nw) return SPEC_ERR_INVALID_ARG;
  for (size_t i = 0; i < nw; ++i)
    if (!d_weights[i] || ((uintptr_t)d_weights[i] & 15)) return SPEC_ERR_INVALID_ARG;
  if ((uintptr_t)d_workspace & (ALIGN - 1)) return SPEC_ERR_INVALID_ARG;
  Layout L = plan(*cfg);
  if (workspace_bytes < L.total) return SPEC_ERR_CAPACITY;

  int devid = 0;
  if (hipGetDevice(&devid) != hipSuccess) return SPEC_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, devid) != hipSuccess) return SPEC_ERR_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return SPEC_ERR_UNSUPPORTED;

  spec_handle* h = new spec_handle();
  h->cfg = *cfg;
  h->device = devid;
  h->w.assign(d_weights, d_weights + nw);
  h->kv = (uint16_t*)d_kv_cache;
  h->ws = (char*)d_workspace;
  h->lay = L;

  // rotary tables: angle = pos * theta^(-2i/D), evaluated in double
  const int D = cfg->head_dim, half = D / 2;
  std::vector<float> cs((size_t)cfg->max_ctx * half), sn((size_t)cfg->max_ctx * half);
  for (int ps = 0; ps < cfg->max_ctx; ++ps)
    for (int i = 0; i < half; ++i) {
      const double inv = std::pow((double)cfg->rope_theta, -(2.0 * i) / D);
      const double a = (double)ps * inv;
      cs[(size_t)ps * half + i] = (float)std::cos(a);
      sn[(size_t)ps * half + i] = (float)std::sin(a);
    }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(h->at<float>(L.rope_cos), cs.data(), cs.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->at<float>(L.rope_sin), sn.data(), sn.size() * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemsetAsync(h->at<uint32_t>(L.flags), 0, 256, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    delete h;
    return SPEC_ERR_DEVICE;
  }
  *out = h;
  return SPEC_OK;
}

namespace {

// The forward of one step: prep + embedding, the recorded layers, the LM head.
spec_status verify_forward(spec_handle* h, const StepShape& sh, const int32_t* d_tokens, const int32_t* d_kv_len,
                           const int32_t* d_tree_parent, const int32_t* d_cu, float* d_logits, hipStream_t s) {
  const spec_config& c = h->cfg;
  if (c.kv_page_size && !h->kv_table) return SPEC_ERR_STATE;
  const Layout& L = h->lay;
  const int M = sh.M, d = c.d_model;
  const int V = c.vocab;
  const size_t wb = c.weight_dtype == SPEC_DTYPE_BF16 ? 2 : 4;
  float* x = h->at<float>(L.x);
  hipError_t e;

  PrepParams pp{d_tokens, d_kv_len, d_tree_parent, h->at<int32_t>(L.tok), h->at<int32_t>(L.pos),
                h->at<int32_t>(L.slot), h->at<uint64_t>(L.anc), h->at<uint32_t>(L.flags), h->W(0),
                c.weight_dtype, x, h->at<int32_t>(L.kvw), sh.B, sh.T, V, c.max_ctx, d,
                d_cu, M, h->at<int32_t>(L.rstart), h->at<int32_t>(L.rlen), h->at<int32_t>(L.rseq), kv_map(h)};
  e = timed(h, K_PREP, (double)M * d * (wb + 4), s, [&] { return launch_prep(pp, s); });
  if (e != hipSuccess) return SPEC_ERR_DEVICE;

  spec_status st = run_layers(h, sh, s);
  if (st != SPEC_OK) return st;

  const float* gf = (const float*)h->W(1 + 6 * (size_t)c.n_layers);
  GemmParams gl{};
  gl.W = h->W(2 + 6 * (size_t)c.n_layers); gl.wdtype = c.weight_dtype; gl.X = final_residual(h, M); gl.ldx = d;
  gl.N = V;
  gl.K = d; gl.epi = EPI_STORE; gl.out = d_logits; gl.ldo = V;
  gl.norm_g = gf; gl.eps = c.rms_eps;
  gl.xs_ready = gl.ssq_ready = down_prepares_next(h, M);  // the last down's finish wrote them
  if ((e = gemm_rows(h, K_LM, gl, M, s)) != hipSuccess) return SPEC_ERR_DEVICE;
  return SPEC_OK;
}

}  // namespace

spec_status spec_verify_step(spec_handle* h, int32_t B, int32_t T, const int32_t* d_tokens,
                             const int32_t* d_kv_len, const int32_t* d_tree_parent, float* d_logits,
                             void* stream) {
  if (!h || !d_tokens || !d_kv_len || !d_logits) return SPEC_ERR_INVALID_ARG;
  const spec_config& c = h->cfg;
  if (B < 1 || T < 1 || B > c.max_batch || T > c.max_rows_per_seq) return SPEC_ERR_CAPACITY;
  return verify_forward(h, StepShape{B, T, B * T, d_tree_parent != nullptr, false}, d_tokens, d_kv_len,
                        d_tree_parent, nullptr, d_logits, (hipStream_t)stream);
}

spec_status spec_verify_step_ragged(spec_handle* h, int32_t B, int32_t max_len, int32_t rows,
                                    const int32_t* d_cu_rows, const int32_t* d_tokens, const int32_t* d_kv_len,
                                    float* d_logits, void* stream) {
  if (!h || !d_cu_rows || !d_tokens || !d_kv_len || !d_logits) return SPEC_ERR_INVALID_ARG;
  const spec_config& c = h->cfg;
  if (B < 1 || max_len < 1 || B > c.max_batch || max_len > c.max_rows_per_seq) return SPEC_ERR_CAPACITY;
  if (rows < 1 || rows > c.max_batch * c.max_rows_per_seq) return SPEC_ERR_CAPACITY;
  return verify_forward(h, StepShape{B, max_len, rows, false, true}, d_tokens, d_kv_len, nullptr, d_cu_rows,
                        d_logits, (hipStream_t)stream);
}

namespace {

// Shared by the chain / tree accept and the ragged chain accept: validate the
// sampling settings and launch.
spec_status accept_impl(spec_handle* h, AcceptParams ap, const spec_sampling* sampling, bool need_q,
                        hipStream_t s) {
  if (!sampling) return SPEC_ERR_INVALID_ARG;
  const float temp = sampling->temperature;
  if (!(temp >= 0.f) || !std::isfinite(temp)) return SPEC_ERR_INVALID_ARG;
  if (sampling->top_k < 0 || !(sampling->top_p >= 0.f && sampling->top_p <= 1.f)) return SPEC_ERR_INVALID_ARG;
  if (temp > 0.f && need_q && !ap.q) return SPEC_ERR_INVALID_ARG;
  if (ap.kv_len_out && !ap.kv_len) return SPEC_ERR_INVALID_ARG;
  const spec_config& c = h->cfg;
  if (c.kv_page_size && !h->kv_table && ap.parent && ap.kv_len_out) return SPEC_ERR_STATE;
  const Layout& L = h->lay;
  ap.temperature = temp; ap.replacement = sampling->tree_replacement ? 1 : 0;
  ap.seed = sampling->seed; ap.round = sampling->round;
  ap.rowstat = h->at<float>(L.rowstat); ap.rowms = h->at<float>(L.rowms); ap.rsum = h->at<float>(L.rsum);
  ap.nacc = h->at<int32_t>(L.nacc); ap.twalk = h->at<char>(L.twalk); ap.tpath = h->at<int32_t>(L.tpath); ap.flags = h->at<uint32_t>(L.flags);
  ap.kv_cache = h->kv; ap.L = c.n_layers; ap.maxB = c.max_batch; ap.Hkv = c.n_kv_heads; ap.D = c.head_dim;
  ap.max_ctx = c.max_ctx; ap.V = c.vocab; ap.nch = accept_chunks(c.vocab);
  ap.top_k = sampling->top_k; ap.top_p = sampling->top_p;
  ap.fcnt = h->at<uint32_t>(L.fcnt); ap.fmass = h->at<double>(L.fmass);
  ap.fstate = h->at<SelState>(L.fstate); ap.fres = h->at<SelRule>(L.fres);
  ap.kvm = kv_map(h);
  const double bytes = (double)ap.rows * c.vocab * 4 + (temp > 0 ? (double)ap.qrows * c.vocab * 4 : 0.0);
  return dev(timed(h, K_ACC, bytes, s, [&] { return launch_accept(ap, s); }));
}

}  // namespace

spec_status spec_accept(spec_handle* h, int32_t B, int32_t T, const float* d_logits, const float* d_q,
                        const int32_t* d_tokens, const int32_t* d_tree_parent,
                        const spec_sampling* sampling, int32_t* d_out_tokens, int32_t* d_num_accepted,
                        const int32_t* d_kv_len, int32_t* d_kv_len_out, void* stream) {
  if (!h || !d_logits || !d_tokens || !sampling || !d_out_tokens || !d_num_accepted)
    return SPEC_ERR_INVALID_ARG;
  const spec_config& c = h->cfg;
  if (B < 1 || T < 1 || B > c.max_batch || T > c.max_rows_per_seq) return SPEC_ERR_CAPACITY;
  AcceptParams ap{};
  ap.logits = d_logits; ap.q = d_q; ap.tokens = d_tokens; ap.parent = d_tree_parent;
  ap.out_tokens = d_out_tokens; ap.num_accepted = d_num_accepted; ap.kv_len = d_kv_len;
  ap.kv_len_out = d_kv_len_out;
  ap.B = B; ap.T = T; ap.rows = B * T; ap.qrows = d_tree_parent ? B * T : B * (T - 1);
  return accept_impl(h, ap, sampling, d_tree_parent || T > 1, (hipStream_t)stream);
}

spec_status spec_accept_ragged(spec_handle* h, int32_t B, int32_t max_len, int32_t rows, int32_t q_rows,
                               const int32_t* d_row_start, const int32_t* d_len, const int32_t* d_q_start,
                               const float* d_logits, const float* d_q, const int32_t* d_tokens,
                               const spec_sampling* sampling, int32_t* d_out_tokens, int32_t* d_num_accepted,
                               const int32_t* d_kv_len, int32_t* d_kv_len_out, void* stream) {
  if (!h || !d_row_start || !d_len || !d_logits || !d_tokens || !sampling || !d_out_tokens || !d_num_accepted)
    return SPEC_ERR_INVALID_ARG;
  const spec_config& c = h->cfg;
  if (B < 1 || max_len < 1 || B > c.max_batch || max_len > c.max_rows_per_seq) return SPEC_ERR_CAPACITY;
  if (rows < 1 || rows > c.max_batch * c.max_rows_per_seq || q_rows < 0) return SPEC_ERR_CAPACITY;
  const bool drafts = max_len > 1;
  if (sampling->temperature > 0.f && drafts && (!d_q || !d_q_start || q_rows < 1)) return SPEC_ERR_INVALID_ARG;
  AcceptParams ap{};
  ap.logits = d_logits; ap.q = d_q; ap.tokens = d_tokens; ap.parent = nullptr;
  ap.out_tokens = d_out_tokens; ap.num_accepted = d_num_accepted; ap.kv_len = d_kv_len;
  ap.kv_len_out = d_kv_len_out;
  ap.B = B; ap.T = max_len; ap.rows = rows; ap.qrows = q_rows;
  ap.rstart = d_row_start; ap.rlen = d_len; ap.qstart = d_q_start;
  return accept_impl(h, ap, sampling, drafts, (hipStream_t)stream);
}

spec_status spec_device_errors(spec_handle* h, uint32_t* flags, void* stream) {
  if (!h || !flags) return SPEC_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  uint32_t v = 0;
  uint32_t* d = h->at<uint32_t>(h->lay.flags);
  if (hipMemcpyAsync(&v, d, 4, hipMemcpyDeviceToHost, s) != hipSuccess) return SPEC_ERR_DEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return SPEC_ERR_DEVICE;
  if (hipMemsetAsync(d, 0, 4, s) != hipSuccess) return SPEC_ERR_DEVICE;
  if (hipStreamSynchronize(s) != hipSuccess) return SPEC_ERR_DEVICE;
  *flags = v;
  return SPEC_OK;
}

spec_status spec_profile_enable(spec_handle* h, int32_t enable) {
  if (!h) return SPEC_ERR_INVALID_ARG;
  h->prof = enable != 0;
  return SPEC_OK;
}

int32_t spec_profile_read(spec_handle* h, spec_kernel_stat* out, int32_t max_out, int32_t reset) {
  if (!h) return -1;
  for (auto& r : h->recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return -1;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return -1;
    h->launches[r.cls] += 1;
    h->ms[r.cls] += t;
    h->bytes[r.cls] += r.bytes;
    h->pool.push_back(r.a);
    h->pool.push_back(r.b);
  }
  h->recs.clear();
  int n = 0;
  for (int k = 0; k < K_N && n < max_out; ++k) {
    if (!out) break;
    std::memset(&out[n], 0, sizeof(spec_kernel_stat));
    std::snprintf(out[n].name, sizeof(out[n].name), "%s", kClassNames[k]);
    out[n].launches = h->launches[k];
    out[n].total_ms = h->ms[k];
    out[n].algo_bytes = h->bytes[k];
    ++n;
  }
  if (reset)
    for (int k = 0; k < K_N; ++k) h->launches[k] = 0, h->ms[k] = 0, h->bytes[k] = 0;
  return n;
}

spec_status spec_profile_gemm(spec_handle* h, const char* cls, int32_t rows, int32_t iters, void* stream,
                              double* ms_out, double* bytes_out) {
  if (!h || !cls || !ms_out || !bytes_out || iters < 1) return SPEC_ERR_INVALID_ARG;
  const spec_config& c = h->cfg;
  if (rows < 1 || rows > c.max_batch * c.max_rows_per_seq) return SPEC_ERR_CAPACITY;
  int k;
  if (!std::strcmp(cls, "gemm_o")) k = K_O;
  else if (!std::strcmp(cls, "gemm_gate_up")) k = K_GU;
  else if (!std::strcmp(cls, "gemm_down")) k = K_DOWN;
  else return SPEC_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  const Layout& L = h->lay;
  const int d = c.d_model, F = c.d_ffn, HD = c.n_heads * c.head_dim;
  const size_t wb = c.weight_dtype == SPEC_DTYPE_BF16 ? 2 : 4;
  float* x = h->at<float>(L.x);
  float* at = h->at<float>(L.attn);
  float* act = h->at<float>(L.act);
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return SPEC_ERR_DEVICE;
  if (hipEventCreate(&b) != hipSuccess) {
    hipEventDestroy(a);
    return SPEC_ERR_DEVICE;
  }
  const bool prof = h->prof;
  h->prof = false;  // one event pair around the whole sequence, none per launch
  spec_status st = SPEC_OK;
  double bytes = 0;
  if (hipEventRecord(a, s) != hipSuccess) st = SPEC_ERR_DEVICE;
  for (int it = 0; it < iters && st == SPEC_OK; ++it) {
    for (int l = 0; l < c.n_layers && st == SPEC_OK; ++l) {
      GemmParams g{};
      g.wdtype = c.weight_dtype;
      if (k == K_O) {
        g.W = h->W(h->layer_w(l, 2)); g.X = at; g.ldx = HD; g.N = d; g.K = HD;
        g.epi = EPI_RESID; g.out = x; g.ldo = d;
        bytes += (double)d * HD * wb + (double)rows * (HD + 2.0 * d) * 4;
      } else if (k == K_GU) {
        g.W = h->W(h->layer_w(l, 4)); g.X = x; g.ldx = d; g.N = 2 * F; g.K = d;
        g.norm_g = (const float*)h->W(h->layer_w(l, 3)); g.eps = c.rms_eps;
        g.epi = EPI_SWIGLU; g.out = act; g.ldo = F; g.F = F;
        bytes += 2.0 * F * d * wb + (double)rows * (d + F) * 4;
      } else {
        g.W = h->W(h->layer_w(l, 5)); g.X = act; g.ldx = F; g.N = d; g.K = F;
        g.epi = EPI_RESID; g.out = x; g.ldo = d;
        bytes += (double)d * F * wb + (double)rows * (F + 2.0 * d) * 4;
      }
      if (gemm_rows(h, k, g, rows, s) != hipSuccess) st = SPEC_ERR_DEVICE;
    }
  }
  if (st == SPEC_OK && hipEventRecord(b, s) != hipSuccess) st = SPEC_ERR_DEVICE;
  float ms = 0.f;
  if (st == SPEC_OK && (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&ms, a, b) != hipSuccess))
    st = SPEC_ERR_DEVICE;
  h->prof = prof;
  hipEventDestroy(a);
  hipEventDestroy(b);
  if (st != SPEC_OK) return st;
  *ms_out = ms;
  *bytes_out = bytes;
  return SPEC_OK;
}

void spec_verify_destroy(spec_handle* h) {
  if (!h) return;
  for (auto& r : h->recs) {
    hipEventDestroy(r.a);
    hipEventDestroy(r.b);
  }
  for (auto e : h->pool) hipEventDestroy(e);
  retire_all(h);
  sweep_retired(h, true);  // a replay may still be running
  if (h->cap) hipStreamDestroy(h->cap);
  delete h;
}

spec_status spec_set_block_table(spec_handle* h, const int32_t* d_table, int32_t pages_per_seq) {
  if (!h || !d_table || pages_per_seq < 1) return SPEC_ERR_INVALID_ARG;
  if (!h->cfg.kv_page_size) return SPEC_ERR_STATE;
  if (h->kv_table != d_table || h->kv_ppseq != pages_per_seq) {
    // the recorded launch sequences hold the old table: drop them (each is
    // destroyed once its last replay has finished)
    retire_all(h);
    sweep_retired(h, false);
  }
  h->kv_table = d_table;
  h->kv_ppseq = pages_per_seq;
  return SPEC_OK;
}

spec_status spec_graph_enable(spec_handle* h, int32_t enable) {
  if (!h) return SPEC_ERR_INVALID_ARG;
  h->graphs = enable != 0;
  return SPEC_OK;
}

spec_status spec_gemm_route(int32_t route) {
  if (route < 0 || route > 3) return SPEC_ERR_INVALID_ARG;
  sv::gemm_route = route;
  return SPEC_OK;
}

}  // extern "C"
