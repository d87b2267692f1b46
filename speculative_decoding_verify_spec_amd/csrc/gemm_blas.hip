// Many-row projections through hipBLASLt.
//
// From 64 activation rows on (many sequences' windows, token trees) the
// projections are dense contractions that a library GEMM runs well on the
// matrix cores.  The fp32 activations stay exact to ~2^-16: the activation
// split kernel of the tiled path writes them as bf16 hi and lo planes
// [2][M][K] (times the RMSNorm gain), and the two planes are stacked as the
// 2M rows of ONE plain GEMM against the bf16 weights, so every weight is
// read once: D [2M][Nw] = [Xhi; Xlo] W^T in fp32 (Nw = weight rows).  The
// finish kernel (gemm_tiled.hip) adds each row's hi and lo products, applies
// the RMSNorm row factor and the fused epilogue (SiLU-gated product, rotary
// embedding and cache write, residual add, logits store).
//
// Algorithms are chosen per (Nw, K, 2M) on first use.  When allowed to tune
// (the stream is not being recorded), every candidate the library proposes is
// run twice and dropped unless both runs give bit-identical output (no
// order-dependent reductions), then the fastest over a few timed runs is
// kept.  Otherwise the library's first proposal is used until a tuning call.
#include <hipblaslt/hipblaslt.h>

#include <vector>

#include "common.h"
#include "launch.h"

namespace sv {

struct BlasPlan {
  int nw, k, m2;
  hipblasLtMatmulDesc_t desc;
  hipblasLtMatrixLayout_t la, lb, lc;
  hipblasLtMatmulAlgo_t algo;
  size_t algo_ws;
  bool tuned;
};

struct BlasCtx {
  hipblasLtHandle_t lt = nullptr;
  void* ws = nullptr;  // the library's workspace (borrowed)
  size_t ws_bytes = 0;
  float* d = nullptr;  // fp32 product scratch (borrowed)
  size_t d_floats = 0;
  std::vector<BlasPlan> plans;
};

BlasCtx* blas_create(void* ws, size_t ws_bytes, float* d, size_t d_floats) {
  BlasCtx* c = new BlasCtx();
  c->ws = ws;
  c->ws_bytes = ws_bytes;
  c->d = d;
  c->d_floats = d_floats;
  return c;
}

void blas_destroy(BlasCtx* c) {
  if (!c) return;
  for (auto& p : c->plans) {
    hipblasLtMatrixLayoutDestroy(p.la);
    hipblasLtMatrixLayoutDestroy(p.lb);
    hipblasLtMatrixLayoutDestroy(p.lc);
    hipblasLtMatmulDescDestroy(p.desc);
  }
  if (c->lt) hipblasLtDestroy(c->lt);
  delete c;
}

namespace {

constexpr int kCandidates = 32;

int weight_rows(const GemmParams& p) { return p.epi == EPI_SWIGLU ? 2 * p.F : p.N; }

// rows per launch so that the [2 rows][Nw] product fits the scratch
int chunk_rows(const GemmParams& p, const BlasCtx* c) {
  const size_t per = (size_t)2 * weight_rows(p);
  const size_t r = c->d_floats / per;
  return (int)(r > (size_t)p.M ? p.M : r);
}

// order-independent digest of a buffer's bit patterns
__global__ void blas_digest_kernel(const uint32_t* v, size_t n, unsigned long long* out) {
  unsigned long long s = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    s += (unsigned long long)v[i] * (2 * i + 1);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) atomicAdd(out, s);
}

hipError_t digest(const BlasCtx* c, size_t n, hipStream_t s, unsigned long long* host) {
  // the library workspace is idle between GEMMs: its first word holds the digest
  unsigned long long* dev = (unsigned long long*)c->ws;
  hipError_t e = hipMemsetAsync(dev, 0, sizeof(unsigned long long), s);
  if (e != hipSuccess) return e;
  blas_digest_kernel<<<512, 256, 0, s>>>((const uint32_t*)c->d, n, dev);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(host, dev, sizeof(*host), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

hipError_t run(const BlasCtx* c, const BlasPlan& pl, const hipblasLtMatmulAlgo_t& algo, const void* W,
               const void* X, hipStream_t s) {
  const float alpha = 1.f, beta = 0.f;
  const hipblasStatus_t st = hipblasLtMatmul(c->lt, pl.desc, &alpha, W, pl.la, X, pl.lb, &beta, c->d, pl.lc, c->d,
                                             pl.lc, &algo, c->ws, c->ws_bytes, s);
  return st == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

// Plan for D [m2][nw] = X [m2][k] W [nw][k]^T, row-major.  In the library's
// column-major terms: D^T (nw x m2) = op(W) X^T with W stored k x nw (op = T)
// and X stored k x m2.
BlasPlan* get_plan(BlasCtx* c, int nw, int k, int m2) {
  for (auto& p : c->plans)
    if (p.nw == nw && p.k == k && p.m2 == m2) return &p;
  BlasPlan p{};
  p.nw = nw;
  p.k = k;
  p.m2 = m2;
  if (hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return nullptr;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta));
  hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb));
  if (hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, k, nw, k) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, k, m2, k) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_32F, nw, m2, nw) != HIPBLAS_STATUS_SUCCESS)
    return nullptr;
  hipblasLtMatmulPreference_t pref;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return nullptr;
  const uint64_t wsl = c->ws_bytes;
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsl, sizeof(wsl));
  hipblasLtMatmulHeuristicResult_t res[kCandidates];
  int n = 0;
  const hipblasStatus_t hs =
      hipblasLtMatmulAlgoGetHeuristic(c->lt, p.desc, p.la, p.lb, p.lc, p.lc, pref, kCandidates, res, &n);
  hipblasLtMatmulPreferenceDestroy(pref);
  int first = -1;
  for (int i = 0; hs == HIPBLAS_STATUS_SUCCESS && i < n; ++i)
    if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= c->ws_bytes) {
      first = i;
      break;
    }
  if (first < 0) return nullptr;
  p.algo = res[first].algo;
  p.algo_ws = res[first].workspaceSize;
  p.tuned = false;
  c->plans.push_back(p);
  return &c->plans.back();
}

// Time the library's candidates on the real operands; keep the fastest whose
// two runs agree bit for bit.  Runs only on a stream that is not recording.
hipError_t tune(BlasCtx* c, BlasPlan* pl, const void* W, const void* X, hipStream_t s) {
  hipblasLtMatmulPreference_t pref;
  if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return hipErrorLaunchFailure;
  const uint64_t wsl = c->ws_bytes;
  hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsl, sizeof(wsl));
  hipblasLtMatmulHeuristicResult_t res[kCandidates];
  int n = 0;
  hipblasStatus_t hs =
      hipblasLtMatmulAlgoGetHeuristic(c->lt, pl->desc, pl->la, pl->lb, pl->lc, pl->lc, pref, kCandidates, res, &n);
  hipblasLtMatmulPreferenceDestroy(pref);
  if (hs != HIPBLAS_STATUS_SUCCESS) return hipErrorLaunchFailure;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess) return hipErrorLaunchFailure;
  if (hipEventCreate(&e1) != hipSuccess) {
    hipEventDestroy(e0);
    return hipErrorLaunchFailure;
  }
  const size_t nd = (size_t)pl->m2 * pl->nw;
  float best = 1e30f;
  hipError_t err = hipSuccess;
  for (int i = 0; i < n && err == hipSuccess; ++i) {
    if (res[i].state != HIPBLAS_STATUS_SUCCESS || res[i].workspaceSize > c->ws_bytes) continue;
    unsigned long long h0 = 0, h1 = 1;
    if (run(c, *pl, res[i].algo, W, X, s) != hipSuccess) continue;
    if ((err = digest(c, nd, s, &h0)) != hipSuccess) break;
    if (run(c, *pl, res[i].algo, W, X, s) != hipSuccess) continue;
    if ((err = digest(c, nd, s, &h1)) != hipSuccess) break;
    if (h0 != h1) continue;  // order-dependent: results would vary run to run
    constexpr int reps = 5;
    if ((err = hipEventRecord(e0, s)) != hipSuccess) break;
    for (int r = 0; r < reps; ++r) run(c, *pl, res[i].algo, W, X, s);
    if ((err = hipEventRecord(e1, s)) != hipSuccess) break;
    if ((err = hipEventSynchronize(e1)) != hipSuccess) break;
    float ms = 0.f;
    hipEventElapsedTime(&ms, e0, e1);
    if (ms < best) {
      best = ms;
      pl->algo = res[i].algo;
      pl->algo_ws = res[i].workspaceSize;
    }
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  if (err != hipSuccess) return err;
  if (best >= 1e30f) return hipErrorLaunchFailure;  // no reproducible candidate
  pl->tuned = true;
  return hipSuccess;
}

}  // namespace

bool blas_ready(const BlasCtx* c) { return c && c->lt; }

// From 64 rows on: below that the deterministic candidates are no faster than
// the tiled kernel (measured at 8 and 32 rows), whose epilogue is fused.
bool gemm_blas_ok(const GemmParams& p) {
  if (!p.blas || p.wdtype != 1 || p.M < 64 || (p.K & 7) || p.K > SSQ_BLK * 1024 || !p.xs) return false;
  if ((size_t)2 * p.M * p.K > p.xs_elems) return false;
  return chunk_rows(p, p.blas) >= 64;
}

hipError_t launch_gemm_blas(const GemmParams& pin, hipStream_t s, bool allow_tune) {
  BlasCtx* c = pin.blas;
  if (!c->lt) {
    if (!allow_tune) return hipErrorNotReady;  // the handle is created outside recording
    if (hipblasLtCreate(&c->lt) != HIPBLAS_STATUS_SUCCESS) {
      c->lt = nullptr;
      return hipErrorLaunchFailure;
    }
  }
  const int nw = weight_rows(pin);
  const int rows = chunk_rows(pin, c);
  for (int m0 = 0; m0 < pin.M; m0 += rows) {
    GemmParams p = pin;
    p.M = pin.M - m0 < rows ? pin.M - m0 : rows;
    p.X = pin.X + (size_t)m0 * pin.ldx;
    p.m0 = pin.m0 + m0;
    if (pin.out) p.out = pin.out + (size_t)m0 * pin.ldo;
    hipError_t e = launch_split_x(p, s);
    if (e != hipSuccess) return e;
    BlasPlan* pl = get_plan(c, nw, p.K, 2 * p.M);
    if (!pl) return hipErrorLaunchFailure;
    if (allow_tune && !pl->tuned && (e = tune(c, pl, p.W, p.xs, s)) != hipSuccess) return e;
    if ((e = run(c, *pl, pl->algo, p.W, p.xs, s)) != hipSuccess) return e;
    if ((e = launch_blas_finish(p, c->d, nw, s)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace sv
