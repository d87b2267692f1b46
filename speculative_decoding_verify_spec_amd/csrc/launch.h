// Internal interface between the runtime (runtime.hip) and the kernel files.
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace sv {

// ---------------------------------------------------------------- prep + embedding
struct PrepParams {
  const int32_t* tokens;  // [B, T]
  const int32_t* kv_len;  // [B]
  const int32_t* parent;  // [B, T] or null (chain)
  int32_t* tok;           // [M] clamped token ids
  int32_t* pos;           // [M] rotary position
  int32_t* slot;          // [M] cache slot, -1 when it would overflow
  uint64_t* anc;          // [M][2] ancestor-or-self bitmask (tree only)
  uint32_t* flags;
  const void* embed;      // [V][d] embedding table (weight dtype)
  int wdtype;             // 0 fp32, 1 bf16
  float* x;               // [M][d] residual stream, written with the rows' embeddings
  int32_t* kv_copy;       // [B] copy of kv_len for the later kernels of the step
  int B, T, vocab, max_ctx, d;
  // ragged (packed) rows: cu [B+1] row offsets of the sequences in the
  // caller's token array (null: B x T rows); rows = padded row count; the
  // kernel writes each sequence's first row and length and each row's
  // sequence for the later kernels
  const int32_t* cu;
  int rows;
  int32_t* rstart;        // [B]
  int32_t* rlen;          // [B]
  int32_t* seq;           // [rows]
  KvMap kvm;              // cache addressing; paged: the table is checked here
};
hipError_t launch_prep(const PrepParams& p, hipStream_t s);

// ---------------------------------------------------------------- GEMM
enum { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_QKV = 3 };

struct GemmParams {
  const void* W;  // [N][K], bf16 or fp32
  int wdtype;     // 0 fp32, 1 bf16
  const float* X; // [M][ldx] fp32
  int ldx;
  int M, N, K;    // N = output rows of W used by the epilogue mapping
  int epi;
  float* out;     // STORE / RESID / SWIGLU: [M][ldo]
  int ldo;
  int F;          // SWIGLU: gate rows [0,F), up rows [F,2F)
  const float* norm_g;  // non-null: RMSNorm the activation rows (gain g, eps) first
  float eps;
  // QKV epilogue
  int m0;                   // global row offset of this launch (row chunking)
  const int32_t* pos;       // [M_total]
  const int32_t* slot;      // [M_total]
  const float* rope_cos;    // [max_ctx][D/2]
  const float* rope_sin;
  float* q_out;             // [M_total][Hq][D]
  float* k_out;             // [M_total][Hkv][D]
  float* v_out;
  uint16_t* kcache;         // this layer's K region [maxB][Hkv][max_ctx][D]
  uint16_t* vcache;         // this layer's V region [maxB][Hkv][D][max_ctx]
  int T, Hq, Hkv, D, max_ctx;
  // split-K scratch for partial sums, or null (then no launch splits K)
  float* part;
  size_t part_floats;
  // tiled kernel: bf16 hi/lo planes of the activations ([2][M][K], xs_elems
  // elements available) and their rows' sums of squares [M]
  uint16_t* xs;
  size_t xs_elems;
  float* xs_ssq;          // [M][SSQ_BLK] partial sums of squares per 1024 k
  // QKV epilogue, ragged rows: sequence of each global row (null: row / T)
  const int32_t* seq;
  KvMap kvm;                // cache addressing of the QKV epilogue's writes
  // Activation rows still owed the K-slice partial sums of a split residual
  // GEMM whose reduce was deferred: with xpart set, row m is taken as
  // X[m][k] + (xpart[(0*8+m)*ldx+k] + ... + xpart[(3*8+m)*ldx+k]), the slices
  // summed in order and the sum added to X as the reduce kernel does, and
  // the launch's first workgroup stores the completed rows to xout ([M][ldx],
  // not X).  Only the k-stationary kernel takes it (gemm_takes_xpart).
  const float* xpart;
  float* xout;
  // split residual GEMM: leave the partial sums in `part` for the next
  // GEMM's prologue instead of launching the reduce
  bool defer_reduce;
  // Activation planes written by the producer: with xs_ready the launch's
  // planes in `xs` are already there (written by the kernel that produced X,
  // with the split's arithmetic) and the tiled launch skips its split; only
  // without a fused norm.  With xs_out a SiLU*up epilogue also writes the
  // bf16 hi/lo planes [2][M][ldo] of its outputs, for the next GEMM.
  bool xs_ready;
  uint16_t* xs_out;
  // ... and xs_ssq holds those rows' sums of squares, so that a launch with a
  // fused norm may skip its split too
  bool ssq_ready;
  // A K-split residual GEMM on the tiled kernels whose finish also prepares
  // the next GEMM's activations: with norm_next set, the finish (one
  // workgroup per 1024 output columns of a row) writes the bf16 hi/lo planes
  // of out * norm_next into xs_next ([2][M][N]) and the rows' sums of squares
  // per 1024 columns into xs_ssq, as the split of the next launch would.
  // Only where gemm_finish_prepares holds.
  const float* norm_next;
  uint16_t* xs_next;
};
constexpr int GEMM_KSPLIT = 2;  // K slices of the skinny residual GEMM
constexpr int SSQ_BLK = 16;     // 1024-k partial sums of squares per activation row (K <= 16384)

// RMSNorm factor of activation row m from the activation split's partial
// sums of squares (added in a fixed order)
__device__ __forceinline__ float row_factor(const GemmParams& p, int m) {
  const int nblk = (p.K + 1023) / 1024;
  float q = 0.f;
  for (int b = 0; b < nblk; ++b) q += p.xs_ssq[m * SSQ_BLK + b];
  return 1.0f / sqrtf(q / (float)p.K + p.eps);
}
hipError_t launch_gemm(const GemmParams& p, hipStream_t s);
// the launch of these parameters (M rows) runs on the tiled kernels as K
// slices whose finish is a separate kernel: the residual GEMMs where
// norm_next can take the next launch's split
bool gemm_finish_prepares(const GemmParams& p);
// the residual GEMM of these parameters runs as K slices + reduce
bool gemm_use_split(const GemmParams& p);
// the launch of these parameters can complete its activation rows from
// deferred partial sums (xpart / xout)
bool gemm_takes_xpart(const GemmParams& p);
// the tiled kernels for M > 8 (bf16 weights, K a multiple of 64)
bool gemm_tiled_ok(const GemmParams& p);
hipError_t launch_gemm_tiled(const GemmParams& p, hipStream_t s);
// the large-tile kernel serves this launch (64 or more rows, or the override)
bool gemm_big_rows(const GemmParams& p);
// measurement override of the tile choice: 0 automatic, 1 the 32-row tiles,
// 2 the large tiles, 3 the large tiles' 4-wave form (set through
// spec_gemm_route)
extern int gemm_route;
// the activation planes of the tiled kernels ([2][M][K] in p.xs, row sums of
// squares in p.xs_ssq)
hipError_t launch_split_x(const GemmParams& p, hipStream_t s);
// compute units of the current device
int device_cus();
// split-K scratch (floats) the large-tile kernel asks for at M rows of
// npairs output pairs over K, on a device of `cus` CUs (0: no split)
size_t gemm_big_part_floats(int M, size_t npairs, int K, int cus);

// ---------------------------------------------------------------- attention
struct AttnParams {
  const float* q;          // [M][Hq][D] rotated queries
  const uint16_t* kc;      // layer K region
  const uint16_t* vc;      // layer V region
  const int32_t* kv_len;   // [B]
  const float* k_suf;      // [M][Hkv][D] the step's own keys, fp32
  const float* v_suf;
  const uint64_t* anc;     // [M][2] ancestor-or-self bits, or null for chain
  float* part_o;           // [nsplit][B][Hkv][nq][D]
  float* part_ml;          // [nsplit][B][Hkv][nq][2]
  int B, T, Hq, Hkv, D, max_ctx;
  int splits;              // context workgroups per (sequence, kv head, query group)
  float scale;
  // ragged rows: first row and length of each sequence (null: b * T, T;
  // T is then the longest length)
  const int32_t* rstart;
  const int32_t* rlen;
  KvMap kvm;               // cache addressing
};
// number of partial slots per query the attention kernel writes: the context
// splits plus one for the step's own (suffix) keys
int attn_nsplit(int splits);
int attn_query_tiles(int nq, int D);    // 16-query tiles per wave of the context attention (1 or 2)
int attn_groups_per_wg(int nq, int D);  // query groups sharing a context workgroup's key blocks (1 or 2)
int attn_suffix_cols(bool tree, int pairs, int QT, int QGW);  // suffix workgroups per unit
hipError_t launch_attention(const AttnParams& p, hipStream_t s);

struct CombineParams {
  const float* part_o;
  const float* part_ml;
  int nsplit;
  float* out;              // [M][Hq][D]
  int B, T, Hq, Hkv, D;
  const int32_t* rstart;   // ragged rows, as in AttnParams
  const int32_t* rlen;
  // or null: the bf16 hi/lo planes [2][M][Hq*D] of `out` as the tiled GEMMs'
  // activation split writes them (M = rows of the step)
  uint16_t* xs;
  int M;
};
hipError_t launch_attn_combine(const CombineParams& p, hipStream_t s);

// ---------------------------------------------------------------- accept
// scratch bytes of the sampled token-tree walk for B sequences of nch chunks
size_t tree_walk_bytes(int B, int nch);
constexpr int TPATH = 130;  // ints per sequence of AcceptParams::tpath (T <= 128)
struct AcceptParams {
  const float* logits;     // [B][T][V]
  const float* q;          // chain [B][T-1][V], tree [B][T][V]
  const int32_t* tokens;   // [B][T]
  const int32_t* parent;   // [B][T] or null
  float temperature;
  int replacement;
  uint64_t seed, round;
  int32_t* out_tokens;     // [B][T]
  int32_t* num_accepted;   // [B]
  const int32_t* kv_len;   // [B]
  int32_t* kv_len_out;     // [B] or null
  // scratch
  float* rowstat;          // [B*T][nch][2]
  float* rowms;            // [B*T][2]
  float* rsum;             // [B][nch]
  int32_t* nacc;           // [B]
  void* twalk;             // sampled token-tree walk: tree_walk_bytes(B, nch)
  int32_t* tpath;          // [B][TPATH]: kv_len, path length, accepted tree path (tree commit)
  uint32_t* flags;
  // cache for the tree commit
  uint16_t* kv_cache;
  int L, maxB, Hkv, D, max_ctx;
  int B, T, V, nch;
  // top-k / top-p adjustment of the target (0 and 1 switch them off) and the
  // selection scratch: chunk histograms [2][SEL_ROWS][nch][256], running
  // state [2][SEL_ROWS], and one keep rule per row [B*T] (null in the
  // sampling kernels when no adjustment applies)
  int top_k;
  float top_p;
  uint32_t* fcnt;
  double* fmass;
  struct SelState* fstate;
  struct SelRule* fres;
  // ragged layout (null: sequence b has T rows from row b*T, its drafts' q
  // rows from b*(T-1)): first logits / token row, length, first q row
  const int32_t* rstart;
  const int32_t* rlen;
  const int32_t* qstart;
  int rows;                // logits (and token) rows: B*T when not ragged
  int qrows;               // rows of q
  KvMap kvm;               // cache addressing of the tree commit
};
// Running state of one row's radix selection: the key bits chosen so far,
// the tokens still to take (top-k) or the mass still to reach (top-p; -1
// until the first digit has been counted), and the mass of the tokens
// already known to be above the threshold.
struct SelState {
  uint32_t prefix;
  uint32_t need;
  double rem;
  double above;
};
// A row's kept set: tokens with key > tau, and those with key == tau and id
// <= cut (keys order logits; equal logits go by id).  tau_k / cut_k /
// mass_k: the top-k set and its unnormalised mass.
struct SelRule {
  uint32_t tau;
  int32_t cut;
  uint32_t tau_k;
  int32_t cut_k;
  double mass_k;
};
constexpr int SEL_ROWS = 128;  // rows per selection batch
int accept_chunks(int V);
hipError_t launch_accept(const AcceptParams& p, hipStream_t s);

}  // namespace sv
