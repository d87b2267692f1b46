/*
 * spec_verify.h -- C ABI of the MI355X speculative verify step.
 *
 * One call of spec_verify_step runs the target model's forward over B
 * sequences x T verify rows, streaming every weight matrix from HBM once for
 * all B*T rows; spec_accept then applies speculative sampling to the logits
 * and commits the accepted prefix to the KV cache.
 *
 * What the calls compute, and where it is defined:
 *   - the verify forward yields p_1 .. p_{gamma+1} in one target pass
 *     (CS349E Lecture 6 "Optimizing Autoregressive Decode", section 6.2,
 *     Leviathan et al.'s Algorithm 1, step 2);
 *   - accept / residual resample / bonus: the same section, steps 3-5, with
 *     the test u * q(x) < p(x) (Kimi-K3 tuning page, "What SGLang actually
 *     runs"); greedy acceptance as argmax match (section 7.4);
 *   - tree verification with an ancestor-only mask (section 10.3);
 *   - the cache commit under the pending-token invariant (section 6.2, KV
 *     handling): after a round the cache holds the confirmed sequence minus its
 *     last token;
 *   - acceptance is per sequence and accept counts differ between sequences
 *     (section 11; the Kimi-K3 tuning page on accept length vs batch).
 *
 * Conventions for every call:
 *   - d_* arguments are device pointers (HIP device memory of the GPU current
 *     when the handle was created); everything else lives on the host.
 *   - `stream` is a hipStream_t passed as void*.  Work is enqueued on it
 *     asynchronously; outputs are valid once the stream has synchronised.
 *     No call synchronises the host except spec_verify_init (its one table
 *     upload), spec_device_errors, spec_profile_read, spec_profile_gemm and
 *     spec_verify_destroy.
 *   - The caller owns every buffer (weights, KV cache, workspace, inputs,
 *     outputs).  The handle only borrows them; they must outlive it.  The
 *     library's kernels use only these buffers: it never calls hipMalloc or
 *     hipFree.  Recording a new shape's launch sequence as a HIP graph (the
 *     first step of each shape, see spec_verify_step) is the one place where
 *     the HIP runtime itself may set up internal state; spec_graph_enable(h,
 *     0) switches recording off.
 *   - Host-detectable errors return a negative spec_status before anything is
 *     enqueued.  Data errors visible only on the device (token id outside
 *     [0, V), bad tree parent, cache overflow) set bits in a sticky flag word
 *     read by spec_device_errors; the kernels clamp or skip the offending
 *     access instead of faulting.  Nothing aborts or throws across the ABI.
 *   - A handle is not thread-safe; calls on one handle must be serialised.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t spec_status;
#define SPEC_OK 0
#define SPEC_ERR_INVALID_ARG (-1) /* null pointer, bad enum, bad temperature   */
#define SPEC_ERR_SHAPE (-2)       /* model shape this build does not support   */
#define SPEC_ERR_CAPACITY (-3)    /* B, T or a buffer beyond what init sized   */
#define SPEC_ERR_UNSUPPORTED (-4) /* dtype or device architecture              */
#define SPEC_ERR_DEVICE (-5)      /* a HIP runtime call failed                 */
#define SPEC_ERR_STATE (-6)       /* handle misuse                             */
#define SPEC_ERR_DATA (-7)        /* device-side data error flagged            */

#define SPEC_DTYPE_F32 0
#define SPEC_DTYPE_BF16 1

/* Device-side error flag bits (spec_device_errors). */
#define SPEC_FLAG_TOKEN_RANGE 1u  /* a token id outside [0, vocab)              */
#define SPEC_FLAG_TREE 2u         /* parent[0] != -1 or parent[i] not in [0,i)   */
#define SPEC_FLAG_KV_OVERFLOW 4u  /* kv_len < 0 or kv_len + T > max_ctx          */
#define SPEC_FLAG_LAYOUT 8u       /* ragged row offsets not increasing from 0,
                                     a length outside [1, max_len], or rows
                                     past the padded row count              */

/* Model shape and capacities, fixed at init.
 *   Llama-style decoder: RMSNorm, rotary embedding (rotate-half, theta),
 *   grouped-query attention (n_heads % n_kv_heads == 0), SiLU-gated FFN,
 *   untied LM head, no biases.
 *   weight_dtype: SPEC_DTYPE_BF16 or SPEC_DTYPE_F32 for every matrix (the
 *   embedding and LM head included); norm gains are always fp32.
 *   max_batch, max_ctx, max_rows_per_seq bound B, the cache length and T.
 *   Supported: head_dim 64 or 128; d_model, d_ffn multiples of 64;
 *   max_rows_per_seq <= 128; max_ctx a multiple of 64 (the cache is laid out
 *   with this stride). */
typedef struct spec_config {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab;
  float rms_eps, rope_theta;
  int32_t weight_dtype;
  int32_t max_batch, max_ctx, max_rows_per_seq;
  /* KV cache layout.  kv_page_size 0: dense, per layer K [max_batch][Hkv]
   * [max_ctx][D] and V [max_batch][Hkv][max_ctx / 64][D][64] (values
   * transposed within blocks of 64 slots: the layout of a page, so a block's
   * values are one contiguous run).  kv_page_size 64: paged
   * (PagedAttention, CS349E Lecture 6's reading list; the page size of the
   * ninfer sweep page), a pool of kv_pages pages shared by all sequences,
   * per layer K [kv_pages][Hkv][64][D] and V [kv_pages][Hkv][D][64]; each
   * sequence's slots are mapped to pages by the block table given to
   * spec_set_block_table. */
  int32_t kv_page_size, kv_pages;
} spec_config;

/* Sampling for one accept call.
 *   temperature > 0: p = softmax(z / temperature), speculative sampling.
 *   temperature == 0: greedy (argmax match, argmax extra token).
 *   seed, round: the Philox4x64-10 key is (seed, 0) and the counter is
 *   (slot, sequence, round, 0); u = (word0 >> 40) * 2^-24.
 *   tree_replacement: 0 if each node's children were drawn from its draft
 *   distribution without replacement (the rejected token is removed from q'
 *   and q' renormalised), 1 if drawn with replacement (q' unchanged).
 *   top_k, top_p: the target is sampled from the adjusted distribution of
 *   CS349E Lecture 6, section 7.3: softmax(z / temperature) restricted to
 *   the top_k most likely tokens and renormalised, then restricted to the
 *   nucleus (the shortest run of most likely tokens whose renormalised mass
 *   reaches top_p) and renormalised.  Most likely = larger logit first,
 *   equal logits by lower token id.  top_k = 0 (or >= vocab) and top_p = 1
 *   switch them off; greedy ignores both.  The output then follows the
 *   adjusted target for any q; q should be the draft's distribution after
 *   the same adjustment, or acceptance drops (same section). */
typedef struct spec_sampling {
  float temperature;
  uint32_t tree_replacement;
  uint64_t seed;
  uint64_t round;
  int32_t top_k;
  float top_p;
} spec_sampling;

typedef struct spec_handle spec_handle;

/* Bytes of device workspace spec_verify_init needs (scratch activations,
 * attention partials, accept partials, rotary tables, flag word).
 * Returns 0 for an invalid config. */
size_t spec_workspace_bytes(const spec_config* cfg);

/* Bytes of the bf16 KV cache: [L][2][max_batch][Hkv][max_ctx * D].
 * The K half stores each head's keys as [max_ctx][D] (row per position,
 * keys already rotated); the V half stores each head's values transposed
 * within blocks of 64 positions, [max_ctx / 64][D][64].  Returns 0 for an
 * invalid config. */
size_t spec_kv_cache_bytes(const spec_config* cfg);

/* Create a handle.
 *   d_weights: n_weights = 1 + 6 * n_layers + 2 device pointers, row-major
 *     [out, in]: embed [V, d]; per layer attn_norm [d], w_qkv [(Hq+2Hkv)D, d]
 *     (q rows, then k rows, then v rows), w_o [d, Hq D], ffn_norm [d],
 *     w_gate_up [2F, d] (gate rows, then up rows), w_down [d, F];
 *     final_norm [d], lm_head [V, d].  Pointers must be 16-byte aligned.
 *   d_kv_cache: spec_kv_cache_bytes(cfg) bytes.
 *   d_workspace: workspace_bytes >= spec_workspace_bytes(cfg), 256-byte aligned.
 *   The rotary tables are computed on the host in double precision and copied
 *   into the workspace on `stream` (the only host-to-device copy); init waits
 *   for that copy before returning.
 *   Errors: INVALID_ARG (null), SHAPE, CAPACITY (workspace too small),
 *   UNSUPPORTED (device is not gfx950), DEVICE. */
spec_status spec_verify_init(const spec_config* cfg, const void* const* d_weights, size_t n_weights,
                             void* d_kv_cache, void* d_workspace, size_t workspace_bytes,
                             void* stream, spec_handle** out);

/* The verify forward: logits for B sequences x T rows in one pass.
 *   d_tokens [B, T] int32: row 0 is the sequence's pending token (the last
 *     confirmed token, not yet cached), rows 1.. its drafts; for a tree, node
 *     ids in an order where every parent precedes its children.
 *   d_kv_len [B] int32: committed cache length of each sequence.
 *   d_tree_parent: NULL for chain verify (row i sees cached rows and rows
 *     0..i, at position kv_len + i); else [B, T] int32 parent ids, root -1
 *     (node i sees cached rows, itself and its ancestors, at position
 *     kv_len + depth(i)).
 *   d_logits [B, T, vocab] fp32 output.
 *   Side effect: every row's K/V (rounded to bf16) is written to cache slot
 *   kv_len[b] + i.  Slots beyond the length spec_accept commits are left as
 *   they are (a position-indexed cache abandons a rejected tail for free).
 *   Launches: a prep kernel, the per-layer kernels, the LM head.  The
 *   per-layer kernels read only weights, cache and workspace, so for each
 *   (B, T, chain or tree) their launch sequence is recorded as a HIP graph on
 *   a private stream of the handle (recording runs nothing) on the first step
 *   of a shape and replayed on `stream` from then on (at most 32 shapes are
 *   kept; the least recently used is dropped, and destroyed once its last
 *   replay has finished, without waiting for it).  When `stream` is itself
 *   being captured by the caller, or graphs are switched off with
 *   spec_graph_enable, the kernels are launched directly.  Every projection
 *   runs in this library's kernels, whatever the row count.
 *   Errors: INVALID_ARG, CAPACITY (B > max_batch, T > max_rows_per_seq,
 *   T < 1), STATE (a paged cache without a block table), DEVICE.
 *   Flags: TOKEN_RANGE, TREE, KV_OVERFLOW, LAYOUT (a paged table entry
 *   outside the pool). */
spec_status spec_verify_step(spec_handle* h, int32_t B, int32_t T, const int32_t* d_tokens,
                             const int32_t* d_kv_len, const int32_t* d_tree_parent,
                             float* d_logits, void* stream);

/* Block table of a paged cache (kv_page_size 64): d_table [max_batch]
 * [pages_per_seq] int32 device, row b listing the pool pages of sequence b's
 * slots 0..63, 64..127, ...  The library keeps the pointer and reads the
 * entries on the device at every later step and accept, so the caller edits
 * them in place between steps (stream-ordered): appending a page as a
 * sequence grows, and on rollback shrinking kv_len and returning the pages
 * past the new length to its pool (CS349E Lecture 6, section 6.2 and its
 * list of serving concerns: a paged rollback edits the table's length and
 * frees the surplus blocks).  A sequence's capacity is min(max_ctx,
 * 64 * pages_per_seq).  Entries outside [0, kv_pages) for slots in use set
 * SPEC_FLAG_LAYOUT and are clamped.
 *   Errors: INVALID_ARG (null handle or table, pages_per_seq < 1),
 *   STATE (the cache is dense). */
spec_status spec_set_block_table(spec_handle* h, const int32_t* d_table, int32_t pages_per_seq);

/* Ragged (compact) verify forward: the DeepSeek-V4 analysis page, section 4
 * (static, cap-accept and compact modes; the RaggedVerifyLayout of
 * per-request verify lengths, their sum, and the graph tier it is padded to).
 * Sequence b verifies its own chain of len_b = cu[b+1] - cu[b] rows,
 * 1 <= len_b <= max_len, packed back to back: rows cu[b] .. cu[b+1] - 1 of
 * d_tokens / d_logits, row i at position and cache slot kv_len[b] + i.  Rows
 * cu[B] .. rows - 1 are padding up to the caller's execution tier: they are
 * computed (their logits are meaningless) but write no cache slot.  Only the
 * packed rows are read from the weights' point of view: the GEMMs run on
 * `rows` rows instead of B * max_len.
 *   d_cu_rows [B+1] int32 device, cu[0] = 0, increasing, cu[B] <= rows.
 *   d_tokens [rows] int32 (row cu[b] is sequence b's pending token).
 *   d_kv_len [B]; d_logits [rows, vocab] fp32 output.
 *   rows <= max_batch * max_rows_per_seq; max_len <= max_rows_per_seq.
 *   Recorded launch sequences are kept per (B, max_len, rows), so a caller
 *   that pads `rows` to a few tiers reuses them.
 *   Errors: INVALID_ARG, CAPACITY, DEVICE.  Flags: TOKEN_RANGE, KV_OVERFLOW,
 *   LAYOUT (offsets not increasing from 0, a length outside [1, max_len] or
 *   rows past `rows`; values are clamped, nothing faults). */
spec_status spec_verify_step_ragged(spec_handle* h, int32_t B, int32_t max_len, int32_t rows,
                                    const int32_t* d_cu_rows, const int32_t* d_tokens,
                                    const int32_t* d_kv_len, float* d_logits, void* stream);

/* Speculative-sampling accept and cache commit.
 *   d_logits [B, T, vocab] fp32 from spec_verify_step.
 *   d_q: draft probabilities, fp32, rows summing to 1.  Chain: [B, T-1, vocab],
 *     row j = the distribution draft j+1 was sampled from.  Tree: [B, T, vocab],
 *     row v = the distribution node v's children were drawn from (rows of
 *     leaves are not read).  May be NULL when temperature == 0 or for a chain
 *     with T == 1 (no drafts).
 *   d_tokens [B, T]: the same tokens given to spec_verify_step.
 *   d_tree_parent: NULL (chain) or the same parent array.
 *   d_out_tokens [B, T] int32 output: the n accepted draft tokens followed by
 *     the resampled / bonus token, then -1 padding.
 *   d_num_accepted [B] int32 output: n (accepted drafts, bonus excluded).
 *   d_kv_len [B] input lengths; d_kv_len_out [B] output lengths
 *     kv_len + n + 1 (may alias d_kv_len).  With a tree, the accepted path's
 *     K/V are also copied to slots kv_len + 0 .. n.  Pass d_kv_len_out = NULL
 *     to skip the commit.
 *   Errors: INVALID_ARG (null where required, temperature < 0 or not finite,
 *   top_k < 0, top_p outside [0, 1]), CAPACITY, DEVICE.
 *   Flags: TOKEN_RANGE (a draft token outside [0, V)),
 *   TREE. */
spec_status spec_accept(spec_handle* h, int32_t B, int32_t T, const float* d_logits,
                        const float* d_q, const int32_t* d_tokens, const int32_t* d_tree_parent,
                        const spec_sampling* sampling, int32_t* d_out_tokens,
                        int32_t* d_num_accepted, const int32_t* d_kv_len, int32_t* d_kv_len_out,
                        void* stream);

/* Accept of ragged chains (same section): sequence b has len_b rows starting
 * at logits / token row row_start[b] (its pending token and len_b - 1
 * drafts), and its drafts' distributions at q rows q_start[b] .. q_start[b] +
 * len_b - 2.  At most len_b - 1 drafts are accepted, the extra token comes
 * from row n, the commit is kv_len + n + 1; the uniforms use slots 0 ..
 * len_b - 1 as a chain of gamma = len_b - 1 does.
 *   Compact mode: row_start = cu[b], q_start = cu[b] - b for q packed without
 *   each sequence's last row, logits from spec_verify_step_ragged.
 *   Cap-accept mode: logits from spec_verify_step at T = max_len, row_start =
 *   b * T, q_start = b * (T - 1), len_b the cap.
 *   rows / q_rows: rows in d_logits and d_tokens / in d_q.
 *   d_out_tokens [B, max_len] (n accepted drafts, the extra token, -1
 *   padding); d_num_accepted [B]; kv_len / kv_len_out as for spec_accept.
 *   d_q and d_q_start may be NULL when temperature == 0 or max_len == 1.
 *   sampling as for spec_accept (tree_replacement unused).
 *   Errors: INVALID_ARG, CAPACITY, DEVICE.  Flags: TOKEN_RANGE, LAYOUT. */
spec_status spec_accept_ragged(spec_handle* h, int32_t B, int32_t max_len, int32_t rows, int32_t q_rows,
                               const int32_t* d_row_start, const int32_t* d_len, const int32_t* d_q_start,
                               const float* d_logits, const float* d_q, const int32_t* d_tokens,
                               const spec_sampling* sampling, int32_t* d_out_tokens,
                               int32_t* d_num_accepted, const int32_t* d_kv_len, int32_t* d_kv_len_out,
                               void* stream);

/* Synchronise `stream`, return the sticky device flag word (SPEC_FLAG_*) in
 * *flags and clear it.  Returns SPEC_OK, or DEVICE if a HIP call failed. */
spec_status spec_device_errors(spec_handle* h, uint32_t* flags, void* stream);

/* Per-kernel timing with HIP events on the launch stream, for measurement.
 * When enabled, every launch of each kernel class is bracketed by events;
 * spec_profile_read synchronises and reports, per class, the launch count,
 * total milliseconds and the algorithmic bytes those launches had to move
 * (weights and activations for the GEMMs, logits and q for accept; each
 * counted once).  Class names: "prep_embed", "gemm_qkv", "attention",
 * "attn_combine", "gemm_o", "gemm_gate_up", "gemm_down", "gemm_lm_head",
 * "accept".  Attention's bytes depend on the device-side kv_len and are
 * reported as 0. */
typedef struct spec_kernel_stat {
  char name[24];
  int64_t launches;
  double total_ms;
  double algo_bytes;
} spec_kernel_stat;
spec_status spec_profile_enable(spec_handle* h, int32_t enable);
int32_t spec_profile_read(spec_handle* h, spec_kernel_stat* out, int32_t max_out, int32_t reset);

/* Back-to-back timing of one GEMM class, for measurement: the class's GEMM
 * of every layer is launched in layer order, `iters` times over, on `stream`
 * with `rows` activation rows, between one pair of HIP events; no event sits
 * between the launches.  Returns the elapsed milliseconds and the algorithmic
 * bytes of all those launches (each weight matrix once per launch, plus the
 * activation rows read and written).  cls: "gemm_o", "gemm_gate_up" or
 * "gemm_down".  The launches read and overwrite the workspace's activation
 * buffers and touch neither the KV cache nor caller memory; call it between
 * verify steps, never while one is in flight on another stream.
 * Errors: SPEC_ERR_INVALID_ARG (null pointer, unknown class, iters < 1),
 * SPEC_ERR_CAPACITY (rows outside [1, max_batch * max_rows_per_seq]),
 * SPEC_ERR_DEVICE (a HIP call failed). */
spec_status spec_profile_gemm(spec_handle* h, const char* cls, int32_t rows, int32_t iters, void* stream,
                              double* ms_out, double* bytes_out);

/* Measurement hook, not part of the verify path: the average launch-to-end
 * time in microseconds of a plain streaming read of `read_bytes`, launched
 * `iters` times back to back on `stream` between one pair of HIP events
 * (after 3 untimed launches).  The read is a grid-stride loop of `grid`
 * workgroups of 256 threads with `unroll` (4 or 8) 16-byte non-temporal
 * loads in flight per thread.  Each launch reads the window after the
 * previous one inside d_buf (wrapping), so that consecutive launches do not
 * hit the memory-side cache; the buffer's last 16 bytes are a sink the
 * kernel may write.  It is the practical ceiling of a weight-streaming GEMM
 * over that many weight bytes, launch, ramp and tail included.  Synchronises
 * the host (it waits for the end event).
 * d_buf: device memory, 4096-byte aligned, buf_bytes a multiple of 16 and at
 * least read_bytes + 8192; read_bytes a multiple of 16.
 * Errors: SPEC_ERR_INVALID_ARG (null pointer, sizes or alignment as above,
 * iters or grid < 1, unroll not 4 or 8), SPEC_ERR_DEVICE (a HIP call failed). */
spec_status spec_profile_stream_read(const void* d_buf, size_t buf_bytes, size_t read_bytes, int32_t iters,
                                     int32_t grid, int32_t unroll, void* stream, double* us_out);

/* Replay the recorded per-layer launch sequence (enable != 0, the default)
 * or launch every kernel directly (enable == 0).  Both run the same kernels
 * with the same arguments, so the results are identical; replay saves the
 * per-launch dispatch overhead of ~190 kernels per step.
 * Errors: INVALID_ARG (null handle). */
spec_status spec_graph_enable(spec_handle* h, int32_t enable);

/* Chain accept that allocates nothing and needs no handle, for callers that
 * cannot allocate device memory or create a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  It computes
 * what spec_accept computes for a chain (T = gamma + 1 rows per sequence,
 * d_tree_parent == NULL) with the same kernels, so for the same inputs the
 * outputs are identical bit for bit; top-k / top-p adjustment is not offered
 * here (SPEC_ERR_UNSUPPORTED).
 *   vocab: V of the logits and q rows; the other arguments as in spec_accept.
 *   d_flags: optional device word that receives the TOKEN_RANGE flag bit
 *     (ORed in; the caller clears it); NULL discards the flags.
 *   Scratch: the kernels' row statistics, residual chunk sums and accept
 *     counts live in a fixed array inside the library (about 2.3 MiB per GPU,
 *     held until the process ends): at most SPEC_STATIC_MAX_ROWS logits rows
 *     (B * T), SPEC_STATIC_MAX_SEQS sequences and a vocabulary of
 *     SPEC_STATIC_MAX_VOCAB.  Every scratch entry a call reads is written
 *     earlier in that call.  All calls on one GPU share the array: calls that
 *     overlap on one GPU (two streams, two threads) race; serialise them.
 *   No hipMalloc, hipFree or allocating library call is made; the first call
 *   on each device looks up the array's device address once.
 *   Errors: INVALID_ARG (null pointer, B < 1, T < 1, vocab < 2, bad sampling,
 *   q missing for a sampled chain), CAPACITY (beyond the limits above, or
 *   T > 128), UNSUPPORTED (top-k / top-p set), DEVICE. */
#define SPEC_STATIC_MAX_ROWS 4096
#define SPEC_STATIC_MAX_SEQS 1024
#define SPEC_STATIC_MAX_VOCAB 262144
spec_status spec_accept_chain_static(int32_t B, int32_t T, int32_t vocab, const float* d_logits, const float* d_q,
                                     const int32_t* d_tokens, const spec_sampling* sampling, int32_t* d_out_tokens,
                                     int32_t* d_num_accepted, const int32_t* d_kv_len, int32_t* d_kv_len_out,
                                     uint32_t* d_flags, void* stream);

/* Measurement hook: the GEMM kernels a launch of 9 or more rows uses, for
 * A/B timing and for parity tests of every path.  route 0: automatic
 * (128-row x 256-weight-row tiles from 64 rows on, 32-row tiles for 9-63;
 * up to 8 rows the weight-streaming kernels); 1: the 32-row tiles at every
 * row count the tiled kernels serve; 2: the large tiles there; 3: automatic,
 * with the large tiles in their 4-wave form (one wave per SIMD).
 * Process-wide; results are within the same fp32 tolerance either way (the
 * sums are taken in a different order).  Takes effect for launch sequences
 * recorded afterwards (switch graphs off, or use a new handle, to apply it
 * to shapes already recorded).
 * Errors: INVALID_ARG (route outside 0..3). */
spec_status spec_gemm_route(int32_t route);

/* Release the handle: host memory, events, recorded graphs and the private
 * recording stream (waits for recorded replays still running). */
void spec_verify_destroy(spec_handle* h);

/* Static string for a status code. */
const char* spec_status_str(spec_status s);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_VERIFY_H */
