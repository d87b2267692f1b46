/*
 * spec_recurrent.h -- C ABI of verify on a recurrent (linear-attention) layer.
 *
 * A recurrent layer carries a per-sequence state that is a value, not a
 * table indexed by position: verifying T = gamma + 1 speculated positions
 * advances it serially through all of them, and the state that survives
 * acceptance (the one after the last committed position) must be
 * recoverable once acceptance has run (Kimi-K3 tuning page, "Verification on
 * a recurrent layer is not a cache write"; the verify recurrence, causal conv
 * and post-verify state scatter are among the hot-path operators listed in
 * "Why it retargets to ROCm without being ported").
 *
 * The layer computed here (the pages name the recurrence but do not write it
 * out; this is the gated delta rule the name refers to), per head h with key
 * and value width D and state S in R^{D x D}, rows = key channels i, columns
 * = value channels j:
 *   raw channels of position t: x~_t = [q~ | k~ | v~], 3*H*D floats
 *   causal depthwise conv:      c_t[ch] = sum_{w<W} conv_w[ch][w] * x~_{t-W+1+w}[ch]
 *                               (positions before the window: the conv state)
 *   activation:                 silu(c) = c / (1 + exp(-c))
 *   normalised q, k per head:   q^ = q / sqrt(|q|^2 + 1e-6) / sqrt(D),
 *                               k^ = k / sqrt(|k|^2 + 1e-6)
 *   decay:                      S <- Diag(exp(gate_t)) S
 *   delta write:                S <- S + beta_t k^ (v - S^T k^)^T
 *   output:                     o_t = S^T q^
 * fp32 throughout.
 *
 * Two ways to recover the survivor, chosen per commit call:
 *   - snapshots: spec_recurrent_verify keeps the state after every window
 *     position (the gamma + 1 candidate states the pages' engines keep
 *     alive) and the commit copies the survivor;
 *   - replay: verify keeps no snapshot; the commit advances the pool state
 *     again through the committed positions from the window inputs, which
 *     the caller keeps until then.  Both run the same per-position
 *     arithmetic in the same order, so the committed states are identical.
 *
 * Conventions: as in spec_verify.h.  d_* are device pointers of the current
 * device, 16-byte aligned; everything is enqueued on `stream` (hipStream_t as
 * void*) with no host synchronisation; the caller owns every buffer.  The
 * calls need no handle and allocate nothing.
 *
 * Layouts (fp32 unless noted; C = 3*H*D channels, q then k then v, head h
 * owning channels h*D .. h*D+D-1 of each third):
 *   x           [B][T][C]        raw channels of the window
 *   gate        [B][T][H][D]     log decay (<= 0 in a trained model)
 *   beta        [B][T][H]        write strength
 *   conv_w      [C][W]           taps, oldest input first
 *   slot        [B] int32        pool row of each sequence; NULL = b.  Rows
 *                                must be distinct within a call.  A row
 *                                outside [0, n_slots) skips the sequence:
 *                                nothing of it is read or written.
 *   conv_state  [n_slots][W-1][C] raw inputs of the W-1 positions before the
 *                                window, oldest first (unused when W = 1)
 *   state       [n_slots][H][D][D]
 *   out         [B][T][H][D]     o_t
 *   snapshots   [B][T][H][D][D]  state after each window position
 */
#ifndef SPEC_RECURRENT_H
#define SPEC_RECURRENT_H

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_recurrent_dims {
  int32_t n_heads;    /* H >= 1                                   */
  int32_t head_dim;   /* D: 64 or 128                             */
  int32_t conv_width; /* W: 1 .. 8                                */
  int32_t n_slots;    /* rows of the state pool, >= 1             */
} spec_recurrent_dims;

/* Advance every sequence's pool state through its T window positions
 * (1 <= T <= 16; B == 0 is a no-op) and write the outputs; with d_snapshots
 * non-NULL also write the state after each position.  Reads the pool
 * (d_conv_state, d_state) without modifying it, so the call can be repeated.
 * Errors: INVALID_ARG (null or misaligned pointer, T or B out of range),
 * SHAPE (dims), DEVICE (launch failed). */
spec_status spec_recurrent_verify(const spec_recurrent_dims* dims, int32_t B, int32_t T, const float* d_x,
                                  const float* d_gate, const float* d_beta, const float* d_conv_w,
                                  const int32_t* d_slot, const float* d_conv_state, const float* d_state,
                                  float* d_out, float* d_snapshots, void* stream);

/* Post-verify state scatter after acceptance.  With n = d_num_accepted[b]
 * clamped into [0, T-1] (the accepted drafts; window positions 0 .. n are
 * committed, as in the chain's cache commit), the sequence's pool row gets
 * the state after window position n and the conv state of the W-1 raw
 * inputs ending at position n.
 *   d_snapshots non-NULL: the snapshots written by spec_recurrent_verify for
 *     the same window; the state is copied from them (d_gate, d_beta,
 *     d_conv_w may be NULL).
 *   d_snapshots NULL: the state is advanced again through positions 0 .. n
 *     from the pool row and the same window inputs the verify call used.
 * d_x is needed in both modes when W > 1.  Modifies d_conv_state and d_state
 * in place.
 * Errors: as spec_recurrent_verify. */
spec_status spec_recurrent_commit(const spec_recurrent_dims* dims, int32_t B, int32_t T, const float* d_x,
                                  const float* d_gate, const float* d_beta, const float* d_conv_w,
                                  const int32_t* d_slot, const int32_t* d_num_accepted,
                                  const float* d_snapshots, float* d_conv_state, float* d_state, void* stream);

/* The two calls of consecutive rounds in one: the replay commit of the
 * previous window (T_prev positions, d_prev_* its inputs, d_prev_accepted its
 * accept counts; T_prev == 0: nothing to commit, the d_prev_* may be NULL),
 * then the verify of the new window (T positions, no snapshots) from the
 * committed state still on chip.  The pool ends committed through the
 * previous window; the new window is committed by the next call (or by
 * spec_recurrent_commit in replay mode).  The results equal
 * spec_recurrent_commit(previous window, replay) followed by
 * spec_recurrent_verify(new window), bit for bit, with one read and one
 * write of each state instead of two reads and a write.
 * Errors: as spec_recurrent_verify; T_prev outside [0, 16] is INVALID_ARG. */
spec_status spec_recurrent_commit_verify(const spec_recurrent_dims* dims, int32_t B, int32_t T_prev,
                                         const float* d_prev_x, const float* d_prev_gate, const float* d_prev_beta,
                                         const int32_t* d_prev_accepted, int32_t T, const float* d_x,
                                         const float* d_gate, const float* d_beta, const float* d_conv_w,
                                         const int32_t* d_slot, float* d_conv_state, float* d_state, float* d_out,
                                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_RECURRENT_H */
