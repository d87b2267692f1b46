// Chain accept with no handle and no allocation: the accept kernels of
// spec_accept (accept.hip) run on a scratch area that lives in a file-scope
// device array of this library, for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array is found once per device with hipGetSymbolAddress (each GPU holds
// its own copy at its own address) and only that address is passed to the
// kernels.  Every scratch entry the kernels read is written earlier in the
// same call (row statistics, per-chunk residual sums, accept counts), so
// nothing has to start at zero; the flag word is the caller's (or a scratch
// word nobody reads).  Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "../../include/spec_verify.h"
#include "launch.h"

using namespace sv;

namespace {

// Capacity of the scratch: rows (B x T) of logits, sequences and vocabulary.
constexpr int kMaxRows = SPEC_STATIC_MAX_ROWS;
constexpr int kMaxSeqs = SPEC_STATIC_MAX_SEQS;
constexpr int kMaxVocab = SPEC_STATIC_MAX_VOCAB;
constexpr int kMaxChunks = (kMaxVocab + 4095) / 4096;

constexpr size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
constexpr size_t kRowstat = 0;                                                  // [rows][chunks][2] fp32
constexpr size_t kRowms = align256(kRowstat + (size_t)kMaxRows * kMaxChunks * 2 * 4);  // [rows][2] fp32
constexpr size_t kRsum = align256(kRowms + (size_t)kMaxRows * 2 * 4);           // [seqs][chunks] fp32
constexpr size_t kNacc = align256(kRsum + (size_t)kMaxSeqs * kMaxChunks * 4);   // [seqs] int32
constexpr size_t kFlags = align256(kNacc + (size_t)kMaxSeqs * 4);               // one word
constexpr size_t kBytes = align256(kFlags + 4);

static __device__ __align__(256) unsigned char scratch[kBytes];

// Device address of this GPU's copy of `scratch`, looked up on the first call
// on each device (the array's name is a host-side stand-in, not an address).
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

hipError_t scratch_ptr(unsigned char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = (unsigned char*)g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" spec_status spec_accept_chain_static(int32_t B, int32_t T, int32_t vocab, const float* d_logits,
                                                const float* d_q, const int32_t* d_tokens,
                                                const spec_sampling* sampling, int32_t* d_out_tokens,
                                                int32_t* d_num_accepted, const int32_t* d_kv_len,
                                                int32_t* d_kv_len_out, uint32_t* d_flags, void* stream) {
  if (!d_logits || !d_tokens || !sampling || !d_out_tokens || !d_num_accepted) return SPEC_ERR_INVALID_ARG;
  if (B < 1 || T < 1 || vocab < 2) return SPEC_ERR_INVALID_ARG;
  if (B > kMaxSeqs || (int64_t)B * T > kMaxRows || vocab > kMaxVocab || T > 128) return SPEC_ERR_CAPACITY;
  const float temp = sampling->temperature;
  if (!(temp >= 0.f) || !std::isfinite(temp)) return SPEC_ERR_INVALID_ARG;
  if (!(sampling->top_p >= 0.f && sampling->top_p <= 1.f) || sampling->top_k < 0) return SPEC_ERR_INVALID_ARG;
  const bool adjust = temp > 0.f && ((sampling->top_k > 0 && sampling->top_k < vocab) || sampling->top_p < 1.f);
  if (adjust) return SPEC_ERR_UNSUPPORTED;  // the top-k / top-p selection scratch is not held here
  if (temp > 0.f && T > 1 && !d_q) return SPEC_ERR_INVALID_ARG;
  if (d_kv_len_out && !d_kv_len) return SPEC_ERR_INVALID_ARG;
  unsigned char* s = nullptr;
  if (scratch_ptr(&s) != hipSuccess) return SPEC_ERR_DEVICE;

  AcceptParams ap{};
  ap.logits = d_logits; ap.q = d_q; ap.tokens = d_tokens; ap.parent = nullptr;
  ap.temperature = temp; ap.replacement = 0; ap.seed = sampling->seed; ap.round = sampling->round;
  ap.out_tokens = d_out_tokens; ap.num_accepted = d_num_accepted; ap.kv_len = d_kv_len;
  ap.kv_len_out = d_kv_len_out;
  ap.rowstat = (float*)(s + kRowstat); ap.rowms = (float*)(s + kRowms); ap.rsum = (float*)(s + kRsum);
  ap.nacc = (int32_t*)(s + kNacc);
  ap.flags = d_flags ? d_flags : (uint32_t*)(s + kFlags);
  ap.B = B; ap.T = T; ap.V = vocab; ap.nch = accept_chunks(vocab);
  ap.rows = B * T; ap.qrows = B * (T - 1);
  ap.top_k = 0; ap.top_p = 1.f;
  return launch_accept(ap, (hipStream_t)stream) == hipSuccess ? SPEC_OK : SPEC_ERR_DEVICE;
}
