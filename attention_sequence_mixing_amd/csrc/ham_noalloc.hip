// ham_noalloc.hip -- the decode step for callers that cannot allocate device memory
// (code under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// ham_decode_step takes its scratch from the caller.  This entry point instead keeps
// the scratch in a file-scope device array of a fixed size, one copy per GPU, held for
// the life of the process; the caller still passes every input and output.  The
// kernels are those of ham_decode_step: none of them reads a scratch region before
// the same call has written it, so nothing is cleared between calls.  Calls that
// overlap on one GPU (two streams, two threads) share the array and race.
#include <cstdio>
#include <mutex>

#include "ham.h"
#include "ham_internal.h"

namespace {

// The decode workload (batch 32, 16 heads of 128, a 33K-entry cache) needs about
// 9 MiB; the split-K partials grow with B * kv_heads * ceil(cap / 1024) * (dv_kv + 2).
static __device__ __align__(256) char scratch[HAM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` on each GPU

// Device address of this GPU's copy of `scratch`, looked up once per device with that
// device current.  The host-side name `scratch` is not a device address.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return ham::api_fail(HAM_EHIP, "ham_decode_step_noalloc: hipGetDevice failed");
  if (dev >= kMaxDevices)
    return ham::api_fail(HAM_EUNSUPPORTED, "ham_decode_step_noalloc: device index beyond 63");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return ham::api_fail(HAM_EHIP, "ham_decode_step_noalloc: hipGetSymbolAddress(scratch) failed");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return HAM_OK;
}

}  // namespace

extern "C" size_t ham_decode_noalloc_scratch_bytes(void) { return HAM_NOALLOC_SCRATCH_BYTES; }

extern "C" int ham_decode_step_noalloc(const ham_dims* d, const void* q, const void* k, const void* v,
                                       const void* q_attn, const void* k_attn, const void* v_attn,
                                       const float* beta, const float* g, const float* tau,
                                       const float* gate_rnn, const float* gate_kv,
                                       const int32_t* doc_start, float* block_score, float* S,
                                       void* Kc, void* Vc, int32_t* pos, int32_t* count,
                                       const int32_t* t_abs, void* o, void* o_rnn, void* o_kv,
                                       float* e, uint8_t* routed, int32_t* status, void* stream) {
  // the argument checks of ham_decode_step come first, before any device query
  const int arc = ham::decode_check(d, q, k, v, q_attn, k_attn, v_attn, beta, g, tau, block_score, S, Kc, Vc, pos,
                                    count, t_abs, o, o_rnn, o_kv, e);
  if (arc != HAM_OK) return arc;
  const size_t need = ham_decode_workspace_size(d);
  if (need > (size_t)HAM_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    snprintf(msg, sizeof msg,
             "ham_decode_step_noalloc: this step needs %zu bytes of scratch, more than the %d it holds "
             "(fewer sequences, heads or cache entries; or ham_decode_step with a workspace)",
             need, HAM_NOALLOC_SCRATCH_BYTES);
    return ham::api_fail(HAM_EWORKSPACE, msg);
  }
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != HAM_OK) return rc;
  return ham_decode_step(d, q, k, v, q_attn, k_attn, v_attn, beta, g, tau, gate_rnn, gate_kv, doc_start,
                         block_score, S, Kc, Vc, pos, count, t_abs, o, o_rnn, o_kv, e, routed, status,
                         ws, (size_t)HAM_NOALLOC_SCRATCH_BYTES, stream);
}
