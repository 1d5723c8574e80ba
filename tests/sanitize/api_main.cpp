// Host-side driver of the C ABI for the sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of ham_api.cpp; the device objects are
// the ordinary build).  Runs only paths that finish on the host: the workspace-size
// functions over a sweep of shapes, and every entry point's argument checks (missing
// pointers, unknown dtypes and flags, bad geometry, short workspaces), which must
// return their documented codes with a message.  No GPU is needed or touched: every
// call here is rejected before anything is enqueued.  Exit status 0 when every
// expectation holds; a sanitizer report aborts the process.
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <vector>

#include "ham.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    std::fprintf(stderr, "%s: returned %d, expected %d (%s)\n", what, got, want, ham_last_error());
    ++failures;
    return;
  }
  if (want != HAM_OK && std::strlen(ham_last_error()) == 0) {
    std::fprintf(stderr, "%s: error %d without a message\n", what, got);
    ++failures;
  }
}

static ham_dims dims(int B, int T, int H, int dk, int dv, int io, int cap) {
  ham_dims d;
  std::memset(&d, 0, sizeof d);
  d.B = B; d.T = T; d.H = H; d.dk = dk; d.dv = dv; d.io_dtype = io;
  d.scale = 0.125f; d.norm_eps = 1e-6f; d.cap = cap;
  return d;
}

// Every workspace-size function over a sweep of shapes, flags and head layouts,
// including shapes whose byte counts pass 2^32 and ones the library rejects.
static void sweep_sizes() {
  const int Bs[] = {0, 1, 3, 64, 4096};
  const int Ts[] = {0, 1, 63, 64, 65, 4096, 1 << 20};
  const int Hs[] = {1, 5, 16, 64};
  const int ds[] = {32, 64, 128, 192, 256, 384};
  const int flags[] = {0, HAM_CONTINUE, HAM_FORCE_RECURRENT, HAM_EXTERNAL_SCORES | HAM_OVERLAP,
                       HAM_TAU_PER_TOKEN, 32};
  size_t total = 0;
  for (int B : Bs)
    for (int T : Ts)
      for (int H : Hs)
        for (int dk : ds)
          for (int dv : ds)
            for (int io = 0; io < 3; ++io)
              for (int f : flags)
                for (int layout = 0; layout < 4; ++layout) {
                  ham_dims d = dims(B, T, H, dk, dv, io, T > 0 ? T : 1);
                  d.flags = f;
                  if (layout == 1) { d.kv_heads = 2 * H; d.dk_kv = 128; d.dv_kv = dv / 2; }
                  if (layout == 2) { d.route_block = 64; d.rope_base = 500000.f; }
                  if (layout == 3) { d.kv_heads = 3 * H; d.cap = 0; }
                  total += ham_forward_workspace_size(&d);
                  total += ham_decode_workspace_size(&d);
                  total += ham_route_stats_workspace_size(&d);
                  total += ham_attention_backward_workspace_size(&d);
                  total += ham_rnn_backward_workspace_size(&d);
                }
  std::printf("workspace sweep done (%zu bytes summed)\n", total);
}

int main() {
  std::printf("ham_version %d\n", ham_version());
  sweep_sizes();

  // fake, aligned, never dereferenced on the host: every call below is rejected
  // before it reaches the device
  void* P = reinterpret_cast<void*>(uintptr_t(1) << 20);
  float* F = static_cast<float*>(P);
  int32_t* I = static_cast<int32_t*>(P);
  uint8_t* U = static_cast<uint8_t*>(P);
  int64_t* L = static_cast<int64_t*>(P);
  double rho = 0;

  const ham_dims ok = dims(2, 128, 4, 64, 64, HAM_BF16, 128);
  ham_dims bad_io = ok; bad_io.io_dtype = 7;
  ham_dims bad_flag = ok; bad_flag.flags = 32;
  ham_dims bad_d = ok; bad_d.dk = 96;
  ham_dims bad_cap = ok; bad_cap.cap = 16;
  ham_dims bad_kvh = ok; bad_kvh.kv_heads = 3 * ok.H;
  ham_dims bad_blk = ok; bad_blk.route_block = 3;
  ham_dims neg = ok; neg.T = -1;

  // ham_forward
  expect("forward null dims", ham_forward(nullptr, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, 0, 0, F, U, P, P, I, I,
                                          P, 1 << 30, 0), HAM_EINVAL);
  expect("forward null q", ham_forward(&ok, nullptr, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, 0, 0, F, U, P, P, I, I,
                                       P, 1 << 30, 0), HAM_EINVAL);
  expect("forward dtype", ham_forward(&bad_io, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, 0, 0, F, U, P, P, I, I,
                                      P, 1 << 30, 0), HAM_EUNSUPPORTED);
  expect("forward flag", ham_forward(&bad_flag, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, 0, 0, F, U, P, P, I, I,
                                     P, 1 << 30, 0), HAM_EUNSUPPORTED);
  expect("forward head size", ham_forward(&bad_d, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, 0, 0, F, U, P, P, I, I,
                                          P, 1 << 30, 0), HAM_EUNSUPPORTED);
  expect("forward capacity", ham_forward(&bad_cap, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, 0, 0, F, U, P, P, I,
                                         I, P, 1 << 30, 0), HAM_ECAPACITY);
  expect("forward kv heads", ham_forward(&bad_kvh, P, P, P, P, P, P, F, F, F, 0, 0, 0, 0, F, P, 0, 0, F, U, P, P, I,
                                         I, P, 1 << 30, 0), HAM_EUNSUPPORTED);
  expect("forward negative T", ham_forward(&neg, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, 0, 0, F, U, P, P, I, I,
                                           P, 1 << 30, 0), HAM_EINVAL);
  expect("forward route block", ham_forward(&bad_blk, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, 0, 0, F, U, P, P,
                                            I, I, P, 1 << 30, 0), HAM_EUNSUPPORTED);
  expect("forward misaligned", ham_forward(&ok, static_cast<char*>(P) + 2, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P,
                                           0, 0, F, U, P, P, I, I, P, 1 << 30, 0), HAM_EINVAL);
  expect("forward workspace", ham_forward(&ok, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, 0, 0, F, U, P, P, I, I,
                                          P, 16, 0), HAM_EWORKSPACE);

  // ham_decode_step and the allocation-free variant
  ham_dims dec = ok; dec.T = 1; dec.flags = HAM_CONTINUE;
  ham_dims dec_io = dec; dec_io.io_dtype = 7;
  expect("decode null S", ham_decode_step(&dec, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, nullptr, P, P, I, I, I, P, 0, 0,
                                          F, U, I, P, 1 << 30, 0), HAM_EINVAL);
  expect("decode dtype", ham_decode_step(&dec_io, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, P, I, I, I, P, 0, 0, F,
                                         U, I, P, 1 << 30, 0), HAM_EUNSUPPORTED);
  expect("decode workspace", ham_decode_step(&dec, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, P, I, I, I, P, 0, 0, F,
                                             U, I, P, 8, 0), HAM_EWORKSPACE);
  expect("noalloc null S", ham_decode_step_noalloc(&dec, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, nullptr, P, P, I, I, I,
                                                   P, 0, 0, F, U, I, 0), HAM_EINVAL);
  expect("noalloc dtype", ham_decode_step_noalloc(&dec_io, P, P, P, 0, 0, 0, F, F, F, 0, 0, 0, 0, F, P, P, I, I, I, P,
                                                  0, 0, F, U, I, 0), HAM_EUNSUPPORTED);
  if (ham_decode_noalloc_scratch_bytes() != HAM_NOALLOC_SCRATCH_BYTES) {
    std::fprintf(stderr, "noalloc scratch size %zu\n", ham_decode_noalloc_scratch_bytes());
    ++failures;
  }

  // ham_route_stats, ham_select_tau
  expect("route_stats null k", ham_route_stats(&ok, P, nullptr, P, F, F, F, 0, F, U, I, L, 0.05f, &rho, P, 1 << 30, 0),
         HAM_EINVAL);
  ham_dims ext = ok; ext.flags = HAM_EXTERNAL_SCORES;
  expect("route_stats external scores", ham_route_stats(&ext, P, P, P, F, F, F, 0, F, U, I, L, 0.05f, &rho, P, 1 << 30,
                                                        0), HAM_EUNSUPPORTED);
  expect("route_stats workspace", ham_route_stats(&ok, P, P, P, F, F, F, 0, F, U, I, L, 0.05f, &rho, P, 4, 0),
         HAM_EWORKSPACE);
  expect("select_tau null e", ham_select_tau(&ok, nullptr, 0.5, F, 0), HAM_EINVAL);
  expect("select_tau rho", ham_select_tau(&ok, F, 1.5, F, 0), HAM_EINVAL);

  // gradients
  expect("attention_backward null dO", ham_attention_backward(&ok, P, P, P, I, I, 0, nullptr, F, F, F, P, 1 << 30, 0),
         HAM_EINVAL);
  ham_dims rope = ok; rope.rope_base = 10000.f;
  expect("attention_backward rope", ham_attention_backward(&rope, P, P, P, I, I, 0, F, F, F, F, P, 1 << 30, 0),
         HAM_EUNSUPPORTED);
  expect("attention_backward workspace", ham_attention_backward(&ok, P, P, P, I, I, 0, F, F, F, F, P, 4, 0),
         HAM_EWORKSPACE);
  ham_dims big = ok; big.dk = 256;
  expect("rnn_backward head size", ham_rnn_backward(&big, P, P, P, F, F, 0, F, 0, F, F, F, F, F, F, P, 1 << 30, 0),
         HAM_EUNSUPPORTED);
  expect("rnn_backward null q", ham_rnn_backward(&ok, nullptr, P, P, F, F, 0, F, 0, F, F, F, F, F, F, P, 1 << 30, 0),
         HAM_EINVAL);
  expect("rnn_backward workspace", ham_rnn_backward(&ok, P, P, P, F, F, 0, F, 0, F, F, F, F, F, F, P, 4, 0),
         HAM_EWORKSPACE);

  // instrumentation
  int n = 0;
  expect("profile_stop null", ham_profile_stop(nullptr, 4, &n, nullptr), HAM_EINVAL);

  std::printf("%d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
