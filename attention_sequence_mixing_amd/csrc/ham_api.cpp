// ham_api.cpp -- the C ABI declared in include/ham.h: argument checks, scratch
// layout and the kernel sequence of each entry point.  Every launch goes to the
// caller's stream; nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "ham.h"
#include "ham_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

bool aligned16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

// attn: the call attends (ham_forward, ham_decode_step), so the KV heads' geometry
// must be one the kernels take; ham_route_stats runs the RNN alone.
int check_dims(const ham_dims* d, bool need_T, bool attn = true) {
  if (!d) return fail(HAM_EINVAL, "dims is NULL");
  if (d->H > 4096) return fail(HAM_EUNSUPPORTED, "H must be <= 4096 (H=%d)", d->H);
  if (d->B <= 0 || d->H <= 0 || (need_T && d->T <= 0))
    return fail(HAM_EINVAL, "B, T and H must be positive (B=%d T=%d H=%d)", d->B, d->T, d->H);
  // 64 or 128 each; or the RNN heads of the paper's layer, dk = 256 with dv = 384
  // (token-serial RNN kernel)
  if (!(((d->dk == 64 || d->dk == 128) && (d->dv == 64 || d->dv == 128)) || (d->dk == 256 && d->dv == 384)))
    return fail(HAM_EUNSUPPORTED, "dk and dv must be 64 or 128, or dk=256 with dv=384 (dk=%d dv=%d)",
                d->dk, d->dv);
  if (d->io_dtype != HAM_F32 && d->io_dtype != HAM_BF16)
    return fail(HAM_EUNSUPPORTED, "io_dtype must be HAM_F32 or HAM_BF16 (got %d)", d->io_dtype);
  if (d->flags & ~(HAM_CONTINUE | HAM_FORCE_RECURRENT | HAM_EXTERNAL_SCORES | HAM_TAU_PER_TOKEN | HAM_OVERLAP))
    return fail(HAM_EUNSUPPORTED, "unknown flag bits 0x%x", d->flags);
  if (d->cap <= 0) return fail(HAM_EINVAL, "cap must be positive (cap=%d)", d->cap);
  // the attention kernels address one head's cache rows with 32-bit byte offsets
  if (d->cap > (1 << 22)) return fail(HAM_EUNSUPPORTED, "cap must be <= 4194304 (cap=%d)", d->cap);
  if (!std::isfinite(d->scale) || !(d->scale > 0.f)) return fail(HAM_EINVAL, "scale must be finite and > 0");
  if (!(d->norm_eps >= 0.f) || !std::isfinite(d->norm_eps)) return fail(HAM_EINVAL, "norm_eps must be finite and >= 0");
  if (d->t0 < 0) return fail(HAM_EINVAL, "t0 must be >= 0");
  if (!std::isfinite(d->rope_base) || d->rope_base < 0.f)
    return fail(HAM_EINVAL, "rope_base must be 0 (none) or a finite positive base");
  if (d->kv_heads < 0 || d->dk_kv < 0 || d->dv_kv < 0)
    return fail(HAM_EINVAL, "kv_heads, dk_kv and dv_kv must be >= 0 (0: as the RNN heads)");
  if (attn) {
    const int HK = d->kv_heads > 0 ? d->kv_heads : d->H;
    const int DKK = d->dk_kv > 0 ? d->dk_kv : d->dk, DVK = d->dv_kv > 0 ? d->dv_kv : d->dv;
    // 64 or 128 each; or the KV heads of the paper's layer, dk_kv = 128 with dv_kv = 192
    if (!(((DKK == 64 || DKK == 128) && (DVK == 64 || DVK == 128)) || (DKK == 128 && DVK == 192)))
      return fail(HAM_EUNSUPPORTED, "dk_kv and dv_kv must be 64 or 128, or 128 with 192 (dk_kv=%d "
                                    "dv_kv=%d)", DKK, DVK);
    // the readout mix across head counts pairs two KV heads with each RNN head
    if (HK != d->H && HK != 2 * d->H)
      return fail(HAM_EUNSUPPORTED, "kv_heads (%d) must equal H or 2*H (H=%d)", HK, d->H);
    if ((long long)HK * DVK != (long long)d->H * d->dv)
      return fail(HAM_EUNSUPPORTED, "the KV heads' values must tile the RNN heads' output: kv_heads*dv_kv "
                                    "(%d*%d) != H*dv (%d*%d)", HK, DVK, d->H, d->dv);
  }
  if (d->route_block < 0 || d->route_block > ham::kChunk || (d->route_block & (d->route_block - 1)))
    return fail(HAM_EUNSUPPORTED, "route_block must be 0, 1 or a power of two up to %d (route_block=%d)",
                ham::kChunk, d->route_block);
  if (need_T && d->route_block > 1 && (d->t0 % d->route_block || d->T % d->route_block))
    return fail(HAM_EINVAL, "with route_block=%d, t0 (%d) and T (%d) must be multiples of it (whole blocks)",
                d->route_block, d->t0, d->T);
  const double elems = (double)d->B * (need_T ? d->T : 1) * d->H * (d->dk > d->dv ? d->dk : d->dv);
  if (elems > 9.0e15) return fail(HAM_EINVAL, "problem too large");
  return HAM_OK;
}

#define HAM_REQUIRE(p) \
  do { if (!(p)) return fail(HAM_EINVAL, "required pointer %s is NULL", #p); } while (0)
#define HAM_ALIGNED(p) \
  do { if (!aligned16(p)) return fail(HAM_EINVAL, "pointer %s is not 16-byte aligned", #p); } while (0)
#define HAM_HIP(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(HAM_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// block size of block-contiguous routing, or 0 for per-token routing
int route_blk(const ham_dims* d) { return d->route_block > 1 ? d->route_block : 0; }

// geometry of the attention (KV) heads; "split": another head count than the RNN's,
// so the mix of the two readouts runs in its own kernel
int kv_heads(const ham_dims* d) { return d->kv_heads > 0 ? d->kv_heads : d->H; }
int dk_kv(const ham_dims* d) { return d->dk_kv > 0 ? d->dk_kv : d->dk; }
int dv_kv(const ham_dims* d) { return d->dv_kv > 0 ? d->dv_kv : d->dv; }
bool split_heads(const ham_dims* d) { return kv_heads(d) != d->H; }
bool own_attn_inputs(const ham_dims* d) { return split_heads(d) || dk_kv(d) != d->dk; }

bool use_chunked(const ham_dims* d) {
  return !(d->flags & HAM_FORCE_RECURRENT) && d->T > ham::kChunk &&
         ham::rnn_chunked_supported(d->io_dtype, d->dk, d->dv);
}

struct SegPlan;
SegPlan seg_plan(const ham_dims* d);

// Segments of the chunked state pass.  Its workgroups (one per 64 state columns of a
// head) walk the chunks in order, one per CU; with few heads most CUs would idle, so
// the chunk sequence is cut into segments that run side by side: each segment's
// zero-start state B_p and transition A_p (the same pass with V = 0 from S = I), the
// entering states S_in[p+1] = A_p S_in[p] + B_p, then the full pass per segment.  Used
// when the heads' column blocks fill at most half the CUs and every segment keeps at
// least 8 chunks.
struct SegPlan {
  int nseg, per;        // segments, chunks per segment (the last may hold fewer)
};
SegPlan seg_plan(const ham_dims* d) {
  const int nchunk = (d->T + ham::kChunk - 1) / ham::kChunk;
  if (d->flags & HAM_OVERLAP) return {1, nchunk};          // the overlapped path is one segment
  if (!use_chunked(d) || d->dk > 128) return {1, nchunk};   // segments: d_k <= 128 only
  const long long nwg = (long long)d->B * d->H * (d->dv / 64);
  if (nwg > 128) return {1, nchunk};
  const long long p = std::max<long long>(1, std::min<long long>(256 / nwg, nchunk / 8));
  const int per = (int)((nchunk + p - 1) / p);
  return {(nchunk + per - 1) / per, per};                  // every segment non-empty
}

// The overlapped learned-router forward (HAM_OVERLAP with HAM_EXTERNAL_SCORES on the
// chunked path): the RNN runs on a second stream beside routing, compaction and
// attention, which write their readout to scratch; the mix follows the join.
bool overlapped(const ham_dims* d) {
  return (d->flags & HAM_OVERLAP) && (d->flags & HAM_EXTERNAL_SCORES) && use_chunked(d);
}

// Scratch regions of ham_forward / ham_route_stats (each 256-byte aligned).
struct FwdLayout {
  size_t o_rnn32, score, e, routed, chunk_count, count_in, ntok, lo, state, rope, prep, okv32;
  size_t seg_a, seg_b, seg_s, total;
  SegPlan seg;
};

FwdLayout fwd_layout(const ham_dims* d, bool with_state) {
  const size_t BTH = (size_t)d->B * d->T * d->H, BH = (size_t)d->B * d->H;
  const size_t BTK = (size_t)d->B * d->T * kv_heads(d), BK = (size_t)d->B * kv_heads(d);
  const size_t nchunk = ((size_t)d->T + ham::kChunk - 1) / ham::kChunk;
  FwdLayout L{};
  size_t off = 0;
  L.o_rnn32 = off;     off += up256(BTH * d->dv * sizeof(float));
  L.score = off;       off += up256(BTH * (d->dv / 16) * sizeof(float4));
  L.e = off;           off += up256(BTH * sizeof(float));
  L.routed = off;      off += up256(BTH);
  L.chunk_count = off; off += up256(BH * nchunk * sizeof(int32_t));
  L.count_in = off;    off += up256(BK * sizeof(int32_t));
  L.ntok = off;        off += up256(BTK * sizeof(int32_t));
  L.lo = off;          off += with_state ? 0 : up256(BTK * sizeof(int32_t));
  L.state = off;       off += with_state ? up256(BH * d->dk * d->dv * sizeof(float)) : 0;
  L.rope = off;        off += (!with_state && d->rope_base > 0.f) ? up256((size_t)d->T * (dk_kv(d) / 2) * sizeof(float2)) : 0;
  // the attention's own readout (fp32), when the mix runs in its own pass: KV heads of
  // another geometry, or the overlapped learned-router forward
  L.okv32 = off;       off += (!with_state && (split_heads(d) || overlapped(d))) ? up256(BTH * d->dv * sizeof(float)) : 0;
  L.prep = off;
  if (d->T > ham::kChunk && ham::rnn_chunked_supported(d->io_dtype, d->dk, d->dv))
    off += up256(BH * nchunk * ham::kPrepRecordBytes);
  L.seg = seg_plan(d);
  const size_t P = (size_t)L.seg.nseg;
  L.seg_a = off;       off += P > 1 ? up256((P - 1) * BH * d->dk * d->dk * sizeof(float)) : 0;
  L.seg_b = off;       off += P > 1 ? up256((P - 1) * BH * d->dk * d->dv * sizeof(float)) : 0;
  L.seg_s = off;       off += P > 1 ? up256(P * BH * d->dk * d->dv * sizeof(float)) : 0;
  L.total = off;
  return L;
}

struct DecLayout {
  size_t o_rnn32, score, e, routed, chunk_count, count_in, part, rope, lo, okv32, total;
  int nseg;
};

DecLayout dec_layout(const ham_dims* d) {
  const size_t BH = (size_t)d->B * d->H, BK = (size_t)d->B * kv_heads(d);
  DecLayout L{};
  L.nseg = (d->cap + ham::kDecodeSeg - 1) / ham::kDecodeSeg;
  size_t off = 0;
  L.o_rnn32 = off;     off += up256(BH * d->dv * sizeof(float));
  L.score = off;       off += up256(BH * (d->dv / 16) * sizeof(float4));
  L.e = off;           off += up256(BH * sizeof(float));
  L.routed = off;      off += up256(BH);
  L.chunk_count = off; off += up256(BH * sizeof(int32_t));
  L.count_in = off;    off += up256(BK * sizeof(int32_t));
  L.part = off;        off += up256(BK * (size_t)L.nseg * (dv_kv(d) + 2) * sizeof(float));
  L.rope = off;        off += d->rope_base > 0.f ? up256((size_t)d->B * (dk_kv(d) / 2) * sizeof(float2)) : 0;
  L.lo = off;          off += up256(BK * sizeof(int32_t));
  L.okv32 = off;       off += split_heads(d) ? up256(BH * d->dv * sizeof(float)) : 0;
  L.total = off;
  return L;
}

// ---- stage timing (ham_profile_*) ------------------------------------------------
struct Profiler {
  std::mutex mu;
  bool armed = false;
  int max_calls = 0, used = 0;
  std::vector<hipEvent_t> ev;      // max_calls x HAM_PROFILE_STAGES x (begin, end)
  std::vector<int> kinds, done;    // done: bit i set when stage i has both events
};
Profiler g_prof;

// One call's recorder: claims a slot when armed.  Stages run one after another on
// the call's stream (mark() ends the current stage and begins the next), or on
// other streams (begin / end name the stage and the stream).
struct CallTimer {
  int slot = -1, stage = 0;
  hipStream_t s;
  CallTimer(int kind, hipStream_t st) : s(st) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (!g_prof.armed || g_prof.used >= g_prof.max_calls) return;
    slot = g_prof.used++;
    g_prof.kinds[slot] = kind;
    g_prof.done[slot] = 0;
    begin(0, s);
  }
  hipEvent_t ev(int st, int which) const { return g_prof.ev[((size_t)slot * HAM_PROFILE_STAGES + st) * 2 + which]; }
  void begin(int st, hipStream_t str) {
    if (slot >= 0 && st < HAM_PROFILE_STAGES) (void)hipEventRecord(ev(st, 0), str);
  }
  void end(int st, hipStream_t str) {
    if (slot < 0 || st >= HAM_PROFILE_STAGES) return;
    (void)hipEventRecord(ev(st, 1), str);
    g_prof.done[slot] |= 1 << st;
  }
  void mark() {
    if (slot < 0 || stage >= HAM_PROFILE_STAGES) return;
    end(stage, s);
    ++stage;
    begin(stage, s);
  }
};

template <class T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

// A second stream per device for the overlapped forward, with a fork and a join
// event.  Created on first use (default priority, non-blocking) and kept for the
// process.  The mutex is held from the fork to the join so that calls from several
// host threads do not interleave their event records and waits.
constexpr int kMaxDevices = 64;
struct SideStream {
  std::mutex mu;
  hipStream_t st[kMaxDevices] = {};
  hipEvent_t fork[kMaxDevices] = {}, join[kMaxDevices] = {};
};
SideStream g_side;

int side_stream(int* dev_out) {
  int dev = -1;
  HAM_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(HAM_EUNSUPPORTED, "device index beyond %d", kMaxDevices - 1);
  if (!g_side.st[dev]) {
    HAM_HIP(hipStreamCreateWithFlags(&g_side.st[dev], hipStreamNonBlocking));
    HAM_HIP(hipEventCreateWithFlags(&g_side.fork[dev], hipEventDisableTiming));
    HAM_HIP(hipEventCreateWithFlags(&g_side.join[dev], hipEventDisableTiming));
  }
  *dev_out = dev;
  return HAM_OK;
}

// The RNN pass shared by ham_forward and ham_route_stats; returns the slice count.
// Two timer stages: the chunk prep (empty on the token-serial path) and the state pass.
int run_rnn(const ham_dims* d, const ham::RnnArgs& ra, hipStream_t s, int* slices, CallTimer& tm,
            const FwdLayout& L, void* ws) {
  if (use_chunked(d)) {
    *slices = ham::rnn_chunked_slices(d->dv);
    HAM_HIP(ham::launch_rnn_chunked_prep(d->io_dtype, d->dk, ra, s));
    tm.mark();
    const int P = L.seg.nseg, per = L.seg.per;
    if (P == 1) {
      HAM_HIP(ham::launch_rnn_chunked_state(d->io_dtype, d->dk, d->dv, ra, s));
    } else {
      const size_t BH = (size_t)d->B * d->H;
      float* Am = at<float>(ws, L.seg_a);
      float* Bm = at<float>(ws, L.seg_b);
      float* Sin = at<float>(ws, L.seg_s);
      // zero-start states and transitions of segments 0 .. P-2
      ham::RnnArgs rb = ra;
      rb.S0 = nullptr; rb.S_out = Bm; rb.o_rnn32 = nullptr; rb.variant = 0;
      rb.seg_chunks = per; rb.seg_stride = BH * d->dk * d->dv;
      HAM_HIP(ham::launch_rnn_chunked_state_seg(d->io_dtype, d->dk, d->dv, 1, P - 1, rb, s));
      ham::RnnArgs rh = rb;
      rh.S_out = Am; rh.seg_stride = BH * d->dk * d->dk;
      HAM_HIP(ham::launch_rnn_chunked_state_seg(d->io_dtype, d->dk, d->dk, 2, P - 1, rh, s));
      ham::SegArgs sg{ra.S0, Am, Bm, Sin, d->B, d->H, P};
      HAM_HIP(ham::launch_seg_combine(d->dk, d->dv, sg, s));
      // the full pass, every segment from its entering state
      ham::RnnArgs rf = ra;
      rf.S0 = Sin; rf.seg_chunks = per; rf.seg_stride = BH * d->dk * d->dv;
      HAM_HIP(ham::launch_rnn_chunked_state_seg(d->io_dtype, d->dk, d->dv, 0, P, rf, s));
    }
  } else {
    *slices = ham::rnn_recurrent_slices(d->dv);
    tm.mark();
    HAM_HIP(ham::launch_rnn_recurrent(d->io_dtype, d->dk, d->dv, ra, s));
  }
  tm.mark();
  return HAM_OK;
}

}  // namespace

namespace ham {
// The error path of entry points defined in other translation units.
int api_fail(int code, const char* msg) { return fail(code, "%s", msg); }
}  // namespace ham

namespace ham {

// The host checks of a decode step's dims and arguments (everything but the workspace).
int decode_check(const ham_dims* d, const void* q, const void* k, const void* v, const void* q_attn,
                      const void* k_attn, const void* v_attn, const float* beta, const float* g,
                      const float* tau, const float* block_score, const float* S, const void* Kc,
                      const void* Vc, const int32_t* pos, const int32_t* count, const int32_t* t_abs,
                      const void* o, const void* o_rnn, const void* o_kv, const float* e) {
  int rc = check_dims(d, false);
  if (rc != HAM_OK) return rc;
  HAM_REQUIRE(q); HAM_REQUIRE(k); HAM_REQUIRE(v); HAM_REQUIRE(beta); HAM_REQUIRE(g);
  HAM_REQUIRE(tau); HAM_REQUIRE(S); HAM_REQUIRE(Kc); HAM_REQUIRE(Vc); HAM_REQUIRE(pos);
  HAM_REQUIRE(count); HAM_REQUIRE(t_abs); HAM_REQUIRE(o);
  if (route_blk(d)) HAM_REQUIRE(block_score);
  if (own_attn_inputs(d) && !(q_attn && k_attn && v_attn))
    return fail(HAM_EINVAL, "the KV heads' geometry differs from the RNN heads': q_attn, k_attn and "
                            "v_attn are required");
  HAM_ALIGNED(q); HAM_ALIGNED(k); HAM_ALIGNED(v); HAM_ALIGNED(q_attn); HAM_ALIGNED(k_attn);
  HAM_ALIGNED(v_attn); HAM_ALIGNED(S); HAM_ALIGNED(o); HAM_ALIGNED(o_rnn); HAM_ALIGNED(o_kv);
  HAM_ALIGNED(Kc); HAM_ALIGNED(Vc);
  if ((d->flags & HAM_EXTERNAL_SCORES) && !e)
    return fail(HAM_EINVAL, "HAM_EXTERNAL_SCORES needs the scores in e (NULL)");
  return HAM_OK;
}

}  // namespace ham

extern "C" {

int ham_version(void) { return 10500; }

const char* ham_last_error(void) { return g_err.c_str(); }

size_t ham_forward_workspace_size(const ham_dims* d) {
  if (check_dims(d, true) != HAM_OK) return 0;
  return fwd_layout(d, false).total;
}

size_t ham_route_stats_workspace_size(const ham_dims* d) {
  if (check_dims(d, true, false) != HAM_OK) return 0;
  return fwd_layout(d, true).total;
}

// Scratch of the attention backward: per-query statistics (32 bytes per token-head);
// with bf16 inputs also the visible range of each 64-query tile and the two bf16 terms
// of dO.
struct AttnBwdLayout {
  size_t stat = 0, rng = 0, dOh = 0, dOl = 0, total = 0;
};
static AttnBwdLayout attn_bwd_layout(const ham_dims* d) {
  AttnBwdLayout L;
  const size_t ntok = (size_t)d->B * d->T * kv_heads(d);
  L.total = up256(ntok * 8 * sizeof(float));
  if (d->io_dtype == HAM_BF16) {
    L.rng = L.total;
    L.total += up256((size_t)d->B * kv_heads(d) * ((d->T + 63) / 64) * 2 * sizeof(int32_t));
    L.dOh = L.total;
    L.total += up256(ntok * dv_kv(d) * 2);
    L.dOl = L.total;
    L.total += up256(ntok * dv_kv(d) * 2);
  }
  return L;
}

size_t ham_attention_backward_workspace_size(const ham_dims* d) {
  if (check_dims(d, true) != HAM_OK) return 0;
  return attn_bwd_layout(d).total;
}

int ham_attention_backward(const ham_dims* d, const void* q_attn, const void* Kc, const void* Vc,
                           const int32_t* pos, const int32_t* count, const int32_t* doc_start,
                           const float* dO, float* dq, float* dKc, float* dVc,
                           void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(d, true);
  if (rc != HAM_OK) return rc;
  if (d->rope_base > 0.f || route_blk(d) || dv_kv(d) > 128)
    return fail(HAM_EUNSUPPORTED, "ham_attention_backward: no RoPE, no block routing, KV sizes 64 or 128");
  HAM_REQUIRE(q_attn); HAM_REQUIRE(Kc); HAM_REQUIRE(Vc); HAM_REQUIRE(pos); HAM_REQUIRE(count);
  HAM_REQUIRE(dO); HAM_REQUIRE(dq); HAM_REQUIRE(dKc); HAM_REQUIRE(dVc);
  HAM_ALIGNED(q_attn); HAM_ALIGNED(Kc); HAM_ALIGNED(Vc); HAM_ALIGNED(dO); HAM_ALIGNED(dq);
  HAM_ALIGNED(dKc); HAM_ALIGNED(dVc); HAM_ALIGNED(ws);
  const size_t need = ham_attention_backward_workspace_size(d);
  if (!ws || ws_bytes < need)
    return fail(HAM_EWORKSPACE, "workspace too small (%zu < %zu bytes)", ws_bytes, need);
  const AttnBwdLayout L = attn_bwd_layout(d);
  char* w = static_cast<char*>(ws);
  ham::AttnBwdArgs a{q_attn, Kc, Vc, pos, count, doc_start, dO, dq, dKc, dVc, reinterpret_cast<float*>(w + L.stat),
                     L.rng ? reinterpret_cast<int2*>(w + L.rng) : nullptr,
                     L.dOh ? reinterpret_cast<uint16_t*>(w + L.dOh) : nullptr,
                     L.dOl ? reinterpret_cast<uint16_t*>(w + L.dOl) : nullptr,
                     d->scale, d->B, d->T, kv_heads(d), d->cap, d->t0};
  HAM_HIP(ham::launch_attention_backward(d->io_dtype, dk_kv(d), dv_kv(d), a, static_cast<hipStream_t>(stream)));
  return HAM_OK;
}

size_t ham_rnn_backward_workspace_size(const ham_dims* d) {
  if (check_dims(d, true, false) != HAM_OK) return 0;
  if (!ham::rnn_backward_supported(d->dk, d->dv)) {
    fail(HAM_EUNSUPPORTED, "ham_rnn_backward: dk and dv must be 64 or 128 (dk=%d dv=%d)", d->dk, d->dv);
    return 0;
  }
  if (!(d->flags & HAM_FORCE_RECURRENT))
    return up256(ham::rnn_backward_chunked_scratch_floats(d->B, d->H, d->T, d->dk, d->dv) * sizeof(float));
  const size_t nchunk = ((size_t)d->T + ham::kChunk - 1) / ham::kChunk;
  const size_t total = ham::rnn_backward_scratch_floats(d->B, d->H, d->T, d->dk, d->dv);
  const size_t ck = total / (nchunk + ham::kChunk) * nchunk;      // the checkpoints come first
  return up256(ck * sizeof(float)) + up256((total - ck) * sizeof(float));
}

int ham_rnn_backward(const ham_dims* d, const void* q, const void* k, const void* v, const float* beta,
                     const float* g, const float* S0, const float* dO, const float* dS_T, float* dq,
                     float* dk, float* dv, float* dbeta, float* dg, float* dS0, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc = check_dims(d, true, false);
  if (rc != HAM_OK) return rc;
  if (!ham::rnn_backward_supported(d->dk, d->dv))
    return fail(HAM_EUNSUPPORTED, "ham_rnn_backward: dk and dv must be 64 or 128 (dk=%d dv=%d)", d->dk, d->dv);
  HAM_REQUIRE(q); HAM_REQUIRE(k); HAM_REQUIRE(v); HAM_REQUIRE(beta); HAM_REQUIRE(g); HAM_REQUIRE(dO);
  HAM_REQUIRE(dq); HAM_REQUIRE(dk); HAM_REQUIRE(dv); HAM_REQUIRE(dbeta); HAM_REQUIRE(dg); HAM_REQUIRE(dS0);
  HAM_ALIGNED(q); HAM_ALIGNED(k); HAM_ALIGNED(v); HAM_ALIGNED(S0); HAM_ALIGNED(dO); HAM_ALIGNED(dS_T);
  HAM_ALIGNED(dq); HAM_ALIGNED(dk); HAM_ALIGNED(dv); HAM_ALIGNED(dS0); HAM_ALIGNED(ws);
  const size_t need = ham_rnn_backward_workspace_size(d);
  if (!ws || ws_bytes < need)
    return fail(HAM_EWORKSPACE, "workspace too small (%zu < %zu bytes)", ws_bytes, need);
  if (!(d->flags & HAM_FORCE_RECURRENT)) {
    ham::RnnBwdArgs a{q, k, v, beta, g, S0, dO, dS_T, dq, dk, dv, dbeta, dg, dS0, nullptr, nullptr,
                      d->B, d->T, d->H, static_cast<float*>(ws)};
    HAM_HIP(ham::launch_rnn_backward_chunked(d->io_dtype, d->dk, d->dv, a, static_cast<hipStream_t>(stream)));
    return HAM_OK;
  }
  const size_t nchunk = ((size_t)d->T + ham::kChunk - 1) / ham::kChunk;
  const size_t total = ham::rnn_backward_scratch_floats(d->B, d->H, d->T, d->dk, d->dv);
  const size_t ck = total / (nchunk + ham::kChunk) * nchunk;
  ham::RnnBwdArgs a{q, k, v, beta, g, S0, dO, dS_T, dq, dk, dv, dbeta, dg, dS0, static_cast<float*>(ws),
                    at<float>(ws, up256(ck * sizeof(float))), d->B, d->T, d->H};
  HAM_HIP(ham::launch_rnn_backward(d->io_dtype, d->dk, d->dv, a, static_cast<hipStream_t>(stream)));
  return HAM_OK;
}

size_t ham_decode_workspace_size(const ham_dims* d) {
  if (check_dims(d, false) != HAM_OK) return 0;
  return dec_layout(d).total;
}

int ham_forward(const ham_dims* d, const void* q, const void* k, const void* v,
                const void* q_attn, const void* k_attn, const void* v_attn,
                const float* beta, const float* g, const float* tau,
                const float* gate_rnn, const float* gate_kv, const int32_t* doc_start,
                const float* S0, float* S_out, void* o, void* o_rnn, void* o_kv,
                float* e, uint8_t* routed, void* Kc, void* Vc, int32_t* pos, int32_t* count,
                void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(d, true);
  if (rc != HAM_OK) return rc;
  HAM_REQUIRE(q); HAM_REQUIRE(k); HAM_REQUIRE(v); HAM_REQUIRE(beta); HAM_REQUIRE(g);
  HAM_REQUIRE(tau); HAM_REQUIRE(S_out); HAM_REQUIRE(o); HAM_REQUIRE(Kc); HAM_REQUIRE(Vc);
  HAM_REQUIRE(pos); HAM_REQUIRE(count);
  HAM_ALIGNED(q); HAM_ALIGNED(k); HAM_ALIGNED(v); HAM_ALIGNED(q_attn); HAM_ALIGNED(k_attn);
  HAM_ALIGNED(v_attn); HAM_ALIGNED(S0); HAM_ALIGNED(S_out); HAM_ALIGNED(o); HAM_ALIGNED(o_rnn);
  HAM_ALIGNED(o_kv); HAM_ALIGNED(Kc); HAM_ALIGNED(Vc); HAM_ALIGNED(ws);
  const bool ext = (d->flags & HAM_EXTERNAL_SCORES) != 0;
  if (ext && !e) return fail(HAM_EINVAL, "HAM_EXTERNAL_SCORES needs the scores in e (NULL)");
  if (own_attn_inputs(d) && !(q_attn && k_attn && v_attn))
    return fail(HAM_EINVAL, "the KV heads' geometry differs from the RNN heads': q_attn, k_attn and "
                            "v_attn are required");
  if (!(d->flags & HAM_CONTINUE) && d->cap < d->T)
    return fail(HAM_ECAPACITY, "cap (%d) < T (%d): the cache cannot hold every token", d->cap, d->T);
  const FwdLayout L = fwd_layout(d, false);
  if (!ws || ws_bytes < L.total)
    return fail(HAM_EWORKSPACE, "workspace too small (%zu < %zu bytes)", ws_bytes, L.total);
  hipStream_t s = static_cast<hipStream_t>(stream);

  float* o_rnn32 = at<float>(ws, L.o_rnn32);
  float4* score = at<float4>(ws, L.score);
  float* e_buf = e ? e : at<float>(ws, L.e);
  uint8_t* r_buf = routed ? routed : at<uint8_t>(ws, L.routed);
  int32_t* chunk_count = at<int32_t>(ws, L.chunk_count);
  int32_t* count_in = at<int32_t>(ws, L.count_in);
  int32_t* ntok = at<int32_t>(ws, L.ntok);

  CallTimer tm(0, s);
  // with learned-router scores the state pass leaves out the score partials
  ham::RnnArgs ra{q, k, v, beta, g, S0, S_out, o_rnn32, score, at<char>(ws, L.prep), d->B, d->T, d->H};
  const bool ovl = overlapped(d);
  if (ext && use_chunked(d) && L.seg.nseg == 1) ra.variant = ovl ? 3 : 1;
  int slices = 0;
  std::unique_lock<std::mutex> side_lk;
  hipStream_t s2 = nullptr;
  int dev = 0;
  if (ovl) {
    // fork: the RNN on the side stream, beside routing, compaction and attention
    side_lk = std::unique_lock<std::mutex>(g_side.mu);
    rc = side_stream(&dev);
    if (rc != HAM_OK) return rc;
    s2 = g_side.st[dev];
    HAM_HIP(hipEventRecord(g_side.fork[dev], s));
    HAM_HIP(hipStreamWaitEvent(s2, g_side.fork[dev], 0));
    tm.begin(0, s2);
    HAM_HIP(ham::launch_rnn_chunked_prep(d->io_dtype, d->dk, ra, s2));
    tm.end(0, s2);
    tm.begin(1, s2);
    HAM_HIP(ham::launch_rnn_chunked_state(d->io_dtype, d->dk, d->dv, ra, s2));
    tm.end(1, s2);
    HAM_HIP(hipEventRecord(g_side.join[dev], s2));
    tm.stage = 2;
    tm.begin(2, s);
  } else {
    rc = run_rnn(d, ra, s, &slices, tm, L, ws);
    if (rc != HAM_OK) return rc;
  }

  ham::RouteArgs ro{score, slices, tau, ext ? nullptr : e_buf, r_buf, chunk_count,
                    (d->flags & HAM_CONTINUE) ? count : nullptr, count_in, d->B, d->T, d->H,
                    ext ? e : nullptr, (d->flags & HAM_TAU_PER_TOKEN) ? 1 : 0, route_blk(d), nullptr,
                    nullptr, kv_heads(d)};
  HAM_HIP(ham::launch_route(ro, s));
  tm.mark();

  // rotary table of the new tokens' positions (read by the key and query rotations)
  float2* rope = d->rope_base > 0.f ? at<float2>(ws, L.rope) : nullptr;
  if (rope) HAM_HIP(ham::launch_rope_table(rope, nullptr, d->t0, d->T, dk_kv(d), (double)d->rope_base, s));
  // one cache per KV head, following the routing of its RNN head
  const int HK = kv_heads(d);
  ham::CompactArgs ca{k_attn ? k_attn : k, v_attn ? v_attn : v, r_buf, chunk_count, count_in,
                      Kc, Vc, pos, count, ntok, nullptr, nullptr, d->t0, d->B, d->T, HK, d->cap,
                      rope, route_blk(d), d->H};
  HAM_HIP(ham::launch_compact(d->io_dtype, dk_kv(d), dv_kv(d), ca, s));
  tm.mark();

  // same-document masking: each query's first visible cache entry
  int32_t* lo = doc_start ? at<int32_t>(ws, L.lo) : nullptr;
  if (lo) {
    ham::DocLoArgs da{doc_start, ntok, count_in, count, pos, lo, d->t0, d->B, d->T, HK, d->cap,
                      route_blk(d)};
    HAM_HIP(ham::launch_doc_lo(da, s));
  }
  // With KV heads of another geometry, or on the overlapped path, the attention writes
  // its readout to scratch and the mix of the two headwise-normalised readouts runs
  // afterwards.
  const bool sep = split_heads(d) || ovl;
  float* okv32 = sep ? at<float>(ws, L.okv32) : nullptr;
  ham::AttnArgs aa{q_attn ? q_attn : q, Kc, Vc, ntok, sep ? nullptr : o_rnn32, gate_rnn, gate_kv, o,
                   o_rnn, o_kv, d->scale, d->norm_eps, d->B, d->T, HK, d->cap, rope,
                   (!sep && use_chunked(d)) ? 1 : 0, lo, okv32};
  HAM_HIP(ham::launch_attention(d->io_dtype, dk_kv(d), dv_kv(d), aa, s));
  if (ovl) {
    tm.end(4, s);                            // attention alone; the join and mix follow
    HAM_HIP(hipStreamWaitEvent(s, g_side.join[dev], 0));
    side_lk.unlock();
  }
  if (sep) {
    ham::MixArgs mx{o_rnn32, okv32, gate_rnn, gate_kv, o, o_rnn, o_kv, d->norm_eps, d->B * d->T, d->H,
                    HK / d->H, use_chunked(d) ? 1 : 0};
    HAM_HIP(ham::launch_mix(d->io_dtype, d->dv, mx, s));
  }
  if (!ovl) tm.mark();
  return HAM_OK;
}

int ham_decode_step(const ham_dims* d, const void* q, const void* k, const void* v,
                    const void* q_attn, const void* k_attn, const void* v_attn,
                    const float* beta, const float* g, const float* tau,
                    const float* gate_rnn, const float* gate_kv, const int32_t* doc_start,
                    float* block_score, float* S, void* Kc, void* Vc, int32_t* pos, int32_t* count,
                    const int32_t* t_abs, void* o, void* o_rnn, void* o_kv,
                    float* e, uint8_t* routed, int32_t* status,
                    void* ws, size_t ws_bytes, void* stream) {
  const int rc = ham::decode_check(d, q, k, v, q_attn, k_attn, v_attn, beta, g, tau, block_score, S, Kc, Vc, pos,
                                   count, t_abs, o, o_rnn, o_kv, e);
  if (rc != HAM_OK) return rc;
  HAM_ALIGNED(ws);
  const bool ext = (d->flags & HAM_EXTERNAL_SCORES) != 0;
  const DecLayout L = dec_layout(d);
  if (!ws || ws_bytes < L.total)
    return fail(HAM_EWORKSPACE, "workspace too small (%zu < %zu bytes)", ws_bytes, L.total);
  hipStream_t s = static_cast<hipStream_t>(stream);

  float* o_rnn32 = at<float>(ws, L.o_rnn32);
  float4* score = at<float4>(ws, L.score);
  float* e_buf = e ? e : at<float>(ws, L.e);
  uint8_t* r_buf = routed ? routed : at<uint8_t>(ws, L.routed);
  int32_t* chunk_count = at<int32_t>(ws, L.chunk_count);
  int32_t* count_in = at<int32_t>(ws, L.count_in);
  float* part = at<float>(ws, L.part);

  CallTimer tm(1, s);
  ham::RnnArgs ra{q, k, v, beta, g, S, S, o_rnn32, score, nullptr, d->B, 1, d->H};
  HAM_HIP(ham::launch_rnn_recurrent(d->io_dtype, d->dk, d->dv, ra, s));
  tm.mark();
  ham::RouteArgs ro{score, ham::rnn_recurrent_slices(d->dv), tau, ext ? nullptr : e_buf, r_buf,
                    chunk_count, count, count_in, d->B, 1, d->H, ext ? e : nullptr,
                    (d->flags & HAM_TAU_PER_TOKEN) ? 1 : 0, route_blk(d), block_score, t_abs, kv_heads(d)};
  HAM_HIP(ham::launch_route(ro, s));
  tm.mark();
  // rotary table of the new tokens' positions t_abs[b] (key and query rotations)
  float2* rope = d->rope_base > 0.f ? at<float2>(ws, L.rope) : nullptr;
  if (rope) HAM_HIP(ham::launch_rope_table(rope, t_abs, 0, d->B, dk_kv(d), (double)d->rope_base, s));
  const int HK = kv_heads(d);
  ham::CompactArgs ca{k_attn ? k_attn : k, v_attn ? v_attn : v, r_buf, chunk_count, count_in,
                      Kc, Vc, pos, count, nullptr, status, t_abs, 0, d->B, 1, HK, d->cap,
                      rope, route_blk(d), d->H};
  HAM_HIP(ham::launch_compact(d->io_dtype, dk_kv(d), dv_kv(d), ca, s));
  tm.mark();
  int32_t* lo = doc_start ? at<int32_t>(ws, L.lo) : nullptr;
  if (lo) {
    ham::DocLoArgs dl{doc_start, nullptr, nullptr, count, pos, lo, 0, d->B, 1, HK, d->cap, 0};
    HAM_HIP(ham::launch_doc_lo(dl, s));
  }
  ham::DecodeAttnArgs da{q_attn ? q_attn : q, Kc, Vc, count, part, d->scale, d->B, HK, d->cap,
                         ham::kDecodeSeg, L.nseg, rope, lo};
  HAM_HIP(ham::launch_decode_attn(d->io_dtype, dk_kv(d), dv_kv(d), da, s));
  tm.mark();
  const bool split = split_heads(d);
  float* okv32 = split ? at<float>(ws, L.okv32) : nullptr;
  ham::DecodeCombineArgs cb{part, count, o_rnn32, gate_rnn, gate_kv, o, o_rnn, o_kv, d->norm_eps,
                            d->B, HK, ham::kDecodeSeg, L.nseg, okv32};
  HAM_HIP(ham::launch_decode_combine(d->io_dtype, dv_kv(d), cb, s));
  if (split) {
    ham::MixArgs mx{o_rnn32, okv32, gate_rnn, gate_kv, o, o_rnn, o_kv, d->norm_eps, d->B, d->H,
                    HK / d->H, 0};
    HAM_HIP(ham::launch_mix(d->io_dtype, d->dv, mx, s));
  }
  tm.mark();
  return HAM_OK;
}

int ham_route_stats(const ham_dims* d, const void* q, const void* k, const void* v,
                    const float* beta, const float* g, const float* tau, const float* S0,
                    float* e, uint8_t* routed, int32_t* count, int64_t* n_near, float near_band,
                    double* rho_host, void* ws, size_t ws_bytes, void* stream) {
  (void)q;
  int rc = check_dims(d, true, false);
  if (rc != HAM_OK) return rc;
  if (d->flags & HAM_EXTERNAL_SCORES)
    return fail(HAM_EUNSUPPORTED, "ham_route_stats takes its scores from the RNN; use ham_select_tau "
                                  "on learned-router scores");
  HAM_REQUIRE(k); HAM_REQUIRE(v); HAM_REQUIRE(beta); HAM_REQUIRE(g); HAM_REQUIRE(tau);
  HAM_REQUIRE(count);
  HAM_ALIGNED(k); HAM_ALIGNED(v); HAM_ALIGNED(S0); HAM_ALIGNED(ws);
  if (n_near && !(near_band >= 0.f)) return fail(HAM_EINVAL, "near_band must be >= 0");
  if (n_near && route_blk(d))
    return fail(HAM_EUNSUPPORTED, "n_near counts per-token scores; pass NULL with route_block > 1");
  const FwdLayout L = fwd_layout(d, true);
  if (!ws || ws_bytes < L.total)
    return fail(HAM_EWORKSPACE, "workspace too small (%zu < %zu bytes)", ws_bytes, L.total);
  hipStream_t s = static_cast<hipStream_t>(stream);

  float4* score = at<float4>(ws, L.score);
  float* e_buf = e ? e : at<float>(ws, L.e);
  uint8_t* r_buf = routed ? routed : at<uint8_t>(ws, L.routed);
  int32_t* chunk_count = at<int32_t>(ws, L.chunk_count);
  int32_t* count_in = at<int32_t>(ws, L.count_in);
  float* S_tmp = at<float>(ws, L.state);

  CallTimer tm(2, s);
  ham::RnnArgs ra{q ? q : k, k, v, beta, g, S0, S_tmp, nullptr, score, at<char>(ws, L.prep),
                  d->B, d->T, d->H};
  int slices = 0;
  rc = run_rnn(d, ra, s, &slices, tm, L, ws);
  if (rc != HAM_OK) return rc;
  ham::RouteArgs ro{score, slices, tau, e_buf, r_buf, chunk_count, nullptr, count_in,
                    d->B, d->T, d->H, nullptr, (d->flags & HAM_TAU_PER_TOKEN) ? 1 : 0, route_blk(d),
                    nullptr, nullptr, 0};
  HAM_HIP(ham::launch_route(ro, s));
  tm.mark();
  ham::StatsArgs sa{e_buf, tau, chunk_count, count, n_near, near_band, d->B, d->T, d->H,
                    (d->flags & HAM_TAU_PER_TOKEN) ? 1 : 0};
  HAM_HIP(ham::launch_stats(sa, s));
  tm.mark();
  if (rho_host) {
    std::vector<int32_t> c((size_t)d->B * d->H);
    HAM_HIP(hipMemcpyAsync(c.data(), count, c.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s));
    HAM_HIP(hipStreamSynchronize(s));
    double tot = 0;
    for (int32_t x : c) tot += x;
    *rho_host = tot / ((double)d->B * d->T * d->H);
  }
  return HAM_OK;
}

int ham_select_tau(const ham_dims* d, const float* e, double rho, float* tau, void* stream) {
  if (!d) return fail(HAM_EINVAL, "dims is NULL");
  if (d->B <= 0 || d->T <= 0 || d->H <= 0)
    return fail(HAM_EINVAL, "B, T and H must be positive (B=%d T=%d H=%d)", d->B, d->T, d->H);
  if ((long long)d->B * d->T > 2147483647LL) return fail(HAM_EINVAL, "B*T must be < 2^31");
  if (!(rho >= 0.0 && rho <= 1.0)) return fail(HAM_EINVAL, "rho must lie in [0, 1]");
  HAM_REQUIRE(e); HAM_REQUIRE(tau);
  const long long N = (long long)d->B * d->T;
  const long long k = (long long)std::nearbyint(rho * (double)N);   // ties to even
  HAM_HIP(ham::launch_select_tau(e, d->B, d->T, d->H, k, tau, static_cast<hipStream_t>(stream)));
  return HAM_OK;
}

int ham_profile_start(int max_calls) {
  if (max_calls <= 0 || max_calls > (1 << 20)) return fail(HAM_EINVAL, "max_calls out of range");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.assign((size_t)max_calls * HAM_PROFILE_STAGES * 2, nullptr);
  for (auto& e : g_prof.ev) HAM_HIP(hipEventCreate(&e));
  g_prof.kinds.assign(max_calls, -1);
  g_prof.done.assign(max_calls, 0);
  g_prof.max_calls = max_calls;
  g_prof.used = 0;
  g_prof.armed = true;
  return HAM_OK;
}

int ham_profile_stop(float* stage_ms, int max_values, int* n_calls, int* kinds) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.armed) return fail(HAM_EINVAL, "profiling is not armed");
  g_prof.armed = false;
  const int used = g_prof.used;
  if (n_calls) *n_calls = used;
  for (int c = 0; c < used; ++c) {
    if (kinds) kinds[c] = g_prof.kinds[c];
    const size_t base = (size_t)c * HAM_PROFILE_STAGES * 2;
    const int done = g_prof.done[c];
    for (int st = 0; st < HAM_PROFILE_STAGES; ++st) {
      const long idx = (long)c * HAM_PROFILE_STAGES + st;
      float ms = 0.f;
      if (done & (1 << st)) {
        HAM_HIP(hipEventSynchronize(g_prof.ev[base + 2 * st + 1]));
        HAM_HIP(hipEventElapsedTime(&ms, g_prof.ev[base + 2 * st], g_prof.ev[base + 2 * st + 1]));
      }
      if (stage_ms && idx < max_values) stage_ms[idx] = ms;
    }
  }
  return HAM_OK;
}

}  // extern "C"
