// ham_bwd.hip -- gradients of the sparse causal attention over the compacted cache.
//
// "Hybrid Associative Memories" §2 KV-memory equation: o_t = sum_c p_tc v_c with
// p_t = softmax_c(scale * q_t . k_c) over the cached entries visible to query t
// (positions <= t; with same-document masking, >= the document start: App. A.1
// "FlexAttention and Block Masks").  Given g_t = dL/do_t, the gradients are those of
// softmax attention: with D_t = sum_c p_tc (g_t . v_c) (= g_t . o_t),
//   dL/dq_t = scale * sum_c p_tc (g_t . v_c - D_t) k_c
//   dL/dk_c = scale * sum_t p_tc (g_t . v_c - D_t) q_t
//   dL/dv_c = sum_t p_tc g_t
// The routing decision is a threshold and passes no gradient.
//
// Visibility comes from the cache itself: entries are in ascending position, so
// query t (absolute position t0 + t) sees entries [lo_t, n_t) with n_t = #{pos <=
// t0 + t} and lo_t = #{pos < doc start}.  Two kernels, both fp32: the query kernel
// (one wave per query) forms the row statistics (m, l, D) and dq; the entry kernel
// (one wave per cache entry) walks the queries that see the entry and forms dk, dv.
// Each takes 64 items at a time with a lane per item for the dot products (rows read
// as 16-byte runs), then turns to a lane per output dimension to accumulate, so no
// lane holds a whole gradient row.
#include "ham_common.h"
#include "ham_internal.h"

namespace ham {

namespace {

HAM_DEVICE int count_at_most(const int32_t* p, int n, long long x) {      // #{p[i] <= x}
  int l = 0, r = n;
  while (l < r) {
    const int m = (l + r) >> 1;
    if ((long long)p[m] <= x) l = m + 1; else r = m;
  }
  return l;
}

// dot product of row r of a [rows, D] tensor of the io type with x (in LDS), read as
// 4-element runs so that no lane holds the whole row
template <class IO, int D>
HAM_DEVICE float dot_row(const typename IO::elem* base, size_t r, const float* x) {
  float acc = 0.f;
#pragma unroll 8
  for (int i = 0; i < D; i += 4) {
    float v[4];
    IO::load4(base, r * D + i, v);
    acc = fmaf(v[0], x[i], acc);
    acc = fmaf(v[1], x[i + 1], acc);
    acc = fmaf(v[2], x[i + 2], acc);
    acc = fmaf(v[3], x[i + 3], acc);
  }
  return acc;
}

// the same for a float row
template <int D>
HAM_DEVICE float dot_row_f32(const float* base, size_t r, const float* x) {
  float acc = 0.f;
#pragma unroll 8
  for (int i = 0; i < D; i += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(base + r * D + i);
    acc = fmaf(v[0], x[i], acc);
    acc = fmaf(v[1], x[i + 1], acc);
    acc = fmaf(v[2], x[i + 2], acc);
    acc = fmaf(v[3], x[i + 3], acc);
  }
  return acc;
}

}  // namespace

// grid (T, H, B), 64 threads.
template <class IO, int DK, int DV>
__global__ __launch_bounds__(64) void attn_bwd_q_kernel(AttnBwdArgs a) {
  using E = typename IO::elem;
  constexpr int PK = DK / 64, PV = DV / 64;      // dimensions per lane
  __shared__ float s_q[DK], s_g[DV], s_w[64];
  const int lane = lane_id();
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.H + h;
  const size_t tok = ((size_t)b * a.T + t) * a.H + h;
  const int32_t* ph = a.pos + (size_t)bh * a.cap;
  const int cnt = a.count[bh];
  const int n = count_at_most(ph, cnt, (long long)a.t0 + t);
  const int lo = a.doc_start ? min(n, count_at_most(ph, cnt, (long long)a.doc_start[(size_t)b * a.T + t] - 1)) : 0;
  const E* q = static_cast<const E*>(a.q);
  const E* Kh = static_cast<const E*>(a.Kc) + (size_t)bh * a.cap * DK;
  const E* Vh = static_cast<const E*>(a.Vc) + (size_t)bh * a.cap * DV;
  for (int i = lane; i < DK; i += 64) s_q[i] = IO::load(q, tok * DK + i);
  for (int i = lane; i < DV; i += 64) s_g[i] = a.dO[tok * DV + i];
  __syncthreads();

  // pass 1: running maximum and sum of the scaled scores (lane per entry)
  float m = -INFINITY, l = 0.f;
  for (int c0 = lo; c0 < n; c0 += 64) {
    const int c = c0 + lane;
    float s = -INFINITY;
    if (c < n) s = a.scale * dot_row<IO, DK>(Kh, c, s_q);
    const float mn = fmaxf(m, wave_max<64>(s));
    l = l * expf(m - mn) + wave_sum<64>(s == -INFINITY ? 0.f : expf(s - mn));
    m = mn;
  }
  const float inv_l = l > 0.f ? 1.f / l : 0.f;

  // pass 2: D = sum_c p_c (g . v_c)
  float D = 0.f;
  for (int c0 = lo; c0 < n; c0 += 64) {
    const int c = c0 + lane;
    float x = 0.f;
    if (c < n)
      x = expf(a.scale * dot_row<IO, DK>(Kh, c, s_q) - m) * inv_l * dot_row<IO, DV>(Vh, c, s_g);
    D += wave_sum<64>(x);
  }

  // pass 3: dq = scale * sum_c p_c (g . v_c - D) k_c; the weights of 64 entries go
  // through LDS, then each lane accumulates its own dimensions
  float dq[PK];
#pragma unroll
  for (int i = 0; i < PK; ++i) dq[i] = 0.f;
  for (int c0 = lo; c0 < n; c0 += 64) {
    const int c = c0 + lane;
    float w = 0.f;
    if (c < n) {
      const float gv = dot_row<IO, DV>(Vh, c, s_g);
      w = a.scale * expf(a.scale * dot_row<IO, DK>(Kh, c, s_q) - m) * inv_l * (gv - D);
    }
    __syncthreads();
    s_w[lane] = w;
    __syncthreads();
    const int nc = min(64, n - c0);
    for (int j = 0; j < nc; ++j) {
      const float wj = s_w[j];
#pragma unroll
      for (int i = 0; i < PK; ++i) dq[i] = fmaf(wj, IO::load(Kh, (size_t)(c0 + j) * DK + lane * PK + i), dq[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < PK; ++i) a.dq[tok * DK + lane * PK + i] = dq[i];
  if (lane == 0) {
    a.stat[tok * 3 + 0] = m;
    a.stat[tok * 3 + 1] = inv_l;
    a.stat[tok * 3 + 2] = D;
  }
}

// grid (cap, H, B), 64 threads: entry c of head (b,h), for c < count.
template <class IO, int DK, int DV>
__global__ __launch_bounds__(64) void attn_bwd_kv_kernel(AttnBwdArgs a) {
  using E = typename IO::elem;
  constexpr int PK = DK / 64, PV = DV / 64;
  __shared__ float s_k[DK], s_v[DV], s_w[64], s_p[64];
  __shared__ int s_t[64];
  const int lane = lane_id();
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.H + h;
  const int cnt = a.count[bh];
  if (c >= cnt) return;                                    // whole workgroup
  const int32_t* ph = a.pos + (size_t)bh * a.cap;
  const E* q = static_cast<const E*>(a.q);
  const E* Kh = static_cast<const E*>(a.Kc) + (size_t)bh * a.cap * DK;
  const E* Vh = static_cast<const E*>(a.Vc) + (size_t)bh * a.cap * DV;
  for (int i = lane; i < DK; i += 64) s_k[i] = IO::load(Kh, (size_t)c * DK + i);
  for (int i = lane; i < DV; i += 64) s_v[i] = IO::load(Vh, (size_t)c * DV + i);
  __syncthreads();
  // the queries of this call that see the entry: positions >= its own (and, with
  // document masks, in a document that starts at or before it)
  const long long pc = ph[c];
  const int t_first = (int)max(0LL, min((long long)a.T, pc - (long long)a.t0));
  float dk[PK], dv[PV];
#pragma unroll
  for (int i = 0; i < PK; ++i) dk[i] = 0.f;
#pragma unroll
  for (int i = 0; i < PV; ++i) dv[i] = 0.f;
  for (int t0q = t_first; t0q < a.T; t0q += 64) {
    const int t = t0q + lane;
    float p = 0.f, w = 0.f;
    if (t < a.T && (!a.doc_start || (long long)a.doc_start[(size_t)b * a.T + t] <= pc)) {
      const size_t tok = ((size_t)b * a.T + t) * a.H + h;
      const float d = dot_row<IO, DK>(q, tok, s_k);
      const float gv = dot_row_f32<DV>(a.dO, tok, s_v);
      const float m = a.stat[tok * 3 + 0], inv_l = a.stat[tok * 3 + 1], D = a.stat[tok * 3 + 2];
      p = expf(a.scale * d - m) * inv_l;
      w = a.scale * p * (gv - D);
    }
    __syncthreads();
    s_p[lane] = p;
    s_w[lane] = w;
    s_t[lane] = t;
    __syncthreads();
    const int nt = min(64, a.T - t0q);
    for (int j = 0; j < nt; ++j) {
      const float pj = s_p[j], wj = s_w[j];
      if (pj == 0.f && wj == 0.f) continue;                 // uniform across the wave
      const size_t tok = ((size_t)b * a.T + s_t[j]) * a.H + h;
#pragma unroll
      for (int i = 0; i < PK; ++i) dk[i] = fmaf(wj, IO::load(q, tok * DK + lane * PK + i), dk[i]);
#pragma unroll
      for (int i = 0; i < PV; ++i) dv[i] = fmaf(pj, a.dO[tok * DV + lane * PV + i], dv[i]);
    }
  }
  const size_t row = (size_t)bh * a.cap + c;
#pragma unroll
  for (int i = 0; i < PK; ++i) a.dKc[row * DK + lane * PK + i] = dk[i];
#pragma unroll
  for (int i = 0; i < PV; ++i) a.dVc[row * DV + lane * PV + i] = dv[i];
}

template <class IO, int DK, int DV>
static hipError_t launch_bwd_t(const AttnBwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_bwd_q_kernel<IO, DK, DV>), dim3(a.T, a.H, a.B), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_kv_kernel<IO, DK, DV>), dim3(a.cap, a.H, a.B), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention_backward(int io, int dk, int dv, const AttnBwdArgs& a, hipStream_t s) {
#define HAM_CASE(IOT, DKV, DVV) \
  if (dk == DKV && dv == DVV) return launch_bwd_t<IOT, DKV, DVV>(a, s);
  if (io == 0) {
    HAM_CASE(IoF32, 64, 64) HAM_CASE(IoF32, 64, 128) HAM_CASE(IoF32, 128, 64) HAM_CASE(IoF32, 128, 128)
  } else {
    HAM_CASE(IoBF16, 64, 64) HAM_CASE(IoBF16, 64, 128) HAM_CASE(IoBF16, 128, 64) HAM_CASE(IoBF16, 128, 128)
  }
#undef HAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace ham
