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
// (one wave per eight queries) forms the row statistics (m, l, D) and dq; the entry kernel
// (one wave per eight cache entries) walks the queries that see them and forms dk, dv.
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

// grid (ceil(T/QB), H, B), 64 threads: QB consecutive queries of one head share each
// cache row they read (lane per entry for the dot products, lane per dimension for dq).
template <class IO, int DK, int DV, int QB>
__global__ __launch_bounds__(64) void attn_bwd_q_kernel(AttnBwdArgs a) {
  using E = typename IO::elem;
  constexpr int PK = DK / 64;                    // dimensions per lane
  __shared__ float s_q[QB][DK], s_g[QB][DV], s_w[QB][64];
  const int lane = lane_id();
  const int tb = blockIdx.x * QB, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.H + h;
  const int32_t* ph = a.pos + (size_t)bh * a.cap;
  const int cnt = a.count[bh];
  const E* q = static_cast<const E*>(a.q);
  const E* Kh = static_cast<const E*>(a.Kc) + (size_t)bh * a.cap * DK;
  const E* Vh = static_cast<const E*>(a.Vc) + (size_t)bh * a.cap * DV;
  int n[QB], lo[QB];
  int cmin = 0x7fffffff, cmax = 0;
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int t = tb + j;
    n[j] = t < a.T ? count_at_most(ph, cnt, (long long)a.t0 + t) : 0;
    lo[j] = (t < a.T && a.doc_start)
                ? min(n[j], count_at_most(ph, cnt, (long long)a.doc_start[(size_t)b * a.T + t] - 1)) : 0;
    if (n[j] > lo[j]) { cmin = min(cmin, lo[j]); cmax = max(cmax, n[j]); }
    const size_t tok = ((size_t)b * a.T + min(t, a.T - 1)) * a.H + h;
    for (int i = lane; i < DK; i += 64) s_q[j][i] = t < a.T ? IO::load(q, tok * DK + i) : 0.f;
    for (int i = lane; i < DV; i += 64) s_g[j][i] = t < a.T ? a.dO[tok * DV + i] : 0.f;
  }
  if (cmax == 0) cmin = 0;
  __syncthreads();

  // the QB scores (and, with g, the QB value products) of entry c
  auto scores = [&](int c, float (&sc)[QB], float (&gv)[QB], bool with_v) {
#pragma unroll
    for (int j = 0; j < QB; ++j) { sc[j] = 0.f; gv[j] = 0.f; }
#pragma unroll 4
    for (int i = 0; i < DK; i += 4) {
      float v[4];
      IO::load4(Kh, (size_t)c * DK + i, v);
#pragma unroll
      for (int j = 0; j < QB; ++j)
        sc[j] = fmaf(v[0], s_q[j][i], fmaf(v[1], s_q[j][i + 1], fmaf(v[2], s_q[j][i + 2], fmaf(v[3], s_q[j][i + 3], sc[j]))));
    }
    if (with_v) {
#pragma unroll 4
      for (int i = 0; i < DV; i += 4) {
        float v[4];
        IO::load4(Vh, (size_t)c * DV + i, v);
#pragma unroll
        for (int j = 0; j < QB; ++j)
          gv[j] = fmaf(v[0], s_g[j][i], fmaf(v[1], s_g[j][i + 1], fmaf(v[2], s_g[j][i + 2], fmaf(v[3], s_g[j][i + 3], gv[j]))));
      }
    }
  };

  // pass 1: running maximum and sum of each query's scaled scores
  float m[QB], l[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) { m[j] = -INFINITY; l[j] = 0.f; }
  for (int c0 = cmin; c0 < cmax; c0 += 64) {
    const int c = c0 + lane;
    float sc[QB], gv[QB];
    if (c < cmax) scores(c, sc, gv, false);
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const float s = (c >= lo[j] && c < n[j]) ? a.scale * sc[j] : -INFINITY;
      const float mn = fmaxf(m[j], wave_max<64>(s));
      if (mn == -INFINITY) continue;                       // nothing visible yet (uniform)
      l[j] = l[j] * expf(m[j] - mn) + wave_sum<64>(s == -INFINITY ? 0.f : expf(s - mn));
      m[j] = mn;
    }
  }
  float inv_l[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) inv_l[j] = l[j] > 0.f ? 1.f / l[j] : 0.f;

  // pass 2: D = sum_c p_c (g . v_c)
  float D[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) D[j] = 0.f;
  for (int c0 = cmin; c0 < cmax; c0 += 64) {
    const int c = c0 + lane;
    float sc[QB], gv[QB];
    if (c < cmax) scores(c, sc, gv, true);
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const float x = (c >= lo[j] && c < n[j]) ? expf(a.scale * sc[j] - m[j]) * inv_l[j] * gv[j] : 0.f;
      D[j] += wave_sum<64>(x);
    }
  }

  // pass 3: dq = scale * sum_c p_c (g . v_c - D) k_c; the weights of 64 entries go
  // through LDS, then each lane accumulates its own dimensions for all QB queries
  float dq[QB][PK];
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int i = 0; i < PK; ++i) dq[j][i] = 0.f;
  for (int c0 = cmin; c0 < cmax; c0 += 64) {
    const int c = c0 + lane;
    float sc[QB], gv[QB];
    if (c < cmax) scores(c, sc, gv, true);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < QB; ++j)
      s_w[j][lane] = (c >= lo[j] && c < n[j])
                         ? a.scale * expf(a.scale * sc[j] - m[j]) * inv_l[j] * (gv[j] - D[j]) : 0.f;
    __syncthreads();
    const int nc = min(64, cmax - c0);
    for (int e = 0; e < nc; ++e) {
      float kd[PK];
#pragma unroll
      for (int i = 0; i < PK; ++i) kd[i] = IO::load(Kh, (size_t)(c0 + e) * DK + lane * PK + i);
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        const float wj = s_w[j][e];
#pragma unroll
        for (int i = 0; i < PK; ++i) dq[j][i] = fmaf(wj, kd[i], dq[j][i]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int t = tb + j;
    if (t >= a.T) continue;
    const size_t tok = ((size_t)b * a.T + t) * a.H + h;
#pragma unroll
    for (int i = 0; i < PK; ++i) a.dq[tok * DK + lane * PK + i] = dq[j][i];
    if (lane == 0) {
      a.stat[tok * 3 + 0] = m[j];
      a.stat[tok * 3 + 1] = inv_l[j];
      a.stat[tok * 3 + 2] = D[j];
    }
  }
}

// grid (ceil(cap/EB), H, B), 64 threads: EB consecutive entries of one head (those
// below count) share each query row they read.
template <class IO, int DK, int DV, int EB>
__global__ __launch_bounds__(64) void attn_bwd_kv_kernel(AttnBwdArgs a) {
  using E = typename IO::elem;
  constexpr int PK = DK / 64, PV = DV / 64;
  __shared__ float s_k[EB][DK], s_v[EB][DV], s_w[EB][64], s_p[EB][64];
  __shared__ int s_t[64];
  const int lane = lane_id();
  const int cb = blockIdx.x * EB, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.H + h;
  const int cnt = a.count[bh];
  if (cb >= cnt) return;                                   // whole workgroup
  const int32_t* ph = a.pos + (size_t)bh * a.cap;
  const E* q = static_cast<const E*>(a.q);
  const E* Kh = static_cast<const E*>(a.Kc) + (size_t)bh * a.cap * DK;
  const E* Vh = static_cast<const E*>(a.Vc) + (size_t)bh * a.cap * DV;
  long long pc[EB];
  int t_first = a.T;
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    const int c = cb + e;
    const bool ok = c < cnt;
    pc[e] = ok ? (long long)ph[c] : (1LL << 62);           // a missing entry is seen by no query
    if (ok) t_first = min(t_first, (int)max(0LL, min((long long)a.T, pc[e] - (long long)a.t0)));
    for (int i = lane; i < DK; i += 64) s_k[e][i] = ok ? IO::load(Kh, (size_t)c * DK + i) : 0.f;
    for (int i = lane; i < DV; i += 64) s_v[e][i] = ok ? IO::load(Vh, (size_t)c * DV + i) : 0.f;
  }
  __syncthreads();
  float dk[EB][PK], dv[EB][PV];
#pragma unroll
  for (int e = 0; e < EB; ++e) {
#pragma unroll
    for (int i = 0; i < PK; ++i) dk[e][i] = 0.f;
#pragma unroll
    for (int i = 0; i < PV; ++i) dv[e][i] = 0.f;
  }
  for (int t0q = t_first; t0q < a.T; t0q += 64) {
    const int t = t0q + lane;
    float p[EB], w[EB];
#pragma unroll
    for (int e = 0; e < EB; ++e) { p[e] = 0.f; w[e] = 0.f; }
    if (t < a.T) {
      // query t sees entry e when the entry's position is <= t0 + t and (document
      // masks) >= the start of t's document
      const long long pt = (long long)a.t0 + t;
      const long long ds = a.doc_start ? (long long)a.doc_start[(size_t)b * a.T + t] : -(1LL << 62);
      const size_t tok = ((size_t)b * a.T + t) * a.H + h;
      float d[EB], gv[EB];
#pragma unroll
      for (int e = 0; e < EB; ++e) { d[e] = 0.f; gv[e] = 0.f; }
#pragma unroll 4
      for (int i = 0; i < DK; i += 4) {
        float x[4];
        IO::load4(q, tok * DK + i, x);
#pragma unroll
        for (int e = 0; e < EB; ++e)
          d[e] = fmaf(x[0], s_k[e][i], fmaf(x[1], s_k[e][i + 1], fmaf(x[2], s_k[e][i + 2], fmaf(x[3], s_k[e][i + 3], d[e]))));
      }
#pragma unroll 4
      for (int i = 0; i < DV; i += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(a.dO + tok * DV + i);
#pragma unroll
        for (int e = 0; e < EB; ++e)
          gv[e] = fmaf(x[0], s_v[e][i], fmaf(x[1], s_v[e][i + 1], fmaf(x[2], s_v[e][i + 2], fmaf(x[3], s_v[e][i + 3], gv[e]))));
      }
      const float m = a.stat[tok * 3 + 0], inv_l = a.stat[tok * 3 + 1], D = a.stat[tok * 3 + 2];
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        if (pc[e] <= pt && pc[e] >= ds) {
          p[e] = expf(a.scale * d[e] - m) * inv_l;
          w[e] = a.scale * p[e] * (gv[e] - D);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EB; ++e) { s_p[e][lane] = p[e]; s_w[e][lane] = w[e]; }
    s_t[lane] = t;
    __syncthreads();
    const int nt = min(64, a.T - t0q);
    for (int j = 0; j < nt; ++j) {
      const size_t tok = ((size_t)b * a.T + s_t[j]) * a.H + h;
      float qd[PK], gd[PV];
#pragma unroll
      for (int i = 0; i < PK; ++i) qd[i] = IO::load(q, tok * DK + lane * PK + i);
#pragma unroll
      for (int i = 0; i < PV; ++i) gd[i] = a.dO[tok * DV + lane * PV + i];
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        const float pj = s_p[e][j], wj = s_w[e][j];
#pragma unroll
        for (int i = 0; i < PK; ++i) dk[e][i] = fmaf(wj, qd[i], dk[e][i]);
#pragma unroll
        for (int i = 0; i < PV; ++i) dv[e][i] = fmaf(pj, gd[i], dv[e][i]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    const int c = cb + e;
    if (c >= cnt) continue;
    const size_t row = (size_t)bh * a.cap + c;
#pragma unroll
    for (int i = 0; i < PK; ++i) a.dKc[row * DK + lane * PK + i] = dk[e][i];
#pragma unroll
    for (int i = 0; i < PV; ++i) a.dVc[row * DV + lane * PV + i] = dv[e][i];
  }
}

template <class IO, int DK, int DV>
static hipError_t launch_bwd_t(const AttnBwdArgs& a, hipStream_t s) {
  constexpr int QB = 8;
  hipLaunchKernelGGL((attn_bwd_q_kernel<IO, DK, DV, QB>), dim3((a.T + QB - 1) / QB, a.H, a.B), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int EB = 8;
  hipLaunchKernelGGL((attn_bwd_kv_kernel<IO, DK, DV, EB>), dim3((a.cap + EB - 1) / EB, a.H, a.B), dim3(64), 0,
                     s, a);
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
