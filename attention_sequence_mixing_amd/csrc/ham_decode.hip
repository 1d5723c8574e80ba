// ham_decode.hip -- single-token attention over the compacted cache (split-K)
// and the combine + mix epilogue of the decode step.
//
// "Hybrid Associative Memories" App. A.1 "Generation": the recurrent state is
// carried and routed tokens accumulate in the KV cache; one new token attends to
// every cached entry (all are at earlier or equal original positions).  The
// readout is the §2 KV-memory softmax; the mix is the §2 headwise-norm gated sum.
//
// Memory-bound: each (b,h) cache is cut into segments of kDecodeSeg keys; one
// workgroup streams one segment with 16-byte loads (16 lanes per key row) and
// keeps a running max / sum / weighted value sum per 16-lane group.  A second
// kernel merges the segments with the usual log-sum-exp rescaling.
#include "ham_common.h"
#include "ham_internal.h"

namespace ham {

constexpr float kLog2eD = 1.4426950408889634f;

// Raw cache rows: a lane holds N consecutive elements of a row as loaded (bf16
// bit patterns or floats) and converts them when they are used.
template <class IO, int N>
struct RawRun;
// The cache rows are streamed once per step, so they are loaded non-temporally (the
// hint keeps them from displacing reused lines: decode attention 0.774 -> 0.673 ms at
// the decode workload, 5.57 -> 6.41 TB/s).
template <int N>
struct RawRun<IoBF16, N> {                    // 16-byte runs (8-byte when N = 4)
  static_assert(N % 4 == 0, "run length");
  static constexpr int W = N % 8 == 0 ? 8 : 4;
  typedef uint16_t vec __attribute__((ext_vector_type(W)));
  vec x[N / W];
  HAM_DEVICE void load(const uint16_t* p) {
#pragma unroll
    for (int i = 0; i < N / W; ++i) x[i] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(p + W * i));
  }
  HAM_DEVICE float operator[](int i) const { return bf16_to_f32(x[i / W][i % W]); }
};
template <int N>
struct RawRun<IoF32, N> {
  static_assert(N % 4 == 0, "16-byte runs");
  f32x4 x[N / 4];
  HAM_DEVICE void load(const float* p) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) x[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4 * i));
  }
  HAM_DEVICE float operator[](int i) const { return x[i >> 2][i & 3]; }
};

// grid (nseg, H, B), 256 threads: one workgroup streams one segment of a head's
// cache.  16 lane groups of 16 lanes; a lane group takes U keys per step (a lane
// holds d/16 elements of each row, 16-byte loads), forms their scores with a row
// reduction, and applies the U keys with one running-maximum update (blocked
// online softmax).  Keys past the end of the segment load the last valid row and
// get probability 0.
template <class IO, int DK, int DV>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeAttnArgs a) {
  using E = typename IO::elem;
  constexpr int KE = DK / 16, VE = DV / 16;   // elements per lane per row
  constexpr int U = 8;                        // keys per lane group per step
  __shared__ float s_m[16], s_l[16];
  __shared__ float s_acc[16][DV];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int grp = wave * 4 + (lane >> 4);     // 16 lane groups per workgroup
  const int sub = lane & 15;
  const int seg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.H + h;
  const int n = a.count[bh];
  if (seg * a.seg >= n) return;
  const int s1 = min(n, seg * a.seg + a.seg);
  // same-document masking: entries before lo belong to earlier documents
  const int s0 = a.lo ? max(seg * a.seg, a.lo[bh]) : seg * a.seg;
  if (s0 >= s1) {                             // nothing visible in this segment
    float* out = a.part + ((size_t)bh * a.nseg + seg) * (DV + 2);
    for (int d = threadIdx.x; d < DV; d += 256) out[d] = 0.f;
    if (threadIdx.x == 0) { out[DV] = -INFINITY; out[DV + 1] = 0.f; }
    return;
  }

  const E* qp = static_cast<const E*>(a.q) + (size_t)bh * DK + sub * KE;
  const E* Kh = static_cast<const E*>(a.Kc) + (size_t)bh * a.cap * DK + sub * KE;
  const E* Vh = static_cast<const E*>(a.Vc) + (size_t)bh * a.cap * DV + sub * VE;
  float qv[KE];
#pragma unroll
  for (int i = 0; i < KE; i += 4) IO::load4(qp, i, qv + i);
  if (a.rope) {
    // the new token's query turned at its absolute position (consecutive pairs)
    const float2* rrow = a.rope + (size_t)b * (DK / 2) + sub * (KE / 2);
#pragma unroll
    for (int j = 0; j < KE / 2; ++j) rope_pair(qv[2 * j], qv[2 * j + 1], rrow[j]);
  }
  const float sl2 = a.scale * kLog2eD;
#pragma unroll
  for (int i = 0; i < KE; ++i) qv[i] *= sl2;

  float m = -INFINITY, l = 0.f, acc[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) acc[i] = 0.f;

  for (int c = s0 + grp; c < s1; c += 16 * U) {
    RawRun<IO, KE> kx[U];
    RawRun<IO, VE> vx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int cc = min(c + 16 * u, s1 - 1);
      kx[u].load(Kh + (size_t)cc * DK);
      vx[u].load(Vh + (size_t)cc * DV);
    }
    float sc[U];
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < KE; ++i) s = fmaf(qv[i], kx[u][i], s);
      s = row16_sum(s);
      sc[u] = (c + 16 * u < s1) ? s : -INFINITY;
      bm = fmaxf(bm, sc[u]);
    }
    const float mn = fmaxf(m, bm);            // finite: key c is always valid
    const float corr = __builtin_amdgcn_exp2f(m - mn);
    l *= corr;
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] *= corr;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = __builtin_amdgcn_exp2f(sc[u] - mn);
      l += p;
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[i] = fmaf(p, vx[u][i], acc[i]);
    }
    m = mn;
  }
  // merge the 16 lane groups
  if (sub == 0) { s_m[grp] = m; s_l[grp] = l; }
#pragma unroll
  for (int i = 0; i < VE; ++i) s_acc[grp][sub * VE + i] = acc[i];
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int q = 0; q < 16; ++q) M = fmaxf(M, s_m[q]);
  float* out = a.part + ((size_t)bh * a.nseg + seg) * (DV + 2);
  for (int d = tid; d < DV; d += 256) {
    float x = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (s_m[q] != -INFINITY) x += s_acc[q][d] * exp2f(s_m[q] - M);
    out[d] = x;
  }
  if (tid == 0) {
    float L = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (s_m[q] != -INFINITY) L += s_l[q] * exp2f(s_m[q] - M);
    out[DV] = M;
    out[DV + 1] = L;
  }
}

template <class IO, int DK, int DV>
static hipError_t launch_dattn_t(const DecodeAttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_attn_kernel<IO, DK, DV>), dim3(a.nseg, a.H, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_attn(int io, int dk, int dv, const DecodeAttnArgs& a, hipStream_t s) {
#define HAM_CASE(IOT, DKV, DVV) \
  if (dk == DKV && dv == DVV) return launch_dattn_t<IOT, DKV, DVV>(a, s);
  if (io == 0) {
    HAM_CASE(IoF32, 64, 64) HAM_CASE(IoF32, 64, 128) HAM_CASE(IoF32, 128, 64) HAM_CASE(IoF32, 128, 128)
    HAM_CASE(IoF32, 128, 192)
  } else {
    HAM_CASE(IoBF16, 64, 64) HAM_CASE(IoBF16, 64, 128) HAM_CASE(IoBF16, 128, 64) HAM_CASE(IoBF16, 128, 128)
    HAM_CASE(IoBF16, 128, 192)
  }
#undef HAM_CASE
  return hipErrorInvalidValue;
}

// grid (H, B), one wave: merge the segments, then mix with the RNN readout.
template <class IO, int DV>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeCombineArgs a) {
  using E = typename IO::elem;
  constexpr int PL = DV / 64;                  // dims per lane
  const int lane = lane_id();
  const int h = blockIdx.x, b = blockIdx.y;
  const int bh = b * a.H + h;
  const int n = a.count[bh];
  const int used = (n + a.seg - 1) / a.seg;
  const float* part = a.part + (size_t)bh * a.nseg * (DV + 2);
  // segment maxima read by the lanes in parallel
  float M = -INFINITY;
  for (int s = lane; s < used; s += 64) M = fmaxf(M, part[(size_t)s * (DV + 2) + DV]);
  M = wave_max<64>(M);
  float L = 0.f, okv[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) okv[i] = 0.f;
#pragma unroll 4
  for (int s = 0; s < used; ++s) {
    const float* ps = part + (size_t)s * (DV + 2);
    const float w = (ps[DV] == -INFINITY) ? 0.f : exp2f(ps[DV] - M);
    L += ps[DV + 1] * w;
#pragma unroll
    for (int i = 0; i < PL; ++i) okv[i] += ps[lane * PL + i] * w;
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  if (a.okv32) {
    // KV heads of another geometry than the RNN's: the readout alone, mixed later
#pragma unroll
    for (int i = 0; i < PL; ++i) a.okv32[(size_t)bh * DV + lane * PL + i] = okv[i] * inv;
    return;
  }
  float orn[PL], ssr = 0.f, ssk = 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    okv[i] *= inv;
    orn[i] = a.o_rnn32[(size_t)bh * DV + lane * PL + i];
    ssr += orn[i] * orn[i];
    ssk += okv[i] * okv[i];
  }
  ssr = wave_sum<64>(ssr);
  ssk = wave_sum<64>(ssk);
  const float gr = a.gate_rnn ? a.gate_rnn[bh] : 1.f;
  const float gk = a.gate_kv ? a.gate_kv[bh] : 1.f;
  const float ir = gr / sqrtf(ssr / (float)DV + a.eps);
  const float ik = gk / sqrtf(ssk / (float)DV + a.eps);
  E* o = static_cast<E*>(a.o);
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const size_t off = (size_t)bh * DV + lane * PL + i;
    IO::store(o, off, orn[i] * ir + okv[i] * ik);
    if (a.o_kv) IO::store(static_cast<E*>(a.o_kv), off, okv[i]);
    if (a.o_rnn) IO::store(static_cast<E*>(a.o_rnn), off, orn[i]);
  }
}

hipError_t launch_decode_combine(int io, int dv, const DecodeCombineArgs& a, hipStream_t s) {
  dim3 grid(a.H, a.B);
  if (io == 0 && dv == 64) hipLaunchKernelGGL((decode_combine_kernel<IoF32, 64>), grid, dim3(64), 0, s, a);
  else if (io == 0 && dv == 128) hipLaunchKernelGGL((decode_combine_kernel<IoF32, 128>), grid, dim3(64), 0, s, a);
  else if (io == 1 && dv == 64) hipLaunchKernelGGL((decode_combine_kernel<IoBF16, 64>), grid, dim3(64), 0, s, a);
  else if (io == 1 && dv == 128) hipLaunchKernelGGL((decode_combine_kernel<IoBF16, 128>), grid, dim3(64), 0, s, a);
  else if (io == 0 && dv == 192) hipLaunchKernelGGL((decode_combine_kernel<IoF32, 192>), grid, dim3(64), 0, s, a);
  else if (io == 1 && dv == 192) hipLaunchKernelGGL((decode_combine_kernel<IoBF16, 192>), grid, dim3(64), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ham
