// ham_rnn_recurrent.hip -- token-serial gated delta-rule kernel.
//
// "Hybrid Associative Memories" §2 (DeltaNet update as one gradient step on
// 1/2|S k - v|^2; readout S_t^T q_t) with the gated-DeltaNet decay of App. A.1,
// and the fit-error score of §2 / App. A.1 ("Router Implementations").
//
// One wave owns a block of columns of the fp32 state S (dk x dv) of one head and
// walks the tokens in order.  The rows are split into RQ groups (2; 8 at dk = 256, so
// that a lane keeps 64 floats of state and a head spreads over twice as many waves):
// lane (rq, cp) = (lane / CPW, lane mod CPW) holds columns 2cp, 2cp+1 of the wave's
// 2*CPW columns (CPW = 64/RQ) for rows [rq*dk/RQ, (rq+1)*dk/RQ), so each row's
// columns are one contiguous run of float2 loads.  Columns of S evolve independently
// under S <- alpha (I - beta k k^T) S + beta k v^T, so waves need no communication;
// the routing score only needs three sums per token, written as partials per
// 16-column slice.  k_t and q_t are staged in LDS as floats each token (every lane
// reads them; the reads broadcast).  This is the decode-step kernel and the forward
// path for short sequences and fp32 I/O.
#include "ham_common.h"
#include "ham_internal.h"

namespace ham {

// row groups per wave and the resulting state columns per wave
template <int DK>
constexpr int rec_groups() { return DK > 128 ? 8 : 2; }
template <int DK>
constexpr int rec_cols() { return 128 / rec_groups<DK>(); }

template <class IO, int DK, int DV>
__global__ __launch_bounds__(64) void rnn_recurrent_kernel(RnnArgs a) {
  constexpr int RQ = rec_groups<DK>();     // row groups
  constexpr int CPW = 64 / RQ;             // column pairs per wave
  constexpr int kRecCols = 2 * CPW;        // state columns per wave
  static_assert(DV % kRecCols == 0, "whole column blocks");
  using E = typename IO::elem;
  constexpr int RH = DK / RQ;              // rows per lane
  constexpr int NS = DV / 16;              // score slices per head
  __shared__ float4 ks4[DK / 4], qs4[DK / 4];
  float* ks = reinterpret_cast<float*>(ks4);
  float* qs = reinterpret_cast<float*>(qs4);
  const int lane = lane_id();
  const int rh = lane / CPW, cp = lane % CPW;
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int j0 = blk * kRecCols + 2 * cp;  // this lane's first column
  const int bh = b * a.H + h;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);

  float2 S[RH];
  const size_t sbase = (size_t)bh * DK * DV + (size_t)(rh * RH) * DV + j0;
  if (a.S0) {
#pragma unroll
    for (int m = 0; m < RH; ++m) S[m] = *reinterpret_cast<const float2*>(a.S0 + sbase + (size_t)m * DV);
  } else {
#pragma unroll
    for (int m = 0; m < RH; ++m) S[m] = make_float2(0.f, 0.f);
  }

  const bool readout = a.o_rnn32 != nullptr;
  // The next token's inputs are loaded into registers while the current token is
  // processed, so the chain from one token to the next waits on LDS, not on memory.
  constexpr int KL = (DK + 63) / 64;       // key / query elements per lane
  float kn[KL], qn[KL], vn0 = 0.f, vn1 = 0.f, gn = 0.f, bn = 0.f;
  auto fetch = [&](int t) {
    const size_t tok = ((size_t)b * a.T + t) * a.H + h;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int e = lane + 64 * i;
      kn[i] = e < DK ? IO::load(k, tok * DK + e) : 0.f;
      qn[i] = (readout && e < DK) ? IO::load(q, tok * DK + e) : 0.f;
    }
    vn0 = IO::load(v, tok * DV + j0);
    vn1 = IO::load(v, tok * DV + j0 + 1);
    gn = a.g[tok];
    bn = a.beta[tok];
  };
  if (a.T > 0) fetch(0);
  for (int t = 0; t < a.T; ++t) {
    const size_t tok = ((size_t)b * a.T + t) * a.H + h;
    const float alpha = expf(gn);
    const float beta = bn;
#pragma unroll
    for (int i = 0; i < KL; ++i) {
      const int e = lane + 64 * i;
      if (e < DK) {
        ks[e] = kn[i];
        if (readout) qs[e] = qn[i];
      }
    }
    const float v0 = vn0, v1 = vn1;
    __syncthreads();
    if (t + 1 < a.T) fetch(t + 1);
    const float4* kr = ks4 + rh * (RH / 4);

    // prediction p_j = sum_i S[i][j] k_i   (S_{t-1}^T k_t), two chains per column
    float pa0 = 0.f, pa1 = 0.f, pb0 = 0.f, pb1 = 0.f;
#pragma unroll
    for (int m = 0; m < RH; m += 4) {
      const float4 kk = kr[m / 4];
      pa0 = fmaf(S[m].x, kk.x, pa0);     pa1 = fmaf(S[m].y, kk.x, pa1);
      pb0 = fmaf(S[m + 1].x, kk.y, pb0); pb1 = fmaf(S[m + 1].y, kk.y, pb1);
      pa0 = fmaf(S[m + 2].x, kk.z, pa0); pa1 = fmaf(S[m + 2].y, kk.z, pa1);
      pb0 = fmaf(S[m + 3].x, kk.w, pb0); pb1 = fmaf(S[m + 3].y, kk.w, pb1);
    }
    float p0 = pa0 + pb0, p1 = pa1 + pb1;
#pragma unroll
    for (int m = CPW; m < 64; m <<= 1) {   // the other row groups
      p0 += __shfl_xor(p0, m, kWave);
      p1 += __shfl_xor(p1, m, kWave);
    }

    // score partials over each 16-column slice (8 lanes of column pairs)
    float pv = p0 * v0 + p1 * v1, pp = p0 * p0 + p1 * p1, vv = v0 * v0 + v1 * v1;
#pragma unroll
    for (int msk = 1; msk < 8; msk <<= 1) {
      pv += __shfl_xor(pv, msk, kWave);
      pp += __shfl_xor(pp, msk, kWave);
      vv += __shfl_xor(vv, msk, kWave);
    }
    if (rh == 0 && (cp & 7) == 0)
      a.score[tok * NS + blk * (kRecCols / 16) + (cp >> 3)] = make_float4(pv, pp, vv, 0.f);

    // S <- alpha*S + k * beta*(v_j - alpha*p_j)
    const float w0 = beta * (v0 - alpha * p0), w1 = beta * (v1 - alpha * p1);
#pragma unroll
    for (int m = 0; m < RH; m += 4) {
      const float4 kk = kr[m / 4];
      S[m].x = fmaf(kk.x, w0, alpha * S[m].x);         S[m].y = fmaf(kk.x, w1, alpha * S[m].y);
      S[m + 1].x = fmaf(kk.y, w0, alpha * S[m + 1].x); S[m + 1].y = fmaf(kk.y, w1, alpha * S[m + 1].y);
      S[m + 2].x = fmaf(kk.z, w0, alpha * S[m + 2].x); S[m + 2].y = fmaf(kk.z, w1, alpha * S[m + 2].y);
      S[m + 3].x = fmaf(kk.w, w0, alpha * S[m + 3].x); S[m + 3].y = fmaf(kk.w, w1, alpha * S[m + 3].y);
    }

    if (readout) {
      const float4* qr = qs4 + rh * (RH / 4);
      float oa0 = 0.f, oa1 = 0.f, ob0 = 0.f, ob1 = 0.f;
#pragma unroll
      for (int m = 0; m < RH; m += 4) {
        const float4 qq = qr[m / 4];
        oa0 = fmaf(S[m].x, qq.x, oa0);     oa1 = fmaf(S[m].y, qq.x, oa1);
        ob0 = fmaf(S[m + 1].x, qq.y, ob0); ob1 = fmaf(S[m + 1].y, qq.y, ob1);
        oa0 = fmaf(S[m + 2].x, qq.z, oa0); oa1 = fmaf(S[m + 2].y, qq.z, oa1);
        ob0 = fmaf(S[m + 3].x, qq.w, ob0); ob1 = fmaf(S[m + 3].y, qq.w, ob1);
      }
      float o0 = oa0 + ob0, o1 = oa1 + ob1;
#pragma unroll
      for (int m = CPW; m < 64; m <<= 1) {
        o0 += __shfl_xor(o0, m, kWave);
        o1 += __shfl_xor(o1, m, kWave);
      }
      if (rh == 0) *reinterpret_cast<float2*>(a.o_rnn32 + tok * DV + j0) = make_float2(o0, o1);
    }
    __syncthreads();                       // k, q of the next token overwrite LDS
  }
#pragma unroll
  for (int m = 0; m < RH; ++m) *reinterpret_cast<float2*>(a.S_out + sbase + (size_t)m * DV) = S[m];
}

int rnn_recurrent_slices(int dv) { return dv / 16; }

template <class IO, int DK, int DV>
static hipError_t launch_t(const RnnArgs& a, hipStream_t s) {
  dim3 grid(DV / rec_cols<DK>(), a.H, a.B);
  hipLaunchKernelGGL((rnn_recurrent_kernel<IO, DK, DV>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rnn_recurrent(int io, int dk, int dv, const RnnArgs& a, hipStream_t s) {
#define HAM_CASE(IOT, DKV, DVV) \
  if (dk == DKV && dv == DVV) return launch_t<IOT, DKV, DVV>(a, s);
  if (io == 0) {
    HAM_CASE(IoF32, 64, 64) HAM_CASE(IoF32, 64, 128) HAM_CASE(IoF32, 128, 64) HAM_CASE(IoF32, 128, 128)
    HAM_CASE(IoF32, 256, 384)
  } else {
    HAM_CASE(IoBF16, 64, 64) HAM_CASE(IoBF16, 64, 128) HAM_CASE(IoBF16, 128, 64) HAM_CASE(IoBF16, 128, 128)
    HAM_CASE(IoBF16, 256, 384)
  }
#undef HAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace ham
