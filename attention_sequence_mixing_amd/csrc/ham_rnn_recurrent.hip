// ham_rnn_recurrent.hip -- token-serial gated delta-rule kernel.
//
// "Hybrid Associative Memories" §2 (DeltaNet update as one gradient step on
// 1/2|S k - v|^2; readout S_t^T q_t) with the gated-DeltaNet decay of App. A.1,
// and the fit-error score of §2 / App. A.1 ("Router Implementations").
//
// One wave owns a 16-column slice of the fp32 state S (dk x dv) of one head and
// walks the tokens in order.  Lane = 4*c + r: column j0+c, rows [r*dk/4, (r+1)*dk/4).
// Columns of S evolve independently under S <- alpha (I - beta k k^T) S + beta k v^T,
// so slices need no communication; the routing score only needs three sums per
// token, written per slice as partials.  This is the decode-step kernel and the
// forward path for short sequences.
#include "ham_common.h"
#include "ham_internal.h"

namespace ham {

template <class IO, int DK, int DV>
__global__ __launch_bounds__(64) void rnn_recurrent_kernel(RnnArgs a) {
  using E = typename IO::elem;
  constexpr int RPL = DK / 4;             // rows per lane
  constexpr int NS = DV / 16;             // slices per head
  const int lane = lane_id();
  const int c = lane >> 2, r = lane & 3;
  const int slice = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int j = slice * 16 + c;
  const int bh = b * a.H + h;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);

  float S[RPL];
  const size_t sbase = (size_t)bh * DK * DV;
  if (a.S0) {
#pragma unroll
    for (int m = 0; m < RPL; ++m) S[m] = a.S0[sbase + (size_t)(r * RPL + m) * DV + j];
  } else {
#pragma unroll
    for (int m = 0; m < RPL; ++m) S[m] = 0.f;
  }

  const bool readout = a.o_rnn32 != nullptr;
  for (int t = 0; t < a.T; ++t) {
    const size_t tok = ((size_t)b * a.T + t) * a.H + h;
    const float alpha = expf(a.g[tok]);
    const float beta = a.beta[tok];
    float kr[RPL];
#pragma unroll
    for (int m = 0; m < RPL; m += 4) IO::load4(k, tok * DK + r * RPL + m, kr + m);
    const float vj = IO::load(v, tok * DV + j);

    // prediction p_j = sum_i S[i][j] k_i   (S_{t-1}^T k_t)
    float p = 0.f;
#pragma unroll
    for (int m = 0; m < RPL; ++m) p = fmaf(S[m], kr[m], p);
    p = wave_sum<4>(p);

    // score partials over this slice's 16 columns (lanes of one column agree)
    float pv = p * vj, pp = p * p, vv = vj * vj;
#pragma unroll
    for (int msk = 4; msk < 64; msk <<= 1) {
      pv += __shfl_xor(pv, msk, kWave);
      pp += __shfl_xor(pp, msk, kWave);
      vv += __shfl_xor(vv, msk, kWave);
    }
    if (lane == 0) a.score[tok * NS + slice] = make_float4(pv, pp, vv, 0.f);

    // S <- alpha*S + k * beta*(v_j - alpha*p_j)
    const float w = beta * (vj - alpha * p);
#pragma unroll
    for (int m = 0; m < RPL; ++m) S[m] = fmaf(kr[m], w, alpha * S[m]);

    if (readout) {
      float qr[RPL];
#pragma unroll
      for (int m = 0; m < RPL; m += 4) IO::load4(q, tok * DK + r * RPL + m, qr + m);
      float o = 0.f;
#pragma unroll
      for (int m = 0; m < RPL; ++m) o = fmaf(S[m], qr[m], o);
      o = wave_sum<4>(o);
      if (r == 0) a.o_rnn32[tok * DV + j] = o;
    }
  }
#pragma unroll
  for (int m = 0; m < RPL; ++m) a.S_out[sbase + (size_t)(r * RPL + m) * DV + j] = S[m];
}

int rnn_recurrent_slices(int dv) { return dv / 16; }

template <class IO, int DK, int DV>
static hipError_t launch_t(const RnnArgs& a, hipStream_t s) {
  dim3 grid(DV / 16, a.H, a.B);
  hipLaunchKernelGGL((rnn_recurrent_kernel<IO, DK, DV>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rnn_recurrent(int io, int dk, int dv, const RnnArgs& a, hipStream_t s) {
#define HAM_CASE(IOT, DKV, DVV) \
  if (dk == DKV && dv == DVV) return launch_t<IOT, DKV, DVV>(a, s);
  if (io == 0) {
    HAM_CASE(IoF32, 64, 64) HAM_CASE(IoF32, 64, 128) HAM_CASE(IoF32, 128, 64) HAM_CASE(IoF32, 128, 128)
  } else {
    HAM_CASE(IoBF16, 64, 64) HAM_CASE(IoBF16, 64, 128) HAM_CASE(IoBF16, 128, 64) HAM_CASE(IoBF16, 128, 128)
  }
#undef HAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace ham
