// ham_rnn_bwd.hip -- gradients of the gated delta-rule RNN (training).
//
// "Hybrid Associative Memories" trains the layer end to end (App. A.1: the chunked
// kernel has a backward pass).  Per head, with alpha_t = exp(g_t):
//   p_t = S_{t-1}^T k_t,  r_t = v_t - alpha_t p_t,  S_t = alpha_t S_{t-1} + beta_t k_t r_t^T,
//   o_t = S_t^T q_t  (§2 DeltaNet update and linear-attention readout; App. A.1 decay).
// Reverse mode, with G = dL/dS_t carried from the last token back:
//   G += q_t dO_t^T;  u_t = G^T k_t;  dq_t = alpha_t S_{t-1} dO_t + beta_t (r_t . dO_t) k_t;
//   dv_t = beta_t u_t;  dbeta_t = u_t . r_t;  dk_t = beta_t (G r_t - alpha_t S_{t-1} u_t);
//   dg_t = alpha_t (<G, S_{t-1}> - beta_t u_t . p_t);  G <- alpha_t (G - beta_t k_t u_t^T).
// (dq_t = S_t dO_t with S_t written out through S_{t-1}.)  The routing threshold passes
// no gradient.
//
// One workgroup per (b, h), DV/16 waves; wave w owns the 16 state columns 16w ..,
// lane l the rows l + 64 m (m < DK/64), so a lane keeps DK/64 x 16 values each of
// S_{t-1} and G.  Column sums over the rows (p, u) are wave reductions; row vectors
// summed over the columns (dq, dk) and the scalars (dbeta, dg) are summed across the
// waves in LDS, double-buffered so one barrier per token suffices.  The states are
// needed in reverse order: a first pass runs the recurrence forward and stores the
// state at every 64-token chunk start; then, chunk by chunk from the end, the chunk's
// states are recomputed from its checkpoint into a per-wave scratch and the reverse
// recurrence walks back through them.  Each token's inputs (and, walking back, its
// stored state) are loaded while the previous token is processed, so a token waits on
// its arithmetic and the barrier rather than on memory.  fp32 throughout.
#include "ham_common.h"
#include "ham_internal.h"

namespace ham {
namespace rnnbwd {

constexpr int kC = 64;        // tokens per checkpointed chunk
constexpr int kCols = 16;     // state columns per wave

// Sum over the 64 lanes of x[j] for each of the 16 columns j; every lane receives all
// 16 sums (uniform values).
HAM_DEVICE void wave_colsum16(const float (&x)[kCols], float (&out)[kCols]) {
  const int n = lane_id() & 15;
  float y = row16_transpose_sum(x, n);        // lane n of each 16-lane row: sum of x[n] over the row
  y += __shfl_xor(y, 16, kWave);
  y += __shfl_xor(y, 32, kWave);              // every lane: the total for column n
#pragma unroll
  for (int j = 0; j < kCols; ++j)
    out[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, y), j));
}

template <int R>
struct Slab {                  // this lane's R rows x 16 columns of a state-shaped matrix
  float x[R][kCols];
};

// A slab in scratch: [4R float4][64 lanes] per state, so each float4 load is one
// contiguous 1 KiB access of the wave.
template <int R>
HAM_DEVICE void slab_store(float* base, const Slab<R>& s) {
  float4* p = reinterpret_cast<float4*>(base);
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int q = 0; q < kCols / 4; ++q)
      p[(m * (kCols / 4) + q) * kWave + lane_id()] =
          make_float4(s.x[m][4 * q], s.x[m][4 * q + 1], s.x[m][4 * q + 2], s.x[m][4 * q + 3]);
}
template <int R>
HAM_DEVICE void slab_load(const float* base, Slab<R>& s) {
  const float4* p = reinterpret_cast<const float4*>(base);
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int q = 0; q < kCols / 4; ++q) {
      const float4 v = p[(m * (kCols / 4) + q) * kWave + lane_id()];
      s.x[m][4 * q] = v.x; s.x[m][4 * q + 1] = v.y; s.x[m][4 * q + 2] = v.z; s.x[m][4 * q + 3] = v.w;
    }
}

template <class IO, int DK, int DV>
__global__ __launch_bounds__(64 * (DV / kCols)) void rnn_bwd_kernel(RnnBwdArgs a) {
  using E = typename IO::elem;
  constexpr int R = DK / 64;                  // rows per lane
  constexpr int NW = DV / kCols;              // waves
  constexpr int SLAB = R * kCols * kWave;     // floats per stored state slab
  __shared__ float s_part[2][NW][2][DK];      // per-wave row partials (dq, dk), two buffers
  __shared__ float s_scal[2][NW][4];          // per-wave (r.dO, u.r, u.p, <G,S>)
  __shared__ float s_k[2][DK];                // k_t (the dq term beta (r.dO) k)

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = blockIdx.x, b = blockIdx.y;
  const int bh = b * a.H + h;
  const int c0 = wave * kCols;                // first state column of this wave
  const int nchunk = (a.T + kC - 1) / kC;
  const E* __restrict__ qp = static_cast<const E*>(a.q);
  const E* __restrict__ kp = static_cast<const E*>(a.k);
  const E* __restrict__ vp = static_cast<const E*>(a.v);
  float* ck = a.ckpt + (size_t)(bh * NW + wave) * nchunk * SLAB;
  float* st = a.states + (size_t)(bh * NW + wave) * kC * SLAB;

  auto tok_of = [&](int t) { return ((size_t)b * a.T + t) * a.H + h; };
  // One token's inputs as loaded: this lane's rows of k_t and q_t, lane j < 16 holding
  // column j of the wave's v_t and dO_t (spread to every lane where they are used), g, beta.
  struct TokIn {
    float kr[R], qr[R], vx, dox, g, beta;
  };
  auto load_in = [&](int t, bool with_q) {
    TokIn in;
    const size_t tok = tok_of(t);
#pragma unroll
    for (int m = 0; m < R; ++m) {
      in.kr[m] = IO::load(kp, tok * DK + lane + 64 * m);
      in.qr[m] = with_q ? IO::load(qp, tok * DK + lane + 64 * m) : 0.f;
    }
    in.vx = lane < kCols ? IO::load(vp, tok * DV + c0 + lane) : 0.f;
    in.dox = (with_q && lane < kCols) ? a.dO[tok * DV + c0 + lane] : 0.f;
    in.g = a.g[tok];
    in.beta = a.beta[tok];
    return in;
  };
  auto spread = [&](float x, float (&out)[kCols]) {
#pragma unroll
    for (int j = 0; j < kCols; ++j)
      out[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), j));
  };
  // one forward step S <- alpha S + beta k (v - alpha S^T k)^T on the slab
  auto forward_step = [&](Slab<R>& S, const TokIn& in) {
    float vj[kCols], x[kCols], p[kCols];
    const float* kr = in.kr;
    spread(in.vx, vj);
    const float alpha = expf(in.g), beta = in.beta;
#pragma unroll
    for (int j = 0; j < kCols; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < R; ++m) acc = fmaf(S.x[m][j], kr[m], acc);
      x[j] = acc;
    }
    wave_colsum16(x, p);
#pragma unroll
    for (int j = 0; j < kCols; ++j) {
      const float w = beta * (vj[j] - alpha * p[j]);
#pragma unroll
      for (int m = 0; m < R; ++m) S.x[m][j] = fmaf(kr[m], w, alpha * S.x[m][j]);
    }
  };

  // ---- pass 1: forward, checkpoint at every chunk start ----
  Slab<R> S;
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int j = 0; j < kCols; ++j)
      S.x[m][j] = a.S0 ? a.S0[(size_t)bh * DK * DV + (size_t)(lane + 64 * m) * DV + c0 + j] : 0.f;
  {
    TokIn cur = load_in(0, false);
    for (int t = 0; t < a.T; ++t) {
      const TokIn nxt = load_in(t + 1 < a.T ? t + 1 : t, false);
      if (t % kC == 0) slab_store(ck + (size_t)(t / kC) * SLAB, S);
      forward_step(S, cur);
      cur = nxt;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);              // the checkpoints are in memory before they are read

  // ---- pass 2: chunks from the end; recompute the chunk's states, then walk back ----
  Slab<R> G;
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int j = 0; j < kCols; ++j)
      G.x[m][j] = a.dS_T ? a.dS_T[(size_t)bh * DK * DV + (size_t)(lane + 64 * m) * DV + c0 + j] : 0.f;
  const int nthr = 64 * NW;
  for (int c = nchunk - 1; c >= 0; --c) {
    const int t0 = c * kC, t1 = min(a.T, t0 + kC);
    slab_load(ck + (size_t)c * SLAB, S);
    {
      TokIn cur = load_in(t0, false);
      for (int t = t0; t < t1; ++t) {
        const TokIn nxt = load_in(t + 1 < t1 ? t + 1 : t, false);
        slab_store(st + (size_t)(t - t0) * SLAB, S);      // S_{t-1} of token t
        forward_step(S, cur);
        cur = nxt;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);            // the chunk's states are in memory before they are read
    Slab<R> Sn;                               // S_{t-1} of the next token walked (t - 1)
    slab_load(st + (size_t)(t1 - 1 - t0) * SLAB, Sn);
    TokIn nin = load_in(t1 - 1, true);
    for (int t = t1 - 1; t >= t0; --t) {
      const int buf = t & 1;
      const size_t tok = tok_of(t);
      S = Sn;                                 // S_{t-1}
      const TokIn in = nin;
      if (t > t0) {
        slab_load(st + (size_t)(t - 1 - t0) * SLAB, Sn);
        nin = load_in(t - 1, true);
      }
      const float* kr = in.kr;
      const float* qr = in.qr;
      float vj[kCols], dOj[kCols];
      spread(in.vx, vj);
      spread(in.dox, dOj);
      const float alpha = expf(in.g), beta = in.beta;
      // G += q dO^T  (G is now dL/dS_t)
#pragma unroll
      for (int m = 0; m < R; ++m)
#pragma unroll
        for (int j = 0; j < kCols; ++j) G.x[m][j] = fmaf(qr[m], dOj[j], G.x[m][j]);
      // p = S_{t-1}^T k, u = G^T k
      float xp[kCols], xu[kCols], p[kCols], u[kCols];
#pragma unroll
      for (int j = 0; j < kCols; ++j) {
        float ap = 0.f, au = 0.f;
#pragma unroll
        for (int m = 0; m < R; ++m) {
          ap = fmaf(S.x[m][j], kr[m], ap);
          au = fmaf(G.x[m][j], kr[m], au);
        }
        xp[j] = ap;
        xu[j] = au;
      }
      wave_colsum16(xp, p);
      wave_colsum16(xu, u);
      float rj[kCols], rdo = 0.f, ur = 0.f, up = 0.f;
#pragma unroll
      for (int j = 0; j < kCols; ++j) {
        rj[j] = vj[j] - alpha * p[j];
        rdo = fmaf(rj[j], dOj[j], rdo);
        ur = fmaf(u[j], rj[j], ur);
        up = fmaf(u[j], p[j], up);
      }
      // row partials over this wave's columns, and <G, S_{t-1}>
      float gs = 0.f;
#pragma unroll
      for (int m = 0; m < R; ++m) {
        float aq = 0.f, ak = 0.f;
#pragma unroll
        for (int j = 0; j < kCols; ++j) {
          aq = fmaf(S.x[m][j], dOj[j], aq);
          ak = fmaf(G.x[m][j], rj[j], ak);
          ak = fmaf(-alpha * S.x[m][j], u[j], ak);
          gs = fmaf(G.x[m][j], S.x[m][j], gs);
        }
        s_part[buf][wave][0][lane + 64 * m] = aq;
        s_part[buf][wave][1][lane + 64 * m] = ak;
        if (wave == 0) s_k[buf][lane + 64 * m] = kr[m];
      }
      gs = wave_sum<64>(gs);
      if (lane == 0) {
        s_scal[buf][wave][0] = rdo;
        s_scal[buf][wave][1] = ur;
        s_scal[buf][wave][2] = up;
        s_scal[buf][wave][3] = gs;
      }
      if (lane < kCols) a.dv[tok * DV + c0 + lane] = beta * u[lane];
      // G <- alpha (G - beta k u^T)   (dL/dS_{t-1})
#pragma unroll
      for (int m = 0; m < R; ++m)
#pragma unroll
        for (int j = 0; j < kCols; ++j) G.x[m][j] = alpha * fmaf(-beta * kr[m], u[j], G.x[m][j]);
      __syncthreads();
      // across the waves: dq, dk rows and the two scalars of token t
      float sr = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sr += s_scal[buf][w][0];
      for (int o = threadIdx.x; o < 2 * DK + 1; o += nthr) {
        if (o < 2 * DK) {
          const int which = o / DK, row = o % DK;
          float acc = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) acc += s_part[buf][w][which][row];
          if (which == 0) a.dq[tok * DK + row] = alpha * acc + beta * sr * s_k[buf][row];
          else a.dk[tok * DK + row] = beta * acc;
        } else {
          float ur_t = 0.f, up_t = 0.f, gs_t = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            ur_t += s_scal[buf][w][1];
            up_t += s_scal[buf][w][2];
            gs_t += s_scal[buf][w][3];
          }
          a.dbeta[tok] = ur_t;
          a.dg[tok] = alpha * (gs_t - beta * up_t);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < R; ++m)
#pragma unroll
    for (int j = 0; j < kCols; ++j) a.dS0[(size_t)bh * DK * DV + (size_t)(lane + 64 * m) * DV + c0 + j] = G.x[m][j];
}

template <class IO, int DK, int DV>
hipError_t launch_t(const RnnBwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((rnn_bwd_kernel<IO, DK, DV>), dim3(a.H, a.B), dim3(64 * (DV / kCols)), 0, s, a);
  return hipGetLastError();
}

}  // namespace rnnbwd

size_t rnn_backward_scratch_floats(int B, int H, int T, int dk, int dv) {
  const size_t nchunk = ((size_t)T + rnnbwd::kC - 1) / rnnbwd::kC;
  const size_t slab = (size_t)(dk / 64) * rnnbwd::kCols * kWave;
  const size_t waves = (size_t)B * H * (dv / rnnbwd::kCols);
  return waves * (nchunk + rnnbwd::kC) * slab;
}

bool rnn_backward_supported(int dk, int dv) { return (dk == 64 || dk == 128) && (dv == 64 || dv == 128); }

hipError_t launch_rnn_backward(int io, int dk, int dv, const RnnBwdArgs& a, hipStream_t s) {
#define HAM_CASE(IOT, DKV, DVV) \
  if (dk == DKV && dv == DVV) return rnnbwd::launch_t<IOT, DKV, DVV>(a, s);
  if (io == 0) {
    HAM_CASE(IoF32, 64, 64) HAM_CASE(IoF32, 64, 128) HAM_CASE(IoF32, 128, 64) HAM_CASE(IoF32, 128, 128)
  } else {
    HAM_CASE(IoBF16, 64, 64) HAM_CASE(IoBF16, 64, 128) HAM_CASE(IoBF16, 128, 64) HAM_CASE(IoBF16, 128, 128)
  }
#undef HAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace ham
