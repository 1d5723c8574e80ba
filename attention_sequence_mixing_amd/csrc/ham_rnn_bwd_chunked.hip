// ham_rnn_bwd_chunked.hip -- chunked gradients of the gated delta-rule RNN (training).
//
// "Hybrid Associative Memories" App. A.1: the chunked kernel of the RNN memory serves
// the backward pass as well.  Per head, the forward recurrence (§2 DeltaNet update and
// linear-attention readout, App. A.1 gated decay) over one 64-token chunk with entering
// state S, cumulative log decay G_t inside the chunk, gamma_t = e^{G_t},
// gamma_C = e^{G_last}, w_t = e^{G_last - G_t}, Gamma_ts = e^{G_t - G_s}, reads
//   X = V - diag(gamma) K S,   (I + diag(beta) A) D = diag(beta) X,
//   S_C = gamma_C S + K^T diag(w) D,   O = diag(gamma) Q S + M D,
// with A = strict_lower(Gamma o K K^T) and M = lower(Gamma o Q K^T) (diagonal kept):
// the residual form of the UT transform that the forward state pass also uses.  Its
// reverse mode, given dO and dS_C = dL/dS_C, is
//   dD = M^T dO + diag(w) K dS_C,   dX = T'^T dD  (T' = (I + diag(beta) A)^-1 diag(beta)),
//   U = dD - A^T dX,   R = X - A D,   dV = dX,   dbeta_t = U_t . R_t,
//   dS = gamma_C dS_C - K^T diag(gamma) dX + Q^T diag(gamma) dO      (entering state),
//   dM = lower(dO D^T),   dA = -strict_lower(dX D^T),
//   dQ = diag(gamma) dO S^T + (dM o Gamma) K,
//   dK = -diag(gamma) dX S^T + diag(w) D dS_C^T + (dM o Gamma)^T Q + (dA o Gamma) K
//        + (dA o Gamma)^T K,
//   dG_t = gamma_t sum_j (dO o QS - dX o KS)_tj - w_t sum_j (K dS_C o D)_tj
//          + sum_s (dM o M + dA o A)_ts - sum_s (dM o M + dA o A)_st,
//   and the chunk's last token's G also takes gamma_C <S, dS_C> + sum_t w_t (K dS_C o D)_t;
//   dg_j = sum_{t >= j} dG_t  (G is the running sum of g inside the chunk).
// Chunks beyond the sequence's end are padded with zero rows, beta = g = 0, which leaves
// every quantity of the real tokens unchanged.
//
// Five kernels, fp32 throughout (products on the fp32 matrix cores, 16x16x4):
//   cbwd_prep   chunk-parallel: G, A, M, T' per chunk (T' by forward substitution);
//   cbwd_fwd    sequential over chunks: the entering state of every chunk and D;
//   cbwd_rev    sequential over chunks, from the end: dS_C of every chunk and dS0, and
//               each chunk's K dS_C, dD and dX = dV;
//   cbwd_cols   chunk-parallel, 16 value columns per wave: the per-token partial sums
//               of dbeta, dgamma, dw over those columns;
//   cbwd_final  chunk-parallel: dM, dA, dQ, dK, dG, dg, dbeta.
// The state chains keep S (or dS) in matrix-core accumulators, 16 value columns per
// wave; a product whose contraction index is held by an accumulator takes it in the
// accumulator's own order (row 16i + 4(lane/16) + r in element r of tile i), and its
// other operand is read from LDS in that order.
#include "ham_common.h"
#include "ham_internal.h"

namespace ham {
namespace cbwd {

constexpr int kC = 64;          // tokens per chunk
constexpr int LP = 4;           // LDS row padding (floats)
constexpr int RW = kC + LP;     // LDS row length of a 64-wide matrix

HAM_DEVICE f32x4 mf(float a, float b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }

// Scratch regions (floats), each 64-float aligned; see chunk_scratch_floats().
struct Scratch {
  size_t G, A, M, T, S, dS, D, dX, dD, KdS, part, total;
};
__host__ __device__ inline Scratch scratch_layout(int B, int H, int T, int DK, int DV) {
  auto up = [](size_t x) { return (x + 63) / 64 * 64; };
  const size_t N = (size_t)(T + kC - 1) / kC, BHN = (size_t)B * H * N;
  Scratch s{};
  size_t o = 0;
  s.G = o;    o += up(BHN * kC);
  s.A = o;    o += up(BHN * kC * kC);
  s.M = o;    o += up(BHN * kC * kC);
  s.T = o;    o += up(BHN * kC * kC);
  s.S = o;    o += up(BHN * DK * DV);
  s.dS = o;   o += up(BHN * DK * DV);
  s.D = o;    o += up(BHN * kC * DV);
  s.dX = o;   o += up(BHN * kC * DV);
  s.dD = o;   o += up(BHN * kC * DV);
  s.KdS = o;  o += up(BHN * kC * DV);
  s.part = o; o += up(BHN * (DV / 16) * 4 * kC);
  s.total = o;
  return s;
}

struct Ctx {                    // per-workgroup indices of a (b, h, chunk)
  int b, h, bh, c, N, t0, Cc;
};
HAM_DEVICE Ctx ctx(const RnnBwdArgs& a, int bh, int c) {
  Ctx x;
  x.bh = bh; x.b = bh / a.H; x.h = bh % a.H; x.c = c;
  x.N = (a.T + kC - 1) / kC;
  x.t0 = c * kC;
  x.Cc = min(kC, a.T - x.t0);
  return x;
}

// rows t < Cc of a [B,T,H,D] tensor (columns col0 .. col0 + W - 1) into LDS [64][W + LP]
// as floats; padded rows are zero
template <class IO, int D, int W>
HAM_DEVICE void load_rows(float* dst, const void* src, const RnnBwdArgs& a, const Ctx& x, int col0) {
  using E = typename IO::elem;
  const E* p = static_cast<const E*>(src);
  for (int i = threadIdx.x; i < kC * W / 4; i += blockDim.x) {
    const int t = i / (W / 4), c4 = (i % (W / 4)) * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (t < x.Cc) IO::load4(p, (((size_t)x.b * a.T + x.t0 + t) * a.H + x.h) * D + col0 + c4, v);
    float* q = dst + t * (W + LP) + c4;
    q[0] = v[0]; q[1] = v[1]; q[2] = v[2]; q[3] = v[3];
  }
}
// a [64][64] fp32 matrix of the chunk from scratch into LDS [64][RW]
HAM_DEVICE void load_mat(float* dst, const float* src) {
  for (int i = threadIdx.x; i < kC * kC / 4; i += blockDim.x) {
    const int t = i / (kC / 4), c4 = (i % (kC / 4)) * 4;
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + t * kC + c4);
    float* q = dst + t * RW + c4;
    q[0] = v[0]; q[1] = v[1]; q[2] = v[2]; q[3] = v[3];
  }
}
// columns col0 .. col0 + W - 1 of R rows with row length LD (scratch) into LDS [R][W + LP]
template <int R, int W>
HAM_DEVICE void load_block(float* dst, const float* src, int LD, int col0) {
  for (int i = threadIdx.x; i < R * W / 4; i += blockDim.x) {
    const int t = i / (W / 4), c4 = (i % (W / 4)) * 4;
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + (size_t)t * LD + col0 + c4);
    float* q = dst + t * (W + LP) + c4;
    q[0] = v[0]; q[1] = v[1]; q[2] = v[2]; q[3] = v[3];
  }
}

// One thread's share (16-byte pieces) of a chunk's rows [64][W] of a [B,T,H,D] tensor
// (columns col0 .., padded rows zero), held in registers from the moment the loads
// are issued until they are written to LDS as floats [64][W + LP]: the state chains
// fetch the next chunk's inputs while the current chunk computes.
template <class IO, int D, int W>
struct RowsPre {
  static constexpr int EPP = 16 / IO::kBytes, PPR = W / EPP, NP = kC * PPR / 256;
  static_assert(kC * PPR % 256 == 0, "whole pieces per thread");
  uint4 x[NP];
  HAM_DEVICE void load(const void* src, const RnnBwdArgs& a, const Ctx& c, int col0) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int p = threadIdx.x + 256 * j, t = p / PPR, e0 = (p % PPR) * EPP;
      x[j] = t < c.Cc ? *reinterpret_cast<const uint4*>(static_cast<const char*>(src) +
                        ((((size_t)c.b * a.T + c.t0 + t) * a.H + c.h) * D + col0 + e0) * IO::kBytes)
                      : make_uint4(0, 0, 0, 0);
    }
  }
  HAM_DEVICE void store(float* dst) const {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int p = threadIdx.x + 256 * j, t = p / PPR, e0 = (p % PPR) * EPP;
      float* q = dst + t * (W + LP) + e0;
      const uint32_t w[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
      if constexpr (IO::kBytes == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          q[2 * i] = __uint_as_float(w[i] << 16);
          q[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = __uint_as_float(w[i]);
      }
    }
  }
};
// the same for a [64][64] fp32 matrix of the chunk in scratch
struct MatPre {
  static constexpr int NP = kC * 16 / 256;
  float4 x[NP];
  HAM_DEVICE void load(const float* src) {
#pragma unroll
    for (int j = 0; j < NP; ++j) x[j] = reinterpret_cast<const float4*>(src)[threadIdx.x + 256 * j];
  }
  HAM_DEVICE void store(float* dst) const {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int p = threadIdx.x + 256 * j, t = p / 16, c4 = (p % 16) * 4;
      float* q = dst + t * RW + c4;
      q[0] = x[j].x; q[1] = x[j].y; q[2] = x[j].z; q[3] = x[j].w;
    }
  }
};

// rows t < Cc of a [B,T,H,D] tensor into LDS in their own element type, rows D + 16 bytes
// apart (padded rows zero); ldf reads one element as a float
template <class IO, int D>
HAM_DEVICE void load_rows_raw(typename IO::elem* dst, const void* src, const RnnBwdArgs& a, const Ctx& x) {
  constexpr int EPP = 16 / IO::kBytes, PPR = D / EPP, RS = D + EPP;
  for (int i = threadIdx.x; i < kC * PPR; i += blockDim.x) {
    const int t = i / PPR, e0 = (i % PPR) * EPP;
    const uint4 v = t < x.Cc ? *reinterpret_cast<const uint4*>(static_cast<const char*>(src) +
                               ((((size_t)x.b * a.T + x.t0 + t) * a.H + x.h) * D + e0) * IO::kBytes)
                             : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(dst + t * RS + e0) = v;
  }
}
// columns col0 .. col0 + W - 1 of the same, rows W + 16 bytes apart
template <class IO, int D, int W>
HAM_DEVICE void load_cols_raw(typename IO::elem* dst, const void* src, const RnnBwdArgs& a, const Ctx& x, int col0) {
  constexpr int EPP = 16 / IO::kBytes, PPR = W / EPP, RS = W + EPP;
  for (int i = threadIdx.x; i < kC * PPR; i += blockDim.x) {
    const int t = i / PPR, e0 = (i % PPR) * EPP;
    const uint4 v = t < x.Cc ? *reinterpret_cast<const uint4*>(static_cast<const char*>(src) +
                               ((((size_t)x.b * a.T + x.t0 + t) * a.H + x.h) * D + col0 + e0) * IO::kBytes)
                             : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(dst + t * RS + e0) = v;
  }
}
HAM_DEVICE float ldf(const float* p, int i) { return p[i]; }
HAM_DEVICE float ldf(const uint16_t* p, int i) { return bf16_to_f32(p[i]); }

// ---- cbwd_prep: G, A, M, T' of one chunk -----------------------------------------
// grid (N, B*H), 256 threads.  Wave w forms row tile w of K K^T and Q K^T.  T' by forward
// substitution, one column per lane of wave 0: T'_tj = beta_t ([t == j] - sum_{s<t} A_ts T'_sj).
template <class IO, int DK>
__global__ __launch_bounds__(256) void cbwd_prep(RnnBwdArgs a, Scratch sc) {
  using E = typename IO::elem;
  constexpr int KW = DK + 16 / IO::kBytes;                 // K and Q rows in their input type
  __shared__ __attribute__((aligned(16))) E Ks[kC * KW];
  __shared__ __attribute__((aligned(16))) E Qs[kC * KW];
  __shared__ float As[kC * RW], Gs[kC], Bs[kC];
  const Ctx x = ctx(a, blockIdx.y, blockIdx.x);
  const int lane = lane_id(), wave = threadIdx.x >> 6, g4 = lane >> 4, n = lane & 15;
  const size_t cid = (size_t)x.bh * x.N + x.c;
  load_rows_raw<IO, DK>(Ks, a.k, a, x);
  load_rows_raw<IO, DK>(Qs, a.q, a, x);
  if (wave == 0) {
    const bool real = lane < x.Cc;
    const size_t tok = ((size_t)x.b * a.T + x.t0 + (real ? lane : 0)) * a.H + x.h;
    float G = real ? a.g[tok] : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(G, o, kWave);
      if (lane >= o) G += y;
    }
    Gs[lane] = G;
    Bs[lane] = real ? a.beta[tok] : 0.f;
    a.scratch[sc.G + cid * kC + lane] = G;
  }
  __syncthreads();
  float* Ag = a.scratch + sc.A + cid * kC * kC;
  float* Mg = a.scratch + sc.M + cid * kC * kC;
#pragma unroll
  for (int si = 0; si < 4; ++si) {
    f32x4 kk = (f32x4)(0.f), qk = (f32x4)(0.f);
    for (int d = 0; d < DK; d += 4) {
      const float kb = ldf(Ks, (16 * si + n) * KW + d + g4);
      kk = mf(ldf(Ks, (16 * wave + n) * KW + d + g4), kb, kk);
      qk = mf(ldf(Qs, (16 * wave + n) * KW + d + g4), kb, qk);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * wave + 4 * g4 + r, s = 16 * si + n;
      const float gam = s <= t ? __expf(Gs[t] - Gs[s]) : 0.f;
      const float av = s < t ? gam * kk[r] : 0.f;
      const float mv = gam * qk[r];
      Ag[t * kC + s] = av;
      Mg[t * kC + s] = mv;
      As[t * RW + s] = av;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int j = lane;
    float col[kC];
#pragma unroll
    for (int t = 0; t < kC; ++t) {
      float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;      // four partial sums for ILP
#pragma unroll
      for (int s = 0; s + 3 < t; s += 4) {
        p0 = fmaf(As[t * RW + s], col[s], p0);
        p1 = fmaf(As[t * RW + s + 1], col[s + 1], p1);
        p2 = fmaf(As[t * RW + s + 2], col[s + 2], p2);
        p3 = fmaf(As[t * RW + s + 3], col[s + 3], p3);
      }
#pragma unroll
      for (int s = t & ~3; s < t; ++s) p0 = fmaf(As[t * RW + s], col[s], p0);
      col[t] = Bs[t] * ((t == j ? 1.f : 0.f) - ((p0 + p1) + (p2 + p3)));
    }
    float* Tg = a.scratch + sc.T + cid * kC * kC;
#pragma unroll
    for (int t = 0; t < kC; ++t) Tg[t * kC + j] = col[t];
  }
}

// ---- cbwd_fwd: the entering state of every chunk, and D --------------------------
// grid (B*H, DV/64), 256 threads: wave w owns value columns 64 y + 16 w .. + 15.
template <class IO, int DK, int DV>
__global__ __launch_bounds__(256) void cbwd_fwd(RnnBwdArgs a, Scratch sc) {
  constexpr int KW = DK + LP, RT = DK / 16;
  __shared__ float Ks[kC * KW], Vs[kC * RW], Ts[kC * RW], Gs[kC];
  const int bh = blockIdx.x, lane = lane_id(), wave = threadIdx.x >> 6, g4 = lane >> 4, n = lane & 15;
  const int cb0 = blockIdx.y * 64, col = cb0 + 16 * wave + n;
  Ctx x = ctx(a, bh, 0);
  f32x4 S[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[rt][r] = a.S0 ? a.S0[((size_t)bh * DK + 16 * rt + 4 * g4 + r) * DV + col] : 0.f;
  RowsPre<IO, DK, DK> pk;
  RowsPre<IO, DV, 64> pv;
  MatPre pt;
  float pg = 0.f;
  auto fetch = [&](int c) {                                 // chunk c's inputs into registers
    const Ctx y = ctx(a, bh, c);
    const size_t cid = (size_t)bh * y.N + c;
    pk.load(a.k, a, y, 0);
    pv.load(a.v, a, y, cb0);
    pt.load(a.scratch + sc.T + cid * kC * kC);
    if (threadIdx.x < kC) pg = a.scratch[sc.G + cid * kC + threadIdx.x];
  };
  fetch(0);
  for (int c = 0; c < x.N; ++c) {
    x = ctx(a, bh, c);
    const size_t cid = (size_t)bh * x.N + c;
    float* Sg = a.scratch + sc.S + cid * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Sg[(size_t)(16 * rt + 4 * g4 + r) * DV + col] = S[rt][r];
    __syncthreads();                                        // the previous chunk's LDS reads
    pk.store(Ks);
    pv.store(Vs);
    pt.store(Ts);
    if (threadIdx.x < kC) Gs[threadIdx.x] = pg;
    __syncthreads();
    if (c + 1 < x.N) fetch(c + 1);                          // in flight under this chunk's products
    // Y = K S
    f32x4 Y[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      Y[tt] = (f32x4)(0.f);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) Y[tt] = mf(Ks[(16 * tt + n) * KW + 16 * rt + 4 * g4 + r], S[rt][r], Y[tt]);
    }
    // X = V - diag(gamma) Y
    f32x4 X[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * g4 + r;
        X[tt][r] = Vs[t * RW + 16 * wave + n] - __expf(Gs[t]) * Y[tt][r];
      }
    // D = T' X (T' lower triangular)
    f32x4 D[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      D[tt] = (f32x4)(0.f);
#pragma unroll
      for (int u = 0; u <= tt; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) D[tt] = mf(Ts[(16 * tt + n) * RW + 16 * u + 4 * g4 + r], X[u][r], D[tt]);
    }
    float* Dg = a.scratch + sc.D + cid * kC * DV;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) Dg[(size_t)(16 * tt + 4 * g4 + r) * DV + col] = D[tt][r];
    // S <- gamma_C S + K^T diag(w) D
    const float GL = Gs[kC - 1], gC = __expf(GL);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) S[rt] *= gC;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * g4 + r;
        const float wd = __expf(GL - Gs[t]) * D[tt][r];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) S[rt] = mf(Ks[t * KW + 16 * rt + n], wd, S[rt]);
      }
  }
}

// ---- cbwd_rev: dS_C of every chunk (from the end), and dS0 -----------------------
template <class IO, int DK, int DV>
__global__ __launch_bounds__(256) void cbwd_rev(RnnBwdArgs a, Scratch sc) {
  constexpr int KW = DK + LP, RT = DK / 16;
  __shared__ float Ks[kC * KW], Qs[kC * KW], Ms[kC * RW], Ts[kC * RW], dOs[kC * RW], Gs[kC];
  const int bh = blockIdx.x, lane = lane_id(), wave = threadIdx.x >> 6, g4 = lane >> 4, n = lane & 15;
  const int cb0 = blockIdx.y * 64, col = cb0 + 16 * wave + n, cw = 16 * wave + n;
  Ctx x = ctx(a, bh, 0);
  f32x4 dS[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dS[rt][r] = a.dS_T ? a.dS_T[((size_t)bh * DK + 16 * rt + 4 * g4 + r) * DV + col] : 0.f;
  RowsPre<IO, DK, DK> pk, pq;
  RowsPre<IoF32, DV, 64> po;
  MatPre pm, pt;
  float pg = 0.f;
  auto fetch = [&](int c) {                                 // chunk c's inputs into registers
    const Ctx y = ctx(a, bh, c);
    const size_t cid = (size_t)bh * y.N + c;
    pk.load(a.k, a, y, 0);
    pq.load(a.q, a, y, 0);
    po.load(a.dO, a, y, cb0);
    pm.load(a.scratch + sc.M + cid * kC * kC);
    pt.load(a.scratch + sc.T + cid * kC * kC);
    if (threadIdx.x < kC) pg = a.scratch[sc.G + cid * kC + threadIdx.x];
  };
  fetch(x.N - 1);
  for (int c = x.N - 1; c >= 0; --c) {
    x = ctx(a, bh, c);
    const size_t cid = (size_t)bh * x.N + c;
    float* dSg = a.scratch + sc.dS + cid * DK * DV;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dSg[(size_t)(16 * rt + 4 * g4 + r) * DV + col] = dS[rt][r];
    __syncthreads();
    pk.store(Ks);
    pq.store(Qs);
    po.store(dOs);
    pm.store(Ms);
    pt.store(Ts);
    if (threadIdx.x < kC) Gs[threadIdx.x] = pg;
    __syncthreads();
    if (c > 0) fetch(c - 1);                                // in flight under this chunk's products
    const float GL = Gs[kC - 1], gC = __expf(GL);
    // dD = M^T dO + diag(w) K dS   (M^T upper triangular)
    f32x4 dD[4], kd[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 md = (f32x4)(0.f);
      kd[tt] = (f32x4)(0.f);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) kd[tt] = mf(Ks[(16 * tt + n) * KW + 16 * rt + 4 * g4 + r], dS[rt][r], kd[tt]);
#pragma unroll
      for (int u = tt; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 16 * u + 4 * g4 + r;
          md = mf(Ms[s * RW + 16 * tt + n], dOs[s * RW + cw], md);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * g4 + r;
        dD[tt][r] = md[r] + __expf(GL - Gs[t]) * kd[tt][r];
      }
    }
    // dX = T'^T dD   (T'^T upper triangular)
    f32x4 dX[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      dX[tt] = (f32x4)(0.f);
#pragma unroll
      for (int u = tt; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) dX[tt] = mf(Ts[(16 * u + 4 * g4 + r) * RW + 16 * tt + n], dD[u][r], dX[tt]);
    }
    // K dS_C, dD and dX of the chunk for the column kernel; dV = dX
    {
      float* dDg = a.scratch + sc.dD + cid * kC * DV;
      float* dXg = a.scratch + sc.dX + cid * kC * DV;
      float* kdg = a.scratch + sc.KdS + cid * kC * DV;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * tt + 4 * g4 + r;
          dDg[(size_t)t * DV + col] = dD[tt][r];
          dXg[(size_t)t * DV + col] = dX[tt][r];
          kdg[(size_t)t * DV + col] = kd[tt][r];
          if (t < x.Cc) a.dv[(((size_t)x.b * a.T + x.t0 + t) * a.H + x.h) * DV + col] = dX[tt][r];
        }
    }
    // dS <- gamma_C dS - K^T diag(gamma) dX + Q^T diag(gamma) dO
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) dS[rt] *= gC;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tt + 4 * g4 + r;
        const float gt = __expf(Gs[t]);
        const float bx = -gt * dX[tt][r], bo = gt * dOs[t * RW + cw];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          dS[rt] = mf(Ks[t * KW + 16 * rt + n], bx, dS[rt]);
          dS[rt] = mf(Qs[t * KW + 16 * rt + n], bo, dS[rt]);
        }
      }
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) a.dS0[((size_t)bh * DK + 16 * rt + 4 * g4 + r) * DV + col] = dS[rt][r];
}

// ---- cbwd_cols: per-token partial sums over 16 value columns per wave -----------
// grid (N, B*H, DV/64), 256 threads.  K dS_C, dD and dX come from the reverse chain;
// this kernel forms KS, QS, A^T dX and A D and the partial sums over the wave's
// columns: [0] U . R (dbeta), [1] dO . QS - dX . KS (dgamma), [2] K dS_C . D (dw);
// [3][0] <S, dS_C> (dgamma_C).  K and Q rows stay in their input type in LDS, so two
// workgroups share a CU.
template <class IO, int DK, int DV>
__global__ __launch_bounds__(256) void cbwd_cols(RnnBwdArgs a, Scratch sc) {
  using E = typename IO::elem;
  constexpr int KW = DK + 16 / IO::kBytes, VW = 64 + 16 / IO::kBytes, RT = DK / 16;
  __shared__ __attribute__((aligned(16))) E Ks[kC * KW];
  __shared__ __attribute__((aligned(16))) E Qs[kC * KW];
  __shared__ __attribute__((aligned(16))) E Vs[kC * VW];
  __shared__ float As[kC * RW], dOs[kC * RW], Gs[kC];
  const Ctx x = ctx(a, blockIdx.y, blockIdx.x);
  const int lane = lane_id(), wave = threadIdx.x >> 6, g4 = lane >> 4, n = lane & 15;
  const int cb0 = blockIdx.z * 64, col = cb0 + 16 * wave + n, cw = 16 * wave + n;
  const size_t cid = (size_t)x.bh * x.N + x.c;
  load_rows_raw<IO, DK>(Ks, a.k, a, x);
  load_rows_raw<IO, DK>(Qs, a.q, a, x);
  load_cols_raw<IO, DV, 64>(Vs, a.v, a, x, cb0);
  load_rows<IoF32, DV, 64>(dOs, a.dO, a, x, cb0);
  load_mat(As, a.scratch + sc.A + cid * kC * kC);
  if (threadIdx.x < kC) Gs[threadIdx.x] = a.scratch[sc.G + cid * kC + threadIdx.x];
  const float* Sg = a.scratch + sc.S + cid * DK * DV;
  const float* dSg = a.scratch + sc.dS + cid * DK * DV;
  f32x4 S[RT], D[4], dD[4], dX[4], kd[4];
  float sds = 0.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const size_t o = (size_t)(16 * rt + 4 * g4 + r) * DV + col;
      S[rt][r] = Sg[o];
      sds = fmaf(S[rt][r], dSg[o], sds);
    }
  {
    const float* Dg = a.scratch + sc.D + cid * kC * DV;
    const float* dDg = a.scratch + sc.dD + cid * kC * DV;
    const float* dXg = a.scratch + sc.dX + cid * kC * DV;
    const float* kdg = a.scratch + sc.KdS + cid * kC * DV;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const size_t o = (size_t)(16 * tt + 4 * g4 + r) * DV + col;
        D[tt][r] = Dg[o];
        dD[tt][r] = dDg[o];
        dX[tt][r] = dXg[o];
        kd[tt][r] = kdg[o];
      }
  }
  __syncthreads();
  f32x4 Y[4], QS[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    Y[tt] = (f32x4)(0.f); QS[tt] = (f32x4)(0.f);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kcol = 16 * rt + 4 * g4 + r;
        Y[tt] = mf(ldf(Ks, (16 * tt + n) * KW + kcol), S[rt][r], Y[tt]);
        QS[tt] = mf(ldf(Qs, (16 * tt + n) * KW + kcol), S[rt][r], QS[tt]);
      }
  }
  // U = dD - A^T dX;  R = X - A D with X = V - diag(gamma) KS
  float pb[16], pg[16], pw[16];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    f32x4 atdx = (f32x4)(0.f), ad = (f32x4)(0.f);
#pragma unroll
    for (int u = tt; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) atdx = mf(As[(16 * u + 4 * g4 + r) * RW + 16 * tt + n], dX[u][r], atdx);
#pragma unroll
    for (int u = 0; u <= tt; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) ad = mf(As[(16 * tt + n) * RW + 16 * u + 4 * g4 + r], D[u][r], ad);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tt + 4 * g4 + r;
      const float X = ldf(Vs, t * VW + cw) - __expf(Gs[t]) * Y[tt][r];
      const float U = dD[tt][r] - atdx[r], R = X - ad[r];
      pb[4 * tt + r] = U * R;
      pg[4 * tt + r] = dOs[t * RW + cw] * QS[tt][r] - dX[tt][r] * Y[tt][r];
      pw[4 * tt + r] = kd[tt][r] * D[tt][r];
    }
  }
  // lane (g4, n) receives the column sums of value index n: token 16 (n/4) + 4 g4 + n%4
  const float sb = row16_transpose_sum(pb, n), sg = row16_transpose_sum(pg, n), sw = row16_transpose_sum(pw, n);
  const int tok = 16 * (n >> 2) + 4 * g4 + (n & 3);
  float* P = a.scratch + sc.part + (cid * (DV / 16) + blockIdx.z * 4 + wave) * 4 * kC;
  P[tok] = sb;
  P[kC + tok] = sg;
  P[2 * kC + tok] = sw;
  sds = wave_sum<64>(sds);
  if (lane == 0) P[3 * kC] = sds;
}

// ---- cbwd_final: dM, dA, dQ, dK, dG -> dg, dbeta ---------------------------------
// grid (N, B*H), 64 NWF threads.  dQ and dK are formed transposed (dk rows x tokens):
// wave w owns dk rows DK/4 * (w mod 4) .. + DK/4 - 1 of JT token tiles, and the dM, dA
// tiles (w mod 4, same JT column tiles).  Phase 1 runs over the value columns in blocks
// of 32 (dO, D, dX, S, dS of the block in LDS); phase 2 takes the Gram terms, with K and
// Q rows in LDS in their input type.  At bf16 two workgroups share a CU, so one stages
// its rows while the other multiplies.
constexpr int NWF = 4;
template <class IO, int DK, int DV>
__global__ __launch_bounds__(64 * NWF) void cbwd_final(RnnBwdArgs a, Scratch sc) {
  using E = typename IO::elem;
  constexpr int NH = NWF / 4, JT = 4 / NH;                    // wave halves, tiles per wave
  constexpr int WR = DK / 4, WT = WR / 16;                    // dk rows and row tiles per wave
  constexpr int CB = 32, BW = CB + LP;                        // phase-1 column block
  constexpr int KW = DK + 16 / IO::kBytes;                    // K, Q rows in their input type
  constexpr int P1 = (3 * kC + 2 * DK) * BW * 4;              // phase-1 bytes
  constexpr int P2 = 2 * kC * KW * IO::kBytes + 2 * kC * RW * 4;
  __shared__ __attribute__((aligned(16))) char L[P1 > P2 ? P1 : P2];
  __shared__ float Gs[kC], rpart[NH][kC], cpart[4][kC];
  const Ctx x = ctx(a, blockIdx.y, blockIdx.x);
  const int lane = lane_id(), wave = threadIdx.x >> 6, g4 = lane >> 4, n = lane & 15;
  const int qw = wave & 3, hw = wave >> 2;
  const size_t cid = (size_t)x.bh * x.N + x.c;
  if (threadIdx.x < kC) Gs[threadIdx.x] = a.scratch[sc.G + cid * kC + threadIdx.x];
  const float* Sg = a.scratch + sc.S + cid * DK * DV;
  const float* dSg = a.scratch + sc.dS + cid * DK * DV;
  const float* Dg = a.scratch + sc.D + cid * kC * DV;
  const float* dXg = a.scratch + sc.dX + cid * kC * DV;
  f32x4 dM[JT], dA[JT], dQT[WT][JT], dKT[WT][JT];
#pragma unroll
  for (int i = 0; i < JT; ++i) {
    dM[i] = (f32x4)(0.f); dA[i] = (f32x4)(0.f);
#pragma unroll
    for (int kt = 0; kt < WT; ++kt) { dQT[kt][i] = (f32x4)(0.f); dKT[kt][i] = (f32x4)(0.f); }
  }
  float* dOs = reinterpret_cast<float*>(L);
  float* Ds = dOs + kC * BW;
  float* dXs = Ds + kC * BW;
  float* Ss = dXs + kC * BW;
  float* dSs = Ss + DK * BW;
  for (int cb0 = 0; cb0 < DV; cb0 += CB) {
    __syncthreads();
    load_rows<IoF32, DV, CB>(dOs, a.dO, a, x, cb0);
    load_block<kC, CB>(Ds, Dg, DV, cb0);
    load_block<kC, CB>(dXs, dXg, DV, cb0);
    load_block<DK, CB>(Ss, Sg, DV, cb0);
    load_block<DK, CB>(dSs, dSg, DV, cb0);
    __syncthreads();
    const float gl = Gs[kC - 1];
    for (int d = 0; d < CB; d += 4) {
      // dM, dA tiles (qw, JT hw + j): sum over the block's columns of dO D^T, dX D^T
      const float o_a = dOs[(16 * qw + n) * BW + d + g4], x_a = dXs[(16 * qw + n) * BW + d + g4];
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const float db = Ds[(16 * (JT * hw + j) + n) * BW + d + g4];
        dM[j] = mf(o_a, db, dM[j]);
        dA[j] = mf(x_a, db, dA[j]);
      }
      // dQ^T += S diag(gamma) dO^T;  dK^T += -S (diag(gamma) dX)^T + dS (diag(w) D)^T
#pragma unroll
      for (int j = 0; j < JT; ++j) {
        const int t = 16 * (JT * hw + j) + n;
        const float gt = __expf(Gs[t]), wt = __expf(gl - Gs[t]);
        const float bo = gt * dOs[t * BW + d + g4], bx = -gt * dXs[t * BW + d + g4], bd = wt * Ds[t * BW + d + g4];
#pragma unroll
        for (int kt = 0; kt < WT; ++kt) {
          const int row = WR * qw + 16 * kt + n;
          const float sa = Ss[row * BW + d + g4], dsa = dSs[row * BW + d + g4];
          dQT[kt][j] = mf(sa, bo, dQT[kt][j]);
          dKT[kt][j] = mf(sa, bx, dKT[kt][j]);
          dKT[kt][j] = mf(dsa, bd, dKT[kt][j]);
        }
      }
    }
  }
  __syncthreads();
  // phase 2: dM o Gamma and dA o Gamma in LDS, K and Q rows; the row and column sums of
  // dM o M + dA o A by wave reductions
  E* Ks = reinterpret_cast<E*>(L);
  E* Qs = Ks + kC * KW;
  float* dMG = reinterpret_cast<float*>(Qs + kC * KW);
  float* dAG = dMG + kC * RW;
  const float* Ag = a.scratch + sc.A + cid * kC * kC;
  const float* Mg = a.scratch + sc.M + cid * kC * kC;
  float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    float cs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * qw + 4 * g4 + r, s = 16 * (JT * hw + j) + n;
      const float gam = s <= t ? __expf(Gs[t] - Gs[s]) : 0.f;
      const float dm = s <= t ? dM[j][r] : 0.f, da = s < t ? -dA[j][r] : 0.f;
      dMG[t * RW + s] = dm * gam;
      dAG[t * RW + s] = da * gam;
      const float gg = dm * Mg[t * kC + s] + da * Ag[t * kC + s];
      rs[r] += gg;
      cs += gg;
    }
    cs += __shfl_xor(cs, 16, kWave);                        // over the four 4-row groups
    cs += __shfl_xor(cs, 32, kWave);
    if (g4 == 0) cpart[qw][16 * (JT * hw + j) + n] = cs;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float v = row16_sum(rs[r]);                       // over the 16 columns of the row
    if (n == 0) rpart[hw][16 * qw + 4 * g4 + r] = v;
  }
  load_rows_raw<IO, DK>(Ks, a.k, a, x);
  load_rows_raw<IO, DK>(Qs, a.q, a, x);
  __syncthreads();
  // dQ^T += K^T (dM o Gamma)^T;  dK^T += Q^T (dM o Gamma) + K^T (dA o Gamma)^T + K^T (dA o Gamma)
  for (int s0 = 0; s0 < kC; s0 += 4) {
    const int s = s0 + g4;
#pragma unroll
    for (int j = 0; j < JT; ++j) {
      const int t = 16 * (JT * hw + j) + n;
      const float mgT = dMG[t * RW + s], mg = dMG[s * RW + t];
      const float agT = dAG[t * RW + s], ag = dAG[s * RW + t];
#pragma unroll
      for (int kt = 0; kt < WT; ++kt) {
        const int row = WR * qw + 16 * kt + n;
        const float ka = ldf(Ks, s * KW + row), qa = ldf(Qs, s * KW + row);
        dQT[kt][j] = mf(ka, mgT, dQT[kt][j]);
        dKT[kt][j] = mf(qa, mg, dKT[kt][j]);
        dKT[kt][j] = mf(ka, agT + ag, dKT[kt][j]);
      }
    }
  }
  // dQ^T / dK^T tiles: lane (g4, n) holds dk rows WR qw + 16 kt + 4 g4 + r of token
  // 16 (JT hw + j) + n
#pragma unroll
  for (int j = 0; j < JT; ++j) {
    const int t = 16 * (JT * hw + j) + n;
    if (t < x.Cc) {
      const size_t o = (((size_t)x.b * a.T + x.t0 + t) * a.H + x.h) * DK;
#pragma unroll
      for (int kt = 0; kt < WT; ++kt) {
        const int row = WR * qw + 16 * kt + 4 * g4;
        *reinterpret_cast<f32x4*>(a.dq + o + row) = dQT[kt][j];
        *reinterpret_cast<f32x4*>(a.dk + o + row) = dKT[kt][j];
      }
    }
  }
  // dG, then dg = reverse cumulative sum over the real tokens; dbeta
  if (wave == 0) {
    const int t = lane;
    const float* P = a.scratch + sc.part + cid * (DV / 16) * 4 * kC;
    float db = 0.f, dgam = 0.f, dw = 0.f, dgC = 0.f;
    for (int cb = 0; cb < DV / 16; ++cb) {
      db += P[cb * 4 * kC + t];
      dgam += P[cb * 4 * kC + kC + t];
      dw += P[cb * 4 * kC + 2 * kC + t];
      dgC += P[cb * 4 * kC + 3 * kC];
    }
    float rsum = 0.f, csum = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < NH; ++h2) rsum += rpart[h2][t];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) csum += cpart[q4][t];
    const bool real = t < x.Cc;
    const float G = Gs[t], GLr = Gs[kC - 1];
    const float wt = __expf(GLr - G);
    float dG = real ? __expf(G) * dgam - wt * dw + rsum - csum : 0.f;
    const float tail = wave_sum<64>(real ? wt * dw : 0.f);
    if (t == x.Cc - 1) dG += __expf(GLr) * dgC + tail;
    // reverse inclusive scan: dg_t = sum_{j >= t} dG_j
    float acc = dG;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_down(acc, o, kWave);
      if (lane + o < 64) acc += y;
    }
    if (real) {
      const size_t tok = ((size_t)x.b * a.T + x.t0 + t) * a.H + x.h;
      a.dg[tok] = acc;
      a.dbeta[tok] = db;
    }
  }
}

template <class IO, int DK, int DV>
hipError_t launch_t(const RnnBwdArgs& a, hipStream_t s) {
  const Scratch sc = scratch_layout(a.B, a.H, a.T, DK, DV);
  const int N = (a.T + kC - 1) / kC, BH = a.B * a.H;
  hipLaunchKernelGGL((cbwd_prep<IO, DK>), dim3(N, BH), dim3(256), 0, s, a, sc);
  hipLaunchKernelGGL((cbwd_fwd<IO, DK, DV>), dim3(BH, DV / 64), dim3(256), 0, s, a, sc);
  hipLaunchKernelGGL((cbwd_rev<IO, DK, DV>), dim3(BH, DV / 64), dim3(256), 0, s, a, sc);
  hipLaunchKernelGGL((cbwd_cols<IO, DK, DV>), dim3(N, BH, DV / 64), dim3(256), 0, s, a, sc);
  hipLaunchKernelGGL((cbwd_final<IO, DK, DV>), dim3(N, BH), dim3(64 * NWF), 0, s, a, sc);
  return hipGetLastError();
}

}  // namespace cbwd

size_t rnn_backward_chunked_scratch_floats(int B, int H, int T, int dk, int dv) {
  return cbwd::scratch_layout(B, H, T, dk, dv).total;
}

hipError_t launch_rnn_backward_chunked(int io, int dk, int dv, const RnnBwdArgs& a, hipStream_t s) {
#define HAM_CASE(IOT, DKV, DVV) \
  if (dk == DKV && dv == DVV) return cbwd::launch_t<IOT, DKV, DVV>(a, s);
  if (io == 0) {
    HAM_CASE(IoF32, 64, 64) HAM_CASE(IoF32, 64, 128) HAM_CASE(IoF32, 128, 64) HAM_CASE(IoF32, 128, 128)
  } else {
    HAM_CASE(IoBF16, 64, 64) HAM_CASE(IoBF16, 64, 128) HAM_CASE(IoBF16, 128, 64) HAM_CASE(IoBF16, 128, 128)
  }
#undef HAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace ham
