// ham_rnn_chunked.hip -- chunked gated delta rule (WY/UT form) on MFMA, with the
// fit-error routing score fused in.
//
// "Hybrid Associative Memories": DeltaNet update (§2) with the gated-DeltaNet
// decay (App. A.1 "RNN Memory"), post-update readout (§2 linear-attention
// equation), fit-error score (§2 "Prediction Error as Routing Metric"; App. A.1
// "Router Implementations"), and the chunk size 64 the paper's training kernels
// use (App. A.1 "Custom Triton Kernels"; Tab. E.11 lists the chunked steps: g
// cumsum, compute A, invert A, recompute w/u, state pass, output).
//
// Per head, with S (dk x dv) the state entering a chunk of C = 64 tokens,
// G = cumsum(g) inside the chunk, gamma = exp(G), Gamma[t,j] = exp(G_t - G_j):
//   A  = strict_lower(Gamma o K K^T)                 (C x C)
//   T' = (I + diag(beta) A)^-1 diag(beta)            (unit-lower solve)
//   X  = V - diag(gamma) K S
//   D  = T' X                                        (the chunk's write vectors)
//   P  = diag(gamma) K S + A D          row t = alpha_t S_{t-1}^T k_t  (score)
//   O  = diag(gamma) Q S + (Gamma o Q K^T o lower_incl) D       (o_rnn)
//   S <- gamma_C S + K^T diag(exp(G_C - G)) D
// These follow from unrolling S_t = alpha_t S_{t-1} + beta_t k_t (v_t - alpha_t
// S_{t-1}^T k_t)^T over the chunk.
//
// Precision: K, Q, V are bf16 inputs, so K K^T and Q K^T are exact on bf16 MFMA
// (fp32 accumulate).  Every product with an fp32 operand (S, D, A, T') splits the
// fp32 value into three bf16 terms hi+mid+lo (24 significant bits) and keeps the
// cross terms down to 2^-16 relative, which is fp32-level accuracy; the routing
// score needs it.  The readout O only feeds bf16 outputs and keeps two terms.
//
// Layout: one workgroup = NW waves = one head's 16*NW state columns.  The fp32 state
// lives in MFMA accumulators (rows of S on the 16x16 tile's M axis).  Products
// whose contraction runs over rows of an accumulator use a k-slot order that
// matches what each lane already holds (k-slot 8g+j <-> rows 4g+j and 16+4g+j-4
// of a 32-row step), and the A operands are read from LDS in that same order, so
// no accumulator is ever shuffled between lanes.
#include "ham_common.h"
#include "ham_internal.h"

namespace ham {
namespace {

constexpr int kC = 64;   // chunk length

HAM_DEVICE f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

HAM_DEVICE __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }
HAM_DEVICE float from_bf16(__bf16 x) { return static_cast<float>(x); }

// x = hi + mid + lo, each a bf16 (nearest-even); the residuals are exact in fp32.
HAM_DEVICE void split3(float x, __bf16& h, __bf16& m, __bf16& l) {
  h = to_bf16(x);
  float r = x - from_bf16(h);
  m = to_bf16(r);
  r -= from_bf16(m);
  l = to_bf16(r);
}

// 8 bf16 from two 4-element (8-byte) runs of a row: k-slots 0..3 and 4..7.
HAM_DEVICE bf16x8 frag2(const uint16_t* p0, const uint16_t* p1) {
  const u16x4 a = *reinterpret_cast<const u16x4*>(p0);
  const u16x4 b = *reinterpret_cast<const u16x4*>(p1);
  u16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return __builtin_bit_cast(bf16x8, r);
}

// B-operand fragments of a 32-row step from two accumulator tiles (rows 4g+i of
// tile lo -> slots 0..3, of tile hi -> slots 4..7), split into three bf16 terms.
HAM_DEVICE void split_pair3(const f32x4& lo, const f32x4& hi, bf16x8& h, bf16x8& m, bf16x8& l,
                            float scale_lo[4] = nullptr, float scale_hi[4] = nullptr) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __bf16 a, b, c;
    split3(scale_lo ? lo[i] * scale_lo[i] : lo[i], a, b, c);
    h[i] = a; m[i] = b; l[i] = c;
    split3(scale_hi ? hi[i] * scale_hi[i] : hi[i], a, b, c);
    h[4 + i] = a; m[4 + i] = b; l[4 + i] = c;
  }
}

template <int DK, int NW>
struct ChunkSmem {
  static constexpr int KS = DK + 8;        // row stride (u16) of K and Q
  static constexpr int TS = kC + 8;        // row stride (u16) of C-wide bf16 matrices and K^T
  static constexpr int VS = 16 * NW + 8;   // row stride (u16) of the V slice
  static constexpr int FS = kC + 1;        // row stride (f32) of C x C fp32 matrices
  uint16_t K[kC * KS];
  uint16_t Q[kC * KS];
  uint16_t Kt[DK * TS];
  uint16_t V[kC * VS];
  uint16_t A[3][kC * TS];                  // strict_lower(Gamma o K K^T): hi, mid, lo
  uint16_t Tm[3][kC * TS];                 // (I + diag(beta)A)^-1 diag(beta): hi, mid, lo
  union {
    uint16_t QK[2][kC * TS];               // Gamma o Q K^T o lower_incl: hi, mid
    float L[kC * FS];                      // diag(beta) A, during the inverse only
  } u;
  float Tf[kC * FS];                       // (I + L)^-1 in fp32
  float W[3 * 256];
  float G[kC], gam[kC], beta[kC], wdec[kC];
};

// Per-thread register stage of one chunk's inputs (prefetched one chunk ahead).
template <int DK, int NW>
struct ChunkRegs {
  static constexpr int NT = 64 * NW;
  static constexpr int KU = kC * (DK / 8);             // 16-byte units of K (and Q)
  static constexpr int KPT = (KU + NT - 1) / NT;
  static constexpr int VU = kC * 2 * NW;               // 16-byte units of the V slice
  static constexpr int VPT = (VU + NT - 1) / NT;
  u16x8 k[KPT], q[KPT], v[VPT];
  float g, beta;
};

template <int DK, int DV, int NW>
HAM_DEVICE void load_chunk(const RnnArgs& a, ChunkRegs<DK, NW>& r, int b, int h, int t0, int colbase,
                           int tid, bool readout) {
  using R = ChunkRegs<DK, NW>;
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  const int nvalid = min(kC, a.T - t0);
#pragma unroll
  for (int p = 0; p < R::KPT; ++p) {
    const int u = tid + p * R::NT;
    const int row = u / (DK / 8), cu = (u % (DK / 8)) * 8;
    r.k[p] = (u16x8)(0);
    r.q[p] = (u16x8)(0);
    if (u < R::KU && row < nvalid) {
      const size_t tok = ((size_t)b * a.T + t0 + row) * a.H + h;
      r.k[p] = *reinterpret_cast<const u16x8*>(k + tok * DK + cu);
      if (readout) r.q[p] = *reinterpret_cast<const u16x8*>(q + tok * DK + cu);
    }
  }
#pragma unroll
  for (int p = 0; p < R::VPT; ++p) {
    const int u = tid + p * R::NT;
    const int row = u / (2 * NW), cu = (u % (2 * NW)) * 8;
    r.v[p] = (u16x8)(0);
    if (u < R::VU && row < nvalid) {
      const size_t tok = ((size_t)b * a.T + t0 + row) * a.H + h;
      r.v[p] = *reinterpret_cast<const u16x8*>(v + tok * DV + colbase + cu);
    }
  }
  r.g = 0.f;
  r.beta = 0.f;
  if (tid < kC && tid < nvalid) {
    const size_t tok = ((size_t)b * a.T + t0 + tid) * a.H + h;
    r.g = a.g[tok];
    r.beta = a.beta[tok];
  }
}

template <int DK, int NW>
HAM_DEVICE void store_chunk(ChunkSmem<DK, NW>& sm, const ChunkRegs<DK, NW>& r, int tid) {
  using R = ChunkRegs<DK, NW>;
  using SM = ChunkSmem<DK, NW>;
#pragma unroll
  for (int p = 0; p < R::KPT; ++p) {
    const int u = tid + p * R::NT;
    if (u < R::KU) {
      const int row = u / (DK / 8), cu = (u % (DK / 8)) * 8;
      *reinterpret_cast<u16x8*>(&sm.K[row * SM::KS + cu]) = r.k[p];
      *reinterpret_cast<u16x8*>(&sm.Q[row * SM::KS + cu]) = r.q[p];
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.Kt[(cu + j) * SM::TS + row] = r.k[p][j];
    }
  }
#pragma unroll
  for (int p = 0; p < R::VPT; ++p) {
    const int u = tid + p * R::NT;
    if (u < R::VU) {
      const int row = u / (2 * NW), cu = (u % (2 * NW)) * 8;
      *reinterpret_cast<u16x8*>(&sm.V[row * SM::VS + cu]) = r.v[p];
    }
  }
  if (tid < kC) {
    // inclusive prefix sum of the log decays over the chunk (wave 0)
    float G = r.g;
#pragma unroll
    for (int off = 1; off < kC; off <<= 1) {
      const float y = __shfl_up(G, off, kWave);
      if (tid >= off) G += y;
    }
    const float Glast = __shfl(G, kC - 1, kWave);
    sm.G[tid] = G;
    sm.gam[tid] = expf(G);
    sm.wdec[tid] = expf(Glast - G);
    sm.beta[tid] = r.beta;
  }
}

// T = (I + L)^-1 for strictly lower L (fp32, 64x64, in sm.u.L) by 16x16 blocks:
// diagonal blocks by forward substitution, then block rows level by level,
// T_ij = -T_ii sum_{k=j}^{i-1} L_ik T_kj.
template <int DK, int NW>
HAM_DEVICE void invert_unit_lower(ChunkSmem<DK, NW>& sm, int tid) {
  using SM = ChunkSmem<DK, NW>;
  constexpr int NT = 64 * NW, FS = SM::FS;
  const float* L = sm.u.L;
  float* Tf = sm.Tf;
  if (tid < 64) {
    const int bb = tid >> 4, c = tid & 15;
    float col[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == c) ? 1.f : 0.f;
      const float* lr = L + (16 * bb + r) * FS + 16 * bb;
#pragma unroll
      for (int j = 0; j < r; ++j) s = fmaf(-lr[j], col[j], s);
      col[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tf[(16 * bb + r) * FS + 16 * bb + c] = col[r];
  }
  __syncthreads();
#pragma unroll
  for (int lev = 1; lev < 4; ++lev) {
    const int nb = 4 - lev;
    for (int e = tid; e < nb * 256; e += NT) {
      const int blk = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      const int i = lev + blk, j = i - lev;
      float s = 0.f;
      const float* lr = L + (16 * i + r) * FS;
      for (int kk = 16 * j; kk < 16 * i; ++kk) s = fmaf(lr[kk], Tf[kk * FS + 16 * j + cc], s);
      sm.W[blk * 256 + r * 16 + cc] = s;
    }
    __syncthreads();
    for (int e = tid; e < nb * 256; e += NT) {
      const int blk = e >> 8, r = (e >> 4) & 15, cc = e & 15;
      const int i = lev + blk, j = i - lev;
      float s = 0.f;
      const float* tr = Tf + (16 * i + r) * FS + 16 * i;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) s = fmaf(tr[kk], sm.W[blk * 256 + kk * 16 + cc], s);
      Tf[(16 * i + r) * FS + 16 * j + cc] = -s;
    }
    __syncthreads();
  }
}

template <int DK, int DV, int NW>
__global__ __launch_bounds__(64 * NW) void rnn_chunked_kernel(RnnArgs a) {
  using SM = ChunkSmem<DK, NW>;
  constexpr int NT = 64 * NW;
  constexpr int KS = SM::KS, TS = SM::TS, VS = SM::VS, FS = SM::FS;
  constexpr int MT = DK / 16;     // 16-row tiles of S
  constexpr int KSD = DK / 32;    // 32-wide k-steps over d
  constexpr int NSL = DV / 16;    // score slices
  __shared__ SM sm;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.H + h;
  const int colbase = blockIdx.x * 16 * NW;
  const int col = colbase + wave * 16 + n;
  const int vcol = wave * 16 + n;
  const int slice = blockIdx.x * NW + wave;
  const bool readout = a.o_rnn32 != nullptr;

  // state tiles: S[16*mt + 4g + i][col]
  f32x4 S[MT];
  const size_t sbase = (size_t)bh * DK * DV;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[mt][i] = a.S0 ? a.S0[sbase + (size_t)(16 * mt + 4 * g + i) * DV + col] : 0.f;

  const int nchunk = (a.T + kC - 1) / kC;
  ChunkRegs<DK, NW> regs;
  load_chunk<DK, DV, NW>(a, regs, b, h, 0, colbase, tid, readout);

  for (int c = 0; c < nchunk; ++c) {
    const int t0 = c * kC;
    const int nvalid = min(kC, a.T - t0);
    __syncthreads();                          // the previous chunk's LDS readers are done
    store_chunk<DK, NW>(sm, regs, tid);
    if (c + 1 < nchunk) load_chunk<DK, DV, NW>(a, regs, b, h, t0 + kC, colbase, tid, readout);
    __syncthreads();

    // ---- A = strict_lower(Gamma o K K^T) (3-way split) and L = diag(beta) A ----
    for (int tile = wave; tile < 16; tile += NW) {
      const int mt = tile >> 2, nt = tile & 3;
      f32x4 acc = (f32x4)(0.f);
      if (nt <= mt) {
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks) {
          const bf16x8 af = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&sm.K[(16 * mt + n) * KS + 32 * ks + 8 * g]));
          const bf16x8 bf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&sm.K[(16 * nt + n) * KS + 32 * ks + 8 * g]));
          acc = mfma_bf16(af, bf, acc);
        }
      }
      const int j = 16 * nt + n;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * g + i;
        const float val = (j < t) ? acc[i] * expf(sm.G[t] - sm.G[j]) : 0.f;
        __bf16 x0, x1, x2;
        split3(val, x0, x1, x2);
        sm.A[0][t * TS + j] = __builtin_bit_cast(uint16_t, x0);
        sm.A[1][t * TS + j] = __builtin_bit_cast(uint16_t, x1);
        sm.A[2][t * TS + j] = __builtin_bit_cast(uint16_t, x2);
        sm.u.L[t * FS + j] = sm.beta[t] * val;
      }
    }
    __syncthreads();
    invert_unit_lower<DK, NW>(sm, tid);
    // T' = T diag(beta), 3-way split, zero above the diagonal
    for (int e = tid; e < kC * kC; e += NT) {
      const int t = e >> 6, j = e & 63;
      const float val = (j <= t) ? sm.Tf[t * FS + j] * sm.beta[j] : 0.f;
      __bf16 x0, x1, x2;
      split3(val, x0, x1, x2);
      sm.Tm[0][t * TS + j] = __builtin_bit_cast(uint16_t, x0);
      sm.Tm[1][t * TS + j] = __builtin_bit_cast(uint16_t, x1);
      sm.Tm[2][t * TS + j] = __builtin_bit_cast(uint16_t, x2);
    }
    __syncthreads();
    // ---- Gamma o Q K^T o lower_incl (2-way split), reusing the L storage ----
    if (readout) {
      for (int tile = wave; tile < 16; tile += NW) {
        const int mt = tile >> 2, nt = tile & 3;
        f32x4 acc = (f32x4)(0.f);
        if (nt <= mt) {
#pragma unroll
          for (int ks = 0; ks < KSD; ++ks) {
            const bf16x8 af = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&sm.Q[(16 * mt + n) * KS + 32 * ks + 8 * g]));
            const bf16x8 bf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&sm.K[(16 * nt + n) * KS + 32 * ks + 8 * g]));
            acc = mfma_bf16(af, bf, acc);
          }
        }
        const int j = 16 * nt + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * mt + 4 * g + i;
          const float val = (j <= t) ? acc[i] * expf(sm.G[t] - sm.G[j]) : 0.f;
          const __bf16 x0 = to_bf16(val);
          const __bf16 x1 = to_bf16(val - from_bf16(x0));
          sm.u.QK[0][t * TS + j] = __builtin_bit_cast(uint16_t, x0);
          sm.u.QK[1][t * TS + j] = __builtin_bit_cast(uint16_t, x1);
        }
      }
    }
    __syncthreads();

    // ---- state phase: this wave's 16 columns ----
    bf16x8 sh[KSD], smd[KSD], sl[KSD];
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) split_pair3(S[2 * ks], S[2 * ks + 1], sh[ks], smd[ks], sl[ks]);

    f32x4 P[4], O[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      P[mt] = (f32x4)(0.f);
      O[mt] = (f32x4)(0.f);
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        const uint16_t* kr = &sm.K[(16 * mt + n) * KS + 32 * ks + 4 * g];
        const bf16x8 af = frag2(kr, kr + 16);
        P[mt] = mfma_bf16(af, sl[ks], P[mt]);
        P[mt] = mfma_bf16(af, smd[ks], P[mt]);
        P[mt] = mfma_bf16(af, sh[ks], P[mt]);
        if (readout) {
          const uint16_t* qr = &sm.Q[(16 * mt + n) * KS + 32 * ks + 4 * g];
          const bf16x8 qf = frag2(qr, qr + 16);
          O[mt] = mfma_bf16(qf, smd[ks], O[mt]);
          O[mt] = mfma_bf16(qf, sh[ks], O[mt]);
        }
      }
    }
    // X = V - gamma K S ; P, O start as gamma K S, gamma Q S
    f32x4 X[4], Vr[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * g + i;
        const float gm = sm.gam[t];
        const float vv = bf16_to_f32(sm.V[t * VS + vcol]);
        Vr[mt][i] = vv;
        P[mt][i] *= gm;
        O[mt][i] *= gm;
        X[mt][i] = vv - P[mt][i];
      }
    bf16x8 xh[2], xm[2], xl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) split_pair3(X[2 * s], X[2 * s + 1], xh[s], xm[s], xl[s]);

    // D = T' X   (6 cross terms per k-step; T' is lower triangular)
    f32x4 D[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      D[mt] = (f32x4)(0.f);
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s) {
        const int off = (16 * mt + n) * TS + 32 * s + 4 * g;
        const bf16x8 th = frag2(&sm.Tm[0][off], &sm.Tm[0][off + 16]);
        const bf16x8 tm = frag2(&sm.Tm[1][off], &sm.Tm[1][off + 16]);
        const bf16x8 tl = frag2(&sm.Tm[2][off], &sm.Tm[2][off + 16]);
        D[mt] = mfma_bf16(tm, xm[s], D[mt]);
        D[mt] = mfma_bf16(tl, xh[s], D[mt]);
        D[mt] = mfma_bf16(th, xl[s], D[mt]);
        D[mt] = mfma_bf16(tm, xh[s], D[mt]);
        D[mt] = mfma_bf16(th, xm[s], D[mt]);
        D[mt] = mfma_bf16(th, xh[s], D[mt]);
      }
    }
    bf16x8 dh[2], dm[2], dl[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) split_pair3(D[2 * s], D[2 * s + 1], dh[s], dm[s], dl[s]);

    // P += A D (6 terms), O += (Gamma o Q K^T) D (3 terms)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s) {
        const int off = (16 * mt + n) * TS + 32 * s + 4 * g;
        const bf16x8 ah = frag2(&sm.A[0][off], &sm.A[0][off + 16]);
        const bf16x8 am = frag2(&sm.A[1][off], &sm.A[1][off + 16]);
        const bf16x8 al = frag2(&sm.A[2][off], &sm.A[2][off + 16]);
        P[mt] = mfma_bf16(am, dm[s], P[mt]);
        P[mt] = mfma_bf16(al, dh[s], P[mt]);
        P[mt] = mfma_bf16(ah, dl[s], P[mt]);
        P[mt] = mfma_bf16(am, dh[s], P[mt]);
        P[mt] = mfma_bf16(ah, dm[s], P[mt]);
        P[mt] = mfma_bf16(ah, dh[s], P[mt]);
        if (readout) {
          const bf16x8 qh = frag2(&sm.u.QK[0][off], &sm.u.QK[0][off + 16]);
          const bf16x8 qm = frag2(&sm.u.QK[1][off], &sm.u.QK[1][off + 16]);
          O[mt] = mfma_bf16(qm, dh[s], O[mt]);
          O[mt] = mfma_bf16(qh, dm[s], O[mt]);
          O[mt] = mfma_bf16(qh, dh[s], O[mt]);
        }
      }
    }

    // score partials of this 16-column slice, and the readout
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * g + i;
        float pv = P[mt][i] * Vr[mt][i], pp = P[mt][i] * P[mt][i], vv = Vr[mt][i] * Vr[mt][i];
        pv = wave_sum<16>(pv);
        pp = wave_sum<16>(pp);
        vv = wave_sum<16>(vv);
        if (t < nvalid) {
          if (n == 0)
            a.score[((size_t)bh * a.T + t0 + t) * NSL + slice] = make_float4(pv, pp, vv, 0.f);
          if (readout)
            a.o_rnn32[(((size_t)b * a.T + t0 + t) * a.H + h) * DV + col] = O[mt][i];
        }
      }

    // S <- gamma_C S + K^T diag(exp(G_C - G)) D
    bf16x8 eh[2], em[2], el[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float w0[4], w1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0[i] = sm.wdec[32 * s + 4 * g + i];
        w1[i] = sm.wdec[32 * s + 16 + 4 * g + i];
      }
      split_pair3(D[2 * s], D[2 * s + 1], eh[s], em[s], el[s], w0, w1);
    }
    const float gl = sm.gam[kC - 1];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      S[mt] *= gl;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint16_t* kr = &sm.Kt[(16 * mt + n) * TS + 32 * s + 4 * g];
        const bf16x8 kf = frag2(kr, kr + 16);
        S[mt] = mfma_bf16(kf, el[s], S[mt]);
        S[mt] = mfma_bf16(kf, em[s], S[mt]);
        S[mt] = mfma_bf16(kf, eh[s], S[mt]);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) a.S_out[sbase + (size_t)(16 * mt + 4 * g + i) * DV + col] = S[mt][i];
}

template <int DK, int DV, int NW>
hipError_t launch_t(const RnnArgs& a, hipStream_t s) {
  dim3 grid(DV / (16 * NW), a.H, a.B);
  hipLaunchKernelGGL((rnn_chunked_kernel<DK, DV, NW>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const RnnArgs& a, hipStream_t s) {
  // widest workgroup that still gives every CU a workgroup
  const long heads = (long)a.B * a.H;
  if (heads * (DV / 64) >= 256) return launch_t<DK, DV, 4>(a, s);
  if (heads * (DV / 32) >= 256) return launch_t<DK, DV, 2>(a, s);
  return launch_t<DK, DV, 1>(a, s);
}

}  // namespace

bool rnn_chunked_supported(int io, int dk, int dv) {
  return io == 1 && (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

int rnn_chunked_slices(int dv) { return dv / 16; }

hipError_t launch_rnn_chunked(int io, int dk, int dv, const RnnArgs& a, hipStream_t s) {
  if (io != 1) return hipErrorInvalidValue;
  if (dk == 64 && dv == 64) return launch_dims<64, 64>(a, s);
  if (dk == 64 && dv == 128) return launch_dims<64, 128>(a, s);
  if (dk == 128 && dv == 64) return launch_dims<128, 64>(a, s);
  if (dk == 128 && dv == 128) return launch_dims<128, 128>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace ham
