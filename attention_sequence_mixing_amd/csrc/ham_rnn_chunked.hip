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
namespace chunked {

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

// ---------------------------------------------------------------------------------
// Chunk record written by the prep kernel and streamed by the state kernel (all
// offsets in bytes; 16-byte lane entries are in MFMA operand order):
//   [0, 18432)       A  fragments: 6 (row tile, k-step) pairs x 3 splits x 64 lanes
//   [18432, 30720)   QK fragments: 6 pairs x 2 splits x 64 lanes
//   [30720, 34816)   T'_ii = (I + diag(beta) A_ii)^-1 diag(beta): 4 blocks x 64 lanes,
//                    lane (g,n) holds row n, columns 4g..4g+3 (fp32)
//   [34816, 35072)   gamma_t = exp(G_t)                (fp32 x 64)
//   [35072, 35328)   w_t = exp(G_last - G_t)           (fp32 x 64)
//   [35328, 35840)   padding to whole 1 KiB blocks
constexpr int kRecA = 0, kRecQK = 18432, kRecTd = 30720, kRecGam = 34816, kRecW = 35072;
constexpr int kRecBlocks = (int)(kPrepRecordBytes / 1024);
static_assert(kPrepRecordBytes % 1024 == 0, "record must be whole 1 KiB blocks");

// Index of the (row tile mt, k-step s) pair among the six with s <= mt/2.
HAM_DEVICE constexpr int pair_index(int mt, int s) { return mt == 0 ? 0 : mt == 1 ? 1 : mt == 2 ? 2 + s : 4 + s; }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

HAM_DEVICE f32x4 mfma_bf16_k16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

HAM_DEVICE void split3x4(const float x[4], bf16x4& h, bf16x4& m, bf16x4& l) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __bf16 a, b, c;
    split3(x[i], a, b, c);
    h[i] = a; m[i] = b; l[i] = c;
  }
}

// Six-term fp32-accurate product accumulation: (ah+am+al)(bh+bm+bl), dropping the
// terms below 2^-16 relative.
template <class F, class V>
HAM_DEVICE f32x4 mma6(F mf, const V& ah, const V& am, const V& al, const V& bh, const V& bm, const V& bl, f32x4 c) {
  c = mf(am, bm, c);
  c = mf(al, bh, c);
  c = mf(ah, bl, c);
  c = mf(am, bh, c);
  c = mf(ah, bm, c);
  c = mf(ah, bh, c);
  return c;
}

// ---------------------------------------------------------------------------------
// Prep kernel: one workgroup (4 waves) per (b, h, chunk); chunks are independent.
// Decayed Gram matrices (S2), their diagonal-block inverses (S3), gamma and the
// state-update decays (S1).
template <int DK>
struct PrepSmem {
  static constexpr int KS = DK + 8;
  uint16_t K[kC * KS];
  uint16_t Q[kC * KS];
  float Ld[4][16][17];                     // diagonal 16x16 blocks of diag(beta) A
  alignas(16) float Td[4][16][20];         // (I + Ld)^-1 diag(beta)
  alignas(16) float G2[kC];
  alignas(16) float beta[kC];
};

// One (row tile mt, k-step s) fragment of a decayed Gram matrix, computed
// transposed so that the MFMA output already sits in A-operand order: lane (g,n)
// ends with entries (t = 16mt + n, j = 32s + 16h + 4g + i) for half h, i = 0..3.
template <int DK, bool kQK>
HAM_DEVICE void gram_fragment(PrepSmem<DK>& sm, char* rec, int mt, int s, int g, int n, int lane) {
  constexpr int KS = PrepSmem<DK>::KS;
  const uint16_t* rowsT = kQK ? sm.Q : sm.K;
  float val[2][4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int jt = 2 * s + hh;
    f32x4 acc = (f32x4)(0.f);
    if (jt <= mt) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const bf16x8 af = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&sm.K[(16 * jt + n) * KS + 32 * ks + 8 * g]));
        const bf16x8 bf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&rowsT[(16 * mt + n) * KS + 32 * ks + 8 * g]));
        acc = mfma_bf16(af, bf, acc);
      }
    }
    const int t = 16 * mt + n;
    const float gt = sm.G2[t];
    const f32x4 gj = *reinterpret_cast<const f32x4*>(&sm.G2[16 * jt + 4 * g]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * jt + 4 * g + i;
      const bool keep = kQK ? (j <= t) : (j < t);
      val[hh][i] = keep ? acc[i] * __builtin_amdgcn_exp2f(gt - gj[i]) : 0.f;
      if (!kQK && jt == mt) sm.Ld[mt][n][4 * g + i] = sm.beta[t] * val[hh][i];
    }
  }
  const int pi = pair_index(mt, s);
  if (kQK) {
    bf16x8 h8, m8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = val[i >> 2][i & 3];
      const __bf16 xh = to_bf16(x);
      h8[i] = xh;
      m8[i] = to_bf16(x - from_bf16(xh));
    }
    bf16x8* dst = reinterpret_cast<bf16x8*>(rec + kRecQK) + pi * 2 * kWave + lane;
    dst[0] = h8;
    dst[kWave] = m8;
  } else {
    bf16x8 h8, m8, l8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __bf16 x0, x1, x2;
      split3(val[i >> 2][i & 3], x0, x1, x2);
      h8[i] = x0; m8[i] = x1; l8[i] = x2;
    }
    bf16x8* dst = reinterpret_cast<bf16x8*>(rec + kRecA) + pi * 3 * kWave + lane;
    dst[0] = h8;
    dst[kWave] = m8;
    dst[2 * kWave] = l8;
  }
}

template <int DK>
__global__ __launch_bounds__(256) void rnn_prep_kernel(RnnArgs a) {
  using SM = PrepSmem<DK>;
  constexpr int KS = SM::KS;
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nchunk = gridDim.x;
  const int t0 = c * kC;
  const int nvalid = min(kC, a.T - t0);
  const bool readout = a.o_rnn32 != nullptr;
  char* rec = static_cast<char*>(a.prep) + ((size_t)(b * a.H + h) * nchunk + c) * kPrepRecordBytes;
  const uint16_t* kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const size_t tok0 = ((size_t)b * a.T + t0) * a.H + h;

  // stage K and Q rows (16-byte units, token-major), zero past T
  for (int u = tid; u < kC * (DK / 8); u += 256) {
    const int row = u % kC, cu = (u / kC) * 8;
    u16x8 kx = (u16x8)(0), qx = (u16x8)(0);
    if (row < nvalid) {
      const size_t off = (tok0 + (size_t)row * a.H) * DK + cu;
      kx = *reinterpret_cast<const u16x8*>(kp + off);
      if (readout) qx = *reinterpret_cast<const u16x8*>(qp + off);
    }
    *reinterpret_cast<u16x8*>(&sm.K[row * KS + cu]) = kx;
    *reinterpret_cast<u16x8*>(&sm.Q[row * KS + cu]) = qx;
  }
  if (wave == 0) {
    float gv = 0.f, bv = 0.f;
    if (lane < nvalid) {
      gv = a.g[tok0 + (size_t)lane * a.H];
      bv = a.beta[tok0 + (size_t)lane * a.H];
    }
    // inclusive prefix sum of the log decays over the chunk
    float G = gv;
#pragma unroll
    for (int off = 1; off < kC; off <<= 1) {
      const float y = __shfl_up(G, off, kWave);
      if (lane >= off) G += y;
    }
    const float Glast = __shfl(G, kC - 1, kWave);
    sm.G2[lane] = G * 1.4426950408889634f;
    sm.beta[lane] = bv;
    reinterpret_cast<float*>(rec + kRecGam)[lane] = expf(G);
    reinterpret_cast<float*>(rec + kRecW)[lane] = expf(Glast - G);
  }
  __syncthreads();

  const int nfrag = readout ? 12 : 6;
#pragma unroll
  for (int rep = 0; rep < 3; ++rep) {
    const int f = wave + rep * 4;
    if (f >= nfrag) break;
    const int pi = f % 6;
    const int mt = pi == 0 ? 0 : pi == 1 ? 1 : pi < 4 ? 2 : 3;
    const int s = pi < 2 ? 0 : (pi - 2) & 1;
    if (f < 6) gram_fragment<DK, false>(sm, rec, mt, s, g, n, lane);
    else gram_fragment<DK, true>(sm, rec, mt, s, g, n, lane);
  }
  __syncthreads();

  // inverses of the four diagonal blocks by forward substitution (lane = block, column)
  if (wave == 0) {
    const int bb = lane >> 4, cc = lane & 15;
    float colv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < r; ++j) part[j & 3] = fmaf(sm.Ld[bb][r][j], colv[j], part[j & 3]);
      colv[r] = ((r == cc) ? 1.f : 0.f) - ((part[0] + part[1]) + (part[2] + part[3]));
    }
    const float bc = sm.beta[16 * bb + cc];
#pragma unroll
    for (int r = 0; r < 16; ++r) sm.Td[bb][r][cc] = colv[r] * bc;
  }
  __syncthreads();
  {
    // lane order: entry (block i, lane (g,n)) = row n, columns 4g..4g+3
    const int i = tid >> 6;
    const f32x4 x = *reinterpret_cast<const f32x4*>(&sm.Td[i][n][4 * g]);
    reinterpret_cast<f32x4*>(rec + kRecTd)[i * kWave + lane] = x;
  }
}

// ---------------------------------------------------------------------------------
// State kernel: one workgroup = NW waves = 16*NW state columns of one head, walking
// the chunks in order.  The chunk record is streamed into LDS one chunk ahead with
// direct global-to-LDS loads; K, Q, K^T and this workgroup's V^T columns are staged
// from registers prefetched one chunk ahead.
template <int DK, int NW>
struct ChunkSmem {
  static constexpr int KS = DK + 8;        // row stride (u16) of K and Q
  static constexpr int TS = kC + 8;        // row stride (u16) of K^T and V^T
  uint16_t K[kC * KS];
  uint16_t Q[kC * KS];
  uint16_t Kt[DK * TS];
  uint16_t Vt[16 * NW * TS];               // this workgroup's V columns, transposed
  alignas(16) char rec[2][kPrepRecordBytes];
};

// Per-thread register stage of one chunk's inputs (prefetched one chunk ahead).
// K and V are fetched as (adjacent pair of elements, 8 consecutive tokens) units
// with 4-byte loads -- a wave's load instruction reads contiguous bytes of one
// token row -- so that the transposed copies K^T and V^T are written with 16-byte
// stores.  Q only needs its row-major copy (16-byte units, token-major).
template <int DK, int NW>
struct ChunkRegs {
  static constexpr int NT = 64 * NW;
  static constexpr int KU = (DK / 2) * (kC / 8);        // (d pair, token group) units of K
  static constexpr int KPT = (KU + NT - 1) / NT;
  static constexpr int QU = kC * (DK / 8);              // 16-byte units of Q
  static constexpr int QPT = (QU + NT - 1) / NT;
  static constexpr int VU = (8 * NW) * (kC / 8);        // (column pair, token group) units of V
  static constexpr int VPT = (VU + NT - 1) / NT;
  uint32_t k[KPT][8], v[VPT][8];
  u16x8 q[QPT];
};

template <int DK, int DV, int NW>
HAM_DEVICE void load_chunk(const RnnArgs& a, ChunkRegs<DK, NW>& r, int b, int h, int t0, int colbase,
                           int tid, bool readout) {
  using R = ChunkRegs<DK, NW>;
  const uint16_t* k = static_cast<const uint16_t*>(a.k);
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  const uint16_t* v = static_cast<const uint16_t*>(a.v);
  const int nvalid = min(kC, a.T - t0);
  const size_t rowstride = (size_t)a.H;                 // tokens are H rows apart
  const size_t tok0 = ((size_t)b * a.T + t0) * a.H + h;
  static_assert(R::KU % R::NT == 0 && R::VU % R::NT == 0 && R::QU % R::NT == 0, "uneven staging");
  if (nvalid == kC) {                       // full chunk: no per-load conditions
#pragma unroll
    for (int p = 0; p < R::KPT; ++p) {
      const int u = tid + p * R::NT;
      const int dp = u % (DK / 2), tg = u / (DK / 2);
      const uint16_t* src = k + (tok0 + (size_t)(tg * 8) * rowstride) * DK + 2 * dp;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        r.k[p][j] = *reinterpret_cast<const uint32_t*>(src + (size_t)j * rowstride * DK);
    }
#pragma unroll
    for (int p = 0; p < R::VPT; ++p) {
      const int u = tid + p * R::NT;
      const int cp = u % (8 * NW), tg = u / (8 * NW);
      const uint16_t* src = v + (tok0 + (size_t)(tg * 8) * rowstride) * DV + colbase + 2 * cp;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        r.v[p][j] = *reinterpret_cast<const uint32_t*>(src + (size_t)j * rowstride * DV);
    }
    if (readout) {
#pragma unroll
      for (int p = 0; p < R::QPT; ++p) {
        const int u = tid + p * R::NT;
        const int row = u % kC, cu = (u / kC) * 8;
        r.q[p] = *reinterpret_cast<const u16x8*>(q + (tok0 + row * rowstride) * DK + cu);
      }
    }
  } else {                                  // tail chunk: zero the rows past T
#pragma unroll
    for (int p = 0; p < R::KPT; ++p) {
      const int u = tid + p * R::NT;
      const int dp = u % (DK / 2), tg = u / (DK / 2);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = tg * 8 + j;
        r.k[p][j] = 0u;
        if (row < nvalid)
          r.k[p][j] = *reinterpret_cast<const uint32_t*>(k + (tok0 + row * rowstride) * DK + 2 * dp);
      }
    }
#pragma unroll
    for (int p = 0; p < R::VPT; ++p) {
      const int u = tid + p * R::NT;
      const int cp = u % (8 * NW), tg = u / (8 * NW);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = tg * 8 + j;
        r.v[p][j] = 0u;
        if (row < nvalid)
          r.v[p][j] = *reinterpret_cast<const uint32_t*>(v + (tok0 + row * rowstride) * DV + colbase + 2 * cp);
      }
    }
#pragma unroll
    for (int p = 0; p < R::QPT; ++p) {
      const int u = tid + p * R::NT;
      const int row = u % kC, cu = (u / kC) * 8;
      r.q[p] = (u16x8)(0);
      if (readout && row < nvalid)
        r.q[p] = *reinterpret_cast<const u16x8*>(q + (tok0 + row * rowstride) * DK + cu);
    }
  }
}

template <int DK, int NW>
HAM_DEVICE void store_chunk(ChunkSmem<DK, NW>& sm, const ChunkRegs<DK, NW>& r, int tid) {
  using R = ChunkRegs<DK, NW>;
  using SM = ChunkSmem<DK, NW>;
#pragma unroll
  for (int p = 0; p < R::KPT; ++p) {
    const int u = tid + p * R::NT;
    const int dp = u % (DK / 2), tg = u / (DK / 2);
    u16x8 lo, hi;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo[j] = (uint16_t)(r.k[p][j] & 0xffffu);
      hi[j] = (uint16_t)(r.k[p][j] >> 16);
      *reinterpret_cast<uint32_t*>(&sm.K[(tg * 8 + j) * SM::KS + 2 * dp]) = r.k[p][j];
    }
    *reinterpret_cast<u16x8*>(&sm.Kt[(2 * dp) * SM::TS + tg * 8]) = lo;
    *reinterpret_cast<u16x8*>(&sm.Kt[(2 * dp + 1) * SM::TS + tg * 8]) = hi;
  }
#pragma unroll
  for (int p = 0; p < R::VPT; ++p) {
    const int u = tid + p * R::NT;
    const int cp = u % (8 * NW), tg = u / (8 * NW);
    u16x8 lo, hi;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      lo[j] = (uint16_t)(r.v[p][j] & 0xffffu);
      hi[j] = (uint16_t)(r.v[p][j] >> 16);
    }
    *reinterpret_cast<u16x8*>(&sm.Vt[(2 * cp) * SM::TS + tg * 8]) = lo;
    *reinterpret_cast<u16x8*>(&sm.Vt[(2 * cp + 1) * SM::TS + tg * 8]) = hi;
  }
#pragma unroll
  for (int p = 0; p < R::QPT; ++p) {
    const int u = tid + p * R::NT;
    const int row = u % kC, cu = (u / kC) * 8;
    *reinterpret_cast<u16x8*>(&sm.Q[row * SM::KS + cu]) = r.q[p];
  }
}

template <int DK, int DV, int NW>
__global__ __launch_bounds__(64 * NW) void rnn_chunked_kernel(RnnArgs a) {
  using SM = ChunkSmem<DK, NW>;
  constexpr int KS = SM::KS, TS = SM::TS;
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
  auto mf32 = [](const bf16x8& x, const bf16x8& y, const f32x4& c) { return mfma_bf16(x, y, c); };
  auto mf16 = [](const bf16x4& x, const bf16x4& y, const f32x4& c) { return mfma_bf16_k16(x, y, c); };

  // state tiles: S[16*mt + 4g + i][col]
  f32x4 S[MT];
  const size_t sbase = (size_t)bh * DK * DV;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[mt][i] = a.S0 ? a.S0[sbase + (size_t)(16 * mt + 4 * g + i) * DV + col] : 0.f;

  const int nchunk = (a.T + kC - 1) / kC;
  const char* recs = static_cast<const char*>(a.prep) + (size_t)bh * nchunk * kPrepRecordBytes;
  // direct global-to-LDS copy of one chunk record (1 KiB per wave instruction); the
  // builtin exists only in the device compilation pass
#if defined(__HIP_DEVICE_COMPILE__)
#define HAM_FETCH_RECORD(BUF, REC)                                                         \
  for (int blk = wave; blk < kRecBlocks; blk += NW)                                        \
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>((REC) + blk * 1024 + lane * 16), \
                                     &sm.rec[(BUF)][blk * 1024], 16, 0, 0)
#else
#define HAM_FETCH_RECORD(BUF, REC) (void)(REC)
#endif
  ChunkRegs<DK, NW> regs;
  load_chunk<DK, DV, NW>(a, regs, b, h, 0, colbase, tid, readout);
  HAM_FETCH_RECORD(0, recs);

  for (int c = 0; c < nchunk; ++c) {
    const int t0 = c * kC;
    const int nvalid = min(kC, a.T - t0);
    __builtin_amdgcn_s_waitcnt(0);            // this chunk's registers and record have arrived
    __syncthreads();                          // the previous chunk's LDS readers are done
    store_chunk<DK, NW>(sm, regs, tid);
    if (c + 1 < nchunk) {
      load_chunk<DK, DV, NW>(a, regs, b, h, t0 + kC, colbase, tid, readout);
      HAM_FETCH_RECORD((c + 1) & 1, recs + (size_t)(c + 1) * kPrepRecordBytes);
    }
    __syncthreads();
    const char* rec = sm.rec[c & 1];
    const bf16x8* Af = reinterpret_cast<const bf16x8*>(rec + kRecA);
    const bf16x8* QKf = reinterpret_cast<const bf16x8*>(rec + kRecQK);
    const f32x4* Tdf = reinterpret_cast<const f32x4*>(rec + kRecTd);
    const float* gam = reinterpret_cast<const float*>(rec + kRecGam);
    const float* wdec = reinterpret_cast<const float*>(rec + kRecW);

    // ---- Y_K = K S, Y_Q = Q S ----
    f32x4 P[4], O[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      P[mt] = (f32x4)(0.f);
      O[mt] = (f32x4)(0.f);
    }
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      bf16x8 sh, smd, sl;
      split_pair3(S[2 * ks], S[2 * ks + 1], sh, smd, sl);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint16_t* kr = &sm.K[(16 * mt + n) * KS + 32 * ks + 4 * g];
        const bf16x8 af = frag2(kr, kr + 16);
        P[mt] = mfma_bf16(af, sl, P[mt]);
        P[mt] = mfma_bf16(af, smd, P[mt]);
        P[mt] = mfma_bf16(af, sh, P[mt]);
        if (readout) {
          const uint16_t* qr = &sm.Q[(16 * mt + n) * KS + 32 * ks + 4 * g];
          const bf16x8 qf = frag2(qr, qr + 16);
          O[mt] = mfma_bf16(qf, smd, O[mt]);
          O[mt] = mfma_bf16(qf, sh, O[mt]);
        }
      }
    }
    // X = V - gamma K S ; P, O start as gamma K S, gamma Q S
    f32x4 X[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 gm = *reinterpret_cast<const f32x4*>(&gam[16 * mt + 4 * g]);
      const u16x4 v4 = *reinterpret_cast<const u16x4*>(&sm.Vt[vcol * TS + 16 * mt + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float vv = bf16_to_f32(v4[i]);
        P[mt][i] *= gm[i];
        O[mt][i] *= gm[i];
        X[mt][i] = vv - P[mt][i];
      }
    }

    // ---- block forward substitution: D_i = T'_ii (X_i - sum_{j<i} A_ij D_j) ----
    // dB[s][*]: B-operand fragments (k-step s) of the D blocks solved so far.
    bf16x8 dB[2][3];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int z = 0; z < 3; ++z) dB[s][z] = (bf16x8)(0);
    f32x4 D[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 R = (f32x4)(0.f);
#pragma unroll
      for (int s = 0; s <= (i - 1) / 2 && i > 0; ++s) {
        const int pi = pair_index(i, s);
        R = mma6(mf32, Af[(pi * 3 + 0) * kWave + lane], Af[(pi * 3 + 1) * kWave + lane],
                 Af[(pi * 3 + 2) * kWave + lane], dB[s][0], dB[s][1], dB[s][2], R);
      }
      float rhs[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) rhs[e] = X[i][e] - R[e];
      bf16x4 rh, rm, rl, th, tm, tl;
      split3x4(rhs, rh, rm, rl);
      const f32x4 tv = Tdf[i * kWave + lane];
      const float tva[4] = {tv[0], tv[1], tv[2], tv[3]};
      split3x4(tva, th, tm, tl);
      D[i] = mma6(mf16, th, tm, tl, rh, rm, rl, (f32x4)(0.f));
      // the diagonal block's share of A D, for the prediction P
      const int half = i & 1;
      bf16x4 dh4, dm4, dl4;
      const float dva[4] = {D[i][0], D[i][1], D[i][2], D[i][3]};
      split3x4(dva, dh4, dm4, dl4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dB[i >> 1][0][4 * half + e] = dh4[e];
        dB[i >> 1][1][4 * half + e] = dm4[e];
        dB[i >> 1][2][4 * half + e] = dl4[e];
      }
      const int pd = pair_index(i, i >> 1);
      const bf16x8 afh = Af[(pd * 3 + 0) * kWave + lane];
      const bf16x8 afm = Af[(pd * 3 + 1) * kWave + lane];
      const bf16x8 afl = Af[(pd * 3 + 2) * kWave + lane];
      bf16x4 ah4, am4, al4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ah4[e] = afh[4 * half + e];
        am4[e] = afm[4 * half + e];
        al4[e] = afl[4 * half + e];
      }
      P[i] = mma6(mf16, ah4, am4, al4, dh4, dm4, dl4, P[i] + R);
    }

    // ---- readout O += (Gamma o Q K^T o lower_incl) D  (bf16 outputs: 3 terms) ----
    if (readout) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int s = 0; s <= (mt >> 1); ++s) {
          const int pi = pair_index(mt, s);
          const bf16x8 qh = QKf[(pi * 2 + 0) * kWave + lane], qm = QKf[(pi * 2 + 1) * kWave + lane];
          O[mt] = mfma_bf16(qm, dB[s][0], O[mt]);
          O[mt] = mfma_bf16(qh, dB[s][1], O[mt]);
          O[mt] = mfma_bf16(qh, dB[s][0], O[mt]);
        }
    }

    // ---- score partials of this 16-column slice, and the readout ----
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const u16x4 v4 = *reinterpret_cast<const u16x4*>(&sm.Vt[vcol * TS + 16 * mt + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * mt + 4 * g + i;
        const float vr = bf16_to_f32(v4[i]);
        const float pv = row16_sum(P[mt][i] * vr);
        const float pp = row16_sum(P[mt][i] * P[mt][i]);
        const float vv = row16_sum(vr * vr);
        if (t < nvalid) {
          if (n == 0)
            a.score[((size_t)bh * a.T + t0 + t) * NSL + slice] = make_float4(pv, pp, vv, 0.f);
          if (readout)
            a.o_rnn32[(((size_t)b * a.T + t0 + t) * a.H + h) * DV + col] = O[mt][i];
        }
      }
    }

    // ---- S <- gamma_C S + K^T diag(exp(G_C - G)) D ----
    bf16x8 eh[2], em[2], el[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float w0[4], w1[4];
      const f32x4 wa = *reinterpret_cast<const f32x4*>(&wdec[32 * s + 4 * g]);
      const f32x4 wb = *reinterpret_cast<const f32x4*>(&wdec[32 * s + 16 + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0[i] = wa[i];
        w1[i] = wb[i];
      }
      split_pair3(D[2 * s], D[2 * s + 1], eh[s], em[s], el[s], w0, w1);
    }
    const float gl = gam[kC - 1];
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
#undef HAM_FETCH_RECORD
}

template <int DK, int DV, int NW>
hipError_t launch_t(const RnnArgs& a, hipStream_t s) {
  const int nchunk = (a.T + kC - 1) / kC;
  hipLaunchKernelGGL((rnn_prep_kernel<DK>), dim3(nchunk, a.H, a.B), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(DV / (16 * NW), a.H, a.B);
  hipLaunchKernelGGL((rnn_chunked_kernel<DK, DV, NW>), grid, dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

// Four waves (64 state columns) per workgroup.
template <int DK, int DV>
hipError_t launch_dims(const RnnArgs& a, hipStream_t s) { return launch_t<DK, DV, 4>(a, s); }

}  // namespace chunked

using chunked::launch_dims;

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
