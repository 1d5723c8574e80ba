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
// (fp32 accumulate).  Every product with an fp32 operand (S, D, A, T') on the path
// of the state and the routing score splits the fp32 value into three bf16 terms
// hi+mid+lo (24 significant bits) and keeps the cross terms down to 2^-16 relative,
// which is fp32-level accuracy; the routing score needs it.  The readout O only
// feeds bf16 outputs: Q S takes the first two terms of S (the mix normalises each
// readout row, so a row of small norm needs the product accurate relative to the
// row), and (Gamma o Q K^T) D the leading term of Gamma o Q K^T against two terms of D
// (about 2^-9 relative, the size of the bf16 rounding of the outputs themselves).
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
// offsets in bytes; lane entries are in MFMA operand order).  A and Gamma o QK^T are
// stored as (row tile mt, 32-column step s) pairs with s <= mt/2; the pairs (0,0)
// and (2,1) reach past the diagonal, so only their first 16 columns are nonzero and
// they are kept as 16-wide fragments (8 bytes per lane), as is the first row tile
// of each 32x32 block inverse.
//   [0, 12288)       A, full pairs (1,0) (2,0) (3,0) (3,1): 3 bf16 terms x 64 lanes x 16 B
//   [12288, 15360)   A, half pairs (0,0) (2,1): 3 terms x 64 lanes x 8 B
//   [15360, 19456)   Gamma o QK^T, full pairs: 1 term x 64 x 16 B
//   [19456, 20480)   Gamma o QK^T, half pairs: 1 term x 64 x 8 B
//   [20480, 26624)   T'_I = (I + diag(beta) A_II)^-1 diag(beta), 32x32 block I = 0, 1,
//                    second row tile: 3 terms x 64 x 16 B
//   [26624, 29696)   first row tile of T'_I (its 16 nonzero columns): 3 terms x 64 x 8 B
//   [29696, 29952)   gamma_t = exp(G_t)                (fp32 x 64)
//   [29952, 30208)   w_t = exp(G_last - G_t)           (fp32 x 64)
//   [30208, 30720)   padding to whole 1 KiB blocks
constexpr int kRecA = 0, kRecAh = 12288, kRecQK = 15360, kRecQKh = 19456, kRecT = 20480, kRecTh = 26624,
              kRecGam = 29696, kRecW = 29952;
static_assert(kPrepRecordBytes % 1024 == 0 && kRecW + 256 <= (int)kPrepRecordBytes, "record layout");

// Index of the (row tile mt, k-step s) pair among the six with s <= mt/2.
HAM_DEVICE constexpr int pair_index(int mt, int s) { return mt == 0 ? 0 : mt == 1 ? 1 : mt == 2 ? 2 + s : 4 + s; }
// pairs (0,0) and (2,1) have 16 nonzero columns; slots within the full / half groups
HAM_DEVICE constexpr bool pair_is_half(int pi) { return pi == 0 || pi == 3; }
HAM_DEVICE constexpr int full_slot(int pi) { return pi == 1 ? 0 : pi == 2 ? 1 : pi == 4 ? 2 : 3; }
HAM_DEVICE constexpr int half_slot(int pi) { return pi == 0 ? 0 : 1; }

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
// About 23 KiB at d_k = 128: K rows are unpadded with their 16-byte chunks XOR-swizzled
// by row, the Q rows of the Q K^T products go from memory straight into registers, and
// the block-inverse scratch reuses K's space once the Gram fragments are done.
template <int DK>
struct PrepSmem {
  static constexpr int NCH = DK / 8;       // 16-byte chunks per K row
  // element offset of chunk c of row r: the 16 rows one fragment read touches fall in
  // different banks
  HAM_DEVICE static int at(int r, int c) { return r * DK + ((c ^ (r & (NCH - 1))) << 3); }
  union {
    uint16_t K[kC * DK];                   // until the Gram fragments are done
    struct {
      alignas(16) float Td[4][16][20];     // (I + Ld)^-1 diag(beta)
      float W[2][16][17];                  // Aoff T'_{2I}
      alignas(16) float Off[2][16][20];    // -T'_{2I+1} Aoff T'_{2I}
    };
  };
  float Ld[4][16][17];                     // diagonal 16x16 blocks of diag(beta) A
  float Aoff[2][16][17];                   // A blocks (rows 16-block 2I+1, cols 16-block 2I)
  alignas(16) float G2[kC];
  alignas(16) float beta[kC];
};

// One (row tile mt, k-step s) fragment of a decayed Gram matrix, computed
// transposed so that the MFMA output already sits in A-operand order: lane (g,n)
// ends with entries (t = 16mt + n, j = 32s + 16h + 4g + i) for half h, i = 0..3.
template <int DK, bool kQK>
HAM_DEVICE void gram_fragment(PrepSmem<DK>& sm, char* rec, int mt, int s, int g, int n, int lane,
                              const u16x8 (&qrow)[DK / 32]) {
  using SM = PrepSmem<DK>;
  float val[2][4];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int jt = 2 * s + hh;
    f32x4 acc = (f32x4)(0.f);
    if (jt <= mt) {
#pragma unroll
      for (int ks = 0; ks < DK / 32; ++ks) {
        const bf16x8 af = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&sm.K[SM::at(16 * jt + n, 4 * ks + g)]));
        // K K^T reads row 16 mt + n of K from LDS; Q K^T takes that row of Q from registers
        const bf16x8 bf = kQK ? __builtin_bit_cast(bf16x8, qrow[ks])
                              : __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&sm.K[SM::at(16 * mt + n, 4 * ks + g)]));
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
      if (!kQK && (mt & 1) && jt == mt - 1) sm.Aoff[mt >> 1][n][4 * g + i] = val[hh][i];
    }
  }
  const int pi = pair_index(mt, s);
  if (kQK) {
    bf16x8 h8;                                  // the readout's one term
#pragma unroll
    for (int i = 0; i < 8; ++i) h8[i] = to_bf16(val[i >> 2][i & 3]);
    if (pair_is_half(pi)) {
      bf16x4* dst = reinterpret_cast<bf16x4*>(rec + kRecQKh) + half_slot(pi) * kWave + lane;
      dst[0] = __builtin_shufflevector(h8, h8, 0, 1, 2, 3);
    } else {
      bf16x8* dst = reinterpret_cast<bf16x8*>(rec + kRecQK) + full_slot(pi) * kWave + lane;
      dst[0] = h8;
    }
  } else {
    bf16x8 h8, m8, l8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __bf16 x0, x1, x2;
      split3(val[i >> 2][i & 3], x0, x1, x2);
      h8[i] = x0; m8[i] = x1; l8[i] = x2;
    }
    if (pair_is_half(pi)) {
      bf16x4* dst = reinterpret_cast<bf16x4*>(rec + kRecAh) + half_slot(pi) * 3 * kWave + lane;
      dst[0] = __builtin_shufflevector(h8, h8, 0, 1, 2, 3);
      dst[kWave] = __builtin_shufflevector(m8, m8, 0, 1, 2, 3);
      dst[2 * kWave] = __builtin_shufflevector(l8, l8, 0, 1, 2, 3);
    } else {
      bf16x8* dst = reinterpret_cast<bf16x8*>(rec + kRecA) + full_slot(pi) * 3 * kWave + lane;
      dst[0] = h8;
      dst[kWave] = m8;
      dst[2 * kWave] = l8;
    }
  }
}

template <int DK>
__global__ __launch_bounds__(256) void rnn_prep_kernel(RnnArgs a) {
  using SM = PrepSmem<DK>;
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

  // stage K and Q rows (16-byte units, token-major), zero past T: every load of the
  // thread is issued before the first LDS store, so the tile costs one memory latency
  constexpr int NU = kC * (DK / 8) / 256;
  static_assert(kC * (DK / 8) % 256 == 0, "staging units must split evenly over the threads");
  u16x8 kx[NU];
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int u = tid + 256 * i, row = u % kC, cu = (u / kC) * 8;
    kx[i] = (u16x8)(0);
    if (row < nvalid) {
      const size_t off = (tok0 + (size_t)row * a.H) * DK + cu;
      kx[i] = *reinterpret_cast<const u16x8*>(kp + off);
    }
  }
  // The Q K^T fragments this wave computes (fragments f = wave + 4 rep with f >= 6 of
  // the twelve below) take their Q rows straight from memory into registers, in the
  // B-operand order of the products: lane (g, n) holds row 16 mt + n, d = 32 ks + 8g ..
  // +7.  Q never goes through LDS, and the block-inverse scratch reuses K's space, so a
  // workgroup needs about 23 KiB and five share a CU.
  constexpr int KSD = DK / 32;
  auto frag_mt = [](int pi) { return pi == 0 ? 0 : pi == 1 ? 1 : pi < 4 ? 2 : 3; };
  u16x8 qrow[2][KSD];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int f = wave + 4 * (rr + 1);
    const int row = 16 * frag_mt(f % 6) + n;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      qrow[rr][ks] = (u16x8)(0);
      if (readout && f >= 6 && row < nvalid)
        qrow[rr][ks] = *reinterpret_cast<const u16x8*>(qp + (tok0 + (size_t)row * a.H) * DK + 32 * ks + 8 * g);
    }
  }
#pragma unroll
  for (int i = 0; i < NU; ++i) {
    const int u = tid + 256 * i, row = u % kC, cu = (u / kC) * 8;
    *reinterpret_cast<u16x8*>(&sm.K[SM::at(row, cu >> 3)]) = kx[i];
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
    if (f < 6) gram_fragment<DK, false>(sm, rec, mt, s, g, n, lane, qrow[0]);
    else gram_fragment<DK, true>(sm, rec, mt, s, g, n, lane, qrow[rep == 1 ? 0 : 1]);
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
  // 32-token diagonal blocks: T'_I = [[T'_{2I}, 0], [-T'_{2I+1} A_{2I+1,2I} T'_{2I}, T'_{2I+1}]]
  // (block inverse of the unit lower-triangular I + diag(beta) A, times diag(beta))
  for (int idx = tid; idx < 512; idx += 256) {
    const int I = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
    float acc = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) acc = fmaf(sm.Aoff[I][r][k2], sm.Td[2 * I][k2][cc], acc);
    sm.W[I][r][cc] = acc;
  }
  __syncthreads();
  for (int idx = tid; idx < 512; idx += 256) {
    const int I = idx >> 8, r = (idx >> 4) & 15, cc = idx & 15;
    float acc = 0.f;
#pragma unroll
    for (int k2 = 0; k2 < 16; ++k2) acc = fmaf(sm.Td[2 * I + 1][r][k2], sm.W[I][k2][cc], acc);
    sm.Off[I][r][cc] = -acc;
  }
  __syncthreads();
  {
    // wave (I, r): row tile r of block I; lane (g,n) holds row n, columns 4g..4g+3
    // (k-slots 0..3) and 16+4g..16+4g+3 (k-slots 4..7) of the 32 block columns
    const int I = wave >> 1, r = wave & 1;
    if (r == 0) {                         // [T'_{2I}, 0]: the 16 nonzero columns
      const f32x4 lo = *reinterpret_cast<const f32x4*>(&sm.Td[2 * I][n][4 * g]);
      const float xa[4] = {lo[0], lo[1], lo[2], lo[3]};
      bf16x4 th, tm, tl;
      split3x4(xa, th, tm, tl);
      bf16x4* dst = reinterpret_cast<bf16x4*>(rec + kRecTh) + (I * 3) * kWave + lane;
      dst[0] = th;
      dst[kWave] = tm;
      dst[2 * kWave] = tl;
    } else {                              // [-T'_{2I+1} A T'_{2I}, T'_{2I+1}]
      const f32x4 lo = *reinterpret_cast<const f32x4*>(&sm.Off[I][n][4 * g]);
      const f32x4 hi = *reinterpret_cast<const f32x4*>(&sm.Td[2 * I + 1][n][4 * g]);
      bf16x8 th, tm, tl;
      split_pair3(lo, hi, th, tm, tl);
      bf16x8* dst = reinterpret_cast<bf16x8*>(rec + kRecT) + (I * 3) * kWave + lane;
      dst[0] = th;
      dst[kWave] = tm;
      dst[2 * kWave] = tl;
    }
  }
}

// ---------------------------------------------------------------------------------
// State kernel: one workgroup = NW waves = 16*NW state columns of one head, walking
// the chunks in order.  Each chunk's K, Q, the workgroup's V columns and the chunk
// record are copied into LDS with direct global-to-LDS loads, one chunk ahead, into
// a two-stage buffer.  K, Q and V stay row-major with their 16-byte chunks
// XOR-swizzled by row; K^T and V-column fragments come from the transposing LDS
// read (for a 16-lane group, lane r addresses X[k0 + r/4][d0 + 4(r mod 4) .. +3]
// and lane i receives X[k0 + j][d0 + i], j = 0..3).
typedef short short4s __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 8-byte transposing LDS read (for a 16-lane group, lane r addresses
// X[k0 + r/4][d0 + 4(r mod 4) .. +3] and lane i receives X[k0 + j][d0 + i], j = 0..3).
HAM_DEVICE u32x2 lds_tr16(const char* base, int byte_off) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) short4s lds_short4;
  const short4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4*)((__attribute__((address_space(3))) const char*)base + byte_off));
  return __builtin_bit_cast(u32x2, r);
#else
  (void)base; (void)byte_off;
  return u32x2{};
#endif
}

HAM_DEVICE u32x4 cat(const u32x2& a, const u32x2& b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3); }
HAM_DEVICE bf16x8 as8(const u32x4& x) { return __builtin_bit_cast(bf16x8, x); }
HAM_DEVICE bf16x4 as4(const u32x2& x) { return __builtin_bit_cast(bf16x4, x); }

// two floats -> two bf16 (nearest even) in one dword, low half first
HAM_DEVICE uint32_t pk_bf16(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){x0, x1}, bf16x2));
}
// (x0, x1) = hi + mid + lo elementwise, each term a packed bf16 pair; the
// residuals are exact in fp32.
HAM_DEVICE void split3_pk(float x0, float x1, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = pk_bf16(x0, x1);
  float r0 = x0 - __uint_as_float(h << 16), r1 = x1 - __uint_as_float(h & 0xffff0000u);
  m = pk_bf16(r0, r1);
  r0 -= __uint_as_float(m << 16);
  r1 -= __uint_as_float(m & 0xffff0000u);
  l = pk_bf16(r0, r1);
}
// four values (one accumulator's rows) -> three 4-element bf16 terms
HAM_DEVICE void split4(const f32x4& x, u32x2& h, u32x2& m, u32x2& l) {
  uint32_t h0, m0, l0, h1, m1, l1;
  split3_pk(x[0], x[1], h0, m0, l0);
  split3_pk(x[2], x[3], h1, m1, l1);
  h = u32x2{h0, h1};
  m = u32x2{m0, m1};
  l = u32x2{l0, l1};
}

template <int DK, int NW, bool LEAN = false>
struct ChunkLayout {
  static constexpr int RK = DK * 2;                  // bytes per K / Q row
  static constexpr int NCK = DK / 8;                 // 16-byte chunks per K / Q row
  static constexpr int RV = NW * 16 * 2;             // bytes per V-slice row
  static constexpr int NCV = NW * 2;
  static constexpr int KB = kC * RK, VB = kC * RV;
  // A stage holds K, Q, the workgroup's V columns and the chunk record.  Up to
  // d_k = 128 two whole stages fit in LDS.  At d_k = 256 (SPLIT) they would need
  // 214 KB, so only K keeps two stages (it is read at both ends of a chunk); Q, V
  // and the record have one buffer each, reloaded for the next chunk as soon as the
  // last read of the current one is behind a barrier (139 KB).  LEAN asks for the
  // same layout at d_k <= 128 (86 KB at 128), so that an attention workgroup fits
  // on the CU beside the state pass; its extra barriers cost about 15% alone.
  static constexpr bool SPLIT = LEAN || DK > 128;
  static constexpr int OFF_K = 0, OFF_Q = SPLIT ? 0 : KB, OFF_V = OFF_Q + KB, OFF_R = OFF_V + VB;
  static constexpr int STAGE = SPLIT ? KB : OFF_R + (int)kPrepRecordBytes;
  static constexpr int SINGLE = SPLIT ? OFF_R + (int)kPrepRecordBytes : 16;   // Q, V, record
  static constexpr int KI = KB / 1024 / NW;          // 1 KiB loads per wave: K (and Q), V
  static constexpr int VI = VB / 1024 / NW;
  static constexpr int RI = (int)(kPrepRecordBytes / 1024);
  static_assert(KB % (1024 * NW) == 0 && VB % (1024 * NW) == 0, "tiles must split evenly over the waves");
  static_assert(kPrepRecordBytes % 1024 == 0, "record must be whole 1 KiB blocks");
  // Byte offset of 16-byte chunk c of row r of a K / Q tile and of a V tile.  The
  // chunks are XOR-swizzled by the row.  K and Q are read two ways: 16-byte row
  // fragments (8 consecutive rows per LDS pass, same chunk) and, for K, transposing
  // 8-byte reads (4 consecutive rows x 4 consecutive chunks per pass).  Taking the
  // row's low three bits rotated by one keeps the first conflict free and the second
  // at two ways, the least a fixed half-chunk allows (the plain row bits gave four).
  // V is read transposed only: 2 (r mod 4) spreads 4 rows x 2 chunks over all banks.
  HAM_DEVICE static int swzk(int r) { return (r & (NCK - 1) & ~7) | ((r & 1) << 2) | ((r >> 1) & 3); }
  HAM_DEVICE static int koff(int r, int c) { return r * RK + ((c ^ swzk(r)) << 4); }
  HAM_DEVICE static int voff(int r, int c) { return r * RV + ((c ^ (2 * (r & (NCV / 2 - 1)))) << 4); }
};

// MODE 0: the full pass (score partials; readout when RO).  MODE 1: the final state
// only.  MODE 2: the homogeneous pass (V = 0 from S0 = I, DV = DK), whose final
// "state" is the product of the chunk transitions of a segment.  With a.seg_chunks
// set, the grid covers several segments of the chunk sequence (see RnnArgs).
// VAR (full pass only): bit 0 leaves out the score partials (the routing scores are
// the caller's, from a learned router); bit 1 takes the LEAN LDS layout.
constexpr int kVarNoScore = 1, kVarLean = 2;
template <int DK, int DV, int NW, bool RO, int MODE, int VAR = 0>
__global__ __launch_bounds__(64 * NW) void rnn_chunked_kernel(RnnArgs a) {
  static_assert(MODE == 0 || !RO, "the readout belongs to the full pass");
  static_assert(MODE == 0 || VAR == 0, "variants of the full pass only");
  static_assert(MODE != 2 || DK == DV, "the transition is dk x dk");
  using LY = ChunkLayout<DK, NW, (VAR & kVarLean) != 0>;
  constexpr int MT = DK / 16;     // 16-row tiles of S
  constexpr int KSD = DK / 32;    // 32-wide k-steps over d
  constexpr int NSL = DV / (16 * NW);   // score slices per token: one per column block
  // Two stages as separate LDS objects: the chunk loop is unrolled by two, so
  // every access names its stage statically and the compiler can tell that reads
  // of the current stage do not depend on the direct loads into the other one.
  __shared__ __attribute__((aligned(16))) char stage0[LY::STAGE];
  __shared__ __attribute__((aligned(16))) char stage1[LY::STAGE];
  __shared__ __attribute__((aligned(16))) char single[LY::SINGLE];
  // Score partials of the waves' 16-column slices, two chunks deep: a chunk's are
  // summed over the workgroup's waves after the next chunk's barrier, so one float4
  // per token and column block goes to memory.
  constexpr bool kScore = MODE == 0 && !(VAR & kVarNoScore);
  static_assert(NW * 16 == kC, "one wave per 16 tokens of a chunk in the score sums");
  __shared__ __attribute__((aligned(16))) float4 sred[kScore ? 2 * NW * kC : 1];

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  // 1-D grid of (head, column block) pairs, renumbered so that the column blocks
  // of one head run on the same XCD and share its L2 (they read the same K, Q and
  // chunk records).
  constexpr int NCB = DV / (16 * NW);                       // column blocks per head
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int cb = lin % NCB, rest = lin / NCB;
  const int bh = rest % (a.B * a.H), seg = rest / (a.B * a.H);
  const int h = bh % a.H, b = bh / a.H;
  const int colbase = cb * 16 * NW;
  const int col = colbase + wave * 16 + n;

  // State tiles: element i of tile mt in lane (g, n) is S[srow(mt, g, i)][col] with
  // srow = 32 (mt/2) + 8g + 4 (mt mod 2) + i.  With this row order the k-slots
  // 8g..8g+7 of a 32-row step (tiles 2ks, 2ks+1) are the consecutive rows
  // 32ks + 8g .. +7, so the matching K and Q operands are single 16-byte reads.
  auto srow = [&](int mt, int i) { return 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i; };
  f32x4 S[MT];
  const size_t sbase = (size_t)bh * DK * DV;
  const size_t soff = (size_t)seg * a.seg_stride;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) S[mt][i] = (MODE == 2 && srow(mt, i) == col) ? 1.f : 0.f;
  if (MODE != 2 && a.S0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] = a.S0[soff + sbase + (size_t)srow(mt, i) * DV + col];
  }

  const int nchunk = (a.T + kC - 1) / kC;
  const int c_begin = a.seg_chunks ? seg * a.seg_chunks : 0;
  const int c_end = a.seg_chunks ? min(nchunk, c_begin + a.seg_chunks) : nchunk;
  const char* recs = static_cast<const char*>(a.prep) + (size_t)bh * nchunk * kPrepRecordBytes;
  const char* kbase = static_cast<const char*>(a.k);
  const char* qbase = static_cast<const char*>(a.q);
  const char* vbase = static_cast<const char*>(a.v);

  // Direct loads of chunk cc into the stage dst.  Wave w issues the 1 KiB blocks
  // w, w + NW, ... of each tile; lane
  // l writes the 16 bytes at 16 l of the block.  The source offset of a lane (bytes
  // from the chunk's first token row of this head) depends on the chunk only through
  // the clamp of rows past T to the last valid token (finite values whose write
  // vectors are zero because beta = 0 there), so full chunks reuse precomputed ones.
  auto k_off = [&](int j, int tlast) {
    const int tp = (wave + NW * j) * 1024 + lane * 16;
    const int r = tp / LY::RK, c = ((tp % LY::RK) >> 4) ^ LY::swzk(r);
    return (uint32_t)(min(r, tlast) * a.H * (DK * 2) + c * 16);
  };
  auto v_off = [&](int j, int tlast) {
    const int tp = (wave + NW * j) * 1024 + lane * 16;
    const int r = tp / LY::RV, c = ((tp % LY::RV) >> 4) ^ (2 * (r & (LY::NCV / 2 - 1)));
    return (uint32_t)(min(r, tlast) * a.H * (DV * 2) + colbase * 2 + c * 16);
  };
  uint32_t koff[LY::KI], voff[LY::VI];
#pragma unroll
  for (int j = 0; j < LY::KI; ++j) koff[j] = k_off(j, kC - 1);
#pragma unroll
  for (int j = 0; j < LY::VI; ++j) voff[j] = v_off(j, kC - 1);

  // The LDS buffers of a stage: K, Q, V and the record (with SPLIT, K from the stage
  // and the other three from the single buffer).
  auto kbuf = [&](char* st) { return st + LY::OFF_K; };
  auto qbuf = [&](char* st) { return (LY::SPLIT ? single : st) + LY::OFF_Q; };
  auto vbuf = [&](char* st) { return (LY::SPLIT ? single : st) + LY::OFF_V; };
  auto rbuf = [&](char* st) { return (LY::SPLIT ? single : st) + LY::OFF_R; };
  // part 1: K (and, without SPLIT, Q and V) tiles; part 2: the chunk record; part 4
  // (SPLIT): Q and V tiles.  The parts are issued at different points of the chunk
  // (measured: issuing all loads at once stalls the loop more than spreading them).
  auto issue_chunk = [&](int cc, char* dst, int part) {
    const int t0 = cc * kC;
    const size_t tok0 = ((size_t)b * a.T + t0) * a.H + h;
    const char* kc = kbase + tok0 * (DK * 2);
    const char* qc = qbase + tok0 * (DK * 2);
    const char* vc = vbase + tok0 * (DV * 2);
    const char* rc = recs + (size_t)cc * kPrepRecordBytes;
    const uint32_t lo = (uint32_t)lane * 16u;
    const bool full = t0 + kC <= a.T;
#if defined(__HIP_DEVICE_COMPILE__)
    const bool kq = LY::SPLIT ? (part & 4) != 0 : (part & 1) != 0;   // Q and V go with this part
    if (part & 1) {
#pragma unroll
    for (int j = 0; j < LY::KI; ++j) {
      const uint32_t ko = full ? koff[j] : k_off(j, a.T - 1 - t0);
      const int blk = (wave + NW * j) * 1024;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kc + ko), kbuf(dst) + blk, 16, 0, 0);
    }
    }
    if (kq) {
    if (RO) {
#pragma unroll
    for (int j = 0; j < LY::KI; ++j) {
      const uint32_t ko = full ? koff[j] : k_off(j, a.T - 1 - t0);
      const int blk = (wave + NW * j) * 1024;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(qc + ko), qbuf(dst) + blk, 16, 0, 0);
    }
    }
    if (MODE != 2) {
#pragma unroll
    for (int j = 0; j < LY::VI; ++j) {
      const uint32_t vo = full ? voff[j] : v_off(j, a.T - 1 - t0);
      const int blk = (wave + NW * j) * 1024;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vc + vo), vbuf(dst) + blk, 16, 0, 0);
    }
    }
    }
    if (part & 2) {
#pragma unroll
    for (int j = 0; j < (LY::RI + NW - 1) / NW; ++j) {
      const int blk = (wave + NW * j) * 1024;
      if (wave + NW * j < LY::RI)
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(rc + blk + lo), rbuf(dst) + blk, 16, 0, 0);
    }
    }
#else
    (void)kc; (void)qc; (void)vc; (void)rc; (void)lo; (void)full; (void)dst; (void)part;
#endif
  };

  // per-lane output offsets (elements) from the chunk's first token row: the
  // readout of tokens 4g + 16mt + i, and the score partials of token s_tok (the
  // token whose row totals this lane ends with after the transposed reduction)
  const uint32_t o_lane = (uint32_t)((4 * g * a.H + h) * DV + col);
  const int s_tok = 16 * (n >> 2) + 4 * g + (n & 3);
  // the waves' partials of chunk cc summed in wave order (lanes 0..15 of wave w take
  // tokens 16w .. 16w + 15) and stored as the column block's slice
  auto flush_scores = [&](int cc) {
    if constexpr (kScore) {
      const int tt = 16 * wave + lane, t0 = cc * kC;
      if (lane < 16 && t0 + tt < a.T) {
        const float4* sr = sred + (cc & 1) * NW * kC + tt;
        float4 acc = sr[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
          const float4 x = sr[w * kC];
          acc.x += x.x;
          acc.y += x.y;
          acc.z += x.z;
        }
        a.score[(((size_t)b * a.T + t0 + tt) * a.H + h) * NSL + cb] = acc;
      }
    }
  };

  auto chunk_step = [&](int c, char* stg, char* nxt) {
    const int t0 = c * kC;
    const int nvalid = min(kC, a.T - t0);
    __builtin_amdgcn_s_waitcnt(0);            // this chunk's tiles and record have arrived
    __syncthreads();                          // ... for every wave; the other stage is free
    if (c > c_begin) flush_scores(c - 1);     // every wave's partials of the last chunk are in
    // this lane's V values V[16mt + 4g + i][wave*16 + n] (transposing reads)
    u32x2 vraw[4] = {};
    if (MODE != 2) {
      const char* Vs = vbuf(stg);
      const int vr = n >> 2, vc = wave * 16 + 4 * (n & 3);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        vraw[mt] = lds_tr16(Vs, LY::voff(16 * mt + 4 * g + vr, vc >> 3) + (vc & 7) * 2);
    }
    auto v4_at = [&](int mt) {
      f32x4 f;
      f[0] = __uint_as_float(vraw[mt][0] << 16);
      f[1] = __uint_as_float(vraw[mt][0] & 0xffff0000u);
      f[2] = __uint_as_float(vraw[mt][1] << 16);
      f[3] = __uint_as_float(vraw[mt][1] & 0xffff0000u);
      return f;
    };
    if (c + 1 < c_end) issue_chunk(c + 1, nxt, 1);    // the next chunk's tiles
    const char* Ks = kbuf(stg);
    const char* Qs = qbuf(stg);
    const char* rec = rbuf(stg);
    const u32x4* Af = reinterpret_cast<const u32x4*>(rec + kRecA);
    const u32x2* Afh = reinterpret_cast<const u32x2*>(rec + kRecAh);
    const u32x4* QKf = reinterpret_cast<const u32x4*>(rec + kRecQK);
    const u32x2* QKfh = reinterpret_cast<const u32x2*>(rec + kRecQKh);
    const float* gam = reinterpret_cast<const float*>(rec + kRecGam);
    const float* wdec = reinterpret_cast<const float*>(rec + kRecW);

    // ---- Y_K = K S, Y_Q = Q S ----
    // A operand of row tile mt, k-step ks: token row 16mt+n, d = 32ks+8g..+7, the
    // 16-byte chunk 4ks + g of the row.
    f32x4 P[4], O[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      P[mt] = (f32x4)(0.f);
      O[mt] = (f32x4)(0.f);
    }
    // fragments of k-step ks are read one step ahead of their products
    u32x4 kf[2][4], qf[2][4];
    auto load_frags = [&](int ks, int buf) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int oa = LY::koff(16 * mt + n, 4 * ks + g);
        kf[buf][mt] = *reinterpret_cast<const u32x4*>(Ks + oa);
        if (RO) qf[buf][mt] = *reinterpret_cast<const u32x4*>(Qs + oa);
      }
    };
    // the three bf16 terms of S rows 32ks..32ks+31 (the B operand of k-step ks).  The
    // readout's Q S takes the first two: the mix normalises each readout row by its own
    // RMS, so a row of small norm (the first tokens of a chunk, early in the sequence)
    // carries the product's rounding relative to the row.  With the leading term alone
    // the worst output slice was 2.2% off at d_k = 256 and 1.6% at d_k = 128 (32 KV
    // heads of 128/64), against the 2% bound; with two, under 0.5%.
    constexpr bool kQS2 = true;
    bf16x8 spl[2][3];
    auto split_step = [&](int ks, int buf) {
      u32x2 h0, m0, l0, h1, m1, l1;
      split4(S[2 * ks], h0, m0, l0);
      split4(S[2 * ks + 1], h1, m1, l1);
      spl[buf][0] = as8(cat(h0, h1));
      spl[buf][1] = as8(cat(m0, m1));
      spl[buf][2] = as8(cat(l0, l1));
    };
    load_frags(0, 0);
    split_step(0, 0);
    // Each k-step's products run while the next step's fragments are read and its S
    // terms are split: the scheduler is asked for the step's LDS reads first, then one
    // MFMA to three VALU instructions.
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks) {
      if (ks + 1 < KSD) {
        load_frags(ks + 1, (ks + 1) & 1);
        split_step(ks + 1, (ks + 1) & 1);
      }
      const bf16x8 sh = spl[ks & 1][0], smd = spl[ks & 1][1], sl = spl[ks & 1][2];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 af = as8(kf[ks & 1][mt]);
        P[mt] = mfma_bf16(af, sl, P[mt]);
        P[mt] = mfma_bf16(af, smd, P[mt]);
        P[mt] = mfma_bf16(af, sh, P[mt]);
        if (RO && kQS2) O[mt] = mfma_bf16(as8(qf[ks & 1][mt]), smd, O[mt]);
        if (RO) O[mt] = mfma_bf16(as8(qf[ks & 1][mt]), sh, O[mt]);
      }
      if (ks + 1 < KSD) {
        __builtin_amdgcn_sched_group_barrier(0x100, RO ? 8 : 4, 0);     // the next step's LDS reads
#pragma unroll
        for (int i = 0; i < 4 * (3 + (RO ? (kQS2 ? 2 : 1) : 0)); ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);            // three VALU
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (LY::SPLIT) {
      // every wave is done with this chunk's Q and V (V is in registers): reload them
      __syncthreads();
      if (c + 1 < c_end) issue_chunk(c + 1, nxt, 4);
    } else if (c + 1 < c_end) {
      issue_chunk(c + 1, nxt, 2);                     // the next chunk's record
    }
    // The record fragments of the block substitution and the prediction below, read
    // ahead of the serial chain of products that consumes them.
    u32x2 pTh[2][3], pAh[2][3];
    u32x4 pT[2][3], pA[4][3];
    {
      const u32x4* Tf = reinterpret_cast<const u32x4*>(rec + kRecT);
      const u32x2* Tfh = reinterpret_cast<const u32x2*>(rec + kRecTh);
#pragma unroll
      for (int z = 0; z < 3; ++z) {
#pragma unroll
        for (int I = 0; I < 2; ++I) {
          pTh[I][z] = Tfh[(I * 3 + z) * kWave + lane];
          pT[I][z] = Tf[(I * 3 + z) * kWave + lane];
          pAh[I][z] = Afh[(I * 3 + z) * kWave + lane];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) pA[j][z] = Af[(j * 3 + z) * kWave + lane];
      }
    }
    u32x4 pQK[4];
    u32x2 pQKh[2];
    if (RO) {
#pragma unroll
      for (int j = 0; j < 4; ++j) pQK[j] = QKf[j * kWave + lane];
#pragma unroll
      for (int j = 0; j < 2; ++j) pQKh[j] = QKfh[j * kWave + lane];
    }
    // X = V - gamma K S ; P, O start as gamma K S, gamma Q S
    f32x4 X[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 gm = *reinterpret_cast<const f32x4*>(&gam[16 * mt + 4 * g]);
      const f32x4 v4 = v4_at(mt);
      P[mt] *= gm;
      if (RO) O[mt] *= gm;
      X[mt] = v4 - P[mt];
    }

    // ---- block forward substitution over the two 32-token blocks ----
    //   D_0 = T'_0 X_0,   D_1 = T'_1 (X_1 - A_10 D_0),   P += A D (strictly lower A)
    // dB[s][z]: B-operand fragments (k-step s, term z) of D rows 32s..32s+31.
    auto mf16 = [](const bf16x4& x, const bf16x4& y, const f32x4& c) { return mfma_bf16_k16(x, y, c); };
    auto lo4 = [](const u32x4& x) { return as4(u32x2{x[0], x[1]}); };
    auto A_at = [&](int mt, int s, int z) { return as8(pA[full_slot(pair_index(mt, s))][z]); };
    auto Ah_at = [&](int mt, int s, int z) { return as4(pAh[half_slot(pair_index(mt, s))][z]); };
    u32x4 dB[2][3];
    f32x4 D[4];
    auto solve_block = [&](int I, const f32x4& x0, const f32x4& x1) {
      u32x2 h0, m0, l0, h1, m1, l1;
      split4(x0, h0, m0, l0);
      split4(x1, h1, m1, l1);
      const bf16x8 rh = as8(cat(h0, h1)), rm = as8(cat(m0, m1)), rl = as8(cat(l0, l1));
      // first row tile: 16 columns
      D[2 * I] = mma6(mf16, as4(pTh[I][0]), as4(pTh[I][1]), as4(pTh[I][2]), as4(h0), as4(m0), as4(l0),
                      (f32x4)(0.f));
      D[2 * I + 1] = mma6(mfma_bf16, as8(pT[I][0]), as8(pT[I][1]), as8(pT[I][2]), rh, rm, rl, (f32x4)(0.f));
      split4(D[2 * I], h0, m0, l0);
      split4(D[2 * I + 1], h1, m1, l1);
      dB[I][0] = cat(h0, h1);
      dB[I][1] = cat(m0, m1);
      dB[I][2] = cat(l0, l1);
    };
    solve_block(0, X[0], X[1]);
    const f32x4 R2 = mma6(mfma_bf16, A_at(2, 0, 0), A_at(2, 0, 1), A_at(2, 0, 2),
                          as8(dB[0][0]), as8(dB[0][1]), as8(dB[0][2]), (f32x4)(0.f));
    const f32x4 R3 = mma6(mfma_bf16, A_at(3, 0, 0), A_at(3, 0, 1), A_at(3, 0, 2),
                          as8(dB[0][0]), as8(dB[0][1]), as8(dB[0][2]), (f32x4)(0.f));
    solve_block(1, X[2] - R2, X[3] - R3);
    // K^T fragments of the state update (below), read here so that their latency
    // falls behind the prediction and the readout (up to d_k = 128: 64 registers)
    const int kr4 = n >> 2;
    auto kt_frag = [&](int mt, int s) {
      // output lane 4c + i needs column srow(mt, c, i); lane (k, c) of the transposing
      // read addresses row k, columns srow(mt, c, 0..3)
      const int dcol = 32 * (mt >> 1) + 8 * (n & 3) + 4 * (mt & 1);
      const int ra = 32 * s + 4 * g + kr4, rb = ra + 16;
      const u32x2 ka = lds_tr16(Ks, LY::koff(ra, dcol >> 3) + (dcol & 7) * 2);
      const u32x2 kb = lds_tr16(Ks, LY::koff(rb, dcol >> 3) + (dcol & 7) * 2);
      return cat(ka, kb);
    };
    constexpr bool kKtAhead = DK <= 128;
    u32x4 ktf[kKtAhead ? MT : 1][2];
    if constexpr (kKtAhead) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int s = 0; s < 2; ++s) ktf[mt][s] = kt_frag(mt, s);
    }
    // the prediction P = gamma K S + A D
    P[0] = mma6(mf16, Ah_at(0, 0, 0), Ah_at(0, 0, 1), Ah_at(0, 0, 2),
                lo4(dB[0][0]), lo4(dB[0][1]), lo4(dB[0][2]), P[0]);
    P[1] = mma6(mfma_bf16, A_at(1, 0, 0), A_at(1, 0, 1), A_at(1, 0, 2),
                as8(dB[0][0]), as8(dB[0][1]), as8(dB[0][2]), P[1]);
    P[2] = mma6(mf16, Ah_at(2, 1, 0), Ah_at(2, 1, 1), Ah_at(2, 1, 2),
                lo4(dB[1][0]), lo4(dB[1][1]), lo4(dB[1][2]), P[2] + R2);
    P[3] = mma6(mfma_bf16, A_at(3, 1, 0), A_at(3, 1, 1), A_at(3, 1, 2),
                as8(dB[1][0]), as8(dB[1][1]), as8(dB[1][2]), P[3] + R3);

    // ---- readout O += (Gamma o Q K^T o lower_incl) D  (bf16 outputs: 2 terms) ----
    if (RO) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int s = 0; s <= (mt >> 1); ++s) {
          const int pi = pair_index(mt, s);
          if (pair_is_half(pi)) {
            // the pair's 16 nonzero columns in k-slots 0..3 of a 32-wide step.  Not the
            // 16x16x16 product: O[2] takes it right after the (2,0) pair's 16x16x32
            // products on the same accumulator, and that back-to-back pairing of the two
            // shapes gave wrong rows 4g, 4g+1 (g = 0, 1) of the tile at d_k = 64 in some
            // builds; with one shape throughout, every build checked gives exact rows.
            const u32x2 qh2 = pQKh[half_slot(pi)];
            const bf16x8 qh = as8(u32x4{qh2[0], qh2[1], 0u, 0u});
            O[mt] = mfma_bf16(qh, as8(dB[s][1]), O[mt]);
            O[mt] = mfma_bf16(qh, as8(dB[s][0]), O[mt]);
          } else {
            const bf16x8 qh = as8(pQK[full_slot(pi)]);
            O[mt] = mfma_bf16(qh, as8(dB[s][1]), O[mt]);
            O[mt] = mfma_bf16(qh, as8(dB[s][0]), O[mt]);
          }
        }
    }

    // ---- score partials of this 16-column slice (summed over the workgroup after
    //      the next barrier), and the readout ----
    const bool full = nvalid == kC;
    if (MODE == 0 && !(VAR & kVarNoScore)) {
      float xpv[16], xpp[16], xvv[16];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 v4 = v4_at(mt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xpv[4 * mt + i] = P[mt][i] * v4[i];
          xpp[4 * mt + i] = P[mt][i] * P[mt][i];
          xvv[4 * mt + i] = v4[i] * v4[i];
        }
      }
      const float pv = row16_transpose_sum(xpv, n);
      const float pp = row16_transpose_sum(xpp, n);
      const float vv = row16_transpose_sum(xvv, n);
      sred[(c & 1) * NW * kC + wave * kC + s_tok] = make_float4(pv, pp, vv, 0.f);
    }
    if (RO) {
      // the readout feeds the bf16 mix and the bf16 o_rnn output: stored as bf16
      uint16_t* oc = reinterpret_cast<uint16_t*>(a.o_rnn32) + ((size_t)b * a.T + t0) * a.H * DV;
      const uint32_t rs = (uint32_t)(a.H * DV);
      if (full) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) oc[o_lane + (uint32_t)(16 * mt + i) * rs] = f32_to_bf16(O[mt][i]);
      } else {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * mt + i + 4 * g < nvalid)
              oc[o_lane + (uint32_t)(16 * mt + i) * rs] = f32_to_bf16(O[mt][i]);
      }
    }

    // ---- S <- gamma_C S + K^T diag(exp(G_C - G)) D ----
    f32x4 wdv[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      wdv[s][0] = *reinterpret_cast<const f32x4*>(&wdec[32 * s + 4 * g]);
      wdv[s][1] = *reinterpret_cast<const f32x4*>(&wdec[32 * s + 16 + 4 * g]);
    }
    const float gl = gam[kC - 1];
    if (LY::SPLIT) {
      // every wave is done with this chunk's record: reload it for the next chunk
      __syncthreads();
      if (c + 1 < c_end) issue_chunk(c + 1, nxt, 2);
    }
    bf16x8 eh[2], em[2], el[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 wa = wdv[s][0];
      const f32x4 wb = wdv[s][1];
      u32x2 h0, m0, l0, h1, m1, l1;
      split4(D[2 * s] * wa, h0, m0, l0);
      split4(D[2 * s + 1] * wb, h1, m1, l1);
      eh[s] = as8(cat(h0, h1));
      em[s] = as8(cat(m0, m1));
      el[s] = as8(cat(l0, l1));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      S[mt] *= gl;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 kt;
        if constexpr (kKtAhead) kt = as8(ktf[mt][s]);
        else kt = as8(kt_frag(mt, s));
        S[mt] = mfma_bf16(kt, el[s], S[mt]);
        S[mt] = mfma_bf16(kt, em[s], S[mt]);
        S[mt] = mfma_bf16(kt, eh[s], S[mt]);
      }
    }
  };

  issue_chunk(c_begin, stage0, 7);
  for (int c = c_begin; c < c_end; c += 2) {
    chunk_step(c, stage0, stage1);
    if (c + 1 < c_end) chunk_step(c + 1, stage1, stage0);
  }
  if (kScore && c_end > c_begin) {
    __syncthreads();
    flush_scores(c_end - 1);
  }
  // the full pass stores the state after the last chunk (its last segment only); the
  // partial passes store each segment's result in its own block
  if (MODE != 0 || c_end == nchunk) {
    float* so = a.S_out + (MODE != 0 ? soff : 0) + sbase;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) so[(size_t)srow(mt, i) * DV + col] = S[mt][i];
  }
}

// S_in of every segment: grid (DV/4, H, B), 256 threads; a workgroup carries 4 state
// columns of one head through the segments (S_in[p+1] = A_p S_in[p] + B_p in fp32;
// every step needs all dk rows of the previous one, so a head's columns split over
// workgroups and its rows do not), each thread DK/64 of the dk x 4 entries.
constexpr int kSegCols = 4;
template <int DK, int DV>
__global__ __launch_bounds__(256) void seg_combine_kernel(SegArgs a) {
  __shared__ float Sc[DK][kSegCols];
  constexpr int PER = DK * kSegCols / 256;    // entries per thread: one row, PER columns
  const int tid = threadIdx.x;
  const int cb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.H + h;
  const int row = tid / (kSegCols / PER), c0 = (tid % (kSegCols / PER)) * PER;
  const size_t BH = (size_t)a.B * a.H;
  const size_t sb = (size_t)bh * DK * DV + (size_t)row * DV + cb * kSegCols + c0;
  float cur[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) cur[j] = a.S0 ? a.S0[sb + j] : 0.f;
  for (int p = 0; p < a.P; ++p) {
#pragma unroll
    for (int j = 0; j < PER; ++j) a.S_in[(size_t)p * BH * DK * DV + sb + j] = cur[j];
    if (p + 1 == a.P) break;
#pragma unroll
    for (int j = 0; j < PER; ++j) Sc[row][c0 + j] = cur[j];
    __syncthreads();
    const float* Ap = a.A + (size_t)p * BH * DK * DK + (size_t)bh * DK * DK + (size_t)row * DK;
    const float* Bp = a.Bm + (size_t)p * BH * DK * DV + sb;
    float acc[PER][2];
#pragma unroll
    for (int j = 0; j < PER; ++j) { acc[j][0] = Bp[j]; acc[j][1] = 0.f; }
#pragma unroll 4
    for (int k = 0; k < DK; k += 4) {
      const float4 ak = *reinterpret_cast<const float4*>(Ap + k);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        acc[j][0] = fmaf(ak.x, Sc[k][c0 + j], acc[j][0]);
        acc[j][1] = fmaf(ak.y, Sc[k + 1][c0 + j], acc[j][1]);
        acc[j][0] = fmaf(ak.z, Sc[k + 2][c0 + j], acc[j][0]);
        acc[j][1] = fmaf(ak.w, Sc[k + 3][c0 + j], acc[j][1]);
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) cur[j] = acc[j][0] + acc[j][1];
    __syncthreads();                          // Sc is rewritten by the next segment
  }
}

template <int DK>
hipError_t launch_prep_t(const RnnArgs& a, hipStream_t s) {
  const int nchunk = (a.T + kC - 1) / kC;
  hipLaunchKernelGGL((rnn_prep_kernel<DK>), dim3(nchunk, a.H, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Four waves (64 state columns) per workgroup; nseg segments of the chunk sequence.
template <int DK, int DV>
hipError_t launch_state_t(const RnnArgs& a, int mode, int nseg, hipStream_t s) {
  constexpr int NW = 4;
  dim3 grid((DV / (16 * NW)) * a.H * a.B * nseg);
  if (mode == 0 && a.o_rnn32 && a.variant == kVarNoScore)
    hipLaunchKernelGGL((rnn_chunked_kernel<DK, DV, NW, true, 0, kVarNoScore>), grid, dim3(64 * NW), 0, s, a);
  else if (mode == 0 && a.o_rnn32 && a.variant == (kVarNoScore | kVarLean))
    hipLaunchKernelGGL((rnn_chunked_kernel<DK, DV, NW, true, 0, kVarNoScore | kVarLean>), grid, dim3(64 * NW), 0,
                       s, a);
  else if (a.variant != 0)
    return hipErrorInvalidValue;
  else if (mode == 0 && a.o_rnn32)
    hipLaunchKernelGGL((rnn_chunked_kernel<DK, DV, NW, true, 0>), grid, dim3(64 * NW), 0, s, a);
  else if (mode == 0)
    hipLaunchKernelGGL((rnn_chunked_kernel<DK, DV, NW, false, 0>), grid, dim3(64 * NW), 0, s, a);
  else if constexpr (DK > 128)            // the segmented passes take d_k <= 128
    return hipErrorInvalidValue;
  else if (mode == 1)
    hipLaunchKernelGGL((rnn_chunked_kernel<DK, DV, NW, false, 1>), grid, dim3(64 * NW), 0, s, a);
  else if constexpr (DK == DV)
    hipLaunchKernelGGL((rnn_chunked_kernel<DK, DK, NW, false, 2>), grid, dim3(64 * NW), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace chunked

bool rnn_chunked_supported(int io, int dk, int dv) {
  return io == 1 && (((dk == 64 || dk == 128) && (dv == 64 || dv == 128)) || (dk == 256 && dv == 384));
}

// one score slice per four-wave workgroup (64 state columns)
int rnn_chunked_slices(int dv) { return dv / 64; }

hipError_t launch_rnn_chunked_prep(int io, int dk, const RnnArgs& a, hipStream_t s) {
  if (io != 1) return hipErrorInvalidValue;
  if (dk == 64) return chunked::launch_prep_t<64>(a, s);
  if (dk == 128) return chunked::launch_prep_t<128>(a, s);
  if (dk == 256) return chunked::launch_prep_t<256>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_rnn_chunked_state_seg(int io, int dk, int dv, int mode, int nseg, const RnnArgs& a,
                                        hipStream_t s) {
  if (io != 1 || nseg < 1 || (mode == 2 && dk != dv)) return hipErrorInvalidValue;
  if (dk == 64 && dv == 64) return chunked::launch_state_t<64, 64>(a, mode, nseg, s);
  if (dk == 64 && dv == 128) return chunked::launch_state_t<64, 128>(a, mode, nseg, s);
  if (dk == 128 && dv == 64) return chunked::launch_state_t<128, 64>(a, mode, nseg, s);
  if (dk == 128 && dv == 128) return chunked::launch_state_t<128, 128>(a, mode, nseg, s);
  // the paper's RNN heads: only the one-segment full pass
  if (dk == 256 && dv == 384 && mode == 0 && nseg == 1) return chunked::launch_state_t<256, 384>(a, 0, 1, s);
  return hipErrorInvalidValue;
}

hipError_t launch_rnn_chunked_state(int io, int dk, int dv, const RnnArgs& a, hipStream_t s) {
  return launch_rnn_chunked_state_seg(io, dk, dv, 0, 1, a, s);
}

hipError_t launch_seg_combine(int dk, int dv, const SegArgs& a, hipStream_t s) {
  const dim3 grid(dv / chunked::kSegCols, a.H, a.B);
  if (dk == 64 && dv == 64) hipLaunchKernelGGL((chunked::seg_combine_kernel<64, 64>), grid, dim3(256), 0, s, a);
  else if (dk == 64 && dv == 128) hipLaunchKernelGGL((chunked::seg_combine_kernel<64, 128>), grid, dim3(256), 0, s, a);
  else if (dk == 128 && dv == 64) hipLaunchKernelGGL((chunked::seg_combine_kernel<128, 64>), grid, dim3(256), 0, s, a);
  else if (dk == 128 && dv == 128) hipLaunchKernelGGL((chunked::seg_combine_kernel<128, 128>), grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ham
