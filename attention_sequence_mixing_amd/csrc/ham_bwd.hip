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
// t0 + t} and lo_t = #{pos < doc start}.  Two kernels per io type: the query kernel
// forms the row statistics (m, l, D) and dq; the entry kernel walks the queries that
// see a block of entries and forms dk, dv.  fp32 inputs run on fp32 VALU kernels (one
// wave per eight queries or entries; each takes 64 items at a time with a lane per item
// for the dot products, rows read as 16-byte runs, then turns to a lane per output
// dimension to accumulate, so no lane holds a whole gradient row).  bf16 inputs run on
// MFMA kernels over 64 x 64 tiles (below).
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

  // pass 1: running maximum and sum of each query's scaled scores, and D = sum_c p_c
  // (g . v_c) accumulated against the same running maximum
  float m[QB], l[QB], D[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) { m[j] = -INFINITY; l[j] = 0.f; D[j] = 0.f; }
  for (int c0 = cmin; c0 < cmax; c0 += 64) {
    const int c = c0 + lane;
    float sc[QB], gv[QB];
    if (c < cmax) scores(c, sc, gv, true);
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const float s = (c >= lo[j] && c < n[j]) ? a.scale * sc[j] : -INFINITY;
      const float mn = fmaxf(m[j], wave_max<64>(s));
      if (mn == -INFINITY) continue;                       // nothing visible yet (uniform)
      const float corr = expf(m[j] - mn);
      const float x = s == -INFINITY ? 0.f : expf(s - mn);
      l[j] = l[j] * corr + wave_sum<64>(x);
      D[j] = D[j] * corr + wave_sum<64>(x * gv[j]);
      m[j] = mn;
    }
  }
  float inv_l[QB];
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    inv_l[j] = l[j] > 0.f ? 1.f / l[j] : 0.f;
    D[j] *= inv_l[j];
  }

  // pass 2: dq = scale * sum_c p_c (g . v_c - D) k_c; the weights of 64 entries go
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

// ---- bf16 inputs: MFMA tiles -------------------------------------------------------
//
// Both kernels run on v_mfma_f32_16x16x32_bf16 (fp32 accumulate) over 64-row tiles,
// 512 threads = 8 waves of 16 rows each (two waves per SIMD).  Q, K and V are bf16
// inputs and enter as they are; the fp32 operands (dO, and P and dS formed in the
// kernels) enter as two bf16 terms hi + lo (16 significant bits), and products of two
// such operands keep the three leading cross terms.  The query kernel writes the two
// terms of dO to scratch once (the entry kernel then stages them like Q), the row
// statistics per query and the visible entry range per 64-query tile.
//
// Tiles come into LDS by direct buffer-to-LDS loads, double-buffered: after the barrier
// that publishes tile i, the loads of the next tile are issued into the other buffer
// and tile i is multiplied.  The two buffers are separate LDS objects and the tile loops
// are unrolled by two, so that every LDS access names its buffer statically: the
// compiler waits on the loads in flight into one buffer only before reads of that one
// (with one array indexed at run time it waited on them before every read, and loads
// never overlapped the products).  Rows are unpadded and the 16-byte chunk c of row r sits at
// slot c ^ f(r).  The LDS has 64 four-byte banks; a 16-byte read serves 16 consecutive
// lanes a pass, an 8-byte read 32, and (measured with the bank-conflict counter on
// probe patterns) the bank of a 16-byte read has its bit 2 flipped by address bit 11,
// so the 16-byte slot of rows 8..15 of a 2 KiB block of 256-byte rows moves by one.  A
// row-fragment read takes one chunk of 16 consecutive rows, a transposing read (below)
// a pair of chunks (2c, 2c + 1) of 8 consecutive rows.  With 128-element rows (16
// chunks, 256 bytes) f(r) = 2 (r mod 8) gives the 16 rows 16 different effective slots
// and the 8 rows 8 different slot pairs; with 64-element rows (8 chunks, two rows per
// 256 bytes, address bit 11 fixed within 16 rows) f(r) = 2 (r / 2 mod 4) + (r / 8 mod 2)
// does the same within each half.  Both reads are then free of bank conflicts.
//
// A-operand fragments: row fragments are 16-byte reads; fragments of a transposed
// tile come from the transposing LDS read (for a 16-lane group, lane r addresses
// X[k0 + r/4][d0 + 4(r mod 4) .. +3] and lane i receives X[k0 + j][d0 + i], j < 4).
// An MFMA output tile holds in lane (g, n) the rows 4g..4g+3 of column n.  A product
// contracting over 32 items whose values sit in such output tiles takes the items in
// the order 8g + j <-> 4g + j (j < 4) and 16 + 4g + j - 4 (j >= 4) on both operands.
namespace mbwd {

constexpr int NW = 8, NTH = 64 * NW;            // waves, threads per workgroup
constexpr int BT = 64;                          // rows per staged tile
constexpr int kMaskWords = 2048;                // visibility bits of up to 65536 query tiles

typedef short s4v __attribute__((ext_vector_type(4)));
typedef short s8v __attribute__((ext_vector_type(8)));

HAM_DEVICE f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <int D>
HAM_DEVICE int swz(int r) {
  static_assert(D == 64 || D == 128, "tile rows of 64 or 128 elements");
  return D == 128 ? 2 * (r & 7) : 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
}
// element offset of (row r, element e) in a swizzled tile of D-element rows
template <int D>
HAM_DEVICE int toff(int r, int e) { return r * D + ((((e >> 3) ^ swz<D>(r))) << 3) + (e & 7); }
// byte offset, from the tile's first row in memory (rows row_bytes apart), of the 16
// bytes that lane `lane` of direct load i brings to LDS bytes 1024 i + 16 lane
template <int D>
HAM_DEVICE int tile_voff(int i, int lane, int row_bytes) {
  const int p = i * 1024 + lane * 16, r = p / (2 * D), s = (p % (2 * D)) >> 4;
  return r * row_bytes + ((s ^ swz<D>(r)) << 4);
}

HAM_DEVICE bf16x8 frag16(const uint16_t* p) { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(p)); }
// row fragment of the 16 x 32 block at rows r0.., elements e0.. (e0 a multiple of 32)
template <int D>
HAM_DEVICE bf16x8 frag_row(const uint16_t* X, int r0, int e0, int g, int n) {
  return frag16(X + toff<D>(r0 + n, e0 + 8 * g));
}
HAM_DEVICE s4v tr16(const uint16_t* base, int elem_off) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) s4v lds_s4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s4*)((__attribute__((address_space(3))) const char*)(const void*)base + elem_off * 2));
#else
  (void)base; (void)elem_off;
  return s4v{0, 0, 0, 0};
#endif
}
// A-operand fragment of X^T for a 32-item step u and the 16 columns d0.. (items
// 32u + 4g + j and 32u + 16 + 4g + j)
template <int D>
HAM_DEVICE bf16x8 frag_tr(const uint16_t* X, int u, int d0, int g, int n) {
  const int col = d0 + 4 * (n & 3);
  const s4v lo = tr16(X, toff<D>(32 * u + 4 * g + (n >> 2), col));
  const s4v hi = tr16(X, toff<D>(32 * u + 16 + 4 * g + (n >> 2), col));
  s8v v;
  v[0] = lo[0]; v[1] = lo[1]; v[2] = lo[2]; v[3] = lo[3];
  v[4] = hi[0]; v[5] = hi[1]; v[6] = hi[2]; v[7] = hi[3];
  return __builtin_bit_cast(bf16x8, v);
}
HAM_DEVICE void split2(float x, __bf16& h, __bf16& l) {
  h = static_cast<__bf16>(x);
  l = static_cast<__bf16>(x - static_cast<float>(h));
}
// B operands (hi, lo) of a 32-item step from two output tiles (items 4g+i of tile 0
// -> slots i, of tile 1 -> slots 4 + i)
HAM_DEVICE void pack2(const f32x4& t0, const f32x4& t1, bf16x8& h, bf16x8& l) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __bf16 a, b;
    split2(t0[i], a, b); h[i] = a; l[i] = b;
    split2(t1[i], a, b); h[4 + i] = a; l[4 + i] = b;
  }
}
HAM_DEVICE int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// grid (B*H, ceil(T/128)), 512 threads: 8 waves x 16 queries of one head.  The query
// blocks with the most visible entries come first (grid y counts down from the end).
// Writes dq, the per-query statistics (m in log2 units, 1/l, D, lo, n), the visible
// entry range of each 64-query tile and the two bf16 terms of dO.
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void attn_bwd_q_mfma(AttnBwdArgs a) {
  constexpr int KSD = DK / 32, VSD = DV / 32, DT = DK / 16;
  constexpr int KB = BT * DK * 2, STAGE = KB + BT * DV * 2;
  constexpr int NKI = DK / 64, NVI = DV / 64;              // direct loads per wave and tile
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE];
  __shared__ int s_rng[2][NW];
  const int tid = threadIdx.x, lane = lane_id(), wave = uniform(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int bh = blockIdx.x, qb = gridDim.y - 1 - blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int nq64 = (a.T + BT - 1) / BT;
  const int32_t* ph = a.pos + (size_t)bh * a.cap;
  const int cnt = a.count[bh];
  const char* Kh = static_cast<const char*>(a.Kc) + (size_t)bh * a.cap * DK * 2;
  const char* Vh = static_cast<const char*>(a.Vc) + (size_t)bh * a.cap * DV * 2;
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const int t = qb * 2 * BT + wave * 16 + n;     // this lane's query
  const bool tv = t < a.T;
  const size_t tok = ((size_t)b * a.T + (tv ? t : 0)) * a.H + h;
  const int nn = tv ? count_at_most(ph, cnt, (long long)a.t0 + t) : 0;
  const int lo = (tv && a.doc_start)
                     ? min(nn, count_at_most(ph, cnt, (long long)a.doc_start[(size_t)b * a.T + t] - 1)) : 0;
  // visible entry ranges of the wave, of each 64-query half and of the block
  int mn = nn > lo ? lo : 0x7fffffff, mx = nn > lo ? nn : 0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) { mn = min(mn, __shfl_xor(mn, o, kWave)); mx = max(mx, __shfl_xor(mx, o, kWave)); }
  if (lane == 0) { s_rng[0][wave] = mn; s_rng[1][wave] = mx; }
  __syncthreads();
  int cmin = 0x7fffffff, cmax = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) { cmin = min(cmin, s_rng[0][w]); cmax = max(cmax, s_rng[1][w]); }
  cmin = uniform(cmin);
  cmax = uniform(cmax);
  if (tid < 2 && 2 * qb + tid < nq64) {
    int hmn = 0x7fffffff, hmx = 0;
#pragma unroll
    for (int w = 0; w < NW / 2; ++w) { hmn = min(hmn, s_rng[0][4 * tid + w]); hmx = max(hmx, s_rng[1][4 * tid + w]); }
    a.tile_rng[(size_t)bh * nq64 + 2 * qb + tid] = make_int2(hmn, hmx);
  }
  const int cfirst = cmax > 0 ? cmin / BT * BT : 0;

  bf16x8 qf[KSD], gh[VSD], gl[VSD];
#pragma unroll
  for (int ks = 0; ks < KSD; ++ks)
    qf[ks] = tv ? frag16(qp + tok * DK + ks * 32 + 8 * g) : __builtin_bit_cast(bf16x8, (u16x8)(0));
#pragma unroll
  for (int ks = 0; ks < VSD; ++ks) {
    f32x4 x0 = (f32x4)(0.f), x1 = (f32x4)(0.f);
    if (tv) {
      const f32x4* p = reinterpret_cast<const f32x4*>(a.dO + tok * DV + ks * 32 + 8 * g);
      x0 = p[0];
      x1 = p[1];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      __bf16 x, y;
      split2(j < 4 ? x0[j] : x1[j - 4], x, y);
      gh[ks][j] = x; gl[ks][j] = y;
    }
    if (tv) {
      *reinterpret_cast<bf16x8*>(a.dOh + tok * DV + ks * 32 + 8 * g) = gh[ks];
      *reinterpret_cast<bf16x8*>(a.dOl + tok * DV + ks * 32 + 8 * g) = gl[ks];
    }
  }
  const float sl2 = a.scale * 1.4426950408889634f;

  int voK[NKI], voV[NVI];
#pragma unroll
  for (int k = 0; k < NKI; ++k) voK[k] = tile_voff<DK>(k * NW + wave, lane, DK * 2);
#pragma unroll
  for (int k = 0; k < NVI; ++k) voV[k] = tile_voff<DV>(k * NW + wave, lane, DV * 2);
  auto issue = [&](int c0, char* st) {
    const int rows = min(BT, cnt - c0);
#pragma unroll
    for (int k = 0; k < NKI; ++k)
      buffer_to_lds(Kh + (size_t)c0 * DK * 2, rows * DK * 2, voK[k], st + (k * NW + wave) * 1024);
#pragma unroll
    for (int k = 0; k < NVI; ++k)
      buffer_to_lds(Vh + (size_t)c0 * DV * 2, rows * DV * 2, voV[k], st + KB + (k * NW + wave) * 1024);
  };
  // Walks the entry tiles [cfirst, cmax), calling body(c0, K, V) on each: wait for the
  // tile's loads, publish it, send the next tile's loads to the other buffer, multiply.
  auto walk = [&](auto&& body) {
    if (cmax <= cfirst) return;
    __syncthreads();                                       // both buffers are free
    issue(cfirst, stage0);
    auto step = [&](int c0, char* cur, char* nxt) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (c0 + BT < cmax) issue(c0 + BT, nxt);
      body(c0, reinterpret_cast<const uint16_t*>(cur), reinterpret_cast<const uint16_t*>(cur + KB));
    };
    for (int c0 = cfirst; c0 < cmax; c0 += 2 * BT) {
      step(c0, stage0, stage1);
      if (c0 + BT < cmax) step(c0 + BT, stage1, stage0);
    }
  };

  // S^T and dP^T of one tile: lane (g, n) gets entries 16 kt + 4g + i of query n
  f32x4 st[4], dp[4];
  auto tile_products = [&](const uint16_t* K, const uint16_t* V) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      st[kt] = (f32x4)(0.f);
      dp[kt] = (f32x4)(0.f);
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) st[kt] = mma(frag_row<DK>(K, 16 * kt, 32 * ks, g, n), qf[ks], st[kt]);
#pragma unroll
      for (int ks = 0; ks < VSD; ++ks) {
        const bf16x8 vf = frag_row<DV>(V, 16 * kt, 32 * ks, g, n);
        dp[kt] = mma(vf, gh[ks], dp[kt]);
        dp[kt] = mma(vf, gl[ks], dp[kt]);
      }
    }
  };

  // pass A: row maximum (log2 units), sum and D = sum_c p_c (dO . v_c), online
  float m = -INFINITY, l = 0.f, accD = 0.f;
  walk([&](int c0, const uint16_t* K, const uint16_t* V) {
    tile_products(K, V);
    float s2[4][4], tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + 16 * kt + 4 * g + i;
        s2[kt][i] = (c >= lo && c < nn) ? st[kt][i] * sl2 : -INFINITY;
        tmax = fmaxf(tmax, s2[kt][i]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float mnew = fmaxf(m, tmax);
    // a query with nothing visible yet keeps m = -inf and adds nothing
    const float corr = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
    l *= corr;
    accD *= corr;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(s2[kt][i] - mnew);
        const float ev = s2[kt][i] == -INFINITY ? 0.f : e;
        l += ev;
        accD = fmaf(ev, dp[kt][i], accD);
      }
    m = mnew;
  });
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  accD += __shfl_xor(accD, 16, kWave);
  accD += __shfl_xor(accD, 32, kWave);
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  const float D = accD * inv_l;
  if (tv && g == 0) {
    f32x4 sv;
    sv[0] = m; sv[1] = inv_l; sv[2] = D; sv[3] = 0.f;
    *reinterpret_cast<f32x4*>(a.stat + tok * 8) = sv;
    *reinterpret_cast<int2*>(a.stat + tok * 8 + 4) = make_int2(lo, nn);
  }

  // pass B: dS = P (dP - D); dq^T = K^T dS^T
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = (f32x4)(0.f);
  walk([&](int c0, const uint16_t* K, const uint16_t* V) {
    tile_products(K, V);
    f32x4 ds[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + 16 * kt + 4 * g + i;
        const float e = __builtin_amdgcn_exp2f(st[kt][i] * sl2 - m) * inv_l;
        const float p = (c >= lo && c < nn) ? e : 0.f;
        ds[kt][i] = p * (dp[kt][i] - D);
      }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 dh, dl;
      pack2(ds[2 * u], ds[2 * u + 1], dh, dl);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 kt = frag_tr<DK>(K, u, 16 * dt, g, n);
        acc[dt] = mma(kt, dh, acc[dt]);
        acc[dt] = mma(kt, dl, acc[dt]);
      }
    }
  });
  if (tv) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(a.dq + tok * DK + 16 * dt + 4 * g) = acc[dt] * a.scale;
  }
}

// grid (B*H, ceil(cap/128)), 512 threads: 8 waves x 16 cache entries of one head.  The
// 64-query tiles whose visible range meets the block are walked in order; the earliest
// entries (seen by the most queries) come first.
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void attn_bwd_kv_mfma(AttnBwdArgs a) {
  constexpr int KSD = DK / 32, VSD = DV / 32, DTK = DK / 16, DTV = DV / 16;
  constexpr int QBY = BT * DK * 2, GBY = BT * DV * 2, SBY = BT * 32;
  constexpr int STAGE = QBY + 2 * GBY + SBY;
  constexpr int NQI = DK / 64, NGI = DV / 64;              // direct loads per wave and tile
  __shared__ __attribute__((aligned(1024))) char stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) char stage1[STAGE];
  __shared__ uint32_t s_mask[kMaskWords];
  const int tid = threadIdx.x, lane = lane_id(), wave = uniform(tid >> 6);
  const int g = lane >> 4, n = lane & 15;
  const int bh = blockIdx.x, cb = blockIdx.y * (NW * 16);
  const int b = bh / a.H, h = bh % a.H;
  const int cnt = a.count[bh];
  if (cb >= cnt) return;                                   // whole workgroup
  const int nq64 = (a.T + BT - 1) / BT;
  const int32_t* ph = a.pos + (size_t)bh * a.cap;
  const uint16_t* Kh = static_cast<const uint16_t*>(a.Kc) + (size_t)bh * a.cap * DK;
  const uint16_t* Vh = static_cast<const uint16_t*>(a.Vc) + (size_t)bh * a.cap * DV;
  const size_t head0 = (size_t)b * a.T * a.H + h;         // token-head index of (b, t = 0, h)
  const char* qh = static_cast<const char*>(a.q) + head0 * DK * 2;
  const char* ghp = reinterpret_cast<const char*>(a.dOh) + head0 * DV * 2;
  const char* glp = reinterpret_cast<const char*>(a.dOl) + head0 * DV * 2;
  const char* sth = reinterpret_cast<const char*>(a.stat) + head0 * 32;
  const int qrow = a.H * DK * 2, grow = a.H * DV * 2, srow = a.H * 32;   // bytes between queries
  const int c = cb + wave * 16 + n;                        // this lane's entry
  const bool cv = c < cnt;
  const int clast = min(cnt, cb + NW * 16) - 1;
  bf16x8 kf[KSD], vf[VSD];
#pragma unroll
  for (int ks = 0; ks < KSD; ++ks)
    kf[ks] = cv ? frag16(Kh + (size_t)c * DK + 32 * ks + 8 * g) : __builtin_bit_cast(bf16x8, (u16x8)(0));
#pragma unroll
  for (int ks = 0; ks < VSD; ++ks)
    vf[ks] = cv ? frag16(Vh + (size_t)c * DV + 32 * ks + 8 * g) : __builtin_bit_cast(bf16x8, (u16x8)(0));
  const float sl2 = a.scale * 1.4426950408889634f;

  // visibility of the query tiles j0.. (tile j0 holds the query at the first entry's
  // position, the first that may see the block), from the query kernel's tile ranges
  const long long p0 = (long long)ph[cb] - (long long)a.t0;
  const int j0 = uniform((int)(max(0LL, min((long long)a.T, p0)) / BT));
  const int nt = nq64 - j0;
  for (int base = 0; base < nt; base += NTH) {
    bool vis = false;
    if (base + tid < nt) {
      const int2 r = a.tile_rng[(size_t)bh * nq64 + j0 + base + tid];
      vis = r.x <= clast && r.y > cb;
    }
    const unsigned long long bal = __ballot(vis);
    if (lane == 0) {
      s_mask[(base >> 5) + 2 * wave] = (uint32_t)bal;
      s_mask[(base >> 5) + 2 * wave + 1] = (uint32_t)(bal >> 32);
    }
  }
  __syncthreads();
  auto next_vis = [&](int j) {                             // first visible tile >= j, or nt
    while (j < nt) {
      const uint32_t w = (uint32_t)uniform((int)s_mask[j >> 5]) >> (j & 31);
      if (w) return j + __builtin_ctz(w);
      j = (j | 31) + 1;
    }
    return nt;
  };

  int voQ[NQI], voG[NGI];
#pragma unroll
  for (int k = 0; k < NQI; ++k) voQ[k] = tile_voff<DK>(k * NW + wave, lane, qrow);
#pragma unroll
  for (int k = 0; k < NGI; ++k) voG[k] = tile_voff<DV>(k * NW + wave, lane, grow);
  // statistics rows: 32 bytes each, waves 0 and 1 bring 32 rows each
  const int voS = ((wave * 1024 + lane * 16) >> 5) * srow + (lane & 1) * 16;
  auto issue = [&](int jt, char* st) {
    const int tq0 = (j0 + jt) * BT, rows = min(BT, a.T - tq0);
#pragma unroll
    for (int k = 0; k < NQI; ++k)
      buffer_to_lds(qh + (size_t)tq0 * qrow, rows * qrow, voQ[k], st + (k * NW + wave) * 1024);
#pragma unroll
    for (int k = 0; k < NGI; ++k) {
      buffer_to_lds(ghp + (size_t)tq0 * grow, rows * grow, voG[k], st + QBY + (k * NW + wave) * 1024);
      buffer_to_lds(glp + (size_t)tq0 * grow, rows * grow, voG[k], st + QBY + GBY + (k * NW + wave) * 1024);
    }
    if (wave < 2) buffer_to_lds(sth + (size_t)tq0 * srow, rows * srow, voS, st + QBY + 2 * GBY + wave * 1024);
  };

  f32x4 dk[DTK], dv[DTV];
#pragma unroll
  for (int i = 0; i < DTK; ++i) dk[i] = (f32x4)(0.f);
#pragma unroll
  for (int i = 0; i < DTV; ++i) dv[i] = (f32x4)(0.f);

  // one visible tile: wait for its loads, publish it, send the next visible tile's
  // loads to the other buffer, multiply; returns that next tile
  auto step = [&](int jt, char* cur, char* nxt) {
    const int jn = next_vis(jt + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (jn < nt) issue(jn, nxt);
    const uint16_t* Q = reinterpret_cast<const uint16_t*>(cur);
    const uint16_t* Gh = reinterpret_cast<const uint16_t*>(cur + QBY);
    const uint16_t* Gl = reinterpret_cast<const uint16_t*>(cur + QBY + GBY);
    const char* S = cur + QBY + 2 * GBY;
    f32x4 sc[4], dpt[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      sc[qt] = (f32x4)(0.f);
      dpt[qt] = (f32x4)(0.f);
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) sc[qt] = mma(frag_row<DK>(Q, 16 * qt, 32 * ks, g, n), kf[ks], sc[qt]);
#pragma unroll
      for (int ks = 0; ks < VSD; ++ks) {
        dpt[qt] = mma(frag_row<DV>(Gh, 16 * qt, 32 * ks, g, n), vf[ks], dpt[qt]);
        dpt[qt] = mma(frag_row<DV>(Gl, 16 * qt, 32 * ks, g, n), vf[ks], dpt[qt]);
      }
    }
    // lane (g, n): rows = queries 16 qt + 4g + i, column = entry n of the wave
    f32x4 P[4], dS[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * qt + 4 * g + i;
        const f32x4 sv = *reinterpret_cast<const f32x4*>(S + r * 32);
        const int2 rg = *reinterpret_cast<const int2*>(S + r * 32 + 16);
        const bool vis = cv & (c >= rg.x) & (c < rg.y);     // no branch per row
        const float e = __builtin_amdgcn_exp2f(sc[qt][i] * sl2 - sv[0]) * sv[1];
        const float p = vis ? e : 0.f;
        P[qt][i] = p;
        dS[qt][i] = p * (dpt[qt][i] - sv[2]);
      }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 ph_, pl_, dh, dl;
      pack2(P[2 * u], P[2 * u + 1], ph_, pl_);
      pack2(dS[2 * u], dS[2 * u + 1], dh, dl);
#pragma unroll
      for (int dt = 0; dt < DTV; ++dt) {
        const bf16x8 ah = frag_tr<DV>(Gh, u, 16 * dt, g, n);
        const bf16x8 al = frag_tr<DV>(Gl, u, 16 * dt, g, n);
        dv[dt] = mma(ah, ph_, dv[dt]);
        dv[dt] = mma(ah, pl_, dv[dt]);
        dv[dt] = mma(al, ph_, dv[dt]);
      }
#pragma unroll
      for (int dt = 0; dt < DTK; ++dt) {
        const bf16x8 aq = frag_tr<DK>(Q, u, 16 * dt, g, n);
        dk[dt] = mma(aq, dh, dk[dt]);
        dk[dt] = mma(aq, dl, dk[dt]);
      }
    }
    return jn;
  };
  int jt = next_vis(0);
  if (jt < nt) issue(jt, stage0);
  while (jt < nt) {
    jt = step(jt, stage0, stage1);
    if (jt >= nt) break;
    jt = step(jt, stage1, stage0);
  }
  if (cv) {
    const size_t row = (size_t)bh * a.cap + c;
#pragma unroll
    for (int dt = 0; dt < DTK; ++dt)
      *reinterpret_cast<f32x4*>(a.dKc + row * DK + 16 * dt + 4 * g) = dk[dt] * a.scale;
#pragma unroll
    for (int dt = 0; dt < DTV; ++dt) *reinterpret_cast<f32x4*>(a.dVc + row * DV + 16 * dt + 4 * g) = dv[dt];
  }
}

}  // namespace mbwd

template <int DK, int DV>
static hipError_t launch_bwd_mfma(const AttnBwdArgs& a, hipStream_t s) {
  const int nq = (a.T + 2 * mbwd::BT - 1) / (2 * mbwd::BT), nc = (a.cap + 16 * mbwd::NW - 1) / (16 * mbwd::NW);
  if ((a.T + mbwd::BT - 1) / mbwd::BT > 32 * mbwd::kMaskWords || nq > 65535 || nc > 65535)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((mbwd::attn_bwd_q_mfma<DK, DV>), dim3(a.B * a.H, nq), dim3(mbwd::NTH), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mbwd::attn_bwd_kv_mfma<DK, DV>), dim3(a.B * a.H, nc), dim3(mbwd::NTH), 0, s, a);
  return hipGetLastError();
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
    // bf16 inputs: the MFMA kernels
    if (dk == 64 && dv == 64) return launch_bwd_mfma<64, 64>(a, s);
    if (dk == 64 && dv == 128) return launch_bwd_mfma<64, 128>(a, s);
    if (dk == 128 && dv == 64) return launch_bwd_mfma<128, 64>(a, s);
    if (dk == 128 && dv == 128) return launch_bwd_mfma<128, 128>(a, s);
  }
#undef HAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace ham
