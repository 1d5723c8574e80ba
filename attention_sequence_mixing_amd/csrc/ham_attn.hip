// ham_attn.hip -- causal softmax attention over the compacted KV cache, with the
// headwise-norm gated mix fused into the epilogue.
//
// "Hybrid Associative Memories": softmax retrieval over the stored pairs (§2
// KV-memory equation), restricted to routed tokens; a query at original position
// t sees cached keys at original positions <= t (App. A.1 "FlexAttention and
// Block Masks": causality by original position, padding excluded).  Because the
// cache is in ascending original position, that set is the prefix c < n_t of the
// cache, with n_t the number of cached tokens at positions <= t (n_t includes t
// itself when t is routed).  With same-document masking (App. A.1 "FlexAttention
// and Block Masks", packed batches) the visible set is cut to keys of t's own document,
// which is the cache range [lo_t, n_t).  Mix: o = g_rnn*rms(o_rnn) +
// g_kv*rms(o_kv) (§2 headwise norm and gated sum; App. A.1 headwise gating).
//
// Each wave computes S^T = K Q^T on 16x16 MFMA tiles (keys on rows), so the
// per-query softmax state lives in the lanes that later hold that query's output
// column of O^T = V^T P^T: no data movement between the two products.  bf16 I/O
// (attn_bf16_v5_kernel): 4 waves x 32 queries of one (b,h) per workgroup on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  fp32 I/O, and bf16 value rows of
// 192 elements (attn_kernel): 4 waves x 16 queries of one (b,h) per workgroup, on
// v_mfma_f32_16x16x4f32 (fp32) or v_mfma_f32_16x16x32_bf16 (bf16).
#include "ham_common.h"
#include "ham_internal.h"

namespace ham {

constexpr float kLog2e = 1.4426950408889634f;

template <class IO>
struct AttnTile;
template <>
struct AttnTile<IoBF16> { static constexpr int BN = 64; };
template <>
struct AttnTile<IoF32> { static constexpr int BN = 32; };

template <class IO, int DK, int DV>
struct AttnSmem;
template <int DK, int DV>
struct AttnSmem<IoBF16, DK, DV> {
  static constexpr int BN = 64;
  static constexpr int KS = DK + 8;   // K row stride (elements), padded
  static constexpr int VS = BN + 8;   // V^T row stride (elements), padded
  uint16_t K[BN * KS];
  uint16_t Vt[DV * VS];
};
template <int DK, int DV>
struct AttnSmem<IoF32, DK, DV> {
  static constexpr int BN = 32;
  static constexpr int KS = DK + 4;
  static constexpr int VS = DV + 4;
  float K[BN * KS];
  float V[BN * VS];
};

// Stage rows [c0, c0+BN) of this head's cache into LDS; rows at or beyond nmax
// are zero so masked lanes multiply finite values.
template <int DK, int DV>
HAM_DEVICE void stage_kv(AttnSmem<IoBF16, DK, DV>& sm, const uint16_t* Kh, const uint16_t* Vh,
                         int c0, int nmax, int tid) {
  constexpr int BN = 64, KS = DK + 8, VS = BN + 8;
  constexpr int KU = DK / 8, VU = DV / 8;
#pragma unroll
  for (int u = tid; u < BN * KU; u += 256) {
    const int row = u / KU, col = (u % KU) * 8;
    u16x8 x = (u16x8)(0);
    if (c0 + row < nmax) x = *reinterpret_cast<const u16x8*>(Kh + (size_t)(c0 + row) * DK + col);
    *reinterpret_cast<u16x8*>(&sm.K[row * KS + col]) = x;
  }
#pragma unroll
  for (int u = tid; u < BN * VU; u += 256) {
    const int row = u / VU, col = (u % VU) * 8;
    u16x8 x = (u16x8)(0);
    if (c0 + row < nmax) x = *reinterpret_cast<const u16x8*>(Vh + (size_t)(c0 + row) * DV + col);
#pragma unroll
    for (int j = 0; j < 8; ++j) sm.Vt[(col + j) * VS + row] = x[j];
  }
}

template <int DK, int DV>
HAM_DEVICE void stage_kv(AttnSmem<IoF32, DK, DV>& sm, const float* Kh, const float* Vh,
                         int c0, int nmax, int tid) {
  constexpr int BN = 32, KS = DK + 4, VS = DV + 4;
  constexpr int KU = DK / 4, VU = DV / 4;
#pragma unroll
  for (int u = tid; u < BN * KU; u += 256) {
    const int row = u / KU, col = (u % KU) * 4;
    f32x4 x = (f32x4)(0.f);
    if (c0 + row < nmax) x = *reinterpret_cast<const f32x4*>(Kh + (size_t)(c0 + row) * DK + col);
    *reinterpret_cast<f32x4*>(&sm.K[row * KS + col]) = x;
  }
#pragma unroll
  for (int u = tid; u < BN * VU; u += 256) {
    const int row = u / VU, col = (u % VU) * 4;
    f32x4 x = (f32x4)(0.f);
    if (c0 + row < nmax) x = *reinterpret_cast<const f32x4*>(Vh + (size_t)(c0 + row) * DV + col);
    *reinterpret_cast<f32x4*>(&sm.V[row * VS + col]) = x;
  }
}

// Query fragments: the B operand of S^T = K Q^T for this lane's query.
template <int DK>
struct QFragBF16 { bf16x8 x[DK / 32]; };
template <int DK>
struct QFragF32 { float x[DK / 4]; };

// Generic kernel: every fp32 shape, and bf16 shapes the tiled kernel below does not
// take (value rows that are not a power-of-two number of 16-byte chunks).
template <class IO, int DK, int DV>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  using E = typename IO::elem;
  constexpr bool kBF16 = (IO::kBytes == 2);
  constexpr int BN = AttnTile<IO>::BN;
  constexpr int NT = BN / 16;              // 16-key subtiles per tile
  constexpr int DT = DV / 16;              // 16-wide d tiles of the output
  __shared__ AttnSmem<IO, DK, DV> sm;

  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int g = lane >> 4, qn = lane & 15;
  const int nqb = (a.T + 63) / 64;
  // longest query blocks first; XCD-aware so one head's blocks share an L2
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lin / nqb;
  const int qb = nqb - 1 - (lin % nqb);
  const int b = bh / a.H, h = bh % a.H;

  const E* __restrict__ qp = static_cast<const E*>(a.q);
  const E* __restrict__ Kh = static_cast<const E*>(a.Kc) + (size_t)bh * a.cap * DK;
  const E* __restrict__ Vh = static_cast<const E*>(a.Vc) + (size_t)bh * a.cap * DV;
  const int32_t* ntok = a.ntok + (size_t)bh * a.T;

  const int t = qb * 64 + wave * 16 + qn;           // this lane's query
  const bool tvalid = t < a.T;
  const int nq = tvalid ? ntok[t] : 0;              // visible keys c < nq
  const int tlast = min(a.T - 1, qb * 64 + 63);
  const int nhi = ntok[tlast];                      // keys any query of the block sees
  // same-document masking: visible keys are lq <= c < nq; the block starts at the
  // tile of its smallest lq
  const int lq = (a.lo && tvalid) ? a.lo[(size_t)bh * a.T + t] : 0;
  __shared__ int s_lomin[4];
  int it0 = 0;
  if (a.lo) {
    int m = tvalid ? lq : 0x7fffffff;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = min(m, __shfl_xor(m, o, kWave));
    if (lane == 0) s_lomin[wave] = m;
    __syncthreads();
    it0 = min(min(s_lomin[0], s_lomin[1]), min(s_lomin[2], s_lomin[3])) / AttnTile<IO>::BN;
  }
  const size_t tok = ((size_t)b * a.T + (tvalid ? t : 0)) * a.H + h;

  // load this lane's query fragment
  QFragBF16<DK> qfb;
  QFragF32<DK> qff;
  // with a rotary table the query is turned at its position first (pairs of
  // consecutive elements; the table row of local token t)
  const float2* rrow = a.rope ? a.rope + (size_t)(tvalid ? t : 0) * (DK / 2) : nullptr;
  if constexpr (kBF16) {
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
      u16x8 x = (u16x8)(0);
      if (tvalid) x = *reinterpret_cast<const u16x8*>(reinterpret_cast<const uint16_t*>(qp) + tok * DK + ks * 32 + 8 * g);
      if (rrow) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x0 = bf16_to_f32(x[2 * j]), x1 = bf16_to_f32(x[2 * j + 1]);
          rope_pair(x0, x1, rrow[(ks * 32 + 8 * g) / 2 + j]);
          x[2 * j] = f32_to_bf16(x0);
          x[2 * j + 1] = f32_to_bf16(x1);
        }
      }
      qfb.x[ks] = __builtin_bit_cast(bf16x8, x);
    }
  } else {
    const float* qf = reinterpret_cast<const float*>(qp) + tok * DK;
#pragma unroll
    for (int ks = 0; ks < DK / 4; ++ks) {
      const int d = ks * 4 + g;
      float x = tvalid ? qf[d] : 0.f;
      if (rrow && tvalid) {
        // element d of pair d/2; its partner is d ^ 1
        const float y = qf[d ^ 1];
        const float2 cs = rrow[d >> 1];
        x = (d & 1) ? (y * cs.y + x * cs.x) : (x * cs.x - y * cs.y);
      }
      qff.x[ks] = x;
    }
  }

  const float sl2 = a.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = (f32x4)(0.f);

  const int ntiles = (nhi + BN - 1) / BN;
  for (int it = it0; it < ntiles; ++it) {
    const int c0 = it * BN;
    __syncthreads();
    stage_kv(sm, Kh, Vh, c0, nhi, tid);
    __syncthreads();

    f32x4 st[NT];
#pragma unroll
    for (int kt = 0; kt < NT; ++kt) {
      st[kt] = (f32x4)(0.f);
      if constexpr (kBF16) {
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
          const u16x8 kx = *reinterpret_cast<const u16x8*>(&sm.K[(kt * 16 + qn) * (DK + 8) + ks * 32 + 8 * g]);
          st[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kx), qfb.x[ks], st[kt], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < DK / 4; ++ks) {
          const float kx = sm.K[(kt * 16 + qn) * (DK + 4) + ks * 4 + g];
          st[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kx, qff.x[ks], st[kt], 0, 0, 0);
        }
      }
    }
    // st[kt][i] = q_t . k_c for c = c0 + kt*16 + 4g + i (this lane's query t)
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int cidx = c0 + kt * 16 + 4 * g + i;
        const float s = (cidx >= lq && cidx < nq) ? st[kt][i] * sl2 : -INFINITY;
        st[kt][i] = s;
        tmax = fmaxf(tmax, s);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    const float m_new = fmaxf(m_run, tmax);
    const float corr = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < NT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = (st[kt][i] == -INFINITY) ? 0.f : exp2f(st[kt][i] - m_new);
        st[kt][i] = p;
        psum += p;
      }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= corr;

    // O^T += V^T P^T
    if constexpr (kBF16) {
#pragma unroll
      for (int u = 0; u < NT / 2; ++u) {
        u16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = f32_to_bf16(st[2 * u][i]);
          pb[4 + i] = f32_to_bf16(st[2 * u + 1][i]);
        }
        const bf16x8 pbf = __builtin_bit_cast(bf16x8, pb);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint16_t* vrow = &sm.Vt[(dt * 16 + qn) * (64 + 8)];
          const u16x4 v0 = *reinterpret_cast<const u16x4*>(vrow + 32 * u + 4 * g);
          const u16x4 v1 = *reinterpret_cast<const u16x4*>(vrow + 32 * u + 16 + 4 * g);
          u16x8 va;
          va[0] = v0[0]; va[1] = v0[1]; va[2] = v0[2]; va[3] = v0[3];
          va[4] = v1[0]; va[5] = v1[1]; va[6] = v1[2]; va[7] = v1[3];
          acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pbf, acc[dt], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < NT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float* vrow = &sm.V[(kt * 16 + 4 * g + i) * (DV + 4)];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[dt * 16 + qn], st[kt][i], acc[dt], 0, 0, 0);
        }
    }
  }

  // ---- epilogue: normalise, mix with the RNN readout, store ----------------------
  float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  const float inv_l = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (a.okv32) {
    // KV heads of another geometry than the RNN's: the readout alone, mixed later
    if (tvalid) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(a.okv32 + tok * DV + dt * 16 + 4 * g) = acc[dt] * inv_l;
    }
    return;
  }
  // lane holds query t, output dims d = dt*16 + 4g + i
  float okv[DT][4], orn[DT][4];
  float ssk = 0.f, ssr = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    f32x4 r4 = (f32x4)(0.f);
    if (tvalid && a.ornn_bf16) {
      const u16x4 x = *reinterpret_cast<const u16x4*>(reinterpret_cast<const uint16_t*>(a.o_rnn32) +
                                                       tok * DV + dt * 16 + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) r4[i] = bf16_to_f32(x[i]);
    } else if (tvalid) {
      r4 = *reinterpret_cast<const f32x4*>(a.o_rnn32 + tok * DV + dt * 16 + 4 * g);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      okv[dt][i] = acc[dt][i] * inv_l;
      orn[dt][i] = r4[i];
      ssk += okv[dt][i] * okv[dt][i];
      ssr += orn[dt][i] * orn[dt][i];
    }
  }
  ssk += __shfl_xor(ssk, 16, kWave);
  ssk += __shfl_xor(ssk, 32, kWave);
  ssr += __shfl_xor(ssr, 16, kWave);
  ssr += __shfl_xor(ssr, 32, kWave);
  if (!tvalid) return;
  const size_t tt = ((size_t)b * a.T + t) * a.H + h;
  const float gr = a.gate_rnn ? a.gate_rnn[tt] : 1.f;
  const float gk = a.gate_kv ? a.gate_kv[tt] : 1.f;
  const float ir = gr / sqrtf(ssr / (float)DV + a.eps);
  const float ik = gk / sqrtf(ssk / (float)DV + a.eps);
  E* o = static_cast<E*>(a.o);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = orn[dt][i] * ir + okv[dt][i] * ik;
    const size_t off = tt * DV + dt * 16 + 4 * g;
    IO::store4(o, off, y);
    if (a.o_kv) IO::store4(static_cast<E*>(a.o_kv), off, okv[dt]);
    if (a.o_rnn) IO::store4(static_cast<E*>(a.o_rnn), off, orn[dt]);
  }
}

// Softmax of the bf16 path: the running maximum m is kept in log2 units of the
// scaled logits.  A tile's probabilities are first formed against the stale m;
// their row sum bounds the largest of them, so when no query's sum exceeds
// 2^12 every probability is at most 2^12 and the tile is accepted as is (fp32 and
// bf16 hold such values exactly enough, and the final division by the running sum
// cancels the common factor).  Otherwise the tile's scores are formed again and
// the exact path runs: row maxima across the four lanes of a query, rescale of the
// accumulators, probabilities against the new maximum.  The first tile of a block
// always takes the exact path.
constexpr float kLazySum = 4096.0f;
constexpr float kLazyRescale = 8.0f;

// ---- bf16 path: direct-to-LDS tile ring ---------------------------------------------
//
// 4 waves x 32 queries per workgroup, two workgroups per CU.  K and V tiles (64
// keys) are copied from HBM into LDS by buffer loads that write LDS directly (no
// staging registers) into a 2-stage ring, one tile ahead of the one being
// consumed.  The buffer descriptors are rebuilt per tile in scalar registers with
// the tile's first row as base and the rows still visible to the block as range,
// so rows past the last visible key read as zero without per-lane clamping; the
// per-lane offsets are fixed for the whole kernel.  Tiles are row-major with the
// 16-byte chunks of each row XOR-swizzled: in K, chunk c of row r sits at slot
// c ^ (r mod chunks-per-row); in V at slot c ^ 2(r mod chunks-per-row/2), which
// keeps both fragment reads free of bank conflicts.  K fragments (A operand of
// S^T = K Q^T) are 16-byte reads; V^T fragments (A operand of O^T = V^T P^T) use
// the transposing LDS read: for each 16-lane group, lane r addresses
// V[k0 + r/4][d0 + 4(r mod 4) .. +3] and lane i receives V[k0 + j][d0 + i] for
// j = 0..3.
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));

HAM_DEVICE short4v lds_read_tr16(const char* base, int byte_off) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) short4v lds_short4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4*)((__attribute__((address_space(3))) const char*)base + byte_off));
#else
  (void)base; (void)byte_off;
  return short4v{0, 0, 0, 0};
#endif
}

// Direct-to-LDS load of 16 bytes per lane at voff + soff of a buffer of range_bytes
// from base (bytes at or past the range read as zero; the scalar offset is part of
// the range check and does not move the LDS address).
HAM_DEVICE void buffer_to_lds_so(const void* base, int range_bytes, int voff, int soff, char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                                               range_bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#else
  (void)base; (void)range_bytes; (void)voff; (void)soff; (void)lds;
#endif
}

// A wave-uniform pointer pinned to scalar registers (a buffer descriptor built from
// vector registers makes the compiler wrap each load in a loop over lanes).
HAM_DEVICE const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Scheduling pattern: NM matrix products in L groups, one vector-memory instruction
// after each group (the first NM mod L groups hold one product more).
template <int NM, int L, int K = 0>
HAM_DEVICE void interleave_loads() {
  if constexpr (K < L) {
    constexpr int n = NM / L + (K < NM % L ? 1 : 0);
    if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x008, n, 0);
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    interleave_loads<NM, L, K + 1>();
  }
}

// Chunk slot swizzles of the K and V tiles (D = row length in elements).
template <int D>
HAM_DEVICE int swz_k(int r) { return r & (D / 8 - 1); }
template <int D>
HAM_DEVICE int swz_v(int r) { return 2 * (r & (D / 16 - 1)); }

// DOC: same-document masking (a.lo set): query t sees keys lo_t <= c < ntok_t; the
// block starts at the tile of its smallest lo.  The queries' (lo, ntok) ranges wait
// in LDS for the tiles that need a mask (registers are at their limit here), and a
// wave in which a row meets its first visible key after the block's first tile
// takes the exact path then.
template <int DK, int DV, int QT, bool DOC>
__global__ __launch_bounds__(256, 2) void attn_bf16_v5_kernel(AttnArgs a) {
  constexpr int NWV = 4;                                   // waves per workgroup
  constexpr int BN = 64, NKT = BN / 16, DT = DV / 16, KSD = DK / 32;
  constexpr int BMW = 16 * QT, BM = NWV * BMW;
  constexpr int KB = BN * DK * 2, VB = BN * DV * 2;        // tile bytes
  constexpr int KI = KB / 1024, VI = VB / 1024;            // 1 KiB load instructions per tile
  static_assert((KI + VI) % NWV == 0, "tile loads must split evenly over the waves");
  constexpr int LPW = (KI + VI) / NWV;                     // load instructions per wave per tile
  constexpr int RBK = DK * 2, RBV = DV * 2;                // row bytes (in memory)
  // In LDS a V tile is kept as column parts of power-of-two width (192 = 128 + 64), each
  // row-major with its own swizzle, so every part has power-of-two rows.
  constexpr int DV1 = DV > 128 ? 128 : DV, DV2 = DV - DV1;
  static_assert((DV1 & (DV1 - 1)) == 0 && (DV2 & (DV2 - 1)) == 0, "value parts must be powers of two");
  constexpr int RB1 = DV1 * 2, RB2 = DV2 * 2;              // LDS row bytes of the parts
  constexpr int VI1 = BN * RB1 / 1024;                     // load instructions of part 1
  constexpr int V2OFF = KB + BN * RB1;                     // LDS offset of part 2 in a stage
  // two ring stages as separate LDS objects, so that reads of one stage are known
  // not to alias the direct loads in flight into the other
  __shared__ __attribute__((aligned(16))) char stage0[KB + VB];
  __shared__ __attribute__((aligned(16))) char stage1[KB + VB];

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, qn = lane & 15;
  const int nqb = (a.T + BM - 1) / BM;
  // global longest-first: all heads' last query block first
  // (the integer divisions run on the vector unit; the results are pinned to scalar
  // registers so that the buffer descriptors built from them stay scalar)
  const int lin = blockIdx.x;
  const int nbh = gridDim.x / nqb;
  const int bh = __builtin_amdgcn_readfirstlane(lin % nbh);
  const int qb = __builtin_amdgcn_readfirstlane(nqb - 1 - (lin / nbh));
  const int b = __builtin_amdgcn_readfirstlane(bh / a.H), h = __builtin_amdgcn_readfirstlane(bh % a.H);

  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const char* Kh = static_cast<const char*>(a.Kc) + (size_t)bh * a.cap * RBK;
  const char* Vh = static_cast<const char*>(a.Vc) + (size_t)bh * a.cap * RBV;
  const int32_t* ntok = a.ntok + (size_t)bh * a.T;

  const int qb0 = qb * BM;
  const int nlo = ntok[qb0];
  const int nhi = ntok[min(a.T - 1, qb0 + BM - 1)];

  // The query fragments carry the logit scale in log2 units (one more bf16 rounding of
  // each query element, the size of the rounding the probabilities get anyway), so the
  // products give scaled logits directly.
  const float sl2 = a.scale * kLog2e;
  int tq[QT], nq[QT];
  bf16x8 qf[QT][KSD];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    tq[qt] = qb0 + wave * BMW + 16 * qt + qn;
    const bool ok = tq[qt] < a.T;
    nq[qt] = ok ? ntok[tq[qt]] : 0;
    const size_t tok = ((size_t)b * a.T + (ok ? tq[qt] : 0)) * a.H + h;
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks)
      qf[qt][ks] = *reinterpret_cast<const bf16x8*>(qp + tok * DK + ks * 32 + 8 * g);
  }
  // The query fragments are turned and scaled after the first tile's loads have gone
  // out (work on them waits for their loads).
  auto prep_queries = [&]() {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      // with a rotary table the query is turned at its position (consecutive pairs)
      const float2* rrow = a.rope ? a.rope + (size_t)(tq[qt] < a.T ? tq[qt] : 0) * (DK / 2) : nullptr;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        u16x8 x = __builtin_bit_cast(u16x8, qf[qt][ks]);
        if (rrow) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float x0 = bf16_to_f32(x[2 * j]), x1 = bf16_to_f32(x[2 * j + 1]);
            rope_pair(x0, x1, rrow[(ks * 32 + 8 * g) / 2 + j]);
            x[2 * j] = f32_to_bf16(x0 * sl2);
            x[2 * j + 1] = f32_to_bf16(x1 * sl2);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = f32_to_bf16(bf16_to_f32(x[j]) * sl2);
        }
        qf[qt][ks] = __builtin_bit_cast(bf16x8, x);
      }
    }
  };

  // Tile loads: 1 KiB instruction i covers bytes [i*1024, i*1024 + 1024) of a stage
  // (K rows first, then V rows); wave w issues i = 4k + w.  Lane l writes 16 bytes at
  // i*1024 + 16*l, which hold chunk (slot ^ swizzle) of its tile row.  The swizzle
  // repeats every PK (PV) instructions, a divisor of 4, so one per-lane offset per
  // tensor serves all of a wave's loads, each adding a constant step.
  static_assert(KI % NWV == 0, "K and V loads must not share a wave step");
  constexpr int PK = (DK / 8) * RBK / 1024 > 1 ? (DK / 8) * RBK / 1024 : 1;
  constexpr int PV1 = (DV1 / 16) * RB1 / 1024 > 1 ? (DV1 / 16) * RB1 / 1024 : 1;
  constexpr int PV2 = DV2 && (DV2 / 16) * RB2 / 1024 > 1 ? (DV2 / 16) * RB2 / 1024 : 1;
  static_assert(NWV % PK == 0 && NWV % PV1 == 0 && NWV % PV2 == 0, "swizzle period must divide the wave count");
  static_assert(KI % NWV == 0 && VI1 % NWV == 0, "K, V part 1 and V part 2 loads must not share a wave step");
  // wave w issues the load instructions i = 4k + w of each tensor part; jX is the
  // instruction of its period that the per-lane offset ldX was computed for
  const int jK = wave % PK, jV1 = wave % PV1, jV2 = wave % PV2;
  int ldK, ldV1, ldV2 = 0;
  {
    const int pk = jK * 1024 + lane * 16, rk = pk / RBK;
    ldK = rk * RBK + ((((pk % RBK) >> 4) ^ swz_k<DK>(rk)) << 4);
    // V parts: LDS rows of RBp bytes, memory rows of RBV bytes
    const int p1 = jV1 * 1024 + lane * 16, r1 = p1 / RB1;
    ldV1 = r1 * RBV + ((((p1 % RB1) >> 4) ^ swz_v<DV1>(r1)) << 4);
    if constexpr (DV2 > 0) {
      const int p2 = jV2 * 1024 + lane * 16, r2 = p2 / RB2;
      ldV2 = r2 * RBV + RB1 + ((((p2 % RB2) >> 4) ^ swz_v<DV2>(r2)) << 4);
    }
  }
  // One descriptor per tensor and tile (base: the tile's first row; range: its rows
  // still visible to the block).  An instruction's place in the tile goes into the
  // scalar offset, which the range check includes, so rows past the last visible key
  // read as zero; the wave's share of the offset is folded into the per-lane offsets.
  ldK += (wave - jK) * 1024;
  ldV1 += (wave - jV1) * (1024 / RB1) * RBV;
  if constexpr (DV2 > 0) ldV2 += (wave - jV2) * (1024 / RB2) * RBV;
  // load k (of LPW) of this wave for tile it into stage st; woff = 1024 * wave (the
  // caller hides its value from the compiler, which otherwise keeps every load's LDS
  // address in a register of its own and runs out of scalar registers)
  auto issue_load = [&](int k, int it, char* st, int woff, int rows) {
    const int c0 = it * BN;
    if (k < KI / NWV) {
      buffer_to_lds_so(Kh + (size_t)c0 * RBK, rows * RBK, ldK, k * NWV * 1024, st + woff + k * NWV * 1024);
    } else if (k < (KI + VI1) / NWV) {
      // part 1 instruction i = kk * NWV + wave covers LDS rows from (i * 1024 / RB1) on
      const int kk = k - KI / NWV;
      buffer_to_lds_so(Vh + (size_t)c0 * RBV, rows * RBV, ldV1, kk * NWV * (1024 / RB1) * RBV,
                       st + KB + woff + kk * NWV * 1024);
    } else {
      const int kk = k - (KI + VI1) / NWV;
      buffer_to_lds_so(Vh + (size_t)c0 * RBV, rows * RBV, ldV2, kk * NWV * (1024 / (RB2 ? RB2 : 1)) * RBV,
                       st + V2OFF + woff + kk * NWV * 1024);
    }
  };
  auto opaque_woff = [&]() {
    int w = wave * 1024;
    asm volatile("" : "+s"(w));
    return w;
  };
  auto issue_tile = [&](int it, char* st, int rows) {
    const int woff = opaque_woff();
#pragma unroll
    for (int k = 0; k < LPW; ++k) issue_load(k, it, st, woff, rows);
  };

  float m_run[QT], l_run[QT];
  f32x4 acc[QT][DT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[qt][dt] = (f32x4)(0.f);
  }

  // Per-lane fragment offsets inside a stage (the swizzle terms depend only on the lane).
  int koff[KSD], voff[DT];
  const int r4 = qn >> 2, c4 = qn & 3;
#pragma unroll
  for (int ks = 0; ks < KSD; ++ks) koff[ks] = qn * RBK + (((ks * 4 + g) ^ swz_k<DK>(qn)) << 4);
  {
    const int ry = 4 * g + r4;                             // tile row of this lane's V run (mod 16)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      if (dt < DV1 / 16)
        voff[dt] = KB + ry * RB1 + (((2 * dt + (c4 >> 1)) ^ swz_v<DV1>(ry)) << 4) + (c4 & 1) * 8;
      else
        voff[dt] = V2OFF + ry * RB2 + (((2 * (dt - DV1 / 16) + (c4 >> 1)) ^ swz_v<DV2 ? DV2 : 16>(ry)) << 4) +
                   (c4 & 1) * 8;
    }
  }

  const int ntiles = (nhi + BN - 1) / BN;
  int it0 = 0, lmax = 0;                                  // first tile; largest lo
  __shared__ int2 s_rng[DOC ? BM : 1];                    // (lo, ntok) of the block's queries
  if constexpr (DOC) {
    __shared__ int s_lo[2][NWV];
    int mn = 0x7fffffff, mx = 0;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int l = tq[qt] < a.T ? a.lo[(size_t)bh * a.T + tq[qt]] : 0;
      s_rng[wave * BMW + 16 * qt + qn] = make_int2(l, nq[qt]);
      if (tq[qt] < a.T) {
        mn = min(mn, l);
        mx = max(mx, l);
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      mn = min(mn, __shfl_xor(mn, o, kWave));
      mx = max(mx, __shfl_xor(mx, o, kWave));
    }
    if (lane == 0) { s_lo[0][wave] = mn; s_lo[1][wave] = mx; }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NWV; ++w) { mn = min(mn, s_lo[0][w]); mx = max(mx, s_lo[1][w]); }
    it0 = __builtin_amdgcn_readfirstlane(mn / BN);
    lmax = __builtin_amdgcn_readfirstlane(mx);
  }
  // The first tile's loads go out while the query fragments are still in flight (the
  // compiler waits for those registers where they are first used; every step waits
  // for all memory before it reads the stage).  Without document masks the first tile
  // is tile 0 and its loads do not wait for the block's visible-key counts either: they
  // take every row the cache holds (up to 64), and once the counts are known the rows
  // past the last visible key, which may be stale, are cleared in the V tile (their
  // scores are masked; a stale value row times probability 0 could still be NaN).
  if constexpr (DOC) {
    if (it0 < ntiles) issue_tile(it0, stage0, min(nhi - it0 * BN, BN));
  } else {
    issue_tile(0, stage0, min(a.cap, BN));
  }
  prep_queries();
  if constexpr (!DOC) {
    const int rmax = min(a.cap, BN);
    if (ntiles == 0) {
      __builtin_amdgcn_s_waitcnt(0);                       // no step waits for the early tile
    } else if (nhi < rmax) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      const int tid = threadIdx.x;
      for (int i = tid; i < (rmax - nhi) * (RB1 / 16); i += 64 * NWV)
        *reinterpret_cast<f32x4*>(stage0 + KB + (nhi + i / (RB1 / 16)) * RB1 + (i % (RB1 / 16)) * 16) = (f32x4)(0.f);
      if constexpr (DV2 > 0) {
        for (int i = tid; i < (rmax - nhi) * (RB2 / 16); i += 64 * NWV)
          *reinterpret_cast<f32x4*>(stage0 + V2OFF + (nhi + i / (RB2 / 16)) * RB2 + (i % (RB2 / 16)) * 16) =
              (f32x4)(0.f);
      }
    }
  }

  f32x4 st[QT][NKT];
  // S^T = K Q^T for the tile in `Kt`.  With `load` set, the loads of tile `itn` into
  // stage `nx` go out between the products (about one per NM / LPW of them), so the
  // texture path takes them spread over the phase rather than all at once after the
  // barrier, where the waves stalled on their issue.
  // The matrix phases (scores, P V) run at raised wave priority: with two waves per
  // SIMD in different phases, the one issuing products is served first and the
  // other's softmax instructions fill its gaps (attention 0.298 -> 0.291 ms at the
  // layer shape, same box).
  auto do_scores = [&](const char* Kt, bool load, char* nx, int itn) {
    constexpr int NM = KSD * NKT * QT;                     // products of the phase
    __builtin_amdgcn_s_setprio(1);
    // the products accumulate onto minus the running maximum (0 while it is -inf), so
    // they end as scaled logits relative to it
    f32x4 c0v[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) c0v[qt] = (f32x4)(m_run[qt] == -INFINITY ? 0.f : -m_run[qt]);
#pragma unroll
    for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const bf16x8 kx = *reinterpret_cast<const bf16x8*>(Kt + koff[ks] + kt * 16 * RBK);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          st[qt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kx, qf[qt][ks], ks == 0 ? c0v[qt] : st[qt][kt], 0, 0, 0);
      }
    if (load) {
      const int woff = opaque_woff();
#pragma unroll
      for (int k = 0; k < LPW; ++k) issue_load(k, itn, nx, woff, min(nhi - itn * BN, BN));
      // order: the fragment reads, then the products in LPW groups, a load after each
      __builtin_amdgcn_sched_group_barrier(0x100, KSD * NKT, 0);
      interleave_loads<NM, LPW>();
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // keys at or past a query's visible count get -inf
  auto do_mask = [&](int c0) {
    if constexpr (DOC) {
      if ((c0 + BN) > nlo || c0 < lmax) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const int2 r = s_rng[wave * BMW + 16 * qt + qn];
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int c = c0 + kt * 16 + 4 * g + i;
              if (c < r.x || c >= r.y) st[qt][kt][i] = -INFINITY;
            }
        }
      }
    } else if ((c0 + BN) > nlo) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((c0 + kt * 16 + 4 * g + i) >= nq[qt]) st[qt][kt][i] = -INFINITY;
    }
  };
  // probabilities against the current maximum, rounded to bf16: the B operand of
  // O^T += V^T P^T.  Within each 32-key half u, B's row k = 8g + j holds key
  // 32u + 4g + j (j < 4) or 32u + 16 + 4g + j - 4 (j >= 4); the V^T fragments
  // follow the same order.  The scores are relative to the maximum they were formed
  // against; off[qt] moves them to the current one (the exact path only).
  bf16x8 pb[NKT / 2][QT];
  auto do_probs = [&](const float (&off)[QT], bool shift) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int u = 0; u < NKT / 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float s0 = shift ? st[qt][2 * u][i] + off[qt] : st[qt][2 * u][i];
          const float s1 = shift ? st[qt][2 * u + 1][i] + off[qt] : st[qt][2 * u + 1][i];
          pb[u][qt][i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(s0));
          pb[u][qt][4 + i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(s1));
        }
    }
  };
  // the tile's row sums of those probabilities, formed on MFMA as 1^T P^T: every
  // lane receives its query's sum over all 64 keys
  auto do_rowsum = [&](float (&ls)[QT]) {
    bf16x8 ones;
#pragma unroll
    for (int j = 0; j < 8; ++j) ones[j] = static_cast<__bf16>(1.0f);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      f32x4 r = (f32x4)(0.f);
#pragma unroll
      for (int u = 0; u < NKT / 2; ++u) r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[u][qt], r, 0, 0, 0);
      ls[qt] = r[0];
    }
  };
  // exact path: row maxima, rescale, probabilities against the new maximum
  auto do_exact = [&]() {
    bool grow = false;
    float m_loc[QT], mref[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      mref[qt] = m_run[qt] == -INFINITY ? 0.f : m_run[qt];   // what the scores are relative to
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
        tmax = fmaxf(tmax, fmaxf(fmaxf(st[qt][kt][0], st[qt][kt][1]), fmaxf(st[qt][kt][2], st[qt][kt][3])));
      m_loc[qt] = tmax + mref[qt];
      grow |= m_loc[qt] > m_run[qt] + kLazyRescale;
    }
    if (__any(grow)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float mrow = fmaxf(m_loc[qt], __shfl_xor(m_loc[qt], 16, kWave));
        mrow = fmaxf(mrow, __shfl_xor(mrow, 32, kWave));
        const float mn = fmaxf(m_run[qt], mrow);
        const float corr = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run[qt] - mn);
        l_run[qt] *= corr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[qt][dt] *= corr;
        m_run[qt] = mn;
      }
    }
    float off[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) off[qt] = m_run[qt] == -INFINITY ? 0.f : mref[qt] - m_run[qt];
    do_probs(off, true);
    float ls[QT];
    do_rowsum(ls);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) l_run[qt] += ls[qt];
  };
  // O^T += V^T P^T for the tile in `stage`
  auto do_pv = [&](const char* Vt) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int u = 0; u < NKT / 2; ++u) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int rbl = dt < DV1 / 16 ? RB1 : RB2;         // LDS row bytes of dt's part
        const short4v lo = lds_read_tr16(Vt, voff[dt] + 32 * u * rbl);
        const short4v hi = lds_read_tr16(Vt, voff[dt] + (32 * u + 16) * rbl);
        short8v va;
        va[0] = lo[0]; va[1] = lo[1]; va[2] = lo[2]; va[3] = lo[3];
        va[4] = hi[0]; va[5] = hi[1]; va[6] = hi[2]; va[7] = hi[3];
        const bf16x8 vb = __builtin_bit_cast(bf16x8, va);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          acc[qt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vb, pb[u][qt], acc[qt][dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Step it: tile it has landed in `cur` (wait, then barrier: every wave is also
  // done with tile it-1, whose stage `nxt` the next load overwrites); fetch tile
  // it+1 into `nxt`; consume tile it.
  // The RNN readout rows of the block (bf16, from the chunked state pass) are copied
  // into the stage the last tile leaves free while that tile is consumed: wave w
  // fetches the rows of its own 32 queries, 16-byte chunks XOR-swizzled by row, so
  // the epilogue reads them from LDS without waiting on memory.
  constexpr int OCH = DV * 2 / 16;                         // 16-byte chunks per row
  constexpr int OWB = BMW * DV * 2;                        // one wave's rows, bytes
  // (not with document masks: that variant has no registers to spare for it)
  constexpr bool kOrnnLds = !DOC && NWV * OWB <= KB + VB && (OCH & (OCH - 1)) == 0;  // they fit in a stage
  const char* ornn_st = nullptr;
  auto issue_ornn = [&](char* st) {
    const int rstride = a.H * DV * 2;
    const char* base = uniform_ptr(reinterpret_cast<const char*>(a.o_rnn32) + (((size_t)b * a.T + qb0) * a.H + h) * DV * 2);
    // rows past T read zero (kept in a scalar register: a clamp the compiler forms on the
    // vector unit would make the descriptor look divergent and wrap each load in a loop)
    const int range = __builtin_amdgcn_readfirstlane(max(0, min(a.T - qb0, BM)) * rstride);
#pragma unroll
    for (int j = 0; j < OCH / 2; ++j) {
      const int r = wave * BMW + j * (64 / OCH) + lane / OCH;
      const int c = (lane % OCH) ^ (r & (OCH - 1));
      buffer_to_lds(base, range, r * rstride + c * 16, st + wave * OWB + j * 1024);
    }
  };
  auto step = [&](int it, char* cur, char* nxt, bool last) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (last && kOrnnLds && a.ornn_bf16) {
      issue_ornn(nxt);
      ornn_st = nxt;
    }
    do_scores(cur, !last, nxt, it + 1);
    do_mask(it * BN);
    // the first tile is exact; with document masks, every tile in which a row meets
    // its first visible key is (the row has no running maximum before it)
    bool exact = !DOC && it == 0;
    if (!exact) {
      const float zero[QT] = {};
      do_probs(zero, false);
      float ls[QT];
      do_rowsum(ls);
      bool over = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) over |= ls[qt] > kLazySum;
      if constexpr (DOC) {
        const int c0 = it * BN;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          if (m_run[qt] == -INFINITY) {
            const int2 r = s_rng[wave * BMW + 16 * qt + qn];
            over |= r.x < r.y && r.x < c0 + BN && r.y > c0;
          }
      }
      if (__any(over)) {
        exact = true;
        do_scores(cur, false, nxt, 0);
        do_mask(it * BN);
      } else {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) l_run[qt] += ls[qt];
      }
    }
    if (exact) do_exact();
    do_pv(cur);
  };
  // tile it sits in stage (it - it0) mod 2; the last tile's step loads no tile.  The
  // loop body holds only steps that load (a choice inside it would let the compiler
  // share the products of both kinds and leave the loads in a block of their own).
  int it = it0;
  for (; it + 2 < ntiles; it += 2) {
    step(it, stage0, stage1, false);
    step(it + 1, stage1, stage0, false);
  }
  if (it + 1 < ntiles) {
    step(it, stage0, stage1, false);
    step(it + 1, stage1, stage0, true);
  } else if (it < ntiles) {
    step(it, stage0, stage1, true);
  }

  // ---- epilogue: normalise, mix with the RNN readout, store ----------------------
  // Straight-line per source, so that all of a wave's reads go out before the first
  // use; reciprocals and reciprocal square roots by the hardware instructions (about
  // one unit in the last place of fp32, far below the bf16 rounding of the outputs).
  float inv_l[QT];
  size_t tt[QT];
  bool tvalid[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    inv_l[qt] = (l_run[qt] > 0.f) ? __builtin_amdgcn_rcpf(l_run[qt]) : 0.f;   // row sum in every lane
    tvalid[qt] = tq[qt] < a.T;
    tt[qt] = ((size_t)b * a.T + (tvalid[qt] ? tq[qt] : 0)) * a.H + h;
  }
  if (a.okv32) {
    // KV heads of another geometry than the RNN's: the readout alone, mixed later
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
      if (tvalid[qt]) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *reinterpret_cast<f32x4*>(a.okv32 + tt[qt] * DV + dt * 16 + 4 * g) = acc[qt][dt] * inv_l[qt];
      }
    return;
  }
  float orn[QT][DT][4];
  if (kOrnnLds && ornn_st) {
    __builtin_amdgcn_s_waitcnt(0);                       // this wave's readout rows are in LDS
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        // row 16 qt + n of this wave's rows; columns dt*16 + 4g .. +3 are half of chunk 2dt + g/2
        const int rr = 16 * qt + qn;
        const int c = (2 * dt + (g >> 1)) ^ ((wave * BMW + rr) & (OCH - 1));
        const u16x4 x = *reinterpret_cast<const u16x4*>(ornn_st + wave * OWB + rr * (DV * 2) + c * 16 + (g & 1) * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) orn[qt][dt][i] = bf16_to_f32(x[i]);
      }
  } else if (a.ornn_bf16) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u16x4 x = *reinterpret_cast<const u16x4*>(reinterpret_cast<const uint16_t*>(a.o_rnn32) +
                                                         tt[qt] * DV + dt * 16 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) orn[qt][dt][i] = bf16_to_f32(x[i]);
      }
  } else {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(a.o_rnn32 + tt[qt] * DV + dt * 16 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) orn[qt][dt][i] = x[i];
      }
  }
  // With the readout rows in LDS, the bf16 results of each wave go over its own rows
  // there, in the layout they were read in, and leave as whole rows (16 bytes per
  // lane, four 256-byte rows per instruction); else 8 bytes per lane from registers.
  const bool staged = kOrnnLds && ornn_st;
  auto stage_put = [&](int qt, int dt, const float (&x)[4]) {
    // row 16 qt + n of this wave's rows; columns dt*16 + 4g .. +3 are half of chunk 2dt + g/2
    const int rr = 16 * qt + qn;
    const int c = (2 * dt + (g >> 1)) ^ ((wave * BMW + rr) & (OCH - 1));
    u16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = f32_to_bf16(x[i]);
    *reinterpret_cast<u16x4*>(const_cast<char*>(ornn_st) + wave * OWB + rr * (DV * 2) + c * 16 + (g & 1) * 8) = v;
  };
  auto stage_store = [&](void* dst) {
    constexpr int RPI = 64 / OCH, NI = BMW / RPI;          // rows per instruction, instructions
    const int cc = lane % OCH;
    u16x8 v[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) {                         // all reads before the first store
      const int r = j * RPI + lane / OCH;
      const int c = cc ^ ((wave * BMW + r) & (OCH - 1));
      v[j] = *reinterpret_cast<const u16x8*>(ornn_st + wave * OWB + r * (DV * 2) + c * 16);
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int t = qb0 + wave * BMW + j * RPI + lane / OCH;
      if (t < a.T)
        *reinterpret_cast<u16x8*>(static_cast<char*>(dst) + (((size_t)b * a.T + t) * a.H + h) * (DV * 2) + cc * 16) = v[j];
    }
  };
  float okv[QT][DT][4];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    float ssk = 0.f, ssr = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        okv[qt][dt][i] = acc[qt][dt][i] * inv_l[qt];
        ssk += okv[qt][dt][i] * okv[qt][dt][i];
        ssr += orn[qt][dt][i] * orn[qt][dt][i];
      }
    ssk += __shfl_xor(ssk, 16, kWave);
    ssk += __shfl_xor(ssk, 32, kWave);
    ssr += __shfl_xor(ssr, 16, kWave);
    ssr += __shfl_xor(ssr, 32, kWave);
    if (!staged && !tvalid[qt]) continue;
    const float gr = a.gate_rnn ? a.gate_rnn[tt[qt]] : 1.f;
    const float gk = a.gate_kv ? a.gate_kv[tt[qt]] : 1.f;
    const float ir = gr * __builtin_amdgcn_rsqf(ssr * (1.f / DV) + a.eps);
    const float ik = gk * __builtin_amdgcn_rsqf(ssk * (1.f / DV) + a.eps);
    uint16_t* o = static_cast<uint16_t*>(a.o);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = orn[qt][dt][i] * ir + okv[qt][dt][i] * ik;
      if (staged) {
        stage_put(qt, dt, y);
      } else {
        const size_t off = tt[qt] * DV + dt * 16 + 4 * g;
        IoBF16::store4(o, off, y);
        if (a.o_kv) IoBF16::store4(static_cast<uint16_t*>(a.o_kv), off, okv[qt][dt]);
        if (a.o_rnn) IoBF16::store4(static_cast<uint16_t*>(a.o_rnn), off, orn[qt][dt]);
      }
    }
  }
  if (staged) {
    // each wave reads back only what it wrote (LDS operations of a wave stay in order)
    stage_store(a.o);
    if (a.o_kv) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) stage_put(qt, dt, okv[qt][dt]);
      stage_store(a.o_kv);
    }
    if (a.o_rnn) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) stage_put(qt, dt, orn[qt][dt]);
      stage_store(a.o_rnn);
    }
  }
}

template <int DK, int DV>
static hipError_t launch_attn_bf16_v5(const AttnArgs& a, hipStream_t s) {
  // two 16-query tiles per wave; one at d_v = 192, where two would not fit the
  // register file of two workgroups per CU
  constexpr int QT = DV > 128 ? 1 : 2, BM = 4 * 16 * QT;
  const int nqb = (a.T + BM - 1) / BM;
  if (a.lo)
    hipLaunchKernelGGL((attn_bf16_v5_kernel<DK, DV, QT, true>), dim3(nqb * a.B * a.H), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_bf16_v5_kernel<DK, DV, QT, false>), dim3(nqb * a.B * a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Gated sum of the headwise-normalised readouts when the KV heads have another
// geometry than the RNN heads ("Hybrid Associative Memories" §2 headwise norm and
// gated sum, App. A.1 headwise gating; §4 model setup: twice the RNN heads, half
// their size, the value columns of a KV head pair tiling one RNN head's).  One wave
// per (token, RNN head), DV/64 columns per lane: the RNN norm runs over the wave,
// each KV head's over the 64/R lanes that hold its columns.
template <class IO, int DV, int R>
__global__ __launch_bounds__(256) void mix_kernel(MixArgs a) {
  using E = typename IO::elem;
  constexpr int PL = DV / 64, LK = 64 / R;
  const int lane = lane_id();
  const long long u = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);   // (token, RNN head)
  if (u >= (long long)a.ntok * a.H) return;                            // whole waves
  const long long tok = u / a.H;
  const int h = (int)(u - tok * a.H);
  const int j = h * R + lane / LK;                                      // this lane's KV head
  const size_t base = (size_t)u * DV + lane * PL;                       // same flat index both sides
  float orn[PL], okv[PL], ssr = 0.f, ssk = 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    orn[i] = a.ornn_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.o_rnn32)[base + i])
                         : a.o_rnn32[base + i];
    okv[i] = a.okv32[base + i];
    ssr += orn[i] * orn[i];
    ssk += okv[i] * okv[i];
  }
  ssr = wave_sum<64>(ssr);
#pragma unroll
  for (int m = 1; m < LK; m <<= 1) ssk += __shfl_xor(ssk, m, kWave);
  const float gr = a.gate_rnn ? a.gate_rnn[u] : 1.f;
  const float gk = a.gate_kv ? a.gate_kv[(size_t)tok * (a.H * R) + j] : 1.f;
  const float ir = gr / sqrtf(ssr / (float)DV + a.eps);
  const float ik = gk / sqrtf(ssk / (float)(DV / R) + a.eps);
  E* o = static_cast<E*>(a.o);
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    IO::store(o, base + i, orn[i] * ir + okv[i] * ik);
    if (a.o_kv) IO::store(static_cast<E*>(a.o_kv), base + i, okv[i]);
    if (a.o_rnn) IO::store(static_cast<E*>(a.o_rnn), base + i, orn[i]);
  }
}

hipError_t launch_mix(int io, int dv, const MixArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(((long long)a.ntok * a.H + 3) / 4));
#define HAM_MIX(IOT, DVV, RR) \
  if (dv == DVV && a.r == RR) { hipLaunchKernelGGL((mix_kernel<IOT, DVV, RR>), grid, dim3(256), 0, s, a); return hipGetLastError(); }
  // r = 2: KV heads of half the RNN heads' value size; r = 1: the overlapped forward
  if (io == 0) { HAM_MIX(IoF32, 128, 2) HAM_MIX(IoF32, 384, 2) HAM_MIX(IoF32, 64, 1) HAM_MIX(IoF32, 128, 1) }
  else { HAM_MIX(IoBF16, 128, 2) HAM_MIX(IoBF16, 384, 2) HAM_MIX(IoBF16, 64, 1) HAM_MIX(IoBF16, 128, 1)
         HAM_MIX(IoBF16, 384, 1) }
#undef HAM_MIX
  return hipErrorInvalidValue;
}

template <class IO, int DK, int DV>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t s) {
  const int nqb = (a.T + 63) / 64;
  hipLaunchKernelGGL((attn_kernel<IO, DK, DV>), dim3(nqb * a.B * a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(int io, int dk, int dv, const AttnArgs& a, hipStream_t s) {
#define HAM_CASE(IOT, DKV, DVV) \
  if (dk == DKV && dv == DVV) return launch_attn_t<IOT, DKV, DVV>(a, s);
  if (io == 0) {
    HAM_CASE(IoF32, 64, 64) HAM_CASE(IoF32, 64, 128) HAM_CASE(IoF32, 128, 64) HAM_CASE(IoF32, 128, 128)
    HAM_CASE(IoF32, 128, 192)
  } else {
    if (dk == 64 && dv == 64) return launch_attn_bf16_v5<64, 64>(a, s);
    if (dk == 64 && dv == 128) return launch_attn_bf16_v5<64, 128>(a, s);
    if (dk == 128 && dv == 64) return launch_attn_bf16_v5<128, 64>(a, s);
    if (dk == 128 && dv == 128) return launch_attn_bf16_v5<128, 128>(a, s);
    if (dk == 128 && dv == 192) return launch_attn_bf16_v5<128, 192>(a, s);
  }
#undef HAM_CASE
  return hipErrorInvalidValue;
}

}  // namespace ham
