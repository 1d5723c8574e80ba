// ham_route.hip -- routing score, threshold, stream compaction and statistics.
//
// "Hybrid Associative Memories": the score e_t = 1 - cos(S_{t-1}^T k_t, v_t)
// (§2 "Prediction Error as Routing Metric"; App. A.1 fit-error router), the
// threshold decision (a token enters the KV memory iff its score exceeds tau,
// App. A.1 "Forward Pass"), the data-dependent KV cache of routed tokens only
// (§2 KV-memory equation restricted to the routed set; App. A.1 "KV Memory"),
// and the KV-usage fraction rho (§5).
//
// Compaction is deterministic: per 64-token chunk one wave64 ballot gives each
// token's rank inside the chunk; a chunk's base is the sum of the earlier chunks'
// routed counts (integer sums, so their order does not matter).  No global atomics:
// the cache order is the ascending original position on every run.
#include <algorithm>

#include "ham_common.h"
#include "ham_internal.h"

namespace ham {

// grid (nchunk, B), 256 threads: all heads of one 64-token chunk.  Thread index
// runs head-fastest so that e and routed ([B,T,H]) are written contiguously; the
// per-head routed counts of the chunk are integer sums in LDS (order-independent).
// NS (score slices per token) is a compile-time constant so that every slice load
// of a thread is in flight at once.  NS = 0: the scores are the caller's (a learned
// input router's sigma(W_r x_t), App. A.1 "Router Implementations"), read from e_in.
template <int NS>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  extern __shared__ int s_cnt[];            // [H], then (block routing, if it fits)
                                            // the chunk's scores [64][H]
  float* s_e = a.blk > 1 && a.e_lds ? reinterpret_cast<float*>(s_cnt + a.H) : nullptr;
  constexpr int PER = NS > 8 ? 1 : 4;       // (token, head) pairs per thread and pass
  const int tid = threadIdx.x;
  const int c = blockIdx.x, b = blockIdx.y;
  const int nchunk = gridDim.x;
  const int H = a.H;
  for (int h = tid; h < H; h += 256) s_cnt[h] = 0;
  __syncthreads();
  const int t0 = c * kChunk;
  const int nv = min(kChunk, a.T - t0);
  const int npair = nv * H;
  for (int base = 0; base < npair; base += 256 * PER) {
    float4 x[PER][NS > 0 ? NS : 1];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = min(base + tid + 256 * j, npair - 1);
      const int tl = idx / H, h = idx - tl * H;
      if constexpr (NS > 0) {
        const float4* sp = a.score + (((size_t)b * a.T + t0 + tl) * H + h) * NS;
#pragma unroll
        for (int s = 0; s < NS; ++s) x[j][s] = sp[s];
      } else {
        x[j][0].x = a.e_in[((size_t)b * a.T + t0 + tl) * H + h];
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = base + tid + 256 * j;
      if (idx >= npair) break;
      const int tl = idx / H, h = idx - tl * H;
      float e;
      if constexpr (NS > 0) {
        float pv = 0.f, pp = 0.f, vv = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          pv += x[j][s].x; pp += x[j][s].y; vv += x[j][s].z;
        }
        float cs = 0.f;
        if (pp > 0.f && vv > 0.f) {
          cs = pv / (sqrtf(pp) * sqrtf(vv));
          cs = fminf(1.f, fmaxf(-1.f, cs));
        }
        e = 1.f - cs;
      } else {
        e = x[j][0].x;
      }
      const size_t tok = ((size_t)b * a.T + t0 + tl) * H + h;
      if constexpr (NS > 0) a.e[tok] = e;
      if (a.blk > 1) {                                               // decided per block below
        if (s_e) s_e[idx] = e;
        continue;
      }
      const bool r = e > a.tau[a.tau_per_token ? tok : (size_t)h];   // strict; NaN never routes
      a.routed[tok] = (uint8_t)r;
      if (r) atomicAdd(&s_cnt[h], 1);
    }
  }
  if (a.blk > 1) {
    // Block-contiguous routing ("Hybrid Associative Memories" §7): a block routes
    // whole on the mean of its scores, summed in token order in fp32 and scaled by
    // 1/blk (exact, blk a power of two), against tau at its last token.
    __syncthreads();                          // the scores stored above are visible
    const float* es = NS > 0 ? a.e : a.e_in;
    const float inv = 1.f / (float)a.blk;
    if (a.t_abs) {
      // decode (T = 1): the open block's sum carries over in blk_acc; the block is
      // decided at its last token
      for (int h = tid; h < H; h += 256) {
        const size_t tok = (size_t)b * H + h;
        const int j = (int)((unsigned)a.t_abs[b] % (unsigned)a.blk);
        const float sum = (j == 0 ? 0.f : a.blk_acc[tok]) + es[tok];
        a.blk_acc[tok] = sum;
        const bool r = j == a.blk - 1 && sum * inv > a.tau[a.tau_per_token ? tok : (size_t)h];
        a.routed[tok] = (uint8_t)r;
        if (r) s_cnt[h] = a.blk;
      }
    } else {
      // forward: the chunk holds whole blocks (t0 and T are multiples of blk)
      const int nb = nv / a.blk;
      for (int idx = tid; idx < nb * H; idx += 256) {
        const int j = idx / H, h = idx - j * H;
        const size_t tok0 = ((size_t)b * a.T + t0 + j * a.blk) * H + h;
        float sum = 0.f;
        if (s_e) {
          // the chunk's scores kept in LDS at (token in chunk) * H + head
          const int loc0 = j * a.blk * H + h;
          for (int i = 0; i < a.blk; ++i) sum += s_e[loc0 + i * H];
        } else {
          for (int i = 0; i < a.blk; ++i) sum += es[tok0 + (size_t)i * H];
        }
        const size_t tlast = tok0 + (size_t)(a.blk - 1) * H;
        const bool r = sum * inv > a.tau[a.tau_per_token ? tlast : (size_t)h];
        for (int i = 0; i < a.blk; ++i) a.routed[tok0 + (size_t)i * H] = (uint8_t)r;
        if (r) atomicAdd(&s_cnt[h], a.blk);
      }
    }
  }
  __syncthreads();
  for (int h = tid; h < H; h += 256) a.chunk_count[(size_t)(b * H + h) * nchunk + c] = s_cnt[h];
  if (c == 0) {
    // entering count of every cache (one per KV head)
    const int HK = a.Hkv ? a.Hkv : H;
    for (int h = tid; h < HK; h += 256) a.count_in[b * HK + h] = a.count ? a.count[b * HK + h] : 0;
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  const int nchunk = (a.T + kChunk - 1) / kChunk;
  const dim3 grid(nchunk, a.B);
  size_t lds = a.H * sizeof(int);
  // block routing keeps the chunk's scores in LDS when they fit
  RouteArgs b = a;
  b.e_lds = a.blk > 1 && !a.t_abs && a.H <= 192 ? 1 : 0;
  if (b.e_lds) lds += (size_t)kChunk * a.H * sizeof(float);
  if (b.e_in) hipLaunchKernelGGL(route_kernel<0>, grid, dim3(256), lds, s, b);
  else if (b.slices == 1) hipLaunchKernelGGL(route_kernel<1>, grid, dim3(256), lds, s, b);
  else if (b.slices == 2) hipLaunchKernelGGL(route_kernel<2>, grid, dim3(256), lds, s, b);
  else if (b.slices == 6) hipLaunchKernelGGL(route_kernel<6>, grid, dim3(256), lds, s, b);
  else if (b.slices == 8) hipLaunchKernelGGL(route_kernel<8>, grid, dim3(256), lds, s, b);
  else if (b.slices == 4) hipLaunchKernelGGL(route_kernel<4>, grid, dim3(256), lds, s, b);
  else if (b.slices == 24) hipLaunchKernelGGL(route_kernel<24>, grid, dim3(256), lds, s, b);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// grid (nchunk, H, B), 256 threads.  Writes the chunk's routed rows to the cache
// at count_in + base + rank, their positions, the per-token visible-key counts,
// and (last chunk) the new count.  ROPE: the key rows are turned by the rotary
// table on the way (a.rope; row of local token t in a forward, row b in decode).
template <class IO, int DK, int DV, bool ROPE>
__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  using E = typename IO::elem;
  constexpr int KU = DK * IO::kBytes / 16;    // 16-byte units per key row
  constexpr int VU = DV * IO::kBytes / 16;
  __shared__ int s_red[4];
  __shared__ int s_tok[kChunk];
  __shared__ int s_cnt, s_rcnt;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int bh = b * a.H + h;
  const int nchunk = gridDim.x;
  // the RNN head whose routing this cache follows
  const int Hr = a.Hr ? a.Hr : a.H;
  const int hr = h / (a.H / Hr), bhr = b * Hr + hr;

  int part = 0;
  for (int i = tid; i < c; i += 256) part += a.chunk_count[(size_t)bhr * nchunk + i];
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) part += __shfl_xor(part, m, kWave);
  if (lane == 0) s_red[wave] = part;
  __syncthreads();
  const int base = a.count_in[bh] + s_red[0] + s_red[1] + s_red[2] + s_red[3];

  // Decode with block-contiguous routing: the new token joins its open block in
  // the row count + (t_abs mod blk), past count (invisible until the block is
  // decided); a routed block is committed at its last token.
  const bool pend = a.blk > 1 && a.t_abs;
  if (wave == 0) {
    const int t = c * kChunk + lane;
    const bool valid = t < a.T;
    const bool r = valid && a.routed[((size_t)b * a.T + t) * Hr + hr];
    const bool w = pend ? valid : r;                     // rows written
    const unsigned long long bal = __ballot(w);
    const unsigned long long balr = __ballot(r);
    const int rank = __popcll(bal & ((1ull << lane) - 1ull));
    if (w) s_tok[rank] = t;
    if (a.ntok && valid) {
      // a query sees the routed tokens up to itself; with blocks, only those of the
      // blocks that end at or before it (blocks align with the chunk's lanes)
      int n = base + rank + (int)r;
      if (a.blk > 1 && (lane & (a.blk - 1)) != a.blk - 1)
        n = base + __popcll(bal & ((1ull << (lane & ~(a.blk - 1))) - 1ull));
      a.ntok[(size_t)bh * a.T + t] = min(a.cap, n);
    }
    if (lane == 0) {
      s_cnt = __popcll(bal);
      s_rcnt = __popcll(balr);
    }
  }
  __syncthreads();
  const int cnt = s_cnt;
  const int tpos0 = a.t_abs ? a.t_abs[b] : a.t0;
  const int slot0 = pend ? base + (int)((unsigned)tpos0 % (unsigned)a.blk) : base;

  const char* kb = static_cast<const char*>(a.k);
  const char* vb = static_cast<const char*>(a.v);
  char* Kb = static_cast<char*>(a.Kc);
  char* Vb = static_cast<char*>(a.Vc);
  for (int u = tid; u < cnt * (KU + VU); u += 256) {
    const int i = u / (KU + VU), w = u % (KU + VU);
    const int slot = slot0 + i;
    if (slot >= a.cap) continue;
    const size_t tok = ((size_t)b * a.T + s_tok[i]) * a.H + h;
    const size_t row = (size_t)bh * a.cap + slot;
    if (w < KU) {
      uint4 x = *reinterpret_cast<const uint4*>(kb + (tok * DK) * IO::kBytes + (size_t)w * 16);
      if constexpr (ROPE) {
        // this 16-byte unit holds the pairs starting at element e0 of the key
        constexpr int EU = 16 / IO::kBytes;
        const int e0 = w * EU;
        float f[EU];
        if constexpr (IO::kBytes == 2) {
          const uint32_t wd[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            f[2 * j] = __uint_as_float(wd[j] << 16);
            f[2 * j + 1] = __uint_as_float(wd[j] & 0xffff0000u);
          }
        } else {
          f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
          f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
        }
#pragma unroll
        for (int j = 0; j < EU / 2; ++j) {
          const int pi = e0 / 2 + j;
          const float2 cs = a.rope[(size_t)(a.t_abs ? b : s_tok[i]) * (DK / 2) + pi];
          rope_pair(f[2 * j], f[2 * j + 1], cs);
        }
        if constexpr (IO::kBytes == 2) {
          uint32_t wd[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) wd[j] = (uint32_t)f32_to_bf16(f[2 * j]) | ((uint32_t)f32_to_bf16(f[2 * j + 1]) << 16);
          x = make_uint4(wd[0], wd[1], wd[2], wd[3]);
        } else {
          x = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
        }
      }
      *reinterpret_cast<uint4*>(Kb + (row * DK) * IO::kBytes + (size_t)w * 16) = x;
    } else {
      const int wv = w - KU;
      const uint4 x = *reinterpret_cast<const uint4*>(vb + (tok * DV) * IO::kBytes + (size_t)wv * 16);
      *reinterpret_cast<uint4*>(Vb + (row * DV) * IO::kBytes + (size_t)wv * 16) = x;
    }
  }
  for (int i = tid; i < cnt; i += 256) {
    const int slot = slot0 + i;
    if (slot < a.cap) a.pos[(size_t)bh * a.cap + slot] = tpos0 + s_tok[i];
  }
  if (tid == 0) {
    if (slot0 + cnt > a.cap && a.status) *a.status = 1;
    if (c == nchunk - 1) a.count[bh] = min(a.cap, base + (pend ? (s_rcnt ? a.blk : 0) : cnt));
  }
}

template <class IO, int DK, int DV>
static hipError_t launch_compact_t(const CompactArgs& a, hipStream_t s) {
  const int nchunk = (a.T + kChunk - 1) / kChunk;
  if (a.rope)
    hipLaunchKernelGGL((compact_kernel<IO, DK, DV, true>), dim3(nchunk, a.H, a.B), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((compact_kernel<IO, DK, DV, false>), dim3(nchunk, a.H, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_compact(int io, int dk, int dv, const CompactArgs& a, hipStream_t s) {
#define HAM_CASE(IOT, DKV, DVV) \
  if (dk == DKV && dv == DVV) return launch_compact_t<IOT, DKV, DVV>(a, s);
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

// grid (H), 256 threads: per-head routed counts and near-threshold counts.
__global__ __launch_bounds__(256) void stats_kernel(StatsArgs a) {
  __shared__ long long s_red[4];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int h = blockIdx.x;
  const int nchunk = (a.T + kChunk - 1) / kChunk;
  for (int b = 0; b < a.B; ++b) {
    long long part = 0;
    for (int i = tid; i < nchunk; i += 256) part += a.chunk_count[(size_t)(b * a.H + h) * nchunk + i];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) part += __shfl_xor(part, m, kWave);
    if (lane == 0) s_red[wave] = part;
    __syncthreads();
    if (tid == 0) a.count[b * a.H + h] = (int32_t)(s_red[0] + s_red[1] + s_red[2] + s_red[3]);
    __syncthreads();
  }
  if (!a.n_near) return;
  long long near = 0;
  const long long n = (long long)a.B * a.T;
  for (long long i = tid; i < n; i += 256) {
    const size_t tok = (size_t)i * a.H + h;
    const float e = a.e[tok];
    near += (fabsf(e - a.tau[a.tau_per_token ? tok : (size_t)h]) < a.near_band) ? 1 : 0;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) near += __shfl_xor(near, m, kWave);
  if (lane == 0) s_red[wave] = near;
  __syncthreads();
  if (tid == 0) a.n_near[h] = s_red[0] + s_red[1] + s_red[2] + s_red[3];
}

hipError_t launch_stats(const StatsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(stats_kernel, dim3(a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---- threshold for a target KV fraction ---------------------------------------------
// "Hybrid Associative Memories" §5 (rho_KV, the fraction of a layer's tokens kept in
// the KV cache) and App. A.1 "Forward Pass" (a token is stored when its score exceeds
// the threshold).  For head h with N = B*T scores and k of them to keep, tau is the
// float nearest to the midpoint of the (N-k)-th and (N-k+1)-th smallest scores.
//
// One workgroup per head finds both order statistics exactly by radix select on
// order-preserving 32-bit keys (sign-magnitude floats mapped to unsigned order; every
// NaN maps to the largest key, so NaN sorts above all numbers): four 8-bit digit
// passes with LDS histograms (integer counts, so the result does not depend on the
// order of the atomic adds) give the lower statistic; one more pass counts the keys
// at or below it and takes the smallest key above it, which gives the upper one.
// Heads of up to 32768 scores keep their keys in LDS for all five passes.
HAM_DEVICE uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  if (x != x) return 0xFFFFFFFFu;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
HAM_DEVICE float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

constexpr int kSelectLdsKeys = 32768;     // a head's keys are staged in LDS up to this many

template <bool STAGED>
__global__ __launch_bounds__(1024) void select_tau_kernel(const float* __restrict__ e, int B, int T, int H,
                                                          long long k, float* __restrict__ tau) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_digit, s_below;
  __shared__ uint32_t s_le[32], s_min[32];
  __shared__ uint32_t s_keys[STAGED ? kSelectLdsKeys : 1];
  const int h = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const long long N = (long long)B * T;
  if (k <= 0 || k >= N) {
    if (tid == 0) tau[h] = (k <= 0) ? INFINITY : -INFINITY;
    return;
  }
  const uint32_t n = (uint32_t)N;
  // i = b*T + t; with STAGED the keys are read from HBM once and kept in LDS
  if constexpr (STAGED) {
    for (uint32_t i = tid; i < n; i += 1024) s_keys[i] = order_key(e[(size_t)i * H + h]);
    __syncthreads();
  }
  auto key_at = [&](uint32_t i) { return STAGED ? s_keys[i] : order_key(e[(size_t)i * H + h]); };
  // lower statistic: rank r = N-k-1 (0-based) of the ascending order
  uint32_t r = (uint32_t)(N - k - 1), prefix = 0, pmask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += 1024) hist[i] = 0;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += 1024) {
      const uint32_t key = key_at(i);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // 256 bins, 4 per lane: inclusive scan over lanes of the lane sums
      uint32_t c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = hist[lane * 4 + j]; sum += c[j]; }
      uint32_t incl = sum;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const uint32_t y = __shfl_up(incl, m, kWave);
        if (lane >= m) incl += y;
      }
      uint32_t run = incl - sum;                 // count in bins before this lane's
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run <= r && r < run + c[j]) { s_digit = (uint32_t)(lane * 4 + j); s_below = run; }
        run += c[j];
      }
    }
    __syncthreads();
    r -= s_below;
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t k1 = prefix;
  // upper statistic: rank N-k; equal to the lower one when more than N-k keys are <= it
  uint32_t le = 0, mn = 0xFFFFFFFFu;
  for (uint32_t i = tid; i < n; i += 1024) {
    const uint32_t key = key_at(i);
    le += (key <= k1);
    if (key > k1) mn = min(mn, key);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    le += __shfl_xor(le, m, kWave);
    mn = min(mn, (uint32_t)__shfl_xor(mn, m, kWave));
  }
  if (lane == 0) { s_le[wave] = le; s_min[wave] = mn; }
  __syncthreads();
  if (tid == 0) {
    uint32_t L = 0, M = 0xFFFFFFFFu;
    for (int w = 0; w < 16; ++w) { L += s_le[w]; M = min(M, s_min[w]); }
    const uint32_t k2 = (L > (uint32_t)(N - k)) ? k1 : M;
    const double mid = 0.5 * ((double)key_value(k1) + (double)key_value(k2));
    tau[h] = (float)mid;
  }
}

hipError_t launch_select_tau(const float* e, int B, int T, int H, long long k, float* tau, hipStream_t s) {
  if ((long long)B * T <= kSelectLdsKeys)
    hipLaunchKernelGGL(select_tau_kernel<true>, dim3(H), dim3(1024), 0, s, e, B, T, H, k, tau);
  else
    hipLaunchKernelGGL(select_tau_kernel<false>, dim3(H), dim3(1024), 0, s, e, B, T, H, k, tau);
  return hipGetLastError();
}

// (cos, sin) of the rotary angles, pair-fastest ([rows][dk/2]); row r is position
// t_abs[r] when t_abs is given, else t0 + r.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* table, const int32_t* t_abs, int t0,
                                                         int rows, int dk, double base) {
  const int half = dk / 2;
  const long long n = (long long)rows * half;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const int r = (int)(i / half), p = (int)(i % half);
    const double pos = t_abs ? (double)t_abs[r] : (double)t0 + r;
    table[i] = rope_cs(pos, p, dk, base);
  }
}

hipError_t launch_rope_table(float2* table, const int32_t* t_abs, int t0, int rows, int dk,
                             double base, hipStream_t s) {
  const long long n = (long long)rows * (dk / 2);
  const int blocks = (int)std::min<long long>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(rope_table_kernel, dim3(blocks), dim3(256), 0, s, table, t_abs, t0, rows, dk, base);
  return hipGetLastError();
}

// Same-document masking: lo = entries at positions < the query's document start.
// Entries are in ascending position; those of this call are counted by ntok (the
// inclusive count after local token j is ntok[j]), earlier ones by a binary search.
HAM_DEVICE int count_before(const int32_t* p, int n, long long ds) {
  int l = 0, r = n;
  while (l < r) {
    const int m = (l + r) >> 1;
    if ((long long)p[m] < ds) l = m + 1; else r = m;
  }
  return l;
}

// grid (ceil(T/256), H, B), 256 threads: one query per thread.
__global__ __launch_bounds__(256) void doc_lo_kernel(DocLoArgs a) {
  const int t = blockIdx.x * 256 + threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (t >= a.T) return;
  const int bh = b * a.H + h;
  const long long ds = a.doc_start[(size_t)b * a.T + t];
  const int32_t* ph = a.pos + (size_t)bh * a.cap;
  int lo;
  if (a.ntok && a.blk > 1) {
    // block routing: ntok counts only decided blocks, so search the whole cache
    lo = min(count_before(ph, a.count[bh], ds), a.ntok[(size_t)bh * a.T + t]);
  } else if (a.ntok) {
    const int32_t* nt = a.ntok + (size_t)bh * a.T;
    const long long j = ds - (long long)a.t0;          // local index of the start
    lo = (j >= 1) ? nt[(int)min(j - 1, (long long)t)] : count_before(ph, a.count_in[bh], ds);
    lo = min(lo, nt[t]);
  } else {
    lo = count_before(ph, a.count[bh], ds);
  }
  a.lo[(size_t)bh * a.T + t] = lo;
}

hipError_t launch_doc_lo(const DocLoArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(doc_lo_kernel, dim3((a.T + 255) / 256, a.H, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace ham
