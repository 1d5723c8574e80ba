// ham_common.h -- device helpers shared by the HAM kernels (gfx950 / CDNA4).
//
// Wave size is 64.  bf16 values travel as raw uint16 bits; conversions to bf16
// round to nearest even.  Nothing here is specific to one kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define HAM_DEVICE __device__ __forceinline__

namespace ham {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// ---- bf16 <-> fp32 ---------------------------------------------------------------
HAM_DEVICE float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950)
HAM_DEVICE uint16_t f32_to_bf16(float x) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x)); }

// ---- element type of q/k/v/cache/outputs ----------------------------------------
// IoF32: float elements.  IoBF16: bf16 bit patterns (uint16_t).
struct IoF32 {
  using elem = float;
  static constexpr int kBytes = 4;
  HAM_DEVICE static float load(const elem* p, size_t i) { return p[i]; }
  HAM_DEVICE static void store(elem* p, size_t i, float x) { p[i] = x; }
  // 4 consecutive elements (16-byte aligned base + i multiple of 4)
  HAM_DEVICE static void load4(const elem* p, size_t i, float out[4]) {
    f32x4 v = *reinterpret_cast<const f32x4*>(p + i);
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  }
  HAM_DEVICE static void store4(elem* p, size_t i, const float x[4]) {
    f32x4 v; v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
    *reinterpret_cast<f32x4*>(p + i) = v;
  }
};

struct IoBF16 {
  using elem = uint16_t;
  static constexpr int kBytes = 2;
  HAM_DEVICE static float load(const elem* p, size_t i) { return bf16_to_f32(p[i]); }
  HAM_DEVICE static void store(elem* p, size_t i, float x) { p[i] = f32_to_bf16(x); }
  HAM_DEVICE static void load4(const elem* p, size_t i, float out[4]) {
    u16x4 v = *reinterpret_cast<const u16x4*>(p + i);
    out[0] = bf16_to_f32(v[0]); out[1] = bf16_to_f32(v[1]);
    out[2] = bf16_to_f32(v[2]); out[3] = bf16_to_f32(v[3]);
  }
  HAM_DEVICE static void store4(elem* p, size_t i, const float x[4]) {
    u16x4 v;
    v[0] = f32_to_bf16(x[0]); v[1] = f32_to_bf16(x[1]);
    v[2] = f32_to_bf16(x[2]); v[3] = f32_to_bf16(x[3]);
    *reinterpret_cast<u16x4*>(p + i) = v;
  }
};

// ---- wave-level reductions (xor butterflies over `width` lanes) -----------------
template <int kWidth>
HAM_DEVICE float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < kWidth; m <<= 1) x += __shfl_xor(x, m, kWave);
  return x;
}
template <int kWidth>
HAM_DEVICE float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < kWidth; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, kWave));
  return x;
}

HAM_DEVICE int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// One 16-byte-per-lane buffer load from `base` + voff with `range_bytes` valid bytes,
// written straight to LDS at `lds` + 16 * lane (`lds` the same for the whole wave);
// offsets at or past the range read zero.  Completion is tracked by vmcnt: wait on it
// (and take a barrier for other waves' loads) before reading the bytes from LDS.
HAM_DEVICE void buffer_to_lds(const void* base, int range_bytes, int voff, char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                                               range_bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
#else
  (void)base; (void)range_bytes; (void)voff; (void)lds;
#endif
}

// Sum over the 16 lanes of a DPP row (lanes 16r..16r+15), result in every lane of
// the row: swap neighbours, swap pairs (quad permutes), then mirror within 8 and 16
// lanes.  Pure VALU (no LDS crossbar traffic).
HAM_DEVICE float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

// Transposed sum over the 16 lanes of a DPP row: every lane holds 16 values x[0..15];
// lane n of the row ends with the row total of x[n].  Four exchange steps with the
// partners n^8 (row rotate by 8), n^7 (half-row mirror), n^2 and n^1 (quad permutes);
// at each step a lane keeps the half of its remaining values selected by one bit of
// n and receives its partner's partial sums of that half.  15 exchanges instead of
// the 64 of sixteen separate row sums.
template <int kCtrl>
HAM_DEVICE float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, true));
}
HAM_DEVICE float row16_transpose_sum(const float (&x)[16], int n) {
  float y[8], z[4], w[2];
  const bool b3 = n & 8, b2 = n & 4, b1 = n & 2, b0 = n & 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = (b3 ? x[j + 8] : x[j]) + dpp_mov<0x128>(b3 ? x[j] : x[j + 8]);
#pragma unroll
  for (int j = 0; j < 4; ++j) z[j] = (b2 ? y[j + 4] : y[j]) + dpp_mov<0x141>(b2 ? y[j] : y[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j) w[j] = (b1 ? z[j + 2] : z[j]) + dpp_mov<0x4E>(b1 ? z[j] : z[j + 2]);
  return (b0 ? w[1] : w[0]) + dpp_mov<0xB1>(b0 ? w[0] : w[1]);
}

// ---- rotary position embedding ------------------------------------------------------
// "Hybrid Associative Memories" §4 model setup: a rotary embedding of base 500000 turns
// the attention path's queries and keys (RoFormer, Su et al.): pair (x_2i, x_2i+1) of a d-dimensional vector
// at absolute position pos turns by pos * base^(-2i/d).  The angle is formed and
// reduced to [-pi, pi] in double precision (at positions in the millions a float
// angle would be off by a good fraction of a radian), then cos and sin are rounded
// to float.
HAM_DEVICE float2 rope_cs(double pos, int i, int d, double base) {
  const double a = pos * exp(-2.0 * (double)i / (double)d * log(base));
  const double r = a - 6.283185307179586 * rint(a * 0.15915494309189535);
  return make_float2((float)cos(r), (float)sin(r));
}
HAM_DEVICE void rope_pair(float& x0, float& x1, float2 cs) {
  const float y0 = x0 * cs.x - x1 * cs.y;
  const float y1 = x0 * cs.y + x1 * cs.x;
  x0 = y0;
  x1 = y1;
}

// ---- XCD-aware workgroup order ----------------------------------------------------
// The dispatcher hands consecutive workgroup ids to the 8 XCDs in turn.  Renumber
// so that each XCD receives a contiguous range of logical ids: neighbouring tiles
// (for example the query blocks of one head, which share K/V) then meet in the
// same L2.
constexpr int kNumXcd = 8;
HAM_DEVICE int xcd_remap(int hw_id, int n) {
  int per = n / kNumXcd, rem = n % kNumXcd;
  int xcd = hw_id % kNumXcd, slot = hw_id / kNumXcd;
  // XCDs [0, rem) get per+1 ids, the rest get per.
  int base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + slot;
}

}  // namespace ham
