// Device helpers shared by the gfx950 kernels: element traits, MFMA fragment
// traits, rounding, wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>
#include <cmath>

#include "anchorkv_internal.hpp"

namespace akv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float -> fp16 bits, round to nearest even, saturating at +-65504.
__device__ __forceinline__ uint16_t f2h_sat(float f) {
  f = fminf(fmaxf(f, -65504.0f), 65504.0f);
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }

// Element traits: DT 1 = bf16 (stored as uint16), 2 = f32.
template <int DT> struct Elem;
template <> struct Elem<ANCHORKV_BF16> {
  using T = uint16_t;
  __device__ __forceinline__ static float f(T x) { return bf2f(x); }
};
template <> struct Elem<ANCHORKV_F32> {
  using T = float;
  __device__ __forceinline__ static float f(T x) { return x; }
};

// MFMA traits.  16x16 output tile, lane l holds rows 4*(l/16)+r (r = 0..3) of
// column l%16.  A operand: lane holds row l%16, K-slice (l/16)*KW .. +KW-1 of
// each KSTEP-wide step; B operand: column l%16, same K-slice.
template <int DT> struct Mfma;
template <> struct Mfma<ANCHORKV_BF16> {
  using frag = bf16x8;
  static constexpr int KW = 8;
  static constexpr int KSTEP = 32;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const uint16_t* p) {  // 16-byte aligned
    return *reinterpret_cast<const frag*>(p);
  }
  __device__ __forceinline__ static frag zero() {
    frag z;
    for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
    return z;
  }
};
template <> struct Mfma<ANCHORKV_F32> {
  using frag = float;
  static constexpr int KW = 1;
  static constexpr int KSTEP = 4;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const float* p) { return *p; }
  __device__ __forceinline__ static frag zero() { return 0.0f; }
};

__device__ __forceinline__ bf16x8 bits_to_frag(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Split 8 floats into bf16 hi + lo so that hi + lo carries ~16 significant bits
// (v_cvt_pk_bf16_f32: round to nearest even, two values per instruction).
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
  for (int i = 0; i < 4; ++i) {
    h[i] = cvt_pk_bf16(v[2 * i], v[2 * i + 1]);
    const float r0 = v[2 * i] - __uint_as_float(h[i] << 16);
    const float r1 = v[2 * i + 1] - __uint_as_float(h[i] & 0xFFFF0000u);
    l[i] = cvt_pk_bf16(r0, r1);
  }
  hi = bits_to_frag(make_uint4(h[0], h[1], h[2], h[3]));
  lo = bits_to_frag(make_uint4(l[0], l[1], l[2], l[3]));
}

// Cross-lane moves inside a row of 16 lanes with DPP (plain VALU, no LDS).
template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;   // quad_perm(1,0,3,2)
constexpr int kDppXor2 = 0x4E;   // quad_perm(2,3,0,1)
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8
constexpr int kDppRowMirror = 0x140;   // lane i of a row of 16 <- lane 15 - i
constexpr int kDppHalfMirror = 0x141;  // lane i of a half-row of 8 <- lane 7 - i

// Sum / max over each group of 4 lanes (l & ~3 .. l | 3); every lane gets it.
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<kDppXor1>(v);
  return v + dpp<kDppXor2>(v);
}
// Sum / max over each row of 16 lanes; every lane gets it.
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<kDppRor8>(v);
  v += dpp<kDppRor4>(v);
  return quad_sum(v);
}
// Sums over each row of 16 lanes of four per-lane values v[0..3], scattered:
// every lane of the quad (l >> 2) & 3 = j ends up with the row sum of v[j]
// (11 VALU operations instead of four full row sums).
__device__ __forceinline__ float row_sum4_scatter(const float (&v)[4], int col) {
  const bool hi8 = (col & 8) != 0, hi4 = (col & 4) != 0;
  // lanes col and 15 - col: keep v[0], v[1] (col < 8) or v[2], v[3]; add the partner's
  const float s0 = hi8 ? v[0] : v[2], s1 = hi8 ? v[1] : v[3];
  const float a0 = (hi8 ? v[2] : v[0]) + dpp<kDppRowMirror>(s0);
  const float a1 = (hi8 ? v[3] : v[1]) + dpp<kDppRowMirror>(s1);
  // lanes col and 7 - col of the half: keep one value
  const float sb = hi4 ? a0 : a1;
  const float b = (hi4 ? a1 : a0) + dpp<kDppHalfMirror>(sb);
  return quad_sum(b);
}
// Sum over the four rows of 16 lanes (lanes l, l^16, l^32, l^48), every lane
// gets it; gfx950 lane-swap instructions, no LDS.  The operand pairs are the
// same for all four lanes, so they all hold the same bits.
__device__ __forceinline__ float sum_rows4(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Integer maximum over each row of 16 lanes; every lane gets it.
template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int row_max_i32(int v) {
  v = max(v, dpp_i<kDppRor8>(v));
  v = max(v, dpp_i<kDppRor4>(v));
  v = max(v, dpp_i<kDppXor1>(v));
  return max(v, dpp_i<kDppXor2>(v));
}
__device__ __forceinline__ int row_sum_i32(int v) {
  v += dpp_i<kDppRor8>(v);
  v += dpp_i<kDppRor4>(v);
  v += dpp_i<kDppXor1>(v);
  return v + dpp_i<kDppXor2>(v);
}
// Whole-wave integer maximum (wave-uniform result).
__device__ __forceinline__ int wave_max_i32(int v) {
  v = row_max_i32(v);
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp<kDppRor8>(v));
  v = fmaxf(v, dpp<kDppRor4>(v));
  v = fmaxf(v, dpp<kDppXor1>(v));
  return fmaxf(v, dpp<kDppXor2>(v));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Whole-wave sum / max (wave-uniform result), fixed combination order.
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max(v);
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier for LDS communication only: waits for this wave's LDS
// (and scalar) operations, not for outstanding global loads, so loads issued
// ahead (prefetch) keep flying across it.  Global memory is not ordered by it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Raw buffer resource over [p, p + bytes) (p uniform): a load at an offset
// outside the range returns zero without a memory access, so a masked load
// needs no branch (and the waitcnt pass sees a fixed number of loads).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

}  // namespace akv
