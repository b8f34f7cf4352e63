// Shared device helpers for the libsrat kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace srat {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- wavefront reductions (64 lanes) --------------------------------------
// DPP lane exchange within rows of 16 lanes (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the 64 lanes, returned to every lane: quad_perm [1,0,3,2] and
// [2,3,0,1], row_half_mirror, row_mirror reduce each row of 16 lanes, then
// the four row sums are read from lanes 0, 16, 32, 48 (fixed order).
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<0xB1>(x);
  x += dpp_f32<0x4E>(x);
  x += dpp_f32<0x141>(x);
  x += dpp_f32<0x140>(x);
  const int xi = __float_as_int(x);
  return (__int_as_float(__builtin_amdgcn_readlane(xi, 0)) + __int_as_float(__builtin_amdgcn_readlane(xi, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(xi, 32)) + __int_as_float(__builtin_amdgcn_readlane(xi, 48)));
}

// ---- bf16 <-> fp32 ---------------------------------------------------------
__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (bf16)lo;   // round to nearest even (v_cvt_pk_bf16_f32)
  r[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- MFMA wrappers (lane layouts verified on gfx950) ------------------------
// 32x32x16 bf16: lane l holds A[l%32][8*(l/32)+e], B[8*(l/32)+e][l%32] (e = 0..7);
// D register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// LDS transpose read (gfx950): within each 16-lane group, lane j receives
// mem16[addr(4*i + j/4) + j%4] for i = 0..3, where addr(x) is the address
// supplied by lane x of the group.  A lane (4*i + t) pointing at row r0+i,
// columns c0+4t.. of a row-major tile makes lane j receive column c0+j,
// rows r0..r0+3.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(uintptr_t)p);
}

// Row stride (bf16 elements) of a D-wide tile in LDS: D/2 + pad dwords with the
// total = 20 (mod 32).  Measured on gfx950, that stride keeps both 16-byte
// row reads across 32 rows and ds_read_b64_tr_b16 4-row groups free of bank
// conflicts (strides = 24 (mod 32) double the row-read cost).
template <int D>
struct TileStride {
  static constexpr int kPadDwords = ((20 - (D / 2) % 32) + 32) % 32;
  static constexpr int kValue = D + 2 * kPadDwords;
};

}  // namespace srat
