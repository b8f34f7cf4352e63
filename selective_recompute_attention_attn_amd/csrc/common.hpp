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

// Max / sum of x over lanes l and l ^ 32 (the two halves of the wave), the
// same value in both, without an LDS round trip: v_permlane32_swap with both
// operands x leaves the lower half's values in both halves of one result and
// the upper half's in the other (lane order of the operands is the same in
// both halves, so the sum is bitwise identical there).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- bf16 <-> fp32 ---------------------------------------------------------
__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (bf16)lo;   // round to nearest even (v_cvt_pk_bf16_f32)
  r[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}
// a & (b | c) in one v_bitop3_b32 (truth table 0xE0 = 0xF0 & (0xCC | 0xAA)):
// keeps the halves of a packed pair selected by the masks b (low) and c (high).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0xE0);
}
// Dropout of a packed bf16 pair by a packed pair of 16-bit draws w: each half
// of `pair` is kept iff its draw is >= T, given tm1 = (T-1) in both halves
// (T >= 1, wave-uniform).  Three packed 16-bit ops: the saturating difference
// draw - (T-1) is 0 exactly for the dropped halves, its minimum with 1 is the
// keep bit, and the 16-bit product of a half's bits with that bit keeps or
// clears it.  Written as instructions because the compiler turns the same
// expression in C into per-half compares and selects (five ops).  ALU only.
__device__ __forceinline__ uint32_t drop_pair(uint32_t pair, uint32_t w, uint32_t tm1) {
  uint32_t d, k, r;
  asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(d) : "v"(w), "s"(tm1));
  asm("v_pk_min_u16 %0, %1, %2" : "=v"(k) : "v"(d), "s"(0x00010001u));
  asm("v_pk_mul_lo_u16 %0, %1, %2" : "=v"(r) : "v"(pair), "v"(k));
  return r;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---- MFMA wrappers (lane layouts verified on gfx950) ------------------------
// 32x32x16 bf16: lane l holds A[l%32][8*(l/32)+e], B[8*(l/32)+e][l%32] (e = 0..7);
// D register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- buffer loads ------------------------------------------------------------
// Raw buffer resource over `nbytes` bytes from `base` (gfx9 word 3): loads at
// offsets >= nbytes return zero without touching memory, so a tile that runs
// past the end of a tensor needs no branch.  Base and size MUST be
// wave-uniform; they are moved to scalar registers explicitly (otherwise the
// compiler may not prove it and wraps every load in a readfirstlane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(nbytes);
  void* b = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voffset, 0, 0));
}

// Buffer -> LDS load of 16 bytes per lane (gfx950): lane l's bytes land at
// LDS address lds + 16 l, with lds wave-uniform (it goes to M0); voffset is
// the lane's byte offset into the buffer, past its end reading zero.  The
// load counts on vmcnt like any buffer load; wait on it (wait_vmcnt) and then
// a barrier before other waves read the bytes.
//
// Written as one asm statement (set M0, issue the load) with no outputs and a
// memory clobber: the compiler then neither reorders memory accesses across
// it nor treats it as a pending LDS store, which would make it wait for every
// such load before the next LDS read (and drain all prefetching).  The caller
// waits with wait_vmcnt; loads the compiler does not see can only make its
// own vmcnt waits stricter, never insufficient.
typedef uint32_t sgpr4 __attribute__((ext_vector_type(4)));
// Buffer resource as four scalar registers: base (48 bits), stride 0, the
// byte count, gfx9 word 3 (as buffer_rsrc above).
__device__ __forceinline__ sgpr4 buffer_rsrc_sgpr(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  sgpr4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xFFFFu;
  r[2] = __builtin_amdgcn_readfirstlane(nbytes);
  r[3] = 0x00020000u;
  return r;
}
__device__ __forceinline__ void buffer_load16_lds(sgpr4 r, uintptr_t lds, uint32_t voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)lds);
  // M0 is reserved to the compiler, which uses it in these kernels for
  // nothing else (no LDS-DMA builtins, no indirect register indexing)
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(m0), "v"(voffset), "s"(r) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Blocks b < nblocks with b = w (mod 4): the buffer -> LDS loads wave w of a
// 4-wave group issues for one tile when the group shares its blocks out.
__host__ __device__ constexpr int blocks_of_wave(int nblocks, int w) { return (nblocks - w + 3) / 4; }
// wait_vmcnt<N> with N = the count of the wave's most recent loads that may
// stay in flight, which differs between the waves of a group (wave-uniform
// branch on w = 0..3)
template <int N0, int N1, int N2, int N3>
__device__ __forceinline__ void wait_vmcnt_by_wave(int w) {
  if (w == 0) wait_vmcnt<N0>();
  else if (w == 1) wait_vmcnt<N1>();
  else if (w == 2) wait_vmcnt<N2>();
  else wait_vmcnt<N3>();
}

// Workgroup barrier that waits only for the wave's own LDS accesses
// (lgkmcnt), not for its loads in flight; one asm statement with a memory
// clobber, so the compiler moves no memory access across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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

// Row stride of a tile that is only ever read as 16-byte rows (MFMA operands
// in row order): 4 dwords of padding, total = 4 or 20 (mod 32) dwords, also
// measured conflict-free for that access and smaller than TileStride.
template <int D>
struct RowStride {
  static_assert((D / 2) % 16 == 0, "D must be a multiple of 32");
  static constexpr int kValue = D + 8;
};

// Launch order of a split grid, longest work first.  Tiles t = 0 .. n-1 are
// modelled to take 2(t+1) units of work (a causal tile's span grows with
// t); the top nsplit tiles run as two halves of t+1 units each.  Workgroup
// `rank` (0 .. n + nsplit - 1) gets tile t and part 0 / 1 (a half) or -1
// (whole), so that ranks come in decreasing modelled work: the dispatcher
// then packs the CUs the way longest-processing-time-first scheduling does.
// Every (tile, part) is produced by exactly one rank.  Wave-uniform.
__device__ __forceinline__ void split_order(int rank, int n, int nsplit, int& t, int& part) {
  int r = rank;
  t = 0;
  part = -1;
  for (int len = 2 * n; len >= 1; --len) {
    if ((len & 1) == 0 && len / 2 - 1 < n - nsplit) {   // whole tile len/2 - 1
      if (r == 0) { t = len / 2 - 1; part = -1; return; }
      --r;
    }
    if (len - 1 >= n - nsplit && len - 1 < n) {        // the halves of tile len - 1
      if (r < 2) { t = len - 1; part = r; return; }
      r -= 2;
    }
  }
}

}  // namespace srat
