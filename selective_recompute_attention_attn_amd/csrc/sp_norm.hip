// Sequence-parallel norm region: hidden dropout + residual + LayerNorm/RMSNorm,
// forward and backward, over one rank's [s_local, b, h] rows.
//
// These are the operations tensor parallelism leaves replicated (the layer
// norm and the dropout after attention or the MLP) and sequence parallelism
// splits along the sequence, each position being independent ("Reducing
// Activation Recomputation in Large Transformer Models", LIT-736 record, Key
// takeaways bullets 1-2).
//
// HBM-bound: one pass over each tensor, 16-byte vector loads/stores, the whole
// row held in registers between the reduction and the output pass, the dropout
// mask regenerated from Philox (one call per 8 columns, matching one 16-byte
// bf16 vector).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"
#include "philox.hpp"

namespace srat {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements <-> fp32 registers (stores non-temporal: each output
// is written once and not read back by this kernel).
__device__ __forceinline__ void load8(const bf16* p, float v[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
  v[0] = bf16_lo(w[0]); v[1] = bf16_hi(w[0]);
  v[2] = bf16_lo(w[1]); v[3] = bf16_hi(w[1]);
  v[4] = bf16_lo(w[2]); v[5] = bf16_hi(w[2]);
  v[6] = bf16_lo(w[3]); v[7] = bf16_hi(w[3]);
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  const u32x4 a = q[0], b = q[1];
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = __uint_as_float(a[e]); v[4 + e] = __uint_as_float(b[e]); }
}
__device__ __forceinline__ void store8_nt(bf16* p, const float v[8]) {
  u32x4 w;
  w[0] = pack_bf16x2(v[0], v[1]);
  w[1] = pack_bf16x2(v[2], v[3]);
  w[2] = pack_bf16x2(v[4], v[5]);
  w[3] = pack_bf16x2(v[6], v[7]);
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store8_nt(float* p, const float v[8]) {
  u32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) { a[e] = __float_as_uint(v[e]); b[e] = __float_as_uint(v[4 + e]); }
  __builtin_nontemporal_store(a, reinterpret_cast<u32x4*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<u32x4*>(p) + 1);
}

// Raw row loads.  A row's 8-column groups are fetched as 16-byte pieces (one
// per group for bf16, two for fp32) through a buffer resource sized to the
// row: groups past the row's end read as zero, so the loads need no branch and
// all of a thread's pieces are in flight before the first is used (a
// bounds-checked load converted on the spot serialises the round trips).
template <typename T>
struct Piece {
  static constexpr int kN = (int)sizeof(T) / 2;   // 16-byte pieces per 8 columns
};
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t row, int hdim) {
  return buffer_rsrc(static_cast<const T*>(base) + row * hdim, (uint32_t)hdim * (uint32_t)sizeof(T));
}
// NT: non-temporal (streamed once)
template <typename T, bool NT>
__device__ __forceinline__ void load_piece(__amdgpu_buffer_rsrc_t r, int c, u32x4 (&w)[Piece<T>::kN]) {
#pragma unroll
  for (int n = 0; n < Piece<T>::kN; ++n)
    w[n] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         r, (int)(16 * (Piece<T>::kN * c + n)), 0, NT ? 2 : 0));
}
__device__ __forceinline__ void unpack8(const u32x4 (&w)[1], float v[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(w[0][i]); v[2 * i + 1] = bf16_hi(w[0][i]); }
}
__device__ __forceinline__ void unpack8(const u32x4 (&w)[2], float v[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = __uint_as_float(w[0][i]); v[4 + i] = __uint_as_float(w[1][i]); }
}

// An fp32 [h] vector (gamma, beta) for the thread's column groups, the same way.
template <int NIT, int BLOCK>
__device__ __forceinline__ void load_vec(const float* v, int hdim, float (&out)[NIT][8]) {
  const __amdgpu_buffer_rsrc_t r = buffer_rsrc(v, (uint32_t)hdim * 4u);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    u32x4 w[2];
    load_piece<float, false>(r, threadIdx.x + it * BLOCK, w);
    unpack8(w, out[it]);
  }
}

// Sum of `n` values per thread over the block; every thread gets the totals.
template <int BLOCK, int N>
__device__ __forceinline__ void block_sum(float (&x)[N], float* red) {
  constexpr int kWaves = BLOCK / kWave;
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = wave_sum(x[i]);
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  if (kWaves > 1) {
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < N; ++i) red[i * kWaves + wv] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float t = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) t += red[i * kWaves + w];
      x[i] = t;
    }
    __syncthreads();
  }
}

// Forward.  A workgroup owns rows blockIdx.x, blockIdx.x + gridDim.x, ...;
// with PIPE the loads of its next row are issued before the current row is
// reduced and written, so each CU keeps reading while it writes.  gamma / beta
// stay in registers across the rows.  Every row is held in registers through
// its two reductions (mean, then the variance of the held values), and h, u
// are streamed out with non-temporal stores.
template <typename T, int NIT, int BLOCK>
__device__ __forceinline__ void fwd_load(const NormFwdParams& p, int64_t row, u32x4 (&x)[NIT][Piece<T>::kN],
                                         u32x4 (&y)[NIT][Piece<T>::kN]) {
  const __amdgpu_buffer_rsrc_t rx = row_rsrc<T>(p.resid, row, p.hdim);
  const __amdgpu_buffer_rsrc_t ry = row_rsrc<T>(p.y, row, p.hdim);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = threadIdx.x + it * BLOCK;   // 8-column group
    load_piece<T, true>(rx, c, x[it]);
    load_piece<T, true>(ry, c, y[it]);
  }
}

// HOLD: gamma / beta come in registers (g, bt); otherwise they are loaded
// here, next to their use (large rows, where registers are short).
template <typename T, int BLOCK, int NIT, bool RMS, bool DROP, bool HOLD>
__device__ __forceinline__ void fwd_row(const NormFwdParams& p, int64_t row, const u32x4 (&xr)[NIT][Piece<T>::kN],
                                        const u32x4 (&yr)[NIT][Piece<T>::kN], const float (&g)[NIT][8],
                                        const float (&bt)[NIT][8], float* red) {
  const int hdim = p.hdim;
  float hv[NIT][8];
  const uint32_t bb = (uint32_t)(row % p.b);
  const uint32_t sg = (uint32_t)(p.seq_offset + row / p.b);
  float acc[1] = {0.f};
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = threadIdx.x + it * BLOCK;
    if (8 * c < hdim) {
      float yv[8];
      unpack8(xr[it], hv[it]);
      unpack8(yr[it], yv);
      uint32_t keep = 0xFFu;
      if (DROP) keep = hidden_keep8(p.k0, p.k1, p.tag, sg, bb, (uint32_t)c, p.thresh);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float yd = ((keep >> e) & 1u) ? yv[e] * p.inv_keep : 0.f;
        hv[it][e] = hv[it][e] + (DROP ? yd : yv[e]);
        acc[0] += RMS ? hv[it][e] * hv[it][e] : hv[it][e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[it][e] = 0.f;
    }
  }
  block_sum<BLOCK>(acc, red);
  const float inv_n = 1.0f / (float)hdim;
  float mu = 0.f, rs;
  if (RMS) {
    rs = 1.0f / sqrtf(acc[0] * inv_n + p.eps);
  } else {
    mu = acc[0] * inv_n;
    float v[1] = {0.f};
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (8 * (int)(threadIdx.x + it * BLOCK) < hdim) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float dlt = hv[it][e] - mu;
          v[0] += dlt * dlt;
        }
      }
    }
    block_sum<BLOCK>(v, red);
    rs = 1.0f / sqrtf(v[0] * inv_n + p.eps);
  }
  T* hout = static_cast<T*>(p.h) + row * hdim;
  T* uout = static_cast<T*>(p.u) + row * hdim;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = threadIdx.x + it * BLOCK;
    if (8 * c < hdim) {
      float u[8], gl[8], bl[8];
      if (!HOLD) {
        load8(p.gamma + 8 * c, gl);
        if (!RMS) load8(p.beta + 8 * c, bl);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ge = HOLD ? g[it][e] : gl[e];
        const float be = RMS ? 0.f : (HOLD ? bt[it][e] : bl[e]);
        u[e] = RMS ? hv[it][e] * rs * ge : (hv[it][e] - mu) * rs * ge + be;
      }
      store8_nt(hout + 8 * c, hv[it]);
      store8_nt(uout + 8 * c, u);
    }
  }
  if (threadIdx.x == 0) {
    if (!RMS) p.mean[row] = mu;
    p.rstd[row] = rs;
  }
}

template <typename T, int BLOCK, int NIT, bool RMS, bool DROP, bool PIPE>
__global__ __launch_bounds__(BLOCK) void sp_norm_fwd_kernel(NormFwdParams p) {
  constexpr bool kHold = NIT <= 3;
  __shared__ float red[2 * (BLOCK / kWave)];
  const int64_t stride = gridDim.x;
  int64_t row = blockIdx.x;             // < rows: the grid never exceeds the row count
  u32x4 xa[NIT][Piece<T>::kN], ya[NIT][Piece<T>::kN];
  fwd_load<T, NIT, BLOCK>(p, row, xa, ya);
  float g[NIT][8], bt[NIT][8];
  if (kHold) {
    load_vec<NIT, BLOCK>(p.gamma, p.hdim, g);
    if (!RMS) load_vec<NIT, BLOCK>(p.beta, p.hdim, bt);
  }
  if (!PIPE) {
    fwd_row<T, BLOCK, NIT, RMS, DROP, kHold>(p, row, xa, ya, g, bt, red);
    return;
  }
  u32x4 xb[NIT][Piece<T>::kN], yb[NIT][Piece<T>::kN];
  while (true) {
    const int64_t r1 = row + stride;
    if (r1 < p.rows) fwd_load<T, NIT, BLOCK>(p, r1, xb, yb);
    fwd_row<T, BLOCK, NIT, RMS, DROP, kHold>(p, row, xa, ya, g, bt, red);
    if (r1 >= p.rows) break;
    const int64_t r2 = r1 + stride;
    if (r2 < p.rows) fwd_load<T, NIT, BLOCK>(p, r2, xa, ya);
    fwd_row<T, BLOCK, NIT, RMS, DROP, kHold>(p, r1, xb, yb, g, bt, red);
    if (r2 >= p.rows) break;
    row = r2;
  }
}

// Backward, one launch with two kinds of workgroup:
//  * the first `col_blocks` workgroups each own a slab of 32 columns and sum
//    dgamma = sum_rows du * xhat and dbeta = sum_rows du over ALL rows (rows
//    split over BLOCK/4 thread groups, then a fixed-order reduction), so the
//    sums need no partials in memory, no atomics, and are reproducible;
//  * the other workgroups each own one row: all loads issued up front, the
//    two row sums, then dh and dy streamed out.
// Both read du and h (the column pass re-reads 4 bytes per element instead of
// writing and reading per-block partials, which cost more when rows are few).
constexpr int kColSlab = 32;

// slab handled by column workgroup `bid`: consecutive slabs (which share
// 128-byte lines of every row) go to the same XCD, which receives every
// eighth workgroup of the launch
__device__ __forceinline__ int xcd_slab(int bid, int col_blocks) {
  const int per = col_blocks / 8;
  return (bid % 8) * per + bid / 8;
}

template <typename T, int BLOCK, bool RMS>
__device__ __forceinline__ void colsum_job(const NormBwdParams& p, int slab, float* red) {
  constexpr int kRG = BLOCK / 4;
  constexpr int kU = BLOCK >= 1024 ? 4 : 8;   // rows in flight per thread (register budget)
  const int v = threadIdx.x & 3, rg = threadIdx.x >> 2;
  const int hdim = p.hdim;
  const int c = kColSlab * slab + 8 * v;
  float ag[8], ab[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ag[e] = ab[e] = 0.f;
  if (c < hdim) {
    const T* du = static_cast<const T*>(p.du) + c;
    const T* h = static_cast<const T*>(p.h) + c;
    int64_t r = rg;
    for (; r + (int64_t)(kU - 1) * kRG < p.rows; r += (int64_t)kU * kRG) {
      float d[kU][8], x[kU][8], mu[kU], rs[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t rr = r + (int64_t)u * kRG;
        load8(du + rr * hdim, d[u]);
        load8(h + rr * hdim, x[u]);
        mu[u] = RMS ? 0.f : p.mean[rr];
        rs[u] = p.rstd[rr];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ag[e] += d[u][e] * ((x[u][e] - mu[u]) * rs[u]);
          ab[e] += d[u][e];
        }
    }
    for (; r < p.rows; r += kRG) {
      float d[8], x[8];
      load8(du + r * hdim, d);
      load8(h + r * hdim, x);
      const float mu = RMS ? 0.f : p.mean[r], rs = p.rstd[r];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ag[e] += d[e] * ((x[e] - mu) * rs);
        ab[e] += d[e];
      }
    }
  }
  // lanes with equal (lane & 3) hold the same columns: sum over lane bits 2..5
#pragma unroll
  for (int off = 4; off < kWave; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ag[e] += __shfl_xor(ag[e], off, kWave);
      ab[e] += __shfl_xor(ab[e], off, kWave);
    }
  constexpr int kWaves = BLOCK / kWave;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  if (lane < 4) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red[(wv * 4 + lane) * 16 + e] = ag[e];
      red[(wv * 4 + lane) * 16 + 8 + e] = ab[e];
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int vv = threadIdx.x >> 4, k = threadIdx.x & 15;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[(w * 4 + vv) * 16 + k];
    const int col = kColSlab * slab + 8 * vv + (k & 7);
    if (col < hdim) {
      if (k < 8) p.dgamma[col] = t;
      else if (!RMS) p.dbeta[col] = t;
    }
  }
}

template <typename T, int NIT, int BLOCK>
__device__ __forceinline__ void bwd_load(const NormBwdParams& p, int64_t row, u32x4 (&x)[NIT][Piece<T>::kN],
                                         u32x4 (&d)[NIT][Piece<T>::kN], u32x4 (&r)[NIT][Piece<T>::kN]) {
  const __amdgpu_buffer_rsrc_t rh = row_rsrc<T>(p.h, row, p.hdim);
  const __amdgpu_buffer_rsrc_t rd = row_rsrc<T>(p.du, row, p.hdim);
  const __amdgpu_buffer_rsrc_t rr = row_rsrc<T>(p.dres, row, p.hdim);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = threadIdx.x + it * BLOCK;
    load_piece<T, false>(rh, c, x[it]);
    load_piece<T, false>(rd, c, d[it]);
    load_piece<T, true>(rr, c, r[it]);
  }
}

template <typename T, int BLOCK, int NIT, bool RMS, bool DROP, bool HOLD>
__device__ __forceinline__ void bwd_row(const NormBwdParams& p, int64_t row, const u32x4 (&xr)[NIT][Piece<T>::kN],
                                        const u32x4 (&dur)[NIT][Piece<T>::kN], const u32x4 (&drr)[NIT][Piece<T>::kN],
                                        const float (&gam)[NIT][8], float* red) {
  float xh[NIT][8], g[NIT][8];
  const int hdim = p.hdim;
  const float inv_n = 1.0f / (float)hdim;
  const float mu = RMS ? 0.f : p.mean[row];
  const float rs = p.rstd[row];
  float sums[2] = {0.f, 0.f};
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = threadIdx.x + it * BLOCK;
    if (8 * c < hdim) {
      float gl[8];
      if (!HOLD) load8(p.gamma + 8 * c, gl);
      unpack8(xr[it], xh[it]);
      unpack8(dur[it], g[it]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xh[it][e] = (xh[it][e] - mu) * rs;
        g[it][e] = g[it][e] * (HOLD ? gam[it][e] : gl[e]);
        sums[0] += g[it][e];
        sums[1] += g[it][e] * xh[it][e];
      }
    }
  }
  block_sum<BLOCK>(sums, red);
  const float mg = RMS ? 0.f : sums[0] * inv_n;
  const float mgx = sums[1] * inv_n;
  const bool separate_dy = p.dy != p.dh;
  const uint32_t bb = (uint32_t)(row % p.b);
  const uint32_t sg = (uint32_t)(p.seq_offset + row / p.b);
  T* dh = static_cast<T*>(p.dh) + row * hdim;
  T* dy = static_cast<T*>(p.dy) + row * hdim;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = threadIdx.x + it * BLOCK;
    if (8 * c < hdim) {
      float o[8], oy[8], dr[8];
      unpack8(drr[it], dr);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = rs * (g[it][e] - mg - xh[it][e] * mgx) + dr[e];
      store8_nt(dh + 8 * c, o);
      if (separate_dy) {
        uint32_t keep = 0xFFu;
        if (DROP) keep = hidden_keep8(p.k0, p.k1, p.tag, sg, bb, (uint32_t)c, p.thresh);
#pragma unroll
        for (int e = 0; e < 8; ++e) oy[e] = ((keep >> e) & 1u) ? o[e] * p.inv_keep : 0.f;
        store8_nt(dy + 8 * c, oy);
      }
    }
  }
}

// Row workgroups: one row each, every load issued up front, gamma held in
// registers.  (Walking two rows with prefetch, as the forward does, measured
// slower here: the column workgroups already keep the memory busy.)
template <typename T, int BLOCK, int NIT, bool RMS, bool DROP>
__device__ __forceinline__ void bwd_rows(const NormBwdParams& p, int64_t row, float* red) {
  constexpr bool kHold = NIT <= 3;
  u32x4 xa[NIT][Piece<T>::kN], da[NIT][Piece<T>::kN], ra[NIT][Piece<T>::kN];
  bwd_load<T, NIT, BLOCK>(p, row, xa, da, ra);
  float gam[NIT][8];
  if (kHold) load_vec<NIT, BLOCK>(p.gamma, p.hdim, gam);
  bwd_row<T, BLOCK, NIT, RMS, DROP, kHold>(p, row, xa, da, ra, gam, red);
}

template <typename T, int BLOCK, int NIT, bool RMS, bool DROP>
__global__ __launch_bounds__(BLOCK) void sp_norm_bwd_kernel(NormBwdParams p) {
  __shared__ float red[(BLOCK / kWave) * 4 * 16];
  const int bid = blockIdx.x;
  if (bid < p.col_blocks) {
    const int slab = xcd_slab(bid, p.col_blocks);
    if (kColSlab * slab < p.hdim) colsum_job<T, BLOCK, RMS>(p, slab, red);
    return;
  }
  bwd_rows<T, BLOCK, NIT, RMS, DROP>(p, bid - p.col_blocks, red);
}

__global__ void hidden_mask_kernel(NormFwdParams p, uint8_t* mask) {
  const int64_t row = blockIdx.x;
  const uint32_t bb = (uint32_t)(row % p.b);
  const uint32_t sg = (uint32_t)(p.seq_offset + row / p.b);
  for (int c = threadIdx.x; 8 * c < p.hdim; c += blockDim.x) {
    const uint32_t keep = p.thresh ? hidden_keep8(p.k0, p.k1, p.tag, sg, bb, (uint32_t)c, p.thresh) : 0xFFu;
    for (int e = 0; e < 8; ++e) mask[row * p.hdim + 8 * c + e] = (keep >> e) & 1u;
  }
}

// Block size so that each thread holds at most 3 groups of 8 columns (4 only
// in 1024-thread blocks, for rows above 24576 elements).
int pick_block(int hdim) {
  const int groups = (hdim + 7) / 8;
  int block = 64;
  while (block < 1024 && (groups + block - 1) / block > 3) block *= 2;
  return block;
}

// Forward workgroups: up to 512, each walking rows with one row of prefetch
// when it has more than one (PIPE; blocks of up to 512 threads keep two rows
// in registers without spilling).  1024-thread blocks take one row each.
constexpr int kMaxRowBlocks = 512;
int64_t row_blocks(int64_t rows, int block) {
  return block <= 512 ? std::min<int64_t>(rows, kMaxRowBlocks) : rows;
}

template <typename T, int BLOCK, bool RMS, bool DROP>
hipError_t fwd_nit(const NormFwdParams& p, hipStream_t st) {
  const int nit = ((p.hdim + 7) / 8 + BLOCK - 1) / BLOCK;
  constexpr bool kPipe = BLOCK <= 512;
  dim3 grid((unsigned)row_blocks(p.rows, BLOCK));
  constexpr int kMaxNit = BLOCK == 1024 ? 4 : 3;
  switch (nit) {
    case 1: sp_norm_fwd_kernel<T, BLOCK, 1, RMS, DROP, kPipe><<<grid, BLOCK, 0, st>>>(p); break;
    case 2: sp_norm_fwd_kernel<T, BLOCK, 2, RMS, DROP, kPipe><<<grid, BLOCK, 0, st>>>(p); break;
    case 3: sp_norm_fwd_kernel<T, BLOCK, 3, RMS, DROP, kPipe><<<grid, BLOCK, 0, st>>>(p); break;
    default: sp_norm_fwd_kernel<T, BLOCK, kMaxNit, RMS, DROP, kPipe><<<grid, BLOCK, 0, st>>>(p); break;
  }
  return hipGetLastError();
}

template <typename T, int BLOCK, bool RMS, bool DROP>
hipError_t bwd_nit(NormBwdParams p, hipStream_t st) {
  const int nit = ((p.hdim + 7) / 8 + BLOCK - 1) / BLOCK;
  dim3 grid((unsigned)(p.col_blocks + p.rows));
  constexpr int kMaxNit = BLOCK == 1024 ? 4 : 3;
  switch (nit) {
    case 1: sp_norm_bwd_kernel<T, BLOCK, 1, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
    case 2: sp_norm_bwd_kernel<T, BLOCK, 2, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
    case 3: sp_norm_bwd_kernel<T, BLOCK, 3, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
    default: sp_norm_bwd_kernel<T, BLOCK, kMaxNit, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
  }
  return hipGetLastError();
}

template <typename T, bool RMS, bool DROP>
hipError_t fwd_block(const NormFwdParams& p, hipStream_t st) {
  switch (pick_block(p.hdim)) {
    case 64: return fwd_nit<T, 64, RMS, DROP>(p, st);
    case 128: return fwd_nit<T, 128, RMS, DROP>(p, st);
    case 256: return fwd_nit<T, 256, RMS, DROP>(p, st);
    case 512: return fwd_nit<T, 512, RMS, DROP>(p, st);
    default: return fwd_nit<T, 1024, RMS, DROP>(p, st);
  }
}

template <typename T, bool RMS, bool DROP>
hipError_t bwd_block(const NormBwdParams& p, hipStream_t st) {
  switch (pick_block(p.hdim)) {
    case 64: return bwd_nit<T, 64, RMS, DROP>(p, st);
    case 128: return bwd_nit<T, 128, RMS, DROP>(p, st);
    case 256: return bwd_nit<T, 256, RMS, DROP>(p, st);
    case 512: return bwd_nit<T, 512, RMS, DROP>(p, st);
    default: return bwd_nit<T, 1024, RMS, DROP>(p, st);
  }
}

template <typename T>
hipError_t fwd_dispatch(const NormFwdParams& p, bool rms, hipStream_t st) {
  const bool drop = p.thresh != 0;
  if (rms) return drop ? fwd_block<T, true, true>(p, st) : fwd_block<T, true, false>(p, st);
  return drop ? fwd_block<T, false, true>(p, st) : fwd_block<T, false, false>(p, st);
}

template <typename T>
hipError_t bwd_dispatch(const NormBwdParams& p, bool rms, hipStream_t st) {
  const bool drop = p.thresh != 0;
  if (rms) return drop ? bwd_block<T, true, true>(p, st) : bwd_block<T, true, false>(p, st);
  return drop ? bwd_block<T, false, true>(p, st) : bwd_block<T, false, false>(p, st);
}

}  // namespace

int norm_bwd_col_blocks(int hdim) {
  const int nslab = (hdim + kColSlab - 1) / kColSlab;
  return 8 * ((nslab + 7) / 8);
}

// The backward grid is col_blocks + rows workgroups of pick_block(h) threads:
// it must stay below 2^32 work-items and 2^31 workgroups.
int64_t norm_bwd_max_rows(int64_t hdim) {
  if (hdim <= 0 || hdim > 32768) return 0;
  const int64_t block = pick_block((int)hdim);
  const int64_t cols = norm_bwd_col_blocks((int)hdim);
  return std::min<int64_t>((((int64_t)1 << 32) - 1) / block, ((int64_t)1 << 31) - 1) - cols;
}

hipError_t launch_norm_fwd(const NormFwdParams& p, bool bf16, bool rms, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  TraceScope ts("sp_norm_fwd", st);
  return bf16 ? fwd_dispatch<srat::bf16>(p, rms, st) : fwd_dispatch<float>(p, rms, st);
}

hipError_t launch_norm_bwd(const NormBwdParams& p0, bool bf16, bool rms, hipStream_t st) {
  NormBwdParams p = p0;
  // no rows: the column workgroups alone run and write dgamma / dbeta = 0
  p.col_blocks = norm_bwd_col_blocks(p.hdim);
  TraceScope ts("sp_norm_bwd", st);
  return bf16 ? bwd_dispatch<srat::bf16>(p, rms, st) : bwd_dispatch<float>(p, rms, st);
}

hipError_t launch_hidden_mask(const NormFwdParams& p, uint8_t* mask, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  hidden_mask_kernel<<<(unsigned)p.rows, 256, 0, st>>>(p, mask);
  return hipGetLastError();
}

}  // namespace srat
