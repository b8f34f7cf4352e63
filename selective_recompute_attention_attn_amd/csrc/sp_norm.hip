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
#include "common.hpp"
#include "kernels.hpp"
#include "philox.hpp"

namespace srat {
namespace {

// 8 consecutive elements <-> fp32 registers
__device__ __forceinline__ void load8(const bf16* p, float v[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const float v[8]) {
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]);
  w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]);
  w.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = w;
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
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

template <typename T, int BLOCK, int NIT, bool RMS, bool DROP>
__global__ __launch_bounds__(BLOCK) void sp_norm_fwd_kernel(NormFwdParams p) {
  __shared__ float red[2 * (BLOCK / kWave)];
  const int64_t row = blockIdx.x;
  const int hdim = p.hdim;
  const uint32_t bb = (uint32_t)(row % p.b);
  const uint32_t sg = (uint32_t)(p.seq_offset + row / p.b);
  const T* resid = static_cast<const T*>(p.resid) + row * hdim;
  const T* y = static_cast<const T*>(p.y) + row * hdim;

  float hv[NIT][8];
  float acc[1] = {0.f};
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = threadIdx.x + it * BLOCK;   // 8-column group
    if (8 * c < hdim) {
      float r[8], yy[8];
      load8(resid + 8 * c, r);
      load8(y + 8 * c, yy);
      uint32_t keep = 0xFFu;
      if (DROP) keep = hidden_keep8(p.k0, p.k1, p.tag, sg, bb, (uint32_t)c, p.thresh);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float yd = ((keep >> e) & 1u) ? yy[e] * p.inv_keep : 0.f;
        hv[it][e] = r[e] + (DROP ? yd : yy[e]);
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
      float g[8], bt[8], u[8];
      load8(p.gamma + 8 * c, g);
      if (!RMS) load8(p.beta + 8 * c, bt);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        u[e] = RMS ? hv[it][e] * rs * g[e] : (hv[it][e] - mu) * rs * g[e] + bt[e];
      store8(hout + 8 * c, hv[it]);
      store8(uout + 8 * c, u);
    }
  }
  if (threadIdx.x == 0) {
    if (!RMS) p.mean[row] = mu;
    p.rstd[row] = rs;
  }
}

template <typename T, int BLOCK, int NIT, bool RMS, bool DROP>
__global__ __launch_bounds__(BLOCK) void sp_norm_bwd_kernel(NormBwdParams p) {
  __shared__ float red[2 * (BLOCK / kWave)];
  const int hdim = p.hdim;
  const float inv_n = 1.0f / (float)hdim;
  const bool separate_dy = p.dy != p.dh;
  float gam[NIT][8], adg[NIT][8], adb[NIT][8];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = threadIdx.x + it * BLOCK;
    if (8 * c < hdim) load8(p.gamma + 8 * c, gam[it]);
#pragma unroll
    for (int e = 0; e < 8; ++e) adg[it][e] = adb[it][e] = 0.f;
  }
  const int64_t r0 = (int64_t)blockIdx.x * p.rows_per_block;
  const int64_t r1 = min(r0 + p.rows_per_block, p.rows);
  for (int64_t row = r0; row < r1; ++row) {
    const T* du = static_cast<const T*>(p.du) + row * hdim;
    const T* dres = static_cast<const T*>(p.dres) + row * hdim;
    const T* h = static_cast<const T*>(p.h) + row * hdim;
    const float mu = RMS ? 0.f : p.mean[row];
    const float rs = p.rstd[row];
    float xh[NIT][8], g[NIT][8];
    float sums[2] = {0.f, 0.f};
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = threadIdx.x + it * BLOCK;
      if (8 * c < hdim) {
        float hh[8], d[8];
        load8(h + 8 * c, hh);
        load8(du + 8 * c, d);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          xh[it][e] = (hh[e] - mu) * rs;
          g[it][e] = d[e] * gam[it][e];
          sums[0] += g[it][e];
          sums[1] += g[it][e] * xh[it][e];
          adg[it][e] += d[e] * xh[it][e];
          adb[it][e] += d[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xh[it][e] = g[it][e] = 0.f;
      }
    }
    block_sum<BLOCK>(sums, red);
    const float mg = RMS ? 0.f : sums[0] * inv_n;
    const float mgx = sums[1] * inv_n;
    const uint32_t bb = (uint32_t)(row % p.b);
    const uint32_t sg = (uint32_t)(p.seq_offset + row / p.b);
    T* dh = static_cast<T*>(p.dh) + row * hdim;
    T* dy = static_cast<T*>(p.dy) + row * hdim;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int c = threadIdx.x + it * BLOCK;
      if (8 * c < hdim) {
        float dr[8], o[8], oy[8];
        load8(dres + 8 * c, dr);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = rs * (g[it][e] - mg - xh[it][e] * mgx) + dr[e];
        store8(dh + 8 * c, o);
        if (separate_dy) {
          uint32_t keep = 0xFFu;
          if (DROP) keep = hidden_keep8(p.k0, p.k1, p.tag, sg, bb, (uint32_t)c, p.thresh);
#pragma unroll
          for (int e = 0; e < 8; ++e) oy[e] = ((keep >> e) & 1u) ? o[e] * p.inv_keep : 0.f;
          store8(dy + 8 * c, oy);
        }
      }
    }
  }
  float* part = p.partial + (int64_t)blockIdx.x * 2 * hdim;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = threadIdx.x + it * BLOCK;
    if (8 * c < hdim) {
      store8(part + 8 * c, adg[it]);
      store8(part + hdim + 8 * c, adb[it]);
    }
  }
}

// dgamma[c] = sum over blocks of partial[blk][0][c]; dbeta likewise
// (blockIdx.y = 0 / 1).  A workgroup owns 64 columns: 16 threads x float4
// across them, 16 thread rows striding over the partial blocks, then a
// reduction of the 16 row sums through LDS.
__global__ __launch_bounds__(256) void sp_norm_colsum_kernel(const float* partial, int nblk, int hdim,
                                                              float* dgamma, float* dbeta) {
  __shared__ float4 red[16][16];
  const int which = blockIdx.y;
  float* out = which ? dbeta : dgamma;
  if (out == nullptr) return;                       // RMSNorm has no dbeta
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int c = blockIdx.x * 64 + 4 * tx;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < hdim) {
    const float* src = partial + (int64_t)which * hdim + c;
    for (int k = ty; k < nblk; k += 16) {
      const float4 v = *reinterpret_cast<const float4*>(src + (int64_t)k * 2 * hdim);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  }
  red[ty][tx] = acc;
  __syncthreads();
  if (ty == 0 && c < hdim) {
    float4 t = red[0][tx];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      const float4 v = red[r][tx];
      t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
    }
    *reinterpret_cast<float4*>(out + c) = t;
  }
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

// Block size so that each thread holds at most 4 groups of 8 columns.
int pick_block(int hdim) {
  const int groups = (hdim + 7) / 8;
  int block = 64;
  while (block < 1024 && (groups + block - 1) / block > 4) block *= 2;
  return block;
}

template <typename T, int BLOCK, bool RMS, bool DROP>
hipError_t fwd_nit(const NormFwdParams& p, hipStream_t st) {
  const int nit = ((p.hdim + 7) / 8 + BLOCK - 1) / BLOCK;
  dim3 grid((unsigned)p.rows);
  switch (nit) {
    case 1: sp_norm_fwd_kernel<T, BLOCK, 1, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
    case 2: sp_norm_fwd_kernel<T, BLOCK, 2, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
    case 3: sp_norm_fwd_kernel<T, BLOCK, 3, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
    default: sp_norm_fwd_kernel<T, BLOCK, 4, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
  }
  return hipGetLastError();
}

template <typename T, int BLOCK, bool RMS, bool DROP>
hipError_t bwd_nit(const NormBwdParams& p, int nblk, hipStream_t st) {
  const int nit = ((p.hdim + 7) / 8 + BLOCK - 1) / BLOCK;
  dim3 grid((unsigned)nblk);
  switch (nit) {
    case 1: sp_norm_bwd_kernel<T, BLOCK, 1, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
    case 2: sp_norm_bwd_kernel<T, BLOCK, 2, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
    case 3: sp_norm_bwd_kernel<T, BLOCK, 3, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
    default: sp_norm_bwd_kernel<T, BLOCK, 4, RMS, DROP><<<grid, BLOCK, 0, st>>>(p); break;
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
hipError_t bwd_block(const NormBwdParams& p, int nblk, hipStream_t st) {
  switch (pick_block(p.hdim)) {
    case 64: return bwd_nit<T, 64, RMS, DROP>(p, nblk, st);
    case 128: return bwd_nit<T, 128, RMS, DROP>(p, nblk, st);
    case 256: return bwd_nit<T, 256, RMS, DROP>(p, nblk, st);
    case 512: return bwd_nit<T, 512, RMS, DROP>(p, nblk, st);
    default: return bwd_nit<T, 1024, RMS, DROP>(p, nblk, st);
  }
}

template <typename T>
hipError_t fwd_dispatch(const NormFwdParams& p, bool rms, hipStream_t st) {
  const bool drop = p.thresh != 0;
  if (rms) return drop ? fwd_block<T, true, true>(p, st) : fwd_block<T, true, false>(p, st);
  return drop ? fwd_block<T, false, true>(p, st) : fwd_block<T, false, false>(p, st);
}

template <typename T>
hipError_t bwd_dispatch(const NormBwdParams& p, int nblk, bool rms, hipStream_t st) {
  const bool drop = p.thresh != 0;
  if (rms) return drop ? bwd_block<T, true, true>(p, nblk, st) : bwd_block<T, true, false>(p, nblk, st);
  return drop ? bwd_block<T, false, true>(p, nblk, st) : bwd_block<T, false, false>(p, nblk, st);
}

}  // namespace

int norm_bwd_blocks(int64_t rows, int hdim) {
  (void)hdim;
  // about 256 row blocks: enough to cover the 256 CUs, few enough that the
  // dgamma/dbeta partials stay small next to the row traffic
  const int64_t rpb = rows >= 512 ? rows / 256 : 1;
  return (int)((rows + rpb - 1) / rpb);
}

static int64_t rows_per_block(int64_t rows, int hdim) {
  const int nblk = norm_bwd_blocks(rows, hdim);
  return (rows + nblk - 1) / nblk;
}

hipError_t launch_norm_fwd(const NormFwdParams& p, bool bf16, bool rms, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  TraceScope ts("sp_norm_fwd", st);
  return bf16 ? fwd_dispatch<srat::bf16>(p, rms, st) : fwd_dispatch<float>(p, rms, st);
}

hipError_t launch_norm_bwd(const NormBwdParams& p0, bool bf16, bool rms, hipStream_t st) {
  NormBwdParams p = p0;
  if (p.rows == 0) {
    // no rows: dgamma / dbeta are empty sums, written as zeros by the column sum
    sp_norm_colsum_kernel<<<dim3((p.hdim + 63) / 64, 2), 256, 0, st>>>(p.partial, 0, p.hdim, p.dgamma,
                                                                        rms ? nullptr : p.dbeta);
    return hipGetLastError();
  }
  p.rows_per_block = (int32_t)rows_per_block(p.rows, p.hdim);
  const int nblk = (int)((p.rows + p.rows_per_block - 1) / p.rows_per_block);
  {
    TraceScope ts("sp_norm_bwd", st);
    hipError_t e = bf16 ? bwd_dispatch<srat::bf16>(p, nblk, rms, st) : bwd_dispatch<float>(p, nblk, rms, st);
    if (e != hipSuccess) return e;
  }
  TraceScope ts("sp_norm_colsum", st);
  sp_norm_colsum_kernel<<<dim3((p.hdim + 63) / 64, 2), 256, 0, st>>>(p.partial, nblk, p.hdim, p.dgamma,
                                                                      rms ? nullptr : p.dbeta);
  return hipGetLastError();
}

hipError_t launch_hidden_mask(const NormFwdParams& p, uint8_t* mask, hipStream_t st) {
  if (p.rows == 0) return hipSuccess;
  hidden_mask_kernel<<<(unsigned)p.rows, 256, 0, st>>>(p, mask);
  return hipGetLastError();
}

}  // namespace srat
