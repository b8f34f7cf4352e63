// Attention core in fp32: the reference-precision path of the library.
//
// Same method as the bf16 kernels -- the forward keeps only O and the per-row
// logsumexp, the backward recomputes scores, softmax and the Philox dropout
// mask ("Reducing Activation Recomputation in Large Transformer Models",
// LIT-736 record, Key takeaways bullet 4) -- and the same tiling: every
// product is a 32 x 32 tile on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32, fp32 operands, fp32 accumulation), with the
// scores transposed so that each lane pair holds one query (forward, dQ) or
// one key (dK, dV).  One wave per workgroup; operands are read straight from
// global memory (this path serves small problems where 1e-5 relative
// accuracy matters more than speed).  exp and log are the accurate fp32
// library functions, not the hardware exp2.
//
// 32x32x2 fp32 MFMA lane layout (lane l, col = l % 32, h = l / 32):
//   A[i][k]: lane (i + 32 k) supplies one float     (rows i, K index k = h)
//   B[k][j]: lane (j + 32 k) supplies one float     (cols j)
//   D[i][j]: lane (j + 32 h), register r holds row 8 (r / 4) + 4 h + r % 4
// A tile's scores come out with one column (query or key) per lane pair and
// 16 rows per lane.  The second product of each kernel (O^T += V^T P^T,
// dQ^T += K^T dS^T, dV^T += dO^T P', dK^T += Q^T dS) runs its K index over
// the same 32 rows in the order of the registers: step r takes, in lane half
// h, row 8 (r / 4) + 4 h + r % 4, so each lane feeds its own register r as
// the B operand and no score crosses lanes.
#include "common.hpp"
#include "kernels.hpp"
#include "philox.hpp"

namespace srat {
namespace {

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// row of output register r in lane half h
__device__ __forceinline__ int tile_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// keep decisions of query i for the keys tile_row(r, h) of the 32-key tile at
// k0 (k0 a multiple of 8): bit r of the result
__device__ __forceinline__ uint32_t keep_row16(const AttnParams& p, uint32_t bb, uint32_t hg, int i, int k0, int h) {
  if (p.thresh == 0) return 0xFFFFu;
  uint32_t out = 0;
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const uint32_t b8 = attn_keep8(p.k0, p.k1, bb, hg, (uint32_t)i, (uint32_t)((k0 >> 3) + g4), p.thresh);
    out |= ((b8 >> (4 * h)) & 0xFu) << (4 * g4);
  }
  return out;
}

// Forward: one workgroup (one wave) per 32 queries of one (batch, q-head).
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(AttnParams p) {
  constexpr int kH = D / 2;    // K steps of the score product
  constexpr int kDB = D / 32;  // 32-row blocks of O^T
  const int lane = threadIdx.x, col = lane & 31, h = lane >> 5;
  const int q0 = blockIdx.x * 32, hh = blockIdx.y, bb = blockIdx.z;
  const int g = hh / (p.hq / p.hkv);
  const int qi = q0 + col;
  const bool qv = qi < p.s;
  const float* qp = static_cast<const float*>(p.q) + bb * p.sq_b + hh * p.sq_h;
  const float* kb = static_cast<const float*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const float* vb = static_cast<const float*>(p.v) + bb * p.sv_b + g * p.sv_h;
  const uint32_t hg = (uint32_t)(p.head_offset + hh);

  float qr[kH];   // Q[qi][2i + h]: the B operand of S^T = K Q^T
#pragma unroll
  for (int i = 0; i < kH; ++i) qr[i] = qv ? qp[(int64_t)qi * p.sq_s + 2 * i + h] : 0.f;
  f32x16 acc[kDB];   // O^T: rows d, column qi
#pragma unroll
  for (int db = 0; db < kDB; ++db) acc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;   // running max (both halves) and this half's sum

  const int kend = p.causal ? min(p.s, q0 + 32) : p.s;
  for (int k0 = 0; k0 < kend; k0 += 32) {
    const int kr = k0 + col;
    const float* krow = kb + (int64_t)(kr < p.s ? kr : 0) * p.sk_s;
    f32x16 st = f32x16{};
#pragma unroll
    for (int i = 0; i < kH; ++i) st = mfma_f32(kr < p.s ? krow[2 * i + h] : 0.f, qr[i], st);
    float sv[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + tile_row(r, h);
      const bool ok = key < p.s && (!p.causal || key <= qi);
      sv[r] = ok ? st[r] * p.scale : -INFINITY;
      tmax = fmaxf(tmax, sv[r]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(m, tmax);   // finite: key k0 is visible to every query of the tile
    const float alpha = m == -INFINITY ? 0.f : expf(m - mn);
    const uint32_t keep = keep_row16(p, (uint32_t)bb, hg, qi, k0, h);
    float pd[16];
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pj = sv[r] == -INFINITY ? 0.f : expf(sv[r] - mn);
      ls += pj;
      pd[r] = ((keep >> r) & 1u) ? pj : 0.f;
    }
    l = l * alpha + ls;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      acc[db] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + tile_row(r, h);
        const float vv = vb[(int64_t)(key < p.s ? key : 0) * p.sv_s + 32 * db + col];
        acc[db] = mfma_f32(vv, pd[r], acc[db]);
      }
    }
    m = mn;
  }
  l += __shfl_xor(l, 32);
  if (!qv) return;
  const float inv = p.inv_keep / l;
  float* o = static_cast<float*>(p.out) + bb * p.so_b + (int64_t)qi * p.so_s + hh * p.so_h;
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[32 * db + tile_row(r, h)] = acc[db][r] * inv;
  if (h == 0) p.lse_out[((int64_t)bb * p.hq + hh) * p.s + qi] = m + logf(l);
}

// dQ for 32 queries of one (batch, q-head); also stores D_i = rowsum(dO * O)
// for the dK/dV kernel.
template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(AttnParams p) {
  constexpr int kH = D / 2;
  constexpr int kDB = D / 32;
  const int lane = threadIdx.x, col = lane & 31, h = lane >> 5;
  const int q0 = blockIdx.x * 32, hh = blockIdx.y, bb = blockIdx.z;
  const int g = hh / (p.hq / p.hkv);
  const int qi = q0 + col;
  const bool qv = qi < p.s;
  const int64_t qoff = bb * p.sq_b + (int64_t)(qv ? qi : 0) * p.sq_s + hh * p.sq_h;
  const int64_t ooff = bb * p.so_b + (int64_t)(qv ? qi : 0) * p.so_s + hh * p.so_h;
  const float* q = static_cast<const float*>(p.q) + qoff;
  const float* o = static_cast<const float*>(p.o) + ooff;
  const float* dout = static_cast<const float*>(p.dout) + ooff;
  const float* kb = static_cast<const float*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const float* vb = static_cast<const float*>(p.v) + bb * p.sv_b + g * p.sv_h;
  const uint32_t hg = (uint32_t)(p.head_offset + hh);

  float qr[kH], dor[kH];   // Q and dO of query qi at columns 2i + h
  float delta = 0.f;
#pragma unroll
  for (int i = 0; i < kH; ++i) {
    qr[i] = qv ? q[2 * i + h] : 0.f;
    dor[i] = qv ? dout[2 * i + h] : 0.f;
    delta = fmaf(dor[i], qv ? o[2 * i + h] : 0.f, delta);
  }
  delta += __shfl_xor(delta, 32);
  const int64_t row = ((int64_t)bb * p.hq + hh) * p.s + qi;
  if (qv && h == 0) p.delta[row] = delta;
  const float lse = qv ? p.lse[row] : 0.f;
  f32x16 acc[kDB];   // dQ^T: rows d, column qi
#pragma unroll
  for (int db = 0; db < kDB; ++db) acc[db] = f32x16{};

  const int kend = p.causal ? min(p.s, q0 + 32) : p.s;
  for (int k0 = 0; k0 < kend; k0 += 32) {
    const int kr = k0 + col;
    const bool kv = kr < p.s;
    const float* krow = kb + (int64_t)(kv ? kr : 0) * p.sk_s;
    const float* vrow = vb + (int64_t)(kv ? kr : 0) * p.sv_s;
    f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
    for (int i = 0; i < kH; ++i) {
      st = mfma_f32(kv ? krow[2 * i + h] : 0.f, qr[i], st);
      dpt = mfma_f32(kv ? vrow[2 * i + h] : 0.f, dor[i], dpt);
    }
    const uint32_t keep = keep_row16(p, (uint32_t)bb, hg, qi, k0, h);
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + tile_row(r, h);
      const bool ok = qv && key < p.s && (!p.causal || key <= qi);
      const float pj = ok ? expf(st[r] * p.scale - lse) : 0.f;
      const float dp = ((keep >> r) & 1u) ? dpt[r] * p.inv_keep : 0.f;
      ds[r] = pj * (dp - delta);
    }
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + tile_row(r, h);
        const float kk = kb[(int64_t)(key < p.s ? key : 0) * p.sk_s + 32 * db + col];
        acc[db] = mfma_f32(kk, ds[r], acc[db]);
      }
  }
  if (!qv) return;
  float* dqo = static_cast<float*>(p.dq) + qoff;
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqo[32 * db + tile_row(r, h)] = acc[db][r] * p.scale;
}

// dK, dV for 32 keys of one kv-head, summed over the q-heads of its group
// (in the workgroup, no partials).
template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dkdv_f32_kernel(AttnParams p) {
  constexpr int kH = D / 2;
  constexpr int kDB = D / 32;
  const int lane = threadIdx.x, col = lane & 31, h = lane >> 5;
  const int k0 = blockIdx.x * 32, g = blockIdx.y, bb = blockIdx.z;
  const int grp = p.hq / p.hkv;
  const int kj = k0 + col;
  const bool kv = kj < p.s;
  const int64_t koff = bb * p.sk_b + (int64_t)(kv ? kj : 0) * p.sk_s + g * p.sk_h;
  const int64_t voff = bb * p.sv_b + (int64_t)(kv ? kj : 0) * p.sv_s + g * p.sv_h;
  float kr[kH], vr[kH];   // K and V of key kj at columns 2i + h: B operands of S and dP
#pragma unroll
  for (int i = 0; i < kH; ++i) {
    kr[i] = kv ? static_cast<const float*>(p.k)[koff + 2 * i + h] : 0.f;
    vr[i] = kv ? static_cast<const float*>(p.v)[voff + 2 * i + h] : 0.f;
  }
  f32x16 dk[kDB], dv[kDB];   // dK^T, dV^T: rows d, column kj
#pragma unroll
  for (int db = 0; db < kDB; ++db) dk[db] = dv[db] = f32x16{};

  for (int hh = g * grp; hh < (g + 1) * grp; ++hh) {
    const uint32_t hg = (uint32_t)(p.head_offset + hh);
    const float* qb = static_cast<const float*>(p.q) + bb * p.sq_b + hh * p.sq_h;
    const float* db_ = static_cast<const float*>(p.dout) + bb * p.so_b + hh * p.so_h;
    const int64_t rowbase = ((int64_t)bb * p.hq + hh) * p.s;
    for (int q0 = p.causal ? k0 : 0; q0 < p.s; q0 += 32) {
      // S = Q K^T and dP = dO V^T: rows queries q0 + tile_row(r, h), column kj
      const int qa = q0 + col;
      const float* qrow = qb + (int64_t)(qa < p.s ? qa : 0) * p.sq_s;
      const float* drow = db_ + (int64_t)(qa < p.s ? qa : 0) * p.so_s;
      f32x16 sm = f32x16{}, dpm = f32x16{};
#pragma unroll
      for (int i = 0; i < kH; ++i) {
        sm = mfma_f32(qa < p.s ? qrow[2 * i + h] : 0.f, kr[i], sm);
        dpm = mfma_f32(qa < p.s ? drow[2 * i + h] : 0.f, vr[i], dpm);
      }
      float pd[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qrr = q0 + tile_row(r, h);
        const bool ok = kv && qrr < p.s && (!p.causal || kj <= qrr);
        const float lse = ok ? p.lse[rowbase + qrr] : 0.f;
        const float delta = ok ? p.delta[rowbase + qrr] : 0.f;
        const float pj = ok ? expf(sm[r] * p.scale - lse) : 0.f;
        const bool keep = p.thresh == 0 ||
                          ((attn_keep8(p.k0, p.k1, (uint32_t)bb, hg, (uint32_t)qrr, (uint32_t)(kj >> 3), p.thresh) >>
                            (kj & 7)) & 1u);
        pd[r] = keep ? pj * p.inv_keep : 0.f;
        ds[r] = pj * ((keep ? dpm[r] * p.inv_keep : 0.f) - delta);
      }
      // dV^T += dO^T P', dK^T += Q^T dS over the tile's queries
#pragma unroll
      for (int d32 = 0; d32 < kDB; ++d32)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrr = q0 + tile_row(r, h);
          const int64_t qo = (int64_t)(qrr < p.s ? qrr : 0);
          dv[d32] = mfma_f32(db_[qo * p.so_s + 32 * d32 + col], pd[r], dv[d32]);
          dk[d32] = mfma_f32(qb[qo * p.sq_s + 32 * d32 + col], ds[r], dk[d32]);
        }
    }
  }
  if (!kv) return;
  float* dko = static_cast<float*>(p.dk) + koff;
  float* dvo = static_cast<float*>(p.dv) + voff;
#pragma unroll
  for (int d32 = 0; d32 < kDB; ++d32)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dko[32 * d32 + tile_row(r, h)] = dk[d32][r] * p.scale;
      dvo[32 * d32 + tile_row(r, h)] = dv[d32][r];
    }
}

template <int D>
hipError_t fwd_d(const AttnParams& p, hipStream_t st) {
  dim3 grid((p.s + 31) / 32, p.hq, p.b);
  TraceScope ts("attn_fwd_f32", st);
  attn_fwd_f32_kernel<D><<<grid, 64, 0, st>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const AttnParams& p, hipStream_t st) {
  {
    TraceScope ts("attn_bwd_dq_f32", st);
    attn_bwd_dq_f32_kernel<D><<<dim3((p.s + 31) / 32, p.hq, p.b), 64, 0, st>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TraceScope ts("attn_bwd_dkdv_f32", st);
  attn_bwd_dkdv_f32_kernel<D><<<dim3((p.s + 31) / 32, p.hkv, p.b), 64, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnParams& p, hipStream_t st) {
  switch (p.d) {
    case 32: return fwd_d<32>(p, st);
    case 64: return fwd_d<64>(p, st);
    case 96: return fwd_d<96>(p, st);
    case 128: return fwd_d<128>(p, st);
    case 160: return fwd_d<160>(p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd_f32(const AttnParams& p, hipStream_t st) {
  switch (p.d) {
    case 32: return bwd_d<32>(p, st);
    case 64: return bwd_d<64>(p, st);
    case 96: return bwd_d<96>(p, st);
    case 128: return bwd_d<128>(p, st);
    case 160: return bwd_d<160>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace srat
