// Attention core in fp32: the reference-precision path of the library.
//
// Same method as the bf16 MFMA kernels -- the forward keeps only O and the
// per-row logsumexp, the backward recomputes scores, softmax and the Philox
// dropout mask ("Reducing Activation Recomputation in Large Transformer
// Models", LIT-736 record, Key takeaways bullet 4) -- written as one thread
// per query row (forward, dQ) or per key row (dK, dV) with fp32 FMA and an
// online softmax.  It serves small fp32 problems where 1e-5 relative accuracy
// matters more than speed; its work per head is O(s^2 d) with no data reuse.
#include "common.hpp"
#include "kernels.hpp"
#include "philox.hpp"

namespace srat {
namespace {

__device__ __forceinline__ bool keep_at(const AttnParams& p, uint32_t bb, uint32_t hg, uint32_t i,
                                        uint32_t j) {
  if (p.thresh == 0) return true;
  return (attn_keep8(p.k0, p.k1, bb, hg, i, j >> 3, p.thresh) >> (j & 7)) & 1u;
}

template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(AttnParams p) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  const int hh = blockIdx.y, bb = blockIdx.z;
  if (i >= p.s) return;
  const int g = hh / (p.hq / p.hkv);
  const float* q = static_cast<const float*>(p.q) + bb * p.sq_b + (int64_t)i * p.sq_s + hh * p.sq_h;
  const float* kb = static_cast<const float*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const float* vb = static_cast<const float*>(p.v) + bb * p.sv_b + g * p.sv_h;
  float qr[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) { qr[c] = q[c]; acc[c] = 0.f; }
  float m = -INFINITY, l = 0.f;
  const int jend = p.causal ? i + 1 : p.s;
  const uint32_t hg = (uint32_t)(p.head_offset + hh);
  for (int j = 0; j < jend; ++j) {
    const float* kr = kb + (int64_t)j * p.sk_s;
    float sdot = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) sdot = fmaf(qr[c], kr[c], sdot);
    const float sv = sdot * p.scale;
    const float mn = fmaxf(m, sv);
    const float alpha = expf(m - mn);
    const float pj = expf(sv - mn);
    l = l * alpha + pj;
    const float pd = keep_at(p, bb, hg, i, j) ? pj : 0.f;
    const float* vr = vb + (int64_t)j * p.sv_s;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] = fmaf(pd, vr[c], acc[c] * alpha);
    m = mn;
  }
  const float inv = p.inv_keep / l;
  float* o = static_cast<float*>(p.out) + bb * p.so_b + (int64_t)i * p.so_s + hh * p.so_h;
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = acc[c] * inv;
  p.lse_out[((int64_t)bb * p.hq + hh) * p.s + i] = m + logf(l);
}

// dQ for one query row; also stores D_i = rowsum(dO * O) for the dK/dV kernel.
template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(AttnParams p) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  const int hh = blockIdx.y, bb = blockIdx.z;
  if (i >= p.s) return;
  const int g = hh / (p.hq / p.hkv);
  const int64_t qoff = bb * p.sq_b + (int64_t)i * p.sq_s + hh * p.sq_h;
  const int64_t ooff = bb * p.so_b + (int64_t)i * p.so_s + hh * p.so_h;
  const float* q = static_cast<const float*>(p.q) + qoff;
  const float* o = static_cast<const float*>(p.o) + ooff;
  const float* dout = static_cast<const float*>(p.dout) + ooff;
  const float* kb = static_cast<const float*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const float* vb = static_cast<const float*>(p.v) + bb * p.sv_b + g * p.sv_h;
  float qr[D], dor[D], dq[D];
  float delta = 0.f;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qr[c] = q[c];
    dor[c] = dout[c];
    delta = fmaf(dor[c], o[c], delta);
    dq[c] = 0.f;
  }
  const int64_t row = ((int64_t)bb * p.hq + hh) * p.s + i;
  p.delta[row] = delta;
  const float lse = p.lse[row];
  const uint32_t hg = (uint32_t)(p.head_offset + hh);
  const int jend = p.causal ? i + 1 : p.s;
  for (int j = 0; j < jend; ++j) {
    const float* kr = kb + (int64_t)j * p.sk_s;
    const float* vr = vb + (int64_t)j * p.sv_s;
    float sdot = 0.f, dp = 0.f;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      sdot = fmaf(qr[c], kr[c], sdot);
      dp = fmaf(dor[c], vr[c], dp);
    }
    const float pj = expf(sdot * p.scale - lse);
    const float dpm = keep_at(p, bb, hg, i, j) ? dp * p.inv_keep : 0.f;
    const float ds = pj * (dpm - delta);
#pragma unroll
    for (int c = 0; c < D; ++c) dq[c] = fmaf(ds, kr[c], dq[c]);
  }
  float* dqo = static_cast<float*>(p.dq) + qoff;
#pragma unroll
  for (int c = 0; c < D; ++c) dqo[c] = dq[c] * p.scale;
}

// dK, dV for one key row of one kv-head, summed over the q-heads of its group.
template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dkdv_f32_kernel(AttnParams p) {
  const int j = blockIdx.x * 64 + threadIdx.x;
  const int g = blockIdx.y, bb = blockIdx.z;
  if (j >= p.s) return;
  const int grp = p.hq / p.hkv;
  const int64_t koff = bb * p.sk_b + (int64_t)j * p.sk_s + g * p.sk_h;
  const int64_t voff = bb * p.sv_b + (int64_t)j * p.sv_s + g * p.sv_h;
  const float* k = static_cast<const float*>(p.k) + koff;
  const float* v = static_cast<const float*>(p.v) + voff;
  float kr[D], vr[D], dk[D], dv[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    kr[c] = k[c];
    vr[c] = v[c];
    dk[c] = dv[c] = 0.f;
  }
  for (int hh = g * grp; hh < (g + 1) * grp; ++hh) {
    const uint32_t hg = (uint32_t)(p.head_offset + hh);
    const float* qb = static_cast<const float*>(p.q) + bb * p.sq_b + hh * p.sq_h;
    const float* db = static_cast<const float*>(p.dout) + bb * p.so_b + hh * p.so_h;
    const int64_t rowbase = ((int64_t)bb * p.hq + hh) * p.s;
    for (int i = p.causal ? j : 0; i < p.s; ++i) {
      const float* qr = qb + (int64_t)i * p.sq_s;
      const float* dor = db + (int64_t)i * p.so_s;
      float sdot = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        sdot = fmaf(qr[c], kr[c], sdot);
        dp = fmaf(dor[c], vr[c], dp);
      }
      const float pj = expf(sdot * p.scale - p.lse[rowbase + i]);
      const bool keep = keep_at(p, bb, hg, i, j);
      const float pd = keep ? pj * p.inv_keep : 0.f;
      const float ds = pj * ((keep ? dp * p.inv_keep : 0.f) - p.delta[rowbase + i]);
#pragma unroll
      for (int c = 0; c < D; ++c) {
        dv[c] = fmaf(pd, dor[c], dv[c]);
        dk[c] = fmaf(ds, qr[c], dk[c]);
      }
    }
  }
  float* dko = static_cast<float*>(p.dk) + koff;
  float* dvo = static_cast<float*>(p.dv) + voff;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    dko[c] = dk[c] * p.scale;
    dvo[c] = dv[c];
  }
}

template <int D>
hipError_t fwd_d(const AttnParams& p, hipStream_t st) {
  dim3 grid((p.s + 63) / 64, p.hq, p.b);
  TraceScope ts("attn_fwd_f32", st);
  attn_fwd_f32_kernel<D><<<grid, 64, 0, st>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_d(const AttnParams& p, hipStream_t st) {
  {
    TraceScope ts("attn_bwd_dq_f32", st);
    attn_bwd_dq_f32_kernel<D><<<dim3((p.s + 63) / 64, p.hq, p.b), 64, 0, st>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TraceScope ts("attn_bwd_dkdv_f32", st);
  attn_bwd_dkdv_f32_kernel<D><<<dim3((p.s + 63) / 64, p.hkv, p.b), 64, 0, st>>>(p);
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
