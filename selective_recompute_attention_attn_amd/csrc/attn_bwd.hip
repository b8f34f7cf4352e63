// Attention-core backward with recomputation, bf16 in / fp32 accumulate, MFMA.
//
// Selective activation recomputation drops the attention core's activations
// (scores, softmax, dropout mask and output) after the forward and re-runs the
// core in the backward pass ("Reducing Activation Recomputation in Large
// Transformer Models", LIT-736 record, Key takeaways bullet 4).  Here the
// re-run is fused into the gradient kernel, tile by tile, so nothing of size
// s x s is ever written:
//
//   S  = Q K^T * scale,  P = exp(S - LSE)          (recomputed)
//   M  = Philox keep mask                           (regenerated, bit-exact)
//   dV = (P*M)^T dO / (1-p)
//   dP = dO V^T * M / (1-p),  dS = P * (dP - D),  D = rowsum(dO * O)
//   dQ = dS K * scale,        dK = dS^T Q * scale
//
// Three kernels on one stream:
//   pre : D = rowsum(dO * O) per query row, zero the fp32 dQ accumulator
//   main: one workgroup per (128-key block, q-head, batch); 4 waves, wave w
//         owns keys 32w .. 32w+31 of the block.  It loops over 32-query tiles:
//         S^T = K Q^T and dP^T = V dO^T with K, V as register-resident MFMA A
//         operands (rows permuted as in the forward, so one lane holds one
//         query and 16 consecutive keys: softmax recompute, mask and dS are
//         lane-local and one Philox call covers 8 keys).  P*M and dS go to LDS
//         once; dV, dK read them back transposed with ds_read_b64_tr_b16, dQ
//         reads dS directly and K transposed; dQ is added to the fp32
//         accumulator with hardware float atomics.
//   post: dQ accumulator -> dQ (x scale, bf16); grouped-query attention: dK,
//         dV summed over the q-heads that share a kv-head.
#include "common.hpp"
#include "kernels.hpp"
#include "philox.hpp"

namespace srat {
namespace {

constexpr int kBNk = 128;      // keys per workgroup
constexpr int kBMq = 32;       // queries per iteration
constexpr int kThreads = 256;  // 4 waves

template <int D>
struct BwdSmem {
  static constexpr int kS = D + 8;       // row stride of K, Q, dO tiles (bf16)
  static constexpr int kP = kBNk + 8;    // row stride of the P*M and dS tiles
  bf16 k[kBNk * kS];
  bf16 q[kBMq * kS];
  bf16 dout[kBMq * kS];
  bf16 pm[kBMq * kP];
  bf16 ds[kBMq * kP];
};

__device__ __forceinline__ int perm32(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// Two ds_read_b64_tr_b16 of a row-major bf16 tile give the 32x32x16 MFMA
// operand "lane (i = l%32, h = l/32) holds column c_base + i, rows
// r_base + 8h .. +7": lane group G = l/16 covers columns c_base + 16*(G%2) ..
// and rows r_base + 8*(G/2) ...
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int stride, int r_base, int c_base, int lane) {
  const int grp = lane >> 4, lg = lane & 15;
  const int r = r_base + 8 * (grp >> 1) + (lg >> 2);
  const int c = c_base + 16 * (grp & 1) + 4 * (lg & 3);
  const s16x4 lo = lds_read_tr16(tile + r * stride + c);
  const s16x4 hi = lds_read_tr16(tile + (r + 4) * stride + c);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int D, bool CAUSAL, bool DROP, bool GQA>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_bf16_kernel(AttnParams p) {
  using SM = BwdSmem<D>;
  constexpr int kS = SM::kS, kP = SM::kP;
  constexpr int kDC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kTileChunks = kBMq * D / 8;                       // 16-byte chunks per Q or dO tile
  constexpr int kTileLoads = (kTileChunks + kThreads - 1) / kThreads;
  __shared__ SM sm;

  const int nkb = (p.s + kBNk - 1) / kBNk;
  const int bh = blockIdx.x % (p.b * p.hq);
  const int kblk = (int)(blockIdx.x / (p.b * p.hq));   // ascending: most work first when causal
  const int hh_q = bh % p.hq, bb = bh / p.hq;
  const int g = hh_q / (p.hq / p.hkv);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int k0 = kblk * kBNk;
  const int kw0 = k0 + 32 * wv;          // first key of this wave
  (void)nkb;

  const bf16* qp = static_cast<const bf16*>(p.q) + bb * p.sq_b + hh_q * p.sq_h;
  const bf16* dop = static_cast<const bf16*>(p.dout) + bb * p.so_b + hh_q * p.so_h;
  const bf16* kp = static_cast<const bf16*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const bf16* vp = static_cast<const bf16*>(p.v) + bb * p.sv_b + g * p.sv_h;
  const int64_t row0 = ((int64_t)bb * p.hq + hh_q) * p.s;
  float* dqa = p.dq_acc + ((int64_t)bb * p.s * p.hq + hh_q) * D;   // [b, s, hq, d] contiguous

  // K block -> LDS (row-major, for the dQ operand)
#pragma unroll
  for (int it = 0; it < kBNk * D / 8 / kThreads; ++it) {
    const int x = tid + kThreads * it;
    const int r = x / (D / 8), c8 = x % (D / 8);
    uint4 w = make_uint4(0, 0, 0, 0);
    if (k0 + r < p.s) w = *reinterpret_cast<const uint4*>(kp + (int64_t)(k0 + r) * p.sk_s + 8 * c8);
    *reinterpret_cast<uint4*>(&sm.k[r * kS + 8 * c8]) = w;
  }
  // K, V rows of this wave as MFMA A operands (rows permuted)
  bf16x8 kreg[kDC], vreg[kDC];
  {
    const int key = kw0 + perm32(col);
#pragma unroll
    for (int c = 0; c < kDC; ++c) {
      if (key < p.s) {
        kreg[c] = *reinterpret_cast<const bf16x8*>(kp + (int64_t)key * p.sk_s + 16 * c + 8 * half);
        vreg[c] = *reinterpret_cast<const bf16x8*>(vp + (int64_t)key * p.sv_s + 16 * c + 8 * half);
      } else {
        kreg[c] = bf16x8{};
        vreg[c] = bf16x8{};
      }
    }
  }

  f32x16 dv_acc[kDB], dk_acc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) dv_acc[db] = dk_acc[db] = f32x16{};

  const int nqt = (p.s + kBMq - 1) / kBMq;
  const int qt0 = CAUSAL ? k0 / kBMq : 0;
  uint4 qpre[kTileLoads], dpre[kTileLoads];
  auto prefetch = [&](int qt) {
#pragma unroll
    for (int it = 0; it < kTileLoads; ++it) {
      const int x = tid + kThreads * it;
      const int r = x / (D / 8), c8 = x % (D / 8);
      const int qrow = qt * kBMq + r;
      qpre[it] = dpre[it] = make_uint4(0, 0, 0, 0);
      if (x < kTileChunks && qrow < p.s) {
        qpre[it] = *reinterpret_cast<const uint4*>(qp + (int64_t)qrow * p.sq_s + 8 * c8);
        dpre[it] = *reinterpret_cast<const uint4*>(dop + (int64_t)qrow * p.so_s + 8 * c8);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int it = 0; it < kTileLoads; ++it) {
      const int x = tid + kThreads * it;
      if (x < kTileChunks) {
        const int r = x / (D / 8), c8 = x % (D / 8);
        *reinterpret_cast<uint4*>(&sm.q[r * kS + 8 * c8]) = qpre[it];
        *reinterpret_cast<uint4*>(&sm.dout[r * kS + 8 * c8]) = dpre[it];
      }
    }
  };

  const uint32_t hg = (uint32_t)(p.head_offset + hh_q);
  if (qt0 < nqt) prefetch(qt0);
  for (int qt = qt0; qt < nqt; ++qt) {
    __syncthreads();
    stash();
    __syncthreads();
    if (qt + 1 < nqt) prefetch(qt + 1);
    const int qi = qt * kBMq + col;       // this lane's query
    const bool qvalid = qi < p.s;
    const float lse2 = qvalid ? p.lse[row0 + qi] * kLog2e : 0.f;
    const float dlt = qvalid ? p.delta[row0 + qi] : 0.f;
    // whole wave above the diagonal of this tile: its P and dS are zero
    const bool dead = (CAUSAL && kw0 > qt * kBMq + kBMq - 1) || kw0 >= p.s;

    float pmv[16], dsv[16];
    if (!dead) {
      f32x16 sacc = f32x16{}, pacc = f32x16{};
      const bf16* qrow = &sm.q[col * kS + 8 * half];
      const bf16* drow = &sm.dout[col * kS + 8 * half];
#pragma unroll
      for (int c = 0; c < kDC; ++c) {
        sacc = mfma32(kreg[c], *reinterpret_cast<const bf16x8*>(qrow + 16 * c), sacc);
        pacc = mfma32(vreg[c], *reinterpret_cast<const bf16x8*>(drow + 16 * c), pacc);
      }
      uint32_t bits = 0xFFFFu;
      if (DROP) {
        const uint32_t g8 = (uint32_t)((kw0 + 16 * half) >> 3);
        bits = attn_keep8(p.k0, p.k1, (uint32_t)bb, hg, (uint32_t)qi, g8, p.thresh) |
               (attn_keep8(p.k0, p.k1, (uint32_t)bb, hg, (uint32_t)qi, g8 + 1, p.thresh) << 8);
      }
      const bool edge = (kw0 + 32 > p.s) || (CAUSAL && kw0 + 31 > qt * kBMq) || !qvalid;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = __builtin_amdgcn_exp2f(sacc[r] * p.scale_log2 - lse2);
        if (edge) {
          const int key = kw0 + 16 * half + r;
          if (key >= p.s || (CAUSAL && key > qi) || !qvalid) pv = 0.f;
        }
        const bool keep = (bits >> r) & 1u;
        pmv[r] = keep ? pv : 0.f;
        dsv[r] = pv * ((keep ? pacc[r] * p.inv_keep : 0.f) - dlt);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) pmv[r] = dsv[r] = 0.f;
    }
    // P*M and dS rows of this lane's query: keys 32w + 16*half .. +15 of the block
    {
      uint4 w0, w1;
      w0.x = pack_bf16x2(pmv[0], pmv[1]);   w0.y = pack_bf16x2(pmv[2], pmv[3]);
      w0.z = pack_bf16x2(pmv[4], pmv[5]);   w0.w = pack_bf16x2(pmv[6], pmv[7]);
      w1.x = pack_bf16x2(pmv[8], pmv[9]);   w1.y = pack_bf16x2(pmv[10], pmv[11]);
      w1.z = pack_bf16x2(pmv[12], pmv[13]); w1.w = pack_bf16x2(pmv[14], pmv[15]);
      uint4* dst = reinterpret_cast<uint4*>(&sm.pm[col * kP + 32 * wv + 16 * half]);
      dst[0] = w0;
      dst[1] = w1;
      w0.x = pack_bf16x2(dsv[0], dsv[1]);   w0.y = pack_bf16x2(dsv[2], dsv[3]);
      w0.z = pack_bf16x2(dsv[4], dsv[5]);   w0.w = pack_bf16x2(dsv[6], dsv[7]);
      w1.x = pack_bf16x2(dsv[8], dsv[9]);   w1.y = pack_bf16x2(dsv[10], dsv[11]);
      w1.z = pack_bf16x2(dsv[12], dsv[13]); w1.w = pack_bf16x2(dsv[14], dsv[15]);
      dst = reinterpret_cast<uint4*>(&sm.ds[col * kP + 32 * wv + 16 * half]);
      dst[0] = w0;
      dst[1] = w1;
    }
    lds_fence();   // this wave's own P*M / dS columns are read back below

    if (!dead) {
      // dV_w += (P*M)^T dO ;  dK_w += dS^T Q   (contraction over the 32 queries)
#pragma unroll
      for (int st = 0; st < kBMq / 16; ++st) {
        const bf16x8 apm = tr_operand(sm.pm, kP, 16 * st, 32 * wv, lane);
        const bf16x8 ads = tr_operand(sm.ds, kP, 16 * st, 32 * wv, lane);
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          dv_acc[db] = mfma32(apm, tr_operand(sm.dout, kS, 16 * st, 32 * db, lane), dv_acc[db]);
          dk_acc[db] = mfma32(ads, tr_operand(sm.q, kS, 16 * st, 32 * db, lane), dk_acc[db]);
        }
      }
    }
    __syncthreads();   // every wave's dS is in LDS

    // dQ (32 queries x D) = dS (32 x 128 keys) K (128 x D); wave w takes d blocks w, w+4, ...
    const int kend = min(kBNk, p.s - k0);           // keys of the block that exist
    const int nst = CAUSAL ? min((kend + 15) / 16, (qt * kBMq + kBMq - 1 - k0) / 16 + 1) : (kend + 15) / 16;
    for (int db = wv; db < kDB; db += 4) {
      f32x16 qacc = f32x16{};
      for (int st = 0; st < nst; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.ds[col * kP + 16 * st + 8 * half]);
        qacc = mfma32(a, tr_operand(sm.k, kS, 16 * st, 32 * db, lane), qacc);
      }
      // lane holds d = 32db + col, queries 8*(r/4) + 4*half + r%4 of the tile
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qq = qt * kBMq + 8 * (r >> 2) + 4 * half + (r & 3);
        if (qq < p.s) unsafeAtomicAdd(dqa + (int64_t)qq * p.hq * D + 32 * db + col, qacc[r]);
      }
    }
  }

  // epilogue: lane holds d = 32db + col, keys kw0 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key >= p.s) continue;
      const float dvv = dv_acc[db][r] * p.inv_keep;
      const float dkv = dk_acc[db][r] * p.scale;
      const int dcol = 32 * db + col;
      if (GQA) {
        const int64_t o = (((int64_t)bb * p.s + key) * p.hq + hh_q) * D + dcol;
        p.dv_part[o] = dvv;
        p.dk_part[o] = dkv;
      } else {
        static_cast<bf16*>(p.dv)[bb * p.sv_b + (int64_t)key * p.sv_s + g * p.sv_h + dcol] = (bf16)dvv;
        static_cast<bf16*>(p.dk)[bb * p.sk_b + (int64_t)key * p.sk_s + g * p.sk_h + dcol] = (bf16)dkv;
      }
    }
  }
}

// D = rowsum(dO * O) for every (b, q-head, query) row; zero the dQ accumulator.
// 8 lanes per row, lane t takes 8-element chunks t, t+8, ...
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(AttnParams p) {
  const int64_t rows = (int64_t)p.b * p.s * p.hq;            // ordered (b, s, hq)
  const int64_t row = (int64_t)blockIdx.x * 32 + threadIdx.x / 8;
  const int t = threadIdx.x & 7;
  float acc = 0.f;
  if (row < rows) {
    const int hh = (int)(row % p.hq);
    const int64_t bs = row / p.hq;
    const int i = (int)(bs % p.s), bb = (int)(bs / p.s);
    const bf16* o = static_cast<const bf16*>(p.o) + bb * p.so_b + (int64_t)i * p.so_s + hh * p.so_h;
    const bf16* d = static_cast<const bf16*>(p.dout) + bb * p.so_b + (int64_t)i * p.so_s + hh * p.so_h;
    float* z = p.dq_acc + row * D;
    for (int c = t; c < D / 8; c += 8) {
      const uint4 a = *reinterpret_cast<const uint4*>(o + 8 * c);
      const uint4 b = *reinterpret_cast<const uint4*>(d + 8 * c);
      acc += bf16_lo(a.x) * bf16_lo(b.x) + bf16_hi(a.x) * bf16_hi(b.x) + bf16_lo(a.y) * bf16_lo(b.y) +
             bf16_hi(a.y) * bf16_hi(b.y) + bf16_lo(a.z) * bf16_lo(b.z) + bf16_hi(a.z) * bf16_hi(b.z) +
             bf16_lo(a.w) * bf16_lo(b.w) + bf16_hi(a.w) * bf16_hi(b.w);
      reinterpret_cast<float4*>(z + 8 * c)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
      reinterpret_cast<float4*>(z + 8 * c)[1] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  acc += __shfl_xor(acc, 1, kWave);
  acc += __shfl_xor(acc, 2, kWave);
  acc += __shfl_xor(acc, 4, kWave);
  if (row < rows && t == 0) {
    const int hh = (int)(row % p.hq);
    const int64_t bs = row / p.hq;
    const int i = (int)(bs % p.s), bb = (int)(bs / p.s);
    p.delta[((int64_t)bb * p.hq + hh) * p.s + i] = acc;
  }
}

// dQ = acc * scale -> bf16; GQA: dK, dV = sum of the group's per-q-head partials.
template <int D, bool GQA>
__global__ __launch_bounds__(256) void attn_bwd_post_kernel(AttnParams p) {
  const int64_t nq = (int64_t)p.b * p.s * p.hq * (D / 8);    // 8-element chunks of dQ
  const int64_t nk = GQA ? (int64_t)p.b * p.s * p.hkv * (D / 8) : 0;
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x < nq) {
    const int c8 = (int)(x % (D / 8));
    const int64_t row = x / (D / 8);                           // (b, s, hq)
    const int hh = (int)(row % p.hq);
    const int64_t bs = row / p.hq;
    const int i = (int)(bs % p.s), bb = (int)(bs / p.s);
    const float* a = p.dq_acc + row * D + 8 * c8;
    const float4 u = reinterpret_cast<const float4*>(a)[0];
    const float4 v = reinterpret_cast<const float4*>(a)[1];
    uint4 w;
    w.x = pack_bf16x2(u.x * p.scale, u.y * p.scale);
    w.y = pack_bf16x2(u.z * p.scale, u.w * p.scale);
    w.z = pack_bf16x2(v.x * p.scale, v.y * p.scale);
    w.w = pack_bf16x2(v.z * p.scale, v.w * p.scale);
    *reinterpret_cast<uint4*>(static_cast<bf16*>(p.dq) + bb * p.sq_b + (int64_t)i * p.sq_s + hh * p.sq_h + 8 * c8) = w;
  } else if (GQA && x < nq + nk) {
    const int64_t y = x - nq;
    const int c8 = (int)(y % (D / 8));
    const int64_t row = y / (D / 8);                           // (b, s, hkv)
    const int gg = (int)(row % p.hkv);
    const int64_t bs = row / p.hkv;
    const int i = (int)(bs % p.s), bb = (int)(bs / p.s);
    const int grp = p.hq / p.hkv;
    float sk[8] = {0, 0, 0, 0, 0, 0, 0, 0}, sv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < grp; ++j) {
      const int64_t o = (((int64_t)bb * p.s + i) * p.hq + gg * grp + j) * D + 8 * c8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sk[e] += p.dk_part[o + e];
        sv[e] += p.dv_part[o + e];
      }
    }
    uint4 wk, wv;
    wk.x = pack_bf16x2(sk[0], sk[1]); wk.y = pack_bf16x2(sk[2], sk[3]);
    wk.z = pack_bf16x2(sk[4], sk[5]); wk.w = pack_bf16x2(sk[6], sk[7]);
    wv.x = pack_bf16x2(sv[0], sv[1]); wv.y = pack_bf16x2(sv[2], sv[3]);
    wv.z = pack_bf16x2(sv[4], sv[5]); wv.w = pack_bf16x2(sv[6], sv[7]);
    *reinterpret_cast<uint4*>(static_cast<bf16*>(p.dk) + bb * p.sk_b + (int64_t)i * p.sk_s + gg * p.sk_h + 8 * c8) = wk;
    *reinterpret_cast<uint4*>(static_cast<bf16*>(p.dv) + bb * p.sv_b + (int64_t)i * p.sv_s + gg * p.sv_h + 8 * c8) = wv;
  }
}

template <int D, bool CAUSAL, bool DROP>
hipError_t main_launch(const AttnParams& p, hipStream_t st) {
  const int nkb = (p.s + kBNk - 1) / kBNk;
  const dim3 grid((unsigned)(nkb * p.hq * p.b));
  if (p.hq != p.hkv) attn_bwd_bf16_kernel<D, CAUSAL, DROP, true><<<grid, kThreads, 0, st>>>(p);
  else attn_bwd_bf16_kernel<D, CAUSAL, DROP, false><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_launch_d(const AttnParams& p, hipStream_t st) {
  const int64_t rows = (int64_t)p.b * p.s * p.hq;
  {
    TraceScope ts("attn_bwd_pre", st);
    attn_bwd_pre_kernel<D><<<(unsigned)((rows + 31) / 32), 256, 0, st>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    TraceScope ts("attn_bwd_bf16", st);
    const bool drop = p.thresh != 0;
    hipError_t e;
    if (p.causal) e = drop ? main_launch<D, true, true>(p, st) : main_launch<D, true, false>(p, st);
    else e = drop ? main_launch<D, false, true>(p, st) : main_launch<D, false, false>(p, st);
    if (e != hipSuccess) return e;
  }
  TraceScope ts("attn_bwd_post", st);
  const bool gqa = p.hq != p.hkv;
  const int64_t n = rows * (D / 8) + (gqa ? (int64_t)p.b * p.s * p.hkv * (D / 8) : 0);
  const unsigned blocks = (unsigned)((n + 255) / 256);
  if (gqa) attn_bwd_post_kernel<D, true><<<blocks, 256, 0, st>>>(p);
  else attn_bwd_post_kernel<D, false><<<blocks, 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_f32(const AttnParams& p, hipStream_t st);

hipError_t launch_attn_bwd(const AttnParams& p, bool bf16_path, hipStream_t st) {
  if (p.s == 0 || p.b == 0) return hipSuccess;
  if (!bf16_path) return launch_attn_bwd_f32(p, st);
  switch (p.d) {
    case 32: return bwd_launch_d<32>(p, st);
    case 64: return bwd_launch_d<64>(p, st);
    case 96: return bwd_launch_d<96>(p, st);
    case 128: return bwd_launch_d<128>(p, st);
    case 160: return bwd_launch_d<160>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace srat
