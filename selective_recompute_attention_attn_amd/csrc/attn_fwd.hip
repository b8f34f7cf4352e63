// Attention-core forward, bf16 in / fp32 accumulate, MFMA on gfx950.
//
//   O = dropout(softmax(Q K^T * scale)) V,  LSE = log-sum-exp of each score row
//
// Only O and LSE leave the kernel; the scores, the softmax and the dropout mask
// live in registers one tile at a time.  That is the selective-recomputation
// contract: the attention core's activations are the large, cheap ones, so they
// are not stored and the backward pass rebuilds them ("Reducing Activation
// Recomputation in Large Transformer Models", LIT-736 record, Key takeaways
// bullet 4), with the K/V tiling of FlashAttention (METP page, Introduction,
// third paragraph).
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one
// (batch, q-head); K/V tiles of 64 keys staged through LDS):
//   * Each wave computes S^T = K Q^T for its 32 queries with
//     v_mfma_f32_32x32x16_bf16: Q^T is the B operand (held in registers for the
//     whole loop), K the A operand (from LDS).  The output layout gives every
//     lane ONE query and 16 keys, so the row max / row sum are lane-local plus
//     one exchange with lane^32.
//   * K rows are fed to the MFMA in a permuted order, so that lane half hh of a
//     32-key block holds the 16 consecutive keys 16*hh .. 16*hh+15: each group
//     of 8 keys of one query is exactly one Philox call (8 x 16-bit draws).
//   * O^T = V^T P^T: P^T (bf16) is the B operand straight from registers; V^T
//     is read from the row-major V tile in LDS with ds_read_b64_tr_b16, which
//     transposes 4x16 blocks on the fly.  The O accumulator is therefore also
//     one query per lane, so the online-softmax rescale is lane-local.
//   * The dropout scale 1/(1-p) is applied once in the epilogue, not per
//     element.
#include "common.hpp"
#include "kernels.hpp"
#include "philox.hpp"

namespace srat {
namespace {

constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // keys per K/V tile
constexpr int kThreads = 256;  // 4 waves
// The running max only moves when a tile's max exceeds it by more than this
// (log2 units): probabilities stay <= 2^8, and the O / l rescale is rare.
constexpr float kMaxSlack = 8.0f;

template <int D>
struct alignas(16) FwdSmem {
  static constexpr int kStride = TileStride<D>::kValue;
  bf16 k[kBN * kStride];
  bf16 v[kBN * kStride];
};

// MFMA row (slot) m of a 32-key block carries key perm32(m): slots
// 8a + 4hh + jj hold keys 16hh + 4a + jj, so output register r of lane half hh
// is key 16hh + r.
__device__ __forceinline__ int perm32(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
// Inverse of perm32: the MFMA slot of key k of a 32-key block.  K rows are
// stored in LDS in slot order, so the A-operand reads are consecutive rows.
__device__ __forceinline__ int slot32(int k) { return 8 * ((k >> 2) & 3) + 4 * (k >> 4) + (k & 3); }

// Causal q-tile order: the first half of the grid runs the longest tiles
// first, the second half the shortest first, so two workgroups that share a
// CU (block i and block i + grid/2) carry equal work.
__device__ __forceinline__ int causal_tile(int rank, int nqt) {
  const int h = (nqt + 1) / 2;
  return rank < h ? nqt - 1 - rank : rank - h;
}

template <int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(AttnParams p) {
  constexpr int kStride = FwdSmem<D>::kStride;
  constexpr int kDC = D / 16;        // 16-wide d chunks (QK^T k-steps)
  constexpr int kDB = D / 32;        // 32-wide d blocks of O^T
  constexpr int kLoads = D / 32;     // 16-byte global loads per thread per tile (each of K, V)
  __shared__ FwdSmem<D> sm;

  const int nqt = (p.s + kBM - 1) / kBM;
  const int nbh = p.b * p.hq;
  const int bh = blockIdx.x % nbh;
  const int rank = (int)(blockIdx.x / nbh);
  const int qt = CAUSAL ? causal_tile(rank, nqt) : rank;
  const int hh_q = bh % p.hq;
  const int bb = bh / p.hq;
  const int g = hh_q / (p.hq / p.hkv);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int q0 = qt * kBM;
  const int qw = q0 + 32 * wv;           // first query of this wave
  const int qi = qw + col;               // this lane's query

  const bf16* qp = static_cast<const bf16*>(p.q) + bb * p.sq_b + hh_q * p.sq_h;
  const bf16* kp = static_cast<const bf16*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const bf16* vp = static_cast<const bf16*>(p.v) + bb * p.sv_b + g * p.sv_h;

  // Q^T B operand: lane (col, half) holds Q[qi][16c + 8*half .. +7]
  bf16x8 qreg[kDC];
#pragma unroll
  for (int c = 0; c < kDC; ++c) qreg[c] = bf16x8{};
  if (qi < p.s) {
#pragma unroll
    for (int c = 0; c < kDC; ++c)
      qreg[c] = *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.sq_s + 16 * c + 8 * half);
  }

  f32x16 oacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) oacc[db] = f32x16{};
  float m_use = -INFINITY;   // running max, log2-scaled units
  float l_run = 0.f;         // lane-partial row sum (this lane's keys)

  const int nkt_all = (p.s + kBN - 1) / kBN;
  const int nkt = CAUSAL ? min(nkt_all, (q0 + kBM + kBN - 1) / kBN) : nkt_all;

  // global -> register prefetch of one K/V tile: 16-byte chunk x = tid + 256*it
  uint4 kpre[kLoads], vpre[kLoads];
  auto prefetch = [&](int kt) {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int x = tid + kThreads * it;
      const int key = kt * kBN + x / (D / 8);
      const int c8 = x % (D / 8);
      kpre[it] = make_uint4(0, 0, 0, 0);
      vpre[it] = make_uint4(0, 0, 0, 0);
      if (key < p.s) {
        kpre[it] = *reinterpret_cast<const uint4*>(kp + (int64_t)key * p.sk_s + 8 * c8);
        vpre[it] = *reinterpret_cast<const uint4*>(vp + (int64_t)key * p.sv_s + 8 * c8);
      }
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int x = tid + kThreads * it;
      const int r = x / (D / 8), c8 = x % (D / 8);
      *reinterpret_cast<uint4*>(&sm.k[((r & ~31) | slot32(r & 31)) * kStride + 8 * c8]) = kpre[it];
      *reinterpret_cast<uint4*>(&sm.v[r * kStride + 8 * c8]) = vpre[it];
    }
  };

  const uint32_t hg = (uint32_t)(p.head_offset + hh_q);
  const uint32_t thr_hi = p.thresh << 16;
  const float c2 = p.scale_log2;
  // LDS element offsets that do not change across tiles
  const int krow = col * kStride + 8 * half;   // K tile rows are in slot order
  const int grp = lane >> 4, lg = lane & 15;
  const int vrow = (16 * (grp >> 1) + (lg >> 2)) * kStride + 16 * (grp & 1) + 4 * (lg & 3);

  prefetch(0);
  for (int kt = 0; kt < nkt; ++kt) {
    __syncthreads();
    stash();
    __syncthreads();
    if (kt + 1 < nkt) prefetch(kt + 1);
    const int key0 = kt * kBN;
    if (CAUSAL && key0 > qw + 31) continue;   // whole tile above this wave's diagonal

    // ---- S^T = K Q^T (raw scores) for two 32-key blocks
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < kDC; ++c) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[32 * kb * kStride + krow + 16 * c]);
        sacc[kb] = mfma32(a, qreg[c], sacc[kb]);
      }
    }

    // ---- mask, tile max (raw units; the scale is positive)
    const bool edge = (key0 + kBN > p.s) || (CAUSAL && key0 + kBN - 1 > qw);
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (edge) {
          const int key = key0 + 32 * kb + 16 * half + r;
          if (key >= p.s || (CAUSAL && key > qi)) sacc[kb][r] = -INFINITY;
        }
        mx = fmaxf(mx, sacc[kb][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave)) * c2;
    const bool grow = mx > m_use + kMaxSlack;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_use;
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);   // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db) oacc[db] *= alpha;
      m_use = m_new;
    }
    const float msub = (m_use == -INFINITY) ? 0.f : m_use;

    // ---- p = exp2(s * c - m); row-sum of the undropped values
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r], c2, -msub));
        sacc[kb][r] = e;
        lsum += e;
      }
    }
    l_run += lsum;

    // ---- dropout: zero the dropped probabilities (1/(1-p) applied in the epilogue)
    if (DROP) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int gh = 0; gh < 2; ++gh) {
          const uint32_t grp8 = (uint32_t)((key0 + 32 * kb + 16 * half + 8 * gh) >> 3);
          const Philox4 rnd = philox4x32_10(grp8, (uint32_t)qi, hg, (uint32_t)bb, p.k0, p.k1);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t w = rnd.w[e >> 1];
            const bool keep = (e & 1) ? (w >= thr_hi) : ((w & 0xFFFFu) >= p.thresh);
            sacc[kb][8 * gh + e] = keep ? sacc[kb][8 * gh + e] : 0.f;
          }
        }
      }
    }

    // ---- P^T as bf16 B operands: step c (16 keys) = block c/2, registers 8*(c%2) ..
    bf16x8 pop[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pop[c][e] = (bf16)sacc[c >> 1][8 * (c & 1) + e];
    }

    // ---- O^T += V^T P^T; V^T operand via LDS transpose reads:
    // lane group G = lane/16 covers d = 32db + 16*(G%2) + (0..15) and the keys
    // 32*kb + 16*(G/2) + 8*c' + (0..7) of step c = 2*kb + c'.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r0 = (32 * (c >> 1) + 8 * (c & 1)) * kStride + vrow;
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const s16x4 lo = lds_read_tr16(&sm.v[r0 + 32 * db]);
        const s16x4 hi = lds_read_tr16(&sm.v[r0 + 4 * kStride + 32 * db]);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = mfma32(a, pop[c], oacc[db]);
      }
    }
  }

  // ---- epilogue: O = O^T / l * 1/(1-p), LSE in natural log
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  if (qi < p.s) {
    const float inv = p.inv_keep / l_tot;
    bf16* op = static_cast<bf16*>(p.out) + bb * p.so_b + (int64_t)qi * p.so_s + hh_q * p.so_h;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 w;
        w.x = pack_bf16x2(oacc[db][4 * a + 0] * inv, oacc[db][4 * a + 1] * inv);
        w.y = pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * a + 4 * half) = w;
      }
    }
    if (half == 0) p.lse_out[((int64_t)bb * p.hq + hh_q) * p.s + qi] = (m_use + __log2f(l_tot)) * kLn2;
  }
}

template <int D>
hipError_t fwd_launch_d(const AttnParams& p, hipStream_t st) {
  const int nqt = (p.s + kBM - 1) / kBM;
  const dim3 grid((unsigned)(nqt * p.hq * p.b));
  const bool drop = p.thresh != 0;
  TraceScope ts("attn_fwd_bf16", st);
  if (p.causal) {
    if (drop) attn_fwd_bf16_kernel<D, true, true><<<grid, kThreads, 0, st>>>(p);
    else attn_fwd_bf16_kernel<D, true, false><<<grid, kThreads, 0, st>>>(p);
  } else {
    if (drop) attn_fwd_bf16_kernel<D, false, true><<<grid, kThreads, 0, st>>>(p);
    else attn_fwd_bf16_kernel<D, false, false><<<grid, kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

__global__ void attn_mask_kernel(AttnParams p, uint8_t* mask) {
  const int i = blockIdx.x, hh = blockIdx.y, bb = blockIdx.z;
  const uint32_t hg = (uint32_t)(p.head_offset + hh);
  uint8_t* row = mask + (((int64_t)bb * p.hq + hh) * p.s + i) * p.s;
  for (int g8 = threadIdx.x; 8 * g8 < p.s; g8 += blockDim.x) {
    const uint32_t bits = p.thresh ? attn_keep8(p.k0, p.k1, (uint32_t)bb, hg, (uint32_t)i, (uint32_t)g8, p.thresh) : 0xFFu;
    for (int e = 0; e < 8 && 8 * g8 + e < p.s; ++e) row[8 * g8 + e] = (bits >> e) & 1u;
  }
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnParams& p, hipStream_t st);

hipError_t launch_attn_fwd(const AttnParams& p, bool bf16_path, hipStream_t st) {
  if (p.s == 0 || p.b == 0) return hipSuccess;
  if (!bf16_path) return launch_attn_fwd_f32(p, st);
  switch (p.d) {
    case 32: return fwd_launch_d<32>(p, st);
    case 64: return fwd_launch_d<64>(p, st);
    case 96: return fwd_launch_d<96>(p, st);
    case 128: return fwd_launch_d<128>(p, st);
    case 160: return fwd_launch_d<160>(p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_mask(const AttnParams& p, uint8_t* mask, hipStream_t st) {
  if (p.s == 0 || p.b == 0) return hipSuccess;
  attn_mask_kernel<<<dim3(p.s, p.hq, p.b), 64, 0, st>>>(p, mask);
  return hipGetLastError();
}

}  // namespace srat
