// Attention-core backward with recomputation, bf16 in / fp32 accumulate, MFMA.
//
// Selective activation recomputation drops the attention core's activations
// (scores, softmax, dropout mask and output) after the forward and re-runs the
// core in the backward pass ("Reducing Activation Recomputation in Large
// Transformer Models", LIT-736 record, Key takeaways bullet 4).  Here the
// re-run is fused into the gradient kernels, tile by tile, so nothing of size
// s x s is ever written:
//
//   S  = Q K^T * scale,  P = exp(S - LSE)          (recomputed)
//   M  = Philox keep mask                           (regenerated, bit-exact)
//   dV = (P*M)^T dO / (1-p)
//   dP = dO V^T * M / (1-p),  dS = P * (dP - D),  D = rowsum(dO * O)
//   dQ = dS K * scale,        dK = dS^T Q * scale
//
// Kernels on one stream, no atomics (results are deterministic):
//   dq  : one workgroup per 128 queries, the forward's shape (at d = 128 two
//         groups of 4 waves over the same queries, alternating key tiles,
//         as the forward at that head dim).  Its prologue
//         forms D = rowsum(dO * O) for its queries (stored for dkdv); then it
//         loops over 64-key tiles, recomputes S^T and dP^T, forms dS^T in
//         registers and accumulates dQ^T += K^T dS^T (K^T through LDS
//         transpose reads).  Re-doing QK^T and dO V^T here costs MFMA work
//         (not counted in the algorithmic FLOPs) but removes every atomic
//         from the backward.
//   dkdv: one workgroup per (128-key block, q-head, batch) (at d = 128, 160 with
//         the chain below split between producer and consumer waves, see
//         attn_bwd_dkdv_pc_kernel).  Waves split the
//         block's keys into four 32-key groups (and, for head dims <= 64, each
//         64-query tile into two 32-query halves, one wave per pair).  A wave
//         computes S^T = K Q^T and dP^T = V dO^T with its K, V rows as
//         register-resident MFMA A operands, rows permuted so that one lane
//         holds one query and 16 consecutive keys: the softmax recompute, the
//         mask (one Philox call per 8 keys) and dS are lane-local.  P*M and
//         dS go through a wave-private LDS tile and come back transposed
//         (ds_read_b64_tr_b16) as the A operands of dV += (P*M)^T dO and
//         dK += dS^T Q.  Under a causal mask the blocks with the lowest keys
//         (the most queries) are launched first; where two workgroups share
//         a CU, the grid's second half runs in the mirrored order so that
//         each pair carries about the same work.
//   sums (one launch after dK/dV, where needed): grouped-query attention or
//         split key blocks: dK, dV = sums, in a fixed order, of the fp32
//         partials of the q-heads that share a kv-head and of the two halves
//         of a split block; split query tiles: dQ = the sum of the two
//         halves' fp32 partials.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "philox.hpp"

namespace srat {
namespace {

constexpr int kBNk = 128;      // keys per dkdv workgroup

__device__ __forceinline__ int perm32(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
// Inverse of perm32: the MFMA slot of key k of a 32-key block (LDS K / V
// tiles of the dq kernel are stored in slot order).
__device__ __forceinline__ int slot32(int k) { return 8 * ((k >> 2) & 3) + 4 * (k >> 4) + (k & 3); }

// ds_read_b64_tr_b16 pair -> 32x32x16 MFMA operand "lane (i = l%32, h = l/32)
// holds column c_base + i, rows r_base + 8h .. +7" of a row-major tile; this is
// the per-lane part of the element offset (lane group G = l/16 covers columns
// c_base + 16*(G%2) .. and rows r_base + 8*(G/2) ..).
__device__ __forceinline__ int tr_off32(int stride, int lane) {
  const int grp = lane >> 4, lg = lane & 15;
  return (8 * (grp >> 1) + (lg >> 2)) * stride + 16 * (grp & 1) + 4 * (lg & 3);
}
__device__ __forceinline__ bf16x8 tr_pair(const bf16* p, int stride) {
  const s16x4 lo = lds_read_tr16(p);
  const s16x4 hi = lds_read_tr16(p + 4 * stride);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The keep decision of element r (0..15) of a lane from its two Philox calls
// (keys 8*g8 .. 8*g8+15 of one query).
__device__ __forceinline__ bool keep16(const Philox4 (&rnd)[2], int r, uint32_t thr, uint32_t thr_hi) {
  const uint32_t w = rnd[r >> 3].w[(r & 7) >> 1];
  return (r & 1) ? (w >= thr_hi) : ((w & 0xFFFFu) >= thr);
}

// ============================================================== dK, dV
// Wave-private P*M and dS tiles: 32 queries x 32 keys, row-major with a row
// stride of 20 dwords.  A lane writes the 16 keys of its query as two
// 16-byte pieces; at this stride the 8 rows a 16-byte write serves per cycle
// land on distinct banks (measured on gfx950: 32 cycles per wave instruction,
// against 64 at a stride of 8 or 24 dwords), and the transpose reads stay
// fast.
constexpr int kWaveRow = 40;              // 32 keys + 8 pad (20 dwords per row)
constexpr int kWaveTile = 32 * kWaveRow;

// Configuration by head dim:
//   d <= 64 : two query halves (8 waves, 2 per SIMD), K and V rows in registers;
//   d == 96 : one query half (4 waves), V rows read from LDS so that a wave
//             fits 256 registers and two workgroups share a CU;
//   d >= 128: one query half, one workgroup per CU (accumulators in AGPRs);
//   d == 192: V rows again through LDS, so that K, the dK/dV accumulators and
//             the tile's values fit the 512 registers of a wave;
//   d == 256: two workgroups per key block, each accumulating and storing
//             half of dK's and dV's columns (both recompute S and dP over
//             the whole head dim): the accumulators of all 256 columns alone
//             would take half of a wave's registers.
template <int D> struct DkdvCfg {
  static constexpr int kQH = D <= 64 ? 2 : 1;
  static constexpr bool kVLds = D == 96 || D == 192;
  static constexpr int kBlocksPerCU = D == 96 ? 2 : 1;
  static constexpr int kDParts = D >= 256 ? 2 : 1;
};

template <int D, int QH>
struct alignas(16) DkdvSmem {
  static constexpr int kS = TileStride<D>::kValue;   // Q / dO tile row stride (bf16)
  static constexpr int kVS = RowStride<D>::kValue;   // V block row stride (row reads only)
  static constexpr int kRows = 32 * QH;              // queries per tile
  static constexpr int kVRows = DkdvCfg<D>::kVLds ? 128 : 1;
  union {
    struct {
      bf16 q[2][kRows * kS];                           // two buffers: tile t read, t+1 written
      bf16 dout[2][kRows * kS];
      bf16 pm[4 * QH][kWaveTile];
      bf16 ds[4 * QH][kWaveTile];
      bf16 v[kVRows * kVS];                            // the block's V rows, slot order
    } t;
    float comb[4][QH == 2 ? 64 * (D / 32) * 16 : 1];   // q-half combine of one accumulator
  };
};

template <bool B>
using bool_c = std::integral_constant<bool, B>;

// configurations whose backward grids may be split (one workgroup per CU:
// d >= 128; causal); elsewhere the split code compiles away
template <int D, bool CAUSAL>
constexpr bool kSplitBwd = CAUSAL && D >= 128;

// VARLEN: per-element valid lengths (padded batch); compiled separately so
// that the plain kernels keep their code.
template <int D, bool CAUSAL, bool DROP, bool PART, bool VARLEN>
__global__ __launch_bounds__(256 * DkdvCfg<D>::kQH, DkdvCfg<D>::kBlocksPerCU) void attn_bwd_dkdv_kernel(AttnParams p) {
  constexpr int QH = DkdvCfg<D>::kQH;
  constexpr bool kVLds = DkdvCfg<D>::kVLds;
  using SM = DkdvSmem<D, QH>;
  constexpr int kS = SM::kS, kRows = SM::kRows;
  constexpr int kThreads = 256 * QH;
  constexpr int kDC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kDParts = DkdvCfg<D>::kDParts;
  constexpr int kDBA = kDB / kDParts;   // 32-column blocks of dK / dV this workgroup accumulates
  constexpr int kTileChunks = kRows * D / 8;
  constexpr int kTileLoads = (kTileChunks + kThreads - 1) / kThreads;
  __shared__ SM sm;

  const int nbh = p.b * p.hq;
  // Key-block order.  Causal, one workgroup per CU: ascending, the blocks
  // with the most queries (lowest keys) first, the dispatcher fills in the
  // rest.  Two per CU: the first half of the grid ascending, the second half
  // descending, so the workgroups that share a CU (block i and i + grid/2)
  // together carry the same number of query tiles.
  const int nkb = (p.s + kBNk - 1) / kBNk;
  const int dpart = (int)(blockIdx.x % kDParts);        // which columns of dK / dV
  const int wg = (int)(blockIdx.x / kDParts);
  const int d0 = dpart * kDBA;                           // first 32-column block of them
  const int rank = wg / nbh;
  const int hkb = (nkb + 1) / 2;
  // Split grids (p.split_kb > 0, causal only): the split_kb blocks with the
  // most queries (the lowest keys) run as two workgroups each (part 0: the
  // first half of the block's query tiles, part 1: the rest), launched in
  // decreasing order of work.
  const int nsk = kSplitBwd<D, CAUSAL> ? p.split_kb : 0;
  int kblk, part = -1;
  if (nsk > 0) {
    int t;
    split_order(rank, nkb, nsk, t, part);
    kblk = nkb - 1 - t;
  } else {
    const bool mirror = CAUSAL && DkdvCfg<D>::kBlocksPerCU == 2 && rank >= hkb;
    kblk = mirror ? nkb - 1 - (rank - hkb) : rank;
  }
  const int bh = wg % nbh;
  const int hh_q = bh % p.hq, bb = bh / p.hq;
  const int g = hh_q / (p.hq / p.hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps tile bounds scalar
  const int kg = wv & 3, qh = wv >> 2;                // key group, query half
  const int half = lane >> 5, col = lane & 31;
  const int k0 = kblk * kBNk;
  const int kw0 = k0 + 32 * kg;                       // first key of this wave
  const int sl = VARLEN ? attn_len(p, bb) : p.s;      // valid length of this batch element

  const bf16* qp = static_cast<const bf16*>(p.q) + bb * p.sq_b + hh_q * p.sq_h;
  const bf16* dop = static_cast<const bf16*>(p.dout) + bb * p.so_b + hh_q * p.so_h;
  const bf16* kp = static_cast<const bf16*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const bf16* vp = static_cast<const bf16*>(p.v) + bb * p.sv_b + g * p.sv_h;
  const int64_t row0 = ((int64_t)bb * p.hq + hh_q) * p.s;

  // K (and, unless V goes through LDS, V) rows of this wave as MFMA A
  // operands (rows permuted)
  bf16x8 kreg[kDC], vreg[kVLds ? 1 : kDC];
  {
    const int key = kw0 + perm32(col);
    const bool ok = key < sl;
    const int64_t ko = (int64_t)(ok ? key : 0) * p.sk_s + 8 * half;
    const int64_t vo = (int64_t)(ok ? key : 0) * p.sv_s + 8 * half;
#pragma unroll
    for (int c = 0; c < kDC; ++c) {
      const uint4 a = *reinterpret_cast<const uint4*>(kp + ko + 16 * c);
      kreg[c] = __builtin_bit_cast(bf16x8, ok ? a : make_uint4(0, 0, 0, 0));
      if (!kVLds) {
        const uint4 b = *reinterpret_cast<const uint4*>(vp + vo + 16 * c);
        vreg[c] = __builtin_bit_cast(bf16x8, ok ? b : make_uint4(0, 0, 0, 0));
      }
    }
  }
  if (kVLds) {
    // the block's 128 V rows -> LDS in slot order (rows past s read as zero);
    // made visible by the first tile's barrier
    constexpr int kVS = SM::kVS;
    const int rows = max(0, min(kBNk, sl - k0));
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vp + (int64_t)k0 * p.sv_s, (uint32_t)((int64_t)rows * p.sv_s * 2));
#pragma unroll
    for (int it = 0; it < kBNk * D / 8 / kThreads; ++it) {
      const int x = tid + kThreads * it;
      const int r = x / (D / 8), c8 = x % (D / 8);
      const uint4 v4 = buffer_load16(rv, (uint32_t)(((int64_t)r * p.sv_s + 8 * c8) * 2));
      *reinterpret_cast<uint4*>(&sm.t.v[((r & ~31) | slot32(r & 31)) * kVS + 8 * c8]) = v4;
    }
  }
  const int v_row = (32 * kg + col) * SM::kVS + 8 * half;   // this lane's V row in LDS
  f32x16 dv_acc[kDBA], dk_acc[kDBA];
#pragma unroll
  for (int db = 0; db < kDBA; ++db) dv_acc[db] = dk_acc[db] = f32x16{};

  const int nqt_all = (sl + kRows - 1) / kRows;
  const int qt_first = CAUSAL ? k0 / kRows : 0;
  // query tiles [qt0, nqt) of this workgroup
  const int qt_mid = qt_first + (nqt_all - qt_first + 1) / 2;
  const int qt0 = part == 1 ? qt_mid : qt_first;
  const int nqt = part == 0 ? qt_mid : nqt_all;

  // ---- Q / dO staging through buffer loads (rows past s read as zero);
  // chunks beyond the tile get an offset past any range
  uint4 qpre[kTileLoads], dpre[kTileLoads];
  uint32_t qoff[kTileLoads], ooff[kTileLoads];
#pragma unroll
  for (int it = 0; it < kTileLoads; ++it) {
    const int x = tid + kThreads * it;
    const bool in = x < kTileChunks;
    qoff[it] = in ? (uint32_t)(((int64_t)(x / (D / 8)) * p.sq_s + 8 * (x % (D / 8))) * 2) : 0xFFFFFFF0u;
    ooff[it] = in ? (uint32_t)(((int64_t)(x / (D / 8)) * p.so_s + 8 * (x % (D / 8))) * 2) : 0xFFFFFFF0u;
  }
  auto tile_bytes = [&](int qt, int64_t stride) -> uint32_t {
    const int rows = min(kRows, max(0, sl - qt * kRows));
    return (uint32_t)((int64_t)rows * stride * 2);
  };
  // per-row LSE / D of the lane's query (zero past s), fetched one tile ahead
  const __amdgpu_buffer_rsrc_t rlse = buffer_rsrc(p.lse + row0, (uint32_t)sl * 4u);
  const __amdgpu_buffer_rsrc_t rdel = buffer_rsrc(p.delta + row0, (uint32_t)sl * 4u);
  float lse_n = 0.f, dlt_n = 0.f;
  auto load_rowstats = [&](int qt) {
    const int qo = (qt * kRows + 32 * qh + col) * 4;
    lse_n = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rlse, qo, 0, 0));
    dlt_n = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rdel, qo, 0, 0));
  };
  auto load_tile = [&](int qt) {
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(qp + (int64_t)qt * kRows * p.sq_s, tile_bytes(qt, p.sq_s));
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(dop + (int64_t)qt * kRows * p.so_s, tile_bytes(qt, p.so_s));
#pragma unroll
    for (int it = 0; it < kTileLoads; ++it) {
      qpre[it] = buffer_load16(rq, qoff[it]);
      dpre[it] = buffer_load16(ro, ooff[it]);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int it = 0; it < kTileLoads; ++it) {
      const int x = tid + kThreads * it;
      if (x < kTileChunks) {
        const int r = x / (D / 8), c8 = x % (D / 8);
        *reinterpret_cast<uint4*>(&sm.t.q[buf][r * kS + 8 * c8]) = qpre[it];
        *reinterpret_cast<uint4*>(&sm.t.dout[buf][r * kS + 8 * c8]) = dpre[it];
      }
    }
  };

  const uint32_t hg = (uint32_t)(p.head_offset + hh_q);
  const uint32_t thr_hi = p.thresh << 16;
  const float c2 = p.scale_log2;
  // the lane's two Philox calls cover keys kw0 + 16half + 8gh .. +7 of its
  // query: fixed key group, the query varies by tile
  // (hoisted state costs 18 registers: only where the waves have room)
  constexpr bool kHoist = QH == 1 && D < 192;   // (at d >= 192 its registers are worth more)
  PhiloxCol pcol[2];
  if (DROP && kHoist) {
#pragma unroll
    for (int gh = 0; gh < 2; ++gh)
      pcol[gh] = philox_col((uint32_t)((kw0 + 16 * half + 8 * gh) >> 3), hg, (uint32_t)bb, p.k0, p.k1);
  }
  const int q_row = (32 * qh + col) * kS + 8 * half;   // this lane's Q / dO row (B operands)
  const int w_row = col * kWaveRow + 16 * half;        // this lane's 16 keys in the wave tiles
  // (P*M)^T, dS^T A operands: lane group G reads keys 16*(G%2) + 4*(lg%4) ..
  // +3, query rows 8*(G/2) + (lg/4) (+4)
  const int tr_w = 16 * ((lane >> 4) & 1) + (8 * (lane >> 5) + ((lane & 15) >> 2)) * kWaveRow + 4 * (lane & 3);
  const int tr_s = tr_off32(kS, lane) + 32 * qh * kS;  // dO, Q rows of this query half (B operands)
  bf16* pmt = sm.t.pm[wv];
  bf16* dst = sm.t.ds[wv];
  const int key_l = kw0 + 16 * half;                   // the lane's first key

  auto tile = [&](int qt, auto mask_c, auto next_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    const int buf = (qt - qt0) & 1;
    const int qi = qt * kRows + 32 * qh + col;
    const float lse2 = lse_n * kLog2e;
    const float dlt = dlt_n;
    __syncthreads();
    if (NEXT) {
      stash(buf ^ 1);             // Q/dO[qt+1] over Q/dO[qt-1]
      load_rowstats(qt + 1);      // before the tile loads: waiting for it later
      load_tile(qt + 2);          // does not wait for them
    }
    // S^T = K Q^T and dP^T = V dO^T (raw, 32 keys x 32 queries); the tile's
    // Philox draws are independent and overlap the MFMAs
    f32x16 sacc = f32x16{}, pacc = f32x16{};
    const bf16* qb_ = sm.t.q[buf];
    const bf16* ob_ = sm.t.dout[buf];
#pragma unroll
    for (int c = 0; c < kDC; ++c) {
      sacc = mfma32(kreg[c], *reinterpret_cast<const bf16x8*>(&qb_[q_row + 16 * c]), sacc);
      const bf16x8 va = kVLds ? *reinterpret_cast<const bf16x8*>(&sm.t.v[v_row + 16 * c]) : vreg[kVLds ? 0 : c];
      pacc = mfma32(va, *reinterpret_cast<const bf16x8*>(&ob_[q_row + 16 * c]), pacc);
    }
    Philox4 rnd[2];
    if (DROP && kHoist) {
      rnd[0] = philox4x32_10_col((uint32_t)qi, pcol[0]);
      rnd[1] = philox4x32_10_col((uint32_t)qi, pcol[1]);
    } else if (DROP) {
      const uint32_t g8 = (uint32_t)(key_l >> 3);
      rnd[0] = philox4x32_10(g8, (uint32_t)qi, hg, (uint32_t)bb, p.k0, p.k1);
      rnd[1] = philox4x32_10(g8 + 1, (uint32_t)qi, hg, (uint32_t)bb, p.k0, p.k1);
    }
    // keys at or past kl are masked for this lane's query (all of them for a
    // query past s)
    const int kl = qi < sl ? (CAUSAL ? min(sl, qi + 1) : sl) : 0;

    // recompute P, regenerate the mask, P*M and dS packed to bf16 pairs
    uint32_t pmw[8], dsw[8];
#pragma unroll
    for (int r2 = 0; r2 < 8; ++r2) {
      float pv[2], dp[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * r2 + e;
        pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[r], c2, -lse2));
        if (MASK) pv[e] = key_l + r >= kl ? 0.f : pv[e];
        dp[e] = pacc[r];
      }
      uint32_t pk = pack_bf16x2(pv[0], pv[1]);
      if (DROP) {
        const uint32_t w = rnd[r2 >> 2].w[r2 & 3];
        const bool keep0 = (w & 0xFFFFu) >= p.thresh, keep1 = w >= thr_hi;
        pk = and_or(pk, keep0 ? 0xFFFFu : 0u, keep1 ? 0xFFFF0000u : 0u);
        dp[0] = keep0 ? dp[0] : 0.f;
        dp[1] = keep1 ? dp[1] : 0.f;
      }
      pmw[r2] = pk;
      dsw[r2] = pack_bf16x2(pv[0] * fmaf(dp[0], p.inv_keep, -dlt), pv[1] * fmaf(dp[1], p.inv_keep, -dlt));
    }
    *reinterpret_cast<uint4*>(&pmt[w_row]) = make_uint4(pmw[0], pmw[1], pmw[2], pmw[3]);
    *reinterpret_cast<uint4*>(&pmt[w_row + 8]) = make_uint4(pmw[4], pmw[5], pmw[6], pmw[7]);
    *reinterpret_cast<uint4*>(&dst[w_row]) = make_uint4(dsw[0], dsw[1], dsw[2], dsw[3]);
    *reinterpret_cast<uint4*>(&dst[w_row + 8]) = make_uint4(dsw[4], dsw[5], dsw[6], dsw[7]);
    lds_fence();   // the wave reads its own tiles back transposed

    // dV += (P*M)^T dO ;  dK += dS^T Q   (contraction over the wave's 32 queries)
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bf16x8 apm = tr_pair(&pmt[16 * st * kWaveRow + tr_w], kWaveRow);
      const bf16x8 ads = tr_pair(&dst[16 * st * kWaveRow + tr_w], kWaveRow);
#pragma unroll
      for (int db = 0; db < kDBA; ++db) {
        dv_acc[db] = mfma32(apm, tr_pair(&ob_[16 * st * kS + tr_s + 32 * (d0 + db)], kS), dv_acc[db]);
        dk_acc[db] = mfma32(ads, tr_pair(&qb_[16 * st * kS + tr_s + 32 * (d0 + db)], kS), dk_acc[db]);
      }
    }
  };

  // a key block past the valid length (padded batch) keeps dK = dV = 0
  if (!VARLEN || k0 < sl) {
    // prologue: Q/dO[qt0] resident, Q/dO[qt0+1] and the row stats of qt0 in flight
    load_tile(qt0);
    stash(0);
    load_rowstats(qt0);
    load_tile(qt0 + 1);
    // Tiles this wave computes without masking: every query of the tile at or
    // past every key of the wave (causal) and everything inside sl.
    const int last = nqt - 1;
    int qa = qt0, qb = qt0;
    if (kw0 + 32 <= sl) {
      qa = CAUSAL ? max(qt0, (kw0 + 31 - 32 * qh + kRows - 1) / kRows) : qt0;   // first q0 >= kw0 + 31
      qb = max(qa, (sl - 32 * qh - 32) / kRows + 1);                             // last q0 + 31 < sl
      qb = min(qb, nqt);
      if ((sl - 32 * qh - 32) < 0) qb = qa;
    }
    // separate straight-line loops (see the forward kernel)
    int qt = qt0;
    for (; qt < min(qa, last); ++qt) tile(qt, bool_c<true>{}, bool_c<true>{});
    for (; qt < min(qb, last); ++qt) tile(qt, bool_c<false>{}, bool_c<true>{});
    for (; qt < last; ++qt) tile(qt, bool_c<true>{}, bool_c<true>{});
    if (qt >= qa && qt < qb) tile(qt, bool_c<false>{}, bool_c<false>{});
    else tile(qt, bool_c<true>{}, bool_c<false>{});
  }

  // two query halves: the second adds its share into the first through LDS
  if (QH == 2) {
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      __syncthreads();
      if (qh == 1) {
#pragma unroll
        for (int db = 0; db < kDBA; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) sm.comb[kg][(db * 16 + r) * 64 + lane] = which ? dk_acc[db][r] : dv_acc[db][r];
      }
      __syncthreads();
      if (qh == 0) {
#pragma unroll
        for (int db = 0; db < kDBA; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = sm.comb[kg][(db * 16 + r) * 64 + lane];
            if (which) dk_acc[db][r] += x;
            else dv_acc[db][r] += x;
          }
      }
    }
    if (qh == 1) return;
  }

  // store: lane holds d = 32(d0 + db) + col, keys kw0 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int db = 0; db < kDBA; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key >= p.s) continue;
      const float dvv = dv_acc[db][r] * p.inv_keep;
      const float dkv = dk_acc[db][r] * p.scale;
      const int dcol = 32 * (d0 + db) + col;
      if (PART || part >= 0) {   // slot 1 holds the second parts of split blocks
        const int64_t o = ((int64_t)max(part, 0) * p.b * p.s * p.hq + ((int64_t)bb * p.s + key) * p.hq + hh_q) * D + dcol;
        p.dv_acc[o] = dvv;
        p.dk_acc[o] = dkv;
      } else {
        static_cast<bf16*>(p.dv)[bb * p.sv_b + (int64_t)key * p.sv_s + g * p.sv_h + dcol] = (bf16)dvv;
        static_cast<bf16*>(p.dk)[bb * p.sk_b + (int64_t)key * p.sk_s + g * p.sk_h + dcol] = (bf16)dkv;
      }
    }
  }
}

// ============================================================== dK, dV: producer and consumer waves (d = 128, 160)
// At d = 128 one wave of the kernel above holds K and V rows (64 registers),
// both accumulators (128) and a tile's scores, so it runs alone on its SIMD
// and each 32-query tile is a serial chain: S^T, dP^T MFMAs -> softmax
// recompute and dS on the VALU -> LDS round trip -> dV, dK MFMAs.  Here the
// two halves of that chain run in different waves.  Waves 0-3 (producers)
// hold the K and V rows of their 32 keys, compute S^T and dP^T, and write
// P*M and dS to LDS; waves 4-7 (consumers, one per SIMD beside a producer)
// hold the dK and dV accumulators of the same keys and, one tile behind,
// read P*M and dS back transposed for dV += (P*M)^T dO and dK += dS^T Q.
// The roles run separate loops with one barrier per step, so each fits 256
// registers and a producer's VALU work overlaps its SIMD neighbour's MFMAs.
// Q, dO and the tile's LSE and D reach LDS through buffer -> LDS loads in a
// four-slot ring, two tiles ahead of the producers.  The producers issue all
// of them, behind their MFMAs: the issue of 24 KB of loads per step stalls
// the issuing waves for hundreds of cycles (address processing), which right
// after the barrier delayed the consumers (the critical path) and the
// producers' MFMAs.
template <int D>
struct alignas(16) DkdvPCSmem {
  static constexpr int kS = TileStride<D>::kValue;            // Q / dO row stride (bf16)
  static constexpr int kQBlocks = (32 * kS * 2 + 1023) / 1024;  // 1 KB blocks of a Q (dO) tile
  static constexpr int kBlocks = (2 * kQBlocks + 2 + 7) / 8 * 8;   // per slot: Q, dO, LSE, D, slack
  unsigned char ring[4][kBlocks * 1024];
  bf16 pm[2][4][kWaveTile];   // [step parity][key group]
  bf16 ds[2][4][kWaveTile];
};

// (at d = 96 the kernel above already runs two workgroups per CU, and the
// split measured slower there: gpt22b-t8 shape 92 -> 98 us)
template <int D>
constexpr bool kDkdvPC = D == 128 || D == 160;

// One 128-key block (kblk; part 0 / 1: one half of its query range, -1: all).
template <int D, bool CAUSAL, bool DROP, bool PART, bool VARLEN>
__device__ __forceinline__ void dkdv_pc_tile(const AttnParams& p, DkdvPCSmem<D>& sm, int bh, int kblk, int part) {
  using SM = DkdvPCSmem<D>;
  constexpr int kS = SM::kS;
  constexpr int kQBlocks = SM::kQBlocks, kBlocks = SM::kBlocks;
  constexpr int kPer = kBlocks / 4;   // ring blocks each producer wave loads per tile
  constexpr int kDC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kRows = 32;

  const int hh_q = bh % p.hq, bb = bh / p.hq;
  const int g = hh_q / (p.hq / p.hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps tile bounds scalar
  const int role = wv >> 2, kg = wv & 3;                      // producer / consumer, key group
  const int half = lane >> 5, col = lane & 31;
  const int k0 = kblk * kBNk;
  const int kw0 = k0 + 32 * kg;
  const int sl = VARLEN ? attn_len(p, bb) : p.s;

  const bf16* qp = static_cast<const bf16*>(p.q) + bb * p.sq_b + hh_q * p.sq_h;
  const bf16* dop = static_cast<const bf16*>(p.dout) + bb * p.so_b + hh_q * p.so_h;
  const bf16* kp = static_cast<const bf16*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const bf16* vp = static_cast<const bf16*>(p.v) + bb * p.sv_b + g * p.sv_h;
  const int64_t row0 = ((int64_t)bb * p.hq + hh_q) * p.s;

  const int nqt_all = (sl + kRows - 1) / kRows;
  const int qt_first = CAUSAL ? k0 / kRows : 0;
  const int qt_mid = qt_first + (nqt_all - qt_first + 1) / 2;
  const int qt0 = part == 1 ? qt_mid : qt_first;
  const int nqt = part == 0 ? qt_mid : nqt_all;
  // tiles of this workgroup (none for a key block past the valid length)
  const int n = (VARLEN && k0 >= sl) ? 0 : nqt - qt0;

  // ---- ring staging: slot = [Q tile | dO tile | LSE of its 32 queries |
  // D of them | slack], 1 KB per load instruction (lane l: bytes 16l ..),
  // producer wave kg loading blocks kg, kg + 4, ...; Q and dO rows land in
  // the padded row layout, padding and everything past the tile read as zero
  uint32_t doff[kPer];
  int dsel[kPer];   // 0 Q, 1 dO, 2 LSE, 3 D, 4 slack
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int blk = kg + 4 * i;
    uint32_t off = 0xFFFFFFF0u;
    int sel = 4;
    if (blk < 2 * kQBlocks) {
      sel = blk < kQBlocks ? 0 : 1;
      const int pos = 1024 * (blk - sel * kQBlocks) + 16 * lane;
      const int row = pos / (2 * kS), cb = pos % (2 * kS);
      const int64_t rs = sel == 0 ? p.sq_s : p.so_s;
      if (row < kRows && cb < 2 * D) off = (uint32_t)((int64_t)row * rs * 2 + cb);
    } else if (blk < 2 * kQBlocks + 2) {
      sel = 2 + (blk - 2 * kQBlocks);
      if (lane < kRows / 4) off = 16u * lane;
    }
    doff[i] = off;
    dsel[i] = sel;
  }
  auto dma = [&](int qt, int slot) {
    if (role != 0) return;   // the producers load the ring; the consumers are the critical path
    const int rows = qt < nqt ? min(kRows, max(0, sl - qt * kRows)) : 0;
    const sgpr4 rq = buffer_rsrc_sgpr(qp + (int64_t)qt * kRows * p.sq_s, (uint32_t)((int64_t)rows * p.sq_s * 2));
    const sgpr4 ro = buffer_rsrc_sgpr(dop + (int64_t)qt * kRows * p.so_s, (uint32_t)((int64_t)rows * p.so_s * 2));
    const sgpr4 rl = buffer_rsrc_sgpr(p.lse + row0 + (int64_t)qt * kRows, (uint32_t)rows * 4u);
    const sgpr4 rd = buffer_rsrc_sgpr(p.delta + row0 + (int64_t)qt * kRows, (uint32_t)rows * 4u);
    const uintptr_t base = (uintptr_t)&sm.ring[slot][0];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int sel = dsel[i];
      const sgpr4 r = sel == 0 ? rq : sel == 1 ? ro : sel == 2 ? rl : rd;
      buffer_load16_lds(r, base + 1024 * (kg + 4 * i), doff[i]);
    }
  };
  auto q_of = [&](int slot) { return reinterpret_cast<const bf16*>(&sm.ring[slot][0]); };
  auto do_of = [&](int slot) { return reinterpret_cast<const bf16*>(&sm.ring[slot][kQBlocks * 1024]); };
  auto stat_of = [&](int slot, int which) {
    return reinterpret_cast<const float*>(&sm.ring[slot][(2 * kQBlocks + which) * 1024]);
  };
  const int w_row = col * kWaveRow + 16 * half;   // this lane's 16 keys in the wave tiles

  if (role == 0) {
    // ================= producer: S^T, dP^T, P*M and dS of each tile
    bf16x8 kreg[kDC], vreg[kDC];
    {
      const int key = kw0 + perm32(col);
      const bool ok = key < sl;
      const int64_t ko = (int64_t)(ok ? key : 0) * p.sk_s + 8 * half;
      const int64_t vo = (int64_t)(ok ? key : 0) * p.sv_s + 8 * half;
#pragma unroll
      for (int c = 0; c < kDC; ++c) {
        const uint4 a = *reinterpret_cast<const uint4*>(kp + ko + 16 * c);
        const uint4 b = *reinterpret_cast<const uint4*>(vp + vo + 16 * c);
        kreg[c] = __builtin_bit_cast(bf16x8, ok ? a : make_uint4(0, 0, 0, 0));
        vreg[c] = __builtin_bit_cast(bf16x8, ok ? b : make_uint4(0, 0, 0, 0));
      }
    }
    // consumed here, so the compiler waits for these loads now and does not
    // guard their later uses with waits that would also drain the ring loads
#pragma unroll
    for (int c = 0; c < kDC; ++c) asm volatile("" ::"v"(kreg[c]), "v"(vreg[c]));
    wait_vmcnt<0>();

    const uint32_t hg = (uint32_t)(p.head_offset + hh_q);
    const uint32_t thr_hi = p.thresh << 16;
    const float c2 = p.scale_log2;
    PhiloxCol pcol[2];
    if (DROP) {
#pragma unroll
      for (int gh = 0; gh < 2; ++gh)
        pcol[gh] = philox_col((uint32_t)((kw0 + 16 * half + 8 * gh) >> 3), hg, (uint32_t)bb, p.k0, p.k1);
    }
    const int q_row = col * kS + 8 * half;   // this lane's Q / dO row (B operands)
    const int key_l = kw0 + 16 * half;
    // tiles this wave computes without masking: [qa, qb)
    int qa = qt0, qb = qt0;
    if (kw0 + 32 <= sl) {
      qa = CAUSAL ? max(qt0, (kw0 + 31 + kRows - 1) / kRows) : qt0;
      qb = (sl - 32) < 0 ? qa : min(nqt, max(qa, (sl - 32) / kRows + 1));
    }

    auto produce = [&](int qt, int slot, int pbuf, int ld_qt, int ld_slot, auto mask_c) {
      constexpr bool MASK = decltype(mask_c)::value;
      const int qi = qt * kRows + col;
      const bf16* qb_ = q_of(slot);
      const bf16* ob_ = do_of(slot);
      const float lse2 = stat_of(slot, 0)[col] * kLog2e;
      const float dlt = stat_of(slot, 1)[col];
      f32x16 sacc = f32x16{}, pacc = f32x16{};
#pragma unroll
      for (int c = 0; c < kDC; ++c) {
        sacc = mfma32(kreg[c], *reinterpret_cast<const bf16x8*>(&qb_[q_row + 16 * c]), sacc);
        pacc = mfma32(vreg[c], *reinterpret_cast<const bf16x8*>(&ob_[q_row + 16 * c]), pacc);
      }
      dma(ld_qt, ld_slot);   // issued behind the MFMAs
      Philox4 rnd[2];
      if (DROP) {
        rnd[0] = philox4x32_10_col((uint32_t)qi, pcol[0]);
        rnd[1] = philox4x32_10_col((uint32_t)qi, pcol[1]);
      }
      const int kl = qi < sl ? (CAUSAL ? min(sl, qi + 1) : sl) : 0;
      uint32_t pmw[8], dsw[8];
#pragma unroll
      for (int r2 = 0; r2 < 8; ++r2) {
        float pv[2], dp[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * r2 + e;
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[r], c2, -lse2));
          if (MASK) pv[e] = key_l + r >= kl ? 0.f : pv[e];
          dp[e] = pacc[r];
        }
        uint32_t pk = pack_bf16x2(pv[0], pv[1]);
        if (DROP) {
          const uint32_t w = rnd[r2 >> 2].w[r2 & 3];
          const bool keep0 = (w & 0xFFFFu) >= p.thresh, keep1 = w >= thr_hi;
          pk = and_or(pk, keep0 ? 0xFFFFu : 0u, keep1 ? 0xFFFF0000u : 0u);
          dp[0] = keep0 ? dp[0] : 0.f;
          dp[1] = keep1 ? dp[1] : 0.f;
        }
        pmw[r2] = pk;
        dsw[r2] = pack_bf16x2(pv[0] * fmaf(dp[0], p.inv_keep, -dlt), pv[1] * fmaf(dp[1], p.inv_keep, -dlt));
      }
      bf16* pmt = sm.pm[pbuf][kg];
      bf16* dst = sm.ds[pbuf][kg];
      *reinterpret_cast<uint4*>(&pmt[w_row]) = make_uint4(pmw[0], pmw[1], pmw[2], pmw[3]);
      *reinterpret_cast<uint4*>(&pmt[w_row + 8]) = make_uint4(pmw[4], pmw[5], pmw[6], pmw[7]);
      *reinterpret_cast<uint4*>(&dst[w_row]) = make_uint4(dsw[0], dsw[1], dsw[2], dsw[3]);
      *reinterpret_cast<uint4*>(&dst[w_row + 8]) = make_uint4(dsw[4], dsw[5], dsw[6], dsw[7]);
    };

    dma(qt0, 0);
    dma(qt0 + 1, 1);
    // step k: tile k of the producers (the consumers take tile k - 1); the
    // barrier bare (see lds_barrier): each wave has completed its own loads
    // of tile k, and the consumers their reads of the slot the next load reuses
    for (int k = 0; k <= n; ++k) {
      wait_vmcnt<kPer>();
      lds_barrier();
      if (k < n) {
        const int qt = qt0 + k;
        if (qt >= qa && qt < qb) produce(qt, k & 3, k & 1, qt0 + k + 2, (k + 2) & 3, bool_c<false>{});
        else produce(qt, k & 3, k & 1, qt0 + k + 2, (k + 2) & 3, bool_c<true>{});
      } else {
        dma(qt0 + k + 2, (k + 2) & 3);
      }
    }
    wait_vmcnt<0>();
    return;
  }

  // ================= consumer: dV += (P*M)^T dO, dK += dS^T Q, one tile behind
  f32x16 dv_acc[kDB], dk_acc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) dv_acc[db] = dk_acc[db] = f32x16{};
  const int tr_w = 16 * ((lane >> 4) & 1) + (8 * (lane >> 5) + ((lane & 15) >> 2)) * kWaveRow + 4 * (lane & 3);
  const int tr_s = tr_off32(kS, lane);
  auto consume = [&](int slot, int pbuf) {
    const bf16* qb_ = q_of(slot);
    const bf16* ob_ = do_of(slot);
    const bf16* pmt = sm.pm[pbuf][kg];
    const bf16* dst = sm.ds[pbuf][kg];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bf16x8 apm = tr_pair(&pmt[16 * st * kWaveRow + tr_w], kWaveRow);
      const bf16x8 ads = tr_pair(&dst[16 * st * kWaveRow + tr_w], kWaveRow);
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        dv_acc[db] = mfma32(apm, tr_pair(&ob_[16 * st * kS + tr_s + 32 * db], kS), dv_acc[db]);
        dk_acc[db] = mfma32(ads, tr_pair(&qb_[16 * st * kS + tr_s + 32 * db], kS), dk_acc[db]);
      }
    }
  };
  for (int k = 0; k <= n; ++k) {
    lds_barrier();
    if (k >= 1) consume((k - 1) & 3, (k - 1) & 1);
  }
  wait_vmcnt<0>();

  // store: lane holds d = 32db + col, keys kw0 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key >= p.s) continue;
      const float dvv = dv_acc[db][r] * p.inv_keep;
      const float dkv = dk_acc[db][r] * p.scale;
      const int dcol = 32 * db + col;
      if (PART || part >= 0) {   // slot 1 holds the second parts of split blocks
        const int64_t o = ((int64_t)max(part, 0) * p.b * p.s * p.hq + ((int64_t)bb * p.s + key) * p.hq + hh_q) * D + dcol;
        p.dv_acc[o] = dvv;
        p.dk_acc[o] = dkv;
      } else {
        static_cast<bf16*>(p.dv)[bb * p.sv_b + (int64_t)key * p.sv_s + g * p.sv_h + dcol] = (bf16)dvv;
        static_cast<bf16*>(p.dk)[bb * p.sk_b + (int64_t)key * p.sk_s + g * p.sk_h + dcol] = (bf16)dkv;
      }
    }
  }
}

// Block order: PAIRED (causal, unsplit) gives workgroup t the key blocks t
// and n-1-t; a split grid runs in decreasing modelled work (split_order);
// otherwise ascending (the blocks with the most queries first).
template <int D, bool CAUSAL, bool DROP, bool PART, bool VARLEN, bool PAIRED>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_pc_kernel(AttnParams p) {
  __shared__ DkdvPCSmem<D> sm;
  const int nbh = p.b * p.hq;
  const int nkb = (p.s + kBNk - 1) / kBNk;
  const int rank = (int)(blockIdx.x / nbh);
  const int bh = (int)(blockIdx.x % nbh);
  if constexpr (PAIRED) {
    const int b1 = nkb - 1 - rank;
    const int nblk = rank < b1 ? 2 : 1;
#pragma nounroll
    for (int i = 0; i < nblk; ++i) {
      if (i > 0) __syncthreads();   // the first block's consumers have read the ring
      dkdv_pc_tile<D, CAUSAL, DROP, PART, VARLEN>(p, sm, bh, i == 0 ? rank : b1, -1);
    }
  } else {
    const int nsk = kSplitBwd<D, CAUSAL> ? p.split_kb : 0;
    int kblk, part = -1;
    if (nsk > 0) {
      int t;
      split_order(rank, nkb, nsk, t, part);
      kblk = nkb - 1 - t;
    } else {
      kblk = rank;
    }
    dkdv_pc_tile<D, CAUSAL, DROP, PART, VARLEN>(p, sm, bh, kblk, part);
  }
}

// ============================================================== dQ
constexpr int kQM = 128;       // queries per dq workgroup
constexpr int kQN = 64;        // keys per K/V tile

// Two K and two V tiles (tile t is consumed while t+1 is written), one
// barrier per tile.  K is read as rows (S^T = K Q^T) and transposed
// (dQ^T += K^T dS^T): TileStride; V only as rows: RowStride.
template <int D>
struct alignas(16) DqSmem {
  static constexpr int kKS = TileStride<D>::kValue;
  static constexpr int kVS = RowStride<D>::kValue;
  bf16 k[2][kQN * kKS];
  bf16 v[2][kQN * kVS];
};

// Causal q-tile order: paired (two workgroups per CU: block i and block
// i + grid/2 carry equal work) or longest first (one per CU), as in the forward.
template <bool PAIRED>
__device__ __forceinline__ int causal_tile(int rank, int nqt) {
  if (!PAIRED) return nqt - 1 - rank;
  const int h = (nqt + 1) / 2;
  return rank < h ? nqt - 1 - rank : rank - h;
}

template <int D> struct DqOcc { static constexpr int kWavesPerEU = D <= 96 ? 2 : 1; };

template <int D, bool CAUSAL, bool DROP, bool VARLEN>
__global__ __launch_bounds__(256, DqOcc<D>::kWavesPerEU) void attn_bwd_dq_kernel(AttnParams p) {
  constexpr int kKS = DqSmem<D>::kKS;
  constexpr int kVS = DqSmem<D>::kVS;
  constexpr int kDC = D / 16;
  constexpr int kDB = D / 32;
  constexpr int kLoads = D / 32;
  constexpr bool kPreK = DqOcc<D>::kWavesPerEU == 1 && D <= 192;   // K^T operands read one phase early
  __shared__ DqSmem<D> sm;

  const int nqt = (p.s + kQM - 1) / kQM;
  const int nbh = p.b * p.hq;
  const int bh = blockIdx.x % nbh;
  const int rank = (int)(blockIdx.x / nbh);
  // Split grids (p.split_qt > 0, causal only): the split_qt longest tiles
  // run as two workgroups each (part 0: the first half of the tile's key
  // tiles, part 1: the rest), launched in decreasing order of work.
  const int nsq = kSplitBwd<D, CAUSAL> ? p.split_qt : 0;
  int qt, part = -1;
  if (nsq > 0) {
    split_order(rank, nqt, nsq, qt, part);
  } else {
    qt = CAUSAL ? causal_tile<DqOcc<D>::kWavesPerEU == 2>(rank, nqt) : rank;
  }
  const int hh_q = bh % p.hq, bb = bh / p.hq;
  const int g = hh_q / (p.hq / p.hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps tile bounds scalar
  const int half = lane >> 5, col = lane & 31;
  const int q0 = qt * kQM;
  const int qw = q0 + 32 * wv;
  const int qi = qw + col;
  const bool qvalid = qi < p.s;
  const int sl = VARLEN ? attn_len(p, bb) : p.s;   // valid length of this batch element
  const bool qlive = VARLEN ? qi < sl : qvalid;      // a query row inside it

  const bf16* qp = static_cast<const bf16*>(p.q) + bb * p.sq_b + hh_q * p.sq_h;
  const bf16* dop = static_cast<const bf16*>(p.dout) + bb * p.so_b + hh_q * p.so_h;
  const bf16* kp = static_cast<const bf16*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const bf16* vp = static_cast<const bf16*>(p.v) + bb * p.sv_b + g * p.sv_h;
  const int64_t row0 = ((int64_t)bb * p.hq + hh_q) * p.s;

  // Q^T and dO^T B operands: lane (col, half) holds row qi, d = 16c + 8*half ..
  bf16x8 qreg[kDC], doreg[kDC];
#pragma unroll
  for (int c = 0; c < kDC; ++c) qreg[c] = doreg[c] = bf16x8{};
  if (qlive) {
#pragma unroll
    for (int c = 0; c < kDC; ++c) {
      qreg[c] = *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.sq_s + 16 * c + 8 * half);
      doreg[c] = *reinterpret_cast<const bf16x8*>(dop + (int64_t)qi * p.so_s + 16 * c + 8 * half);
    }
  }
  // rows past the valid length see no key (dQ = 0, D = 0); rows past s are not stored
  const float lse2 = qlive ? p.lse[row0 + qi] * kLog2e : 0.f;
  // D = rowsum(dO * O) of the lane's query: the lane's d-slices of O against
  // the same slices of dO (doreg), plus the other lane half's complementary
  // slices; stored for the dK/dV kernel, which runs after this one
  float dlt = 0.f;
  if (qlive) {
    const bf16* orow = static_cast<const bf16*>(p.o) + bb * p.so_b + hh_q * p.so_h + (int64_t)qi * p.so_s;
#pragma unroll
    for (int c = 0; c < kDC; ++c) {
      const bf16x8 ov = *reinterpret_cast<const bf16x8*>(orow + 16 * c + 8 * half);
#pragma unroll
      for (int e = 0; e < 8; ++e) dlt = fmaf(bf2f(ov[e]), bf2f(doreg[c][e]), dlt);
    }
  }
  dlt = halves_sum(dlt);
  if (qvalid && half == 0 && part <= 0) p.delta[row0 + qi] = dlt;

  f32x16 qacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) qacc[db] = f32x16{};

  const int nkt_all = (sl + kQN - 1) / kQN;
  const int nkt = CAUSAL ? min(nkt_all, (q0 + kQM + kQN - 1) / kQN) : nkt_all;
  // tiles this wave computes without masking (none if it holds a row past sl)
  const int n_int = (VARLEN && qw + 31 >= sl) ? 0 : CAUSAL ? min(sl / kQN, (qw + 1) / kQN) : sl / kQN;
  // key tiles [kt_lo, kt_hi) of this workgroup
  const int kt_mid = (nkt + 1) / 2;
  const int kt_lo = part == 1 ? kt_mid : 0;
  const int kt_hi = part == 0 ? kt_mid : nkt;
  const int key_lim = VARLEN ? (qlive ? (CAUSAL ? min(sl, qi + 1) : sl) : 0) : (CAUSAL ? min(p.s, qi + 1) : p.s);

  // ---- K/V staging through buffer loads (keys past s read as zero)
  uint4 kpre[kLoads], vpre[kLoads];
  uint32_t koff[kLoads], voff[kLoads];
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int x = tid + 256 * it;
    koff[it] = (uint32_t)(((int64_t)(x / (D / 8)) * p.sk_s + 8 * (x % (D / 8))) * 2);
    voff[it] = (uint32_t)(((int64_t)(x / (D / 8)) * p.sv_s + 8 * (x % (D / 8))) * 2);
  }
  auto tile_bytes = [&](int kt, int64_t stride) -> uint32_t {
    const int rows = min(kQN, max(0, sl - kt * kQN));
    return (uint32_t)((int64_t)rows * stride * 2);
  };
  auto load_kv = [&](int kt) {
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kp + (int64_t)kt * kQN * p.sk_s, tile_bytes(kt, p.sk_s));
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vp + (int64_t)kt * kQN * p.sv_s, tile_bytes(kt, p.sv_s));
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      kpre[it] = buffer_load16(rk, koff[it]);
      vpre[it] = buffer_load16(rv, voff[it]);
    }
  };
  auto stash_kv = [&](int buf) {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int x = tid + 256 * it;
      const int r = x / (D / 8), c8 = x % (D / 8);
      const int sr = (r & ~31) | slot32(r & 31);   // slot order
      *reinterpret_cast<uint4*>(&sm.k[buf][sr * kKS + 8 * c8]) = kpre[it];
      *reinterpret_cast<uint4*>(&sm.v[buf][sr * kVS + 8 * c8]) = vpre[it];
    }
  };

  const uint32_t hg = (uint32_t)(p.head_offset + hh_q);
  const PhiloxRow prow = philox_row((uint32_t)qi, hg, (uint32_t)bb, p.k0, p.k1);
  const uint32_t thr_hi = p.thresh << 16;
  const float c2 = p.scale_log2;
  const int kro = col * kKS + 8 * half;    // K, V tile rows are in slot order
  const int vro = col * kVS + 8 * half;
  // K^T operand of step c (keys 32*(c/2) + 16*h + 8*(c%2) + e of lane half h):
  // in slot order those are rows 16*(c%2) + 4*h + (0..3) and the same + 8
  const int grp = lane >> 4, lg = lane & 15;
  const int ktr = (4 * (grp >> 1) + (lg >> 2)) * kKS + 16 * (grp & 1) + 4 * (lg & 3);

  // K^T A operand of dQ step c (keys 32(c/2) + 16(c%2) ..), d block db, from
  // a row-major K tile through two transposing reads
  auto kt_operand = [&](const bf16* kb_, int c, int db) -> bf16x8 {
    const int r0 = (32 * (c >> 1) + 16 * (c & 1)) * kKS + ktr;
    const s16x4 lo = lds_read_tr16(&kb_[r0 + 32 * db]);
    const s16x4 hi = lds_read_tr16(&kb_[r0 + 8 * kKS + 32 * db]);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto tile = [&](int kt, auto mask_c, auto next_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    const int key0 = kt * kQN;
    const int buf = kt & 1;
    __syncthreads();
    if (NEXT) {
      stash_kv(buf ^ 1);          // K/V[kt+1] over K/V[kt-1]
      load_kv(kt + 2);
    }
    // keep the loads at the top of the tile, a whole tile ahead of their use
    // (left alone, the scheduler sinks them to the end of the loop body to
    // reuse their registers, and the next stash waits the full load latency);
    // at d > 96 the pinned registers cost more than the latency they hide
    if constexpr (D <= 96) __builtin_amdgcn_sched_barrier(0);
    // ---- S^T = K Q^T, dP^T = V dO^T for two 32-key blocks; the Philox draws
    // of the tile are independent and overlap the MFMAs
    f32x16 sacc[2], pacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sacc[kb] = pacc[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < kDC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = mfma32(*reinterpret_cast<const bf16x8*>(&sm.k[buf][32 * kb * kKS + kro + 16 * c]), qreg[c], sacc[kb]);
        pacc[kb] = mfma32(*reinterpret_cast<const bf16x8*>(&sm.v[buf][32 * kb * kVS + vro + 16 * c]), doreg[c], pacc[kb]);
      }
    // with one wave per SIMD nothing else hides the LDS latency of the K^T
    // operands of dQ, so they are read here, behind the MFMAs above
    bf16x8 kop[kPreK ? 4 : 1][kPreK ? kDB : 1];
    if (kPreK) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int db = 0; db < kDB; ++db) kop[c][db] = kt_operand(sm.k[buf], c, db);
    }
    uint32_t w[16];
    if (DROP) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int gh = 0; gh < 2; ++gh) {
          const Philox4 rnd = philox4x32_10_row((uint32_t)((key0 + 32 * kb + 16 * half + 8 * gh) >> 3), prow);
#pragma unroll
          for (int j = 0; j < 4; ++j) w[8 * kb + 4 * gh + j] = rnd.w[j];
        }
    }

    // ---- dS^T = P * (dP * M / (1-p) - D), packed to bf16 pairs
    uint32_t dsw[16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float pv[2], dp[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + e], c2, -lse2));
          if (MASK) pv[e] = key0 + 32 * kb + 16 * half + r + e >= key_lim ? 0.f : pv[e];
          dp[e] = pacc[kb][r + e];
        }
        if (DROP) {
          const uint32_t ww = w[8 * kb + (r >> 1)];
          dp[0] = (ww & 0xFFFFu) >= p.thresh ? dp[0] : 0.f;
          dp[1] = ww >= thr_hi ? dp[1] : 0.f;
        }
        dsw[8 * kb + (r >> 1)] =
            pack_bf16x2(pv[0] * fmaf(dp[0], p.inv_keep, -dlt), pv[1] * fmaf(dp[1], p.inv_keep, -dlt));
      }

    // ---- dQ^T += K^T dS^T; K^T operand through LDS transpose reads
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 dsop = __builtin_bit_cast(bf16x8, make_uint4(dsw[4 * c], dsw[4 * c + 1], dsw[4 * c + 2], dsw[4 * c + 3]));
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        qacc[db] = mfma32(kPreK ? kop[c][db] : kt_operand(sm.k[buf], c, db), dsop, qacc[db]);
    }
  };

  // a query tile past the valid length (padded batch) sees no key (key_lim
  // is 0 for all its rows): its tiles leave dQ = 0
  // prologue: K/V[kt_lo] resident, K/V[kt_lo+1] in flight
  load_kv(kt_lo);
  stash_kv(kt_lo & 1);
  load_kv(kt_lo + 1);
  // separate straight-line loops (see the forward kernel)
  int kt = kt_lo;
  for (; kt < min(n_int, kt_hi - 1); ++kt) tile(kt, bool_c<false>{}, bool_c<true>{});
  for (; kt < kt_hi - 1; ++kt) tile(kt, bool_c<true>{}, bool_c<true>{});
  if (kt < n_int) tile(kt, bool_c<false>{}, bool_c<false>{});
  else tile(kt, bool_c<true>{}, bool_c<false>{});


  // a split tile's part: the raw fp32 dQ^T partial, [2][b, hq, s, d]
  if (part >= 0) {
    if (qvalid) {
      float* dst = p.dq_part + (((int64_t)part * p.b * p.hq * p.s) + row0 + qi) * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<float4*>(dst + 32 * db + 8 * a + 4 * half) =
              make_float4(qacc[db][4 * a], qacc[db][4 * a + 1], qacc[db][4 * a + 2], qacc[db][4 * a + 3]);
    }
    return;
  }
  // dQ = dQ^T * scale; lane holds query qi, d = 32db + 8a + 4*half + j
  if (qvalid) {
    bf16* dq = static_cast<bf16*>(p.dq) + bb * p.sq_b + (int64_t)qi * p.sq_s + hh_q * p.sq_h;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 wo;
        wo.x = pack_bf16x2(qacc[db][4 * a + 0] * p.scale, qacc[db][4 * a + 1] * p.scale);
        wo.y = pack_bf16x2(qacc[db][4 * a + 2] * p.scale, qacc[db][4 * a + 3] * p.scale);
        *reinterpret_cast<uint2*>(dq + 32 * db + 8 * a + 4 * half) = wo;
      }
    }
  }
}

// ============================================================== dQ, two key groups (d = 128)
// At d = 128 the one-group dQ kernel needs ~400 registers per wave, so it
// runs one wave per SIMD and nothing hides its latencies.  This variant runs
// 8 waves in two groups of 4 over the same 128 queries; group g takes the
// key tiles kt_lo + 2j + g, so each wave fits 256 registers and two waves
// share a SIMD.  Group 1 runs one barrier phase behind group 0: while one
// wave of a SIMD issues its MFMAs (phase M: dQ^T += K^T dS^T of its previous
// tile, then S^T and dP^T of its current tile), the other forms dS on the
// VALU (phase V).  At the end group 1 hands its dQ^T to group 0 through LDS.
// K/V tiles go from the buffer to LDS without passing through registers
// (buffer_load ... lds), K one step ahead (it is read again, transposed, in
// the step after its own) and V two steps ahead.
template <int D>
struct alignas(16) DqPPSmem {
  static constexpr int kKS = TileStride<D>::kValue;   // K: rows (S^T) and transposed (dQ^T)
  static constexpr int kVS = RowStride<D>::kValue;    // V: rows only
  union {
    struct {
      bf16 k[2][2][kQN * kKS];   // [group][buffer], rows in slot order
      bf16 v[2][2][kQN * kVS];
    } t;
    float x[4][(D / 32) * 16][64];   // group 1's dQ^T accumulators
  };
};

// (at d = 96 two one-group workgroups already share a CU, and the two-group
// form measured slower there: gpt22b-t8 shape 67 -> 88 us)
template <int D>
constexpr bool kDqPingPong = D == 128;

template <int D, bool CAUSAL, bool DROP, bool VARLEN>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_pp_kernel(AttnParams p) {
  using SM = DqPPSmem<D>;
  constexpr int kKS = SM::kKS;
  constexpr int kVS = SM::kVS;
  constexpr int kDC = D / 16;
  constexpr int kDB = D / 32;
  __shared__ SM sm;

  const int nqt = (p.s + kQM - 1) / kQM;
  const int nbh = p.b * p.hq;
  const int bh = blockIdx.x % nbh;
  const int rank = (int)(blockIdx.x / nbh);
  const int nsq = kSplitBwd<D, CAUSAL> ? p.split_qt : 0;
  int qt, part = -1;
  if (nsq > 0) {
    split_order(rank, nqt, nsq, qt, part);
  } else {
    qt = CAUSAL ? causal_tile<false>(rank, nqt) : rank;
  }
  const int hh_q = bh % p.hq, bb = bh / p.hq;
  const int g = hh_q / (p.hq / p.hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps tile bounds scalar
  const int grp = wv >> 2, wq = wv & 3;                       // key group, query block
  const int half = lane >> 5, col = lane & 31;
  const int q0 = qt * kQM;
  const int qw = q0 + 32 * wq;
  const int qi = qw + col;
  const bool qvalid = qi < p.s;
  const int sl = VARLEN ? attn_len(p, bb) : p.s;
  const bool qlive = VARLEN ? qi < sl : qvalid;

  const bf16* qp = static_cast<const bf16*>(p.q) + bb * p.sq_b + hh_q * p.sq_h;
  const bf16* dop = static_cast<const bf16*>(p.dout) + bb * p.so_b + hh_q * p.so_h;
  const bf16* kp = static_cast<const bf16*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const bf16* vp = static_cast<const bf16*>(p.v) + bb * p.sv_b + g * p.sv_h;
  const int64_t row0 = ((int64_t)bb * p.hq + hh_q) * p.s;

  // Q^T and dO^T B operands (as the one-group kernel), D = rowsum(dO * O)
  bf16x8 qreg[kDC], doreg[kDC];
#pragma unroll
  for (int c = 0; c < kDC; ++c) qreg[c] = doreg[c] = bf16x8{};
  if (qlive) {
#pragma unroll
    for (int c = 0; c < kDC; ++c) {
      qreg[c] = *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.sq_s + 16 * c + 8 * half);
      doreg[c] = *reinterpret_cast<const bf16x8*>(dop + (int64_t)qi * p.so_s + 16 * c + 8 * half);
    }
  }
  const float lse2 = qlive ? p.lse[row0 + qi] * kLog2e : 0.f;
  float dlt = 0.f;
  if (qlive) {
    const bf16* orow = static_cast<const bf16*>(p.o) + bb * p.so_b + hh_q * p.so_h + (int64_t)qi * p.so_s;
#pragma unroll
    for (int c = 0; c < kDC; ++c) {
      const bf16x8 ov = *reinterpret_cast<const bf16x8*>(orow + 16 * c + 8 * half);
#pragma unroll
      for (int e = 0; e < 8; ++e) dlt = fmaf(bf2f(ov[e]), bf2f(doreg[c][e]), dlt);
    }
  }
  dlt = halves_sum(dlt);
  if (grp == 0 && qvalid && half == 0 && part <= 0) p.delta[row0 + qi] = dlt;
  // consumed here, so the compiler waits for these loads now and does not
  // guard their later uses with waits that would also drain the tile loads
#pragma unroll
  for (int c = 0; c < kDC; ++c) asm volatile("" ::"v"(qreg[c]), "v"(doreg[c]));
  asm volatile("" ::"v"(lse2));
  // the tile loads are counted on vmcnt after everything issued so far
  wait_vmcnt<0>();

  f32x16 qacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) qacc[db] = f32x16{};

  const int nkt_all = (sl + kQN - 1) / kQN;
  const int nkt_q = CAUSAL ? min(nkt_all, (q0 + kQM + kQN - 1) / kQN) : nkt_all;
  const int kt_mid = (nkt_q + 1) / 2;
  const int kt_lo = part == 1 ? kt_mid : 0;
  const int nkt = part == 0 ? kt_mid : nkt_q;                      // key tiles [kt_lo, nkt)
  const int nsteps = (nkt - kt_lo + 1) / 2;                        // steps of both groups
  const int n_int = (VARLEN && qw + 31 >= sl) ? 0 : CAUSAL ? min(sl / kQN, (qw + 1) / kQN) : sl / kQN;
  const int key_lim = VARLEN ? (qlive ? (CAUSAL ? min(sl, qi + 1) : sl) : 0) : (CAUSAL ? min(p.s, qi + 1) : p.s);
  auto tile_of = [&](int j) { return kt_lo + 2 * j + grp; };

  // ---- staging: buffer -> LDS loads, 1 KB of LDS per instruction (lane l
  // the bytes 16l .. 16l+15), per-lane global offsets that land K and V in
  // slot order in the padded layouts; padding reads from past the buffer's
  // end, which gives zero.  The 4 waves of a group share a tile's blocks.
  constexpr int kKBytes = kQN * kKS * 2, kVBytes = kQN * kVS * 2;
  constexpr int kKBlocks = kKBytes / 1024, kVBlocks = kVBytes / 1024;
  static_assert(kKBytes % 1024 == 0 && kVBytes % 1024 == 0, "tiles must be whole 1 KB blocks");
  constexpr int kKPer = (kKBlocks + 3) / 4, kVPer = (kVBlocks + 3) / 4;
  // the V blocks wave w issues per tile: the wait at the end of a V phase
  // leaves exactly those (its most recent loads: V, two steps ahead) in
  // flight and completes everything before them
  auto wait_recent = [&] {
    wait_vmcnt_by_wave<blocks_of_wave(kVBlocks, 0), blocks_of_wave(kVBlocks, 1), blocks_of_wave(kVBlocks, 2),
                       blocks_of_wave(kVBlocks, 3)>(wq);
  };
  uint32_t kdo[kKPer], vdo[kVPer];
#pragma unroll
  for (int i = 0; i < kKPer; ++i) {
    const int pos = 1024 * (wq + 4 * i) + 16 * lane;
    const int row = pos / (2 * kKS), cb = pos % (2 * kKS);
    const int key = (row & ~31) | perm32(row & 31);
    kdo[i] = (row < kQN && cb < 2 * D) ? (uint32_t)((int64_t)key * p.sk_s * 2 + cb) : 0xFFFFFFF0u;
  }
#pragma unroll
  for (int i = 0; i < kVPer; ++i) {
    const int pos = 1024 * (wq + 4 * i) + 16 * lane;
    const int row = pos / (2 * kVS), cb = pos % (2 * kVS);
    const int key = (row & ~31) | perm32(row & 31);
    vdo[i] = (row < kQN && cb < 2 * D) ? (uint32_t)((int64_t)key * p.sv_s * 2 + cb) : 0xFFFFFFF0u;
  }
  auto tile_bytes = [&](int kt, int64_t stride) -> uint32_t {
    const int rows = kt < nkt ? min(kQN, max(0, sl - kt * kQN)) : 0;
    return (uint32_t)((int64_t)rows * stride * 2);
  };
  auto dma_k = [&](int kt, int buf) {
    const sgpr4 rk = buffer_rsrc_sgpr(kp + (int64_t)kt * kQN * p.sk_s, tile_bytes(kt, p.sk_s));
    const uintptr_t base = (uintptr_t)&sm.t.k[grp][buf][0];
#pragma unroll
    for (int i = 0; i < kKPer; ++i)
      if (wq + 4 * i < kKBlocks) buffer_load16_lds(rk, base + 1024 * (wq + 4 * i), kdo[i]);
  };
  auto dma_v = [&](int kt, int buf) {
    const sgpr4 rv = buffer_rsrc_sgpr(vp + (int64_t)kt * kQN * p.sv_s, tile_bytes(kt, p.sv_s));
    const uintptr_t base = (uintptr_t)&sm.t.v[grp][buf][0];
#pragma unroll
    for (int i = 0; i < kVPer; ++i)
      if (wq + 4 * i < kVBlocks) buffer_load16_lds(rv, base + 1024 * (wq + 4 * i), vdo[i]);
  };

  const uint32_t hg = (uint32_t)(p.head_offset + hh_q);
  const PhiloxRow prow = philox_row((uint32_t)qi, hg, (uint32_t)bb, p.k0, p.k1);
  const uint32_t thr_hi = p.thresh << 16;
  const float c2 = p.scale_log2;
  const int kro = col * kKS + 8 * half;
  const int vro = col * kVS + 8 * half;
  const int lgp = lane >> 4, lg = lane & 15;
  const int ktr = (4 * (lgp >> 1) + (lg >> 2)) * kKS + 16 * (lgp & 1) + 4 * (lg & 3);
  auto kt_operand = [&](const bf16* kb_, int c, int db) -> bf16x8 {
    const int r0 = (32 * (c >> 1) + 16 * (c & 1)) * kKS + ktr;
    const s16x4 lo = lds_read_tr16(&kb_[r0 + 32 * db]);
    const s16x4 hi = lds_read_tr16(&kb_[r0 + 8 * kKS + 32 * db]);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 sacc[2], pacc[2];   // S^T, dP^T of the current tile
  uint32_t dsw[16];          // dS^T of the previous tile, packed bf16 pairs

  // M phase of step j: dQ^T += K^T dS^T of step j-1 (if it had a tile), then
  // S^T = K Q^T and dP^T = V dO^T of step j
  auto phase_m = [&](int j, bool dq, bool sp) {
    if (dq) {
      const bf16* kb_ = sm.t.k[grp][(j - 1) & 1];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 dsop =
            __builtin_bit_cast(bf16x8, make_uint4(dsw[4 * c], dsw[4 * c + 1], dsw[4 * c + 2], dsw[4 * c + 3]));
#pragma unroll
        for (int db = 0; db < kDB; ++db) qacc[db] = mfma32(kt_operand(kb_, c, db), dsop, qacc[db]);
      }
    }
    if (sp) {
      const bf16* kb_ = sm.t.k[grp][j & 1];
      const bf16* vb = sm.t.v[grp][j & 1];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = pacc[kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < kDC; ++c)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          sacc[kb] = mfma32(*reinterpret_cast<const bf16x8*>(&kb_[32 * kb * kKS + kro + 16 * c]), qreg[c], sacc[kb]);
          pacc[kb] = mfma32(*reinterpret_cast<const bf16x8*>(&vb[32 * kb * kVS + vro + 16 * c]), doreg[c], pacc[kb]);
        }
    }
  };

  // V phase of step j: load K of step j+1 (its buffer's tile, step j-1, was
  // last read by M(j)) and V of step j+2 (its buffer's tile, step j, too);
  // form dS^T of step j into dsw (MASK: causal / tail masking needed)
  auto phase_v = [&](int j, bool have, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    dma_k(tile_of(j + 1), (j + 1) & 1);
    dma_v(tile_of(j + 2), j & 1);
    if (!have) return;
    const int key0 = tile_of(j) * kQN;
    uint32_t w[16];
    if (DROP) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int gh = 0; gh < 2; ++gh) {
          const Philox4 rnd = philox4x32_10_row((uint32_t)((key0 + 32 * kb + 16 * half + 8 * gh) >> 3), prow);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) w[8 * kb + 4 * gh + jj] = rnd.w[jj];
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float pv[2], dp[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][r + e], c2, -lse2));
          if (MASK) pv[e] = key0 + 32 * kb + 16 * half + r + e >= key_lim ? 0.f : pv[e];
          dp[e] = pacc[kb][r + e];
        }
        if (DROP) {
          const uint32_t ww = w[8 * kb + (r >> 1)];
          dp[0] = (ww & 0xFFFFu) >= p.thresh ? dp[0] : 0.f;
          dp[1] = ww >= thr_hi ? dp[1] : 0.f;
        }
        dsw[8 * kb + (r >> 1)] =
            pack_bf16x2(pv[0] * fmaf(dp[0], p.inv_keep, -dlt), pv[1] * fmaf(dp[1], p.inv_keep, -dlt));
      }
  };

  // ---- prologue: K and V of step 0 resident, V of step 1 in flight
  dma_k(tile_of(0), 0);
  dma_v(tile_of(0), 0);
  dma_v(tile_of(1), 1);
  wait_recent();
  __syncthreads();
  if (grp == 1) __syncthreads();   // group 1 runs one phase behind

  // steps whose tile needs no masking for this wave: tile_of(j) < n_int
  const int j_int = max(0, min(nsteps, (min(n_int, nkt) - kt_lo - grp + 1) / 2));
  int j = 0;
  // bare barriers in the loop (see lds_barrier): each wave completes its own
  // LDS reads and, at the end of a V phase, the loads the next M phase reads
  for (; j < j_int; ++j) {
    phase_m(j, j > 0, true);
    lds_barrier();
    phase_v(j, true, bool_c<false>{});
    wait_recent();
    lds_barrier();
  }
  for (; j < nsteps; ++j) {
    const bool have = tile_of(j) < nkt;
    phase_m(j, j > 0, have);
    lds_barrier();
    phase_v(j, have, bool_c<true>{});
    wait_recent();
    lds_barrier();
  }
  phase_m(nsteps, nsteps > 0 && tile_of(nsteps - 1) < nkt, false);
  wait_vmcnt<0>();                 // no load may land in LDS once it is reused below
  __syncthreads();
  if (grp == 0) __syncthreads();   // balances group 1's extra barrier

  // ---- group 1's dQ^T into group 0's (both over the same queries)
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.x[wq][db * 16 + r][lane] = qacc[db][r];
  }
  __syncthreads();
  if (grp == 1) return;
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) qacc[db][r] += sm.x[wq][db * 16 + r][lane];

  // ---- store (as the one-group kernel)
  if (part >= 0) {
    if (qvalid) {
      float* dst = p.dq_part + (((int64_t)part * p.b * p.hq * p.s) + row0 + qi) * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<float4*>(dst + 32 * db + 8 * a + 4 * half) =
              make_float4(qacc[db][4 * a], qacc[db][4 * a + 1], qacc[db][4 * a + 2], qacc[db][4 * a + 3]);
    }
    return;
  }
  if (qvalid) {
    bf16* dq = static_cast<bf16*>(p.dq) + bb * p.sq_b + (int64_t)qi * p.sq_s + hh_q * p.sq_h;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 wo;
        wo.x = pack_bf16x2(qacc[db][4 * a + 0] * p.scale, qacc[db][4 * a + 1] * p.scale);
        wo.y = pack_bf16x2(qacc[db][4 * a + 2] * p.scale, qacc[db][4 * a + 3] * p.scale);
        *reinterpret_cast<uint2*>(dq + 32 * db + 8 * a + 4 * half) = wo;
      }
    }
  }
}

// ============================================================== partial sums
// dK, dV of a kv-head = the sum of its fp32 partials: over the q-heads that
// share it (grouped-query attention) and over the two parts of a split key
// block (slot 1, keys below 128 * split_kb), in a fixed order; written as
// bf16 in 8-element chunks.  Keys [0, nkeys) are covered.
template <int D>
__device__ __forceinline__ void kv_sum_job(const AttnParams& p, int nkeys, int64_t x) {
  const int64_t nk = (int64_t)p.b * nkeys * p.hkv * (D / 8);
  if (x >= 2 * nk) return;
  const bool is_v = x >= nk;
  const int64_t y = is_v ? x - nk : x;
  const int c8 = (int)(y % (D / 8));
  const int64_t row = y / (D / 8);                           // (b, key, hkv)
  const int gg = (int)(row % p.hkv);
  const int64_t bk = row / p.hkv;
  const int i = (int)(bk % nkeys), bb = (int)(bk / nkeys);
  const int grp = p.hq / p.hkv;
  const int nslot = i < 128 * p.split_kb ? 2 : 1;
  const int64_t slot_stride = (int64_t)p.b * p.s * p.hq * D;
  const float* src = (is_v ? p.dv_acc : p.dk_acc) + (((int64_t)bb * p.s + i) * p.hq + (int64_t)gg * grp) * D + 8 * c8;
  float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int sl = 0; sl < nslot; ++sl)
    for (int j = 0; j < grp; ++j) {
      const float* q = src + sl * slot_stride + (int64_t)j * D;
      const float4 u = reinterpret_cast<const float4*>(q)[0];
      const float4 v = reinterpret_cast<const float4*>(q)[1];
      a[0] += u.x; a[1] += u.y; a[2] += u.z; a[3] += u.w;
      a[4] += v.x; a[5] += v.y; a[6] += v.z; a[7] += v.w;
    }
  uint4 w;
  w.x = pack_bf16x2(a[0], a[1]); w.y = pack_bf16x2(a[2], a[3]);
  w.z = pack_bf16x2(a[4], a[5]); w.w = pack_bf16x2(a[6], a[7]);
  bf16* dst = is_v ? static_cast<bf16*>(p.dv) + bb * p.sv_b + (int64_t)i * p.sv_s + gg * p.sv_h
                   : static_cast<bf16*>(p.dk) + bb * p.sk_b + (int64_t)i * p.sk_s + gg * p.sk_h;
  *reinterpret_cast<uint4*>(dst + 8 * c8) = w;
}

// dQ of the queries of split tiles (rows from q_lo) = (part 0 + part 1) * scale.
template <int D>
__device__ __forceinline__ void dq_sum_job(const AttnParams& p, int q_lo, int64_t x) {
  const int nrows = p.s - q_lo;
  const int64_t n = (int64_t)p.b * p.hq * nrows * (D / 8);
  if (x >= n) return;
  const int c8 = (int)(x % (D / 8));
  const int64_t r = x / (D / 8);                             // (b, hq, query)
  const int qi = q_lo + (int)(r % nrows);
  const int64_t bh = r / nrows;
  const int hh = (int)(bh % p.hq), bb = (int)(bh / p.hq);
  const int64_t part_stride = (int64_t)p.b * p.hq * p.s * D;
  const float* src = p.dq_part + (bh * p.s + qi) * D + 8 * c8;
  const float4 u0 = reinterpret_cast<const float4*>(src)[0], v0 = reinterpret_cast<const float4*>(src)[1];
  const float4 u1 = reinterpret_cast<const float4*>(src + part_stride)[0];
  const float4 v1 = reinterpret_cast<const float4*>(src + part_stride)[1];
  const float sc = p.scale;
  uint4 w;
  w.x = pack_bf16x2((u0.x + u1.x) * sc, (u0.y + u1.y) * sc);
  w.y = pack_bf16x2((u0.z + u1.z) * sc, (u0.w + u1.w) * sc);
  w.z = pack_bf16x2((v0.x + v1.x) * sc, (v0.y + v1.y) * sc);
  w.w = pack_bf16x2((v0.z + v1.z) * sc, (v0.w + v1.w) * sc);
  bf16* dst = static_cast<bf16*>(p.dq) + bb * p.sq_b + (int64_t)qi * p.sq_s + hh * p.sq_h;
  *reinterpret_cast<uint4*>(dst + 8 * c8) = w;
}

// The partial sums of one backward pass in one launch (after the dK/dV
// kernel): workgroups [0, dq_blocks) sum the dQ halves of split query tiles
// (q_lo >= 0), the rest the dK/dV partials of keys [0, nkeys) (nkeys > 0).
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_sums_kernel(AttnParams p, int q_lo, int nkeys, int dq_blocks) {
  const int blk = (int)blockIdx.x;
  if (blk < dq_blocks) dq_sum_job<D>(p, q_lo, (int64_t)blk * 256 + threadIdx.x);
  else kv_sum_job<D>(p, nkeys, (int64_t)(blk - dq_blocks) * 256 + threadIdx.x);
}

template <int D, bool CAUSAL, bool DROP, bool VARLEN>
hipError_t bwd_main(const AttnParams& p, hipStream_t st) {
  const bool part = p.hq != p.hkv;
  const unsigned nbh = (unsigned)(p.hq * p.b);
  {
    TraceScope ts("attn_bwd_dq", st);
    const unsigned nqt = (unsigned)((p.s + kQM - 1) / kQM);
    if constexpr (kDqPingPong<D>)
      attn_bwd_dq_pp_kernel<D, CAUSAL, DROP, VARLEN><<<(nqt + p.split_qt) * nbh, 512, 0, st>>>(p);
    else
      attn_bwd_dq_kernel<D, CAUSAL, DROP, VARLEN><<<(nqt + p.split_qt) * nbh, 256, 0, st>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    TraceScope ts("attn_bwd_dkdv", st);
    const unsigned nkb = (unsigned)((p.s + kBNk - 1) / kBNk);
    const dim3 grid((nkb + p.split_kb) * nbh * DkdvCfg<D>::kDParts);
    const int threads = 256 * DkdvCfg<D>::kQH;
    if constexpr (kDkdvPC<D>) {
      if (CAUSAL && attn_pair_tiles(p, (int)nkb, p.split_kb)) {
        const dim3 gp((nkb + 1) / 2 * nbh);
        if (part) attn_bwd_dkdv_pc_kernel<D, CAUSAL, DROP, true, VARLEN, CAUSAL><<<gp, 512, 0, st>>>(p);
        else attn_bwd_dkdv_pc_kernel<D, CAUSAL, DROP, false, VARLEN, CAUSAL><<<gp, 512, 0, st>>>(p);
      } else {
        if (part) attn_bwd_dkdv_pc_kernel<D, CAUSAL, DROP, true, VARLEN, false><<<grid, 512, 0, st>>>(p);
        else attn_bwd_dkdv_pc_kernel<D, CAUSAL, DROP, false, VARLEN, false><<<grid, 512, 0, st>>>(p);
      }
    } else {
      if (part) attn_bwd_dkdv_kernel<D, CAUSAL, DROP, true, VARLEN><<<grid, threads, 0, st>>>(p);
      else attn_bwd_dkdv_kernel<D, CAUSAL, DROP, false, VARLEN><<<grid, threads, 0, st>>>(p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // partial sums, one launch: dQ of split query tiles, dK/dV of grouped
  // query heads or of split key blocks
  const int q_lo = p.split_qt > 0 ? (int)(((p.s + kQM - 1) / kQM - p.split_qt) * kQM) : -1;
  const int64_t n_dq = q_lo >= 0 ? (int64_t)p.b * p.hq * (p.s - q_lo) * (D / 8) : 0;
  const int nkeys = part ? p.s : min(p.s, 128 * p.split_kb);
  const int64_t n_kv = nkeys > 0 ? 2 * (int64_t)p.b * nkeys * p.hkv * (D / 8) : 0;
  if (n_dq == 0 && n_kv == 0) return hipSuccess;
  TraceScope ts("attn_bwd_sums", st);
  const int dq_blocks = (int)((n_dq + 255) / 256);
  const int kv_blocks = (int)((n_kv + 255) / 256);
  attn_bwd_sums_kernel<D><<<(unsigned)(dq_blocks + kv_blocks), 256, 0, st>>>(p, q_lo, nkeys, dq_blocks);
  return hipGetLastError();
}

template <int D, bool VARLEN>
hipError_t bwd_launch_v(const AttnParams& p, hipStream_t st) {
  const bool drop = p.thresh != 0;
  if (p.causal) return drop ? bwd_main<D, true, true, VARLEN>(p, st) : bwd_main<D, true, false, VARLEN>(p, st);
  return drop ? bwd_main<D, false, true, VARLEN>(p, st) : bwd_main<D, false, false, VARLEN>(p, st);
}

template <int D>
hipError_t bwd_launch_d(const AttnParams& p, hipStream_t st) {
  return p.seqlens ? bwd_launch_v<D, true>(p, st) : bwd_launch_v<D, false>(p, st);
}

}  // namespace

AttnSplit attn_grid_split(int64_t b, int64_t s, int64_t hq, int64_t d, bool causal, bool bf16) {
  AttnSplit r{0, 0};
  // the one-workgroup-per-CU kernels (d >= 128) of causal grids with at most
  // one 128-row workgroup per CU of a 256-CU MI355X
  if (!bf16 || !causal || d < 128 || s <= 0 || b <= 0) return r;
  const int64_t nqt = (s + kQM - 1) / kQM;
  if (nqt * b * hq > 256) return r;
  const int64_t nkt_all = (s + kQN - 1) / kQN;
  for (int64_t qt = 0; qt < nqt; ++qt) {
    const int64_t nkt = std::min(nkt_all, (qt * kQM + kQM + kQN - 1) / kQN);
    if (nkt >= 2 && nkt > (nkt_all + 1) / 2) ++r.split_qt;
  }
  const int64_t nq32 = (s + 31) / 32;
  for (int64_t kb = 0; kb < (s + kBNk - 1) / kBNk; ++kb) {
    const int64_t len = nq32 - kb * kBNk / 32;
    if (len >= 2 && len > (nq32 + 1) / 2) ++r.split_kb;
  }
  return r;
}

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
    case 192: return bwd_launch_d<192>(p, st);
    case 256: return bwd_launch_d<256>(p, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace srat
