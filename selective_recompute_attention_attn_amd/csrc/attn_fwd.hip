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
#include <type_traits>

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

// Two K and two V tiles: while tile t is consumed, tile t+1 (K) / t+1 (V) are
// already resident and the next ones are being written, so one barrier per
// tile suffices.  K is read as 16-byte rows only (RowStride), V through the
// transposing reads (TileStride).
template <int D>
struct alignas(16) FwdSmem {
  static constexpr int kKS = RowStride<D>::kValue;
  static constexpr int kVS = TileStride<D>::kValue;
  bf16 k[2][kBN * kKS];
  bf16 v[2][kBN * kVS];
};
// two workgroups per CU where the registers of the software pipeline allow it
template <int D>
constexpr int fwd_occupancy() { return D <= 96 ? 2 : 1; }

// MFMA row (slot) m of a 32-key block carries key perm32(m): slots
// 8a + 4hh + jj hold keys 16hh + 4a + jj, so output register r of lane half hh
// is key 16hh + r.
__device__ __forceinline__ int perm32(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }
// Inverse of perm32: the MFMA slot of key k of a 32-key block.  K rows are
// stored in LDS in slot order, so the A-operand reads are consecutive rows.
__device__ __forceinline__ int slot32(int k) { return 8 * ((k >> 2) & 3) + 4 * (k >> 4) + (k & 3); }

// Causal q-tile order.  Two workgroups per CU: the first half of the grid
// runs the longest tiles first, the second half the shortest first, so two
// workgroups that share a CU (block i and block i + grid/2) carry equal work.
// One workgroup per CU: longest first throughout; each CU that frees up takes
// the longest tile left (longest-processing-time-first scheduling), which
// evens the CUs' totals (the paired order leaves the CUs that start with the
// shortest of the long tiles to collect the short ones one by one: at
// llama3-70b-t8 a makespan of ~97 tile-steps per CU against ~75).
template <bool PAIRED>
__device__ __forceinline__ int causal_tile(int rank, int nqt) {
  if (!PAIRED) return nqt - 1 - rank;
  const int h = (nqt + 1) / 2;
  return rank < h ? nqt - 1 - rank : rank - h;
}

template <bool B>
using bool_c = std::integral_constant<bool, B>;

// configurations whose forward grid may be split (one workgroup per CU:
// d >= 128; causal); elsewhere the split code compiles away
template <int D, bool CAUSAL>
constexpr bool kSplitFwd = CAUSAL && fwd_occupancy<D>() == 1;

// Loop structure (tile t = keys 64t .. 64t+63), software-pipelined by one
// tile inside each wave:
//   barrier; write K[t+2], V[t+1] (fetched from global memory during tile t-1)
//   into the free buffers; start the global loads of K[t+3], V[t+2];
//   row max of S[t] (computed during tile t-1), rare rescale;
//   issue the MFMAs of S[t+1] = K[t+1] Q^T   || exp / row sum / dropout of S[t]
//   issue the MFMAs of O^T += V[t]^T P[t]^T  || Philox draws for tile t+1
// so the matrix cores and the vector ALUs of a wave work on different tiles.
// VARLEN: per-element valid lengths (padded batch); compiled separately so
// that the plain kernels keep their code.
template <int D, bool CAUSAL, bool DROP, bool VARLEN>
__global__ __launch_bounds__(kThreads, fwd_occupancy<D>()) void attn_fwd_bf16_kernel(AttnParams p) {
  constexpr int kKS = FwdSmem<D>::kKS;
  constexpr int kVS = FwdSmem<D>::kVS;
  constexpr int kDC = D / 16;        // 16-wide d chunks (QK^T k-steps)
  constexpr int kDB = D / 32;        // 32-wide d blocks of O^T
  constexpr int kLoads = D / 32;     // 16-byte global loads per thread per tile (each of K, V)
  constexpr bool kPreV = D >= 128 && D <= 192;   // V^T operands read one phase early (registers allow it)
  __shared__ FwdSmem<D> sm;

  const int nqt = (p.s + kBM - 1) / kBM;
  const int nbh = p.b * p.hq;
  const int bh = blockIdx.x % nbh;
  const int rank = (int)(blockIdx.x / nbh);
  // Split grids (p.split_qt > 0: causal, d >= 128, a workspace given): the
  // split_qt longest tiles run as two workgroups each (part 0: the first
  // half of the tile's key tiles, part 1: the rest); all workgroups are
  // launched in decreasing order of work.
  const int nsq = kSplitFwd<D, CAUSAL> ? p.split_qt : 0;
  int qt, part = -1;
  if (nsq > 0) {
    split_order(rank, nqt, nsq, qt, part);
  } else {
    qt = CAUSAL ? causal_tile<fwd_occupancy<D>() == 2>(rank, nqt) : rank;
  }
  const int hh_q = bh % p.hq;
  const int bb = bh / p.hq;
  const int g = hh_q / (p.hq / p.hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps tile bounds scalar
  const int half = lane >> 5, col = lane & 31;
  const int q0 = qt * kBM;
  const int qw = q0 + 32 * wv;           // first query of this wave
  const int qi = qw + col;               // this lane's query
  const int sl = VARLEN ? attn_len(p, bb) : p.s;   // valid length of this batch element

  const bf16* qp = static_cast<const bf16*>(p.q) + bb * p.sq_b + hh_q * p.sq_h;
  const bf16* kp = static_cast<const bf16*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const bf16* vp = static_cast<const bf16*>(p.v) + bb * p.sv_b + g * p.sv_h;

  // a tile past the valid length (padded batch): O = 0, LSE = -inf (a split
  // tile's parts: O / l = 0, LSE = -inf, which the merge turns into the same)
  if (VARLEN && q0 >= sl) {
    if (qi < p.s) {
      const int64_t row = ((int64_t)bb * p.hq + hh_q) * p.s + qi;
      if (part >= 0) {
        const int64_t prow = (int64_t)part * p.b * p.hq * p.s + row;
#pragma unroll
        for (int j = 0; j < D / 4; ++j)
          if (j % 2 == half) *reinterpret_cast<float4*>(p.o_part + prow * D + 4 * j) = make_float4(0.f, 0.f, 0.f, 0.f);
        if (half == 0) p.lse_part[prow] = -INFINITY;
      } else {
        bf16* op = static_cast<bf16*>(p.out) + bb * p.so_b + (int64_t)qi * p.so_s + hh_q * p.so_h;
#pragma unroll
        for (int c = 0; c < D / 8; ++c)
          if (c % 2 == half) *reinterpret_cast<uint4*>(op + 8 * c) = make_uint4(0, 0, 0, 0);
        if (half == 0) p.lse_out[row] = -INFINITY;
      }
    }
    return;
  }

  // Q^T B operand: lane (col, half) holds Q[qi][16c + 8*half .. +7]
  bf16x8 qreg[kDC];
#pragma unroll
  for (int c = 0; c < kDC; ++c) qreg[c] = bf16x8{};
  if (qi < sl) {
#pragma unroll
    for (int c = 0; c < kDC; ++c)
      qreg[c] = *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.sq_s + 16 * c + 8 * half);
  }

  f32x16 oacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) oacc[db] = f32x16{};
  float m_use = -INFINITY;   // running max, log2-scaled units
  float l_run = 0.f;         // lane-partial row sum (this lane's keys)

  const int nkt_all = (sl + kBN - 1) / kBN;
  const int nkt_q = CAUSAL ? min(nkt_all, (q0 + kBM + kBN - 1) / kBN) : nkt_all;
  // key tiles [kt_lo, nkt) of this workgroup
  const int kt_mid = (nkt_q + 1) / 2;
  const int kt_lo = part == 1 ? kt_mid : 0;
  const int nkt = part == 0 ? kt_mid : nkt_q;
  // tiles 0 .. n_int-1 need no masking for any query of this wave
  const int n_int = CAUSAL ? min(sl / kBN, (qw + 1) / kBN) : sl / kBN;
  // keys at or beyond key_lim are masked for this lane's query
  const int key_lim = CAUSAL ? min(sl, qi + 1) : sl;

  // ---- global <-> LDS staging; chunk x = tid + 256*it of a 64 x D tile.
  // Buffer loads: the tile's base and its valid byte count are scalars, keys
  // at or beyond s read as zero, each chunk has a fixed 32-bit offset.
  uint4 kpre[kLoads], vpre[kLoads];
  uint32_t koff[kLoads], voff[kLoads];
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int x = tid + kThreads * it;
    koff[it] = (uint32_t)(((int64_t)(x / (D / 8)) * p.sk_s + 8 * (x % (D / 8))) * 2);
    voff[it] = (uint32_t)(((int64_t)(x / (D / 8)) * p.sv_s + 8 * (x % (D / 8))) * 2);
  }
  auto tile_bytes = [&](int kt, int64_t stride) -> uint32_t {
    const int rows = min(kBN, max(0, sl - kt * kBN));
    return (uint32_t)((int64_t)rows * stride * 2);
  };
  auto load_k = [&](int kt) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(kp + (int64_t)kt * kBN * p.sk_s, tile_bytes(kt, p.sk_s));
#pragma unroll
    for (int it = 0; it < kLoads; ++it) kpre[it] = buffer_load16(r, koff[it]);
  };
  auto load_v = [&](int kt) {
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(vp + (int64_t)kt * kBN * p.sv_s, tile_bytes(kt, p.sv_s));
#pragma unroll
    for (int it = 0; it < kLoads; ++it) vpre[it] = buffer_load16(r, voff[it]);
  };
  auto stash_k = [&](int buf) {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int x = tid + kThreads * it;
      const int r = x / (D / 8), c8 = x % (D / 8);
      *reinterpret_cast<uint4*>(&sm.k[buf][((r & ~31) | slot32(r & 31)) * kKS + 8 * c8]) = kpre[it];
    }
  };
  auto stash_v = [&](int buf) {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      const int x = tid + kThreads * it;
      const int r = x / (D / 8), c8 = x % (D / 8);
      *reinterpret_cast<uint4*>(&sm.v[buf][r * kVS + 8 * c8]) = vpre[it];
    }
  };

  const int krow = col * kKS + 8 * half;   // K tile rows are in slot order
  const int grp = lane >> 4, lg = lane & 15;
  const int vrow = (16 * (grp >> 1) + (lg >> 2)) * kVS + 16 * (grp & 1) + 4 * (lg & 3);
  // V^T A operand of PV step c (keys 32(c/2) + 8(c%2) ..), d block db, from a
  // row-major V tile through two transposing reads
  auto v_operand = [&](const bf16* vb, int c, int db) -> bf16x8 {
    const int r0 = (32 * (c >> 1) + 8 * (c & 1)) * kVS + vrow;
    const s16x4 lo = lds_read_tr16(&vb[r0 + 32 * db]);
    const s16x4 hi = lds_read_tr16(&vb[r0 + 4 * kVS + 32 * db]);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T = K Q^T (raw scores) of the tile in K buffer `buf`, two 32-key blocks
  auto qk = [&](int buf, f32x16 (&s)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < kDC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.k[buf][32 * kb * kKS + krow + 16 * c]);
        s[kb] = mfma32(a, qreg[c], s[kb]);
      }
  };

  // Philox words of tile kt for this lane: call (kb, gh) covers keys
  // 64kt + 32kb + 16half + 8gh .. +7 of query qi
  const uint32_t hg = (uint32_t)(p.head_offset + hh_q);
  const PhiloxRow prow = philox_row((uint32_t)qi, hg, (uint32_t)bb, p.k0, p.k1);
  auto draws = [&](int kt, uint32_t (&w)[16]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int gh = 0; gh < 2; ++gh) {
        const uint32_t grp8 = (uint32_t)((kt * kBN + 32 * kb + 16 * half + 8 * gh) >> 3);
        const Philox4 rnd = philox4x32_10_row(grp8, prow);
#pragma unroll
        for (int j = 0; j < 4; ++j) w[8 * kb + 4 * gh + j] = rnd.w[j];
      }
  };

  const uint32_t tm1 = (p.thresh - 1u) * 0x10001u;   // T - 1 in both halves (T >= 1 when DROP)
  const float c2 = p.scale_log2;

  // one tile: MASK = causal / tail masking needed, NEXT = tile kt+1 exists
  f32x16 scur[2];
  uint32_t wcur[16];
  auto tile = [&](int kt, auto mask_c, auto next_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    constexpr bool NEXT = decltype(next_c)::value;
    const int key0 = kt * kBN;
    __syncthreads();
    if (NEXT) {
      stash_k(kt & 1);            // K[kt+2] over K[kt] (read during tile kt-1)
      stash_v((kt + 1) & 1);      // V[kt+1] over V[kt-1]
      load_k(kt + 3);
      load_v(kt + 2);
    }
    // ---- mask, row max (raw units; the scale is positive)
    if (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb + 16 * half + r;
          scur[kb][r] = key >= key_lim ? -INFINITY : scur[kb][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[kb][r]);
    mx = halves_max(mx) * c2;
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
    // phases are kept apart (sched_barrier) so that the scheduler interleaves
    // matrix and vector work inside each phase without hoisting the next
    // phase's LDS reads (and their registers) into it; explicit interleave
    // patterns inside the phases measured slower than the scheduler's own
    __builtin_amdgcn_sched_barrier(0);

    // ---- next tile's scores on the matrix cores
    f32x16 snext[2];
    if (NEXT) qk((kt + 1) & 1, snext);
    // with one wave per SIMD nothing else hides the LDS latency of the V^T
    // operands, so they are read here, behind the exp work of this phase
    bf16x8 vop[kPreV ? 4 : 1][kPreV ? kDB : 1];
    if (kPreV) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int db = 0; db < kDB; ++db) vop[c][db] = v_operand(sm.v[kt & 1], c, db);
    }

    // ---- p = exp2(s * c - m), row sum of the undropped values, dropout
    // (1/(1-p) is applied in the epilogue), P^T as bf16 B operands
    float lsum = 0.f;
    uint32_t pw[16];           // P^T pairs: keys 16half + r, r+1 of block kb -> pw[8kb + r/2]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(scur[kb][r], c2, -msub));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(scur[kb][r + 1], c2, -msub));
        lsum += e0;
        lsum += e1;
        uint32_t pk = pack_bf16x2(e0, e1);
        if (DROP) {   // zero the dropped halves of the packed pair
          const uint32_t w = wcur[8 * kb + (r >> 1)];
          pk = drop_pair(pk, w, tm1);
        }
        pw[8 * kb + (r >> 1)] = pk;
      }
    l_run += lsum;
    bf16x8 pop[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      pop[c] = __builtin_bit_cast(bf16x8, make_uint4(pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]));
    __builtin_amdgcn_sched_barrier(0);

    // ---- O^T += V^T P^T; V^T operand via LDS transpose reads:
    // lane group G = lane/16 covers d = 32db + 16*(G%2) + (0..15) and the keys
    // 32*kb + 16*(G/2) + 8*c' + (0..7) of step c = 2*kb + c'.
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        oacc[db] = mfma32(kPreV ? vop[c][db] : v_operand(sm.v[kt & 1], c, db), pop[c], oacc[db]);
    if (NEXT) {
      if (DROP) draws(kt + 1, wcur);
      scur[0] = snext[0];
      scur[1] = snext[1];
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- prologue: K[kt_lo], K[kt_lo+1], V[kt_lo] resident, S[kt_lo] and its
  // draws computed, K[kt_lo+2] and V[kt_lo+1] in flight
  load_k(kt_lo);
  load_v(kt_lo);
  stash_k(kt_lo & 1);
  stash_v(kt_lo & 1);
  load_k(kt_lo + 1);
  stash_k((kt_lo + 1) & 1);
  __syncthreads();
  load_k(kt_lo + 2);
  load_v(kt_lo + 1);
  qk(kt_lo & 1, scur);
  if (DROP) draws(kt_lo, wcur);

  // separate loops (not one loop switching between tile variants): each loop
  // body is one straight-line variant, which keeps register allocation tight
  int kt = kt_lo;
  for (; kt < min(n_int, nkt - 1); ++kt) tile(kt, bool_c<false>{}, bool_c<true>{});
  for (; kt < nkt - 1; ++kt) tile(kt, bool_c<true>{}, bool_c<true>{});
  if (kt < n_int) tile(kt, bool_c<false>{}, bool_c<false>{});
  else tile(kt, bool_c<true>{}, bool_c<false>{});

  // ---- epilogue: O = O^T / l * 1/(1-p), LSE in natural log
  const float l_tot = halves_sum(l_run);
  if (part >= 0) {   // a split tile's part: O / l (fp32) and its LSE, merged later
    if (qi < p.s) {
      const int64_t row = (int64_t)part * p.b * p.hq * p.s + ((int64_t)bb * p.hq + hh_q) * p.s + qi;
      // a row can have no visible key in one part (the first tile's early
      // rows in part 1): O = 0 and LSE = -inf give it zero weight in the merge
      const bool any = l_tot > 0.f && (!VARLEN || qi < sl);
      const float inv = any ? 1.0f / l_tot : 0.f;
      float* dst = p.o_part + row * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<float4*>(dst + 32 * db + 8 * a + 4 * half) =
              make_float4(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv, oacc[db][4 * a + 2] * inv,
                          oacc[db][4 * a + 3] * inv);
      if (half == 0) p.lse_part[row] = any ? (m_use + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
  if (qi < p.s) {
    const bool valid = !VARLEN || qi < sl;   // rows past the valid length: O = 0, LSE = -inf
    const float inv = valid ? p.inv_keep / l_tot : 0.f;
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
    if (half == 0)
      p.lse_out[((int64_t)bb * p.hq + hh_q) * p.s + qi] = valid ? (m_use + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- ping-pong
// The same forward with two waves on every SIMD, paired so that one wave's
// softmax (VALU) runs while the other's matrix products (MFMA) run.
//
// A workgroup has 8 waves in two groups of 4 over the same 128 queries (wave
// w of either group owns queries 32w .. 32w+31).  Group g takes the key tiles
// kt_lo + 2j + g (j = 0, 1, ...): each group keeps its own running max, row
// sum and O accumulator, and the two are merged through LDS at the end (the
// same exact combination as a split tile's merge).
//
// Each group alternates two barrier-separated phases per tile:
//   M(j): O^T += V[j-1]^T P[j-1]^T  and  S[j]^T = K[j] Q^T   (MFMA)
//   V(j): stage the group's next K/V tile into LDS, start the loads of the one
//         after; row max, rare rescale, exp, row sum, dropout, pack P[j] (VALU)
// and group 1 runs one phase behind group 0, so that in every interval between
// two barriers one group issues MFMAs and the other VALU work.  Row sums are
// taken from the packed bf16 probabilities with v_dot2c_f32_bf16 (two per
// instruction), the values the PV product uses.
template <int D>
struct alignas(16) FwdPPSmem {
  static constexpr int kKS = RowStride<D>::kValue;
  static constexpr int kVS = TileStride<D>::kValue;
  union {
    struct {
      bf16 k[2][2][kBN * kKS];   // [group][buffer]: K rows in slot order
      bf16 v[2][2][kBN * kVS];   // V rows (read transposed)
    } t;
    struct {                     // group 1's state handed to group 0
      float o[4][(D / 32) * 16][64];
      float m[4][64];
      float l[4][64];
    } x;
  };
};

__device__ __forceinline__ float dot2_sum(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                         __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
}

template <int D, bool CAUSAL, bool DROP, bool VARLEN>
__global__ __launch_bounds__(512, 1) void attn_fwd_pp_kernel(AttnParams p) {
  using SM = FwdPPSmem<D>;
  constexpr int kKS = SM::kKS;
  constexpr int kVS = SM::kVS;
  constexpr int kDC = D / 16;
  constexpr int kDB = D / 32;
  __shared__ SM sm;

  const int nqt = (p.s + kBM - 1) / kBM;
  const int nbh = p.b * p.hq;
  const int bh = blockIdx.x % nbh;
  const int rank = (int)(blockIdx.x / nbh);
  const int nsq = kSplitFwd<D, CAUSAL> ? p.split_qt : 0;
  int qt, part = -1;
  if (nsq > 0) {
    split_order(rank, nqt, nsq, qt, part);
  } else {
    qt = CAUSAL ? causal_tile<false>(rank, nqt) : rank;
  }
  const int hh_q = bh % p.hq;
  const int bb = bh / p.hq;
  const int g = hh_q / (p.hq / p.hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps tile bounds scalar
  const int grp = wv >> 2, wq = wv & 3;                       // key group, query block
  const int half = lane >> 5, col = lane & 31;
  const int q0 = qt * kBM;
  const int qw = q0 + 32 * wq;
  const int qi = qw + col;
  const int sl = VARLEN ? attn_len(p, bb) : p.s;

  const bf16* qp = static_cast<const bf16*>(p.q) + bb * p.sq_b + hh_q * p.sq_h;
  const bf16* kp = static_cast<const bf16*>(p.k) + bb * p.sk_b + g * p.sk_h;
  const bf16* vp = static_cast<const bf16*>(p.v) + bb * p.sv_b + g * p.sv_h;

  if (VARLEN && q0 >= sl) {   // a tile past the valid length: O = 0, LSE = -inf
    if (grp == 0 && qi < p.s) {
      const int64_t row = ((int64_t)bb * p.hq + hh_q) * p.s + qi;
      if (part >= 0) {
        const int64_t prow = (int64_t)part * p.b * p.hq * p.s + row;
#pragma unroll
        for (int j = 0; j < D / 4; ++j)
          if (j % 2 == half) *reinterpret_cast<float4*>(p.o_part + prow * D + 4 * j) = make_float4(0.f, 0.f, 0.f, 0.f);
        if (half == 0) p.lse_part[prow] = -INFINITY;
      } else {
        bf16* op = static_cast<bf16*>(p.out) + bb * p.so_b + (int64_t)qi * p.so_s + hh_q * p.so_h;
#pragma unroll
        for (int c = 0; c < D / 8; ++c)
          if (c % 2 == half) *reinterpret_cast<uint4*>(op + 8 * c) = make_uint4(0, 0, 0, 0);
        if (half == 0) p.lse_out[row] = -INFINITY;
      }
    }
    return;
  }

  bf16x8 qreg[kDC];
#pragma unroll
  for (int c = 0; c < kDC; ++c) qreg[c] = bf16x8{};
  if (qi < sl) {
#pragma unroll
    for (int c = 0; c < kDC; ++c)
      qreg[c] = *reinterpret_cast<const bf16x8*>(qp + (int64_t)qi * p.sq_s + 16 * c + 8 * half);
  }
  // consumed here, so the compiler waits for these loads now and does not
  // guard their later uses with waits that would also drain the tile loads
#pragma unroll
  for (int c = 0; c < kDC; ++c) asm volatile("" ::"v"(qreg[c]));

  f32x16 oacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db) oacc[db] = f32x16{};
  float m_use = -INFINITY;
  float l_run = 0.f;

  const int nkt_all = (sl + kBN - 1) / kBN;
  const int nkt_q = CAUSAL ? min(nkt_all, (q0 + kBM + kBN - 1) / kBN) : nkt_all;
  const int kt_mid = (nkt_q + 1) / 2;
  const int kt_lo = part == 1 ? kt_mid : 0;
  const int nkt = part == 0 ? kt_mid : nkt_q;
  const int nsteps = (nkt - kt_lo + 1) / 2;                       // steps of both groups
  const int n_int = CAUSAL ? min(sl / kBN, (qw + 1) / kBN) : sl / kBN;
  const int key_lim = CAUSAL ? min(sl, qi + 1) : sl;
  auto tile_of = [&](int j) { return kt_lo + 2 * j + grp; };

  // ---- staging: buffer -> LDS loads.  One instruction fills 1 KB of LDS
  // (lane l the bytes 16l .. 16l+15) from per-lane global offsets chosen so
  // that the block lands in the padded layouts -- K rows in slot order, V
  // rows in order -- without passing through registers; padding bytes are
  // loaded from past the buffer's end, which reads zero.  The 4 waves of a
  // group share a tile's blocks (wave w: blocks w, w+4, ...).
  constexpr int kKBytes = kBN * kKS * 2, kVBytes = kBN * kVS * 2;
  constexpr int kKBlocks = kKBytes / 1024, kVBlocks = kVBytes / 1024;
  static_assert(kKBytes % 1024 == 0 && kVBytes % 1024 == 0, "tiles must be whole 1 KB blocks");
  constexpr int kKPer = (kKBlocks + 3) / 4, kVPer = (kVBlocks + 3) / 4;   // blocks of wave 0
  // the loads wave w issues per phase: the wait at the end of a VALU phase
  // leaves exactly those (its most recent) in flight and completes the rest
  auto wait_recent = [&] {
    wait_vmcnt_by_wave<blocks_of_wave(kKBlocks, 0) + blocks_of_wave(kVBlocks, 0),
                       blocks_of_wave(kKBlocks, 1) + blocks_of_wave(kVBlocks, 1),
                       blocks_of_wave(kKBlocks, 2) + blocks_of_wave(kVBlocks, 2),
                       blocks_of_wave(kKBlocks, 3) + blocks_of_wave(kVBlocks, 3)>(wq);
  };
  uint32_t kdo[kKPer], vdo[kVPer];
#pragma unroll
  for (int i = 0; i < kKPer; ++i) {
    const int pos = 1024 * (wq + 4 * i) + 16 * lane;
    const int row = pos / (2 * kKS), cb = pos % (2 * kKS);
    const int key = (row & ~31) | perm32(row & 31);
    kdo[i] = (row < kBN && cb < 2 * D) ? (uint32_t)((int64_t)key * p.sk_s * 2 + cb) : 0xFFFFFFF0u;
  }
#pragma unroll
  for (int i = 0; i < kVPer; ++i) {
    const int pos = 1024 * (wq + 4 * i) + 16 * lane;
    const int row = pos / (2 * kVS), cb = pos % (2 * kVS);
    vdo[i] = (row < kBN && cb < 2 * D) ? (uint32_t)((int64_t)row * p.sv_s * 2 + cb) : 0xFFFFFFF0u;
  }
  auto tile_bytes = [&](int kt, int64_t stride) -> uint32_t {
    const int rows = kt < nkt ? min(kBN, max(0, sl - kt * kBN)) : 0;
    return (uint32_t)((int64_t)rows * stride * 2);
  };
  auto dma_k = [&](int kt, int buf) {
    const sgpr4 rk = buffer_rsrc_sgpr(kp + (int64_t)kt * kBN * p.sk_s, tile_bytes(kt, p.sk_s));
    const uintptr_t base = (uintptr_t)&sm.t.k[grp][buf][0];
#pragma unroll
    for (int i = 0; i < kKPer; ++i)
      if (wq + 4 * i < kKBlocks) buffer_load16_lds(rk, base + 1024 * (wq + 4 * i), kdo[i]);
  };
  auto dma_v = [&](int kt, int buf) {
    const sgpr4 rv = buffer_rsrc_sgpr(vp + (int64_t)kt * kBN * p.sv_s, tile_bytes(kt, p.sv_s));
    const uintptr_t base = (uintptr_t)&sm.t.v[grp][buf][0];
#pragma unroll
    for (int i = 0; i < kVPer; ++i)
      if (wq + 4 * i < kVBlocks) buffer_load16_lds(rv, base + 1024 * (wq + 4 * i), vdo[i]);
  };

  const int krow = col * kKS + 8 * half;
  const int lgp = lane >> 4, lg = lane & 15;
  const int vrow = (16 * (lgp >> 1) + (lg >> 2)) * kVS + 16 * (lgp & 1) + 4 * (lg & 3);
  auto v_operand = [&](const bf16* vb, int c, int db) -> bf16x8 {
    const int r0 = (32 * (c >> 1) + 8 * (c & 1)) * kVS + vrow;
    const s16x4 lo = lds_read_tr16(&vb[r0 + 32 * db]);
    const s16x4 hi = lds_read_tr16(&vb[r0 + 4 * kVS + 32 * db]);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  const uint32_t hg = (uint32_t)(p.head_offset + hh_q);
  const PhiloxRow prow = philox_row((uint32_t)qi, hg, (uint32_t)bb, p.k0, p.k1);
  const uint32_t tm1 = (p.thresh - 1u) * 0x10001u;
  const float c2 = p.scale_log2;

  f32x16 s[2];        // S^T of the current tile (raw scores)
  uint32_t pw[16];    // P^T of the previous tile, packed bf16 pairs

  // M phase of step j: PV of step j-1 (if it had a tile), QK^T of step j
  auto phase_m = [&](int j, bool pv, bool qk) {
    if (pv) {
      const bf16* vb = sm.t.v[grp][(j - 1) & 1];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bf16x8 pop =
            __builtin_bit_cast(bf16x8, make_uint4(pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]));
#pragma unroll
        for (int db = 0; db < kDB; ++db) oacc[db] = mfma32(v_operand(vb, c, db), pop, oacc[db]);
      }
    }
    if (qk) {
      const bf16* kb_ = sm.t.k[grp][j & 1];
      s[0] = s[1] = f32x16{};
#pragma unroll
      for (int c = 0; c < kDC; ++c)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(&kb_[32 * kb * kKS + krow + 16 * c]), qreg[c], s[kb]);
    }
  };

  // V phase of step j: stage the group's tile of step j+1, load step j+2;
  // softmax of step j's scores into pw (MASK: causal / tail masking needed)
  // loads issued here: V of step j+1 (its buffer's tile was last read by
  // PV(j-1) in M(j)) and K of step j+2 (its buffer's tile by QK(j) in M(j));
  // the wait at the end of the phase completes those of V(j-1): K of step
  // j+1 and V of step j, which M(j+1) reads
  auto phase_v = [&](int j, bool have, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    dma_v(tile_of(j + 1), (j + 1) & 1);
    dma_k(tile_of(j + 2), j & 1);
    if (!have) return;
    const int key0 = tile_of(j) * kBN;
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
    if (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb + 16 * half + r;
          s[kb][r] = key >= key_lim ? -INFINITY : s[kb][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = halves_max(mx) * c2;
    const bool grow = mx > m_use + kMaxSlack;
    if (__any(grow)) {
      const float m_new = grow ? mx : m_use;
      const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; ++db) oacc[db] *= alpha;
      m_use = m_new;
    }
    const float msub = (m_use == -INFINITY) ? 0.f : m_use;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -msub));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], c2, -msub));
        uint32_t pk = pack_bf16x2(e0, e1);
        l_run = dot2_sum(pk, l_run);
        if (DROP) pk = drop_pair(pk, w[8 * kb + (r >> 1)], tm1);
        pw[8 * kb + (r >> 1)] = pk;
      }
  };

  // ---- prologue: K of step 0 resident; V of step 0 and K of step 1 in flight
  dma_k(tile_of(0), 0);
  dma_v(tile_of(0), 0);
  dma_k(tile_of(1), 1);
  wait_recent();
  __syncthreads();
  if (grp == 1) __syncthreads();   // group 1 runs one phase behind

  // steps whose tile needs no masking for this wave: tile_of(j) < n_int
  const int j_int = max(0, min(nsteps, (min(n_int, nkt) - kt_lo - grp + 1) / 2));
  int j = 0;
  // Inside the loop the barriers are bare (lds_barrier): a __syncthreads
  // would also wait for every load in flight, the prefetched tiles included.
  // Each wave instead completes its own LDS reads (lgkmcnt) and, at the end
  // of a VALU phase, the loads the next MFMA phase reads (wait_vmcnt).
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

  // ---- merge group 1 into group 0 (both over the same queries)
  l_run = halves_sum(l_run);
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.x.o[wq][db * 16 + r][lane] = oacc[db][r];
    sm.x.m[wq][lane] = m_use;
    sm.x.l[wq][lane] = l_run;
  }
  __syncthreads();
  if (grp == 1) return;
  {
    const float m1 = sm.x.m[wq][lane], l1 = sm.x.l[wq][lane];
    const float mm = fmaxf(m_use, m1);
    const float a0 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_use - mm);
    const float a1 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = oacc[db][r] * a0 + sm.x.o[wq][db * 16 + r][lane] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_use = mm;
  }

  // ---- epilogue (as the one-group kernel): O = O^T / l * 1/(1-p), LSE
  const float l_tot = l_run;
  if (part >= 0) {
    if (qi < p.s) {
      const int64_t row = (int64_t)part * p.b * p.hq * p.s + ((int64_t)bb * p.hq + hh_q) * p.s + qi;
      const bool any = l_tot > 0.f && (!VARLEN || qi < sl);
      const float inv = any ? 1.0f / l_tot : 0.f;
      float* dst = p.o_part + row * D;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<float4*>(dst + 32 * db + 8 * a + 4 * half) =
              make_float4(oacc[db][4 * a] * inv, oacc[db][4 * a + 1] * inv, oacc[db][4 * a + 2] * inv,
                          oacc[db][4 * a + 3] * inv);
      if (half == 0) p.lse_part[row] = any ? (m_use + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
  if (qi < p.s) {
    const bool valid = !VARLEN || qi < sl;
    const float inv = valid ? p.inv_keep / l_tot : 0.f;
    bf16* op = static_cast<bf16*>(p.out) + bb * p.so_b + (int64_t)qi * p.so_s + hh_q * p.so_h;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint2 w2;
        w2.x = pack_bf16x2(oacc[db][4 * a + 0] * inv, oacc[db][4 * a + 1] * inv);
        w2.y = pack_bf16x2(oacc[db][4 * a + 2] * inv, oacc[db][4 * a + 3] * inv);
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * a + 4 * half) = w2;
      }
    }
    if (half == 0)
      p.lse_out[((int64_t)bb * p.hq + hh_q) * p.s + qi] = valid ? (m_use + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Merge of the two parts of a split tile's rows (from q_lo): LSE =
// log(e^LSE0 + e^LSE1), O = (e^(LSE0-LSE) O0 + e^(LSE1-LSE) O1) / (1-p).
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_merge_kernel(AttnParams p, int q_lo) {
  const int nrows = p.s - q_lo;
  const int64_t n = (int64_t)p.b * p.hq * nrows * (D / 8);
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= n) return;
  const int c8 = (int)(x % (D / 8));
  const int64_t r = x / (D / 8);                             // (b, hq, query)
  const int qi = q_lo + (int)(r % nrows);
  const int64_t bh = r / nrows;
  const int hh = (int)(bh % p.hq), bb = (int)(bh / p.hq);
  const int64_t row = bh * p.s + qi;
  const int64_t part_rows = (int64_t)p.b * p.hq * p.s;
  const float l0 = p.lse_part[row], l1 = p.lse_part[part_rows + row];
  const float mx = fmaxf(l0, l1);
  const bool none = mx == -INFINITY;     // a padded row: no visible key in either part
  const float lse = none ? -INFINITY : mx + log1pf(__expf(fminf(l0, l1) - mx));
  const float w0 = none ? 0.f : __expf(l0 - lse) * p.inv_keep;
  const float w1 = none ? 0.f : __expf(l1 - lse) * p.inv_keep;
  const float* s0 = p.o_part + row * D + 8 * c8;
  const float* s1 = s0 + part_rows * D;
  const float4 a0 = reinterpret_cast<const float4*>(s0)[0], b0 = reinterpret_cast<const float4*>(s0)[1];
  const float4 a1 = reinterpret_cast<const float4*>(s1)[0], b1 = reinterpret_cast<const float4*>(s1)[1];
  uint4 w;
  w.x = pack_bf16x2(w0 * a0.x + w1 * a1.x, w0 * a0.y + w1 * a1.y);
  w.y = pack_bf16x2(w0 * a0.z + w1 * a1.z, w0 * a0.w + w1 * a1.w);
  w.z = pack_bf16x2(w0 * b0.x + w1 * b1.x, w0 * b0.y + w1 * b1.y);
  w.w = pack_bf16x2(w0 * b0.z + w1 * b1.z, w0 * b0.w + w1 * b1.w);
  bf16* dst = static_cast<bf16*>(p.out) + bb * p.so_b + (int64_t)qi * p.so_s + hh * p.so_h;
  *reinterpret_cast<uint4*>(dst + 8 * c8) = w;
  if (c8 == 0) p.lse_out[row] = lse;
}

// head dims whose forward runs as the ping-pong kernel (8 waves)
template <int D>
constexpr bool kFwdPingPong = D == 128;

template <int D, bool VARLEN>
hipError_t fwd_launch_v(const AttnParams& p, hipStream_t st) {
  const int nqt = (p.s + kBM - 1) / kBM;
  const dim3 grid((unsigned)((nqt + p.split_qt) * p.hq * p.b));
  const bool drop = p.thresh != 0;
  {
    TraceScope ts("attn_fwd_bf16", st);
    if constexpr (kFwdPingPong<D>) {
      if (p.causal) {
        if (drop) attn_fwd_pp_kernel<D, true, true, VARLEN><<<grid, 512, 0, st>>>(p);
        else attn_fwd_pp_kernel<D, true, false, VARLEN><<<grid, 512, 0, st>>>(p);
      } else {
        if (drop) attn_fwd_pp_kernel<D, false, true, VARLEN><<<grid, 512, 0, st>>>(p);
        else attn_fwd_pp_kernel<D, false, false, VARLEN><<<grid, 512, 0, st>>>(p);
      }
    } else if (p.causal) {
      if (drop) attn_fwd_bf16_kernel<D, true, true, VARLEN><<<grid, kThreads, 0, st>>>(p);
      else attn_fwd_bf16_kernel<D, true, false, VARLEN><<<grid, kThreads, 0, st>>>(p);
    } else {
      if (drop) attn_fwd_bf16_kernel<D, false, true, VARLEN><<<grid, kThreads, 0, st>>>(p);
      else attn_fwd_bf16_kernel<D, false, false, VARLEN><<<grid, kThreads, 0, st>>>(p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.split_qt == 0) return e;
  }
  TraceScope ts("attn_fwd_merge", st);
  const int q_lo = (nqt - p.split_qt) * kBM;
  const int64_t n = (int64_t)p.b * p.hq * (p.s - q_lo) * (D / 8);
  attn_fwd_merge_kernel<D><<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, q_lo);
  return hipGetLastError();
}

template <int D>
hipError_t fwd_launch_d(const AttnParams& p, hipStream_t st) {
  return p.seqlens ? fwd_launch_v<D, true>(p, st) : fwd_launch_v<D, false>(p, st);
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
    case 192: return fwd_launch_d<192>(p, st);
    case 256: return fwd_launch_d<256>(p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_mask(const AttnParams& p, uint8_t* mask, hipStream_t st) {
  if (p.s == 0 || p.b == 0) return hipSuccess;
  attn_mask_kernel<<<dim3(p.s, p.hq, p.b), 64, 0, st>>>(p, mask);
  return hipGetLastError();
}

}  // namespace srat
