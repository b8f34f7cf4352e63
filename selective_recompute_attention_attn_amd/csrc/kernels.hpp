// Launch parameters and launchers shared between the kernels and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace srat {

// ---------------------------------------------------------------- norm region
struct NormFwdParams {
  const void* resid;
  const void* y;
  const float* gamma;
  const float* beta;
  void* h;
  void* u;
  float* mean;
  float* rstd;
  int64_t rows;
  int32_t b;
  int32_t hdim;
  int64_t seq_offset;
  float eps;
  float inv_keep;      // 1 / (1 - p)
  uint32_t thresh;     // 16-bit drop threshold, 0 = no dropout
  uint32_t k0, k1;     // Philox key
  uint32_t tag;        // word 3 of the hidden-dropout counter
};

struct NormBwdParams {
  const void* du;
  const void* dres;
  const void* h;
  const float* gamma;
  const float* mean;
  const float* rstd;
  void* dh;
  void* dy;            // == dh allowed when thresh == 0
  float* dgamma;
  float* dbeta;
  int64_t rows;
  int32_t col_blocks;  // set by the launcher: workgroups summing dgamma / dbeta
  int32_t b;
  int32_t hdim;
  int64_t seq_offset;
  float inv_keep;
  uint32_t thresh, k0, k1, tag;
};

hipError_t launch_norm_fwd(const NormFwdParams& p, bool bf16, bool rms, hipStream_t st);
// largest row count whose backward grid fits the launch limits, for row width hdim
int64_t norm_bwd_max_rows(int64_t hdim);
hipError_t launch_norm_bwd(const NormBwdParams& p, bool bf16, bool rms, hipStream_t st);
hipError_t launch_hidden_mask(const NormFwdParams& p, uint8_t* mask, hipStream_t st);

// ------------------------------------------------------------ attention core
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;       // forward output (read by the backward)
  const float* lse;
  const void* dout;
  void* out;           // forward: O
  float* lse_out;      // forward: LSE
  void* dq;
  void* dk;
  void* dv;
  float* dk_acc;       // fp32 dK partials [slot][b, s, hq, d] (grouped-query heads, split key blocks)
  float* dv_acc;       // ... and dV partials
  float* dq_part;      // fp32 dQ partials [2][b, hq, s, d] of split query tiles
  float* o_part;       // forward: fp32 O / l of the two parts of split query tiles [2][b, hq, s, d]
  float* lse_part;     // forward: their LSEs [2][b, hq, s]
  float* delta;        // [b, hq, s] rowsum(dO * O)
  int64_t sq_b, sq_s, sq_h;
  int64_t sk_b, sk_s, sk_h;
  int64_t sv_b, sv_s, sv_h;
  int64_t so_b, so_s, so_h;
  int32_t b, s, hq, hkv, d;
  int32_t causal;
  float scale;
  float scale_log2;    // scale * log2(e)
  float inv_keep;      // 1 / (1 - p)
  uint32_t thresh;     // 16-bit drop threshold, 0 = no dropout
  uint32_t k0, k1;
  int32_t head_offset;
  const int32_t* seqlens;  // [b] valid lengths of a padded batch, or null (all s)
  int32_t split_qt;    // 128-query tiles whose keys are split over two workgroups (forward, dQ)
  int32_t split_kb;    // backward: 128-key blocks whose queries are split over two dK/dV workgroups
};

// Compute units of the MI355X (gfx950).  An unsplit causal dK/dV grid whose
// workgroups, taking two key blocks each (t and n-1-t: the same work for
// every workgroup), still cover them all runs paired: one dispatch per CU
// and no longest-first tail.
constexpr int kNumCUs = 256;
inline bool attn_pair_tiles(const AttnParams& p, int ntiles, int nsplit) {
  return p.causal && nsplit == 0 && (int64_t)p.b * p.hq * (ntiles / 2) >= kNumCUs;
}

// Work split for grids too small to fill the chip (causal, one workgroup per
// CU): the longest query tiles / key blocks are halved so that no workgroup
// carries much more than half the longest one's work; the halves write fp32
// partials that a final kernel sums (dQ, dK, dV) or merges through the rows'
// LSEs (O).  Depends on the shape only, so workspace queries and launches
// agree.
struct AttnSplit {
  int32_t split_qt;
  int32_t split_kb;
};
AttnSplit attn_grid_split(int64_t b, int64_t s, int64_t hq, int64_t d, bool causal, bool bf16);

// Valid length of batch element bb: seqlens[bb] clamped to [0, s], or s.
// Wave-uniform (bb is), read through the scalar cache.
__device__ __forceinline__ int attn_len(const AttnParams& p, int bb) {
  if (!p.seqlens) return p.s;
  return min(max(p.seqlens[bb], 0), p.s);
}

hipError_t launch_attn_fwd(const AttnParams& p, bool bf16, hipStream_t st);
hipError_t launch_attn_bwd(const AttnParams& p, bool bf16, hipStream_t st);
hipError_t launch_attn_mask(const AttnParams& p, uint8_t* mask, hipStream_t st);

// tracing: records a start event before and a stop event after a launch
struct TraceScope {
  TraceScope(const char* name, hipStream_t st);
  ~TraceScope();
  const char* name_;
  hipStream_t st_;
  void* ev_[2];
};

}  // namespace srat
