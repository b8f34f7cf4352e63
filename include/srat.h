/*
 * srat.h -- C ABI of libsrat: the selective-recompute attention core and the
 * sequence-parallel norm region, hand-written HIP for AMD MI355X (gfx950).
 *
 * What the calls compute.
 *
 * The attention core O = dropout(softmax(Q K^T * scale)) V is the part of a
 * transformer layer that selective activation recomputation does not store:
 * its activations (scores, softmax, dropout mask and output, 5as^2b bytes per
 * layer) are large while its FLOPs are few, so the backward pass recomputes it
 * ("Reducing Activation Recomputation in Large Transformer Models", LIT-736
 * record, Key takeaways bullet 4; "Recomputing Activations" plate, second
 * paragraph and the per-token formula under "What you will learn").
 * srat_attn_core_fwd keeps only O and the per-row logsumexp; srat_attn_core_bwd
 * recomputes Q K^T, the softmax and the dropout mask tile by tile (the tiling of
 * FlashAttention as the METP page describes it, Introduction, third paragraph),
 * so no s x s tensor is ever written to memory.
 *
 * The norm region is what tensor parallelism leaves replicated -- the layer
 * norm and the dropout (+ residual) after attention or the MLP -- and what
 * sequence parallelism splits along the sequence (LIT-736 record, Key
 * takeaways bullets 1-2).  One call processes one rank's [s_local, b, h] slice.
 *
 * Dropout masks are never stored either: both are drawn from Philox4x32-10
 * (Salmon et al., SC'11) keyed by position, so the backward pass regenerates
 * them bit-exactly.
 *   key       = (seed mod 2^32, seed div 2^32)
 *   attention : element (query i, key j) of batch bb, global q-head hg uses
 *               counter (j div 8, i, hg, bb); hidden dropout: element (global
 *               sequence position sg, batch bb, column c) of site `site` uses
 *               counter (c div 8, sg, bb, site * 2^24 + 2^31).
 *   decision  : the call's four words are eight little-endian 16-bit values;
 *               element j takes value j mod 8 (word (j mod 8) div 2, half
 *               (j mod 2)); keep iff value >= T, T = floor(p * 65536 + 0.5)
 *               with p the float drop probability evaluated in double.
 *               T must stay below 65536: a p that rounds to 65536 (p at or
 *               above 1 - 2^-17) is refused with SRAT_ERR_INVALID.
 *   scaling   : kept elements are multiplied by 1 / (1 - p) (inverted dropout).
 *
 * Conventions for every call.
 *   - Pointers are caller-owned device buffers (hipMalloc / torch) unless said
 *     otherwise; the library allocates nothing and keeps no pointer after the
 *     call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     is asynchronous: the call returns before the kernels finish.
 *   - Outputs are fully overwritten, never accumulated into.
 *   - Returns SRAT_OK (0) or a negative SRAT_ERR_* code.  Arguments are
 *     validated before any HIP call; on error nothing is enqueued and
 *     srat_last_error() (thread-local) describes the problem.
 *   - Calls are reentrant; concurrent calls on different streams do not share
 *     state (workspaces are caller-provided).
 */
#ifndef SRAT_H
#define SRAT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SRAT_VERSION 2

enum srat_status {
  SRAT_OK = 0,
  SRAT_ERR_INVALID = -1,     /* bad pointer, shape, stride or probability */
  SRAT_ERR_UNSUPPORTED = -2, /* valid but not implemented (head dim, dtype, size) */
  SRAT_ERR_WORKSPACE = -3,   /* workspace missing or smaller than the query said */
  SRAT_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
};

enum srat_dtype { SRAT_F32 = 1, SRAT_BF16 = 2 };
enum srat_norm_kind { SRAT_LAYERNORM = 1, SRAT_RMSNORM = 2 };

/*
 * Attention-core problem of one tensor-parallel rank.
 *
 * Layout: Q, O, dO, dQ are [b, s, hq, d]; K, V, dK, dV are [b, s, hkv, d],
 * addressed through the (batch, sequence, head) strides below, in elements;
 * the head dimension d is contiguous.  dO and dQ share O's and Q's strides,
 * dK and dV share K's and V's.  Strides and base pointers must be multiples of
 * 8 elements (16 bytes) for bf16 and of 4 elements for fp32.
 * Grouped-query attention: q-head hh reads kv-head hh / (hq / hkv).
 * Padded batches: with seqlens != NULL, batch element bb acts on its first
 * L = seqlens[bb] positions only, as if its sequence had length L: keys at or
 * past L are invisible, the dropout mask keeps its global counters, and the
 * padded positions get O = 0, LSE = -inf and dQ = dK = dV = 0.  Lengths are
 * read on the device and clamped to [0, s].  bf16 path only.
 */
typedef struct {
  int32_t dtype;          /* SRAT_BF16 (MFMA path) or SRAT_F32 (reference-precision path) */
  int32_t causal;         /* 1: key j is visible to query i iff j <= i; 0: all keys visible */
  int64_t b, s, hq, hkv, d;  /* d in {32, 64, 96, 128, 160}, and 192, 256 for bf16; hq % hkv == 0; s >= 1 */
  int64_t q_stride[3];    /* (batch, seq, head) strides of Q, dQ */
  int64_t k_stride[3];    /* ... of K, dK */
  int64_t v_stride[3];    /* ... of V, dV */
  int64_t o_stride[3];    /* ... of O, dO */
  float scale;            /* softmax scale > 0, or 0 for the default 1/sqrt(d) (rounded to float) */
  float p_drop;           /* attention-dropout probability in [0, 1 - 2^-17); 0 disables it */
  uint64_t seed;          /* Philox key of the attention dropout */
  int64_t head_offset;    /* global index of local q-head 0 (TP rank * hq) */
  const int32_t* seqlens; /* NULL, or device pointer to b valid lengths (int32, 4-byte aligned) */
} srat_attn_desc;

/*
 * Forward of the attention core (LIT-736 record, Key takeaways bullet 4).
 * o   : [b, s, hq, d] output, dtype of the descriptor.
 * lse : [b, hq, s] float32, natural-log logsumexp of each scaled score row
 *       (undropped), the only statistic the backward needs.
 */
int srat_attn_core_fwd(const srat_attn_desc* desc, const void* q, const void* k,
                       const void* v, void* o, float* lse, void* stream);

/*
 * Workspace bytes srat_attn_core_fwd_ws can use: 0 except for causal bf16
 * grids too small to fill the GPU (head dim >= 128, at most 256 workgroups
 * of 128 query rows), where the longest query tiles are split over two
 * workgroups each and need fp32 partials (8 b hq s (d + 1) bytes, rounded up
 * to 256-byte blocks).  Depends on the descriptor only.  Never O(s^2).
 */
int srat_attn_core_fwd_workspace(const srat_attn_desc* desc, size_t* bytes);

/*
 * srat_attn_core_fwd with a caller-owned device workspace (256-byte aligned).
 * With ws != NULL and a nonzero workspace query, ws_bytes must be at least
 * that size (else SRAT_ERR_WORKSPACE) and the split grid runs: each half of
 * a split tile writes O / l and its LSE, and a final kernel merges the halves
 * through their LSEs.  With ws == NULL this is srat_attn_core_fwd.
 */
int srat_attn_core_fwd_ws(const srat_attn_desc* desc, const void* q, const void* k,
                          const void* v, void* o, float* lse, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Workspace bytes srat_attn_core_bwd needs: the per-row D = rowsum(dO * O)
 * (4 b hq s bytes); for grouped-query attention, per-q-head fp32 dK / dV
 * partials (8 b s hq d bytes); and, for causal bf16 grids too small to fill
 * the GPU (head dim >= 128, at most 256 workgroups of 128 rows), the fp32
 * partials of the split query tiles and key blocks (up to 24 b s hq d bytes
 * in all).  Depends on the descriptor only.  Never O(s^2).
 */
int srat_attn_core_bwd_workspace(const srat_attn_desc* desc, size_t* bytes);

/*
 * Backward with recomputation: rebuilds S = Q K^T * scale, P = exp(S - lse)
 * and the dropout mask instead of reading stored activations, then
 * dV = P_d^T dO, dS = P * (dP - rowsum(dO * O)), dQ = dS K * scale,
 * dK = dS^T Q * scale (summed over each kv-head's q-heads).  No atomics: the
 * gradients are bitwise reproducible.
 * q, k, v, o, lse are the forward's inputs/outputs; dout is dL/dO.
 * ws: device workspace of at least srat_attn_core_bwd_workspace() bytes,
 * 256-byte aligned.  dq, dk, dv: outputs with the strides of q, k, v.
 */
int srat_attn_core_bwd(const srat_attn_desc* desc, const void* q, const void* k,
                       const void* v, const void* o, const float* lse, const void* dout,
                       void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * backward as srat_attn_core_bwd, with its workspace taken from a scratch
 * array of SRAT_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on from the moment its code is loaded until the process ends.  The
 * call allocates nothing and calls no allocating routine.
 *   - Shapes whose srat_attn_core_bwd_workspace() exceeds
 *     SRAT_NOALLOC_SCRATCH_BYTES are refused with SRAT_ERR_UNSUPPORTED, before
 *     any HIP call.
 *   - The scratch is found on the device current at the call, which must be
 *     the device of `stream` and of the tensors.
 *   - Every call on one GPU shares that GPU's scratch and leaves its contents
 *     behind; the kernels write every scratch byte before they read it, so no
 *     clearing is needed.  Calls whose execution overlaps on one GPU (several
 *     streams or threads) race on the scratch: serialise them.
 * Arguments, layouts, outputs and errors otherwise as srat_attn_core_bwd.
 */
#define SRAT_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int srat_attn_core_bwd_noalloc(const srat_attn_desc* desc, const void* q, const void* k,
                               const void* v, const void* o, const float* lse, const void* dout,
                               void* dq, void* dk, void* dv, void* stream);

/*
 * Sequence-parallel norm region of one rank: rows [s_local, b, h], contiguous,
 * h contiguous; row (sl, bb) is global sequence position seq_offset + sl.
 */
typedef struct {
  int32_t dtype;          /* SRAT_BF16 or SRAT_F32 for resid, y, h, u, du, dres, dh, dy */
  int32_t norm;           /* SRAT_LAYERNORM or SRAT_RMSNORM */
  int64_t s_local, b, h;  /* h % 8 == 0, h <= 32768; rows s_local * b below about
                             2^32 / (threads per row workgroup) (SRAT_ERR_UNSUPPORTED) */
  int64_t seq_offset;     /* global sequence index of local row 0 (SP rank * s_local) */
  float eps;              /* normaliser epsilon, e.g. 1e-5 */
  float p_drop;           /* hidden-dropout probability in [0, 1 - 2^-17) */
  uint64_t seed;          /* Philox key of the hidden dropout */
  int32_t site;           /* which dropout of the layer, 0..127 (e.g. 1 attention, 2 MLP) */
} srat_norm_desc;

/*
 * Forward (LIT-736 record, Key takeaways bullets 1-2):
 *   h = resid + y * mask / (1 - p)
 *   LayerNorm: u = (h - mean) * rstd * gamma + beta, rstd = 1/sqrt(var + eps)
 *   RMSNorm:   u = h * rstd * gamma,                rstd = 1/sqrt(mean(h^2) + eps)
 * gamma, beta: [h] float32 (beta ignored and may be NULL for RMSNorm).
 * h_out, u_out: [s_local, b, h]; mean (NULL for RMSNorm), rstd: [s_local * b] float32.
 */
int srat_sp_norm_fwd(const srat_norm_desc* desc, const void* resid, const void* y,
                     const float* gamma, const float* beta, void* h_out, void* u_out,
                     float* mean, float* rstd, void* stream);

/* Workspace bytes srat_sp_norm_bwd needs.  Currently 0 for every shape:
 * dgamma / dbeta are summed over all rows by dedicated workgroups of the same
 * launch, without scratch memory.  Kept so callers need not change should a
 * later version use scratch. */
int srat_sp_norm_bwd_workspace(const srat_norm_desc* desc, size_t* bytes);

/*
 * Backward: du = dL/du, dres = dL/dh from the residual path; h, mean, rstd
 * from the forward (the mask is regenerated).
 *   dh = d(norm)/dh applied to du, plus dres  (= dL/dresid)
 *   dy = dh * mask / (1 - p)
 *   dgamma = sum over rows of du * xhat;  dbeta = sum over rows of du
 * dy may equal dh only when p_drop == 0.  dbeta is ignored (may be NULL) for
 * RMSNorm.  ws: at least srat_sp_norm_bwd_workspace() bytes, 256-byte aligned
 * (may be NULL when that is 0).  dgamma / dbeta are reproducible bit for bit
 * (fixed summation order).
 */
int srat_sp_norm_bwd(const srat_norm_desc* desc, const void* du, const void* dres,
                     const void* h, const float* gamma, const float* mean, const float* rstd,
                     void* dh, void* dy, float* dgamma, float* dbeta, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * Test aid: write the keep mask (1 kept, 0 dropped) the kernels use.
 * kind 0: attention, desc is srat_attn_desc*, mask is [b, hq, s, s] bytes;
 * kind 1: hidden dropout, desc is srat_norm_desc*, mask is [s_local, b, h] bytes.
 * Same device function as the compute kernels.  Refused (SRAT_ERR_UNSUPPORTED)
 * above 2^28 mask bytes: for small shapes only.
 */
int srat_dropout_mask_dump(int kind, const void* desc, uint8_t* mask, void* stream);

/*
 * Optional tracing: when enabled, every kernel launch is bracketed with HIP
 * events on its stream; srat_trace_read() synchronises those events and
 * reports, per kernel name, the number of launches and the summed duration.
 * Costs two event records per launch; off by default.
 */
int srat_trace_enable(int on);
/* Fills up to `cap` entries; returns the number of kernels traced (may exceed cap). */
typedef struct { char name[48]; int64_t launches; double total_ms; } srat_trace_entry;
int srat_trace_read(srat_trace_entry* out, int cap, int reset);

/*
 * Recompute policy: the activation-memory ledger of a transformer layer and a
 * planner that picks, layer by layer, what to keep and what to recompute.
 * Host-only (no HIP call, no device pointer).
 *
 * Stored activation bytes of one layer, 2-byte activations (the per-token
 * byte formula of the "Recomputing Activations" plate, "What you will learn",
 * multiplied out per layer):
 *   SRAT_RECOMPUTE_NONE       sbh(34 + 5as/h)
 *   SRAT_RECOMPUTE_SELECTIVE  34sbh        (the attention core is recomputed,
 *                                           what srat_attn_core_bwd does)
 *   SRAT_RECOMPUTE_FULL       2sbh         (the layer input only)
 * On one of t tensor-parallel ranks the layer norms and the dropouts after
 * attention and the MLP (10sbh) stay whole and the rest divides by t; with
 * sequence parallelism everything divides by t (LIT-736 record, Key
 * takeaways bullets 1-2).  Reading: a fully recomputed layer keeps its input
 * whole under tensor parallelism alone and its s/t slice with sequence
 * parallelism (the input sits in the sequence-parallel region).
 *
 * Extra compute, per token over the layers described: selective re-does the
 * attention-score FLOPs of the forward pass, A = 4sh per layer (2sh causal);
 * full re-does the whole forward pass of the layer, 2N/L + A (one more
 * forward pass, about a third more training FLOPs: the plate's second
 * paragraph).  The
 * base is the training FLOPs 6N + 3LA (forward plus backward of the weights
 * and of the attention scores).  All of it divides by t, so the fractions do
 * not depend on t.
 */
enum srat_recompute_policy { SRAT_RECOMPUTE_NONE = 0, SRAT_RECOMPUTE_SELECTIVE = 1, SRAT_RECOMPUTE_FULL = 2 };

typedef struct {
  int64_t s, b, h, a;          /* sequence length, micro-batch, hidden size, attention heads (all > 0) */
  int64_t layers;              /* layers held on this device (> 0) */
  int64_t n_params;            /* parameters N of those layers (>= 0; 0 counts attention FLOPs only) */
  int64_t t;                   /* tensor-parallel size (>= 1) */
  int32_t sequence_parallel;   /* 0/1 */
  int32_t causal;              /* 0/1: causal attention computes half the scores */
} srat_layer_desc;               /* limits (SRAT_ERR_INVALID beyond): s, b, h, a < 2^31;
                                    layers, t < 2^20; n_params < 2^50; s*b*h < 2^60;
                                    a*s*s*b < 2^70 */

typedef struct {
  int64_t layers_none, layers_selective, layers_full;   /* sum = desc->layers */
  double activation_bytes;     /* stored on this device, all layers */
  double extra_compute;        /* extra FLOPs / base training FLOPs */
} srat_recompute_plan;

/* Bytes one layer stores on this device under `policy`, and the extra-compute
 * fraction that policy costs when every layer uses it.  Either output may be
 * NULL. */
int srat_activation_bytes(const srat_layer_desc* desc, int policy, double* bytes_per_layer,
                          double* extra_compute);

/* The assignment of policies to layers with the least extra compute whose
 * stored bytes fit `budget_bytes` (ties: fewer stored bytes, then fewer fully
 * recomputed layers); layers differ only in count.  Exact integer arithmetic.
 * SRAT_ERR_UNSUPPORTED (plan zeroed) when even full recomputation of every
 * layer does not fit; SRAT_ERR_INVALID for a negative or NaN budget. */
int srat_plan_recompute(const srat_layer_desc* desc, double budget_bytes, srat_recompute_plan* plan);

/* Thread-local text of the last error of this thread ("" if none). */
const char* srat_last_error(void);
int srat_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SRAT_H */
