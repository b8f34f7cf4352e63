// C ABI of libsrat: argument validation, workspace layout, kernel dispatch,
// launch tracing and thread-local error text.  Every check runs before the
// first HIP call so that a bad descriptor never enqueues work.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/srat.h"
#include "kernels.hpp"
#include "philox.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SRAT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ----------------------------------------------------------------- tracing
struct TraceState {
  std::mutex mu;
  bool on = false;
  struct Pending { std::string name; hipEvent_t a, b; };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;   // recorded-and-read events, reused
  struct Acc { int64_t n = 0; double ms = 0; };
  std::map<std::string, Acc> acc;
  bool take(hipEvent_t* e) {
    if (!pool.empty()) {
      *e = pool.back();
      pool.pop_back();
      return true;
    }
    // timing-only events: without the system-scope fence an event record
    // costs no cache writeback / invalidation between the traced kernels
    return hipEventCreateWithFlags(e, hipEventDisableSystemFence) == hipSuccess;
  }
};
TraceState& trace() {
  static TraceState t;
  return t;
}

// Drop probability: in [0, 1) and with a 16-bit threshold T = round(p 2^16)
// below 2^16, so that every draw can pass the comparison "value >= T" and the
// threshold fits the 16-bit halves the kernels compare against.
int check_p(float p) {
  if (!(p >= 0.f && p < 1.f)) return fail(SRAT_ERR_INVALID, "p_drop %g not in [0, 1)", p);
  if (srat::drop_threshold16(p) > 0xFFFFu)
    return fail(SRAT_ERR_INVALID, "p_drop %.9g rounds to a 16-bit threshold of 65536: use p < 1 - 2^-17", p);
  return SRAT_OK;
}

// ----------------------------------------------------------------- attention
int check_attn(const srat_attn_desc* d) {
  if (!d) return fail(SRAT_ERR_INVALID, "attn desc is NULL");
  if (d->dtype != SRAT_BF16 && d->dtype != SRAT_F32) return fail(SRAT_ERR_INVALID, "dtype %d", d->dtype);
  if (d->causal != 0 && d->causal != 1) return fail(SRAT_ERR_INVALID, "causal must be 0 or 1");
  if (d->b < 0 || d->s < 0 || d->hq <= 0 || d->hkv <= 0) return fail(SRAT_ERR_INVALID, "negative or zero size");
  if (d->hq % d->hkv) return fail(SRAT_ERR_INVALID, "hq (%lld) not a multiple of hkv (%lld)", (long long)d->hq, (long long)d->hkv);
  if (d->d != 32 && d->d != 64 && d->d != 96 && d->d != 128 && d->d != 160 && d->d != 192 && d->d != 256)
    return fail(SRAT_ERR_UNSUPPORTED, "head dim %lld not in {32,64,96,128,160,192,256}", (long long)d->d);
  if (d->d > 160 && d->dtype != SRAT_BF16)
    return fail(SRAT_ERR_UNSUPPORTED, "head dims above 160 are implemented for bf16 only");
  if (d->s > (1 << 30) || d->b > (1 << 20) || d->hq > (1 << 16))
    return fail(SRAT_ERR_UNSUPPORTED, "size beyond the 32-bit counter ranges");
  if (d->head_offset < 0 || d->head_offset + d->hq > ((int64_t)1 << 31))
    return fail(SRAT_ERR_INVALID, "head_offset out of range");
  if (int e = check_p(d->p_drop)) return e;
  if (!std::isfinite(d->scale) || !(d->scale >= 0.f))
    return fail(SRAT_ERR_INVALID, "scale must be finite and >= 0 (0: 1/sqrt(d))");
  if (d->seqlens && d->dtype != SRAT_BF16)
    return fail(SRAT_ERR_UNSUPPORTED, "per-element sequence lengths need the bf16 path");
  if (d->seqlens && !aligned(d->seqlens, 4)) return fail(SRAT_ERR_INVALID, "seqlens must be 4-byte aligned");
  const int64_t al = d->dtype == SRAT_BF16 ? 8 : 4;
  const int64_t* st[4] = {d->q_stride, d->k_stride, d->v_stride, d->o_stride};
  for (int t = 0; t < 4; ++t)
    for (int i = 0; i < 3; ++i)
      if (st[t][i] < 0 || st[t][i] % al)
        return fail(SRAT_ERR_INVALID, "stride %d of tensor %d is %lld: must be >= 0 and a multiple of %lld",
                    i, t, (long long)st[t][i], (long long)al);
  // the row of one (batch, position, head) must not overlap the next head's
  if (d->q_stride[2] < d->d && d->hq > 1) return fail(SRAT_ERR_INVALID, "q head stride < d");
  if (d->o_stride[2] < d->d && d->hq > 1) return fail(SRAT_ERR_INVALID, "o head stride < d");
  if (d->k_stride[2] < d->d && d->hkv > 1) return fail(SRAT_ERR_INVALID, "k head stride < d");
  if (d->v_stride[2] < d->d && d->hkv > 1) return fail(SRAT_ERR_INVALID, "v head stride < d");
  return SRAT_OK;
}

srat::AttnParams attn_params(const srat_attn_desc* d) {
  srat::AttnParams p{};
  p.sq_b = d->q_stride[0]; p.sq_s = d->q_stride[1]; p.sq_h = d->q_stride[2];
  p.sk_b = d->k_stride[0]; p.sk_s = d->k_stride[1]; p.sk_h = d->k_stride[2];
  p.sv_b = d->v_stride[0]; p.sv_s = d->v_stride[1]; p.sv_h = d->v_stride[2];
  p.so_b = d->o_stride[0]; p.so_s = d->o_stride[1]; p.so_h = d->o_stride[2];
  p.b = (int32_t)d->b; p.s = (int32_t)d->s; p.hq = (int32_t)d->hq; p.hkv = (int32_t)d->hkv;
  p.d = (int32_t)d->d;
  p.causal = d->causal;
  // scale 0 asks for the default 1/sqrt(d), rounded to float
  p.scale = d->scale > 0.f ? d->scale : (float)(1.0 / std::sqrt((double)d->d));
  p.scale_log2 = p.scale * 1.4426950408889634f;
  p.inv_keep = 1.0f / (1.0f - d->p_drop);
  p.thresh = srat::drop_threshold16(d->p_drop);
  p.k0 = (uint32_t)(d->seed & 0xFFFFFFFFu);
  p.k1 = (uint32_t)(d->seed >> 32);
  p.head_offset = (int32_t)d->head_offset;
  p.seqlens = d->seqlens;
  return p;
}

struct AttnWs {
  size_t delta, dk_part, dv_part, dq_part, total;
  srat::AttnSplit split;
};
// rowsum(dO * O) per query row; fp32 dK / dV partials when several q-heads
// share a kv-head or key blocks are split (one slot, or two with split key
// blocks); fp32 dQ partials (two slots) when query tiles are split
AttnWs attn_ws(const srat_attn_desc* d) {
  AttnWs w{};
  w.split = srat::attn_grid_split(d->b, d->s, d->hq, d->d, d->causal != 0, d->dtype == SRAT_BF16);
  const size_t rows = (size_t)d->b * d->s * d->hq;
  size_t off = 0;
  w.delta = off; off += align256(rows * sizeof(float));
  if (d->hq != d->hkv || w.split.split_kb > 0) {
    const size_t slots = w.split.split_kb > 0 ? 2 : 1;
    w.dk_part = off; off += align256(slots * rows * d->d * sizeof(float));
    w.dv_part = off; off += align256(slots * rows * d->d * sizeof(float));
  }
  if (w.split.split_qt > 0) {
    w.dq_part = off; off += align256(2 * rows * d->d * sizeof(float));
  }
  w.total = off;
  return w;
}

// ----------------------------------------------------------------- norm region
int check_norm(const srat_norm_desc* d) {
  if (!d) return fail(SRAT_ERR_INVALID, "norm desc is NULL");
  if (d->dtype != SRAT_BF16 && d->dtype != SRAT_F32) return fail(SRAT_ERR_INVALID, "dtype %d", d->dtype);
  if (d->norm != SRAT_LAYERNORM && d->norm != SRAT_RMSNORM) return fail(SRAT_ERR_INVALID, "norm kind %d", d->norm);
  if (d->s_local < 0 || d->b <= 0 || d->h <= 0) return fail(SRAT_ERR_INVALID, "bad sizes");
  if (d->h % 8) return fail(SRAT_ERR_UNSUPPORTED, "h (%lld) must be a multiple of 8", (long long)d->h);
  if (d->h > 32768) return fail(SRAT_ERR_UNSUPPORTED, "h (%lld) above 32768", (long long)d->h);
  if (d->s_local * d->b > ((int64_t)1 << 31)) return fail(SRAT_ERR_UNSUPPORTED, "too many rows");
  if (d->seq_offset < 0 || d->seq_offset + d->s_local > ((int64_t)1 << 32))
    return fail(SRAT_ERR_INVALID, "seq_offset out of range");
  if (d->b > ((int64_t)1 << 24)) return fail(SRAT_ERR_UNSUPPORTED, "batch above 2^24");
  if (d->site < 0 || d->site > 127) return fail(SRAT_ERR_INVALID, "site %d not in 0..127", d->site);
  if (int e = check_p(d->p_drop)) return e;
  if (!(d->eps >= 0.f) || !std::isfinite(d->eps)) return fail(SRAT_ERR_INVALID, "eps must be finite and >= 0");
  // the backward launches one workgroup per row after the column workgroups;
  // the grid must stay within 2^32 work-items
  if (d->s_local * d->b > srat::norm_bwd_max_rows(d->h))
    return fail(SRAT_ERR_UNSUPPORTED, "%lld rows exceed the %lld the backward grid can hold at h = %lld",
                (long long)(d->s_local * d->b), (long long)srat::norm_bwd_max_rows(d->h), (long long)d->h);
  return SRAT_OK;
}

void norm_common(const srat_norm_desc* d, int64_t& rows, uint32_t& thresh, uint32_t& k0, uint32_t& k1,
                 uint32_t& tag, float& inv_keep) {
  rows = d->s_local * d->b;
  thresh = srat::drop_threshold16(d->p_drop);
  k0 = (uint32_t)(d->seed & 0xFFFFFFFFu);
  k1 = (uint32_t)(d->seed >> 32);
  tag = srat::hidden_tag((uint32_t)d->site);
  inv_keep = 1.0f / (1.0f - d->p_drop);
}

// forward partials of split query tiles: O / l [2][b, hq, s, d] and LSE [2][b, hq, s], fp32
size_t attn_fwd_ws_bytes(const srat_attn_desc* d) {
  const srat::AttnSplit sp = srat::attn_grid_split(d->b, d->s, d->hq, d->d, d->causal != 0, d->dtype == SRAT_BF16);
  if (sp.split_qt == 0) return 0;
  const size_t rows = (size_t)d->b * d->hq * d->s;
  return align256(2 * rows * d->d * sizeof(float)) + align256(2 * rows * sizeof(float));
}

int attn_fwd_impl(const srat_attn_desc* desc, const void* q, const void* k, const void* v, void* o, float* lse,
                  void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (int e = check_attn(desc)) return e;
  const size_t al = 16;
  if (desc->b * desc->s > 0) {
    if (!q || !k || !v || !o || !lse) return fail(SRAT_ERR_INVALID, "NULL tensor pointer");
    if (!aligned(q, al) || !aligned(k, al) || !aligned(v, al) || !aligned(o, al) || !aligned(lse, 4))
      return fail(SRAT_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  }
  srat::AttnParams p = attn_params(desc);
  p.q = q; p.k = k; p.v = v; p.out = o; p.lse_out = lse;
  const size_t need = attn_fwd_ws_bytes(desc);
  if (need > 0 && ws) {   // split grid: needs the workspace; without one, the unsplit launch
    if (ws_bytes < need) return fail(SRAT_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
    if (!aligned(ws, 256)) return fail(SRAT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    const srat::AttnSplit sp = srat::attn_grid_split(desc->b, desc->s, desc->hq, desc->d, desc->causal != 0, true);
    const size_t rows = (size_t)desc->b * desc->hq * desc->s;
    char* base = static_cast<char*>(ws);
    p.o_part = reinterpret_cast<float*>(base);
    p.lse_part = reinterpret_cast<float*>(base + align256(2 * rows * desc->d * sizeof(float)));
    p.split_qt = sp.split_qt;
  }
  hipError_t e = srat::launch_attn_fwd(p, desc->dtype == SRAT_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_core_fwd launch");
  return SRAT_OK;
}

int check_bwd_tensors(const srat_attn_desc* desc, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, const void* dq, const void* dk, const void* dv) {
  if (desc->b * desc->s == 0) return SRAT_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
    return fail(SRAT_ERR_INVALID, "NULL tensor pointer");
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (!aligned(ptr, 16)) return fail(SRAT_ERR_INVALID, "tensor pointers must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(SRAT_ERR_INVALID, "lse must be 4-byte aligned");
  return SRAT_OK;
}

int attn_bwd_launch(const srat_attn_desc* desc, const AttnWs& w, const void* q, const void* k, const void* v,
                    const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                    void* stream);

// ---- scratch of the allocation-free backward entry point.  One array per
// GPU, reserved when the code object is loaded and held until the process
// ends.  In host code the array's name is only a stand-in: its device address
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is passed to kernels.
constexpr size_t kScratchBytes = SRAT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int scratch_ptr(void** out) {
  static std::mutex mu;
  static std::map<int, void*> addr;   // device ordinal -> address of its copy of `scratch`
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256)) return fail(SRAT_ERR_HIP, "scratch address %p is not 256-byte aligned", p);
    it = addr.emplace(dev, p).first;
  }
  *out = it->second;
  return SRAT_OK;
}

}  // namespace

namespace srat {
int activation_bytes(const srat_layer_desc* d, int policy, double* bytes, double* extra, std::string* err);
int plan_recompute(const srat_layer_desc* d, double budget, srat_recompute_plan* plan, std::string* err);
}  // namespace srat

namespace srat {

TraceScope::TraceScope(const char* name, hipStream_t st) : name_(name), st_(st) {
  ev_[0] = ev_[1] = nullptr;
  TraceState& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  if (!t.on) return;
  hipEvent_t a, b;
  if (!t.take(&a)) return;
  if (!t.take(&b)) { t.pool.push_back(a); return; }
  ev_[0] = a;
  ev_[1] = b;
  (void)hipEventRecord(a, st);
}

TraceScope::~TraceScope() {
  if (!ev_[0]) return;
  (void)hipEventRecord((hipEvent_t)ev_[1], st_);
  TraceState& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  t.pending.push_back({name_, (hipEvent_t)ev_[0], (hipEvent_t)ev_[1]});
}

}  // namespace srat

extern "C" {

const char* srat_last_error(void) { return g_err.c_str(); }
int srat_version(void) { return SRAT_VERSION; }

int srat_attn_core_bwd_workspace(const srat_attn_desc* desc, size_t* bytes) {
  g_err.clear();
  if (int e = check_attn(desc)) return e;
  if (!bytes) return fail(SRAT_ERR_INVALID, "bytes is NULL");
  *bytes = attn_ws(desc).total;
  return SRAT_OK;
}

int srat_attn_core_fwd(const srat_attn_desc* desc, const void* q, const void* k, const void* v, void* o,
                       float* lse, void* stream) {
  return attn_fwd_impl(desc, q, k, v, o, lse, nullptr, 0, stream);
}

int srat_attn_core_fwd_workspace(const srat_attn_desc* desc, size_t* bytes) {
  g_err.clear();
  if (int e = check_attn(desc)) return e;
  if (!bytes) return fail(SRAT_ERR_INVALID, "bytes is NULL");
  *bytes = attn_fwd_ws_bytes(desc);
  return SRAT_OK;
}

int srat_attn_core_fwd_ws(const srat_attn_desc* desc, const void* q, const void* k, const void* v, void* o,
                          float* lse, void* ws, size_t ws_bytes, void* stream) {
  return attn_fwd_impl(desc, q, k, v, o, lse, ws, ws_bytes, stream);
}

int srat_attn_core_bwd(const srat_attn_desc* desc, const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                       size_t ws_bytes, void* stream) {
  g_err.clear();
  if (int e = check_attn(desc)) return e;
  if (int e = check_bwd_tensors(desc, q, k, v, o, lse, dout, dq, dk, dv)) return e;
  const AttnWs w = attn_ws(desc);
  if (desc->b * desc->s > 0) {
    if (!ws || ws_bytes < w.total)
      return fail(SRAT_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, w.total);
    if (!aligned(ws, 256)) return fail(SRAT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  return attn_bwd_launch(desc, w, q, k, v, o, lse, dout, dq, dk, dv, ws, stream);
}

int srat_attn_core_bwd_noalloc(const srat_attn_desc* desc, const void* q, const void* k, const void* v,
                               const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               void* stream) {
  g_err.clear();
  if (int e = check_attn(desc)) return e;
  if (int e = check_bwd_tensors(desc, q, k, v, o, lse, dout, dq, dk, dv)) return e;
  const AttnWs w = attn_ws(desc);
  if (w.total > kScratchBytes)
    return fail(SRAT_ERR_UNSUPPORTED, "this shape needs %zu bytes of workspace; the no-allocation entry point "
                "has %zu (use srat_attn_core_bwd with a caller workspace)", w.total, kScratchBytes);
  if (desc->b * desc->s == 0) return SRAT_OK;
  void* ws = nullptr;
  if (int e = scratch_ptr(&ws)) return e;
  return attn_bwd_launch(desc, w, q, k, v, o, lse, dout, dq, dk, dv, ws, stream);
}

}  // extern "C"

namespace {

int attn_bwd_launch(const srat_attn_desc* desc, const AttnWs& w, const void* q, const void* k, const void* v,
                    const void* o, const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                    void* stream) {
  srat::AttnParams p = attn_params(desc);
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.dout = dout;
  p.dq = dq; p.dk = dk; p.dv = dv;
  char* base = static_cast<char*>(ws);
  p.delta = reinterpret_cast<float*>(base + w.delta);
  if (desc->hq != desc->hkv || w.split.split_kb > 0) {
    p.dk_acc = reinterpret_cast<float*>(base + w.dk_part);
    p.dv_acc = reinterpret_cast<float*>(base + w.dv_part);
  }
  if (w.split.split_qt > 0) p.dq_part = reinterpret_cast<float*>(base + w.dq_part);
  p.split_qt = w.split.split_qt;
  p.split_kb = w.split.split_kb;
  hipError_t e = srat::launch_attn_bwd(p, desc->dtype == SRAT_BF16, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_core_bwd launch");
  return SRAT_OK;
}

}  // namespace

extern "C" {

int srat_sp_norm_bwd_workspace(const srat_norm_desc* desc, size_t* bytes) {
  g_err.clear();
  if (int e = check_norm(desc)) return e;
  if (!bytes) return fail(SRAT_ERR_INVALID, "bytes is NULL");
  *bytes = 0;   // dgamma / dbeta are summed without scratch memory
  return SRAT_OK;
}

int srat_sp_norm_fwd(const srat_norm_desc* desc, const void* resid, const void* y, const float* gamma,
                     const float* beta, void* h_out, void* u_out, float* mean, float* rstd, void* stream) {
  g_err.clear();
  if (int e = check_norm(desc)) return e;
  const bool rms = desc->norm == SRAT_RMSNORM;
  if (desc->s_local > 0) {
    if (!resid || !y || !gamma || !h_out || !u_out || !rstd || (!rms && (!beta || !mean)))
      return fail(SRAT_ERR_INVALID, "NULL tensor pointer");
    const void* ptrs[] = {resid, y, gamma, h_out, u_out};
    for (const void* ptr : ptrs)
      if (!aligned(ptr, 16)) return fail(SRAT_ERR_INVALID, "tensor pointers must be 16-byte aligned");
    if (!rms && !aligned(beta, 16)) return fail(SRAT_ERR_INVALID, "beta must be 16-byte aligned");
  }
  srat::NormFwdParams p{};
  norm_common(desc, p.rows, p.thresh, p.k0, p.k1, p.tag, p.inv_keep);
  p.resid = resid; p.y = y; p.gamma = gamma; p.beta = beta; p.h = h_out; p.u = u_out;
  p.mean = mean; p.rstd = rstd;
  p.b = (int32_t)desc->b; p.hdim = (int32_t)desc->h; p.seq_offset = desc->seq_offset; p.eps = desc->eps;
  hipError_t e = srat::launch_norm_fwd(p, desc->dtype == SRAT_BF16, rms, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sp_norm_fwd launch");
  return SRAT_OK;
}

int srat_sp_norm_bwd(const srat_norm_desc* desc, const void* du, const void* dres, const void* h,
                     const float* gamma, const float* mean, const float* rstd, void* dh, void* dy, float* dgamma,
                     float* dbeta, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (int e = check_norm(desc)) return e;
  const bool rms = desc->norm == SRAT_RMSNORM;
  size_t need = 0;
  srat_sp_norm_bwd_workspace(desc, &need);
  if (!gamma || !dgamma || (!rms && !dbeta)) return fail(SRAT_ERR_INVALID, "NULL tensor pointer");
  if (desc->s_local > 0) {
    if (!du || !dres || !h || !rstd || !dh || !dy || (!rms && !mean))
      return fail(SRAT_ERR_INVALID, "NULL tensor pointer");
    const void* ptrs[] = {du, dres, h, gamma, dh, dy};
    for (const void* ptr : ptrs)
      if (!aligned(ptr, 16)) return fail(SRAT_ERR_INVALID, "tensor pointers must be 16-byte aligned");
    if (dy == dh && desc->p_drop != 0.f) return fail(SRAT_ERR_INVALID, "dy may alias dh only when p_drop == 0");
    if (need && (!ws || ws_bytes < need))
      return fail(SRAT_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
    if (need && !aligned(ws, 256)) return fail(SRAT_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  (void)ws;
  (void)ws_bytes;
  srat::NormBwdParams p{};
  norm_common(desc, p.rows, p.thresh, p.k0, p.k1, p.tag, p.inv_keep);
  p.du = du; p.dres = dres; p.h = h; p.gamma = gamma; p.mean = mean; p.rstd = rstd;
  p.dh = dh; p.dy = dy; p.dgamma = dgamma; p.dbeta = dbeta;
  p.b = (int32_t)desc->b; p.hdim = (int32_t)desc->h; p.seq_offset = desc->seq_offset;
  hipError_t e = srat::launch_norm_bwd(p, desc->dtype == SRAT_BF16, rms, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sp_norm_bwd launch");
  return SRAT_OK;
}

int srat_dropout_mask_dump(int kind, const void* desc, uint8_t* mask, void* stream) {
  g_err.clear();
  if (kind == 0) {
    const srat_attn_desc* d = static_cast<const srat_attn_desc*>(desc);
    if (int e = check_attn(d)) return e;
    const double bytes = (double)d->b * d->hq * d->s * d->s;
    if (bytes > (double)(1 << 28)) return fail(SRAT_ERR_UNSUPPORTED, "mask dump above 2^28 bytes");
    if (bytes > 0 && !mask) return fail(SRAT_ERR_INVALID, "mask is NULL");
    hipError_t e = srat::launch_attn_mask(attn_params(d), mask, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "mask dump launch");
    return SRAT_OK;
  }
  if (kind == 1) {
    const srat_norm_desc* d = static_cast<const srat_norm_desc*>(desc);
    if (int e = check_norm(d)) return e;
    const double bytes = (double)d->s_local * d->b * d->h;
    if (bytes > (double)(1 << 28)) return fail(SRAT_ERR_UNSUPPORTED, "mask dump above 2^28 bytes");
    if (bytes > 0 && !mask) return fail(SRAT_ERR_INVALID, "mask is NULL");
    srat::NormFwdParams p{};
    norm_common(d, p.rows, p.thresh, p.k0, p.k1, p.tag, p.inv_keep);
    p.b = (int32_t)d->b; p.hdim = (int32_t)d->h; p.seq_offset = d->seq_offset;
    hipError_t e = srat::launch_hidden_mask(p, mask, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "mask dump launch");
    return SRAT_OK;
  }
  return fail(SRAT_ERR_INVALID, "mask kind %d", kind);
}

int srat_trace_enable(int on) {
  TraceState& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  t.on = on != 0;
  return SRAT_OK;
}

int srat_trace_read(srat_trace_entry* out, int cap, int reset) {
  g_err.clear();
  TraceState& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& pd : t.pending) {
    hipError_t e = hipEventSynchronize(pd.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pd.a, pd.b);
    t.pool.push_back(pd.a);
    t.pool.push_back(pd.b);
    if (e != hipSuccess) {
      t.pending.clear();
      return hip_fail(e, "trace event");
    }
    auto& a = t.acc[pd.name];
    a.n += 1;
    a.ms += ms;
  }
  t.pending.clear();
  int n = 0;
  for (auto& kv : t.acc) {
    if (out && n < cap) {
      std::memset(&out[n], 0, sizeof(srat_trace_entry));
      std::snprintf(out[n].name, sizeof(out[n].name), "%s", kv.first.c_str());
      out[n].launches = kv.second.n;
      out[n].total_ms = kv.second.ms;
    }
    ++n;
  }
  if (reset) t.acc.clear();
  return n;
}

// ---- recompute policy (host only)
int srat_activation_bytes(const srat_layer_desc* desc, int policy, double* bytes_per_layer,
                          double* extra_compute) {
  std::string err;
  const int rc = srat::activation_bytes(desc, policy, bytes_per_layer, extra_compute, &err);
  if (rc != SRAT_OK) return fail(rc, "%s", err.c_str());
  return SRAT_OK;
}

int srat_plan_recompute(const srat_layer_desc* desc, double budget_bytes, srat_recompute_plan* plan) {
  std::string err;
  const int rc = srat::plan_recompute(desc, budget_bytes, plan, &err);
  if (rc != SRAT_OK) return fail(rc, "%s", err.c_str());
  return SRAT_OK;
}

}  // extern "C"
