"""Python binding of libsrat (ctypes): argument marshalling only.

Every step of the attention core and of the norm region runs in the HIP
library; this module builds descriptors, allocates outputs and workspaces
with torch on the tensors' device, and passes raw pointers plus torch's
current HIP stream.  If libsrat.so is missing, every call raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsrat.so")

SRAT_F32, SRAT_BF16 = 1, 2
SRAT_LAYERNORM, SRAT_RMSNORM = 1, 2
ERRORS = {-1: "SRAT_ERR_INVALID", -2: "SRAT_ERR_UNSUPPORTED", -3: "SRAT_ERR_WORKSPACE", -4: "SRAT_ERR_HIP"}
EXPORTS = ("srat_attn_core_fwd", "srat_attn_core_fwd_workspace", "srat_attn_core_fwd_ws", "srat_attn_core_bwd",
           "srat_attn_core_bwd_workspace", "srat_attn_core_bwd_noalloc", "srat_sp_norm_fwd",
           "srat_sp_norm_bwd", "srat_sp_norm_bwd_workspace", "srat_dropout_mask_dump", "srat_trace_enable",
           "srat_trace_read", "srat_last_error", "srat_version", "srat_activation_bytes",
           "srat_plan_recompute")
RECOMPUTE_POLICIES = {"none": 0, "selective": 1, "full": 2}


class AttnDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("b", ctypes.c_int64), ("s", ctypes.c_int64), ("hq", ctypes.c_int64),
                ("hkv", ctypes.c_int64), ("d", ctypes.c_int64),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
                ("scale", ctypes.c_float), ("p_drop", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("head_offset", ctypes.c_int64), ("seqlens", ctypes.c_void_p)]


class NormDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("norm", ctypes.c_int32),
                ("s_local", ctypes.c_int64), ("b", ctypes.c_int64), ("h", ctypes.c_int64),
                ("seq_offset", ctypes.c_int64), ("eps", ctypes.c_float), ("p_drop", ctypes.c_float),
                ("seed", ctypes.c_uint64), ("site", ctypes.c_int32)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("s", ctypes.c_int64), ("b", ctypes.c_int64), ("h", ctypes.c_int64), ("a", ctypes.c_int64),
                ("layers", ctypes.c_int64), ("n_params", ctypes.c_int64), ("t", ctypes.c_int64),
                ("sequence_parallel", ctypes.c_int32), ("causal", ctypes.c_int32)]


class RecomputePlan(ctypes.Structure):
    _fields_ = [("layers_none", ctypes.c_int64), ("layers_selective", ctypes.c_int64),
                ("layers_full", ctypes.c_int64), ("activation_bytes", ctypes.c_double),
                ("extra_compute", ctypes.c_double)]


class TraceEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class SratError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Open libsrat.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise SratError(f"{LIB_PATH} not found: build it with "
                            "`python -m selective_recompute_attention_attn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.srat_attn_core_fwd.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp]
        L.srat_attn_core_fwd_workspace.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(sz)]
        L.srat_attn_core_fwd_ws.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, sz, vp]
        L.srat_attn_core_bwd.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.srat_attn_core_bwd_workspace.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(sz)]
        L.srat_attn_core_bwd_noalloc.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.srat_sp_norm_fwd.argtypes = [ctypes.POINTER(NormDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.srat_sp_norm_bwd.argtypes = [ctypes.POINTER(NormDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.srat_sp_norm_bwd_workspace.argtypes = [ctypes.POINTER(NormDesc), ctypes.POINTER(sz)]
        L.srat_dropout_mask_dump.argtypes = [ctypes.c_int, vp, vp, vp]
        L.srat_trace_enable.argtypes = [ctypes.c_int]
        L.srat_trace_read.argtypes = [ctypes.POINTER(TraceEntry), ctypes.c_int, ctypes.c_int]
        dp = ctypes.POINTER(ctypes.c_double)
        L.srat_activation_bytes.argtypes = [ctypes.POINTER(LayerDesc), ctypes.c_int, dp, dp]
        L.srat_plan_recompute.argtypes = [ctypes.POINTER(LayerDesc), ctypes.c_double, ctypes.POINTER(RecomputePlan)]
        L.srat_last_error.restype = ctypes.c_char_p
        for f in EXPORTS:
            if f != "srat_last_error":
                getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        msg = lib().srat_last_error().decode()
        raise SratError(f"{what}: {ERRORS.get(rc, rc)}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SRAT_BF16
    if t.dtype == torch.float32:
        return SRAT_F32
    raise SratError(f"unsupported dtype {t.dtype}")


def _strides(t: torch.Tensor):
    if t.dim() != 4 or t.stride(3) != 1:
        raise SratError("attention tensors are [b, s, heads, d] with d contiguous")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def _seqlens_ptr(seqlens: torch.Tensor, b: int, device) -> int:
    if seqlens.dtype != torch.int32 or seqlens.shape != (b,) or not seqlens.is_contiguous() \
            or seqlens.device != device:
        raise SratError("seqlens must be a contiguous int32 [b] tensor on the tensors' device")
    return seqlens.data_ptr()


def attn_desc(q, k, v, o, *, causal: bool, scale: Optional[float], p_drop: float, seed: int,
              head_offset: int, seqlens: Optional[torch.Tensor] = None) -> AttnDesc:
    """Descriptor of one attention problem.  seqlens: optional int32 [b] device
    tensor of valid lengths (padded batch)."""
    b, s, hq, d = q.shape
    hkv = k.shape[2]
    if k.shape != (b, s, hkv, d) or v.shape != k.shape or o.shape != q.shape:
        raise SratError("shape mismatch between q, k, v, o")
    if not (q.dtype == k.dtype == v.dtype == o.dtype):
        raise SratError("q, k, v, o must share a dtype")
    return AttnDesc(dtype=_dtype_code(q), causal=int(bool(causal)), b=b, s=s, hq=hq, hkv=hkv, d=d,
                    q_stride=_strides(q), k_stride=_strides(k), v_stride=_strides(v), o_stride=_strides(o),
                    scale=0.0 if scale is None else float(scale), p_drop=float(p_drop),
                    seed=int(seed) & 0xFFFFFFFFFFFFFFFF, head_offset=int(head_offset),
                    seqlens=None if seqlens is None else _seqlens_ptr(seqlens, b, q.device))


class Call:
    """One library call with every argument marshalled once: descriptor, device
    pointers, workspace and stream.  Calling it re-issues the same operation on
    the same buffers through a single foreign call, which is what a training
    loop that re-runs a layer on fixed buffers needs.  The object keeps the
    tensors it was built from alive; their storage must not be resized."""
    __slots__ = ("_fn", "_args", "_name", "_keep")

    def __init__(self, name: str, args: tuple, keep: tuple):
        self._fn = getattr(lib(), name)
        self._args = args
        self._name = name
        self._keep = keep

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != 0:
            _check(rc, self._name)


def _stream_arg(device: torch.device, stream):
    if stream is None:
        return _stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def attn_fwd_workspace_bytes(desc: AttnDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().srat_attn_core_fwd_workspace(ctypes.byref(desc), ctypes.byref(n)),
           "srat_attn_core_fwd_workspace")
    return n.value


def prepare_attn_fwd(q, k, v, o, lse, *, causal: bool = False, scale: Optional[float] = None,
                     p_drop: float = 0.0, seed: int = 0, head_offset: int = 0, workspace=None,
                     seqlens: Optional[torch.Tensor] = None, stream=None) -> Call:
    """srat_attn_core_fwd_ws on fixed buffers (o, lse preallocated; workspace of
    attn_fwd_workspace_bytes or None); stream defaults to torch's current stream
    at preparation time."""
    b, s, hq, d = q.shape
    if lse.shape != (b, hq, s) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise SratError("lse must be a contiguous float32 [b, hq, s] tensor")
    desc = attn_desc(q, k, v, o, causal=causal, scale=scale, p_drop=p_drop, seed=seed, head_offset=head_offset,
                     seqlens=seqlens)
    ws_ptr, ws_bytes = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), ws_ptr, ws_bytes,
            _stream_arg(q.device, stream))
    return Call("srat_attn_core_fwd_ws", args, (desc, q, k, v, o, lse, workspace, seqlens))


def attn_core_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
                  scale: Optional[float] = None, p_drop: float = 0.0, seed: int = 0, head_offset: int = 0,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, seqlens: Optional[torch.Tensor] = None
                  ) -> Tuple[torch.Tensor, torch.Tensor]:
    """O = dropout(softmax(q k^T * scale)) v and the per-row LSE [b, hq, s] (fp32).

    workspace: None allocates the one the shape can use (none for most shapes).
    seqlens: optional int32 [b] device tensor of valid lengths (padded batch).
    """
    b, s, hq, d = q.shape
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    l = torch.empty((b, hq, s), dtype=torch.float32, device=q.device) if lse is None else lse
    if workspace is None:
        need = attn_fwd_workspace_bytes(attn_desc(q, k, v, o, causal=causal, scale=scale, p_drop=p_drop,
                                                  seed=seed, head_offset=head_offset))
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    prepare_attn_fwd(q, k, v, o, l, causal=causal, scale=scale, p_drop=p_drop, seed=seed,
                     head_offset=head_offset, workspace=workspace, seqlens=seqlens)()
    return o, l


def attn_bwd_workspace_bytes(desc: AttnDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().srat_attn_core_bwd_workspace(ctypes.byref(desc), ctypes.byref(n)),
           "srat_attn_core_bwd_workspace")
    return n.value


def prepare_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, *, causal: bool = False,
                     scale: Optional[float] = None, p_drop: float = 0.0, seed: int = 0, head_offset: int = 0,
                     seqlens: Optional[torch.Tensor] = None, stream=None) -> Call:
    """srat_attn_core_bwd on fixed buffers: gradients (with the strides of q, k, v)
    and the workspace (attn_bwd_workspace_bytes) preallocated."""
    if dout.shape != o.shape or dout.stride() != o.stride():
        raise SratError("dout must have o's shape and strides")
    desc = attn_desc(q, k, v, o, causal=causal, scale=scale, p_drop=p_drop, seed=seed, head_offset=head_offset,
                     seqlens=seqlens)
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.shape != ref.shape or t.stride() != ref.stride() or t.dtype != ref.dtype:
            raise SratError("preallocated gradients must match q, k, v")
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(workspace), workspace.numel(), _stream_arg(q.device, stream))
    return Call("srat_attn_core_bwd", args, (desc, q, k, v, o, lse, dout, dq, dk, dv, workspace, seqlens))


def attn_core_bwd(q, k, v, o, lse, dout, *, causal: bool = False, scale: Optional[float] = None,
                  p_drop: float = 0.0, seed: int = 0, head_offset: int = 0,
                  workspace: Optional[torch.Tensor] = None, outs=None, seqlens: Optional[torch.Tensor] = None):
    """dq, dk, dv by recomputation of scores, softmax and dropout mask.

    outs: optional preallocated (dq, dk, dv) with the strides of (q, k, v).
    seqlens: the forward's valid lengths (padded batch), or None.
    """
    if outs is None:
        dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
        dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
        dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device)
    else:
        dq, dk, dv = outs
    if workspace is None:
        desc = attn_desc(q, k, v, o, causal=causal, scale=scale, p_drop=p_drop, seed=seed,
                         head_offset=head_offset)
        workspace = torch.empty(max(attn_bwd_workspace_bytes(desc), 1), dtype=torch.uint8, device=q.device)
    prepare_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, causal=causal, scale=scale, p_drop=p_drop,
                     seed=seed, head_offset=head_offset, seqlens=seqlens)()
    return dq, dk, dv


def attn_core_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, *, causal: bool = False,
                          scale: Optional[float] = None, p_drop: float = 0.0, seed: int = 0, head_offset: int = 0,
                          seqlens: Optional[torch.Tensor] = None, stream=None) -> None:
    """srat_attn_core_bwd_noalloc into preallocated dq, dk, dv (strides of q, k,
    v): the backward with the library's own scratch, no workspace argument."""
    if dout.shape != o.shape or dout.stride() != o.stride():
        raise SratError("dout must have o's shape and strides")
    for t, ref in ((dq, q), (dk, k), (dv, v)):
        if t.shape != ref.shape or t.stride() != ref.stride() or t.dtype != ref.dtype:
            raise SratError("preallocated gradients must match q, k, v")
    desc = attn_desc(q, k, v, o, causal=causal, scale=scale, p_drop=p_drop, seed=seed, head_offset=head_offset,
                     seqlens=seqlens)
    _check(lib().srat_attn_core_bwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                            _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                            _stream_arg(q.device, stream)),
           "srat_attn_core_bwd_noalloc")


def norm_desc(x: torch.Tensor, *, norm: str, eps: float, p_drop: float, seed: int, site: int,
              seq_offset: int) -> NormDesc:
    if x.dim() != 3 or not x.is_contiguous():
        raise SratError("norm-region tensors are contiguous [s_local, b, h]")
    kind = {"layernorm": SRAT_LAYERNORM, "rmsnorm": SRAT_RMSNORM}[norm]
    s_local, b, h = x.shape
    return NormDesc(dtype=_dtype_code(x), norm=kind, s_local=s_local, b=b, h=h, seq_offset=int(seq_offset),
                    eps=float(eps), p_drop=float(p_drop), seed=int(seed) & 0xFFFFFFFFFFFFFFFF, site=int(site))


def prepare_sp_norm_fwd(resid, y, gamma, beta, h, u, mean, rstd, *, norm: str = "layernorm",
                        eps: float = 1e-5, p_drop: float = 0.0, seed: int = 0, site: int = 1,
                        seq_offset: int = 0, stream=None) -> Call:
    """srat_sp_norm_fwd on fixed buffers (h, u, mean, rstd preallocated; mean None for RMSNorm)."""
    if y.shape != resid.shape or y.dtype != resid.dtype:
        raise SratError("resid and y must match")
    desc = norm_desc(resid, norm=norm, eps=eps, p_drop=p_drop, seed=seed, site=site, seq_offset=seq_offset)
    for t in (h, u):
        if t.shape != resid.shape or t.dtype != resid.dtype or not t.is_contiguous():
            raise SratError("h and u must be contiguous and match resid")
    args = (ctypes.byref(desc), _ptr(resid), _ptr(y), _ptr(gamma), _ptr(beta), _ptr(h), _ptr(u), _ptr(mean),
            _ptr(rstd), _stream_arg(resid.device, stream))
    return Call("srat_sp_norm_fwd", args, (desc, resid, y, gamma, beta, h, u, mean, rstd))


def sp_norm_fwd(resid, y, gamma, beta=None, *, norm: str = "layernorm", eps: float = 1e-5,
                p_drop: float = 0.0, seed: int = 0, site: int = 1, seq_offset: int = 0, outs=None):
    """h = resid + dropout(y); u = norm(h) * gamma (+ beta).  Returns h, u, mean, rstd.

    outs: optional preallocated (h, u, mean, rstd); mean is None for RMSNorm.
    """
    rows = resid.shape[0] * resid.shape[1]
    if outs is None:
        h = torch.empty_like(resid)
        u = torch.empty_like(resid)
        mean = torch.empty(rows, dtype=torch.float32, device=resid.device) if norm == "layernorm" else None
        rstd = torch.empty(rows, dtype=torch.float32, device=resid.device)
    else:
        h, u, mean, rstd = outs
    prepare_sp_norm_fwd(resid, y, gamma, beta, h, u, mean, rstd, norm=norm, eps=eps, p_drop=p_drop, seed=seed,
                        site=site, seq_offset=seq_offset)()
    return h, u, mean, rstd


def sp_norm_bwd_workspace_bytes(desc: NormDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().srat_sp_norm_bwd_workspace(ctypes.byref(desc), ctypes.byref(n)), "srat_sp_norm_bwd_workspace")
    return n.value


def prepare_sp_norm_bwd(du, dres, h, gamma, mean, rstd, dh, dy, dgamma, dbeta, workspace=None, *,
                        norm: str = "layernorm", p_drop: float = 0.0, seed: int = 0, site: int = 1,
                        seq_offset: int = 0, stream=None) -> Call:
    """srat_sp_norm_bwd on fixed buffers (dy may be dh when p_drop == 0; dbeta None for
    RMSNorm; workspace None when sp_norm_bwd_workspace_bytes is 0)."""
    desc = norm_desc(h, norm=norm, eps=0.0, p_drop=p_drop, seed=seed, site=site, seq_offset=seq_offset)
    ws_ptr, ws_bytes = (_ptr(workspace), workspace.numel()) if workspace is not None else (None, 0)
    args = (ctypes.byref(desc), _ptr(du), _ptr(dres), _ptr(h), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dh),
            _ptr(dy), _ptr(dgamma), _ptr(dbeta), ws_ptr, ws_bytes, _stream_arg(h.device, stream))
    return Call("srat_sp_norm_bwd", args, (desc, du, dres, h, gamma, mean, rstd, dh, dy, dgamma, dbeta, workspace))


def sp_norm_bwd(du, dres, h, gamma, mean, rstd, *, norm: str = "layernorm", p_drop: float = 0.0,
                seed: int = 0, site: int = 1, seq_offset: int = 0, alias_dy: bool = False,
                workspace: Optional[torch.Tensor] = None, outs=None):
    """dh (= d resid), dy, dgamma, dbeta (None for RMSNorm).

    outs: optional preallocated (dh, dy, dgamma, dbeta); dy may be dh when p_drop == 0.
    """
    hdim = h.shape[2]
    if outs is None:
        dh = torch.empty_like(h)
        dy = dh if alias_dy else torch.empty_like(h)
        dgamma = torch.empty(hdim, dtype=torch.float32, device=h.device)
        dbeta = torch.empty(hdim, dtype=torch.float32, device=h.device) if norm == "layernorm" else None
    else:
        dh, dy, dgamma, dbeta = outs
    if workspace is None:
        desc = norm_desc(h, norm=norm, eps=0.0, p_drop=p_drop, seed=seed, site=site, seq_offset=seq_offset)
        need = sp_norm_bwd_workspace_bytes(desc)
        workspace = torch.empty(need, dtype=torch.uint8, device=h.device) if need else None
    prepare_sp_norm_bwd(du, dres, h, gamma, mean, rstd, dh, dy, dgamma, dbeta, workspace, norm=norm,
                        p_drop=p_drop, seed=seed, site=site, seq_offset=seq_offset)()
    return dh, dy, dgamma, dbeta


def attn_dropout_mask(b, s, hq, *, p_drop, seed, head_offset=0, device="cuda"):
    """The attention keep mask [b, hq, s, s] (uint8) the kernels use (small shapes only)."""
    d = 32
    z = torch.empty((b, s, hq, d), dtype=torch.bfloat16, device=device)
    desc = attn_desc(z, z, z, z, causal=False, scale=1.0, p_drop=p_drop, seed=seed, head_offset=head_offset)
    m = torch.empty((b, hq, s, s), dtype=torch.uint8, device=device)
    _check(lib().srat_dropout_mask_dump(0, ctypes.cast(ctypes.pointer(desc), ctypes.c_void_p), _ptr(m),
                                        _stream(m.device)), "srat_dropout_mask_dump")
    return m


def hidden_dropout_mask(s_local, b, h, *, p_drop, seed, site=1, seq_offset=0, device="cuda"):
    """The hidden-dropout keep mask [s_local, b, h] (uint8) the kernels use."""
    z = torch.empty((s_local, b, h), dtype=torch.bfloat16, device=device)
    desc = norm_desc(z, norm="layernorm", eps=1e-5, p_drop=p_drop, seed=seed, site=site, seq_offset=seq_offset)
    m = torch.empty((s_local, b, h), dtype=torch.uint8, device=device)
    _check(lib().srat_dropout_mask_dump(1, ctypes.cast(ctypes.pointer(desc), ctypes.c_void_p), _ptr(m),
                                        _stream(m.device)), "srat_dropout_mask_dump")
    return m


def trace_enable(on: bool = True) -> None:
    _check(lib().srat_trace_enable(int(on)), "srat_trace_enable")


def trace_read(reset: bool = True):
    """{kernel name: (launches, total_ms)} accumulated since the last reset."""
    cap = 64
    buf = (TraceEntry * cap)()
    n = lib().srat_trace_read(buf, cap, int(reset))
    if n < 0:
        _check(n, "srat_trace_read")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n, cap))}


# ---- recompute policy (host only: no device, no stream)
def layer_desc(*, s: int, b: int, h: int, a: int, layers: int, n_params: int = 0, t: int = 1,
               sequence_parallel: bool = False, causal: bool = True) -> LayerDesc:
    return LayerDesc(s, b, h, a, layers, int(n_params), t, int(bool(sequence_parallel)), int(bool(causal)))


def activation_bytes(policy: str, **dims) -> Tuple[float, float]:
    """(bytes one layer stores on this device, extra-compute fraction) when every
    layer uses `policy` ("none", "selective" or "full")."""
    d = layer_desc(**dims)
    nb, ex = ctypes.c_double(), ctypes.c_double()
    _check(lib().srat_activation_bytes(ctypes.byref(d), RECOMPUTE_POLICIES[policy], ctypes.byref(nb),
                                       ctypes.byref(ex)), "srat_activation_bytes")
    return nb.value, ex.value


def plan_recompute(budget_bytes: float, **dims) -> dict:
    """Least-extra-compute assignment of none / selective / full recomputation to
    the layers whose stored activations fit `budget_bytes` on this device."""
    d = layer_desc(**dims)
    plan = RecomputePlan()
    _check(lib().srat_plan_recompute(ctypes.byref(d), float(budget_bytes), ctypes.byref(plan)),
           "srat_plan_recompute")
    return {"none": plan.layers_none, "selective": plan.layers_selective, "full": plan.layers_full,
            "activation_bytes": plan.activation_bytes, "extra_compute": plan.extra_compute}
