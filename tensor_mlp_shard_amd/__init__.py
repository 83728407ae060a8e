"""Python binding of ``libtpmlp.so``: the tensor-parallel MLP shard on MI355X.

Argument marshalling only: every step of the computation runs in the HIP kernels
of the library.  PyTorch supplies device memory and the current stream.  If the
library is not built, every call raises; there is no CPU fallback.

The functions carry the names of the C ABI (``include/tp_mlp_shard.h``):

* ``tp_mlp_shard_plan``, ``tp_mlp_shard_create``, ``tp_mlp_shard_fwd``,
  ``tp_mlp_shard_destroy``, ``tp_partials_reduce``,
  ``tp_partials_reduce_add_rmsnorm``, ``tp_partials_quantize_fp8``,
  ``tp_partials_reduce_fp8``, ``tp_proj_create``, ``tp_proj_fwd``,
  ``tp_proj_destroy``, ``tp_moe_create``, ``tp_moe_fwd``, ``tp_moe_destroy``,
  ``tpm_status_str``,
  ``tp_mlp_shard_set_timing_events``;

plus conveniences: ``Shard`` (one rank's MLP handle), ``Projection`` (one rank's
shard of a single projection, e.g. the attention QKV or output projection),
``GroupedExperts`` (the experts of one GPU as a grouped MLP) and
``tensor_parallel_output(x, a_shards, b_shards, activation="tanh")``, the pages'
statement Z = sum_i act(x @ a_i) @ b_i (page "LLM 推理并行化：先找瓶颈，再决定怎么
切", section 三.2), which raises ``ValueError`` when the shard lists differ in length.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "tp_mlp_shard_plan", "tp_mlp_shard_create", "tp_mlp_shard_fwd", "tp_mlp_shard_fwd_noalloc",
    "tp_mlp_shard_destroy",
    "tp_partials_reduce", "tp_partials_reduce_add_rmsnorm", "tp_partials_quantize_fp8",
    "tp_partials_reduce_fp8", "tp_attn_partials_merge", "attn_partials_merge", "tp_proj_create", "tp_proj_fwd", "tp_proj_destroy",
    "Projection", "tp_moe_create", "tp_moe_fwd", "tp_moe_destroy", "GroupedExperts",
    "tpm_status_str", "tp_mlp_shard_set_timing_events", "Shard",
    "partials_reduce", "tensor_parallel_output", "TpmError", "LIB_PATH", "ACT", "PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtpmlp.so")

ACT = {"tanh": 0, "silu_gate": 1, "identity": 2}
PATH = {"auto": 0, "stream": 1, "tiled": 2}
F32, BF16 = 0, 1

STATUS_NAMES = {0: "TPM_OK", 1: "TPM_ERR_INVALID_ARG", 2: "TPM_ERR_SHAPE", 3: "TPM_ERR_ALIGN",
                4: "TPM_ERR_HIP", 5: "TPM_ERR_OOM"}


class TpmDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int64), ("ffn_shard", ctypes.c_int64),
                ("max_tokens", ctypes.c_int64), ("act", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("path", ctypes.c_int32)]


class TpmPlanInfo(ctypes.Structure):
    _fields_ = [("packed_weight_bytes", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("ffn_padded", ctypes.c_int64), ("stream_max_tokens", ctypes.c_int64),
                ("kernels_per_fwd", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class TpmProjDesc(ctypes.Structure):
    _fields_ = [("in_features", ctypes.c_int64), ("out_features", ctypes.c_int64),
                ("max_tokens", ctypes.c_int64), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("path", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class TpmMoeDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int64), ("ffn_expert", ctypes.c_int64),
                ("n_experts", ctypes.c_int64), ("max_tokens", ctypes.c_int64),
                ("act", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("path", ctypes.c_int32)]


class TpmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, STATUS_NAMES.get(status, status),
                                           tpm_status_str(status)))


_lib = None


def capi():
    """The loaded library with its C signatures declared (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libtpmlp.so is not built (%s); run __graft_entry__.build() "
                           "-- there is no CPU fallback" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.tpm_status_str.argtypes = [ctypes.c_int]
    lib.tpm_status_str.restype = ctypes.c_char_p
    lib.tp_mlp_shard_plan.argtypes = [ctypes.POINTER(TpmDesc), ctypes.POINTER(TpmPlanInfo)]
    lib.tp_mlp_shard_plan.restype = ctypes.c_int
    lib.tp_mlp_shard_create.argtypes = [ctypes.POINTER(TpmDesc), vp, vp, vp, ctypes.POINTER(vp)]
    lib.tp_mlp_shard_create.restype = ctypes.c_int
    lib.tp_mlp_shard_fwd.argtypes = [vp, vp, i64, vp, vp]
    lib.tp_mlp_shard_fwd.restype = ctypes.c_int
    lib.tp_mlp_shard_fwd_noalloc.argtypes = [vp, vp, i64, vp, vp]
    lib.tp_mlp_shard_fwd_noalloc.restype = ctypes.c_int
    lib.tp_partials_reduce.argtypes = [ctypes.POINTER(vp), i32, i64, i32, vp, i32, vp]
    lib.tp_partials_reduce.restype = ctypes.c_int
    lib.tp_partials_reduce_add_rmsnorm.argtypes = [ctypes.POINTER(vp), i32, i64, i64, i32, vp, vp,
                                                   i32, vp, ctypes.c_float, vp, i32, vp]
    lib.tp_partials_reduce_add_rmsnorm.restype = ctypes.c_int
    lib.tp_partials_quantize_fp8.argtypes = [vp, i64, i64, i32, vp, vp, vp]
    lib.tp_partials_quantize_fp8.restype = ctypes.c_int
    lib.tp_partials_reduce_fp8.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, i64, i64,
                                           vp, i32, vp]
    lib.tp_partials_reduce_fp8.restype = ctypes.c_int
    lib.tp_attn_partials_merge.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp),
                                           ctypes.POINTER(vp), i32, i64, i64, i32, vp, i32, vp,
                                           vp, vp]
    lib.tp_attn_partials_merge.restype = ctypes.c_int
    lib.tp_proj_create.argtypes = [ctypes.POINTER(TpmProjDesc), vp, vp, ctypes.POINTER(vp)]
    lib.tp_proj_create.restype = ctypes.c_int
    lib.tp_proj_fwd.argtypes = [vp, vp, i64, vp, vp]
    lib.tp_proj_fwd.restype = ctypes.c_int
    lib.tp_proj_destroy.argtypes = [vp]
    lib.tp_proj_destroy.restype = ctypes.c_int
    lib.tp_moe_create.argtypes = [ctypes.POINTER(TpmMoeDesc), vp, vp, vp, ctypes.POINTER(vp)]
    lib.tp_moe_create.restype = ctypes.c_int
    lib.tp_moe_fwd.argtypes = [vp, vp, vp, i64, vp, vp]
    lib.tp_moe_fwd.restype = ctypes.c_int
    lib.tp_moe_destroy.argtypes = [vp]
    lib.tp_moe_destroy.restype = ctypes.c_int
    lib.tp_mlp_shard_destroy.argtypes = [vp]
    lib.tp_mlp_shard_destroy.restype = ctypes.c_int
    lib.tp_mlp_shard_set_timing_events.argtypes = [vp, ctypes.POINTER(vp), i32]
    lib.tp_mlp_shard_set_timing_events.restype = ctypes.c_int
    _lib = lib
    return lib


def tpm_status_str(status: int) -> str:
    return capi().tpm_status_str(int(status)).decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise TpmError(rc, what)


def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % dt)


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _dev_ptr(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous (row-major, no padding)" % name)
    return ctypes.c_void_p(t.data_ptr())


def make_desc(d_model, ffn_shard, max_tokens, activation="silu_gate", in_dtype=BF16,
              out_dtype=F32, path="auto") -> TpmDesc:
    return TpmDesc(int(d_model), int(ffn_shard), int(max_tokens), ACT[activation],
                   int(in_dtype), int(out_dtype), PATH[path])


def tp_mlp_shard_plan(desc: TpmDesc) -> dict:
    info = TpmPlanInfo()
    _check(capi().tp_mlp_shard_plan(ctypes.byref(desc), ctypes.byref(info)), "tp_mlp_shard_plan")
    return {f: getattr(info, f) for f, _ in TpmPlanInfo._fields_ if f != "reserved"}


def tp_mlp_shard_create(desc: TpmDesc, A, B, stream=None) -> int:
    """Create a shard handle from device tensors A [d, F or 2F] and B [F, d]."""
    h = ctypes.c_void_p()
    _check(capi().tp_mlp_shard_create(ctypes.byref(desc), _dev_ptr(A, "A"), _dev_ptr(B, "B"),
                                      _stream_ptr(stream), ctypes.byref(h)), "tp_mlp_shard_create")
    return h.value


def tp_mlp_shard_fwd(handle: int, X, M: int, partial, stream=None) -> None:
    _check(capi().tp_mlp_shard_fwd(ctypes.c_void_p(handle), _dev_ptr(X, "X"), int(M),
                                   _dev_ptr(partial, "partial"), _stream_ptr(stream)),
           "tp_mlp_shard_fwd")


def tp_mlp_shard_fwd_noalloc(handle: int, X, M: int, partial, stream=None) -> None:
    """The decode-path forward with the library's per-device scratch array instead of
    the handle's workspace (1 <= M <= 64, bf16 handles; allocates nothing)."""
    _check(capi().tp_mlp_shard_fwd_noalloc(ctypes.c_void_p(handle), _dev_ptr(X, "X"), int(M),
                                           _dev_ptr(partial, "partial"), _stream_ptr(stream)),
           "tp_mlp_shard_fwd_noalloc")


def tp_partials_reduce(partials, out, stream=None) -> None:
    """out = sum of the partials (rank order, fp32 accumulation)."""
    parts = list(partials)
    if not parts:
        raise ValueError("need at least one partial")
    numel = parts[0].numel()
    in_dt = parts[0].dtype
    for p in parts:
        if p.numel() != numel or p.dtype != in_dt:
            raise ValueError("partials must agree in size and dtype")
    if out.numel() != numel:
        raise ValueError("out has %d elements, partials %d" % (out.numel(), numel))
    arr = (ctypes.c_void_p * len(parts))(*[_dev_ptr(p, "partial").value for p in parts])
    _check(capi().tp_partials_reduce(arr, len(parts), numel, _dtype_code(in_dt),
                                     _dev_ptr(out, "out"), _dtype_code(out.dtype),
                                     _stream_ptr(stream)), "tp_partials_reduce")


def tp_partials_reduce_add_rmsnorm(partials, residual, gamma, eps, y, residual_out=None,
                                   stream=None) -> None:
    """Partials sum + residual add + RMSNorm per row (see the C header).

    partials: k tensors [rows, cols]; residual, residual_out (default: residual,
    in place) [rows, cols]; gamma [cols] with the residual's dtype; y [rows, cols]."""
    parts = list(partials)
    if not parts:
        raise ValueError("need at least one partial")
    if residual.dim() != 2:
        raise ValueError("residual must be [rows, cols]")
    rows, cols = residual.shape
    in_dt = parts[0].dtype
    for p in parts:
        if tuple(p.shape) != (rows, cols) or p.dtype != in_dt:
            raise ValueError("partials must be [rows, cols] of one dtype")
    if residual_out is None:
        residual_out = residual
    if tuple(residual_out.shape) != (rows, cols) or residual_out.dtype != residual.dtype:
        raise ValueError("residual_out must match residual")
    if tuple(gamma.shape) != (cols,) or gamma.dtype != residual.dtype:
        raise ValueError("gamma must be [cols] with the residual's dtype")
    if tuple(y.shape) != (rows, cols):
        raise ValueError("y must be [rows, cols]")
    arr = (ctypes.c_void_p * len(parts))(*[_dev_ptr(p, "partial").value for p in parts])
    _check(capi().tp_partials_reduce_add_rmsnorm(
        arr, len(parts), rows, cols, _dtype_code(in_dt), _dev_ptr(residual, "residual"),
        _dev_ptr(residual_out, "residual_out"), _dtype_code(residual.dtype),
        _dev_ptr(gamma, "gamma"), float(eps), _dev_ptr(y, "y"), _dtype_code(y.dtype),
        _stream_ptr(stream)), "tp_partials_reduce_add_rmsnorm")


def tp_partials_quantize_fp8(partial, q, scale, stream=None) -> None:
    """FP8 (E4M3) codes of a partial [rows, cols] with one fp32 scale per row:
    q uint8 [rows, cols], scale float32 [rows] (see the C header)."""
    torch = _torch()
    if partial.dim() != 2:
        raise ValueError("partial must be [rows, cols]")
    rows, cols = partial.shape
    if tuple(q.shape) != (rows, cols) or q.dtype != torch.uint8:
        raise ValueError("q must be uint8 [rows, cols]")
    if tuple(scale.shape) != (rows,) or scale.dtype != torch.float32:
        raise ValueError("scale must be float32 [rows]")
    _check(capi().tp_partials_quantize_fp8(_dev_ptr(partial, "partial"), rows, cols,
                                           _dtype_code(partial.dtype), _dev_ptr(q, "q"),
                                           _dev_ptr(scale, "scale"), _stream_ptr(stream)),
           "tp_partials_quantize_fp8")


def tp_partials_reduce_fp8(qs, scales, out, stream=None) -> None:
    """out = sum over ranks of value(q_i) * scale_i[row], fp32 accumulation."""
    torch = _torch()
    qs, scales = list(qs), list(scales)
    if not qs or len(qs) != len(scales):
        raise ValueError("need matching, non-empty lists of codes and scales")
    rows, cols = qs[0].shape
    for q, s in zip(qs, scales):
        if tuple(q.shape) != (rows, cols) or q.dtype != torch.uint8:
            raise ValueError("codes must be uint8 [rows, cols]")
        if tuple(s.shape) != (rows,) or s.dtype != torch.float32:
            raise ValueError("scales must be float32 [rows]")
    if tuple(out.shape) != (rows, cols):
        raise ValueError("out must be [rows, cols]")
    qa = (ctypes.c_void_p * len(qs))(*[_dev_ptr(q, "q").value for q in qs])
    sa = (ctypes.c_void_p * len(qs))(*[_dev_ptr(s, "scale").value for s in scales])
    _check(capi().tp_partials_reduce_fp8(qa, sa, len(qs), rows, cols, _dev_ptr(out, "out"),
                                         _dtype_code(out.dtype), _stream_ptr(stream)),
           "tp_partials_reduce_fp8")


def tp_attn_partials_merge(values, maxima, expsums, out, max_out=None, expsum_out=None,
                           stream=None) -> None:
    """Merge k attention partials (page "LLM 推理并行化", section 三.4): values[i]
    [rows, dim] (float32 or bfloat16), maxima[i] and expsums[i] float32 [rows];
    out [rows, dim]; optional merged statistics max_out, expsum_out float32 [rows]."""
    torch = _torch()
    vals, maxs, sums = list(values), list(maxima), list(expsums)
    if not vals or not (len(vals) == len(maxs) == len(sums)):
        raise ValueError("need matching, non-empty lists of values, maxima and expsums")
    if vals[0].dim() != 2:
        raise ValueError("values must be [rows, dim]")
    rows, dim = vals[0].shape
    in_dt = vals[0].dtype
    for v, m, e in zip(vals, maxs, sums):
        if tuple(v.shape) != (rows, dim) or v.dtype != in_dt:
            raise ValueError("values must be [rows, dim] of one dtype")
        if tuple(m.shape) != (rows,) or tuple(e.shape) != (rows,) or \
                m.dtype != torch.float32 or e.dtype != torch.float32:
            raise ValueError("maxima and expsums must be float32 [rows]")
    if tuple(out.shape) != (rows, dim):
        raise ValueError("out must be [rows, dim]")
    if (max_out is None) != (expsum_out is None):
        raise ValueError("give both merged statistics or neither")
    if max_out is not None:
        for t in (max_out, expsum_out):
            if tuple(t.shape) != (rows,) or t.dtype != torch.float32:
                raise ValueError("merged statistics must be float32 [rows]")
    k = len(vals)
    va = (ctypes.c_void_p * k)(*[_dev_ptr(v, "values") for v in vals])
    ma = (ctypes.c_void_p * k)(*[_dev_ptr(m, "maxima") for m in maxs])
    ea = (ctypes.c_void_p * k)(*[_dev_ptr(e, "expsums") for e in sums])
    mo = _dev_ptr(max_out, "max_out") if max_out is not None else None
    eo = _dev_ptr(expsum_out, "expsum_out") if expsum_out is not None else None
    _check(capi().tp_attn_partials_merge(va, ma, ea, k, rows, dim, _dtype_code(in_dt),
                                         _dev_ptr(out, "out"), _dtype_code(out.dtype), mo, eo,
                                         _stream_ptr(stream)), "tp_attn_partials_merge")


def attn_partials_merge(values, maxima, expsums, out_dtype=None, stream=None):
    """Merged output and merged statistics (out, max, expsum) of k attention partials."""
    torch = _torch()
    v0 = values[0]
    out = torch.empty(v0.shape, dtype=out_dtype or torch.float32, device=v0.device)
    mo = torch.empty(v0.shape[0], dtype=torch.float32, device=v0.device)
    eo = torch.empty_like(mo)
    tp_attn_partials_merge(values, maxima, expsums, out, mo, eo, stream)
    return out, mo, eo


def tp_mlp_shard_destroy(handle: int) -> None:
    _check(capi().tp_mlp_shard_destroy(ctypes.c_void_p(handle)), "tp_mlp_shard_destroy")


def tp_mlp_shard_set_timing_events(handle: int, events) -> None:
    """events: sequence of raw hipEvent_t values (ints), or None to switch off."""
    if events is None:
        _check(capi().tp_mlp_shard_set_timing_events(ctypes.c_void_p(handle), None, 0),
               "tp_mlp_shard_set_timing_events")
        return
    arr = (ctypes.c_void_p * len(events))(*[int(e) for e in events])
    _check(capi().tp_mlp_shard_set_timing_events(ctypes.c_void_p(handle), arr, len(events)),
           "tp_mlp_shard_set_timing_events")


class Shard:
    """One rank's shard: owns a library handle with repacked weights.

    a: first-weight shard [d, F] (tanh, identity) or [d, 2F] (silu_gate: F gate
       columns then F up columns), b: second-weight shard [F, d]; both GPU tensors
       of the same dtype (float32 or bfloat16)."""

    def __init__(self, a, b, activation="tanh", max_tokens=None, out_dtype=None, path="auto",
                 stream=None):
        torch = _torch()
        if a.dim() != 2 or b.dim() != 2:
            raise ValueError("a and b must be 2-D")
        if a.dtype != b.dtype:
            raise ValueError("a and b must share a dtype")
        d, F = a.shape[0], b.shape[0]
        ncol = 2 * F if activation == "silu_gate" else F
        if a.shape[1] != ncol or b.shape[1] != d:
            raise ValueError("shard shapes %s, %s do not fit activation %s"
                             % (tuple(a.shape), tuple(b.shape), activation))
        self.d_model, self.ffn_shard, self.activation = d, F, activation
        self.in_dtype = a.dtype
        self.out_dtype = out_dtype if out_dtype is not None else torch.float32
        self.max_tokens = int(max_tokens) if max_tokens is not None else 8192
        self.desc = make_desc(d, F, self.max_tokens, activation, _dtype_code(a.dtype),
                              _dtype_code(self.out_dtype), path)
        self.plan = tp_mlp_shard_plan(self.desc)
        self.handle = tp_mlp_shard_create(self.desc, a, b, stream)

    def forward(self, x, out=None, stream=None):
        torch = _torch()
        if x.dim() != 2 or x.shape[1] != self.d_model or x.dtype != self.in_dtype:
            raise ValueError("x must be [M, %d] of %s" % (self.d_model, self.in_dtype))
        M = x.shape[0]
        if out is None:
            out = torch.empty((M, self.d_model), dtype=self.out_dtype, device=x.device)
        elif out.shape != (M, self.d_model) or out.dtype != self.out_dtype:
            raise ValueError("out must be [M, d] of %s" % self.out_dtype)
        tp_mlp_shard_fwd(self.handle, x, M, out, stream)
        return out

    __call__ = forward

    def set_timing_events(self, events):
        tp_mlp_shard_set_timing_events(self.handle, events)

    def close(self):
        if getattr(self, "handle", None):
            tp_mlp_shard_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tp_proj_create(desc: TpmProjDesc, W, stream=None) -> int:
    """Create a projection handle from a device tensor W [in_features, out_features]."""
    h = ctypes.c_void_p()
    _check(capi().tp_proj_create(ctypes.byref(desc), _dev_ptr(W, "W"), _stream_ptr(stream),
                                 ctypes.byref(h)), "tp_proj_create")
    return h.value


def tp_proj_fwd(handle: int, X, M: int, Y, stream=None) -> None:
    _check(capi().tp_proj_fwd(ctypes.c_void_p(handle), _dev_ptr(X, "X"), int(M), _dev_ptr(Y, "Y"),
                              _stream_ptr(stream)), "tp_proj_fwd")


def tp_proj_destroy(handle: int) -> None:
    _check(capi().tp_proj_destroy(ctypes.c_void_p(handle)), "tp_proj_destroy")


class Projection:
    """One rank's shard of a single projection, Y = X W (the handle owns a packed
    copy of W).  For the attention block: the column shard of [Wq | Wk | Wv] with
    bf16 output, or the row shard of Wo with an fp32 partial output."""

    def __init__(self, w, max_tokens=None, out_dtype=None, path="auto", stream=None):
        torch = _torch()
        if w.dim() != 2:
            raise ValueError("w must be [in_features, out_features]")
        self.in_features, self.out_features = w.shape
        self.in_dtype = w.dtype
        self.out_dtype = out_dtype if out_dtype is not None else torch.float32
        self.max_tokens = int(max_tokens) if max_tokens is not None else 8192
        self.desc = TpmProjDesc(int(self.in_features), int(self.out_features), self.max_tokens,
                                _dtype_code(w.dtype), _dtype_code(self.out_dtype), PATH[path], 0)
        self.handle = tp_proj_create(self.desc, w, stream)

    def forward(self, x, out=None, stream=None):
        torch = _torch()
        if x.dim() != 2 or x.shape[1] != self.in_features or x.dtype != self.in_dtype:
            raise ValueError("x must be [M, %d] of %s" % (self.in_features, self.in_dtype))
        M = x.shape[0]
        if out is None:
            out = torch.empty((M, self.out_features), dtype=self.out_dtype, device=x.device)
        elif tuple(out.shape) != (M, self.out_features) or out.dtype != self.out_dtype:
            raise ValueError("out must be [M, %d] of %s" % (self.out_features, self.out_dtype))
        tp_proj_fwd(self.handle, x, M, out, stream)
        return out

    __call__ = forward

    def close(self):
        if getattr(self, "handle", None):
            tp_proj_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tp_moe_create(desc: TpmMoeDesc, W1, W2, stream=None) -> int:
    h = ctypes.c_void_p()
    _check(capi().tp_moe_create(ctypes.byref(desc), _dev_ptr(W1, "W1"), _dev_ptr(W2, "W2"),
                                _stream_ptr(stream), ctypes.byref(h)), "tp_moe_create")
    return h.value


def tp_moe_fwd(handle: int, X, counts, T: int, Y, stream=None) -> None:
    _check(capi().tp_moe_fwd(ctypes.c_void_p(handle), _dev_ptr(X, "X"), _dev_ptr(counts, "counts"),
                             int(T), _dev_ptr(Y, "Y"), _stream_ptr(stream)), "tp_moe_fwd")


def tp_moe_destroy(handle: int) -> None:
    _check(capi().tp_moe_destroy(ctypes.c_void_p(handle)), "tp_moe_destroy")


class GroupedExperts:
    """The experts held by one GPU as one grouped MLP.  w1: [E, d, 2F] (silu_gate:
    gate then up columns) or [E, d, F]; w2: [E, F, d]; bf16 on the GPU.  path:
    "stream" (both projections stream each expert's weights once per 128 of its
    tokens), "tiled" (256-token matrix-core tiles) or "auto" (stream when the
    tokens number at most 128 per expert)."""

    def __init__(self, w1, w2, activation="silu_gate", max_tokens=8192, out_dtype=None,
                 path="auto", stream=None):
        torch = _torch()
        if w1.dim() != 3 or w2.dim() != 3 or w1.shape[0] != w2.shape[0]:
            raise ValueError("w1 [E, d, n1] and w2 [E, F, d] with the same E")
        E, d, F = w1.shape[0], w1.shape[1], w2.shape[1]
        if w1.shape[2] != (2 * F if activation == "silu_gate" else F) or w2.shape[2] != d:
            raise ValueError("expert weight shapes do not fit activation %s" % activation)
        self.n_experts, self.d_model, self.ffn_expert = E, d, F
        self.out_dtype = out_dtype if out_dtype is not None else torch.float32
        self.max_tokens = int(max_tokens)
        self.desc = TpmMoeDesc(d, F, E, self.max_tokens, ACT[activation], _dtype_code(w1.dtype),
                               _dtype_code(self.out_dtype), PATH[path])
        self.handle = tp_moe_create(self.desc, w1, w2, stream)

    def forward(self, x, counts, out=None, stream=None):
        """x: [T, d] tokens grouped by expert; counts: int32 [E] on the GPU."""
        torch = _torch()
        if x.dim() != 2 or x.shape[1] != self.d_model or x.dtype != torch.bfloat16:
            raise ValueError("x must be [T, %d] of torch.bfloat16" % self.d_model)
        T = x.shape[0]
        if counts.dtype != torch.int32 or counts.numel() != self.n_experts:
            raise ValueError("counts must be int32 [%d]" % self.n_experts)
        if out is None:
            out = torch.zeros((T, self.d_model), dtype=self.out_dtype, device=x.device)
        elif tuple(out.shape) != (T, self.d_model) or out.dtype != self.out_dtype:
            raise ValueError("out must be [%d, %d] of %s" % (T, self.d_model, self.out_dtype))
        tp_moe_fwd(self.handle, x, counts, T, out, stream)
        return out

    __call__ = forward

    def close(self):
        if getattr(self, "handle", None):
            tp_moe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def partials_reduce(partials, out=None, out_dtype=None, stream=None):
    torch = _torch()
    parts = list(partials)
    if out is None:
        out = torch.empty_like(parts[0], dtype=out_dtype or torch.float32)
    tp_partials_reduce(parts, out, stream)
    return out


def tensor_parallel_output(x, a_shards, b_shards, activation="tanh", path="auto",
                           out_dtype=None):
    """Z = sum_i act(x @ a_i) @ b_i over matched shard pairs, all on the GPU."""
    a_shards, b_shards = list(a_shards), list(b_shards)
    if len(a_shards) != len(b_shards):
        raise ValueError("a_shards and b_shards differ in count (%d vs %d)"
                         % (len(a_shards), len(b_shards)))
    shards = [Shard(a, b, activation, max_tokens=x.shape[0], path=path) for a, b in
              zip(a_shards, b_shards)]
    try:
        partials = [s.forward(x) for s in shards]
        return partials_reduce(partials, out_dtype=out_dtype)
    finally:
        for s in shards:
            s.close()
