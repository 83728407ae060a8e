"""Oracle for the tensor-parallel MLP shard (fp64, plain loops in ``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the GPU library in ``tensor_mlp_shard_amd`` and imports nothing from it.

It follows the pages' statement of the method:

* page "LLM 推理并行化：先找瓶颈，再决定怎么切", section 三.2 (tensor parallel):
  for each matched pair of shards the partial is ``act(x @ a_shard) @ b_shard``,
  a count mismatch between the two shard lists is an error, and the output is the
  element-wise sum of the partials;
* page "大模型推理系统揭秘（07）Multi-GPU", sections 1.2.2-1.2.3: the first
  weight is split by columns, the second by the matching rows, and the sum of the
  rank partials equals the unsplit two-layer product;
* same page, section 1.4.3: SwiGLU applies SiLU to the gate branch and multiplies
  by the up branch;
* page "7.4 推理侧并行", section 7.4.2 (kernel fusion after the all-reduce): the
  residual add and RMSNorm that follow the sum (``reduce_add_rmsnorm``; RMSNorm in
  its textbook form, which the pages name without defining);
* same page, MoE section: an expert is the SwiGLU MLP of the tokens routed to it,
  the tokens of a GPU grouped by expert (``grouped_experts``);
* page "大模型推理系统揭秘（07）Multi-GPU", section 1.2.4: the attention block's
  QKV projection is column-parallel and its output projection row-parallel
  (``projection``, one matrix product);
* page "LLM 推理并行化：先找瓶颈，再决定怎么切", section 三.4 (decode context
  parallelism): each rank attends over its own part of the KV history and reports
  its local score maximum, its sum of exponentials and its exponential-weighted sum
  of values; the merge rescales every rank to the global maximum and divides the
  summed values by the summed exponentials (``attn_partials_merge``);
* page "7.4 推理侧并行", section 7.4.2 (communication quantization): partials travel as FP8 with a
  per-token scale and are summed in high precision (``e4m3_value``,
  ``e4m3_encode``, ``quantize_fp8``, ``reduce_fp8``).  FP8 is the OCP E4M3 format,
  written here from its definition (the pages name FP8 without fixing it).

Activation names: ``"tanh"``, ``"silu_gate"``, ``"identity"``.  For ``silu_gate``
a shard's first weight has ``2F`` columns: the ``F`` gate columns, then the ``F``
up columns over the same hidden indices.

Pins (what ties this oracle to something other than itself) live in
``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

ACT_CODES = {"tanh": 0, "silu_gate": 1, "identity": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc and OpenMP."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.orc_shard_forward.argtypes = [dp, ctypes.c_int64, ctypes.c_int64, dp,
                                          ctypes.c_int64, dp, ctypes.c_int64, ctypes.c_int, dp]
        lib.orc_shard_forward.restype = ctypes.c_int
        lib.orc_partials_sum.argtypes = [ctypes.POINTER(dp), ctypes.c_int32,
                                         ctypes.c_int64, dp]
        lib.orc_partials_sum.restype = ctypes.c_int
        lib.orc_matmul.argtypes = [dp, ctypes.c_int64, ctypes.c_int64, dp, ctypes.c_int64, dp]
        lib.orc_matmul.restype = ctypes.c_int
        lib.orc_num_threads.argtypes = []
        lib.orc_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    """Exact widening to a C-contiguous float64 array (fp32 and bf16 values are exact in fp64)."""
    if hasattr(a, "detach"):  # a torch tensor: widen through float32 (exact for bf16/fp16)
        a = a.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().orc_num_threads())


def _check_shapes(X, A, B, activation):
    if X.ndim != 2 or A.ndim != 2 or B.ndim != 2:
        raise ValueError("x, a_shard and b_shard must be 2-D")
    d = X.shape[1]
    F = B.shape[0]
    ncol = 2 * F if activation == "silu_gate" else F
    if A.shape != (d, ncol):
        raise ValueError("shape mismatch: x %s, a %s, b %s (activation %s)"
                         % (X.shape, A.shape, B.shape, activation))
    return X.shape[0], d, F, B.shape[1]


def shard_forward(x, a_shard, b_shard, activation: str = "tanh") -> np.ndarray:
    """One rank's partial ``act(x @ a_shard) @ b_shard`` in fp64, shape [M, N]
    (N = d for the MLP block)."""
    act = ACT_CODES[activation]
    X, A, B = _f64(x), _f64(a_shard), _f64(b_shard)
    M, d, F, N = _check_shapes(X, A, B, activation)
    P = np.zeros((M, N), dtype=np.float64)
    rc = _load().orc_shard_forward(_ptr(X), M, d, _ptr(A), F, _ptr(B), N, act, _ptr(P))
    if rc != 0:
        raise RuntimeError("orc_shard_forward failed with code %d" % rc)
    return P


def partials_sum(partials) -> np.ndarray:
    """Element-wise sum of the rank partials, in rank order, fp64."""
    parts = [_f64(p) for p in partials]
    if not parts:
        raise ValueError("need at least one partial")
    shape = parts[0].shape
    for p in parts:
        if p.shape != shape:
            raise ValueError("partials differ in shape")
    Z = np.zeros(shape, dtype=np.float64)
    arr = (ctypes.POINTER(ctypes.c_double) * len(parts))(*[_ptr(p) for p in parts])
    rc = _load().orc_partials_sum(arr, len(parts), Z.size, _ptr(Z))
    if rc != 0:
        raise RuntimeError("orc_partials_sum failed with code %d" % rc)
    return Z


def tensor_parallel_output(x, a_shards, b_shards, activation: str = "tanh") -> np.ndarray:
    """Sum over matched shard pairs of ``act(x @ a_i) @ b_i``; a count mismatch raises."""
    a_shards, b_shards = list(a_shards), list(b_shards)
    if len(a_shards) != len(b_shards):
        raise ValueError("a_shards and b_shards differ in count (%d vs %d)"
                         % (len(a_shards), len(b_shards)))
    partials = [shard_forward(x, a, b, activation) for a, b in zip(a_shards, b_shards)]
    return partials_sum(partials)


def unsplit_weights(a_shards, b_shards, activation: str = "tanh"):
    """Reassemble the full first and second weights from rank shards.

    The first weight's column blocks and the second weight's row blocks are laid
    side by side in rank order.  For ``silu_gate`` the gate halves and the up halves
    are gathered separately, so the result again holds all gate columns, then all
    up columns.
    """
    As = [_f64(a) for a in a_shards]
    Bs = [_f64(b) for b in b_shards]
    if activation == "silu_gate":
        gates = [a[:, : a.shape[1] // 2] for a in As]
        ups = [a[:, a.shape[1] // 2:] for a in As]
        A = np.concatenate(gates + ups, axis=1)
    else:
        A = np.concatenate(As, axis=1)
    B = np.concatenate(Bs, axis=0)
    return A, B


def unsplit_output(x, a_shards, b_shards, activation: str = "tanh") -> np.ndarray:
    """The same MLP computed without splitting: one shard holding all hidden features."""
    A, B = unsplit_weights(a_shards, b_shards, activation)
    return shard_forward(x, A, B, activation)


def grouped_experts(x, counts, w1s, w2s, activation: str = "silu_gate") -> np.ndarray:
    """The experts of one GPU (page "大模型推理系统揭秘（07）Multi-GPU", MoE section):
    rows [o_e, o_e + n_e) of x, o_e = n_0 + ... + n_{e-1}, go through expert e's MLP
    act(x_e @ w1_e) @ w2_e; returns all rows in order, fp64."""
    X = _f64(x)
    out = np.zeros((X.shape[0], _f64(w2s[0]).shape[1]), dtype=np.float64)
    off = 0
    for n, a, b in zip(counts, w1s, w2s):
        n = int(n)
        if n:
            out[off:off + n] = shard_forward(X[off:off + n], a, b, activation)
        off += n
    if off != X.shape[0]:
        raise ValueError("counts sum to %d, x has %d rows" % (off, X.shape[0]))
    return out


def projection(x, w) -> np.ndarray:
    """One projection ``x @ w`` in fp64 (page "大模型推理系统揭秘（07）Multi-GPU",
    section 1.2.2: Y = XW; column shards of W give column blocks of Y, row shards of
    W with the matching column blocks of X give partials that sum to Y)."""
    X, W = _f64(x), _f64(w)
    if X.ndim != 2 or W.ndim != 2 or X.shape[1] != W.shape[0]:
        raise ValueError("shapes %s and %s do not chain" % (X.shape, W.shape))
    Y = np.zeros((X.shape[0], W.shape[1]), dtype=np.float64)
    rc = _load().orc_matmul(_ptr(X), X.shape[0], X.shape[1], _ptr(W), W.shape[1], _ptr(Y))
    if rc != 0:
        raise RuntimeError("orc_matmul failed with code %d" % rc)
    return Y


def reduce_add_rmsnorm(partials, residual, gamma, eps: float):
    """The step after the all-reduce, in fp64: for each row,
    ``h = residual + sum_i partials[i]`` (rank order) and
    ``y = h / sqrt(mean(h^2) + eps) * gamma``.  Returns ``(h, y)``, both [rows, cols].
    """
    z = partials_sum(partials)
    R = _f64(residual)
    g = _f64(gamma)
    if R.shape != z.shape or R.ndim != 2 or g.shape != (R.shape[1],):
        raise ValueError("residual must match the partials, gamma must be [cols]")
    h = R + z
    ms = np.mean(h * h, axis=1, keepdims=True)
    y = h / np.sqrt(ms + float(eps)) * g[None, :]
    return h, y


def attn_partials_merge(values, maxima, expsums):
    """Merge of k attention partials, in fp64 (page "LLM 推理并行化", section 三.4).

    ``values[i]`` [rows, dim], ``maxima[i]`` and ``expsums[i]`` [rows]: rank i's
    exponential-weighted value sum, local score maximum and sum of exponentials,
    both taken relative to that maximum.  In the page's order: the global maximum
    over the ranks, each rank's scale ``exp(m_i - max)``, the denominator
    ``sum_i scale_i * s_i`` and numerator ``sum_i scale_i * v_i`` (rank order), and
    their quotient.  Returns ``(out [rows, dim], max [rows], expsum [rows])``: the
    merged output and the merged statistics (the denominator is the merged sum of
    exponentials relative to the global maximum), so a merged result can be
    merged again.  A row with no keys on any rank (every maximum -inf) is taken as
    an empty attention: output 0, maximum -inf, sum 0.
    """
    if not (len(values) == len(maxima) == len(expsums)) or not values:
        raise ValueError("need matching, non-empty lists of partials")
    v = [_f64(x) for x in values]
    m = [_f64(x) for x in maxima]
    e = [_f64(x) for x in expsums]
    rows, dim = v[0].shape
    for vi, mi, ei in zip(v, m, e):
        if vi.shape != (rows, dim) or mi.shape != (rows,) or ei.shape != (rows,):
            raise ValueError("partials must be [rows, dim] with [rows] statistics")
    gmax = m[0].copy()
    for mi in m[1:]:
        gmax = np.maximum(gmax, mi)
    empty = np.isneginf(gmax)
    ref = np.where(empty, 0.0, gmax)  # any finite reference for empty rows
    scales = [np.where(np.isneginf(mi), 0.0, np.exp(mi - ref)) for mi in m]
    den = np.zeros(rows)
    num = np.zeros((rows, dim))
    for sc, ei, vi in zip(scales, e, v):
        den = den + sc * ei
        num = num + sc[:, None] * vi
    safe = np.where(empty | (den == 0.0), 1.0, den)
    out = np.where(empty[:, None], 0.0, num / safe[:, None])
    return out, gmax, np.where(empty, 0.0, den)


def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 byte: sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 is subnormal (m / 8 * 2^-6); 0x7f and 0xff are NaN."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3_POS = np.array([e4m3_value(c) for c in range(0x7F)], dtype=np.float64)  # codes 0..126


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code), saturating to
    +-448; NaN gives 0x7f.  Works on the exact values given (no rescaling): the
    magnitude is located in the table of the 127 non-negative finite values and
    the nearer neighbour is taken."""
    a = np.asarray(x, dtype=np.float64)
    mag = np.abs(a)
    nan = np.isnan(a)
    m = np.where(nan, 0.0, mag)
    hi = np.clip(np.searchsorted(_E4M3_POS, m, side="left"), 1, len(_E4M3_POS) - 1)
    lo = hi - 1
    dl = m - _E4M3_POS[lo]
    dh = _E4M3_POS[hi] - m
    code = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(m >= _E4M3_POS[-1], 0x7E, code)
    sign = np.where(np.signbit(a), 0x80, 0)
    out = np.where(nan, 0x7F, sign | code)
    return out.astype(np.uint8)


def quantize_fp8(x):
    """Per-row FP8 quantization of a partial [rows, cols] given in fp32 or bf16:
    amax per row, scale = amax / 448 and codes of x * (448 / amax), each of the
    two divisions and the product taken in fp32 with correct rounding (the
    precision the codes are decided in).  Zero rows: scale 1, all codes 0.
    Returns (codes uint8 [rows, cols], scales float32 [rows])."""
    X = np.asarray(_f64(x), dtype=np.float32)  # exact: the inputs are fp32 or bf16
    rows = X.shape[0]
    codes = np.zeros(X.shape, dtype=np.uint8)
    scales = np.ones(rows, dtype=np.float32)
    for r in range(rows):
        amax = np.float32(np.max(np.abs(X[r]))) if X.shape[1] else np.float32(0)
        if not amax > 0:
            continue
        inv = np.float32(448.0) / amax
        scales[r] = amax / np.float32(448.0)
        codes[r] = e4m3_encode((X[r] * inv).astype(np.float32))
    return codes, scales


def reduce_fp8(codes, scales) -> np.ndarray:
    """Sum over ranks of value(code_i) * scale_i[row], in fp64, rank order."""
    table = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
    total = None
    for q, s in zip(codes, scales):
        d = table[np.asarray(q, dtype=np.uint8)] * np.asarray(s, dtype=np.float64)[:, None]
        total = d if total is None else total + d
    return total


def rel_err(got, ref) -> float:
    """max|got - ref| / sqrt(mean(ref^2)), the error measure the parity tests use."""
    g = _f64(got)
    r = _f64(ref)
    if g.shape != r.shape:
        raise ValueError("shape mismatch %s vs %s" % (g.shape, r.shape))
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    diff = float(np.max(np.abs(g - r)))
    if rms == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return diff / rms


def timed_shard_forward(x, a_shard, b_shard, activation: str = "tanh"):
    """``shard_forward`` plus the wall time of the compute call alone (seconds)."""
    act = ACT_CODES[activation]
    X, A, B = _f64(x), _f64(a_shard), _f64(b_shard)
    M, d, F, N = _check_shapes(X, A, B, activation)
    P = np.zeros((M, N), dtype=np.float64)
    lib = _load()
    t0 = time.perf_counter()
    rc = lib.orc_shard_forward(_ptr(X), M, d, _ptr(A), F, _ptr(B), N, act, _ptr(P))
    t1 = time.perf_counter()
    if rc != 0:
        raise RuntimeError("orc_shard_forward failed with code %d" % rc)
    return P, t1 - t0
