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
  its textbook form, which the pages name without defining).

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
