"""Parity bounds shared by the GPU tests, in the measure
err = max|got - ref| / sqrt(mean(ref^2)) (``oracle.rel_err``).

TOL_F32: fp32 inputs, fp32 arithmetic.  TOL_BF16: bf16 inputs and bf16 hidden
activations with fp32 accumulation, fp32 output.  A bf16 output is rounded once
more, by at most half an ulp (2^-8 of the value) per element, which adds
2^-8 max|ref| / rms(ref) to the bound (``tol_for``)."""
import numpy as np
import torch

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def _f64(a):
    if isinstance(a, torch.Tensor):
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def tol_for(out_dtype, ref):
    """The bf16-input bound for an output of `out_dtype` against the reference `ref`."""
    if out_dtype != torch.bfloat16:
        return TOL_BF16
    r = _f64(ref)
    rms = float(np.sqrt(np.mean(r * r)))
    return TOL_BF16 + (2.0 ** -8 * float(np.abs(r).max()) / rms if rms > 0 else 0.0)


def tol_hidden_rounding(h, b, ref):
    """Bound for shards too narrow for the rounding of the hidden activations to average
    out (one or two hidden features): the GPU rounds H to bf16 once (unit roundoff 2^-8),
    so |P_gpu - P| <= 2^-8 (|H| |B|) elementwise, plus fp32 accumulation (1e-3 of the RMS
    here).  Never below TOL_BF16.  `h` is the oracle's hidden activations [M, F], `b`
    the second weight [F, d], `ref` the oracle's partial [M, d]."""
    h = np.abs(_f64(h))
    bb = np.abs(_f64(b))
    r = _f64(ref)
    rms = float(np.sqrt(np.mean(r * r)))
    if rms == 0:
        return TOL_BF16
    return max(TOL_BF16, 2.0 ** -8 * float((h @ bb).max()) / rms + 1e-3)
