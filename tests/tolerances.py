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


def tol_for(out_dtype, ref):
    """The bf16-input bound for an output of `out_dtype` against the reference `ref`."""
    if out_dtype != torch.bfloat16:
        return TOL_BF16
    r = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(r * r)))
    return TOL_BF16 + (2.0 ** -8 * float(np.abs(r).max()) / rms if rms > 0 else 0.0)
