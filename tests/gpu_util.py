"""Helpers of the GPU parity tests: host <-> device transfer and the tolerances.

Tolerances:
* fp32 stages (align, FWHT, pre-quant values): per-token normwise error
  max_i |g - o| / max_i |o| <= 1e-5 against the float64 oracle;
* bf16 outputs of an fp32 computation: |g - o| <= 1e-2 |o| elementwise
  (one bf16 ulp is at most 2^-7 relative);
* integer results (codes, scales, int32 accumulators): bit-exact, with the
  oracle fed the GPU's own fp32 inputs of that stage.
"""
import sys

import numpy as np

FP32_TOL = 1e-5
BF16_TOL = 1e-2


def torch():
    import torch as _t
    return _t


def dev(a: np.ndarray, dtype=None):
    t = torch()
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16).copy()).view(t.bfloat16).cuda()
    x = t.from_numpy(np.ascontiguousarray(a)).cuda()
    return x if dtype is None else x.to(dtype)


def host(x) -> np.ndarray:
    t = torch()
    x = x.detach()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def normwise(g: np.ndarray, o: np.ndarray) -> float:
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    den = np.maximum(np.abs(o).max(axis=-1), 1e-300)
    return float((np.abs(g - o).max(axis=-1) / den).max())


def bf16_rel(g_bits: np.ndarray, o_bits: np.ndarray, tol: float = BF16_TOL):
    import oracle
    g = oracle.bf16_to_f64(g_bits)
    o = oracle.bf16_to_f64(o_bits)
    bad = np.abs(g - o) > tol * np.abs(o)
    return int(bad.sum()), float(np.max(np.abs(g - o) / np.maximum(np.abs(o), 1e-30)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
