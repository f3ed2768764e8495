"""Seeded synthetic inputs for the rotated W4A4 linear workloads.

This module is the only code shared by the CPU oracle and the HIP path. It
draws random numbers and builds test inputs; it computes no step of the
method (no alignment, Hadamard transform, quantization or GEMM).

Recipes (reading of the workload descriptions):

* activations ``x``: bf16, entries N(0, 1); ``k`` outlier channels, the first
  ``k`` entries of a seeded permutation of ``range(D)``, are multiplied by the
  outlier factor in fp32; then one bf16 round-to-nearest-even cast.  The same
  channels are outliers for every token.
* basis ``Q``: reduced QR of a seeded N(0, 1) float64 ``D x r`` matrix, column
  signs flipped so that diag(R) > 0, cast to fp32.  Columns are orthonormal.
* sub-rotation ``M``: Cayley transform ``(I - A)^-1 (I + A)`` of a skew matrix
  ``A`` whose strict upper triangle is iid N(0, 0.02^2); float64 solve, then
  fp32.  ``M`` is orthogonal with det +1.
* weights ``W``: fp32 N(0, std^2), ``[N][K]`` (output channel major).

Every stream has its own seed: ``SeedSequence([1000 + config_id, crc32(name)])``.
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, Tuple

import numpy as np

__all__ = [
    "Linear", "Workload", "CONFIGS", "rng", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "gen_x", "gen_basis", "gen_weight", "gen_gate_up", "workload_inputs",
]


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Linear:
    """One quantized linear: ``K`` inputs, ``N`` outputs.

    ``rotate`` says that an online Hadamard transform precedes it, so its
    weight rows are Hadamard-rotated along K before quantization.
    ``swiglu`` says its input is a gate|up pair of width ``2K``.
    """
    name: str
    K: int
    N: int
    rotate: bool = False
    swiglu: bool = False


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    D: int
    T: int
    r: int
    n_outliers: int
    outlier_scale: float
    w_std: float
    kind: str                      # "linear" (align -> FWHT -> quant -> GEMM) or "layer"
    linears: Tuple[Linear, ...]
    ffn: int = 0

    @property
    def is_layer(self) -> bool:
        return self.kind == "layer"


def _layer_linears(D: int, F: int) -> Tuple[Linear, ...]:
    return (
        Linear("qkv", D, 3 * D),
        Linear("o", D, D),
        Linear("gate_up", D, 2 * F),
        Linear("down", F, D, rotate=True, swiglu=True),
    )


CONFIGS: Dict[int, Workload] = {
    0: Workload(0, "tiny D=256 T=64 r=8 256->256", 256, 64, 8, 2, 50.0, 0.02, "linear",
                (Linear("lin", 256, 256, rotate=True),)),
    1: Workload(1, "prefill linear D=4096 T=2048 r=32 4096->4096", 4096, 2048, 32, 8, 80.0, 0.02,
                "linear", (Linear("lin", 4096, 4096, rotate=True),)),
    2: Workload(2, "decode layer D=4096 T=8 r=32 FFN=16384", 4096, 8, 32, 8, 80.0, 0.02, "layer",
                _layer_linears(4096, 16384), ffn=16384),
    3: Workload(3, "prefill layer D=4096 T=4096 r=32 FFN=16384", 4096, 4096, 32, 8, 80.0, 0.02,
                "layer", _layer_linears(4096, 16384), ffn=16384),
    4: Workload(4, "large prefill linear D=8192 T=8192 r=64 8192->28672", 8192, 8192, 64, 16, 100.0,
                0.015, "linear", (Linear("lin", 8192, 28672, rotate=True),)),
}


# ----------------------------------------------------------------------------
# random streams and bf16 bit patterns
# ----------------------------------------------------------------------------
def rng(key: int, stream: str) -> np.random.Generator:
    """Independent generator for (key, stream name)."""
    return np.random.default_rng(np.random.SeedSequence([int(key), zlib.crc32(stream.encode())]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even. Finite input only."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# generators
# ----------------------------------------------------------------------------
def gen_x(key: int, T: int, D: int, n_outliers: int, outlier_scale: float,
          stream: str = "x") -> np.ndarray:
    """bf16 activations [T][D] as uint16 bit patterns."""
    g = rng(key, stream)
    x = g.standard_normal((T, D), dtype=np.float32)
    if n_outliers:
        ch = rng(key, stream + ".outliers").permutation(D)[:n_outliers]
        x[:, ch] *= np.float32(outlier_scale)
    return f32_to_bf16_bits(x)


def gen_basis(key: int, D: int, r: int, stream: str = "basis",
              skew_std: float = 0.02) -> Tuple[np.ndarray, np.ndarray]:
    """(Q fp32 [D][r] orthonormal columns, M fp32 [r][r] orthogonal, det +1)."""
    if r == 0:
        return np.zeros((D, 0), np.float32), np.zeros((0, 0), np.float32)
    g = rng(key, stream + ".Q")
    G = g.standard_normal((D, r))
    Qm, R = np.linalg.qr(G, mode="reduced")
    sgn = np.sign(np.diag(R))
    sgn[sgn == 0] = 1.0
    Qm = Qm * sgn[None, :]
    ga = rng(key, stream + ".A")
    U = np.triu(ga.normal(0.0, skew_std, size=(r, r)), k=1)
    A = U - U.T
    I = np.eye(r)
    M = np.linalg.solve(I - A, I + A)
    return Qm.astype(np.float32), M.astype(np.float32)


def gen_hadamard_transition(key: int, D: int, n_big: int, big=(0.3, 1.0),
                            small: float = 0.01) -> np.ndarray:
    """fp32 [D][D] synthetic residual transition near the identity, of the kind
    the pages describe (rotations that stay close to a shared Hadamard start):
    T = Hn G Hn^T with Hn the normalized Sylvester matrix and G block-diagonal
    plane rotations on the coordinate pairs (2k, 2k+1): n_big seeded pairs
    turn by angles in ``big``, all others by angles below ``small``. D must
    be a power of two."""
    import scipy.linalg
    g = rng(key, "transition.angles")
    theta = g.uniform(0.0, small, D // 2)
    pick = g.permutation(D // 2)[:n_big]
    theta[pick] = g.uniform(big[0], big[1], n_big)
    Hn = scipy.linalg.hadamard(D).astype(np.float64) / np.sqrt(D)
    c, s = np.cos(theta), np.sin(theta)
    # Y = G Hn^T: rotate row pairs of Hn^T (= Hn)
    Y = Hn.copy()
    Y[0::2], Y[1::2] = c[:, None] * Hn[0::2] - s[:, None] * Hn[1::2], \
        s[:, None] * Hn[0::2] + c[:, None] * Hn[1::2]
    return (Hn @ Y).astype(np.float32)


def gen_weight(key: int, N: int, K: int, std: float, stream: str = "w") -> np.ndarray:
    """fp32 weights [N][K], entries N(0, std^2)."""
    g = rng(key, stream)
    return (g.standard_normal((N, K), dtype=np.float32) * np.float32(std)).astype(np.float32)


def gen_gate_up(key: int, T: int, F: int, stream: str = "gu") -> np.ndarray:
    """bf16 gate|up pair [T][2F] (uint16 bits), entries N(0, 1); test input for the gated front."""
    g = rng(key, stream)
    return f32_to_bf16_bits(g.standard_normal((T, 2 * F), dtype=np.float32))


def workload_inputs(wl: Workload, with_weights: bool = True):
    """All inputs of a workload: dict with x, (Q, M) pair(s) and fp32 weights per linear."""
    key = 1000 + wl.cid
    out = {"x": gen_x(key, wl.T, wl.D, wl.n_outliers, wl.outlier_scale)}
    n_basis = 2 if wl.is_layer else 1
    out["basis"] = [gen_basis(key, wl.D, wl.r, stream=f"basis{i}") for i in range(n_basis)]
    if with_weights:
        out["W"] = {lin.name: gen_weight(key, lin.N, lin.K, wl.w_std, stream="w." + lin.name)
                    for lin in wl.linears}
    return out
