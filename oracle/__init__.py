"""CPU oracle for the rotated W4A4 linear data path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library never
calls it, and it shares no code with the HIP path; the only common module is
the seeded input generator (``workloads``), which computes no step of the
method.

Plain, slow, obviously correct NumPy.  Floating-point stages run in float64;
the quantizer runs in float32 because its integer decisions must be taken in
the precision the kernel uses (the pages fix no precision for it).

Sources (web pages; cited as [key, section]):

* [RSQ]  "ReSpinQuant: Efficient Layer-Wise LLM Quantization via Subspace
  Residual Rotation Approximation" -- paper notes (m0rtzz).  Sections
  "整体框架" (framework flowchart) and "关键设计" 1-3.
* [QS]   "QuaRot 与 SpinQuant" (lizn-zn scholia log).  §1.2 (rotation as a basis
  change), §1.3 (worked 4x4 Hadamard example), §2.2 (why Hadamard).
* [IQ2]  "Infra Quant II" (taking-lying-flat).  QuaRot "Background" and
  "Method" (online Hadamard before the down projection; activation, weight
  and GEMM quantization), SpinQuant "MOTIVATION" (symmetric quantizer),
  FlatQuant "Preliminaries" (signed b-bit grid, Y = (XH)(H^T W^T)).

Where the pages are silent or ambiguous, the reading taken is stated next to
the code it shapes.

Pins: every function below is pinned by ``tests/test_oracle_pins.py`` against
something other than itself (worked example, closed forms, library routines,
invariants, brute force); ``residual`` against the dense T_hat and a case that
tells one bf16 rounding from two.  The pages give no SiLU value; ``silu_gate``
is pinned against SciPy's logistic function (``scipy.special.expit``, a
library routine) and the closed forms SiLU(0) = 0 and SiLU(g) - SiLU(-g) = g.
A decoder layer is not an oracle function: the layer tests feed each oracle
stage the GPU's own previous stage.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64", "f64_to_bf16", "align", "align_dense", "t_hat", "construct_basis", "fwht",
    "hadamard",
    "quant_sym", "quant_int4", "pack_int4", "unpack_int4", "gemm_int", "gemm_int_loop",
    "epilogue", "silu_gate", "prep_weight", "prequant", "rotated_linear", "residual",
    "quadratic_character", "jacobsthal", "paley_hadamard", "hadamard_kron", "head_hadamard",
    "FLAG_ALIGN", "FLAG_FWHT", "FLAG_SWIGLU", "FLAG_KRON_SHIFT", "FLAG_HEADS_SHIFT",
]

FLAG_ALIGN = 1
FLAG_FWHT = 2
FLAG_SWIGLU = 4
FLAG_KRON_SHIFT = 16     # with FLAG_FWHT: H_{2^n} (x) H_m, m in bits 16..23
FLAG_HEADS_SHIFT = 24    # H_{n_h} (x) I across heads, log2(n_h) in bits 24..28


# ----------------------------------------------------------------------------
# bf16 values
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even) in one rounding, as uint16 bit patterns.

    bf16 keeps 8 significant bits and fp32's exponent range; below 2^-126 the
    spacing is fixed at 2^-133.  Finite inputs only.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                         # v = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                    # subnormal range: fixed spacing 2^-133
    q = np.rint(np.ldexp(v, 8 - e))            # integer count of units 2^(e-8); half-even
    r = np.ldexp(q, e - 8)
    r32 = r.astype(np.float32)                 # exact: r has <= 8 significant bits
    return (r32.view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# S1: low-rank residual alignment  [RSQ 关键设计 2, 3; framework flowchart]
# ----------------------------------------------------------------------------
def align(x: np.ndarray, Q: np.ndarray, M: np.ndarray) -> np.ndarray:
    """Online residual alignment, the three-step path of [RSQ 关键设计 3].

    Per token (rows of ``x``): project to the r-dim subspace y = Q^T x, apply
    the small matrix z = (M - I_r) y, lift and add: out = x + Q z.

    ``M`` is the orthogonal sub-rotation R_sub; the page folds the identity
    into its small matrix (its M is R_sub - I_r), so the step applies M - I.
    With r = 0 the path is the identity.
    """
    x = np.asarray(x, np.float64)
    Q = np.asarray(Q, np.float64)
    M = np.asarray(M, np.float64)
    r = Q.shape[1]
    y = x @ Q                                   # row t: (Q^T x_t)^T
    z = y @ (M - np.eye(r)).T                   # row t: ((M - I) y_t)^T
    return x + z @ Q.T                          # row t: x_t + Q z_t


def t_hat(Q: np.ndarray, M: np.ndarray) -> np.ndarray:
    """Dense aligned transition T_hat = I + Q (M - I) Q^T  [RSQ 关键设计 2]."""
    Q = np.asarray(Q, np.float64)
    M = np.asarray(M, np.float64)
    D, r = Q.shape
    return np.eye(D) + Q @ (M - np.eye(r)) @ Q.T


def construct_basis(T: np.ndarray, r: int):
    """Offline (Q, R_sub) of a residual transition T = R_out R_in^T, the steps of
    [RSQ 关键设计 2] in order:
      1. Delta T = T - I;
      2. its SVD; Q = the top-r left singular vectors ([D][r]);
      3. T_sub = Q^T T Q (r x r);
      4. polar decomposition of T_sub = U_sub S V_sub^T: R_sub = U_sub V_sub^T.
    T_hat = I + Q (R_sub - I) Q^T (t_hat) is then orthogonal. Q is unique up
    to a rotation inside degenerate singular subspaces (the planes of T come
    in pairs of equal singular values); T_hat depends only on span(Q).
    Returns (Q, R_sub, singular values of Delta T), float64."""
    T = np.asarray(T, np.float64)
    D = T.shape[0]
    U, S, _ = np.linalg.svd(T - np.eye(D))
    Q = U[:, :r]
    Tsub = Q.T @ T @ Q
    Us, _, Vts = np.linalg.svd(Tsub)
    return Q, Us @ Vts, S


def align_dense(x: np.ndarray, Q: np.ndarray, M: np.ndarray) -> np.ndarray:
    """Brute force: materialize T_hat and multiply every token by it."""
    return np.asarray(x, np.float64) @ t_hat(Q, M).T


# ----------------------------------------------------------------------------
# S2: Walsh-Hadamard transform  [QS §2.2; IQ2 QuaRot Background]
# ----------------------------------------------------------------------------
def hadamard(D: int) -> np.ndarray:
    """Normalized Walsh-Hadamard matrix of order D = 2^n, natural (Sylvester) order.

    Entry (i, j) is (-1)^popcount(i & j) / sqrt(D)  (entries +-1/sqrt(D) per
    [IQ2 QuaRot Background]; Sylvester order as in the printed H_4 of [QS §1.3]).
    """
    i = np.arange(D)
    bits = np.bitwise_and.outer(i, i)
    par = np.zeros_like(bits)
    while bits.any():
        par ^= bits & 1
        bits >>= 1
    return np.where(par == 1, -1.0, 1.0) / np.sqrt(D)


def fwht(v: np.ndarray) -> np.ndarray:
    """Fast Walsh-Hadamard transform of every row, normalized: H_D v / sqrt(D).

    Butterflies (a, b) -> (a + b, a - b) on index pairs (i, i + h) inside
    blocks of 2h, for h = 1, 2, 4, ..., D/2; O(D log D)  [QS §2.2;
    IQ2 QuaRot Background].  The last dimension must be a power of two.
    """
    a = np.array(v, dtype=np.float64, copy=True)
    D = a.shape[-1]
    if D & (D - 1) or D < 1:
        raise ValueError("FWHT size must be a power of two")
    lead = a.shape[:-1]
    h = 1
    while h < D:
        b = a.reshape(lead + (D // (2 * h), 2, h))
        lo = b[..., 0, :].copy()
        hi = b[..., 1, :].copy()
        b[..., 0, :] = lo + hi
        b[..., 1, :] = lo - hi
        h *= 2
    return a / np.sqrt(D)


# ----------------------------------------------------------------------------
# Structured Hadamard transforms  [IQ2 QuaRot Background, QuaRot Method]
# ----------------------------------------------------------------------------
def _is_prime(q: int) -> bool:
    return q >= 2 and all(q % d for d in range(2, int(q ** 0.5) + 1))


def quadratic_character(q: int) -> np.ndarray:
    """chi over the integers mod a prime q: chi(0) = 0, chi(a) = +1 if a is a
    nonzero square mod q, else -1 (the Legendre symbol)."""
    if not _is_prime(q) or q == 2:
        raise ValueError("odd prime q required")
    chi = -np.ones(q, dtype=np.int64)
    chi[0] = 0
    for y in range(1, q):
        chi[(y * y) % q] = 1
    return chi


def jacobsthal(q: int) -> np.ndarray:
    """Jacobsthal matrix of a prime q: J[a][b] = chi(a - b mod q)."""
    chi = quadratic_character(q)
    a = np.arange(q)
    return chi[(a[:, None] - a[None, :]) % q]


def paley_hadamard(m: int) -> np.ndarray:
    """A +-1 Hadamard matrix of order m by Paley's construction (the pages need
    one of non-power-of-two order m [IQ2 QuaRot Background] and print none).

    * Paley I, q = m - 1 prime with q = 3 (mod 4): the Jacobsthal matrix J is
      skew, S = [[0, 1^T], [-1, J]] (index 0 first, then 0..q-1 of the
      integers mod q), H = I + S.
    * Paley II, q = m/2 - 1 prime with q = 1 (mod 4): J is symmetric,
      C = [[0, 1^T], [1, J]], H = C (x) [[1, 1], [1, -1]] + I (x) [[1, -1], [-1, -1]].
    """
    if m >= 4 and _is_prime(m - 1) and (m - 1) % 4 == 3:
        q = m - 1
        S = np.zeros((m, m), dtype=np.int64)
        S[0, 1:] = 1
        S[1:, 0] = -1
        S[1:, 1:] = jacobsthal(q)
        return np.eye(m, dtype=np.int64) + S
    if m % 2 == 0 and m >= 4 and _is_prime(m // 2 - 1) and (m // 2 - 1) % 4 == 1:
        q = m // 2 - 1
        C = np.zeros((q + 1, q + 1), dtype=np.int64)
        C[0, 1:] = 1
        C[1:, 0] = 1
        C[1:, 1:] = jacobsthal(q)
        A = np.array([[1, 1], [1, -1]], dtype=np.int64)
        B = np.array([[1, -1], [-1, -1]], dtype=np.int64)
        return np.kron(C, A) + np.kron(np.eye(q + 1, dtype=np.int64), B)
    raise ValueError(f"no Paley construction of order {m} over a prime field")


def hadamard_kron(v: np.ndarray, m: int, signs=None) -> np.ndarray:
    """(H_{2^n} (x) H_m) diag(s) v / sqrt(D) for every row, D = 2^n m
    [IQ2 QuaRot Background: H_d = H_{2^n} (x) H_m for d = 2^n m, and the
    randomized H diag(s) with s in {+1, -1}^d]. m = 1 is the plain WHT; H_m
    for m > 1 is paley_hadamard(m). Index f = i m + j (i < 2^n, j < m), so
    the row as a 2^n x m matrix V becomes H_{2^n} V H_m^T."""
    a = np.array(v, dtype=np.float64, copy=True)
    D = a.shape[-1]
    if D % m:
        raise ValueError("D must be a multiple of m")
    A = D // m
    if signs is not None:
        a = a * np.asarray(signs, dtype=np.float64)
    V = a.reshape(a.shape[:-1] + (A, m))
    if m > 1:
        V = V @ paley_hadamard(m).T.astype(np.float64)
    # H_{2^n} along i: the normalized transform of the columns, times sqrt(A)
    V = np.swapaxes(fwht(np.swapaxes(V, -1, -2)), -1, -2) * np.sqrt(A)
    return V.reshape(a.shape) / np.sqrt(D)


def head_hadamard(v: np.ndarray, n_h: int) -> np.ndarray:
    """(H_{n_h} (x) I_{d_h}) v / sqrt(n_h) for every row, d_h = D / n_h: the
    online transform across attention heads before the output projection
    [IQ2 QuaRot Method, value projection: Z <- Z (H_{n_h} (x) I), by reshaping
    and a Walsh-Hadamard transform; H_{n_h} is symmetric, so the row form
    equals the column form]."""
    a = np.array(v, dtype=np.float64, copy=True)
    D = a.shape[-1]
    if D % n_h:
        raise ValueError("D must be a multiple of n_h")
    V = a.reshape(a.shape[:-1] + (n_h, D // n_h))
    V = np.swapaxes(fwht(np.swapaxes(V, -1, -2)), -1, -2)
    return V.reshape(a.shape)


# ----------------------------------------------------------------------------
# S3: symmetric absmax quantization  [IQ2 SpinQuant MOTIVATION; QuaRot Method]
# ----------------------------------------------------------------------------
def quant_sym(v: np.ndarray, bits: int = 4):
    """Per-row symmetric absmax quantization to signed ``bits``-bit integers.

    Step alpha = max|row| / (2^(bits-1) - 1)  [IQ2 SpinQuant MOTIVATION,
    symmetric case]; code = round(row / alpha)  [IQ2 QuaRot Method: per-token,
    absmax / 7 for 4 bits]; projected onto the signed grid
    {-2^(bits-1), ..., 2^(bits-1) - 1}  [IQ2 FlatQuant Preliminaries].

    Decided in float32 (the kernel's precision): alpha = fl32(absmax / qmax)
    with IEEE division; quotient fl32(v / alpha) rounded to fp32 before it is
    rounded to an integer; integer rounding is half-to-even.  An all-zero row
    gets alpha = 0 and codes 0.
    Returns (codes int8 [..., D], alpha float32 [...]).
    """
    v = np.asarray(v, dtype=np.float32)
    qmax = (1 << (bits - 1)) - 1
    qmin = -(1 << (bits - 1))
    a = np.max(np.abs(v), axis=-1)                          # exact in fp32
    s = (a / np.float32(qmax)).astype(np.float32)           # IEEE fp32 division
    safe = np.where(s == 0, np.float32(1), s).astype(np.float32)
    qf = (v / safe[..., None]).astype(np.float32)           # fp32 quotient
    q = np.clip(np.rint(qf), qmin, qmax)
    q = np.where((s == 0)[..., None], 0, q)
    return q.astype(np.int8), s


def quant_int4(v: np.ndarray):
    """4-bit case of ``quant_sym``: step absmax / 7, grid {-8..7}."""
    return quant_sym(v, 4)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, element 2j in the low nibble of byte j."""
    q = np.asarray(q, dtype=np.int16)
    if q.shape[-1] % 2:
        raise ValueError("row length must be even")
    lo = (q[..., 0::2] & 0xF).astype(np.uint8)
    hi = (q[..., 1::2] & 0xF).astype(np.uint8)
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    p = np.asarray(p, dtype=np.uint8).astype(np.int16)
    lo = p & 0xF
    hi = p >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ----------------------------------------------------------------------------
# S4: integer GEMM and dequantization  [IQ2 QuaRot Method]
# ----------------------------------------------------------------------------
def gemm_int(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[t, n] = sum_k qa[t, k] * qw[n, k], exact, as int32.

    A float64 matrix product of integer-valued matrices is exact here: every
    partial sum is an integer of magnitude <= 64 K < 2^53.
    """
    qa = np.asarray(qa)
    qw = np.asarray(qw)
    if qa.shape[-1] * 64 >= 2 ** 53:
        raise ValueError("K too large for exact float64 accumulation")
    acc = qa.astype(np.float64) @ qw.astype(np.float64).T
    return acc.astype(np.int64).astype(np.int32)


def gemm_int_loop(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """Triple loop over integers (tiny shapes only)."""
    T, K = qa.shape
    N = qw.shape[0]
    out = np.zeros((T, N), np.int64)
    for t in range(T):
        for n in range(N):
            s = 0
            for k in range(K):
                s += int(qa[t, k]) * int(qw[n, k])
            out[t, n] = s
    return out.astype(np.int32)


def epilogue(acc: np.ndarray, s_a: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """Dequantize: acc * (row scale of the activation) * (column scale of the weight),
    then one rounding to bf16  [IQ2 QuaRot Method; bf16 output]."""
    y = (np.asarray(acc, np.float64) * np.asarray(s_a, np.float64)[:, None]
         * np.asarray(s_w, np.float64)[None, :])
    return f64_to_bf16(y)


# ----------------------------------------------------------------------------
# S5: gated FFN front  (SiLU(gate) * up; the Hadamard goes after the gating)
# ----------------------------------------------------------------------------
def silu_gate(gu: np.ndarray) -> np.ndarray:
    """h = SiLU(g) * u with g, u the first and second halves of each row, float64.

    SiLU(g) = g / (1 + exp(-g)).  A rotation cannot cross the SiLU [QS §2.1],
    so the online Hadamard is applied to h, before the down projection
    [IQ2 QuaRot Method].
    """
    gu = np.asarray(gu, np.float64)
    F = gu.shape[-1] // 2
    g = gu[..., :F]
    u = gu[..., F:]
    return g / (1.0 + np.exp(-g)) * u


# ----------------------------------------------------------------------------
# chains
# ----------------------------------------------------------------------------
def prep_weight(W: np.ndarray, rotate: bool, bits: int = 4, m: int = 1, signs=None):
    """Offline weight preparation: optional Hadamard rotation of every row along K
    (the online Hadamard's inverse folded into the weight, [IQ2 QuaRot Method]:
    with x' = H x online, W' = W H^T, i.e. every row w becomes H w; H may be the
    Kronecker H_{2^n} (x) H_m and randomized by signs), then per-output-channel
    symmetric quantization (rows of W [N][K]).
    Returns (codes int8 [N][K], s_w float32 [N], the fp32 values that were quantized)."""
    if rotate:
        Wr = (fwht(W) if m == 1 and signs is None else hadamard_kron(W, m, signs)).astype(np.float32)
    else:
        Wr = np.asarray(W, np.float32)
    q, s = quant_sym(Wr, bits)
    return q, s, Wr


def prequant(x: np.ndarray, flags: int, Q=None, M=None) -> np.ndarray:
    """float64 values that reach the activation quantizer.

    ``x`` is float64 [T][D] (or [T][2D] gate|up with FLAG_SWIGLU).  Order:
    align -> gate -> Hadamard, as selected by ``flags``; the Hadamard is H_D
    (power-of-two D), H_{2^n} (x) H_m (m in the FLAG_KRON_SHIFT field), or
    the transform across heads (log2 n_h in the FLAG_HEADS_SHIFT field).
    """
    v = np.asarray(x, np.float64)
    m = (flags >> FLAG_KRON_SHIFT) & 0xFF
    lg = (flags >> FLAG_HEADS_SHIFT) & 0x1F
    if flags & FLAG_ALIGN:
        v = align(v, Q, M)
    if flags & FLAG_SWIGLU:
        v = silu_gate(v)
    if flags & FLAG_FWHT:
        v = hadamard_kron(v, m) if m else fwht(v)
    if lg:
        v = head_hadamard(v, 1 << lg)
    return v


def rotated_linear(x_bits: np.ndarray, flags: int, wq: np.ndarray, s_w: np.ndarray,
                   Q=None, M=None, bits: int = 4):
    """Whole unit on bf16 input bits: pre-quant values -> fp32 -> per-token
    ``bits``-bit codes (4: INT4; 3: the W3A3 setting [RSQ 实验]) -> integer GEMM
    -> dequantized bf16.  Returns a dict of every stage."""
    v = prequant(bf16_to_f64(x_bits), flags, Q, M)
    v32 = v.astype(np.float32)
    qa, s_a = quant_sym(v32, bits)
    acc = gemm_int(qa, wq)
    y = epilogue(acc, s_a, s_w)
    return {"prequant": v, "prequant32": v32, "codes": qa, "s_a": s_a, "acc": acc, "y": y}


def residual(x_bits: np.ndarray, Q, M, addend_bits: np.ndarray) -> np.ndarray:
    """bf16(align(x) + addend): the aligned skip plus the block output, one rounding.

    The alignment acts on the residual stream [RSQ framework flowchart: the
    transition sits on the skip connection between two blocks]; the block
    output joins after it, and the sum is rounded to bf16 once, from float64."""
    return f64_to_bf16(align(bf16_to_f64(x_bits), Q, M) + bf16_to_f64(addend_bits))
