"""Python binding of librotw4a4 (gfx950): the rotated W4A4 linear data path.

Argument marshalling only: every step runs in the HIP library behind the C ABI
declared in include/rotw4a4.h. PyTorch provides device memory and streams.
The functions keep the ABI's names; they take CUDA (HIP) tensors and enqueue
on torch's current stream. There is no CPU fallback: without the built
library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "RW4_ALIGN", "RW4_FWHT", "RW4_SWIGLU", "RW4_WPACKED", "Rw4Error", "lib", "library_path",
    "respin_align", "fwht", "quant_act_int4", "w4a4_gemm", "rotated_linear",
    "rotated_linear_workspace_size", "respin_align_workspace_size", "workspace_views",
    "respin_basis_size", "respin_prepare_basis", "rotated_linear_prepared",
    "respin_align_prepared", "respin_align_prepared_workspace_size",
    "rotated_linear_prepared_workspace_size",
    "w4a4_tiles_size", "w4a4_tile_codes", "w4a4_gemm_tiles", "prep_weight", "layer",
    "quant_act_sym", "RW4_ABITS", "RW4_KRON", "RW4_HEADS", "hadamard_transform", "head_hadamard",
    "respin_construct", "respin_construct_workspace_size", "rotated_linear_prepared_noalloc",
    "NOALLOC_SCRATCH_BYTES", "respin_align_project_prepared", "respin_align_project_size",
    "rotated_linear_prepared_residual", "rotated_linear_prepared_project",
]

RW4_ALIGN, RW4_FWHT, RW4_SWIGLU = 1, 2, 4
RW4_WPACKED = 1 << 29     # weights as packed INT4 rows [N][K/2] instead of FP6 tiles


def RW4_ABITS(bits: int) -> int:
    """rotated_linear flag field for b-bit activation codes (b = 2, 3, 4)."""
    return bits << 8


def RW4_KRON(m: int) -> int:
    """rotated_linear flag field (with RW4_FWHT): H_{2^n} (x) H_m, m = 12, 20, 28."""
    return m << 16


def RW4_HEADS(n_h: int) -> int:
    """rotated_linear flag field: the transform across n_h heads (a power of two)."""
    if n_h < 2 or n_h & (n_h - 1):
        raise ValueError("n_h must be a power of two >= 2")
    return (n_h.bit_length() - 1) << 24
_BF16, _F32, _I32 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "librotw4a4.so")
_lib = None

EXPORTS = ("respin_align", "respin_align_workspace_size", "fwht", "quant_act_int4",
           "quant_act_sym", "w4a4_gemm",
           "w4a4_tiles_size", "w4a4_tile_codes", "w4a4_gemm_tiles", "rotated_linear",
           "rotated_linear_workspace_size", "respin_basis_size", "respin_prepare_basis",
           "rotated_linear_prepared", "rotated_linear_prepared_workspace_size",
           "respin_align_prepared", "respin_align_prepared_workspace_size",
           "hadamard_transform", "head_hadamard", "respin_construct",
           "respin_construct_workspace_size", "rotated_linear_prepared_noalloc",
           "respin_align_project_prepared", "respin_align_project_size",
           "rotated_linear_prepared_residual", "rotated_linear_prepared_project", "rw4_align256",
           "rw4_status_string", "rw4_abi_version")


class Rw4Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the HIP library (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(
            f"{library_path} is missing: build it with "
            "`python -m rotation_w4a4_quantized_amd.build` (no CPU fallback exists)")
    L = ctypes.CDLL(library_path)
    vp, i64, u32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint, ctypes.c_size_t
    i32 = ctypes.c_int
    L.respin_align.argtypes = [vp, i32, vp, i32, vp, vp, vp, i64, i64, i64, vp, sz, vp]
    L.respin_align_workspace_size.argtypes = [i64, i64, i64]
    L.respin_align_workspace_size.restype = sz
    L.fwht.argtypes = [vp, i32, vp, i64, i64, vp]
    L.quant_act_int4.argtypes = [vp, i32, vp, vp, i64, i64, vp]
    L.quant_act_sym.argtypes = [vp, i32, vp, vp, i64, i64, i32, vp]
    L.w4a4_gemm.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    L.w4a4_tiles_size.argtypes = [i64, i64]
    L.w4a4_tiles_size.restype = sz
    L.w4a4_tile_codes.argtypes = [vp, i64, i64, vp, vp, vp]
    L.w4a4_gemm_tiles.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i64, vp]
    L.rotated_linear.argtypes = [vp, i64, i64, i64, vp, vp, i64, u32, vp, vp, i64, vp, vp, sz,
                                 vp, vp]
    L.rotated_linear_workspace_size.argtypes = [i64, i64, i64, u32]
    L.rotated_linear_workspace_size.restype = sz
    L.respin_basis_size.argtypes = [i64, i64]
    L.respin_basis_size.restype = sz
    L.respin_prepare_basis.argtypes = [vp, vp, i64, i64, vp, sz, vp]
    L.rotated_linear_prepared.argtypes = [vp, i64, i64, i64, vp, i64, u32, vp, vp, i64, vp, vp,
                                          sz, vp, vp]
    L.rotated_linear_prepared_noalloc.argtypes = [vp, i64, i64, i64, vp, i64, u32, vp, vp, i64,
                                                  vp, vp, vp]
    L.respin_align_project_prepared.argtypes = [vp, i64, i64, vp, i64, vp, sz, vp]
    L.respin_align_project_size.argtypes = [i64, i64, i64]
    L.respin_align_project_size.restype = sz
    L.rotated_linear_prepared_residual.argtypes = [vp, i64, i64, i64, vp, i64, u32, vp, vp, i64,
                                                   vp, vp, sz, vp, vp, vp, i64, vp, sz, vp, vp]
    L.rotated_linear_prepared_project.argtypes = [vp, i64, i64, i64, vp, i64, u32, vp, vp, i64,
                                                  vp, vp, sz, vp, vp, i64, vp, sz, vp]
    L.rotated_linear_prepared_workspace_size.argtypes = [i64, i64, i64, u32]
    L.rotated_linear_prepared_workspace_size.restype = sz
    L.respin_align_prepared.argtypes = [vp, vp, i32, vp, vp, i64, i64, i64, vp, sz, vp]
    L.respin_align_prepared_workspace_size.argtypes = [i64, i64, i64]
    L.respin_align_prepared_workspace_size.restype = sz
    L.hadamard_transform.argtypes = [vp, i32, i64, vp, i64, i64, i64, vp, vp]
    L.respin_construct.argtypes = [vp, i64, i64, i32, vp, vp, vp, sz, vp]
    L.respin_construct_workspace_size.argtypes = [i64, i64]
    L.respin_construct_workspace_size.restype = sz
    L.head_hadamard.argtypes = [vp, i32, i64, vp, i64, i64, i64, vp]
    L.rw4_align256.argtypes = [sz]
    L.rw4_align256.restype = sz
    L.rw4_status_string.argtypes = [i32]
    L.rw4_status_string.restype = ctypes.c_char_p
    L.rw4_abi_version.restype = i32
    for f in ("respin_align", "fwht", "quant_act_int4", "quant_act_sym", "w4a4_gemm",
              "w4a4_tile_codes",
              "w4a4_gemm_tiles", "rotated_linear", "respin_prepare_basis",
              "rotated_linear_prepared", "rotated_linear_prepared_noalloc",
              "respin_align_prepared", "respin_align_project_prepared",
              "rotated_linear_prepared_residual", "rotated_linear_prepared_project",
              "hadamard_transform",
              "head_hadamard", "respin_construct"):
        getattr(L, f).restype = i32
    _lib = L
    return L


# ---------------------------------------------------------------- helpers
def _torch():
    import torch
    return torch


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _check(fn: str, st: int):
    if st != 0:
        raise Rw4Error(fn, st, lib().rw4_status_string(st).decode())


def _fdt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise TypeError(f"expected bf16 or fp32 tensor, got {t.dtype}")


def _rows(x):
    if x.dim() != 2 or not x.is_cuda:
        raise ValueError("expected a 2-D CUDA tensor [T][D]")
    if x.numel() and x.stride(1) != 1:
        raise ValueError("rows must be contiguous")


def _contig(x):
    _rows(x)
    if x.numel() and not x.is_contiguous():
        raise ValueError("expected a contiguous tensor")


# ---------------------------------------------------------------- entry points
def respin_align_workspace_size(T: int, D: int, r: int) -> int:
    return int(lib().respin_align_workspace_size(T, D, r))


def respin_align(x, Q, M, out=None, addend=None, out_dtype=None, workspace=None, direct=False):
    """out = x + Q (M - I) Q^T x (+ addend), per token row; see include/rotw4a4.h.

    With bf16 x (and D % 32 == 0) it runs on matrix cores using ``workspace``
    (allocated here if not given); ``direct=True`` selects the fp32-FMA kernel."""
    torch = _torch()
    _contig(x)
    T, D = x.shape
    r = Q.shape[1] if Q is not None else 0
    if out is None:
        out = torch.empty((T, D), dtype=out_dtype or torch.float32, device=x.device)
    if addend is not None:
        _contig(addend)
        if addend.dtype != out.dtype or addend.shape != out.shape:
            raise ValueError("addend must match out in dtype and shape")
    if r > 0:
        if Q.dtype != torch.float32 or M.dtype != torch.float32:
            raise TypeError("Q and M must be fp32")
        Q, M = Q.contiguous(), M.contiguous()
    need = 0 if direct else respin_align_workspace_size(T, D, r)
    if need and workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    if not need:
        workspace = None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().respin_align(_p(x), _fdt(x), _p(out), _fdt(out), _p(Q) if r else None,
                            _p(M) if r else None, _p(addend), T, D, r, _p(workspace), nbytes,
                            _stream())
    _check("respin_align", st)
    return out


def respin_align_prepared_workspace_size(T: int, D: int, r: int) -> int:
    return int(lib().respin_align_prepared_workspace_size(T, D, r))


def respin_align_prepared(x, basis, r: int, out=None, addend=None, out_dtype=None,
                          workspace=None):
    """``respin_align`` with a basis from ``respin_prepare_basis`` (rank r) in
    place of (Q, M); x bf16 [T][D]. Returns out."""
    torch = _torch()
    _contig(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bf16")
    T, D = x.shape
    if basis.numel() * basis.element_size() < respin_basis_size(D, r):
        raise ValueError("basis: buffer too small for (D, r)")
    if out is None:
        out = torch.empty((T, D), dtype=out_dtype or torch.float32, device=x.device)
    if addend is not None:
        _contig(addend)
        if addend.dtype != out.dtype or addend.shape != out.shape:
            raise ValueError("addend must match out in dtype and shape")
    need = respin_align_prepared_workspace_size(T, D, r)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    st = lib().respin_align_prepared(_p(x), _p(out), _fdt(out), _p(basis), _p(addend), T, D, r,
                                     _p(workspace), workspace.numel() * workspace.element_size(),
                                     _stream())
    _check("respin_align_prepared", st)
    return out


def respin_align_project_size(T: int, D: int, r: int) -> int:
    return int(lib().respin_align_project_size(T, D, r))


def respin_align_project_prepared(x, basis, r: int, z=None):
    """The projection half of ``respin_align_prepared`` for short batches
    (1 <= T <= 16): z for ``rotated_linear_prepared_residual``. Returns z."""
    torch = _torch()
    _contig(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bf16")
    T, D = x.shape
    if basis.numel() * basis.element_size() < respin_basis_size(D, r):
        raise ValueError("basis: buffer too small for (D, r)")
    need = respin_align_project_size(T, D, r)
    if z is None:
        z = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    st = lib().respin_align_project_prepared(_p(x), T, D, _p(basis), r, _p(z),
                                             z.numel() * z.element_size(), _stream())
    _check("respin_align_project_prepared", st)
    return z


def fwht(x, out=None):
    """Normalized Walsh-Hadamard transform of every row -> fp32 (in place if out is x)."""
    torch = _torch()
    _contig(x)
    T, D = x.shape
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    st = lib().fwht(_p(x), _fdt(x), _p(out), T, D, _stream())
    _check("fwht", st)
    return out


def hadamard_transform(x, m: int = 1, signs=None, out=None, D: int = None):
    """(H_{2^n} (x) H_m) diag(signs) x / sqrt(D) for every row -> fp32 [T][D]
    (H_m by Paley's construction, m = 12, 20, 28; m = 1 the plain transform).
    x may be row-strided; D defaults to its width; out may be x (fp32)."""
    torch = _torch()
    _rows(x)
    T = x.shape[0]
    D = x.shape[1] if D is None else D
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    if signs is not None and (signs.dtype != torch.float32 or signs.numel() != D
                              or not signs.is_cuda or not signs.is_contiguous()):
        raise ValueError("signs: contiguous fp32 [D] on the device")
    st = lib().hadamard_transform(_p(x), _fdt(x), x.stride(0), _p(out), T, D, m, _p(signs),
                                  _stream())
    _check("hadamard_transform", st)
    return out


def head_hadamard(x, n_h: int, out=None):
    """(H_{n_h} (x) I_{d_h}) x / sqrt(n_h) for every row -> fp32 [T][D]."""
    torch = _torch()
    _rows(x)
    T, D = x.shape
    if D % n_h:
        raise ValueError("D must be a multiple of n_h")
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    st = lib().head_hadamard(_p(x), _fdt(x), x.stride(0), _p(out), T, n_h, D // n_h, _stream())
    _check("head_hadamard", st)
    return out


def quant_act_int4(x, codes=None, scales=None) -> Tuple:
    """Per-row absmax INT4: (codes uint8 [T][D/2], scales fp32 [T])."""
    torch = _torch()
    _contig(x)
    T, D = x.shape
    if codes is None:
        codes = torch.empty((T, D // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((T,), dtype=torch.float32, device=x.device)
    st = lib().quant_act_int4(_p(x), _fdt(x), _p(codes), _p(scales), T, D, _stream())
    _check("quant_act_int4", st)
    return codes, scales


def quant_act_sym(x, bits: int, codes=None, scales=None) -> Tuple:
    """Per-row absmax b-bit codes (b = 2, 3, 4) stored as INT4 nibbles:
    (codes uint8 [T][D/2], scales fp32 [T])."""
    torch = _torch()
    _contig(x)
    T, D = x.shape
    if codes is None:
        codes = torch.empty((T, D // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((T,), dtype=torch.float32, device=x.device)
    st = lib().quant_act_sym(_p(x), _fdt(x), _p(codes), _p(scales), T, D, bits, _stream())
    _check("quant_act_sym", st)
    return codes, scales


def w4a4_gemm(a, s_a, w, s_w, out=None, out_dtype=None):
    """y = bf16(acc * s_a[t] * s_w[n]) or raw int32 acc (out_dtype=torch.int32)."""
    torch = _torch()
    _contig(a)
    _contig(w)
    T, KB = a.shape
    N = w.shape[0]
    if w.shape[1] != KB:
        raise ValueError("a and w must have the same K")
    odt = out_dtype or (out.dtype if out is not None else torch.bfloat16)
    if out is None:
        out = torch.empty((T, N), dtype=odt, device=a.device)
    ydt = _I32 if odt == torch.int32 else _BF16
    st = lib().w4a4_gemm(_p(a), _p(s_a), _p(w), _p(s_w), _p(out), ydt, T, 2 * KB, N, _stream())
    _check("w4a4_gemm", st)
    return out


def w4a4_tiles_size(R: int, K: int) -> int:
    """Bytes of the FP6 tile form of an [R][K] code matrix (layout in include/rotw4a4.h)."""
    return int(lib().w4a4_tiles_size(R, K))


def w4a4_tile_codes(codes, tiles=None, check: bool = True):
    """Packed INT4 rows uint8 [R][K/2] -> FP6 tiles (flat uint8). With ``check``
    the call synchronizes and raises if any code was -8 (no FP6 value)."""
    torch = _torch()
    _contig(codes)
    R, KB = codes.shape
    K = 2 * KB
    n = w4a4_tiles_size(R, K)
    if n == 0 and R > 0:
        raise Rw4Error("w4a4_tile_codes", -2, lib().rw4_status_string(-2).decode())
    if tiles is None:
        tiles = torch.empty((max(n, 16),), dtype=torch.uint8, device=codes.device)
    bad = torch.zeros((1,), dtype=torch.int32, device=codes.device) if check else None
    st = lib().w4a4_tile_codes(_p(codes), R, K, _p(tiles), _p(bad), _stream())
    _check("w4a4_tile_codes", st)
    if check and int(bad.item()) != 0:
        raise ValueError("w4a4_tile_codes: code -8 has no FP6 value (codes must lie in [-7, 7])")
    return tiles


def w4a4_gemm_tiles(a, s_a, w, s_w, T: int, K: int, N: int, out=None, out_dtype=None):
    """The W4A4 GEMM on FP6 tiles: bf16(acc * s_a[t] * s_w[n]) or int32 acc."""
    torch = _torch()
    for name, t, R in (("a", a, T), ("w", w, N)):
        if t.numel() * t.element_size() < w4a4_tiles_size(R, K):
            raise ValueError(f"{name}: tile buffer too small")
    odt = out_dtype or (out.dtype if out is not None else torch.bfloat16)
    if out is None:
        out = torch.empty((T, N), dtype=odt, device=a.device)
    ydt = _I32 if odt == torch.int32 else _BF16
    st = lib().w4a4_gemm_tiles(_p(a), _p(s_a), _p(w), _p(s_w), _p(out), ydt, T, K, N, _stream())
    _check("w4a4_gemm_tiles", st)
    return out


def _check_weights(w, N: int, D: int, flags: int):
    need = N * D // 2 if flags & RW4_WPACKED else w4a4_tiles_size(N, D)
    if w.numel() * w.element_size() < need:
        raise ValueError("w: weight buffer too small for [N][D] (packed INT4 rows with "
                         "RW4_WPACKED, FP6 tiles otherwise)")


def rotated_linear_workspace_size(T: int, D: int, r: int, flags: int) -> int:
    return int(lib().rotated_linear_workspace_size(T, D, r, flags))


def rotated_linear(x, w, s_w, flags: int, Q=None, M=None, out=None, workspace=None,
                   dbg_prequant=None):
    """[align] -> [SiLU gate] -> [FWHT] -> INT4 quant -> W4A4 GEMM -> bf16 [T][N].

    ``x`` is bf16 [T][D] (or [T][2D] with RW4_SWIGLU); a row-strided view is
    allowed. ``w`` holds the weight codes as FP6 tiles (``prep_weight`` /
    ``w4a4_tile_codes``), ``s_w`` their fp32 scales [N]. Returns (y,
    workspace); the workspace holds the activation tiles and scales after the
    call (layout in include/rotw4a4.h).
    """
    torch = _torch()
    _rows(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bf16")
    T = x.shape[0]
    D = x.shape[1] // 2 if flags & RW4_SWIGLU else x.shape[1]
    N = s_w.shape[0]
    _check_weights(w, N, D, flags)
    r = Q.shape[1] if (flags & RW4_ALIGN) and Q is not None else 0
    need = rotated_linear_workspace_size(T, D, r, flags)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    st = lib().rotated_linear(_p(x), x.stride(0), T, D, _p(Q) if r else None,
                              _p(M) if r else None, r, flags, _p(w), _p(s_w), N, _p(out),
                              _p(workspace), workspace.numel() * workspace.element_size(),
                              _p(dbg_prequant), _stream())
    _check("rotated_linear", st)
    return out, workspace


def respin_construct_workspace_size(D: int, r: int) -> int:
    return int(lib().respin_construct_workspace_size(D, r))


def respin_construct(T, r: int, iters: int = 4, workspace=None):
    """(Q fp32 [D][r], R_sub fp32 [r][r]) of a residual transition T fp32 [D][D]:
    the top-r left singular vectors of T - I and the polar factor of Q^T T Q."""
    torch = _torch()
    _contig(T)
    if T.dtype != torch.float32 or T.shape[0] != T.shape[1]:
        raise TypeError("T must be a square fp32 matrix")
    D = T.shape[0]
    need = respin_construct_workspace_size(D, r)
    if need == 0:
        raise Rw4Error("respin_construct", -2, lib().rw4_status_string(-2).decode())
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=T.device)
    Q = torch.empty((D, r), dtype=torch.float32, device=T.device)
    R = torch.empty((r, r), dtype=torch.float32, device=T.device)
    st = lib().respin_construct(_p(T), D, r, iters, _p(Q), _p(R), _p(workspace),
                                workspace.numel() * workspace.element_size(), _stream())
    _check("respin_construct", st)
    return Q, R


def respin_basis_size(D: int, r: int) -> int:
    return int(lib().respin_basis_size(D, r))


def respin_prepare_basis(Q, M, basis=None):
    """The alignment's per-layer basis from Q fp32 [D][r] and M fp32 [r][r]
    (flat uint8 device buffer, layout internal to the library)."""
    torch = _torch()
    _contig(Q)
    _contig(M)
    D, r = Q.shape
    n = respin_basis_size(D, r)
    if n == 0:
        raise Rw4Error("respin_prepare_basis", -2, lib().rw4_status_string(-2).decode())
    if basis is None:
        basis = torch.empty((n,), dtype=torch.uint8, device=Q.device)
    st = lib().respin_prepare_basis(_p(Q), _p(M), D, r, _p(basis),
                                    basis.numel() * basis.element_size(), _stream())
    _check("respin_prepare_basis", st)
    return basis


def rotated_linear_prepared_workspace_size(T: int, D: int, r: int, flags: int) -> int:
    return int(lib().rotated_linear_prepared_workspace_size(T, D, r, flags))


def rotated_linear_prepared(x, w, s_w, flags: int, basis=None, r: int = 0, out=None,
                            workspace=None, dbg_prequant=None):
    """``rotated_linear`` with a basis from ``respin_prepare_basis`` (r = its
    rank) in place of (Q, M). Returns (y, workspace)."""
    torch = _torch()
    _rows(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bf16")
    T = x.shape[0]
    D = x.shape[1] // 2 if flags & RW4_SWIGLU else x.shape[1]
    N = s_w.shape[0]
    _check_weights(w, N, D, flags)
    r = r if flags & RW4_ALIGN else 0
    if r and basis.numel() * basis.element_size() < respin_basis_size(D, r):
        raise ValueError("basis: buffer too small for (D, r)")
    need = rotated_linear_prepared_workspace_size(T, D, r, flags)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    st = lib().rotated_linear_prepared(_p(x), x.stride(0), T, D, _p(basis) if r else None, r,
                                       flags, _p(w), _p(s_w), N, _p(out), _p(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _p(dbg_prequant), _stream())
    _check("rotated_linear_prepared", st)
    return out, workspace


def rotated_linear_prepared_residual(x, w, s_w, flags: int, res_x, res_basis, res_r: int, res_z,
                                     basis=None, r: int = 0, out=None, res_out=None,
                                     workspace=None, dbg_prequant=None):
    """``rotated_linear_prepared`` (packed INT4 weights, 1 <= T <= 16) whose
    product also finishes the residual alignment of ``res_x`` (projection
    ``res_z`` from ``respin_align_project_prepared``): res_out = bf16(res_x +
    Q z + y), bit for bit ``respin_align_prepared(res_x, ..., addend=y)``.
    Returns (y, res_out, workspace)."""
    torch = _torch()
    _rows(x)
    _contig(res_x)
    if x.dtype != torch.bfloat16 or res_x.dtype != torch.bfloat16:
        raise TypeError("x and res_x must be bf16")
    T = x.shape[0]
    D = x.shape[1] // 2 if flags & RW4_SWIGLU else x.shape[1]
    N = s_w.shape[0]
    if tuple(res_x.shape) != (T, N):
        raise ValueError("res_x must be [T][N]")
    _check_weights(w, N, D, flags)
    r = r if flags & RW4_ALIGN else 0
    need = rotated_linear_prepared_workspace_size(T, D, r, flags)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    if res_out is None:
        res_out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    st = lib().rotated_linear_prepared_residual(
        _p(x), x.stride(0), T, D, _p(basis) if r else None, r, flags, _p(w), _p(s_w), N,
        _p(out), _p(workspace), workspace.numel() * workspace.element_size(), _p(dbg_prequant),
        _p(res_x), _p(res_basis), res_r, _p(res_z), res_z.numel() * res_z.element_size(),
        _p(res_out), _stream())
    _check("rotated_linear_prepared_residual", st)
    return out, res_out, workspace


def rotated_linear_prepared_project(x, w, s_w, flags: int, proj_basis, proj_r: int, out=None,
                                    proj_z=None, workspace=None, dbg_prequant=None):
    """``rotated_linear_prepared`` (1 <= T <= 16, contiguous x, no alignment
    in the unit) that also writes ``respin_align_project_prepared(x,
    proj_basis, proj_r)``. Returns (y, proj_z, workspace)."""
    torch = _torch()
    _contig(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bf16")
    T, D = x.shape
    N = s_w.shape[0]
    _check_weights(w, N, D, flags)
    need = rotated_linear_prepared_workspace_size(T, D, 0, flags)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    if proj_z is None:
        proj_z = torch.empty((max(respin_align_project_size(T, D, proj_r), 256),),
                             dtype=torch.uint8, device=x.device)
    st = lib().rotated_linear_prepared_project(
        _p(x), x.stride(0), T, D, None, 0, flags, _p(w), _p(s_w), N, _p(out), _p(workspace),
        workspace.numel() * workspace.element_size(), _p(dbg_prequant), _p(proj_basis), proj_r,
        _p(proj_z), proj_z.numel() * proj_z.element_size(), _stream())
    _check("rotated_linear_prepared_project", st)
    return out, proj_z, workspace


NOALLOC_SCRATCH_BYTES = 64 << 20   # RW4_NOALLOC_SCRATCH_BYTES of include/rotw4a4.h


def rotated_linear_prepared_noalloc(x, w, s_w, flags: int, basis=None, r: int = 0, out=None,
                                    dbg_prequant=None):
    """``rotated_linear_prepared`` without a workspace: the library's own
    per-GPU scratch array holds the intermediates, and the call allocates no
    device memory (``out`` must then be given). Calls that overlap on one GPU
    race. Returns y."""
    torch = _torch()
    _rows(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bf16")
    T = x.shape[0]
    D = x.shape[1] // 2 if flags & RW4_SWIGLU else x.shape[1]
    N = s_w.shape[0]
    _check_weights(w, N, D, flags)
    r = r if flags & RW4_ALIGN else 0
    if r and basis.numel() * basis.element_size() < respin_basis_size(D, r):
        raise ValueError("basis: buffer too small for (D, r)")
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    st = lib().rotated_linear_prepared_noalloc(_p(x), x.stride(0), T, D,
                                               _p(basis) if r else None, r, flags, _p(w),
                                               _p(s_w), N, _p(out), _p(dbg_prequant), _stream())
    _check("rotated_linear_prepared_noalloc", st)
    return out


def workspace_views(workspace, T: int, D: int, packed: bool = False):
    """(activation codes, scales fp32 [T]) inside a rotated_linear workspace: the
    codes as FP6 tiles (flat uint8), or as packed INT4 rows uint8 [T][D/2] for a
    call with RW4_WPACKED."""
    n = w4a4_tiles_size(T, D)
    off = int(lib().rw4_align256(n))
    codes = workspace[:T * D // 2].view(T, D // 2) if packed else workspace[:n]
    scales = workspace[off: off + 4 * T].view(_torch().float32)
    return codes, scales


def prep_weight(W, rotate: bool, bits: int = 4, m: int = 1, signs=None):
    """Offline weight preparation on the GPU: optional row-wise Hadamard along K
    (fwht; H_{2^n} (x) H_m and random signs with hadamard_transform), per-output-
    channel b-bit codes (quant_act_sym), then FP6 tiles.
    W fp32 [N][K]. Returns (tiles, s_w, codes [N][K/2], rotated W)."""
    _contig(W)
    if rotate:
        src = fwht(W) if m == 1 and signs is None else hadamard_transform(W, m, signs)
    else:
        src = W
    codes, s_w = quant_act_sym(src, bits)
    tiles = w4a4_tile_codes(codes)
    return tiles, s_w, codes, src


def layer(x0, aligns, weights, D: int, dbg_down=None, packed: bool = False):
    """One decoder layer's quantized path (each token attends only to itself):
    qkv = L(x0); o = L(V part of qkv); x1 = bf16(align1(x0) + o);
    gu = L(x1); d = L_down(FWHT(SiLU(g) * u)); x2 = bf16(align2(x1) + d).
    ``aligns``: ((basis1, r1), (basis2, r2)), each alignment's basis from
    ``respin_prepare_basis`` (prepared once per layer) with its rank.
    ``weights``: name -> (tiles, s_w) for qkv, o, gate_up, down; with
    ``packed`` (codes, s_w), the packed INT4 rows (RW4_WPACKED: the decode
    format).
    ``dbg_down``: optional fp32 [T][D_ffn] that receives the down projection's
    pre-quant values. Returns a dict of every stage's output tensor, plus
    "down_ws", the down projection's workspace (its activation tiles and
    scales, see ``workspace_views``)."""
    torch = _torch()
    (B1, r1), (B2, r2) = aligns
    st = {}
    wf = RW4_WPACKED if packed else 0
    T = x0.shape[0]
    if packed and 1 <= T <= 16:
        # short batches: each alignment's projection runs with the quantizer
        # of the same input, and the product that makes the residual's addend
        # finishes the alignment in its epilogue (the same bits as the
        # sequence below)
        st["qkv"], z1, _ = rotated_linear_prepared_project(x0, *weights["qkv"], wf, B1, r1)
        st["o"], st["x1"], _ = rotated_linear_prepared_residual(
            st["qkv"][:, 2 * D:3 * D], *weights["o"], wf, x0, B1, r1, z1)
        st["gate_up"], z2, _ = rotated_linear_prepared_project(st["x1"], *weights["gate_up"], wf,
                                                               B2, r2)
        st["down"], st["x2"], st["down_ws"] = rotated_linear_prepared_residual(
            st["gate_up"], *weights["down"], RW4_SWIGLU | RW4_FWHT | wf, st["x1"], B2, r2, z2,
            dbg_prequant=dbg_down)
        return st
    st["qkv"], _ = rotated_linear(x0, *weights["qkv"], flags=wf)
    st["o"], _ = rotated_linear(st["qkv"][:, 2 * D:3 * D], *weights["o"], flags=wf)
    st["x1"] = respin_align_prepared(x0, B1, r1, addend=st["o"], out_dtype=torch.bfloat16)
    st["gate_up"], _ = rotated_linear(st["x1"], *weights["gate_up"], flags=wf)
    st["down"], st["down_ws"] = rotated_linear(st["gate_up"], *weights["down"],
                                               flags=RW4_SWIGLU | RW4_FWHT | wf,
                                               dbg_prequant=dbg_down)
    st["x2"] = respin_align_prepared(st["x1"], B2, r2, addend=st["down"],
                                     out_dtype=torch.bfloat16)
    return st
