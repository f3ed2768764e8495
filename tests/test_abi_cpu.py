"""The C ABI library on the CPU: it loads, exports what the header declares, and
rejects invalid arguments on the host before any device work (no GPU calls)."""
import ctypes
import os
import re

import pytest

import rotation_w4a4_quantized_amd as rw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rotw4a4.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "return")))


def test_library_built_and_loads():
    assert os.path.exists(rw.library_path), "build the HIP library first"
    L = rw.lib()
    assert L.rw4_abi_version() == 13


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(rw.EXPORTS), names
    L = ctypes.CDLL(rw.library_path)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = rw.lib()
    for code, text in [(0, b"ok"), (-1, b"invalid argument"), (-3, b"pointer not 16-byte aligned"),
                       (-4, b"workspace missing or too small"), (-5, b"HIP runtime error at launch")]:
        assert L.rw4_status_string(code) == text
    assert L.rw4_status_string(7) == b"unknown status"


def test_workspace_size():
    L = rw.lib()
    assert L.rw4_align256(1) == 256 and L.rw4_align256(256) == 256 and L.rw4_align256(0) == 0
    T, D = 2048, 4096
    assert L.w4a4_tiles_size(T, D) == T * D * 3 // 4          # 2048 rows: already a multiple of 256
    assert L.w4a4_tiles_size(1, 64) == 256 * 64 * 3 // 4      # rows padded to 256
    assert L.w4a4_tiles_size(257, 128) == 512 * 128 * 3 // 4
    assert L.w4a4_tiles_size(4, 96) == 0 and L.w4a4_tiles_size(4, 32) == 0
    assert L.w4a4_tiles_size(-1, 64) == 0 and L.w4a4_tiles_size(0, 64) == 0
    base = L.rw4_align256(L.w4a4_tiles_size(T, D)) + L.rw4_align256(4 * T)
    assert L.rotated_linear_workspace_size(T, D, 32, 0) == base
    assert L.rotated_linear_workspace_size(T, D, 32, 2) == base
    aws = L.respin_align_workspace_size(T, D, 32)
    assert aws > 0
    # projection parts: D / 512 parts x T tokens x r padded to 32, fp32
    zpart = L.rw4_align256((D // 512) * T * 32 * 4)
    assert L.rotated_linear_prepared_workspace_size(T, D, 32, 3) == base + zpart
    assert L.rotated_linear_prepared_workspace_size(T, D, 32, 2) == base
    assert L.rotated_linear_workspace_size(T, D, 32, 3) == (
        base + zpart + L.rw4_align256(L.respin_basis_size(D, 32)))
    # D = 8192 is past the fused prologue: aligned rows go through an fp32 buffer
    T8, D8 = 64, 8192
    base8 = L.rw4_align256(L.w4a4_tiles_size(T8, D8)) + L.rw4_align256(4 * T8)
    assert L.rotated_linear_prepared_workspace_size(T8, D8, 64, 3) == (
        base8 + L.rw4_align256(16 * T8 * 64 * 4) + 4 * T8 * D8)
    assert L.rotated_linear_workspace_size(T, D, 0, 3) == base
    assert L.rotated_linear_workspace_size(-1, D, 0, 0) == 0
    assert L.rotated_linear_workspace_size(4, 7, 0, 0) == 0
    assert L.rotated_linear_workspace_size(4, 32, 0, 0) == 0   # tiles need D >= 64
    # matrix-core alignment needs D % 64 == 0
    assert L.respin_align_workspace_size(4, 1000, 12) == 0


def test_basis_size():
    L = rw.lib()
    # bf16 hi/lo of the projection operand [r padded to 16][D] (twice: rows,
    # and in the projection's fragment order) and of Q [D][r padded to 32],
    # plus the Hadamard image of Q (hi/lo, [D][r padded to 32]) for D a power
    # of two in [256, 4096] with r <= 64
    assert L.respin_basis_size(4096, 32) == 8 * (4096 * 32 * 2)
    assert L.respin_basis_size(8192, 64) == 6 * (8192 * 64 * 2)
    assert L.respin_basis_size(256, 8) == 4 * (256 * 16 * 2) + 4 * (256 * 32 * 2)
    assert L.respin_basis_size(4096, 0) == 0 and L.respin_basis_size(4096, 6) == 0
    assert L.respin_basis_size(4096, 132) == 0 and L.respin_basis_size(1000, 8) == 0
    assert L.respin_basis_size(64, 68) == 0


# fake, 256-byte aligned addresses: validation must reject before dereferencing
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)
C = ctypes.c_void_p(0x30000)
Dp = ctypes.c_void_p(0x40000)
ODD = ctypes.c_void_p(0x10004)
NUL = None
INV, UNS, MIS, WSE = -1, -2, -3, -4


@pytest.mark.parametrize("args,expect", [
    ((NUL, 0, B, 1, C, Dp, NUL, 4, 64, 8, NUL, 0, NUL), INV),        # null x
    ((A, 0, B, 1, NUL, Dp, NUL, 4, 64, 8, NUL, 0, NUL), INV),        # null Q with r > 0
    ((A, 5, B, 1, C, Dp, NUL, 4, 64, 8, NUL, 0, NUL), INV),          # bad dtype
    ((A, 0, B, 1, C, Dp, NUL, -1, 64, 8, NUL, 0, NUL), INV),         # negative T
    ((A, 0, B, 1, C, Dp, NUL, 4, 64, 6, NUL, 0, NUL), UNS),          # r % 4
    ((A, 0, B, 1, C, Dp, NUL, 4, 64, 132, NUL, 0, NUL), UNS),        # r > 128
    ((A, 0, B, 1, C, Dp, NUL, 4, 60, 8, NUL, 0, NUL), UNS),          # D % 8
    ((ODD, 0, B, 1, C, Dp, NUL, 4, 64, 8, NUL, 0, NUL), MIS),        # misaligned x
    ((A, 0, A, 1, C, Dp, NUL, 4, 64, 8, NUL, 0, NUL), INV),          # out aliases x
    ((A, 0, B, 1, C, Dp, NUL, 0, 64, 8, NUL, 0, NUL), 0),            # T = 0: valid, nothing launched
    ((A, 0, B, 1, C, Dp, NUL, 4, 64, 8, C, 16, NUL), WSE),           # workspace too small
    ((A, 0, B, 1, C, Dp, NUL, 4, 64, 8, ODD, 1 << 20, NUL), WSE),    # workspace misaligned
])
def test_respin_align_validation(args, expect):
    assert rw.lib().respin_align(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((A, 0, B, 4, 12, NUL), UNS),            # D not a power of two
    ((A, 0, B, 4, 65536, NUL), UNS),         # D too large
    ((A, 0, B, 4, 1, NUL), UNS),             # D too small
    ((A, 0, A, 4, 64, NUL), INV),            # in place needs fp32 input
    ((A, 2, B, 4, 64, NUL), INV),            # int32 input
    ((ODD, 1, B, 4, 64, NUL), MIS),
    ((A, 1, A, 0, 64, NUL), 0),              # T = 0 in place
    ((NUL, 1, NUL, 0, 64, NUL), 0),          # empty call: pointers not inspected
])
def test_fwht_validation(args, expect):
    assert rw.lib().fwht(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((A, 0, B, NUL, 4, 64, NUL), INV),
    ((A, 0, B, C, 4, 63, NUL), UNS),
    ((A, 0, B, C, 4, 0, NUL), UNS),
    ((A, 0, ODD, C, 4, 64, NUL), MIS),
    ((A, 0, B, C, 0, 64, NUL), 0),
    ((NUL, 0, NUL, NUL, 0, 64, NUL), 0),     # empty call: pointers not inspected
])
def test_quant_validation(args, expect):
    assert rw.lib().quant_act_int4(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((A, B, C, Dp, A, 0, 4, 48, 16, NUL), UNS),     # K % 32
    ((A, B, C, Dp, A, 0, 4, 262144, 16, NUL), UNS), # K too large for int32 accumulators
    ((A, NUL, C, Dp, A, 0, 4, 64, 16, NUL), INV),   # bf16 output needs scales
    ((A, NUL, C, NUL, A, 2, 0, 64, 16, NUL), 0),    # int32 output needs none; T = 0
    ((NUL, NUL, NUL, NUL, NUL, 0, 0, 64, 16, NUL), 0),  # empty call: pointers not inspected
    ((A, B, C, Dp, A, 1, 4, 64, 16, NUL), INV),     # fp32 output not offered
    ((A, B, C, Dp, A, 0, 4, 64, 0, NUL), INV),      # N = 0
    ((A, B, ODD, Dp, A, 0, 4, 64, 16, NUL), MIS),
])
def test_gemm_validation(args, expect):
    assert rw.lib().w4a4_gemm(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((A, 4, 96, B, NUL, NUL), UNS),                 # K % 64
    ((A, 4, 32, B, NUL, NUL), UNS),                 # K < 64
    ((A, -1, 64, B, NUL, NUL), INV),
    ((NUL, 4, 64, B, NUL, NUL), INV),
    ((ODD, 4, 64, B, NUL, NUL), MIS),
    ((A, 4, 64, B, ctypes.c_void_p(0x20002), NUL), MIS),   # flag word alignment
    ((NUL, 0, 64, NUL, NUL, NUL), 0),               # empty call
])
def test_tile_codes_validation(args, expect):
    assert rw.lib().w4a4_tile_codes(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((A, B, C, Dp, A, 0, 4, 96, 16, NUL), UNS),     # K % 64
    ((A, B, C, Dp, A, 0, 4, 262144, 16, NUL), UNS), # K too large for exact fp32 sums
    ((A, NUL, C, Dp, A, 0, 4, 64, 16, NUL), INV),   # bf16 output needs scales
    ((A, NUL, C, NUL, A, 2, 0, 64, 16, NUL), 0),    # T = 0
    ((NUL, NUL, NUL, NUL, NUL, 0, 0, 64, 16, NUL), 0),
    ((A, B, C, Dp, A, 1, 4, 64, 16, NUL), INV),     # fp32 output not offered
    ((A, B, C, Dp, A, 0, 4, 64, 0, NUL), INV),      # N = 0
    ((A, B, ODD, Dp, A, 0, 4, 64, 16, NUL), MIS),
])
def test_gemm_tiles_validation(args, expect):
    assert rw.lib().w4a4_gemm_tiles(*args) == expect


def _rl(x=A, ldx=64, T=4, D=64, Q=B, M=C, r=8, flags=3, w=Dp, sw=A, N=16, y=B, ws=C,
        wsb=1 << 20, dbg=NUL):
    return rw.lib().rotated_linear(x, ldx, T, D, Q, M, r, flags, w, sw, N, y, ws, wsb, dbg, NUL)


def _prep(Q=A, M=B, D=256, r=8, basis=C, nb=1 << 20):
    return rw.lib().respin_prepare_basis(Q, M, D, r, basis, nb, NUL)


def test_prepare_basis_validation():
    assert _prep(Q=NUL) == INV and _prep(M=NUL) == INV and _prep(r=0) == INV
    assert _prep(r=6) == UNS and _prep(D=1000) == UNS and _prep(r=132) == UNS
    assert _prep(Q=ODD) == MIS
    assert _prep(M=ctypes.c_void_p(0x20002)) == MIS
    assert _prep(basis=NUL) == WSE and _prep(nb=100) == WSE
    assert _prep(basis=ctypes.c_void_p(0x30010)) == WSE


def _rlp(x=A, ldx=64, T=4, D=64, basis=B, r=8, flags=3, w=Dp, sw=A, N=16, y=B, ws=C,
         wsb=1 << 20, dbg=NUL):
    return rw.lib().rotated_linear_prepared(x, ldx, T, D, basis, r, flags, w, sw, N, y, ws, wsb,
                                            dbg, NUL)


def test_rotated_linear_prepared_validation():
    assert _rlp(flags=8) == INV
    assert _rlp(flags=1 | 4) == INV
    assert _rlp(D=48) == UNS
    assert _rlp(r=6) == UNS
    assert _rlp(ldx=128) == UNS
    assert _rlp(basis=NUL) == INV                  # align with r > 0 needs a basis
    assert _rlp(basis=ctypes.c_void_p(0x20010)) == INV
    assert _rlp(ws=ctypes.c_void_p(0x30010)) == WSE
    assert _rlp(wsb=100) == WSE
    assert _rlp(x=ODD) == MIS
    assert _rlp(T=0) == 0
    assert _rlp(T=0, x=NUL, w=NUL, sw=NUL, y=NUL, basis=NUL) == 0


def _rap(x=A, out=B, odt=1, basis=C, add=NUL, T=4, D=256, r=8, ws=Dp, wsb=1 << 20):
    return rw.lib().respin_align_prepared(x, out, odt, basis, add, T, D, r, ws, wsb, NUL)


def test_respin_align_prepared_validation():
    L = rw.lib()
    # the per-call workspace is the projection's parts alone
    assert L.respin_align_prepared_workspace_size(2048, 4096, 32) == \
        L.rw4_align256((4096 // 512) * 2048 * 32 * 4)
    assert L.respin_align_prepared_workspace_size(4, 1000, 8) == 0
    assert L.respin_align_prepared_workspace_size(-1, 256, 8) == 0
    assert _rap(x=NUL) == INV and _rap(out=NUL) == INV and _rap(basis=NUL) == INV
    assert _rap(odt=2) == INV and _rap(T=-1) == INV and _rap(r=0) == INV
    assert _rap(r=6) == UNS and _rap(D=1000) == UNS and _rap(r=132) == UNS
    assert _rap(x=ODD) == MIS and _rap(add=ODD) == MIS
    assert _rap(basis=ctypes.c_void_p(0x30010)) == INV
    assert _rap(out=A) == INV                      # out aliases x
    assert _rap(ws=NUL) == WSE and _rap(wsb=100) == WSE
    assert _rap(ws=ctypes.c_void_p(0x40010)) == WSE
    assert _rap(T=0, ws=NUL) == 0
    assert _rap(T=0, x=NUL, out=NUL, basis=NUL, ws=NUL) == 0   # empty call: no pointer read


def _proj(x=A, T=8, D=4096, basis=B, r=32, z=C, zb=1 << 20):
    return rw.lib().respin_align_project_prepared(x, T, D, basis, r, z, zb, NUL)


def _rlr(x=A, T=8, D=4096, flags=(1 << 29), N=4096, y=B, ws=C, wsb=1 << 22, rx=Dp,
         rbasis=ctypes.c_void_p(0x50000), rr=32, rz=ctypes.c_void_p(0x60000), rzb=1 << 20,
         rout=ctypes.c_void_p(0x70000)):
    return rw.lib().rotated_linear_prepared_residual(x, D, T, D, NUL, 0, flags, Dp, A, N, y, ws,
                                                     wsb, NUL, rx, rbasis, rr, rz, rzb, rout, NUL)


def test_residual_entries_validation():
    L = rw.lib()
    # the projection of short batches only: sized like respin_align's parts
    assert L.respin_align_project_size(8, 4096, 32) == L.rw4_align256(16 * 8 * 32 * 4)
    assert L.respin_align_project_size(17, 4096, 32) == 0      # past 16 tokens
    assert L.respin_align_project_size(8, 1000, 32) == 0
    assert _proj(T=17) == UNS and _proj(r=6) == UNS
    assert _proj(x=NUL) == INV and _proj(basis=NUL) == INV and _proj(r=0) == INV
    assert _proj(x=ODD) == MIS
    assert _proj(basis=ctypes.c_void_p(0x20010)) == INV
    assert _proj(z=NUL) == WSE and _proj(zb=100) == WSE
    assert _proj(z=ctypes.c_void_p(0x30010)) == WSE
    assert _proj(T=0, x=NUL, basis=NUL, z=NUL) == 0
    # the residual product: packed weights, short batches, N = the alignment's D
    assert _rlr(flags=0) == UNS                     # FP6 tiles
    assert _rlr(T=17) == UNS
    assert _rlr(N=1000) == UNS                      # no alignment of width 1000
    assert _rlr(rr=0) == INV
    assert _rlr(rx=NUL) == INV and _rlr(rbasis=NUL) == INV and _rlr(rout=NUL) == INV
    assert _rlr(rx=ODD) == MIS and _rlr(rout=ODD) == MIS
    assert _rlr(rbasis=ctypes.c_void_p(0x50010)) == INV
    assert _rlr(rout=Dp) == INV and _rlr(rout=B) == INV   # aliases res_x, y
    assert _rlr(rz=NUL) == WSE and _rlr(rzb=100) == WSE
    assert _rlr(ws=NUL) == WSE
    assert _rlr(T=0) == 0


def _rlj(x=A, ldx=4096, T=8, D=4096, flags=(1 << 29), N=4096, y=B, ws=C, wsb=1 << 22,
         pb=ctypes.c_void_p(0x50000), pr=32, pz=ctypes.c_void_p(0x60000), pzb=1 << 20):
    return rw.lib().rotated_linear_prepared_project(x, ldx, T, D, NUL, 0, flags, Dp, A, N, y, ws,
                                                    wsb, NUL, pb, pr, pz, pzb, NUL)


def test_projecting_unit_validation():
    assert _rlj() is not None
    assert _rlj(T=17) == UNS                        # short batches only
    assert _rlj(flags=(1 << 29) | 1) == UNS         # the unit aligns nothing itself
    assert _rlj(flags=(1 << 29) | 4, ldx=8192) == UNS
    assert _rlj(ldx=8192) == UNS                    # contiguous rows
    assert _rlj(pr=0) == INV and _rlj(pr=6) == UNS
    assert _rlj(pb=NUL) == INV and _rlj(pb=ctypes.c_void_p(0x50010)) == INV
    assert _rlj(pz=NUL) == WSE and _rlj(pzb=100) == WSE
    assert _rlj(pz=ctypes.c_void_p(0x60010)) == WSE
    assert _rlj(ws=NUL) == WSE and _rlj(wsb=100) == WSE
    assert _rlj(x=ODD) == MIS
    assert _rlj(T=0) == 0


def test_structured_transform_validation():
    L = rw.lib()
    ht = lambda x=A, dt=0, ldx=192, y=B, T=4, D=192, m=12, sg=NUL: L.hadamard_transform(
        x, dt, ldx, y, T, D, m, sg, NUL)
    assert ht(m=16) == UNS and ht(m=52) == UNS and ht(D=200) == UNS   # order, D not 2^n m
    assert ht(D=12 * 2048) == UNS                 # beyond 16384
    assert ht(dt=2) == INV and ht(T=-1) == INV
    assert ht(ldx=100) == INV and ht(ldx=194) == INV
    assert ht(x=NUL) == INV and ht(y=NUL) == INV
    assert ht(x=ODD) == MIS and ht(sg=ODD) == MIS
    assert ht(y=A) == INV                         # in place needs fp32 input
    assert ht(y=A, dt=1, ldx=256) == INV          # ... and ldx == D
    assert ht(T=0, x=NUL, y=NUL) == 0
    hh = lambda x=A, dt=0, ldx=4096, y=B, T=4, nh=32, dh=128: L.head_hadamard(
        x, dt, ldx, y, T, nh, dh, NUL)
    assert hh(nh=24) == UNS and hh(nh=256, dh=128) == UNS and hh(nh=1, dh=6) == UNS
    assert hh(nh=0) == INV and hh(dh=0) == INV and hh(ldx=4000) == INV
    assert hh(x=ODD) == MIS and hh(y=A) == INV
    assert hh(T=0, x=NUL, y=NUL) == 0
    # rotated_linear flag fields
    K28, H5 = 28 << 16, 5 << 24
    assert L.rotated_linear_prepared_workspace_size(64, 28 * 512, 0, 2 | K28) > 0
    assert L.rotated_linear_prepared_workspace_size(64, 28 * 512, 0, K28) == 0   # needs FWHT
    assert L.rotated_linear_prepared_workspace_size(64, 28 * 1024, 0, 2 | K28) == 0  # > 16384
    assert L.rotated_linear_prepared_workspace_size(64, 12 * 4, 0, 2 | (12 << 16)) == 0  # D % 64
    assert L.rotated_linear_prepared_workspace_size(64, 4096, 0, H5) > 0
    assert L.rotated_linear_prepared_workspace_size(64, 4096, 0, H5 | 2) == 0
    assert L.rotated_linear_prepared_workspace_size(64, 4096, 0, H5 | K28 | 2) == 0
    assert _rl(D=28 * 16, ldx=28 * 16, flags=K28, r=0) == INV
    assert _rl(D=28 * 16, ldx=28 * 16, flags=2 | (16 << 16), r=0) == UNS
    assert _rl(D=4096, ldx=4096, flags=H5 | 1, r=0) == INV
    assert _rl(D=4096, ldx=4096, flags=(15 << 24), r=0) == UNS
    assert _rl(D=4096, ldx=4096, flags=(1 << 30), r=0) == INV   # unknown bit
    # packed INT4 weights: same workspace (packed codes fit the tile area)
    assert (L.rotated_linear_prepared_workspace_size(64, 4096, 32, 3 | (1 << 29))
            == L.rotated_linear_prepared_workspace_size(64, 4096, 32, 3))


def test_construct_validation():
    L = rw.lib()
    # Y and Z (D x p fp64, p = r + 16) plus two small fp64 matrices
    p = 48
    # two [D][p] fp64 blocks, two 80 x 80 fp64 matrices, and the K-part sums
    # of the products (8 parts at D = 4096)
    assert L.respin_construct_workspace_size(4096, 32) == (
        2 * 4096 * p * 8 + 2 * L.rw4_align256(80 * 80 * 8) + 8 * 4096 * p * 8)
    assert L.respin_construct_workspace_size(4096, 30) == 0 and L.respin_construct_workspace_size(4000, 32) == 0
    assert L.respin_construct_workspace_size(4096, 68) == 0 and L.respin_construct_workspace_size(32768, 32) == 0
    cs = lambda T=A, D=256, r=32, it=4, Q=B, R=C, ws=Dp, wsb=1 << 24: L.respin_construct(
        T, D, r, it, Q, R, ws, wsb, NUL)
    assert cs(T=NUL) == INV and cs(Q=NUL) == INV and cs(R=NUL) == INV
    assert cs(it=-1) == INV and cs(it=33) == INV
    assert cs(D=200) == UNS and cs(r=6) == UNS and cs(r=72) == UNS and cs(D=64, r=68) == UNS
    assert cs(T=ODD) == MIS and cs(Q=ODD) == MIS
    assert cs(ws=NUL) == WSE and cs(wsb=100) == WSE and cs(ws=ctypes.c_void_p(0x40010)) == WSE


def test_quant_sym_validation():
    L = rw.lib()
    for bits in (0, 1, 5, 8):
        assert L.quant_act_sym(A, 0, B, C, 4, 64, bits, NUL) == INV
    assert L.quant_act_sym(A, 0, B, C, 4, 63, 3, NUL) == UNS
    assert L.quant_act_sym(A, 0, B, NUL, 4, 64, 3, NUL) == INV
    assert L.quant_act_sym(ODD, 0, B, C, 4, 64, 3, NUL) == MIS
    assert L.quant_act_sym(NUL, 0, NUL, NUL, 0, 64, 2, NUL) == 0


def test_rotated_linear_validation():
    assert _rl(flags=8) == INV                     # unknown flag
    assert _rl(flags=3 | (1 << 8)) == INV          # 1-bit codes
    assert _rl(flags=3 | (5 << 8)) == INV          # 5-bit codes
    assert _rl(flags=3 | (1 << 12)) == INV         # unknown flag above the bit field
    assert _rl(T=0, flags=3 | (3 << 8)) == 0       # 3-bit codes accepted
    assert _rl(flags=1 | 4) == INV                 # align + swiglu
    assert _rl(D=48) == UNS                        # not a power of two
    assert _rl(D=32, ldx=32, flags=0) == UNS       # below the 64-code tile width
    assert _rl(ldx=32) == INV                      # stride below width
    assert _rl(flags=4, ldx=64) == INV             # swiglu needs 2D wide rows
    assert _rl(r=6) == UNS
    assert _rl(ldx=128) == UNS                     # align needs contiguous rows
    assert _rl(ws=ctypes.c_void_p(0x30010)) == WSE # workspace alignment
    assert _rl(wsb=100) == WSE
    assert _rl(ws=NUL) == WSE
    assert _rl(x=ODD) == MIS
    assert _rl(T=0) == 0
    assert _rl(T=0, x=NUL, w=NUL, sw=NUL, y=NUL) == 0


# rotated_linear_prepared_noalloc(x, ldx, T, D, basis, r, flags, w, s_w, N, y, dbg, stream):
# sizes past the library's scratch and invalid arguments are refused on the host
E = ctypes.c_void_p(0x50000)


@pytest.mark.parametrize("args,expect", [
    ((A, 8192, 8192, 8192, B, 64, 3, C, Dp, 64, E, NUL, NUL), UNS),       # needs > the scratch
    ((A, 4096, 4, 4096, B, 32, 3 | (1 << 31), C, Dp, 64, E, NUL, NUL), INV),  # unknown flag
    ((A, 4096, 4, 100, B, 32, 3, C, Dp, 64, E, NUL, NUL), UNS),           # D not a power of two
    ((A, 4096, -1, 4096, B, 32, 3, C, Dp, 64, E, NUL, NUL), INV),         # negative T
    ((A, 4096, 0, 4096, B, 32, 3, C, Dp, 64, E, NUL, NUL), 0),            # T = 0: nothing launched
])
def test_noalloc_validation(args, expect):
    L = rw.lib()
    assert L.rotated_linear_prepared_noalloc(*args) == expect
    if expect == UNS and args[2] == 8192:
        assert L.rotated_linear_prepared_workspace_size(8192, 8192, 64, 3) > rw.NOALLOC_SCRATCH_BYTES
