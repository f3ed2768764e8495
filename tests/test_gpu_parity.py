"""Stage parity of the HIP path against the CPU oracle (needs an MI355X).

Every call goes through the C ABI (via the ctypes binding). Inputs come from
the seeded generators; expected values come only from the oracle.
"""
import numpy as np
import pytest

import fp6_layout as F
import oracle as O
import workloads as W
from gpu_util import BF16_TOL, FP32_TOL, bf16_rel, dev, host, normwise, say, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rw():
    import rotation_w4a4_quantized_amd as m
    m.lib()
    return m


def _sync():
    torch().cuda.synchronize()


# ---------------------------------------------------------------- quantizer
def _quant_input(T, D, seed, special=True):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, D)) * rng.uniform(0.01, 50, (T, 1))).astype(np.float32)
    if special and T >= 4:
        x[0] = 0.0                                     # all-zero row
        x[1] = 0.0
        x[1, D // 3] = -5.0                            # one nonzero (negative) entry
        # ties: absmax 7 -> step exactly 1, values on k + 1/2
        x[2] = (rng.integers(-7, 7, D) + 0.5).astype(np.float32)
        x[2, 0] = 7.0
        x[3] = np.float32(1e-40) * rng.standard_normal(D).astype(np.float32)   # denormal row
    return x


@pytest.mark.parametrize("T,D", [(1, 2), (4, 6), (64, 256), (300, 4096), (5, 16384), (3, 32768),
                                 (7, 12288), (2, 65536), (0, 64)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_quant_act_int4(rw, T, D, dt):
    say(f"quant_act_int4 T={T} D={D} {dt}")
    x = _quant_input(T, D, seed=T * 7 + D)
    if dt == "bf16":
        xb = W.f32_to_bf16_bits(x)
        xg = dev(xb)
        x = W.bf16_bits_to_f32(xb)
    else:
        xg = dev(x)
    codes, scales = rw.quant_act_int4(xg)
    _sync()
    if T == 0:
        return
    q, s = O.quant_int4(x)
    np.testing.assert_array_equal(host(scales), s)
    np.testing.assert_array_equal(host(codes), O.pack_int4(q))


@pytest.mark.parametrize("T,D", [(3, 64), (300, 4096), (5, 1000), (17, 16384)])
@pytest.mark.parametrize("bits", [2, 3])
def test_quant_act_sym(rw, T, D, bits):
    say(f"quant_act_sym T={T} D={D} bits={bits}")
    x = _quant_input(T, D, seed=T * 5 + D + bits)
    codes, scales = rw.quant_act_sym(dev(x), bits)
    _sync()
    q, s = O.quant_sym(x, bits)
    np.testing.assert_array_equal(host(scales), s)
    np.testing.assert_array_equal(host(codes), O.pack_int4(q))


def test_quant_near_half_integers(rw):
    """Values whose quotient by the step sits within a few ulps of k + 1/2, the
    case where the fp32 quotient's rounding decides the code (R6)."""
    rng = np.random.default_rng(11)
    T, D = 48, 4096
    x = np.zeros((T, D), np.float32)
    for t in range(T):
        m = np.float32(rng.uniform(0.1, 100.0))
        s = np.float32(m / np.float32(7))
        k = rng.integers(-7, 7, D).astype(np.float32) + np.float32(0.5)
        base = (k.astype(np.float64) * np.float64(s)).astype(np.float32)
        steps = rng.integers(-3, 4, D).astype(np.int32)
        v = base.view(np.int32) + steps                    # a few ulps either way
        x[t] = v.view(np.float32)
        x[t] = np.clip(x[t], -m, m)
        x[t, 0] = m                                        # absmax: step is fl(m / 7)
    codes, scales = rw.quant_act_int4(dev(x))
    q, s = O.quant_int4(x)
    np.testing.assert_array_equal(host(scales), s)
    np.testing.assert_array_equal(host(codes), O.pack_int4(q))
    # the tiled writer of the unit takes the same decisions
    Wq = np.random.default_rng(12).integers(-7, 8, (64, D))
    wt = rw.w4a4_tile_codes(dev(O.pack_int4(Wq)))
    dbg = torch().empty((T, D), dtype=torch().float32, device="cuda")
    y, ws = rw.rotated_linear(dev(W.f32_to_bf16_bits(x)), wt, dev(np.ones(64, np.float32)), 0,
                              dbg_prequant=dbg)
    pre = host(dbg)
    tiles_g, sa_g = (host(v) for v in rw.workspace_views(ws, T, D))
    q2, s2 = O.quant_int4(pre)
    np.testing.assert_array_equal(sa_g, s2)
    np.testing.assert_array_equal(F.untile(tiles_g, T, D), q2)


# ---------------------------------------------------------------- Hadamard
def test_fwht_worked_example(rw):
    x = dev(np.array([[20, 0, 0, 0], [10, 10, 10, 10]], np.float32))
    y = host(rw.fwht(x))
    np.testing.assert_array_equal(y, np.array([[10, 10, 10, 10], [20, 0, 0, 0]], np.float32))


@pytest.mark.parametrize("D", [2 ** k for k in range(1, 16)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fwht(rw, D, dt):
    T = 37 if D <= 4096 else 5
    say(f"fwht T={T} D={D} {dt}")
    x32 = W.bf16_bits_to_f32(W.gen_x(D, T, D, min(8, D // 2), 80.0))
    xg = dev(W.f32_to_bf16_bits(x32)) if dt == "bf16" else dev(x32)
    y = host(rw.fwht(xg))
    assert normwise(y, O.fwht(x32)) <= FP32_TOL


def test_fwht_in_place_and_involution(rw):
    x = W.bf16_bits_to_f32(W.gen_x(9, 16, 4096, 8, 80.0))
    g = dev(x)
    rw.fwht(g, out=g)
    rw.fwht(g, out=g)
    assert normwise(host(g), x) <= 2 * FP32_TOL


# Long batches of wide rows (many workgroups per CU over the launch): every
# row equals the same row run in a slice of 256 rows, bit for bit, and the
# oracle's.
def _same_as_slices(full, run, xg, T, step=256):
    tt = torch()
    for t0 in range(0, T, step):
        part = run(xg[t0:t0 + step].contiguous())
        for a, b in zip(part if isinstance(part, tuple) else (part,),
                        full if isinstance(full, tuple) else (full,)):
            if not tt.equal(a, b[t0:t0 + step]):
                raise AssertionError(f"rows {t0}..{t0 + step} differ from the slice's")


@pytest.mark.parametrize("T,D,dt", [(1100, 16384, "f32"), (1030, 32768, "bf16")])
def test_fwht_long_batches(rw, T, D, dt):
    say(f"fwht long batch T={T} D={D} {dt}")
    x32 = W.bf16_bits_to_f32(W.gen_x(D + T, T, D, 8, 80.0))
    xg = dev(W.f32_to_bf16_bits(x32)) if dt == "bf16" else dev(x32)
    y = rw.fwht(xg)
    _same_as_slices(y, rw.fwht, xg, T)
    assert normwise(host(y), O.fwht(x32)) <= FP32_TOL


@pytest.mark.parametrize("T,D,dt", [(1100, 16384, "f32"), (2100, 8192, "bf16"), (1030, 32768, "f32")])
def test_quant_act_int4_long_batches(rw, T, D, dt):
    say(f"quant_act_int4 long batch T={T} D={D} {dt}")
    x = _quant_input(T, D, seed=T + D)
    if dt == "bf16":
        xb = W.f32_to_bf16_bits(x)
        xg = dev(xb)
        x = W.bf16_bits_to_f32(xb)
    else:
        xg = dev(x)
    codes, scales = rw.quant_act_int4(xg)
    _same_as_slices((codes, scales), rw.quant_act_int4, xg, T)
    q, s = O.quant_int4(x)
    np.testing.assert_array_equal(host(scales), s)
    np.testing.assert_array_equal(host(codes), O.pack_int4(q))


# ---------------------------------------------------------------- structured Hadamard
@pytest.mark.parametrize("T,n,m", [(37, 4, 12), (9, 5, 20), (5, 9, 28), (20, 12, 1), (3, 14, 1),
                                   (2, 1, 12), (4, 0, 28), (6, 8, 20)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("randomized", [False, True])
def test_hadamard_transform(rw, T, n, m, dt, randomized):
    """(H_{2^n} (x) H_m) diag(s) x / sqrt(D) against the oracle (Paley H_m)."""
    D = (1 << n) * m
    say(f"hadamard_transform T={T} D={D} m={m} {dt} signs={randomized}")
    rng = np.random.default_rng(D + T + m)
    x32 = W.bf16_bits_to_f32(W.gen_x(D + T, T, D, min(4, D // 2), 40.0))
    s = rng.choice([-1.0, 1.0], D).astype(np.float32) if randomized else None
    xg = dev(W.f32_to_bf16_bits(x32)) if dt == "bf16" else dev(x32)
    out = host(rw.hadamard_transform(xg, m, dev(s) if s is not None else None))
    assert normwise(out, O.hadamard_kron(x32, m, s)) <= FP32_TOL


def test_hadamard_transform_in_place_strided_and_inverse(rw):
    T, m, n = 11, 28, 6
    D = (1 << n) * m
    x32 = W.bf16_bits_to_f32(W.gen_x(3, T, D, 4, 40.0))
    g = dev(x32)
    rw.hadamard_transform(g, m, out=g)                     # in place
    y = host(g)
    assert normwise(y, O.hadamard_kron(x32, m)) <= FP32_TOL
    # the transpose undoes it (orthogonal): H_D^T y = x
    Hd = np.kron(O.hadamard(1 << n) * np.sqrt(1 << n), O.paley_hadamard(m)) / np.sqrt(D)
    assert normwise(y.astype(np.float64) @ Hd, x32) <= 2 * FP32_TOL
    # row-strided input: the middle third of wider rows
    big = W.gen_x(4, T, 3 * D, 4, 40.0)
    gb = dev(big)[:, D:2 * D]
    out = host(rw.hadamard_transform(gb, m))
    assert normwise(out, O.hadamard_kron(W.bf16_bits_to_f32(big[:, D:2 * D]), m)) <= FP32_TOL


@pytest.mark.parametrize("T,n_h,d_h", [(33, 32, 128), (7, 8, 32), (5, 64, 64), (4, 4, 6),
                                       (3, 128, 128), (9, 2, 48)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_head_hadamard(rw, T, n_h, d_h, dt):
    D = n_h * d_h
    say(f"head_hadamard T={T} n_h={n_h} d_h={d_h} {dt}")
    x32 = W.bf16_bits_to_f32(W.gen_x(D + 7, T, D, min(4, D // 2), 40.0))
    xg = dev(W.f32_to_bf16_bits(x32)) if dt == "bf16" else dev(x32)
    out = host(rw.head_hadamard(xg, n_h))
    assert normwise(out, O.head_hadamard(x32, n_h)) <= FP32_TOL


def test_head_hadamard_completes_the_transform(rw):
    """The page's identity on the GPU: the transform within heads (fwht of
    each head's d_h values) followed by the one across heads is H_D."""
    T, n_h, d_h = 12, 32, 128
    x32 = W.bf16_bits_to_f32(W.gen_x(8, T, n_h * d_h, 4, 40.0))
    within = rw.fwht(dev(x32.reshape(T * n_h, d_h))).reshape(T, n_h * d_h)
    out = host(rw.head_hadamard(within, n_h))
    assert normwise(out, O.fwht(x32)) <= 2 * FP32_TOL


# ---------------------------------------------------------------- offline construction
@pytest.mark.parametrize("D,r,n_big,iters", [(256, 32, 16, 4), (1024, 64, 32, 4), (512, 16, 8, 2),
                                             (64, 64, 16, 2)])
def test_respin_construct_against_oracle(rw, D, r, n_big, iters):
    """(Q, R_sub) of a perturbed-Hadamard transition: the GPU's T_hat and span(Q)
    against the oracle's full SVD and polar factor."""
    say(f"respin_construct D={D} r={r} iters={iters}")
    T = W.gen_hadamard_transition(D + r, D, n_big)
    Qg, Rg = rw.respin_construct(dev(T), r, iters)
    Qg, Rg = host(Qg).astype(np.float64), host(Rg).astype(np.float64)
    Qo, Ro, S = O.construct_basis(T, r)
    X = np.random.default_rng(D).standard_normal((16, D))
    err = np.linalg.norm(O.align(X, Qg, Rg) - O.align(X, Qo, Ro)) / np.linalg.norm(X)
    assert err <= 1e-5, err
    assert np.linalg.norm(Qg @ Qg.T - Qo @ Qo.T) / np.sqrt(r) <= 1e-5
    np.testing.assert_allclose(Rg.T @ Rg, np.eye(r), rtol=0, atol=1e-5)
    assert np.linalg.det(Rg) == pytest.approx(np.linalg.det(Ro), abs=1e-4)


@pytest.mark.parametrize("D,r", [(4096, 32), (8192, 64)])
def test_respin_construct_recovers_exact_rank(rw, D, r):
    """At the workload sizes: an exact rank-r transition is recovered (T_hat = T),
    checked on random vectors without a dense SVD; the basis then drives the
    online alignment."""
    say(f"respin_construct exact rank D={D} r={r}")
    # the transition is the oracle's dense T_hat of a seeded (Q0, M0) of rank r
    Q0, M0 = W.gen_basis(D + 1, D, r, stream="transition", skew_std=0.3)
    T = O.t_hat(Q0, M0).astype(np.float32)
    Qg, Rg = rw.respin_construct(dev(T), r, 2)
    X = np.random.default_rng(r).standard_normal((8, D))
    Q64, R64 = host(Qg).astype(np.float64), host(Rg).astype(np.float64)
    want = X @ T.astype(np.float64).T
    assert np.linalg.norm(O.align(X, Q64, R64) - want) / np.linalg.norm(X) <= 1e-5
    # the same through the device alignment (bf16 tokens)
    xb = W.f32_to_bf16_bits(X.astype(np.float32))
    out = host(rw.respin_align(dev(xb), Qg, Rg))
    assert normwise(out, W.bf16_bits_to_f32(xb).astype(np.float64) @ T.astype(np.float64).T) <= 1e-5


# ---------------------------------------------------------------- alignment
@pytest.mark.parametrize("T,D,r", [(64, 256, 8), (37, 4096, 32), (19, 8192, 64), (9, 4096, 128),
                                   (13, 1000, 12), (1, 64, 4)])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("direct", [False, True])
def test_respin_align_f32(rw, T, D, r, xdt, direct):
    """bf16 x with D % 32 == 0 runs the matrix-core path unless direct=True."""
    say(f"respin_align T={T} D={D} r={r} x={xdt} direct={direct}")
    Q, M = W.gen_basis(D + r, D, r)
    xb = W.gen_x(D, T, D, 8, 80.0)
    x = W.bf16_bits_to_f32(xb)
    xg = dev(xb) if xdt == "bf16" else dev(x)
    out = host(rw.respin_align(xg, dev(Q), dev(M), direct=direct))
    assert normwise(out, O.align(x, Q, M)) <= FP32_TOL


@pytest.mark.parametrize("T,D,r", [(2048, 4096, 32), (8, 4096, 32), (4096, 4096, 32)])
def test_respin_align_workload_sizes(rw, T, D, r):
    """The alignment at the workload sizes (prefill linear, decode, prefill layer)."""
    say(f"respin_align workload T={T} D={D} r={r}")
    Q, M = W.gen_basis(1001, D, r)
    xb = W.gen_x(1001, T, D, 8, 80.0)
    out = host(rw.respin_align(dev(xb), dev(Q), dev(M)))
    assert normwise(out, O.align(W.bf16_bits_to_f32(xb), Q, M)) <= FP32_TOL


def test_respin_align_identity_cases(rw):
    T, D = 20, 4096
    Q, M = W.gen_basis(5, D, 32)
    xb = W.gen_x(5, T, D, 8, 80.0)
    x = W.bf16_bits_to_f32(xb)
    # M = I: M - I is exactly zero, the output equals the input bit for bit
    out = host(rw.respin_align(dev(xb), dev(Q), dev(np.eye(32, dtype=np.float32))))
    np.testing.assert_array_equal(out, x)
    outb = host(rw.respin_align(dev(xb), dev(Q), dev(np.eye(32, dtype=np.float32)),
                                out_dtype=torch().bfloat16))
    np.testing.assert_array_equal(outb, xb)
    out = host(rw.respin_align(dev(xb), dev(Q), dev(np.eye(32, dtype=np.float32)), direct=True))
    np.testing.assert_array_equal(out, x)
    # r = 0: identity
    out0 = host(rw.respin_align(dev(x), None, None))
    np.testing.assert_array_equal(out0, x)
    # norm preserved (T_hat is orthogonal)
    out = host(rw.respin_align(dev(xb), dev(Q), dev(M))).astype(np.float64)
    np.testing.assert_allclose(np.linalg.norm(out, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)


@pytest.mark.parametrize("T,D,r", [(37, 4096, 32), (2048, 4096, 32), (9, 256, 8), (70, 1024, 64),
                                   (13, 2048, 40), (5, 4096, 128), (11, 8192, 64), (6, 576, 16),
                                   # short batches (up to 16 tokens) take the D-parallel path
                                   (1, 4096, 32), (16, 8192, 128), (17, 4096, 32), (8, 320, 4),
                                   # 16 and 32 D parts over several 64-token blocks with a
                                   # ragged tail: the partials summed once before the lift,
                                   # the projection's workgroups dealt part-major
                                   (200, 8192, 64), (70, 16384, 32)])
@pytest.mark.parametrize("odt", ["f32", "bf16"])
@pytest.mark.parametrize("add", [False, True])
def test_respin_align_prepared(rw, T, D, r, odt, add):
    """respin_align_prepared equals respin_align (given a workspace) bit for bit,
    and the oracle's alignment within the fp32 (bf16) tolerance."""
    say(f"respin_align_prepared T={T} D={D} r={r} out={odt} addend={add}")
    tt = torch()
    Q, M = W.gen_basis(D * 3 + r, D, r)
    xb = W.gen_x(D + T, T, D, 8, 80.0)
    x = W.bf16_bits_to_f32(xb)
    out_dtype = tt.float32 if odt == "f32" else tt.bfloat16
    addend = None
    if add:
        a32 = W.bf16_bits_to_f32(W.gen_x(D + T + 1, T, D, 0, 1.0))
        addend = dev(a32) if odt == "f32" else dev(W.f32_to_bf16_bits(a32))
    basis = rw.respin_prepare_basis(dev(Q), dev(M))
    out = host(rw.respin_align_prepared(dev(xb), basis, r, addend=addend, out_dtype=out_dtype))
    ref = host(rw.respin_align(dev(xb), dev(Q), dev(M), addend=addend, out_dtype=out_dtype))
    np.testing.assert_array_equal(out, ref)
    want = O.align(x, Q, M)
    if add:
        want = want + (host(addend) if odt == "f32" else O.bf16_to_f64(host(addend)))
    got = out if odt == "f32" else O.bf16_to_f64(out)
    tol = FP32_TOL if odt == "f32" else BF16_TOL
    assert normwise(got, want) <= tol


# From 16 D parts of 512 columns (D > 7680), batches of at least 2 * floor(256 / S)
# blocks of 64 tokens (S parts, 256 CUs) take the looping lift when r <= 64
# (with an addend, 32 < r <= 64): one workgroup per (D part, token stride)
# keeps its basis slice in registers across blocks. A 64-token slice takes
# the one-block lift; the rows of both must agree bit for bit, and both the
# oracle's alignment.
@pytest.mark.parametrize("T,D,r,odt,add", [
    (2053, 8192, 64, "f32", False),      # the 70B-shaped prologue's lift, ragged tail
    (2048, 8192, 32, "f32", False),      # exactly two blocks per workgroup
    (1100, 16384, 32, "f32", False),     # 32 parts, 18 blocks over 8 strides
    (2000, 8256, 64, "bf16", False),     # a last part of 64 columns (7 idle waves)
    (2100, 8192, 48, "bf16", True),      # r padded to 64, bf16 addend
    (1030, 16384, 64, "bf16", True)])
def test_respin_align_looping_lift(rw, T, D, r, odt, add):
    say(f"looping lift T={T} D={D} r={r} out={odt} addend={add}")
    tt = torch()
    Q, M = W.gen_basis(D + 7 * r, D, r)
    xb = W.gen_x(D + T + 3, T, D, 8, 80.0)
    out_dtype = tt.float32 if odt == "f32" else tt.bfloat16
    addend = None
    if add:
        addend = dev(W.f32_to_bf16_bits(W.bf16_bits_to_f32(W.gen_x(D + T + 4, T, D, 0, 1.0))))
    basis = rw.respin_prepare_basis(dev(Q), dev(M))
    xg = dev(xb)
    out = rw.respin_align_prepared(xg, basis, r, addend=addend, out_dtype=out_dtype)
    for t0 in range(0, T, 64):
        t1 = min(T, t0 + 64)
        # a slice of up to 16 rows would take the short-batch kernels: the tail
        # is checked inside the last 64 rows (each token's z and lift do not
        # depend on the other tokens of its block)
        s0 = t1 - 64 if t1 - t0 <= 16 else t0
        part = rw.respin_align_prepared(xg[s0:t1].contiguous(), basis, r,
                                        addend=None if addend is None else addend[s0:t1].contiguous(),
                                        out_dtype=out_dtype)[t0 - s0:]
        if not tt.equal(part, out[t0:t1]):
            bad = (part != out[t0:t1]).nonzero()[:4].tolist()
            raise AssertionError(f"rows {t0}..{t1}: looping lift differs at {bad}")
    want = O.align(W.bf16_bits_to_f32(xb), Q, M)
    if add:
        want = want + O.bf16_to_f64(host(addend))
    got = host(out) if odt == "f32" else O.bf16_to_f64(host(out))
    assert normwise(got, want) <= (FP32_TOL if odt == "f32" else BF16_TOL)


@pytest.mark.parametrize("T,D,r", [(33, 4096, 32), (8, 4096, 32), (70, 256, 8)])
@pytest.mark.parametrize("direct", [False, True])
def test_respin_align_bf16_residual(rw, T, D, r, direct):
    Q, M = W.gen_basis(77, D, r)
    xb = W.gen_x(77, T, D, 8, 80.0)
    ab = W.gen_x(78, T, D, 0, 1.0)
    out = host(rw.respin_align(dev(xb), dev(Q), dev(M), addend=dev(ab),
                               out_dtype=torch().bfloat16, direct=direct))
    ref = O.residual(xb, Q, M, ab)
    # The fp32 alignment may be off by its own tolerance (FP32_TOL times the row's
    # max |align(x)|); the fp32 add then costs a few fp32 ulps of the summands and
    # the single bf16 rounding one bf16 ulp. Where align(x) + addend cancels, those
    # errors span several ulps of the tiny sum, which this bound allows.
    aligned = O.align(W.bf16_bits_to_f32(xb), Q, M)
    addv = W.bf16_bits_to_f32(ab).astype(np.float64)
    g, o = O.bf16_to_f64(out), O.bf16_to_f64(ref)
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(o), 2.0 ** -126))[1] - 8)
    bound = (ulp + 2.0 ** -20 * (np.abs(aligned) + np.abs(addv))
             + FP32_TOL * np.abs(aligned).max(axis=1, keepdims=True))
    assert np.all(np.abs(g - o) <= bound)
    diff = np.abs(out.astype(np.int32) - ref.astype(np.int32))
    assert (diff > 0).mean() < 0.01


def _check_residual(rw, x_bits, add_bits, basis, r, Q, M, out_bits):
    """bf16(align(x) + addend) as the kernels form it: the fp32 alignment, one
    fp32 add of the bf16 addend, one round-to-nearest-even to bf16.
    * identical inputs: the GPU's own fp32 alignment of x (the same entry point
      with fp32 output) is within the fp32 bar of the float64 oracle, and the
      bf16 result equals the oracle's rounding of (that + addend) bit for bit;
    * against the float64 chain (O.residual): within the error those steps
      allow, which spans many ulps of a sum that cancels."""
    a32 = host(rw.respin_align_prepared(dev(x_bits), basis, r))
    aligned = O.align(O.bf16_to_f64(x_bits), Q, M)
    assert normwise(a32, aligned) <= FP32_TOL
    s32 = a32 + O.bf16_to_f64(add_bits).astype(np.float32)        # IEEE fp32 add
    np.testing.assert_array_equal(out_bits, O.f64_to_bf16(s32.astype(np.float64)))
    ref = O.residual(x_bits, Q, M, add_bits)
    addv = O.bf16_to_f64(add_bits)
    g, o = O.bf16_to_f64(out_bits), O.bf16_to_f64(ref)
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(o), 2.0 ** -126))[1] - 8)
    bound = (ulp + 2.0 ** -20 * (np.abs(aligned) + np.abs(addv))
             + FP32_TOL * np.abs(aligned).max(axis=1, keepdims=True))
    assert np.all(np.abs(g - o) <= bound)
    diff = np.abs(out_bits.astype(np.int32) - ref.astype(np.int32))
    say(f"   residual: {(diff > 1).sum()} of {diff.size} outputs more than one bf16 ulp "
        f"from the float64 chain (cancelling sums), {(diff > 0).mean():.2e} differ")
    assert (diff > 0).mean() < 0.01


# ---------------------------------------------------------------- GEMM
def _codes(seed, rows, K):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)   # every byte is two valid codes


# T <= 16 takes the weight-streaming decode kernel (K steps of 256 codes with
# a partial last step, ragged N, fewer waves as the workgroups multiply)
@pytest.mark.parametrize("T,K,N", [(1, 32, 1), (64, 256, 256), (300, 512, 384), (129, 4096, 130),
                                   (17, 16384, 64), (8, 4096, 12288), (257, 96, 1000),
                                   (16, 96, 70), (9, 160, 33), (3, 32, 17), (8, 16384, 4096),
                                   (16, 4096, 4100), (1, 4128, 9000), (8, 4096, 32768)])
def test_w4a4_gemm(rw, T, K, N):
    say(f"w4a4_gemm T={T} K={K} N={N}")
    a = _codes(T + K, T, K)
    w = _codes(N + K + 1, N, K)
    rng = np.random.default_rng(K)
    s_a = rng.uniform(1e-3, 1.0, T).astype(np.float32)
    s_w = rng.uniform(1e-3, 0.1, N).astype(np.float32)
    acc = host(rw.w4a4_gemm(dev(a), None, dev(w), None, out_dtype=torch().int32))
    ref = O.gemm_int(O.unpack_int4(a), O.unpack_int4(w))
    np.testing.assert_array_equal(acc, ref)
    y = host(rw.w4a4_gemm(dev(a), dev(s_a), dev(w), dev(s_w)))
    nbad, worst = bf16_rel(y, O.epilogue(ref, s_a, s_w))
    assert nbad == 0, worst


@pytest.mark.parametrize("T,K,N", [(40, 16384, 72), (3, 131072, 40), (66, 131072, 64)])
def test_w4a4_gemm_extremes(rw, T, K, N):
    """Codes at the ends of the INT4 range on the packed-row (int8) path, up to
    the largest K: all -8 against all -8 sums to 64 K, which is 2^23 at
    K = 131072 (the int8 path holds 256 times the sum in int32, so this one
    value needs the exact decoding of its epilogue); -8 against +7 gives -56 K."""
    say(f"w4a4_gemm extremes T={T} K={K} N={N}")
    a = np.full((T, K // 2), 0x88, np.uint8)            # all codes -8
    w = np.full((N, K // 2), 0x88, np.uint8)
    acc = host(rw.w4a4_gemm(dev(a), None, dev(w), None, out_dtype=torch().int32))
    assert np.all(acc == 64 * K)
    s_a = np.full(T, 0.5, np.float32)
    s_w = np.full(N, 0.25, np.float32)
    y = host(rw.w4a4_gemm(dev(a), dev(s_a), dev(w), dev(s_w)))
    np.testing.assert_array_equal(y, O.epilogue(np.full((T, N), 64 * K), s_a, s_w))
    w[:, :] = 0x77                                      # all codes +7
    acc = host(rw.w4a4_gemm(dev(a), None, dev(w), None, out_dtype=torch().int32))
    assert np.all(acc == -56 * K)
    # mixed rows: every sum against the oracle
    qa = np.random.default_rng(K + T).choice([-8, 7, -7, 0], (T, K))
    qw = np.random.default_rng(K + N).choice([-8, 7, -1], (N, K))
    acc = host(rw.w4a4_gemm(dev(O.pack_int4(qa)), None, dev(O.pack_int4(qw)), None,
                            out_dtype=torch().int32))
    np.testing.assert_array_equal(acc, O.gemm_int(qa, qw))


# ---------------------------------------------------------------- FP6 tiles and the tiled GEMM
def _oracle_gemm_chunks(qa, qw, elems=1 << 24):
    """(n0, oracle int32 acc [T][n0:n0 + step]) over column chunks of about
    ``elems`` outputs, so that full-size products stay within host memory."""
    T = qa.shape[0]
    step = max(64, elems // max(T, 1))
    chunks = -(-qw.shape[0] // step)
    for n0 in range(0, qw.shape[0], step):
        if chunks > 8:
            say(f"   oracle GEMM columns {n0}..{min(n0 + step, qw.shape[0])} of {qw.shape[0]}")
        yield n0, O.gemm_int(qa, qw[n0:n0 + step])


def _check_gemm_out(y_bits, q, s, qw, sw):
    """bf16 GEMM outputs [T][N] against the oracle's epilogue on the same codes,
    every element, in column chunks."""
    for n0, ref in _oracle_gemm_chunks(q, qw):
        n1 = n0 + ref.shape[1]
        nbad, worst = bf16_rel(y_bits[:, n0:n1], O.epilogue(ref, s, sw[n0:n1]))
        assert nbad == 0, (n0, worst)


def _codes7(seed, rows, K):
    """packed INT4 rows with codes in [-7, 7] (the symmetric quantizer's range)"""
    q = np.random.default_rng(seed).integers(-7, 8, (rows, K))
    return O.pack_int4(q), q


@pytest.mark.parametrize("R,K", [(1, 64), (33, 128), (300, 192), (256, 4096), (70, 16384)])
def test_tile_codes(rw, R, K):
    say(f"w4a4_tile_codes R={R} K={K}")
    packed, q = _codes7(R * 3 + K, R, K)
    tiles = host(rw.w4a4_tile_codes(dev(packed)))
    assert len(tiles) == F.tiles_size(R, K) == rw.w4a4_tiles_size(R, K)
    np.testing.assert_array_equal(tiles, F.tile(q))


def test_tile_codes_rejects_minus8(rw):
    packed, _ = _codes7(9, 40, 128)
    packed[17, 5] = 0x8F                                 # codes -1 and -8
    with pytest.raises(ValueError):
        rw.w4a4_tile_codes(dev(packed))


# T >= 128 with K % 128 == 0 takes the LDS-staged kernel (one stage of 128 k:
# K = 128; stage-ring tails: K / 128 = 4, 5, 32), the rest the direct kernel
@pytest.mark.parametrize("T,K,N", [(1, 64, 1), (64, 256, 256), (300, 512, 384), (129, 4096, 130),
                                   (17, 16384, 64), (8, 4096, 12288), (257, 192, 1000),
                                   (256, 128, 256), (200, 640, 520),
                                   (4096, 4096, 4096), (4100, 1024, 4104),
                                   # decode products (split-K workgroups): a full token
                                   # tile, ragged N, K with fewer k-tiles than waves, an
                                   # odd k-tile count; 16-row workgroups of 16, 8 and 4
                                   # waves (N up to 4096, 8192, 16384), 32-row ones past
                                   # 16 tokens or N = 16384
                                   (32, 4096, 4096), (5, 192, 100), (31, 1088, 4000),
                                   (8, 16384, 4096), (2, 64, 16383), (8, 1024, 32768),
                                   (8, 1024, 8192), (16, 1088, 12288), (17, 256, 4096),
                                   (1, 64, 16400),
                                   # the largest K (sums stay exact in fp32: 49 K < 2^24)
                                   (2, 131072, 40), (130, 131072, 64),
                                   # each split of the tile grid into 8 XCD rectangles
                                   # (rt along T = 1, 8, 4, 2 with ragged edges; 4 on
                                   # the large-block variant)
                                   (256, 384, 1024), (1024, 256, 128), (1024, 640, 256),
                                   (1000, 640, 1000), (8192, 256, 4096),
                                   # 256 x 256 blocks (chosen where they take fewer
                                   # weighted waves): ragged T and N, an even XCD split,
                                   # a grid no split divides
                                   (3000, 512, 4100), (2048, 384, 8192), (2304, 256, 5000),
                                   # whole tiles, several per CU (256 x 256 blocks with
                                   # 2, 3, 8 stages; 256 x 128 blocks with 16)
                                   (8192, 256, 8192), (4096, 384, 8192), (4096, 1024, 8192),
                                   (2048, 2048, 12288),
                                   # an XCD's rectangle larger than its resident tiles,
                                   # walked in super-tiles: 4 x 16 of 128 x 128 blocks
                                   # (12 x 16 rectangle), 4 x 8 of 256 x 256 (16 x 8)
                                   (1536, 256, 16384), (4096, 128, 16384)])
def test_w4a4_gemm_tiles(rw, T, K, N):
    say(f"w4a4_gemm_tiles T={T} K={K} N={N}")
    a, qa = _codes7(T + K, T, K)
    w, qw = _codes7(N + K + 1, N, K)
    rng = np.random.default_rng(K)
    s_a = rng.uniform(1e-3, 1.0, T).astype(np.float32)
    s_w = rng.uniform(1e-3, 0.1, N).astype(np.float32)
    at = rw.w4a4_tile_codes(dev(a))
    wt = rw.w4a4_tile_codes(dev(w))
    acc = host(rw.w4a4_gemm_tiles(at, None, wt, None, T, K, N, out_dtype=torch().int32))
    y = host(rw.w4a4_gemm_tiles(at, dev(s_a), wt, dev(s_w), T, K, N))
    # the packed-row (int8) path on the same codes
    acc8 = host(rw.w4a4_gemm(dev(a), None, dev(w), None, out_dtype=torch().int32))
    y8 = host(rw.w4a4_gemm(dev(a), dev(s_a), dev(w), dev(s_w)))
    # every output of both paths against the oracle, in column chunks
    for n0, ref in _oracle_gemm_chunks(qa, qw):
        n1 = n0 + ref.shape[1]
        np.testing.assert_array_equal(acc[:, n0:n1], ref)
        np.testing.assert_array_equal(acc8[:, n0:n1], ref)
        ref_y = O.epilogue(ref, s_a, s_w[n0:n1])
        for out in (y, y8):
            nbad, worst = bf16_rel(out[:, n0:n1], ref_y)
            assert nbad == 0, (n0, worst)


def test_w4a4_gemm_tiles_ignores_rows_past_T(rw):
    """Activation tiles hold 32-row blocks; rows past T (unwritten workspace in
    the unit) must not reach the T valid rows, on the decode path as elsewhere."""
    K, N = 1024, 300
    a, qa = _codes7(77, 32, K)
    w, qw = _codes7(78, N, K)
    at = rw.w4a4_tile_codes(dev(a))          # all 32 rows nonzero
    for T in (1, 8, 31):
        acc = host(rw.w4a4_gemm_tiles(at, None, rw.w4a4_tile_codes(dev(w)), None, T, K, N,
                                      out_dtype=torch().int32))
        np.testing.assert_array_equal(acc, O.gemm_int(qa[:T], qw))


@pytest.mark.parametrize("T,K,N", [(40, 16384, 72), (8, 131072, 48), (128, 131072, 128)])
def test_w4a4_gemm_tiles_extremes(rw, T, K, N):
    """All codes at +-7: every sum is +-49 K, exact up to the largest K."""
    say(f"w4a4_gemm_tiles extremes T={T} K={K} N={N}")
    qa = np.full((T, K), -7)
    for wv, expect in ((-7, 49 * K), (7, -49 * K)):
        qw = np.full((N, K), wv)
        at = rw.w4a4_tile_codes(dev(O.pack_int4(qa)))
        wt = rw.w4a4_tile_codes(dev(O.pack_int4(qw)))
        acc = host(rw.w4a4_gemm_tiles(at, None, wt, None, T, K, N, out_dtype=torch().int32))
        assert np.all(acc == expect)


# ---------------------------------------------------------------- weight prep and the unit
def _prep(rw, Wf, rotate, bits=4, m=1, signs=None):
    tiles, s_w, codes, src = rw.prep_weight(dev(Wf), rotate, bits, m,
                                            dev(signs) if signs is not None else None)
    src_h = host(src)
    if rotate:
        assert normwise(src_h, O.hadamard_kron(Wf, m, signs)) <= FP32_TOL
    q, s = O.quant_sym(src_h, bits)
    np.testing.assert_array_equal(host(s_w), s)
    np.testing.assert_array_equal(host(codes), O.pack_int4(q))
    np.testing.assert_array_equal(host(tiles), F.tile(q))
    return tiles, s_w, q, s


def _check_unit(rw, xb, Q, M, flags, codes_w, s_w, qw, sw_h, rows=None):
    """Run rotated_linear on the GPU and check every stage against the oracle.
    rows: optional token sample for the expensive float checks."""
    t = torch()
    T = xb.shape[0]
    D = xb.shape[1] // 2 if flags & O.FLAG_SWIGLU else xb.shape[1]
    dbg = t.empty((T, D), dtype=t.float32, device="cuda")
    y, ws = rw.rotated_linear(dev(xb), codes_w, s_w, flags, dev(Q) if Q is not None else None,
                              dev(M) if M is not None else None, dbg_prequant=dbg)
    _sync()
    packed = bool(flags & rw.RW4_WPACKED)
    codes_ws, sa_g = (host(v) for v in rw.workspace_views(ws, T, D, packed))
    codes_g = O.unpack_int4(codes_ws) if packed else F.untile(codes_ws, T, D)
    pre = host(dbg)
    y = host(y)
    sel = np.arange(T) if rows is None else rows
    # 1. pre-quant fp32 values vs the float64 chain
    ref_pre = O.prequant(O.bf16_to_f64(xb[sel]), flags, Q, M)
    assert normwise(pre[sel], ref_pre) <= FP32_TOL
    # 2. codes and scales: bit-exact on the GPU's own fp32 values
    bits = (flags >> 8) & 0xF or 4
    q, s = O.quant_sym(pre[sel], bits)
    np.testing.assert_array_equal(sa_g[sel], s)
    np.testing.assert_array_equal(codes_g[sel], q)
    # 3. GEMM + epilogue on those codes
    _check_gemm_out(y[sel], q, s, qw, sw_h)
    # 4. end to end against the oracle's own chain: rare code flips only
    q_own, _ = O.quant_sym(ref_pre.astype(np.float32), bits)
    flips = float((q_own != q).mean())
    say(f"   end-to-end code flips vs float64 chain: {flips:.2e}")
    assert flips < 1e-3
    return y


@pytest.mark.parametrize("cid", [0, 1])
def test_rotated_linear_config(rw, cid):
    wl = W.CONFIGS[cid]
    say(f"rotated_linear {wl.name}")
    inp = W.workload_inputs(wl)
    Q, M = inp["basis"][0]
    lin = wl.linears[0]
    codes_w, s_w, qw, sw_h = _prep(rw, inp["W"]["lin"], lin.rotate)
    _check_unit(rw, inp["x"], Q, M, O.FLAG_ALIGN | O.FLAG_FWHT, codes_w, s_w, qw, sw_h)


@pytest.mark.timeout(900)
def test_rotated_linear_config4(rw):
    """Full 70B-shaped size (T=8192, D=8192, r=64, N=28672): every token's
    pre-quant values, codes and scales, every weight row's rotation and codes,
    and every one of the 235 M outputs against the oracle (GEMM in column
    chunks)."""
    wl = W.CONFIGS[4]
    say(f"rotated_linear {wl.name}")
    inp = W.workload_inputs(wl)
    Q, M = inp["basis"][0]
    Wf = inp["W"]["lin"]
    tiles_w, s_w, codes_w, src = rw.prep_weight(dev(Wf), True)
    sw_h = host(s_w)
    codes_h = host(codes_w)
    for r0 in range(0, Wf.shape[0], 4096):             # weight rows in chunks
        src_h = host(src[r0:r0 + 4096])
        assert normwise(src_h, O.fwht(Wf[r0:r0 + 4096])) <= FP32_TOL
        q_s, s_s = O.quant_int4(src_h)
        np.testing.assert_array_equal(codes_h[r0:r0 + 4096], O.pack_int4(q_s))
        np.testing.assert_array_equal(sw_h[r0:r0 + 4096], s_s)
    del src
    qw = O.unpack_int4(codes_h)
    _check_unit(rw, inp["x"], Q, M, O.FLAG_ALIGN | O.FLAG_FWHT, tiles_w, s_w, qw, sw_h)


@pytest.mark.parametrize("T,D,N,flags", [(77, 512, 200, 0), (77, 512, 200, 2), (50, 256, 64, 4 | 2),
                                         (33, 1024, 96, 4), (130, 2048, 260, 1),
                                         (1, 4096, 4096, 3), (21, 4096, 64, 4 | 2),
                                         (6, 8192, 64, 4 | 2), (9, 2048, 64, 2),
                                         # the down projection's width in the layers
                                         (8, 16384, 64, 4 | 2), (300, 16384, 128, 4 | 2),
                                         # long batches (at D = 8192 the looping lift)
                                         (1100, 16384, 64, 4 | 2), (2100, 8192, 64, 1 | 2),
                                         (4100, 4096, 64, 0)])
def test_rotated_linear_flags(rw, T, D, N, flags):
    say(f"rotated_linear T={T} D={D} N={N} flags={flags}")
    width = 2 * D if flags & 4 else D
    xb = W.gen_x(T + D, T, width, 4, 30.0)
    Q, M = W.gen_basis(T + D, D, 16) if flags & 1 else (None, None)
    Wf = W.gen_weight(N, N, D, 0.02)
    codes_w, s_w, qw, sw_h = _prep(rw, Wf, bool(flags & 2))
    _check_unit(rw, xb, Q, M, flags, codes_w, s_w, qw, sw_h)


# the prepared basis gives the same results bit for bit; the fused prologue's
# geometry changes with D (lane bits of a row), r (32 or 64 padded), and the
# transform flag (without it the lift operand is Q itself); D = 8192 runs the
# unfused path on the same basis layout (short and multi-block batches)
@pytest.mark.parametrize("T,D,N,r,flags", [(45, 512, 128, 16, 3), (61, 1024, 64, 48, 3),
                                           (200, 2048, 96, 64, 3), (9, 4096, 64, 64, 1),
                                           (70, 256, 64, 8, 1), (3, 8192, 64, 64, 3),
                                           (100, 8192, 64, 64, 3)])
def test_rotated_linear_prepared(rw, T, D, N, r, flags):
    say(f"rotated_linear_prepared T={T} D={D} N={N} r={r} flags={flags}")
    t = torch()
    xb = W.gen_x(T + D + r, T, D, 4, 30.0)
    Q, M = W.gen_basis(T + r, D, r)
    Wf = W.gen_weight(N + r, N, D, 0.02)
    codes_w, s_w, qw, sw_h = _prep(rw, Wf, bool(flags & 2))
    y_ref = _check_unit(rw, xb, Q, M, flags, codes_w, s_w, qw, sw_h)
    d1 = t.empty((T, D), dtype=t.float32, device="cuda")
    _, ws1 = rw.rotated_linear(dev(xb), codes_w, s_w, flags, dev(Q), dev(M), dbg_prequant=d1)
    basis = rw.respin_prepare_basis(dev(Q), dev(M))
    d2 = t.empty((T, D), dtype=t.float32, device="cuda")
    y2, ws2 = rw.rotated_linear_prepared(dev(xb), codes_w, s_w, flags, basis, r, dbg_prequant=d2)
    _sync()
    np.testing.assert_array_equal(host(y2), y_ref)
    np.testing.assert_array_equal(host(d2), host(d1))
    (t1, s1), (t2, s2) = rw.workspace_views(ws1, T, D), rw.workspace_views(ws2, T, D)
    np.testing.assert_array_equal(host(s2), host(s1))
    # rows past T of the padded tiles are not written by either call
    np.testing.assert_array_equal(F.untile(host(t2), T, D), F.untile(host(t1), T, D))


# Without dbg_prequant the fused prologue is a separate kernel instance: the
# one the benchmark times. Its tiles, scales and outputs must equal those of
# the dumping run (checked against the oracle) bit for bit, through both entry
# points, at the prefill-linear shape and at token counts that leave a partial
# 8-token block; also without the transform and with 3-bit codes.
@pytest.mark.parametrize("T,flags,bits", [(2048, 3, 4), (77, 3, 4), (1001, 1, 4), (13, 3, 3)])
def test_rotated_linear_without_dump(rw, T, flags, bits):
    say(f"rotated_linear without dump T={T} flags={flags} bits={bits}")
    t = torch()
    wl = W.CONFIGS[1]
    D, r, N = wl.D, wl.r, 512
    inp = W.workload_inputs(wl, with_weights=False)
    Q, M = inp["basis"][0]
    xb = inp["x"][:T]
    Wf = W.gen_weight(T + flags, N, D, 0.02)
    codes_w, s_w, qw, sw_h = _prep(rw, Wf, bool(flags & 2), bits)
    fl = flags | rw.RW4_ABITS(bits)
    y_ref = _check_unit(rw, xb, Q, M, fl, codes_w, s_w, qw, sw_h)
    dbg = t.empty((T, D), dtype=t.float32, device="cuda")
    _, ws_d = rw.rotated_linear(dev(xb), codes_w, s_w, fl, dev(Q), dev(M), dbg_prequant=dbg)
    y1, ws1 = rw.rotated_linear(dev(xb), codes_w, s_w, fl, dev(Q), dev(M))
    basis = rw.respin_prepare_basis(dev(Q), dev(M))
    y2, ws2 = rw.rotated_linear_prepared(dev(xb), codes_w, s_w, fl, basis, r)
    _sync()
    td, sd = (host(v) for v in rw.workspace_views(ws_d, T, D))
    for y, ws in ((y1, ws1), (y2, ws2)):
        np.testing.assert_array_equal(host(y), y_ref)
        tg, sg = (host(v) for v in rw.workspace_views(ws, T, D))
        np.testing.assert_array_equal(sg, sd)
        np.testing.assert_array_equal(F.untile(tg, T, D), F.untile(td, T, D))


# Packed INT4 weight rows (RW4_WPACKED: the survey's weight layout, the decode
# format): the activation codes are packed rows too and the product runs on the
# packed-row GEMM (weight-streaming kernel for T <= 16). Every stage against
# the oracle, and the outputs bit-identical to the FP6-tile path on the same
# weight codes.
@pytest.mark.parametrize("T,D,N,r,flags,bits", [
    (8, 4096, 4096, 32, 3, 4), (77, 4096, 512, 32, 3, 4), (8, 16384, 64, 0, 6, 4),
    (9, 8192, 64, 64, 3, 4), (13, 4096, 96, 32, 1, 3), (16, 640, 64, 16, 3 | (20 << 16), 4)])
def test_rotated_linear_packed(rw, T, D, N, r, flags, bits):
    say(f"rotated_linear packed weights T={T} D={D} N={N} r={r} flags={flags:#x} bits={bits}")
    m = (flags >> 16) & 0xFF
    width = 2 * D if flags & 4 else D
    xb = W.gen_x(T + D + bits, T, width, 4, 30.0)
    Q, M = W.gen_basis(T + r, D, r) if flags & 1 else (None, None)
    Wf = W.gen_weight(N + D, N, D, 0.02)
    tiles, s_w, codes, src = rw.prep_weight(dev(Wf), bool(flags & 2), bits, m if m else 1)
    q_w, s_wh = O.quant_sym(host(src), bits)
    np.testing.assert_array_equal(host(codes), O.pack_int4(q_w))
    np.testing.assert_array_equal(host(s_w), s_wh)
    fl = flags | rw.RW4_ABITS(bits)
    y_p = _check_unit(rw, xb, Q, M, fl | rw.RW4_WPACKED, codes, s_w, q_w, s_wh)
    y_t, _ = rw.rotated_linear(dev(xb), tiles, s_w, fl, dev(Q) if r else None,
                               dev(M) if r else None)
    _sync()
    np.testing.assert_array_equal(y_p, host(y_t))


# lower code widths [RSQ 实验: W3A3]: 3-bit weights and activations through the
# fused prologue (D = 4096), the tiny workload's shape, the unfused path
# (D = 8192), and 2-bit activations on the transform-only path
@pytest.mark.parametrize("T,D,N,r,flags,bits", [(64, 256, 256, 8, 3, 3), (300, 4096, 384, 32, 3, 3),
                                                (40, 8192, 96, 64, 3, 3), (50, 1024, 64, 0, 2, 2)])
def test_rotated_linear_low_bits(rw, T, D, N, r, flags, bits):
    say(f"rotated_linear W{bits}A{bits} T={T} D={D} N={N} r={r} flags={flags}")
    xb = W.gen_x(T + D + bits, T, D, 4, 30.0)
    Q, M = W.gen_basis(T + r, D, r) if flags & 1 else (None, None)
    Wf = W.gen_weight(N + bits, N, D, 0.02)
    codes_w, s_w, qw, sw_h = _prep(rw, Wf, bool(flags & 2), bits)
    assert np.abs(qw).max() == 2 ** (bits - 1) - 1
    _check_unit(rw, xb, Q, M, flags | rw.RW4_ABITS(bits), codes_w, s_w, qw, sw_h)


# structured transforms inside the unit: H_{2^n} (x) H_m (the FFN width
# 14336 = 512 x 28 of the pages' 8B model, gated), after the alignment on the
# unfused path, and the transform across heads before the output projection
@pytest.mark.parametrize("T,D,N,r,flags,m,bits", [
    (50, 14336, 64, 0, 4 | 2, 28, 4), (37, 28 * 512, 96, 0, 2, 28, 4),
    (21, 640, 64, 16, 1 | 2, 20, 4), (130, 768, 128, 0, 2, 12, 3),
    (33, 4096, 128, 0, 0, 0, 4), (9, 2048, 64, 0, 0, 0, 3)])
def test_rotated_linear_structured(rw, T, D, N, r, flags, m, bits):
    fl = flags | rw.RW4_ABITS(bits)
    if m:
        fl |= rw.RW4_KRON(m)
    else:
        fl |= rw.RW4_HEADS(32 if D == 4096 else 16)
    say(f"rotated_linear structured T={T} D={D} N={N} r={r} flags={fl:#x}")
    width = 2 * D if flags & 4 else D
    xb = W.gen_x(T + D + m, T, width, 4, 30.0)
    Q, M = W.gen_basis(T + r, D, r) if flags & 1 else (None, None)
    Wf = W.gen_weight(N + m, N, D, 0.02)
    rotate = m > 0
    signs = np.random.default_rng(D).choice([-1.0, 1.0], D).astype(np.float32) if m == 12 else None
    if signs is not None:
        # a randomized rotation of the weights exercises the signs; the unit's
        # own online transform is the plain one, so the weights it sees are
        # only used for the GEMM stage check
        _prep(rw, Wf, True, bits, m, signs)
    codes_w, s_w, qw, sw_h = _prep(rw, Wf, rotate, bits, m if m else 1)
    _check_unit(rw, xb, Q, M, fl, codes_w, s_w, qw, sw_h)


def test_rotated_linear_strided_input(rw):
    """Row-strided bf16 input (the V third of a QKV output)."""
    T, D, N = 24, 256, 64
    big = W.gen_x(3, T, 3 * D, 2, 10.0)
    Wf = W.gen_weight(4, N, D, 0.02)
    codes_w, s_w, qw, sw_h = _prep(rw, Wf, False)
    g = dev(big)[:, 2 * D:3 * D]
    y, ws = rw.rotated_linear(g, codes_w, s_w, 0)
    q, s = O.quant_int4(W.bf16_bits_to_f32(big[:, 2 * D:]))
    ref = O.epilogue(O.gemm_int(q, qw), s, sw_h)
    nbad, worst = bf16_rel(host(y), ref)
    assert nbad == 0, worst


def _special_rows(T, D, seed):
    """bf16 bits [T][D]: degenerate rows first, then ordinary activations."""
    rng = np.random.default_rng(seed)
    x = W.bf16_bits_to_f32(W.gen_x(seed, T, D, 4, 30.0))
    x[0] = 0.0                                                    # all zero
    x[1] = 0.0
    x[1, D // 3] = -3.0                                           # one entry
    x[2] = W.bf16_bits_to_f32((rng.integers(1, 0x80, D) | (rng.integers(0, 2, D) << 15))
                              .astype(np.uint16))                 # bf16 subnormals only
    x[3] = rng.standard_normal(D).astype(np.float32) * np.float32(1e30)   # large
    x[4] = 1.0                                                    # constant: one Walsh row
    x[5] = np.where(np.arange(D) % 2 == 0, 1.0, -1.0)             # alternating: another
    return W.f32_to_bf16_bits(x)


# degenerate token rows through the fused prologue (D = 4096, r = 32), the
# unfused path (D = 8192) and the quantizer alone; 3-bit codes on one case
@pytest.mark.parametrize("T,D,r,flags,bits,prepared", [
    (40, 4096, 32, 3, 4, True), (40, 4096, 32, 3, 4, False), (40, 4096, 32, 3, 3, True),
    (12, 8192, 64, 3, 4, True), (12, 4096, 0, 2, 4, False), (12, 4096, 0, 0, 4, False)])
def test_rotated_linear_special_rows(rw, T, D, r, flags, bits, prepared):
    say(f"rotated_linear special rows T={T} D={D} r={r} flags={flags} bits={bits} "
        f"prepared={prepared}")
    t = torch()
    N = 64
    xb = _special_rows(T, D, seed=D + r + flags)
    Q, M = W.gen_basis(D + r, D, r) if r else (None, None)
    Wf = W.gen_weight(N + D, N, D, 0.02)
    codes_w, s_w, qw, sw_h = _prep(rw, Wf, bool(flags & 2), bits)
    fl = flags | rw.RW4_ABITS(bits)
    dbg = t.empty((T, D), dtype=t.float32, device="cuda")
    if prepared:
        basis = rw.respin_prepare_basis(dev(Q), dev(M)) if r else None
        y, ws = rw.rotated_linear_prepared(dev(xb), codes_w, s_w, fl, basis, r, dbg_prequant=dbg)
    else:
        y, ws = rw.rotated_linear(dev(xb), codes_w, s_w, fl, dev(Q) if r else None,
                                  dev(M) if r else None, dbg_prequant=dbg)
    _sync()
    pre, y = host(dbg), host(y)
    tiles_g, sa_g = (host(v) for v in rw.workspace_views(ws, T, D))
    ref_pre = O.prequant(O.bf16_to_f64(xb), fl, Q, M)
    assert np.isfinite(pre).all()
    # the zero row stays exactly zero, with zero codes and a zero scale
    assert not pre[0].any() and sa_g[0] == 0.0 and not y[0].any()
    # every row with normal-range values on its own
    for i in [1, 3, 4, 5] + list(range(6, T)):
        assert normwise(pre[i:i + 1], ref_pre[i:i + 1]) <= FP32_TOL, i
    # The subnormal row: the alignment's correction multiplies the r
    # projections z = Q^T x as bf16 (hi, lo) pairs, and for |z_j| near 1e-39
    # the low half underflows bf16's subnormal spacing 2^-133, so each z_j is
    # off by at most 2^-134. Q is orthonormal and the Hadamard orthogonal,
    # hence ||err||_inf <= ||err||_2 <= ||M - I||_2 sqrt(r) 2^-134, plus fp32's
    # own subnormal rounding (2^-150 per step, log2 D steps of the transform).
    floor = np.log2(D) * 2.0 ** -149
    if r:
        floor += np.linalg.norm(M.astype(np.float64) - np.eye(r), 2) * np.sqrt(r) * 2.0 ** -133
    err2 = np.abs(pre[2] - ref_pre[2]).max()
    say(f"   subnormal row: max error {err2:.3e}, bound {FP32_TOL * np.abs(ref_pre[2]).max() + floor:.3e}")
    assert err2 <= FP32_TOL * np.abs(ref_pre[2]).max() + floor
    q, s = O.quant_sym(pre, bits)
    np.testing.assert_array_equal(sa_g, s)
    np.testing.assert_array_equal(F.untile(tiles_g, T, D), q)
    nbad, worst = bf16_rel(y, O.epilogue(O.gemm_int(q, qw), s, sw_h))
    assert nbad == 0, worst


def test_empty_batches(rw):
    """T = 0 through every entry point that takes token rows: no error, no write."""
    say("empty batches")
    t = torch()
    D, N, r = 4096, 64, 32
    x0 = t.empty((0, D), dtype=t.bfloat16, device="cuda")
    xf = t.empty((0, D), dtype=t.float32, device="cuda")
    Q, M = (dev(v) for v in W.gen_basis(5, D, r))
    basis = rw.respin_prepare_basis(Q, M)
    codes_w, s_w, _, _ = _prep(rw, W.gen_weight(6, N, D, 0.02), True)
    for direct in (False, True):
        assert rw.respin_align(x0, Q, M, direct=direct).shape == (0, D)
    assert rw.respin_align_prepared(x0, basis, r).shape == (0, D)
    assert rw.fwht(xf).shape == (0, D)
    assert rw.hadamard_transform(t.empty((0, 28 * 64), dtype=t.float32, device="cuda"),
                                 28).shape == (0, 28 * 64)
    assert rw.head_hadamard(x0, 32).shape == (0, D)
    c, s = rw.quant_act_sym(xf, 3)
    assert c.shape == (0, D // 2) and s.shape == (0,)
    a = t.empty((0, D // 2), dtype=t.uint8, device="cuda")
    w_codes = t.zeros((N, D // 2), dtype=t.uint8, device="cuda")
    assert rw.w4a4_gemm(a, t.empty((0,), device="cuda"), w_codes, s_w).shape == (0, N)
    guard = t.full((4, N), 7.0, dtype=t.bfloat16, device="cuda")
    for fl in (3, 0, 2 | rw.RW4_ABITS(3), rw.RW4_HEADS(32)):
        y, _ = rw.rotated_linear(x0, codes_w, s_w, fl, Q, M, out=guard[:0])
        y2, _ = rw.rotated_linear_prepared(x0, codes_w, s_w, fl, basis, r, out=guard[:0])
        assert y.shape == (0, N) and y2.shape == (0, N)
    _sync()
    assert bool((guard == 7.0).all())


# ---------------------------------------------------------------- decoder layer
def _layer_check(rw, cid, packed=False):
    wl = W.CONFIGS[cid]
    say(f"layer {wl.name} packed={packed}")
    t = torch()
    D, T, F_ = wl.D, wl.T, wl.ffn
    inp = W.workload_inputs(wl)
    weights, qws, sws = {}, {}, {}
    for lin in wl.linears:
        tl, s, c, src = rw.prep_weight(dev(inp["W"][lin.name]), lin.rotate)
        weights[lin.name] = (c if packed else tl, s)
        qws[lin.name] = O.unpack_int4(host(c))
        sws[lin.name] = host(s)
        del src, c
    aligns = [(rw.respin_prepare_basis(dev(Q), dev(M)), Q.shape[1]) for Q, M in inp["basis"]]
    dbg = t.empty((T, F_), dtype=t.float32, device="cuda")
    st = rw.layer(dev(inp["x"]), aligns, weights, D, dbg_down=dbg, packed=packed)
    _sync()
    down_codes, down_sa = (host(v) for v in rw.workspace_views(st.pop("down_ws"), T, F_, packed))
    g = {k: host(v) for k, v in st.items()}
    pre_down = host(dbg)
    del st, dbg

    # identical-input stage parity: every oracle stage is fed the GPU's previous stage
    def lin_check(name, xin_bits, out_bits):
        q, s = O.quant_int4(O.bf16_to_f64(xin_bits).astype(np.float32))
        _check_gemm_out(out_bits, q, s, qws[name], sws[name])
    x0 = inp["x"]
    say("   qkv")
    lin_check("qkv", x0, g["qkv"])
    say("   o")
    lin_check("o", np.ascontiguousarray(g["qkv"][:, 2 * D:3 * D]), g["o"])
    (Q1, M1), (Q2, M2) = inp["basis"]
    for name, xin, add, Qm, Mm, (basis, r) in (("x1", x0, g["o"], Q1, M1, aligns[0]),
                                               ("x2", g["x1"], g["down"], Q2, M2, aligns[1])):
        say(f"   {name}")
        _check_residual(rw, xin, add, basis, r, Qm, Mm, g[name])
    say("   gate_up")
    lin_check("gate_up", g["x1"], g["gate_up"])
    # the down projection (SiLU gate -> FWHT 16384 -> INT4 -> GEMM) on the
    # GPU's own gate|up output: pre-quant values within the fp32 bar, codes
    # and scales bit-exact on the GPU's own fp32 values, every output element
    say("   down")
    ref_pre = O.prequant(O.bf16_to_f64(g["gate_up"]), O.FLAG_SWIGLU | O.FLAG_FWHT)
    assert normwise(pre_down, ref_pre) <= FP32_TOL
    del ref_pre
    q, s = O.quant_int4(pre_down)
    np.testing.assert_array_equal(down_sa, s)
    np.testing.assert_array_equal(O.unpack_int4(down_codes) if packed else F.untile(down_codes, T, F_), q)
    _check_gemm_out(g["down"], q, s, qws["down"], sws["down"])


# the unit that also projects its own input for an alignment: the same bits
# as the unit and the projection called apart (one launch at D = 4096, the
# projection then the quantizer otherwise); packed and tiled weights, the
# transform in the unit, ragged token counts, both basis widths
@pytest.mark.parametrize("T,D,N,rr,flags,packed", [(8, 4096, 12288, 32, 0, True),
                                                   (3, 4096, 4096, 64, 0, True),
                                                   (16, 4096, 640, 32, 2, False),
                                                   (1, 4096, 4096, 8, 2, True),
                                                   (8, 1024, 512, 32, 0, True),
                                                   (5, 8192, 256, 64, 2, False)])
def test_rotated_linear_project(rw, T, D, N, rr, flags, packed):
    say(f"rotated_linear_prepared_project T={T} D={D} N={N} r={rr} flags={flags} packed={packed}")
    t = torch()
    fl = flags | (rw.RW4_WPACKED if packed else 0)
    x = dev(W.gen_x(720 + T, T, D, 8, 80.0))
    Wf = W.gen_weight(721, N, D, 0.02)
    tiles, s_w, codes, _ = rw.prep_weight(dev(Wf), bool(flags & O.FLAG_FWHT))
    w = codes if packed else tiles
    Q, M = W.gen_basis(722, D, rr)
    B = rw.respin_prepare_basis(dev(Q), dev(M))
    d1 = t.empty((T, D), dtype=t.float32, device="cuda")
    y, z, ws = rw.rotated_linear_prepared_project(x, w, s_w, fl, B, rr, dbg_prequant=d1)
    d2 = t.empty((T, D), dtype=t.float32, device="cuda")
    y_ref, ws_ref = rw.rotated_linear_prepared(x, w, s_w, fl, dbg_prequant=d2)
    z_ref = rw.respin_align_project_prepared(x, B, rr)
    _sync()
    n = rw.respin_align_project_size(T, D, rr)
    np.testing.assert_array_equal(host(y), host(y_ref))
    np.testing.assert_array_equal(host(d1), host(d2))
    np.testing.assert_array_equal(host(z)[:n], host(z_ref)[:n])
    (c1, s1), (c2, s2) = rw.workspace_views(ws, T, D, packed), rw.workspace_views(ws_ref, T, D, packed)
    np.testing.assert_array_equal(host(s1), host(s2))
    # the codes of the T rows (tiles pad to 256 rows that nobody writes)
    dec = (lambda c: host(c)) if packed else (lambda c: F.untile(host(c), T, D))
    np.testing.assert_array_equal(dec(c1), dec(c2))
    # the projection finishes into the oracle's alignment: the residual
    # product on it against respin_align_prepared is checked by the residual
    # test; here its lift through the residual entry with a zero block output
    if packed and N == D:
        zero_x = t.zeros((T, 2 * D if fl & O.FLAG_SWIGLU else D), dtype=t.bfloat16, device="cuda")
        _, res_out, _ = rw.rotated_linear_prepared_residual(zero_x, w, s_w, fl, x, B, rr, z)
        res_ref = rw.respin_align_prepared(x, B, rr, out_dtype=t.bfloat16)
        _sync()
        np.testing.assert_array_equal(host(res_out), host(res_ref))


# the product that finishes a residual alignment (short batches, packed
# weights): the same bits as the product and the aligned residual computed
# apart; decode shapes (o and down projections), ragged token counts, both
# basis widths, the gated input, an alignment narrower than 4096
@pytest.mark.parametrize("T,Din,N,rr,flags", [(8, 4096, 4096, 32, 0), (3, 4096, 4096, 32, 0),
                                              (16, 4096, 4096, 64, 0), (1, 512, 1024, 8, 0),
                                              (8, 16384, 4096, 32, 6), (5, 16384, 4096, 64, 6)])
def test_rotated_linear_residual(rw, T, Din, N, rr, flags):
    say(f"rotated_linear_prepared_residual T={T} D={Din} N={N} r={rr} flags={flags}")
    t = torch()
    fl = flags | rw.RW4_WPACKED
    xb = W.gen_x(700 + T, T, 2 * Din if flags & O.FLAG_SWIGLU else Din, 8, 80.0)
    Wf = W.gen_weight(701, N, Din, 0.02)
    _, s_w, codes, _ = rw.prep_weight(dev(Wf), bool(flags & O.FLAG_FWHT))
    res_x = dev(W.gen_x(702 + T, T, N, 8, 80.0))
    Q, M = W.gen_basis(703, N, rr)
    B = rw.respin_prepare_basis(dev(Q), dev(M))
    z = rw.respin_align_project_prepared(res_x, B, rr)
    d_fused = t.empty((T, Din), dtype=t.float32, device="cuda")
    y, res_out, ws = rw.rotated_linear_prepared_residual(dev(xb), codes, s_w, fl, res_x, B, rr, z,
                                                         dbg_prequant=d_fused)
    d_ref = t.empty((T, Din), dtype=t.float32, device="cuda")
    y_ref, ws_ref = rw.rotated_linear_prepared(dev(xb), codes, s_w, fl, dbg_prequant=d_ref)
    res_ref = rw.respin_align_prepared(res_x, B, rr, addend=y_ref, out_dtype=t.bfloat16)
    _sync()
    np.testing.assert_array_equal(host(y), host(y_ref))
    np.testing.assert_array_equal(host(res_out), host(res_ref))
    np.testing.assert_array_equal(host(d_fused), host(d_ref))
    for a, b in zip(rw.workspace_views(ws, T, Din, True), rw.workspace_views(ws_ref, T, Din, True)):
        np.testing.assert_array_equal(host(a), host(b))
    # and the aligned residual against the oracle, as the layer tests check it
    _check_residual(rw, host(res_x), host(y), B, rr, Q, M, host(res_out))


@pytest.mark.parametrize("packed", [False, True])
def test_layer_decode_config2(rw, packed):
    _layer_check(rw, 2, packed)


@pytest.mark.timeout(900)
def test_layer_prefill_config3(rw):
    _layer_check(rw, 3)
