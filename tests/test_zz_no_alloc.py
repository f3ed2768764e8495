"""rotated_linear_prepared_noalloc (the unit with the library's own scratch
array, for callers that cannot allocate) against rotated_linear_prepared
(needs an MI355X). Every call goes through the C ABI."""
import numpy as np
import pytest

import fp6_layout as F
import oracle as O
import workloads as W
from gpu_util import FP32_TOL, bf16_rel, dev, host, normwise, say, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rw():
    import rotation_w4a4_quantized_amd as m
    m.lib()
    return m


def _operands(rw, T, D, N, r, flags, key):
    xb = W.gen_x(key, T, 2 * D if flags & rw.RW4_SWIGLU else D, 8, 80.0)
    Wf = W.gen_weight(key + 1, N, D, 0.02)
    tiles, s_w, codes, _ = rw.prep_weight(dev(Wf), bool(flags & rw.RW4_FWHT))
    basis = None
    Q = M = None
    if r:
        Q, M = W.gen_basis(key + 2, D, r)
        basis = rw.respin_prepare_basis(dev(Q), dev(M))
    return xb, tiles, s_w, codes, basis, Q, M


PK = 1 << 29  # RW4_WPACKED: packed INT4 weight rows (the decode format)


# two calls in a row on one GPU, the second smaller than the first (the scratch
# keeps the first call's contents), then a third on the unfused alignment path
# and a gated one; and the decode shapes on packed INT4 weight rows
@pytest.mark.parametrize("seq", [((2048, 4096, 4096, 32, 3), (77, 4096, 512, 32, 3),
                                  (9, 8192, 256, 64, 3), (300, 16384, 128, 0, 6)),
                                 ((8, 4096, 12288, 32, 3 | PK), (3, 4096, 640, 32, 3 | PK),
                                  (8, 16384, 4096, 0, 6 | PK))])
def test_noalloc_matches_workspace_entry(rw, seq):
    t = torch()
    for i, (T, D, N, r, flags) in enumerate(seq):
        say(f"noalloc call {i}: T={T} D={D} N={N} r={r} flags={flags}")
        xb, tiles, s_w, codes, basis, Q, M = _operands(rw, T, D, N, r, flags, 100 + i)
        packed = bool(flags & PK)
        if packed:
            tiles = codes  # the weight operand of the call
        x = dev(xb)
        d_ref = t.empty((T, D), dtype=t.float32, device="cuda")
        y_ref, ws = rw.rotated_linear_prepared(x, tiles, s_w, flags, basis, r, dbg_prequant=d_ref)
        d_na = t.full((T, D), float("nan"), dtype=t.float32, device="cuda")
        y_na = t.full((T, N), 7.0, dtype=t.bfloat16, device="cuda")
        rw.rotated_linear_prepared_noalloc(x, tiles, s_w, flags, basis, r, out=y_na,
                                           dbg_prequant=d_na)
        y_plain = rw.rotated_linear_prepared_noalloc(x, tiles, s_w, flags, basis, r)
        t.cuda.synchronize()
        np.testing.assert_array_equal(host(y_na), host(y_ref))
        np.testing.assert_array_equal(host(y_plain), host(y_ref))
        np.testing.assert_array_equal(host(d_na), host(d_ref))
        # and the workspace entry's own results against the oracle (the same
        # stage checks as the unit tests: pre-quant values, codes, GEMM)
        pre = host(d_ref)
        ref_pre = O.prequant(O.bf16_to_f64(xb), flags, Q, M)
        assert normwise(pre, ref_pre) <= FP32_TOL
        q, s = O.quant_int4(pre)
        acts, s_a = (host(v) for v in rw.workspace_views(ws, T, D, packed))
        np.testing.assert_array_equal(s_a, s)
        np.testing.assert_array_equal(O.unpack_int4(acts) if packed else F.untile(acts, T, D), q)
        nbad, worst = bf16_rel(host(y_na), O.epilogue(O.gemm_int(q, O.unpack_int4(host(codes))),
                                                      s, host(s_w)))
        assert nbad == 0, worst


def test_noalloc_rejects_sizes_past_its_scratch(rw):
    """The 70B-shaped linear needs more than the scratch holds: refused before
    any launch, with the output untouched."""
    t = torch()
    T, D, N, r, flags = 8192, 8192, 64, 64, 3
    assert rw.rotated_linear_prepared_workspace_size(T, D, r, flags) > rw.NOALLOC_SCRATCH_BYTES
    x = t.zeros((T, D), dtype=t.bfloat16, device="cuda")
    tiles = t.zeros((rw.w4a4_tiles_size(N, D),), dtype=t.uint8, device="cuda")
    s_w = t.ones((N,), dtype=t.float32, device="cuda")
    basis = t.zeros((rw.respin_basis_size(D, r),), dtype=t.uint8, device="cuda")
    y = t.full((T, N), 7.0, dtype=t.bfloat16, device="cuda")
    with pytest.raises(rw.Rw4Error) as e:
        rw.rotated_linear_prepared_noalloc(x, tiles, s_w, flags, basis, r, out=y)
    assert e.value.status == -2
    t.cuda.synchronize()
    assert bool((y == 7.0).all())
