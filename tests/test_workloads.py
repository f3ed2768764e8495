"""The seeded generators: reproducible, and shaped as the workload recipes say."""
import numpy as np

import workloads as W


def test_reproducible_and_distinct_streams():
    a = W.gen_x(1001, 8, 256, 8, 80.0)
    b = W.gen_x(1001, 8, 256, 8, 80.0)
    c = W.gen_x(1002, 8, 256, 8, 80.0)
    assert a.dtype == np.uint16 and a.shape == (8, 256)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)
    q1, m1 = W.gen_basis(1001, 256, 8, stream="basis0")
    q2, m2 = W.gen_basis(1001, 256, 8, stream="basis1")
    assert not np.array_equal(q1, q2)


def test_outlier_channels():
    x = W.bf16_bits_to_f32(W.gen_x(1000, 64, 256, 2, 50.0))
    col = np.abs(x).mean(axis=0)
    top = np.argsort(col)[-3:]
    assert col[top[-1]] > 20 and col[top[-2]] > 20 and col[top[-3]] < 2


def test_basis_properties():
    Q, M = W.gen_basis(1001, 512, 32)
    assert Q.dtype == np.float32 and M.dtype == np.float32
    np.testing.assert_allclose(Q.T.astype(np.float64) @ Q, np.eye(32), atol=1e-6)
    np.testing.assert_allclose(M.T.astype(np.float64) @ M, np.eye(32), atol=1e-6)
    assert abs(np.linalg.det(M.astype(np.float64)) - 1.0) < 1e-5
    assert np.all(np.diag(M) > 0.5) and np.all(np.diag(M) < 1.0 + 1e-6)
    Q0, M0 = W.gen_basis(1, 16, 0)
    assert Q0.shape == (16, 0) and M0.shape == (0, 0)


def test_weights_and_configs():
    w = W.gen_weight(1000, 32, 64, 0.02)
    assert w.dtype == np.float32 and abs(w.std() - 0.02) < 0.003
    assert W.CONFIGS[1].D == 4096 and W.CONFIGS[1].T == 2048 and W.CONFIGS[1].r == 32
    lin = {l.name: l for l in W.CONFIGS[3].linears}
    assert (lin["qkv"].N, lin["gate_up"].N, lin["down"].K) == (12288, 32768, 16384)
    assert lin["down"].rotate and lin["down"].swiglu and not lin["qkv"].rotate
    assert (W.CONFIGS[4].D, W.CONFIGS[4].linears[0].N) == (8192, 28672)
