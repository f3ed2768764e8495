"""Benchmark of the rotated W4A4 linear on one MI355X.

One step = one rotated_linear_prepared call (align -> FWHT -> per-token INT4 ->
W4A4 GEMM -> bf16) over the 4096-wide prefill workload (D=4096, T=2048 tokens,
r=32, K=N=4096), synthetic seeded inputs already resident in HBM. The layer's
constants are prepared once per operand set before timing: the weight tiles
and the alignment basis of (Q, M). Several copies of all operands are rotated
so that the per-step working set does not stay in the 256 MB last-level cache.
The K timed steps are the same calls captured once as a HIP graph and
replayed, as a serving loop issues them; the eager host-launched rate is
reported beside it.

Prints ONE JSON line (rank 0): tokens/s, the dominant kernel's roofline
(W4A4 GEMM, int8 MFMA), and the CPU oracle timed on a bounded token sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_I8_TOPS = 5000.0          # MI355X dense int8 MFMA, TOP/s
PEAK_FP6_TFLOPS = 10100.0      # MI355X dense FP6/FP4 MFMA, TFLOP/s (the GEMM's operand type)
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector, TFLOP/s
PEAK_FP64_TFLOPS = 78.6       # MI355X fp64 vector, TFLOP/s
METRIC = "rotated W4A4 linear tokens/s; GEMM int8-MFMA TOPS and align/quant GB/s vs peak"
# the GEMM kernel's sources: its file and the headers it compiles in
GEMM_SRC = [os.path.join(ROOT, "rotation_w4a4_quantized_amd", "csrc", f)
            for f in ("gemm6.hip", "common.hpp", "launch.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a4_gemm_D4096_T2048_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=1)
    p.add_argument("--buffers", type=int, default=8, help="operand sets rotated per step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy (counter calibration)")
    p.add_argument("--profile-configs", action="store_true",
                   help="only the other configurations (70B-shaped linear, decode and prefill "
                        "layers; short runs under a profiler)")
    p.add_argument("--profile-step", action="store_true",
                   help="only the unit's steps, the GEMM, the cold stages and the 256 MiB "
                        "calibration copy (short runs under a profiler)")
    return p.parse_args()


def _src_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_bytes():
    """HBM bytes per GEMM launch from committed counter runs, or None when the
    kernel source changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("gemm_src_sha256_16") != _src_hash(GEMM_SRC):
        return None
    return rec.get("bytes_per_launch")


def _host_threads():
    """(cores this process may run on, BLAS threads numpy uses)."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        blas = max(int(i.get("num_threads", 1)) for i in info) if info else 1
    except Exception:
        blas = None
    return cores, blas


def gpu_clocks():
    """Current and maximum shader / memory clocks as amd-smi reports them right
    after the timed runs (best effort: None when the tool is unavailable)."""
    import subprocess
    try:
        p = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True,
                           text=True, timeout=20)
        if p.returncode != 0:
            return None
        rec = json.loads(p.stdout)
        if isinstance(rec, dict) and "gpu_data" in rec:
            rec = rec["gpu_data"]
        rec = rec[0] if isinstance(rec, list) else rec
        clk = rec.get("clock", rec)
        out = {}
        for key in ("gfx_0", "mem_0"):
            c = clk.get(key) if isinstance(clk, dict) else None
            if isinstance(c, dict):
                out[key] = {k: (v.get("value") if isinstance(v, dict) else v)
                            for k, v in c.items() if k in ("clk", "max_clk", "min_clk")}
        return out or None
    except Exception:
        return None


def cpu_baseline(wl, inp, seconds):
    """The oracle, as it stands, on a bounded token sample of the same workload."""
    import oracle as O
    cores, threads = _host_threads()
    Q, M = inp["basis"][0]
    qw, s_w, _ = O.prep_weight(inp["W"]["lin"], rotate=True)      # offline, untimed
    sample = 128
    x = inp["x"]
    done, t_total, i = 0, 0.0, 0
    while t_total < seconds and done < wl.T * 64:
        rows = x[(i * sample) % wl.T:(i * sample) % wl.T + sample]
        t0 = time.perf_counter()
        O.rotated_linear(rows, O.FLAG_ALIGN | O.FLAG_FWHT, qw, s_w, Q, M)
        t_total += time.perf_counter() - t0
        done += rows.shape[0]
        i += 1
    return {"value": done / t_total, "unit": "tokens/s", "cores": cores, "blas_threads": threads,
            "kind": "oracle",
            "sample": f"{done} tokens of the same workload in {sample}-token batches "
                      f"(float64 align+FWHT, fp32 quant, float64-BLAS integer GEMM), "
                      f"{t_total:.1f} s"}


def _oracle_layer(O, x_bits, basis, wq, sw, D):
    """One decoder layer's chain through the oracle's stages (each token attends
    only to itself): qkv, o on the V third, the first residual alignment, gate+up,
    the gated down projection behind the transform, the second residual."""
    (Q1, M1), (Q2, M2) = basis
    qkv = O.rotated_linear(x_bits, 0, wq["qkv"], sw["qkv"])["y"]
    o = O.rotated_linear(np.ascontiguousarray(qkv[:, 2 * D:3 * D]), 0, wq["o"], sw["o"])["y"]
    x1 = O.residual(x_bits, Q1, M1, o)
    gu = O.rotated_linear(x1, 0, wq["gate_up"], sw["gate_up"])["y"]
    d = O.rotated_linear(gu, O.FLAG_SWIGLU | O.FLAG_FWHT, wq["down"], sw["down"])["y"]
    return O.residual(x1, Q2, M2, d)


def cpu_baseline_configs(seconds):
    """The oracle on the other workloads, each on a bounded token sample of its
    own inputs (weights prepared untimed): the decode layer (T = 8) and the
    prefill layer (T = 4096) through the layer chain, the 70B-shaped linear
    through the unit."""
    import oracle as O
    import workloads as W
    cores, threads = _host_threads()
    out = {}
    for cid, sample in ((2, 8), (3, 32), (4, 16)):
        wl = W.CONFIGS[cid]
        inp = W.workload_inputs(wl)
        wq, sw = {}, {}
        for lin in wl.linears:
            q, s_, _ = O.prep_weight(inp["W"][lin.name], rotate=lin.rotate)
            wq[lin.name], sw[lin.name] = q, s_
        del inp["W"]
        done, t_total, i = 0, 0.0, 0
        while t_total < seconds and done < wl.T * 8:
            r0 = (i * sample) % wl.T
            rows = inp["x"][r0:r0 + sample]
            t0 = time.perf_counter()
            if wl.is_layer:
                _oracle_layer(O, rows, inp["basis"], wq, sw, wl.D)
            else:
                Q, M = inp["basis"][0]
                O.rotated_linear(rows, O.FLAG_ALIGN | O.FLAG_FWHT, wq["lin"], sw["lin"], Q, M)
            t_total += time.perf_counter() - t0
            done += rows.shape[0]
            i += 1
        out[wl.name] = {"value": done / t_total, "unit": "tokens/s", "cores": cores,
                        "blas_threads": threads, "kind": "oracle",
                        "sample": f"{done} tokens in {sample}-token batches, {t_total:.1f} s"}
        del wq, sw, inp
    return out


def structured_rows(rw, torch, dev, timed, with_oracle):
    """The structured transforms on their workload shapes: H_{2^n} (x) H_m with
    random signs at the gated FFN width of the pages' 8B model (T = 4096
    tokens of the prefill layer, D = 14336 = 512 x 28), and the transform
    across 32 heads at the prefill linear (T = 2048, D = 4096, d_h = 128);
    bf16 in, fp32 out. Algorithmic bytes: T D (2 + 4), plus 4 D of signs."""
    import workloads as W
    out = {}
    g = torch.Generator().manual_seed(7)
    cases = [("hadamard_kron_m28_signs", 4096, 14336, 28), ("head_hadamard_nh32", 2048, 4096, 0)]
    for name, T, D, m in cases:
        x = torch.randn((T, D), generator=g).to(torch.bfloat16).to(dev)
        y = torch.empty((T, D), dtype=torch.float32, device=dev)
        if m:
            s = (torch.randint(0, 2, (D,), generator=g).float() * 2 - 1).to(dev)
            fn = lambda: rw.hadamard_transform(x, m, s, out=y)
            nbytes = T * D * 6 + 4 * D
        else:
            fn = lambda: rw.head_hadamard(x, 32, out=y)
            nbytes = T * D * 6
        ms = timed(fn)
        gbs = nbytes / (ms * 1e-3) / 1e9
        rec = {"T": T, "D": D, "us": ms * 1e3, "bytes": nbytes, "GB/s": gbs,
               "frac_hbm": gbs / PEAK_HBM_GBS, "rows_per_s": T / (ms * 1e-3)}
        if with_oracle:
            import oracle as O
            xs = W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.random.default_rng(1).standard_normal((256, D)).astype(np.float32)))
            t0 = time.perf_counter()
            if m:
                O.hadamard_kron(xs, m, np.ones(D))
            else:
                O.head_hadamard(xs, 32)
            rec["oracle_rows_per_s"] = 256 / (time.perf_counter() - t0)
        out[name] = rec
    # decode (T = 8 tokens) through the GEMM of the decode layer's linears:
    # weight-streaming, so against HBM; eight weight sets rotated so that
    # they do not stay in the 256 MB last-level cache
    dec = {}
    for name, K, N in (("qkv", 4096, 12288), ("o", 4096, 4096), ("gate_up", 4096, 32768),
                       ("down", 16384, 4096)):
        wbytes = N * K // 2                      # algorithmic: INT4 codes
        fp6_bytes = N * K * 3 // 4               # what the kernel streams (FP6 tiles)
        nset = min(24, max(2, -(-(320 << 20) // fp6_bytes)))   # >= 320 MiB of tiles in rotation
        Tdec = 8
        codes_w = [torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, generator=g).to(dev) & 0x77
                   for _ in range(nset)]
        wt = [rw.w4a4_tile_codes(c) for c in codes_w]
        del codes_w
        at = rw.w4a4_tile_codes(torch.randint(0, 256, (Tdec, K // 2), dtype=torch.uint8, generator=g).to(dev) & 0x77)
        sa = torch.rand(Tdec, device=dev)
        sw = torch.rand(N, device=dev)
        yd = torch.empty((Tdec, N), dtype=torch.bfloat16, device=dev)
        cnt = [0]

        def call():
            i = cnt[0] % nset
            cnt[0] += 1
            rw.w4a4_gemm_tiles(at, sa, wt[i], sw, Tdec, K, N, out=yd)
        ms = timed(call, n=2 * nset)
        gbs = wbytes / (ms * 1e-3) / 1e9
        # the same product on packed INT4 rows (w4a4_gemm: the weight-streaming
        # int8 kernel at T <= 16), weights rotated the same way
        nset4 = min(24, max(2, -(-(320 << 20) // wbytes)))
        pw = [torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, generator=g).to(dev) & 0x77
              for _ in range(nset4)]
        pa = torch.randint(0, 256, (Tdec, K // 2), dtype=torch.uint8, generator=g).to(dev) & 0x77
        cnt4 = [0]

        def call4():
            i = cnt4[0] % nset4
            cnt4[0] += 1
            rw.w4a4_gemm(pa, sa, pw[i], sw, out=yd)
        ms4 = timed(call4, n=2 * nset4)
        gbs4 = wbytes / (ms4 * 1e-3) / 1e9
        dec[name] = {"K": K, "N": N, "us": ms * 1e3, "weight_bytes_int4": wbytes, "GB/s": gbs,
                     "frac_hbm": gbs / PEAK_HBM_GBS,
                     "fp6_tile_bytes_streamed": fp6_bytes,
                     "GB/s_fp6_streamed": fp6_bytes / (ms * 1e-3) / 1e9,
                     "packed_int4_us": ms4 * 1e3, "packed_int4_GB/s": gbs4,
                     "packed_int4_frac_hbm": gbs4 / PEAK_HBM_GBS}
        del wt, pw
    out["decode_gemm_T8"] = dec

    # offline construction of (Q, R_sub) at the prefill shape (D = 4096, r = 32,
    # 4 subspace iterations): ten products with T (fp32 in, fp64 FMA), 2 D^2 p
    # flops each (p = r + 16)
    import workloads as W
    D, r, iters = 4096, 32, 4
    # a transition whose deviation from the identity has rank r: I + Q0 (M0 - I) Q0^T
    # for a seeded (Q0, M0), assembled on the device (a timing input only)
    Q0, M0 = (torch.from_numpy(v).to(dev).double() for v in
              W.gen_basis(11, D, r, stream="transition", skew_std=0.3))
    Tg = (torch.eye(D, dtype=torch.float64, device=dev)
          + Q0 @ (M0 - torch.eye(r, dtype=torch.float64, device=dev)) @ Q0.T).float()
    del Q0, M0
    ws = torch.empty((rw.respin_construct_workspace_size(D, r),), dtype=torch.uint8, device=dev)
    ms = timed(lambda: rw.respin_construct(Tg, r, iters, workspace=ws), n=5)
    p = r + 16
    flops = (2 * iters + 2) * 2.0 * D * D * p + 2.0 * D * D * r
    rec = {"D": D, "r": r, "iters": iters, "us": ms * 1e3, "flop": flops,
           "TFLOP/s": flops / (ms * 1e-3) / 1e12,
           "frac_fp64": flops / (ms * 1e-3) / 1e12 / PEAK_FP64_TFLOPS}
    if with_oracle:
        import oracle as O
        Ts = O.t_hat(*W.gen_basis(11, 1024, r, stream="transition", skew_std=0.3))
        t0 = time.perf_counter()
        O.construct_basis(Ts, r)
        rec["oracle_s_at_D1024"] = time.perf_counter() - t0
    out["construct_D4096_r32"] = rec
    return out


def config_rows(rw, torch, dev, timed):
    """The other configurations of the path, each timed whole: the 70B-shaped
    linear (T = 8192, D = 8192, r = 64, 8192 -> 28672, align|fwht, basis
    prepared), and the decode (T = 8) and prefill (T = 4096) layers of
    D = 4096 (QKV 4096 -> 12288, O 4096 -> 4096, the two alignments with their
    residual adds on bases prepared once, gate+up 4096 -> 32768, down
    16384 -> 4096 behind the SwiGLU gate and the FWHT). Operands are drawn on the device (their values do not
    change the time); the layers' weights are rotated over two sets (402 MB of
    FP6 tiles), so that they do not stay in the 256 MB last-level cache."""
    import workloads as W
    gd = torch.Generator(device=dev).manual_seed(11)
    out = {}

    def weight(N, K, rotate, packed=False):
        Wf = torch.randn((N, K), generator=gd, device=dev).mul_(0.02)
        tl, s, codes, _ = rw.prep_weight(Wf, rotate)
        del Wf
        return (codes, s) if packed else (tl, s)

    def basis_pair(key, D, r):
        Q, M = W.gen_basis(key, D, r)
        return torch.from_numpy(Q).to(dev), torch.from_numpy(M).to(dev)

    # 70B-shaped linear
    T, D, r, N = 8192, 8192, 64, 28672
    Q, M = basis_pair(5, D, r)
    basis = rw.respin_prepare_basis(Q, M)
    x = torch.randn((T, D), generator=gd, device=dev).to(torch.bfloat16)
    tl, sw = weight(N, D, True)
    flags = rw.RW4_ALIGN | rw.RW4_FWHT
    ws = torch.empty((rw.rotated_linear_prepared_workspace_size(T, D, r, flags),),
                     dtype=torch.uint8, device=dev)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    ms = timed(lambda: rw.rotated_linear_prepared(x, tl, sw, flags, basis, r, out=y, workspace=ws),
               n=5)
    a_t, s_a = rw.workspace_views(ws, T, D)
    gms = timed(lambda: rw.w4a4_gemm_tiles(a_t, s_a, tl, sw, T, D, N, out=y), n=5)
    ops = 2.0 * T * D * N
    out["linear_70b_T8192"] = {"T": T, "D": D, "r": r, "N": N, "us": ms * 1e3,
                               "tokens_per_s": T / (ms * 1e-3), "gemm_us": gms * 1e3,
                               "gemm_frac_fp6": ops / (gms * 1e-3) / 1e12 / PEAK_FP6_TFLOPS,
                               "gemm_frac_int8": ops / (gms * 1e-3) / 1e12 / PEAK_I8_TOPS,
                               "prologue_us": (ms - gms) * 1e3}
    del x, tl, sw, ws, y, basis, a_t, s_a

    # decoder layers
    D = 4096
    shapes = {"qkv": (3 * D, D, False), "o": (D, D, False), "gate_up": (8 * D, D, False),
              "down": (D, 4 * D, True)}
    sets = [{k: weight(N, K, rot) for k, (N, K, rot) in shapes.items()} for _ in range(2)]
    psets = [{k: weight(N, K, rot, True) for k, (N, K, rot) in shapes.items()} for _ in range(3)]
    wbytes = sum(N * K // 2 for N, K, _ in shapes.values())          # INT4 codes
    lops = sum(2.0 * N * K for N, K, _ in shapes.values())            # per token
    aligns = tuple((rw.respin_prepare_basis(*basis_pair(k, D, 32)), 32) for k in (21, 22))
    # the decode layer on packed INT4 weight rows (RW4_WPACKED, three sets: 402 MB)
    # and on FP6 tiles (two sets: 402 MB); the prefill layer on FP6 tiles
    for name, T, packed in (("layer_decode_T8", 8, True), ("layer_decode_T8_fp6_tiles", 8, False),
                            ("layer_prefill_T4096", 4096, False)):
        x0 = torch.randn((T, D), generator=gd, device=dev).to(torch.bfloat16)
        cnt = [0]
        ws_sets = psets if packed else sets

        def call():
            i = cnt[0] % len(ws_sets)
            cnt[0] += 1
            rw.layer(x0, aligns, ws_sets[i], D, packed=packed)
        ms = timed(call, n=4 if T > 8 else 24)
        rec = {"T": T, "D": D, "us": ms * 1e3, "tokens_per_s": T / (ms * 1e-3),
               "gemm_ops": lops * T, "TOPS": lops * T / (ms * 1e-3) / 1e12}
        if T <= 32:
            rec["weight_bytes_int4"] = wbytes
            rec["GB/s_int4_weights"] = wbytes / (ms * 1e-3) / 1e9
            rec["frac_hbm"] = rec["GB/s_int4_weights"] / PEAK_HBM_GBS
        else:
            rec["frac_int8"] = rec["TOPS"] / PEAK_I8_TOPS
        out[name] = rec
    del sets, psets
    return out


def graph_timed(torch, fn, n=20):
    """Average device time of one call: n calls captured once in a HIP graph
    and replayed between two events, so that the host's per-call cost (the
    Python binding) does not leave the device idle between short kernels;
    eager back-to-back calls if capture is not possible."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side), torch.cuda.graph(g, stream=side):
            for _ in range(n):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n
    except Exception:
        torch.cuda.synchronize()
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch

    import rotation_w4a4_quantized_amd as rw
    import workloads as W

    rw.lib()
    if args.profile_configs:
        dev = torch.device("cuda:0")
        rec = config_rows(rw, torch, dev, lambda fn, n=20: graph_timed(torch, fn, n))
        print(json.dumps({"profile_configs": rec}), flush=True)
        return
    wl = W.CONFIGS[args.config]
    if wl.is_layer:
        raise SystemExit("bench workloads are the single-linear configs (0, 1, 4)")
    dev = torch.device("cuda:0")
    inp = W.workload_inputs(wl)
    Q, M = inp["basis"][0]
    T, D, r = wl.T, wl.D, wl.r
    N = wl.linears[0].N
    flags = rw.RW4_ALIGN | rw.RW4_FWHT

    def g(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    Qg, Mg = g(Q), g(M)
    x0 = g(inp["x"])
    Wg = g(inp["W"]["lin"])
    tiles0, sw0, _, _ = rw.prep_weight(Wg, True)
    del Wg
    nb = max(1, args.buffers)
    sets = []
    ws_bytes = rw.rotated_linear_prepared_workspace_size(T, D, r, flags)
    for i in range(nb):
        sets.append({
            "x": x0.clone(), "w": tiles0.clone(), "sw": sw0.clone(),
            "basis": rw.respin_prepare_basis(Qg, Mg),
            "y": torch.empty((T, N), dtype=torch.bfloat16, device=dev),
            "ws": torch.empty((ws_bytes,), dtype=torch.uint8, device=dev),
        })
    torch.cuda.synchronize()

    def step(i):
        s = sets[i % nb]
        rw.rotated_linear_prepared(s["x"], s["w"], s["sw"], flags, s["basis"], r, out=s["y"],
                                   workspace=s["ws"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # context: the K steps launched one by one from the host (the binding and
    # three launches per step, ~5 us of host time, leave the device idle
    # between steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    eager_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # the measured run: the same K steps (same calls, operand sets in the same
    # rotation) captured once as a HIP graph, as a serving loop issues them,
    # and replayed between two synchronizations
    graph = None
    try:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side), torch.cuda.graph(g, stream=side):
            for i in range(args.steps):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        graph = g
    except Exception:
        torch.cuda.synchronize()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ea.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    eb.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms_ev = ea.elapsed_time(eb) / args.steps
    ms_per_step = elapsed * 1e3 / args.steps

    # The dominant kernel alone: the GEMM entry point on the same operands and
    # launch configuration, HIP events on the stream the kernel is launched on.
    def gemm(i):
        s = sets[i % nb]
        tiles, s_a = rw.workspace_views(s["ws"], T, D)
        rw.w4a4_gemm_tiles(tiles, s_a, s["w"], s["sw"], T, D, N, out=s["y"])

    for i in range(args.warmup):
        gemm(i)
    # back-to-back launches between one pair of events: the queue stays full,
    # so the average is the kernel's duration plus the dispatch gap
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ga.record()
    for i in range(args.steps):
        gemm(i)
    gb.record()
    torch.cuda.synchronize()
    gemm_ms = ga.elapsed_time(gb) / args.steps
    gemm_ops = 2.0 * T * D * N
    achieved = gemm_ops / (gemm_ms * 1e-3) / 1e12

    # stage split of the prologue (same entry points the unit uses)
    s0 = sets[0]
    tmp = torch.empty((T, D), dtype=torch.float32, device=dev)
    codes_t = torch.empty((T, D // 2), dtype=torch.uint8, device=dev)
    sa_t = torch.empty((T,), dtype=torch.float32, device=dev)

    def timed(fn, n=20):
        return graph_timed(torch, fn, n)

    # the same unit with the basis prepared inside every call (rotated_linear)
    uws = torch.empty((rw.rotated_linear_workspace_size(T, D, r, flags),), dtype=torch.uint8,
                      device=dev)
    unprepared_ms = timed(lambda: rw.rotated_linear(s0["x"], s0["w"], s0["sw"], flags, Qg, Mg,
                                                    out=s0["y"], workspace=uws))
    basis_ms = timed(lambda: rw.respin_prepare_basis(Qg, Mg, basis=s0["basis"]))
    aws = torch.empty((rw.respin_align_workspace_size(T, D, r),), dtype=torch.uint8, device=dev)
    align_unprep_ms = timed(lambda: rw.respin_align(s0["x"], Qg, Mg, out=tmp, workspace=aws))
    pws = torch.empty((rw.respin_align_prepared_workspace_size(T, D, r),), dtype=torch.uint8,
                      device=dev)
    # warm: one buffer set, replayed (it stays in the 256 MB last-level cache)
    align_warm_ms = timed(lambda: rw.respin_align_prepared(s0["x"], s0["basis"], r, out=tmp,
                                                           workspace=pws))
    fwht_warm_ms = timed(lambda: rw.fwht(tmp, out=tmp))
    quant_warm_ms = timed(lambda: rw.quant_act_int4(tmp, codes_t, sa_t))
    del tmp, codes_t, sa_t
    # cold: every call on the next of NC buffer sets (bf16 x, fp32 rows, codes,
    # scales: 52 MiB a set, 520 MiB in rotation), so that a set has left the
    # last-level cache before it comes round again
    NC = 10
    cold = [{"x": sets[i % nb]["x"], "f": torch.empty((T, D), dtype=torch.float32, device=dev),
             "c": torch.empty((T, D // 2), dtype=torch.uint8, device=dev),
             "s": torch.empty((T,), dtype=torch.float32, device=dev)} for i in range(NC)]
    for c in cold:
        c["f"].normal_()
    ctr = [0]

    def rot(fn):
        def call():
            c = cold[ctr[0] % NC]
            ctr[0] += 1
            fn(c)
        return call
    align_ms = timed(rot(lambda c: rw.respin_align_prepared(c["x"], s0["basis"], r, out=c["f"],
                                                             workspace=pws)), n=2 * NC)
    fwht_ms = timed(rot(lambda c: rw.fwht(c["f"], out=c["f"])), n=2 * NC)
    quant_ms = timed(rot(lambda c: rw.quant_act_int4(c["f"], c["c"], c["s"])), n=2 * NC)
    del cold

    # the packed-INT4 GEMM (int8 matrix cores, nibbles widened in registers) at
    # the same shape, on the same codes (packed rows of the weight, activation
    # codes from the unit's own quantizer), eight operand sets rotated as above
    codes_w0 = rw.quant_act_int4(rw.fwht(torch.from_numpy(inp["W"]["lin"]).to(dev)))[0]
    i8sets = [{"a": rw.quant_act_int4(sets[i % nb]["x"])[0], "w": codes_w0.clone(),
               "sa": torch.rand(T, device=dev), "sw": torch.rand(N, device=dev)}
              for i in range(nb)]
    del codes_w0
    for i in range(args.warmup):
        q = i8sets[i % nb]
        rw.w4a4_gemm(q["a"], q["sa"], q["w"], q["sw"], out=sets[i % nb]["y"])
    torch.cuda.synchronize()
    ga.record()
    for i in range(args.steps):
        q = i8sets[i % nb]
        rw.w4a4_gemm(q["a"], q["sa"], q["w"], q["sw"], out=sets[i % nb]["y"])
    gb.record()
    torch.cuda.synchronize()
    gemm_i8_ms = ga.elapsed_time(gb) / args.steps
    del i8sets

    if args.profile_step:
        src = torch.empty((256 << 20,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_step": wl.name, "ms_per_step": ms_per_step,
                          "gemm_us": gemm_ms * 1e3, "gemm_int8_packed_us": gemm_i8_ms * 1e3,
                          "align_cold_us": align_ms * 1e3, "fwht_cold_us": fwht_ms * 1e3,
                          "quant_cold_us": quant_ms * 1e3}), flush=True)
        return

    rows = structured_rows(rw, torch, dev, timed, not args.no_cpu_baseline)
    configs = config_rows(rw, torch, dev, timed)

    if args.copy_calibration:
        src = torch.empty((256 << 20,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # standalone stages against HBM: algorithmic bytes per call (x in, result
    # out, plus the layer's basis for the alignment) over the measured time
    stage_bytes = {"align": T * 6 * D + 4 * D * r + 4 * r * r, "fwht": T * 8 * D,
                   "quant": T * (4 * D + D // 2 + 4)}
    stage_ms = {"align": align_ms, "fwht": fwht_ms, "quant": quant_ms}
    warm_ms = {"align": align_warm_ms, "fwht": fwht_warm_ms, "quant": quant_warm_ms}
    bw = {}
    for k, nbytes in stage_bytes.items():
        gbs = nbytes / (stage_ms[k] * 1e-3) / 1e9
        bw[k] = {"bytes": nbytes, "us": stage_ms[k] * 1e3, "GB/s": gbs,
                 "frac_hbm": gbs / PEAK_HBM_GBS, "cache": "cold (10 buffer sets rotated)",
                 "us_warm": warm_ms[k] * 1e3,
                 "frac_hbm_warm": nbytes / (warm_ms[k] * 1e-3) / 1e9 / PEAK_HBM_GBS}
    align_flop = T * (4 * D * r + 2 * r * r)
    bw["align"]["TFLOP/s"] = align_flop / (align_ms * 1e-3) / 1e12
    bw["align"]["frac_fp32"] = bw["align"]["TFLOP/s"] / PEAK_FP32_TFLOPS

    traffic = traffic_bytes()
    out = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": wl.name, "D": D, "T": T, "r": r, "K": D, "N": N, "basis": "prepared once per operand set",
                   "flags": "align|fwht", "operand_sets_rotated": nb},
        "roofline": {"bound": "mfma", "kernel": "w4a4_gemm_tiles (gemm6_lds_kernel, FP6 E2M3 operands)",
                     "achieved": achieved, "peak": PEAK_FP6_TFLOPS, "unit": "TFLOP/s",
                     "unit_note": "2 ops per int4 multiply-add; codes run as exact FP6 E2M3 "
                                  "numbers, so the peak is the FP6 one",
                     "frac": achieved / PEAK_FP6_TFLOPS,
                     "frac_of_int8_peak": achieved / PEAK_I8_TOPS, "traffic": traffic,
                     "avg_launch_us": gemm_ms * 1e3, "ops_per_launch": gemm_ops},
        "gemm_int8_packed": {"kernel": "w4a4_gemm (gemm_kernel, packed INT4 rows, int8 MFMA)",
                             "avg_launch_us": gemm_i8_ms * 1e3,
                             "TOP/s": gemm_ops / (gemm_i8_ms * 1e-3) / 1e12,
                             "frac_of_int8_peak": gemm_ops / (gemm_i8_ms * 1e-3) / 1e12 / PEAK_I8_TOPS},
        "step_launch": "one captured HIP graph of the K steps" if graph is not None
                       else "eager launches",
        "eager_ms_per_step": eager_ms_per_step,
        "stages_us": {"step_events": step_ms_ev * 1e3, "align_cold": align_ms * 1e3,
                      "fwht_cold": fwht_ms * 1e3, "quant_cold": quant_ms * 1e3,
                      "gemm": gemm_ms * 1e3, "gemm_int8_packed": gemm_i8_ms * 1e3,
                      "basis_prep": basis_ms * 1e3,
                      "align_with_basis_prep": align_unprep_ms * 1e3,
                      "step_with_basis_prep": unprepared_ms * 1e3},
        "stages_vs_hbm": bw,
        "structured_transforms": rows,
        "configs": configs,
    }
    out["gpu_clocks_after_run"] = gpu_clocks()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
        out["cpu_baseline_other_configs"] = cpu_baseline_configs(args.cpu_seconds / 2)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
