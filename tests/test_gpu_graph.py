"""Runs captured in a HIP graph: qmatmul_run enqueues kernels only (no device
allocation, no memset, no synchronization), so a captured sequence of runs
replays to the same bits as the eager runs.  Each replay is checked against
the eager result, with eager work on the same buffers between replays."""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import block_quantized_matmul_gguf_amd as qmm  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    qmm.lib()


CASES = [(qmm.Q8_0, qmm.MODE_F32ACT, 1), (qmm.Q8_0, qmm.MODE_QACT, 8), (qmm.Q4_K, qmm.MODE_QACT, 1),
         (qmm.Q8_0, qmm.MODE_QACT, 96), (qmm.Q4_K, qmm.MODE_F32ACT, 96), (qmm.Q8_0, qmm.MODE_DEQUANT, 4),
         # the other formats: one-row kernel, staged decode (in-kernel and separate activation
         # quantization), the Q8_0 rewrite for the prefill, Q6_K's eight-row launches
         (qmm.Q5_0, qmm.MODE_QACT, 1), (qmm.Q5_0, qmm.MODE_F32ACT, 1), (qmm.Q4_0, qmm.MODE_QACT, 8),
         (qmm.Q4_0, qmm.MODE_F32ACT, 96), (qmm.Q6_K, qmm.MODE_QACT, 1), (qmm.Q6_K, qmm.MODE_QACT, 12),
         (qmm.Q6_K, qmm.MODE_F32ACT, 96),
         # the register-operand decode (2..8 rows) in both modes, and the one-row Q6_K kernel
         (qmm.Q8_0, qmm.MODE_F32ACT, 8), (qmm.Q4_K, qmm.MODE_F32ACT, 5), (qmm.Q5_0, qmm.MODE_F32ACT, 3),
         (qmm.Q6_K, qmm.MODE_QACT, 8), (qmm.Q6_K, qmm.MODE_F32ACT, 1),
         # the short-row prefill (activations prepared in the launch)
         (qmm.Q8_0, qmm.MODE_F32ACT, 96), (qmm.Q5_0, qmm.MODE_QACT, 40),
         # an odd block count (the padded copies)
         (qmm.Q8_0, qmm.MODE_QACT, 1), ]


@pytest.mark.parametrize("fmt,mode", [(qmm.Q8_0, qmm.MODE_F32ACT), (qmm.Q8_0, qmm.MODE_QACT), (qmm.Q4_K, qmm.MODE_QACT),
                                      (qmm.Q5_0, qmm.MODE_QACT), (qmm.Q6_K, qmm.MODE_F32ACT)])
def test_graph_replays_of_grouped_prefill(fmt, mode):
    # a layer's q/k/v (576, 192, 192 rows) as one grouped run at M = 307, captured
    k, m, ns = (1536 if fmt in (qmm.Q4_K, qmm.Q6_K) else 576), 307, [576, 192, 192]
    dev = torch.device("cuda")
    w = [torch.from_numpy(oracle.quantize(fmt, synth.weights_f32(7200 + n + i, n, k))).to(dev) for i, n in enumerate(ns)]
    x = torch.from_numpy(synth.acts_f32(7300, m, k)).to(dev)
    ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for n in ns]
    plans = [qmm.Plan(fmt, n, k, m, mode) for n in ns]
    try:
        stream = torch.cuda.current_stream()
        qmm.run_group(plans, w, x, ys, stream)
        torch.cuda.synchronize()
        ref = [t.clone() for t in ys]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            qmm.run_group(plans, w, x, ys, torch.cuda.current_stream())
        for rep in range(4):
            for t in ys:
                t.fill_(float("nan"))
            qmm.run_group(plans, w, x, ys, stream)  # eager work between replays
            torch.cuda.synchronize()
            assert all(torch.equal(a, b) for a, b in zip(ys, ref))
            for t in ys:
                t.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(zip(ys, ref)):
                assert torch.equal(a, b), f"replay {rep}, plan {i} differs from the eager grouped run"
        del g
    finally:
        for p in plans:
            p.close()


@pytest.mark.parametrize("fmt,mode,m", CASES, ids=[f"fmt{f}-mode{md}-M{m}" for f, md, m in CASES])
def test_graph_replays_match_eager_runs(fmt, mode, m):
    n, k = 640, 1536 if fmt in (qmm.Q4_K, qmm.Q6_K) else 576
    if (fmt, mode, m) == CASES[-1]:
        k = 608  # 19 blocks
    dev = torch.device("cuda")
    w = [torch.from_numpy(oracle.quantize(fmt, synth.weights_f32(7000 + i, n, k))).to(dev) for i in range(3)]
    x = torch.from_numpy(synth.acts_f32(7100 + m, m, k)).to(dev)
    ys = [torch.empty((m, n), dtype=torch.float32, device=dev) for _ in w]
    with qmm.Plan(fmt, n, k, m, mode) as p:
        stream = torch.cuda.current_stream()
        for wi, yi in zip(w, ys):  # eager runs (also set the kernels' launch attributes before capture)
            p.run(wi, x, yi, stream)
        torch.cuda.synchronize()
        ref = [t.clone() for t in ys]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            for wi, yi in zip(w, ys):
                p.run(wi, x, yi, cap)
        for rep in range(4):
            for t in ys:
                t.fill_(float("nan"))
            p.run(w[0], x, ys[0], stream)  # eager work on the same plan and buffers between replays
            torch.cuda.synchronize()
            assert torch.equal(ys[0], ref[0])
            g.replay()
            torch.cuda.synchronize()
            for i, (a, b) in enumerate(zip(ys, ref)):
                assert torch.equal(a, b), f"replay {rep}, run {i} differs from the eager run"
        del g
