"""The no-allocation entry point (qmatmul_run_noalloc) against qmatmul_run.

The no-allocation call lays the workspace out in a static device array shared
by every call on the GPU; it must give the values a plan's run gives (same
kernels, deterministic, so bit-equal), which themselves meet the parity bar
against the oracle: |y - y_ref| <= 1e-5 * sum_k |w_k x_k|.  Calls come in
pairs, the second on a smaller input, so the second call runs on scratch
that still holds the first call's contents.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import block_quantized_matmul_gguf_amd as qmm  # noqa: E402

TOL = 1e-5
A, B = qmm.MODE_F32ACT, qmm.MODE_QACT


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    qmm.lib()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_one(fmt, mode, n, k, m, seed):
    print(f"noalloc fmt={fmt} mode={mode} N={n} K={k} M={m}", flush=True)
    wq = oracle.quantize(fmt, synth.weights_f32(seed, n, k))
    x = synth.acts_f32(seed + 1, m, k)
    wd, xd = dev(wq), dev(x)
    got = host(qmm.run_noalloc(fmt, n, k, mode, wd, xd))
    with qmm.Plan(fmt, n, k, m, mode) as p:
        want = host(p.run(wd, xd))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "no-alloc run differs from the plan's run"
    yr, acc = (oracle.matmul_a if mode == A else oracle.matmul_b)(fmt, wq, n, k, x)
    err = np.abs(got.astype(np.float64) - yr)
    assert np.all(err <= TOL * acc) and np.all((acc != 0) | (got == 0)), float((err / np.maximum(acc, 1e-300)).max())


# (format, mode, first (N, K, M), second smaller (N, K, M))
PAIRS = [
    (qmm.Q8_0, B, (576, 1536, 37), (192, 576, 9)),
    (qmm.Q8_0, A, (1000, 1536, 37), (576, 576, 1)),
    (qmm.Q8_0, B, (14336, 4096, 8), (576, 1536, 1)),
    (qmm.Q8_0, A, (14336, 4096, 8), (576, 1536, 5)),
    (qmm.Q4_K, A, (600, 4096, 8), (130, 4096, 2)),
    (qmm.Q4_K, B, (576, 1536, 37), (300, 512, 8)),
    (qmm.Q4_K, A, (576, 4096, 130), (192, 1536, 1)),
    (qmm.Q4_0, B, (576, 1536, 20), (192, 576, 1)),
    (qmm.Q5_0, A, (1536, 4096, 8), (576, 576, 3)),
    (qmm.Q5_0, A, (576, 1536, 8), (192, 576, 3)),
    (qmm.Q6_K, B, (576, 1536, 37), (192, 512, 8)),
    (qmm.Q6_K, A, (576, 1536, 37), (192, 512, 1)),
]


@pytest.mark.parametrize("fmt,mode,first,second", PAIRS)
def test_noalloc_matches_plan_run_twice(fmt, mode, first, second):
    check_one(fmt, mode, *first, seed=7000 + fmt)
    check_one(fmt, mode, *second, seed=7100 + fmt)


def test_noalloc_rejects_what_does_not_fit():
    # Q4_0 prefill rewrites the weights as Q8_0 blocks in the workspace: 14336 x 4096 needs ~62 MB
    n, k, m = 14336, 4096, 64
    need = qmm.workspace_bytes(qmm.Q4_0, n, k, m, B)
    assert need > qmm.NOALLOC_SCRATCH_BYTES
    w = torch.zeros(n * qmm.row_bytes(qmm.Q4_0, k), dtype=torch.uint8, device="cuda")
    x = torch.zeros((m, k), dtype=torch.float32, device="cuda")
    with pytest.raises(qmm.QmmError) as e:
        qmm.run_noalloc(qmm.Q4_0, n, k, B, w, x)
    assert e.value.status == qmm.EINVAL and "scratch" in str(e.value)
    with pytest.raises(qmm.QmmError) as e:
        qmm.run_noalloc(qmm.Q8_0, 64, 64, qmm.MODE_DEQUANT, torch.zeros(64 * 68, dtype=torch.uint8, device="cuda"),
                        torch.zeros((1, 64), dtype=torch.float32, device="cuda"))
    assert e.value.status == qmm.EUNSUPPORTED
    # M = 0 enqueues nothing
    y = torch.full((0, 64), 1.0, device="cuda")
    qmm.run_noalloc(qmm.Q8_0, 64, 64, B, torch.zeros(64 * 68, dtype=torch.uint8, device="cuda"),
                    torch.zeros((0, 64), dtype=torch.float32, device="cuda"), y)
