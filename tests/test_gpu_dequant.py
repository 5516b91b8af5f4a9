"""GPU parity of the dequantize-all form (page "同一个 GGUF，CPU 和 Metal
生成的文字不一样", section 修法: CANDLE_DEQUANTIZE_ALL decodes every weight to
f32, then a plain f32 matmul).

Bars: the decoded weights are bit-exact against the oracle's exact
dequantization rounded once to f32; outputs satisfy the mode (a) tolerance
|y - y_ref| <= 1e-5 * sum_k |w_k x_k| (the same plain definition: the f64 matmul
of the dequantized weights); runs are deterministic.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import block_quantized_matmul_gguf_amd as qmm  # noqa: E402

from test_gpu_parity import FMT_NAME, assert_within, dev, host  # noqa: E402

SHAPES = [
    (qmm.Q8_0, 576, 576),
    (qmm.Q8_0, 200, 576),     # ragged N
    (qmm.Q8_0, 130, 4096),
    (qmm.Q4_K, 576, 1536),
    (qmm.Q4_K, 70, 256),      # one super-block per row
    (qmm.Q4_K, 100, 4096),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    qmm.lib()


@pytest.mark.parametrize("fmt,n,k", SHAPES, ids=[f"{FMT_NAME[f]}-{n}x{k}" for f, n, k in SHAPES])
def test_dequantized_weights_bit_exact(fmt, n, k):
    wq = oracle.quantize(fmt, synth.weights_f32(6000 + n + k, n, k))
    got = host(qmm.dequantize_weights(fmt, dev(wq), n, k))
    want = oracle.dequantize(fmt, wq, k).astype(np.float32)  # exact value, rounded once
    assert got.dtype == np.float32
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_dequantized_weights_extreme_blocks():
    # int8 extremes, a negative and a subnormal f16 scale, an all-zero block
    blk = np.zeros((2, 2, 34), np.uint8)
    blk[0, 0, 0:2] = [0x00, 0xBC]                       # d = -1
    blk[0, 0, 2:] = np.arange(-128, 128, 8).astype(np.int8).view(np.uint8)
    blk[0, 1, 0:2] = [0x01, 0x00]                       # d = 2^-24 (subnormal)
    blk[0, 1, 2:] = np.array([127, -128] * 16, np.int8).view(np.uint8)
    blk[1, 1, 0:2] = [0xFF, 0x7B]                       # d = 65504
    blk[1, 1, 2:] = 127
    got = host(qmm.dequantize_weights(qmm.Q8_0, dev(blk), 2, 64))
    want = oracle.dequantize(qmm.Q8_0, blk, 64).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("fmt,n,k", SHAPES, ids=[f"{FMT_NAME[f]}-{n}x{k}" for f, n, k in SHAPES])
@pytest.mark.parametrize("m", [1, 3, 8, 37])
def test_dequant_form_parity(fmt, n, k, m):
    wq = oracle.quantize(fmt, synth.weights_f32(6100 + n + k, n, k))
    x = synth.acts_f32(6200 + m, m, k)
    with qmm.Plan(fmt, n, k, m, qmm.MODE_DEQUANT) as p:
        y = host(p.run(dev(wq), dev(x)))
    yr, a = oracle.matmul_a(fmt, wq, n, k, x)
    assert_within(y, yr, a, f"dequantize-all {FMT_NAME[fmt]} {n}x{k} M={m}")


@pytest.mark.parametrize("fmt,k", [(qmm.Q8_0, 4096), (qmm.Q4_K, 1536)])
def test_run_dequantized_matches_run_and_repeats(fmt, k):
    n, m = 300, 12
    wq = dev(oracle.quantize(fmt, synth.weights_f32(6300, n, k)))
    x = dev(synth.acts_f32(6301, m, k))
    with qmm.Plan(fmt, n, k, m, qmm.MODE_DEQUANT) as p:
        y1 = host(p.run(wq, x))
        wf = qmm.dequantize_weights(fmt, wq, n, k)
        y2 = host(p.run_dequantized(wf, x))
        y3 = host(p.run_dequantized(wf, x))
    assert np.array_equal(y1, y2) and np.array_equal(y2, y3)


def test_f32_weights_need_a_dequant_plan():
    n, k = 64, 576
    with qmm.Plan(qmm.Q8_0, n, k, 4, qmm.MODE_F32ACT) as p:
        with pytest.raises(qmm.QmmError) as e:
            p.run_dequantized(torch.zeros((n, k), device="cuda"), torch.zeros((2, k), device="cuda"))
        assert e.value.status == qmm.EUNSUPPORTED
