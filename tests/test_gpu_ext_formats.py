"""GPU parity of the Q4_0, Q5_0 and Q6_K weight formats: the HIP kernels,
called through the C ABI, against the CPU oracle on the same seeded inputs.

The formats are the other types of the pages' files (page "自己量化": the Q4_0
file, the Q5_0 fallback for rows K-quants cannot take, the downloaded file's
Q6K tensors); mode (b) pairs Q4_0 and Q5_0 with Q8_0 activations and Q6_K with
Q8K (page "同一个 GGUF，CPU 和 Metal 生成的文字不一样", section 出处).

Bars as for Q8_0 and Q4_K: quantized weights, decoded weights and integer
block sums bit-exact; outputs within |y - y_ref| <= 1e-5 * sum_k |w_k x_k|,
and y == 0 exactly where that sum is 0.  M <= 8 takes the decode kernels;
Q4_0/Q5_0 at M > 8 take the Q8_0 prefill kernels on weights rewritten as
Q8_0 blocks; Q6_K at M > 8 takes the decode kernels eight rows at a time.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import block_quantized_matmul_gguf_amd as qmm  # noqa: E402

from test_gpu_parity import assert_within, dev, host  # noqa: E402

NAME = {qmm.Q4_0: "Q4_0", qmm.Q5_0: "Q5_0", qmm.Q6_K: "Q6_K"}
BYTES = {qmm.Q4_0: 18, qmm.Q5_0: 22, qmm.Q6_K: 210}
MODES = [qmm.MODE_F32ACT, qmm.MODE_QACT]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    qmm.lib()


def random_blocks(fmt, n, k, seed):
    """Every byte random except a finite f16 scale: every code and bit pattern."""
    g = np.random.default_rng(seed)
    nb = k // (256 if fmt == qmm.Q6_K else 32)
    blk = g.integers(0, 256, size=(n, nb, BYTES[fmt]), dtype=np.uint8)
    dpos = 209 if fmt == qmm.Q6_K else 1          # high byte of d
    blk[..., dpos] &= 0x1F                         # |d| below 2^-8: keeps sums modest
    return blk.reshape(n, -1)


def run(fmt, mode, wq, n, k, x, m_max=None):
    with qmm.Plan(fmt, n, k, m_max or max(x.shape[0], 1), mode) as p:
        return host(p.run(dev(wq), dev(x)))


def ref(fmt, mode, wq, n, k, x):
    return (oracle.matmul_a if mode == qmm.MODE_F32ACT else oracle.matmul_b)(fmt, wq, n, k, x)


# ------------------------------------------------------ weight codecs ----

@pytest.mark.parametrize("fmt,n,k", [(qmm.Q4_0, 96, 576), (qmm.Q5_0, 200, 576), (qmm.Q5_0, 33, 4096),
                                     (qmm.Q6_K, 64, 1536), (qmm.Q6_K, 7, 768)])
def test_quantize_weights_bit_exact(fmt, n, k):
    w = synth.weights_f32(7000 + n + k, n, k)
    w[0, :32] = 0.0                                # an all-zero block
    w[1, :32] = np.arange(32) - 16.0               # exact ties at x/d + offset + 1/2
    w[2, 40] = -w[2, 32:64].__abs__().max()        # sign of the block maximum
    w[3, :] = np.random.default_rng(n + k).integers(-4, 5, k)  # magnitude ties of both signs everywhere
    w[4, :32] = 0.0
    w[4, 0], w[4, 1] = 4.0, -4.0                   # the first of the tied maxima sets d's sign
    got = host(qmm.quantize_weights(fmt, dev(w)))
    assert np.array_equal(got, oracle.quantize(fmt, w)), NAME[fmt]


@pytest.mark.parametrize("fmt,n,k", [(qmm.Q4_0, 70, 576), (qmm.Q5_0, 70, 4160), (qmm.Q6_K, 33, 768),
                                     (qmm.Q6_K, 20, 4096)])
def test_dequantized_weights_bit_exact_on_random_bytes(fmt, n, k):
    # Q6_K K = 768: three super-blocks per row, so every other row starts at
    # an address that is 2 mod 4
    wq = random_blocks(fmt, n, k, 7100 + k)
    got = host(qmm.dequantize_weights(fmt, dev(wq), n, k))
    want = oracle.dequantize(fmt, wq, k).astype(np.float32)  # exact value, rounded once
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), NAME[fmt]


# ----------------------------------------------------- matmul parity ----

SHAPES = [
    (qmm.Q4_0, 576, 576),
    (qmm.Q4_0, 200, 576),     # ragged N
    (qmm.Q4_0, 130, 4096),
    (qmm.Q5_0, 192, 576),     # attn_k
    (qmm.Q5_0, 1536, 576),    # ffn_gate
    (qmm.Q5_0, 100, 4160),    # 65 block pairs: a second pass over the lanes
    (qmm.Q6_K, 576, 1536),    # ffn_down
    (qmm.Q6_K, 70, 256),      # one super-block per row
    (qmm.Q6_K, 45, 768),      # odd super-block count: misaligned rows
    (qmm.Q6_K, 33, 4352),     # 17 super-blocks, 136 pieces: three passes
]


@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
@pytest.mark.parametrize("fmt,n,k", SHAPES, ids=[f"{NAME[f]}-{n}x{k}" for f, n, k in SHAPES])
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8, 9, 37])
def test_matmul_parity(fmt, n, k, mode, m):
    wq = oracle.quantize(fmt, synth.weights_f32(7200 + n + k, n, k))
    x = synth.acts_f32(7300 + m, m, k)
    y = run(fmt, mode, wq, n, k, x)
    yr, a = ref(fmt, mode, wq, n, k, x)
    assert_within(y, yr, a, f"{NAME[fmt]} {n}x{k} M={m} mode={mode}")


@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
@pytest.mark.parametrize("fmt,k", [(qmm.Q4_0, 1536), (qmm.Q5_0, 576), (qmm.Q6_K, 768), (qmm.Q6_K, 1024)])
@pytest.mark.parametrize("m", [1, 4, 12])
def test_matmul_parity_on_random_bytes(fmt, k, mode, m):
    n = 50
    wq = random_blocks(fmt, n, k, 7400 + k + m)
    x = synth.acts_f32(7500 + m, m, k)
    y = run(fmt, mode, wq, n, k, x)
    yr, a = ref(fmt, mode, wq, n, k, x)
    assert_within(y, yr, a, f"{NAME[fmt]} random bytes M={m} mode={mode}")


# Q6_K at M = 1 with an even super-block count runs on the one-row kernel (four
# lanes per super-block, odd super-blocks two bytes into a dword): partial
# segments (2 and 6 super-blocks), a whole one, mode (b)'s two and four segments,
# ragged N; three runs bit-equal.
Q6_ROW = [(77, 512), (1000, 1536), (130, 4096), (40, 8192), (33, 16384)]


@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
@pytest.mark.parametrize("n,k", Q6_ROW, ids=[f"{n}x{k}" for n, k in Q6_ROW])
def test_q6_k_one_row_parity(n, k, mode):
    wq = oracle.quantize(qmm.Q6_K, synth.weights_f32(7600 + n + k, n, k))
    x = synth.acts_f32(7601 + k, 1, k)
    with qmm.Plan(qmm.Q6_K, n, k, 1, mode) as p:
        wd, xd = dev(wq), dev(x)
        ys = [host(p.run(wd, xd)) for _ in range(3)]
    for y in ys[1:]:
        assert np.array_equal(y.view(np.uint32), ys[0].view(np.uint32))
    yr, a = ref(qmm.Q6_K, mode, wq, n, k, x)
    assert_within(ys[0], yr, a, f"Q6_K {n}x{k} M=1 mode={mode}")


@pytest.mark.parametrize("fmt,n,k", [(qmm.Q4_0, 40, 256), (qmm.Q5_0, 40, 256), (qmm.Q6_K, 24, 512)])
@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
@pytest.mark.parametrize("m", [1, 3, 10])
def test_integer_special_case_is_exact(fmt, n, k, mode, m):
    # d = 1 (and Q6_K scales 1): weights are q - offset; integer activations
    # with a +-127 in every block quantize losslessly, and every partial sum is
    # an integer below 2^24: both modes must equal the integer matmul exactly
    g = np.random.default_rng(7600 + fmt + m)
    if fmt == qmm.Q6_K:
        blk = random_blocks(fmt, n, k, 7601).reshape(n, k // 256, 210)
        blk[..., 192:208] = 1
        blk[..., 208:210] = [0x00, 0x3C]
        wq = blk.reshape(n, -1)
        x = synth.integer_acts(7602 + m, m, k, 256)
    else:
        blk = random_blocks(fmt, n, k, 7603).reshape(n, k // 32, BYTES[fmt])
        blk[..., 0:2] = [0x00, 0x3C]
        wq = blk.reshape(n, -1)
        x = synth.integer_acts(7604 + m, m, k, 32)
    want = x.astype(np.int64) @ np.rint(oracle.dequantize(fmt, wq, k)).astype(np.int64).T
    y = run(fmt, mode, wq, n, k, x)
    assert np.array_equal(y, want.astype(np.float32)), (NAME[fmt], mode, m)
    assert g is not None


@pytest.mark.parametrize("fmt,n,k", [(qmm.Q4_0, 70, 576), (qmm.Q5_0, 33, 1536), (qmm.Q6_K, 45, 768),
                                     (qmm.Q4_0, 41, 16384), (qmm.Q6_K, 30, 4096)])
@pytest.mark.parametrize("m", [1, 2, 3, 8, 11])
def test_traced_run_integer_parts_bit_exact(fmt, n, k, m):
    # the run's own kernels (one-row decode, staged decode with the activations
    # quantized in its prologue or by the preparation launch, the Q8_0 prefill
    # on the rewritten weights) with their integer parts written out
    wq = oracle.quantize(fmt, synth.weights_f32(7700 + n, n, k))
    x = synth.acts_f32(7701 + m, m, k)
    ties = synth.tie_rows(7702 + m, k)
    if m == 1:
        x[0] = ties[1 if fmt == qmm.Q6_K else 0]
    else:
        x[:2] = ties
    want = oracle.block_sums(fmt, wq, n, k, x)
    with qmm.Plan(fmt, n, k, m, qmm.MODE_QACT) as p:
        wd, xd = dev(wq), dev(x)
        y, sums, act = p.run_traced(wd, xd)
        y_run = host(p.run(wd, xd))
    y, got, act = host(y), host(sums).astype(np.int64), host(act)
    assert np.array_equal(y.view(np.uint32), y_run.view(np.uint32)), (NAME[fmt], m, "traced y")
    assert np.array_equal(act, oracle.quantize(qmm.ACT_FORMAT[fmt], x)), (NAME[fmt], m, "activations")
    got = got.reshape(want.shape)
    if fmt == qmm.Q6_K and m > qmm.GEMV_MAX_M:
        # the prefill kernel carries the scales in its weight operand: it forms
        # each super-block's sumi exactly, and no per-16 sums
        got, want = got.reshape(m, n, -1, 17), want.reshape(m, n, -1, 17)
        assert np.all(got[..., :16] == np.iinfo(np.int32).min)
        got, want = got[..., 16], want[..., 16]
    assert np.array_equal(got, want), (NAME[fmt], m)


@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
@pytest.mark.parametrize("n,k", [(576, 1536), (45, 768), (300, 4352), (1000, 256)])
@pytest.mark.parametrize("m", [9, 64, 130, 307])
def test_q6_k_prefill_parity(n, k, mode, m):
    # the Q6_K prefill kernel: several row and column tiles, ragged edges,
    # rows that start two bytes into a dword (odd super-block counts)
    wq = oracle.quantize(qmm.Q6_K, synth.weights_f32(7800 + n + k, n, k))
    x = synth.acts_f32(7801 + m, m, k)
    y = run(qmm.Q6_K, mode, wq, n, k, x)
    yr, a = ref(qmm.Q6_K, mode, wq, n, k, x)
    assert_within(y, yr, a, f"Q6_K {n}x{k} M={m} mode={mode}")


@pytest.mark.parametrize("fmt,n,k", [(qmm.Q4_0, 200, 576), (qmm.Q6_K, 45, 768)])
@pytest.mark.parametrize("m", [1, 5, 37])
def test_dequant_form_parity(fmt, n, k, m):
    wq = oracle.quantize(fmt, synth.weights_f32(7800 + n, n, k))
    x = synth.acts_f32(7801 + m, m, k)
    y = run(fmt, qmm.MODE_DEQUANT, wq, n, k, x)
    yr, a = oracle.matmul_a(fmt, wq, n, k, x)
    assert_within(y, yr, a, f"{NAME[fmt]} dequantize-all M={m}")


@pytest.mark.parametrize("fmt", [qmm.Q4_0, qmm.Q5_0, qmm.Q6_K], ids=["Q4_0", "Q5_0", "Q6_K"])
@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
def test_runs_are_deterministic_and_m_below_plan_maximum(fmt, mode):
    n, k = 96, 1536
    wq = dev(oracle.quantize(fmt, synth.weights_f32(7900, n, k)))
    x = synth.acts_f32(7901, 12, k)
    with qmm.Plan(fmt, n, k, 12, mode) as p:
        y12 = host(p.run(wq, dev(x)))
        y3 = host(p.run(wq, dev(x[:3])))
        y12b = host(p.run(wq, dev(x)))
    assert np.array_equal(y12, y12b)
    yr, a = ref(fmt, mode, oracle.quantize(fmt, synth.weights_f32(7900, n, k)), n, k, x[:3])
    assert_within(y3, yr, a, f"{NAME[fmt]} M=3 on a plan for 12")


# ------------------------------------------------- full-size, sampled ----

@pytest.mark.parametrize("fmt", [qmm.Q4_0, qmm.Q5_0, qmm.Q6_K], ids=["Q4_0", "Q5_0", "Q6_K"])
@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
@pytest.mark.parametrize("m", [1, 8, 512])
def test_scaleup_shape_sampled_rows(fmt, mode, m):
    # 14336 x 4096 (the scale-up projection), every output computed on the
    # GPU, 64 sampled weight rows checked against the oracle
    n, k = 14336, 4096
    w = synth.weights_f32(5000, n, k)
    x = synth.acts_f32(5100, 512, k)[:m]
    wg = qmm.quantize_weights(fmt, dev(w))
    y = run(fmt, mode, host(wg), n, k, x)
    g = np.random.default_rng(7950 + m)
    rows = g.choice(n, 64, replace=False)
    if m > qmm.GEMV_MAX_M:  # the prefill: a row in every 32 (every output tile)
        rows = np.unique(np.concatenate([rows, np.arange(0, n, 32) + g.integers(0, 32, n // 32), [n - 1]]))
    wq = oracle.quantize(fmt, w[rows])
    assert np.array_equal(host(wg)[rows], wq)
    yr, a = ref(fmt, mode, wq, len(rows), k, x)
    assert_within(y[:, rows], yr, a, f"{NAME[fmt]} 14336x4096 M={m} mode={mode}")


# Rows with an odd number of 32-value blocks (K % 64 == 32): the plan runs
# them on copies one all-zero block longer.  Every path (the one-row decode,
# the staged and tile decodes, the prefill) in both modes, single and traced
# runs, grouped runs and the dequantize-all decode.
ODD = [(qmm.Q8_0, 96), (qmm.Q8_0, 608), (qmm.Q8_0, 4128), (qmm.Q4_0, 96), (qmm.Q4_0, 608), (qmm.Q5_0, 608),
       (qmm.Q5_0, 4128)]
ODD_NAME = {qmm.Q8_0: "Q8_0", **NAME}


@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
@pytest.mark.parametrize("fmt,k", ODD, ids=[f"{ODD_NAME[f]}-{k}" for f, k in ODD])
@pytest.mark.parametrize("m", [1, 3, 8, 37])
def test_odd_block_count_parity(fmt, k, mode, m):
    n = 77
    wq = oracle.quantize(fmt, synth.weights_f32(7850 + k, n, k))
    x = synth.acts_f32(7851 + m, m, k)
    assert qmm.check(fmt, n, k, m, mode) == qmm.OK
    y = run(fmt, mode, wq, n, k, x)
    yr, a = ref(fmt, mode, wq, n, k, x)
    assert_within(y, yr, a, f"{ODD_NAME[fmt]} {n}x{k} M={m} mode={mode}")
    if mode == qmm.MODE_QACT:
        with qmm.Plan(fmt, n, k, m, mode) as p:
            yt, sums, act = p.run_traced(dev(wq), dev(x))
            yt, sums, act = host(yt), host(sums).astype(np.int64), host(act)
        assert np.array_equal(yt.view(np.uint32), y.view(np.uint32))
        assert np.array_equal(sums, oracle.block_sums(fmt, wq, n, k, x))
        assert np.array_equal(act, oracle.quantize(qmm.Q8_0, x))


@pytest.mark.parametrize("fmt,k", [(qmm.Q8_0, 608), (qmm.Q4_0, 96), (qmm.Q5_0, 4128)])
def test_odd_block_count_dequantize_and_group(fmt, k):
    ns = [64, 33]
    wqs = [oracle.quantize(fmt, synth.weights_f32(7860 + n, n, k)) for n in ns]
    want = oracle.dequantize(fmt, wqs[0], k).astype(np.float32)
    assert np.array_equal(host(qmm.dequantize_weights(fmt, dev(wqs[0]), ns[0], k)), want)
    x = synth.acts_f32(7870, 1, k)
    for mode in (qmm.MODE_F32ACT, qmm.MODE_QACT):
        plans = [qmm.Plan(fmt, n, k, 1, mode) for n in ns]
        try:
            wg = [dev(w) for w in wqs]
            sep = [host(p.run(w, dev(x))) for p, w in zip(plans, wg)]
            grp = [host(y) for y in qmm.run_group(plans, wg, dev(x))]
        finally:
            for p in plans:
                p.close()
        for a_, b_ in zip(sep, grp):
            assert np.array_equal(a_, b_)


# Long rows: more units than two per lane (each lane walks its units), and
# activations too large to stage in LDS (read from global memory).
LONG = [(qmm.Q4_0, 40, 16384), (qmm.Q5_0, 24, 9216), (qmm.Q6_K, 40, 14336)]


@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
@pytest.mark.parametrize("fmt,n,k", LONG, ids=[f"{NAME[f]}-{n}x{k}" for f, n, k in LONG])
@pytest.mark.parametrize("m", [1, 3, 8])
def test_long_rows(fmt, n, k, mode, m):
    wq = oracle.quantize(fmt, synth.weights_f32(8000 + k, n, k))
    x = synth.acts_f32(8001 + m, m, k)
    y = run(fmt, mode, wq, n, k, x)
    yr, a = ref(fmt, mode, wq, n, k, x)
    assert_within(y, yr, a, f"{NAME[fmt]} {n}x{k} M={m} mode={mode}")


# Grouped runs: up to four plans sharing format, K, mode and x in one decode
# launch, their rows end to end; each output must equal its separate run bit
# for bit (the same per-row arithmetic), and the oracle within the bar.
GROUPS = [
    (qmm.Q5_0, 576, [576, 192, 192]),            # q, k, v of a SmolLM2 layer in the page's Q4K file
    (qmm.Q5_0, 576, [1536, 1536]),               # gate, up
    (qmm.Q4_0, 1536, [96, 200, 64, 130, 50]),    # five plans: two launches
    (qmm.Q6_K, 768, [45, 70]),                   # misaligned super-blocks
]


@pytest.mark.parametrize("m", [1, 3, 8])
@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
@pytest.mark.parametrize("fmt,k,ns", GROUPS, ids=[f"{NAME[f]}-{k}-{len(ns)}" for f, k, ns in GROUPS])
def test_grouped_run_equals_separate_runs(fmt, k, ns, mode, m):
    x = synth.acts_f32(8300 + k + m, m, k)
    wqs = [oracle.quantize(fmt, synth.weights_f32(8400 + i + n, n, k)) for i, n in enumerate(ns)]
    plans = [qmm.Plan(fmt, n, k, 8, mode) for n in ns]
    try:
        xg, wg = dev(x), [dev(w) for w in wqs]
        sep = [host(p.run(w, xg)) for p, w in zip(plans, wg)]
        grp = [host(y) for y in qmm.run_group(plans, wg, xg)]
    finally:
        for p in plans:
            p.close()
    for i, (n, wq) in enumerate(zip(ns, wqs)):
        assert np.array_equal(grp[i], sep[i]), f"plan {i} ({n} rows)"
        yr, a = ref(fmt, mode, wq, n, k, x)
        assert_within(grp[i], yr, a, f"group plan {i} {NAME[fmt]} {n}x{k} M={m} mode={mode}")


# M = 1 on the one-row kernel (Q4_0, Q5_0): rows of one to four 64-pair
# segments, short last segments, and (mode (a)) past its one-segment limit.
ROW_K = [(f, k) for f in (qmm.Q4_0, qmm.Q5_0) for k in (64, 960, 2048, 4096, 4160, 8192, 12352, 16384)]


@pytest.mark.parametrize("mode", MODES, ids=["a", "b"])
@pytest.mark.parametrize("fmt,k", ROW_K, ids=[f"{NAME[f]}-{k}" for f, k in ROW_K])
def test_single_row_decode_row_lengths(fmt, k, mode):
    n = 300
    wq = oracle.quantize(fmt, synth.weights_f32(8500 + k, n, k))
    x = synth.acts_f32(8501 + k, 1, k)
    y = run(fmt, mode, wq, n, k, x)
    yr, a = ref(fmt, mode, wq, n, k, x)
    assert_within(y, yr, a, f"{NAME[fmt]} {n}x{k} M=1 mode={mode}")
