"""GPU parity: the HIP kernels, called through the C ABI, against the CPU
oracle on the same seeded inputs.

Bars: quantized activations, quantized weights and integer block sums are
bit-exact; outputs satisfy |y - y_ref| <= 1e-5 * sum_k |w_k x_k| per element
(x = the f32 activations in mode (a), the dequantized quantized activations in
mode (b)), and y == 0 exactly where that sum is 0.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import block_quantized_matmul_gguf_amd as qmm  # noqa: E402

TOL = 1e-5
FMT_NAME = {qmm.Q8_0: "Q8_0", qmm.Q4_K: "Q4_K", qmm.Q4_0: "Q4_0", qmm.Q5_0: "Q5_0", qmm.Q6_K: "Q6_K"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    qmm.lib()  # fails loudly when the library is missing


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_within(y, ref, absacc, what):
    y = y.astype(np.float64)
    err = np.abs(y - ref)
    bound = TOL * absacc
    bad = (err > bound) | ((absacc == 0) & (y != 0)) | ~np.isfinite(y)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        rows = [f"(m={i},n={j}) y={y[i, j]!r} ref={ref[i, j]!r} err={err[i, j]:.3e} bound={bound[i, j]:.3e}"
                for i, j in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; " + "; ".join(rows))
    return float((err / np.maximum(absacc, 1e-300)).max())


def run_plan(fmt, mode, wq, n, k, x, m_max=None):
    m = x.shape[0]
    with qmm.Plan(fmt, n, k, m_max or max(m, 1), mode) as p:
        return host(p.run(dev(wq), dev(x)))


def ref(fmt, mode, wq, n, k, x):
    return (oracle.matmul_a if mode == qmm.MODE_F32ACT else oracle.matmul_b)(fmt, wq, n, k, x)


# --------------------------------------------------------- quantizers ----

@pytest.mark.parametrize("m,k", [(1, 576), (3, 1536), (37, 1536), (8, 4096), (307, 576)])
def test_quantize_act_q8_0_bit_exact(m, k):
    x = synth.acts_f32(900 + m, m, k)
    got = host(qmm.quantize_act(qmm.Q8_0, dev(x)))
    assert np.array_equal(got, oracle.quantize(oracle.Q8_0, x))


@pytest.mark.parametrize("m,k", [(1, 1536), (37, 1536), (8, 4096), (5, 256)])
def test_quantize_act_q8k_bit_exact(m, k):
    x = synth.acts_f32(910 + m, m, k)
    got = host(qmm.quantize_act(qmm.Q8_K, dev(x)))
    assert np.array_equal(got, oracle.quantize(oracle.Q8_K, x))


def test_quantize_act_edge_blocks_bit_exact():
    # zero blocks, ties at x*id = k + 1/2, a +-max tie on |x| (first index wins), subnormal scales
    k = 512
    x = np.zeros((4, k), np.float32)
    x[1, :32] = np.arange(32) - 15.5          # d = 16.5/127: many values near ties
    x[1, 32:64] = 2.5
    x[1, 64] = 127.0
    x[1, 65] = -2.5
    x[2, 5], x[2, 9] = 2.0, -2.0               # Q8K sign tie: first index decides
    x[2, 300], x[2, 301] = -3.0, 3.0
    x[3] = synth.acts_f32(920, 1, k)[0] * 1e-6  # f16 d goes subnormal
    for fmt in (qmm.Q8_0, qmm.Q8_K):
        got = host(qmm.quantize_act(fmt, dev(x)))
        assert np.array_equal(got, oracle.quantize(fmt, x)), FMT_NAME.get(fmt, "Q8K")


@pytest.mark.parametrize("fmt,n,k", [(qmm.Q8_0, 96, 576), (qmm.Q4_K, 96, 1536), (qmm.Q4_K, 33, 4096)])
def test_quantize_weights_bit_exact(fmt, n, k):
    w = synth.weights_f32(930 + n, n, k)
    got = host(qmm.quantize_weights(fmt, dev(w)))
    assert np.array_equal(got, oracle.quantize(fmt, w))


@pytest.mark.parametrize("n,k", [(96, 1536), (33, 4096), (7, 256)])
def test_quantize_q4_k_search_bit_exact(n, k):
    w = synth.weights_f32(935 + n, n, k)
    w[0, :256] = 0.0
    w[0, 7:256:32], w[0, 20:256:32] = 0.5, 1.0  # the hand-worked block (the search moves it)
    w[1, :32] = np.linspace(-0.75, 3.0, 32, dtype=np.float32)
    got = host(qmm.quantize_q4_k_search(dev(w)))
    assert np.array_equal(got, oracle.quantize_q4_k_search(w))


def test_activation_quantization_is_row_local_on_gpu():
    x = synth.acts_f32(940, 37, 1536)
    full = host(qmm.quantize_act(qmm.Q8_K, dev(x)))
    one = host(qmm.quantize_act(qmm.Q8_K, dev(x[:1])))
    assert np.array_equal(one[0], full[0])
    perm = np.random.default_rng(941).permutation(37)
    assert np.array_equal(host(qmm.quantize_act(qmm.Q8_K, dev(x[perm]))), full[perm])


# ---------------------------------------------------- matmul parity ----

SHAPES = [
    (qmm.Q8_0, 576, 576),     # q_proj
    (qmm.Q8_0, 200, 576),     # ragged N (not a multiple of 16 or 64)
    (qmm.Q8_0, 192, 1536),    # split K, 48 blocks
    (qmm.Q8_0, 130, 4096),    # split K x4
    (qmm.Q4_K, 576, 1536),    # ffn_down
    (qmm.Q4_K, 100, 4096),
    (qmm.Q4_K, 70, 256),      # one super-block per row
]


@pytest.mark.parametrize("mode", [qmm.MODE_F32ACT, qmm.MODE_QACT], ids=["a", "b"])
@pytest.mark.parametrize("fmt,n,k", SHAPES, ids=[f"{FMT_NAME[f]}-{n}x{k}" for f, n, k in SHAPES])
@pytest.mark.parametrize("m", [1, 2, 5, 8, 9, 37, 130])
def test_matmul_parity(fmt, n, k, mode, m):
    wq = oracle.quantize(fmt, synth.weights_f32(1000 + n + k, n, k))
    x = synth.acts_f32(2000 + m, m, k)
    y = run_plan(fmt, mode, wq, n, k, x)
    yr, a = ref(fmt, mode, wq, n, k, x)
    assert_within(y, yr, a, f"{FMT_NAME[fmt]} {n}x{k} M={m} mode={mode}")


# One activation row streams weight rows whole, in segments of 64 block pairs
# (Q8_0) or 8 super-blocks (Q4_K), several rows per wave: rows longer than one
# segment with a short last segment, one-pair last segments, more rows than
# waves by far (outputs leave a wave 64 at a time), fewer rows than waves, and
# rows past the segment limit (the tile kernel takes those).
ROW_SHAPES = [
    (qmm.Q8_0, 70, 14336),    # four segments, the last 32 pairs
    (qmm.Q8_0, 33, 8256),     # three segments, the last one pair
    (qmm.Q8_0, 5, 576),       # fewer rows than waves
    (qmm.Q8_0, 140000, 64),   # about 69 rows per wave
    (qmm.Q8_0, 24, 16448),    # past the segment limit
    (qmm.Q4_K, 70, 14336),    # seven segments of super-blocks
    (qmm.Q4_K, 37, 2304),     # one short segment
    (qmm.Q4_K, 140000, 256),  # one super-block per row, about 69 rows per wave
]


# Every row length the one-row kernel compiles for: 1 to 5 load instructions per
# segment (Q8_0 rows of 64 to 4352 bytes, Q4_K of 144 to 2304), 1 to 4 segments
# per row, two or three segment buffers per wave.
ROW_K = [(qmm.Q8_0, k) for k in (64, 960, 1600, 2048, 3072, 4032, 4096, 4160, 8192, 12352, 16384)] + \
        [(qmm.Q4_K, k) for k in (256, 1792, 2304, 2560, 4352, 8192, 12288, 16384)]


@pytest.mark.parametrize("mode", [qmm.MODE_F32ACT, qmm.MODE_QACT], ids=["a", "b"])
@pytest.mark.parametrize("fmt,k", ROW_K, ids=[f"{FMT_NAME[f]}-{k}" for f, k in ROW_K])
def test_single_row_decode_row_lengths(fmt, k, mode):
    n = 41
    wq = oracle.quantize(fmt, synth.weights_f32(7000 + k, n, k))
    x = synth.acts_f32(7001 + k, 1, k)
    y = run_plan(fmt, mode, wq, n, k, x)
    yr, a = ref(fmt, mode, wq, n, k, x)
    assert_within(y, yr, a, f"{FMT_NAME[fmt]} {n}x{k} M=1 mode={mode}")


@pytest.mark.parametrize("mode", [qmm.MODE_F32ACT, qmm.MODE_QACT], ids=["a", "b"])
@pytest.mark.parametrize("fmt,n,k", ROW_SHAPES, ids=[f"{FMT_NAME[f]}-{n}x{k}" for f, n, k in ROW_SHAPES])
def test_single_row_decode_shapes(fmt, n, k, mode):
    wq = oracle.quantize(fmt, synth.weights_f32(6000 + n + k, n, k))
    x = synth.acts_f32(6001 + k, 1, k)
    y = run_plan(fmt, mode, wq, n, k, x)
    yr, a = ref(fmt, mode, wq, n, k, x)
    assert_within(y, yr, a, f"{FMT_NAME[fmt]} {n}x{k} M=1 mode={mode}")


@pytest.mark.parametrize("mode", [qmm.MODE_F32ACT, qmm.MODE_QACT], ids=["a", "b"])
@pytest.mark.parametrize("fmt", [qmm.Q8_0, qmm.Q4_K], ids=["Q8_0", "Q4_K"])
@pytest.mark.parametrize("m", [1, 8, 40])
def test_integer_special_case_is_exact(fmt, mode, m):
    # d = 1 weights (Q4_K: sc = m = 1, dmin = 1) and integer activations whose
    # every block reaches +-127: both modes equal the integer matmul exactly.
    n, k = 48, 512
    g = np.random.default_rng(77)
    if fmt == qmm.Q8_0:
        q = g.integers(-127, 128, size=(n, k))
        blk = np.zeros((n, k // 32, 34), np.uint8)
        blk[..., 0:2] = [0x00, 0x3C]
        blk[..., 2:] = q.reshape(n, k // 32, 32).astype(np.int8).view(np.uint8)
        wint = q
        x = synth.integer_acts(78, m, k, 32)
    else:
        q = g.integers(0, 16, size=(n, k))
        blk = np.zeros((n, k // 256, 144), np.uint8)
        blk[..., 0:2] = [0x00, 0x3C]
        blk[..., 2:4] = [0x00, 0x3C]
        blk[..., 4:12] = 1
        blk[..., 12:16] = 0x11
        for e in range(256):
            c, l = divmod(e, 64)
            blk[..., 16 + 32 * c + l % 32] |= (q.reshape(n, k // 256, 256)[..., e] << (0 if l < 32 else 4)).astype(np.uint8)
        wint = q - 1
        x = synth.integer_acts(78, m, k, 256)
    exact = (x.astype(np.int64) @ wint.T).astype(np.float64)
    y = run_plan(fmt, mode, blk, n, k, x)
    assert np.array_equal(y.astype(np.float64), exact)


# The traced run: the kernels that compute y (the one-row decode at M = 1,
# the tile decode at M <= 8 and past the one-row kernel's K, the int8 prefill
# at M > 8), with their integer parts written out.  Its y equals the plain
# run's bit for bit; its block sums and the quantized activations its own
# prologue or preparation formed equal the oracle's.  Rows built around the
# tie rules (half-way values; two maxima of opposite sign) are part of x.
TRACED = [
    (qmm.Q8_0, 200, 576, 1), (qmm.Q8_0, 130, 4096, 1), (qmm.Q8_0, 41, 16384, 1), (qmm.Q8_0, 30, 20480, 1),
    (qmm.Q4_K, 100, 1536, 1), (qmm.Q4_K, 41, 16384, 1), (qmm.Q4_K, 30, 20480, 1),
    (qmm.Q8_0, 200, 576, 3), (qmm.Q8_0, 130, 4096, 8), (qmm.Q4_K, 100, 1536, 2), (qmm.Q4_K, 300, 4096, 8),
    (qmm.Q8_0, 200, 576, 20), (qmm.Q8_0, 130, 4096, 37), (qmm.Q8_0, 300, 4096, 130),
    (qmm.Q4_K, 100, 1536, 37), (qmm.Q4_K, 300, 4096, 130), (qmm.Q4_K, 70, 256, 9),
    (qmm.Q8_0, 100, 1088, 20), (qmm.Q8_0, 70, 1536, 37), (qmm.Q8_0, 40, 64, 9),
    (qmm.Q4_0, 70, 576, 37), (qmm.Q5_0, 100, 1088, 20), (qmm.Q5_0, 130, 1536, 9),
    (qmm.Q4_K, 70, 1536, 307), (qmm.Q4_K, 200, 512, 20),
]


def traced_inputs(fmt, n, k, m, seed):
    wq = oracle.quantize(fmt, synth.weights_f32(seed, n, k))
    x = synth.acts_f32(seed + 1, m, k)
    ties = synth.tie_rows(seed + 2, k)
    if m == 1:
        x[0] = ties[1 if k % 256 == 0 and fmt != qmm.Q8_0 else 0]
    else:
        x[:2] = ties
    return wq, x


@pytest.mark.parametrize("fmt,n,k,m", TRACED, ids=[f"{FMT_NAME[f]}-{n}x{k}-M{m}" for f, n, k, m in TRACED])
def test_traced_run_integer_parts_bit_exact(fmt, n, k, m):
    wq, x = traced_inputs(fmt, n, k, m, 3000 + n + m)
    with qmm.Plan(fmt, n, k, m, qmm.MODE_QACT) as p:
        wd, xd = dev(wq), dev(x)
        y, sums, act = p.run_traced(wd, xd)
        y_run = host(p.run(wd, xd))
        sums_only = host(p.block_sums(wd, xd))
    y, sums, act = host(y), host(sums).astype(np.int64), host(act)
    assert np.array_equal(y.view(np.uint32), y_run.view(np.uint32)), "traced y differs from the plain run"
    assert np.array_equal(act, oracle.quantize(qmm.ACT_FORMAT[fmt], x)), "quantized activations"
    assert np.array_equal(sums, oracle.block_sums(fmt, wq, n, k, x)), "block sums"
    assert np.array_equal(sums_only.astype(np.int64), sums)
    yr, a = ref(fmt, qmm.MODE_QACT, wq, n, k, x)
    assert_within(y, yr, a, f"traced {FMT_NAME[fmt]} {n}x{k} M={m}")


@pytest.mark.parametrize("fmt,mode,m", [(qmm.Q8_0, 0, 1), (qmm.Q8_0, 1, 8), (qmm.Q4_K, 0, 8),
                                        (qmm.Q4_K, 1, 1), (qmm.Q8_0, 1, 37), (qmm.Q4_K, 0, 37)])
def test_runs_are_deterministic_and_reuse_the_plan(fmt, mode, m):
    n, k = 300, 4096
    wq = dev(oracle.quantize(fmt, synth.weights_f32(4000, n, k)))
    x = dev(synth.acts_f32(4001, m, k))
    x2 = dev(synth.acts_f32(4002, m, k))
    with qmm.Plan(fmt, n, k, 64, mode) as p:
        y1 = host(p.run(wq, x))
        p.run(wq, x2)
        y2 = host(p.run(wq, x))
    assert np.array_equal(y1, y2)


# Mode (a) decode with 2..8 rows (K <= 4096) runs with each wave's slice of
# the activation operand in registers, K split over the eight waves.  Shapes:
# one tile, ragged N, the largest slices (Q8_0 K = 4096: eight block pairs per
# wave), slices past the row's end (K = 1536: six of eight slices real; K =
# 576: the fifth slice one pair, the rest empty).  Q4_0 and Q5_0 (the page's
# own Q4K file) take the same kernel with their block pairs, every stage width
# (four pairs, two, one); Q6_K (the downloaded file's ffn_down) with super-block
# pairs (K % 512 == 0; K = 1536: three of eight slices real).  Three runs of
# one plan must agree bit for bit.
REG_SHAPES = [
    (qmm.Q8_0, 16, 2048, 3),
    (qmm.Q8_0, 200, 4096, 8),
    (qmm.Q8_0, 4100, 1024, 2),
    (qmm.Q8_0, 130, 1536, 5),
    (qmm.Q8_0, 77, 576, 7),
    (qmm.Q4_K, 130, 4096, 5),
    (qmm.Q4_K, 64, 2048, 8),
    (qmm.Q4_K, 33, 1536, 8),
    (qmm.Q4_0, 130, 4096, 8),
    (qmm.Q4_0, 300, 1024, 6),
    (qmm.Q4_0, 77, 576, 3),
    (qmm.Q4_0, 40, 128, 2),
    (qmm.Q5_0, 130, 4096, 8),
    (qmm.Q5_0, 4100, 1024, 2),
    (qmm.Q5_0, 33, 1536, 7),
    (qmm.Q5_0, 64, 128, 4),
    (qmm.Q6_K, 130, 4096, 8),
    (qmm.Q6_K, 4100, 1024, 2),
    (qmm.Q6_K, 77, 1536, 3),
    (qmm.Q6_K, 40, 512, 5),
]


@pytest.mark.parametrize("fmt,n,k,m", REG_SHAPES, ids=[f"{FMT_NAME[f]}-{n}x{k}-M{m}" for f, n, k, m in REG_SHAPES])
def test_decode_register_operand_and_k_halves(fmt, n, k, m):
    wq = oracle.quantize(fmt, synth.weights_f32(4100 + n, n, k))
    x = synth.acts_f32(4200 + m, m, k)
    with qmm.Plan(fmt, n, k, m, qmm.MODE_F32ACT) as p:
        wd, xd = dev(wq), dev(x)
        ys = [host(p.run(wd, xd)) for _ in range(3)]
    for y in ys[1:]:
        assert np.array_equal(y, ys[0])
    yr, a = ref(fmt, qmm.MODE_F32ACT, wq, n, k, x)
    assert_within(ys[0], yr, a, f"{FMT_NAME[fmt]} {n}x{k} M={m}")


# Grouped runs: plans sharing format, K and mode and one x.  At M = 1 the
# one-row kernel takes all of their rows in one launch (per four plans) and
# must give what separate runs give, bit for bit; other M run the plans in turn.
GROUPS = [
    (qmm.Q8_0, 576, [576, 192, 192]),             # q, k, v of a SmolLM2 layer
    (qmm.Q8_0, 576, [1536, 1536]),                # gate, up
    (qmm.Q8_0, 4096, [300, 77, 41, 129, 64]),     # five plans: two launches
    (qmm.Q4_K, 1536, [576, 100]),
]


@pytest.mark.parametrize("m", [1, 3])
@pytest.mark.parametrize("mode", [qmm.MODE_F32ACT, qmm.MODE_QACT], ids=["a", "b"])
@pytest.mark.parametrize("fmt,k,ns", GROUPS, ids=[f"{FMT_NAME[f]}-{k}-{len(ns)}" for f, k, ns in GROUPS])
def test_grouped_run_equals_separate_runs(fmt, k, ns, mode, m):
    x = synth.acts_f32(8000 + k + m, m, k)
    wqs = [oracle.quantize(fmt, synth.weights_f32(8100 + i + n, n, k)) for i, n in enumerate(ns)]
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
        assert_within(grp[i], yr, a, f"group plan {i} {FMT_NAME[fmt]} {n}x{k} M={m} mode={mode}")


# Prefill with short rows (Q8_0, Q4_0, Q5_0, Q4_K; K <= 1536, at most 8192 columns, a
# one-round grid): one launch that prepares its own activations.  Whole rows
# staged at once and in pieces (mode (a) at K = 1536: four of 384, two buffers
# per wave), block pairs from K = 64 up, ragged M and N, the widest launch; rows
# 0 and 1 built around the tie rules.
SHORT = [(qmm.Q8_0, 40, 64, 9), (qmm.Q8_0, 200, 576, 17), (qmm.Q8_0, 576, 576, 307), (qmm.Q8_0, 130, 1024, 37),
         (qmm.Q8_0, 100, 1088, 20), (qmm.Q8_0, 576, 1536, 37), (qmm.Q8_0, 8192, 576, 10),
         (qmm.Q8_0, 70, 1536, 307), (qmm.Q8_0, 8100, 1536, 9),
         (qmm.Q4_0, 40, 64, 9), (qmm.Q4_0, 576, 576, 307), (qmm.Q4_0, 100, 1088, 20), (qmm.Q4_0, 576, 1536, 37),
         (qmm.Q5_0, 40, 128, 9), (qmm.Q5_0, 576, 576, 307), (qmm.Q5_0, 130, 1024, 37), (qmm.Q5_0, 70, 1536, 307),
         # Q4_K: super-blocks, whole rows (mode (b): Q8K values and sums formed in the launch)
         (qmm.Q4_K, 100, 256, 9), (qmm.Q4_K, 300, 512, 20), (qmm.Q4_K, 576, 1536, 37), (qmm.Q4_K, 70, 1536, 307)]


@pytest.mark.parametrize("mode", [qmm.MODE_F32ACT, qmm.MODE_QACT], ids=["a", "b"])
@pytest.mark.parametrize("fmt,n,k,m", SHORT, ids=[f"{FMT_NAME[f]}-{n}x{k}-M{m}" for f, n, k, m in SHORT])
def test_short_row_prefill(fmt, n, k, m, mode):
    wq = oracle.quantize(fmt, synth.weights_f32(7000 + n + k, n, k))
    x = synth.acts_f32(7001 + m + k, m, k)
    x[:2] = synth.tie_rows(7002 + k, k)
    with qmm.Plan(fmt, n, k, m, mode) as p:
        wd, xd = dev(wq), dev(x)
        ys = [host(p.run(wd, xd)) for _ in range(2)]
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32)), "two runs differ"
    yr, a = ref(fmt, mode, wq, n, k, x)
    assert_within(ys[0], yr, a, f"short-row prefill {FMT_NAME[fmt]} {n}x{k} M={m} mode={mode}")


# Grouped prefill (M > 8): the activations prepared once, the plans' output
# tiles in one launch per four plans; bit for bit the separate runs.
PGROUPS = [
    (qmm.Q8_0, 576, [576, 192, 192]),             # q, k, v
    (qmm.Q8_0, 576, [1536, 1536]),                # gate, up
    (qmm.Q4_K, 1536, [576, 100, 300, 64, 33]),    # five plans: two launches
    (qmm.Q6_K, 512, [200, 77]),
    (qmm.Q4_0, 576, [576, 192]),                  # rewritten as Q8_0 blocks per plan
    (qmm.Q5_0, 1536, [96, 130]),
    # at M = 307 the wide plan takes the K-staged kernel and the others the short-row kernel
    (qmm.Q8_0, 576, [2048, 192, 64]),
    (qmm.Q5_0, 576, [4096, 100]),
]


@pytest.mark.parametrize("m", [9, 37, 307])
@pytest.mark.parametrize("mode", [qmm.MODE_F32ACT, qmm.MODE_QACT], ids=["a", "b"])
@pytest.mark.parametrize("fmt,k,ns", PGROUPS, ids=[f"fmt{f}-{k}-{len(ns)}" for f, k, ns in PGROUPS])
def test_grouped_prefill_equals_separate_runs(fmt, k, ns, mode, m):
    x = synth.acts_f32(8300 + k + m, m, k)
    wqs = [oracle.quantize(fmt, synth.weights_f32(8400 + i + n, n, k)) for i, n in enumerate(ns)]
    plans = [qmm.Plan(fmt, n, k, m, mode) for n in ns]
    try:
        xg, wg = dev(x), [dev(w) for w in wqs]
        sep = [host(p.run(w, xg)) for p, w in zip(plans, wg)]
        grp = [host(y) for y in qmm.run_group(plans, wg, xg)]
    finally:
        for p in plans:
            p.close()
    for i, (n, wq) in enumerate(zip(ns, wqs)):
        assert np.array_equal(grp[i].view(np.uint32), sep[i].view(np.uint32)), f"plan {i} ({n} rows)"
        yr, a = ref(fmt, mode, wq, n, k, x)
        assert_within(grp[i], yr, a, f"grouped prefill plan {i} fmt={fmt} {n}x{k} M={m} mode={mode}")


def test_grouped_run_rejects_mixed_plans():
    x = dev(synth.acts_f32(8200, 1, 576))
    w = dev(oracle.quantize(oracle.Q8_0, synth.weights_f32(8201, 64, 576)))
    y = [torch.empty((1, 64), device="cuda") for _ in range(2)]
    with qmm.Plan(qmm.Q8_0, 64, 576, 1, qmm.MODE_QACT) as p1, qmm.Plan(qmm.Q8_0, 64, 1536, 1, qmm.MODE_QACT) as p2, \
            qmm.Plan(qmm.Q8_0, 64, 576, 1, qmm.MODE_F32ACT) as p3:
        for other in (p2, p3):  # another K, another mode
            harr = (qmm._p * 2)(p1._h, other._h)
            warr = (qmm._p * 2)(qmm._ptr(w), qmm._ptr(w))
            yarr = (qmm._p * 2)(qmm._ptr(y[0]), qmm._ptr(y[1]))
            assert qmm.lib().qmatmul_run_group(harr, 2, warr, qmm._ptr(x), yarr, 1, None) == qmm.EINVAL


def test_m_zero_is_a_no_op():
    with qmm.Plan(qmm.Q8_0, 64, 576, 4, 0) as p:
        y = torch.full((0, 64), 7.0, device="cuda")
        p.run(dev(oracle.quantize(oracle.Q8_0, synth.weights_f32(5, 64, 576))), torch.empty((0, 576), device="cuda"), y)
    torch.cuda.synchronize()


def test_run_rejects_m_above_plan_maximum():
    with qmm.Plan(qmm.Q8_0, 64, 576, 4, 0) as p:
        wq = dev(oracle.quantize(oracle.Q8_0, synth.weights_f32(6, 64, 576)))
        with pytest.raises(qmm.QmmError) as e:
            p.run(wq, dev(synth.acts_f32(7, 5, 576)))
        assert e.value.status == qmm.EINVAL
