"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one plan per shape and mode, weights quantized on the GPU by
the library).  The oracle computes sampled output columns (every activation
row) from its own quantization of the same float weight rows; those rows'
bytes are first checked equal to the GPU's, so the oracle's inputs never come
from the GPU path.

Workloads (seeded synthetic stand-ins for SmolLM2-135M's trained weights):
q_proj 576x576 decode, lm_head 49152x576 decode, ffn_down 576x1536 (Q4_K)
decode and 37-token prefill, the 30-layer 307-token prefill with lm_head, and
the 8-layer 14336x4096 scale-up at M = 1, 8 and 512.
"""
import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import block_quantized_matmul_gguf_amd as qmm  # noqa: E402

TOL = 1e-5
MODES = [(qmm.MODE_F32ACT, "a"), (qmm.MODE_QACT, "b")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    qmm.lib()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check(fmt, mode, w_f32, w_gpu_blocks, x, y_gpu, cols, what):
    """Oracle on columns `cols`: bytes equal, then outputs within tolerance."""
    k = w_f32.shape[1]
    wq = oracle.quantize(fmt, w_f32[cols])
    got_bytes = host(w_gpu_blocks[torch.as_tensor(cols, device=w_gpu_blocks.device)])
    assert np.array_equal(got_bytes, wq), f"{what}: GPU weight quantization differs from the oracle"
    fn = oracle.matmul_a if mode == qmm.MODE_F32ACT else oracle.matmul_b
    yr, a = fn(fmt, wq, len(cols), k, x)
    y = y_gpu[:, cols].astype(np.float64)
    err = np.abs(y - yr)
    bad = (err > TOL * a) | ((a == 0) & (y != 0)) | ~np.isfinite(y)
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs outside tolerance, worst "
                           f"{float((err / np.maximum(a, 1e-300)).max()):.3e}")


def sample_cols(n, count, seed, stripe=None):
    """`count` random columns, the first and last (ragged tile tails) and, with
    `stripe`, one random column in every `stripe`-wide run of columns, so that
    every output tile of that width (and its place in the XCD remapping of the
    workgroups) is compared."""
    g = np.random.default_rng(seed)
    cols = set(g.choice(n, size=min(count, n), replace=False).tolist())
    cols.update({0, n - 1})
    if stripe:
        for c0 in range(0, n, stripe):
            cols.add(int(c0 + g.integers(0, min(stripe, n - c0))))
    return np.array(sorted(cols))


# The prefill kernels' output tiles are 64 to 224 columns wide (every width a
# multiple of 32, the narrowest 64); the decode kernels' tiles are 16 rows of
# the weights.  Sampling one column per 32 covers every prefill tile, one per
# 16 every decode tile.
PREFILL_STRIPE, DECODE_STRIPE = 32, 16


def run_problem(fmt, mode, prob, m_max=None, cols=48, seed=0):
    w = prob.weights()
    x = prob.acts()
    wg = qmm.quantize_weights(fmt, torch.from_numpy(w).cuda())
    with qmm.Plan(fmt, prob.n, prob.k, m_max or prob.m, mode) as p:
        y = host(p.run(wg, torch.from_numpy(x).cuda()))
    check(fmt, mode, w, wg, x, y, sample_cols(prob.n, cols, seed), prob.name)


@pytest.mark.parametrize("mode,mname", MODES)
def test_q_proj_decode(mode, mname):
    run_problem(qmm.Q8_0, mode, synth.c1_q_proj(), cols=576)


@pytest.mark.parametrize("mode,mname", MODES)
def test_lm_head_decode(mode, mname):
    run_problem(qmm.Q8_0, mode, synth.c2_lm_head(), cols=4096, seed=2)


@pytest.mark.parametrize("mode,mname", MODES)
@pytest.mark.parametrize("m", [1, 37])
def test_ffn_down_q4_k(mode, mname, m):
    run_problem(qmm.Q4_K, mode, synth.c3_ffn_down(m), cols=576, seed=3)


@pytest.mark.parametrize("mode,mname", MODES)
def test_smollm2_prefill_all_layers(mode, mname):
    """All 210 layer projections (Q8_0) plus the tied lm_head at M = 307, with
    ffn_down also as Q4_K; every GEMM checked on sampled columns."""
    probs = synth.c4_prefill()
    plans = {}
    try:
        for i, prob in enumerate(probs):
            fmts = [qmm.Q8_0] + ([qmm.Q4_K] if prob.name.split()[0].endswith("down") else [])
            w = prob.weights()
            x = prob.acts()
            xg = torch.from_numpy(x).cuda()
            for fmt in fmts:
                key = (fmt, prob.n, prob.k)
                if key not in plans:
                    plans[key] = qmm.Plan(fmt, prob.n, prob.k, synth.PREFILL_TOKENS, mode)
                wg = qmm.quantize_weights(fmt, torch.from_numpy(w).cuda())
                y = host(plans[key].run(wg, xg))
                check(fmt, mode, w, wg, x, y, sample_cols(prob.n, 8, 40 + i, PREFILL_STRIPE),
                      f"{prob.name} fmt={fmt}")
    finally:
        for p in plans.values():
            p.close()


@pytest.fixture(scope="module")
def scaleup():
    """Layers 0 and 7 of the 8-layer 14336x4096 scale-up, both formats on the GPU."""
    layers = {}
    for layer in (0, 7):
        prob = synth.c5_layer(layer, 512)
        w = prob.weights()
        wt = torch.from_numpy(w).cuda()
        layers[layer] = (w, {fmt: qmm.quantize_weights(fmt, wt) for fmt in (qmm.Q8_0, qmm.Q4_K)})
        del wt
    x = synth.c5_layer(0, 512).acts()
    return layers, x


@pytest.mark.parametrize("mode,mname", MODES)
@pytest.mark.parametrize("fmt", [qmm.Q8_0, qmm.Q4_K], ids=["Q8_0", "Q4_K"])
def test_scaleup_all_batch_sizes(scaleup, fmt, mode, mname):
    layers, x = scaleup
    n, k = synth.C5_N, synth.C5_K
    with qmm.Plan(fmt, n, k, synth.C5_MMAX, mode) as p:
        for layer, (w, wg) in layers.items():
            for m in (1, 8, 512):
                xm = np.ascontiguousarray(x[:m])
                y = host(p.run(wg[fmt], torch.from_numpy(xm).cuda()))
                stripe = PREFILL_STRIPE if m == 512 else DECODE_STRIPE
                check(fmt, mode, w, wg[fmt], xm, y, sample_cols(n, 24, layer * 10 + m, stripe),
                      f"scale-up L{layer} fmt={fmt} M={m}")
