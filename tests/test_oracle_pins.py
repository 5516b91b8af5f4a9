"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or the mathematics
fix: byte counts the pages print, hand-built blocks with hand-worked values,
IEEE binary16 as NumPy implements it, closed-form error bounds, special cases
that reduce to an exact integer matmul, and brute force on tiny inputs.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import Q4_0, Q4_K, Q5_0, Q6_K, Q8_0, Q8_K

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def le16(v):
    return [v & 0xFF, (v >> 8) & 0xFF]


def f16val(bits):
    return float(np.array([bits], np.uint16).view(np.float16)[0])


# --------------------------------------------------------------- binary16 --

def test_f16_decode_matches_numpy_on_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_bits_to_f64(int(b)) for b in bits])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_f16_encode_is_round_to_nearest_even():
    g = np.random.default_rng(3)
    vals = [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e30, 2.0 ** -25, 3 * 2.0 ** -25,
            2.0 ** -24, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 / 127, 8.0 / 63]
    vals += list((g.standard_normal(4000) * np.exp2(g.uniform(-30, 17, 4000))).astype(np.float32))
    # every midpoint between adjacent positive finite f16 values is a tie
    p = np.arange(0, 0x7BFF, 7, dtype=np.uint16)
    lo = p.view(np.float16).astype(np.float64)
    hi = (p + 1).view(np.float16).astype(np.float64)
    vals += list(((lo + hi) / 2).astype(np.float32))
    vals = np.array(vals, dtype=np.float32)
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_bits(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------ block byte sizes --

def test_block_sizes_reproduce_the_pages_byte_counts():
    g = gold("page_byte_counts.json")
    for t in g["tensor_type_totals"]:
        fmt = {"Q8_0": Q8_0, "Q4_K": Q4_K, "Q5_0": Q5_0}[t["fmt"]]
        q = oracle.quantize(fmt, synth.weights_f32(7, t["n"], t["k"]))
        assert q.nbytes * t["tensors"] == t["bytes"], t["what"]
    f = g["whole_files"]
    layer = [(n, k) for _, n, k in synth.SMOLLM2_LAYER]
    vocab, hidden = synth.SMOLLM2_VOCAB, synth.SMOLLM2_HIDDEN
    norms = f["norm_weights_f32"] * hidden * 4
    payload_f32 = 4 * (synth.SMOLLM2_LAYERS * sum(n * k for n, k in layer) + vocab * hidden) + norms
    payload_q8 = (synth.SMOLLM2_LAYERS * sum(n * oracle.row_bytes(Q8_0, k) for n, k in layer)
                  + vocab * oracle.row_bytes(Q8_0, hidden) + norms)
    overhead = f["f32_bytes"] - payload_f32
    assert 0 < overhead < 1 << 20
    assert f["q8_0_bytes"] - payload_q8 == overhead
    # the Q4_0 file: every matrix Q4_0; the Q4K file: K-quants only where K is a
    # multiple of 256 (ffn_down, K = 1536), Q5_0 for the rest
    payload_q4_0 = (synth.SMOLLM2_LAYERS * sum(n * oracle.row_bytes(Q4_0, k) for n, k in layer)
                    + vocab * oracle.row_bytes(Q4_0, hidden) + norms)
    assert f["q4_0_bytes"] - payload_q4_0 == overhead
    fallback = [(n, oracle.row_bytes(Q4_K if k % 256 == 0 else Q5_0, k)) for n, k in layer]
    assert sum(k % 256 == 0 for _, _, k in synth.SMOLLM2_LAYER) == 1
    payload_q4k = (synth.SMOLLM2_LAYERS * sum(n * rb for n, rb in fallback)
                   + vocab * oracle.row_bytes(Q5_0, hidden) + norms)
    assert f["q4k_q5_0_bytes"] - payload_q4k == overhead


# ------------------------------------------------------------------ Q8_0 --

def test_q8_0_handbuilt_blocks_decode():
    for case in gold("q8_0_handbuilt.json")["decode"]:
        blk = np.array(le16(case["d_bits"]) + list(np.array(case["q"], np.int8).view(np.uint8)), np.uint8)
        w = oracle.dequantize(Q8_0, blk, 32)[0]
        assert np.array_equal(w, np.array(case["w"])), case["why"]


def test_q8_0_handbuilt_quantization():
    for case in gold("q8_0_handbuilt.json")["quantize"]:
        xh = case["x_head"]
        x = np.zeros((1, 32), np.float32)
        x[0, :len(xh)] = xh
        for variant, key in ((0, "q_head"), (2, "q_head_ties_even")):
            blk = oracle.quantize(Q8_0, x, variant)[0]
            assert int(blk[0]) | (int(blk[1]) << 8) == case["d_bits"], case["why"]
            q = blk[2:].view(np.int8)
            assert list(q[:len(xh)]) == case[key], case["why"]
            assert not q[len(xh):].any()


def test_q8_0_scale_is_block_absmax_over_127():
    # "the scale is max|x| / 127" (page 自己量化, section 和下载的 Q8_0 逐字节比)
    x = synth.weights_f32(21, 64, 1024)
    blk = oracle.quantize(Q8_0, x).reshape(64, 32, 34)
    amax = np.abs(x).reshape(64, 32, 32).max(-1)
    want = (amax / np.float32(127)).astype(np.float16).view(np.uint16)
    got = blk[..., 0].astype(np.uint16) | (blk[..., 1].astype(np.uint16) << 8)
    assert np.array_equal(got, want)
    q = blk[..., 2:].view(np.int8)
    # the largest element of every nonzero block lands on +-127
    assert np.all(np.abs(q).max(-1) == 127)


def test_q8_0_round_trip_bounds():
    x = synth.weights_f32(22, 256, 1024)
    blk = oracle.quantize(Q8_0, x).reshape(256, 32, 34)
    q = blk[..., 2:].view(np.int8).astype(np.float64)
    xb = x.reshape(256, 32, 32).astype(np.float64)
    d32 = (np.abs(x).reshape(256, 32, 32).max(-1) / np.float32(127)).astype(np.float64)[..., None]
    d16 = oracle.dequantize(Q8_0, blk, 1024).reshape(256, 32, 32) / np.where(q == 0, 1, q)
    d16 = np.where(q == 0, np.nan, d16)
    d16 = np.nanmax(np.abs(d16), -1, keepdims=True) * np.sign(d32)
    assert np.all(np.abs(xb - d32 * q) <= (0.5 + 1e-4) * d32)
    assert np.all(np.abs(xb - d16 * q) <= (0.5 + 1e-4) * d32 + np.abs(q) * np.abs(d32 - d16))


def test_q8_0_random_bytes_decode_like_a_direct_reading():
    g = np.random.default_rng(23)
    blk = g.integers(0, 256, size=(200, 34), dtype=np.uint8)
    blk[:, 1] &= 0x7B  # keep the f16 exponent below 31 (finite)
    d = blk[:, 0:2].copy().view(np.float16).astype(np.float64)
    want = d * blk[:, 2:].view(np.int8).astype(np.float64)
    assert np.array_equal(oracle.dequantize(Q8_0, blk, 32 * 200).reshape(200, 32), want)


# ------------------------------------------------------------------ Q4_K --

def py_q4k_decode(blk):
    """Direct reading of one 144-byte super-block (independent of the oracle)."""
    d = f16val(int(blk[0]) | int(blk[1]) << 8)
    dmin = f16val(int(blk[2]) | int(blk[3]) << 8)
    s = [int(v) for v in blk[4:16]]
    qs = [int(v) for v in blk[16:144]]
    out, sc_m = [], []
    for j in range(8):
        if j < 4:
            sc, m = s[j] & 63, s[j + 4] & 63
        else:
            sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4)
            m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4)
        sc_m.append((sc, m))
    qv = []
    for e in range(256):
        c, l = divmod(e, 64)
        byte = qs[32 * c + l % 32]
        q = byte & 15 if l < 32 else byte >> 4
        sc, m = sc_m[e // 32]
        qv.append(q)
        out.append(d * sc * q - dmin * m)
    return np.array(out), qv, sc_m, d, dmin


def handbuilt_q4k():
    g = gold("q4_k_handbuilt.json")
    i = np.arange(128)
    blk = np.array(le16(g["d_bits"]) + le16(g["dmin_bits"]) + g["scales12"]
                   + list((i % 16) | ((15 - i % 16) << 4)), np.uint8)
    return g, blk


def test_q4_k_handbuilt_block_decodes_to_hand_worked_values():
    g, blk = handbuilt_q4k()
    w = oracle.dequantize(Q4_K, blk, 256)[0]
    for el in g["elements"]:
        assert w[el["e"]] == el["w"], el
    _, qv, sc_m, _, _ = py_q4k_decode(blk)
    assert [sc for sc, _ in sc_m] == g["sc"]
    assert [m for _, m in sc_m] == g["m"]
    for el in g["elements"]:
        assert qv[el["e"]] == el["q"]


def test_q4_k_handbuilt_quantization():
    g = gold("q4_k_handbuilt.json")
    e = np.arange(256)
    i = np.arange(128)
    for case in g["quantize"]:
        x = (e % 16 - (8 if "- 8" in case["x_rule"] else 0)).astype(np.float32)[None, :]
        blk = oracle.quantize(Q4_K, x)[0]
        assert list(blk[0:2]) == le16(case["d_bits"]), case["why"]
        assert list(blk[2:4]) == le16(case["dmin_bits"]), case["why"]
        assert list(blk[4:16]) == case["scales12"], case["why"]
        assert np.array_equal(blk[16:], (17 * (i % 16)).astype(np.uint8)), case["why"]


def test_q4_k_random_bytes_decode_like_a_direct_reading():
    g = np.random.default_rng(31)
    blk = g.integers(0, 256, size=(6, 144), dtype=np.uint8)
    blk[:, 1] &= 0x7B
    blk[:, 3] &= 0x7B
    got = oracle.dequantize(Q4_K, blk, 256 * 6).reshape(6, 256)
    for r in range(6):
        assert np.array_equal(got[r], py_q4k_decode(blk[r])[0])


def test_q4_k_quantizer_round_trip_bound():
    w = synth.weights_f32(32, 24, 1536)
    blk = oracle.quantize(Q4_K, w).reshape(24, 6, 144)
    worst = 0.0
    for r in range(24):
        for b in range(6):
            deq, qv, sc_m, d, dmin = py_q4k_decode(blk[r, b])
            x = w[r, 256 * b:256 * (b + 1)].astype(np.float64)
            qv = np.array(qv)
            d_eff = np.array([d * sc_m[e // 32][0] for e in range(256)])
            inside = (qv > 0) & (qv < 15)
            err = np.abs(x - deq)
            assert np.all(err[inside] <= 0.5 * d_eff[inside] * (1 + 1e-5))
            # clamped values sit on the side the clamp pushed them from
            assert np.all(x[qv == 0] <= deq[qv == 0] + 0.5 * d_eff[qv == 0] * (1 + 1e-5))
            assert np.all(x[qv == 15] >= deq[qv == 15] - 0.5 * d_eff[qv == 15] * (1 + 1e-5))
            worst = max(worst, float(np.sqrt(np.mean(err ** 2))))
    assert worst < 0.25 * synth.W_SIGMA


# ------------------------------------------------ Q4_K with the search --
# The search tries code assignments for 22 scales around the min/max rule's
# and keeps the least-squares line of smallest squared error (the min/max
# rule's own fit competing first), then packs like the min/max rule.

def test_q4_k_search_hand_worked_block():
    # Every sub-block: 30 zeros, 0.5 and 1.0.  The min/max rule spans [0, 1]
    # with 15 steps (scale 1/15): 0.5 falls at 7.5 steps, so one of the two
    # nonzero values is off by half a step.  The codes 7 and 14 lie on the
    # line x = q/14 exactly (the candidate c = 14/r, k = 0): the search takes
    # it (scale 1/14, min about 0).  Packing: d = f16((1/14)/63), whose bits
    # are 0x14A5 (1/882 = 2^-10 * 1.1610..., mantissa 165); dmin = 0 (the min
    # is far below the f16 range); sc_j = m_j = 63; requantized against
    # d_eff = f16(d) * 63 = 0.0714369: 0.5 -> 7, 1.0 -> 14.  The min/max rule
    # instead stores d = f16((1/15)/63) = 0x1456 and codes 7 and 15.
    x = np.zeros((1, 256), np.float32)
    for j in range(8):
        x[0, 32 * j + 7], x[0, 32 * j + 20] = 0.5, 1.0
    for fn, dbits, codes in ((oracle.quantize_q4_k_search, 0x14A5, (7, 14)),
                             (lambda v: oracle.quantize(Q4_K, v), 0x1456, (7, 15))):
        blk = fn(x)[0]
        assert (int(blk[0]) | int(blk[1]) << 8) == dbits and blk[2] == 0 and blk[3] == 0
        deq, qv, sc_m, d, dmin = py_q4k_decode(blk)
        assert [sm[0] for sm in sc_m] == [63] * 8
        for j in range(8):
            assert (qv[32 * j + 7], qv[32 * j + 20]) == codes
            assert not any(qv[32 * j + l] for l in range(32) if l not in (7, 20))


def test_q4_k_search_round_trip_bound_and_gain():
    # the packing stage is the min/max rule's, so its bound holds; the search
    # lowers the error on N(0, 0.02) weights
    w = synth.weights_f32(33, 64, 1536)
    blk = oracle.quantize_q4_k_search(w).reshape(64, 6, 144)
    sq_search = 0.0
    for r in range(64):
        for b in range(6):
            deq, qv, sc_m, d, dmin = py_q4k_decode(blk[r, b])
            x = w[r, 256 * b:256 * (b + 1)].astype(np.float64)
            qv = np.array(qv)
            d_eff = np.array([d * sc_m[e // 32][0] for e in range(256)])
            inside = (qv > 0) & (qv < 15)
            assert np.all(np.abs(x - deq)[inside] <= 0.5 * d_eff[inside] * (1 + 1e-5))
            sq_search += float(((x - deq) ** 2).sum())
    plain = oracle.dequantize(Q4_K, oracle.quantize(Q4_K, w), 1536).astype(np.float64)
    sq_plain = float(((plain - w) ** 2).sum())
    assert sq_search < 0.9 * sq_plain


# ------------------------------------------------------------------- Q8K --

def test_q8_k_handbuilt_quantization():
    maxes = [2.0, -3.0, 0.0]
    for case, mx in zip(gold("q8_k_handbuilt.json")["cases"], maxes):
        x = np.zeros((1, 256), np.float32)
        for k, v in case["x_sparse"].items():
            x[0, int(k)] = v
        blk = oracle.quantize(Q8_K, x)[0]
        d = blk[:4].copy().view(np.float32)[0]
        q = blk[4:260].view(np.int8)
        bs = blk[260:292].copy().view(np.int16)
        want = np.zeros(256, np.int8)
        for k, v in case["q_sparse"].items():
            want[int(k)] = v
        assert np.array_equal(q, want), case["why"]
        assert list(bs[:3]) == case["bsums_head"], case["why"]
        assert np.array_equal(bs, q.astype(np.int32).reshape(16, 16).sum(1))
        if mx == 0.0:
            assert d == 0.0
        else:
            iscale = np.float32(-127.0) / np.float32(mx)
            assert d == np.float32(1.0) / iscale
            assert np.sign(d) == -np.sign(mx)


def test_q8_k_round_trip_bound_and_range():
    x = synth.acts_f32(41, 16, 2048)
    blk = oracle.quantize(Q8_K, x).reshape(16, 8, 292)
    d = blk[..., :4].copy().view(np.float32).astype(np.float64)
    q = blk[..., 4:260].view(np.int8).astype(np.float64)
    xb = x.reshape(16, 8, 256).astype(np.float64)
    assert np.all(np.abs(xb - d * q) <= (0.5 + 1e-4) * np.abs(d))
    assert q.min() >= -127 and q.max() <= 127
    assert np.all(np.abs(q).max(-1) == 127)


# ------------------------------------------------ the flagged variants --
# The oracle carries the readings the pages leave open behind variant flags
# (Q8_0: x / d in place of x * (1/d), ties to even; Q8K: -128/max in place of
# -127/max, ties to even).  Only the default reading runs anywhere else; the
# variants are pinned here so that a flag means what it says.

def test_q8_0_variants_on_a_hand_worked_block():
    # amax 127 makes d = 1 and 1/d = 1 exactly: x * id = x / d = x
    x = np.zeros((1, 32), np.float32)
    x[0, :6] = [127.0, 2.5, -2.5, 0.5, 1.5, -0.5]
    away = [127, 3, -3, 1, 2, -1]   # half away from zero (the default)
    even = [127, 2, -2, 0, 2, 0]    # ties to even (variant bit 1)
    for variant, want in ((0, away), (1, away), (2, even), (3, even)):
        q = oracle.quantize(Q8_0, x, variant)[0, 2:].view(np.int8)
        assert list(q[:6]) == want, variant
        assert not q[6:].any()


def test_q8_0_division_variant_differs_rarely_and_where_predicted():
    # The survey measured that x / d and x * (1/d) disagree on a few values
    # per million.  Predict every disagreement with NumPy's IEEE f32 division
    # and multiplication (one correctly rounded operation each), then require
    # the oracle's two variants to land on the predicted sides of it.
    w = synth.weights_f32(5000, 2048, 4096)            # 8.4M values of the scale-up's layer 0
    blocks = w.reshape(-1, 32)
    d = (np.abs(blocks).max(1) / np.float32(127.0)).astype(np.float32)[:, None]
    id_ = np.where(d != 0, np.float32(1.0) / np.where(d != 0, d, 1), 0).astype(np.float32)
    t_mul = (blocks * id_).astype(np.float64)
    t_div = (blocks / np.where(d != 0, d, 1)).astype(np.float64)

    def half_away(t):
        return np.sign(t) * np.floor(np.abs(t) + 0.5)

    q_mul, q_div = half_away(t_mul), half_away(t_div)
    differ = q_mul != q_div
    count = int(differ.sum())
    print(f"x/d and x*(1/d) differ on {count} of {differ.size} values")
    assert 0 < count < 1e-5 * differ.size
    rows = np.unique(np.argwhere(differ)[:, 0])
    sel = blocks[rows]
    got0 = oracle.quantize(Q8_0, sel, 0).reshape(len(rows), 34)[:, 2:].view(np.int8)
    got1 = oracle.quantize(Q8_0, sel, 1).reshape(len(rows), 34)[:, 2:].view(np.int8)
    assert np.array_equal(got0, q_mul[rows].astype(np.int8))
    assert np.array_equal(got1, q_div[rows].astype(np.int8))
    assert not np.array_equal(got0, got1)


def test_q8_k_variants_on_a_hand_worked_block():
    # max 2.0: iscale = -127/2 = -63.5 (default) or -128/2 = -64 (bit 0), both exact
    x = np.zeros((1, 256), np.float32)
    x[0, :5] = [2.0, 1.0, -0.5, 0.25, 0.0078125]
    cases = {
        0: ([-127, -64, 32, -16, 0], np.float32(1.0) / np.float32(-63.5)),  # -63.5, 31.75, -15.875, -0.496
        1: ([-128, -64, 32, -16, -1], np.float32(-0.015625)),               # ..., -0.5 -> -1 (away)
        2: ([-127, -64, 32, -16, 0], np.float32(1.0) / np.float32(-63.5)),  # -63.5 -> -64 either way
        3: ([-128, -64, 32, -16, 0], np.float32(-0.015625)),                # -0.5 -> 0 (even)
    }
    for variant, (want, dwant) in cases.items():
        blk = oracle.quantize(Q8_K, x, variant)[0]
        q = blk[4:260].view(np.int8)
        assert list(q[:5]) == want, variant
        assert not q[5:].any()
        assert blk[:4].copy().view(np.float32)[0] == dwant, variant
        assert blk[260:262].copy().view(np.int16)[0] == sum(want), variant


# ------------------------------------------------- integer special cases --

def test_integer_case_q8_0_both_modes_exact():
    # d = 1 weights and integer activations whose every 32-block reaches +-127:
    # activation quantization is lossless, so both modes equal x_int . q_int^T.
    n, k, m = 40, 256, 3
    g = np.random.default_rng(11)
    qw = g.integers(-127, 128, size=(n, k))
    blk = np.zeros((n, k // 32, 34), np.uint8)
    blk[..., 0:2] = le16(0x3C00)
    blk[..., 2:] = qw.reshape(n, k // 32, 32).astype(np.int8).view(np.uint8)
    x = synth.integer_acts(12, m, k, 32)
    ref = x.astype(np.int64) @ qw.T
    ya, _ = oracle.matmul_a(Q8_0, blk, n, k, x)
    yb, _ = oracle.matmul_b(Q8_0, blk, n, k, x)
    assert np.array_equal(ya, ref) and np.array_equal(yb, ref)
    s = oracle.block_sums(Q8_0, blk, n, k, x)
    assert np.array_equal(s.sum(-1), ref)


@pytest.mark.parametrize("dmin", [0, 1])
def test_integer_case_q4_k_both_modes_exact(dmin):
    # d = 1, every sc_j = m_j = 1, dmin in {0, 1}: w = q - dmin.  Integer
    # activations with a +-127 in every 256-block make Q8K lossless.
    n, k, m = 24, 512, 3
    g = np.random.default_rng(13 + dmin)
    q = g.integers(0, 16, size=(n, k))
    blk = np.zeros((n, k // 256, 144), np.uint8)
    blk[..., 0:2] = le16(0x3C00)
    blk[..., 2:4] = le16(0x3C00 if dmin else 0)
    blk[..., 4:8] = 1
    blk[..., 8:12] = 1
    blk[..., 12:16] = 0x11
    for e in range(256):
        c, l = divmod(e, 64)
        byte = 16 + 32 * c + l % 32
        blk[..., byte] |= (q.reshape(n, k // 256, 256)[..., e] << (0 if l < 32 else 4)).astype(np.uint8)
    x = synth.integer_acts(14, m, k, 256)
    ref = x.astype(np.int64) @ (q - dmin).T
    ya, _ = oracle.matmul_a(Q4_K, blk, n, k, x)
    yb, _ = oracle.matmul_b(Q4_K, blk, n, k, x)
    assert np.array_equal(ya, ref) and np.array_equal(yb, ref)


# -------------------------------------------------------- mode relations --

@pytest.mark.parametrize("fmt,k", [(Q8_0, 576), (Q4_K, 1536), (Q4_0, 576), (Q5_0, 576), (Q6_K, 1536)])
def test_mode_a_is_the_matmul_of_the_dequantized_weights(fmt, k):
    n, m = 48, 5
    w = oracle.quantize(fmt, synth.weights_f32(51, n, k))
    x = synth.acts_f32(52, m, k)
    ref = x.astype(np.float64) @ oracle.dequantize(fmt, w, k).T
    y, a = oracle.matmul_a(fmt, w, n, k, x)
    assert np.all(np.abs(y - ref) <= 1e-12 * a)
    assert np.allclose(a, np.abs(x.astype(np.float64)) @ np.abs(oracle.dequantize(fmt, w, k)).T, rtol=1e-12)


@pytest.mark.parametrize("fmt,k", [(Q8_0, 576), (Q4_K, 1536), (Q4_0, 576), (Q5_0, 576), (Q6_K, 1536)])
def test_mode_b_is_the_matmul_of_requantized_activations(fmt, k):
    # sum_b dw*dx*S_b (and the Q4_K sumi/summins combination) equals, in exact
    # arithmetic, the plain product of the dequantized weights with the
    # dequantized quantized activations.
    n, m = 48, 5
    w = oracle.quantize(fmt, synth.weights_f32(53, n, k))
    x = synth.acts_f32(54, m, k)
    afmt = oracle.ACT_FORMAT[fmt]
    xt = oracle.dequantize(afmt, oracle.quantize(afmt, x), k)
    wd = oracle.dequantize(fmt, w, k)
    y, a = oracle.matmul_b(fmt, w, n, k, x)
    assert np.all(np.abs(y - xt @ wd.T) <= 1e-12 * a)
    assert np.allclose(a, np.abs(xt) @ np.abs(wd).T, rtol=1e-12)
    # mode (b) differs from mode (a) by at most sum_k |w_k| * |x~_k - x_k|
    ya, _ = oracle.matmul_a(fmt, w, n, k, x)
    bound = np.abs(xt - x.astype(np.float64)) @ np.abs(wd).T
    assert np.all(np.abs(y - ya) <= bound * (1 + 1e-9) + 1e-12)
    assert np.abs(y - ya).max() > 1e3 * np.abs(ya - x.astype(np.float64) @ wd.T).max()


def test_q4_k_block_sums_by_brute_force():
    n, k, m = 3, 512, 2
    w = oracle.quantize(Q4_K, synth.weights_f32(61, n, k))
    x = synth.acts_f32(62, m, k)
    s = oracle.block_sums(Q4_K, w, n, k, x)
    xq = oracle.quantize(Q8_K, x).reshape(m, k // 256, 292)
    wb = w.reshape(n, k // 256, 144)
    for mi in range(m):
        for ni in range(n):
            for i in range(k // 256):
                _, qv, sc_m, _, _ = py_q4k_decode(wb[ni, i])
                q8 = xq[mi, i, 4:260].view(np.int8).astype(int)
                bs = xq[mi, i, 260:].copy().view(np.int16).astype(int)
                S = [sum(qv[32 * j + l] * q8[32 * j + l] for l in range(32)) for j in range(8)]
                sumi = sum(sc_m[j][0] * S[j] for j in range(8))
                summins = sum(sc_m[j][1] * (bs[2 * j] + bs[2 * j + 1]) for j in range(8))
                assert list(s[mi, ni, 10 * i:10 * i + 10]) == S + [sumi, summins]


def test_activation_quantization_is_row_local():
    # candle quantizes each activation row on its own, per 32 (Q8_0) or per
    # 256 (Q8K) values (page 自己量化, section 动脑筋答案): permuting or
    # sub-setting rows permutes or sub-sets the quantized blocks bit-exactly.
    x = synth.acts_f32(71, 9, 512)
    perm = np.random.default_rng(72).permutation(9)
    for fmt in (Q8_0, Q8_K):
        full = oracle.quantize(fmt, x)
        assert np.array_equal(oracle.quantize(fmt, x[perm]), full[perm])
        for r in range(9):
            assert np.array_equal(oracle.quantize(fmt, x[r:r + 1])[0], full[r])
    w = oracle.quantize(Q8_0, synth.weights_f32(73, 16, 512))
    s = oracle.block_sums(Q8_0, w, 16, 512, x)
    assert np.array_equal(oracle.block_sums(Q8_0, w, 16, 512, x[perm][:4]), s[perm][:4])


def test_shape_check_rejects_k_not_divisible_by_block():
    # K-quants need the last dim divisible by 256 (page 自己量化, section 3. 量化)
    with pytest.raises(ValueError):
        oracle.quantize(Q4_K, np.zeros((2, 576), np.float32))
    with pytest.raises(ValueError):
        oracle.quantize(Q8_0, np.zeros((2, 40), np.float32))


# ---------------------------------------------------------- Q4_0 and Q5_0 --

def handbuilt_q4_q5():
    g = gold("q4_0_q5_0_handbuilt.json")
    qs = [i | ((15 - i) << 4) for i in range(16)]
    b4 = np.array(le16(g["q4_0"]["d_bits"]) + qs, np.uint8)
    b5 = np.array(le16(g["q5_0"]["d_bits"]) + g["q5_0"]["qh_bytes"] + qs, np.uint8)
    return g, b4, b5


def py_q4_q5_decode(blk, five):
    """A direct reading of one Q4_0 / Q5_0 block: (values, codes)."""
    d = f16val(int(blk[0]) | (int(blk[1]) << 8))
    qs = blk[6:22] if five else blk[2:18]
    qh = int.from_bytes(bytes(blk[2:6]), "little") if five else 0
    codes = []
    for j in range(32):
        lo = int(qs[j]) & 15 if j < 16 else int(qs[j - 16]) >> 4
        codes.append(lo | (((qh >> j) & 1) << 4))
    off = 16 if five else 8
    return np.array([d * (c - off) for c in codes]), codes


def test_q4_0_q5_0_handbuilt_blocks_decode_to_hand_worked_values():
    g, b4, b5 = handbuilt_q4_q5()
    for fmt, blk, key, five in ((Q4_0, b4, "q4_0", False), (Q5_0, b5, "q5_0", True)):
        w = oracle.dequantize(fmt, blk, 32)[0]
        _, codes = py_q4_q5_decode(blk, five)
        for el in g[key]["elements"]:
            assert w[el["e"]] == el["w"], (key, el)
            assert codes[el["e"]] == el["q"], (key, el)


def test_q4_0_q5_0_handbuilt_quantization():
    j = np.arange(32)
    for case in gold("q4_0_q5_0_handbuilt.json")["quantize"]:
        x = {"x[j] = j - 16": j - 16, "x[j] = 16 - j": 16 - j, "x[j] = 0": 0 * j}[case["x_rule"]]
        five = case["fmt"] == "Q5_0"
        blk = oracle.quantize(Q5_0 if five else Q4_0, x.astype(np.float32)[None, :])[0]
        assert list(blk[0:2]) == le16(case["d_bits"]), case["why"]
        _, codes = py_q4_q5_decode(blk, five)
        assert codes == case["q"], case["why"]
        if five:
            assert list(blk[2:6]) == case["qh_bytes"], case["why"]


def test_q4_0_q5_0_signed_maximum_ties_take_the_first():
    # x = [4, -4, 0, ...]: both ends have magnitude 4 and the first one met
    # (+4) is the signed maximum, so d = 4 / -offset is negative.  Worked by
    # hand from the scale and rounding rule (truncate v/d + offset + 1/2,
    # capped at the top code):
    #   Q4_0: d = -0.5 (f16 0xB800), codes 0, 15 (16.5 capped), 8 for the zeros;
    #         bytes j = c[j] | c[j + 16] << 4: 0x80, 0x8F, then 0x88.
    #   Q5_0: d = -0.25 (f16 0xB400), codes 0, 31 (32.5 capped), 16 for the zeros;
    #         fifth bits: all but element 0; low nibbles 0, 15, 0, ...
    # Taking the last of the tied magnitudes (-4) would flip d's sign and
    # every code.
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0], x[0, 1] = 4.0, -4.0
    q4 = oracle.quantize(Q4_0, x)[0]
    assert list(q4) == [0x00, 0xB8, 0x80, 0x8F] + [0x88] * 14
    q5 = oracle.quantize(Q5_0, x)[0]
    assert list(q5) == [0x00, 0xB4, 0xFE, 0xFF, 0xFF, 0xFF, 0x00, 0x0F] + [0x00] * 14


@pytest.mark.parametrize("fmt", [Q4_0, Q5_0])
def test_q4_0_q5_0_random_bytes_decode_like_a_direct_reading(fmt):
    five = fmt == Q5_0
    nbytes = 22 if five else 18
    g = np.random.default_rng(33 + fmt)
    blk = g.integers(0, 256, size=(8, nbytes), dtype=np.uint8)
    blk[:, 1] &= 0x7B  # finite f16 d
    got = oracle.dequantize(fmt, blk, 32 * 8).reshape(8, 32)
    for r in range(8):
        assert np.array_equal(got[r], py_q4_q5_decode(blk[r], five)[0])


@pytest.mark.parametrize("fmt", [Q4_0, Q5_0])
def test_q4_0_q5_0_quantizer_scale_rule_and_round_trip(fmt):
    # d = (signed absmax) / -offset stored as f16; the absmax element takes
    # code 0; unclamped values round to within half a step of the stored d
    five = fmt == Q5_0
    off, qmax = (16, 31) if five else (8, 15)
    w = synth.weights_f32(81 + fmt, 16, 576)
    blk = oracle.quantize(fmt, w).reshape(16, 18, 22 if five else 18)
    for r in range(16):
        for b in range(18):
            x = w[r, 32 * b:32 * b + 32]
            mx = x[np.argmax(np.abs(x))]
            d_bits = int(blk[r, b, 0]) | (int(blk[r, b, 1]) << 8)
            assert d_bits == int(np.array([np.float32(mx) / np.float32(-off)], np.float32)
                                 .astype(np.float16).view(np.uint16)[0])
            deq, codes = py_q4_q5_decode(blk[r, b], five)
            codes = np.array(codes)
            assert codes[np.argmax(np.abs(x))] == 0
            # codes are rounded against the f32 d and decoded with the f16 d
            d32 = float(np.float32(mx) / np.float32(-off))
            drift = off * abs(d32 - f16val(d_bits))
            inside = codes < qmax
            err = np.abs(x.astype(np.float64) - deq)
            assert np.all(err[inside] <= 0.5 * abs(d32) * (1 + 1e-6) + drift)
            # the one-sided range: only values near +-|max| on the far side clamp
            assert np.all(err <= abs(d32) * (1 + 1e-6) + drift)


# ------------------------------------------------------------------ Q6_K --

def handbuilt_q6k():
    g = gold("q6_k_handbuilt.json")
    blk = np.zeros(210, np.uint8)
    blk[:128] = [(37 * i + 11) % 256 for i in range(128)]
    blk[128:192] = [(53 * i + 7) % 256 for i in range(64)]
    blk[192:208] = np.array(g["scales"], np.int8).view(np.uint8)
    blk[208:210] = le16(g["d_bits"])
    return g, blk


def py_q6k_decode(blk):
    """A direct reading of one Q6_K super-block: (values, codes, scales, d)."""
    d = f16val(int(blk[208]) | (int(blk[209]) << 8))
    sc = blk[192:208].view(np.int8).astype(int)
    codes = []
    for e in range(256):
        n, el = divmod(e, 128)
        g, l = divmod(el, 32)
        lo_byte = int(blk[64 * n + 32 * (g & 1) + l])
        lo = (lo_byte >> 4) if g >= 2 else (lo_byte & 15)
        hi = (int(blk[128 + 32 * n + l]) >> (2 * g)) & 3
        codes.append(lo | (hi << 4))
    vals = np.array([d * sc[e // 16] * (codes[e] - 32) for e in range(256)])
    return vals, codes, sc, d


def test_q6_k_handbuilt_block_decodes_to_hand_worked_values():
    g, blk = handbuilt_q6k()
    w = oracle.dequantize(Q6_K, blk, 256)[0]
    _, codes, _, _ = py_q6k_decode(blk)
    for el in g["elements"]:
        assert w[el["e"]] == el["w"], el
        assert codes[el["e"]] == el["q"], el


def test_q6_k_handbuilt_quantization():
    case = gold("q6_k_handbuilt.json")["quantize"]
    e = np.arange(256)
    x = (e % 16 - 8).astype(np.float32)[None, :]
    blk = oracle.quantize(Q6_K, x)[0]
    assert list(blk[208:210]) == le16(case["d_bits"]), case["why"]
    assert list(blk[192:208].view(np.int8)) == case["scales"], case["why"]
    vals, codes, _, _ = py_q6k_decode(blk)
    assert codes == list(4 * (e % 16)), case["why"]
    assert np.array_equal(vals, x[0].astype(np.float64)), case["why"]


def test_q6_k_random_bytes_decode_like_a_direct_reading():
    g = np.random.default_rng(35)
    blk = g.integers(0, 256, size=(4, 210), dtype=np.uint8)
    blk[:, 209] &= 0x7B
    got = oracle.dequantize(Q6_K, blk, 256 * 4).reshape(4, 256)
    for r in range(4):
        assert np.array_equal(got[r], py_q6k_decode(blk[r])[0])


def test_q6_k_quantizer_round_trip_bound():
    w = synth.weights_f32(37, 12, 1536)
    blk = oracle.quantize(Q6_K, w).reshape(12, 6, 210)
    for r in range(12):
        for b in range(6):
            deq, codes, sc, d = py_q6k_decode(blk[r, b])
            x = w[r, 256 * b:256 * (b + 1)].astype(np.float64)
            step = np.abs(np.repeat(d * sc, 16))
            codes = np.array(codes)
            inside = (codes > 0) & (codes < 63)
            err = np.abs(x - deq)
            assert np.all(err[inside] <= 0.5 * step[inside] * (1 + 1e-5))
            assert np.all(sc <= 127) and np.all(sc >= -128)


# -------------------------------- integer special cases, other formats --

@pytest.mark.parametrize("fmt", [Q4_0, Q5_0])
def test_integer_case_q4_0_q5_0_both_modes_exact(fmt):
    # d = 1: w = q - offset.  Integer activations with a +-127 in every
    # 32-block make their Q8_0 quantization lossless.
    five = fmt == Q5_0
    n, k, m = 24, 256, 3
    g = np.random.default_rng(15 + fmt)
    q = g.integers(0, 32 if five else 16, size=(n, k // 32, 32))
    blk = np.zeros((n, k // 32, 22 if five else 18), np.uint8)
    blk[..., 0:2] = le16(0x3C00)
    base = 6 if five else 2
    blk[..., base:base + 16] = (q[..., :16] & 15) | ((q[..., 16:] & 15) << 4)
    if five:
        qh = ((q >> 4) << np.arange(32)).sum(-1)
        for t in range(4):
            blk[..., 2 + t] = (qh >> (8 * t)) & 255
    x = synth.integer_acts(16 + fmt, m, k, 32)
    ref = x.astype(np.int64) @ (q.reshape(n, k) - (16 if five else 8)).T
    ya, _ = oracle.matmul_a(fmt, blk, n, k, x)
    yb, _ = oracle.matmul_b(fmt, blk, n, k, x)
    assert np.array_equal(ya, ref) and np.array_equal(yb, ref)
    assert np.array_equal(oracle.block_sums(fmt, blk, n, k, x).sum(-1), ref)


def test_integer_case_q6_k_both_modes_exact():
    # d = 1 and sc_j = 1: w = q - 32; Q8K lossless on integer activations
    # with a +-127 in every 256-block.
    n, k, m = 16, 512, 3
    g = np.random.default_rng(17)
    q = g.integers(0, 64, size=(n, k // 256, 256))
    blk = np.zeros((n, k // 256, 210), np.uint8)
    for e in range(256):
        half, el = divmod(e, 128)
        gg, l = divmod(el, 32)
        lo = (q[..., e] & 15) << (4 if gg >= 2 else 0)
        blk[..., 64 * half + 32 * (gg & 1) + l] |= lo.astype(np.uint8)
        blk[..., 128 + 32 * half + l] |= ((q[..., e] >> 4) << (2 * gg)).astype(np.uint8)
    blk[..., 192:208] = 1
    blk[..., 208:210] = le16(0x3C00)
    x = synth.integer_acts(18, m, k, 256)
    ref = x.astype(np.int64) @ (q.reshape(n, k) - 32).T
    ya, _ = oracle.matmul_a(Q6_K, blk, n, k, x)
    yb, _ = oracle.matmul_b(Q6_K, blk, n, k, x)
    assert np.array_equal(ya, ref) and np.array_equal(yb, ref)


def test_q6_k_block_sums_by_brute_force():
    n, k, m = 3, 512, 2
    w = oracle.quantize(Q6_K, synth.weights_f32(63, n, k))
    x = synth.acts_f32(64, m, k)
    s = oracle.block_sums(Q6_K, w, n, k, x)
    xq = oracle.quantize(Q8_K, x).reshape(m, k // 256, 292)
    wb = w.reshape(n, k // 256, 210)
    for mi in range(m):
        for ni in range(n):
            for i in range(k // 256):
                _, codes, sc, _ = py_q6k_decode(wb[ni, i])
                q8 = xq[mi, i, 4:260].view(np.int8).astype(int)
                S = [sum((codes[16 * j + l] - 32) * q8[16 * j + l] for l in range(16)) for j in range(16)]
                sumi = sum(int(sc[j]) * S[j] for j in range(16))
                assert list(s[mi, ni, 17 * i:17 * i + 17]) == S + [sumi]


def test_q4_0_q5_0_block_sums_by_brute_force():
    n, k, m = 3, 128, 2
    x = synth.acts_f32(66, m, k)
    xq = oracle.quantize(Q8_0, x).reshape(m, k // 32, 34)
    for fmt in (Q4_0, Q5_0):
        five = fmt == Q5_0
        w = oracle.quantize(fmt, synth.weights_f32(65, n, k))
        s = oracle.block_sums(fmt, w, n, k, x)
        wb = w.reshape(n, k // 32, 22 if five else 18)
        for mi in range(m):
            for ni in range(n):
                for b in range(k // 32):
                    _, codes = py_q4_q5_decode(wb[ni, b], five)
                    q8 = xq[mi, b, 2:].view(np.int8).astype(int)
                    off = 16 if five else 8
                    assert s[mi, ni, b] == sum((codes[j] - off) * q8[j] for j in range(32))
