"""The C-ABI library on the host (no GPU needed): it loads, exports every
symbol include/qmatmul.h declares, and rejects bad arguments with the right
status code before any HIP call."""
import ctypes
import os
import re

import pytest

import block_quantized_matmul_gguf_amd as qmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmatmul.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmatmul_\w+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for must in ("qmatmul_create", "qmatmul_run", "qmatmul_destroy", "qmatmul_quantize_act",
                 "qmatmul_run_block_sums", "qmatmul_status_string", "qmatmul_last_error"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = qmm.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in qmm.SIGNATURES, f"binding lacks a signature for {name}"


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define (QMM_\w+) (\d+)", text))
    assert consts["QMM_Q8_0"] == qmm.Q8_0 == 8
    assert consts["QMM_Q4_K"] == qmm.Q4_K == 12
    assert consts["QMM_Q8_K"] == qmm.Q8_K == 15
    assert consts["QMM_Q4_0"] == qmm.Q4_0 == 2
    assert consts["QMM_Q5_0"] == qmm.Q5_0 == 6
    assert consts["QMM_Q6_K"] == qmm.Q6_K == 14
    assert consts["QMM_MODE_F32ACT"] == qmm.MODE_F32ACT
    assert consts["QMM_MODE_QACT"] == qmm.MODE_QACT
    assert consts["QMM_MODE_DEQUANT"] == qmm.MODE_DEQUANT == 2
    for name, v in (("QMM_OK", qmm.OK), ("QMM_EINVAL", qmm.EINVAL), ("QMM_EBLOCK", qmm.EBLOCK),
                    ("QMM_EUNSUPPORTED", qmm.EUNSUPPORTED), ("QMM_ENOMEM", qmm.ENOMEM), ("QMM_EHIP", qmm.EHIP)):
        assert consts[name] == v


def test_row_bytes_and_block_sums_sizes():
    assert qmm.row_bytes(qmm.Q8_0, 576) == 612
    assert qmm.row_bytes(qmm.Q4_K, 1536) == 864
    assert qmm.row_bytes(qmm.Q8_K, 4096) == 16 * 292
    assert qmm.row_bytes(qmm.Q4_K, 576) == -1
    assert qmm.row_bytes(99, 576) == -1
    assert qmm.block_sums_per_row(qmm.Q8_0, 576) == 18
    assert qmm.block_sums_per_row(qmm.Q4_K, 1536) == 60
    # the pages' byte counts: Q5_0 attn_k 192 x 576 is 76,032 B per tensor
    assert 192 * qmm.row_bytes(qmm.Q5_0, 576) == 2280960 // 30
    assert qmm.row_bytes(qmm.Q4_0, 576) == 324
    assert qmm.row_bytes(qmm.Q6_K, 1536) == 1260
    assert qmm.row_bytes(qmm.Q6_K, 576) == -1
    assert qmm.block_sums_per_row(qmm.Q5_0, 576) == 18
    assert qmm.block_sums_per_row(qmm.Q6_K, 1536) == 6 * 17


@pytest.mark.parametrize("args,status", [
    ((qmm.Q4_K, 576, 576, 1, 0), qmm.EBLOCK),        # K-quants need K % 256 == 0
    ((qmm.Q8_0, 576, 40, 1, 0), qmm.EBLOCK),
    ((7, 576, 576, 1, 0), qmm.EUNSUPPORTED),          # unknown format
    ((qmm.Q8_K, 576, 512, 1, 1), qmm.EUNSUPPORTED),   # activation-only format as weights
    ((qmm.Q8_0, 576, 576, 1, 3), qmm.EUNSUPPORTED),   # unknown mode
    ((qmm.Q8_0, 576, 576, 1, 2), qmm.OK),             # dequantize-all
    ((qmm.Q4_K, 576, 576, 1, 2), qmm.EBLOCK),
    ((qmm.Q8_0, 0, 576, 1, 0), qmm.EINVAL),
    ((qmm.Q8_0, 576, 576, 0, 0), qmm.EINVAL),
    ((qmm.Q8_0, -5, 576, 1, 0), qmm.EINVAL),
    ((qmm.Q8_0, 576, 576, 307, 1), qmm.OK),
    ((qmm.Q4_K, 14336, 4096, 512, 0), qmm.OK),
    ((qmm.Q5_0, 192, 576, 307, 1), qmm.OK),
    ((qmm.Q4_0, 576, 96, 1, 0), qmm.OK),       # an odd number of 32-value blocks
    ((qmm.Q8_0, 576, 96, 1, 1), qmm.OK),
    ((qmm.Q5_0, 100, 4128, 40, 0), qmm.OK),
    ((qmm.Q4_0, 576, 40, 1, 0), qmm.EBLOCK),
    ((qmm.Q6_K, 576, 576, 1, 1), qmm.EBLOCK),
    ((qmm.Q6_K, 576, 768, 512, 0), qmm.OK),
    ((qmm.Q6_K, 576, 1536, 1, 2), qmm.OK),
])
def test_check_status_codes(args, status):
    assert qmm.check(*args) == status


def test_shape_error_names_the_shape_and_block_size():
    assert qmm.check(qmm.Q4_K, 576, 576, 1, 0) == qmm.EBLOCK
    assert qmm.last_error() == "quantized tensor must have their last dim divisible by block size [576, 576] 256"


def test_create_rejects_before_touching_the_gpu():
    lib = qmm.lib()
    h = ctypes.c_void_p(1234)
    assert lib.qmatmul_create(ctypes.byref(h), qmm.Q4_K, 576, 576, 1, 0) == qmm.EBLOCK
    assert h.value is None
    assert lib.qmatmul_create(None, qmm.Q8_0, 576, 576, 1, 0) == qmm.EINVAL


def test_run_rejects_null_plan_and_bad_m():
    lib = qmm.lib()
    assert lib.qmatmul_run(None, None, None, None, 1, None) == qmm.EINVAL
    assert lib.qmatmul_run_block_sums(None, None, None, None, 1, None) == qmm.EINVAL
    assert lib.qmatmul_run_dequantized(None, None, None, None, 1, None) == qmm.EINVAL
    assert lib.qmatmul_destroy(None) == qmm.OK
    arr = (ctypes.c_void_p * 2)()  # null plans, null pointers
    assert lib.qmatmul_run_group(None, 1, None, None, None, 1, None) == qmm.EINVAL
    assert lib.qmatmul_run_group(arr, 0, arr, None, arr, 1, None) == qmm.EINVAL   # count out of range
    assert lib.qmatmul_run_group(arr, qmm.GROUP_MAX + 1, arr, None, arr, 1, None) == qmm.EINVAL
    assert lib.qmatmul_run_group(arr, 2, arr, None, arr, 1, None) == qmm.EINVAL   # null plan


def test_quantize_entry_points_validate_on_host():
    lib = qmm.lib()
    assert lib.qmatmul_quantize_act(qmm.Q4_K, None, 1, 256, None, None) == qmm.EUNSUPPORTED
    assert lib.qmatmul_quantize_act(qmm.Q8_K, None, 1, 300, None, None) == qmm.EBLOCK
    assert lib.qmatmul_quantize_act(qmm.Q8_0, None, 0, 64, None, None) == qmm.OK   # M = 0: nothing to do
    assert lib.qmatmul_quantize_act(qmm.Q8_0, None, 2, 64, None, None) == qmm.EINVAL
    assert lib.qmatmul_quantize_act(qmm.Q8_0, ctypes.c_void_p(8), 2, 64, ctypes.c_void_p(64), None) == qmm.EINVAL
    assert lib.qmatmul_quantize_weights(qmm.Q8_K, None, 1, 256, None, None) == qmm.EUNSUPPORTED
    assert lib.qmatmul_quantize_weights(qmm.Q4_K, None, 1, 576, None, None) == qmm.EBLOCK
    assert lib.qmatmul_quantize_weights(qmm.Q6_K, None, 1, 576, None, None) == qmm.EBLOCK
    assert lib.qmatmul_quantize_weights(qmm.Q5_0, None, 2, 64, None, None) == qmm.EINVAL
    assert lib.qmatmul_dequantize_weights(qmm.Q4_0, None, 2, 96, None, None) == qmm.EINVAL  # odd block count: ok, null
    assert lib.qmatmul_dequantize_weights(qmm.Q8_K, None, 1, 256, None, None) == qmm.EUNSUPPORTED
    assert lib.qmatmul_dequantize_weights(qmm.Q4_K, None, 1, 576, None, None) == qmm.EBLOCK
    assert lib.qmatmul_dequantize_weights(qmm.Q8_0, None, 0, 64, None, None) == qmm.OK   # N = 0
    assert lib.qmatmul_dequantize_weights(qmm.Q8_0, None, 2, 64, None, None) == qmm.EINVAL
    assert lib.qmatmul_dequantize_weights(qmm.Q8_0, ctypes.c_void_p(16), 2, 64, ctypes.c_void_p(8), None) == qmm.EINVAL


def test_status_strings():
    for s in range(6):
        assert qmm.status_string(s)
    assert qmm.status_string(99) == "unknown status"
    assert qmm.lib().qmatmul_version() >= 1


def test_workspace_sizes_are_modest():
    # decode-only plans stay small; the prefill activation buffers scale with M_max * K
    assert 0 < qmm.workspace_bytes(qmm.Q8_0, 49152, 576, 1, 0) < 8 << 20
    big = qmm.workspace_bytes(qmm.Q4_K, 14336, 4096, 512, 0)
    assert 4 * 512 * 4096 <= big < 64 << 20
    assert qmm.workspace_bytes(qmm.Q4_K, 576, 576, 1, 0) == -1
    # Q4_0 decode plans keep only the quantized activations; prefill plans add
    # the weights as Q8_0 blocks
    small = qmm.workspace_bytes(qmm.Q4_0, 14336, 4096, 8, 1)
    assert 0 < small < 1 << 20
    assert qmm.workspace_bytes(qmm.Q4_0, 14336, 4096, 512, 1) >= 14336 * 128 * 34
    # dequantize-all plans hold the decoded f32 weights
    assert qmm.workspace_bytes(qmm.Q8_0, 576, 576, 1, 2) == 4 * 576 * 576
