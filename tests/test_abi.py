"""The C ABI on the host (no GPU): exports, sizes and every validation error, all decided before any launch."""
import ctypes as C
import math
import os
import re

import pytest

import workloads as W

R = pytest.importorskip("int4_quantized_flashattention_amd")
from int4_quantized_flashattention_amd import binding as Bd  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    try:
        return Bd.load_library()
    except RuntimeError as e:
        pytest.skip(str(e))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "rotattn.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(rotattn_\w+)\(", src, flags=re.M)))


def test_exports_match_header():
    lib = _lib()
    names = _header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(Bd.EXPORTS) == names


def test_version_and_strerror():
    lib = _lib()
    assert lib.rotattn_version() == 5
    for code in (0, -1, -2, -3, -4, -5, -6, 7):
        assert lib.rotattn_strerror(code)


def _p(**kw):
    w = W.WORKLOADS["tiny"]
    p = Bd.problem_from_workload(w)
    for k, v in kw.items():
        if k == "rope_split":
            p.rope_split[0], p.rope_split[1], p.rope_split[2] = v
        else:
            setattr(p, k, v)
    return p


def test_sizes_720p():
    _lib()
    p = Bd.problem_from_workload(W.WORKLOADS["720p"])
    s = Bd.get_sizes(p)
    assert (s.Lp, s.NB, s.Dp) == (75648, 1182, 128)
    assert s.qk_codes_bytes == 40 * 75648 * 64
    assert s.v_codes_bytes == 40 * 1182 * 128 * 32
    assert s.v_colsum_bytes == 40 * 1182 * 128 * 4
    p2 = Bd.problem_from_workload(W.WORKLOADS["480p"])
    assert Bd.get_sizes(p2).Dp == 192
    # the attention workspace holds one LDS image per (head, key block): at D' = D = 128 the dense
    # 12288-byte form (64 K rows and 128 V rows of 24-byte FP6 slots, 4 and 2 slots per row)
    img = 40 * 1182 * 12288
    vt = 40 * 1182 * 64 * 128 * 2   # transposed fp16 V blocks of the FP16 path
    # without routing and without a head mask the FP16 path cannot run: no V^T blocks
    assert Bd.workspace_bytes(p, Bd.CALL_ATTENTION) == img
    assert Bd.workspace_bytes(p, Bd.CALL_ATTENTION_HEAD_FALLBACK) == img + vt
    assert Bd.workspace_bytes(p, Bd.CALL_FORWARD_HEAD_FALLBACK) - Bd.workspace_bytes(p, Bd.CALL_FORWARD) == vt
    assert Bd.workspace_bytes(p, Bd.CALL_DEBUG_DUMP) == img
    assert Bd.workspace_bytes(p, Bd.CALL_SPARSE_ATTENTION) == img
    # block-sparse mask: one row per 128 query rows, ceil(1182 / 32) = 37 words per row
    assert (s.mask_rows, s.mask_words, s.mask_bytes) == (591, 37, 40 * 591 * 37 * 4)
    assert s.bsum_bytes == 40 * 1182 * 128 * 4
    # with block routing: the V^T blocks with or without a head mask, and the INT4 partial results of rows
    # that mix both paths (float32 O [Lp, D] and m, l [Lp] per head)
    pm = Bd.problem_from_workload(W.WORKLOADS["mixed"])
    img_m = 12 * 512 * 16384   # D' = 192: dense, 64 x 6 + 128 x 2 slots of 24 bytes (15360), padded to 16384
    vt_m = 12 * 512 * 64 * 128 * 2
    part = 12 * 32768 * 128 * 4 + 2 * 12 * 32768 * 4
    assert Bd.workspace_bytes(pm, Bd.CALL_ATTENTION) == img_m + vt_m + part
    assert Bd.workspace_bytes(pm, Bd.CALL_ATTENTION_HEAD_FALLBACK) == img_m + vt_m + part


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), -2),
    (dict(D=64), -1),                      # split no longer sums to D
    (dict(rope_split=(40, 42, 42)), -1),
    (dict(L=255), -1),                     # L != prefix + T*Hh*W
    (dict(B=0), -1),
    (dict(rotation=7), -1),
    (dict(stride_l=100), -1),              # stride_l < D
    (dict(stride_l=132), -3),              # rows not 16-byte aligned
    (dict(rope_base=-1.0), -1),
    (dict(block_err_tau=float("nan")), -1),
    (dict(rotation=1, rope_split=(100, 14, 14)), -2),
    (dict(H=70000), -2),                   # grid y limit
    (dict(B=40000), -2),                   # grid z limit (two tensors per batch)
    (dict(B=1000, H=5000), -2),            # B*H*NB = 2e7 workgroups of 256 on one grid axis
    # RoPE tables of 2 * 2^25 positions * 64 pairs = 2^32 floats: more than 32-bit offsets address
    (dict(L=2 ** 25, grid_t=2 ** 25, grid_h=1, grid_w=1, rope_split=(128, 0, 0)), -2),
    (dict(L=2 ** 23, grid_t=2 ** 23, grid_h=1, grid_w=1, rope_split=(128, 0, 0)), 0),   # 2^30 floats: fine
])
def test_problem_validation(kw, code):
    _lib()
    p = _p(**kw)
    s = Bd.Sizes()
    assert Bd.load_library().rotattn_get_sizes(C.byref(p), C.byref(s)) == code


def test_call_validation_before_launch():
    """Null, misaligned and short-workspace arguments are rejected on the host (fake addresses are never touched)."""
    lib = _lib()
    p = _p()
    good = 0x10000
    qk = Bd.QKBuffers(*([good] * 7 + [None, None]))
    stream = C.c_void_p(None)
    n = Bd.workspace_bytes(p, Bd.CALL_QUANTIZE_QK)
    assert n > 0
    # null q
    assert lib.rotattn_quantize_qk(C.byref(p), None, C.c_void_p(good), C.byref(qk), C.c_void_p(good), n, stream) == -1
    # misaligned k
    assert lib.rotattn_quantize_qk(C.byref(p), C.c_void_p(good), C.c_void_p(good + 2), C.byref(qk),
                                   C.c_void_p(good), n, stream) == -3
    # short workspace
    assert lib.rotattn_quantize_qk(C.byref(p), C.c_void_p(good), C.c_void_p(good), C.byref(qk),
                                   C.c_void_p(good), n - 1, stream) == -4
    # missing code buffer
    bad = Bd.QKBuffers(*([good] * 6 + [None, None, None]))
    assert lib.rotattn_quantize_qk(C.byref(p), C.c_void_p(good), C.c_void_p(good), C.byref(bad),
                                   C.c_void_p(good), n, stream) == -1
    # the FP16 path needs the RoPE'd copies when routing is possible
    vb = Bd.VBuffers(good, good, good)
    mask = C.c_void_p(good)
    assert lib.rotattn_attention(C.byref(p), C.byref(qk), C.byref(vb), C.c_void_p(good), mask, C.c_void_p(good),
                                 None, 0, stream) == -1
    # out missing
    assert lib.rotattn_forward(C.byref(p), C.byref(qk), C.c_void_p(good), None, None, None, 0, stream) == -1
    # fp16 forward without workspace
    assert lib.rotattn_fp16_forward(C.byref(p), C.c_void_p(good), C.c_void_p(good), C.c_void_p(good),
                                    C.c_void_p(good), None, 0, stream) == -4
    # dump with a negative unit count
    assert lib.rotattn_debug_dump(C.byref(p), C.byref(qk), C.byref(vb), None, None, None, -1, None, None, None,
                                  None, None, None, 0, stream) == -1
    # dump without its workspace (the K/V block images)
    one = C.c_void_p(good)
    assert lib.rotattn_debug_dump(C.byref(p), C.byref(qk), C.byref(vb), None, None, one, 1, one, one, one, one,
                                  None, None, 0, stream) == -4
    # dump with a block mask and a head mask together
    assert lib.rotattn_debug_dump(C.byref(p), C.byref(qk), C.byref(vb), one, one, one, 1, one, one, one, one,
                                  None, None, 0, stream) == -1
    # block mask: needs the block sums; topn < 1; null or misaligned mask (no workspace needed)
    assert Bd.workspace_bytes(p, Bd.CALL_BLOCK_MASK) == 0
    qks = Bd.QKBuffers(*([good] * 7 + [None, None, good, good]))
    assert lib.rotattn_block_mask(C.byref(p), C.byref(qk), 4, one, None, 0, stream) == -1
    assert lib.rotattn_block_mask(C.byref(p), C.byref(qks), 0, one, None, 0, stream) == -1
    assert lib.rotattn_block_mask(C.byref(p), C.byref(qks), 4, None, None, 0, stream) == -1
    assert lib.rotattn_block_mask(C.byref(p), C.byref(qks), 4, C.c_void_p(good + 2), None, 0, stream) == -3
    qkm = Bd.QKBuffers(*([good] * 7 + [None, None, good + 4, good]))
    assert lib.rotattn_block_mask(C.byref(p), C.byref(qkm), 4, one, None, 0, stream) == -3
    # sparse attention: null mask; block routing on; no workspace
    assert lib.rotattn_sparse_attention(C.byref(p), C.byref(qk), C.byref(vb), None, one, one, 1 << 30,
                                        stream) == -1
    pr = _p(block_err_tau=0.05)
    assert lib.rotattn_sparse_attention(C.byref(pr), C.byref(qk), C.byref(vb), one, one, one, 1 << 30,
                                        stream) == -1
    assert lib.rotattn_sparse_attention(C.byref(p), C.byref(qk), C.byref(vb), one, one, None, 0, stream) == -4


def test_empty_problem_is_a_no_op():
    """L = 0 (no tokens) validates and enqueues nothing."""
    lib = _lib()
    p = _p(L=0, grid_t=0, text_prefix=0)
    good = 0x10000
    qk = Bd.QKBuffers(*([good] * 7 + [None, None]))
    ws = C.c_void_p(0x100000)
    n = Bd.workspace_bytes(p, Bd.CALL_QUANTIZE_QK)
    assert lib.rotattn_quantize_qk(C.byref(p), C.c_void_p(good), C.c_void_p(good), C.byref(qk), ws, n,
                                   C.c_void_p(None)) == 0


def test_static_quantize_qk_validation():
    """The allocation-free Q/K entry point: argument errors, and problems whose RoPE tables exceed its 1 MiB static
    scratch, are refused before any device call."""
    lib = _lib()
    good = 1 << 20
    qk = Bd.QKBuffers(*([good] * 7 + [None] * 4))
    p = _p()
    assert lib.rotattn_quantize_qk_static(C.byref(p), None, C.c_void_p(good), C.byref(qk), None) == -1
    assert lib.rotattn_quantize_qk_static(C.byref(p), C.c_void_p(good + 2), C.c_void_p(good), C.byref(qk), None) == -3
    big = _p(L=2 ** 23, grid_t=2 ** 23, grid_h=1, grid_w=1, rope_split=(128, 0, 0))   # 4 GiB of tables
    assert Bd.workspace_bytes(big, Bd.CALL_QUANTIZE_QK) > (1 << 20)
    assert lib.rotattn_quantize_qk_static(C.byref(big), C.c_void_p(good), C.c_void_p(good), C.byref(qk), None) == -6
    # the 720p tables (21 + 45 + 80 positions) fit easily
    assert Bd.workspace_bytes(Bd.problem_from_workload(W.WORKLOADS["720p"]), Bd.CALL_QUANTIZE_QK) < (1 << 20)

