"""ctypes binding of librotattn.so (include/rotattn.h), same names, argument marshalling only.

PyTorch supplies device memory and the current stream; every step of the
attention path runs in the library's HIP kernels. If the library is missing
the calls raise: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import functools
import inspect
import math
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
# ROTATTN_LIBRARY: another build of the same library (e.g. one with host-side sanitizers)
LIB_PATH = os.environ.get("ROTATTN_LIBRARY") or os.path.join(HERE, "librotattn.so")

ROT_FULL = 0
ROT_GROUP64 = 1
ROT_PAIR = 2

CALL_QUANTIZE_QK = 0
CALL_QUANTIZE_V = 1
CALL_ATTENTION = 2
CALL_FORWARD = 3
CALL_FP16_FORWARD = 4
CALL_DEBUG_DUMP = 5
CALL_BLOCK_MASK = 6
CALL_SPARSE_ATTENTION = 7
CALL_ATTENTION_HEAD_FALLBACK = 8
CALL_FORWARD_HEAD_FALLBACK = 9

ERRORS = {0: "ROTATTN_OK", -1: "ROTATTN_EINVAL", -2: "ROTATTN_EUNSUPPORTED", -3: "ROTATTN_EALIGN",
          -4: "ROTATTN_EWORKSPACE", -5: "ROTATTN_ELAUNCH", -6: "ROTATTN_ESCRATCH"}

EXPORTS = ["rotattn_version", "rotattn_strerror", "rotattn_get_sizes", "rotattn_workspace_bytes",
           "rotattn_quantize_qk", "rotattn_quantize_v", "rotattn_attention", "rotattn_forward",
           "rotattn_fp16_forward", "rotattn_debug_dump", "rotattn_block_mask", "rotattn_sparse_attention",
           "rotattn_quantize_qk_static"]


class Problem(C.Structure):
    _fields_ = [("B", C.c_int32), ("H", C.c_int32), ("L", C.c_int32), ("D", C.c_int32),
                ("grid_t", C.c_int32), ("grid_h", C.c_int32), ("grid_w", C.c_int32),
                ("text_prefix", C.c_int32), ("rope_split", C.c_int32 * 3), ("rotation", C.c_int32),
                ("rope_base", C.c_double), ("stride_b", C.c_int64), ("stride_h", C.c_int64),
                ("stride_l", C.c_int64), ("block_err_tau", C.c_float), ("reserved", C.c_int32)]


class QKBuffers(C.Structure):
    _fields_ = [("q_codes", C.c_void_p), ("k_codes", C.c_void_p), ("q_scale", C.c_void_p),
                ("k_scale", C.c_void_p), ("q_flag", C.c_void_p), ("k_flag", C.c_void_p),
                ("head_kflag", C.c_void_p), ("q_rope", C.c_void_p), ("k_rope", C.c_void_p),
                ("q_bsum", C.c_void_p), ("k_bsum", C.c_void_p)]


class VBuffers(C.Structure):
    _fields_ = [("v_codes", C.c_void_p), ("v_scale", C.c_void_p), ("v_colsum", C.c_void_p)]


class Sizes(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("Lp", "NB", "Dp", "qk_codes_bytes", "qk_scale_bytes", "qk_flag_bytes",
                                         "head_flag_bytes", "rope_bytes", "v_codes_bytes", "v_scale_bytes",
                                         "v_colsum_bytes", "out_min_elems", "bsum_bytes", "mask_rows", "mask_words",
                                         "mask_bytes")]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load librotattn.so once and declare the argument types of every export."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m int4_quantized_flashattention_amd.build`")
    lib = C.CDLL(path)
    P = C.POINTER
    vp = C.c_void_p
    lib.rotattn_version.restype = C.c_int
    lib.rotattn_strerror.restype = C.c_char_p
    lib.rotattn_strerror.argtypes = [C.c_int]
    lib.rotattn_get_sizes.argtypes = [P(Problem), P(Sizes)]
    lib.rotattn_workspace_bytes.argtypes = [P(Problem), C.c_int, P(C.c_size_t)]
    lib.rotattn_quantize_qk.argtypes = [P(Problem), vp, vp, P(QKBuffers), vp, C.c_size_t, vp]
    lib.rotattn_quantize_qk_static.argtypes = [P(Problem), vp, vp, P(QKBuffers), vp]
    lib.rotattn_quantize_v.argtypes = [P(Problem), vp, P(VBuffers), vp, C.c_size_t, vp]
    lib.rotattn_attention.argtypes = [P(Problem), P(QKBuffers), P(VBuffers), vp, vp, vp, vp, C.c_size_t, vp]
    lib.rotattn_forward.argtypes = [P(Problem), P(QKBuffers), vp, vp, vp, vp, C.c_size_t, vp]
    lib.rotattn_fp16_forward.argtypes = [P(Problem), vp, vp, vp, vp, vp, C.c_size_t, vp]
    lib.rotattn_debug_dump.argtypes = [P(Problem), P(QKBuffers), P(VBuffers), vp, vp, vp, C.c_int32,
                                       vp, vp, vp, vp, vp, vp, C.c_size_t, vp]
    lib.rotattn_block_mask.argtypes = [P(Problem), P(QKBuffers), C.c_int32, vp, vp, C.c_size_t, vp]
    lib.rotattn_sparse_attention.argtypes = [P(Problem), P(QKBuffers), P(VBuffers), vp, vp, vp, C.c_size_t, vp]
    for name in EXPORTS:
        if name not in ("rotattn_strerror",):
            getattr(lib, name).restype = C.c_int
    _lib = lib
    return lib


class RotattnError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = load_library().rotattn_strerror(code).decode()
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({msg})")
        self.code = code


def _check(code: int, where: str):
    if code != 0:
        raise RotattnError(code, where)


def make_problem(B, H, L, D, grid, prefix, split, rotation=ROT_FULL, base=10000.0, tau=math.inf,
                 strides=None) -> Problem:
    """strides: (stride_b, stride_h, stride_l) in elements; default dense [B, H, L, D]."""
    if strides is None:
        strides = (H * L * D, L * D, D)
    p = Problem()
    p.B, p.H, p.L, p.D = B, H, L, D
    p.grid_t, p.grid_h, p.grid_w = grid
    p.text_prefix = prefix
    p.rope_split[0], p.rope_split[1], p.rope_split[2] = split
    p.rotation = rotation
    p.rope_base = base
    p.stride_b, p.stride_h, p.stride_l = strides
    p.block_err_tau = tau
    p.reserved = 0
    return p


def problem_from_workload(w, strides=None, tau=None) -> Problem:
    return make_problem(w.B, w.H, w.L, w.D, w.grid, w.prefix, w.split, w.rotation, w.base,
                        w.tau if tau is None else tau, strides)


def get_sizes(p: Problem) -> Sizes:
    s = Sizes()
    _check(load_library().rotattn_get_sizes(C.byref(p), C.byref(s)), "rotattn_get_sizes")
    return s


def workspace_bytes(p: Problem, call: int) -> int:
    n = C.c_size_t(0)
    _check(load_library().rotattn_workspace_bytes(C.byref(p), call, C.byref(n)), "rotattn_workspace_bytes")
    return n.value


# --------------------------------------------------------------------------
# torch-facing helpers
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _on_stream(fn):
    """Run an entry point with the caller's `stream` (if given) as torch's current stream, so that the
    buffers the binding allocates for the call (workspace, outputs) belong to that stream: the caching
    allocator then reuses a freed workspace only for work ordered after the call on the same stream."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapped(*args, **kwargs):
        s = sig.bind(*args, **kwargs).arguments.get("stream")
        if s is None:
            return fn(*args, **kwargs)
        with _torch().cuda.stream(s):
            return fn(*args, **kwargs)
    return wrapped


def _workspace(p: Problem, call: int, device, ws=None):
    torch = _torch()
    n = workspace_bytes(p, call)
    if ws is not None:
        if ws.numel() * ws.element_size() < n:
            raise ValueError(f"workspace of {ws.numel()} bytes is smaller than the {n} bytes needed")
        return ws, n
    if n == 0:
        return None, 0
    return torch.empty(n, dtype=torch.uint8, device=device), n


def _strides_of(t):
    """(stride_b, stride_h, stride_l) of a [B, H, L, D] tensor with a contiguous last axis."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, H, L, D] tensor with a contiguous head dim")
    return (t.stride(0), t.stride(1), t.stride(2))


@dataclass
class QKCodes:
    q_codes: object
    k_codes: object
    q_scale: object
    k_scale: object
    q_flag: object
    k_flag: object
    head_kflag: object
    q_rope: object = None
    k_rope: object = None
    q_bsum: object = None
    k_bsum: object = None

    def struct(self) -> QKBuffers:
        s = QKBuffers()
        for name, _ in QKBuffers._fields_:
            t = getattr(self, name)
            setattr(s, name, None if t is None else t.data_ptr())
        return s


@dataclass
class VCodes:
    v_codes: object
    v_scale: object
    v_colsum: object

    def struct(self) -> VBuffers:
        s = VBuffers()
        s.v_codes, s.v_scale, s.v_colsum = (self.v_codes.data_ptr(), self.v_scale.data_ptr(),
                                            self.v_colsum.data_ptr())
        return s


def alloc_qk(p: Problem, device, rope_copy: bool, block_sums: bool = False) -> QKCodes:
    torch = _torch()
    s = get_sizes(p)
    B, H = p.B, p.H
    u8, f32 = torch.uint8, torch.float32
    return QKCodes(
        q_codes=torch.empty((B, H, s.Lp, s.Dp // 2), dtype=u8, device=device),
        k_codes=torch.empty((B, H, s.Lp, s.Dp // 2), dtype=u8, device=device),
        q_scale=torch.empty((B, H, s.NB), dtype=f32, device=device),
        k_scale=torch.empty((B, H, s.NB), dtype=f32, device=device),
        q_flag=torch.empty((B, H, s.NB), dtype=u8, device=device),
        k_flag=torch.empty((B, H, s.NB), dtype=u8, device=device),
        head_kflag=torch.empty((B * H,), dtype=torch.int32, device=device),
        q_rope=torch.empty((B, H, p.L, p.D), dtype=torch.float16, device=device) if rope_copy else None,
        k_rope=torch.empty((B, H, p.L, p.D), dtype=torch.float16, device=device) if rope_copy else None,
        q_bsum=torch.empty((B, H, s.NB, p.D), dtype=f32, device=device) if block_sums else None,
        k_bsum=torch.empty((B, H, s.NB, p.D), dtype=f32, device=device) if block_sums else None,
    )


def alloc_v(p: Problem, device) -> VCodes:
    torch = _torch()
    s = get_sizes(p)
    return VCodes(
        v_codes=torch.empty((p.B, p.H, s.NB, p.D, 32), dtype=torch.uint8, device=device),
        v_scale=torch.empty((p.B, p.H, p.D), dtype=torch.float32, device=device),
        v_colsum=torch.empty((p.B, p.H, s.NB, p.D), dtype=torch.int32, device=device),
    )


@_on_stream
def rotattn_quantize_qk(p: Problem, q, k, out: QKCodes = None, rope_copy: bool = False, ws=None, stream=None,
                        block_sums: bool = False):
    """RoPE + rotation + per-block INT4 quantization of Q and K (see include/rotattn.h); block_sums also writes
    the RoPE'd block sums that rotattn_block_mask reads."""
    if out is None:
        out = alloc_qk(p, q.device, rope_copy, block_sums)
    ws, n = _workspace(p, CALL_QUANTIZE_QK, q.device, ws)
    st = out.struct()
    _check(load_library().rotattn_quantize_qk(C.byref(p), _ptr(q), _ptr(k), C.byref(st), _ptr(ws), n,
                                              _stream(stream)), "rotattn_quantize_qk")
    return out


@_on_stream
def rotattn_quantize_qk_static(p: Problem, q, k, out: QKCodes = None, rope_copy: bool = False, stream=None,
                               block_sums: bool = False):
    """rotattn_quantize_qk with the library's static scratch instead of a workspace (no device allocation inside
    the call; `out` must be given for that: allocating it here is only a convenience)."""
    if out is None:
        out = alloc_qk(p, q.device, rope_copy, block_sums)
    st = out.struct()
    _check(load_library().rotattn_quantize_qk_static(C.byref(p), _ptr(q), _ptr(k), C.byref(st), _stream(stream)),
           "rotattn_quantize_qk_static")
    return out


@_on_stream
def rotattn_quantize_v(p: Problem, v, out: VCodes = None, ws=None, stream=None):
    if out is None:
        out = alloc_v(p, v.device)
    ws, n = _workspace(p, CALL_QUANTIZE_V, v.device, ws)
    st = out.struct()
    _check(load_library().rotattn_quantize_v(C.byref(p), _ptr(v), C.byref(st), _ptr(ws), n, _stream(stream)),
           "rotattn_quantize_v")
    return out


@_on_stream
def rotattn_attention(p: Problem, qk: QKCodes, vq: VCodes, v=None, head_fallback=None, out=None, ws=None,
                      stream=None):
    torch = _torch()
    dev = qk.q_codes.device
    if out is None:
        out = torch.empty((p.B, p.H, p.L, p.D), dtype=torch.float16, device=dev)
    ws, n = _workspace(p, CALL_ATTENTION if head_fallback is None else CALL_ATTENTION_HEAD_FALLBACK, dev, ws)
    qs, vs = qk.struct(), vq.struct()
    _check(load_library().rotattn_attention(C.byref(p), C.byref(qs), C.byref(vs), _ptr(v), _ptr(head_fallback),
                                            _ptr(out), _ptr(ws), n, _stream(stream)), "rotattn_attention")
    return out


@_on_stream
def rotattn_forward(p: Problem, qk: QKCodes, v, head_fallback=None, out=None, ws=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((p.B, p.H, p.L, p.D), dtype=torch.float16, device=v.device)
    ws, n = _workspace(p, CALL_FORWARD if head_fallback is None else CALL_FORWARD_HEAD_FALLBACK, v.device, ws)
    qs = qk.struct()
    _check(load_library().rotattn_forward(C.byref(p), C.byref(qs), _ptr(v), _ptr(head_fallback), _ptr(out),
                                          _ptr(ws), n, _stream(stream)), "rotattn_forward")
    return out


@_on_stream
def rotattn_fp16_forward(p: Problem, q, k, v, out=None, ws=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((p.B, p.H, p.L, p.D), dtype=torch.float16, device=q.device)
    ws, n = _workspace(p, CALL_FP16_FORWARD, q.device, ws)
    _check(load_library().rotattn_fp16_forward(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ws), n,
                                               _stream(stream)), "rotattn_fp16_forward")
    return out


@_on_stream
def rotattn_block_mask(p: Problem, qk: QKCodes, topn: int, out=None, ws=None, stream=None):
    """Block-sparse mask from the block sums of rotattn_quantize_qk(block_sums=True) (see include/rotattn.h):
    int32 view of uint32 [B, H, mask_rows, mask_words], one row per 128 query rows."""
    torch = _torch()
    s = get_sizes(p)
    dev = qk.q_codes.device
    if out is None:
        out = torch.empty((p.B, p.H, s.mask_rows, s.mask_words), dtype=torch.int32, device=dev)
    ws, n = _workspace(p, CALL_BLOCK_MASK, dev, ws)
    qs = qk.struct()
    _check(load_library().rotattn_block_mask(C.byref(p), C.byref(qs), int(topn), _ptr(out), _ptr(ws), n,
                                             _stream(stream)), "rotattn_block_mask")
    return out


@_on_stream
def rotattn_sparse_attention(p: Problem, qk: QKCodes, vq: VCodes, block_mask, out=None, ws=None, stream=None):
    """Block-sparse INT4 attention over the key blocks `block_mask` keeps (see include/rotattn.h)."""
    torch = _torch()
    dev = qk.q_codes.device
    if out is None:
        out = torch.empty((p.B, p.H, p.L, p.D), dtype=torch.float16, device=dev)
    ws, n = _workspace(p, CALL_SPARSE_ATTENTION, dev, ws)
    qs, vs = qk.struct(), vq.struct()
    _check(load_library().rotattn_sparse_attention(C.byref(p), C.byref(qs), C.byref(vs), _ptr(block_mask),
                                                   _ptr(out), _ptr(ws), n, _stream(stream)),
           "rotattn_sparse_attention")
    return out


def mask_to_bool(mask_words, NB: int):
    """Host helper: int32/uint32 words [..., rows, mask_words] -> bool [..., rows, NB]."""
    import numpy as np
    w = np.asarray(mask_words).astype(np.uint32)
    bits = (w[..., :, :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(w.shape[:-1] + (w.shape[-1] * 32,))[..., :NB].astype(bool)


@_on_stream
def rotattn_debug_dump(p: Problem, qk: QKCodes, vq: VCodes, units, head_fallback=None, ws=None, stream=None,
                       block_mask=None, p15: bool = True):
    """Intermediate integers of the INT4 kernel for 64-row query blocks `units` ((b*H+h)*NB + block), and (p15)
    the float32 15 P each P code is rounded from."""
    torch = _torch()
    dev = qk.q_codes.device
    s = get_sizes(p)
    units = torch.as_tensor(units, dtype=torch.int32, device=dev)
    n = units.numel()
    acc = torch.zeros((n, 64, s.Lp), dtype=torch.int32, device=dev)
    pq = torch.zeros((n, 64, s.Lp), dtype=torch.int8, device=dev)
    pv = torch.zeros((n, 64, s.NB, p.D), dtype=torch.int32, device=dev)
    m = torch.full((n, 64, s.NB), float("nan"), dtype=torch.float32, device=dev)
    y = torch.zeros((n, 64, s.Lp), dtype=torch.float32, device=dev) if p15 else None
    ws, nws = _workspace(p, CALL_DEBUG_DUMP, dev, ws)
    qs, vs = qk.struct(), vq.struct()
    _check(load_library().rotattn_debug_dump(C.byref(p), C.byref(qs), C.byref(vs), _ptr(head_fallback),
                                             _ptr(block_mask), _ptr(units), n, _ptr(acc), _ptr(pq), _ptr(pv),
                                             _ptr(m), _ptr(y),
                                             _ptr(ws), nws, _stream(stream)), "rotattn_debug_dump")
    out = {"acc": acc, "pq": pq, "accpv": pv, "m": m}
    if y is not None:
        out["p15"] = y
    return out


# short aliases
quantize_qk = rotattn_quantize_qk
quantize_qk_static = rotattn_quantize_qk_static
quantize_v = rotattn_quantize_v
attention = rotattn_attention
forward = rotattn_forward
fp16_forward = rotattn_fp16_forward
debug_dump = rotattn_debug_dump
block_mask = rotattn_block_mask
sparse_attention = rotattn_sparse_attention
