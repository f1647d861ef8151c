"""rotattn for MI355X: RoPE-aware rotated mixed-precision INT4 FlashAttention (HIP, gfx950).

The C ABI is include/rotattn.h; `binding` is its ctypes mirror. Importing the
package does not load the library; the first call does, and raises if
librotattn.so has not been built.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    ROT_FULL, ROT_GROUP64, ROT_PAIR, Problem, QKCodes, VCodes, RotattnError, make_problem, problem_from_workload,
    get_sizes, workspace_bytes, rotattn_quantize_qk, rotattn_quantize_qk_static, rotattn_quantize_v,
    rotattn_attention, rotattn_forward, rotattn_fp16_forward, rotattn_debug_dump, rotattn_block_mask, rotattn_sparse_attention, mask_to_bool,
    load_library,
)

__all__ = [n for n in dir() if n.startswith("rotattn_") or n in (
    "ROT_FULL", "ROT_GROUP64", "ROT_PAIR", "Problem", "QKCodes", "VCodes", "RotattnError", "make_problem",
    "problem_from_workload", "get_sizes", "workspace_bytes", "load_library")]
