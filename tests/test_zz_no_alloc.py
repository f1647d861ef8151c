"""The allocation-free Q/K entry point (rotattn_quantize_qk_static, static device scratch) against
rotattn_quantize_qk (caller's workspace): identical codes, scales, flags, head flags and RoPE'd copies, on two
calls in a row, the second with a smaller problem whose tables differ (its scratch keeps the first call's
larger tables underneath)."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as G

torch = G.torch
pytestmark = pytest.mark.gpu

FIELDS = ("q_codes", "k_codes", "q_scale", "k_scale", "q_flag", "k_flag", "head_kflag", "q_rope", "k_rope")


def _compare(w, tau=None, plant=False):
    x = W.full_inputs(w)
    if plant:   # one high-norm key token, so that a K block is flagged and head_kflag is set
        x["k"][0, 0, 70] *= np.float16(12)
    p = G.R.problem_from_workload(w, tau=tau)
    q, k = G.dev(x["q"]), G.dev(x["k"])
    print(f"[gpu] static quantize_qk L={w.L} H={w.H} D={w.D} rotation={w.rotation} tau={tau}", flush=True)
    ref = G.R.rotattn_quantize_qk(p, q, k, rope_copy=True)
    out = G.R.binding.alloc_qk(p, q.device, True)
    for f in FIELDS:
        getattr(out, f).fill_(0x5A if getattr(out, f).dtype == torch.uint8 else 7)
    G.R.rotattn_quantize_qk_static(p, q, k, out=out)
    torch.cuda.synchronize()
    for f in FIELDS:
        a, b = G.host(getattr(ref, f)), G.host(getattr(out, f))
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f
    return G.host(out.head_kflag)


def test_static_quantize_qk_matches_workspace_call():
    G.require_gpu()
    # first call: 720p-shaped tables (21 + 45 + 80 positions), full Hadamard
    _compare(W.WORKLOADS["720p"].replace(H=2))
    # second call, smaller: 4 x 8 x 8 grid, the mergeable rotation (every table entry shifted by pi/4) and the
    # block rule on, with a flagged K block
    hk = _compare(W.WORKLOADS["tiny"].replace(rotation=W.ROT_PAIR), tau=0.05, plant=True)
    assert hk[0] != 0
