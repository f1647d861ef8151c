"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI, decode its layouts, and compare with the oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest

import workloads as W
from oracle import core as O

torch = pytest.importorskip("torch")

import int4_quantized_flashattention_amd as R  # noqa: E402

# Output tolerance of the quantized path against the oracle's float64 result:
# the 2e-3 absolute bar, plus the float16 output's own rounding (2^-11 of the
# value) doubled to cover float32 accumulation-order differences.
ATOL = 2e-3
RTOL = 2.0 ** -10


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R.load_library()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def variant(name, **kw) -> W.Workload:
    return W.WORKLOADS[name].replace(**kw)


def inputs(w: W.Workload, heads=None):
    """Full [B, H, L, D] inputs (all heads) as numpy fp16."""
    return W.full_inputs(w)


def unpack_qk_codes(packed):
    """GPU Q/K codes [..., Lp, D'/2] -> int8 [..., Lp, D'] (low nibble = even dim)."""
    return O.unpack_nibbles(packed)


def _v_key_maps():
    lo = np.zeros(32, dtype=np.int64)
    hi = np.zeros(32, dtype=np.int64)
    for hh in range(2):
        for s in range(2):
            for w in range(2):
                for b in range(4):
                    pos = 16 * hh + 8 * s + 4 * w + b
                    lo[pos] = 32 * s + 16 * w + 4 * hh + b
                    hi[pos] = 32 * s + 16 * w + 8 + 4 * hh + b
    return lo, hi


V_KEY_LO, V_KEY_HI = _v_key_maps()


def decode_v_codes(vc):
    """GPU V codes [B, H, NB, D, 32] (operand order) -> int8 [B, H, NB*64, D]."""
    B, H, NB, D, _ = vc.shape
    x = vc.astype(np.int16)
    lo = x & 0xF
    hi = (x >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.zeros((B, H, NB, 64, D), dtype=np.int8)
    out[:, :, :, V_KEY_LO, :] = np.moveaxis(lo, -1, -2)
    out[:, :, :, V_KEY_HI, :] = np.moveaxis(hi, -1, -2)
    return out.reshape(B, H, NB * 64, D)


def oracle_head(w: W.Workload, x, b, h, tau=None, head_masked=False, q_flags=None, k_flags=None, rows=None):
    return O.forward_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], prefix=w.prefix, grid=w.grid,
                          split=w.split, base=w.base, rotation=w.rotation,
                          tau=w.tau if tau is None else tau, head_masked=head_masked,
                          q_flags=q_flags, k_flags=k_flags, rows=rows)


def flags_agree(gpu_flags, nsr, tau, rel=1e-4):
    """Block flags equal NSR > tau except where NSR sits within `rel` of tau (float32 sum order)."""
    want = nsr > tau
    near = np.abs(nsr - tau) <= rel * tau
    return bool(np.all((gpu_flags.astype(bool) == want) | near))


def fp16_weight_bound(qr16, kr16, v16, L, D, rows, key_blocks=None):
    """Worst-case effect of rounding the softmax weights to fp16 in the P.V product, per output element.

    Each weight P_j/l carries a relative rounding error of at most 2^-11 (or an
    absolute 2^-25 in the fp16 subnormal range), so the output moves by at most
    2^-11 sum_j (P_j/l)|v_j| + 2^-25 sum_j |v_j| / l.
    """
    p = O.fp16_rows(qr16, kr16, v16, L, D, rows, key_blocks)
    nb = O.n_blocks(L)
    kb = np.ones(nb, bool) if key_blocks is None else key_blocks
    keys = np.nonzero(np.repeat(kb, 64)[:L])[0]
    q = qr16[rows].astype(np.float64)
    k = kr16[keys].astype(np.float64)
    va = np.abs(v16[keys].astype(np.float64))
    S2 = (q @ k.T) * (math.log2(math.e) / math.sqrt(D))
    P = np.exp2(S2 - p["m"][:, None])
    return p, 2.0 ** -11 * (P @ va) / p["l"][:, None] + 2.0 ** -25 * va.sum(0)[None, :] / p["l"][:, None]


def tie_mismatch_ok(gpu_pq, oracle_pq, P15_oracle, eps=1e-5):
    """P codes may differ by 1 where 15 P sits within eps of a rounding boundary (the exp2 evaluations differ)."""
    diff = gpu_pq.astype(int) - oracle_pq.astype(int)
    bad = diff != 0
    if not bad.any():
        return True, 0
    if np.abs(diff[bad]).max() > 1:
        return False, int(bad.sum())
    x = P15_oracle[bad].astype(np.float64)
    near = np.abs(x - np.floor(x) - 0.5) < eps
    return bool(near.all()), int(bad.sum())
