"""Parity past the 2^22-token mark: one head of L = 2^22 + 7 tokens (7 text tokens before a 64x256x256
video grid) at D = 64. The prologue's grid coordinates leave their reciprocal path (exact for L <= 2^22)
for integer division there, every query row visits 65536 key blocks, and the last query block is ragged.
Both prologue kernels are covered: even RoPE groups (22/22/20) take the register kernel, odd ones
(22/21/21) the LDS-tile kernel. Checked against the oracle: Q/K/V codes, scales and flags of the whole
head bitwise (flags to the derived window), and the outputs of the first, a middle and the last (ragged)
64-row query block to the derived tolerance."""
import numpy as np
import pytest

import workloads as W
from tests import gpu_common as G

torch = G.torch
pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
@pytest.mark.parametrize("split", [(22, 22, 20), (22, 21, 21)])
def test_long_sequence_past_2p22(split):
    G.require_gpu()
    w = W.WORKLOADS["smalld"].replace(H=1, grid=(64, 256, 256), prefix=7, split=split)
    assert w.L == (1 << 22) + 7
    print(f"[gpu] long sequence L={w.L} D={w.D} split={split}: inputs", flush=True)
    x = W.full_inputs(w, threads=16)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[t]).to(dev) for t in ("q", "k", "v"))
    p = G.R.problem_from_workload(w)
    print("[gpu] long sequence: quantize_qk, quantize_v, attention", flush=True)
    qk = G.R.rotattn_quantize_qk(p, q, k)
    vq = G.R.rotattn_quantize_v(p, v)
    out = G.R.rotattn_attention(p, qk, vq)
    torch.cuda.synchronize()
    NB = G.R.get_sizes(p).NB
    rows = np.concatenate([np.arange(0, 64), np.arange((NB // 2) * 64, (NB // 2) * 64 + 64),
                           np.arange((NB - 1) * 64, w.L)])
    got = out[0, 0].index_select(0, torch.from_numpy(rows).to(dev)).float().cpu().numpy().astype(np.float64)
    print(f"[gpu] long sequence: oracle over {w.L} tokens, {rows.size} rows", flush=True)
    o = G.oracle_head(w, x, 0, 0, rows=rows)
    for t in ("q", "k"):
        codes = G.unpack_qk_codes(getattr(qk, f"{t}_codes")[0, 0].cpu().numpy())
        assert np.array_equal(codes, o[t]["codes"]), t
        assert np.array_equal(getattr(qk, f"{t}_scale")[0, 0].cpu().numpy(), o[t]["scale"]), t
        assert G.flags_agree(getattr(qk, f"{t}_flag")[0, 0].cpu().numpy(), o[t]["nsr"], w.tau, w.Dp), t
    vc = G.decode_v_codes(vq.v_codes.cpu().numpy())[0, 0]
    assert np.array_equal(vc, o["v_codes"])
    assert np.array_equal(vq.v_scale[0, 0].cpu().numpy(), o["v_scale"])
    assert np.array_equal(vq.v_colsum[0, 0].cpu().numpy(), o["v_colsum"])
    print("[gpu] long sequence: output tolerance", flush=True)
    tol = G.head_output_tol(w, x, 0, 0, o, False, rows=rows)
    err = np.abs(got - o["out"])
    assert (err <= tol).all(), (float(err.max()), np.argwhere(err > tol)[:4].tolist())
