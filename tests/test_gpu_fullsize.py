"""Parity at the full workload sizes, in the launch configuration bench.py times.

For each workload (480p, small head dim with text prefix, mixed precision,
720p) the whole path runs on the GPU exactly as the benchmark runs it
(rotattn_quantize_qk, rotattn_quantize_v, rotattn_attention). Two heads are
then checked against the oracle: their Q/K/V codes, scales and flags in full,
and the INT4 kernel's integers and the outputs on sampled 64-row query blocks
(first, middle, last, which is ragged) that the oracle computes over all keys.
"""
import numpy as np
import pytest

import workloads as W
from oracle import core as O
from tests import gpu_common as G

torch = G.torch
pytestmark = pytest.mark.gpu

FULL = ["480p", "smalld", "mixed", "720p"]


def _sample_blocks(NB):
    return sorted({0, NB // 2, NB - 1})


@pytest.mark.parametrize("name", FULL)
def test_fullsize_sampled(name):
    G.require_gpu()
    w = W.WORKLOADS[name]
    print(f"[gpu] fullsize {name}: B={w.B} H={w.H} L={w.L} D={w.D}", flush=True)
    x = W.full_inputs(w, threads=16)
    p = G.R.problem_from_workload(w)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[t]).to(dev) for t in ("q", "k", "v"))
    mask_np = W.head_fallback_mask(w)
    mask = torch.from_numpy(mask_np).to(dev) if mask_np is not None else None
    need_rope = mask is not None or np.isfinite(w.tau)
    qk = G.R.rotattn_quantize_qk(p, q, k, rope_copy=need_rope)
    vq = G.R.rotattn_quantize_v(p, v)
    out = G.R.rotattn_attention(p, qk, vq, v=v if need_rope else None, head_fallback=mask)
    s = G.R.get_sizes(p)
    NB, Lp, L = s.NB, s.Lp, w.L
    rng = np.random.default_rng(2024)
    heads = sorted(rng.choice(w.H, size=2, replace=False).tolist())
    if mask_np is not None:   # include one masked and one unmasked head
        heads = [int(np.nonzero(mask_np)[0][0]), int(np.nonzero(mask_np == 0)[0][0])]
    qbs = _sample_blocks(NB)
    units = np.array([h * NB + qb for h in heads for qb in qbs], dtype=np.int32)
    dump = G.R.rotattn_debug_dump(p, qk, vq, G.dev(units), head_fallback=mask)
    torch.cuda.synchronize()
    acc = {kk: t.cpu().numpy() for kk, t in dump.items()}
    del dump
    total = mism = 0
    for h in heads:
        masked = bool(mask_np[h]) if mask_np is not None else False
        qf_gpu = qk.q_flag[0, h].cpu().numpy().astype(bool)
        kf_gpu = qk.k_flag[0, h].cpu().numpy().astype(bool)
        rows = np.concatenate([np.arange(qb * 64, min(qb * 64 + 64, L)) for qb in qbs])
        o = G.oracle_head(w, x, 0, h, head_masked=masked, q_flags=qf_gpu, k_flags=kf_gpu, rows=rows)
        # prologue, whole head
        for t in ("q", "k"):
            codes = G.unpack_qk_codes(getattr(qk, f"{t}_codes")[0, h].cpu().numpy())
            assert np.array_equal(codes, o[t]["codes"]), (name, h, t)
            assert np.array_equal(getattr(qk, f"{t}_scale")[0, h].cpu().numpy(), o[t]["scale"]), (name, h, t)
            assert G.flags_agree(getattr(qk, f"{t}_flag")[0, h].cpu().numpy(), o[t]["nsr"], w.tau), (name, h, t)
        vc = G.decode_v_codes(vq.v_codes[:, h:h + 1].cpu().numpy())[0, 0]
        assert np.array_equal(vc, o["v_codes"])
        assert np.array_equal(vq.v_scale[0, h].cpu().numpy(), o["v_scale"])
        assert np.array_equal(vq.v_colsum[0, h].cpu().numpy(), o["v_colsum"])
        # INT4 loop integers and outputs on the sampled query blocks
        got_all = out[0, h].float().cpu().numpy().astype(np.float64)
        for bi, qb in enumerate(qbs):
            rr = np.arange(qb * 64, min(qb * 64 + 64, L))
            sel = np.searchsorted(rows, rr)
            ref_out = o["out"][sel]
            tol = G.ATOL + G.RTOL * np.abs(ref_out)
            fp16_row = masked or qf_gpu[qb]
            flip = np.zeros(rr.size, bool)
            if not fp16_row:
                u = heads.index(h) * len(qbs) + bi
                ref = O.int4_flash_rows(o["q"]["codes"], o["q"]["scale"], o["k"]["codes"], o["k"]["scale"],
                                        o["v_codes"], o["v_scale"], o["v_colsum"], L, w.D, rr,
                                        key_blocks=~kf_gpu, dump=True)
                keep = np.repeat(~kf_gpu, 64)[:L]
                n = rr.size
                assert np.array_equal(acc["acc"][u, :n, :L][:, keep], ref["acc"][:, :L][:, keep]), (name, h, qb)
                assert np.array_equal(acc["m"][u, :n][:, ~kf_gpu], ref["m_hist"][:, ~kf_gpu]), (name, h, qb)
                gp = acc["pq"][u, :n, :L][:, keep]
                op = ref["pq"][:, :L][:, keep]
                kidx = np.nonzero(keep)[0]
                cq = np.float32(o["q"]["scale"][qb] * O.softmax_c0(w.D))
                c = (cq * o["k"]["scale"][kidx // 64]).astype(np.float32).astype(np.float64)
                m15 = (ref["m_hist"][:, kidx // 64] - O.LOG2_15).astype(np.float32).astype(np.float64)
                accf = ref["acc"][:, :L][:, keep].astype(np.float32).astype(np.float64)
                P15 = np.exp2((accf * c[None, :] - m15).astype(np.float32).astype(np.float64))
                ok, nb = G.tie_mismatch_ok(gp, op, P15)
                assert ok, (name, h, qb, nb)
                total += gp.size
                mism += nb
                same = np.all(gp == op, axis=1)
                assert np.array_equal(acc["accpv"][u, :n][same][:, ~kf_gpu], ref["accpv"][same][:, ~kf_gpu])
                flip = ~same
                if kf_gpu.any():   # mixed rows: the FP16 half carries the fp16 weight bound
                    _, bound = G.fp16_weight_bound(o["q"]["rope16"], o["k"]["rope16"], x["v"][0, h], L, w.D, rr,
                                                   key_blocks=kf_gpu)
                    tol = tol + bound
            else:
                _, bound = G.fp16_weight_bound(o["q"]["rope16"], o["k"]["rope16"], x["v"][0, h], L, w.D, rr)
                tol = tol + bound
            err = np.abs(got_all[rr] - ref_out)
            bad = (err > tol) & ~flip[:, None]
            assert not bad.any(), (name, h, qb, float(err[~flip].max()) if (~flip).any() else 0.0)
    assert mism <= 1e-4 * max(total, 1), (mism, total)
