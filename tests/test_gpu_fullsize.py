"""Parity at the full workload sizes, in the launch configuration bench.py times.

For each workload (tiny, 480p, small head dim with text prefix, mixed precision,
720p) the whole path runs on the GPU exactly as the benchmark runs it
(rotattn_quantize_qk, rotattn_quantize_v, rotattn_attention). Sampled heads
are then checked against the oracle: their Q/K/V codes, scales and flags in
full, and the INT4 kernel's integers, P codes and outputs on sampled 64-row
query blocks (the first, quarter points, the middle and the last, which is
ragged) that the oracle computes over all keys. The same rows also give the
fidelity report: cosine similarity of the GPU output to exact float64
attention (softmax(RoPE(Q) RoPE(K)^T / sqrt(D)) V, no quantization).
"""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import core as O
from tests import gpu_common as G

torch = G.torch
pytestmark = pytest.mark.gpu

FULL = ["tiny", "480p", "smalld", "mixed", "720p"]


def _sample_blocks(NB, n):
    qbs = {0, NB // 2, NB - 1}
    for i in range(1, n):
        if len(qbs) >= n:
            break
        qbs.add(i * NB // n)
    return sorted(qbs)


def _sample_heads(w, mask_np, rng):
    if mask_np is not None:   # two masked heads and two unmasked ones
        masked = np.nonzero(mask_np)[0]
        unmasked = np.nonzero(mask_np == 0)[0]
        return sorted([int(masked[0]), int(masked[-1]), int(unmasked[0]), int(unmasked[-1])])
    return sorted(rng.choice(w.H, size=min(4, w.H), replace=False).tolist())


def _report(name, rec):
    d = os.environ.get("ROTATTN_REPORT_DIR")
    if d:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, f"fidelity_{name}.json"), "w") as f:
            json.dump(rec, f, indent=1)


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
    NB, L = s.NB, w.L
    rng = np.random.default_rng(2024)
    heads = _sample_heads(w, mask_np, rng)
    qbs = _sample_blocks(NB, 6)
    units = np.array([h * NB + qb for h in heads for qb in qbs], dtype=np.int32)
    dump = G.R.rotattn_debug_dump(p, qk, vq, G.dev(units), head_fallback=mask)
    torch.cuda.synchronize()
    acc = {kk: t.cpu().numpy() for kk, t in dump.items()}
    del dump
    total = mism = flipped_rows = int4_rows = 0
    exp_err = 0.0
    gpu_rows, exact_rows, oracle_rows = [], [], []
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
            assert G.flags_agree(getattr(qk, f"{t}_flag")[0, h].cpu().numpy(), o[t]["nsr"], w.tau, w.Dp), (name, h, t)
        vc = G.decode_v_codes(vq.v_codes[:, h:h + 1].cpu().numpy())[0, 0]
        assert np.array_equal(vc, o["v_codes"])
        assert np.array_equal(vq.v_scale[0, h].cpu().numpy(), o["v_scale"])
        assert np.array_equal(vq.v_colsum[0, h].cpu().numpy(), o["v_colsum"])
        # INT4 loop integers, P codes and outputs on the sampled query blocks
        got_all = out[0, h].float().cpu().numpy().astype(np.float64)
        exact = O.exact_attention(x["q"][0, h], x["k"][0, h], x["v"][0, h], prefix=w.prefix, grid=w.grid,
                                  split=w.split, base=w.base, rows=rows)
        gpu_rows.append(got_all[rows])
        exact_rows.append(exact)
        oracle_rows.append(o["out"])
        nvis = int(np.count_nonzero(~kf_gpu))
        for bi, qb in enumerate(qbs):
            rr = np.arange(qb * 64, min(qb * 64 + 64, L))
            sel = np.searchsorted(rows, rr)
            ref_out = o["out"][sel]
            tol = G.ATOL + G.RTOL * np.abs(ref_out)
            if not (masked or qf_gpu[qb]):
                u = heads.index(h) * len(qbs) + bi
                ref = O.int4_flash_rows(o["q"]["codes"], o["q"]["scale"], o["k"]["codes"], o["k"]["scale"],
                                        o["v_codes"], o["v_scale"], o["v_colsum"], L, w.D, rr,
                                        key_blocks=~kf_gpu, dump=True)
                keep = np.repeat(~kf_gpu, 64)[:L]
                n = rr.size
                assert np.array_equal(acc["acc"][u, :n, :L][:, keep], ref["acc"][:, :L][:, keep]), (name, h, qb)
                assert np.array_equal(acc["m"][u, :n][:, ~kf_gpu], ref["m_hist"][:, ~kf_gpu]), (name, h, qb)
                kidx = np.nonzero(keep)[0]
                cq = np.float32(o["q"]["scale"][qb] * O.softmax_c0(w.D))
                c = (cq * o["k"]["scale"][kidx // 64]).astype(np.float32)
                chk = G.check_p_codes(acc["pq"][u, :n, :L][:, keep], acc["p15"][u, :n, :L][:, keep],
                                      ref["acc"][:, :L][:, keep], c, ref["m_hist"][:, kidx // 64])
                total += chk["entries"]
                mism += chk["mismatch"]
                exp_err = max(exp_err, chk["exp_err"])
                same = ~chk["flips"].any(axis=1)
                assert np.array_equal(acc["accpv"][u, :n][same][:, ~kf_gpu], ref["accpv"][same][:, ~kf_gpu])
                flipped_rows += int((~same).sum())
                int4_rows += n
                flips = np.zeros((n, L), bool)
                flips[:, keep] = chk["flips"]
                tol = G.int4_output_tol(ref_out, ref, o["v_scale"], nvis, chk["eta"], flips=flips,
                                        vcodes=o["v_codes"])
                if kf_gpu.any():   # mixed rows: the FP16 half carries its own bound
                    _, bound = G.fp16_weight_bound(o["q"]["rope16"], o["k"]["rope16"], x["v"][0, h], L, w.D, rr,
                                                   key_blocks=kf_gpu)
                    tol = tol + bound
            else:
                _, bound = G.fp16_weight_bound(o["q"]["rope16"], o["k"]["rope16"], x["v"][0, h], L, w.D, rr)
                tol = tol + bound
            err = np.abs(got_all[rr] - ref_out)
            bad = err > tol
            assert not bad.any(), (name, h, qb, float(err.max()), np.argwhere(bad)[:4].tolist())
    cos_gpu = O.cosine_similarity(np.concatenate(gpu_rows), np.concatenate(exact_rows))
    cos_oracle = O.cosine_similarity(np.concatenate(oracle_rows), np.concatenate(exact_rows))
    rec = {"workload": name, "heads": heads, "query_blocks": qbs, "rows_per_head": int(rows.size),
           "cosine_gpu_vs_exact": cos_gpu, "cosine_oracle_vs_exact": cos_oracle,
           "p_code_boundary_flips": mism, "p_codes_compared": total, "int4_rows": int4_rows,
           "rows_with_a_flip": flipped_rows, "device_exp2_max_rel_err": exp_err}
    print(f"[gpu] fidelity {json.dumps(rec)}", flush=True)
    _report(name, rec)
    assert mism <= 1e-4 * max(total, 1), (mism, total)
    # the GPU output is the oracle's to within the tolerances, so the two cosines agree closely
    assert abs(cos_gpu - cos_oracle) < 1e-3, (cos_gpu, cos_oracle)
