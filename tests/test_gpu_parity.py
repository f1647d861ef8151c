"""GPU parity: the HIP path through the C ABI against the CPU oracle, element by element.

Bars (bit-exact for integers, the stated tolerance for floating point):
  Q/K/V codes, scales, column sums, int32 Q.K^T and P.V accumulators: bitwise;
  block flags: exact except where the block's NSR is within 1e-6 tau of tau;
  P codes: those of the plain quantizer rne(fl(15 P)) - 8, except +-1 where
  the rounding boundary lies within the derived bound of the oracle's 15 P
  (gpu_common.p15_plain_and_bound), on at most 1e-4 of the entries; P.V
  accumulators compared on the rows whose P codes all match; running max:
  bitwise;
  outputs: |gpu - oracle| <= 2e-3 + 2^-11 |oracle| plus the derived float32
  terms of gpu_common.int4_output_tol (INT4 rows, with one code step per
  boundary flip) and gpu_common.fp16_weight_bound (tiles on the FP16 path).
"""
import numpy as np
import pytest

import workloads as W
from oracle import core as O
from tests import gpu_common as G

torch = G.torch
pytestmark = pytest.mark.gpu

CASES = {
    # name: (workload, heads to check)
    "tiny": W.WORKLOADS["tiny"],
    "ragged_prefix": W.WORKLOADS["tiny"].replace(grid=(2, 5, 19), prefix=8),
    "group64": W.WORKLOADS["480p"].replace(H=2, grid=(2, 7, 23)),
    "d64_prefix": W.WORKLOADS["smalld"].replace(H=3, grid=(2, 5, 11)),
    "d64_group64": W.WORKLOADS["smalld"].replace(H=2, grid=(1, 3, 30), prefix=5, rotation=W.ROT_GROUP64),
    "lognormal": W.WORKLOADS["720p"].replace(H=2, grid=(3, 9, 16)),
    "mixed": W.WORKLOADS["mixed"].replace(H=4, grid=(2, 9, 20)),
    "pair": W.WORKLOADS["tiny"].replace(rotation=W.ROT_PAIR),
    "d64_pair_prefix": W.WORKLOADS["smalld"].replace(H=2, grid=(2, 5, 11), prefix=37, rotation=W.ROT_PAIR),
    # even RoPE groups at D = 64: the register prologue, with its RoPE'd copies
    "d64_even": W.WORKLOADS["smalld"].replace(H=2, grid=(2, 5, 11), split=(22, 22, 20)),
    "d64_even_pair": W.WORKLOADS["smalld"].replace(H=2, grid=(2, 5, 11), prefix=37, split=(22, 22, 20),
                                                   rotation=W.ROT_PAIR),
    "d64_even_group64": W.WORKLOADS["smalld"].replace(H=2, grid=(1, 3, 30), prefix=5, split=(22, 22, 20),
                                                      rotation=W.ROT_GROUP64),
    "pair_mixed": W.WORKLOADS["mixed"].replace(H=4, grid=(2, 9, 20), rotation=W.ROT_PAIR),
}

_cache = {}


def _run(name):
    """Run quantize_qk + quantize_v + forward + dump of every query block for a case (cached)."""
    if name in _cache:
        return _cache[name]
    G.require_gpu()
    w = CASES[name]
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    q, k, v = G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"])
    mask_np = W.head_fallback_mask(w)
    mask = G.dev(mask_np) if mask_np is not None else None
    need_rope = mask is not None or np.isfinite(w.tau)
    print(f"[gpu] case={name} L={w.L} H={w.H} D={w.D} rot={w.rotation}", flush=True)
    qk = G.R.rotattn_quantize_qk(p, q, k, rope_copy=True)
    vq = G.R.rotattn_quantize_v(p, v)
    out = G.R.rotattn_forward(p, qk, v, head_fallback=mask)
    s = G.R.get_sizes(p)
    units = np.arange(w.B * w.H * s.NB, dtype=np.int32)
    dump = G.R.rotattn_debug_dump(p, qk, vq, G.dev(units), head_fallback=mask)
    torch.cuda.synchronize()
    res = {
        "w": w, "x": x, "p": p, "mask": mask_np, "need_rope": need_rope, "NB": s.NB, "Lp": s.Lp,
        "q_codes": G.unpack_qk_codes(G.host(qk.q_codes)), "k_codes": G.unpack_qk_codes(G.host(qk.k_codes)),
        "q_scale": G.host(qk.q_scale), "k_scale": G.host(qk.k_scale),
        "q_flag": G.host(qk.q_flag), "k_flag": G.host(qk.k_flag), "head_kflag": G.host(qk.head_kflag),
        "q_rope": G.host(qk.q_rope), "k_rope": G.host(qk.k_rope),
        "v_codes": G.decode_v_codes(G.host(vq.v_codes)), "v_scale": G.host(vq.v_scale),
        "v_colsum": G.host(vq.v_colsum), "out": G.host(out).astype(np.float64),
        "dump": {kk: G.host(t) for kk, t in dump.items()},
    }
    res["oracle"] = {}
    for b in range(w.B):
        for h in range(w.H):
            masked = bool(mask_np[b * w.H + h]) if mask_np is not None else False
            # follow the GPU's block flags where the oracle agrees up to the threshold tolerance
            o = G.oracle_head(w, x, b, h, head_masked=masked)
            qf = res["q_flag"][b, h].astype(bool)
            kf = res["k_flag"][b, h].astype(bool)
            if not (np.array_equal(qf, o["q_flags"]) and np.array_equal(kf, o["k_flags"])):
                o = G.oracle_head(w, x, b, h, head_masked=masked, q_flags=qf, k_flags=kf)
            res["oracle"][(b, h)] = o
    _cache[name] = res
    return res


@pytest.mark.parametrize("name", list(CASES))
def test_prologue_parity(name):
    r = _run(name)
    w = r["w"]
    for (b, h), o in r["oracle"].items():
        for t in ("q", "k"):
            assert np.array_equal(r[f"{t}_codes"][b, h], o[t]["codes"]), (t, b, h)
            assert np.array_equal(r[f"{t}_scale"][b, h], o[t]["scale"]), (t, b, h)
            assert G.flags_agree(r[f"{t}_flag"][b, h], o[t]["nsr"], w.tau, w.Dp), (t, b, h)
            assert np.array_equal(r[f"{t}_rope"][b, h], o[t]["rope16"]), (t, b, h)
        assert bool(r["head_kflag"][b * w.H + h]) == bool(r["k_flag"][b, h].any())


@pytest.mark.parametrize("name", list(CASES))
def test_vquant_parity(name):
    r = _run(name)
    for (b, h), o in r["oracle"].items():
        assert np.array_equal(r["v_codes"][b, h], o["v_codes"]), (b, h)
        assert np.array_equal(r["v_scale"][b, h], o["v_scale"]), (b, h)
        assert np.array_equal(r["v_colsum"][b, h], o["v_colsum"]), (b, h)


def _int4_blocks(r):
    """Oracle loop (with its dump) and the P-code check of every INT4 query block of a case (cached)."""
    if "int4" in r:
        return r["int4"]
    w, NB, L = r["w"], r["NB"], r["w"].L
    d = r["dump"]
    out = {}
    for (b, h), o in r["oracle"].items():
        masked = r["mask"] is not None and r["mask"][b * w.H + h]
        qf, kf = o["q_flags"], o["k_flags"]
        for qb in range(NB):
            if masked or qf[qb]:
                continue
            u = (b * w.H + h) * NB + qb
            rows = np.arange(qb * 64, min(qb * 64 + 64, L))
            ref = O.int4_flash_rows(o["q"]["codes"], o["q"]["scale"], o["k"]["codes"], o["k"]["scale"],
                                    o["v_codes"], o["v_scale"], o["v_colsum"], L, w.D, rows,
                                    key_blocks=~kf, dump=True)
            n = rows.size
            keep = np.repeat(~kf, 64)[:L]
            kidx = np.nonzero(keep)[0]
            cq = np.float32(o["q"]["scale"][qb] * O.softmax_c0(w.D))
            c = (cq * o["k"]["scale"][kidx // 64]).astype(np.float32)
            chk = G.check_p_codes(d["pq"][u, :n, :L][:, keep], d["p15"][u, :n, :L][:, keep],
                                  ref["acc"][:, :L][:, keep], c, ref["m_hist"][:, kidx // 64])
            flips = np.zeros((n, L), bool)
            flips[:, keep] = chk["flips"]
            out[(b, h, qb)] = {"u": u, "rows": rows, "ref": ref, "chk": chk, "flips": flips, "keep": keep}
    r["int4"] = out
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_int4_loop_parity(name):
    """Dump of the INT4 kernel (every query block) against the oracle's loop on the same codes and routing.

    Integers (q.k, P.V accumulators) and the running max bitwise; P codes
    equal to the plain quantizer's except at rounding boundaries within the
    derived bound, on at most 1e-4 of the entries; the kernel's float32 15 P
    within the derived bound of the oracle's everywhere.
    """
    r = _run(name)
    d = r["dump"]
    L = r["w"].L
    total = mism = 0
    exp_err = 0.0
    for (b, h, qb), e in _int4_blocks(r).items():
        kf = r["oracle"][(b, h)]["k_flags"]
        u, ref, keep, n = e["u"], e["ref"], e["keep"], e["rows"].size
        assert np.array_equal(d["acc"][u, :n, :L][:, keep], ref["acc"][:, :L][:, keep]), (b, h, qb)
        mh = d["m"][u, :n]
        dm = np.argwhere(mh[:, ~kf] != ref["m_hist"][:, ~kf])
        assert dm.size == 0, (b, h, qb, dm[:6].tolist())
        total += e["chk"]["entries"]
        mism += e["chk"]["mismatch"]
        exp_err = max(exp_err, e["chk"]["exp_err"])
        same_rows = ~e["flips"].any(axis=1)
        pv = d["accpv"][u, :n][same_rows][:, ~kf]
        assert np.array_equal(pv, ref["accpv"][same_rows][:, ~kf]), (b, h, qb)
    print(f"[gpu] {name}: P codes {mism} of {total} differ at boundaries; device 2^x max rel err {exp_err:.3g}")
    assert mism <= 1e-4 * max(total, 1), (mism, total)


@pytest.mark.parametrize("name", list(CASES))
def test_forward_parity(name):
    """Final fp16 output of rotattn_forward against the oracle, to the derived per-element tolerance.

    The tolerance (gpu_common.head_output_tol) comes from the oracle alone:
    every key whose 15 P lies within the derived bound of a rounding
    boundary may move its code by one step. The P-code check of
    test_int4_loop_parity confirms the kernel's flips are among those keys.
    """
    r = _run(name)
    w = r["w"]
    blocks = _int4_blocks(r)
    for (b, h), o in r["oracle"].items():
        masked = r["mask"] is not None and bool(r["mask"][b * w.H + h])
        tol = G.head_output_tol(w, r["x"], b, h, o, masked)
        err = np.abs(r["out"][b, h] - o["out"])
        bad = err > tol
        assert not bad.any(), (b, h, float(err.max()), np.argwhere(bad)[:5].tolist(),
                               [(float(err[i, j]), float(tol[i, j])) for i, j in np.argwhere(bad)[:5]])
    flipped = sum(int(e["flips"].any(axis=1).sum()) for e in blocks.values())
    print(f"[gpu] {name}: {flipped} rows carry a P-code boundary flip")


@pytest.mark.parametrize("name", ["tiny", "d64_prefix", "ragged_prefix"])
def test_fp16_forward_parity(name):
    """Whole-call FP16 path (RoPE, no rotation or quantization) against exact float64 attention on the fp16-rounded RoPE'd inputs."""
    G.require_gpu()
    w = CASES[name]
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    out = G.host(G.R.rotattn_fp16_forward(p, G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"]))).astype(np.float64)
    for b in range(w.B):
        for h in range(w.H):
            qr = O.apply_rope(x["q"][b, h].astype(np.float32), w.prefix, w.grid, w.split, w.base).astype(np.float16)
            kr = O.apply_rope(x["k"][b, h].astype(np.float32), w.prefix, w.grid, w.split, w.base).astype(np.float16)
            rows = np.arange(w.L)
            pp, bound = G.fp16_weight_bound(qr, kr, x["v"][b, h], w.L, w.D, rows)
            ref = pp["O"] / pp["l"][:, None]
            tol = G.ATOL + G.RTOL * np.abs(ref) + bound
            assert (np.abs(out[b, h] - ref) <= tol).all(), (b, h, np.abs(out[b, h] - ref).max())


def test_all_heads_masked_equals_fp16_forward():
    """A head mask of all ones routes every tile to FP16: identical bits to the whole-call FP16 forward."""
    G.require_gpu()
    w = CASES["ragged_prefix"]
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    q, k, v = G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"])
    qk = G.R.rotattn_quantize_qk(p, q, k, rope_copy=True)
    mask = torch.ones(w.B * w.H, dtype=torch.uint8, device="cuda")
    a = G.host(G.R.rotattn_forward(p, qk, v, head_fallback=mask))
    bb = G.host(G.R.rotattn_fp16_forward(p, q, k, v))
    assert np.array_equal(a.view(np.uint16), bb.view(np.uint16))


def test_tau_zero_equals_fp16_forward():
    """tau = 0 flags every block with any energy, so every row runs whole on FP16 through the Q flags (the
    routing path, not the head mask): identical bits to the whole-call FP16 forward."""
    G.require_gpu()
    w = CASES["ragged_prefix"]
    x = W.full_inputs(w)
    q, k, v = G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"])
    p = G.R.problem_from_workload(w, tau=0.0)
    qk = G.R.rotattn_quantize_qk(p, q, k, rope_copy=True)
    assert G.host(qk.q_flag).all() and G.host(qk.k_flag).all()
    a = G.host(G.R.rotattn_forward(p, qk, v))
    bb = G.host(G.R.rotattn_fp16_forward(G.R.problem_from_workload(w), q, k, v))
    assert np.array_equal(a.view(np.uint16), bb.view(np.uint16))


def test_routing_without_flags_equals_unrouted():
    """A finite tau that flags nothing switches block routing on (the routed INT4 instance, the side stream)
    with nothing to route: identical bits to the call with routing off."""
    G.require_gpu()
    w = CASES["ragged_prefix"]
    x = W.full_inputs(w)
    q, k, v = G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"])
    p_on = G.R.problem_from_workload(w, tau=1e30)
    qk_on = G.R.rotattn_quantize_qk(p_on, q, k, rope_copy=True)
    assert not G.host(qk_on.q_flag).any() and not G.host(qk_on.k_flag).any()
    a = G.host(G.R.rotattn_forward(p_on, qk_on, v))
    p_off = G.R.problem_from_workload(w)
    b_ = G.host(G.R.rotattn_forward(p_off, G.R.rotattn_quantize_qk(p_off, q, k), v))
    assert np.array_equal(a.view(np.uint16), b_.view(np.uint16))


def test_determinism():
    """Two runs give bitwise-equal outputs and dumps."""
    G.require_gpu()
    w = CASES["mixed"]
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    q, k, v = G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"])
    mask = G.dev(W.head_fallback_mask(w))
    outs = []
    for _ in range(2):
        qk = G.R.rotattn_quantize_qk(p, q, k, rope_copy=True)
        outs.append(G.host(G.R.rotattn_forward(p, qk, v, head_fallback=mask)).view(np.uint16))
    assert np.array_equal(outs[0], outs[1])
