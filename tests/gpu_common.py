"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI, decode its layouts, and compare with the oracle."""
from __future__ import annotations

import math

import numpy as np
import pytest

import workloads as W
from oracle import core as O

torch = pytest.importorskip("torch")

import int4_quantized_flashattention_amd as R  # noqa: E402

# Output tolerance against the oracle's float64 result: the 2e-3 absolute bar
# plus the float16 output's own rounding (half an ulp, 2^-11 of the value);
# the tests add the derived float32 accumulation and P-rounding terms below.
ATOL = 2e-3
RTOL = 2.0 ** -11
U32 = 2.0 ** -24                                  # unit roundoff of float32
# relative error allowed for the device's 2^x (v_exp_f32); the tests measure
# the actual error on every element they dump and check it against this
EXP2_REL = 2.0 ** -22
LOG2_15_F32 = np.float32(math.log2(15.0))
LOG2_15_ERR = abs(float(LOG2_15_F32) - math.log2(15.0))


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


def nsr_rel_bound(Dp: int) -> float:
    """Relative error bound of the prologue's float32 NSR against the oracle's float64 one.

    Each thread sums 32 * ceil(Dp / 128) terms of one token chunk per round
    with fused multiply-adds (each residual x - s c is rounded once, so a
    squared term carries at most 2 roundings), then a workgroup tree of 8
    additions: each of the two sums is within (32 ceil(Dp / 128) + 10) 2^-24
    of its value relative (first-order bound for sums of positive terms),
    and the quotient adds one rounding.
    """
    return (2 * (32 * -(-Dp // 128) + 10) + 4) * U32


def flags_agree(gpu_flags, nsr, tau, Dp):
    """Block flags equal NSR > tau except where NSR sits within the derived float32 bound of tau."""
    want = nsr > tau
    near = np.abs(nsr - tau) <= nsr_rel_bound(Dp) * max(tau, 0.0) * 1.01
    return bool(np.all((gpu_flags.astype(bool) == want) | near))


def fp16_weight_bound(qr16, kr16, v16, L, D, rows, key_blocks=None):
    """Derived bound on the FP16 path's float arithmetic, per output element (beyond 2e-3 + 2^-11 |ref|).

    Against exact float64 attention on the same fp16 inputs, the kernel
      - rounds each weight P_j / l to fp16 for the P.V product: relative
        2^-11 (absolute 2^-25 in the fp16 subnormal range), so the output
        moves by at most 2^-11 W + 2^-25 sum_j |v_j| / l with
        W = sum_j (P_j / l) |v_j|;
      - forms each score q.k in float32 from exact fp16 products (D - 1
        additions), scales it and subtracts the running max (two more
        roundings): the exponent is off by at most
        eps_j = (D + 2) 2^-24 c0 sum_d |q_d k_jd| + 2^-23 (|S2_j| + |m|), and
        2^x on the device adds a relative EXP2_REL, so P_j is off by a
        factor within 1 + e_j, e_j = 2^eps_j (1 + EXP2_REL) - 1; that moves O
        by sum_j P_j e_j |v_j| / l and l by sum_j P_j e_j / l relative;
      - accumulates O and l in float32 over nvis key blocks: at most
        (3 nvis + 40) 2^-24 W.
    Returns (the oracle's exact partial, the bound [R, D]).
    """
    p = O.fp16_rows(qr16, kr16, v16, L, D, rows, key_blocks)
    nb = O.n_blocks(L)
    kb = np.ones(nb, bool) if key_blocks is None else key_blocks
    nvis = int(np.count_nonzero(kb))
    keys = np.nonzero(np.repeat(kb, 64)[:L])[0]
    q = qr16[rows].astype(np.float64)
    k = kr16[keys].astype(np.float64)
    va = np.abs(v16[keys].astype(np.float64))
    c0 = math.log2(math.e) / math.sqrt(D)
    S2 = (q @ k.T) * c0
    P = np.exp2(S2 - p["m"][:, None])
    l = p["l"][:, None]
    W = (P @ va) / l
    eps = (D + 2) * U32 * c0 * (np.abs(q) @ np.abs(k).T) + 2 * U32 * (np.abs(S2) + np.abs(p["m"])[:, None])
    e = np.exp2(eps) * (1 + EXP2_REL) - 1
    Pe = P * e
    bound = (2.0 ** -11 * W + 2.0 ** -25 * va.sum(0)[None, :] / l + (Pe @ va) / l + (Pe.sum(1)[:, None] / l) * W
             + (3 * nvis + 40) * U32 * W)
    return p, bound


def half_ulp(x32) -> np.ndarray:
    """Upper bound of half an ulp of each float32 value (the rounding error of a result rounded to it)."""
    return np.spacing(np.abs(np.asarray(x32, dtype=np.float32))).astype(np.float64) / 2


def p15_plain_and_bound(acc, c, m):
    """The oracle's float32 15 P of every score, the kernel's exponent argument, and a bound on their gap.

    acc: exact integer q.k [R, K]; c: float32 softmax factor of each key's
    block [K]; m: float32 running max (after the key's block) [R, K], the same
    bits on both sides (the dump tests check it).
    Oracle (the plain quantizer): S2 = fl(acc c), d = fl(S2 - m),
    P = fl(2^d), X = fl(15 P). Kernel: m15 = fl(m - fl(log2 15)),
    t = fl(acc c - m15) (one fused multiply-add), Y = exp2(t) on the device.
    Writing every rounding as an error term, log2 Y - log2 X is at most
      Delta = |fl(log2 15) - log2 15| + hu(m15) + hu(t) + hu(S2) + hu(d)
    (hu = half an ulp of the rounded value) plus the relative errors of P,
    of 15 P and of the device's 2^x, so
      |Y - X| <= B = X (2^Delta (1 + EXP2_REL) / (1 - 2^-24)^2 - 1) + 2^-126
    (the last term: results in the float32 subnormal range, which the device
    may flush to zero; far below any rounding boundary of a code).
    Returns (X float32, t float32, B float64, rel float64), all [R, K]; rel
    is the relative part of the bound, (B - 2^-126) / X.
    """
    x = np.asarray(acc, dtype=np.float64).astype(np.float32).astype(np.float64) * np.asarray(c, np.float32).astype(np.float64)
    m = np.asarray(m, dtype=np.float32)
    s2 = x.astype(np.float32)
    d = (s2 - m).astype(np.float32)
    X = (np.float32(15.0) * O.exp2_f32(d)).astype(np.float32)
    m15 = (m - LOG2_15_F32).astype(np.float32)
    t = (x - m15.astype(np.float64)).astype(np.float32)
    with np.errstate(invalid="ignore"):
        delta = LOG2_15_ERR + half_ulp(m15) + half_ulp(t) + half_ulp(s2) + half_ulp(d)
        rho = np.exp2(delta) * (1 + EXP2_REL) / (1 - U32) ** 2
        rel = (rho - 1) * 1.001
        B = X.astype(np.float64) * rel + 2.0 ** -126
    return X, t, B, np.where(np.isfinite(rel), rel, 0.0)


def check_p_codes(gpu_pq, gpu_p15, acc, c, m, valid=None):
    """P codes of the kernel against the plain quantizer rne(fl(15 P)) - 8 of the oracle.

    Every code must be equal, or differ by one where the rounding boundary
    between the two codes lies within B (p15_plain_and_bound) of the oracle's
    15 P. With the kernel's own float32 15 P (gpu_p15) also checked: it lies
    within B of the oracle's everywhere, its codes are its rne exactly, and
    the device's 2^x stays within EXP2_REL of the exact 2^t.
    Returns a dict: mismatch (count), entries (count), exp_err (max relative
    error of the device 2^x), flips (bool [R, K] where the codes differ) and
    eta (per row, the largest relative gap B / X the bound allows between the
    two 15 P; it bounds the relative gap of the two row sums l).
    """
    X, t, B, relb = p15_plain_and_bound(acc, c, m)
    gpu_pq = np.asarray(gpu_pq).astype(np.int64)
    want = np.rint(X.astype(np.float64)).astype(np.int64) - 8
    if valid is None:
        valid = np.ones(X.shape, bool)
    valid = np.broadcast_to(valid, X.shape)
    diff = np.where(valid, gpu_pq - want, 0)
    bad = diff != 0
    assert np.abs(diff).max(initial=0) <= 1, "P code off by more than one step"
    if bad.any():
        boundary = np.minimum(gpu_pq, want)[bad] + 8 + 0.5
        gap = np.abs(X[bad].astype(np.float64) - boundary)
        assert np.all(gap <= B[bad]), ("P code differs away from a rounding boundary",
                                       float((gap - B[bad]).max()))
    exp_err = 0.0
    if gpu_p15 is not None:
        Y = np.asarray(gpu_p15, dtype=np.float32).astype(np.float64)
        assert np.array_equal(np.where(valid, np.rint(Y).astype(np.int64) - 8, 0), np.where(valid, gpu_pq, 0)), \
            "P code is not rne of the kernel's 15 P"
        gap = np.abs(Y - X.astype(np.float64))
        assert np.all(~valid | (gap <= B)), ("kernel's 15 P outside the derived bound", float(np.max(np.where(valid, gap - B, -1))))
        ok = valid & (t.astype(np.float64) >= -100)
        if ok.any():
            ex = np.exp2(t.astype(np.float64)[ok])
            exp_err = float(np.max(np.abs(Y[ok] - ex) / ex))
            assert exp_err <= EXP2_REL, ("device 2^x error", exp_err)
    rel = np.where(valid, relb, 0.0)
    return {"mismatch": int(bad.sum()), "entries": int(valid.sum()), "exp_err": exp_err, "flips": bad,
            "eta": rel.max(axis=1, initial=0.0)}


def int4_output_tol(ref_out, od, sv, nvis, eta, flips=None, vcodes=None):
    """Per-element tolerance of INT4 rows against the oracle, derived from the arithmetic.

    ref_out [R, D]: the oracle's output of the rows (merged when the row also
    has FP16 tiles). od: the oracle's int4_flash_rows(dump=True) of the
    rows. A_c = sum_j 2^(m_j - m) |accPV_jc| s_v,c / (15 l) bounds the INT4
    part of the output and the float32 values it is summed from. Terms:
      2e-3 + 2^-11 |ref|                the stated bar and the fp16 output rounding
      ((5 nvis + 32) 2^-24 + eta) A_c   float32 accumulation of O and l over
                                        nvis key blocks (first-order recursive
                                        summation bound) and the row's largest
                                        relative gap eta between the kernel's
                                        and the oracle's P (check_p_codes), in l
      flips: sum over keys whose P code differs by one of
             2^(m_j - m) |cv_kc| s_v,c / (15 l)   (one code step each).
    """
    m_hist = od["m_hist"].astype(np.float64)            # [R, nb]
    m_fin = od["m"].astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        alpha = np.where(np.isneginf(m_hist), 0.0, np.exp2(m_hist - m_fin[:, None]))   # [R, nb]
    scale = sv.astype(np.float64)[None, :] / (15.0 * od["l"][:, None])              # [R, D]
    A = np.einsum("rj,rjd->rd", alpha, np.abs(od["accpv"].astype(np.float64))) * scale
    tol = ATOL + RTOL * np.abs(ref_out) + ((5 * nvis + 32) * U32 + np.asarray(eta)[:, None]) * A
    if flips is not None and flips.any():
        fa = np.repeat(alpha, 64, axis=1)[:, :flips.shape[1]] * flips        # [R, K]
        tol = tol + (fa @ np.abs(vcodes[:flips.shape[1]].astype(np.float64))) * scale
    return tol


def flip_candidates(od, c_of_key, keys):
    """Keys of each row whose P code may legitimately differ between kernel and oracle.

    From the oracle alone: those whose 15 P lies within the derived bound B
    of a rounding boundary k + 1/2. Returns (bool [R, K], eta [R]).
    """
    X, _, B, rel = p15_plain_and_bound(od["acc"][:, keys], c_of_key, od["m_hist"][:, keys // 64])
    Xd = X.astype(np.float64)
    near = (np.abs(Xd - np.floor(Xd) - 0.5) <= B) & (Xd >= 0.5 - B)
    return near, rel.max(axis=1, initial=0.0)


def int4_rows_tol(w, o, rows, ref_out, key_blocks):
    """Derived tolerance (int4_output_tol) of INT4 rows of one head, with every flip candidate allowed one step."""
    L, nb = w.L, O.n_blocks(w.L)
    od = O.int4_flash_rows(o["q"]["codes"], o["q"]["scale"], o["k"]["codes"], o["k"]["scale"], o["v_codes"],
                           o["v_scale"], o["v_colsum"], L, w.D, rows, key_blocks=key_blocks, dump=True)
    keys = np.nonzero(np.repeat(key_blocks, 64)[:L])[0]
    tol = np.zeros_like(ref_out) + ATOL + RTOL * np.abs(ref_out)
    qb_of = rows // 64
    for qb in np.unique(qb_of):
        sel = qb_of == qb
        cq = np.float32(o["q"]["scale"][qb] * O.softmax_c0(w.D))
        c = (cq * o["k"]["scale"][keys // 64]).astype(np.float32)
        sub = {kk: od[kk][sel] for kk in ("acc", "m_hist", "accpv", "l", "m")}
        near, eta = flip_candidates(sub, c, keys)
        flips = np.zeros((int(sel.sum()), L), bool)
        flips[:, keys] = near
        tol[sel] = int4_output_tol(ref_out[sel], sub, o["v_scale"], int(np.count_nonzero(key_blocks)), eta,
                                   flips=flips, vcodes=o["v_codes"])
    return tol


def head_output_tol(w, x, b, h, o, masked, rows=None):
    """Derived per-element tolerance of one head's output against the oracle's (o = oracle_head(...)).

    Rows that run whole on the FP16 path: the bar plus fp16_weight_bound over
    every key. INT4 rows: int4_rows_tol, plus fp16_weight_bound over the
    flagged key blocks when the row mixes both paths.
    """
    L = w.L
    rows = np.arange(L) if rows is None else np.asarray(rows)
    ref = o["out"]
    qf, kf = o["q_flags"], o["k_flags"]
    fp16 = masked | qf[rows // 64]
    tol = ATOL + RTOL * np.abs(ref)
    v16 = x["v"][b, h]
    if fp16.any():
        _, bound = fp16_weight_bound(o["q"]["rope16"], o["k"]["rope16"], v16, L, w.D, rows[fp16])
        tol[fp16] += bound
    if (~fp16).any():
        r4 = rows[~fp16]
        tol[~fp16] = int4_rows_tol(w, o, r4, ref[~fp16], ~kf)
        if kf.any():
            _, bound = fp16_weight_bound(o["q"]["rope16"], o["k"]["rope16"], v16, L, w.D, r4, key_blocks=kf)
            tol[~fp16] += bound
    return tol

