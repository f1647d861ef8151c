"""Block-sparse path on the GPU against the oracle (RainFusion2.0 sections 3.1, 3.2 and 3.4).

rotattn_block_mask (query blocks of 128 rows, key blocks of 64) is checked
against the oracle's float64 block scores: the sink rows and columns are
kept, every key block scoring clearly above the query block's n-th largest
score is kept, every one clearly below is dropped (near-ties may go either
way: the GPU ranks float32 scores). The block-sparse INT4 loop is then
checked with the GPU's own mask: bit-exact integers on the kept blocks of
sampled 64-row blocks (first, first past the sink, middle, last), P codes
equal to the plain quantizer's up to the derived rounding-boundary window,
and outputs within the derived tolerance.
"""
import numpy as np
import pytest

import workloads as W
from oracle import core as O
from tests import gpu_common as G

torch = G.torch
pytestmark = pytest.mark.gpu


def _sinks(w):
    se = O.sink_end(w.L, w.prefix, w.grid)
    return -(-se // O.SPARSE_BQ), -(-se // O.SPARSE_BK)


def _check_mask(sel, s_hat, topn, nsr, ns):
    """One head's GPU mask (bool [NBq, NB]) against the oracle's scores."""
    NQ, NB = s_hat.shape
    assert sel.shape == (NQ, NB)
    assert sel[:nsr].all() and sel[:, :ns].all()
    n = min(topn, NB)
    for i in range(nsr, NQ):
        row = s_hat[i]
        t = np.sort(row)[::-1][n - 1]
        eps = 1e-4 * (np.abs(row).max() + 1e-6)
        must = row > t + eps
        never = row < t - eps
        never[:ns] = False
        assert sel[i][must].all(), i
        assert not sel[i][never].any(), i
        cnt = int(sel[i].sum())
        assert max(n, ns) <= cnt <= n + ns, (i, cnt)


def _compare_blocks(w, x, h, gsel, qbs, out_gpu, dump, unit0, L, D):
    """Integers and outputs of query blocks qbs of head h against the oracle run with the GPU mask."""
    o = O.sparse_forward_head(x["q"][0, h], x["k"][0, h], x["v"][0, h], prefix=w.prefix, grid=w.grid,
                              split=w.split, base=w.base, rotation=w.rotation, topn=1, block_mask=gsel,
                              rows=np.concatenate([np.arange(qb * 64, min(L, qb * 64 + 64)) for qb in qbs]))
    total = mism = 0
    for bi, qb in enumerate(qbs):
        rr = np.arange(qb * 64, min(L, qb * 64 + 64))
        n = rr.size
        kb = gsel[qb * 64 // O.SPARSE_BQ]
        ref = O.int4_flash_rows(o["q"]["codes"], o["q"]["scale"], o["k"]["codes"], o["k"]["scale"], o["v_codes"],
                                o["v_scale"], o["v_colsum"], L, D, rr, key_blocks=kb, dump=True)
        u = unit0 + bi
        keep = np.repeat(kb, 64)[:L]
        assert np.array_equal(dump["acc"][u, :n, :L][:, keep], ref["acc"][:, :L][:, keep]), (h, qb)
        assert np.array_equal(dump["m"][u, :n][:, kb], ref["m_hist"][:, kb]), (h, qb)
        kidx = np.nonzero(keep)[0]
        cq = np.float32(o["q"]["scale"][qb] * O.softmax_c0(D))
        c = (cq * o["k"]["scale"][kidx // 64]).astype(np.float32)
        chk = G.check_p_codes(dump["pq"][u, :n, :L][:, keep], dump["p15"][u, :n, :L][:, keep],
                              ref["acc"][:, :L][:, keep], c, ref["m_hist"][:, kidx // 64])
        total += chk["entries"]
        mism += chk["mismatch"]
        same = ~chk["flips"].any(axis=1)
        assert np.array_equal(dump["accpv"][u, :n][same][:, kb], ref["accpv"][same][:, kb]), (h, qb)
        want = ref["O_scaled"] / ref["l"][:, None]
        flips = np.zeros((n, L), bool)
        flips[:, keep] = chk["flips"]
        tol = G.int4_output_tol(want, ref, o["v_scale"], int(np.count_nonzero(kb)), chk["eta"], flips=flips,
                                vcodes=o["v_codes"])
        err = np.abs(out_gpu[rr] - want)
        bad = err > tol
        assert not bad.any(), (h, qb, float(err.max()))
    return total, mism


def _sparse_tol(w, o, rows, M):
    """Derived tolerance (gpu_common.int4_rows_tol) of sparse rows, per 128-row query block of mask M."""
    tol = np.zeros_like(o["out"])
    qb = rows // O.SPARSE_BQ
    for i in np.unique(qb):
        sel = qb == i
        tol[sel] = G.int4_rows_tol(w, o, rows[sel], o["out"][sel], M[i])
    return tol


CASES = [("tiny", {}, 2), ("smalld", dict(H=2), 56), ("480p", dict(H=2), 102),
         ("smalld", dict(H=2, split=(22, 22, 20)), 56),   # even groups: block sums from the register prologue
         ("tiny", dict(rotation=W.ROT_PAIR, grid=(3, 9, 15), prefix=5), 3)]   # mergeable rotation, ragged


@pytest.mark.parametrize("name,kw,topn", CASES)
def test_sparse_mask_and_attention(name, kw, topn):
    G.require_gpu()
    w = W.WORKLOADS[name].replace(**kw)
    print(f"[gpu] sparse {name} H={w.H} L={w.L} D={w.D} topn={topn}", flush=True)
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    s = G.R.get_sizes(p)
    NB, L, D = s.NB, w.L, w.D
    q, k, v = (G.dev(x[t]) for t in ("q", "k", "v"))
    qk = G.R.rotattn_quantize_qk(p, q, k, block_sums=True)
    vq = G.R.rotattn_quantize_v(p, v)
    mask = G.R.rotattn_block_mask(p, qk, topn)
    out = G.R.rotattn_sparse_attention(p, qk, vq, mask)
    mw = G.host(mask).astype(np.uint32)
    assert mw.shape == (1, w.H, s.mask_rows, s.mask_words) and s.mask_rows == -(-NB // 2)
    gm = G.R.mask_to_bool(mw, NB)
    tail = NB % 32
    if tail:
        assert not (mw[..., -1] >> np.uint32(tail)).any()   # no bits at or beyond NB
    nsr, ns = _sinks(w)
    qbs = sorted({0, min(2 * nsr, NB - 1), NB // 2, NB - 1})
    units = np.array([h * NB + qb for h in range(w.H) for qb in qbs], dtype=np.int32)
    dump = G.R.rotattn_debug_dump(p, qk, vq, G.dev(units), block_mask=mask)
    torch.cuda.synchronize()
    dump = {kk: t.cpu().numpy() for kk, t in dump.items()}
    out_np = G.host(out).astype(np.float64)
    total = mism = 0
    cnt = np.minimum(64, L - 64 * np.arange(NB)).astype(np.float64)[:, None]
    for h in range(w.H):
        # block sums of the RoPE'd rows from the Q/K prologue
        # (with the mergeable rotation, of the RoPE'd rows with the pair rotation folded in, as the
        # prologue holds them; S_hat is the same, the rotation being orthogonal and shared by Q and K)
        phase = O.pair_phase() if w.rotation == W.ROT_PAIR else 0.0
        for t in ("q", "k"):
            r32 = O.apply_rope(x[t][0, h].astype(np.float32), w.prefix, w.grid, w.split, w.base, phase)
            want = np.add.reduceat(r32.astype(np.float64), np.arange(0, L, 64), axis=0)
            xr = np.abs(r32)
            bound = 64 * 2.0 ** -23 * np.add.reduceat(xr.astype(np.float64), np.arange(0, L, 64), axis=0)
            got = G.host(getattr(qk, f"{t}_bsum")[0, h]).astype(np.float64)
            assert (np.abs(got - want) <= bound + 1e-30).all(), (h, t)
        s_hat = O.block_scores(O.block_means(x["q"][0, h], w.prefix, w.grid, w.split, w.base, O.SPARSE_BQ),
                               O.block_means(x["k"][0, h], w.prefix, w.grid, w.split, w.base, O.SPARSE_BK))
        _check_mask(gm[0, h], s_hat, topn, nsr, ns)
        t, m = _compare_blocks(w, x, h, gm[0, h], qbs, out_np[0, h], dump, h * len(qbs), L, D)
        total += t
        mism += m
    assert mism <= 1e-4 * max(total, 1), (mism, total)


def test_sparse_full_mask_equals_dense():
    """topn >= NB keeps every block: the block-sparse kernel gives the dense kernel's output bit for bit."""
    G.require_gpu()
    w = W.WORKLOADS["smalld"].replace(H=2)
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    NB = G.R.get_sizes(p).NB
    q, k, v = (G.dev(x[t]) for t in ("q", "k", "v"))
    qk = G.R.rotattn_quantize_qk(p, q, k, block_sums=True)
    vq = G.R.rotattn_quantize_v(p, v)
    mask = G.R.rotattn_block_mask(p, qk, NB + 5)
    assert G.R.mask_to_bool(G.host(mask).astype(np.uint32), NB).all()
    sparse = G.R.rotattn_sparse_attention(p, qk, vq, mask)
    dense = G.R.rotattn_attention(p, qk, vq)
    assert torch.equal(sparse, dense)


@pytest.mark.parametrize("sel", [
    [[0, 0, 0, 0], [0, 0, 0, 1]],      # an empty query block (zeros); one that keeps only the ragged last block
    [[1, 0, 1, 1], [0, 1, 0, 1]],      # scattered blocks
])
def test_sparse_custom_mask_edges(sel):
    """A caller's mask, against the oracle with the same mask; a query block that keeps no key block gets zeros."""
    G.require_gpu()
    w = W.WORKLOADS["tiny"].replace(grid=(4, 8, 7))        # L = 224: NB = 4, last key block 32 keys
    sel = np.array(sel, dtype=bool)
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    s = G.R.get_sizes(p)
    NB, L = s.NB, w.L
    assert sel.shape == (s.mask_rows, NB)
    words = np.zeros((1, w.H, s.mask_rows, s.mask_words), dtype=np.uint32)
    for i in range(s.mask_rows):
        for j in range(NB):
            if sel[i, j]:
                words[0, :, i, j // 32] |= np.uint32(1 << (j % 32))
    mask = G.dev(words.view(np.int32))
    q, k, v = (G.dev(x[t]) for t in ("q", "k", "v"))
    qk = G.R.rotattn_quantize_qk(p, q, k)
    vq = G.R.rotattn_quantize_v(p, v)
    out = G.host(G.R.rotattn_sparse_attention(p, qk, vq, mask)).astype(np.float64)
    for h in range(w.H):
        rows = []
        for i in range(s.mask_rows):
            rr = np.arange(128 * i, min(L, 128 * i + 128))
            if sel[i].any():
                rows.append(rr)
            else:
                assert (out[0, h, rr] == 0).all()
        rows = np.concatenate(rows)
        o = O.sparse_forward_head(x["q"][0, h], x["k"][0, h], x["v"][0, h], prefix=w.prefix, grid=w.grid,
                                  split=w.split, base=w.base, rotation=w.rotation, topn=1, block_mask=sel,
                                  rows=rows)
        err = np.abs(out[0, h, rows] - o["out"])
        assert (err <= _sparse_tol(w, o, rows, sel)).all(), float(err.max())


def test_sparse_strided_batch():
    """B = 2 with tokens-major [B, L, H, D] storage, D = 64, a text prefix and a ragged last block: the mask and
    every output row against the oracle (run with the GPU's mask after checking it)."""
    G.require_gpu()
    w = W.WORKLOADS["smalld"].replace(B=2, H=3, grid=(3, 10, 20), prefix=9)     # L = 609, NB = 10, 5 mask rows
    x = W.full_inputs(w)
    B, H, L, D = w.B, w.H, w.L, w.D
    topn = 2

    def put(a):
        return torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3))).cuda().permute(0, 2, 1, 3)
    p = G.R.problem_from_workload(w, strides=(L * H * D, D, H * D))
    s = G.R.get_sizes(p)
    q, k, v = put(x["q"]), put(x["k"]), put(x["v"])
    out = torch.empty((B, L, H, D), dtype=torch.float16, device="cuda").permute(0, 2, 1, 3)
    qk = G.R.rotattn_quantize_qk(p, q, k, block_sums=True)
    vq = G.R.rotattn_quantize_v(p, v)
    mask = G.R.rotattn_block_mask(p, qk, topn)
    G.R.rotattn_sparse_attention(p, qk, vq, mask, out=out)
    gm = G.R.mask_to_bool(G.host(mask).astype(np.uint32), s.NB)
    got = G.host(out).astype(np.float64)
    nsr, ns = _sinks(w)
    assert (nsr, ns) == (2, 4)
    for b in range(B):
        for h in range(H):
            s_hat = O.block_scores(O.block_means(x["q"][b, h], w.prefix, w.grid, w.split, w.base, O.SPARSE_BQ),
                                   O.block_means(x["k"][b, h], w.prefix, w.grid, w.split, w.base, O.SPARSE_BK))
            _check_mask(gm[b, h], s_hat, topn, nsr, ns)
            o = O.sparse_forward_head(x["q"][b, h], x["k"][b, h], x["v"][b, h], prefix=w.prefix, grid=w.grid,
                                      split=w.split, base=w.base, rotation=w.rotation, topn=topn,
                                      block_mask=gm[b, h])
            err = np.abs(got[b, h] - o["out"])
            assert (err <= _sparse_tol(w, o, np.arange(L), gm[b, h])).all(), (b, h, float(err.max()))
