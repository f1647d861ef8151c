"""Edge cases of the HIP path against the oracle: tiny and ragged lengths, text-only
sequences, strided layouts with B > 1, degenerate inputs, the empty problem and
the dump hook's bounds handling."""
import numpy as np
import pytest

import workloads as W
from oracle import core as O
from tests import gpu_common as G

torch = G.torch
pytestmark = pytest.mark.gpu


def _run_and_check(w, x, layout="bhld", tau=None, head_mask=None):
    """quantize_qk + forward through the C ABI; check codes and outputs against the oracle for every head."""
    B, H, L, D = w.B, w.H, w.L, w.D
    if layout == "blhd":   # [B, L, H, D] storage viewed as [B, H, L, D]
        def put(a):
            return torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3))).cuda().permute(0, 2, 1, 3)
        strides = (L * H * D, D, H * D)
        out = torch.empty((B, L, H, D), dtype=torch.float16, device="cuda").permute(0, 2, 1, 3)
    else:
        def put(a):
            return G.dev(a)
        strides = None
        out = torch.empty((B, H, L, D), dtype=torch.float16, device="cuda")
    q, k, v = put(x["q"]), put(x["k"]), put(x["v"])
    p = G.R.problem_from_workload(w, strides=strides, tau=tau)
    need_rope = head_mask is not None or (tau is not None and np.isfinite(tau))
    qk = G.R.rotattn_quantize_qk(p, q, k, rope_copy=need_rope)
    m = G.dev(head_mask) if head_mask is not None else None
    G.R.rotattn_forward(p, qk, v, head_fallback=m, out=out)
    got = G.host(out).astype(np.float64)
    qc = G.unpack_qk_codes(G.host(qk.q_codes))
    for b in range(B):
        for h in range(H):
            masked = head_mask is not None and bool(head_mask[b * H + h])
            o = G.oracle_head(w, x, b, h, tau=tau, head_masked=masked,
                              q_flags=G.host(qk.q_flag)[b, h].astype(bool),
                              k_flags=G.host(qk.k_flag)[b, h].astype(bool))
            assert np.array_equal(qc[b, h], o["q"]["codes"]), (b, h)
            tol = G.head_output_tol(w, x, b, h, o, masked)
            err = np.abs(got[b, h] - o["out"])
            assert (err <= tol).all(), (b, h, float(err.max()))
    return got


@pytest.mark.parametrize("grid,prefix", [((1, 1, 1), 0), ((1, 8, 8), 0), ((1, 5, 13), 0), ((0, 0, 0), 100),
                                         ((1, 1, 3), 61)])
def test_lengths(grid, prefix):
    """L = 1, one full block, one block plus one token, a text-only sequence, a block boundary inside the prefix."""
    G.require_gpu()
    w = W.WORKLOADS["tiny"].replace(grid=grid, prefix=prefix)
    _run_and_check(w, W.full_inputs(w))


def test_strided_batch_layout():
    """B = 2 with tokens-major [B, L, H, D] storage (non-dense strides), D = 64, text prefix."""
    G.require_gpu()
    w = W.WORKLOADS["smalld"].replace(B=2, H=3, grid=(2, 3, 17), prefix=9)
    _run_and_check(w, W.full_inputs(w), layout="blhd")


def test_degenerate_inputs():
    """Q = 0 (every P = 1), an all-zero K block (scale 0), negative scores everywhere (K = -Q)."""
    G.require_gpu()
    w = W.WORKLOADS["tiny"].replace(H=3, grid=(1, 10, 20))
    x = W.full_inputs(w)
    x["q"][:, 0] = 0
    x["k"][:, 1, 64:128] = 0
    x["k"][:, 2] = -x["q"][:, 2]
    _run_and_check(w, x)


def test_mask_and_block_rule_small():
    """Head mask and the 5% block rule together at a small size, against the oracle's routing."""
    G.require_gpu()
    w = W.WORKLOADS["mixed"].replace(H=4, grid=(3, 7, 9))
    x = W.full_inputs(w)
    # plant a high-norm token so that one K block is flagged for sure
    x["k"][0, 1, 70] *= np.float16(12)
    mask = np.array([0, 0, 1, 0], dtype=np.uint8)
    _run_and_check(w, x, tau=0.05, head_mask=mask)


def test_routing_strided_batch():
    """The mask and the block rule with B = 2 in tokens-major [B, L, H, D] storage: masked heads in both batch
    entries, planted high-norm key tokens flagging K blocks in a head of the second entry (its rows mix both
    paths) and a flagged Q block in the first; every head against the oracle."""
    G.require_gpu()
    w = W.WORKLOADS["mixed"].replace(B=2, H=3, grid=(2, 9, 15))    # L = 270: five key blocks, ragged
    x = W.full_inputs(w)
    x["k"][1, 2, 70] *= np.float16(12)
    x["k"][1, 2, 200] *= np.float16(12)
    x["q"][0, 0, 5] *= np.float16(12)
    mask = np.array([0, 1, 0, 0, 0, 1], dtype=np.uint8)
    _run_and_check(w, x, layout="blhd", tau=0.05, head_mask=mask)


def test_empty_problem():
    """L = 0: every call returns success and touches nothing."""
    G.require_gpu()
    p = G.R.make_problem(1, 2, 0, 128, (0, 0, 0), 0, (44, 42, 42))
    z = torch.zeros(16, dtype=torch.float16, device="cuda")
    qk = G.R.binding.alloc_qk(p, "cuda", False)
    G.R.rotattn_quantize_qk(p, z, z, out=qk)
    G.R.rotattn_forward(p, qk, z, out=z)
    torch.cuda.synchronize()


def test_dump_ignores_out_of_range_units():
    """Units outside [0, B*H*NB) are skipped by the kernel: their dump rows stay as the caller filled them."""
    G.require_gpu()
    w = W.WORKLOADS["tiny"]
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    qk = G.R.rotattn_quantize_qk(p, G.dev(x["q"]), G.dev(x["k"]))
    vq = G.R.rotattn_quantize_v(p, G.dev(x["v"]))
    d = G.R.rotattn_debug_dump(p, qk, vq, G.dev(np.array([-1, 10**6, 1], dtype=np.int32)))
    acc = G.host(d["acc"])
    assert not acc[0].any() and not acc[1].any() and acc[2].any()


def test_fp16_forward_strided():
    """The whole-call FP16 path with [B, L, H, D] storage."""
    G.require_gpu()
    w = W.WORKLOADS["tiny"].replace(B=2, H=2, grid=(1, 6, 25), prefix=5)
    x = W.full_inputs(w)
    B, H, L, D = w.B, w.H, w.L, w.D

    def put(a):
        return torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3))).cuda().permute(0, 2, 1, 3)
    out = torch.empty((B, L, H, D), dtype=torch.float16, device="cuda").permute(0, 2, 1, 3)
    p = G.R.problem_from_workload(w, strides=(L * H * D, D, H * D))
    G.R.rotattn_fp16_forward(p, put(x["q"]), put(x["k"]), put(x["v"]), out=out)
    got = G.host(out).astype(np.float64)
    for b in range(B):
        for h in range(H):
            qr = O.apply_rope(x["q"][b, h].astype(np.float32), w.prefix, w.grid, w.split, w.base).astype(np.float16)
            kr = O.apply_rope(x["k"][b, h].astype(np.float32), w.prefix, w.grid, w.split, w.base).astype(np.float16)
            pp, bound = G.fp16_weight_bound(qr, kr, x["v"][b, h], L, D, np.arange(L))
            ref = pp["O"] / pp["l"][:, None]
            assert (np.abs(got[b, h] - ref) <= G.ATOL + G.RTOL * np.abs(ref) + bound).all()


def test_prologue_rounding_ties():
    """Q/K values that land exactly on half-integers of the quantization step: text-only tokens (no RoPE),
    D = 64 (the rotation's 1/8 is exact), rows x = H y / 8 with y in {+-0.5, +-1.5, ..., +-6.5, +-7}, so the
    rotated values are y and s = 1: every tie must round to even, as in the oracle."""
    G.require_gpu()
    w = W.WORKLOADS["smalld"].replace(H=1, grid=(0, 0, 0), prefix=128)
    rng = np.random.default_rng(77)
    halves = np.arange(-6.5, 7.0, 1.0)                      # -6.5 .. 6.5
    H64 = np.array([[1.0]])
    while H64.shape[0] < 64:
        H64 = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), H64)
    x = {}
    for t in ("q", "k"):
        y = rng.choice(halves, size=(128, 64))
        y[:, 0] = 7.0                                        # absmax 7 in every token: s = 1 in every block
        x[t] = ((y @ H64) / 8.0).astype(np.float16)[None, None]
        assert np.array_equal(x[t][0, 0].astype(np.float64), (y @ H64) / 8.0)   # exact in fp16
    x["v"] = rng.standard_normal((1, 1, 128, 64)).astype(np.float16)
    p = G.R.problem_from_workload(w)
    qk = G.R.rotattn_quantize_qk(p, G.dev(x["q"]), G.dev(x["k"]))
    o = G.oracle_head(w, x, 0, 0)
    for t in ("q", "k"):
        assert np.array_equal(G.host(getattr(qk, f"{t}_scale"))[0, 0], np.ones(2, np.float32))
        codes = G.unpack_qk_codes(G.host(getattr(qk, f"{t}_codes")))[0, 0]
        assert np.array_equal(codes, o[t]["codes"]), t
        assert (np.abs(o[t]["rot"][:, 1:] % 1.0 - 0.5) < 1e-12).all()   # every rotated value but dim 0 is a tie


def test_vquant_rounding_ties():
    """V values on exact half-integers of the quantization step: each channel holds one token at 7 (s = 1)
    and the rest in {+-0.5, +-1.5, ..., +-6.5}, exact in fp16, so every code but the 7s is a rounding tie
    that must go to even, as in the oracle; an all-zero channel gets scale 0 and codes 0."""
    G.require_gpu()
    w = W.WORKLOADS["tiny"].replace(H=1, grid=(1, 5, 30))   # L = 150: two full key blocks and a ragged one
    L, D = w.L, w.D
    rng = np.random.default_rng(78)
    halves = np.arange(-6.5, 7.0, 1.0)
    y = rng.choice(halves, size=(L, D))
    y[rng.integers(0, L, size=D), np.arange(D)] = 7.0          # absmax 7 in every channel
    y[:, 5] = 0.0                                              # one all-zero channel
    v = y.astype(np.float16)[None, None]
    assert np.array_equal(v[0, 0].astype(np.float64), y)
    x = {"q": rng.standard_normal((1, 1, L, D)).astype(np.float16),
         "k": rng.standard_normal((1, 1, L, D)).astype(np.float16), "v": v}
    p = G.R.problem_from_workload(w)
    vq = G.R.rotattn_quantize_v(p, G.dev(x["v"]))
    o = G.oracle_head(w, x, 0, 0)
    scale = G.host(vq.v_scale)[0, 0]
    want_scale = np.ones(D, np.float32)
    want_scale[5] = 0.0
    assert np.array_equal(scale, want_scale)
    assert np.array_equal(scale, o["v_scale"])
    codes = G.decode_v_codes(G.host(vq.v_codes))[0, 0]
    assert np.array_equal(codes, o["v_codes"])
    assert np.array_equal(G.host(vq.v_colsum)[0, 0], o["v_colsum"])
    # the ties really are ties, and they went to even
    c = o["v_codes"][:L].astype(np.float64)
    tie = np.abs(y % 1.0 - 0.5) < 1e-12
    assert tie.sum() > L * D // 2
    assert (c[tie] % 2 == 0).all()


@pytest.mark.parametrize("name,w", [
    ("group64_d128", W.WORKLOADS["480p"].replace(H=2, grid=(2, 7, 23))),
    ("group64_d64_even", W.WORKLOADS["smalld"].replace(H=2, grid=(1, 3, 30), prefix=5, split=(22, 22, 20),
                                                       rotation=W.ROT_GROUP64)),
    ("full_d128", W.WORKLOADS["tiny"].replace(grid=(2, 5, 19), prefix=8)),
])
def test_prologue_paths_agree(name, w):
    """The Q/K prologue with and without RoPE'd copies runs different kernels (per-group layout:
    the register kernel without copies, the LDS tile with them; full rotation: the register kernel
    without and with its copy-writing instance); both give the same codes, scales and flags, equal
    to the oracle's."""
    G.require_gpu()
    print(f"[gpu] prologue paths {name} L={w.L} D={w.D} rotation={w.rotation}", flush=True)
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    q, k = G.dev(x["q"]), G.dev(x["k"])
    a = G.R.rotattn_quantize_qk(p, q, k)
    c = G.R.rotattn_quantize_qk(p, q, k, rope_copy=True)
    torch.cuda.synchronize()
    for f in ("q_codes", "k_codes", "q_scale", "k_scale", "q_flag", "k_flag"):
        assert np.array_equal(G.host(getattr(a, f)), G.host(getattr(c, f))), (name, f)
    for h in range(w.H):
        o = G.oracle_head(w, x, 0, h)
        for t in ("q", "k"):
            assert np.array_equal(G.unpack_qk_codes(G.host(getattr(a, f"{t}_codes"))[0, h]), o[t]["codes"]), (name, h, t)
            assert np.array_equal(G.host(getattr(a, f"{t}_scale"))[0, h], o[t]["scale"]), (name, h, t)


@pytest.mark.parametrize("grid,prefix", [((1, 1, 523), 0), ((523, 1, 1), 3), ((7, 1, 97), 0), ((1, 61, 67), 5),
                                         ((3, 113, 1), 0), ((2, 3, 251), 11)])
def test_prologue_grid_coordinates(grid, prefix):
    """Token coordinates on degenerate and prime-sized grids (the prologue divides by H*W and W with a
    reciprocal estimate and a correction step): codes, scales and RoPE'd copies equal the oracle's."""
    G.require_gpu()
    w = W.WORKLOADS["tiny"].replace(H=1, grid=grid, prefix=prefix)
    print(f"[gpu] prologue grid {grid} prefix {prefix} L={w.L}", flush=True)
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    for copies in (False, True):
        qk = G.R.rotattn_quantize_qk(p, G.dev(x["q"]), G.dev(x["k"]), rope_copy=copies)
        torch.cuda.synchronize()
        for t in ("q", "k"):
            o = O.qk_prologue(x[t][0, 0], w.prefix, w.grid, w.split, w.base, w.rotation)
            assert np.array_equal(G.unpack_qk_codes(G.host(getattr(qk, f"{t}_codes"))[0, 0]), o["codes"]), (grid, t)
            assert np.array_equal(G.host(getattr(qk, f"{t}_scale"))[0, 0], o["scale"]), (grid, t)
            if copies:   # the RoPE'd fp16 copy, rounded to nearest even
                assert np.array_equal(G.host(getattr(qk, f"{t}_rope"))[0, 0], o["rope16"][:w.L]), (grid, t)


@pytest.mark.parametrize("name,w", [
    ("720p", W.WORKLOADS["720p"].replace(H=1)),
    ("smalld_odd_groups", W.WORKLOADS["smalld"].replace(H=1)),
    ("pair", W.WORKLOADS["tiny"].replace(rotation=W.ROT_PAIR)),
    ("480p_group64", W.WORKLOADS["480p"].replace(H=1)),
])
def test_rope_tables_bitwise(name, w):
    """The RoPE tables the prologue computed on the device (left in its workspace) equal the oracle's bit for bit:
    cos/sin of pos * base^(-2i / g_rot) (+ pi/4 for the mergeable rotation) in double, rounded once to float."""
    G.require_gpu()
    print(f"[gpu] rope tables {name} grid={w.grid} split={w.split}", flush=True)
    x = W.full_inputs(w)
    p = G.R.problem_from_workload(w)
    n = G.R.workspace_bytes(p, G.R.binding.CALL_QUANTIZE_QK)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    G.R.rotattn_quantize_qk(p, G.dev(x["q"]), G.dev(x["k"]), ws=ws)
    tab = G.host(ws).view(np.float32)
    phase = O.pair_phase() if w.rotation == W.ROT_PAIR else 0.0
    off = 0
    for a, (c, s) in enumerate(O.rope_tables(w.grid, w.split, w.base, phase)):
        cnt = c.size
        assert np.array_equal(tab[off:off + cnt].view(np.uint32), c.ravel().view(np.uint32)), (name, a, "cos")
        assert np.array_equal(tab[off + cnt:off + 2 * cnt].view(np.uint32), s.ravel().view(np.uint32)), (name, a, "sin")
        off += 2 * cnt


@pytest.mark.parametrize("n_flag", [3, 20])
def test_mixed_rows_inline_and_merged(n_flag):
    """Rows that mix both paths, in a head with few flagged K blocks (at most 16: the INT4 kernel finishes their
    FP16 tiles after its loop) and in one with many (the FP16 kernel merges the INT4 partials): planted
    high-norm key tokens flag n_flag K blocks of head 0; head 1 is masked; outputs against the oracle."""
    G.require_gpu()
    w = W.WORKLOADS["mixed"].replace(H=2, grid=(1, 40, 64))      # L = 2560, NB = 40
    x = W.full_inputs(w)
    rng = np.random.default_rng(n_flag)
    blocks = rng.choice(40, size=n_flag, replace=False)
    for j in blocks:
        x["k"][0, 0, 64 * j + 17] *= np.float16(14)
    print(f"[gpu] mixed rows: {n_flag} planted K blocks L={w.L}", flush=True)
    p = G.R.problem_from_workload(w, tau=0.05)
    q, k, v = G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"])
    qk = G.R.rotattn_quantize_qk(p, q, k, rope_copy=True)
    mask = np.array([0, 1], dtype=np.uint8)
    out = G.host(G.R.rotattn_forward(p, qk, v, head_fallback=G.dev(mask))).astype(np.float64)
    kf = G.host(qk.k_flag)[0, 0].astype(bool)
    assert kf.sum() >= n_flag and (kf.sum() > 16) == (n_flag > 16), int(kf.sum())
    assert int(G.host(qk.head_kflag)[0]) == int(kf.sum())          # the head's count of flagged K blocks
    for h in range(2):
        o = G.oracle_head(w, x, 0, h, tau=0.05, head_masked=bool(mask[h]),
                          q_flags=G.host(qk.q_flag)[0, h].astype(bool), k_flags=G.host(qk.k_flag)[0, h].astype(bool))
        tol = G.head_output_tol(w, x, 0, h, o, bool(mask[h]))
        err = np.abs(out[0, h] - o["out"])
        assert (err <= tol).all(), (h, float(err.max()))


def test_routed_call_on_user_stream():
    """A call that routes rows to FP16 forks the library's side stream from the caller's stream and joins it back
    before returning. On a non-default stream, with the output buffer filled with NaN first and read back by a
    copy on that stream, synchronizing that stream alone must expose the whole output, bit-identical to the same
    call on the default stream, on each of three calls. Head 0 has 18 flagged K blocks (merge), head 2 three
    (inline), heads 1 and 3 are masked (whole-row FP16)."""
    G.require_gpu()
    w = W.WORKLOADS["mixed"].replace(H=4, grid=(1, 40, 64))      # L = 2560, NB = 40
    x = W.full_inputs(w)
    for j in (2, 3, 5, 7, 9, 11, 13, 17, 19, 21, 23, 25, 27, 29, 31, 33, 35, 37):
        x["k"][0, 0, 64 * j + 17] *= np.float16(14)
    for j in (4, 14, 24):
        x["k"][0, 2, 64 * j + 40] *= np.float16(14)
    print(f"[gpu] routed call on a user stream L={w.L}", flush=True)
    p = G.R.problem_from_workload(w, tau=0.05)
    q, k, v = G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"])
    qk = G.R.rotattn_quantize_qk(p, q, k, rope_copy=True)
    m = G.dev(np.array([0, 1, 0, 1], dtype=np.uint8))
    kcount = G.host(qk.head_kflag)
    assert kcount[0] > 16 and 0 < kcount[2] <= 16, kcount
    ref = G.host(G.R.rotattn_forward(p, qk, v, head_fallback=m))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        with torch.cuda.stream(s):
            out = torch.full((w.B, w.H, w.L, w.D), float("nan"), dtype=torch.float16, device="cuda")
            G.R.rotattn_forward(p, qk, v, head_fallback=m, out=out, stream=s)
            host = torch.empty(out.shape, dtype=out.dtype, pin_memory=True)
            host.copy_(out, non_blocking=True)
        s.synchronize()
        assert np.array_equal(host.numpy().view(np.uint16), ref.view(np.uint16)), rep


def test_routed_call_graph_replay():
    """The routed forward (side-stream fork and join, inline and merged mixed rows, masked heads) captured in a
    HIP graph through torch's stream capture: every replay, with the output filled with NaN before it and an
    eager call of the library between replays, equals the eager result bit for bit."""
    G.require_gpu()
    w = W.WORKLOADS["mixed"].replace(H=4, grid=(1, 40, 64))      # L = 2560, NB = 40
    x = W.full_inputs(w)
    for j in (2, 3, 5, 7, 9, 11, 13, 17, 19, 21, 23, 25, 27, 29, 31, 33, 35, 37):
        x["k"][0, 0, 64 * j + 17] *= np.float16(14)
    for j in (4, 14, 24):
        x["k"][0, 2, 64 * j + 40] *= np.float16(14)
    print(f"[gpu] routed call in a graph L={w.L}", flush=True)
    p = G.R.problem_from_workload(w, tau=0.05)
    q, k, v = G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"])
    qk = G.R.rotattn_quantize_qk(p, q, k, rope_copy=True)
    m = G.dev(np.array([0, 1, 0, 1], dtype=np.uint8))
    ref = G.host(G.R.rotattn_forward(p, qk, v, head_fallback=m))
    n = G.R.workspace_bytes(p, G.R.binding.CALL_FORWARD_HEAD_FALLBACK)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.H, w.L, w.D), dtype=torch.float16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                                 # warm-up on the capture's kind of stream
        G.R.rotattn_forward(p, qk, v, head_fallback=m, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.R.rotattn_forward(p, qk, v, head_fallback=m, out=out, ws=ws)
    other = torch.empty_like(out)
    for rep in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), ref.view(np.uint16)), rep
        G.R.rotattn_forward(p, qk, v, head_fallback=m, out=other)   # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(other.cpu().numpy().view(np.uint16), ref.view(np.uint16)), rep


def test_routed_calls_from_two_threads():
    """Two host threads issue routed forwards on their own streams at the same time (the library's one side
    stream per device and its fork/join events are shared under a lock): every output is bit-identical to the
    serial result."""
    import threading
    G.require_gpu()
    w = W.WORKLOADS["mixed"].replace(H=4, grid=(1, 40, 64))      # L = 2560, NB = 40
    x = W.full_inputs(w)
    for j in (2, 3, 5, 7, 9, 11, 13, 17, 19, 21, 23, 25, 27, 29, 31, 33, 35, 37):
        x["k"][0, 0, 64 * j + 17] *= np.float16(14)
    for j in (4, 14, 24):
        x["k"][0, 2, 64 * j + 40] *= np.float16(14)
    print(f"[gpu] routed calls from two threads L={w.L}", flush=True)
    p = G.R.problem_from_workload(w, tau=0.05)
    q, k, v = G.dev(x["q"]), G.dev(x["k"]), G.dev(x["v"])
    qk = G.R.rotattn_quantize_qk(p, q, k, rope_copy=True)
    m = G.dev(np.array([0, 1, 0, 1], dtype=np.uint8))
    ref = G.host(G.R.rotattn_forward(p, qk, v, head_fallback=m)).view(np.uint16)
    n = G.R.workspace_bytes(p, G.R.binding.CALL_FORWARD_HEAD_FALLBACK)
    results, errors = {}, []

    def worker(tid):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                ws = torch.empty(n, dtype=torch.uint8, device="cuda")
                outs = [torch.empty((w.B, w.H, w.L, w.D), dtype=torch.float16, device="cuda") for _ in range(5)]
                for o in outs:
                    G.R.rotattn_forward(p, qk, v, head_fallback=m, out=o, ws=ws, stream=s)
            s.synchronize()
            results[tid] = [o.cpu().numpy().view(np.uint16) for o in outs]
        except Exception as e:   # reported below
            errors.append(repr(e))

    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for tid in range(2):
        for i, o in enumerate(results[tid]):
            assert np.array_equal(o, ref), (tid, i)
