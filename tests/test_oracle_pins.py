"""Pins of the CPU oracle to facts other than itself (no GPU needed).

Each test names the fact it checks: a hand-derived worked value, a closed
form, an invariant of the mathematics, a special case that reduces to a
textbook computation, or brute force on a tiny input.
"""
import math
import os

import numpy as np
import pytest

import workloads as W
from oracle import core as O
from tests import brute_force as BF

HERE = os.path.dirname(os.path.abspath(__file__))
F32 = np.float32


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# worked values
# --------------------------------------------------------------------------

def _golden_rows(name):
    rows = []
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line)
    return rows


def test_p_codes_golden():
    """Hand-derived codes of the range-optimized P quantizer (tests/golden/p_quant.txt)."""
    rows = _golden_rows("p_quant.txt")
    assert len(rows) >= 10
    for r in rows:
        p, want = r.split()
        got = int(O.p_codes(np.array([F32(float(p))], dtype=F32))[0])
        assert got == int(want), (p, got, want)


def test_p_codes_cover_int4_range():
    """The quantizer is the affine map of [0, 1] onto [-8, 7]: every INT4 value is reached, none outside."""
    P = np.linspace(0, 1, 100001, dtype=np.float64).astype(F32)
    pq = O.p_codes(P)
    assert pq.min() == -8 and pq.max() == 7
    assert set(np.unique(pq).tolist()) == set(range(-8, 8))
    # monotone non-decreasing in P
    assert np.all(np.diff(pq.astype(int)) >= 0)
    # step k is reached exactly where 15 P crosses k - 1/2
    for k in range(1, 16):
        lo = F32((k - 0.5) / 15 * (1 - 1e-6))
        hi = F32((k - 0.5) / 15 * (1 + 1e-6))
        assert O.p_codes(np.array([lo]))[0] == k - 1 - 8
        assert O.p_codes(np.array([hi]))[0] == k - 8


def test_fwht_golden():
    """Hand-derived small Walsh-Hadamard transforms (tests/golden/fwht_small.txt)."""
    for r in _golden_rows("fwht_small.txt"):
        n, x, y = [s.strip() for s in r.split("|")]
        n = int(n)
        x = np.array([float(v) for v in x.split()], dtype=F32)
        y = np.array([float(v) for v in y.split()]) / math.sqrt(n)
        got = O.fwht(x[None, :])[0]
        assert np.allclose(got, y, rtol=1e-6, atol=1e-7), (n, got, y)


# --------------------------------------------------------------------------
# token positions and RoPE
# --------------------------------------------------------------------------

def test_token_coords_roundtrip():
    """Frame-major [F, H, W] flattening: n = prefix + (t*Hh + h)*W + w, text tokens first."""
    grid = (3, 5, 7)
    prefix = 11
    L = prefix + 3 * 5 * 7
    coords, video = O.token_coords(L, prefix, grid)
    assert not video[:prefix].any() and video[prefix:].all()
    for n in range(prefix, L):
        t, h, w = coords[n]
        assert n == prefix + (t * 5 + h) * 7 + w
        assert BF.coords_of(n, prefix, grid) == (t, h, w)
    assert set(map(tuple, coords[prefix:])) == {(t, h, w) for t in range(3) for h in range(5) for w in range(7)}


@pytest.mark.parametrize("split,D", [((44, 42, 42), 128), ((22, 21, 21), 64)])
def test_rope_equals_dense_rotation(split, D):
    """RoPE equals x @ M with M built from 2x2 rotation blocks (brute force, float64), to float32 rounding."""
    grid = (3, 4, 5)
    prefix = 3
    L = prefix + 60
    x = _rng(1).standard_normal((L, D)).astype(F32)
    y = O.apply_rope(x, prefix, grid, split, 10000.0)
    for n in range(L):
        c = BF.coords_of(n, prefix, grid)
        if c is None:
            assert np.array_equal(y[n], x[n])
            continue
        want = x[n].astype(np.float64) @ BF.rope_matrix(c, split, 10000.0)
        assert np.allclose(y[n], want, rtol=0, atol=4e-6 * (1 + np.abs(want).max()))


def test_rope_orthogonal_and_identity_at_origin():
    """RoPE preserves each token's norm; position (0,0,0) and text tokens are the identity."""
    split = (44, 42, 42)
    grid = (4, 8, 8)
    L = 256
    x = _rng(2).standard_normal((L, 128)).astype(F32)
    y = O.apply_rope(x, 0, grid, split, 10000.0)
    nx = np.linalg.norm(x.astype(np.float64), axis=1)
    ny = np.linalg.norm(y.astype(np.float64), axis=1)
    assert np.allclose(nx, ny, rtol=1e-6)
    assert np.array_equal(y[0], x[0])
    # first pair of the t group turns by exactly t radians (frequency base**0 = 1)
    n = 2 * 64  # t = 2, h = w = 0
    ang = math.atan2(float(y[n, 1]) * x[n, 0] - float(y[n, 0]) * x[n, 1],
                     float(y[n, 0]) * x[n, 0] + float(y[n, 1]) * x[n, 1])
    assert abs(ang - 2.0) < 1e-5


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_relative_position(axis):
    """3D RoPE depends only on coordinate differences: moving both tokens one step along an axis leaves q.k unchanged."""
    split = (44, 42, 42)
    grid = (4, 6, 6)
    L = 4 * 6 * 6
    rng = _rng(3)
    q = rng.standard_normal(128).astype(F32)
    k = rng.standard_normal(128).astype(F32)
    step = (36, 6, 1)[axis]
    pairs = [(0, 37), (40, 75), (1, 3)]  # chosen so the shifted copies neither overlap nor wrap
    for a, b in pairs:
        X = np.zeros((L, 128), dtype=F32)
        X[a] = q
        X[b] = k
        X[a + step] = q
        X[b + step] = k
        Y = O.apply_rope(X, 0, grid, split, 10000.0).astype(np.float64)
        d0 = Y[a] @ Y[b]
        d1 = Y[a + step] @ Y[b + step]
        assert abs(d0 - d1) < 1e-4 * (1 + abs(d0))


# --------------------------------------------------------------------------
# Hadamard rotation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [2, 8, 64, 128])
def test_fwht_equals_dense_sylvester(n):
    """Butterfly WHT equals x @ H_n / sqrt(n) with H_n from the Kronecker recursion."""
    x = _rng(n).standard_normal((17, n)).astype(F32)
    want = x.astype(np.float64) @ BF.sylvester(n) / math.sqrt(n)
    got = O.fwht(x)
    assert np.allclose(got, want, rtol=0, atol=2e-6 * np.abs(want).max())


@pytest.mark.parametrize("n", [64, 128])
def test_fwht_orthonormal_involution(n):
    """H_n/sqrt(n) is symmetric and orthonormal: applying it twice gives x back; R R^T = I."""
    x = _rng(5).standard_normal((9, n)).astype(F32)
    back = O.fwht(O.fwht(x))
    assert np.allclose(back, x, atol=3e-6)
    R = O.fwht(np.eye(n, dtype=F32)).astype(np.float64)
    assert np.allclose(R @ R.T, np.eye(n), atol=1e-6)
    assert np.allclose(R, R.T, atol=0)


@pytest.mark.parametrize("rotation,split,D", [(O.ROT_FULL, (44, 42, 42), 128),
                                              (O.ROT_GROUP64, (44, 42, 42), 128),
                                              (O.ROT_FULL, (22, 21, 21), 64)])
def test_rotation_preserves_qk(rotation, split, D):
    """The rotation after RoPE leaves Q K^T unchanged (to float32 rounding)."""
    rng = _rng(6)
    q = rng.standard_normal((40, D)).astype(F32)
    k = rng.standard_normal((50, D)).astype(F32)
    qr = O.rotate(q, rotation, split)
    kr = O.rotate(k, rotation, split)
    assert qr.shape[1] == O.rotated_dim(D, rotation)
    S0 = q.astype(np.float64) @ k.astype(np.float64).T
    S1 = qr.astype(np.float64) @ kr.astype(np.float64).T
    assert np.allclose(S0, S1, atol=2e-5 * np.abs(S0).max())


def test_group64_layout():
    """Per-group padded rotation: group g occupies dims [64g, 64g+64) and is H_64/8 of the zero-padded group."""
    split = (44, 42, 42)
    x = _rng(7).standard_normal((5, 128)).astype(F32)
    y = O.rotate(x, O.ROT_GROUP64, split)
    H = BF.sylvester(64) / 8.0
    off = 0
    for g, size in enumerate(split):
        pad = np.zeros((5, 64))
        pad[:, :size] = x[:, off:off + size]
        assert np.allclose(y[:, 64 * g:64 * g + 64], pad @ H, atol=1e-5)
        off += size


# --------------------------------------------------------------------------
# INT4 quantization of Q, K, V
# --------------------------------------------------------------------------

def test_qk_quant_properties():
    """Symmetric INT4 block codes: range [-7, 7], absmax -> +-7, |x - s c| <= s/2, requantizing s*c returns c."""
    x = (_rng(8).standard_normal((200, 128)) * 3).astype(F32)   # ragged: 200 = 3*64 + 8
    codes, scales, nsr = O.quantize_qk_blocks(x)
    assert codes.shape == (256, 128) and scales.shape == (4,)
    assert codes.min() >= -7 and codes.max() <= 7
    for b in range(4):
        xb = x[64 * b:min(64 * b + 64, 200)]
        cb = codes[64 * b:64 * b + xb.shape[0]]
        s = scales[b]
        assert s == F32(np.abs(xb).max() / F32(7))
        i = np.unravel_index(np.argmax(np.abs(xb)), xb.shape)
        assert abs(int(cb[i])) == 7
        err = np.abs(xb.astype(np.float64) - float(s) * cb)
        assert err.max() <= float(s) * 0.5 * (1 + 1e-6)
        again = O.quantize_sym((F32(s) * cb.astype(F32)).astype(F32), s)
        assert np.array_equal(again, cb)
    # padded rows of the ragged block are zero
    assert not codes[200:].any()


def test_qk_quant_tail_uses_valid_tokens_only():
    """The ragged last block's scale ignores the padding; an all-zero block gets scale 0 and codes 0."""
    x = np.zeros((130, 64), dtype=F32)
    x[:64] = 1.0
    x[128:130] = 0.5
    codes, scales, nsr = O.quantize_qk_blocks(x)
    assert scales[0] == F32(1.0) / F32(7.0)
    assert scales[1] == 0 and not codes[64:128].any() and nsr[1] == 0
    assert scales[2] == F32(0.5) / F32(7.0)
    assert (codes[128:130] == 7).all()


def test_qk_quant_power_of_two_invariance():
    """Scaling a block by 2**k scales s by 2**k and leaves the codes alone (exact in float32)."""
    x = _rng(9).standard_normal((64, 128)).astype(F32)
    c1, s1, _ = O.quantize_qk_blocks(x)
    c2, s2, _ = O.quantize_qk_blocks(x * F32(8))
    assert np.array_equal(c1, c2) and s2[0] == s1[0] * 8


def test_nsr_matches_uniform_noise_model():
    """Block NSR of a Gaussian block is close to the uniform-noise closed form s^2/12 / E[x^2]."""
    rng = _rng(10)
    vals = []
    for _ in range(50):
        x = rng.standard_normal((64, 128)).astype(F32)
        c, s, nsr = O.quantize_qk_blocks(x)
        model = float(s[0]) ** 2 / 12 / float(np.mean(x.astype(np.float64) ** 2))
        vals.append((nsr[0], model))
    v = np.array(vals)
    assert np.allclose(v[:, 0], v[:, 1], rtol=0.08)
    assert 0.02 < v[:, 0].mean() < 0.04


def test_nsr_flags_high_norm_token_not_single_spike():
    """One token scaled x10 raises NSR above 5% (flagged); one huge element dominates the energy and does not."""
    rng = _rng(11)
    x = O.fwht(rng.standard_normal((64, 128)).astype(F32))
    _, _, n0 = O.quantize_qk_blocks(x)
    y = x.copy()
    y[5] *= 10
    _, _, n1 = O.quantize_qk_blocks(y)
    z = x.copy()
    z[5, 3] = 1000.0
    _, _, n2 = O.quantize_qk_blocks(z)
    assert n0[0] < 0.05 < n1[0]
    assert n2[0] < 0.05


def test_v_quant_properties():
    """Per-channel V codes: range, absmax -> +-7, |v - s c| <= s/2; colsum is the integer column sum of each key block."""
    v = (_rng(12).standard_normal((150, 64)) * np.exp(_rng(13).standard_normal(64))).astype(np.float16)
    codes, scale, colsum = O.quantize_v(v)
    v64 = v.astype(np.float64)
    assert codes.shape == (192, 64) and colsum.shape == (3, 64)
    assert not codes[150:].any()
    assert codes.min() >= -7 and codes.max() <= 7
    for c in range(64):
        assert scale[c] == F32(np.abs(v64[:, c]).max()) / F32(7)
        assert abs(codes[np.argmax(np.abs(v64[:, c])), c]) == 7
        assert np.abs(v64[:, c] - float(scale[c]) * codes[:150, c]).max() <= float(scale[c]) * 0.5 * (1 + 1e-6)
    assert np.array_equal(colsum.sum(axis=0), codes.astype(np.int64).sum(axis=0))
    for j in range(3):
        for c in (0, 17, 63):
            assert colsum[j, c] == sum(int(codes[k, c]) for k in range(64 * j, 64 * j + 64))


def test_nibble_packing_layout():
    """Byte k holds dim 2k in the low nibble and dim 2k+1 in the high nibble, two's complement."""
    codes = np.array([[1, -1, 7, -7, -8, 0, 3, -2]], dtype=np.int8)
    p = O.pack_nibbles(codes)
    assert p.tolist() == [[0xF1, 0x97, 0x08, 0xE3]]
    assert np.array_equal(O.unpack_nibbles(p), codes)
    r = _rng(14).integers(-7, 8, size=(33, 192)).astype(np.int8)
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(r)), r)


# --------------------------------------------------------------------------
# the flash loop
# --------------------------------------------------------------------------

def _tiny_codes(L, Dq, Dv, seed):
    rng = _rng(seed)
    nb = O.n_blocks(L)
    qc = np.zeros((nb * 64, Dq), np.int8)
    kc = np.zeros((nb * 64, Dq), np.int8)
    vc = np.zeros((nb * 64, Dv), np.int8)
    qc[:L] = rng.integers(-7, 8, (L, Dq))
    kc[:L] = rng.integers(-7, 8, (L, Dq))
    vc[:L] = rng.integers(-7, 8, (L, Dv))
    sq = rng.uniform(0.02, 0.3, nb).astype(F32)
    sk = rng.uniform(0.02, 0.3, nb).astype(F32)
    sv = rng.uniform(0.1, 1.0, Dv).astype(F32)
    colsum = vc.reshape(nb, 64, Dv).astype(np.int32).sum(1).astype(np.int32)
    return qc, sq, kc, sk, vc, sv, colsum


@pytest.mark.parametrize("L,Dq,Dv", [(150, 16, 8), (64, 8, 4), (7, 8, 4), (129, 12, 6)])
def test_flash_matches_scalar_brute_force(L, Dq, Dv):
    """Vectorized flash loop equals a per-row, per-key scalar loop: identical P codes, outputs to 1e-12."""
    qc, sq, kc, sk, vc, sv, colsum = _tiny_codes(L, Dq, Dv, L)
    rows = list(range(0, L, max(1, L // 9))) + [L - 1]
    r = O.int4_flash_rows(qc, sq, kc, sk, vc, sv, colsum, L, 128, rows, dump=True)
    out = r["O_scaled"] / r["l"][:, None]
    bout, bpq = BF.flash_brute(qc, sq, kc, sk, vc, sv, L, 128, rows)
    assert np.array_equal(r["pq"][:, :L], bpq[:, :L])
    assert np.allclose(out, bout, rtol=1e-12, atol=1e-12)


def test_flash_skip_list_matches_brute_force():
    """Skipping key blocks (the block mask of RainFusion2.0 sec. 3.1) in the vectorized loop equals the scalar loop."""
    L = 200
    qc, sq, kc, sk, vc, sv, colsum = _tiny_codes(L, 16, 8, 99)
    kb = np.array([True, False, True, True])
    rows = [0, 63, 64, 130, 199]
    r = O.int4_flash_rows(qc, sq, kc, sk, vc, sv, colsum, L, 64, rows, key_blocks=kb, dump=True)
    bout, bpq = BF.flash_brute(qc, sq, kc, sk, vc, sv, L, 64, rows, key_blocks=list(kb))
    assert np.allclose(r["O_scaled"] / r["l"][:, None], bout, rtol=1e-12)
    keep = np.repeat(kb, 64)[:L]
    assert np.array_equal(r["pq"][:, :L][:, keep], bpq[:, :L][:, keep])


def test_flash_integer_invariants():
    """acc equals the int64 dot product; pq in [-8, 7]; the running-max key gets 7; P < 1/30 gives -8; accPV = sum (pq+8) v."""
    L = 300
    qc, sq, kc, sk, vc, sv, colsum = _tiny_codes(L, 32, 16, 5)
    rows = np.arange(0, L, 7)
    r = O.int4_flash_rows(qc, sq, kc, sk, vc, sv, colsum, L, 128, rows, dump=True)
    acc = qc[rows].astype(np.int64) @ kc.astype(np.int64).T
    assert np.array_equal(r["acc"][:, :L], acc[:, :L])
    pq = r["pq"][:, :L].astype(int)
    assert pq.min() >= -8 and pq.max() <= 7
    nb = O.n_blocks(L)
    c0 = O.softmax_c0(128)
    for ri, row in enumerate(rows):
        for j in range(nb):
            keys = np.arange(64 * j, min(64 * j + 64, L))
            # the key holding the running max after block j (if it is in block j) has P = 1 -> code 7
            cq = F32(sq[row // 64] * c0)
            c = F32(cq * sk[j])
            exact = acc[ri, keys].astype(F32).astype(np.float64) * float(c)
            S2 = exact.astype(F32)
            if S2.max() == r["m_hist"][ri, j]:
                assert pq[ri, keys[np.argmax(S2)]] == 7
            # P = 2**(S2 - m) below 1/30 (15 P below 1/2, with margin for rounding) gives -8
            P = np.exp2(exact - float(r["m_hist"][ri, j]))
            assert (pq[ri, keys[P < 1 / 30 * (1 - 1e-5)]] == -8).all()
            # and every code is within one rounding step of 15 P - 8
            assert (np.abs(pq[ri, keys] + 8 - 15 * P) <= 0.5 + 1e-4).all()
            want = ((pq[ri, keys] + 8)[:, None] * vc[keys].astype(np.int64)).sum(0)
            assert np.array_equal(r["accpv"][ri, j], want)


def test_flash_identity_without_quantization():
    """With codes replaced by real values and P unquantized, the blockwise online recurrence equals one-pass softmax attention (RainFusion2.0 sec. 3.1)."""
    rng = _rng(21)
    L, D = 333, 64
    q = rng.standard_normal((L, D))
    k = rng.standard_normal((L, D))
    v = rng.standard_normal((L, D))
    nb = O.n_blocks(L)
    pad = lambda a: np.concatenate([a, np.zeros((nb * 64 - L, a.shape[1]))])
    ones = np.ones(nb, dtype=F32)
    rows = np.arange(0, L, 5)
    r = O.int4_flash_rows(pad(q), ones, pad(k), ones, pad(v), np.ones(D, F32), None, L, D, rows,
                          quantize_p=False)
    out = r["O"] if "O" in r else r["O_scaled"]
    out = out / r["l"][:, None]
    # textbook softmax with natural exp on the same float32-rounded logits (S2 rounding is part of the loop)
    want = BF.softmax_attention_brute(q[rows], k, v, 1.0 / math.sqrt(D))
    assert np.allclose(out, want, rtol=0, atol=2e-5)


def test_q_zero_closed_form():
    """Q = 0: every S2 is 0, every P is 1 and every code is 7, so out_c = s_v,c * mean_j(cv_jc) exactly."""
    L, D = 150, 128
    rng = _rng(22)
    q = np.zeros((L, D), np.float16)
    k = rng.standard_normal((L, D)).astype(np.float16)
    v = rng.standard_normal((L, D)).astype(np.float16)
    res = O.forward_head(q, k, v, prefix=0, grid=(1, 5, 30), split=(44, 42, 42), base=10000.0,
                         rotation=O.ROT_FULL)
    vc, sv = res["v_codes"][:L].astype(np.float64), res["v_scale"].astype(np.float64)
    want = sv[None, :] * vc.mean(axis=0)[None, :]
    assert np.allclose(res["out"], np.broadcast_to(want, (L, D)), rtol=1e-12, atol=1e-15)


def test_constant_v_columns():
    """Constant V columns a and b get codes 7 sign(a), 7 sign(b) and outputs in exact ratio a : b, close to a and b.

    The output of a constant column is a times sum(pq+8) / (15 l), the same
    channel-independent factor for every constant column; it is 1 up to the
    rounding of 15 P to integers, which averages out over many keys.
    """
    L, D = 100, 64
    rng = _rng(23)
    q = rng.standard_normal((L, D)).astype(np.float16)
    k = rng.standard_normal((L, D)).astype(np.float16)
    v = rng.standard_normal((L, D)).astype(np.float16)
    v[:, 5] = np.float16(-1.25)
    v[:, 9] = np.float16(2.5)
    res = O.forward_head(q, k, v, prefix=10, grid=(2, 5, 9), split=(22, 21, 21), base=10000.0,
                         rotation=O.ROT_FULL)
    assert (res["v_codes"][:L, 5] == -7).all() and (res["v_codes"][:L, 9] == 7).all()
    r5 = res["out"][:, 5] / -1.25
    r9 = res["out"][:, 9] / 2.5
    assert np.allclose(r5, r9, rtol=1e-12)
    assert abs(r5.mean() - 1) < 0.05


def test_single_block_is_plain_quantized_softmax():
    """L <= 64: one key block, so the loop is one softmax with P codes taken against the row max.

    Reference computed in float64 without any of the loop's float32 steps:
    codes rne(15 P) with P = 2**(S2 - max S2), out = sum codes v * s_v / 15 / sum P.
    """
    L, D = 50, 64
    qc, sq, kc, sk, vc, sv, colsum = _tiny_codes(L, 64, 64, 24)
    rows = np.arange(L)
    r = O.int4_flash_rows(qc, sq, kc, sk, vc, sv, colsum, L, D, rows, dump=True)
    c0 = O.softmax_c0(D)
    acc = qc[:L].astype(np.int64) @ kc[:L].astype(np.int64).T
    S2 = acc.astype(np.float64) * float(F32(F32(sq[0] * c0) * sk[0]))
    P = np.exp2(S2 - S2.max(1, keepdims=True))
    codes = np.rint(15 * P)  # pq + 8
    assert np.array_equal(r["pq"][:, :L] + 8, codes)
    want = (codes @ vc[:L].astype(np.float64)) * sv / 15 / P.sum(1, keepdims=True)
    assert np.allclose(r["O_scaled"] / r["l"][:, None], want, rtol=2e-6)


# --------------------------------------------------------------------------
# FP16 path, merge, routing
# --------------------------------------------------------------------------

def test_fp16_rows_is_textbook_softmax():
    """The FP16 path's exact partial equals softmax(q k^T / sqrt(D)) v with natural exp (scalar loops)."""
    rng = _rng(31)
    L, D = 70, 16
    q = rng.standard_normal((L, D)).astype(np.float16)
    k = rng.standard_normal((L, D)).astype(np.float16)
    v = rng.standard_normal((L, D)).astype(np.float16)
    rows = [0, 33, 69]
    p = O.fp16_rows(q, k, v, L, D, rows)
    want = BF.softmax_attention_brute(q[rows], k, v, 1 / math.sqrt(D))
    assert np.allclose(p["O"] / p["l"][:, None], want, rtol=1e-12, atol=1e-13)


def test_merge_reassembles_split():
    """Merging the partials of two disjoint key sets reproduces the unsplit softmax (log-sum-exp identity)."""
    rng = _rng(32)
    L, D = 256, 32
    q = rng.standard_normal((L, D)).astype(np.float16)
    k = rng.standard_normal((L, D)).astype(np.float16)
    v = rng.standard_normal((L, D)).astype(np.float16)
    rows = np.arange(0, L, 3)
    kb = np.array([True, False, False, True])
    a = O.fp16_rows(q, k, v, L, D, rows, key_blocks=kb)
    b = O.fp16_rows(q, k, v, L, D, rows, key_blocks=~kb)
    full = O.fp16_rows(q, k, v, L, D, rows)
    got = O.merge(a["O"], a["m"], a["l"], b["O"], b["m"], b["l"])
    assert np.allclose(got, full["O"] / full["l"][:, None], rtol=1e-12, atol=1e-13)
    # an empty partial (m = -inf) has no weight
    e = O.merge(np.zeros_like(a["O"]), np.full(rows.size, -np.inf), np.zeros(rows.size),
                full["O"], full["m"], full["l"])
    assert np.allclose(e, full["O"] / full["l"][:, None], rtol=1e-14)


def _head(name="tiny", h=0, L=None):
    w = W.WORKLOADS[name]
    if L is not None:
        w = w.replace(grid=(1, 1, L - w.prefix))
    return w, W.head_inputs(w, 0, h)


def test_merge_equals_continued_recurrence():
    """Continuing the online softmax (RainFusion2.0 sec. 3.1) over the FP16 key blocks from the INT4 loop's final
    state (m, l, O in V's units) gives the log-sum-exp merge of the two partials: the order in which a row with
    both paths is finished does not change the oracle's result (float64, to 1e-12)."""
    rng = _rng(41)
    L, D = 300, 64
    q = rng.standard_normal((L, D)).astype(np.float16)
    k = rng.standard_normal((L, D)).astype(np.float16)
    v = rng.standard_normal((L, D)).astype(np.float16)
    grid, split = (1, 10, 30), (22, 21, 21)
    qp = O.qk_prologue(q, 0, grid, split, 10000.0, O.ROT_FULL)
    kp = O.qk_prologue(k, 0, grid, split, 10000.0, O.ROT_FULL)
    vc, sv, cs = O.quantize_v(v)
    fk = np.array([False, True, False, False, True])
    rows = np.arange(0, L, 3)
    p1 = O.int4_flash_rows(qp["codes"], qp["scale"], kp["codes"], kp["scale"], vc, sv, cs, L, D, rows,
                           key_blocks=~fk)
    p2 = O.fp16_rows(qp["rope16"], kp["rope16"], v, L, D, rows, key_blocks=fk)
    want = O.merge(p1["O_scaled"], p1["m"], p1["l"], p2["O"], p2["m"], p2["l"])
    # the continuation, block by block in ascending order
    m = p1["m"].astype(np.float64).copy()
    lsum = p1["l"].copy()
    acc = p1["O_scaled"].copy()
    c = math.log2(math.e) / math.sqrt(D)
    qq = qp["rope16"][rows].astype(np.float64)
    for j in np.nonzero(fk)[0]:
        keys = np.arange(64 * j, min(64 * j + 64, L))
        S2 = (qq @ kp["rope16"][keys].astype(np.float64).T) * c
        m_new = np.maximum(m, S2.max(axis=1))
        alpha = np.exp2(m - m_new)
        P = np.exp2(S2 - m_new[:, None])
        acc = alpha[:, None] * acc + P @ v[keys].astype(np.float64)
        lsum = alpha * lsum + P.sum(axis=1)
        m = m_new
    assert np.allclose(acc / lsum[:, None], want, rtol=1e-12, atol=1e-13)


def test_routing_all_fp16_equals_fp16_forward():
    """A masked head runs every tile on the FP16 path: identical to the whole-call FP16 forward."""
    w, x = _head()
    kw = dict(prefix=w.prefix, grid=w.grid, split=w.split, base=w.base)
    a = O.forward_head(x["q"], x["k"], x["v"], rotation=w.rotation, head_masked=True, **kw)
    b = O.fp16_forward_head(x["q"], x["k"], x["v"], **kw)
    assert np.array_equal(a["out"], b)


def test_routing_tau_zero_equals_fp16_forward():
    """tau = 0 flags every non-empty block: again every tile is FP16."""
    w, x = _head()
    kw = dict(prefix=w.prefix, grid=w.grid, split=w.split, base=w.base)
    a = O.forward_head(x["q"], x["k"], x["v"], rotation=w.rotation, tau=0.0, **kw)
    b = O.fp16_forward_head(x["q"], x["k"], x["v"], **kw)
    assert a["q_flags"].all() and a["k_flags"].all()
    assert np.allclose(a["out"], b, rtol=1e-14, atol=1e-14)


def test_routing_mixed_rows():
    """Flagging only some K blocks: unflagged rows merge an INT4 partial (unflagged keys) with an exact FP16 partial (flagged keys)."""
    w, x = _head()
    kw = dict(prefix=w.prefix, grid=w.grid, split=w.split, base=w.base, rotation=w.rotation)
    L = w.L
    fk = np.array([False, True, False, False])
    fq = np.array([False, False, True, False])
    res = O.forward_head(x["q"], x["k"], x["v"], q_flags=fq, k_flags=fk, **kw)
    qp, kp = res["q"], res["k"]
    rows = np.arange(0, 64)
    p1 = O.int4_flash_rows(qp["codes"], qp["scale"], kp["codes"], kp["scale"], res["v_codes"],
                           res["v_scale"], res["v_colsum"], L, w.D, rows, key_blocks=~fk)
    p2 = O.fp16_rows(qp["rope16"], kp["rope16"], x["v"], L, w.D, rows, key_blocks=fk)
    assert np.allclose(res["out"][rows], O.merge(p1["O_scaled"], p1["m"], p1["l"], p2["O"], p2["m"], p2["l"]))
    fp16 = O.fp16_forward_head(x["q"], x["k"], x["v"], prefix=w.prefix, grid=w.grid, split=w.split, base=w.base)
    assert np.array_equal(res["out"][128:192], fp16[128:192])


def test_quantized_path_tracks_exact_attention():
    """On plain Gaussian inputs the quantized path stays close to unquantized attention (cosine similarity).

    Flat attention is the hard case for a fixed-scale P code (most P are far
    below 1/15), so the bar is loose: it catches a broken path (cosine near 0),
    not small numerical differences.
    """
    x = W.random_qkv(300, 128, seed=3)
    kw = dict(prefix=0, grid=(3, 10, 10), split=(44, 42, 42), base=10000.0)
    q, k, v = x["q"][0, 0], x["k"][0, 0], x["v"][0, 0]
    res = O.forward_head(q, k, v, rotation=O.ROT_FULL, **kw)
    ex = O.exact_attention(q, k, v, **kw)
    assert O.cosine_similarity(res["out"], ex) > 0.93


def test_exact_attention_brute():
    """exact_attention equals textbook softmax on float64 RoPE'd vectors built from dense rotation matrices."""
    rng = _rng(41)
    grid, split, prefix = (2, 3, 4), (22, 21, 21), 5
    L, D = prefix + 24, 64
    q = rng.standard_normal((L, D)).astype(np.float16)
    k = rng.standard_normal((L, D)).astype(np.float16)
    v = rng.standard_normal((L, D)).astype(np.float16)

    def rope(x):
        y = x.astype(np.float64).copy()
        for n in range(L):
            c = BF.coords_of(n, prefix, grid)
            if c is not None:
                y[n] = x[n].astype(np.float64) @ BF.rope_matrix(c, split, 10000.0)
        return y

    got = O.exact_attention(q, k, v, prefix=prefix, grid=grid, split=split, base=10000.0)
    want = BF.softmax_attention_brute(rope(q), rope(k), v, 1 / math.sqrt(D))
    assert np.allclose(got, want, rtol=1e-10, atol=1e-12)


# --------------------------------------------------------------------------
# block-sparse mask (RainFusion2.0 sections 3.1, 3.2, 3.4)
# --------------------------------------------------------------------------

def test_sink_end_closed_forms():
    """The sink is the text prefix plus the grid_h * grid_w tokens of frame 0 (clamped to L)."""
    assert O.sink_end(226 + 13 * 30 * 45, 226, (13, 30, 45)) == 226 + 30 * 45
    assert O.sink_end(75600, 0, (21, 45, 80)) == 45 * 80
    assert O.sink_end(100, 100, (0, 4, 4)) == 100            # no video: the prefix only
    assert O.sink_end(20, 4, (1, 4, 8)) == 20                 # one frame: everything


def test_block_means_brute_force_and_tail():
    """Block means equal a per-dim summation loop over the RoPE'd rows (3 text + 64 video tokens); the ragged block averages its 3 valid rows only."""
    rng = _rng(31)
    L, D, prefix, grid, split = 64 + 3, 16, 3, (1, 8, 8), (6, 5, 5)
    x = rng.standard_normal((L, D)).astype(np.float16)
    got = O.block_means(x, prefix, grid, split, 10000.0)
    xr = O.apply_rope(x.astype(F32), prefix, grid, split, 10000.0)
    for i, (a, b) in enumerate([(0, 64), (64, L)]):
        for d in range(D):
            acc = 0.0
            for t in range(a, b):
                acc += float(xr[t, d])
            assert got[i, d] == pytest.approx(acc / (b - a), rel=1e-12, abs=1e-15)
    # the ragged block is not diluted by the 61 padded rows
    assert not np.allclose(got[1], xr[64:].astype(np.float64).sum(0) / 64, rtol=1e-3)
    # one 128-token block (67 valid tokens) is the count-weighted mean of the two 64-token means
    got128 = O.block_means(x, prefix, grid, split, 10000.0, 128)
    assert got128.shape == (1, D)
    assert np.allclose(got128[0], (64 * got[0] + 3 * got[1]) / 67, rtol=1e-12, atol=1e-15)


def test_block_scores_are_tile_means_of_scores():
    """S_hat[i, j] = q_hat_i . k_hat_j equals the mean of q_a . k_b over the 128 x 64 tile (a in Q_i, b in K_j), by bilinearity."""
    rng = _rng(32)
    L, D, prefix, grid, split = 150, 16, 0, (1, 10, 15), (6, 5, 5)
    q = rng.standard_normal((L, D)).astype(np.float16)
    k = rng.standard_normal((L, D)).astype(np.float16)
    bq, bk = O.SPARSE_BQ, O.SPARSE_BK
    s_hat = O.block_scores(O.block_means(q, prefix, grid, split, 10000.0, bq),
                           O.block_means(k, prefix, grid, split, 10000.0, bk))
    qr = O.apply_rope(q.astype(F32), prefix, grid, split, 10000.0).astype(np.float64)
    kr = O.apply_rope(k.astype(F32), prefix, grid, split, 10000.0).astype(np.float64)
    S = qr @ kr.T
    assert s_hat.shape == (-(-L // bq), -(-L // bk)) == (2, 3)
    for i in range(s_hat.shape[0]):
        for j in range(s_hat.shape[1]):
            tile = S[bq * i:min(L, bq * i + bq), bk * j:min(L, bk * j + bk)]
            assert s_hat[i, j] == pytest.approx(tile.mean(), rel=1e-10, abs=1e-12)


def test_block_scores_invariant_under_hadamard():
    """Means of the Hadamard-rotated rows give the same S_hat (the rotation is orthonormal and linear)."""
    rng = _rng(33)
    L, D, grid, split = 128, 128, (2, 8, 8), (44, 42, 42)
    q = rng.standard_normal((L, D)).astype(np.float16)
    k = rng.standard_normal((L, D)).astype(np.float16)
    qm = O.block_means(q, 0, grid, split, 10000.0)
    km = O.block_means(k, 0, grid, split, 10000.0)
    H = BF.sylvester(D) / math.sqrt(D)
    assert np.allclose(O.block_scores(qm @ H, km @ H), O.block_scores(qm, km), rtol=1e-10, atol=1e-12)


def test_sparse_mask_rank_count_brute_force():
    """Top-n per query block equals the rank-count rule (fewer than n keys rank above it, ties to lower j), plus the sink rows and columns."""
    rng = _rng(34)
    nb, n = 9, 3
    s = rng.integers(-3, 4, (nb, nb)).astype(np.float64)     # many ties
    L, prefix, grid = nb * 64, 10, (3, 10, 17)                # sink_end = 10 + 170 = 180 -> key blocks 0..2
    M = O.sparse_block_mask(s, n, L, prefix, grid, bq=64)
    for i in range(nb):
        for j in range(nb):
            rank = sum(1 for kk in range(nb) if s[i, kk] > s[i, j] or (s[i, kk] == s[i, j] and kk < j))
            want = rank < n or j <= 2 or i <= 2
            assert M[i, j] == want, (i, j)
    assert M[:3].all() and M[:, :3].all()
    # 128-row query blocks: the sink (tokens < 180) lies in query blocks 0 and 1
    M2 = O.sparse_block_mask(s[:5], n, L, prefix, grid, bq=128)
    assert M2[:2].all() and M2[:, :3].all() and not M2[2:, 3:].all()


def test_sparse_mask_worked_example():
    """Hand-checked: scores with a clear order select the expected blocks; topn >= NB keeps everything."""
    s = np.array([[5., 1., 4., 2., 3.],
                  [1., 2., 3., 4., 5.],
                  [0., 0., 0., 0., 0.],
                  [9., 8., 7., 6., 5.],
                  [2., 9., 2., 9., 1.]])
    L, prefix, grid = 5 * 64, 0, (5, 8, 8)                    # frame 0 = block 0 is the sink
    M = O.sparse_block_mask(s, 2, L, prefix, grid, bq=64)
    want = np.array([[1, 1, 1, 1, 1],                         # sink query block
                     [1, 0, 0, 1, 1],
                     [1, 1, 0, 0, 0],                         # all equal: lowest j
                     [1, 1, 0, 0, 0],
                     [1, 1, 0, 1, 0]], dtype=bool)
    assert np.array_equal(M, want)
    assert O.sparse_block_mask(s, 5, L, prefix, grid, bq=64).all()


def test_sparse_forward_dense_mask_equals_dense_path():
    """With every block kept the block-sparse path is the dense INT4 path (same loop, same codes)."""
    w = W.WORKLOADS["tiny"]
    x = W.head_inputs(w, 0, 1)
    kw = dict(prefix=w.prefix, grid=w.grid, split=w.split, base=w.base, rotation=w.rotation)
    nb = O.n_blocks(w.L)
    sp = O.sparse_forward_head(x["q"], x["k"], x["v"], topn=nb, **kw)
    dn = O.forward_head(x["q"], x["k"], x["v"], **kw)
    assert sp["mask"].all()
    assert np.array_equal(sp["out"], dn["out"])


def test_sparse_forward_masked_softmax_identity():
    """Unquantized, the block-skipping loop with a per-query-block mask equals softmax restricted to the kept keys."""
    rng = _rng(35)
    L, D = 200, 32
    nb = O.n_blocks(L)
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    pad = lambda a: np.concatenate([a, np.zeros((nb * 64 - L, a.shape[1]))])
    M = np.array([[1, 0, 1, 1], [0, 1, 0, 1], [1, 1, 1, 0], [0, 0, 1, 1]], dtype=bool)
    ones = np.ones(nb, dtype=F32)
    for qb in range(nb):
        rows = np.arange(64 * qb, min(L, 64 * qb + 64), 7)
        r = O.int4_flash_rows(pad(q), ones, pad(k), ones, pad(v), np.ones(D, F32), None, L, D, rows,
                              key_blocks=M[qb], quantize_p=False)
        keys = np.nonzero(np.repeat(M[qb], 64)[:L])[0]
        want = BF.softmax_attention_brute(q[rows], k[keys], v[keys], 1.0 / math.sqrt(D))
        assert np.allclose(r["O_scaled"] / r["l"][:, None], want, rtol=0, atol=2e-5)


def test_sparse_sink_rows_are_dense():
    """Query blocks (128 rows) that hold first-frame tokens keep every key block, so their outputs equal the dense path's."""
    w = W.WORKLOADS["tiny"]
    x = W.head_inputs(w, 0, 0)
    kw = dict(prefix=w.prefix, grid=w.grid, split=w.split, base=w.base, rotation=w.rotation)
    rows = np.arange(0, 128)                                  # frame 0 of the 4x8x8 grid is in query block 0
    sp = O.sparse_forward_head(x["q"], x["k"], x["v"], topn=1, rows=rows, **kw)
    dn = O.forward_head(x["q"], x["k"], x["v"], rows=rows, **kw)
    assert not sp["mask"][1:, 1:].all()
    assert np.array_equal(sp["out"], dn["out"])


# --------------------------------------------------------------------------
# the mergeable RoPE-aware rotation (RotateAttention abstract)
# --------------------------------------------------------------------------

def _pair_matrix(split, phase):
    """Dense D x D per-pair plane rotation by `phase` (row-vector convention), identity on unpaired dims."""
    D = sum(split)
    R = np.eye(D)
    c, s = math.cos(phase), math.sin(phase)
    off = 0
    for g in split:
        for i in range(g // 2):
            d0, d1 = off + 2 * i, off + 2 * i + 1
            R[d0, d0], R[d1, d0], R[d0, d1], R[d1, d1] = c, -s, s, c
        off += g
    return R


@pytest.mark.parametrize("split", [(44, 42, 42), (22, 21, 21)])
def test_pair_rotation_commutes_with_rope(split):
    """The per-pair rotation commutes with every 3D-RoPE rotation (so it can be merged into RoPE), is orthogonal,
    and a Hadamard mixing of pairs does not commute (the reason the Hadamard variant runs after RoPE)."""
    R = _pair_matrix(split, O.pair_phase())
    D = sum(split)
    assert np.allclose(R @ R.T, np.eye(D), atol=1e-14)
    rng = _rng(41)
    for _ in range(5):
        coord = rng.integers(0, 50, 3)
        M = BF.rope_matrix(coord, split, 10000.0)
        assert np.allclose(M @ R, R @ M, atol=1e-12)
    if D == 128:
        H = BF.sylvester(D) / math.sqrt(D)
        M = BF.rope_matrix((3, 5, 7), split, 10000.0)
        assert not np.allclose(M @ H, H @ M, atol=1e-3)


@pytest.mark.parametrize("split,prefix", [((44, 42, 42), 0), ((22, 21, 21), 5)])
def test_pair_rotation_folded_equals_rope_then_rotation(split, prefix):
    """RoPE with the phase folded into its angles equals the dense RoPE matrix followed by the dense pair rotation
    (text tokens: the pair rotation alone), to float32 rounding."""
    rng = _rng(42)
    grid = (2, 3, 4)
    D = sum(split)
    L = prefix + 24
    x = rng.standard_normal((L, D)).astype(np.float32)
    got = O.apply_rope(x, prefix, grid, split, 10000.0, O.pair_phase()).astype(np.float64)
    R = _pair_matrix(split, O.pair_phase())
    for n in range(L):
        c = BF.coords_of(n, prefix, grid)
        M = np.eye(D) if c is None else BF.rope_matrix(c, split, 10000.0)
        want = x[n].astype(np.float64) @ M @ R
        assert np.allclose(got[n], want, rtol=0, atol=4e-6 * (1 + np.abs(want).max())), n


def test_pair_rotation_preserves_qk_and_spreads_outliers():
    """Q' K'^T equals RoPE(Q) RoPE(K)^T; a pair whose energy sits in one dim is split evenly over both."""
    rng = _rng(43)
    grid, split = (1, 4, 8), (44, 42, 42)
    q = rng.standard_normal((32, 128)).astype(np.float32)
    k = rng.standard_normal((32, 128)).astype(np.float32)
    a = O.apply_rope(q, 0, grid, split, 10000.0, O.pair_phase()).astype(np.float64)
    b = O.apply_rope(k, 0, grid, split, 10000.0, O.pair_phase()).astype(np.float64)
    qr = O.apply_rope(q, 0, grid, split, 10000.0).astype(np.float64)
    kr = O.apply_rope(k, 0, grid, split, 10000.0).astype(np.float64)
    assert np.allclose(a @ b.T, qr @ kr.T, rtol=1e-5, atol=1e-4)
    # text token with (x0, x1) = (1, 0) in every pair: both dims become 1/sqrt(2)
    e = np.zeros((1, 128), np.float32)
    e[0, 0::2] = 1.0
    y = O.apply_rope(e, 1, (0, 0, 0), split, 10000.0, O.pair_phase())
    assert np.allclose(np.abs(y[0]), 1 / math.sqrt(2), atol=1e-7)
