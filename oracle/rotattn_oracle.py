"""CPU oracle for RoPE-aware-rotated INT4 FlashAttention (test infrastructure).

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module. The GPU library
never calls it and shares no code, table or constant generator with it.

What it computes, step by step, in the pages' order:

  1. 3D RoPE on Q and K (RotateAttention abstract: video DiTs with 3D rotary
     position embeddings; the head dim is partitioned into temporal / height /
     width frequency groups). Token order is frame-major [F, H, W]
     (RainFusion2.0, section "3D Window Permutation", default layout).
  2. A Walsh-Hadamard rotation applied after RoPE to Q and K (RotateAttention
     abstract, "RoPE-aware Rotation": the variant applied online at little cost),
     or the mergeable variant folded into RoPE (pair_phase). Either rotation
     is orthonormal, so Q K^T is unchanged.
  3. Symmetric INT4 quantization of Q and K per 64-token block, and of V per
     channel (RotateAttention abstract: mixed-precision INT4 FlashAttention).
  4. The flash loop of RainFusion2.0 section 3.1 "Blockwise Sparse" (the
     online-softmax recurrences for m, P~, l and O, and the final
     O = diag(l)^-1 O), computed here in the log2 domain with integer Q K^T,
     then the range-optimized P quantization of the RotateAttention abstract:
     P = exp(S - max S) lies in [0, 1], and a fixed scale 1/15 with zero-point
     -8 maps it onto the whole INT4 range [-8, 7]; then integer P.V against
     per-channel INT4 V with the zero-point correction 8 * column-sum.
  5. An FP16 path for the blocks and heads where INT4 would lose too much
     accuracy (RotateAttention abstract), using the block mask of RainFusion2.0
     section 3.1 (a tile is skipped by one path and computed by the other),
     and a log-sum-exp merge of the two partial results.
  6. Block-sparse attention (RainFusion2.0 sections 3.1, 3.2, 3.4): block
     means as representative tokens (query blocks of 128 rows, key blocks of
     64), top-n key blocks per query block by the score of the means, the
     first-frame sink on top, and the INT4 loop over the kept key blocks.

Floating point: every step that decides an integer (a Q/K/V code, a block
flag, a P code) is evaluated in float32 with the operation order stated in each
function, because the GPU path takes those decisions in float32. Accumulations
that feed only the floating-point output (O, l) are done in float64. Integer
dot products are computed as float64 matrix products of small integers, which
is exact (|sum| < 2**53).

Where the pages leave a step open, the reading taken is stated in the
docstring of the function that implements it.
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32
F64 = np.float64

BLOCK = 64          # tokens per quantization block and per flash key block
ROT_FULL = 0
ROT_GROUP64 = 1
ROT_PAIR = 2        # the mergeable rotation, fused into RoPE (see pair_phase)


# --------------------------------------------------------------------------
# 1. token positions and 3D RoPE
# --------------------------------------------------------------------------

def token_coords(L: int, prefix: int, grid) -> tuple[np.ndarray, np.ndarray]:
    """(t, h, w) coordinates of every token and a mask of video tokens.

    Reading: text tokens come first (``prefix`` of them) and take no RoPE;
    video tokens follow, flattened frame-major over (t, h, w) as in the
    default [F, H, W] layout of RainFusion2.0 ("3D Window Permutation").
    Coordinates start at 0.
    """
    T, Hh, W = grid
    n = np.arange(L, dtype=np.int64)
    idx = n - prefix
    video = idx >= 0
    ic = np.where(video, idx, 0)
    hw, ww, hh = max(Hh * W, 1), max(W, 1), max(Hh, 1)      # a text-only sequence has an empty grid
    coords = np.stack([ic // hw, (ic // ww) % hh, ic % ww], axis=1)
    return coords, video


def group_offsets(split) -> list[int]:
    offs, o = [], 0
    for g in split:
        offs.append(o)
        o += g
    return offs


def rope_thetas(split, base: float) -> list[list[float]]:
    """Rotation frequency of every pair of every axis group, in float64.

    Reading: each axis group of g dims holds floor(g/2) adjacent pairs
    (2i, 2i+1) counted from the start of the group; an odd group leaves its
    last dim unrotated. Pair i turns by pos * theta_i with
    theta_i = base ** (-2 i / g_rot), g_rot = 2 * floor(g / 2), the usual 1D
    RoPE schedule applied per axis.
    """
    out = []
    for g in split:
        npair = g // 2
        g_rot = 2 * npair
        out.append([base ** (-(2.0 * i) / g_rot) for i in range(npair)])
    return out


def rope_tables(grid, split, base: float, phase: float = 0.0):
    """float32 cos/sin tables per axis: list of (cos[n_pos, npair], sin[n_pos, npair]).

    Angles pos * theta_i + phase and their cos/sin are evaluated in float64
    and rounded once to float32.
    """
    tabs = []
    for a, thetas in enumerate(rope_thetas(split, base)):
        n_pos = grid[a]
        c = np.empty((n_pos, len(thetas)), dtype=F32)
        s = np.empty((n_pos, len(thetas)), dtype=F32)
        for p in range(n_pos):
            for i, th in enumerate(thetas):
                ang = float(p) * th + phase
                c[p, i] = F32(math.cos(ang))
                s[p, i] = F32(math.sin(ang))
        tabs.append((c, s))
    return tabs


def pair_phase() -> float:
    """Angle of the mergeable RoPE-aware rotation (RotateAttention abstract, "RoPE-aware Rotation").

    Reading: the abstract names rotation matrices that can be merged into
    RoPE but does not construct them. An orthogonal R can be merged
    into RoPE (RoPE_pos(x) R = RoPE_pos(x R) for every position, so R can be
    folded into the Q/K projections or into RoPE's tables) exactly when it
    commutes with every 3D-RoPE rotation; with the distinct frequencies of an
    axis group and the independent positions of the three axes, those are the
    matrices that turn each RoPE pair (2i, 2i+1) by a fixed angle in its own
    plane and leave an odd group's unpaired dim alone. The angle taken here
    is pi/4 for every pair: it spreads a pair's energy evenly over its two
    dims, the most a within-pair rotation can flatten a one-dim outlier.
    Folded into RoPE, every pair of a video token turns by pos * theta_i +
    pi/4 and every pair of a text token by pi/4.
    """
    return math.pi / 4


def apply_rope(x32: np.ndarray, prefix: int, grid, split, base: float, phase: float = 0.0) -> np.ndarray:
    """3D RoPE in float32: per pair y0 = x0*c - x1*s, y1 = x0*s + x1*c.

    Each product and each sum is rounded to float32 separately (no fused
    multiply-add). With phase = 0 text tokens are returned unchanged; with a
    phase (the mergeable rotation folded into RoPE, see pair_phase) every
    pair of a video token turns by pos * theta_i + phase and every pair of a
    text token by phase alone, with float32(cos phase), float32(sin phase).
    """
    assert x32.dtype == F32
    L, D = x32.shape
    assert sum(split) == D
    coords, video = token_coords(L, prefix, grid)
    text = ~video
    y = x32.copy()
    tabs = rope_tables(grid, split, base, phase)
    ct, st = F32(math.cos(phase)), F32(math.sin(phase))
    for a, off in enumerate(group_offsets(split)):
        c_tab, s_tab = tabs[a]
        pos = coords[video, a]
        for i in range(c_tab.shape[1]):
            d0, d1 = off + 2 * i, off + 2 * i + 1
            c = c_tab[pos, i]
            s = s_tab[pos, i]
            x0 = x32[video, d0]
            x1 = x32[video, d1]
            y[video, d0] = (x0 * c) - (x1 * s)
            y[video, d1] = (x0 * s) + (x1 * c)
            if phase != 0.0 and text.any():
                t0 = x32[text, d0]
                t1 = x32[text, d1]
                y[text, d0] = (t0 * ct) - (t1 * st)
                y[text, d1] = (t0 * st) + (t1 * ct)
    return y


# --------------------------------------------------------------------------
# 2. Walsh-Hadamard rotation after RoPE
# --------------------------------------------------------------------------

def hadamard_scale(n: int) -> np.float32:
    """float32 nearest to 1/sqrt(n)."""
    return F32(1.0 / math.sqrt(n))


def fwht(x32: np.ndarray) -> np.ndarray:
    """Normalized Walsh-Hadamard transform (Sylvester order) of the last axis, float32.

    Reading: butterfly stages with half-width h = 1, 2, 4, ..., n/2; each
    stage replaces the pair (x[j], x[j+h]) inside every block of 2h values by
    (x[j] + x[j+h], x[j] - x[j+h]) in float32; one float32 multiply by
    float32(1/sqrt(n)) at the end. The result is x . H_n / sqrt(n) with the
    symmetric Sylvester matrix H_1 = [1], H_2n = [[H, H], [H, -H]].
    """
    assert x32.dtype == F32
    n = x32.shape[-1]
    assert n & (n - 1) == 0
    lead = x32.shape[:-1]
    y = x32.copy()
    h = 1
    while h < n:
        y = y.reshape(lead + (n // (2 * h), 2, h))
        a = y[..., 0, :]
        b = y[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2)
        h *= 2
    y = y.reshape(lead + (n,))
    return y * hadamard_scale(n)


def rotate(x32: np.ndarray, rotation: int, split) -> np.ndarray:
    """RoPE-aware rotation x' = x . R applied after RoPE (float32).

    ROT_PAIR: the mergeable rotation; it is applied inside RoPE (see
    pair_phase), so nothing is left to do here.
    ROT_FULL: R = H_D / sqrt(D) over the whole head dim.
    ROT_GROUP64 (reading of "block-diagonal Hadamard per RoPE group, 44 -> pad
    64, 42 -> pad 64"): each RoPE group is zero padded to 64 dims and turned
    by H_64 / 8; the three results are concatenated, so the rotated head dim
    is 192. The kept rows of an orthonormal matrix are orthonormal, so
    x' y'^T = x y^T.
    """
    if rotation == ROT_PAIR:   # already folded into RoPE (apply_rope with pair_phase)
        return x32
    if rotation == ROT_FULL:
        return fwht(x32)
    if rotation == ROT_GROUP64:
        L = x32.shape[0]
        parts = []
        for off, g in zip(group_offsets(split), split):
            assert g <= 64
            pad = np.zeros((L, 64), dtype=F32)
            pad[:, :g] = x32[:, off:off + g]
            parts.append(fwht(pad))
        return np.concatenate(parts, axis=1)
    raise ValueError(rotation)


def rotated_dim(D: int, rotation: int) -> int:
    return 192 if rotation == ROT_GROUP64 else D


# --------------------------------------------------------------------------
# 3. INT4 quantization
# --------------------------------------------------------------------------

def n_blocks(L: int) -> int:
    return (L + BLOCK - 1) // BLOCK


def quantize_sym(x32: np.ndarray, scale: np.float32) -> np.ndarray:
    """Symmetric INT4 codes: clamp(rne(x / s), -7, 7), IEEE float32 division.

    A zero scale gives zero codes.
    """
    if scale == 0:
        return np.zeros(x32.shape, dtype=np.int8)
    q = np.rint(x32 / scale)            # float32 / float32 -> float32, then round half to even
    return np.clip(q, -7, 7).astype(np.int8)


def quantize_qk_blocks(x32: np.ndarray):
    """Per-64-token symmetric INT4 quantization of a rotated Q or K head.

    Reading: the block is 64 consecutive tokens by all rotated dims; the scale
    is s = float32(absmax / 7) over the valid tokens of the block (a ragged
    last block uses only its valid tokens); codes lie in [-7, 7] ("symmetric"
    in the abstract; -8 is never produced). Padded token rows get code 0.

    Also returns the block's quantization noise-to-signal ratio
    NSR = sum (x - s c)^2 / sum x^2 (float64; 0 for an all-zero block), the
    "quantization error" that the 5% block rule compares against.

    Returns codes int8 [Lp, D'], scales float32 [nb], nsr float64 [nb].
    """
    L, Dp = x32.shape
    nb = n_blocks(L)
    codes = np.zeros((nb * BLOCK, Dp), dtype=np.int8)
    scales = np.zeros(nb, dtype=F32)
    nsr = np.zeros(nb, dtype=F64)
    for b in range(nb):
        xb = x32[b * BLOCK:min((b + 1) * BLOCK, L)]
        amax = F32(np.max(np.abs(xb))) if xb.size else F32(0)
        s = F32(amax / F32(7.0))
        c = quantize_sym(xb, s)
        codes[b * BLOCK:b * BLOCK + xb.shape[0]] = c
        scales[b] = s
        x64 = xb.astype(F64)
        sig = float(np.sum(x64 * x64))
        err = x64 - F64(s) * c.astype(F64)
        nsr[b] = float(np.sum(err * err)) / sig if sig > 0 else 0.0
    return codes, scales, nsr


def quantize_v(v16: np.ndarray):
    """Per-channel symmetric INT4 quantization of V over all tokens of a head.

    Reading: s_v[c] = float32(absmax over the L tokens of channel c / 7);
    codes clamp(rne(v / s_v), -7, 7); V is not rotated. colsum[j, c] is the
    integer sum of the codes of key block j in channel c (padded keys are 0).

    Returns codes int8 [Lp, D], scale float32 [D], colsum int32 [nb, D].
    """
    L, D = v16.shape
    nb = n_blocks(L)
    v32 = v16.astype(F32)
    codes = np.zeros((nb * BLOCK, D), dtype=np.int8)
    scale = np.zeros(D, dtype=F32)
    for c in range(D):
        amax = F32(np.max(np.abs(v32[:, c]))) if L else F32(0)
        s = F32(amax / F32(7.0))
        scale[c] = s
        codes[:L, c] = quantize_sym(v32[:, c], s)
    colsum = codes.reshape(nb, BLOCK, D).astype(np.int32).sum(axis=1).astype(np.int32)
    return codes, scale, colsum


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two INT4 codes per byte: dim 2k in the low nibble, dim 2k+1 in the high nibble (two's complement)."""
    c = codes.astype(np.int16)
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    p = packed.astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# --------------------------------------------------------------------------
# 4. the INT4 flash loop
# --------------------------------------------------------------------------

def softmax_c0(D: int) -> np.float32:
    """float32(log2(e) / sqrt(D)): the softmax scale 1/sqrt(d) of RainFusion2.0 section 3.1, in the log2 domain.

    Reading: d is the nominal head dim (128 or 64), also when the rotated
    dim is 192.
    """
    return F32(math.log2(math.e) / math.sqrt(D))


def p_codes(P32: np.ndarray) -> np.ndarray:
    """Range-optimized P quantization: pq = rne(float32(15 * P)) - 8.

    P = exp(S - max S) is in [0, 1]; the fixed scale 1/15 and zero-point -8
    send 0 to -8 and 1 to 7, the whole INT4 range (RotateAttention abstract,
    "Range-optimized P Quantization"). The product 15 * P is rounded to
    float32, then to the nearest integer with ties to even.
    """
    return (np.rint(F32(15.0) * np.asarray(P32, dtype=F32)) - 8).astype(np.int8)


def exp2_f32(x32: np.ndarray) -> np.ndarray:
    """2 ** x for float32 x, evaluated in float64 and rounded once to float32 (-inf -> 0)."""
    return np.exp2(np.asarray(x32, dtype=F32).astype(F64)).astype(F32)


def int4_flash_rows(qc, sq, kc, sk, vc, sv, colsum, L: int, D: int, rows, key_blocks=None,
                    quantize_p: bool = True, dump: bool = False):
    """The INT4 flash loop for a set of query rows of one head.

    qc, kc: int8 codes [Lp, D'] (any real-valued arrays when quantize_p is
    False and the caller wants the unquantized loop); sq, sk: float32 block
    scales; vc: V codes [Lp, D]; sv: float32 [D]; colsum: int32 [nb, D].
    rows: query token indices. key_blocks: bool [nb] of key blocks this
    path processes (default all), visited in ascending order.

    Per key block j, for every row (RainFusion2.0 section 3.1, with
    exp -> exp2 and the scale folded into the log2 domain):
      acc   = q . k over the rotated dims                 (exact integer)
      c     = float32(float32(sq * c0) * sk[j])
      S2    = float32(float32(acc) * c)                   (padded keys: -inf)
      m'    = max(m, rowmax S2)                           (m starts at -inf)
      P     = float32(2 ** float32(S2 - m'))              in [0, 1]
      pq    = p_codes(P) = rne(float32(15 P)) - 8         (in [-8, 7])
      l     = 2**(m - m') l + rowsum P                    (the unquantized P)
      accPV = pq . v + 8 * colsum[j]                      (exact integer)
      O     = 2**(m - m') O + accPV
    Final: O_scaled = O * s_v / 15 and out = O_scaled / l.

    Reading: the running max advances per key block of 64 keys in ascending
    order (the P codes depend on it), skipping blocks not in key_blocks; the
    row sum l uses the unquantized P. 2 ** x is evaluated in float64 and
    rounded once to float32; l and O accumulate in float64.

    With quantize_p=False the loop keeps P unquantized and accumulates
    P . v directly (no codes, no colsum): the plain FlashAttention recurrence.

    Returns a dict with O_scaled [R, D] float64, m [R] (float32 values), l [R]
    float64, and when dump=True the per-block int32 acc [R, Lp], int8 pq
    [R, Lp], float32 P [R, Lp], int32 accPV [R, nb, D] (0 for skipped blocks)
    and the running max after every block m_hist [R, nb].
    """
    rows = np.asarray(rows, dtype=np.int64)
    R = rows.size
    nb = n_blocks(L)
    if key_blocks is None:
        key_blocks = np.ones(nb, dtype=bool)
    c0 = softmax_c0(D)
    cq = (sq[rows // BLOCK].astype(F32) * c0).astype(F32)
    Qf = np.asarray(qc[rows], dtype=F64)
    Dv = vc.shape[1]
    m = np.full(R, -np.inf, dtype=F32)
    l = np.zeros(R, dtype=F64)
    O = np.zeros((R, Dv), dtype=F64)
    if dump:
        d_acc = np.zeros((R, nb * BLOCK), dtype=np.int32)
        d_pq = np.zeros((R, nb * BLOCK), dtype=np.int8)
        d_p = np.zeros((R, nb * BLOCK), dtype=F32)
        d_pv = np.zeros((R, nb, Dv), dtype=np.int32)
        d_m = np.full((R, nb), -np.inf, dtype=F32)
    for j in range(nb):
        if not key_blocks[j]:
            if dump:
                d_m[:, j] = m
            continue
        k0 = j * BLOCK
        kk = np.asarray(kc[k0:k0 + BLOCK], dtype=F64)
        valid = (np.arange(k0, k0 + BLOCK) < L)
        acc = Qf @ kk.T                                   # exact small integers (or reals)
        c = (cq * F32(sk[j])).astype(F32)
        S2 = (acc.astype(F32) * c[:, None]).astype(F32)   # float32 product
        S2[:, ~valid] = -np.inf
        m_new = np.maximum(m, S2.max(axis=1)).astype(F32)
        alpha = np.exp2((m - m_new).astype(F64))          # -inf - finite -> -inf -> 0
        P = exp2_f32((S2 - m_new[:, None]).astype(F32))   # float32 difference, then 2 ** x
        P[:, ~valid] = 0
        l = alpha * l + P.astype(F64).sum(axis=1)
        vv = np.asarray(vc[k0:k0 + BLOCK], dtype=F64)
        if quantize_p:
            pq = p_codes(P)
            accpv = pq.astype(F64) @ vv + 8.0 * colsum[j].astype(F64)[None, :]
        else:
            accpv = P.astype(F64) @ vv
        O = alpha[:, None] * O + accpv
        m = m_new
        if dump:
            d_acc[:, k0:k0 + BLOCK] = acc.astype(np.int64)
            d_pq[:, k0:k0 + BLOCK] = pq
            d_p[:, k0:k0 + BLOCK] = P
            d_pv[:, j, :] = accpv.astype(np.int64)
            d_m[:, j] = m
    out = {"O_scaled": O * (sv.astype(F64) / 15.0)[None, :] if quantize_p else O,
           "m": m, "l": l}
    if dump:
        out.update(acc=d_acc, pq=d_pq, P=d_p, accpv=d_pv, m_hist=d_m)
    return out


# --------------------------------------------------------------------------
# 5. FP16 fallback path and merge
# --------------------------------------------------------------------------

def fp16_rows(qr16, kr16, v16, L: int, D: int, rows, key_blocks=None):
    """Exact float64 attention partial of the FP16 fallback path.

    Reading: the fallback path sees RoPE'd, unrotated Q and K rounded to
    float16 and the raw float16 V. Here it is evaluated exactly in float64:
    S2 = (q . k) * log2(e) / sqrt(D) over the keys of ``key_blocks``;
    m = max S2, P = 2**(S2 - m), l = sum P, O = P . V.
    Returns dict(O [R, D], m [R], l [R]) in float64.
    """
    rows = np.asarray(rows, dtype=np.int64)
    nb = n_blocks(L)
    if key_blocks is None:
        key_blocks = np.ones(nb, dtype=bool)
    keymask = np.repeat(key_blocks, BLOCK)[:L]
    keys = np.nonzero(keymask)[0]
    q = qr16[rows].astype(F64)
    k = kr16[keys].astype(F64)
    v = v16[keys].astype(F64)
    S2 = (q @ k.T) * (math.log2(math.e) / math.sqrt(D))
    m = S2.max(axis=1)
    P = np.exp2(S2 - m[:, None])
    return {"O": P @ v, "m": m, "l": P.sum(axis=1)}


def merge(O1, m1, l1, O2, m2, l2):
    """Log-sum-exp merge of two partial results over disjoint key sets (log2 domain).

    m = max(m1, m2); out = (2**(m1-m) O1 + 2**(m2-m) O2) / (2**(m1-m) l1 + 2**(m2-m) l2).
    A partial with m = -inf (no keys) has weight 0.
    """
    m1 = np.asarray(m1, dtype=F64)
    m2 = np.asarray(m2, dtype=F64)
    m = np.maximum(m1, m2)
    a1 = np.where(np.isneginf(m1), 0.0, np.exp2(m1 - m))
    a2 = np.where(np.isneginf(m2), 0.0, np.exp2(m2 - m))
    return (a1[:, None] * O1 + a2[:, None] * O2) / (a1 * l1 + a2 * l2)[:, None]


# --------------------------------------------------------------------------
# 6. block-sparse mask (RainFusion2.0, sections 3.1, 3.2 and 3.4)
# --------------------------------------------------------------------------

def sink_end(L: int, prefix: int, grid) -> int:
    """Tokens [0, sink_end) take part in full attention: the text prefix and the first video frame.

    RainFusion2.0 section 3.4 "First Frame Sink": the queries of the first
    frame attend to every key and every query attends to the keys of the
    first frame; the first-frame tokens are grouped with the text tokens so
    that both take part in full attention. Reading: in the token order used
    here (text prefix, then frames 0, 1, ... in [F, H, W] order) that set is
    the prefix followed by the grid_h * grid_w tokens of frame 0.
    """
    T, Hh, W = grid
    return min(L, prefix + (Hh * W if T > 0 else 0))


def block_means(x16, prefix, grid, split, base, size: int = BLOCK) -> np.ndarray:
    """Representative token of every block of `size` tokens (RainFusion2.0 section 3.2).

    The block mean of the RoPE'd rows (RoPE in float32 as in apply_rope),
    averaged in float64 over the block's valid tokens (a ragged last block
    averages only its tokens below L). Reading: the means are taken on the
    RoPE'd Q and K, the vectors whose products the attention scores are;
    the Hadamard rotation would not change any score (it is orthonormal).
    Returns float64 [ceil(L / size), D].
    """
    xr = apply_rope(x16.astype(F32), prefix, grid, split, base)
    L, D = xr.shape
    nb = -(-L // size)
    out = np.zeros((nb, D), dtype=F64)
    for i in range(nb):
        out[i] = xr[i * size:min(L, (i + 1) * size)].astype(F64).mean(axis=0)
    return out


# Query and key block sizes of the block-sparse mask. RainFusion2.0 section
# 3.1 lets b_q and b_k differ; b_k is the 64-key block of the flash loop and
# b_q = 128 query rows (two quantization blocks) share one mask row.
SPARSE_BQ = 128
SPARSE_BK = BLOCK


def block_scores(q_means, k_means) -> np.ndarray:
    """S_hat[i, j] = q_hat_i . k_hat_j (RainFusion2.0 section 3.2), float64 [NBq, NBk].

    No 1/sqrt(d) factor: S_hat only ranks the key blocks of each query block.
    """
    return np.asarray(q_means, dtype=F64) @ np.asarray(k_means, dtype=F64).T


def sparse_block_mask(s_hat, topn: int, L: int, prefix: int, grid, bq: int = SPARSE_BQ,
                      bk: int = SPARSE_BK) -> np.ndarray:
    """Block mask M [ceil(L/bq), ceil(L/bk)] of the block-sparse flash loop (RainFusion2.0 sections 3.1, 3.2, 3.4).

    M[i, j] = 1 for the topn key blocks j with the largest S_hat[i, j]
    (the page selects the n most important key blocks for each query block;
    its top-n over dimension 0 of S_hat is read the same way, per query block;
    equal scores are taken in ascending j), then the first-frame sink on top: every key block
    that holds a sink token is kept for every query block, and every query
    block that holds a sink token keeps every key block.
    """
    s_hat = np.asarray(s_hat, dtype=F64)
    nq, nk = s_hat.shape
    M = np.zeros((nq, nk), dtype=bool)
    n = min(int(topn), nk)
    for i in range(nq):
        order = sorted(range(nk), key=lambda j: (-s_hat[i, j], j))
        M[i, order[:n]] = True
    se = sink_end(L, prefix, grid)
    M[:, :-(-se // bk)] = True                       # key blocks holding a sink token
    M[:-(-se // bq), :] = True                       # query blocks holding a sink token
    return M


def sparse_forward_head(q16, k16, v16, *, prefix, grid, split, base, rotation, topn, block_mask=None,
                        rows=None):
    """Block-sparse INT4 attention of one head (RainFusion2.0 section 3.1: Q_i K_j^T and P_ij V_j
    are skipped where M[i, j] = 0), with the quantized loop of int4_flash_rows.

    Query blocks of SPARSE_BQ rows, key blocks of SPARSE_BK = 64 keys; query
    row r uses mask row r // SPARSE_BQ. block_mask: bool [NBq, NB] to use
    instead of the one computed from the block means (the GPU tests pass the
    mask the GPU chose after checking it against s_hat). Returns dict(out,
    rows, mask, s_hat, q, k, v codes).
    """
    L, D = q16.shape
    qp = qk_prologue(q16, prefix, grid, split, base, rotation)
    kp = qk_prologue(k16, prefix, grid, split, base, rotation)
    vc, sv, colsum = quantize_v(v16)
    s_hat = block_scores(block_means(q16, prefix, grid, split, base, SPARSE_BQ),
                         block_means(k16, prefix, grid, split, base, SPARSE_BK))
    M = sparse_block_mask(s_hat, topn, L, prefix, grid) if block_mask is None else np.asarray(block_mask, bool)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, D), dtype=F64)
    for qb in np.unique(rows // SPARSE_BQ):
        sel = (rows // SPARSE_BQ) == qb
        p1 = int4_flash_rows(qp["codes"], qp["scale"], kp["codes"], kp["scale"], vc, sv, colsum,
                             L, D, rows[sel], key_blocks=M[qb])
        out[sel] = p1["O_scaled"] / p1["l"][:, None]
    return {"out": out, "rows": rows, "mask": M, "s_hat": s_hat, "q": qp, "k": kp, "v_codes": vc,
            "v_scale": sv, "v_colsum": colsum}


# --------------------------------------------------------------------------
# whole path for one head
# --------------------------------------------------------------------------

def qk_prologue(x16, prefix, grid, split, base, rotation):
    """RoPE, rotation and block quantization of one Q or K head [L, D] float16.

    With ROT_PAIR the rotation is folded into RoPE, so "rope32"/"rope16" (the
    FP16 path's inputs) are the rotated vectors; Q K^T is the same either way.
    """
    x32 = x16.astype(F32)
    xr = apply_rope(x32, prefix, grid, split, base, pair_phase() if rotation == ROT_PAIR else 0.0)
    xrot = rotate(xr, rotation, split)
    codes, scales, nsr = quantize_qk_blocks(xrot)
    return {"rope32": xr, "rope16": xr.astype(np.float16), "rot": xrot,
            "codes": codes, "scale": scales, "nsr": nsr}


def forward_head(q16, k16, v16, *, prefix, grid, split, base, rotation, tau=math.inf,
                 head_masked=False, q_flags=None, k_flags=None, rows=None):
    """The whole mixed-precision path for one (batch, head); returns float64 outputs.

    Routing (reading of "Q/K blocks whose quantization error exceeds 5% are
    routed to FP16" and of the per-head fallback mask): block flags are
    NSR > tau; tile (i, j) runs on the FP16 path if the head is masked, or
    query block i is flagged, or key block j is flagged. Query blocks whose
    tiles are all FP16 are computed by the FP16 path alone; query blocks that
    mix both run the INT4 loop over the unflagged key blocks and the FP16
    path over the flagged ones, then merge. ``q_flags``/``k_flags`` override
    the computed flags (used where a flag sits on the threshold).

    rows: query rows to compute (default all). Returns dict(out [R, D]
    float64, rows, q/k prologue dicts, v codes, flags).
    """
    L, D = q16.shape
    nb = n_blocks(L)
    qp = qk_prologue(q16, prefix, grid, split, base, rotation)
    kp = qk_prologue(k16, prefix, grid, split, base, rotation)
    vc, sv, colsum = quantize_v(v16)
    fq = qp["nsr"] > tau if q_flags is None else np.asarray(q_flags, dtype=bool)
    fk = kp["nsr"] > tau if k_flags is None else np.asarray(k_flags, dtype=bool)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, D), dtype=F64)
    rblk = rows // BLOCK
    fp16_row = np.full(rows.size, bool(head_masked)) | fq[rblk]
    any_k = bool(fk.any())
    int4_sel = ~fp16_row
    if int4_sel.any():
        r = rows[int4_sel]
        p1 = int4_flash_rows(qp["codes"], qp["scale"], kp["codes"], kp["scale"], vc, sv, colsum,
                             L, D, r, key_blocks=~fk)
        if any_k:
            p2 = fp16_rows(qp["rope16"], kp["rope16"], v16, L, D, r, key_blocks=fk)
            out[int4_sel] = merge(p1["O_scaled"], p1["m"], p1["l"], p2["O"], p2["m"], p2["l"])
        else:
            out[int4_sel] = p1["O_scaled"] / p1["l"][:, None]
    if fp16_row.any():
        r = rows[fp16_row]
        p2 = fp16_rows(qp["rope16"], kp["rope16"], v16, L, D, r)
        out[fp16_row] = p2["O"] / p2["l"][:, None]
    return {"out": out, "rows": rows, "q": qp, "k": kp, "v_codes": vc, "v_scale": sv,
            "v_colsum": colsum, "q_flags": fq, "k_flags": fk}


def fp16_forward_head(q16, k16, v16, *, prefix, grid, split, base, rows=None):
    """The whole-call FP16 path (fallback for a whole denoising step)."""
    L, D = q16.shape
    qr = apply_rope(q16.astype(F32), prefix, grid, split, base).astype(np.float16)
    kr = apply_rope(k16.astype(F32), prefix, grid, split, base).astype(np.float16)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    p = fp16_rows(qr, kr, v16, L, D, rows)
    return p["O"] / p["l"][:, None]


def exact_attention(q16, k16, v16, *, prefix, grid, split, base, rows=None):
    """Unquantized attention in float64: softmax(RoPE(Q) RoPE(K)^T / sqrt(D)) V.

    RoPE here is evaluated in float64 with float64 cos/sin (no float32
    rounding anywhere), so this is the full-precision reference that the
    cosine-similarity report compares against.
    """
    L, D = q16.shape
    coords, video = token_coords(L, prefix, grid)

    def rope64(x):
        y = x.astype(F64).copy()
        for a, (off, th) in enumerate(zip(group_offsets(split), rope_thetas(split, base))):
            pos = coords[video, a].astype(F64)
            for i, t in enumerate(th):
                ang = pos * t
                c, s = np.cos(ang), np.sin(ang)
                x0 = x[video, off + 2 * i].astype(F64)
                x1 = x[video, off + 2 * i + 1].astype(F64)
                y[video, off + 2 * i] = x0 * c - x1 * s
                y[video, off + 2 * i + 1] = x0 * s + x1 * c
        return y

    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    qq = rope64(q16)[rows]
    kk = rope64(k16)
    S = qq @ kk.T / math.sqrt(D)
    S -= S.max(axis=1, keepdims=True)
    P = np.exp(S)
    return (P @ v16.astype(F64)) / P.sum(axis=1, keepdims=True)


def cosine_similarity(a, b) -> float:
    a = np.asarray(a, dtype=F64).ravel()
    b = np.asarray(b, dtype=F64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
