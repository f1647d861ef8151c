"""Scalar brute-force re-computations for pinning the vectorized oracle on tiny inputs.

Everything here is written with explicit Python loops over tokens, pairs,
blocks and keys, so that an indexing, transposition or vectorization mistake
in the numpy oracle shows up as a disagreement. Dense matrices are built from
their definitions (Sylvester's Kronecker recursion, 2x2 rotation blocks) rather
than from butterflies.
"""
from __future__ import annotations

import math

import numpy as np

F32 = np.float32


def sylvester(n: int) -> np.ndarray:
    """Dense H_n by the Kronecker recursion H_2n = H_2 (x) H_n."""
    H = np.array([[1.0]])
    H2 = np.array([[1.0, 1.0], [1.0, -1.0]])
    while H.shape[0] < n:
        H = np.kron(H2, H)
    return H


def rope_matrix(coord, split, base: float) -> np.ndarray:
    """Dense D x D float64 rotation of one video token, from 2x2 blocks.

    Pair (2i, 2i+1) of group a (counted from the group start) turns by
    coord[a] * base ** (-2i / (2 * floor(g / 2))); an odd group's last dim
    is left alone. Applied as a row vector: y = x @ M.
    """
    D = sum(split)
    M = np.eye(D)
    off = 0
    for a, g in enumerate(split):
        npair = g // 2
        for i in range(npair):
            th = base ** (-(2.0 * i) / (2 * npair))
            ang = coord[a] * th
            c, s = math.cos(ang), math.sin(ang)
            d0, d1 = off + 2 * i, off + 2 * i + 1
            # y0 = x0 c - x1 s ; y1 = x0 s + x1 c   (row-vector convention)
            M[d0, d0] = c
            M[d1, d0] = -s
            M[d0, d1] = s
            M[d1, d1] = c
        off += g
    return M


def coords_of(n: int, prefix: int, grid):
    T, Hh, W = grid
    if n < prefix:
        return None
    i = n - prefix
    t = i // (Hh * W)
    rem = i - t * Hh * W
    return (t, rem // W, rem % W)


def flash_brute(qc, sq, kc, sk, vc, sv, L: int, D: int, rows, key_blocks=None):
    """Per-row, per-key scalar loop of the INT4 flash recurrence (float32 scalars).

    S2 = float32(float32(acc) * c); P = float32(2 ** float32(S2 - m)); the P
    code is rne(float32(15 P)) - 8 and the row sum adds P.

    Returns (out float64 [R, Dv], pq int [R, Lp]).
    """
    nb = (L + 63) // 64
    if key_blocks is None:
        key_blocks = [True] * nb
    c0 = F32(math.log2(math.e) / math.sqrt(D))
    Dv = vc.shape[1]
    Dq = qc.shape[1]
    outs = []
    pqs = []
    for r in rows:
        m = F32(-np.inf)
        l = 0.0
        O = [0.0] * Dv
        pq_row = [0] * (nb * 64)
        cq = F32(F32(sq[r // 64]) * c0)
        for j in range(nb):
            if not key_blocks[j]:
                continue
            c = F32(cq * F32(sk[j]))
            s2 = []
            for kk in range(64 * j, 64 * j + 64):
                if kk >= L:
                    s2.append(None)
                    continue
                acc = 0
                for d in range(Dq):
                    acc += int(qc[r, d]) * int(kc[kk, d])
                s2.append(F32(F32(acc) * c))
            mb = max(e for e in s2 if e is not None)
            m_new = F32(max(m, mb))
            alpha = 0.0 if m == -np.inf else 2.0 ** float(F32(m - m_new))
            psum = 0.0
            accpv = [0] * Dv
            for t, kk in enumerate(range(64 * j, 64 * j + 64)):
                P = F32(0.0) if s2[t] is None else F32(2.0 ** float(F32(s2[t] - m_new)))
                q = int(np.rint(F32(F32(15.0) * P))) - 8
                pq_row[kk] = q
                psum += float(P)
                for c_ in range(Dv):
                    accpv[c_] += q * int(vc[kk, c_])
            for c_ in range(Dv):
                colsum = sum(int(vc[kk, c_]) for kk in range(64 * j, 64 * j + 64))
                O[c_] = alpha * O[c_] + (accpv[c_] + 8 * colsum)
            l = alpha * l + psum
            m = m_new
        outs.append([O[c_] * float(sv[c_]) / 15.0 / l for c_ in range(Dv)])
        pqs.append(pq_row)
    return np.array(outs), np.array(pqs)


def softmax_attention_brute(q, k, v, scale: float):
    """Textbook softmax(q k^T * scale) v with natural exp, per row, float64 loops."""
    R, Dq = q.shape
    N = k.shape[0]
    out = np.zeros((R, v.shape[1]))
    for r in range(R):
        s = [sum(float(q[r, d]) * float(k[n, d]) for d in range(Dq)) * scale for n in range(N)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = sum(e)
        for n in range(N):
            out[r] += e[n] / z * v[n].astype(np.float64)
    return out
