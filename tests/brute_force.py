"""Pure-Python brute force for tiny cases: the definitions written as loops.

Used only to pin the numpy oracle.  Every quantity is computed element by
element with `math`, with no numpy, so a mistake in the oracle's vectorised
indexing (a transposed operand, a wrong head mapping, an off-by-one mask)
shows up as a mismatch.
"""
import math

NEG = float("-inf")


def dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def softmax_attend_row(logit_by_key, v_rows):
    """logit_by_key: dict key -> logit; v_rows: dict key -> vector."""
    if not logit_by_key:
        return None, NEG
    m = max(logit_by_key.values())
    w = {j: math.exp(s - m) for j, s in logit_by_key.items()}
    z = sum(w.values())
    D = len(next(iter(v_rows.values())))
    o = [sum(w[j] * v_rows[j][d] for j in w) / z for d in range(D)]
    return o, m + math.log(z)


def attention(q, k, v, scale, visible):
    """q[i][h][d], k[j][g][d]; visible(i, j) -> bool.  Returns O[i][h], LSE[h][i]."""
    L, Hq = len(q), len(q[0])
    Hkv = len(k[0])
    G = Hq // Hkv
    O = [[None] * Hq for _ in range(L)]
    lse = [[NEG] * L for _ in range(Hq)]
    for i in range(L):
        for h in range(Hq):
            g = h // G
            lg = {j: scale * dot(q[i][h], k[j][g]) for j in range(len(k)) if visible(i, j)}
            vr = {j: v[j][g] for j in lg}
            o, l = softmax_attend_row(lg, vr)
            O[i][h] = o
            lse[h][i] = l
    return O, lse


def block_scores(q, k, scale, block):
    L, Hq = len(q), len(q[0])
    G = Hq // len(k[0])
    nblk = (len(k) + block - 1) // block
    M = [[NEG] * nblk for _ in range(L)]
    for i in range(L):
        for h in range(Hq):
            for j in range(len(k)):
                if j <= i:
                    s = scale * dot(q[i][h], k[j][h // G])
                    c = j // block
                    if s > M[i][c]:
                        M[i][c] = s
    return M


def tile_token_scores(q, k, scale, tile):
    L, Hq = len(q), len(q[0])
    G = Hq // len(k[0])
    nt = (L + tile - 1) // tile
    T = [[NEG] * len(k) for _ in range(nt)]
    for i in range(L):
        t = i // tile
        for h in range(Hq):
            for j in range(len(k)):
                if j <= i:
                    s = scale * dot(q[i][h], k[j][h // G])
                    if s > T[t][j]:
                        T[t][j] = s
    return T


def topk(x, k):
    cand = [c for c in range(len(x)) if x[c] == x[c] and x[c] > NEG]
    chosen = sorted(sorted(cand, key=lambda c: (-x[c], c))[:k])
    return chosen + [-1] * (k - len(chosen)), len(chosen)


def sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z))
