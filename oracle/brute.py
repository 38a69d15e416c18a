"""Brute-force pair enumeration for tiny cases (n <= 64), pure Python.

TEST INFRASTRUCTURE ONLY. Written independently of ``oracle.c``: every
(i, j) pair is tested with the pages' own description of the pattern --
nearby tokens always see each other (|i - j| <= w), far tokens only when they
share a group, and never a later token (Korean page "Why Attend to
Everything? Focus is the Key", technical summary §2.1; Japanese page "Focus:
Learning Which Attention Pairs Matter", technical summary §2.1-§2.2) -- and
the softmax is taken over exactly the kept pairs (exact softmax, §2.1 of the
Korean page).
"""
import math


def bf16_to_float(bits: int) -> float:
    """Value of a bf16 bit pattern, decoded from sign, exponent and mantissa."""
    sign = -1.0 if bits & 0x8000 else 1.0
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0:
        return sign * man * 2.0 ** (-133)          # subnormal: man/2^7 * 2^-126
    if exp == 0xFF:
        return sign * math.inf if man == 0 else math.nan
    return sign * (1.0 + man / 128.0) * 2.0 ** (exp - 127)


def keeps(i: int, j: int, w: int, gi: int, gj: int) -> bool:
    if j > i:                      # causal
        return False
    near = abs(i - j) <= w         # local window, any group
    return near or gi == gj        # far: same group only


def attention(q, k, v, ids, w, scale):
    """q: [Hq][n][d], k/v: [Hkv][n][d] nested lists of bf16 bit patterns
    (one batch element); ids: [n]. Returns (out [Hq][n][d], weights [Hq][n][n])."""
    Hq, Hkv = len(q), len(k)
    n, d = len(q[0]), len(q[0][0])
    share = Hq // Hkv
    out, weights = [], []
    for h in range(Hq):
        kv = h // share
        Kf = [[bf16_to_float(x) for x in row] for row in k[kv]]
        Vf = [[bf16_to_float(x) for x in row] for row in v[kv]]
        oh, wh = [], []
        for i in range(n):
            qi = [bf16_to_float(x) for x in q[h][i]]
            scores = {}
            for j in range(n):
                if keeps(i, j, w, ids[i], ids[j]):
                    scores[j] = scale * math.fsum(a * b for a, b in zip(qi, Kf[j]))
            top = max(scores.values())
            ex = {j: math.exp(s - top) for j, s in scores.items()}
            tot = math.fsum(ex.values())
            row_w = [ex.get(j, 0.0) / tot for j in range(n)]
            oh.append([math.fsum(row_w[j] * Vf[j][c] for j in scores) for c in range(d)])
            wh.append(row_w)
        out.append(oh)
        weights.append(wh)
    return out, weights


def keeps_sets(i: int, j: int, w: int, gi, gj) -> bool:
    """Multi-membership rule (Korean page §2.3, Japanese page §2.2: a token
    may belong to its top-k groups): far pairs are kept when the two tokens
    have at least one group in common."""
    if j > i:
        return False
    if abs(i - j) <= w:
        return True
    return len(set(gi) & set(gj)) > 0


def attention_sets(q, k, v, groups, w, scale):
    """As attention(), with groups[i] the collection of token i's groups.
    Returns (out [Hq][n][d], kept-pair counts [Hq][n])."""
    Hq, Hkv = len(q), len(k)
    n, d = len(q[0]), len(q[0][0])
    share = Hq // Hkv
    out, counts = [], []
    for h in range(Hq):
        kv = h // share
        Kf = [[bf16_to_float(x) for x in row] for row in k[kv]]
        Vf = [[bf16_to_float(x) for x in row] for row in v[kv]]
        oh, ch = [], []
        for i in range(n):
            qi = [bf16_to_float(x) for x in q[h][i]]
            scores = {}
            for j in range(n):
                if keeps_sets(i, j, w, groups[i], groups[j]):
                    scores[j] = scale * math.fsum(a * b for a, b in zip(qi, Kf[j]))
            top = max(scores.values())
            ex = {j: math.exp(s - top) for j, s in scores.items()}
            tot = math.fsum(ex.values())
            oh.append([math.fsum(ex[j] / tot * Vf[j][c] for j in scores) for c in range(d)])
            ch.append(len(scores))
        out.append(oh)
        counts.append(ch)
    return out, counts


def soft_gate_attention(q, k, v, G, w, scale, lam):
    """Training-time soft gate (Japanese page §2.1-§2.2, Korean page §2.1),
    pair by pair: every causal pair is kept; a pair further apart than the
    window is weighted by the logistic function of lam times the dot product
    of the two tokens' soft assignments; the softmax is renormalised over the
    weighted pairs. G: [n][K] floats. Returns out [Hq][n][d]."""
    Hq, Hkv = len(q), len(k)
    n, d = len(q[0]), len(q[0][0])
    share = Hq // Hkv
    out = []
    for h in range(Hq):
        kv = h // share
        Kf = [[bf16_to_float(x) for x in row] for row in k[kv]]
        Vf = [[bf16_to_float(x) for x in row] for row in v[kv]]
        oh = []
        for i in range(n):
            qi = [bf16_to_float(x) for x in q[h][i]]
            logits = [scale * math.fsum(a * b for a, b in zip(qi, Kf[j])) for j in range(i + 1)]
            top = max(logits)
            wts = []
            for j in range(i + 1):
                g = 1.0
                if i - j > w:
                    aff = math.fsum(x * y for x, y in zip(G[i], G[j]))
                    g = 1.0 / (1.0 + math.exp(-lam * aff))
                wts.append(g * math.exp(logits[j] - top))
            tot = math.fsum(wts)
            oh.append([math.fsum(wts[j] / tot * Vf[j][c] for j in range(i + 1)) for c in range(d)])
        out.append(oh)
    return out
