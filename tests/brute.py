"""Pure-Python, loop-by-loop brute force of the block and the DiT for tiny
shapes.  It is written element by element from the pages' definitions, in a
different form from the vectorised oracle (no NumPy arithmetic: lists and the
`math` module only), so that an indexing, transposition or sign slip in the
oracle shows up as a disagreement.  Only usable for a handful of rows.

Definitions followed ("gizai:dit" reference: Block.forward, Modulation,
gluRows, prepOf, sinusoids; "Host contract -- RGBA-Image-2.1-Turbo" s.4 for
positions and rotary angles, s.6 for the Euler loop).
"""

import math


def mat(a):
    return [list(map(float, r)) for r in a]


def vec(a):
    return [float(v) for v in a]


def matvec(W, x):
    # y[o] = sum_i W[o][i] * x[i]   (W stored [out][in])
    out = []
    for o in range(len(W)):
        s = 0.0
        for i in range(len(x)):
            s += W[o][i] * x[i]
        out.append(s)
    return out


def silu(z):
    return z / (1.0 + math.exp(-z))


def time_embed(t, dim):
    half = dim // 2
    arg = 1000.0 * t
    c = [math.cos(arg * 10000.0 ** (-i / half)) for i in range(half)]
    s = [math.sin(arg * 10000.0 ** (-i / half)) for i in range(half)]
    return c + s


def angles(pos_row, axes, theta=10000.0):
    """Per pair p of the head: the angle of its axis at this token."""
    out = []
    for a, d in enumerate(axes):
        for j in range(d // 2):
            out.append(pos_row[a] * theta ** (-(2.0 * j) / d))
    return out


def layernorm(row, eps):
    n = len(row)
    mu = sum(row) / n
    var = sum((v - mu) ** 2 for v in row) / n
    return [(v - mu) / math.sqrt(var + eps) for v in row]


def rmsnorm(row, w, eps):
    n = len(row)
    ms = sum(v * v for v in row) / n
    r = 1.0 / math.sqrt(ms + eps)
    return [row[i] * r * (1.0 if w is None else w[i]) for i in range(n)]


def block(x, W, vecc, ang, D, H, hd, F, eps=1e-6, qk_eps=1e-6, rms=False):
    """x: list of S rows (lists of D); W: dict of nested lists; vecc: [D];
    ang: per row the list of hd/2 pair angles.  Returns the new rows."""
    S = len(x)
    sv = [silu(v) for v in vecc]
    m = matvec(W["w_mod"], sv)
    shift_a, scale_a, gate_a = m[0:D], m[D:2 * D], m[2 * D:3 * D]
    shift_m, scale_m, gate_m = m[3 * D:4 * D], m[4 * D:5 * D], m[5 * D:6 * D]

    def modnorm(row, shift, scale, nw):
        n = rmsnorm(row, nw, eps) if rms else layernorm(row, eps)
        return [n[i] * (1.0 + scale[i]) + shift[i] for i in range(D)]

    # queries, keys, values per row and head
    Q = [[None] * H for _ in range(S)]
    K = [[None] * H for _ in range(S)]
    V = [[None] * H for _ in range(S)]
    for r in range(S):
        hrow = modnorm(x[r], shift_a, scale_a, W.get("norm1"))
        qkv = matvec(W["w_qkv"], hrow)
        for h in range(H):
            q = qkv[h * hd:(h + 1) * hd]
            k = qkv[H * hd + h * hd:H * hd + (h + 1) * hd]
            v = qkv[2 * H * hd + h * hd:2 * H * hd + (h + 1) * hd]
            q = rmsnorm(q, W["q_norm"], qk_eps)
            k = rmsnorm(k, W["k_norm"], qk_eps)
            qr, kr = [0.0] * hd, [0.0] * hd
            for p in range(hd // 2):
                c, s = math.cos(ang[r][p]), math.sin(ang[r][p])
                qr[2 * p] = q[2 * p] * c - q[2 * p + 1] * s
                qr[2 * p + 1] = q[2 * p] * s + q[2 * p + 1] * c
                kr[2 * p] = k[2 * p] * c - k[2 * p + 1] * s
                kr[2 * p + 1] = k[2 * p] * s + k[2 * p + 1] * c
            Q[r][h], K[r][h], V[r][h] = qr, kr, v
    y = []
    for r in range(S):
        o = []
        for h in range(H):
            sc = []
            for j in range(S):
                sc.append(sum(Q[r][h][e] * K[j][h][e] for e in range(hd)) / math.sqrt(hd))
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            den = sum(ex)
            for e in range(hd):
                o.append(sum(ex[j] * V[j][h][e] for j in range(S)) / den)
        proj = matvec(W["w_out"], o)
        x1 = [x[r][i] + gate_a[i] * proj[i] for i in range(D)]
        h2 = modnorm(x1, shift_m, scale_m, W.get("norm2"))
        u = matvec(W["w_up"], h2)
        a = [silu(u[2 * j]) * u[2 * j + 1] for j in range(F)]
        dn = matvec(W["w_down"], a)
        y.append([x1[i] + gate_m[i] * dn[i] for i in range(D)])
    return y
