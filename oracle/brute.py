"""Pure-Python brute force of the CSA/HCA step, for tiny sizes only.

TEST INFRASTRUCTURE ONLY (see csa_oracle.py).  This is a second, independent
realisation of the same definitions, written with explicit loops over Python
floats and complex numbers and sharing no helper with the vectorised oracle:

* pooling walks each window token by token (no sliding-window views);
* rotation multiplies complex numbers (x0 + i x1) * exp(i * pos * f), the
  complex view of rotating a dim pair, instead of the cos/sin formulas;
* selection sorts (score, index) pairs with Python's sort;
* attention sums exponentials in plain loops.

Sources as in csa_oracle.py ("DeepSeek-V4-Pro vs Inkling", Component-by-component
table: CSA, HCA, sink and partial-RoPE rows).
"""
from __future__ import annotations

import cmath
import math


def inv_freq(theta, rope_dim):
    return [theta ** (-(2.0 * i) / rope_dim) for i in range(rope_dim // 2)]


def rotate(vec, pos, freqs):
    """Rotate the last 2*len(freqs) entries of a list, pair by pair, as complex numbers."""
    out = list(vec)
    D = len(vec)
    R = 2 * len(freqs)
    for i, f in enumerate(freqs):
        a = D - R + 2 * i
        zc = complex(vec[a], vec[a + 1]) * cmath.exp(1j * pos * f)
        out[a], out[a + 1] = zc.real, zc.imag
    return out


def compress(kv, z, window, stride, pos0, freqs):
    """kv, z: lists of T rows of C floats.  Returns (entries, positions)."""
    T = len(kv)
    C = len(kv[0]) if T else 0
    entries, positions = [], []
    j = 0
    while j * stride + window <= T:
        first = j * stride
        row = []
        for c in range(C):
            top = max(z[first + t][c] for t in range(window))
            num = 0.0
            den = 0.0
            for t in range(window):
                a = math.exp(z[first + t][c] - top)
                num += a * kv[first + t][c]
                den += a
            row.append(num / den)
        p = pos0 + first + window - 1
        entries.append(rotate(row, p, freqs))
        positions.append(p)
        j += 1
    return entries, positions


def scores(q_idx, w, keys):
    out = []
    for key in keys:
        s = 0.0
        for h in range(len(q_idx)):
            dot = sum(q_idx[h][d] * key[d] for d in range(len(key)))
            if dot > 0.0:
                s += w[h] * dot
        out.append(s)
    return out


def select(sc, positions, q_pos, k):
    cand = [(-sc[j], j) for j in range(len(sc)) if positions[j] <= q_pos]
    cand.sort()
    return sorted(j for _, j in cand[:k])


def attend(q, q_pos, rows, sink, scale, freqs):
    """q: H lists of D floats; rows: U lists of D floats (stored, rotated)."""
    outs, lses = [], []
    for h in range(len(q)):
        qh = rotate(q[h], q_pos, freqs)
        logits = [scale * sum(qh[d] * r[d] for d in range(len(r))) for r in rows]
        top = max(logits + [sink[h]])
        ex = [math.exp(v - top) for v in logits]
        Z = math.exp(sink[h] - top) + sum(ex)
        D = len(qh)
        o = [0.0] * D
        for u, r in enumerate(rows):
            wgt = ex[u] / Z
            for d in range(D):
                o[d] += wgt * r[d]
        outs.append(rotate(o, -q_pos, freqs))
        lses.append(top + math.log(Z))
    return outs, lses


def csa_step(kv, z, pos0, q, q_pos, q_idx, w, keys, sink, k, W, scale, freqs,
             window=8, stride=4):
    """Whole CSA step for one query from the raw stream.

    Raw token i has position pos0 + i; the window rows are the raw tokens with
    positions in (q_pos - W, q_pos], rotated at their own positions.
    """
    entries, positions = compress(kv, z, window, stride, pos0, freqs)
    sc = scores(q_idx, w, keys[:len(entries)])
    sel = select(sc, positions, q_pos, k)
    win = [rotate(kv[i], pos0 + i, freqs) for i in range(len(kv))
           if q_pos - W < pos0 + i <= q_pos]
    rows = [entries[j] for j in sel] + win
    o, lse = attend(q, q_pos, rows, sink, scale, freqs)
    return o, lse, sel, sc


def hca_step(kv, z, pos0, q, q_pos, sink, W, scale, freqs, window, stride):
    entries, positions = compress(kv, z, window, stride, pos0, freqs)
    rows = [entries[j] for j in range(len(entries)) if positions[j] <= q_pos]
    rows += [rotate(kv[i], pos0 + i, freqs) for i in range(len(kv))
             if q_pos - W < pos0 + i <= q_pos]
    return attend(q, q_pos, rows, sink, scale, freqs)


def out_projection(o, wa, wb):
    """Grouped low-rank output projection with explicit loops (tiny sizes only).
    o: T x H x D nested lists; wa: G x R x (H/G * D); wb: hidden x (G * R).  Returns y: T x hidden."""
    T, H, D = len(o), len(o[0]), len(o[0][0])
    G, R = len(wa), len(wa[0])
    hg = H // G
    y = []
    for t in range(T):
        cat = []
        for g in range(G):
            flat = []
            for h in range(g * hg, (g + 1) * hg):
                flat.extend(o[t][h])
            for r in range(R):
                acc = 0.0
                for k, x in enumerate(flat):
                    acc += wa[g][r][k] * x
                cat.append(acc)
        row = []
        for j in range(len(wb)):
            acc = 0.0
            for k, x in enumerate(cat):
                acc += wb[j][k] * x
            row.append(acc)
        y.append(row)
    return y
