"""A second, independent statement of the CSA/HCA chain in plain Python loops.

Test infrastructure: it exists only to check the float64 oracle on tiny inputs.
It uses lists of Python floats and the math/cmath modules (no numpy arithmetic,
no code shared with the oracle), and follows the page "CSA And HCA: Definition,
State, And Cost Model":

  section 1    completed entries s < floor((t+1)/r)
  section 2.1  CSA entry i: one per-channel softmax over the a-rows of block i
               (logit Z^a + B^a) and the b-rows of block i-1 (logit Z^b + B^b)
  section 2.2  HCA entry i: one stream over block i
  section 3.1  I[t][s] = sum_h w[t][h] * ReLU(q[t][h] . K[s]); top-k entries
  section 5.1  one candidate list: compressed entries, then the window
  section 5.2  RMSNorm; RoPE on the last rope_dims channels (pairs as complex numbers);
               inverse RoPE of the output at t
  section 5.3  sink logit in the denominator only

Readings shared with the oracle (they are readings of the pages, not code):
bias rows B^a then B^b; i = 0 has no b-stream; top-k ties to the lower index;
RoPE pairs (2i, 2i+1) of the rotated slice with angle pos * base^(-2i/rope_dims).
"""
from __future__ import annotations

import cmath
import math


def rmsnorm(x, gamma=None, eps=0.0):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * (1.0 if gamma is None else gamma[i]) for i, v in enumerate(x)]


def rope(x, pos, rd, base=10000.0):
    y = list(x)
    c = len(y)
    for i in range(rd // 2):
        a = c - rd + 2 * i
        z = complex(y[a], y[a + 1]) * cmath.exp(1j * pos * base ** (-2.0 * i / rd))
        y[a], y[a + 1] = z.real, z.imag
    return y


def entry(C, Z, B, i, c, m, overlap, gamma=None, eps=1e-6, rd=0, base=10000.0):
    """C, Z: lists of rows (absolute positions from 0); B: list of bias rows."""
    out = []
    for ch in range(c):
        terms = []  # (logit, value)
        for j in range(m):
            p = m * i + j
            terms.append((Z[p][ch] + B[j][ch], C[p][ch]))
        if overlap and i > 0:
            for j in range(m):
                p = m * (i - 1) + j
                terms.append((Z[p][c + ch] + B[m + j][ch], C[p][c + ch]))
        mx = max(l for l, _ in terms)
        den = sum(math.exp(l - mx) for l, _ in terms)
        out.append(sum(math.exp(l - mx) * v for l, v in terms) / den)
    if gamma is not None:
        out = rmsnorm(out, gamma, eps)
    if rd:
        out = rope(out, r_anchor(i, m), rd, base)
    return out


def r_anchor(i, r):
    return float(r * i)


def score(qI_t, KI_s, wI_t):
    tot = 0.0
    for h, qh in enumerate(qI_t):
        d = sum(a * b for a, b in zip(qh, KI_s))
        tot += wI_t[h] * (d if d > 0.0 else 0.0)
    return tot


def topk(scores, k):
    """Indices of the k largest scores (lower index first among equals), ascending."""
    order = sorted(range(len(scores)), key=lambda s: (-scores[s], s))
    return sorted(order[:k])


def attend(q_t, t, comp_rows, local, w, *, q_gamma=None, kv_gamma=None, eps=1e-6, rd=0,
           base=10000.0, sink=None, scale=None):
    """All heads of query t.  comp_rows: stored compressed rows (used as given); local:
    raw local rows by absolute position (normalised, turned at their position)."""
    c = len(q_t[0])
    scale = 1.0 / math.sqrt(c) if scale is None else scale
    cands = [list(r) for r in comp_rows]
    for j in range(max(0, t - w + 1), t + 1):
        v = rmsnorm(local[j], kv_gamma, eps) if kv_gamma is not None else list(local[j])
        cands.append(rope(v, float(j), rd, base) if rd else v)
    outs = []
    for h, qh in enumerate(q_t):
        qv = rmsnorm(qh, q_gamma, eps) if q_gamma is not None else list(qh)
        if rd:
            qv = rope(qv, float(t), rd, base)
        z = [scale * sum(a * b for a, b in zip(qv, v)) for v in cands]
        mx = max(z + ([sink[h]] if sink is not None else []))
        e = [math.exp(x - mx) for x in z]
        den = sum(e) + (math.exp(sink[h] - mx) if sink is not None else 0.0)
        o = [sum(e[u] * cands[u][i] for u in range(len(cands))) / den for i in range(c)]
        outs.append(rope(o, -float(t), rd, base) if rd else o)
    return outs


def csa_chain(P):
    """Whole CSA prefill of P['n'] tokens from t = 0: both compressors, indexer, top-k and
    attention.  Returns dict(kv, KI, scores, idx, out)."""
    n, c, cI, m, k, w, rd = (P[x] for x in ("n", "c", "cI", "m", "k", "w", "rd"))
    E = n // m
    kv = [entry(P["C"], P["Z"], P["B"], i, c, m, True, P["gamma"], P["eps"], rd) for i in range(E)]
    KI = [entry(P["CI"], P["ZI"], P["BI"], i, cI, m, True, P["gammaI"], P["eps"], 0)
          for i in range(E)]
    scores, sel, out = [], [], []
    for t in range(n):
        Et = (t + 1) // m
        s = [score(P["qI"][t], KI[e], P["wI"][t]) for e in range(Et)]
        chosen = topk(s, k)
        scores.append(s)
        sel.append(chosen)
        out.append(attend(P["q"][t], t, [kv[e] for e in chosen], P["local"], w,
                          q_gamma=P["gamma"], kv_gamma=P["gamma"], eps=P["eps"], rd=rd,
                          sink=P["sink"]))
    return dict(kv=kv, KI=KI, scores=scores, idx=sel, out=out)


def hca_chain(P):
    """Whole HCA prefill: one-stream compressor with ratio m', dense attention."""
    n, c, mp, w, rd = (P[x] for x in ("n", "c", "mp", "w", "rd"))
    E = n // mp
    kv = [entry(P["C"], P["Z"], P["B"], i, c, mp, False, P["gamma"], P["eps"], rd)
          for i in range(E)]
    out = [attend(P["q"][t], t, kv[: (t + 1) // mp], P["local"], w, q_gamma=P["gamma"],
                  kv_gamma=P["gamma"], eps=P["eps"], rd=rd, sink=P["sink"]) for t in range(n)]
    return dict(kv=kv, out=out)
