"""Pure-Python brute force for tiny MoE layers.  TEST INFRASTRUCTURE ONLY.

No numpy, no BLAS: nested loops over Python floats, so that the numpy oracle
(moe_oracle) can be checked against an implementation with a different shape.
The forward is the dense reading of the layer: every token visits EVERY
expert and multiplies its output by a dense gate row that is zero outside the
token's selected experts (the "loop over all experts regardless of tokens"
form of the Nemotron hub code, page "Accelerating Transformers fine-tuning
with NVIDIA NeMo AutoModel", note under the Nemotron 3 Nano table; the eager
backend is the for-loop over selected experts, section 专家后端).

Inputs are nested lists (or anything indexable): x[T][d], Wr[d][E], b[E] or
None, Wg/Wu[E][d][I], Wd[E][I][d].
"""
from __future__ import annotations

import math


def _sig(z):
    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    ez = math.exp(z)
    return ez / (1.0 + ez)


def logits(x, Wr, b, E):
    T, d = len(x), len(x[0])
    out = []
    for t in range(T):
        row = []
        for e in range(E):
            s = 0.0
            for i in range(d):
                s += float(x[t][i]) * float(Wr[i][e])
            if b is not None:
                s += float(b[e])
            row.append(s)
        out.append(row)
    return out


def select(L_row, k):
    """k expert ids, largest logit first, equal logits by lower id."""
    E = len(L_row)
    return sorted(range(E), key=lambda e: (-L_row[e], e))[:k]


def dense_gate(x, Wr, b, E, k, gate):
    """Dense gate matrix G[t][e] (zero for unselected experts) and the selections."""
    T = len(x)
    G = [[0.0] * E for _ in range(T)]
    sel_all = []
    if gate == "balanced":
        P = E // k
        for t in range(T):
            sel = [(t % P) + i * P for i in range(k)]
            for e in sel:
                G[t][e] = 1.0 / k
            sel_all.append(sel)
        return G, sel_all
    L = logits(x, Wr, b, E)
    for t in range(T):
        sel = select(L[t], k)
        m = max(L[t][e] for e in sel)
        z = [math.exp(L[t][e] - m) for e in sel]
        Z = sum(z)
        for e, ze in zip(sel, z):
            G[t][e] = ze / Z
        sel_all.append(sel)
    return G, sel_all


def ffn(v, Wg_e, Wu_e, Wd_e):
    d, I = len(Wg_e), len(Wg_e[0])
    a = []
    for j in range(I):
        hg = 0.0
        hu = 0.0
        for i in range(d):
            hg += float(v[i]) * float(Wg_e[i][j])
            hu += float(v[i]) * float(Wu_e[i][j])
        a.append(hg * _sig(hg) * hu)
    out = []
    for n in range(d):
        s = 0.0
        for j in range(I):
            s += a[j] * float(Wd_e[j][n])
        out.append(s)
    return out


def layer_forward(x, Wr, b, Wg, Wu, Wd, k, gate, E):
    """y[t] = sum over all experts e of G[t][e] * FFN_e(x[t])."""
    G, _ = dense_gate(x, Wr, b, E, k, gate)
    T, d = len(x), len(x[0])
    y = []
    for t in range(T):
        acc = [0.0] * d
        for e in range(E):
            out = ffn(x[t], Wg[e], Wu[e], Wd[e])
            for n in range(d):
                acc[n] += G[t][e] * out[n]
        y.append(acc)
    return y


def stable_groups(idx, E, e_lo=0, e_hi=None):
    """perm and group sizes by definition: for each expert in ascending order,
    every flattened row t*k+j with that expert, in ascending row order; a
    token that names one expert in several slots visits it once, through the
    first of those slots."""
    e_hi = E if e_hi is None else e_hi
    T, k = len(idx), len(idx[0])
    perm, counts = [], []
    for e in range(e_lo, e_hi):
        c = 0
        for t in range(T):
            for j in range(k):
                if int(idx[t][j]) == e:
                    perm.append(t * k + j)
                    c += 1
                    break  # the token's later slots naming e are not visited
        counts.append(c)
    return perm, counts


def loss(x, Wr, b, Wg, Wu, Wd, k, gate, E, dY):
    """Scalar <dY, y>, whose gradients are the layer's backward for upstream dY."""
    y = layer_forward(x, Wr, b, Wg, Wu, Wd, k, gate, E)
    return sum(dY[t][n] * y[t][n] for t in range(len(y)) for n in range(len(y[0])))
