"""Plain, slow, obviously correct CPU implementation of the MoE expert layer.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are its only callers.  It shares no code
with the HIP path and imports nothing from it.

Arithmetic is numpy float64 throughout (inputs that are bf16 on the device are
read as their exact bf16 values, upcast); no intermediate rounding is applied.

What the layer computes, with the passage each step follows:

* Pages used (cited by title and section):
  [P3] "Accelerating Transformers fine-tuning with NVIDIA NeMo AutoModel"
       (neows.pages.dev, zh-CN translation of the blog post);
  [P1] "NVIDIA NeMo AutoModel MoE 微調的 3.7 倍加速突破" (wiki digest);
  [P4] the Japanese translation of [P3] (agentlenshq.com).
* Routing each token over many experts: [P3] section 背景 (background), first
  paragraph, names routing tokens across hundreds of experts as the problem.
  The pages leave the gate open; this oracle takes softmax over the top-k
  logits (equal to a full softmax renormalised over the selected experts),
  ties broken toward the lower expert id, slots ordered by descending logit.
* Balanced gate: [P3] section 单节点30B MoE基准测试, note on the routing gate
  (tokens are forced to spread evenly over the experts).  The mechanism is not
  given; this oracle uses expert (t mod P) + i*P for slot i, P = E/k.
* Permutation: [P3] section 专家后端 (expert backends), grouped_mm row and the
  paragraph under the table: tokens are sorted by their assigned expert and a
  single grouped GEMM runs over the groups.  Order inside a group is by the
  flattened (token, slot) row, which makes the sort stable and unique.
* Expert FFN: experts are stored as fused 3-D weight tensors ([P3] v4 deadlock
  note under the Qwen3 table).  The FFN form is not on the pages; this oracle
  uses SwiGLU, silu(x Wg) * (x Wu) then Wd, without biases.
* Combine: dispatch and combine are the two token-movement steps that DeepEP
  fuses ([P3] section 加速来源, DeepEP item); combine is the gate-weighted sum
  of a token's expert outputs.
* Auxiliary load-balancing loss (optional, natural gate): named by [P1]
  section 延伸觀點 and the routing-gate note of [P3]; the formula is the
  Switch Transformer balancing loss (see ``aux_loss``).
* Backward: full-parameter fine-tuning reports a separate backward time
  ([P3] Qwen3 and Nemotron tables, row 平均反向); the gradients below are the
  exact derivatives of the forward definition.
"""
from __future__ import annotations

import numpy as np

GATE_SOFTMAX_TOPK = "softmax_topk"
GATE_BALANCED = "balanced"


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------
def router_logits(x, Wr, b=None):
    """L = x Wr (+ b): the router's per-token score of every expert."""
    L = _f64(x) @ _f64(Wr)
    if b is not None:
        L = L + _f64(b)[None, :]
    return L


def topk_select(L, k):
    """Indices of the k largest logits per row.

    Slot order: descending logit; equal logits by ascending expert id.  This is
    a library sort (numpy lexsort) on the key (-logit, id)."""
    L = np.asarray(L)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("k must lie in [1, E]")
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -L), axis=-1)
    return order[:, :k].astype(np.int32)


def sigmoid(z):
    z = _f64(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def topk_softmax_weights(L, idx):
    """Gate weights: softmax over the selected logits of each token.

    Equal to the full softmax over all E logits renormalised over the selected
    set, because the common normaliser cancels."""
    sel = np.take_along_axis(_f64(L), idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def balanced_gate(T, E, k):
    """Balanced gate: slot i of token t goes to expert (t mod P) + i*P, P = E/k.

    Every token gets k distinct experts and every expert receives the same
    number of rows when P divides T; gate weights are 1/k."""
    if E % k:
        raise ValueError("balanced gate needs k | E")
    P = E // k
    t = np.arange(T)[:, None]
    i = np.arange(k)[None, :]
    idx = ((t % P) + i * P).astype(np.int32)
    g = np.full((T, k), 1.0 / k)
    return idx, g


def route(x, Wr, b, k, gate):
    """Returns (logits or None, idx int32 [T,k], g float64 [T,k])."""
    if gate == GATE_BALANCED:
        idx, g = balanced_gate(x.shape[0], Wr.shape[1], k)
        return None, idx, g
    L = router_logits(x, Wr, b)
    idx = topk_select(L, k)
    return L, idx, topk_softmax_weights(L, idx)


# ----------------------------------------------------------------------------
# permutation (sort rows by expert)
# ----------------------------------------------------------------------------
def permute(idx, x, E, e_lo=0, e_hi=None, R_cap=None):
    """Group the T*k (token, slot) rows by expert, stably.

    Returns dict(counts [E_loc], offsets [E_loc+1], perm [R], inv [T*k], Xp [R,d]).
    Only rows whose expert lies in [e_lo, e_hi) are kept; ``inv`` is -1 for the
    others.  Rows whose sorted position is >= R_cap are dropped as well (their
    ``inv`` is -1 and the offsets are clamped to R_cap).

    A routing table handed in by a caller may name one expert in several
    slots of a token (the router never does: its k experts are distinct).
    The pages do not cover this; the reading taken is that a token visits an
    expert once, through the first slot that names it, and its later slots
    with the same id are dropped like non-local ones (``inv`` = -1)."""
    e_hi = E if e_hi is None else e_hi
    T, k = idx.shape
    ids = np.asarray(idx, dtype=np.int64)
    first = np.ones((T, k), dtype=bool)   # slot j names an id no earlier slot of its token names
    for j in range(1, k):
        first[:, j] = ~np.any(ids[:, :j] == ids[:, j:j + 1], axis=1)
    flat = ids.reshape(-1)
    E_loc = e_hi - e_lo
    local = (flat >= e_lo) & (flat < e_hi) & first.reshape(-1)
    counts = np.bincount(flat[local] - e_lo, minlength=E_loc).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    rows = np.nonzero(local)[0]                       # ascending flattened row
    perm = rows[np.argsort(flat[rows], kind="stable")]
    cap = T * k if R_cap is None else int(R_cap)
    offsets = np.minimum(offsets, cap)
    perm = perm[:cap]
    inv = np.full(T * k, -1, dtype=np.int64)
    inv[perm] = np.arange(perm.size)
    Xp = _f64(x)[perm // k] if x is not None else None
    return dict(counts=counts, offsets=offsets.astype(np.int64), perm=perm.astype(np.int64),
                inv=inv, Xp=Xp)


def unpermute_sum(Zp, inv, T, k):
    """Z[t] = sum over slots j (ascending) of Zp[inv[t,j]], slots with inv < 0 skipped."""
    Zp = _f64(Zp)
    inv = np.asarray(inv).reshape(T, k)
    Z = np.zeros((T, Zp.shape[1]))
    for j in range(k):
        p = inv[:, j]
        m = p >= 0
        Z[m] += Zp[p[m]]
    return Z


# ----------------------------------------------------------------------------
# expert FFN (SwiGLU) over expert groups
# ----------------------------------------------------------------------------
def silu(z):
    z = _f64(z)
    return z * sigmoid(z)


def expert_ffn_fwd(Xp, offsets, Wg, Wu, Wd):
    """Per local expert e over rows [o_e, o_{e+1}):
    Hg = Xp Wg[e], Hu = Xp Wu[e], A = silu(Hg) * Hu, Yp = A Wd[e]."""
    Xp = _f64(Xp)
    R = Xp.shape[0]
    E_loc, d, I = Wg.shape
    Hg = np.zeros((R, I)); Hu = np.zeros((R, I)); A = np.zeros((R, I))
    Yp = np.zeros((R, Wd.shape[2]))
    for e in range(E_loc):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if s == t:
            continue
        xe = Xp[s:t]
        Hg[s:t] = xe @ _f64(Wg[e])
        Hu[s:t] = xe @ _f64(Wu[e])
        A[s:t] = silu(Hg[s:t]) * Hu[s:t]
        Yp[s:t] = A[s:t] @ _f64(Wd[e])
    return dict(Hg=Hg, Hu=Hu, A=A, Yp=Yp)


def expert_ffn_bwd(Xp, offsets, Wg, Wu, Wd, Hg, Hu, A, dYp):
    """Exact gradients of expert_ffn_fwd.

    dWd[e] = A_e^T dYp_e; dA = dYp_e Wd[e]^T; with s = sigmoid(Hg):
    dHg = dA * Hu * s * (1 + Hg (1 - s)), dHu = dA * Hg * s;
    dXp = dHg Wg[e]^T + dHu Wu[e]^T; dWg[e] = Xp_e^T dHg; dWu[e] = Xp_e^T dHu.
    Experts with no rows get all-zero weight gradients."""
    Xp, dYp = _f64(Xp), _f64(dYp)
    E_loc, d, I = Wg.shape
    dXp = np.zeros_like(Xp)
    dHg = np.zeros((Xp.shape[0], I)); dHu = np.zeros((Xp.shape[0], I))
    dWg = np.zeros((E_loc, d, I)); dWu = np.zeros((E_loc, d, I))
    dWd = np.zeros((E_loc, I, Wd.shape[2]))
    for e in range(E_loc):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if s == t:
            continue
        hg, hu, a, dy, xe = _f64(Hg[s:t]), _f64(Hu[s:t]), _f64(A[s:t]), dYp[s:t], Xp[s:t]
        dWd[e] = a.T @ dy
        dA = dy @ _f64(Wd[e]).T
        sg = sigmoid(hg)
        dHg[s:t] = dA * hu * sg * (1.0 + hg * (1.0 - sg))
        dHu[s:t] = dA * hg * sg
        dXp[s:t] = dHg[s:t] @ _f64(Wg[e]).T + dHu[s:t] @ _f64(Wu[e]).T
        dWg[e] = xe.T @ dHg[s:t]
        dWu[e] = xe.T @ dHu[s:t]
    return dict(dXp=dXp, dHg=dHg, dHu=dHu, dWg=dWg, dWu=dWu, dWd=dWd)


# ----------------------------------------------------------------------------
# combine (gate-weighted sum back to token order) and its backward
# ----------------------------------------------------------------------------
def combine(Yp, inv, g, T, k):
    """y[t] = sum_j g[t,j] * Yp[inv[t,j]] over slots with inv >= 0, j ascending."""
    Yp, g = _f64(Yp), _f64(g)
    inv = np.asarray(inv).reshape(T, k)
    y = np.zeros((T, Yp.shape[1]))
    for j in range(k):
        p = inv[:, j]
        m = p >= 0
        y[m] += g[m, j, None] * Yp[p[m]]
    return y


def combine_bwd(dY, Yp, inv, g, T, k):
    """dYp[inv[t,j]] = g[t,j] dY[t];  dG[t,j] = <dY[t], Yp[inv[t,j]]> (0 if dropped)."""
    dY, Yp, g = _f64(dY), _f64(Yp), _f64(g)
    inv = np.asarray(inv).reshape(T, k)
    dYp = np.zeros_like(Yp)
    dG = np.zeros((T, k))
    for j in range(k):
        p = inv[:, j]
        m = p >= 0
        dYp[p[m]] = g[m, j, None] * dY[m]
        dG[m, j] = np.sum(dY[m] * Yp[p[m]], axis=1)
    return dYp, dG


def permute_bwd(dXp, inv, T, k):
    """dX[t] = sum_j dXp[inv[t,j]] (the adjoint of the row gather)."""
    return unpermute_sum(dXp, inv, T, k)


# ----------------------------------------------------------------------------
# load-balancing auxiliary loss
# ----------------------------------------------------------------------------
def softmax_rows(L):
    """Softmax of every row of L over all of its entries (max subtracted)."""
    L = _f64(L)
    z = np.exp(L - L.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def aux_loss(L, idx, E, alpha):
    """Load-balancing auxiliary loss of the router.

    The pages name the practice but not a formula: an auxiliary loss keeps
    the naturally uneven routing even while fine-tuning ([P1] section
    延伸觀點), and a trained model's load-balancing loss drives expert
    utilisation toward uniform ([P3] section 单节点30B MoE基准测试,
    routing-gate note).  This oracle takes the differentiable balancing loss
    of the Switch Transformer (Fedus, Zoph and Shazeer, 2021), the k routed
    slots of a token counted as k dispatches:

        f_e  = c_e / (T k)            share of the T*k routed rows on expert e
                                      (c_e counted over all E experts),
        P_e  = (1/T) sum_t p[t, e]    mean router probability, p = softmax of
                                      the full logit row,
        loss = alpha * E * sum_e f_e P_e.

    The counts are piecewise constant in the logits, so the gradient flows
    through P only; w_e = alpha * E * f_e / T is its weight per probability.
    """
    L = _f64(L)
    T = L.shape[0]
    k = idx.shape[1]
    p = softmax_rows(L)
    c = np.bincount(np.asarray(idx, dtype=np.int64).ravel(), minlength=E).astype(np.float64)
    f = c / (T * k)
    P = p.mean(axis=0)
    return dict(loss=float(alpha * E * np.sum(f * P)), f=f, P=P, w=alpha * E * f / T, counts=c)


def aux_loss_dlogits(L, w):
    """Gradient of the auxiliary loss with respect to the logits:
    d loss / d L[t, j] = sum_e w_e d p[t, e] / d L[t, j]
                       = p[t, j] (w_j - sum_e w_e p[t, e])  (softmax Jacobian)."""
    p = softmax_rows(L)
    w = _f64(w)
    return p * (w[None, :] - (p @ w)[:, None])


# ----------------------------------------------------------------------------
# router backward
# ----------------------------------------------------------------------------
def route_bwd(x, Wr, idx, g, dG, gate, dL_aux=None):
    """Gradients through the gate.

    softmax over the selected logits: dL[t, idx[t,j]] = g_j (dG_j - sum_i g_i dG_i),
    every other logit gets 0 (the selection is piecewise constant);
    dWr = x^T dL, db = sum_t dL, dX_router = dL Wr^T.
    Balanced gate: the weights are constants, so dL, dWr, db and dX_router are 0.
    dL_aux (optional): a further gradient on the logits (the auxiliary loss's),
    added to dL before dWr, db and dX_router are formed."""
    T, k = idx.shape
    E = Wr.shape[1]
    if gate == GATE_BALANCED:
        return dict(dL=np.zeros((T, E)), dWr=np.zeros(Wr.shape), db=np.zeros(E),
                    dX=np.zeros(x.shape))
    g, dG = _f64(g), _f64(dG)
    s = np.sum(g * dG, axis=1, keepdims=True)
    dsel = g * (dG - s)
    dL = np.zeros((T, E))
    np.put_along_axis(dL, idx.astype(np.int64), dsel, axis=1)
    if dL_aux is not None:
        dL = dL + _f64(dL_aux)
    return dict(dL=dL, dWr=_f64(x).T @ dL, db=dL.sum(axis=0), dX=dL @ _f64(Wr).T)


# ----------------------------------------------------------------------------
# the whole layer
# ----------------------------------------------------------------------------
def layer_fwd(x, Wr, b, Wg, Wu, Wd, k, gate, E, e_lo=0, e_hi=None, R_cap=None):
    """Route, permute, expert FFN, combine.  Returns a dict of every intermediate."""
    L, idx, g = route(x, Wr, b, k, gate)
    p = permute(idx, x, E, e_lo, e_hi, R_cap)
    f = expert_ffn_fwd(p["Xp"], p["offsets"], Wg, Wu, Wd)
    y = combine(f["Yp"], p["inv"], g, x.shape[0], k)
    out = dict(logits=L, idx=idx, g=g, y=y)
    out.update(p)
    out.update(f)
    return out


def layer_bwd(fwd, dY, x, Wr, Wg, Wu, Wd, k, gate):
    """Backward of layer_fwd for upstream gradient dY.

    Returns dX (expert path plus router path), dWg, dWu, dWd, dWr, db, dG, dL and
    the permuted intermediates dYp, dXp, dHg, dHu."""
    T = x.shape[0]
    dYp, dG = combine_bwd(dY, fwd["Yp"], fwd["inv"], fwd["g"], T, k)
    fb = expert_ffn_bwd(fwd["Xp"], fwd["offsets"], Wg, Wu, Wd, fwd["Hg"], fwd["Hu"],
                        fwd["A"], dYp)
    dX = permute_bwd(fb["dXp"], fwd["inv"], T, k)
    rb = route_bwd(x, Wr, fwd["idx"], fwd["g"], dG, gate)
    out = dict(dYp=dYp, dG=dG, dX=dX + rb["dX"], dX_expert=dX, dL=rb["dL"],
               dWr=rb["dWr"], db=rb["db"])
    out.update(fb)
    return out
