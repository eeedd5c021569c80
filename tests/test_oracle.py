"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against a value or property fixed by the pages or
by mathematics: a hand-worked example, brute force in pure Python, closed
forms, library routines for special cases, invariants and finite differences.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

from moe_inputs import round_bf16
from oracle import brute
from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _tiny(seed, T=7, d=4, E=5, k=2, I=3, bias=True, scale=1.0):
    r = _rng(seed)
    x = r.standard_normal((T, d)) * scale
    Wr = r.standard_normal((d, E))
    b = r.standard_normal(E) if bias else None
    Wg = r.standard_normal((E, d, I)) * 0.5
    Wu = r.standard_normal((E, d, I)) * 0.5
    Wd = r.standard_normal((E, I, d)) * 0.5
    return x, Wr, b, Wg, Wu, Wd


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def test_hand_routing_example():
    gold = json.load(open(os.path.join(GOLD, "hand_routing_example.json")))
    L = np.array(gold["logits"], dtype=np.float64)
    k, E = gold["k"], gold["E"]
    idx = O.topk_select(L, k)
    assert idx.tolist() == gold["idx"]
    g = O.topk_softmax_weights(L, idx)
    e3 = math.exp(-3.0)
    want = np.array([[0.5, 0.5], [1 / (1 + e3), e3 / (1 + e3)], [0.5, 0.5]])
    np.testing.assert_allclose(g, want, rtol=0, atol=1e-15)
    p = O.permute(idx, np.zeros((3, 1)), E)
    assert p["counts"].tolist() == gold["counts"]
    assert p["offsets"].tolist() == gold["offsets"]
    assert p["perm"].tolist() == gold["perm"]
    assert p["inv"].tolist() == gold["inv"]
    q = O.permute(idx, np.zeros((3, 1)), E, e_lo=1, e_hi=3)
    loc = gold["local_1_3"]
    assert q["counts"].tolist() == loc["counts"]
    assert q["offsets"].tolist() == loc["offsets"]
    assert q["perm"].tolist() == loc["perm"]
    assert q["inv"].tolist() == loc["inv"]


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_python_sort_with_ties(seed):
    r = _rng(seed)
    T, E, k = 40, 9, 4
    L = r.integers(-3, 4, size=(T, E)).astype(np.float64)   # many exact ties
    idx = O.topk_select(L, k)
    for t in range(T):
        assert idx[t].tolist() == brute.select(L[t].tolist(), k)


def test_zero_router_gives_lowest_ids_and_uniform_weights():
    T, d, E, k = 5, 6, 8, 3
    L, idx, g = O.route(np.ones((T, d)), np.zeros((d, E)), None, k, O.GATE_SOFTMAX_TOPK)
    assert (idx == np.arange(k)[None, :]).all()
    np.testing.assert_allclose(g, 1.0 / k, rtol=0, atol=1e-15)


def test_k_equals_E_is_full_softmax():
    r = _rng(3)
    L = r.standard_normal((11, 6)) * 3
    idx = O.topk_select(L, 6)
    g = O.topk_softmax_weights(L, idx)
    full = scipy.special.softmax(L, axis=1)
    np.testing.assert_allclose(g, np.take_along_axis(full, idx.astype(np.int64), 1),
                               rtol=1e-13, atol=0)


def test_topk_weights_equal_renormalised_full_softmax():
    r = _rng(4)
    L = r.standard_normal((13, 10)) * 2
    idx = O.topk_select(L, 3)
    g = O.topk_softmax_weights(L, idx)
    full = scipy.special.softmax(L, axis=1)
    sel = np.take_along_axis(full, idx.astype(np.int64), 1)
    np.testing.assert_allclose(g, sel / sel.sum(1, keepdims=True), rtol=1e-13)


@pytest.mark.parametrize("gate", ["softmax_topk", "balanced"])
def test_gate_invariants(gate):
    r = _rng(5)
    T, d, E, k = 64, 8, 16, 4
    x = r.standard_normal((T, d))
    Wr = r.standard_normal((d, E))
    _, idx, g = O.route(x, Wr, None, k, gate)
    for t in range(T):
        assert len(set(idx[t].tolist())) == k             # k distinct experts
    assert ((idx >= 0) & (idx < E)).all()
    assert np.abs(g.sum(1) - 1).max() <= 1e-12             # renormalised weights sum to 1
    if gate == "softmax_topk":
        assert (np.diff(np.take_along_axis(O.router_logits(x, Wr), idx.astype(np.int64), 1), axis=1) <= 0).all()


def test_router_logits_vs_brute():
    x, Wr, b, *_ = _tiny(7)
    L = O.router_logits(x, Wr, b)
    Lb = np.array(brute.logits(x.tolist(), Wr.tolist(), b.tolist(), Wr.shape[1]))
    np.testing.assert_allclose(L, Lb, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# permutation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed,e_lo,e_hi", [(0, 0, 7), (1, 2, 5), (2, 0, 1), (3, 6, 7)])
def test_permute_matches_definition(seed, e_lo, e_hi):
    r = _rng(seed)
    T, E, k = 23, 7, 3
    idx = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = r.standard_normal((T, 5))
    p = O.permute(idx, x, E, e_lo, e_hi)
    perm, counts = brute.stable_groups(idx.tolist(), E, e_lo, e_hi)
    assert p["perm"].tolist() == perm
    assert p["counts"].tolist() == counts
    assert p["offsets"].tolist() == np.concatenate([[0], np.cumsum(counts)]).tolist()


def test_permute_invariants_and_roundtrip():
    r = _rng(9)
    T, E, k, d = 50, 12, 4, 6
    idx = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = r.standard_normal((T, d))
    p = O.permute(idx, x, E)
    assert p["counts"].sum() == T * k                       # group sizes sum to T*k
    assert (np.diff(p["offsets"]) >= 0).all()
    assert sorted(p["perm"].tolist()) == list(range(T * k))  # a permutation
    assert (p["inv"][p["perm"]] == np.arange(T * k)).all()   # inv o perm = id
    assert (p["perm"][p["inv"]] == np.arange(T * k)).all()
    # permute then un-permute (gather back through inv) is the identity, bit for bit
    back = p["Xp"][p["inv"]].reshape(T, k, d)
    for j in range(k):
        assert np.array_equal(back[:, j], x)
    # each group holds only its expert
    flat = idx.reshape(-1)
    for e in range(E):
        s, t = p["offsets"][e], p["offsets"][e + 1]
        assert (flat[p["perm"][s:t]] == e).all()
        assert (np.diff(p["perm"][s:t]) > 0).all()          # stable


@pytest.mark.parametrize("T,E,k", [(4096, 128, 8), (32768, 256, 8), (64, 8, 2)])
def test_balanced_closed_form(T, E, k):
    idx, g = O.balanced_gate(T, E, k)
    P = E // k
    p = O.permute(idx, None, E)
    assert (p["counts"] == T * k // E).all()                # evenly spread
    e = np.arange(E)
    assert (p["offsets"][:-1] == e * T * k // E).all()
    m = np.arange(T // P)
    for ee in [0, 1, P - 1, P, E - 1, E // 2 + 3]:
        want = ((ee % P) + m * P) * k + ee // P
        got = p["perm"][p["offsets"][ee]:p["offsets"][ee + 1]]
        assert (got == want).all()


def test_repeated_and_foreign_ids_hand_example():
    """A caller's table with repeated and out-of-range ids (hand-worked)."""
    gold = json.load(open(os.path.join(GOLD, "repeated_ids_example.json")))
    idx = np.array(gold["idx"], dtype=np.int32)
    E = gold["E"]
    p = O.permute(idx, None, E)
    assert p["counts"].tolist() == gold["counts"]
    assert p["offsets"].tolist() == gold["offsets"]
    assert p["perm"].tolist() == gold["perm"]
    assert p["inv"].tolist() == gold["inv"]
    kept = (p["inv"] >= 0).reshape(idx.shape)
    assert kept.tolist() == gold["kept_slots"]
    q = O.permute(idx, None, E, e_lo=2, e_hi=6)
    loc = gold["local_2_6"]
    assert q["counts"].tolist() == loc["counts"]
    assert q["offsets"].tolist() == loc["offsets"]
    assert q["perm"].tolist() == loc["perm"]
    assert q["inv"].tolist() == loc["inv"]


@pytest.mark.parametrize("seed,e_lo,e_hi", [(0, 0, 6), (1, 1, 4), (2, 5, 6)])
def test_permute_with_repeated_ids_matches_definition(seed, e_lo, e_hi):
    """Random tables drawn with replacement (repeats) and ids outside [0, E)."""
    r = _rng(100 + seed)
    T, E, k = 31, 6, 4
    idx = r.integers(-1, E + 2, size=(T, k)).astype(np.int32)
    p = O.permute(idx, None, E, e_lo, e_hi)
    perm, counts = brute.stable_groups(idx.tolist(), E, e_lo, e_hi)
    assert p["perm"].tolist() == perm
    assert p["counts"].tolist() == counts
    # every kept slot is the first of its token to name its (local) expert
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(idx[t, j])
            keep = e_lo <= e < e_hi and e not in seen
            seen.add(e)
            assert (p["inv"][t * k + j] >= 0) == keep


def test_forward_with_caller_table_vs_brute():
    """y for a table with repeats: each token's distinct local experts, each
    weighted by the gate weight of the first slot that names it."""
    x, Wr, b, Wg, Wu, Wd = _tiny(77, T=6, d=3, E=4, k=3, I=2)
    idx = np.array([[1, 1, 2], [3, 0, 3], [2, 2, 2], [0, 1, 3], [5, 1, -2], [0, 0, 1]],
                   dtype=np.int32)
    g = _rng(78).random(idx.shape)
    T, k = idx.shape
    p = O.permute(idx, x, 4)
    f = O.expert_ffn_fwd(p["Xp"], p["offsets"], Wg, Wu, Wd)
    y = O.combine(f["Yp"], p["inv"], g, T, k)
    want = []
    for t in range(T):
        acc = [0.0] * x.shape[1]
        seen = set()
        for j in range(k):
            e = int(idx[t, j])
            if e in seen or not 0 <= e < 4:
                continue
            seen.add(e)
            out = brute.ffn(x[t].tolist(), Wg[e].tolist(), Wu[e].tolist(), Wd[e].tolist())
            acc = [a + g[t, j] * o for a, o in zip(acc, out)]
        want.append(acc)
    np.testing.assert_allclose(y, np.array(want), rtol=1e-12, atol=1e-14)


def test_capacity_drop_keeps_sorted_prefix():
    r = _rng(11)
    T, E, k = 30, 5, 2
    idx = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    full = O.permute(idx, None, E)
    cap = 37
    p = O.permute(idx, None, E, R_cap=cap)
    assert (p["perm"] == full["perm"][:cap]).all()
    assert (p["offsets"] == np.minimum(full["offsets"], cap)).all()
    assert (p["inv"] >= 0).sum() == cap
    dropped = full["perm"][cap:]
    assert (p["inv"][dropped] == -1).all()


# --------------------------------------------------------------------------
# expert FFN and the whole forward
# --------------------------------------------------------------------------
def test_silu_special_values():
    z = np.array([0.0, 1e-3, -1e-3, 2.0, -2.0, 40.0, -40.0, 800.0, -800.0])
    s = O.silu(z)
    np.testing.assert_allclose(s, z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert s[0] == 0.0
    assert s[7] == 800.0 and abs(s[8]) < 1e-300


@pytest.mark.parametrize("gate,bias", [("softmax_topk", True), ("softmax_topk", False), ("balanced", False)])
def test_forward_vs_dense_brute_force(gate, bias):
    T, d, E, k, I = (8, 4, 4, 2, 3)
    x, Wr, b, Wg, Wu, Wd = _tiny(21, T=T, d=d, E=E, k=k, I=I, bias=bias)
    f = O.layer_fwd(x, Wr, b, Wg, Wu, Wd, k, gate, E)
    yb = brute.layer_forward(x.tolist(), Wr.tolist(), None if b is None else b.tolist(),
                             Wg.tolist(), Wu.tolist(), Wd.tolist(), k, gate, E)
    np.testing.assert_allclose(f["y"], np.array(yb), rtol=1e-12, atol=1e-12)


def test_single_expert_is_dense_swiglu_mlp():
    r = _rng(2)
    T, d, I = 9, 6, 5
    x = r.standard_normal((T, d))
    Wg, Wu, Wd = r.standard_normal((1, d, I)), r.standard_normal((1, d, I)), r.standard_normal((1, I, d))
    f = O.layer_fwd(x, np.zeros((d, 1)), None, Wg, Wu, Wd, 1, "softmax_topk", 1)
    h = x @ Wg[0]
    want = (h * scipy.special.expit(h) * (x @ Wu[0])) @ Wd[0]
    np.testing.assert_allclose(f["y"], want, rtol=1e-12, atol=1e-12)


def test_identical_experts_ignore_routing():
    r = _rng(8)
    T, d, E, k, I = 20, 6, 6, 3, 4
    x = r.standard_normal((T, d))
    Wr = r.standard_normal((d, E))
    wg, wu, wd = r.standard_normal((d, I)), r.standard_normal((d, I)), r.standard_normal((I, d))
    Wg, Wu, Wd = (np.repeat(w[None], E, 0) for w in (wg, wu, wd))
    f = O.layer_fwd(x, Wr, None, Wg, Wu, Wd, k, "softmax_topk", E)
    single = O.layer_fwd(x, np.zeros((d, 1)), None, wg[None], wu[None], wd[None], 1, "softmax_topk", 1)
    np.testing.assert_allclose(f["y"], single["y"], rtol=1e-12, atol=1e-12)


def test_hand_ffn_closed_form():
    # d = I = 1, one expert: y = g * Wd * silu(Wg x) * (Wu x) with x=2, Wg=1, Wu=0.5, Wd=3.
    s2 = 1.0 / (1.0 + math.exp(-2.0))
    f = O.layer_fwd(np.array([[2.0]]), np.zeros((1, 1)), None, np.array([[[1.0]]]),
                    np.array([[[0.5]]]), np.array([[[3.0]]]), 1, "softmax_topk", 1)
    assert abs(f["y"][0, 0] - 3.0 * 2.0 * s2 * 1.0) < 1e-14
    bw = O.layer_bwd(f, np.array([[1.0]]), np.array([[2.0]]), np.zeros((1, 1)), np.array([[[1.0]]]),
                     np.array([[[0.5]]]), np.array([[[3.0]]]), 1, "softmax_topk")
    # dy/dWd = A = 2*s2; dy/dWu = Wd*silu(2)*x = 3*2*s2*2; dy/dWg = Wd*Hu*silu'(2)*x
    dsilu = s2 * (1 + 2.0 * (1 - s2))
    assert abs(bw["dWd"][0, 0, 0] - 2 * s2) < 1e-14
    assert abs(bw["dWu"][0, 0, 0] - 3 * 2 * s2 * 2) < 1e-13
    assert abs(bw["dWg"][0, 0, 0] - 3 * 1.0 * dsilu * 2) < 1e-13
    # dy/dx = Wd * (silu'(Wg x) Wg (Wu x) + silu(Wg x) Wu)
    assert abs(bw["dX"][0, 0] - 3 * (dsilu * 1.0 * 1.0 + 2 * s2 * 0.5)) < 1e-13


def test_ep_shards_partition_the_layer():
    facts = json.load(open(os.path.join(GOLD, "pages_facts.json")))
    ep = facts["ep_size"]["value"]
    r = _rng(12)
    T, d, E, k, I = 64, 8, 16, 2, 4
    x = r.standard_normal((T, d))
    Wr = r.standard_normal((d, E))
    Wg, Wu, Wd = r.standard_normal((E, d, I)), r.standard_normal((E, d, I)), r.standard_normal((E, I, d))
    full = O.layer_fwd(x, Wr, None, Wg, Wu, Wd, k, "softmax_topk", E)
    per = E // ep
    acc = np.zeros_like(full["y"])
    rows = 0
    for rank in range(ep):
        lo, hi = rank * per, (rank + 1) * per
        part = O.layer_fwd(x, Wr, None, Wg[lo:hi], Wu[lo:hi], Wd[lo:hi], k, "softmax_topk", E, lo, hi)
        acc += part["y"]
        rows += int(part["offsets"][-1])
        assert Wg[lo:hi].nbytes * ep == Wg.nbytes              # 1/ep of the expert weights
    assert rows == T * k
    np.testing.assert_allclose(acc, full["y"], rtol=1e-12, atol=1e-12)
    # balanced gate over ep ranks with P = E/k experts per "column": equal rows per rank
    idx, _ = O.balanced_gate(facts["seq_len_tokens_per_gpu"]["value"], 256, 8)
    sizes = [int(O.permute(idx, None, 256, q * 32, (q + 1) * 32)["offsets"][-1]) for q in range(ep)]
    assert sizes == [4096] * ep


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def _min_gap(L, k):
    s = -np.sort(-L, axis=1)
    return float((s[:, k - 1] - s[:, k]).min()) if L.shape[1] > k else np.inf


@pytest.mark.parametrize("gate", ["softmax_topk", "balanced"])
def test_backward_finite_differences_brute(gate):
    T, d, E, k, I = 5, 3, 4, 2, 3
    x, Wr, b, Wg, Wu, Wd = _tiny(31, T=T, d=d, E=E, k=k, I=I, bias=(gate != "balanced"))
    dY = _rng(32).standard_normal((T, d))
    if gate == "softmax_topk":
        assert _min_gap(O.router_logits(x, Wr, b), k) > 1e-3      # no routing flip under h
    f = O.layer_fwd(x, Wr, b, Wg, Wu, Wd, k, gate, E)
    g = O.layer_bwd(f, dY, x, Wr, Wg, Wu, Wd, k, gate)
    h = 1e-6
    params = {"x": x, "Wr": Wr, "Wg": Wg, "Wu": Wu, "Wd": Wd}
    if b is not None:
        params["b"] = b
    grads = {"x": g["dX"], "Wr": g["dWr"], "Wg": g["dWg"], "Wu": g["dWu"], "Wd": g["dWd"], "b": g["db"]}

    def L_of(p):
        return brute.loss(p["x"].tolist(), p["Wr"].tolist(), None if "b" not in p else p["b"].tolist(),
                          p["Wg"].tolist(), p["Wu"].tolist(), p["Wd"].tolist(), k, gate, E, dY.tolist())

    for name, arr in params.items():
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            p = {n: a.copy() for n, a in params.items()}
            p[name][i] += h
            up = L_of(p)
            p[name][i] -= 2 * h
            dn = L_of(p)
            fd[i] = (up - dn) / (2 * h)
        np.testing.assert_allclose(grads[name], fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_backward_directional_derivative_larger():
    T, d, E, k, I = 40, 12, 8, 3, 10
    x, Wr, b, Wg, Wu, Wd = _tiny(41, T=T, d=d, E=E, k=k, I=I)
    dY = _rng(42).standard_normal((T, d))
    assert _min_gap(O.router_logits(x, Wr, b), k) > 1e-4
    f = O.layer_fwd(x, Wr, b, Wg, Wu, Wd, k, "softmax_topk", E)
    g = O.layer_bwd(f, dY, x, Wr, Wg, Wu, Wd, k, "softmax_topk")
    r = _rng(43)
    v = {n: r.standard_normal(a.shape) for n, a in dict(x=x, Wr=Wr, b=b, Wg=Wg, Wu=Wu, Wd=Wd).items()}
    h = 1e-6

    def loss(s):
        ff = O.layer_fwd(x + s * v["x"], Wr + s * v["Wr"], b + s * v["b"], Wg + s * v["Wg"],
                         Wu + s * v["Wu"], Wd + s * v["Wd"], k, "softmax_topk", E)
        return float(np.sum(ff["y"] * dY))

    fd = (loss(h) - loss(-h)) / (2 * h)
    an = sum(float(np.sum(g[gn] * v[pn])) for gn, pn in
             [("dX", "x"), ("dWr", "Wr"), ("db", "b"), ("dWg", "Wg"), ("dWu", "Wu"), ("dWd", "Wd")])
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an))


def test_combine_backward_by_finite_differences():
    r = _rng(51)
    T, k, R, d = 6, 3, 18, 4
    inv = r.permutation(R)
    inv[[2, 7]] = -1                                   # two dropped slots
    Yp = r.standard_normal((R, d))
    g = r.random((T, k))
    dY = r.standard_normal((T, d))
    dYp, dG = O.combine_bwd(dY, Yp, inv, g, T, k)
    h = 1e-6
    for (t, j) in [(0, 0), (0, 2), (2, 1), (5, 2)]:
        gp, gm = g.copy(), g.copy()
        gp[t, j] += h
        gm[t, j] -= h
        fd = (np.sum(O.combine(Yp, inv, gp, T, k) * dY) - np.sum(O.combine(Yp, inv, gm, T, k) * dY)) / (2 * h)
        assert abs(fd - dG[t, j]) < 1e-7
    for p in [0, 5, 11, 17]:
        for n in range(d):
            Ypp, Ypm = Yp.copy(), Yp.copy()
            Ypp[p, n] += h
            Ypm[p, n] -= h
            fd = (np.sum(O.combine(Ypp, inv, g, T, k) * dY) - np.sum(O.combine(Ypm, inv, g, T, k) * dY)) / (2 * h)
            assert abs(fd - dYp[p, n]) < 1e-7
    assert (dYp[np.setdiff1d(np.arange(R), inv[inv >= 0])] == 0).all()


def test_regrouped_gate_products_equal_the_definition():
    """The backward's dY form regroups where the gate weight g of row p
    (token t, slot j) is applied: dA = g (dY[t] Wd^T) instead of (g dY[t]) Wd^T,
    dWd = sum_p (g A[p])^T dY[t] instead of A^T dYp, and dG = <dY[t] Wd^T, A[p]>
    instead of <dY[t], Yp[p]>.  In exact arithmetic both sides are the same;
    here in fp64 against the oracle's backward, per expert, with empty and
    dropped rows (R_cap < T*k)."""
    r = _rng(53)
    T, d, E, k, I = 40, 16, 6, 3, 12
    x = r.standard_normal((T, d))
    Wr = r.standard_normal((d, E))
    Wg, Wu = r.standard_normal((E, d, I)) / 4, r.standard_normal((E, d, I)) / 4
    Wd = r.standard_normal((E, I, d)) / 4
    dY = r.standard_normal((T, d))
    f = O.layer_fwd(x, Wr, None, Wg, Wu, Wd, k, "softmax_topk", E, R_cap=100)
    off, perm = f["offsets"], f["perm"]
    R = int(off[-1])
    assert R == 100  # 20 of the 120 slots dropped
    dYp, dG = O.combine_bwd(dY, f["Yp"], f["inv"], f["g"], T, k)
    fb = O.expert_ffn_bwd(f["Xp"], off, Wg, Wu, Wd, f["Hg"], f["Hu"], f["A"], dYp)
    tok, gw = perm // k, f["g"].reshape(-1)[perm]
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        dA0 = dY[tok[rows]] @ Wd[e].T                     # before the gate weight
        assert np.allclose(gw[rows, None] * dA0, dYp[rows] @ Wd[e].T, rtol=0, atol=1e-12)
        dWd = (gw[rows, None] * f["A"][rows]).T @ dY[tok[rows]]
        assert np.allclose(dWd, fb["dWd"][e], rtol=0, atol=1e-12)
        dg = np.einsum("pi,pi->p", dA0, f["A"][rows])
        assert np.allclose(dg, dG.reshape(-1)[perm[rows]], rtol=0, atol=1e-12)
    # every kept slot's dG comes from its row; dropped slots stay 0
    kept = f["inv"] >= 0
    assert not dG.reshape(-1)[~kept].any() and kept.sum() == R


def test_permute_backward_is_adjoint_of_gather():
    r = _rng(52)
    T, k, d, E = 10, 3, 5, 6
    idx = np.stack([r.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    x = r.standard_normal((T, d))
    p = O.permute(idx, x, E, 1, 5)
    dXp = r.standard_normal(p["Xp"].shape)
    dX = O.permute_bwd(dXp, p["inv"], T, k)
    assert abs(np.sum(p["Xp"] * dXp) - np.sum(x * dX)) < 1e-12   # <P x, v> = <x, P^T v>


def test_router_gradient_invariants():
    r = _rng(61)
    T, d, E, k = 30, 7, 9, 4
    x = r.standard_normal((T, d))
    Wr = r.standard_normal((d, E))
    L, idx, g = O.route(x, Wr, None, k, "softmax_topk")
    dG = r.standard_normal((T, k))
    rb = O.route_bwd(x, Wr, idx, g, dG, "softmax_topk")
    sel = np.take_along_axis(rb["dL"], idx.astype(np.int64), 1)
    assert np.abs(sel.sum(1)).max() < 1e-13                # softmax gradient sums to zero
    mask = np.ones((T, E), bool)
    np.put_along_axis(mask, idx.astype(np.int64), False, 1)
    assert (rb["dL"][mask] == 0).all()                      # unselected logits get nothing
    Wr8 = r.standard_normal((d, 8))
    bidx, bg = O.balanced_gate(T, 8, k)
    bal = O.route_bwd(x, Wr8, bidx, bg, dG, "balanced")
    assert not bal["dWr"].any() and not bal["dX"].any()     # balanced gate: dWr = 0


def test_empty_experts_get_exactly_zero_weight_grads():
    r = _rng(71)
    T, d, E, k, I = 12, 5, 6, 2, 4
    idx = np.stack([r.choice([0, 2, 3], size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = r.standard_normal((T, d))
    p = O.permute(idx, x, E)
    Wg, Wu, Wd = r.standard_normal((E, d, I)), r.standard_normal((E, d, I)), r.standard_normal((E, I, d))
    f = O.expert_ffn_fwd(p["Xp"], p["offsets"], Wg, Wu, Wd)
    bw = O.expert_ffn_bwd(p["Xp"], p["offsets"], Wg, Wu, Wd, f["Hg"], f["Hu"], f["A"],
                          r.standard_normal(f["Yp"].shape))
    for e in (1, 4, 5):
        assert p["counts"][e] == 0
        assert not bw["dWg"][e].any() and not bw["dWu"][e].any() and not bw["dWd"][e].any()


def test_bf16_rounding_of_inputs_is_rne():
    # the input generator's rounding, pinned on values with known bf16 neighbours
    v = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-9, 1.0 + 2**-9, -2.5, 3.0e-3], dtype=np.float32)
    r = round_bf16(v)
    assert r[0] == 1.0
    assert r[1] == 1.0                                # exactly half-way: ties to even
    assert r[2] == 1.0 + 2**-7                        # 1.5 ulp rounds up
    assert r[3] == 1.0                                # half ulp, even below
    assert r[4] == -2.5
    assert abs(r[5] - 3.0e-3) <= 3.0e-3 * 2**-8


def test_gate_weights_stable_for_large_logits():
    L = np.array([[1000.0, 999.0, -5.0, 998.0]])
    idx = O.topk_select(L, 3)
    g = O.topk_softmax_weights(L, idx)
    z = np.array([1.0, math.exp(-1.0), math.exp(-2.0)])
    np.testing.assert_allclose(g[0], z / z.sum(), rtol=1e-14)


# --------------------------------------------------------------------------
# load-balancing auxiliary loss
# --------------------------------------------------------------------------
def test_aux_loss_hand_example():
    """tests/golden/aux_loss_example.json: the loss re-derived by hand from
    its definition, each softmax row written out term by term."""
    g = json.load(open(os.path.join(GOLD, "aux_loss_example.json")))
    e = math.e
    Z0 = e + 2 * e ** 3 + 1
    Z1 = 2 * e ** 2 + 1 + e ** 5
    p0 = [e / Z0, e ** 3 / Z0, e ** 3 / Z0, 1 / Z0]
    p1 = [e ** 2 / Z1, 1 / Z1, e ** 2 / Z1, e ** 5 / Z1]
    P = [(a + b + 0.25) / 3 for a, b in zip(p0, p1)]
    hand = 0.01 * 4 * (P[0] / 3 + P[1] / 3 + P[2] / 6 + P[3] / 6)
    assert hand == pytest.approx(g["loss_closed_form_value"], rel=1e-13)
    r = O.aux_loss(np.array(g["logits"], float), np.array(g["idx"]), g["E"], g["alpha"])
    assert r["loss"] == pytest.approx(hand, rel=1e-13)
    assert r["f"] == pytest.approx([1 / 3, 1 / 3, 1 / 6, 1 / 6], rel=1e-15)
    assert r["counts"].tolist() == [2, 2, 1, 1]


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (60, 16, 4), (7, 4, 4)])
def test_aux_loss_uniform_routing_is_alpha(T, E, k):
    """Equal logits give P_e = 1/E; a routing that puts T*k/E rows on every
    expert gives f_e = 1/E; then loss = alpha * E * E * (1/E)(1/E) = alpha."""
    L = np.full((T, E), 0.37)
    idx = np.array([[(t * k + j) % E for j in range(k)] for t in range(T)])
    if (T * k) % E:
        pytest.skip("rows do not divide evenly")
    r = O.aux_loss(L, idx, E, 0.25)
    assert r["loss"] == pytest.approx(0.25, rel=1e-14)
    # the gradient vanishes: every w_e equal, softmax Jacobian rows sum to zero
    assert np.abs(O.aux_loss_dlogits(L, r["w"])).max() < 1e-15


def test_aux_loss_all_on_one_expert():
    """Every token routed to expert 0 (k = 1), logits strongly favouring it:
    f = (1, 0, ...), P_0 -> 1, so loss -> alpha * E (its largest value)."""
    T, E = 16, 8
    L = np.zeros((T, E))
    L[:, 0] = 60.0
    idx = np.zeros((T, 1), dtype=np.int32)
    r = O.aux_loss(L, idx, E, 1.0)
    assert r["loss"] == pytest.approx(E * (1.0 / (1.0 + (E - 1) * math.exp(-60.0))), rel=1e-14)


def test_aux_loss_gradient_by_finite_differences():
    """Central differences of loss(L) with the routing held fixed (the counts
    are piecewise constant) against the closed-form gradient."""
    r = _rng(41)
    T, E, k = 6, 5, 2
    L = r.standard_normal((T, E))
    idx = O.topk_select(L, k)
    w = O.aux_loss(L, idx, E, 0.7)["w"]
    G = O.aux_loss_dlogits(L, w)
    h = 1e-6
    num = np.zeros_like(L)
    for t in range(T):
        for e in range(E):
            Lp, Lm = L.copy(), L.copy()
            Lp[t, e] += h
            Lm[t, e] -= h
            num[t, e] = (O.aux_loss(Lp, idx, E, 0.7)["loss"] - O.aux_loss(Lm, idx, E, 0.7)["loss"]) / (2 * h)
    np.testing.assert_allclose(G, num, rtol=1e-7, atol=1e-10)


def test_aux_loss_router_parameter_gradients_by_finite_differences():
    """The auxiliary gradient pushed through the router (dWr = x^T dL,
    db = column sums of dL, dX = dL Wr^T) against central differences of
    loss(x Wr + b) in Wr, b and x, the routing held fixed."""
    r = _rng(43)
    T, d, E, k = 5, 3, 4, 2
    x, Wr, b = r.standard_normal((T, d)), r.standard_normal((d, E)), r.standard_normal(E)
    idx = O.topk_select(O.router_logits(x, Wr, b), k)
    alpha = 0.3

    def loss(x_, Wr_, b_):
        return O.aux_loss(O.router_logits(x_, Wr_, b_), idx, E, alpha)["loss"]

    L = O.router_logits(x, Wr, b)
    dL = O.aux_loss_dlogits(L, O.aux_loss(L, idx, E, alpha)["w"])
    zero_g = np.zeros((T, k))
    rb = O.route_bwd(x, Wr, idx, zero_g, zero_g, O.GATE_SOFTMAX_TOPK, dL_aux=dL)
    h = 1e-6
    for name, arr, grad in (("Wr", Wr, rb["dWr"]), ("b", b, rb["db"]), ("x", x, rb["dX"])):
        num = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[i] += h
            am[i] -= h
            args_p = dict(x_=x, Wr_=Wr, b_=b)
            args_m = dict(x_=x, Wr_=Wr, b_=b)
            key = {"Wr": "Wr_", "b": "b_", "x": "x_"}[name]
            args_p[key], args_m[key] = ap, am
            num[i] = (loss(**args_p) - loss(**args_m)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-10, err_msg=name)


def test_aux_loss_invariant_under_expert_relabelling():
    """Renaming the experts (permuting logit columns and routed ids alike)
    changes neither the loss nor, relabelled, its gradient."""
    r = _rng(47)
    T, E, k = 9, 6, 3
    L = r.standard_normal((T, E))
    idx = O.topk_select(L, k)
    perm = r.permutation(E)
    inv = np.argsort(perm)
    a = O.aux_loss(L, idx, E, 0.1)
    b = O.aux_loss(L[:, perm], inv[idx], E, 0.1)
    assert b["loss"] == pytest.approx(a["loss"], rel=1e-14)
    ga = O.aux_loss_dlogits(L, a["w"])
    gb = O.aux_loss_dlogits(L[:, perm], b["w"])
    np.testing.assert_allclose(gb, ga[:, perm], rtol=1e-12, atol=1e-16)
