"""The oracle's pins catch plausible mistakes (CPU only).

Each case copies oracle/, moe_inputs/ and tests/ to a temporary directory,
plants one mistake in the copy of the oracle (a dropped term, a wrong sign, a
swapped operand, a wrong index, an unstable sort, ...) and runs the pin tests
(tests/test_oracle.py) on the copy.  The case passes when the pins fail.
The repository's own oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (what the mistake is, original text, planted text)
MUTATIONS = [
    ("router bias dropped", "L = L + _f64(b)[None, :]", "L = L"),
    ("tie order reversed", "order = np.lexsort((ids, -L), axis=-1)",
     "order = np.lexsort((-ids, -L), axis=-1)"),
    ("smallest logits selected", "return order[:, :k].astype(np.int32)",
     "return order[:, -k:].astype(np.int32)"),
    ("softmax max-shift dropped", "z = np.exp(sel - sel.max(axis=1, keepdims=True))",
     "z = np.exp(sel)"),
    ("sigmoid negative branch wrong", "out[~pos] = ez / (1.0 + ez)", "out[~pos] = 1.0 / (1.0 + ez)"),
    ("balanced gate index transposed", "idx = ((t % P) + i * P).astype(np.int32)",
     "idx = ((t % P) * k + i).astype(np.int32)"),
    ("balanced gate weight not 1/k", "g = np.full((T, k), 1.0 / k)", "g = np.full((T, k), 1.0)"),
    ("repeated expert ids all kept", "local = (flat >= e_lo) & (flat < e_hi) & first.reshape(-1)",
     "local = (flat >= e_lo) & (flat < e_hi)"),
    ("repeat test against slot 0 only", "first[:, j] = ~np.any(ids[:, :j] == ids[:, j:j + 1], axis=1)",
     "first[:, j] = ~np.any(ids[:, :1] == ids[:, j:j + 1], axis=1)"),
    ("unstable sort",'perm = rows[np.argsort(flat[rows], kind="stable")]',
     'perm = rows[np.argsort(flat[rows], kind="quicksort")]'),
    ("capacity keeps the tail", "perm = perm[:cap]", "perm = perm[-cap:]"),
    ("offsets not clamped to capacity", "offsets = np.minimum(offsets, cap)", "offsets = offsets"),
    ("gather by slot instead of token", "Xp = _f64(x)[perm // k]", "Xp = _f64(x)[perm % k]"),
    ("gate weight used for up", "Hg[s:t] = xe @ _f64(Wg[e])", "Hg[s:t] = xe @ _f64(Wu[e])"),
    ("silu without x", "return z * sigmoid(z)", "return sigmoid(z)"),
    ("dWd halved", "dWd[e] = a.T @ dy", "dWd[e] = a.T @ dy * 0.5"),
    ("dsilu term dropped", "dHg[s:t] = dA * hu * sg * (1.0 + hg * (1.0 - sg))",
     "dHg[s:t] = dA * hu * sg"),
    ("dHu sign", "dHu[s:t] = dA * hg * sg", "dHu[s:t] = -dA * hg * sg"),
    ("dXp uses Wg twice", "dXp[s:t] = dHg[s:t] @ _f64(Wg[e]).T + dHu[s:t] @ _f64(Wu[e]).T",
     "dXp[s:t] = dHg[s:t] @ _f64(Wg[e]).T + dHu[s:t] @ _f64(Wg[e]).T"),
    ("dWg from dHu", "dWg[e] = xe.T @ dHg[s:t]", "dWg[e] = xe.T @ dHu[s:t]"),
    ("combine ignores gate", "y[m] += g[m, j, None] * Yp[p[m]]", "y[m] += Yp[p[m]] / k"),
    ("combine bwd ignores gate", "dYp[p[m]] = g[m, j, None] * dY[m]", "dYp[p[m]] = dY[m]"),
    ("dG scaled by gate", "dG[m, j] = np.sum(dY[m] * Yp[p[m]], axis=1)",
     "dG[m, j] = np.sum(dY[m] * Yp[p[m]], axis=1) * g[m, j]"),
    ("unpermute overwrites", "Z[m] += Zp[p[m]]", "Z[m] = Zp[p[m]]"),
    ("softmax Jacobian term dropped", "dsel = g * (dG - s)", "dsel = g * dG"),
    ("db averaged", "db=dL.sum(axis=0)", "db=dL.mean(axis=0)"),
    ("router dX dropped", "dX=dL @ _f64(Wr).T)", "dX=0 * dL @ _f64(Wr).T)"),
    ("aux loss without the expert count factor", "loss=float(alpha * E * np.sum(f * P))",
     "loss=float(alpha * np.sum(f * P))"),
    ("aux shares over tokens not rows", "f = c / (T * k)", "f = c / T"),
    ("aux mean probability not averaged", "P = p.mean(axis=0)", "P = p.sum(axis=0)"),
    ("aux gradient Jacobian term dropped", "return p * (w[None, :] - (p @ w)[:, None])",
     "return p * w[None, :]"),
    ("aux gradient not added to the router", "dL = dL + _f64(dL_aux)", "dL = dL"),
]


@pytest.mark.parametrize("what,orig,planted", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, what, orig, planted):
    for d in ("oracle", "moe_inputs", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    f = tmp_path / "oracle" / "moe_oracle.py"
    src = f.read_text()
    assert src.count(orig) == 1, f"mutation site not unique or missing: {orig}"
    f.write_text(src.replace(orig, planted))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle.py"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 1, f"pins did not catch: {what}\n{r.stdout[-2000:]}"
