"""Element-wise comparison of GPU outputs with the oracle that accounts for
the call's quantized decisions (oracle/decisions.py).

The bar is max-abs relative error <= 2e-2 (of the tensor's largest oracle
value) and cosine >= 0.999 per output.  Where admissible fp32 evaluations can
take a quantized decision either way, the element-wise part is applied to what
is unique:
* O, dV: |got - want| <= 2e-2 max|want| + allowance (the width the admissible
  P^ and bf16 decisions span; zero for almost every element);
* dQ: a row within 2e-2 max|want| passes as it is.  A row beyond it passes
  if the oracle, recomputing that row with D_i shifted by an admissible
  amount (|a| <= e(D_i), the shift the O decisions allow) and the row's dS^
  codes re-rounded, lands within 2e-2 max|want| of it for some listed a
  (rows beyond half the bar are scanned, so the reported error shows what
  the shift explains);
* dK: |got - want| <= 2e-2 max|want|.
The cosine is always taken on the raw outputs.
"""

import numpy as np

TOL_REL = 2e-2
TOL_COS = 0.999


def cosine(got, want):
    g, w = got.ravel().astype(np.float64), want.ravel().astype(np.float64)
    return float(g @ w / np.sqrt((g @ g) * (w @ w)))


def _doc_of(al, t):
    """(document start, local row) of slice token t."""
    for s, e in al["docs"]:
        if s <= t < e:
            return s, t - s
    raise KeyError(t)


def dq_rows_under_shift(got, want, al, bar):
    """For each dQ row of ``got`` ([T, heads, d]) beyond half the bar: the
    smallest residual over the admissible D shifts the oracle lists (the scan
    stops once a shift brings the row within a tenth of the bar), and the
    shift that gives it.  Returns {(t, h): (residual, a)}."""
    out = {}
    diff = np.abs(got - want).max(axis=-1)
    for t, h in zip(*np.nonzero(diff > 0.5 * bar)):
        s, i = _doc_of(al, int(t))
        ev = al["dq_rows"][(s, int(h))]
        eD = float(al["e_D"][t, h])
        best = (float(diff[t, h]), 0.0)
        for a in ev.shifts(i, -eD, eD):
            r = float(np.abs(got[t, h] - ev.row(i, a)).max())
            if r < best[0]:
                best = (r, float(a))
            if r <= 0.1 * bar:
                break
        out[(int(t), int(h))] = best
    return out


def compare(name, got, want, al=None, tol=TOL_REL):
    """Returns (rel_plain, rel_applied, cosine, extra) for one output tensor
    ([T, heads, d]); ``al`` is oracle/decisions.allowances of the same inputs
    (None: plain comparison)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    M = max(np.max(np.abs(want)), 1e-30)
    diff = got - want
    rel_plain = float(np.max(np.abs(diff)) / M)
    extra = {}
    if al is None or name == "dk":
        rel = rel_plain
    elif name == "dq":
        shifted = dq_rows_under_shift(got, want, al, tol * M)
        rest = np.abs(diff).max(axis=-1)
        for (t, h), (r, _) in shifted.items():
            rest[t, h] = r
        rel = float(rest.max() / M)
        extra["rows_shifted"] = len(shifted)
        extra["max_shift_over_eD"] = max((abs(a) / max(float(al["e_D"][t, h]), 1e-300)
                                          for (t, h), (_, a) in shifted.items()), default=0.0)
    else:
        excess = np.abs(diff) - al[name]
        rel = float(max(np.max(excess), 0.0) / M)
        extra["allowed_elems"] = float(np.mean(al[name] > 1e-3 * M))
    return rel_plain, rel, cosine(got, want), extra


def check_outputs(outs, ref, al, tag, names=("o", "dq", "dk", "dv")):
    """outs: name -> GPU array; ref: oracle result; al: oracle/decisions.allowances
    of the same inputs.  Asserts the bar and returns the metrics."""
    res = {}
    for n in names:
        got = outs[n]
        assert np.all(np.isfinite(got)), n
        res[n] = compare(n, got, ref[n], al)
    print(f"[{tag}] " + ", ".join(
        f"{n} rel={r[0]:.2e}" + (f"->{r[1]:.2e}" if r[1] != r[0] else "") + f" cos={r[2]:.6f}"
        + (f" {r[3]}" if r[3] else "")
        for n, r in res.items()), flush=True)
    for n, (_, rel, cos, extra) in res.items():
        assert cos >= TOL_COS, (n, cos)
        assert rel <= TOL_REL, (n, rel, extra)
    return res
