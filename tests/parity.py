"""Parity metrics shared by the GPU tests.

Every comparison is relative L2 in fp64, taken twice: over the whole tensor,
and over each independent unit of the computation (a (sequence, value head)
pair of an output, one 128 x 128 state plane), where the largest unit error
must meet the same bar.  A unit that carries a small share of the tensor's
norm cannot hide a large error behind the whole-tensor figure that way.

Each unit's error is divided by its own reference norm, floored at half of
what a unit of its size typically carries: the tensor's RMS token-row norm
times sqrt(rows) for outputs, the RMS plane norm for states.

Short output units hold to a bar scaled by sqrt(64 / rows) (rows < 64: a
sequence shorter than one chunk), the standard-error scaling of an average
over fewer rows.  A one-token output row is rank one in the scalar qn.kn,
which for random unit vectors is ~N(0, 1/128); bf16 operands (8 significant
bits) give that scalar an absolute error of ~3e-4, so across thousands of
one-to-three-token units the worst relative error reaches the 1e-2 bar from
rounding alone.  The floor keeps an accidentally tiny reference from doing
the same.  A real fault in a unit (a wrong head, state, sequence boundary or
missing term) moves it by the order of its typical norm and is caught at
any length; units of 64 tokens or more meet the plain bar.
"""
from __future__ import annotations

import numpy as np

PLANE = (128, 128)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _units(a, cu):
    """Rows of `a` split into (unit, rows) pairs: per plane for [..., 128, 128]
    states (one row each), per (sequence, head) for token-major [T, H, D]
    tensors (sequences from cu, or all tokens as one sequence; rows = tokens),
    else the whole tensor as one unit."""
    if a.ndim >= 3 and a.shape[-2:] == PLANE:
        return [(x, 1) for x in a.reshape(-1, PLANE[0] * PLANE[1])]
    if a.ndim == 3:
        T, H = a.shape[0], a.shape[1]
        bounds = [0, T] if cu is None else [int(x) for x in np.asarray(cu).reshape(-1)]
        out = []
        for n in range(len(bounds) - 1):
            s, e = bounds[n], bounds[n + 1]
            if e > s:
                for h in range(H):
                    out.append((a[s:e, h].reshape(-1), e - s))
        return out
    return [(a.reshape(-1), 1)]


def unit_errors(got, ref, cu=None):
    """(whole-tensor rel-L2, per-unit relative errors, rows per unit)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    whole = _rel(got, ref)
    ug, ur = _units(got, cu), _units(ref, cu)
    if not ur:
        return whole, np.zeros(0), np.zeros(0)
    norms = np.array([np.linalg.norm(x) for x, _ in ur])
    rows = np.array([n for _, n in ur], dtype=np.float64)
    row_rms = float(np.sqrt(np.sum(norms ** 2) / np.sum(rows)))
    floors = 0.5 * row_rms * np.sqrt(rows)
    errs = np.array([np.linalg.norm(g - r) / max(nr, fl, 1e-300)
                     for (g, _), (r, _), nr, fl in zip(ug, ur, norms, floors)])
    return whole, errs, rows


def _scaled(errs, rows, planes):
    """Unit errors over their bars' multiple of the tolerance."""
    if planes:
        return errs
    return errs / np.sqrt(64.0 / np.minimum(np.maximum(rows, 1.0), 64.0))


def _is_planes(a):
    a = np.asarray(a)
    return a.ndim >= 3 and a.shape[-2:] == PLANE


def rel(got, ref, cu=None):
    """max(whole-tensor rel-L2, worst unit error over its bar's multiple of
    the tolerance): the figure tested against the tolerance."""
    whole, errs, rows = unit_errors(got, ref, cu)
    sc = _scaled(errs, rows, _is_planes(got))
    return max(whole, float(sc.max()) if sc.size else 0.0)


def report(name, got, ref, cu=None):
    """The figures, printed, and the tested one returned."""
    whole, errs, rows = unit_errors(got, ref, cu)
    sc = _scaled(errs, rows, _is_planes(got))
    worst = float(errs.max()) if errs.size else 0.0
    tested = max(whole, float(sc.max()) if sc.size else 0.0)
    print(f"  {name}: rel-L2 whole {whole:.3e}, worst of {errs.size} units {worst:.3e}, "
          f"tested {tested:.3e}", flush=True)
    return tested


def first_rows(x, cu, rows=64):
    """The first `rows` tokens of every sequence of a token-major tensor (the
    tokens where the initial state still shows under strong decay)."""
    x = np.asarray(x)
    b = [int(v) for v in np.asarray(cu).reshape(-1)]
    idx = np.concatenate([np.arange(b[n], min(b[n + 1], b[n] + rows))
                          for n in range(len(b) - 1)] or [np.zeros(0, dtype=np.int64)])
    return x[idx.astype(np.int64)]


def first_cu(cu, rows=64):
    """cu_seqlens of first_rows' result."""
    b = [int(v) for v in np.asarray(cu).reshape(-1)]
    lens = [min(b[n + 1] - b[n], rows) for n in range(len(b) - 1)]
    return np.concatenate([[0], np.cumsum(lens)])
