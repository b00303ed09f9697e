"""Independent fp64 forms of KDA, used to pin the token recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function takes the
inputs already widened to fp64 numpy arrays, in the varlen layout
q, k [T, Hqk, 128]; v, g [T, Hv, 128]; beta [T, Hv] (logits); cu [N+1];
s0 [N, Hv, 128(V), 128(K)] (V-first, or None) -- and returns fp64 arrays.

Forms and what pins each (the tests under tests/test_oracle_*.py):

``chunked``     the WY chunked form: per chunk of C tokens (chunks restart at
                every sequence start, the last one may be short), with the
                in-chunk cumulative log-decay G, the gated operands
                qg = qn e^G, kg = kn e^(G_last - G), d = e^G_last, the
                couplings A_kk (strictly lower, rows scaled by b) and A_qk
                (lower incl. diagonal) with per-element factors e^(G_t - G_i),
                T = (I + A_kk)^-1 by forward substitution, w = T (b kn e^G),
                u = T (b v), then U = u - w S, O = scale (qg S + A_qk U),
                S <- diag(d) S + kg^T U.  This is the operand set of page
                "vllm.models.kimi_k3.amd.ops.kda_chunk" (fused_kda_prologue
                workspaces qg / w / u / kg_t / aqk / decay, and the transfer
                diag(d_c) - w_c^T kg_c named in _chunk_groups).  Pinned against
                the recurrence to 1e-10 for C in {16, 32, 64}.
``window``      the short-window closed form of page
                "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify"
                (KdaTcVerify): probes p_t = e^cum_t kn_t, r_t = scale e^cum_t qn_t,
                w_i = e^-cum_i kn_i, couplings c_ti = w_i . p_t (i < t) and
                d_ti = w_i . r_t (i <= t), u_t = b_t (v_t - S0^T p_t - sum c_ti u_i),
                o_t = S0^T r_t + sum d_ti u_i.  Pinned against the recurrence at
                T <= 8 to 1e-12.
``brute``       dense transition matrices A_t = (I - b kn kn^T) diag(e^g),
                S_t = A_t S_{t-1} + b kn v^T, o_t = scale S_t^T qn: the problem
                statement's formula written out.  Pinned at T <= 8 to 1e-12.
``closed_b0``   b = 0: S_t = diag(e^G_t) S0, o_t = scale S0^T (e^G_t * qn_t).
``transfer``    the chunk-group composition S_out = P S_in + B with
                P = prod_c (diag(d_c) - kg_c^T w_c) over a run of chunks, and
                B the same run walked from zero (the exact transfer of
                _chunk_groups on the kda_chunk page).  Pinned to 1e-10 against
                a plain walk.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def l2n(x: np.ndarray) -> np.ndarray:
    """x / sqrt(sum(x^2) + 1e-6) along the last axis (KdaTcVerify's norm)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + EPS)


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _prep(q, k, beta, use_l2norm):
    if use_l2norm:
        q, k = l2n(q), l2n(k)
    return q, k, sigmoid(beta)


def _s_of(s0, n, h):
    """K x V state from the V-first buffer (element [v][k] holds S[k][v])."""
    if s0 is None:
        return np.zeros((128, 128))
    return np.array(s0[n, h].T, dtype=np.float64)


def unit_inverse_lower(A: np.ndarray) -> np.ndarray:
    """(I + A)^-1 for strictly lower-triangular A, by forward substitution."""
    L = A.shape[0]
    T = np.zeros_like(A)
    for t in range(L):
        row = np.zeros(L)
        row[t] = 1.0
        for i in range(t):
            row -= A[t, i] * T[i]
        T[t] = row
    return T


def chunk_operands(qn, kn, vv, gg, b):
    """Per-chunk operands of the WY form for one (sequence, head) chunk.

    qn, kn [L, K] (normalised), vv [L, V], gg [L, K] (natural-log decay per
    step), b [L].  Returns a dict with G, qg, kg, d, Akk, Aqk, T, w, u.
    """
    L = qn.shape[0]
    G = np.cumsum(gg, axis=0)
    tri = np.tril(np.ones((L, L), dtype=bool), -1)
    tri_d = np.tril(np.ones((L, L), dtype=bool), 0)
    diff = G[:, None, :] - G[None, :, :]                    # [t, i, c]
    E = np.exp(np.where(tri_d[:, :, None], diff, 0.0))      # only i <= t used
    Akk = np.where(tri, b[:, None] * np.einsum("tc,ic,tic->ti", kn, kn, E), 0.0)
    Aqk = np.where(tri_d, np.einsum("tc,ic,tic->ti", qn, kn, E), 0.0)
    T = unit_inverse_lower(Akk)
    eG = np.exp(G)
    w = T @ (b[:, None] * kn * eG)
    u = T @ (b[:, None] * vv)
    return dict(G=G, qg=qn * eG, kg=kn * np.exp(G[-1][None, :] - G), d=np.exp(G[-1]),
                Akk=Akk, Aqk=Aqk, T=T, w=w, u=u)


def chunked(q, k, v, g, beta, cu, scale, use_l2norm=True, s0=None, C=64,
            intermediates=False):
    """Naive fp64 chunked (WY) form.  Returns (out, final) or, with
    intermediates=True, (out, final, inter) where inter holds token-major
    qg, kg, w, u [T, Hv, 128], aqk [T, Hv, C] (column = token index inside its
    chunk) and decay d [n_chunks, Hv, 128] with chunks ordered by sequence,
    then position.
    """
    Ttot, hqk, K = q.shape
    hv = v.shape[1]
    grp = hv // hqk
    N = len(cu) - 1
    out = np.zeros((Ttot, hv, v.shape[2]))
    fin = np.zeros((N, hv, v.shape[2], K))
    if intermediates:
        nch = sum((int(cu[n + 1]) - int(cu[n]) + C - 1) // C for n in range(N))
        inter = dict(qg=np.zeros((Ttot, hv, K)), kg=np.zeros((Ttot, hv, K)),
                     w=np.zeros((Ttot, hv, K)), u=np.zeros((Ttot, hv, v.shape[2])),
                     aqk=np.zeros((Ttot, hv, C)), d=np.zeros((nch, hv, K)))
    for h in range(hv):
        hq = h // grp
        qh, kh, b = _prep(q[:, hq, :], k[:, hq, :], beta[:, h], use_l2norm)
        ci = 0
        for n in range(N):
            S = _s_of(s0, n, h)
            bos, eos = int(cu[n]), int(cu[n + 1])
            for s in range(bos, eos, C):
                e = min(s + C, eos)
                op = chunk_operands(qh[s:e], kh[s:e], v[s:e, h], g[s:e, h], b[s:e])
                U = op["u"] - op["w"] @ S
                out[s:e, h] = scale * (op["qg"] @ S + op["Aqk"] @ U)
                S = op["d"][:, None] * S + op["kg"].T @ U
                if intermediates:
                    L = e - s
                    for key in ("qg", "kg", "w", "u"):
                        inter[key][s:e, h] = op[key]
                    inter["aqk"][s:e, h, :L] = op["Aqk"]
                    inter["d"][ci, h] = op["d"]
                ci += 1
            fin[n, h] = S.T
    if intermediates:
        return out, fin, inter
    return out, fin


def window(q, k, v, g, beta, scale, use_l2norm=True, s0=None):
    """Short-window closed form for one sequence (T <= 8 tokens), all heads."""
    Tw, hqk, K = q.shape
    hv = v.shape[1]
    grp = hv // hqk
    out = np.zeros((Tw, hv, v.shape[2]))
    fin = np.zeros((1, hv, v.shape[2], K))
    for h in range(hv):
        qh, kh, b = _prep(q[:, h // grp, :], k[:, h // grp, :], beta[:, h], use_l2norm)
        S0 = _s_of(s0, 0, h)
        cum = np.cumsum(g[:, h, :], axis=0)
        p = np.exp(cum) * kh
        r = np.exp(cum) * qh * scale
        wv = np.exp(-cum) * kh
        u = np.zeros((Tw, v.shape[2]))
        for t in range(Tw):
            acc = v[t, h] - S0.T @ p[t]
            for i in range(t):
                acc = acc - np.dot(wv[i], p[t]) * u[i]
            u[t] = b[t] * acc
            o = S0.T @ r[t]
            for i in range(t + 1):
                o = o + np.dot(wv[i], r[t]) * u[i]
            out[t, h] = o
        S = np.exp(cum[-1])[:, None] * (S0 + wv.T @ u)
        fin[0, h] = S.T
    return out, fin


def brute(q, k, v, g, beta, scale, use_l2norm=True, s0=None):
    """Dense 128x128 transition matrices, one sequence, all heads."""
    Tw, hqk, K = q.shape
    hv = v.shape[1]
    grp = hv // hqk
    out = np.zeros((Tw, hv, v.shape[2]))
    fin = np.zeros((1, hv, v.shape[2], K))
    eye = np.eye(K)
    for h in range(hv):
        qh, kh, b = _prep(q[:, h // grp, :], k[:, h // grp, :], beta[:, h], use_l2norm)
        S = _s_of(s0, 0, h)
        for t in range(Tw):
            A = (eye - b[t] * np.outer(kh[t], kh[t])) @ np.diag(np.exp(g[t, h]))
            S = A @ S + b[t] * np.outer(kh[t], v[t, h])
            out[t, h] = scale * S.T @ qh[t]
        fin[0, h] = S.T
    return out, fin


def closed_b0(q, g, cu, scale, s0, hv, use_l2norm=True):
    """Closed form when every write strength is zero: the state only decays."""
    Ttot, hqk, K = q.shape
    grp = hv // hqk
    N = len(cu) - 1
    out = np.zeros((Ttot, hv, 128))
    fin = np.zeros((N, hv, 128, K))
    qh = l2n(q) if use_l2norm else q
    for n in range(N):
        bos, eos = int(cu[n]), int(cu[n + 1])
        for h in range(hv):
            S0 = _s_of(s0, n, h)
            G = np.cumsum(g[bos:eos, h], axis=0)
            for j, t in enumerate(range(bos, eos)):
                out[t, h] = scale * S0.T @ (np.exp(G[j]) * qh[t, h // grp])
            GL = G[-1] if eos > bos else np.zeros(K)
            fin[n, h] = (np.exp(GL)[:, None] * S0).T
    return out, fin


def transfer(qn, kn, vv, gg, b, chunk=64):
    """(P, B) for a run of tokens of one head: S_out = P S_in + B.

    P = prod over chunks (last first) of (diag(d_c) - kg_c^T w_c); B is the run
    walked from a zero state.  qn, kn, gg [L, K]; vv [L, V]; b [L].
    """
    K = qn.shape[1]
    P = np.eye(K)
    B = np.zeros((K, vv.shape[1]))
    for s in range(0, qn.shape[0], chunk):
        e = min(s + chunk, qn.shape[0])
        op = chunk_operands(qn[s:e], kn[s:e], vv[s:e], gg[s:e], b[s:e])
        M = np.diag(op["d"]) - op["kg"].T @ op["w"]
        P = M @ P
        B = M @ B + op["kg"].T @ op["u"]
    return P, B
