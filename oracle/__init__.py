"""KDA oracle -- TEST INFRASTRUCTURE, not part of the product.

Plain, slow, fp64 CPU implementations of what the KDA chunked forward and the
T=1 decode compute.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import anything from here; the product
package never does, and nothing here imports the product package.

Contents
--------
``recurrence``      the definition, token by token (C, fp64, threaded): see
                    ``kda_oracle.c`` for the formula and its sources.
``decode``, ``decode_multi``, ``checkpoints``
                    one-token and multi-token decode over a paged cache, and
                    mid-prefill state snapshots, as the recurrence.
``verify``, ``commit``
                    the record-based speculative window (outputs and records
                    by the window form, no state) and the state rebuilt from
                    the records once the accepted count is known.
``forms``           independent fp64 forms used to pin the recurrence: the naive
                    chunked (WY) form, the short-window closed form, brute force
                    with dense 128x128 transition matrices, and special cases.

Parity status of each function is listed in ``forms``' module docstring.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np
import torch

from . import forms

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None
_lock = threading.Lock()

_DT = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/libkda_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            f = lib.oracle_kda_recurrence
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 6 + [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
            f = lib.oracle_kda_recurrence_gated
            f.restype = ctypes.c_int
            f.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 6 + [
                ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
            _lib = lib
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, min(n, 16))


def _cpu_contig(x: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    return x.detach().to("cpu").contiguous()


def recurrence(q, k, v, g, beta, cu_seqlens=None, scale=None, use_qk_l2norm=True,
               initial_state=None, heads=None, threads=None, want_state=True,
               A_log=None, dt_bias=None, lower_bound=-5.0):
    """Token-by-token fp64 KDA recurrence.

    With A_log [Hv] and dt_bias [Hv, 128] (both or neither, any float dtype,
    widened exactly) g is a raw gate and the step log-decay is
    lower_bound * sigmoid(exp(A_log[h]) * (g + dt_bias[h, c])).

    q, k: [T, Hqk, 128]; v, g: [T, Hv, 128]; beta: [T, Hv] (logits), all one of
    fp32/bf16/fp16 (read at their stored precision).  Dense [B, T, H, 128]
    inputs are accepted and flattened with cu_seqlens = [0, T, 2T, ...].
    initial_state: [N, Hv, 128(V), 128(K)] (any float dtype, widened) or None.
    heads: optional list of value heads to compute (others are left 0).

    Returns (out [T, Hv, 128] fp64 numpy, final_state [N, Hv, 128, 128] fp64
    numpy V-first, or None).
    """
    q = _cpu_contig(q, "q"); k = _cpu_contig(k, "k"); v = _cpu_contig(v, "v")
    g = _cpu_contig(g, "g"); beta = _cpu_contig(beta, "beta")
    if q.dim() == 4:
        B, T = q.shape[:2]
        if cu_seqlens is not None:
            raise ValueError("dense 4-D input takes no cu_seqlens")
        q, k = q.reshape(B * T, *q.shape[2:]), k.reshape(B * T, *k.shape[2:])
        v, g = v.reshape(B * T, *v.shape[2:]), g.reshape(B * T, *g.shape[2:])
        beta = beta.reshape(B * T, beta.shape[-1])
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if cu_seqlens is None:
            cu = np.array([0, q.shape[0]], dtype=np.int64)
        else:
            cu = np.asarray(torch.as_tensor(cu_seqlens).cpu().numpy(), dtype=np.int64)
    dt = q.dtype
    for name, x in (("k", k), ("v", v), ("g", g), ("beta", beta)):
        if x.dtype != dt:
            raise TypeError(f"{name} dtype {x.dtype} != q dtype {dt}")
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    Ttot, hqk, D = q.shape
    hv = v.shape[1]
    if D != 128 or v.shape[2] != 128 or hv % hqk:
        raise ValueError("bad head shapes")
    if scale is None:
        scale = 128 ** -0.5
    N = len(cu) - 1
    cu = np.ascontiguousarray(cu)
    s0 = None
    if initial_state is not None:
        s0 = np.ascontiguousarray(
            torch.as_tensor(initial_state).detach().cpu().double().numpy())
        if s0.shape != (N, hv, 128, 128):
            raise ValueError(f"initial_state shape {s0.shape} != {(N, hv, 128, 128)}")
    out = np.zeros((Ttot, hv, 128), dtype=np.float64)
    sf = np.zeros((N, hv, 128, 128), dtype=np.float64) if want_state else None
    hs = None
    if heads is not None:
        hs = np.ascontiguousarray(np.asarray(list(heads), dtype=np.int32))

    def ptr(t):
        if t is None:
            return None
        if isinstance(t, torch.Tensor):
            return ctypes.c_void_p(t.data_ptr())
        return t.ctypes.data_as(ctypes.c_void_p)

    if (A_log is None) != (dt_bias is None):
        raise ValueError("A_log and dt_bias must be given together")
    al = db = None
    if A_log is not None:
        al = np.ascontiguousarray(torch.as_tensor(A_log).detach().cpu().double().numpy())
        db = np.ascontiguousarray(torch.as_tensor(dt_bias).detach().cpu().double().numpy())
        if al.shape != (hv,) or db.shape != (hv, 128):
            raise ValueError("A_log must be [Hv] and dt_bias [Hv, 128]")
    lib = _load()
    rc = lib.oracle_kda_recurrence_gated(
        _DT[dt], ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(cu), N, hqk, hv,
        float(scale), int(bool(use_qk_l2norm)), ptr(al), ptr(db), float(lower_bound),
        ptr(s0), ptr(out), ptr(sf), ptr(hs), 0 if hs is None else len(hs),
        threads if threads else default_threads())
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out, sf


def decode(q, k, v, g, beta, state_cache, state_indices, scale=None,
           use_qk_l2norm=True, threads=None, A_log=None, dt_bias=None, lower_bound=-5.0):
    """One-token decode over a paged V-first state cache, as the recurrence.

    q, k: [N, Hqk, 128]; v, g: [N, Hv, 128]; beta: [N, Hv];
    state_cache: [slots, Hv, 128, 128]; state_indices: [N] (negative = skip).
    Returns (out [N, Hv, 128] fp64, new_cache fp64 copy of the cache with the
    touched rows replaced).  A skipped request has a zero output row and leaves
    the cache alone.
    """
    idx = np.asarray(torch.as_tensor(state_indices).cpu().numpy(), dtype=np.int64)
    cache = torch.as_tensor(state_cache).detach().cpu().double().numpy()
    n = idx.shape[0]
    live = np.nonzero(idx >= 0)[0]
    out = np.zeros((n,) + tuple(v.shape[1:]), dtype=np.float64)
    new_cache = cache.copy()
    if live.size == 0:
        return out, new_cache
    sel = torch.as_tensor(live)
    s0 = cache[idx[live]]
    o, sf = recurrence(q[sel], k[sel], v[sel], g[sel], beta[sel],
                       cu_seqlens=np.arange(live.size + 1, dtype=np.int64),
                       scale=scale, use_qk_l2norm=use_qk_l2norm,
                       initial_state=s0, threads=threads, A_log=A_log, dt_bias=dt_bias,
                       lower_bound=lower_bound)
    out[live] = o
    new_cache[idx[live]] = sf
    return out, new_cache


def checkpoints(q, k, v, g, beta, cu_seqlens, offsets, scale=None, use_qk_l2norm=True,
                initial_state=None, A_log=None, dt_bias=None, lower_bound=-5.0,
                alignment=64, threads=None):
    """Mid-prefill state snapshots: for each sequence n with a usable offset
    (0 < offsets[n] <= length, a multiple of ``alignment``) the recurrent state
    after its first offsets[n] tokens, V-first fp64 [Hv, 128, 128]; None for
    the others.  The snapshot of fused_kda_chunk (kda_chunk page): offsets are
    relative to each sequence's first token, 0 disables, unaligned ones are
    skipped.  Computed as the recurrence over each prefix alone.
    """
    cu = np.asarray(torch.as_tensor(cu_seqlens).cpu().numpy(), dtype=np.int64)
    offs = np.asarray(torch.as_tensor(offsets).cpu().numpy(), dtype=np.int64)
    q = _cpu_contig(q, "q"); k = _cpu_contig(k, "k"); v = _cpu_contig(v, "v")
    g = _cpu_contig(g, "g"); beta = _cpu_contig(beta, "beta")
    s0 = None if initial_state is None else torch.as_tensor(initial_state).detach().cpu()
    res = []
    for n in range(len(cu) - 1):
        length = cu[n + 1] - cu[n]
        o = int(offs[n])
        if o <= 0 or o > length or o % alignment:
            res.append(None)
            continue
        sl = slice(int(cu[n]), int(cu[n]) + o)
        _, sf = recurrence(q[sl], k[sl], v[sl], g[sl], beta[sl], scale=scale,
                           use_qk_l2norm=use_qk_l2norm,
                           initial_state=None if s0 is None else s0[n:n + 1],
                           A_log=A_log, dt_bias=dt_bias, lower_bound=lower_bound,
                           threads=threads)
        res.append(sf[0])
    return res


def round_bf16(x):
    """fp64 -> nearest bf16 value (ties to even), returned as fp64.  Done in
    integer arithmetic on the fp64 bit pattern (no intermediate fp32
    rounding): bf16 keeps the top 7 of fp64's 52 mantissa bits, with fp32's
    exponent range (values below bf16's smallest normal are flushed to
    zero here, far below anything a state holds)."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    bits = a.view(np.uint64)
    drop = np.uint64(52 - 7)
    half = np.uint64(1) << (drop - np.uint64(1))
    lsb = (bits >> drop) & np.uint64(1)
    r = ((bits + half - np.uint64(1) + lsb) >> drop) << drop
    out = r.view(np.float64).copy()
    out[np.abs(a) < 2.0 ** -126] = 0.0
    return out


def decode_multi(q, k, v, g, beta, state_cache, state_indices, num_accepted_tokens=None,
                 scale=None, use_qk_l2norm=True, A_log=None, dt_bias=None, lower_bound=-5.0,
                 threads=None, state_bf16=False):
    """Multi-token (speculative) decode over a paged V-first state cache.

    q, k: [B, T, Hqk, 128]; v, g: [B, T, Hv, 128]; beta: [B, T, Hv];
    state_indices: [B, C] with C >= T; num_accepted_tokens: [B] or None.
    Request b starts from cache row state_indices[b, a - 1] with
    a = num_accepted_tokens[b] (row state_indices[b, 0] without it), runs its
    T tokens in order, and after token t writes its state to row
    state_indices[b, t] when that index is >= 0.  A start row < 0 (or an
    accepted count outside [1, C]) skips the request: zero outputs, no writes.
    Each state is the recurrence over the request's tokens so far (computed
    here one prefix at a time).  With state_bf16 the state is stored in bf16:
    it is widened for each token's arithmetic and rounded back (to nearest
    even) after each token, as repeated single-token decode over a bf16 cache
    would do (mate.kda, gated_delta_rule_decode's bf16 state); outputs read
    the unrounded state of their token.  Returns (out [B, T, Hv, 128] fp64,
    new cache fp64).
    """
    idx = np.asarray(torch.as_tensor(state_indices).cpu().numpy(), dtype=np.int64)
    cache = torch.as_tensor(state_cache).detach().cpu().double().numpy()
    B, T = q.shape[0], q.shape[1]
    cols = idx.shape[1]
    acc = None if num_accepted_tokens is None else \
        np.asarray(torch.as_tensor(num_accepted_tokens).cpu().numpy(), dtype=np.int64)
    out = np.zeros(tuple(v.shape), dtype=np.float64)
    new_cache = cache.copy()
    for b in range(B):
        a = 1 if acc is None else int(acc[b])
        if a < 1 or a > cols or idx[b, a - 1] < 0:
            continue
        s0 = cache[idx[b, a - 1]][None]
        if state_bf16:
            s = round_bf16(s0)
            for t in range(T):
                o, sf = recurrence(q[b, t:t + 1], k[b, t:t + 1], v[b, t:t + 1], g[b, t:t + 1],
                                   beta[b, t:t + 1], scale=scale,
                                   use_qk_l2norm=use_qk_l2norm, initial_state=s,
                                   A_log=A_log, dt_bias=dt_bias, lower_bound=lower_bound,
                                   threads=threads)
                out[b, t] = o[0]
                s = round_bf16(sf)
                if idx[b, t] >= 0:
                    new_cache[idx[b, t]] = s[0]
            continue
        for t in range(T):
            o, sf = recurrence(q[b, :t + 1], k[b, :t + 1], v[b, :t + 1], g[b, :t + 1],
                               beta[b, :t + 1], scale=scale, use_qk_l2norm=use_qk_l2norm,
                               initial_state=s0, A_log=A_log, dt_bias=dt_bias,
                               lower_bound=lower_bound, threads=threads)
            out[b, t] = o[t]
            if idx[b, t] >= 0:
                new_cache[idx[b, t]] = sf[0]
    return out, new_cache


# ------------------------------------------------ verify window and commit
#
# The record-based speculative step of page
# "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify" (class KdaTcVerify):
# a request's window of at most Q <= 8 draft tokens is run from the slot's
# state S0 by the window closed form, writing the outputs and two records per
# (request, head, token) -- corr = the delta correction u_t, and kg = the raw
# key followed by the raw gate -- and no state.  Once the accepted count a is
# known, the commit rebuilds the state after the first a tokens from S0 and
# the records alone.  The pages show the verify step and name the records;
# the commit is our reading of what they are for (the recurrence with its
# corrections given, see ``commit``).


def _f64(x):
    return torch.as_tensor(x).detach().cpu().double().numpy()


def gate_log_decay(g_raw, h, A_log=None, dt_bias=None, lower_bound=-5.0):
    """Step log-decay of value head h from a raw gate [..., 128]: with gate
    parameters lower_bound * sigmoid(exp(A_log[h]) * (g_raw + dt_bias[h])),
    KdaTcVerify's activation (page
    "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify", step 2); without
    them g_raw already is the log-decay."""
    g_raw = np.asarray(g_raw, dtype=np.float64)
    if A_log is None:
        return g_raw
    a = np.exp(float(_f64(A_log)[h]))
    return lower_bound / (1.0 + np.exp(-a * (g_raw + _f64(dt_bias)[h])))


def verify(q, k, v, g, beta, query_start, state_cache, state_indices, window,
           scale=None, use_qk_l2norm=True, A_log=None, dt_bias=None, lower_bound=-5.0):
    """The verify step: outputs and records of each request's window.

    q, k: [T, Hqk, 128]; v, g: [T, Hv, 128]; beta: [T, Hv] logits; request b
    owns rows [query_start[b], query_start[b+1]) and its first
    min(length, window) tokens are run; state_cache [slots, Hv, 128(V),
    128(K)] (read only); state_indices [B] (a slot outside [0, slots) skips
    the request: zero output rows, no records).

    Per (request, head), with cum_t the inclusive cumulative log-decay over the
    window and qn, kn the (optionally L2-normalised) query and key, the page's
    window form (step 4 of KdaTcVerify): probes p_t = e^cum_t kn_t and
    r_t = scale e^cum_t qn_t, weights w_i = e^-cum_i kn_i, couplings
    c_ti = w_i . p_t (i < t) and d_ti = w_i . r_t (i <= t), then in token order
      u_t = b_t (v_t - S0^T p_t - sum_{i<t} c_ti u_i),
      o_t = S0^T r_t + sum_{i<=t} d_ti u_i,
    with S0 the K x V state (S0[k][v] = cache[slot, h, v, k]).

    Returns (out [T, Hv, 128], corr [B, Hv, window, 128] = u_t,
    kg [B, Hv, window, 256] = raw k of the head's query-key head, then raw g),
    fp64; record rows a request does not write are NaN.
    """
    qs = np.asarray(_f64(query_start), dtype=np.int64)
    idx = np.asarray(_f64(state_indices), dtype=np.int64)
    cache = _f64(state_cache)
    qd, kd, vd, gd, bd = (_f64(x) for x in (q, k, v, g, beta))
    Ttot, hqk, K = qd.shape
    hv = vd.shape[1]
    grp = hv // hqk
    B = len(qs) - 1
    Q = int(window)
    if scale is None:
        scale = K ** -0.5
    out = np.zeros((Ttot, hv, 128))
    corr = np.full((B, hv, Q, 128), np.nan)
    kg = np.full((B, hv, Q, 2 * K), np.nan)
    for b in range(B):
        bos = int(qs[b])
        n = max(0, min(int(qs[b + 1]) - bos, Q))
        slot = int(idx[b])
        if n == 0 or slot < 0 or slot >= cache.shape[0]:
            continue
        rows = slice(bos, bos + n)
        for h in range(hv):
            hq = h // grp
            qn, kn = qd[rows, hq], kd[rows, hq]
            if use_qk_l2norm:
                qn, kn = forms.l2n(qn), forms.l2n(kn)
            bt = forms.sigmoid(bd[rows, h])
            cum = np.cumsum(gate_log_decay(gd[rows, h], h, A_log, dt_bias, lower_bound), axis=0)
            S0 = cache[slot, h].T
            p = np.exp(cum) * kn
            r = scale * np.exp(cum) * qn
            w = np.exp(-cum) * kn
            u = np.zeros((n, 128))
            for t in range(n):
                acc = vd[bos + t, h] - S0.T @ p[t]
                for i in range(t):
                    acc = acc - np.dot(w[i], p[t]) * u[i]
                u[t] = bt[t] * acc
                o = S0.T @ r[t]
                for i in range(t + 1):
                    o = o + np.dot(w[i], r[t]) * u[i]
                out[bos + t, h] = o
            corr[b, h, :n] = u
            kg[b, h, :n, :K] = kd[rows, hq]
            kg[b, h, :n, K:] = gd[rows, h]
    return out, corr, kg


def commit(state_cache, state_indices, num_accepted_tokens, corr, kg, use_qk_l2norm=True,
           A_log=None, dt_bias=None, lower_bound=-5.0, state_bf16=False):
    """The state after each request's first a = num_accepted_tokens[b] window
    tokens, rebuilt from the slot's state and the verify records alone.

    The recurrence's step is S_t = diag(e^g_t) S_{t-1} + kn_t u_t^T, where
    u_t = b_t (v_t - (diag(e^g_t) S_{t-1})^T kn_t) is exactly the correction
    the verify step records; so with the records given the state after token
    a - 1 is that step applied for t = 0 .. a-1, with kn_t and g_t recomputed
    from the raw key and raw gate in kg.  A request with a slot outside the
    pool, or a count outside [0, window], is skipped; a = 0 leaves the state.
    With state_bf16 the new state is rounded (to nearest even) once, as it
    is stored once.  Returns the new cache, fp64 (a copy).
    """
    idx = np.asarray(_f64(state_indices), dtype=np.int64)
    acc = np.asarray(_f64(num_accepted_tokens), dtype=np.int64)
    cache = _f64(state_cache)
    u_all, kg_all = _f64(corr), _f64(kg)
    B, hv, Q = u_all.shape[:3]
    K = kg_all.shape[-1] // 2
    new = cache.copy()
    for b in range(B):
        slot, a = int(idx[b]), int(acc[b])
        if slot < 0 or slot >= cache.shape[0] or a < 0 or a > Q or a == 0:
            continue
        for h in range(hv):
            kn = kg_all[b, h, :a, :K]
            if use_qk_l2norm:
                kn = forms.l2n(kn)
            gl = gate_log_decay(kg_all[b, h, :a, K:], h, A_log, dt_bias, lower_bound)
            S = cache[slot, h].T.copy()
            for t in range(a):
                S = np.exp(gl[t])[:, None] * S + np.outer(kn[t], u_all[b, h, t])
            new[slot, h] = round_bf16(S.T) if state_bf16 else S.T
    return new
