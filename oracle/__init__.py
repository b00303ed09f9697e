"""KDA oracle -- TEST INFRASTRUCTURE, not part of the product.

Plain, slow, fp64 CPU implementations of what the KDA chunked forward and the
T=1 decode compute.  Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import anything from here; the product
package never does, and nothing here imports the product package.

Contents
--------
``recurrence``      the definition, token by token (C, fp64, threaded): see
                    ``kda_oracle.c`` for the formula and its sources.
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
