"""ctypes binding of libkda.so (include/kda.h).

Argument marshalling only: tensors are checked for the shapes the ABI sizes
describe (chunk_kda's checks on page "mate.kda"), outputs and the workspace are
allocated with torch, and the call goes through the C ABI on torch's current
stream.  Every step of the computation runs in the library's HIP kernels; there
is no fallback of any kind, and a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

D = 128
CHUNK = 64
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_ERR_SHAPE, KDA_ERR_DTYPE, KDA_ERR_UNSUPPORTED = 0, 1, 2, 3
KDA_ERR_WORKSPACE, KDA_ERR_HIP, KDA_ERR_ARG = 4, 5, 6
PATH_AUTO, PATH_STAGED, PATH_FUSED, PATH_ONCHIP = 0, 1, 2, 3

_DTYPES = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


class KdaError(RuntimeError):
    """The HIP runtime refused a launch, or the library is missing."""


class ChunkArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
        ("total_tokens", ctypes.c_int64),
        ("cu_seqlens", ctypes.c_void_p),
        ("hqk", ctypes.c_int32), ("hv", ctypes.c_int32),
        ("scale", ctypes.c_float), ("use_qk_l2norm", ctypes.c_int32),
        ("initial_state", ctypes.c_void_p), ("final_state", ctypes.c_void_p),
        ("state_cache", ctypes.c_void_p), ("state_indices", ctypes.c_void_p),
        ("has_initial_state", ctypes.c_void_p), ("num_slots", ctypes.c_int32),
        ("out", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("path", ctypes.c_int32), ("groups", ctypes.c_int32),
        ("walk_waves", ctypes.c_int32),
        ("stage_events", ctypes.c_void_p), ("num_stage_events", ctypes.c_int32),
        ("stream", ctypes.c_void_p),
        ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("dt_bias_dtype", ctypes.c_int32), ("lower_bound", ctypes.c_float),
        ("checkpoint_state", ctypes.c_void_p), ("checkpoint_offsets", ctypes.c_void_p),
        ("checkpoint_state_indices", ctypes.c_void_p), ("checkpoint_rows", ctypes.c_int32),
        ("state_dtype", ctypes.c_int32),
        ("q_stride", ctypes.c_int64), ("k_stride", ctypes.c_int64),
        ("v_stride", ctypes.c_int64), ("g_stride", ctypes.c_int64),
        ("beta_stride", ctypes.c_int64), ("state_slot_stride", ctypes.c_int64),
        ("max_seqlen", ctypes.c_int64),
    ]


NUM_STAGE_EVENTS = 7


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("chunk_offsets", "zero", "table", "qg", "kg_t", "decay", "w", "u", "aqk", "scan",
                 "total")
                ] + [("max_chunks", ctypes.c_int64), ("groups", ctypes.c_int32),
                     ("walk_waves", ctypes.c_int32)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("n", ctypes.c_int32),
        ("hqk", ctypes.c_int32), ("hv", ctypes.c_int32),
        ("scale", ctypes.c_float), ("use_qk_l2norm", ctypes.c_int32),
        ("state_cache", ctypes.c_void_p), ("state_indices", ctypes.c_void_p),
        ("num_slots", ctypes.c_int32), ("out", ctypes.c_void_p),
        ("stream", ctypes.c_void_p),
        ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("dt_bias_dtype", ctypes.c_int32), ("lower_bound", ctypes.c_float),
        ("tokens", ctypes.c_int32), ("state_index_cols", ctypes.c_int32),
        ("num_accepted_tokens", ctypes.c_void_p), ("state_dtype", ctypes.c_int32),
        ("q_stride", ctypes.c_int64), ("k_stride", ctypes.c_int64),
        ("v_stride", ctypes.c_int64), ("g_stride", ctypes.c_int64),
        ("beta_stride", ctypes.c_int64), ("state_slot_stride", ctypes.c_int64),
    ]


class VerifyArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("dtype", ctypes.c_int32), ("query_start", ctypes.c_void_p), ("n", ctypes.c_int32),
        ("hqk", ctypes.c_int32), ("hv", ctypes.c_int32), ("window", ctypes.c_int32),
        ("scale", ctypes.c_float), ("use_qk_l2norm", ctypes.c_int32),
        ("state_cache", ctypes.c_void_p), ("state_dtype", ctypes.c_int32),
        ("state_slot_stride", ctypes.c_int64), ("state_indices", ctypes.c_void_p),
        ("num_slots", ctypes.c_int32),
        ("corr", ctypes.c_void_p), ("kg", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("dt_bias_dtype", ctypes.c_int32), ("lower_bound", ctypes.c_float),
        ("q_stride", ctypes.c_int64), ("k_stride", ctypes.c_int64),
        ("v_stride", ctypes.c_int64), ("g_stride", ctypes.c_int64),
        ("beta_stride", ctypes.c_int64),
        ("stream", ctypes.c_void_p),
    ]


class CommitArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("state_cache", ctypes.c_void_p), ("state_dtype", ctypes.c_int32),
        ("state_slot_stride", ctypes.c_int64), ("num_slots", ctypes.c_int32),
        ("state_indices", ctypes.c_void_p), ("num_accepted_tokens", ctypes.c_void_p),
        ("corr", ctypes.c_void_p), ("kg", ctypes.c_void_p), ("dtype", ctypes.c_int32),
        ("n", ctypes.c_int32), ("hv", ctypes.c_int32), ("window", ctypes.c_int32),
        ("use_qk_l2norm", ctypes.c_int32),
        ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
        ("dt_bias_dtype", ctypes.c_int32), ("lower_bound", ctypes.c_float),
        ("stream", ctypes.c_void_p),
    ]


_lib = None
_lock = threading.Lock()
EXPORTS = ("kda_chunk_fwd", "kda_chunk_fwd_workspace_size", "kda_chunk_ws_layout",
           "kda_decode", "kda_status_str", "kda_last_error", "kda_version",
           "kda_chunk_fwd_noalloc", "kda_verify", "kda_commit")


def library_path() -> str:
    return os.environ.get("KDA_LIBRARY", _LIB_PATH)


def load_library():
    """Load libkda.so once; raise KdaError if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise KdaError(f"{path} is missing: build it with "
                               "`python -m gated_delta_rule_65_amd.build`")
            lib = ctypes.CDLL(path)
            P = ctypes.POINTER
            lib.kda_chunk_fwd.argtypes = [P(ChunkArgs)]
            lib.kda_chunk_fwd.restype = ctypes.c_int
            lib.kda_chunk_fwd_noalloc.argtypes = [P(ChunkArgs)]
            lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
            lib.kda_chunk_fwd_workspace_size.argtypes = [P(ChunkArgs), P(ctypes.c_size_t)]
            lib.kda_chunk_fwd_workspace_size.restype = ctypes.c_int
            lib.kda_chunk_ws_layout.argtypes = [P(ChunkArgs), P(WsLayout)]
            lib.kda_chunk_ws_layout.restype = ctypes.c_int
            lib.kda_decode.argtypes = [P(DecodeArgs)]
            lib.kda_decode.restype = ctypes.c_int
            lib.kda_status_str.argtypes = [ctypes.c_int32]
            lib.kda_status_str.restype = ctypes.c_char_p
            lib.kda_last_error.argtypes = []
            lib.kda_last_error.restype = ctypes.c_char_p
            lib.kda_version.argtypes = []
            lib.kda_version.restype = ctypes.c_char_p
            _lib = lib
    return _lib


def _raise(lib, status: int):
    msg = lib.kda_last_error().decode() or lib.kda_status_str(status).decode()
    if status == KDA_ERR_DTYPE:
        raise TypeError(msg)
    if status == KDA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if status in (KDA_ERR_SHAPE, KDA_ERR_WORKSPACE, KDA_ERR_ARG):
        raise ValueError(msg)
    raise KdaError(msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    if dev.type != "cuda":
        return None
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _gate(A_log, dt_bias, lower_bound, hv, dev):
    """Checked gate parameters (chunk_kda's A_log / dt_bias / lower_bound):
    (A_log, dt_bias, dt_bias dtype code, lower_bound), or Nones."""
    if A_log is None and dt_bias is None:
        return None, None, 0, float(lower_bound)
    _need(A_log is not None and dt_bias is not None,
          "A_log and dt_bias must be provided together.")
    _need(A_log.dtype == torch.float32, "A_log must be float32", TypeError)
    _need(dt_bias.dtype in (torch.float32, torch.bfloat16),
          "dt_bias must be float32 or bfloat16", TypeError)
    _need(tuple(A_log.shape) == (hv,), f"A_log must have shape [{hv}]")
    _need(tuple(dt_bias.shape) == (hv, D), f"dt_bias must have shape [{hv}, {D}]")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        _contig(name, t)
        _need(t.device == dev, f"{name} must be on {dev}")
    return A_log, dt_bias, _DTYPES[dt_bias.dtype], float(lower_bound)


def _checkpoints(state, offsets, indices, N, hv, dev):
    """Checked snapshot arguments: (state, int32 offsets, int32 indices or
    None), or None."""
    if state is None and offsets is None and indices is None:
        return None
    _need(state is not None and offsets is not None,
          "checkpoint_state and checkpoint_offsets must be given together")
    _need(state.dtype == torch.float32, "checkpoint_state must be float32", TypeError)
    _need(state.dim() == 4 and tuple(state.shape[1:]) == (hv, D, D) and state.shape[0] > 0,
          f"checkpoint_state must be [rows, {hv}, 128, 128]")
    _need(tuple(offsets.shape) == (N,), f"checkpoint_offsets must have shape [{N}]")
    _need(offsets.dtype in (torch.int32, torch.int64), "checkpoint_offsets must be integer")
    offs = offsets.to(device=dev, dtype=torch.int32).contiguous()
    idx = None
    if indices is not None:
        _need(tuple(indices.shape) == (N,), f"checkpoint_state_indices must have shape [{N}]")
        _need(indices.dtype in (torch.int32, torch.int64),
              "checkpoint_state_indices must be integer")
        idx = indices.to(device=dev, dtype=torch.int32).contiguous()
    else:
        _need(state.shape[0] >= N, "checkpoint_state needs a row per sequence")
    _contig("checkpoint_state", state)
    _need(state.device == dev, f"checkpoint_state must be on {dev}")
    return state, offs, idx


def _set_gate(a, gate):
    al, db, code, lb = gate
    a.A_log, a.dt_bias, a.dt_bias_dtype, a.lower_bound = _ptr(al), _ptr(db), code, lb


def _need(cond, msg, exc=ValueError):
    if not cond:
        raise exc(msg)


def _contig(name, t):
    _need(t.is_contiguous(), f"{name} must be contiguous")
    return t


def _token_stride(name, t, inner):
    """Elements between consecutive tokens of an input laid out as
    [token dims..., H, 128] (inner = 2) or [token dims..., H] (inner = 1, beta),
    0 when the tensor is contiguous.  A view into a wider projection output
    (each token's block dense, tokens a fixed stride apart) is passed as it
    is, without a copy."""
    if t.is_contiguous():
        return 0
    msg = (f"{name} must be contiguous, or a view whose tokens lie a fixed stride apart "
           f"with each token's last {inner} dims dense")
    dense = 1
    for d in range(t.dim() - 1, t.dim() - 1 - inner, -1):
        _need(t.shape[d] == 1 or t.stride(d) == dense, msg)
        dense *= t.shape[d]
    lead = [(t.shape[d], t.stride(d)) for d in range(t.dim() - inner) if t.shape[d] != 1]
    if not lead:
        return 0
    stride = run = lead[-1][1]
    for size, st in reversed(lead):
        _need(st == run, msg)
        run *= size
    _need(stride >= dense, msg)
    return 0 if stride == dense else stride


def _slot_stride(cache):
    """Elements between the slots of a [slots, Hv, 128, 128] state pool, 0 when
    dense (a pool whose slots are padded keeps each slot's planes dense)."""
    if cache is None or cache.is_contiguous():
        return 0
    hv = cache.shape[1]
    msg = "state pool slots must each be dense [Hv, 128, 128] blocks"
    _need(cache.stride(3) == 1 and cache.stride(2) == D and (hv == 1 or cache.stride(1) == D * D),
          msg)
    if cache.shape[0] == 1:
        return 0
    _need(cache.stride(0) >= hv * D * D, msg)
    return 0 if cache.stride(0) == hv * D * D else cache.stride(0)


def _set_strides(a, q, k, v, g, beta, cache):
    a.q_stride, a.k_stride = _token_stride("q", q, 2), _token_stride("k", k, 2)
    a.v_stride, a.g_stride = _token_stride("v", v, 2), _token_stride("g", g, 2)
    a.beta_stride = _token_stride("beta", beta, 1)
    a.state_slot_stride = _slot_stride(cache)


def _as_varlen(x, name, cu_seqlens):
    """[B, T, H, 128] dense, or [S, H, 128] / [1, S, H, 128] with cu_seqlens."""
    if cu_seqlens is None:
        _need(x.dim() == 4, f"{name} must be a 4D tensor [B, T, H, 128].")
        return x.reshape(x.shape[0] * x.shape[1], *x.shape[2:]), x.shape[0], x.shape[1]
    if x.dim() == 3:
        return x, 1, x.shape[0]
    _need(x.dim() == 4 and x.shape[0] == 1,
          f"{name} must be [S, H, 128] or [1, S, H, 128] for varlen.")
    return x[0], 1, x.shape[1]


def _chunk_struct(q, k, v, g, beta, out, cu, N, T, hqk, hv, scale, l2, init, fin, cache,
                  idx, has_init, path, groups, stream, walk_waves=0, gate=None, max_seqlen=0):
    a = ChunkArgs()
    a.struct_size = ctypes.sizeof(ChunkArgs)
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.dtype = _DTYPES[q.dtype]
    a.num_seqs, a.total_tokens = N, T
    a.cu_seqlens = _ptr(cu)
    a.hqk, a.hv = hqk, hv
    a.scale = scale
    a.use_qk_l2norm = 1 if l2 else 0
    a.initial_state, a.final_state = _ptr(init), _ptr(fin)
    st = init if init is not None else (fin if fin is not None else cache)
    a.state_dtype = _DTYPES[st.dtype] if st is not None else 0
    a.state_cache, a.state_indices, a.has_initial_state = _ptr(cache), _ptr(idx), _ptr(has_init)
    a.num_slots = 0 if cache is None else cache.shape[0]
    a.out = _ptr(out)
    a.path, a.groups, a.walk_waves = path, groups, walk_waves
    a.stream = stream
    _set_gate(a, gate if gate is not None else (None, None, 0, -5.0))
    _set_strides(a, q, k, v, g, beta, cache)
    a.max_seqlen = max_seqlen
    return a


def _prepare_chunk(q, k, v, g, beta, scale, initial_state, output_final_state, cu_seqlens,
                   use_qk_l2norm_in_kernel, output, final_state, state_cache, state_indices,
                   has_initial_state):
    varlen = cu_seqlens is not None
    q3, B, Tq = _as_varlen(q, "q", cu_seqlens)
    k3, _, _ = _as_varlen(k, "k", cu_seqlens)
    v3, _, _ = _as_varlen(v, "v", cu_seqlens)
    g3, _, _ = _as_varlen(g, "g", cu_seqlens)
    if varlen and beta.dim() == 3:
        _need(beta.shape[0] == 1, "beta must be [S, Hv] or [1, S, Hv] for varlen.")
        beta = beta[0]
    _need(q3.shape[-1] == D and k3.shape[-1] == D and v3.shape[-1] == D and g3.shape[-1] == D,
          "chunk_kda currently requires D=128.")
    _need(k.shape == q.shape, "k must have the same shape as q.")
    _need(q3.shape[0] == v3.shape[0] == g3.shape[0],
          "q, v and g must have matching [B, T] dimensions.")
    _need(g.shape == v.shape, "g must have the same shape as v.")
    hqk, hv = q3.shape[1], v3.shape[1]
    _need(hv % hqk == 0, "GVA requires v/g heads to be divisible by q/k heads.")
    T = q3.shape[0]
    beta2 = beta.reshape(T, -1) if not varlen else beta
    _need(tuple(beta2.shape) == (T, hv), "beta must have shape [B, T, Hv].")
    _need(q.dtype in (torch.float32, torch.bfloat16, torch.float16),
          "chunk_kda supports torch.float32, torch.bfloat16 and torch.float16 inputs.",
          TypeError)
    for name, t in (("k", k), ("v", v), ("g", g), ("beta", beta)):
        _need(t.dtype == q.dtype, "k, v, g and beta must have the same dtype as q.", TypeError)
    dev = q.device
    if varlen:
        _need(cu_seqlens.dtype in (torch.int32, torch.int64),
              "cu_seqlens must have dtype torch.int32 or torch.int64.", TypeError)
        cu = cu_seqlens.to(device=dev, dtype=torch.int32).contiguous()
        N = cu.numel() - 1
        # planning hint: known without a device sync only for host offsets
        max_seqlen = (int((cu_seqlens[1:] - cu_seqlens[:-1]).max())
                      if cu_seqlens.device.type == "cpu" and N > 0 else 0)
    else:
        cu = None
        N = B
        max_seqlen = 0
    if scale is None:
        scale = D ** -0.5
    paged = state_cache is not None
    init = fin = idx = hinit = None
    if paged:
        _need(initial_state is None and not output_final_state and final_state is None,
              "state_cache replaces initial_state/output_final_state")
        _need(state_indices is not None and has_initial_state is not None,
              "state_cache needs state_indices and has_initial_state")
        _need(state_cache.dtype in (torch.float32, q.dtype) and
              state_cache.dtype != torch.float16,
              f"state_cache must have dtype torch.float32 or {q.dtype} (not float16).",
              TypeError)
        _need(state_cache.dim() == 4 and tuple(state_cache.shape[1:]) == (hv, D, D),
              f"state_cache must be [slots, {hv}, 128, 128]")
        _slot_stride(state_cache)
        idx = state_indices.to(device=dev, dtype=torch.int32).contiguous()
        hinit = has_initial_state.to(device=dev, dtype=torch.uint8).contiguous()
        _need(idx.numel() == N and hinit.numel() == N,
              "state_indices and has_initial_state need one entry per sequence")
    else:
        # states are fp32 or of q's dtype (chunk_kda's rule), both alike; a new
        # final state takes the initial state's dtype, else fp32
        ok_state = (torch.float32,) if q.dtype == torch.float16 else (torch.float32, q.dtype)
        if initial_state is not None:
            _need(initial_state.dtype in ok_state,
                  f"initial_state must have dtype {q.dtype} or torch.float32.", TypeError)
            _need(tuple(initial_state.shape) == (N, hv, D, D),
                  f"initial_state must be [{N}, {hv}, 128, 128]")
            init = _contig("initial_state", initial_state)
        if output_final_state:
            if final_state is None:
                sdt = initial_state.dtype if initial_state is not None else torch.float32
                final_state = torch.empty((N, hv, D, D), device=dev, dtype=sdt)
            _need(final_state.dtype in ok_state,
                  f"final_state must have dtype {q.dtype} or torch.float32.", TypeError)
            _need(tuple(final_state.shape) == (N, hv, D, D),
                  f"final_state must be [{N}, {hv}, 128, 128]")
            fin = _contig("final_state", final_state)
        if init is not None and fin is not None:
            _need(init.dtype == fin.dtype, "initial_state and final_state must have the same dtype.",
                  TypeError)
    if output is None:
        output = torch.empty_like(v)
    _need(output.shape == v.shape or (varlen and output.shape == v3.shape),
          "output must have the same shape as v.")
    _need(output.dtype == q.dtype, "output must have the same dtype as q.", TypeError)
    for name, t in (("q", q3), ("k", k3), ("v", v3), ("g", g3), ("beta", beta2)):
        _token_stride(name, t, 1 if name == "beta" else 2)
        _need(t.device == dev, f"{name} must be on {dev}")
    _contig("output", output)
    _need(output.device == dev, f"output must be on {dev}")
    return dict(q=q3, k=k3, v=v3, g=g3, beta=beta2, out=output, cu=cu, N=N, T=T, hqk=hqk,
                hv=hv, scale=float(scale), l2=bool(use_qk_l2norm_in_kernel), init=init,
                fin=fin, cache=state_cache if paged else None, idx=idx, has_init=hinit,
                max_seqlen=max(0, max_seqlen))


def _run_chunk(p, path=PATH_AUTO, groups=0, workspace=None, keep=None, events=None,
               walk_waves=0, gate=None, ckpt=None, no_alloc=False):
    lib = load_library()
    dev = p["q"].device
    a = _chunk_struct(p["q"], p["k"], p["v"], p["g"], p["beta"], p["out"], p["cu"], p["N"],
                      p["T"], p["hqk"], p["hv"], p["scale"], p["l2"], p["init"], p["fin"],
                      p["cache"], p["idx"], p["has_init"], path, groups, _stream(dev),
                      walk_waves, gate, p["max_seqlen"])
    if ckpt is not None:
        cs, co, ci = ckpt
        a.checkpoint_state, a.checkpoint_offsets = _ptr(cs), _ptr(co)
        a.checkpoint_state_indices, a.checkpoint_rows = _ptr(ci), cs.shape[0]
        if keep is not None:
            keep["ckpt"] = ckpt
    if events is not None:
        arr = (ctypes.c_void_p * len(events))(*events)
        a.stage_events = ctypes.cast(arr, ctypes.c_void_p)
        a.num_stage_events = len(events)
    if no_alloc:
        # the library's static scratch replaces the workspace
        st = lib.kda_chunk_fwd_noalloc(ctypes.byref(a))
        if st != KDA_OK:
            _raise(lib, st)
        if keep is not None:
            keep["args"] = a
        return a
    nbytes = ctypes.c_size_t(0)
    st = lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(nbytes))
    if st != KDA_OK:
        _raise(lib, st)
    if workspace is None:
        workspace = torch.empty(max(int(nbytes.value), 1), dtype=torch.uint8, device=dev)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    st = lib.kda_chunk_fwd(ctypes.byref(a))
    if st != KDA_OK:
        _raise(lib, st)
    if keep is not None:
        keep["workspace"] = workspace
        keep["args"] = a
    return a


def chunk_kda(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=False,
              cu_seqlens=None, use_qk_l2norm_in_kernel=True, output=None, final_state=None,
              state_cache=None, state_indices=None, has_initial_state=None, groups=0,
              workspace=None, stage_events=None, walk_waves=0, path=PATH_AUTO,
              A_log=None, dt_bias=None, lower_bound=-5.0, checkpoint_state=None,
              checkpoint_offsets=None, checkpoint_state_indices=None, max_seqlen=None,
              no_alloc=False):
    """Chunked KDA forward (chunk_kda's argument set, plus the paged state of
    fused_kda_chunk).  Returns out, or (out, final_state) when
    output_final_state; in paged mode the final states land in state_cache.
    stage_events: optional list of up to 7 hipEvent_t handles (ints) recorded
    at the stage boundaries (profiling).  groups / walk_waves: 0 lets the
    planner choose; otherwise they fix the walk's launch shape (tuning only,
    the result is the same up to rounding order).  path: PATH_AUTO,
    PATH_STAGED (prep as its own kernel) or PATH_FUSED.  A_log [Hv] fp32 and
    dt_bias [Hv, 128] fp32/bf16 (both or neither) make g a raw gate with
    log-decay lower_bound * sigmoid(exp(A_log) * (g + dt_bias)).
    checkpoint_state [rows, Hv, 128, 128] fp32 with checkpoint_offsets [N]
    (and optionally checkpoint_state_indices [N]) snapshots each sequence's
    state after its first checkpoint_offsets[n] tokens (0 or a multiple of 64;
    fused_kda_chunk's checkpoint arguments).  max_seqlen: the longest sequence's
    length, a planning hint for varlen batches (taken from cu_seqlens when it
    is a host tensor; results never depend on it).  no_alloc: run through
    kda_chunk_fwd_noalloc, whose workspace is the library's static 64 MiB
    per-device scratch (no workspace argument; calls on one device must not
    overlap)."""
    _need(not (no_alloc and workspace is not None), "no_alloc takes no workspace")
    p = _prepare_chunk(q, k, v, g, beta, scale, initial_state, output_final_state,
                       cu_seqlens, use_qk_l2norm_in_kernel, output, final_state,
                       state_cache, state_indices, has_initial_state)
    if max_seqlen is not None:
        p["max_seqlen"] = int(max_seqlen)
    gate = _gate(A_log, dt_bias, lower_bound, p["hv"], p["q"].device)
    ck = _checkpoints(checkpoint_state, checkpoint_offsets, checkpoint_state_indices, p["N"],
                      p["hv"], p["q"].device)
    _run_chunk(p, path=path, groups=groups, workspace=workspace, events=stage_events,
               walk_waves=walk_waves, gate=gate, ckpt=ck, no_alloc=no_alloc)
    out = p["out"]
    if output_final_state:
        return out, p["fin"]
    return out


def chunk_workspace_bytes(q, k, v, g, beta, scale=None, initial_state=None,
                          output_final_state=False, cu_seqlens=None,
                          use_qk_l2norm_in_kernel=True, state_cache=None, state_indices=None,
                          has_initial_state=None, groups=0, walk_waves=0, path=PATH_AUTO,
                          max_seqlen=None):
    """Workspace bytes chunk_kda needs for these arguments (host-side only),
    so that a caller can allocate it once and pass it to every call."""
    p = _prepare_chunk(q, k, v, g, beta, scale, initial_state, output_final_state,
                       cu_seqlens, use_qk_l2norm_in_kernel, None, None,
                       state_cache, state_indices, has_initial_state)
    if max_seqlen is not None:
        p["max_seqlen"] = int(max_seqlen)
    a = _chunk_struct(p["q"], p["k"], p["v"], p["g"], p["beta"], p["out"], p["cu"], p["N"],
                      p["T"], p["hqk"], p["hv"], p["scale"], p["l2"], p["init"], p["fin"],
                      p["cache"], p["idx"], p["has_init"], path, groups, None, walk_waves,
                      None, p["max_seqlen"])
    lib = load_library()
    nbytes = ctypes.c_size_t(0)
    st = lib.kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(nbytes))
    if st != KDA_OK:
        _raise(lib, st)
    return int(nbytes.value)


def chunk_stages(q, k, v, g, beta, cu_seqlens=None, scale=None, initial_state=None,
                 use_qk_l2norm_in_kernel=True, groups=1, path=PATH_STAGED):
    """Run the chunk path (PATH_STAGED: prep as its own kernel; PATH_FUSED:
    prep folded into WY) and return its intermediates as raw views of the
    workspace (layouts and the packed fragment order as kda.h documents them):
    chunk_offsets, order (the sequences longest first), nch_max (the longest
    sequence's chunk count), qg, kg_t, decay, w, u_t, aqk, plus out and the
    final state.  For tests and tools."""
    p = _prepare_chunk(q, k, v, g, beta, scale, initial_state, True, cu_seqlens,
                       use_qk_l2norm_in_kernel, None, None, None, None, None)
    keep = {}
    a = _run_chunk(p, path=path, groups=groups, keep=keep)
    lib = load_library()
    lay = WsLayout()
    st = lib.kda_chunk_ws_layout(ctypes.byref(a), ctypes.byref(lay))
    if st != KDA_OK:
        _raise(lib, st)
    ws = keep["workspace"]
    dt = p["q"].dtype
    es = 4 if dt == torch.float32 else 2
    T, H, N, mc = p["T"], p["hv"], p["N"], lay.max_chunks

    def view(off, shape, dtype, esz):
        n = 1
        for s in shape:
            n *= s
        return ws[off:off + n * esz].view(dtype).view(*shape)

    return dict(
        out=p["out"], final_state=p["fin"],
        chunk_offsets=view(lay.chunk_offsets, (N + 1,), torch.int32, 4),
        order=view(lay.chunk_offsets + 4 * (N + 1), (N,), torch.int32, 4),
        nch_max=view(lay.zero + 1040, (1,), torch.int32, 4),
        qg=view(lay.qg, (T, H, D), dt, es),
        kg_t=view(lay.kg_t, (mc, H, D, CHUNK), dt, es),
        decay=view(lay.decay, (mc, H, D), torch.float32, 4),
        w=view(lay.w, (T, H, D), dt, es),
        u_t=view(lay.u, (mc, H, D, CHUNK), dt, es),
        aqk=view(lay.aqk, (T, H, CHUNK), dt, es),
    )


def kda_decode(q, k, v, g, beta, state_cache, state_indices=None, scale=None,
               use_qk_l2norm=True, output=None, A_log=None, dt_bias=None, lower_bound=-5.0,
               num_accepted_tokens=None):
    """Paged decode over the V-first fp32 state cache, updated in place
    (gated_delta_rule_decode's argument set).

    One token per request: q, k [N, Hqk, 128] or [N, 1, Hqk, 128]; v, g
    [N, Hv, 128] or [N, 1, Hv, 128]; beta [N, Hv] or [N, 1, Hv]; state_indices
    [N] (negative = skip) or None (identity).  T tokens per request (T <= 8,
    speculative / multi-token): q, k [N, T, Hqk, 128], v, g [N, T, Hv, 128],
    beta [N, T, Hv], state_indices [N, C >= T]: the request starts from row
    state_indices[n, a - 1] (a = num_accepted_tokens[n], column 0 without it)
    and writes its state after token t to row state_indices[n, t].  With
    A_log / dt_bias, g is a raw gate (the form chunk_kda takes).  Returns out
    shaped like v."""
    shape_v = v.shape
    if q.dim() == 4:
        T = q.shape[1]
        _need(1 <= T <= 8, "kda_decode takes 1 to 8 tokens per request", NotImplementedError)
        _need(q.shape[-1] == D, "q must be [N, T, Hqk, 128]")
        _need(k.shape == q.shape, "k must match q")
        _need(v.dim() == 4 and v.shape[:2] == q.shape[:2] and v.shape[-1] == D,
              "v must be [N, T, Hv, 128]")
        n, hqk, hv = q.shape[0], q.shape[2], v.shape[2]
        _need(g.shape == v.shape, "g must have the same shape as v")
        _need(tuple(beta.shape) == (n, T, hv), "beta must be [N, T, Hv]")
    else:
        T = 1
        _need(q.dim() == 3 and q.shape[-1] == D, "q must be [N, Hqk, 128]")
        _need(k.shape == q.shape, "k must match q")
        n, hqk = q.shape[0], q.shape[1]
        _need(v.dim() == 3 and v.shape[0] == n and v.shape[-1] == D, "v must be [N, Hv, 128]")
        hv = v.shape[1]
        _need(g.shape == v.shape, "g must have the same shape as v")
        _need(tuple(beta.shape) == (n, hv), "beta must be [N, Hv]")
    _need(hv % hqk == 0, f"Expected HV to be divisible by H, got HV={hv}, H={hqk}.")
    _need(q.dtype in _DTYPES, f"unsupported dtype {q.dtype}", TypeError)
    for name, t in (("k", k), ("v", v), ("g", g), ("beta", beta)):
        _need(t.dtype == q.dtype, f"{name} must have q's dtype", TypeError)
    _need(state_cache.dtype in (torch.float32, torch.bfloat16),
          "state must have dtype torch.float32 or torch.bfloat16", ValueError)
    _need(state_cache.dim() == 4 and tuple(state_cache.shape[1:]) == (hv, D, D),
          "state must have shape [pool, HV, V, K]")
    _need(state_cache.shape[0] > 0, "state pool must contain at least one slot.")
    dev = q.device
    idx, cols = None, 0
    if state_indices is not None:
        _need(state_indices.dim() in (1, 2) and state_indices.shape[0] == n,
              f"state_indices must have shape [{n}] or [{n}, T]")
        _need(state_indices.dtype in (torch.int32, torch.int64),
              "state_indices must have dtype torch.int32 or torch.int64", ValueError)
        if state_indices.dim() == 2:
            cols = state_indices.shape[1]
            _need(cols >= T, f"state_indices needs at least {T} columns, got {cols}")
        idx = state_indices.to(device=dev, dtype=torch.int32).contiguous()
    _need(cols > 0 or (T == 1 and num_accepted_tokens is None),
          "1D state_indices only support non-speculative single-token decode; use [B, T] "
          "state_indices for speculative or multi-token decode.")
    acc = None
    if num_accepted_tokens is not None:
        _need(tuple(num_accepted_tokens.shape) == (n,),
              f"num_accepted_tokens must have shape [B={n}]")
        _need(num_accepted_tokens.dtype in (torch.int32, torch.int64),
              "num_accepted_tokens must be integer")
        acc = num_accepted_tokens.to(device=dev, dtype=torch.int32).contiguous()
    if output is None:
        output = torch.empty(tuple(shape_v), dtype=q.dtype, device=dev)
    _need(output.numel() == n * T * hv * D and output.dtype == q.dtype,
          "output must be shaped like v, of q's dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _token_stride(name, t, 1 if name == "beta" else 2)
        _need(t.device == dev, f"{name} must be on {dev}")
    _slot_stride(state_cache)
    _contig("output", output)
    _need(state_cache.device == dev and output.device == dev,
          f"state_cache and output must be on {dev}")
    lib = load_library()
    a = DecodeArgs()
    a.struct_size = ctypes.sizeof(DecodeArgs)
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.dtype = _DTYPES[q.dtype]
    a.n, a.hqk, a.hv = n, hqk, hv
    a.scale = float(D ** -0.5 if scale is None else scale)
    a.use_qk_l2norm = 1 if use_qk_l2norm else 0
    a.state_cache = _ptr(state_cache)
    a.state_indices = _ptr(idx)
    a.num_slots = state_cache.shape[0]
    a.out = _ptr(output)
    a.stream = _stream(dev)
    _set_gate(a, _gate(A_log, dt_bias, lower_bound, hv, dev))
    a.tokens, a.state_index_cols, a.num_accepted_tokens = T, cols, _ptr(acc)
    a.state_dtype = _DTYPES[state_cache.dtype]
    _set_strides(a, q, k, v, g, beta, state_cache)
    st = lib.kda_decode(ctypes.byref(a))
    if st != KDA_OK:
        _raise(lib, st)
    return output.view(shape_v) if output.numel() == v.numel() else output


def _pool_checks(state_cache, hv, dev):
    _need(state_cache.dtype in (torch.float32, torch.bfloat16),
          "state must have dtype torch.float32 or torch.bfloat16", ValueError)
    _need(state_cache.dim() == 4 and tuple(state_cache.shape[1:]) == (hv, D, D),
          "state must have shape [pool, HV, V, K]")
    _need(state_cache.shape[0] > 0, "state pool must contain at least one slot.")
    _need(state_cache.device == dev, f"state_cache must be on {dev}")
    _slot_stride(state_cache)


def _int32_vec(x, n, name, dev):
    _need(tuple(x.shape) == (n,), f"{name} must have shape [{n}]")
    _need(x.dtype in (torch.int32, torch.int64), f"{name} must be integer", ValueError)
    return x.to(device=dev, dtype=torch.int32).contiguous()


def kda_verify(q, k, v, g, beta, query_start, state_cache, state_indices, window,
               scale=None, use_qk_l2norm=True, A_log=None, dt_bias=None, lower_bound=-5.0,
               output=None, corr=None, kg=None):
    """The record-based speculative verify step (KdaTcVerify's window form):
    request b runs its tokens q[query_start[b]:query_start[b+1]] (at most
    `window` <= 8 of them) from slot state_indices[b] of the paged state, and
    the step writes the outputs and, per (request, head, token), the records
    corr = the delta correction u_t (fp32) and kg = raw key then raw gate (q's
    dtype), but no state.

    q, k [T, Hqk, 128]; v, g [T, Hv, 128]; beta [T, Hv]; query_start [B + 1];
    state_cache [pool, Hv, 128, 128] fp32 or bf16 (read only); state_indices
    [B] (outside the pool: zero outputs, no records).  Returns (out [T, Hv,
    128], corr [B, Hv, window, 128], kg [B, Hv, window, 256])."""
    _need(q.dim() == 3 and q.shape[-1] == D, "q must be [T, Hqk, 128]")
    _need(k.shape == q.shape, "k must match q")
    T, hqk = q.shape[0], q.shape[1]
    _need(v.dim() == 3 and v.shape[0] == T and v.shape[-1] == D, "v must be [T, Hv, 128]")
    hv = v.shape[1]
    _need(g.shape == v.shape, "g must have the same shape as v")
    _need(tuple(beta.shape) == (T, hv), "beta must be [T, Hv]")
    _need(hv % hqk == 0, f"Expected HV to be divisible by H, got HV={hv}, H={hqk}.")
    _need(q.dtype in _DTYPES, f"unsupported dtype {q.dtype}", TypeError)
    for name, t in (("k", k), ("v", v), ("g", g), ("beta", beta)):
        _need(t.dtype == q.dtype, f"{name} must have q's dtype", TypeError)
    _need(1 <= int(window) <= 8, "window must lie in [1, 8]")
    dev = q.device
    n = query_start.numel() - 1
    _need(query_start.dim() == 1 and n >= 0, "query_start must be [B + 1]")
    qs = query_start.to(device=dev, dtype=torch.int32).contiguous()
    idx = _int32_vec(state_indices, n, "state_indices", dev)
    _pool_checks(state_cache, hv, dev)
    W = int(window)
    if output is None:
        output = torch.zeros((T, hv, D), dtype=q.dtype, device=dev)
    if corr is None:
        corr = torch.zeros((n, hv, W, D), dtype=torch.float32, device=dev)
    if kg is None:
        kg = torch.zeros((n, hv, W, 2 * D), dtype=q.dtype, device=dev)
    _need(tuple(output.shape) == (T, hv, D) and output.dtype == q.dtype,
          "output must be [T, Hv, 128] of q's dtype")
    _need(tuple(corr.shape) == (n, hv, W, D) and corr.dtype == torch.float32,
          "corr must be [B, Hv, window, 128] fp32")
    _need(tuple(kg.shape) == (n, hv, W, 2 * D) and kg.dtype == q.dtype,
          "kg must be [B, Hv, window, 256] of q's dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _token_stride(name, t, 1 if name == "beta" else 2)
        _need(t.device == dev, f"{name} must be on {dev}")
    for name, t in (("output", output), ("corr", corr), ("kg", kg)):
        _contig(name, t)
        _need(t.device == dev, f"{name} must be on {dev}")
    lib = load_library()
    a = VerifyArgs()
    a.struct_size = ctypes.sizeof(VerifyArgs)
    a.q, a.k, a.v, a.g, a.beta = _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta)
    a.dtype = _DTYPES[q.dtype]
    a.query_start, a.n, a.hqk, a.hv, a.window = _ptr(qs), n, hqk, hv, W
    a.scale = float(D ** -0.5 if scale is None else scale)
    a.use_qk_l2norm = 1 if use_qk_l2norm else 0
    a.state_cache, a.state_dtype = _ptr(state_cache), _DTYPES[state_cache.dtype]
    a.state_indices, a.num_slots = _ptr(idx), state_cache.shape[0]
    a.corr, a.kg, a.out = _ptr(corr), _ptr(kg), _ptr(output)
    _set_gate(a, _gate(A_log, dt_bias, lower_bound, hv, dev))
    _set_strides(a, q, k, v, g, beta, state_cache)
    a.stream = _stream(dev)
    st = lib.kda_verify(ctypes.byref(a))
    if st != KDA_OK:
        _raise(lib, st)
    return output, corr, kg


def kda_commit(state_cache, state_indices, num_accepted_tokens, corr, kg, use_qk_l2norm=True,
               A_log=None, dt_bias=None, lower_bound=-5.0):
    """Rebuild each request's state after its first a = num_accepted_tokens[b]
    window tokens from its slot's state and the kda_verify records, in place
    (a = 0, a count outside [0, window] or a slot outside the pool: left
    alone).  corr [B, Hv, window, 128] fp32 and kg [B, Hv, window, 256] as
    kda_verify returned them; the key normalisation and gate parameters must
    be the ones the verify step used."""
    _need(corr.dim() == 4 and corr.shape[-1] == D and corr.dtype == torch.float32,
          "corr must be [B, Hv, window, 128] fp32")
    n, hv, W = corr.shape[:3]
    _need(1 <= W <= 8, "window must lie in [1, 8]")
    _need(tuple(kg.shape) == (n, hv, W, 2 * D) and kg.dtype in _DTYPES,
          "kg must be [B, Hv, window, 256]")
    dev = corr.device
    idx = _int32_vec(state_indices, n, "state_indices", dev)
    acc = _int32_vec(num_accepted_tokens, n, "num_accepted_tokens", dev)
    _pool_checks(state_cache, hv, dev)
    for name, t in (("corr", corr), ("kg", kg)):
        _contig(name, t)
        _need(t.device == dev, f"{name} must be on {dev}")
    lib = load_library()
    a = CommitArgs()
    a.struct_size = ctypes.sizeof(CommitArgs)
    a.state_cache, a.state_dtype = _ptr(state_cache), _DTYPES[state_cache.dtype]
    a.state_slot_stride = _slot_stride(state_cache)
    a.num_slots = state_cache.shape[0]
    a.state_indices, a.num_accepted_tokens = _ptr(idx), _ptr(acc)
    a.corr, a.kg, a.dtype = _ptr(corr), _ptr(kg), _DTYPES[kg.dtype]
    a.n, a.hv, a.window = n, hv, W
    a.use_qk_l2norm = 1 if use_qk_l2norm else 0
    _set_gate(a, _gate(A_log, dt_bias, lower_bound, hv, dev))
    a.stream = _stream(dev)
    st = lib.kda_commit(ctypes.byref(a))
    if st != KDA_OK:
        _raise(lib, st)
    return state_cache


def chunk_plan(q, k, v, g, beta, cu_seqlens=None, initial_state=None, output_final_state=False,
               groups=0, walk_waves=0, max_seqlen=None, path=PATH_AUTO):
    """The walk's launch plan (groups, walk_waves) that chunk_kda takes for
    these arguments.  Host-side only: nothing runs on the device."""
    p = _prepare_chunk(q, k, v, g, beta, None, initial_state, output_final_state, cu_seqlens,
                       True, None, None, None, None, None)
    if max_seqlen is not None:
        p["max_seqlen"] = int(max_seqlen)
    a = _chunk_struct(p["q"], p["k"], p["v"], p["g"], p["beta"], p["out"], p["cu"], p["N"],
                      p["T"], p["hqk"], p["hv"], p["scale"], True, p["init"], p["fin"], None,
                      None, None, path, groups, None, walk_waves, None, p["max_seqlen"])
    lay = WsLayout()
    lib = load_library()
    st = lib.kda_chunk_ws_layout(ctypes.byref(a), ctypes.byref(lay))
    if st != KDA_OK:
        _raise(lib, st)
    return lay.groups, lay.walk_waves

