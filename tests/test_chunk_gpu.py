"""Chunked forward on the GPU against the fp64 oracle.

Tolerances (relative L2): <= 1e-2 for bf16 inputs, <= 1e-4 for fp32 inputs,
for outputs and final states alike, met both over the whole tensor and by
the worst unit: each (sequence, value head) of an output, each state plane
(tests/parity.py).  Stage
intermediates (qg, kg_t, decay, w, u, aqk) are checked against the oracle's
chunked form at the same bars.  Exactness cases (zero write strength with no
decay, overwrite with orthonormal keys) are checked bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import stress
from oracle import forms
from gated_delta_rule_65_amd import binding as B
from gated_delta_rule_65_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


# max(whole-tensor, worst (sequence, head) / state-plane) relative L2
from parity import rel, report, first_rows, first_cu  # noqa: E402


_PATH = {"path": B.PATH_AUTO}


@pytest.fixture(autouse=True, params=["auto", "onchip"])
def chunk_path(request):
    """Every case runs twice: on the library's default plan, and with bf16
    calls sent down the on-chip path (the intra-chunk stage recomputed inside
    the walk).  fp32 calls keep the default plan, the on-chip path being
    bf16-only; calls that name a path keep it."""
    _PATH["path"] = B.PATH_ONCHIP if request.param == "onchip" else B.PATH_AUTO
    yield request.param
    _PATH["path"] = B.PATH_AUTO


def chunk_kda(q, *a, **kw):
    if kw.get("path", B.PATH_AUTO) == B.PATH_AUTO and q.dtype == torch.bfloat16:
        kw["path"] = _PATH["path"]
    return B.chunk_kda(q, *a, **kw)


def tol(dtype):
    return 1e-4 if dtype == torch.float32 else 1e-2


def say(*a):
    print(*a, flush=True)


def gpu(batch):
    return [t.to(DEV) for t in (batch.q, batch.k, batch.v, batch.g, batch.beta)]


def run_dense_state(batch, groups=0, l2=True, walk_waves=0):
    """Varlen call with dense initial/final states."""
    q, k, v, g, beta = gpu(batch)
    init = None if batch.initial_state is None else batch.initial_state.to(DEV)
    out, fin = chunk_kda(q, k, v, g, beta, scale=batch.scale, initial_state=init,
                           output_final_state=True, cu_seqlens=batch.cu_seqlens.to(DEV),
                           use_qk_l2norm_in_kernel=l2, groups=groups,
                           walk_waves=walk_waves)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), fin.cpu().numpy()


def oracle_dense(batch, heads=None, l2=True):
    return oracle.recurrence(batch.q, batch.k, batch.v, batch.g, batch.beta,
                             cu_seqlens=batch.cu_seqlens, scale=batch.scale,
                             use_qk_l2norm=l2, initial_state=batch.initial_state, heads=heads)


def f64(x):
    return x.detach().cpu().double().numpy()


# ------------------------------------------------------------------ workloads

def test_tiny_fp32_workload():
    """B=1, T=256, H=1, fp32, zero initial state, output + final state."""
    b = inputs.make_workload("tiny_fp32")
    say("tiny_fp32")
    out, fin = run_dense_state(b)
    o_ref, s_ref = oracle_dense(b)
    assert rel(out, o_ref) < 1e-4
    assert rel(fin, s_ref) < 1e-4


CASES = [
    # (name, lengths, hqk, hv, dtype, g_scale, init)
    ("ragged_bf16", [1, 63, 64, 65, 200, 7], 1, 2, torch.bfloat16, 5.0, True),
    ("ragged_fp32", [1, 63, 64, 65, 200, 7], 1, 2, torch.float32, 5.0, True),
    ("gva_bf16", [130, 77], 2, 8, torch.bfloat16, 5.0, True),
    ("slow_decay_bf16", [700, 300], 2, 2, torch.bfloat16, 0.5, True),
    ("weak_decay_bf16", [1500], 1, 2, torch.bfloat16, 0.01, True),
    ("weak_decay_fp32", [1000], 1, 1, torch.float32, 0.01, True),
    ("no_decay_fp32", [513], 1, 1, torch.float32, 0.0, True),
    ("zero_start_bf16", [256, 5], 1, 1, torch.bfloat16, 5.0, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunk_cases(case):
    name, lengths, hqk, hv, dt, gs, init = case
    b = inputs.make_chunk(lengths, hqk, hv, dtype=dt, g_scale=gs, seed=len(name), init=init)
    say("case", name, lengths, hqk, hv, dt, gs)
    out, fin = run_dense_state(b)
    o_ref, s_ref = oracle_dense(b)
    assert rel(out, o_ref, b.cu_seqlens) < tol(dt), report('out', out, o_ref, b.cu_seqlens)
    assert rel(fin, s_ref) < tol(dt), report('state', fin, s_ref)


def test_no_l2norm_custom_scale():
    b = inputs.make_chunk([100, 40], 1, 2, dtype=torch.float32, seed=4, init=True)
    b.q = b.q * 0.05
    b.k = b.k * 0.05   # un-normalised keys must keep the delta rule contractive
    b.scale = 0.7
    say("no_l2norm")
    out, fin = run_dense_state(b, l2=False)
    o_ref, s_ref = oracle_dense(b, l2=False)
    assert rel(out, o_ref, b.cu_seqlens) < 1e-4 and rel(fin, s_ref) < 1e-4


@pytest.mark.parametrize("nb,T,hqk,hv,dt,groups", [
    (2, 96, 2, 2, torch.bfloat16, 0),     # ragged last chunk
    (3, 1000, 1, 4, torch.bfloat16, 3),   # GVA, forced group scan
    (1, 4160, 2, 2, torch.bfloat16, 0),   # one sequence: the planner's group scan
    (2, 200, 1, 2, torch.float32, 2),     # fp32 operands
], ids=["ragged", "gva_scan", "single", "fp32_scan"])
def test_dense_4d_input_matches_varlen(nb, T, hqk, hv, dt, groups):
    """A dense batch given as [B, T, H, 128] (no cu_seqlens) equals the same
    batch given in varlen form, bit for bit, and the oracle."""
    b = inputs.make_chunk([T] * nb, hqk, hv, dtype=dt, seed=8 + T, init=True)
    q, k, v, g, beta = gpu(b)
    d4 = lambda x, h: x.view(nb, T, h, 128)
    out4, fin4 = chunk_kda(d4(q, hqk), d4(k, hqk), d4(v, hv), d4(g, hv), beta.view(nb, T, hv),
                           scale=b.scale, initial_state=b.initial_state.to(DEV),
                           output_final_state=True, groups=groups)
    out, fin = chunk_kda(q, k, v, g, beta, scale=b.scale,
                         initial_state=b.initial_state.to(DEV), output_final_state=True,
                         cu_seqlens=b.cu_seqlens.to(DEV), groups=groups)
    torch.cuda.synchronize()
    assert torch.equal(out4.view_as(out), out) and torch.equal(fin4, fin)
    o_ref, s_ref = oracle_dense(b)
    assert rel(out.float().cpu().numpy(), o_ref, b.cu_seqlens) < tol(dt)
    assert rel(fin.cpu().numpy(), s_ref) < tol(dt)


# ------------------------------------------------------- stage intermediates

def packed_to_logical(n):
    """Index array: logical element x of an axis of length n (a multiple of
    32) sits at packed position idx[x] (the fragment order kda.h states)."""
    idx = np.zeros(n, dtype=np.int64)
    for blk in range(0, n, 32):
        for gq in range(4):
            for j in range(8):
                x = 4 * gq + j if j < 4 else 16 + 4 * gq + (j - 4)
                idx[blk + x] = blk + 8 * gq + j
    return idx


def test_packed_order_is_a_permutation():
    for n in (32, 64, 128):
        assert sorted(packed_to_logical(n).tolist()) == list(range(n))


@pytest.mark.parametrize("path", [B.PATH_STAGED, B.PATH_FUSED], ids=["staged", "fused"])
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_stage_intermediates_match_chunked_form(dt, path):
    lengths = [70, 1, 128, 33]
    b = inputs.make_chunk(lengths, 1, 2, dtype=dt, seed=12, init=True)
    say("stages", dt, path)
    q, k, v, g, beta = gpu(b)
    st = B.chunk_stages(q, k, v, g, beta, cu_seqlens=b.cu_seqlens.to(DEV), scale=b.scale,
                        initial_state=b.initial_state.to(DEV), path=path)
    torch.cuda.synchronize()
    o_ref, s_ref, inter = forms.chunked(f64(b.q), f64(b.k), f64(b.v), f64(b.g), f64(b.beta),
                                        b.cu_seqlens.numpy(), b.scale, True,
                                        f64(b.initial_state), C=64, intermediates=True)
    offs = st["chunk_offsets"].cpu().numpy()
    expect = np.concatenate([[0], np.cumsum([(x + 63) // 64 for x in lengths])])
    assert np.array_equal(offs, expect)
    nch = int(offs[-1])
    t_ = tol(dt)
    p128, p64 = packed_to_logical(128), packed_to_logical(64)
    for key in ("qg", "w"):
        got = st[key].float().cpu().numpy()[..., p128]
        assert rel(got, inter[key]) < t_, key
    assert rel(st["aqk"].float().cpu().numpy()[..., p64], inter["aqk"]) < t_
    assert rel(st["decay"][:nch].cpu().numpy(), inter["d"]) < t_
    # kg_t and u_t: chunk-major and transposed; tokens past a short chunk are zero
    kgt = st["kg_t"][:nch].float().cpu().numpy()[..., p64]
    ut = st["u_t"][:nch].float().cpu().numpy()[..., p64]
    ref_k = np.zeros_like(kgt)
    ref_u = np.zeros_like(ut)
    cu = b.cu_seqlens.tolist()
    ci = 0
    for n in range(len(lengths)):
        for s in range(cu[n], cu[n + 1], 64):
            e = min(s + 64, cu[n + 1])
            ref_k[ci, :, :, :e - s] = inter["kg"][s:e].transpose(1, 2, 0)
            ref_u[ci, :, :, :e - s] = inter["u"][s:e].transpose(1, 2, 0)
            ci += 1
    assert rel(kgt, ref_k) < t_
    assert rel(ut, ref_u) < t_
    assert rel(st["out"].float().cpu().numpy(), o_ref, b.cu_seqlens) < t_
    assert rel(st["final_state"].cpu().numpy(), s_ref) < t_


# ------------------------------------------------------------- exactness cases

def test_zero_write_strength_no_decay_keeps_state_bitwise():
    """b = 0 (logit -1e4 -> sigmoid 0) and g = 0: the state passes through
    bit for bit and the output is the frozen-state read-out."""
    b = inputs.make_chunk([150, 64], 1, 2, dtype=torch.bfloat16, seed=2, init=True)
    b.beta.fill_(-1e4)
    b.g.zero_()
    say("b=0,g=0")
    out, fin = run_dense_state(b)
    assert np.array_equal(fin, b.initial_state.numpy())
    o_ref, _ = forms.closed_b0(f64(b.q), f64(b.g), b.cu_seqlens.numpy(), b.scale,
                               f64(b.initial_state), 2)
    assert rel(out, o_ref, b.cu_seqlens) < 1e-2


def test_zero_write_strength_with_decay_closed_form():
    b = inputs.make_chunk([300], 1, 1, dtype=torch.float32, g_scale=0.05, seed=3, init=True)
    b.beta.fill_(-1e4)
    say("b=0 decay")
    out, fin = run_dense_state(b)
    o_ref, s_ref = forms.closed_b0(f64(b.q), f64(b.g), b.cu_seqlens.numpy(), b.scale,
                                   f64(b.initial_state), 1)
    assert rel(out, o_ref) < 1e-4 and rel(fin, s_ref) < 1e-4


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_exact_overwrite_with_orthonormal_keys(dt):
    """b = 1 (logit 40), g = 0, distinct basis keys, q = k, scale 1, no norm,
    zero start: every product is x1 or +0, so o_t = v_t and row pi(t) of the
    state equals v_t exactly.  The fp32 path carries MFMA operands as a
    hi + lo bf16 pair, so its values are drawn on the bf16 grid (lo = 0)."""
    T, hv = 128, 2
    gen = torch.Generator().manual_seed(5)
    perm = torch.randperm(128, generator=gen)[:T]
    k = torch.zeros(T, 1, 128, dtype=dt)
    k[torch.arange(T), 0, perm] = 1
    v = torch.randn(T, hv, 128, generator=gen).to(torch.bfloat16).to(dt)
    g = torch.zeros(T, hv, 128, dtype=dt)
    beta = torch.full((T, hv), 40.0, dtype=dt)
    cu = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    say("overwrite", dt)
    out, fin = chunk_kda(k.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), beta.to(DEV), scale=1.0,
                           output_final_state=True, cu_seqlens=cu,
                           use_qk_l2norm_in_kernel=False)
    assert torch.equal(out.cpu(), v)
    fin = fin.cpu()
    for t in range(T):
        assert torch.equal(fin[0, :, :, perm[t]], v[t].float())


# ------------------------------------------------------------------ paged state

def test_paged_state_equals_dense_and_leaves_other_rows():
    lengths = [90, 0, 64, 131]
    b = inputs.make_chunk(lengths, 2, 4, dtype=torch.bfloat16, seed=21, paged_slots=9)
    b.has_initial_state = torch.tensor([1, 1, 0, 1], dtype=torch.uint8)
    say("paged")
    q, k, v, g, beta = gpu(b)
    cache = b.state_cache.to(DEV)
    out = chunk_kda(q, k, v, g, beta, scale=b.scale, cu_seqlens=b.cu_seqlens.to(DEV),
                      state_cache=cache, state_indices=b.state_indices.to(DEV),
                      has_initial_state=b.has_initial_state.to(DEV))
    torch.cuda.synchronize()
    idx = b.state_indices.long()
    s0 = b.state_cache[idx].clone()
    s0[2] = 0.0
    o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                     scale=b.scale, initial_state=s0)
    assert rel(out.float().cpu().numpy(), o_ref, b.cu_seqlens) < 1e-2
    got = cache.cpu()
    assert rel(got[idx].numpy(), s_ref) < 1e-2
    # the zero-length sequence passes its row through bit for bit
    assert torch.equal(got[idx[1]], b.state_cache[idx[1]])
    others = torch.ones(9, dtype=torch.bool)
    others[idx] = False
    assert torch.equal(got[others], b.state_cache[others])


def test_paged_null_slot_gives_zero_rows_and_no_state_io():
    lengths = [40, 70]
    b = inputs.make_chunk(lengths, 1, 2, dtype=torch.bfloat16, seed=22, paged_slots=4)
    b.state_indices = torch.tensor([-1, 2], dtype=torch.int32)
    say("null slot")
    q, k, v, g, beta = gpu(b)
    cache = b.state_cache.to(DEV)
    out = chunk_kda(q, k, v, g, beta, scale=b.scale, cu_seqlens=b.cu_seqlens.to(DEV),
                      state_cache=cache, state_indices=b.state_indices.to(DEV),
                      has_initial_state=b.has_initial_state.to(DEV))
    torch.cuda.synchronize()
    assert torch.all(out[:40].cpu() == 0)
    got = cache.cpu()
    for r in (0, 1, 3):
        assert torch.equal(got[r], b.state_cache[r])
    sl = slice(40, 110)
    o_ref, s_ref = oracle.recurrence(b.q[sl], b.k[sl], b.v[sl], b.g[sl], b.beta[sl],
                                     scale=b.scale, initial_state=b.state_cache[2:3])
    assert rel(out[40:].float().cpu().numpy(), o_ref) < 1e-2
    assert rel(got[2].numpy(), s_ref[0]) < 1e-2


def test_empty_batch_and_all_empty_sequences():
    b = inputs.make_chunk([0, 0], 1, 1, seed=1, init=True)
    q, k, v, g, beta = gpu(b)
    init = b.initial_state.to(DEV)
    out, fin = chunk_kda(q, k, v, g, beta, initial_state=init, output_final_state=True,
                           cu_seqlens=b.cu_seqlens.to(DEV))
    torch.cuda.synchronize()
    assert out.numel() == 0 and torch.equal(fin, init)


def test_deterministic():
    b = inputs.make_chunk([300, 77], 2, 4, seed=31, init=True)
    r1 = run_dense_state(b)
    r2 = run_dense_state(b)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])


def test_stage_events_sparse():
    """Stage events with NULL entries: only the given boundaries are recorded,
    the events complete, and the results equal a call without events bit for bit
    (also under the group scan, whose boundaries differ)."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventQuery.argtypes = [ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    b = inputs.make_chunk([300, 77, 0, 129], 2, 4, seed=33, init=True)
    q, k, v, g, beta = gpu(b)
    init = b.initial_state.to(DEV)
    cu = b.cu_seqlens.to(DEV)
    for groups in (1, 2):
        ref_o, ref_s = chunk_kda(q, k, v, g, beta, scale=b.scale, initial_state=init,
                                   output_final_state=True, cu_seqlens=cu, groups=groups)
        evs = []
        for _ in range(2):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e.value)
        # boundaries: after the table and after WY; every other entry NULL
        o, s = chunk_kda(q, k, v, g, beta, scale=b.scale, initial_state=init,
                           output_final_state=True, cu_seqlens=cu, groups=groups,
                           stage_events=[None, evs[0], None, evs[1], None, None, None])
        torch.cuda.synchronize()
        for e in evs:
            assert hip.hipEventSynchronize(ctypes.c_void_p(e)) == 0
            assert hip.hipEventQuery(ctypes.c_void_p(e)) == 0  # recorded and complete
            hip.hipEventDestroy(ctypes.c_void_p(e))
        assert torch.equal(o, ref_o) and torch.equal(s, ref_s)


# --------------------------------------------------------------- full workloads

def check_workload(out, o_ref, fin, s_ref, cu, t_=1e-2):
    """Whole-tensor and worst-unit figures for outputs and final states, plus
    the first 64 tokens of every sequence (where the initial state's
    influence is confined under strong decay), each held to the bar."""
    e_o = report("out", out, o_ref, cu)
    e_s = report("state", fin, s_ref)
    f_o = report("out, first 64 tokens per sequence", first_rows(out, cu),
                 first_rows(o_ref, cu), first_cu(cu))
    assert e_o < t_ and e_s < t_ and f_o < t_, (e_o, e_s, f_o)


def run_batched(batch, nb, tl):
    """The call bench.py times for a dense workload: [B, T, H, 128] tensors,
    no cu_seqlens, the library's own plan; returns varlen-shaped results."""
    q, k, v, g, beta = gpu(batch)
    d4 = lambda x: x.view(nb, tl, *x.shape[1:])
    out, fin = chunk_kda(d4(q), d4(k), d4(v), d4(g), d4(beta), scale=batch.scale,
                         initial_state=batch.initial_state.to(DEV), output_final_state=True)
    torch.cuda.synchronize()
    return out.reshape(nb * tl, *out.shape[2:]).float().cpu().numpy(), fin.cpu().numpy()


def test_dense_prefill_workload():
    """B=4, T=4096, H=16, bf16, fp32 initial state, as bench.py calls it:
    every output and state."""
    b = inputs.make_workload("dense_prefill")
    say("dense_prefill")
    out, fin = run_batched(b, 4, 4096)
    o_ref, s_ref = oracle_dense(b)
    check_workload(out, o_ref, fin, s_ref, b.cu_seqlens)


def test_varlen_gva_paged_workload():
    """24 log-uniform sequences (S = 32768), Hqk=8, Hv=32, paged cache [64,...]."""
    b = inputs.make_workload("varlen_gva_paged")
    say("varlen_gva_paged", b.meta["lengths"])
    q, k, v, g, beta = gpu(b)
    cache = b.state_cache.to(DEV)
    out = chunk_kda(q, k, v, g, beta, scale=b.scale, cu_seqlens=b.cu_seqlens.to(DEV),
                      state_cache=cache, state_indices=b.state_indices.to(DEV),
                      has_initial_state=b.has_initial_state.to(DEV))
    torch.cuda.synchronize()
    idx = b.state_indices.long()
    o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                     scale=b.scale, initial_state=b.state_cache[idx])
    got = cache.cpu()
    check_workload(out.float().cpu().numpy(), o_ref, got[idx].numpy(), s_ref, b.cu_seqlens)
    others = torch.ones(64, dtype=torch.bool)
    others[idx] = False
    assert torch.equal(got[others], b.state_cache[others])


def test_long_single_workload():
    """B=1, T=131072, H=32, slow decay, as bench.py calls it: every output
    and final state of all 32 heads."""
    b = inputs.make_workload("long_single")
    say("long_single")
    out, fin = run_batched(b, 1, 131072)
    o_ref, s_ref = oracle_dense(b)
    check_workload(out, o_ref, fin, s_ref, b.cu_seqlens)


# --------------------------------------------------- exponent-range limits

@pytest.mark.parametrize("groups", [1, 3])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_strongest_decay_everywhere(dt, groups):
    """g = -5 on every element (the strongest per-step decay the interface
    accepts), over ragged tails, with and without the group scan."""
    b = inputs.make_chunk([1, 63, 64, 65, 200, 7, 300], 1, 2, dtype=dt, seed=61, init=True)
    b.g.fill_(-5.0)
    say("g = -5", dt, groups)
    out, fin = run_dense_state(b, groups=groups)
    o_ref, s_ref = oracle_dense(b)
    assert report("out", out, o_ref, b.cu_seqlens) < tol(dt)
    assert report("state", fin, s_ref) < tol(dt)


@pytest.mark.parametrize("groups", [1, 4])
def test_gate_at_its_lower_bound(groups):
    """Gate parameters with lower_bound = -5 and dt_bias = +/-60 per channel:
    the sigmoid saturates, so every step's log-decay is exactly -5 or 0
    (alternating over channel pairs), the range limit of the interface."""
    b = inputs.make_chunk([700, 65], 1, 2, dtype=torch.bfloat16, g_scale=0.5, seed=62,
                          init=True)
    gen = torch.Generator().manual_seed(63)
    b.g = torch.randn(b.g.shape, generator=gen).to(torch.bfloat16)
    a_log = torch.zeros(2)
    sign = torch.tensor([1.0, 1.0, -1.0, -1.0]).repeat(32)
    dt_bias = (60.0 * sign).expand(2, 128).contiguous()
    say("gate at lower bound", groups)
    q, k, v, g, beta = gpu(b)
    out, fin = chunk_kda(q, k, v, g, beta, scale=b.scale, initial_state=b.initial_state.to(DEV),
                           output_final_state=True, cu_seqlens=b.cu_seqlens.to(DEV),
                           groups=groups, A_log=a_log.to(DEV), dt_bias=dt_bias.to(DEV),
                           lower_bound=-5.0)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                     scale=b.scale, initial_state=b.initial_state,
                                     A_log=a_log.double(), dt_bias=dt_bias.double(),
                                     lower_bound=-5.0)
    assert report("out", out.float().cpu().numpy(), o_ref, b.cu_seqlens) < 1e-2
    assert report("state", fin.cpu().numpy(), s_ref) < 1e-2


# ------------------------------------------------------------- group scan

SCAN_CASES = [
    # (name, lengths, hqk, hv, dtype, g_scale)
    ("weak_bf16", [2500], 1, 2, torch.bfloat16, 0.01),
    ("slow_bf16", [3000], 2, 2, torch.bfloat16, 0.5),
    ("nodecay_fp32", [1100], 1, 1, torch.float32, 0.0),
    ("varlen_bf16", [1300, 70, 1, 640, 200], 1, 2, torch.bfloat16, 0.05),
]


@pytest.mark.parametrize("groups,waves", [(2, 2), (4, 4), (8, 8), (3, 2), (1, 4), (1, 8)])
@pytest.mark.parametrize("case", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_group_scan_matches_oracle_and_plain_walk(case, groups, waves):
    """The chunk-group scan (pass one, compose, pass two) against the oracle,
    and against the plain walk (G = 1) on the same inputs.  Weak or no decay
    keeps the carried state visible in every output."""
    name, lengths, hqk, hv, dt, gs = case
    b = inputs.make_chunk(lengths, hqk, hv, dtype=dt, g_scale=gs, seed=40 + len(name), init=True)
    say("scan", name, groups, waves)
    o1, s1 = run_dense_state(b, groups=1, walk_waves=2)
    og, sg = run_dense_state(b, groups=groups, walk_waves=waves)
    o_ref, s_ref = oracle_dense(b)
    t_ = tol(dt)
    say("  rel vs oracle", rel(og, o_ref), rel(sg, s_ref), "vs plain walk", rel(og, o1),
        rel(sg, s1))
    assert rel(og, o_ref, b.cu_seqlens) < t_, report('out', og, o_ref, b.cu_seqlens)
    assert rel(sg, s_ref) < t_, report('state', sg, s_ref)
    # the scan reorders the same products; it must agree with the plain walk
    # well inside the oracle tolerance
    assert rel(og, o1, b.cu_seqlens) < t_ / 2 and rel(sg, s1) < t_ / 2


def test_group_scan_more_groups_than_chunks():
    b = inputs.make_chunk([100, 30], 1, 1, dtype=torch.float32, g_scale=0.1, seed=77, init=True)
    o, s = run_dense_state(b, groups=16)
    o_ref, s_ref = oracle_dense(b)
    assert rel(o, o_ref, b.cu_seqlens) < 1e-4 and rel(s, s_ref) < 1e-4


def test_group_scan_paged_with_null_slot():
    lengths = [900, 500, 64]
    b = inputs.make_chunk(lengths, 1, 2, dtype=torch.bfloat16, g_scale=0.05, seed=78,
                          paged_slots=6)
    b.state_indices = torch.tensor([4, -1, 1], dtype=torch.int32)
    b.has_initial_state = torch.tensor([1, 1, 0], dtype=torch.uint8)
    q, k, v, g, beta = gpu(b)
    cache = b.state_cache.to(DEV)
    out = chunk_kda(q, k, v, g, beta, scale=b.scale, cu_seqlens=b.cu_seqlens.to(DEV),
                      state_cache=cache, state_indices=b.state_indices.to(DEV),
                      has_initial_state=b.has_initial_state.to(DEV), groups=4)
    torch.cuda.synchronize()
    cu = b.cu_seqlens.tolist()
    assert torch.all(out[cu[1]:cu[2]].cpu() == 0)
    got = cache.cpu()
    for n, slot, start in ((0, 4, b.state_cache[4]), (2, 1, torch.zeros(2, 128, 128))):
        sl = slice(cu[n], cu[n + 1])
        o_ref, s_ref = oracle.recurrence(b.q[sl], b.k[sl], b.v[sl], b.g[sl], b.beta[sl],
                                         scale=b.scale, initial_state=start[None])
        assert rel(out[sl].float().cpu().numpy(), o_ref) < 1e-2
        assert rel(got[slot].numpy(), s_ref[0]) < 1e-2
    for r in (0, 2, 3, 5):
        assert torch.equal(got[r], b.state_cache[r])


def test_auto_plan_uses_groups_for_long_single_sequence():
    """The planner takes the group scan for one long sequence over few heads
    (and the result still matches the plain walk)."""
    b = inputs.make_chunk([16384], 2, 2, dtype=torch.bfloat16, g_scale=0.5, seed=79, init=True)
    q, k, v, g, beta = gpu(b)
    G, W = B.chunk_plan(q, k, v, g, beta, cu_seqlens=b.cu_seqlens.to(DEV),
                        initial_state=b.initial_state.to(DEV), output_final_state=True)
    assert G > 1 and W in (2, 4, 8)
    out_auto, fin_auto = chunk_kda(q, k, v, g, beta, scale=b.scale,
                                     initial_state=b.initial_state.to(DEV),
                                     output_final_state=True, cu_seqlens=b.cu_seqlens.to(DEV))
    out1, fin1 = chunk_kda(q, k, v, g, beta, scale=b.scale,
                             initial_state=b.initial_state.to(DEV), output_final_state=True,
                             cu_seqlens=b.cu_seqlens.to(DEV), groups=1)
    torch.cuda.synchronize()
    assert rel(out_auto.float().cpu().numpy(), out1.float().cpu().numpy()) < 5e-3
    assert rel(fin_auto.cpu().numpy(), fin1.cpu().numpy()) < 5e-3


def test_staged_and_fused_paths_agree():
    """Prep as its own kernel or folded into WY: the same intermediates up to
    the order of the gate cumsum, so outputs agree far inside the tolerance."""
    b = inputs.make_chunk([300, 64, 1, 900], 2, 8, dtype=torch.bfloat16, seed=81, init=True)
    q, k, v, g, beta = gpu(b)
    res = []
    for path in (B.PATH_STAGED, B.PATH_FUSED):
        o, s = chunk_kda(q, k, v, g, beta, scale=b.scale, initial_state=b.initial_state.to(DEV),
                           output_final_state=True, cu_seqlens=b.cu_seqlens.to(DEV), path=path)
        torch.cuda.synchronize()
        res.append((o.float().cpu().numpy(), s.cpu().numpy()))
    say("staged vs fused", rel(res[1][0], res[0][0]), rel(res[1][1], res[0][1]))
    assert rel(res[1][0], res[0][0], b.cu_seqlens) < 2e-3 and rel(res[1][1], res[0][1]) < 2e-3
    o_ref, s_ref = oracle_dense(b)
    assert rel(res[1][0], o_ref, b.cu_seqlens) < 1e-2 and rel(res[1][1], s_ref) < 1e-2


# ------------------------------------------------------------ gate parameters

GATE_CASES = [
    # (name, lengths, hqk, hv, dtype, path, groups, dt_bias dtype)
    ("bf16_fused", [300, 64, 1, 200], 2, 4, torch.bfloat16, B.PATH_FUSED, 0, torch.float32),
    ("bf16_staged", [300, 64, 1, 200], 2, 4, torch.bfloat16, B.PATH_STAGED, 0, torch.float32),
    ("bf16_bias_bf16", [257, 100], 1, 2, torch.bfloat16, B.PATH_FUSED, 0, torch.bfloat16),
    ("fp32", [130, 70], 1, 2, torch.float32, B.PATH_FUSED, 0, torch.float32),
    ("bf16_scan", [1500], 1, 2, torch.bfloat16, B.PATH_FUSED, 4, torch.float32),
]


@pytest.mark.parametrize("case", GATE_CASES, ids=[c[0] for c in GATE_CASES])
def test_gate_parameters_match_oracle(case):
    """g as a raw gate: log-decay lower_bound * sigmoid(exp(A_log) (g + dt_bias)),
    applied in the kernels, against the oracle with the same stored values."""
    name, lengths, hqk, hv, dt, path, groups, bdt = case
    b = inputs.make_chunk(lengths, hqk, hv, dtype=dt, seed=90, init=True)
    gen = torch.Generator().manual_seed(91)
    b.g = torch.randn(b.g.shape, generator=gen).to(dt)
    a_log = (torch.rand(hv, generator=gen) * 2 - 1).float()
    dt_bias = (torch.randn(hv, 128, generator=gen) * 0.5).to(bdt)
    say("gate", name)
    q, k, v, g, beta = gpu(b)
    out, fin = chunk_kda(q, k, v, g, beta, scale=b.scale, initial_state=b.initial_state.to(DEV),
                           output_final_state=True, cu_seqlens=b.cu_seqlens.to(DEV),
                           path=path, groups=groups, A_log=a_log.to(DEV),
                           dt_bias=dt_bias.to(DEV), lower_bound=-5.0)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                     scale=b.scale, initial_state=b.initial_state,
                                     A_log=a_log.double(), dt_bias=dt_bias.double(),
                                     lower_bound=-5.0)
    t_ = tol(dt)
    assert rel(out.float().cpu().numpy(), o_ref, b.cu_seqlens) < t_
    assert rel(fin.cpu().numpy(), s_ref) < t_


# ---------------------------------------------------- mid-prefill checkpoints

SENTINEL = 7.0


def run_checkpoints(b, offsets, rows, indices=None, groups=0, dtype=None):
    q, k, v, g, beta = gpu(b)
    hv = b.v.shape[1]
    ck = torch.full((rows, hv, 128, 128), SENTINEL, dtype=torch.float32, device=DEV)
    offs = torch.tensor(offsets, dtype=torch.int32)
    idx = None if indices is None else torch.tensor(indices, dtype=torch.int32)
    out, fin = chunk_kda(q, k, v, g, beta, scale=b.scale, initial_state=b.initial_state.to(DEV),
                           output_final_state=True, cu_seqlens=b.cu_seqlens.to(DEV),
                           groups=groups, checkpoint_state=ck, checkpoint_offsets=offs.to(DEV),
                           checkpoint_state_indices=None if idx is None else idx.to(DEV))
    torch.cuda.synchronize()
    refs = oracle.checkpoints(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, offs, scale=b.scale,
                              initial_state=b.initial_state)
    return ck.cpu().numpy(), refs, out, fin


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_checkpoints_match_oracle_and_skip_unusable_offsets(dt):
    lengths = [300, 64, 1, 200, 128]
    b = inputs.make_chunk(lengths, 1, 2, dtype=dt, g_scale=0.5, seed=95, init=True)
    offsets = [128, 64, 0, 96, 128]     # aligned, = length, disabled, unaligned, = length
    say("checkpoints", dt)
    ck, refs, _, fin = run_checkpoints(b, offsets, rows=5)
    t_ = tol(dt)
    for n, r in enumerate(refs):
        if r is None:
            assert np.all(ck[n] == SENTINEL), n
        else:
            assert rel(ck[n], r) < t_, n
    # an offset equal to the length is the final state, bit for bit
    assert np.array_equal(ck[4], fin[4].cpu().numpy())
    assert np.array_equal(ck[1], fin[1].cpu().numpy())


def test_checkpoints_through_row_indices():
    lengths = [300, 64, 200]
    b = inputs.make_chunk(lengths, 2, 4, dtype=torch.bfloat16, g_scale=0.5, seed=96, init=True)
    ck, refs, _, _ = run_checkpoints(b, [256, 64, 192], rows=4, indices=[3, -1, 0])
    assert rel(ck[3], refs[0]) < 1e-2
    assert rel(ck[0], refs[2]) < 1e-2
    assert np.all(ck[1] == SENTINEL) and np.all(ck[2] == SENTINEL)


def test_checkpoints_under_the_group_scan():
    b = inputs.make_chunk([1500], 1, 2, dtype=torch.bfloat16, g_scale=0.05, seed=97, init=True)
    ck, refs, _, _ = run_checkpoints(b, [640], rows=1, groups=4)
    assert rel(ck[0], refs[0]) < 1e-2


# ------------------------------------------------------- bf16 initial / final

@pytest.mark.parametrize("groups", [1, 4])
def test_bf16_initial_and_final_state(groups):
    """States stored in bf16 (chunk_kda allows q's dtype): the initial state is
    widened exactly, the final state rounded to nearest even."""
    b = inputs.make_chunk([700, 300], 1, 2, dtype=torch.bfloat16, g_scale=0.5, seed=98,
                          init=True)
    init16 = b.initial_state.to(torch.bfloat16)
    q, k, v, g, beta = gpu(b)
    out, fin = chunk_kda(q, k, v, g, beta, scale=b.scale, initial_state=init16.to(DEV),
                           output_final_state=True, cu_seqlens=b.cu_seqlens.to(DEV),
                           groups=groups)
    torch.cuda.synchronize()
    assert fin.dtype == torch.bfloat16
    o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                     scale=b.scale, initial_state=init16)
    assert rel(out.float().cpu().numpy(), o_ref, b.cu_seqlens) < 1e-2
    assert rel(fin.float().cpu().numpy(), s_ref) < 1e-2


def test_bf16_state_b0_passes_through_bitwise():
    """b = 0, g = 0: a bf16 initial state comes back bit for bit."""
    b = inputs.make_chunk([150, 64], 1, 2, dtype=torch.bfloat16, seed=99, init=True)
    b.beta.fill_(-1e4)
    b.g.zero_()
    init16 = b.initial_state.to(torch.bfloat16)
    q, k, v, g, beta = gpu(b)
    _, fin = chunk_kda(q, k, v, g, beta, scale=b.scale, initial_state=init16.to(DEV),
                         output_final_state=True, cu_seqlens=b.cu_seqlens.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(fin.cpu(), init16)


# ------------------------------------------------- strided (projection) inputs

def projection_views(tensors, dev, pad=8):
    """q, k, v, g ([T, H, 128]) and beta ([T, Hv]) copied into bands of one
    [T, W] buffer, as the slices of a fused projection output; returns views.
    W keeps every token row 16-byte aligned."""
    T = tensors[0].shape[0]
    flat = [t.reshape(T, -1) for t in tensors]
    W = sum(f.shape[1] for f in flat) + pad
    W += (-W) % 8
    proj = torch.full((T, W), float("nan"), dtype=tensors[0].dtype, device=dev)
    views, off = [], 0
    for t, f in zip(tensors, flat):
        proj[:, off:off + f.shape[1]] = f.to(dev)
        views.append(proj[:, off:off + f.shape[1]].view(t.shape))
        off += f.shape[1]
    return views, proj


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("path,groups", [(B.PATH_FUSED, 1), (B.PATH_STAGED, 1),
                                         (B.PATH_FUSED, 3)])
def test_strided_projection_inputs(dtype, path, groups):
    """Inputs read through a per-token stride (bands of one projection buffer,
    NaN padding between them) equal the contiguous run bit for bit, and the
    oracle at the usual bar."""
    b = inputs.make_chunk([300, 190, 64], 2, 4, dtype=dtype, g_scale=0.5, seed=97, init=True)
    say("strided", dtype, path, groups)
    (qv, kv, vv, gv, bv), proj = projection_views([b.q, b.k, b.v, b.g, b.beta], DEV)
    assert not qv.is_contiguous() and qv.stride(0) == proj.shape[1]
    init = b.initial_state.to(DEV)
    cu = b.cu_seqlens.to(DEV)
    kw = dict(scale=b.scale, initial_state=init, output_final_state=True, cu_seqlens=cu,
              path=path, groups=groups)
    out_s, fin_s = chunk_kda(qv, kv, vv, gv, bv, **kw)
    out_c, fin_c = chunk_kda(*gpu(b), **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_c) and torch.equal(fin_s, fin_c)
    o_ref, s_ref = oracle_dense(b)
    assert rel(out_s.float().cpu().numpy(), o_ref, b.cu_seqlens) < tol(dtype)
    assert rel(fin_s.cpu().numpy(), s_ref) < tol(dtype)


def test_strided_inputs_with_gate_and_padded_paged_pool():
    """Projection views with the gate parameters, into a paged pool whose slots
    are padded (slot stride above Hv*128*128)."""
    b = inputs.make_chunk([200, 130], 1, 2, dtype=torch.bfloat16, seed=96,
                          paged_slots=5)
    hv = 2
    al = torch.tensor([0.3, -0.2])
    dtb = torch.randn(hv, 128, generator=torch.Generator().manual_seed(3)) * 0.5
    (qv, kv, vv, gv, bv), _ = projection_views([b.q, b.k, b.v, b.g, b.beta], DEV)
    plane = hv * 128 * 128
    pool = torch.full((5, plane + 192), float("nan"), device=DEV)
    cache = pool[:, :plane].view(5, hv, 128, 128)
    cache.copy_(b.state_cache.to(DEV))
    ref_cache = b.state_cache.to(DEV).clone()
    kw = dict(scale=b.scale, cu_seqlens=b.cu_seqlens.to(DEV),
              state_indices=b.state_indices.to(DEV), has_initial_state=b.has_initial_state.to(DEV),
              A_log=al.to(DEV), dt_bias=dtb.to(DEV))
    out_s = chunk_kda(qv, kv, vv, gv, bv, state_cache=cache, **kw)
    out_c = chunk_kda(*gpu(b), state_cache=ref_cache, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_c)
    assert torch.equal(cache, ref_cache)
    assert torch.isnan(pool[:, plane:]).all()   # the padding is never written
    o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                     scale=b.scale, initial_state=b.state_cache[
                                         b.state_indices.long()] * b.has_initial_state.view(
                                         -1, 1, 1, 1).float(),
                                     A_log=al.double(), dt_bias=dtb.double())
    assert rel(out_s.float().cpu().numpy(), o_ref, b.cu_seqlens) < 1e-2
    live = b.state_indices.long().numpy()
    assert rel(cache.cpu().numpy()[live], s_ref) < 1e-2


# -------------------------------------------- exactness under the group scan

@pytest.mark.parametrize("groups", [2, 4])
def test_group_scan_keeps_empty_sequences_and_end_checkpoints_exact(groups):
    """With the group scan, a zero-length sequence keeps its state bit for
    bit (empty groups compose exactly) and a checkpoint at a sequence's end
    equals its final state bit for bit (the group holding the last chunk
    writes the final state), also when later groups are empty."""
    lengths = [300, 0, 64, 130]
    b = inputs.make_chunk(lengths, 1, 2, dtype=torch.bfloat16, g_scale=0.5, seed=88, init=True)
    say("scan exactness", groups)
    offsets = [0, 0, 64, 128]
    ck, refs, out, fin = run_checkpoints(b, offsets, rows=4, groups=groups)
    fin = fin.cpu()
    assert torch.equal(fin[1], b.initial_state[1])
    assert np.array_equal(ck[2], fin[2].numpy())
    o_ref, s_ref = oracle_dense(b)
    assert rel(out.float().cpu().numpy(), o_ref, b.cu_seqlens) < 1e-2
    assert rel(fin.numpy(), s_ref) < 1e-2
    assert rel(ck[3], refs[3]) < 1e-2


# ------------------------------------------------------------- chunk table

def chunk_class(nc):
    """Quarter-octave class of a chunk count: 0 for none, else
    4 floor(log2 nc) + the two bits after the leading one, plus 1 (capped
    at 63); the walks start sequences in decreasing class."""
    if nc <= 0:
        return 0
    e = nc.bit_length() - 1
    f = (nc >> (e - 2)) & 3 if e >= 2 else (nc << (2 - e)) & 3
    return min(63, 4 * e + f + 1)


def test_chunk_class_orders_counts():
    assert [chunk_class(n) for n in (0, 1, 2, 3, 4, 5, 6, 7, 8)] == [0, 1, 5, 7, 9, 10, 11, 12, 13]
    cls = [chunk_class(n) for n in range(1, 5000)]
    assert all(a <= b for a, b in zip(cls, cls[1:]))


@pytest.mark.parametrize("n_seqs,max_len,init", [(2000, 200, True), (9000, 3, False)])
def test_chunk_table_for_many_sequences(n_seqs, max_len, init):
    """Thousands of sequences (some empty): the chunk offsets are the prefix
    sums of ceil(length / 64), and the outputs and final states match the
    oracle.  9000 sequences exceed the chunk-table kernel's LDS offset cache
    (8192) and take its per-thread path."""
    gen = torch.Generator().manual_seed(n_seqs)
    lengths = torch.randint(0, max_len + 1, (n_seqs,), generator=gen).tolist()
    b = inputs.make_chunk(lengths, 1, 1, dtype=torch.bfloat16, g_scale=0.5, seed=n_seqs,
                          init=init)
    say("chunk table", n_seqs)
    st = B.chunk_stages(*gpu(b), cu_seqlens=b.cu_seqlens.to(DEV), scale=b.scale,
                        initial_state=None if b.initial_state is None else
                        b.initial_state.to(DEV), path=B.PATH_FUSED)
    torch.cuda.synchronize()
    counts = torch.tensor([(L + 63) // 64 for L in lengths])
    want = torch.cat([torch.zeros(1, dtype=torch.long), counts.cumsum(0)])
    assert torch.equal(st["chunk_offsets"].cpu().long(), want)
    # the walk order: every sequence once, chunk counts non-increasing by
    # quarter-octave class; and the longest count
    order = st["order"].cpu().long()
    assert sorted(order.tolist()) == list(range(n_seqs))
    cls = [chunk_class(int(counts[n])) for n in order.tolist()]
    assert all(a >= b for a, b in zip(cls, cls[1:]))
    assert int(st["nch_max"].cpu()[0]) == int(counts.max())
    o_ref, s_ref = oracle_dense(b)
    assert rel(st["out"].float().cpu().numpy(), o_ref, b.cu_seqlens) < 1e-2
    assert rel(st["final_state"].cpu().numpy(), s_ref) < 1e-2


# ------------------------------------------------ seeded mixed configurations

def _mixed_case(i):
    """Configuration i of a fixed seeded draw: sequence lengths (some empty,
    ragged tails), GVA ratio, dtype, gate parameters, dense or paged state,
    projection-view inputs, and an explicit or planned walk shape."""
    gen = torch.Generator().manual_seed(1000 + i)
    r = lambda n: int(torch.randint(0, n, (1,), generator=gen))
    n_seqs = 1 + r(5)
    lengths = [r(4) * 64 + r(65) if r(5) else 0 for _ in range(n_seqs)]
    if sum(lengths) == 0:
        lengths[0] = 70
    hqk = [1, 2][r(2)]
    hv = hqk * [1, 2, 4][r(3)]
    dtype = [torch.bfloat16, torch.bfloat16, torch.float32][r(3)]
    return dict(lengths=lengths, hqk=hqk, hv=hv, dtype=dtype, gate=bool(r(2)), paged=bool(r(2)),
                strided=bool(r(2)) and dtype == torch.bfloat16, groups=[0, 1, 2, 3][r(4)],
                waves=[0, 2, 4, 8][r(4)], seed=2000 + i)


@pytest.mark.parametrize("i", range(24))
def test_mixed_configurations_match_oracle(i):
    cfg = _mixed_case(i)
    say("mixed", i, cfg)
    b = inputs.make_chunk(cfg["lengths"], cfg["hqk"], cfg["hv"], dtype=cfg["dtype"], g_scale=0.5,
                          seed=cfg["seed"], init=not cfg["paged"],
                          paged_slots=len(cfg["lengths"]) + 3 if cfg["paged"] else 0)
    hv = cfg["hv"]
    gk = {}
    if cfg["gate"]:
        gg = torch.Generator().manual_seed(cfg["seed"])
        gk = dict(A_log=torch.randn(hv, generator=gg) * 0.3,
                  dt_bias=torch.randn(hv, 128, generator=gg) * 0.5)
    if cfg["strided"]:
        (q, k, v, g, beta), _ = projection_views([b.q, b.k, b.v, b.g, b.beta], DEV)
    else:
        q, k, v, g, beta = gpu(b)
    kw = dict(scale=b.scale, cu_seqlens=b.cu_seqlens.to(DEV), groups=cfg["groups"],
              walk_waves=cfg["waves"], **{k_: v_.to(DEV) for k_, v_ in gk.items()})
    if cfg["paged"]:
        cache = b.state_cache.to(DEV)
        out = chunk_kda(q, k, v, g, beta, state_cache=cache,
                          state_indices=b.state_indices.to(DEV),
                          has_initial_state=b.has_initial_state.to(DEV), **kw)
        s0 = b.state_cache[b.state_indices.long()] * b.has_initial_state.view(-1, 1, 1, 1).float()
    else:
        out, fin = chunk_kda(q, k, v, g, beta, initial_state=b.initial_state.to(DEV),
                               output_final_state=True, **kw)
        s0 = b.initial_state
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                     scale=b.scale, initial_state=s0,
                                     **{k_: v_.double() for k_, v_ in gk.items()})
    t_ = tol(cfg["dtype"])
    assert rel(out.float().cpu().numpy(), o_ref, b.cu_seqlens) < t_
    got = cache.cpu()[b.state_indices.long()] if cfg["paged"] else fin.cpu()
    assert rel(got.numpy(), s_ref) < t_


# ------------------------------------------------ fp16 inputs, bf16 paged pool

FP16_CASES = [
    # (name, lengths, hqk, hv, g_scale, groups)
    ("ragged", [1, 63, 64, 65, 200, 7], 1, 2, 5.0, 0),
    ("gva", [130, 77], 2, 8, 5.0, 0),
    ("weak_decay_scan", [3000], 1, 2, 0.01, 4),
]


@pytest.mark.parametrize("case", FP16_CASES, ids=[c[0] for c in FP16_CASES])
def test_fp16_inputs(case):
    """fp16 inputs run on the fp32 kernels (widened exactly, split MFMA
    operands): outputs are stored in fp16 (the 1e-2 bar of 16-bit outputs), the
    fp32 final states keep the fp32 bar (1e-4)."""
    name, lengths, hqk, hv, gs, groups = case
    b = inputs.make_chunk(lengths, hqk, hv, dtype=torch.float16, g_scale=gs, seed=130,
                          init=True)
    say("fp16", name)
    q, k, v, g, beta = gpu(b)
    out, fin = chunk_kda(q, k, v, g, beta, scale=b.scale, initial_state=b.initial_state.to(DEV),
                         output_final_state=True, cu_seqlens=b.cu_seqlens.to(DEV),
                         groups=groups)
    torch.cuda.synchronize()
    assert out.dtype == torch.float16 and fin.dtype == torch.float32
    o_ref, s_ref = oracle_dense(b)
    cu = b.cu_seqlens.numpy()
    assert report("out", out.float().cpu().numpy(), o_ref, cu) < 1e-2
    assert report("state", fin.cpu().numpy(), s_ref) < 1e-4
    assert report("first 64", first_rows(out.float().cpu().numpy(), cu),
                  first_rows(o_ref, cu), first_cu(cu)) < 1e-2


def test_fp16_paged_pool_with_gate_parameters():
    lengths = [90, 0, 64, 131]
    hv = 4
    b = inputs.make_chunk(lengths, 2, hv, dtype=torch.float16, seed=131, paged_slots=9)
    b.has_initial_state = torch.tensor([1, 1, 0, 1], dtype=torch.uint8)
    gen = torch.Generator().manual_seed(132)
    b.g = torch.randn(b.g.shape, generator=gen).to(torch.float16)  # raw gate ~ N(0, 1)
    a_log = (torch.rand(hv, generator=gen) * 2 - 1).float()
    dt_bias = torch.randn(hv, 128, generator=gen).float()
    say("fp16 paged gate")
    q, k, v, g, beta = gpu(b)
    cache = b.state_cache.to(DEV)
    out = chunk_kda(q, k, v, g, beta, scale=b.scale, cu_seqlens=b.cu_seqlens.to(DEV),
                    state_cache=cache, state_indices=b.state_indices.to(DEV),
                    has_initial_state=b.has_initial_state.to(DEV), A_log=a_log.to(DEV),
                    dt_bias=dt_bias.to(DEV))
    torch.cuda.synchronize()
    idx = b.state_indices.long()
    s0 = b.state_cache[idx].clone()
    s0[2] = 0.0
    o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                     scale=b.scale, initial_state=s0, A_log=a_log,
                                     dt_bias=dt_bias)
    assert report("out", out.float().cpu().numpy(), o_ref, b.cu_seqlens.numpy()) < 1e-2
    got = cache.cpu()
    assert report("state", got[idx].numpy(), s_ref) < 1e-4
    others = torch.ones(9, dtype=torch.bool)
    others[idx] = False
    assert torch.equal(got[others], b.state_cache[others])


@pytest.mark.parametrize("groups", [1, 4])
def test_bf16_paged_pool(groups):
    """A bf16 state pool (chunk_kda's states may take q's dtype): each row is
    widened exactly as the start state and the final state is rounded to
    nearest even; a zero-length sequence passes its row through bit for bit,
    rows of other slots are untouched."""
    lengths = [900, 0, 64, 1300]
    b = inputs.make_chunk(lengths, 2, 4, dtype=torch.bfloat16, g_scale=0.5, seed=133,
                          paged_slots=9)
    b.has_initial_state = torch.tensor([1, 1, 0, 1], dtype=torch.uint8)
    pool = (b.state_cache * 25.0).to(torch.bfloat16)
    say("bf16 pool", groups)
    q, k, v, g, beta = gpu(b)
    cache = pool.to(DEV)
    out = chunk_kda(q, k, v, g, beta, scale=b.scale, cu_seqlens=b.cu_seqlens.to(DEV),
                    state_cache=cache, state_indices=b.state_indices.to(DEV),
                    has_initial_state=b.has_initial_state.to(DEV), groups=groups)
    torch.cuda.synchronize()
    idx = b.state_indices.long()
    s0 = pool[idx].float()
    s0[2] = 0.0
    o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                     scale=b.scale, initial_state=s0)
    assert report("out", out.float().cpu().numpy(), o_ref, b.cu_seqlens.numpy()) < 1e-2
    got = cache.cpu()
    assert got.dtype == torch.bfloat16
    live = [0, 2, 3]
    assert report("state", got[idx[live]].float().numpy(),
                  oracle.round_bf16(s_ref[live])) < 1e-2
    assert torch.equal(got[idx[1]], pool[idx[1]])
    others = torch.ones(9, dtype=torch.bool)
    others[idx] = False
    assert torch.equal(got[others], pool[others])


# ------------------------------------------- randomised stress (opt-in)

def _stress_case(i):
    """Case i of a wider seeded family than the mixed configurations: up to
    120 sequences with log-uniform lengths up to 3000 tokens (some empty), GVA
    1 / 2 / 4, bf16 / fp16 / fp32, gate parameters, paged pools, G up to 16,
    every walk width and path."""
    gen = torch.Generator().manual_seed(190000 + i)
    r = lambda n: int(torch.randint(0, n, (1,), generator=gen))
    n_seqs = 1 + r([40, 120][r(2)])
    lengths = [0 if r(8) == 0 else int(np.exp(np.log(3000) * float(torch.rand(1, generator=gen))))
               for _ in range(n_seqs)]
    if sum(lengths) == 0:
        lengths[0] = 100
    hqk = [1, 2, 4][r(3)]
    hv = hqk * [1, 2, 4][r(3)]
    dtype = [torch.bfloat16, torch.bfloat16, torch.float32, torch.float16][r(4)]
    paths = [B.PATH_AUTO, B.PATH_STAGED] + ([B.PATH_ONCHIP] if dtype == torch.bfloat16 else [])
    return dict(lengths=lengths, hqk=hqk, hv=hv, dtype=dtype, gate=r(3) == 0, paged=bool(r(2)),
                groups=[0, 0, 1, 2, 3, 5, 8, 16][r(8)], waves=[0, 0, 2, 4, 8][r(5)],
                path=paths[r(len(paths))], seed=195000 + i)


@pytest.mark.parametrize("i", stress.cases())
def test_random_configurations_match_oracle(i):
    """Opt-in (KDA_STRESS=<cases>): outputs and final states of seeded random
    configurations against the oracle at the usual bars, per unit."""
    cfg = _stress_case(i)
    say("stress", i, {k: v for k, v in cfg.items() if k != "lengths"}, len(cfg["lengths"]))
    b = inputs.make_chunk(cfg["lengths"], cfg["hqk"], cfg["hv"], dtype=cfg["dtype"], g_scale=0.5,
                          seed=cfg["seed"], init=not cfg["paged"],
                          paged_slots=len(cfg["lengths"]) + 3 if cfg["paged"] else 0)
    hv = cfg["hv"]
    gk = {}
    if cfg["gate"]:
        gg = torch.Generator().manual_seed(cfg["seed"])
        gk = dict(A_log=torch.randn(hv, generator=gg) * 0.3,
                  dt_bias=torch.randn(hv, 128, generator=gg) * 0.5)
    q, k, v, g, beta = gpu(b)
    kw = dict(scale=b.scale, cu_seqlens=b.cu_seqlens.to(DEV), groups=cfg["groups"],
              walk_waves=cfg["waves"], path=cfg["path"],
              **{k_: v_.to(DEV) for k_, v_ in gk.items()})
    if cfg["paged"]:
        cache = b.state_cache.to(DEV)
        out = B.chunk_kda(q, k, v, g, beta, state_cache=cache,
                          state_indices=b.state_indices.to(DEV),
                          has_initial_state=b.has_initial_state.to(DEV), **kw)
        s0 = b.state_cache[b.state_indices.long()] * b.has_initial_state.view(-1, 1, 1, 1).float()
    else:
        out, fin = B.chunk_kda(q, k, v, g, beta, initial_state=b.initial_state.to(DEV),
                               output_final_state=True, **kw)
        s0 = b.initial_state
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                     scale=b.scale, initial_state=s0,
                                     **{k_: v_.double() for k_, v_ in gk.items()})
    t_ = tol(cfg["dtype"])
    assert rel(out.float().cpu().numpy(), o_ref, b.cu_seqlens) < t_
    got = cache.cpu()[b.state_indices.long()] if cfg["paged"] else fin.cpu()
    assert rel(got.float().numpy(), s_ref) < t_
