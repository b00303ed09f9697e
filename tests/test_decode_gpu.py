"""Decode (T = 1, paged V-first fp32 state, in place) against the fp64 oracle.

Tolerance: relative L2 <= 1e-2 for bf16/fp16 inputs (bf16 output rounding alone
is ~2e-3) and <= 1e-4 for fp32 inputs; the state is fp32 throughout, so the
updated cache rows are held to 1e-5 (the only error is fp32 arithmetic).  Each
bar holds over the whole tensor and for the worst unit: every (request, token,
head) output row, every state plane (tests/parity.py).
"""
import numpy as np
import pytest
import torch

import oracle
import parity
import stress
from gated_delta_rule_65_amd import binding as B
from gated_delta_rule_65_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def rel(a, b):
    """max(whole-tensor rel-L2, worst unit): units are the state planes of a
    cache, and each (request, token, head) row of an output."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.ndim >= 3 and a.shape[-2:] == (128, 128):
        return parity.rel(a, b)
    if a.ndim >= 3:
        a = a.reshape(-1, a.shape[-2], a.shape[-1])
        b = b.reshape(-1, b.shape[-2], b.shape[-1])
        return parity.rel(a, b, np.arange(a.shape[0] + 1))
    return parity.rel(a, b)


def run_case(batch, l2=True, scale=None, null=()):
    idx = batch.state_indices.clone()
    for i in null:
        idx[i] = -1
    cache_dev = batch.state_cache.to(DEV)
    before = batch.state_cache  # CPU copy, untouched
    args = [t.to(DEV) for t in (batch.q, batch.k, batch.v, batch.g, batch.beta)]
    print(f"decode n={batch.q.shape[0]} hqk={batch.q.shape[1]} hv={batch.v.shape[1]} "
          f"dtype={batch.q.dtype} null={list(null)}", flush=True)
    out = B.kda_decode(*args, cache_dev, idx.to(DEV), scale=scale, use_qk_l2norm=l2)
    torch.cuda.synchronize()
    live = torch.nonzero(idx >= 0).flatten()
    ref_out = np.zeros(out.shape)
    if live.numel():
        s0 = before[idx[live].long()]
        o, sf = oracle.recurrence(batch.q[live], batch.k[live], batch.v[live], batch.g[live],
                                  batch.beta[live],
                                  cu_seqlens=np.arange(live.numel() + 1), scale=scale,
                                  use_qk_l2norm=l2, initial_state=s0)
        ref_out[live.numpy()] = o
    else:
        sf = None
    return out.float().cpu().numpy(), ref_out, cache_dev, before, idx, live, sf


def test_decode_full_workload():
    """256 requests x 32 heads, cache [1024, 32, 128, 128], distinct random slots."""
    b = inputs.make_workload("decode_paged")
    out, ref, cache, before, idx, live, sf = run_case(b)
    assert rel(out, ref) < 1e-2
    rows = idx[live].long()
    got = cache[rows.to(DEV)].cpu().numpy()
    assert rel(got, sf) < 1e-5
    mask = torch.ones(cache.shape[0], dtype=torch.bool)
    mask[rows] = False
    assert torch.equal(cache[mask.to(DEV)].cpu(), before[mask])


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16])
@pytest.mark.parametrize("hqk,hv", [(1, 1), (2, 8), (4, 4)])
def test_decode_dtypes_and_gva(dtype, hqk, hv):
    b = inputs.make_decode(37, hqk, hv, 50, dtype=dtype, seed=3)
    out, ref, cache, before, idx, live, sf = run_case(b, null=(3, 17))
    tol = 1e-4 if dtype == torch.float32 else 1e-2
    assert rel(out, ref) < tol
    assert np.all(out[[3, 17]] == 0.0)
    got = cache[idx[live].long().to(DEV)].cpu().numpy()
    assert rel(got, sf) < 1e-5


def test_decode_no_l2norm_custom_scale_identity_slots():
    b = inputs.make_decode(16, 2, 4, 16, dtype=torch.float32, seed=5)
    b.state_indices = torch.arange(16, dtype=torch.int32)
    out, ref, cache, *_ = run_case(b, l2=False, scale=0.37)
    assert rel(out, ref) < 1e-4
    # the same call with no index array (identity map) gives the same result
    c2 = b.state_cache.to(DEV)
    args = [t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)]
    out2 = B.kda_decode(*args, c2, None, scale=0.37, use_qk_l2norm=False)
    assert torch.equal(out2.cpu(), torch.from_numpy(out).to(out2.dtype))
    assert torch.equal(c2, cache)


def test_decode_all_null_slots_touch_nothing():
    b = inputs.make_decode(8, 1, 2, 8, seed=6)
    out, ref, cache, before, *_ = run_case(b, null=tuple(range(8)))
    assert np.all(out == 0.0)
    assert torch.equal(cache.cpu(), before)


def test_decode_repeated_equals_multi_token_recurrence():
    """Repeated single-token decode equals the T-token recurrence."""
    T, hqk, hv = 12, 2, 4
    bb = inputs.make_chunk([T], hqk, hv, dtype=torch.float32, seed=9, init=True)
    cache = torch.zeros(5, hv, 128, 128)
    cache[3] = bb.initial_state[0]
    c_dev = cache.to(DEV)
    idx = torch.tensor([3], dtype=torch.int32, device=DEV)
    outs = []
    for t in range(T):
        sl = slice(t, t + 1)
        o = B.kda_decode(bb.q[sl].to(DEV), bb.k[sl].to(DEV), bb.v[sl].to(DEV),
                         bb.g[sl].to(DEV), bb.beta[sl].to(DEV), c_dev, idx)
        outs.append(o[0].cpu())
    o_ref, s_ref = oracle.recurrence(bb.q, bb.k, bb.v, bb.g, bb.beta,
                                     initial_state=bb.initial_state)
    assert rel(torch.stack(outs).numpy(), o_ref) < 1e-4
    assert rel(c_dev[3].cpu().numpy(), s_ref[0]) < 1e-5


def test_decode_is_deterministic():
    b = inputs.make_decode(64, 4, 8, 80, seed=11)
    args = [t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)]
    c1, c2 = b.state_cache.to(DEV), b.state_cache.to(DEV)
    idx = b.state_indices.to(DEV)
    o1 = B.kda_decode(*args, c1, idx)
    o2 = B.kda_decode(*args, c2, idx)
    assert torch.equal(o1, o2) and torch.equal(c1, c2)


@pytest.mark.parametrize("dtype,bias_dtype", [(torch.bfloat16, torch.float32),
                                              (torch.bfloat16, torch.bfloat16),
                                              (torch.float32, torch.float32)])
def test_decode_gate_parameters(dtype, bias_dtype):
    """g as a raw gate with A_log / dt_bias / lower_bound, against the oracle
    with the same stored parameters."""
    b = inputs.make_decode(40, 2, 4, 64, dtype=dtype, seed=11)
    gen = torch.Generator().manual_seed(12)
    b.g = torch.randn(b.g.shape, generator=gen).to(dtype)
    a_log = (torch.rand(4, generator=gen) * 2 - 1).float()
    dt_bias = (torch.randn(4, 128, generator=gen) * 0.5).to(bias_dtype)
    idx = b.state_indices.clone()
    idx[5] = -1
    cache = b.state_cache.to(DEV)
    args = [t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)]
    print("decode gate", dtype, bias_dtype, flush=True)
    out = B.kda_decode(*args, cache, idx.to(DEV), A_log=a_log.to(DEV),
                       dt_bias=dt_bias.to(DEV), lower_bound=-4.0)
    torch.cuda.synchronize()
    ref_out, ref_cache = oracle.decode(b.q, b.k, b.v, b.g, b.beta, b.state_cache, idx,
                                       A_log=a_log.double(), dt_bias=dt_bias.double(),
                                       lower_bound=-4.0)
    tol = 1e-4 if dtype == torch.float32 else 1e-2
    assert rel(out.float().cpu().numpy(), ref_out) < tol
    live = idx >= 0
    rows = idx[live].long()
    assert rel(cache.cpu()[rows].numpy(), ref_cache[rows.numpy()]) < 1e-5
    assert np.all(out[5].float().cpu().numpy() == 0.0)


# ------------------------------------------------- multi-token (spec) decode

def spec_case(B, T, hqk, hv, slots, dtype, seed):
    d = inputs.make_decode(B * T, hqk, hv, slots, dtype=dtype, seed=seed)
    rs = lambda x: x.reshape(B, T, *x.shape[1:]).contiguous()
    return rs(d.q), rs(d.k), rs(d.v), rs(d.g), rs(d.beta), d.state_cache


def run_spec(q, k, v, g, beta, cache, idx, acc=None, **gate):
    cd = cache.to(DEV)
    out = B.kda_decode(*(t.to(DEV) for t in (q, k, v, g, beta)), cd, idx.to(DEV),
                       num_accepted_tokens=None if acc is None else acc.to(DEV), **gate)
    torch.cuda.synchronize()
    og = {k_: (v_.double() if isinstance(v_, torch.Tensor) else v_) for k_, v_ in gate.items()}
    for k_ in ("A_log", "dt_bias"):
        if k_ in og:
            og[k_] = og[k_].cpu()
    ro, rc = oracle.decode_multi(q, k, v, g, beta, cache, idx, acc, **og)
    return out.float().cpu().numpy(), ro, cd.cpu().numpy(), rc


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
@pytest.mark.parametrize("T,hqk,hv", [(4, 1, 2), (8, 2, 4), (3, 4, 4)])
def test_multi_token_decode_matches_oracle(dtype, T, hqk, hv):
    Bn = 7
    q, k, v, g, beta, cache = spec_case(Bn, T, hqk, hv, 70, dtype, seed=20 + T)
    idx = torch.arange(Bn * T, dtype=torch.int32).reshape(Bn, T)
    idx[2, 1] = -1                      # no store after that token
    idx[4, 0] = -1                      # null start: skipped request
    print("spec decode", dtype, T, hqk, hv, flush=True)
    o, ro, c, rc = run_spec(q, k, v, g, beta, cache, idx)
    tol = 1e-4 if dtype == torch.float32 else 1e-2
    assert rel(o, ro) < tol
    assert np.all(o[4] == 0)
    assert rel(c, rc) < 1e-5


def test_multi_token_decode_accepted_counts():
    Bn, T = 6, 4
    q, k, v, g, beta, cache = spec_case(Bn, T, 1, 2, 40, torch.bfloat16, seed=41)
    idx = torch.arange(Bn * T, dtype=torch.int32).reshape(Bn, T)
    acc = torch.tensor([1, 2, 3, 4, 0, 5], dtype=torch.int32)   # 0 and 5: skipped
    o, ro, c, rc = run_spec(q, k, v, g, beta, cache, idx, acc)
    assert rel(o, ro) < 1e-2
    assert np.all(o[4] == 0) and np.all(o[5] == 0)
    assert rel(c, rc) < 1e-5


def test_multi_token_decode_single_column_equals_single_token():
    q, k, v, g, beta, cache = spec_case(9, 1, 2, 4, 20, torch.bfloat16, seed=42)
    idx = torch.randperm(20)[:9].to(torch.int32)
    c1, c2 = cache.to(DEV), cache.to(DEV)
    o1 = B.kda_decode(*(t[:, 0].to(DEV) for t in (q, k, v, g, beta)), c1, idx.to(DEV))
    o2 = B.kda_decode(*(t.to(DEV) for t in (q, k, v, g, beta)), c2, idx[:, None].to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1.cpu(), o2[:, 0].cpu()) and torch.equal(c1.cpu(), c2.cpu())


def test_multi_token_decode_with_gate():
    Bn, T = 5, 6
    q, k, v, g, beta, cache = spec_case(Bn, T, 1, 2, 40, torch.bfloat16, seed=43)
    gen = torch.Generator().manual_seed(44)
    g = torch.randn(g.shape, generator=gen).to(torch.bfloat16)
    idx = torch.arange(Bn * T, dtype=torch.int32).reshape(Bn, T)
    gate = dict(A_log=(torch.rand(2, generator=gen) - 0.5).to(DEV),
                dt_bias=torch.randn(2, 128, generator=gen).to(DEV), lower_bound=-3.0)
    o, ro, c, rc = run_spec(q, k, v, g, beta, cache, idx, **gate)
    assert rel(o, ro) < 1e-2 and rel(c, rc) < 1e-5


# ------------------------------------------------------------ bf16 state cache

def test_decode_bf16_state_cache():
    """bf16 cache: widened for the token's arithmetic, stored rounded to
    nearest even; against the oracle on the same stored values."""
    b = inputs.make_decode(60, 2, 4, 80, dtype=torch.bfloat16, seed=61)
    cache = b.state_cache.to(torch.bfloat16)
    idx = b.state_indices.clone()
    idx[7] = -1
    cd = cache.to(DEV)
    out = B.kda_decode(*(t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)), cd, idx.to(DEV))
    torch.cuda.synchronize()
    ro, rc = oracle.decode(b.q, b.k, b.v, b.g, b.beta, cache, idx)
    assert rel(out.float().cpu().numpy(), ro) < 1e-2
    live = idx[idx >= 0].long()
    got = cd.cpu().float().numpy()[live.numpy()]
    want = oracle.round_bf16(rc[live.numpy()])
    assert rel(got, want) < 1e-2
    # most elements round to the same bf16 value as the fp64 state
    assert np.mean(got == want) > 0.9
    untouched = torch.ones(80, dtype=torch.bool)
    untouched[live] = False
    assert torch.equal(cd.cpu()[untouched], cache[untouched])


def test_multi_token_decode_bf16_state_cache():
    Bn, T = 6, 5
    q, k, v, g, beta, cache = spec_case(Bn, T, 1, 2, 40, torch.bfloat16, seed=62)
    cache = cache.to(torch.bfloat16)
    idx = torch.arange(Bn * T, dtype=torch.int32).reshape(Bn, T)
    acc = torch.tensor([1, 1, 2, 3, 5, 4], dtype=torch.int32)
    cd = cache.to(DEV)
    out = B.kda_decode(*(t.to(DEV) for t in (q, k, v, g, beta)), cd, idx.to(DEV),
                       num_accepted_tokens=acc.to(DEV))
    torch.cuda.synchronize()
    ro, rc = oracle.decode_multi(q, k, v, g, beta, cache, idx, acc, state_bf16=True)
    assert rel(out.float().cpu().numpy(), ro) < 1e-2
    assert rel(cd.cpu().float().numpy(), rc) < 1e-2


# ------------------------------------------------- strided (projection) inputs

def projection_views(tensors, pad=8):
    """Tensors copied into bands of one [tokens, W] buffer (NaN between
    bands), returned as views with a per-token stride of W elements."""
    n = tensors[0].shape[0] * (tensors[0].shape[1] if tensors[0].dim() == 4 else 1)
    flat = [t.reshape(n, -1) for t in tensors]
    W = sum(f.shape[1] for f in flat) + pad
    W += (-W) % 8
    proj = torch.full((n, W), float("nan"), dtype=tensors[0].dtype, device=DEV)
    views, off = [], 0
    for t, f in zip(tensors, flat):
        proj[:, off:off + f.shape[1]] = f.to(DEV)
        views.append(proj[:, off:off + f.shape[1]].view(t.shape))
        off += f.shape[1]
    return views


def padded_pool(cache, pad=64):
    """The cache as a pool whose slots are padded by `pad` elements (NaN)."""
    slots, plane = cache.shape[0], cache[0].numel()
    pool = torch.full((slots, plane + pad), float("nan"), dtype=cache.dtype, device=DEV)
    view = pool[:, :plane].view(cache.shape)
    view.copy_(cache.to(DEV))
    return pool, view


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_decode_strided_inputs_and_padded_pool(dtype):
    b = inputs.make_decode(40, 2, 4, 64, dtype=dtype, seed=63)
    idx = b.state_indices.clone()
    idx[3] = -1
    views = projection_views([b.q, b.k, b.v, b.g, b.beta])
    assert not views[0].is_contiguous()
    pool, cache_s = padded_pool(b.state_cache)
    cache_c = b.state_cache.to(DEV)
    out_s = B.kda_decode(*views, cache_s, idx.to(DEV))
    out_c = B.kda_decode(*(t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)), cache_c,
                         idx.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_c) and torch.equal(cache_s, cache_c)
    assert torch.isnan(pool[:, 4 * 128 * 128:]).all()
    ro, rc = oracle.decode(b.q, b.k, b.v, b.g, b.beta, b.state_cache, idx)
    assert rel(out_s.float().cpu().numpy(), ro) < (1e-4 if dtype == torch.float32 else 1e-2)


def test_multi_token_decode_strided_inputs_bf16_padded_pool():
    Bn, T = 5, 4
    q, k, v, g, beta, cache = spec_case(Bn, T, 1, 2, 30, torch.bfloat16, seed=64)
    cache = cache.to(torch.bfloat16)
    idx = torch.arange(Bn * T, dtype=torch.int32).reshape(Bn, T)
    acc = torch.tensor([1, 2, 4, 3, 1], dtype=torch.int32)
    views = projection_views([q, k, v, g, beta])
    pool, cache_s = padded_pool(cache)
    cache_c = cache.to(DEV)
    out_s = B.kda_decode(*views, cache_s, idx.to(DEV), num_accepted_tokens=acc.to(DEV))
    out_c = B.kda_decode(*(t.to(DEV) for t in (q, k, v, g, beta)), cache_c, idx.to(DEV),
                         num_accepted_tokens=acc.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(out_s, out_c) and torch.equal(cache_s, cache_c)
    assert torch.isnan(pool[:, 2 * 128 * 128:].float()).all()
    ro, rc = oracle.decode_multi(q, k, v, g, beta, cache, idx, acc, state_bf16=True)
    assert rel(out_s.float().cpu().numpy(), ro) < 1e-2


# ------------------------------------------------ seeded mixed configurations

@pytest.mark.parametrize("i", range(10))
def test_mixed_decode_configurations_match_oracle(i):
    """Configuration i of a fixed seeded draw: request count, tokens per
    request (1..8), GVA ratio, input dtype, fp32 or bf16 pool, gate
    parameters, projection-view inputs, accepted-token counts."""
    gen = torch.Generator().manual_seed(3000 + i)
    r = lambda n: int(torch.randint(0, n, (1,), generator=gen))
    Bn, T = 1 + r(9), 1 + r(8)
    hqk = [1, 2][r(2)]
    hv = hqk * [1, 2, 4][r(3)]
    dtype = [torch.bfloat16, torch.float16, torch.float32][r(3)]
    state_bf16 = bool(r(2))
    print("mixed decode", i, Bn, T, hqk, hv, dtype, state_bf16, flush=True)
    q, k, v, g, beta, cache = spec_case(Bn, T, hqk, hv, Bn * T + 4, dtype, seed=4000 + i)
    if state_bf16:
        cache = cache.to(torch.bfloat16)
    idx = torch.randperm(Bn * T + 4, generator=gen)[:Bn * T].to(torch.int32).reshape(Bn, T)
    idx[0, T - 1] = -1                                   # one skipped store
    acc = torch.randint(1, T + 1, (Bn,), generator=gen).to(torch.int32)
    gk = {}
    if r(2):
        gk = dict(A_log=torch.randn(hv, generator=gen) * 0.3,
                  dt_bias=torch.randn(hv, 128, generator=gen) * 0.5)
    views = projection_views([q, k, v, g, beta]) if r(2) and dtype != torch.float32 else \
        [t.to(DEV) for t in (q, k, v, g, beta)]
    cd = cache.to(DEV)
    out = B.kda_decode(*views, cd, idx.to(DEV), num_accepted_tokens=acc.to(DEV),
                       **{k_: v_.to(DEV) for k_, v_ in gk.items()})
    torch.cuda.synchronize()
    ro, rc = oracle.decode_multi(q, k, v, g, beta, cache, idx, acc, state_bf16=state_bf16,
                                 **{k_: v_.double() for k_, v_ in gk.items()})
    t_ = 1e-4 if dtype == torch.float32 and not state_bf16 else 1e-2
    assert rel(out.float().cpu().numpy(), ro) < t_
    assert rel(cd.cpu().float().numpy(), rc) < t_


@pytest.mark.parametrize("i", stress.cases())
def test_random_decode_configurations_match_oracle(i):
    """Opt-in (KDA_STRESS=<cases>): seeded random single-token ([N, H, 128])
    and multi-token ([B, T, H, 128]) decodes over request counts up to 64,
    GVA, input dtypes, fp32 or bf16 pools, null slots, accepted-token counts
    and gate parameters, against the oracle."""
    gen = torch.Generator().manual_seed(310000 + i)
    r = lambda n: int(torch.randint(0, n, (1,), generator=gen))
    Bn, T = 1 + r(64), 1 + r(8)
    single = T == 1 and bool(r(2))
    hqk = [1, 2, 4, 8][r(4)]
    hv = min(16, hqk * [1, 2, 4][r(3)])
    dtype = [torch.bfloat16, torch.float16, torch.float32][r(3)]
    state_bf16 = bool(r(2))
    slots = Bn * T + r(32)
    print("random decode", i, Bn, T, single, hqk, hv, dtype, state_bf16, flush=True)
    q, k, v, g, beta, cache = spec_case(Bn, T, hqk, hv, slots, dtype, seed=320000 + i)
    if state_bf16:
        cache = cache.to(torch.bfloat16)
    idx = torch.randperm(slots, generator=gen)[:Bn * T].to(torch.int32).reshape(Bn, T)
    for b_ in range(Bn):
        if r(8) == 0:
            idx[b_, r(T)] = -1
    acc = None if single or r(3) == 0 else \
        torch.randint(1, T + 1, (Bn,), generator=gen).to(torch.int32)
    gk = {}
    if r(3) == 0:
        gk = dict(A_log=torch.randn(hv, generator=gen) * 0.3,
                  dt_bias=torch.randn(hv, 128, generator=gen) * 0.5,
                  lower_bound=-float(1 + r(5)))
    cd = cache.to(DEV)
    dev = {k_: (v_.to(DEV) if isinstance(v_, torch.Tensor) else v_) for k_, v_ in gk.items()}
    ref = {k_: (v_.double() if isinstance(v_, torch.Tensor) else v_) for k_, v_ in gk.items()}
    if single:
        flat = [t[:, 0].contiguous() for t in (q, k, v, g, beta)]
        out = B.kda_decode(*(t.to(DEV) for t in flat), cd, idx[:, 0].contiguous().to(DEV),
                           **dev)
        torch.cuda.synchronize()
        ro, rc = oracle.decode_multi(q, k, v, g, beta, cache, idx, None,
                                     state_bf16=state_bf16, **ref)
        ro = ro[:, 0]
    else:
        out = B.kda_decode(*(t.to(DEV) for t in (q, k, v, g, beta)), cd, idx.to(DEV),
                           num_accepted_tokens=None if acc is None else acc.to(DEV), **dev)
        torch.cuda.synchronize()
        ro, rc = oracle.decode_multi(q, k, v, g, beta, cache, idx, acc,
                                     state_bf16=state_bf16, **ref)
    t_ = 1e-4 if dtype == torch.float32 and not state_bf16 else 1e-2
    assert rel(out.float().cpu().numpy(), ro) < t_
    assert rel(cd.cpu().float().numpy(), rc) < t_
