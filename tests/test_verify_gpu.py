"""Record-based verify window and commit on the GPU against the fp64 oracle.

Bars (relative L2, over the whole tensor and the worst unit, tests/parity.py).
Both sides read the same stored inputs, so the corrections (fp32) and an fp32
committed state differ from the oracle by fp32 arithmetic alone: 1e-4 for the
corrections, 1e-5 for the state planes, whatever the input dtype.  Outputs
are stored in the input dtype: 1e-2 for bf16 / fp16 (rounding to 8 or 11
significant bits), 1e-4 for fp32.  A bf16 committed state is rounded once on
both sides, so it agrees up to an ulp where the two land on opposite sides
of a rounding boundary: 1e-2.  The kg records are copies of the raw inputs
and are compared bit for bit; record rows and cache slots a call must not
touch are checked unchanged.
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
SENT_CORR, SENT_KG = 7.0, 3.0


def tol_out(dt):
    return 1e-4 if dt == torch.float32 else 1e-2


TOL_CORR = 1e-4


def tol_state(state_dt):
    return 1e-2 if state_dt == torch.bfloat16 else 1e-5


def rel_rows(got, ref):
    """max(whole, worst row) over [units, 128] rows."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, 1, 128)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, 1, 128)
    return parity.rel(got, ref, np.arange(got.shape[0] + 1))


def gate_params(hv, seed):
    gen = torch.Generator().manual_seed(seed)
    al = (torch.rand(hv, generator=gen) * 2 - 1).float()
    db = torch.randn(hv, 128, generator=gen).float()
    return al, db


def run(b, window, state_dt=torch.float32, gate=None, scale=None, l2=True):
    """Verify then commit on the GPU; returns everything the checks need."""
    hv = b.v.shape[1]
    n = b.cu_seqlens.numel() - 1
    print(f"verify n={n} hqk={b.q.shape[1]} hv={hv} window={window} dtype={b.q.dtype} "
          f"state={state_dt} gate={gate is not None}", flush=True)
    cache0 = b.state_cache.to(state_dt)
    cache = cache0.to(DEV)
    al = db = None
    if gate is not None:
        al, db = gate
    dal = None if al is None else al.to(DEV)
    ddb = None if db is None else db.to(DEV)
    args = [t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)]
    corr = torch.full((n, hv, window, 128), SENT_CORR, device=DEV)
    kg = torch.full((n, hv, window, 256), SENT_KG, dtype=b.q.dtype, device=DEV)
    out = torch.full((b.q.shape[0], hv, 128), 5.0, dtype=b.q.dtype, device=DEV)
    B.kda_verify(*args, b.cu_seqlens.to(DEV), cache, b.state_indices.to(DEV), window,
                 scale=scale, use_qk_l2norm=l2, A_log=dal, dt_bias=ddb, output=out,
                 corr=corr, kg=kg)
    torch.cuda.synchronize()
    assert torch.equal(cache.cpu(), cache0), "verify must not write the state"
    acc = b.meta["accepted"]
    B.kda_commit(cache, b.state_indices.to(DEV), acc.to(DEV), corr, kg, use_qk_l2norm=l2,
                 A_log=dal, dt_bias=ddb)
    torch.cuda.synchronize()
    ro, rc, rk = oracle.verify(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, cache0.float(),
                               b.state_indices, window, scale=scale, use_qk_l2norm=l2,
                               A_log=al, dt_bias=db)
    rnew = oracle.commit(cache0.float(), b.state_indices, acc, rc, rk, use_qk_l2norm=l2,
                         A_log=al, dt_bias=db, state_bf16=state_dt == torch.bfloat16)
    return dict(out=out.float().cpu().numpy(), corr=corr.cpu().numpy(),
                kg=kg.float().cpu().numpy(), cache=cache.float().cpu().numpy(),
                cache0=cache0.float().numpy(), ro=ro, rc=rc, rk=rk, rnew=rnew, acc=acc)


def check(b, r, dt, state_dt, window):
    lengths = (b.cu_seqlens[1:] - b.cu_seqlens[:-1]).tolist()
    idx = b.state_indices.tolist()
    slots = r["cache"].shape[0]
    live = [q for q, (n, s) in enumerate(zip(lengths, idx)) if n > 0 and 0 <= s < slots]
    # outputs: every token row of every request (null ones must be zero)
    e_out = parity.report("out", r["out"], r["ro"], b.cu_seqlens.numpy())
    assert e_out < tol_out(dt)
    # records: written rows against the oracle, the rest untouched
    mask = ~np.isnan(r["rc"])
    assert np.all(r["corr"][~mask] == SENT_CORR)
    e_corr = rel_rows(r["corr"][mask].reshape(-1, 128), r["rc"][mask].reshape(-1, 128))
    print(f"  corr: tested {e_corr:.3e}", flush=True)
    assert e_corr < TOL_CORR
    kmask = ~np.isnan(r["rk"])
    assert np.array_equal(r["kg"][kmask], r["rk"][kmask])
    assert np.all(r["kg"][~kmask] == SENT_KG)
    # committed states: the live requests' slots; every other slot bit-identical
    acc = r["acc"].tolist()
    moved = [idx[q] for q in live if acc[q] > 0]
    if moved:
        e_st = parity.report("state", r["cache"][moved], r["rnew"][moved])
        assert e_st < tol_state(state_dt)
    rest = [s for s in range(slots) if s not in moved]
    assert np.array_equal(r["cache"][rest], r["cache0"][rest])


@pytest.mark.parametrize("gate", [False, True])
@pytest.mark.parametrize("state_dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
def test_verify_and_commit_match_the_oracle(dt, state_dt, gate):
    lengths = [3, 8, 1, 0, 5, 8, 2, 7, 4, 6]
    b = inputs.make_verify(lengths, 8, 2, 4, 40, dtype=dt, seed=70, null=(5,))
    b.state_cache = b.state_cache * 25.0
    gp = None
    if gate:
        gp = gate_params(4, 71)
        gen = torch.Generator().manual_seed(72)
        b.g = torch.randn(b.g.shape, generator=gen).to(dt)  # raw gate ~ N(0, 1)
    r = run(b, 8, state_dt, gate=gp)
    check(b, r, dt, state_dt, 8)


@pytest.mark.parametrize("window", [1, 2, 3, 5])
def test_short_windows_and_clamped_lengths(window):
    """Windows under 8 (record stride = window); a request longer than the
    window runs only its first `window` tokens and leaves the rest of its out
    rows alone."""
    lengths = [window, 1, window + 2, window]
    b = inputs.make_verify(lengths, window, 1, 2, 16, dtype=torch.bfloat16, seed=73)
    b.state_cache = b.state_cache * 25.0
    b.meta["accepted"] = torch.tensor([window, 1, window, max(1, window - 1)], dtype=torch.int32)
    r = run(b, window)
    s = int(b.cu_seqlens[2])
    assert np.all(r["out"][s + window:s + window + 2] == 5.0)
    r["out"][s + window:s + window + 2] = 0.0   # the oracle leaves them at 0
    check(b, r, torch.bfloat16, torch.float32, window)


def test_no_l2norm_custom_scale():
    b = inputs.make_verify([4, 6, 2], 8, 2, 2, 12, dtype=torch.float32, seed=74)
    b.state_cache = b.state_cache * 25.0
    # unnormalised keys: small enough that the delta step stays a contraction
    b.q, b.k = b.q * 0.05, b.k * 0.05
    r = run(b, 8, scale=0.7, l2=False)
    check(b, r, torch.float32, torch.float32, 8)


def test_decode_workload_with_a_4_token_window():
    """256 requests x 32 heads over a [1024, 32, 128, 128] fp32 cache, 4 draft
    tokens each: every output and record on the GPU; the oracle on a sample of
    48 requests (all heads)."""
    B_, W, hv = 256, 4, 32
    b = inputs.make_verify([W] * B_, W, 32, hv, 1024, dtype=torch.bfloat16, seed=75,
                           null=(7, 100))
    cache = b.state_cache.to(DEV)
    cache0 = b.state_cache
    args = [t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)]
    out, corr, kg = B.kda_verify(*args, b.cu_seqlens.to(DEV), cache, b.state_indices.to(DEV), W)
    acc = b.meta["accepted"]
    B.kda_commit(cache, b.state_indices.to(DEV), acc.to(DEV), corr, kg)
    torch.cuda.synchronize()
    sample = list(range(0, B_, 16)) + [7, 100] + list(range(200, 232))
    sel = torch.tensor(sorted(set(sample)))
    rows = torch.cat([torch.arange(int(b.cu_seqlens[q]), int(b.cu_seqlens[q + 1])) for q in sel])
    qs = torch.arange(sel.numel() + 1, dtype=torch.int32) * W
    ro, rc, rk = oracle.verify(b.q[rows], b.k[rows], b.v[rows], b.g[rows], b.beta[rows], qs,
                               cache0, b.state_indices[sel], W)
    got = out[rows.to(DEV)].float().cpu().numpy()
    assert parity.report("out", got, ro, qs.numpy()) < 1e-2
    c = corr[sel.to(DEV)].cpu().numpy()
    m = ~np.isnan(rc)
    assert rel_rows(c[m].reshape(-1, 128), rc[m].reshape(-1, 128)) < TOL_CORR
    assert np.array_equal(kg[sel.to(DEV)].float().cpu().numpy()[m.repeat(2, -1)],
                          rk[m.repeat(2, -1)])
    rnew = oracle.commit(cache0, b.state_indices[sel], acc[sel], rc, rk)
    slots = [int(b.state_indices[q]) for q in sel if int(b.state_indices[q]) >= 0]
    got = cache[torch.tensor(slots, device=DEV)].cpu().numpy()
    assert parity.report("state", got, rnew[slots]) < tol_state(torch.float32)
    idx = b.state_indices
    untouched = torch.ones(1024, dtype=torch.bool)
    untouched[idx[idx >= 0].long()] = False
    assert torch.equal(cache[untouched.to(DEV)].cpu(), cache0[untouched])


def test_commit_equals_multi_token_decode_state():
    """The same windows through multi-token decode (a state stored after each
    token): equal outputs, and the commit at count a equals the state decode
    stored after token a - 1, on the GPU."""
    Bn, T, hv = 6, 5, 4
    b = inputs.make_verify([T] * Bn, T, 2, hv, 64, dtype=torch.bfloat16, seed=76)
    b.state_cache = b.state_cache * 25.0
    cache_v = b.state_cache.to(DEV)
    args = [t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)]
    out_v, corr, kg = B.kda_verify(*args, b.cu_seqlens.to(DEV), cache_v,
                                   b.state_indices.to(DEV), T)
    acc = torch.tensor([1, 2, 3, 4, 5, 3], dtype=torch.int32)
    B.kda_commit(cache_v, b.state_indices.to(DEV), acc.to(DEV), corr, kg)
    # decode: start rows = the verify slots, token t stored to a fresh row
    idx = b.state_indices.long()
    free = [s for s in range(64) if s not in set(idx.tolist())]
    rows = torch.zeros(Bn, T, dtype=torch.int32)
    rows[:, 0] = idx.to(torch.int32)
    rows[:, 1:] = torch.tensor(free[:Bn * (T - 1)], dtype=torch.int32).reshape(Bn, T - 1)
    cache_d = b.state_cache.to(DEV)
    rs = lambda x: x.reshape(Bn, T, *x.shape[1:]).contiguous()
    out_d = B.kda_decode(*[rs(a) for a in args], cache_d, rows.to(DEV))
    torch.cuda.synchronize()
    # the decode's first stored row overwrote the start slot: compare per count
    assert rel_rows(out_v.float().cpu().numpy(), out_d.reshape(-1, hv, 128).float().cpu().numpy()) \
        < 1e-2
    for q in range(Bn):
        a = int(acc[q])
        want = cache_d[int(rows[q, a - 1])].cpu().numpy()
        got = cache_v[int(idx[q])].cpu().numpy()
        assert parity.rel(got[None], want[None]) < 1e-5


def test_fused_projection_views_equal_contiguous_inputs():
    """q, k, v as column bands of one [T, 3 H 128] projection and the gate and
    beta as bands of wider rows (KdaTcVerify's qkv layout): same results bit
    for bit as contiguous copies."""
    lengths = [4, 8, 3]
    H = 2
    b = inputs.make_verify(lengths, 8, H, H, 12, dtype=torch.bfloat16, seed=77)
    T = b.q.shape[0]
    qkv = torch.cat([b.q.reshape(T, -1), b.k.reshape(T, -1), b.v.reshape(T, -1)], 1).to(DEV)
    gw = torch.cat([b.g.reshape(T, -1), torch.zeros(T, 64, dtype=b.g.dtype)], 1).to(DEV)
    bw = torch.cat([b.beta, torch.zeros(T, 6, dtype=b.beta.dtype)], 1).to(DEV)
    qv = qkv[:, :H * 128].view(T, H, 128)
    kv = qkv[:, H * 128:2 * H * 128].view(T, H, 128)
    vv = qkv[:, 2 * H * 128:].view(T, H, 128)
    gv = gw[:, :H * 128].view(T, H, 128)
    bv = bw[:, :H]
    cache = b.state_cache.to(DEV)
    qs, idx = b.cu_seqlens.to(DEV), b.state_indices.to(DEV)
    o1, c1, k1 = B.kda_verify(qv, kv, vv, gv, bv, qs, cache, idx, 8)
    o2, c2, k2 = B.kda_verify(*[t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)], qs, cache,
                              idx, 8)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(c1, c2) and torch.equal(k1, k2)


def test_padded_pool_slots():
    """A pool whose slots are padded past Hv planes (a cache page)."""
    lengths = [5, 3]
    b = inputs.make_verify(lengths, 8, 1, 2, 6, dtype=torch.bfloat16, seed=78)
    b.state_cache = b.state_cache * 25.0
    big = torch.zeros(6, 3, 128, 128)
    big[:, :2] = b.state_cache
    pool = big.to(DEV)[:, :2]
    args = [t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)]
    out, corr, kg = B.kda_verify(*args, b.cu_seqlens.to(DEV), pool, b.state_indices.to(DEV), 8)
    dense = b.state_cache.to(DEV)
    out2, corr2, kg2 = B.kda_verify(*args, b.cu_seqlens.to(DEV), dense,
                                    b.state_indices.to(DEV), 8)
    acc = torch.tensor([5, 2], dtype=torch.int32, device=DEV)
    B.kda_commit(pool, b.state_indices.to(DEV), acc, corr, kg)
    B.kda_commit(dense, b.state_indices.to(DEV), acc, corr2, kg2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(corr, corr2)
    assert torch.equal(pool.cpu(), dense.cpu())


@pytest.mark.parametrize("i", stress.cases())
def test_random_verify_and_commit_match_the_oracle(i):
    """Opt-in (KDA_STRESS=<cases>): seeded random windows (1..8), request
    counts (up to 300, some empty, some null slots), GVA, input dtypes, bf16
    pools and gate parameters; outputs, records and committed states against
    the oracle."""
    gen = torch.Generator().manual_seed(290000 + i)
    r = lambda n: int(torch.randint(0, n, (1,), generator=gen))
    window = 1 + r(8)
    n = 1 + r(300)
    lengths = [r(window + 1) for _ in range(n)]
    hqk = [1, 2, 4, 8][r(4)]
    hv = hqk * [1, 2, 4][r(3)]
    dt = [torch.bfloat16, torch.float32, torch.float16][r(3)]
    state_dt = torch.bfloat16 if dt == torch.bfloat16 and r(2) else torch.float32
    null = tuple(q for q in range(n) if r(10) == 0)
    gate = gate_params(hv, 299000 + i) if r(3) == 0 else None
    b = inputs.make_verify(lengths, window, hqk, hv, n + r(16), dtype=dt, seed=295000 + i,
                           null=null)
    res = run(b, window, state_dt=state_dt, gate=gate)
    check(b, res, dt, state_dt, window)
