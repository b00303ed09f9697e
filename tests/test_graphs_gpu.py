"""The library's calls captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed, as a serving loop runs them.

Every call queues kernels only: no allocation when the caller passes the
outputs and the workspace (or uses the no-allocation entry point), and no
memset (counters and flags are cleared by the kernels themselves).  Each
test captures once, then replays several times with new inputs copied in
eagerly between the replays and an eager call of the same function on the
same inputs as the reference; every replay must match it bit for bit (the
kernels are deterministic).
"""
import pytest
import torch

from gated_delta_rule_65_amd import binding as B
from gated_delta_rule_65_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def capture(fn):
    """Warm up on a side stream (first-call set-up happens outside the
    graph), then capture one call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def test_decode_graph_replays_match_eager():
    n, hqk, hv, slots = 64, 2, 4, 96
    b = inputs.make_decode(n, hqk, hv, slots, dtype=torch.bfloat16, seed=71)
    static = [t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)]
    idx = b.state_indices.clone()
    idx[5] = -1                                   # a skipped request
    idx = idx.to(DEV)
    cache0 = b.state_cache.to(DEV)
    cache = cache0.clone()
    out = torch.empty_like(static[2])
    graph = capture(lambda: B.kda_decode(*static, cache, idx, output=out))
    for r in range(3):
        nxt = inputs.make_decode(n, hqk, hv, slots, dtype=torch.bfloat16, seed=80 + r)
        for dst, src in zip(static, (nxt.q, nxt.k, nxt.v, nxt.g, nxt.beta)):
            dst.copy_(src.to(DEV))
        cache.copy_(cache0)
        ref_cache = cache0.clone()
        ref = B.kda_decode(*static, ref_cache, idx)
        torch.cuda.synchronize()
        print("decode graph replay", r, flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        assert torch.equal(cache, ref_cache), r


def test_multi_token_decode_graph_replays_match_eager():
    n, T, hqk, hv = 24, 4, 2, 4
    slots = n * T + 8

    def draw(seed):
        d = inputs.make_decode(n * T, hqk, hv, slots, dtype=torch.bfloat16, seed=seed)
        rs = lambda x: x.reshape(n, T, *x.shape[1:]).contiguous()
        return [rs(t) for t in (d.q, d.k, d.v, d.g, d.beta)], d.state_cache

    ins, cache_cpu = draw(73)
    static = [t.to(DEV) for t in ins]
    idx = torch.arange(n * T, dtype=torch.int32).reshape(n, T).to(DEV)
    acc = (torch.arange(n, dtype=torch.int32) % T + 1).to(DEV)
    cache0 = cache_cpu.to(DEV)
    cache = cache0.clone()
    out = torch.empty_like(static[2])
    graph = capture(lambda: B.kda_decode(*static, cache, idx, output=out,
                                         num_accepted_tokens=acc))
    for r in range(3):
        nxt, _ = draw(85 + r)
        for dst, src in zip(static, nxt):
            dst.copy_(src.to(DEV))
        cache.copy_(cache0)
        ref_cache = cache0.clone()
        ref = B.kda_decode(*static, ref_cache, idx, num_accepted_tokens=acc)
        torch.cuda.synchronize()
        print("multi-token decode graph replay", r, flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        assert torch.equal(cache, ref_cache), r


@pytest.mark.parametrize("no_alloc", [False, True], ids=["workspace", "no_alloc"])
@pytest.mark.parametrize("groups", [1, 2])
def test_chunk_forward_graph_replays_match_eager(groups, no_alloc):
    """A dense [B, T, H, 128] batch with a ragged last chunk, initial and final
    states, on the plain walk and the group scan; the workspace is passed in,
    or the call uses the library's static scratch (no_alloc)."""
    nb, T, hqk, hv = 2, 700, 2, 4

    def draw(seed):
        b = inputs.make_chunk([T] * nb, hqk, hv, dtype=torch.bfloat16, g_scale=0.5, seed=seed,
                              init=True)
        d4 = lambda x: x.to(DEV).view(nb, T, *x.shape[1:])
        return [d4(x) for x in (b.q, b.k, b.v, b.g, b.beta)], b.initial_state.to(DEV), b.scale

    ins, init, scale = draw(90)
    static = [t.clone() for t in ins]
    init = init.clone()
    out = torch.empty_like(static[2])
    fin = torch.empty((nb, hv, 128, 128), dtype=torch.float32, device=DEV)
    kw = dict(scale=scale, initial_state=init, output_final_state=True, groups=groups)
    if no_alloc:
        extra = dict(no_alloc=True)
    else:
        nbytes = B.chunk_workspace_bytes(*static, **kw)
        extra = dict(workspace=torch.empty(max(nbytes, 1), dtype=torch.uint8, device=DEV))
    graph = capture(lambda: B.chunk_kda(*static, output=out, final_state=fin, **kw, **extra))
    for r in range(3):
        nxt, nxt_init, _ = draw(91 + r)
        for dst, src in zip(static, nxt):
            dst.copy_(src)
        init.copy_(nxt_init)
        ref_out, ref_fin = B.chunk_kda(*static, **kw)
        torch.cuda.synchronize()
        print("chunk graph replay", r, "groups", groups, "no_alloc", no_alloc, flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), r
        assert torch.equal(fin, ref_fin), r


def test_verify_and_commit_graph_replays_match_eager():
    """One serving step as one graph: the verify window (outputs and records,
    no state), then the commit of each request's accepted prefix."""
    lengths, window, hqk, hv, slots = [4, 0, 3, 4, 1, 4, 2, 4], 4, 2, 4, 20

    def draw(seed):
        return inputs.make_verify(lengths, window, hqk, hv, slots, dtype=torch.bfloat16,
                                  seed=seed, null=(2,))

    b = draw(95)
    static = [t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)]
    qs, idx = b.cu_seqlens.to(DEV), b.state_indices.to(DEV)
    acc = b.meta["accepted"].to(DEV)
    cache0 = b.state_cache.to(DEV)
    cache = cache0.clone()
    n = len(lengths)
    out = torch.zeros_like(static[2])
    corr = torch.zeros((n, hv, window, 128), dtype=torch.float32, device=DEV)
    kg = torch.zeros((n, hv, window, 256), dtype=torch.bfloat16, device=DEV)

    def step():
        B.kda_verify(*static, qs, cache, idx, window, output=out, corr=corr, kg=kg)
        B.kda_commit(cache, idx, acc, corr, kg)

    graph = capture(step)
    for r in range(3):
        nxt = draw(96 + r)
        for dst, src in zip(static, (nxt.q, nxt.k, nxt.v, nxt.g, nxt.beta)):
            dst.copy_(src.to(DEV))
        acc.copy_(nxt.meta["accepted"].to(DEV))
        cache.copy_(cache0)
        for t in (out, corr, kg):
            t.zero_()
        ref_cache = cache0.clone()
        ro, rc, rk = B.kda_verify(*static, qs, ref_cache, idx, window)
        B.kda_commit(ref_cache, idx, acc, rc, rk)
        torch.cuda.synchronize()
        print("verify + commit graph replay", r, flush=True)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ro) and torch.equal(corr, rc) and torch.equal(kg, rk), r
        assert torch.equal(cache, ref_cache), r
