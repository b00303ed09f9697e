"""kda_chunk_fwd_noalloc (the entry point for callers that cannot allocate)
against kda_chunk_fwd on the same inputs: two calls in a row through the
C ABI, the second smaller than the first, so the shared static scratch is
reused with stale contents from the first call.  The two entry points run
the same kernels, so outputs and final states must agree bit for bit; both
also meet the oracle at the usual bar."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_65_amd import binding as B
from gated_delta_rule_65_amd import inputs
from parity import report

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(b, **kw):
    q, k, v, g, beta = [t.to(DEV) for t in (b.q, b.k, b.v, b.g, b.beta)]
    init = None if b.initial_state is None else b.initial_state.to(DEV)
    out, fin = B.chunk_kda(q, k, v, g, beta, scale=b.scale, initial_state=init,
                           output_final_state=True, cu_seqlens=b.cu_seqlens.to(DEV), **kw)
    torch.cuda.synchronize()
    return out.cpu(), fin.cpu()


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_noalloc_matches_workspace_entry_on_two_calls(dt):
    big = inputs.make_chunk([700, 1, 300, 130], 2, 4, dtype=dt, g_scale=0.5, seed=501, init=True)
    small = inputs.make_chunk([90, 65], 1, 2, dtype=dt, g_scale=0.5, seed=502, init=True)
    for name, b in (("first (larger)", big), ("second (smaller)", small)):
        print("noalloc", dt, name, b.meta["lengths"], flush=True)
        o_na, s_na = _run(b, no_alloc=True)
        o_ws, s_ws = _run(b)
        assert torch.equal(o_na, o_ws) and torch.equal(s_na, s_ws), name
        o_ref, s_ref = oracle.recurrence(b.q, b.k, b.v, b.g, b.beta, cu_seqlens=b.cu_seqlens,
                                         scale=b.scale, initial_state=b.initial_state)
        t_ = 1e-4 if dt == torch.float32 else 1e-2
        assert report("out", o_na.float().numpy(), o_ref, b.cu_seqlens) < t_
        assert report("state", s_na.numpy(), s_ref) < t_


def test_noalloc_rejects_calls_beyond_its_scratch():
    """A call whose workspace exceeds the static scratch (here through 64
    chunk groups of 8 heads: 64 x 8 group-scan planes of 192 KiB) is refused
    with KDA_ERR_WORKSPACE, and nothing is written."""
    T, hv = 4096, 8
    dev = torch.device(DEV)
    q = torch.zeros(T, 1, 128, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(T, hv, 128, dtype=torch.bfloat16, device=dev)
    beta = torch.zeros(T, hv, dtype=torch.bfloat16, device=dev)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    need = B.chunk_workspace_bytes(q, q, v, v, beta, cu_seqlens=cu, groups=64)
    assert need > 64 << 20, need
    out = torch.full_like(v, 3.0)
    with pytest.raises(ValueError, match="workspace"):
        B.chunk_kda(q, q, v, v, beta, cu_seqlens=cu, output=out, groups=64, no_alloc=True)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
