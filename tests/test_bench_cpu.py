"""bench.py's work model and contract on the CPU.

The roofline fractions bench.py reports divide algorithmic flops and bytes by
measured time, so the model is checked here against counts derived from the
operand shapes alone: per (token, value head) of a full 64-token chunk, the
intra-chunk (WY) stage multiplies A_kk (strictly lower), A_qk (lower with the
diagonal), the unit-lower inverse (a triangular solve, L^3 / 3), and w and u
(the strictly lower T times a 64 x 128 block each); the walk multiplies w S,
qg S and kg^T U (64 x 128 x 128 each), A_qk U (lower) and scales the state by
its decay.  Byte counts are the tensors each kernel must read or write once.
"""
import subprocess
import sys

import pytest

import bench

D, C = 128, 64


def tri(n, diag):
    """Entries of an n x n lower triangle (with or without the diagonal)."""
    return n * (n + 1) // 2 if diag else n * (n - 1) // 2


def test_intra_chunk_flops_per_token_head():
    akk = 2 * D * tri(C, False)          # strictly lower dots of length 128
    aqk = 2 * D * tri(C, True)           # lower with the diagonal
    inv = C ** 3 / 3                     # unit-lower triangular inverse
    wu = 2 * (2 * D * tri(C, False))     # T (strictly lower part) x 64 x 128, twice
    per_chunk = akk + aqk + inv + wu
    assert bench.wy_flops(C) == pytest.approx(per_chunk, rel=1e-12)
    assert bench.wy_flops(C) / C == pytest.approx(33877.33, abs=0.01)


def test_walk_flops_per_token_head():
    dense = 3 * 2 * C * D * D            # w S, qg S (64 x 128 x 128), kg^T U (128 x 64 x 128)
    aqk_u = 2 * D * tri(C, True)         # lower A_qk times U
    decay = D * D                        # diag(d) S
    assert bench.walk_flops(C) == dense + aqk_u + decay
    assert bench.walk_flops(C) / C == 106880


def test_long_sequence_intermediate_bytes():
    """One 131072-token sequence, 32 heads, bf16: the fused WY kernel reads q,
    k, v, g and beta and writes qg, w, kg_t, u_t, aqk and the fp32 decay."""
    T, H, es = 131072, 32, 2
    nch = T // C
    inputs = 4 * T * H * D * es + T * H * es
    token_major = 2 * T * H * D * es + T * H * C * es      # qg, w, aqk
    chunk_major = 2 * nch * H * D * C * es + nch * H * D * 4  # kg_t, u_t, decay
    w = bench.chunk_work([T], H, H, es, True, True, groups=8)
    assert w["intra"]["bytes"] == inputs + token_major + chunk_major == 9168748544
    # pass two: qg, w, aqk, kg_t, u_t, decay in; out, the start and final states
    plane = D * D * 4
    p2 = (2 * T * H * D * es + T * H * C * es + 2 * nch * H * D * C * es + nch * H * D * 4
          + T * H * D * es + 2 * H * plane + 8 * H * plane)
    assert w["pass_two"]["bytes"] == p2
    # the floor of an on-chip path: inputs, outputs and states only
    assert w["onchip"]["bytes"] == inputs + T * H * D * es + 2 * H * plane


def test_decode_bytes():
    """256 requests x 32 heads: every touched 64 KiB fp32 state read and
    written, plus the token's inputs, its output row and the slot index."""
    n, hqk, hv, es = 256, 32, 32, 2
    state = 2 * n * hv * D * D * 4
    io = n * (2 * hqk * D + 2 * hv * D + hv + hv * D) * es + n * 4
    got = bench.decode_work(n, hqk, hv, es)
    assert got["state_bytes"] == state
    assert got["bytes"] == state + io == 1084244992


def test_roofline_bound_follows_the_ridge_point():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    assert ridge == pytest.approx(312.5)
    low = bench.roofline_of(100.0 * 1e9, 1e9, 1.0)      # 100 flop/B: bytes bound
    assert low["bound"] == "hbm" and low["achieved"] == pytest.approx(1000.0)
    assert low["frac"] == pytest.approx(1000.0 / bench.PEAK_HBM_GBS, abs=1e-4)
    high = bench.roofline_of(1000.0 * 1e9, 1e9, 1.0)    # 1000 flop/B: MFMA bound
    assert high["bound"] == "mfma" and high["achieved"] == pytest.approx(1000.0)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", str(n)],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout + r.stderr
