#!/usr/bin/env python3
"""Throughput of the KDA hot path on one MI355X.

One step = one chunked forward over the long single-sequence prefill
(B=1, T=131072, Hqk=Hv=32, D=128, bf16, slow decay g = -0.5 sigmoid(N(0,1)),
fp32 initial and final state), the largest of the workloads, inputs resident
in HBM.  W untimed warm-up steps, then K timed steps bracketed by device
synchronisation, with nothing else queued between them.  ``value`` is its
tokens/s: 131072 tokens over the mean wall time of a step.

After the timed region, each with HIP events on the library's stream:
  * K more calls with the library's stage events: the per-kernel breakdown
    of the headline workload (``kernels``: one row per kernel launch, each
    with its algorithmic flops and bytes and its roofline bound, HBM when its
    arithmetic intensity is below the ridge point of 312.5 flop/B, MFMA
    above) and ``roofline``, the row of its longest kernel;
  * the chunk path as a whole (all kernels of a call) against the bf16 MFMA
    peak: ``roofline_chunk_path``;
  * the other prefill workloads, each timed alone (``legs``): the dense
    prefill (B=4, T=4096, H=16) and the varlen GVA batch (24 sequences,
    32768 tokens, Hqk=8, Hv=32, paged fp32 state);
  * the paged decode (256 requests x 32 heads, fp32 pool [1024, 32, 128,
    128], updated in place) after a dense-prefill chunk forward and back to
    back: ``decode`` and ``roofline_decode`` (state bytes against HBM).
``cpu_baseline`` times the fp64 CPU oracle over the headline workload on the
host.  ``--copy-calibration`` adds the reference copy kernel for scaling HBM
byte counters.
"""
from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("chunk_kda fwd tokens/s + TFLOP/s (% bf16 MFMA peak); "
          "decode state GB/s (% HBM)")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
K = V = 128
C = 64


# ------------------------------------------------------------ work accounting

def wy_flops(L: int) -> float:
    """Triangle-aware WY work of one chunk of L tokens for one value head:
    A_kk (strictly lower) + A_qk (lower) + the unit-lower inverse + w and u."""
    return K * L * (L - 1) + K * L * (L + 1) + L ** 3 / 3 + (K + V) * L * (L - 1)


def walk_flops(L: int) -> float:
    """Walk work of one chunk: w S, qg S, kg^T U (2 L K V each), A_qk U
    (lower), and the diagonal decay of S."""
    return V * L * (L + 1) + 6 * L * K * V + K * V


def chunk_lengths(lengths):
    out = []
    for n in lengths:
        out += [C] * (n // C) + ([n % C] if n % C else [])
    return out


def chunk_work(lengths, hqk, hv, es, state_in, state_out, groups=1):
    """Algorithmic flops and bytes per kernel for one chunked forward (groups:
    the chunk groups of the walk's group scan, 1 for the plain walk)."""
    T = sum(lengths)
    chunks = chunk_lengths(lengths)
    nch = len(chunks)
    N = len(lengths)
    plane = 128 * 128 * 4
    prep_b = (2 * T * hqk + T * hv) * 128 * es + T * hv * 128 * es + nch * hv * 128 * (64 * es + 4)
    wy_b = (2 * T * hqk + 2 * T * hv) * 128 * es + T * hv * es + T * hv * (2 * 128 + 64) * es
    walk_b = (T * hv * (3 * 128 + 64) * es + nch * hv * 128 * (64 * es + 4)
              + T * hv * 128 * es + (state_in + state_out) * N * hv * 128 * 128 * 4)
    # prep folded into WY: the inputs once, all six intermediates out
    intra_b = ((2 * T * hqk + 2 * T * hv) * 128 * es + T * hv * es
               + T * hv * (2 * 128 + 64) * es + nch * hv * 128 * (2 * 64 * es + 4))
    wyf = hv * sum(wy_flops(L) for L in chunks)
    wkf = hv * sum(walk_flops(L) for L in chunks)
    G = max(1, groups)
    planes = G * N * hv * plane
    # pass one walks every group but the last: its chunks, per sequence
    p1_chunks, p1_T = [], 0
    for n_ in lengths:
        cl = chunk_lengths([n_])
        cpg = -(-len(cl) // G) if cl else 0
        keep = cl[:min(len(cl), (G - 1) * cpg)]
        p1_chunks += keep
        p1_T += sum(keep)
    # group scan.  Pass one reads w, kg_t, u_t and decay and writes a group's
    # transfer and partial state; compose reads those and the start states and
    # writes each group's start state; pass two is the plain walk from them.
    # Work: pass one walks the 128 value and the 128 transfer columns without
    # outputs (w S and kg^T U for both), compose G - 1 products of 128^3 per
    # (sequence, head).
    p1_b = (p1_T * hv * 128 * es + len(p1_chunks) * hv * 128 * (2 * 64 * es + 4)
            + 2 * planes * (G - 1) // G)
    p1_f = 2 * hv * sum(4 * L * K * V + K * V for L in p1_chunks)
    cmp_b = 2 * planes + (state_in * N * hv * plane) + planes
    cmp_f = 2.0 * (G - 1) * N * hv * (2 * K * K * V)
    p2_b = walk_b + planes
    # on-chip path: inputs once per pass, outputs and states; nothing else
    in_b = (2 * T * hqk + 2 * T * hv) * 128 * es + T * hv * es
    oc_b = in_b + T * hv * 128 * es + (state_in + state_out) * N * hv * plane
    oc1_b = ((2 * p1_T * hv + p1_T * hqk) * 128 * es + p1_T * hv * es
             + 2 * planes * (G - 1) // G)
    return dict(
        tokens=T,
        prep=dict(bytes=prep_b, flops=0.0),
        intra=dict(bytes=intra_b, flops=wyf),
        wy=dict(bytes=wy_b, flops=wyf),
        walk=dict(bytes=walk_b, flops=wkf),
        pass_one=dict(bytes=p1_b, flops=p1_f),
        compose=dict(bytes=cmp_b, flops=cmp_f),
        pass_two=dict(bytes=p2_b, flops=wkf),
        onchip=dict(bytes=oc_b, flops=wyf + wkf),
        onchip_pass_one=dict(bytes=oc1_b,
                             flops=hv * sum(wy_flops(L) for L in p1_chunks) + p1_f),
        onchip_pass_two=dict(bytes=oc_b + planes, flops=wyf + wkf),
        table=dict(bytes=4 * (2 * N + 1), flops=0.0),
    )


def decode_work(n, hqk, hv, es):
    state = n * hv * 128 * 128 * 4 * 2
    io = n * (2 * hqk * 128 + 2 * hv * 128 + hv + hv * 128) * es + n * 4
    return dict(bytes=state + io, state_bytes=state)


# ------------------------------------------------------------------ HIP events

class HipEvents:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def record(self, e, stream):
        if self.lib.hipEventRecord(ctypes.c_void_p(e), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        out = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(out), ctypes.c_void_p(a),
                                        ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(out.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(ctypes.c_void_p(e))


# ------------------------------------------------------------------- helpers

def source_hash():
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "gated_delta_rule_65_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, row: str):
    """Counter-derived HBM bytes per launch of kernel row `row` on `workload`
    (profiles/traffic.json), or None when absent or taken from a different
    kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    rec = t.get("workloads", {}).get(workload, {}).get(row)
    return None if not rec else rec.get("bytes_per_launch")


def roofline_of(flops, nbytes, ms):
    """The roofline bound of a kernel from its arithmetic intensity against
    the ridge point (bf16 MFMA peak / HBM peak = 312.5 flop per byte), and
    the achieved rate against that bound's peak."""
    s = ms / 1e3
    if nbytes and flops / nbytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        gbs = nbytes / s / 1e9
        return dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(gbs / PEAK_HBM_GBS, 4))
    tf = flops / s / 1e12
    return dict(bound="mfma", achieved=round(tf, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                frac=round(tf / PEAK_BF16_TFLOPS, 4))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


CPU_BASELINE_SECONDS = 10.0  # whole calls are repeated until this much time has passed


def cpu_baseline(batch_cpu, name):
    """The fp64 oracle on the host over whole calls of the headline workload
    (every sequence, head and token), repeated until CPU_BASELINE_SECONDS have
    passed.  Threads: the oracle's default (the host's cores, capped at the
    16-thread CPU share of one GPU); the host's core count is reported
    beside it."""
    import oracle
    threads = oracle.default_threads()
    T = batch_cpu.q.shape[0]
    hv = batch_cpu.v.shape[1]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.recurrence(batch_cpu.q, batch_cpu.k, batch_cpu.v, batch_cpu.g, batch_cpu.beta,
                          cu_seqlens=batch_cpu.cu_seqlens, scale=batch_cpu.scale,
                          initial_state=batch_cpu.initial_state, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= CPU_BASELINE_SECONDS:
            break
    per = el / reps
    units = batch_cpu.num_seqs * hv
    return dict(value=round(T / per, 1), unit="tokens/s", cores=threads,
                host_cores=os.cpu_count(), kind="oracle",
                sample=(f"{reps} whole call(s) of {name} ({T} tokens x {hv} heads, "
                        f"{units} independent (sequence, head) chains), fp64 token "
                        f"recurrence on {threads} threads, {per:.2f} s per call, "
                        f"{el:.1f} s in all on {cpu_model()}"))


# ---------------------------------------------------------------------- main

CAL_BYTES = 256 << 20  # bytes read (and written) by one calibration copy


def copy_calibration(dev):
    """A plain copy kernel of known size (fp32 x * 1.0 into another buffer),
    launched three times, for scaling FETCH_SIZE / WRITE_SIZE readings."""
    import torch
    src = torch.ones(CAL_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    return dict(kernel="elementwise mul (copy)", bytes_read=CAL_BYTES, bytes_written=CAL_BYTES,
                launches=3)


def next_rows(dev):
    """The rows beyond the hot path, each timed against its plain counterpart:
    gate parameters, mid-prefill checkpoints and inputs read through a
    per-token stride on the dense-prefill chunked forward; multi-token
    (speculative) decode and a bf16 state pool on the decode workload.  Inputs
    are resident in HBM.  The clocks drift with the recent load by several
    percent, so a row and its plain counterpart are timed alternately (three
    rounds of 20 calls after 3 warm-up calls, CUDA events) and the medians are
    compared."""
    import torch
    from gated_delta_rule_65_amd import binding as B
    from gated_delta_rule_65_amd import inputs

    def timed(fn, reps=20, warm=3):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def against(plain_fn, fn, rounds=3):
        tp, tv = [], []
        for _ in range(rounds):
            tp.append(timed(plain_fn))
            tv.append(timed(fn))
        return sorted(tp)[rounds // 2], sorted(tv)[rounds // 2]

    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    res = {}
    # ---- chunked forward: dense prefill in varlen form with the max_seqlen hint
    wl = inputs.WORKLOADS["dense_prefill"]
    cb = inputs.make_workload("dense_prefill", device=dev)
    T, N, hv = cb.q.shape[0], wl["B"], wl["hv"]
    base = dict(scale=cb.scale, initial_state=cb.initial_state, output_final_state=True,
                cu_seqlens=cb.cu_seqlens, max_seqlen=wl["T"])

    def plain():
        B.chunk_kda(cb.q, cb.k, cb.v, cb.g, cb.beta, **base)

    def chunk_row(fn, **extra):
        p_ms, ms = against(plain, fn)
        return dict(ms=round(ms, 4), plain_ms=round(p_ms, 4),
                    tokens_per_s=round(T / ms * 1e3, 1), vs_plain=round(p_ms / ms, 3), **extra)

    # f1: g as a raw gate, lower_bound * sigmoid(exp(A_log) (g + dt_bias)); with
    # A_log = 0, dt_bias = 0 and g ~ N(0, 1) this is the workload's own g draw
    g_raw = torch.randn(cb.g.shape, generator=gen, device=dev).to(cb.g.dtype)
    a_log = torch.zeros(hv, device=dev)
    dt_bias = torch.zeros(hv, 128, device=dev)
    res["f1_gate_parameters"] = chunk_row(
        lambda: B.chunk_kda(cb.q, cb.k, cb.v, g_raw, cb.beta, A_log=a_log, dt_bias=dt_bias,
                            **base))
    # f2: one mid-prefill snapshot per sequence, at half its length
    ck_state = torch.empty(N, hv, 128, 128, device=dev)
    ck_off = torch.full((N,), wl["T"] // 2, dtype=torch.int32, device=dev)
    res["f2_checkpoints"] = chunk_row(
        lambda: B.chunk_kda(cb.q, cb.k, cb.v, cb.g, cb.beta, checkpoint_state=ck_state,
                            checkpoint_offsets=ck_off, **base),
        snapshot=f"1 per sequence at token {wl['T'] // 2}")
    # f4: q, k, v, g, beta as bands of one [T, W] projection output (per-token stride)
    flat = [x.reshape(T, -1) for x in (cb.q, cb.k, cb.v, cb.g, cb.beta)]
    W = sum(f.shape[1] for f in flat) + 8
    W += (-W) % 8
    proj = torch.empty((T, W), dtype=cb.q.dtype, device=dev)
    views, off = [], 0
    for x, f in zip((cb.q, cb.k, cb.v, cb.g, cb.beta), flat):
        proj[:, off:off + f.shape[1]] = f
        views.append(proj[:, off:off + f.shape[1]].view(x.shape))
        off += f.shape[1]
    res["f4_strided_inputs"] = chunk_row(lambda: B.chunk_kda(*views, **base),
                                         layout=f"bands of one [{T}, {W}] bf16 buffer")
    del cb, proj, views, g_raw
    torch.cuda.empty_cache()
    # ---- decode: 256 requests x 32 heads over a [1024, 32, 128, 128] pool
    dwl = inputs.WORKLOADS["decode_paged"]
    db = inputs.make_workload("decode_paged", device=dev)
    n, hqk, dhv = dwl["N"], dwl["hqk"], dwl["hv"]
    state1 = n * dhv * 128 * 128 * 4 * 2
    io1 = decode_work(n, hqk, dhv, 2)["bytes"] - state1

    def dplain():
        B.kda_decode(db.q, db.k, db.v, db.g, db.beta, db.state_cache, db.state_indices,
                     scale=db.scale)

    def decode_row(fn, byt, **extra):
        p_ms, ms = against(dplain, fn)
        return dict(ms=round(ms, 4), plain_ms=round(p_ms, 4), gb_s=round(byt / ms / 1e6, 1),
                    hbm_frac=round(byt / ms / 1e6 / PEAK_HBM_GBS, 4),
                    plain_gb_s=round((state1 + io1) / p_ms / 1e6, 1), **extra)

    # f4: the same decode over a bf16 pool (rounded after each token)
    cache16 = db.state_cache.to(torch.bfloat16)
    res["f4_bf16_state_decode"] = decode_row(
        lambda: B.kda_decode(db.q, db.k, db.v, db.g, db.beta, cache16, db.state_indices,
                             scale=db.scale),
        n * dhv * 128 * 128 * 2 * 2 + io1)
    del cache16
    torch.cuda.empty_cache()
    # f3: 4 tokens per request, each token's state stored to its own pool row
    tt = 4
    slots = db.state_cache.shape[0]

    def draw(shape, s=1.0):
        return (s * torch.randn(shape, generator=gen, device=dev)).to(torch.bfloat16)
    qm, km = draw((n, tt, hqk, 128)), draw((n, tt, hqk, 128))
    vm, bm = draw((n, tt, dhv, 128)), draw((n, tt, dhv))
    gm = (-5.0 * torch.sigmoid(torch.randn((n, tt, dhv, 128), generator=gen,
                                           device=dev))).to(torch.bfloat16)
    idx = torch.randperm(slots, generator=gen, device=dev)[:n * tt].to(torch.int32).view(n, tt)
    row = decode_row(
        lambda: B.kda_decode(qm, km, vm, gm, bm, db.state_cache, idx, scale=db.scale),
        n * dhv * 128 * 128 * 4 * (1 + tt) + tt * io1, tokens_per_request=tt)
    row["tokens_per_s"] = round(n * tt / row["ms"] * 1e3, 1)
    res["f3_multi_token_decode"] = row
    # f3: the record-based verify of the same windows (outputs and records, no
    # state), then the commit of a random accepted prefix from the records
    qs = torch.arange(n + 1, dtype=torch.int32, device=dev) * tt
    flat = [x.reshape(n * tt, *x.shape[2:]) for x in (qm, km, vm, gm, bm)]
    sidx = idx[:, 0].contiguous()
    outv = torch.empty((n * tt, dhv, 128), dtype=torch.bfloat16, device=dev)
    corr = torch.empty((n, dhv, tt, 128), device=dev)
    kgr = torch.empty((n, dhv, tt, 256), dtype=torch.bfloat16, device=dev)
    acc = torch.randint(1, tt + 1, (n,), generator=gen, device=dev, dtype=torch.int32)

    def multi():
        B.kda_decode(qm, km, vm, gm, bm, db.state_cache, idx, scale=db.scale)

    def verify():
        B.kda_verify(*flat, qs, db.state_cache, sidx, tt, scale=db.scale, output=outv, corr=corr,
                     kg=kgr)

    def commit():
        B.kda_commit(db.state_cache, sidx, acc, corr, kgr)

    units = n * dhv
    io_tok = 2 * hqk * 256 + dhv * (3 * 256 + 2)       # q, k; v, g, out; beta
    rec_tok = 128 * 4 + 256 * 2                         # corr fp32, kg bf16
    v_bytes = units * 128 * 128 * 4 + n * tt * io_tok + units * tt * rec_tok
    c_bytes = units * 128 * 128 * 4 * 2 + dhv * int(acc.sum()) * rec_tok
    m_ms, v_ms = against(multi, verify)
    c_ms = timed(commit)
    res["f3_verify_window"] = dict(
        tokens_per_request=tt, verify_ms=round(v_ms, 4), commit_ms=round(c_ms, 4),
        multi_token_decode_ms=round(m_ms, 4),
        vs_multi_token_decode=round(m_ms / (v_ms + c_ms), 3),
        verify_gb_s=round(v_bytes / v_ms / 1e6, 1),
        verify_hbm_frac=round(v_bytes / v_ms / 1e6 / PEAK_HBM_GBS, 4),
        commit_gb_s=round(c_bytes / c_ms / 1e6, 1),
        commit_hbm_frac=round(c_bytes / c_ms / 1e6 / PEAK_HBM_GBS, 4),
        bytes_per_unit=dict(verify=round(v_bytes / units), commit=round(c_bytes / units),
                            multi_token_decode=128 * 128 * 4 * (1 + tt) + round(tt * io1 / units)),
        accepted_mean=round(float(acc.float().mean()), 3))
    return res


STAGES = ["table", "prep", "wy", "walk", "compose", "pass2"]
class ChunkCase:
    """One prefill workload resident in HBM with preallocated outputs and
    workspace; call() queues one kda_chunk_fwd on the current stream."""

    def __init__(self, name, dev, args):
        import torch
        from gated_delta_rule_65_amd import binding as B
        from gated_delta_rule_65_amd import inputs
        self.B, self.name, self.args = B, name, args
        wl = inputs.WORKLOADS[name]
        self.b = b = inputs.make_workload(name, device=dev)
        self.lengths = b.meta["lengths"]
        self.hqk, self.hv = b.q.shape[1], b.v.shape[1]
        self.T = b.q.shape[0]
        self.paged = b.state_cache is not None
        self.out = torch.empty_like(b.v)
        self.fin = None if self.paged else torch.empty(
            (b.num_seqs, self.hv, 128, 128), device=dev, dtype=torch.float32)
        self.max_seqlen = max(self.lengths)
        self.path = {"auto": B.PATH_AUTO, "staged": B.PATH_STAGED,
                     "fused": B.PATH_FUSED, "onchip": B.PATH_ONCHIP}[args.path]
        # A dense workload (B sequences of T tokens) is passed as chunk_kda's
        # [B, T, H, 128] tensors without cu_seqlens, as a caller holds it; the
        # varlen batch as [S, H, 128] with cu_seqlens.
        self.dense = wl["kind"] == "chunk"
        if self.dense:
            nb, tl = wl["B"], wl["T"]
            d4 = lambda x: x.view(nb, tl, *x.shape[1:])
            self.inputs = tuple(d4(x) for x in (b.q, b.k, b.v, b.g, b.beta))
            self.kw = dict(scale=b.scale, output=d4(self.out))
        else:
            self.inputs = (b.q, b.k, b.v, b.g, b.beta)
            self.kw = dict(scale=b.scale, cu_seqlens=b.cu_seqlens, max_seqlen=self.max_seqlen,
                           output=self.out)
        self.kw.update(groups=args.groups, walk_waves=args.walk_waves, path=self.path)
        if self.paged:
            self.kw.update(state_cache=b.state_cache, state_indices=b.state_indices,
                           has_initial_state=b.has_initial_state)
        else:
            self.kw.update(initial_state=b.initial_state, output_final_state=True,
                           final_state=self.fin)
        self.plan = B.chunk_plan(*self.inputs,
                                 cu_seqlens=None if self.dense else b.cu_seqlens,
                                 initial_state=None if self.paged else b.initial_state,
                                 output_final_state=not self.paged, groups=args.groups,
                                 walk_waves=args.walk_waves,
                                 max_seqlen=None if self.dense else self.max_seqlen,
                                 path=self.path)
        nbytes = B.chunk_workspace_bytes(*self.inputs, **self._ws_kw())
        self.ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        es = 2 if b.q.dtype == torch.bfloat16 else 4
        self.work = chunk_work(self.lengths, self.hqk, self.hv, es, True, True,
                               groups=self.plan[0])
        self.flops = self.work["wy"]["flops"] + self.work["walk"]["flops"]

    def _ws_kw(self):
        kw = dict(self.kw)
        kw.pop("output", None)
        kw.pop("final_state", None)
        return kw

    def call(self, events=None):
        self.B.chunk_kda(*self.inputs, workspace=self.ws, stage_events=events, **self.kw)

    def cpu_batch(self):
        from gated_delta_rule_65_amd import inputs
        b = self.b
        return inputs.Batch(b.q.cpu(), b.k.cpu(), b.v.cpu(), b.g.cpu(), b.beta.cpu(),
                            b.cu_seqlens.cpu(), b.scale,
                            initial_state=None if b.initial_state is None
                            else b.initial_state.cpu())


def timed_calls(ev, stream, fn, n, warm=3):
    """Mean ms of n back-to-back calls of fn, by two HIP events on stream."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a_, b_ = ev.create(), ev.create()
    ev.record(a_, stream)
    for _ in range(n):
        fn()
    ev.record(b_, stream)
    torch.cuda.synchronize()
    ms = ev.ms(a_, b_) / n
    ev.destroy(a_)
    ev.destroy(b_)
    return ms


def stage_breakdown(ev, case, n):
    """Mean ms per stage over n calls with the library's stage events."""
    import torch
    sets = [[ev.create() for _ in range(len(STAGES) + 1)] for _ in range(n)]
    for i in range(n):
        case.call(sets[i])
    torch.cuda.synchronize()
    per = {st: 0.0 for st in STAGES}
    for i in range(n):
        for j, st in enumerate(STAGES):
            per[st] += ev.ms(sets[i][j], sets[i][j + 1]) / n
    for es in sets:
        for e in es:
            ev.destroy(e)
    return per


def kernel_rows(case, per):
    """One row per kernel launch of a chunked forward, from its stage times:
    algorithmic work, time, and the roofline bound with the achieved rate."""
    w = case.work
    onchip = case.path == case.B.PATH_ONCHIP
    fused_prep = case.path != case.B.PATH_STAGED
    groups = case.plan[0]
    rows = {}

    def row(name, kernel, key, ms, note=None):
        if ms <= 0:
            return
        r = dict(kernel=kernel, ms=round(ms, 4), algorithmic_flops=w[key]["flops"],
                 algorithmic_bytes=w[key]["bytes"])
        r.update(roofline_of(w[key]["flops"], w[key]["bytes"], ms))
        s_ = ms / 1e3
        r["tflops"] = round(w[key]["flops"] / s_ / 1e12, 2)
        r["gb_s"] = round(w[key]["bytes"] / s_ / 1e9, 1)
        if note:
            r["note"] = note
        rows[name] = r

    if per["table"] > 0:
        rows["table"] = dict(kernel="chunk_offsets_kernel", ms=round(per["table"], 4))
    if onchip:
        if groups > 1:
            row("pass_one", "onchip_kernel<1>", "onchip_pass_one", per["walk"],
                "group scan pass one: the intra-chunk stage and the walk of the value and "
                "transfer columns, per chunk, on chip")
            row("compose", "compose_kernel", "compose", per["compose"])
            row("pass_two", "onchip_kernel<2>", "onchip_pass_two", per["pass2"],
                "group scan pass two: the intra-chunk stage and the walk, on chip")
        else:
            row("walk", "onchip_kernel<0>", "onchip", per["walk"],
                "the intra-chunk stage and the walk, per chunk, on chip")
        return rows
    if not fused_prep:
        row("prep", "prep_kernel", "prep", per["prep"])
    row("wy", "wy_kernel", "intra" if fused_prep else "wy", per["wy"],
        "prep folded in (reads q, k, v, g, beta; writes all intermediates)"
        if fused_prep else None)
    if groups > 1:
        bf16 = str(case.b.q.dtype) == "torch.bfloat16"
        row("pass_one", "pass_one_kernel" if bf16 else "walk_kernel<1>", "pass_one",
            per["walk"],
            f"group scan (G = {groups}) pass one: each group walked from zero and from the "
            "identity (value and transfer columns), no outputs")
        row("compose", "compose_kernel", "compose", per["compose"])
        row("pass_two", "walk_kernel<2>", "pass_two", per["pass2"],
            f"group scan (G = {groups}) pass two: the plain walk from the composed start "
            "states")
    else:
        row("walk", "walk_kernel<0>", "walk", per["walk"])
    return rows


def chunk_leg(ev, stream, case, n):
    """A prefill workload timed alone: whole call and its kernels."""
    ms = timed_calls(ev, stream, case.call, n)
    per = stage_breakdown(ev, case, max(3, n // 2))
    s = ms / 1e3
    return dict(workload=case.name, tokens=case.T, ms=round(ms, 4),
                tokens_per_s=round(case.T / s, 1), tflops=round(case.flops / s / 1e12, 2),
                mfma_frac=round(case.flops / s / 1e12 / PEAK_BF16_TFLOPS, 4),
                groups=case.plan[0], walk_waves=case.plan[1],
                kernels=kernel_rows(case, per))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_single",
                    choices=["long_single", "dense_prefill", "varlen_gva_paged"],
                    help="the headline prefill workload (default: the largest)")
    ap.add_argument("--groups", type=int, default=0, help="chunk groups (0 = auto)")
    ap.add_argument("--walk-waves", type=int, default=0,
                    help="waves per walk workgroup: 0 = auto, 2, 4 or 8")
    ap.add_argument("--path", choices=["auto", "staged", "fused", "onchip"], default="auto",
                    help="chunk path: prep as its own kernel (staged), folded into WY "
                         "(fused), or the intra-chunk stage inside the walk (onchip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the other prefill workloads and the decode")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run a plain elementwise copy of "
                         f"{CAL_BYTES >> 20} MiB (reads and writes that many bytes) three "
                         "times: the reference kernel for scaling HBM byte counters")
    ap.add_argument("--next-rows", action="store_true",
                    help="instead of the step: time the rows beyond the hot path (gate "
                         "parameters, checkpoints, strided inputs, multi-token decode, bf16 "
                         "state) against their plain counterparts; one JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by head or sequence with no communication; see the "
              "design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_65_amd import binding as B
    from gated_delta_rule_65_amd import inputs

    B.load_library()   # raises if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.next_rows:
        print(json.dumps(dict(kind="next_rows", data="synthetic", dtype="bf16",
                              rows=next_rows(dev))))
        return
    ev = HipEvents()
    stream = torch.cuda.current_stream(dev).cuda_stream

    # ---- the headline step: one chunked forward over the headline workload
    print(f"bench: {args.workload}: inputs", file=sys.stderr, flush=True)
    case = ChunkCase(args.workload, dev, args)
    for _ in range(args.warmup):
        case.call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        case.call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_s = wall / args.steps
    print(f"bench: {args.workload}: {step_s * 1e3:.3f} ms per step", file=sys.stderr,
          flush=True)
    call_ms = timed_calls(ev, stream, case.call, args.steps, warm=0)
    per = stage_breakdown(ev, case, args.steps)
    kernels = kernel_rows(case, per)
    # the dominant kernel of the step (its algorithmic work per launch over its
    # event-timed launch duration)
    dom = max((k for k in kernels if k != "table"), key=lambda k: kernels[k]["ms"])
    kd = kernels[dom]
    roof = {k: kd[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof.update(kernel=kd["kernel"], algorithmic_bytes=kd["algorithmic_bytes"],
                algorithmic_flops=kd["algorithmic_flops"])
    # (counters are recorded per workload for the default path, and under
    # "workload@path" for the others: the kernels and their rows differ)
    tkey = args.workload if args.path == "auto" else f"{args.workload}@{args.path}"
    roof["traffic"] = load_traffic(tkey, dom)
    roof["launch_ms"] = kd["ms"]
    if "note" in kd:
        roof["note"] = kd["note"]
    cs = call_ms / 1e3
    min_b = case.work["onchip"]["bytes"]
    roof_path = dict(bound="mfma", achieved=round(case.flops / cs / 1e12, 2),
                     peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                     frac=round(case.flops / cs / 1e12 / PEAK_BF16_TFLOPS, 4),
                     kernel="whole chunked forward (every kernel of one call)",
                     algorithmic_flops=case.flops, launch_ms=round(call_ms, 4),
                     min_bytes=min_b,
                     min_bytes_gb_s=round(min_b / cs / 1e9, 1),
                     min_bytes_hbm_frac=round(min_b / cs / 1e9 / PEAK_HBM_GBS, 4),
                     note="min_bytes: inputs, outputs and states only, the HBM floor of a "
                          "path that keeps every intermediate on chip")
    wl = inputs.WORKLOADS[args.workload]
    config = dict(workload=args.workload, B=len(case.lengths), T=max(case.lengths),
                  tokens=case.T, hqk=case.hqk, hv=case.hv, head_dim=128, chunk=64,
                  dtype="bf16", g="-%g*sigmoid(N(0,1))" % wl["g_scale"],
                  state="paged fp32" if case.paged else "fp32 initial+final",
                  groups=case.plan[0], walk_waves=case.plan[1], path=args.path)
    res = dict(
        metric=METRIC, value=round(case.T / step_s, 1), unit="tokens/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=round(step_s * 1e3, 4),
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
        data="synthetic", config=config,
        chunk_ms=round(call_ms, 4), tflops=roof_path["achieved"], mfma_frac=roof_path["frac"],
        kernels=kernels, roofline=roof, roofline_chunk_path=roof_path,
    )
    cpu_in = None
    if not args.no_cpu_baseline:
        cpu_in = case.cpu_batch()
    del case
    torch.cuda.empty_cache()

    # ---- the other prefill workloads and the decode, each timed alone
    if not args.no_legs:
        legs = {}
        for name in ("dense_prefill", "varlen_gva_paged", "long_single"):
            if name == args.workload:
                continue
            print(f"bench: leg {name}", file=sys.stderr, flush=True)
            c = ChunkCase(name, dev, args)
            legs[name] = chunk_leg(ev, stream, c, 10)
            if name == "dense_prefill":
                dense = c
            else:
                del c
            torch.cuda.empty_cache()
        res["legs"] = legs
        print("bench: decode", file=sys.stderr, flush=True)
        if args.workload == "dense_prefill" or "dense" not in locals():
            dense = ChunkCase("dense_prefill", dev, args)
        dwl = inputs.WORKLOADS["decode_paged"]
        db = inputs.make_workload("decode_paged", device=dev)
        dout = torch.empty_like(db.v)

        def decode():
            B.kda_decode(db.q, db.k, db.v, db.g, db.beta, db.state_cache, db.state_indices,
                         scale=db.scale, output=dout)
        # in a step after a chunk forward (its writes still draining), and back to back
        for _ in range(3):
            dense.call()
            decode()
        torch.cuda.synchronize()
        tev = [ev.create() for _ in range(2 * args.steps)]
        for i in range(args.steps):
            dense.call()
            ev.record(tev[2 * i], stream)
            decode()
            ev.record(tev[2 * i + 1], stream)
        torch.cuda.synchronize()
        dec_ms = sum(ev.ms(tev[2 * i], tev[2 * i + 1]) for i in range(args.steps)) / args.steps
        for e in tev:
            ev.destroy(e)
        b2b_ms = timed_calls(ev, stream, decode, args.steps)
        dw = decode_work(dwl["N"], dwl["hqk"], dwl["hv"], 2)
        gbs = dw["bytes"] / (dec_ms / 1e3) / 1e9
        gbs_b2b = dw["bytes"] / (b2b_ms / 1e3) / 1e9
        res["decode"] = dict(
            workload=f"{dwl['N']} requests x {dwl['hv']} heads, cache [{dwl['slots']}, "
                     f"{dwl['hv']}, 128, 128] fp32, in place",
            ms=round(dec_ms, 4), gb_s=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4),
            back_to_back_ms=round(b2b_ms, 4), back_to_back_gb_s=round(gbs_b2b, 1),
            back_to_back_hbm_frac=round(gbs_b2b / PEAK_HBM_GBS, 4),
            tokens_per_s=round(dwl["N"] / (dec_ms / 1e3), 1))
        res["roofline_decode"] = dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS,
                                      unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4),
                                      kernel="decode_kernel", algorithmic_bytes=dw["bytes"],
                                      traffic=load_traffic("decode_paged", "decode"),
                                      launch_ms=round(dec_ms, 4),
                                      note="launched after a dense-prefill chunked forward")
        del dense, db
        torch.cuda.empty_cache()
    if args.copy_calibration:
        res["copy_calibration"] = copy_calibration(dev)
    if cpu_in is not None:
        print("bench: cpu baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cpu_in, args.workload)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res))


if __name__ == "__main__":
    main()
