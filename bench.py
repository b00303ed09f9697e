#!/usr/bin/env python3
"""Throughput of the KDA hot path on one MI355X.

One step = one chunked forward over the dense-prefill workload (B=4, T=4096,
Hqk=Hv=16, D=128, bf16, fp32 initial and final state) followed by one paged
decode over the decode workload (256 requests x 32 heads, fp32 cache
[1024, 32, 128, 128]), inputs resident in HBM.  W untimed warm-up steps, then K
timed steps bracketed by device synchronisation, with nothing else queued
between them.  After the timed region: K more steps with two HIP events per
step on the library's stream (chunk start, decode start) for the launch
durations of the two calls, K chunk forwards with the library's stage events
for the per-kernel breakdown, and K decode launches back to back.

Printed: one JSON line.  ``value`` is whole-step throughput: the tokens of a
step (16384 prefill + 256 decode) over the mean wall time of a timed step.
``chunk_tokens_per_s`` is the chunk forward alone.  ``roofline`` describes the
kernel that takes the most time in a step (HBM traffic from rocprofv3 byte
counters scaled by a plain copy kernel, when recorded for the current kernel
sources); ``kernels`` lists all of them.  ``cpu_baseline`` times the fp64 CPU
oracle on the host.  ``--copy-calibration`` adds the reference copy kernel
after the timed region.
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


def chunk_work(lengths, hqk, hv, es, state_in, state_out):
    """Algorithmic flops and bytes per kernel for one chunked forward."""
    T = sum(lengths)
    chunks = chunk_lengths(lengths)
    nch = len(chunks)
    N = len(lengths)
    prep_b = (2 * T * hqk + T * hv) * 128 * es + T * hv * 128 * es + nch * hv * 128 * (64 * es + 4)
    wy_b = (2 * T * hqk + 2 * T * hv) * 128 * es + T * hv * es + T * hv * (2 * 128 + 64) * es
    walk_b = (T * hv * (3 * 128 + 64) * es + nch * hv * 128 * (64 * es + 4)
              + T * hv * 128 * es + (state_in + state_out) * N * hv * 128 * 128 * 4)
    # prep folded into WY: the inputs once, all six intermediates out
    intra_b = ((2 * T * hqk + 2 * T * hv) * 128 * es + T * hv * es
               + T * hv * (2 * 128 + 64) * es + nch * hv * 128 * (2 * 64 * es + 4))
    return dict(
        tokens=T,
        prep=dict(bytes=prep_b, flops=0.0),
        intra=dict(bytes=intra_b, flops=hv * sum(wy_flops(L) for L in chunks)),
        wy=dict(bytes=wy_b, flops=hv * sum(wy_flops(L) for L in chunks)),
        walk=dict(bytes=walk_b, flops=hv * sum(walk_flops(L) for L in chunks)),
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


def load_traffic(kernel: str):
    """Counter-derived HBM bytes per launch (profiles/traffic.json), or None
    when absent or taken from a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    rec = t.get("kernels", {}).get(kernel)
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


CPU_BASELINE_SECONDS = 10.0  # whole steps are repeated until this much time has passed


def cpu_baseline(batch_cpu, lengths, dec_cpu):
    """The fp64 oracle on the host, over whole steps: the prefill batch (all
    sequences and heads) and, when given, the decode batch.  The decode batch
    carries only the pool rows its requests touch (gathered, indices
    renumbered), which is the same work.  Steps repeat until
    CPU_BASELINE_SECONDS have passed."""
    import torch
    import oracle
    threads = oracle.default_threads()
    n_dec = 0
    if dec_cpu is not None:
        rows = dec_cpu.state_indices.long()
        dcache = dec_cpu.state_cache[rows]
        didx = torch.arange(rows.numel(), dtype=torch.int32)
        n_dec = rows.numel()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.recurrence(batch_cpu.q, batch_cpu.k, batch_cpu.v, batch_cpu.g, batch_cpu.beta,
                          cu_seqlens=batch_cpu.cu_seqlens, scale=batch_cpu.scale,
                          initial_state=batch_cpu.initial_state, threads=threads)
        if dec_cpu is not None:
            oracle.decode(dec_cpu.q, dec_cpu.k, dec_cpu.v, dec_cpu.g, dec_cpu.beta, dcache, didx,
                          scale=dec_cpu.scale, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= CPU_BASELINE_SECONDS:
            break
    per_step = el / reps
    dec_txt = (f" + decode batch ({n_dec} requests x {dec_cpu.v.shape[1]} heads)"
               if dec_cpu is not None else "")
    return dict(value=(sum(lengths) + n_dec) / per_step, unit="tokens/s", cores=threads,
                kind="oracle",
                sample=(f"{reps} whole steps: prefill batch ({len(lengths)} x {lengths[0]} "
                        f"tokens, {batch_cpu.v.shape[1]} heads){dec_txt}, fp64 token "
                        f"recurrence, {per_step:.2f} s per step, {el:.1f} s in all on "
                        f"{cpu_model()}"))


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
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--groups", type=int, default=0, help="chunk groups (0 = auto)")
    ap.add_argument("--walk-waves", type=int, default=0,
                    help="waves per walk workgroup: 0 = auto, 2, 4 or 8")
    ap.add_argument("--path", choices=["auto", "staged", "fused"], default="auto",
                    help="chunk path: prep as its own kernel (staged) or folded into WY")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-decode-back-to-back", action="store_true",
                    help="skip timing decode launched back to back (after the timed region), "
                         "as a serving loop runs it")
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

    # inputs resident in HBM
    wl = inputs.WORKLOADS["dense_prefill"]
    lengths = [wl["T"]] * wl["B"]
    cb = inputs.make_workload("dense_prefill", device=dev)
    hqk, hv = wl["hqk"], wl["hv"]
    T = sum(lengths)
    q4 = cb.q.view(wl["B"], wl["T"], hqk, 128)
    k4 = cb.k.view(wl["B"], wl["T"], hqk, 128)
    v4 = cb.v.view(wl["B"], wl["T"], hv, 128)
    g4 = cb.g.view(wl["B"], wl["T"], hv, 128)
    b4 = cb.beta.view(wl["B"], wl["T"], hv)
    out = torch.empty_like(v4)
    fin = torch.empty((wl["B"], hv, 128, 128), device=dev, dtype=torch.float32)
    dwl = inputs.WORKLOADS["decode_paged"]
    db = inputs.make_workload("decode_paged", device=dev)
    dout = torch.empty_like(db.v)
    # one workspace, sized once
    p = B._prepare_chunk(q4, k4, v4, g4, b4, cb.scale, cb.initial_state, True, None, True,
                         out, fin, None, None, None)
    nbytes = ctypes.c_size_t(0)
    a = B._chunk_struct(p["q"], p["k"], p["v"], p["g"], p["beta"], p["out"], None, p["N"],
                        p["T"], hqk, hv, p["scale"], True, p["init"], p["fin"], None, None,
                        None, 0, args.groups, ctypes.c_void_p(stream), args.walk_waves)
    B.load_library().kda_chunk_fwd_workspace_size(ctypes.byref(a), ctypes.byref(nbytes))
    ws = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)

    nev = B.NUM_STAGE_EVENTS
    ev_sets = [[ev.create() for _ in range(nev)] for _ in range(args.steps)]

    path = {"auto": B.PATH_AUTO, "staged": B.PATH_STAGED, "fused": B.PATH_FUSED}[args.path]

    def chunk(evs=None):
        B.chunk_kda(q4, k4, v4, g4, b4, scale=cb.scale, initial_state=cb.initial_state,
                    output_final_state=True, output=out, final_state=fin,
                    groups=args.groups, walk_waves=args.walk_waves, workspace=ws,
                    stage_events=evs, path=path)

    def decode():
        B.kda_decode(db.q, db.k, db.v, db.g, db.beta, db.state_cache, db.state_indices,
                     scale=db.scale, output=dout)

    def step():
        chunk()
        if not args.no_decode:
            decode()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed region: exactly `steps` whole steps and nothing else (an event
    # recorded between the calls of a step adds a few microseconds of queue
    # idle time at each boundary, so the per-call figures come from the pass
    # below).
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # An instrumented pass of `steps` more steps: two events per step on the
    # library's stream (chunk start, decode start; the next step's chunk start
    # closes the decode) give the launch durations of the two calls.
    tev = [ev.create() for _ in range(2 * args.steps + 1)]
    for i in range(args.steps):
        ev.record(tev[2 * i], stream)
        chunk()
        if not args.no_decode:
            ev.record(tev[2 * i + 1], stream)
            decode()
    ev.record(tev[2 * args.steps], stream)
    torch.cuda.synchronize()
    if args.no_decode:
        chunk_ms = [ev.ms(tev[2 * i], tev[2 * i + 2]) for i in range(args.steps)]
        dec_ms = []
    else:
        chunk_ms = [ev.ms(tev[2 * i], tev[2 * i + 1]) for i in range(args.steps)]
        dec_ms = [ev.ms(tev[2 * i + 1], tev[2 * i + 2]) for i in range(args.steps)]
    for e in tev:
        ev.destroy(e)

    # After the timed region: the per-kernel breakdown from the library's
    # stage events, and decode launched back to back (each launch then also
    # waits out the write-back of the previous one's state rows).
    for i in range(args.steps):
        chunk(ev_sets[i])
    torch.cuda.synchronize()
    dec_b2b_ms = None
    if not args.no_decode_back_to_back and not args.no_decode:
        a_, b_ = ev.create(), ev.create()
        ev.record(a_, stream)
        for _ in range(args.steps):
            decode()
        ev.record(b_, stream)
        torch.cuda.synchronize()
        dec_b2b_ms = ev.ms(a_, b_) / args.steps
        ev.destroy(a_)
        ev.destroy(b_)

    names = ["table", "prep", "wy", "walk", "compose", "pass2"]
    per = {n: [] for n in names}
    for i in range(args.steps):
        e = ev_sets[i]
        for j, n in enumerate(names):
            per[n].append(ev.ms(e[j], e[j + 1]))
    mean = lambda xs: sum(xs) / max(len(xs), 1)
    t_chunk = mean(chunk_ms) / 1e3
    work = chunk_work(lengths, hqk, hv, 2, True, True)
    flops = work["wy"]["flops"] + work["walk"]["flops"]

    # the fused path records an empty prep stage: its WY kernel carries prep
    fused = args.path != "staged"
    kernels = {}
    stages = (("wy", "intra", "mfma"),) if fused else (("prep", "prep", "hbm"),
                                                      ("wy", "wy", "mfma"))
    for n, wk, bound in stages + (("walk", "walk", "mfma"),):
        ms = mean(per[n])
        if ms <= 0:
            continue
        s = ms / 1e3
        gbs = work[wk]["bytes"] / s / 1e9
        tfl = work[wk]["flops"] / s / 1e12
        kernels[n] = dict(ms=round(ms, 4), bound=bound, gb_s=round(gbs, 1),
                          tflops=round(tfl, 2), hbm_frac=round(gbs / PEAK_HBM_GBS, 4),
                          frac=round((gbs / PEAK_HBM_GBS) if bound == "hbm"
                                     else (tfl / PEAK_BF16_TFLOPS), 4))
        if n == "wy" and fused:
            kernels[n]["note"] = "prep folded in (reads q, k, v, g, beta; writes all intermediates)"
    for n in ("compose", "pass2"):
        ms = mean(per[n])
        if ms > 0.003:
            kernels[n] = dict(ms=round(ms, 4))
    dec = None
    if not args.no_decode:
        dw = decode_work(dwl["N"], dwl["hqk"], dwl["hv"], 2)
        s = mean(dec_ms) / 1e3
        gbs = dw["bytes"] / s / 1e9
        kernels["decode"] = dict(ms=round(s * 1e3, 4), bound="hbm", gb_s=round(gbs, 1),
                                 frac=round(gbs / PEAK_HBM_GBS, 4))
        dec = dict(ms=round(s * 1e3, 4), gb_s=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4),
                   state_gb_s=round(dw["state_bytes"] / s / 1e9, 1),
                   back_to_back_ms=None if dec_b2b_ms is None else round(dec_b2b_ms, 4),
                   back_to_back_gb_s=None if dec_b2b_ms is None else
                   round(dw["bytes"] / (dec_b2b_ms / 1e3) / 1e9, 1),
                   workload=f"{dwl['N']} requests x {dwl['hv']} heads, cache "
                            f"[{dwl['slots']}, {dwl['hv']}, 128, 128] fp32")

    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    kd = kernels[dom]
    kname = {"prep": "prep_kernel", "wy": "wy_kernel", "walk": "walk_kernel",
             "decode": "decode_kernel"}[dom]
    wkey = "intra" if (dom == "wy" and fused) else dom
    if kd["bound"] == "hbm":
        wb = work[wkey]["bytes"] if dom != "decode" else decode_work(
            dwl["N"], dwl["hqk"], dwl["hv"], 2)["bytes"]
        roof = dict(bound="hbm", achieved=kd["gb_s"], peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=kd["frac"], kernel=kname, algorithmic_bytes=wb)
    else:
        roof = dict(bound="mfma", achieved=kd["tflops"], peak=PEAK_BF16_TFLOPS,
                    unit="TFLOP/s", frac=kd["frac"], kernel=kname,
                    algorithmic_flops=work[wkey]["flops"])
    roof["traffic"] = load_traffic(kname)
    roof["launch_ms"] = kd["ms"]

    n_dec = 0 if args.no_decode else dwl["N"]
    step_s = wall / args.steps
    res = dict(
        metric=METRIC, value=round((T + n_dec) / step_s, 1), unit="tokens/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup,
        ms_per_step=round(wall / args.steps * 1e3, 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload="dense_prefill", B=wl["B"], T=wl["T"], hqk=hqk, hv=hv,
                    head_dim=128, chunk=64, state="fp32 initial+final",
                    groups=args.groups, walk_waves=args.walk_waves,
                    path="fused" if fused else "staged",
                    decode=None if dec is None else dec["workload"],
                    value_counts=f"{T} prefill + {n_dec} decode tokens per step"),
        chunk_ms=round(t_chunk * 1e3, 4),
        chunk_tokens_per_s=round(T / t_chunk, 1),
        tflops=round(flops / t_chunk / 1e12, 2),
        mfma_frac=round(flops / t_chunk / 1e12 / PEAK_BF16_TFLOPS, 4),
        decode=dec, kernels=kernels, roofline=roof,
    )
    if args.copy_calibration:
        res["copy_calibration"] = copy_calibration(dev)
    if not args.no_cpu_baseline:
        cpu = inputs.Batch(cb.q.cpu(), cb.k.cpu(), cb.v.cpu(), cb.g.cpu(), cb.beta.cpu(),
                           cb.cu_seqlens.cpu(), cb.scale, initial_state=cb.initial_state.cpu())
        dcpu = None
        if not args.no_decode:
            dcpu = inputs.Batch(db.q.cpu(), db.k.cpu(), db.v.cpu(), db.g.cpu(), db.beta.cpu(),
                                db.cu_seqlens.cpu(), db.scale, state_cache=db.state_cache.cpu(),
                                state_indices=db.state_indices.cpu())
        res["cpu_baseline"] = cpu_baseline(cpu, lengths, dcpu)
    else:
        res["cpu_baseline"] = None
    for es in ev_sets:
        for e in es:
            ev.destroy(e)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
