"""Throughput of the chunked gated-delta-rule prefill on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--workload 3]

One step = one gdn_prefill_ex call (both kernels: stage 1, then the spine with
the output fused in) over the whole synthetic workload, inputs resident in HBM.
Default workload: B=4 sequences of T=8192 tokens, nk=16 k-heads, nv=32
v-heads, dk=dv=128, carried float32 state updated in place, per-chunk entry
states emitted (the one workload that asks for them; the others run without).
--raw-qk draws q and k unnormalised and has the kernels normalise them.
Prints one JSON line.

Warm-up: the W untimed warm-up steps run first; if they took less than 50 ms
of GPU time, untimed steps continue until 50 ms have passed.  An idle MI355X
sits in a low-power state, and the first ~25 ms of this workload run 5-40 %
slower than the steady state while clocks settle; the timed K steps are then
all at steady state.  The line reports the warm-up actually run
("warmup_steps_run", "warmup_ms").

roofline: the dominant kernel's irreducible bytes per launch -- what the
method must move at least, whatever the implementation: q and k once per
k-head, v, the output, the entry states where the workload asks for them, and
the state read and written -- over its average launch time, timed live with
HIP events on the launch stream (timing-only events, without the
system-scope fence: "timing_events"); "whole_step" gives the same for the whole
step (g and beta added).  The implementation's own byte model (its
intermediates included) is reported beside it as "impl_*".
traffic: HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE, read
from profiles/traffic_<kernel>_<workload>.json when that file was taken on the
current kernel source (its sha256 matches), else null.
cpu_baseline: the oracle (float64 token recurrence) timed on the host cores
over a bounded sample of the same workload's chains.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN chunked prefill tokens/sec on 1 MI355X; % bf16 MFMA / HBM roofline"
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, AMD published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, AMD published
WARMUP_MIN_S = 0.05            # untimed warm-up floor: clocks reach steady state (see docstring)
KERNELS = {1: "chunk_cumsum_recompute_wu", 2: "chunk_delta_h_fwd_o"}
KERNEL_SRC = {1: "k1_chunk_cumsum_recompute_wu.hip", 2: "k2_chunk_delta_h_fwd_o.hip", 3: "k3_recurrent_decode.hip"}


# ---------------------------------------------------------------------------
# byte and flop model (algorithmic: every byte each stage must move once)


OPT_ENTRY_STATES, OPT_L2NORM_QK = 0x1, 0x2  # include/gdn_prefill.h


def irreducible(p, entry):
    """The bytes the method must move at least, for problem p: per kernel
    (the spine moves q, k, v, the output, the entry states and the state;
    stage 1 the gates g, beta) and for the whole step.  q and k are counted
    once per k-head; the entry states only where the workload asks for them
    (32 KB per chunk-head); the float32 state is read and written once per
    (sequence, v-head)."""
    N, nk, nv = p.n_tokens, p.nk, p.nv
    slots = int(p.cu_chunks[-1]) * nv
    d = 128
    qk = 2 * N * nk * d * 2
    v = N * nv * d * 2
    o = N * nv * d * 2
    gb = N * nv * 8
    s_out = slots * d * d * 2 if entry else 0
    state = 2 * p.nseq * nv * d * d * 4
    per = {1: gb, 2: qk + v + o + s_out + state}
    return per, sum(per.values())


def algorithmic(p, flags=OPT_ENTRY_STATES):
    """Per-kernel bytes and flops of this implementation for problem p
    (inputs.Problem) and call options.

    Bytes: every operand each kernel reads or writes once (q, k counted once
    per k-head).  Stage 1 reads k, g, beta (and q with normalisation) and
    writes gc and T' (10 KB per chunk-head, a bf16 hi + lo pair; with
    normalisation the row scales, 512 B); stage 2 reads q, k, v, gc, T' (and
    the row scales) and the state, and writes o, the state and (when asked
    for) the entry states (32 KB per chunk-head).
    Flops: the dense-tile MFMA work per chunk-head of what each kernel computes
    (Gram in stage 1; K h, T' R, K^T uc, Q h, the scores Q K^T and A uc in
    stage 2), each product counted once."""
    N, nk, nv = p.n_tokens, p.nk, p.nv
    slots = int(p.cu_chunks[-1]) * nv
    nseq = p.nseq
    d, C = 128, 64
    norm = bool(flags & OPT_L2NORM_QK)
    k_bytes = N * nk * d * 2
    q_bytes = N * nk * d * 2
    v_bytes = N * nv * d * 2
    gb_bytes = N * nv * 8
    gc_bytes = slots * C * 4
    tp_bytes = slots * 2 * 2560 * 2  # hi + lo, 2560 bf16 each
    nrm_bytes = slots * 2 * C * 4 if norm else 0
    s_bytes = slots * d * d * 2 if flags & OPT_ENTRY_STATES else 0
    state_bytes = nseq * nv * d * d * 4
    o_bytes = N * nv * d * 2
    by = {
        1: k_bytes + (q_bytes if norm else 0) + gb_bytes + gc_bytes + tp_bytes + nrm_bytes,
        2: q_bytes + k_bytes + v_bytes + gc_bytes + tp_bytes + nrm_bytes + 2 * state_bytes + s_bytes + o_bytes,
    }
    fl = {1: slots * (2 * C * C * d),
          2: slots * (6 * C * d * d + 6 * C * C * d)}
    return by, fl


def read_write_bytes(p, flags):
    """Per kernel, the (read, write) split of algorithmic()'s bytes."""
    N, nk, nv = p.n_tokens, p.nk, p.nv
    slots = int(p.cu_chunks[-1]) * nv
    d, C = 128, 64
    norm = bool(flags & OPT_L2NORM_QK)
    qk = N * nk * d * 2
    small = slots * C * 4 + slots * 2 * 2560 * 2 + (slots * 2 * C * 4 if norm else 0)  # gc, T', row scales
    state = p.nseq * nv * d * d * 4
    s_out = slots * d * d * 2 if flags & OPT_ENTRY_STATES else 0
    return {1: (qk * (2 if norm else 1) + N * nv * 8, small),
            2: (2 * qk + N * nv * d * 2 + small + state, N * nv * d * 2 + s_out + state)}


def workload_flags(meta, raw_qk=False, entry_states="auto"):
    """Call options for a workload: entry states where it asks for them (or as
    ``entry_states`` = "on" / "off" forces), q/k normalisation in the kernels
    for raw q, k."""
    entry = bool(meta.get("entry_states")) if entry_states == "auto" else entry_states == "on"
    return (OPT_ENTRY_STATES if entry else 0) | (OPT_L2NORM_QK if raw_qk else 0)


def source_sha(stage):
    """Hash of what a kernel is built from: its source, the device headers and
    the build flags."""
    from linear_attention_ssm_chunk_amd import build
    csrc = os.path.join(ROOT, "linear_attention_ssm_chunk_amd", "csrc")
    h = hashlib.sha256()
    for f in [KERNEL_SRC[stage]] + sorted(f for f in os.listdir(csrc) if f.endswith(".h")):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(build.FLAGS[:-2]).encode())  # without the include path
    return h.hexdigest()


def traffic_for(stage, workload_name):
    path = os.path.join(ROOT, "profiles", f"traffic_{KERNELS[stage]}_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_sha(stage):
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample, forked workers (before the GPU
# is touched)


def _oracle_worker(args):
    w, workers, seconds = args
    from threadpoolctl import threadpool_limits
    from oracle import gdn_recurrence, kv_head_map, l2_normalize
    from linear_attention_ssm_chunk_amd.inputs import bf16_to_f64
    p = _SAMPLE_PROBLEM
    kmap = kv_head_map(p.nk, p.nv)
    norm = p.meta.get("raw_qk", False)
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        # chains (sequence, v-head) in a fixed order, worker w takes every
        # workers-th one, until its time is up
        for chain in range(w, p.nseq * p.nv, workers):
            i, h = chain % p.nseq, (chain // p.nseq * 7) % p.nv
            a, L = int(p.cu_seqlens[i]), int(p.lengths[i])
            kap = kmap[[h]]
            q = bf16_to_f64(p.q[a:a + L][:, kap])
            k = bf16_to_f64(p.k[a:a + L][:, kap])
            if norm:  # the method's per-token normalisation, as the kernels are asked to do it
                q, k = l2_normalize(q), l2_normalize(k)
            v = bf16_to_f64(p.v[a:a + L][:, [h]])
            g = p.g[a:a + L][:, [h]].astype("float64")
            b = p.beta[a:a + L][:, [h]].astype("float64")
            h0 = p.h0[i][[h]].astype("float64")
            pos, step = 0, 256
            while pos < L and time.perf_counter() - t0 < seconds:
                n = min(step, L - pos)
                _, h0, _ = gdn_recurrence(q[pos:pos + n], k[pos:pos + n], v[pos:pos + n],
                                          g[pos:pos + n], b[pos:pos + n], h0)
                pos += n
                done += n
            if time.perf_counter() - t0 >= seconds:
                break
    return done, time.perf_counter() - t0


_SAMPLE_PROBLEM = None


def cpu_baseline(p, seconds_per_worker=1.5):
    import multiprocessing as mp
    global _SAMPLE_PROBLEM
    _SAMPLE_PROBLEM = p
    workers = max(1, min(16, os.cpu_count() or 1))
    jobs = [(w, workers, seconds_per_worker) for w in range(workers)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.map(_oracle_worker, jobs)
    wall = time.perf_counter() - t0
    token_heads = sum(r[0] for r in res)
    cpu_s = sum(r[1] for r in res)
    return {
        "value": token_heads / wall / p.nv,
        "unit": "tokens/s",
        "cores": workers,
        "host_cores": os.cpu_count(),
        "kind": "oracle",
        "sample": (f"{workers} workers (one BLAS thread each; the host reports {os.cpu_count()} cores) running "
                   f"(sequence, v-head) chains of this workload through the float64 token recurrence for "
                   f"{seconds_per_worker}s each: {token_heads} token-heads, {cpu_s:.1f} core-s, wall {wall:.1f}s; "
                   f"tokens/s = token-heads/s / nv"),
    }


# ---------------------------------------------------------------------------
# decode: one recurrent step per sequence (gdn_decode), a serving batch

DECODE_METRIC = "GDN recurrent decode tokens/sec on 1 MI355X; % HBM roofline"
DECODE_SHAPE = dict(B=256, nk=16, nv=32)


def decode_bytes(B, nk, nv):
    """Algorithmic bytes of one decode step: the float32 state read and
    written (64 KB each way per head), q and k once per k-head, v, g, beta, o."""
    d = 128
    return B * (nv * d * d * 4 * 2 + 2 * nk * d * 2 + nv * d * 2 + nv * 8 + nv * d * 2)


def _oracle_decode_worker(args):
    w, workers, seconds = args
    from threadpoolctl import threadpool_limits
    from oracle import gdn_recurrence, kv_head_map, l2_normalize
    from linear_attention_ssm_chunk_amd.inputs import bf16_to_f64
    p = _SAMPLE_PROBLEM
    raw = p.meta.get("raw_qk", False)
    kmap = kv_head_map(p.nk, p.nv)
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        chain = w
        while time.perf_counter() - t0 < seconds:
            i, h = chain % p.nseq, (chain // p.nseq) % p.nv
            kap = kmap[[h]]
            q, k = bf16_to_f64(p.q[i:i + 1][:, kap]), bf16_to_f64(p.k[i:i + 1][:, kap])
            if raw:
                q, k = l2_normalize(q), l2_normalize(k)
            gdn_recurrence(q, k, bf16_to_f64(p.v[i:i + 1][:, [h]]), p.g[i:i + 1][:, [h]].astype("float64"),
                           p.beta[i:i + 1][:, [h]].astype("float64"), p.h0[i][[h]].astype("float64"))
            done += 1
            chain += workers
    return done, time.perf_counter() - t0


def bench_decode(args):
    import multiprocessing as mp
    global _SAMPLE_PROBLEM
    from linear_attention_ssm_chunk_amd import inputs as I
    sh = DECODE_SHAPE
    raw = bool(args.raw_qk)
    p = I.make_problem([1] * sh["B"], sh["nk"], sh["nv"], seed=6, raw_qk=raw)
    p.meta["raw_qk"] = raw
    cpu = None
    if not args.no_cpu_baseline:
        _SAMPLE_PROBLEM = p
        workers = max(1, min(16, os.cpu_count() or 1))
        t0 = time.perf_counter()
        with mp.get_context("fork").Pool(workers) as pool:
            res = pool.map(_oracle_decode_worker, [(w, workers, 1.5) for w in range(workers)])
        wall = time.perf_counter() - t0
        heads = sum(r[0] for r in res)
        cpu = {"value": heads / wall / p.nv, "unit": "tokens/s", "cores": workers, "host_cores": os.cpu_count(),
               "kind": "oracle",
               "sample": (f"{workers} workers (one BLAS thread each) running single-token steps of this batch's "
                          f"(sequence, v-head) pairs through the float64 recurrence for 1.5 s each: {heads} "
                          f"head-steps, wall {wall:.1f}s; tokens/s = head-steps/s / nv")}
    import torch
    from linear_attention_ssm_chunk_amd.device import DeviceProblem
    # the decode takes the problem's q/k normalisation bit (GDN_OPT_L2NORM_QK with --raw-qk)
    dp = DeviceProblem(p, ragged=False, flags=OPT_L2NORM_QK if raw else 0)
    warm_t0 = time.perf_counter()
    warm_steps = 0
    while warm_steps < args.warmup or time.perf_counter() - warm_t0 < WARMUP_MIN_S:
        for _ in range(10):
            dp.decode_step(0)
        warm_steps += 10
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        dp.decode_step(0)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_kernel = e0.elapsed_time(e1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    by = decode_bytes(sh["B"], sh["nk"], sh["nv"])
    achieved = by / (ms_kernel / 1e3) / 1e9
    line = {
        "metric": DECODE_METRIC, "value": round(sh["B"] / (ms_per_step / 1e3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": warm_steps,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "decode_B256", "B": sh["B"], "nk": sh["nk"], "nv": sh["nv"], "dk": 128, "dv": 128,
                   "tokens_per_sequence": 1, "qk_normalised_in_kernels": raw},
        "roofline": {"bound": "hbm", "kernel": "recurrent_decode", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     # the committed counters are of the call without normalisation
                     "traffic": None if raw else traffic_for_decode()},
        "kernels": {"recurrent_decode": {"ms": round(ms_kernel, 4), "alg_bytes": by}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def traffic_for_decode():
    path = os.path.join(ROOT, "profiles", "traffic_recurrent_decode_decode_B256.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_sha(3):
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# section stamps: cycles per section of the spine's step, from the profiling
# build (libgdn_prefill_stamps.so, built with -DGDN_SECTION_STAMPS)

STAMP_FIRST, STAMP_STEPS, STAMP_SLOTS, STAMP_WAVES = 8, 32, 16, 8  # gdn_params.h
COMPUTE_SECTIONS = {  # mark k closes the section that began at mark k-1 (k2_chunk_delta_h_fwd_o.hip)
    4: {  # four strips per workgroup: the compute waves form the output
        1: "split h (first pair), entry-state tile write, previous chunk's A uc and output tile",
        2: "Q h (output state term) with the rest of the split",
        3: "K h rows 0..31 (entry states 0..63 out)",
        4: "K h rows 32..63, R rows 0..31 (entry states 64..127 out)",
        5: "T' R rows 0..31 and R rows 32..63",
        6: "T' R rows 32..63; uc rows 0..31 decayed and split",
        7: "K^T uc rows 0..31; uc rows 32..63 decayed and split",
        8: "K^T uc rows 32..63",
        9: "barrier wait",
    },
    2: {  # one or two strips: the output is formed on a loader
        1: "split h (first pair), bf16 h and entry-state tile writes, operand reads",
        2: "K h rows 0..31 with the rest of the split",
        3: "(no section)",
        4: "K h rows 32..63, R rows 0..31",
        5: "T' R rows 0..31 and R rows 32..63",
        6: "T' R rows 32..63; uc rows 0..31 to the output tile, decayed and split",
        7: "K^T uc rows 0..31; uc rows 32..63 to the output tile, decayed and split",
        8: "K^T uc rows 32..63",
        9: "barrier wait",
    },
}
# loader roles: (name, what marks 1, 2, 3 close in a step where the pair stages
# the next chunk ("active"), what mark 3 closes in the other steps ("idle"))
LOADER_ROLES = {
    (4, 0): ("Q rows, K rows 0..31; output stores; score rows 0 and 3", "stage", "issue fetch", "-",
             "output stores, scores"),
    (4, 1): ("K rows 32..63, T', V, gate factors; score rows 1 and 2", "stage", "issue fetch", "-", "scores"),
    (2, 0): ("Q rows; output stores", "delay and stage", "issue fetch", "-", "delay and output stores"),
    (2, 1): ("T', V, gate factors; scores; output", "stage", "issue fetch", "output", "scores"),
    (2, 2): ("K rows", "delay and stage", "issue fetch", "-", "delay"),
}


def section_stamps(args):
    """Run the workload with the profiling build, stamp one step window of
    workgroup 0 (sequence 0, v-head 0), and print cycles per section."""
    import numpy as np
    import torch
    from linear_attention_ssm_chunk_amd import binding, build
    L = binding.load(build.LIB_STAMPS)
    import ctypes
    L.gdn_debug_set_stamps.argtypes = [ctypes.c_void_p]
    from linear_attention_ssm_chunk_amd import inputs as I
    from linear_attention_ssm_chunk_amd.device import DeviceProblem
    p = I.make_workload(args.workload, raw_qk=args.raw_qk)
    flags = workload_flags(p.meta, args.raw_qk, args.entry_states)
    kw = dict(flags=flags)
    if p.meta["layout"] == "conv":
        kw["layout"] = "conv"
    elif p.meta["layout"] == "varlen_table":
        kw.update(state="table", ragged=True)
    dp = DeviceProblem(p, **kw)
    t0 = time.perf_counter()
    n = 0
    while n < args.warmup or time.perf_counter() - t0 < WARMUP_MIN_S:
        dp.run()
        n += 1
        torch.cuda.synchronize()
    buf = torch.zeros(STAMP_WAVES * STAMP_STEPS * STAMP_SLOTS, dtype=torch.int64, device="cuda")
    L.gdn_debug_set_stamps(buf.data_ptr())
    dp.run()
    torch.cuda.synchronize()
    L.gdn_debug_set_stamps(None)
    st = buf.cpu().numpy().astype(np.int64).reshape(STAMP_WAVES, STAMP_STEPS, STAMP_SLOTS)
    chains = p.nseq * p.nv
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    strips = 1 if chains * 8 <= cus else 2 if chains * 4 <= cus else 4
    nch = int(p.cu_chunks[1] - p.cu_chunks[0])
    steps = min(STAMP_STEPS, nch - STAMP_FIRST) - 1  # full steps in the window
    w0 = st[0]
    step_cyc = np.diff(w0[:steps + 1, 0])
    step_rt = np.diff(w0[:steps + 1, 15])  # 100 MHz ticks
    clock = float(step_cyc.sum() / step_rt.sum() * 0.1)  # GHz
    names = COMPUTE_SECTIONS[4 if strips == 4 else 2]
    comp = {names[k]: round(float(np.mean(w0[:steps, k] - w0[:steps, k - 1])), 1) for k in range(1, 10)}
    loaders = {}
    nload = 4 if strips == 4 else 6
    for w in range(strips, min(strips + nload, STAMP_WAVES)):
        li = w - strips
        role = (li >> 1) if strips == 4 else (1, 0, 2)[li >> 1]
        name, m1, m2, m3, idle3 = LOADER_ROLES[(4 if strips == 4 else 2, role)]
        pair = li & 1
        t = st[w].astype(np.float64)
        # a loader stages in step c when (c + 1) % 2 == pair and is idle otherwise
        act = [c for c in range(steps) if (STAMP_FIRST + c + 1) % 2 == pair]
        idle = [c for c in range(steps) if (STAMP_FIRST + c) % 2 == pair]
        mean = lambda cs, k1, k0: round(float(np.mean([t[c, k1] - t[c, k0] for c in cs])), 1)  # noqa: E731
        loaders[f"wave {w}: {name}"] = {
            "active: " + m1: mean(act, 1, 0), "active: " + m2: mean(act, 2, 1), "active: " + m3: mean(act, 3, 2),
            "active: barrier wait": mean(act, 4, 3),
            "idle: " + idle3: mean(idle, 3, 0), "idle: barrier wait": mean(idle, 4, 3)}
    out = {"workload": p.meta["name"], "entry_states": bool(flags & OPT_ENTRY_STATES),
           "strips_per_workgroup": strips, "chunks": nch,
           "stamped_steps": f"{STAMP_FIRST}..{STAMP_FIRST + steps - 1} of sequence 0, v-head 0, workgroup 0",
           "clock_GHz": round(clock, 3), "cycles_per_step": round(float(step_cyc.mean()), 1),
           "us_per_step": round(float(step_rt.mean()) / 100.0, 3),
           "compute_wave_0": comp, "loaders": loaders}
    print(json.dumps(out), flush=True)


def workload_shape(index):
    """The sizes the byte models read, without drawing the workload's values:
    token count, heads, sequence count and chunk offsets."""
    from types import SimpleNamespace
    import numpy as np
    from linear_attention_ssm_chunk_amd import inputs as I
    w = I.WORKLOADS[index]
    lengths = I.ragged_lengths(index, w["nseq"])[0] if "nseq" in w else [w["T"]] * w["B"]
    cu_chunks = np.concatenate([[0], np.cumsum([-(-L // 64) for L in lengths])])
    return SimpleNamespace(n_tokens=int(sum(lengths)), nk=w["nk"], nv=w["nv"], nseq=len(lengths),
                           cu_chunks=cu_chunks, meta=dict(w))


def stream_ceiling(args):
    """The achievable HBM rate for each kernel's read:write mix on this GPU:
    a streaming kernel (profiling build) reads and writes the same byte counts
    as the kernel does on the workload, interleaved in the same ratio; best of
    three grid sizes, 20 timed launches each after warm-up."""
    import ctypes
    import torch
    from linear_attention_ssm_chunk_amd import binding, build
    L = binding.load(build.LIB_STAMPS)
    L.gdn_debug_stream_mix.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.gdn_debug_stream_mix.restype = ctypes.c_int
    p = workload_shape(args.workload)
    flags = workload_flags(p.meta, args.raw_qk, args.entry_states)
    rw = read_write_bytes(p, flags)
    mixes = {KERNELS[st]: rw[st] for st in sorted(rw)}
    mixes["whole step"] = (rw[1][0] + rw[2][0], rw[1][1] + rw[2][1])
    mixes["copy 1:1"] = (max(rw[2]), max(rw[2]))
    biggest = max(max(r, w) for r, w in mixes.values())
    src = torch.zeros(biggest // 4 + 4, dtype=torch.int32, device="cuda")
    dst = torch.empty(biggest // 4 + 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    out = {"workload": p.meta["name"], "entry_states": bool(flags & OPT_ENTRY_STATES), "mixes": {}}
    for name, (r, w) in mixes.items():
        r, w = r // 16 * 16, w // 16 * 16
        best = None
        for blocks in (1024, 2048, 4096):
            def launch():
                rc = L.gdn_debug_stream_mix(src.data_ptr(), r, dst.data_ptr(), w, sink.data_ptr(), blocks, stream)
                if rc != 0:
                    raise RuntimeError(f"stream_mix failed ({rc})")
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < WARMUP_MIN_S:
                launch()
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                launch()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 20
            gbs = (r + w) / (ms / 1e3) / 1e9
            if best is None or gbs > best[0]:
                best = (gbs, blocks, ms)
        out["mixes"][name] = {"read_bytes": r, "write_bytes": w, "read_share": round(r / (r + w), 3),
                              "GBps": round(best[0], 1), "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4),
                              "blocks": best[1], "ms": round(best[2], 4)}
    print(json.dumps(out), flush=True)


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it skips the system-scope cache write-back and invalidation that
    a default event performs (and that slows the kernel after it).  The times
    are read only after a device synchronisation.  The HIP runtime is the one
    torch has loaded (the process holds one copy, found by its mapped path)."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000  # hip_runtime_api.h

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            hip = ctypes.CDLL(path)
            vp = ctypes.c_void_p
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [vp, vp]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            hip.hipEventDestroy.argtypes = [vp]
            for fn in (hip.hipEventCreateWithFlags, hip.hipEventRecord, hip.hipEventElapsedTime, hip.hipEventDestroy):
                fn.restype = ctypes.c_int
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        self._ctypes = ctypes
        self.ev = ctypes.c_void_p()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: error {rc}")

    def record(self, stream):
        rc = self._runtime().hipEventRecord(self.ev, self._ctypes.c_void_p(int(stream)))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord: error {rc}")

    def elapsed_time(self, end):
        ms = self._ctypes.c_float()
        rc = self._runtime().hipEventElapsedTime(self._ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime: error {rc}")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--entry-states", choices=("auto", "on", "off"), default="auto",
                    help="emit the per-chunk entry states: auto = where the workload asks for them")
    ap.add_argument("--raw-qk", action="store_true",
                    help="draw q and k unnormalised and have the kernels normalise them (GDN_OPT_L2NORM_QK)")
    ap.add_argument("--events", choices=("nofence", "torch"), default="nofence",
                    help="timing events: HIP events without the system-scope fence (default), or torch's")
    ap.add_argument("--decode", action="store_true",
                    help="measure the recurrent decode step (gdn_decode) on a batch of 256 sequences instead")
    ap.add_argument("--section-stamps", action="store_true",
                    help="cycles per section of the spine's step from the profiling build (not a timing run)")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="the achievable HBM rate of each kernel's read:write mix (profiling build's streaming kernel)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB mebibytes (three times), to "
                         "calibrate the FETCH_SIZE / WRITE_SIZE counters against known bytes")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        # the same copy timed at steady clocks: the achievable read+write rate
        for _ in range(20):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        print(json.dumps({"copy_bytes_per_launch": n * 4, "launches": 43,
                          "copy_ms": round(ms, 4), "copy_GBps_read_plus_write": round(2 * n * 4 / ms / 1e6, 1)}),
              flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (--gpus {args.gpus} "
              f"requested); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.decode:
        bench_decode(args)
        return
    if args.section_stamps:
        section_stamps(args)
        return
    if args.stream_ceiling:
        stream_ceiling(args)
        return

    from linear_attention_ssm_chunk_amd import inputs as I
    p = I.make_workload(args.workload, raw_qk=args.raw_qk)
    wname = p.meta["name"] + ("_raw_qk" if args.raw_qk else "")
    flags = workload_flags(p.meta, args.raw_qk, args.entry_states)
    if args.entry_states != "auto":
        wname += f"_entry_{args.entry_states}"

    cpu = None if args.no_cpu_baseline else cpu_baseline(p)

    import torch
    from linear_attention_ssm_chunk_amd.device import DeviceProblem
    kw = dict(flags=flags)
    if p.meta["layout"] == "conv":
        kw["layout"] = "conv"
    elif p.meta["layout"] == "varlen_table":
        kw.update(state="table", ragged=True)
    dp = DeviceProblem(p, **kw)

    # warm-up: W steps, then more untimed steps until 50 ms of GPU time have run
    warm_t0 = time.perf_counter()
    warm_steps = 0
    while True:
        for _ in range(max(args.warmup - warm_steps, 1) if warm_steps < args.warmup else 10):
            dp.run()
            warm_steps += 1
        torch.cuda.synchronize()
        if warm_steps >= args.warmup and time.perf_counter() - warm_t0 >= WARMUP_MIN_S:
            break
    warm_ms = (time.perf_counter() - warm_t0) * 1e3

    stages = sorted(KERNELS)
    stream = torch.cuda.current_stream().cuda_stream  # the stream the stages are launched on
    if args.events == "torch":
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
        rec = lambda e: e.record()  # noqa: E731
    else:
        ev = [[TimingEvent() for _ in range(len(stages) + 1)] for _ in range(args.steps)]
        rec = lambda e: e.record(stream)  # noqa: E731
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        e = ev[s]
        rec(e[0])
        for st in stages:
            dp.run_stage(st)
            rec(e[st])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {st: sum(ev[s][st - 1].elapsed_time(ev[s][st]) for s in range(args.steps)) / args.steps
           for st in stages}
    ms_per_step = wall * 1e3 / args.steps
    tokens = p.n_tokens
    value = tokens / (ms_per_step / 1e3)

    entry = bool(flags & OPT_ENTRY_STATES)
    io, io_total = irreducible(p, entry)
    by, fl = algorithmic(p, flags)
    dom = max(per, key=per.get)
    gbps = lambda b, ms: b / (ms / 1e3) / 1e9  # noqa: E731
    achieved = gbps(io[dom], per[dom])
    kernels = {KERNELS[st]: {"ms": round(per[st], 4), "io_bytes": io[st],
                             "io_GBps": round(gbps(io[st], per[st]), 1),
                             "io_frac": round(gbps(io[st], per[st]) / HBM_PEAK_GBS, 4),
                             "impl_bytes": by[st], "impl_GBps": round(gbps(by[st], per[st]), 1),
                             "impl_frac": round(gbps(by[st], per[st]) / HBM_PEAK_GBS, 4),
                             "mfma_frac": round(fl[st] / (per[st] / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
               for st in stages}
    total_bytes = sum(by.values())
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "warmup_ms": round(warm_ms, 1),
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wname, "B": p.nseq, "T": max(p.lengths), "n_tokens": tokens, "nk": p.nk,
                   "nv": p.nv, "dk": 128, "dv": 128, "chunk": 64, "global_batch": p.nseq,
                   "seq_len": max(p.lengths), "parallelism": "single_gpu", "entry_states": entry,
                   "qk_normalised_in_kernels": bool(flags & OPT_L2NORM_QK)},
        "roofline": {"bound": "hbm", "kernel": KERNELS[dom], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(dom, wname), "bytes_per_launch": io[dom],
                     "bytes": "irreducible: q and k once per k-head, v, o, entry states where asked for, "
                              "state in and out",
                     "impl_bytes_per_launch": by[dom],
                     "impl_frac": round(gbps(by[dom], per[dom]) / HBM_PEAK_GBS, 4)},
        "kernels": kernels,
        "timing_events": "HIP, no system-scope fence" if args.events == "nofence" else "torch (default HIP events)",
        "whole_step": {"io_bytes": io_total, "io_GBps": round(gbps(io_total, ms_per_step), 1),
                       "io_frac": round(gbps(io_total, ms_per_step) / HBM_PEAK_GBS, 4),
                       "impl_bytes": total_bytes, "impl_GBps": round(gbps(total_bytes, ms_per_step), 1),
                       "mfma_frac": round(sum(fl.values()) / (ms_per_step / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
