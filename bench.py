"""Throughput of the chunked gated-delta-rule prefill on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--workload 3]

One step = one gdn_prefill call (both kernels: stage 1, then the spine with the
output fused in) over the whole synthetic workload, inputs resident in HBM.
Default workload: B=4 sequences of T=8192 tokens, nk=16 k-heads, nv=32
v-heads, dk=dv=128, carried float32 state updated in place, per-chunk entry
states emitted.  Prints one JSON line.

Warm-up: the W untimed warm-up steps run first; if they took less than 50 ms
of GPU time, untimed steps continue until 50 ms have passed.  An idle MI355X
sits in a low-power state, and the first ~25 ms of this workload run 5-40 %
slower than the steady state while clocks settle; the timed K steps are then
all at steady state.  The line reports the warm-up actually run
("warmup_steps_run", "warmup_ms").

roofline: the dominant kernel's algorithmic bytes per launch (the byte model
below, per token-head / per slot, times the units one launch processes) over
its average launch time, timed live with HIP events on the launch stream.
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


def algorithmic(p):
    """Per-kernel algorithmic bytes and flops for problem p (inputs.Problem).

    Bytes: every operand each kernel must read or write once (q, k counted once
    per k-head).  Stage 1 reads k, g, beta and writes gc, the decays and T'
    (5 KB per chunk-head); stage 2 reads q, k, v, gc, the decays, T' and the
    state, and writes the entry states (32 KB per chunk-head), o and the state.
    Flops: the dense-tile MFMA work per chunk-head of what each kernel computes
    (Gram in stage 1; K h, T' R, K^T uc, Q h, the scores Q K^T and A uc in
    stage 2), each product counted once."""
    N, nk, nv = p.n_tokens, p.nk, p.nv
    slots = int(p.cu_chunks[-1]) * nv
    nseq = p.nseq
    d, C = 128, 64
    k_bytes = N * nk * d * 2
    q_bytes = N * nk * d * 2
    v_bytes = N * nv * d * 2
    gb_bytes = N * nv * 8
    gc_bytes = slots * C * 4
    dec_bytes = slots * 2 * C * 4
    tp_bytes = slots * 2560 * 2  # 2560 float16
    s_bytes = slots * d * d * 2
    state_bytes = nseq * nv * d * d * 4
    o_bytes = N * nv * d * 2
    by = {
        1: k_bytes + gb_bytes + gc_bytes + dec_bytes + tp_bytes,
        2: q_bytes + k_bytes + v_bytes + gc_bytes + dec_bytes + tp_bytes + 2 * state_bytes + s_bytes + o_bytes,
    }
    fl = {1: slots * (2 * C * C * d),
          2: slots * (6 * C * d * d + 6 * C * C * d)}
    return by, fl


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
    from oracle import gdn_recurrence, kv_head_map
    from linear_attention_ssm_chunk_amd.inputs import bf16_to_f64
    p = _SAMPLE_PROBLEM
    kmap = kv_head_map(p.nk, p.nv)
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
        "kind": "oracle",
        "sample": (f"{workers} workers (one BLAS thread each) running (sequence, v-head) chains of this "
                   f"workload through the float64 token recurrence for {seconds_per_worker}s each: "
                   f"{token_heads} token-heads, {cpu_s:.1f} core-s, wall {wall:.1f}s; "
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
    from oracle import gdn_recurrence, kv_head_map
    from linear_attention_ssm_chunk_amd.inputs import bf16_to_f64
    p = _SAMPLE_PROBLEM
    kmap = kv_head_map(p.nk, p.nv)
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        chain = w
        while time.perf_counter() - t0 < seconds:
            i, h = chain % p.nseq, (chain // p.nseq) % p.nv
            kap = kmap[[h]]
            gdn_recurrence(bf16_to_f64(p.q[i:i + 1][:, kap]), bf16_to_f64(p.k[i:i + 1][:, kap]),
                           bf16_to_f64(p.v[i:i + 1][:, [h]]), p.g[i:i + 1][:, [h]].astype("float64"),
                           p.beta[i:i + 1][:, [h]].astype("float64"), p.h0[i][[h]].astype("float64"))
            done += 1
            chain += workers
    return done, time.perf_counter() - t0


def bench_decode(args):
    import multiprocessing as mp
    global _SAMPLE_PROBLEM
    from linear_attention_ssm_chunk_amd import inputs as I
    sh = DECODE_SHAPE
    p = I.make_problem([1] * sh["B"], sh["nk"], sh["nv"], seed=6)
    cpu = None
    if not args.no_cpu_baseline:
        _SAMPLE_PROBLEM = p
        workers = max(1, min(16, os.cpu_count() or 1))
        t0 = time.perf_counter()
        with mp.get_context("fork").Pool(workers) as pool:
            res = pool.map(_oracle_decode_worker, [(w, workers, 1.5) for w in range(workers)])
        wall = time.perf_counter() - t0
        heads = sum(r[0] for r in res)
        cpu = {"value": heads / wall / p.nv, "unit": "tokens/s", "cores": workers, "kind": "oracle",
               "sample": (f"{workers} workers (one BLAS thread each) running single-token steps of this batch's "
                          f"(sequence, v-head) pairs through the float64 recurrence for 1.5 s each: {heads} "
                          f"head-steps, wall {wall:.1f}s; tokens/s = head-steps/s / nv")}
    import torch
    from linear_attention_ssm_chunk_amd.device import DeviceProblem
    dp = DeviceProblem(p, ragged=False)
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
                   "tokens_per_sequence": 1},
        "roofline": {"bound": "hbm", "kernel": "recurrent_decode", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for_decode()},
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="measure the recurrent decode step (gdn_decode) on a batch of 256 sequences instead")
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

    from linear_attention_ssm_chunk_amd import inputs as I
    p = I.make_workload(args.workload)
    wname = p.meta["name"]

    cpu = None if args.no_cpu_baseline else cpu_baseline(p)

    import torch
    from linear_attention_ssm_chunk_amd.device import DeviceProblem
    kw = {}
    if p.meta["layout"] == "conv":
        kw = dict(layout="conv")
    elif p.meta["layout"] == "varlen_table":
        kw = dict(state="table", ragged=True)
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
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        e = ev[s]
        e[0].record()
        for st in stages:
            dp.run_stage(st)
            e[st].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {st: sum(ev[s][st - 1].elapsed_time(ev[s][st]) for s in range(args.steps)) / args.steps
           for st in stages}
    ms_per_step = wall * 1e3 / args.steps
    tokens = p.n_tokens
    value = tokens / (ms_per_step / 1e3)

    by, fl = algorithmic(p)
    dom = max(per, key=per.get)
    achieved = by[dom] / (per[dom] / 1e3) / 1e9
    kernels = {KERNELS[st]: {"ms": round(per[st], 4), "alg_bytes": by[st],
                             "alg_GBps": round(by[st] / (per[st] / 1e3) / 1e9, 1),
                             "hbm_frac": round(by[st] / (per[st] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
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
                   "seq_len": max(p.lengths), "parallelism": "single_gpu"},
        "roofline": {"bound": "hbm", "kernel": KERNELS[dom], "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(dom, wname)},
        "kernels": kernels,
        "whole_step": {"alg_bytes": total_bytes,
                       "alg_GBps": round(total_bytes / (ms_per_step / 1e3) / 1e9, 1),
                       "mfma_frac": round(sum(fl.values()) / (ms_per_step / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
