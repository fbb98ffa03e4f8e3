#!/usr/bin/env python3
"""Benchmark of the batched paged MLA decode on one MI355X.

One step = one mla_decode call (split-KV kernel + LSE combine) over the
whole batch of the DeepSeek-style decode workload: 64 requests, 1 query
token, 128 heads, 576-wide bf16 latent rows in 64-token pages, sequence
lengths uniform in [1024, 4096], scattered block tables, N(0,1) values.
Inputs are generated on the host once and copied to the GPU before the
timed region.  To keep the KV pool from being served by the 256 MB
last-level cache instead of HBM, the timed steps rotate over several
device copies of the pool and the query (together at least --rotate-gib).

Prints one JSON line (see the keys below).  --gpus above 1 is refused: the
decode runs on one GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode KV-cache GB/s + TFLOPS (% of HBM/MFMA roofline), 128 heads bf16"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense fp8


# Timing-only events: no system-scope fence (cache writeback and invalidate)
# when the event completes.  With the default flags, three events per step add
# about 9 us to a 73 us step; two of these around the split kernel add about 1 us.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """Timing-only hipEvent_t handles through the HIP runtime already loaded by torch."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(int(stream.cuda_stream))) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, ev):
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def cpu_baseline(inp, budget_s: float = 10.0, rg=None):
    """The CPU oracle on the host cores over a bounded sample of the same workload:
    whole requests (all query rows) in batch order, cycling through the batch
    again if it is done early, until about budget_s seconds of oracle work (at
    least one request).  rg: the ragged packing of inp, if the workload has one."""
    import numpy as np
    import oracle
    from oracle import ragged as oracle_ragged
    import paged_mla_decode_06_amd as mla
    orc = oracle.default()
    kv_bytes = 1 if inp.kv_fp8 else 2
    done, t_total = 0, 0.0
    while done == 0 or t_total < budget_s:
        b = done % inp.batch
        t0 = time.perf_counter()
        if rg is None:
            orc.decode_rows(inp, [(b, j, h) for j in range(inp.q_len) for h in range(inp.heads)])
        else:
            oracle_ragged.decode_rows(orc, rg, [(t, h) for t in range(int(rg.qo_indptr[b]), int(rg.qo_indptr[b + 1]))
                                                for h in range(inp.heads)])
        t_total += time.perf_counter() - t0
        done += 1
    idx = np.arange(done) % inp.batch
    lens = np.asarray(inp.seq_lens)[idx]
    if rg is None:
        nbytes, _ = mla.algorithmic_work(lens, inp.q_len, inp.heads, inp.page_size, kv_bytes)
    else:
        nbytes, _ = mla.algorithmic_work_ragged(lens, rg.q_lens[idx], inp.heads, inp.page_size, kv_bytes)
    passes = f", {done / inp.batch:.2f} passes over the batch" if done > inp.batch else ""
    q_tokens = int(np.sum(rg.q_lens[idx])) if rg is not None else done * inp.q_len
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": orc.threads(), "kind": "oracle",
            "seconds": round(t_total, 3), "decode_tokens_per_s": round(q_tokens / t_total, 3),
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model,
            "sample": f"{done} whole requests in batch order{passes} (all their query rows, "
                      f"{int(lens.sum())} cached tokens), fp64 C oracle, OpenMP over query rows; "
                      f"rate = the sample's algorithmic bytes / its time"}


def time_kv_append(ev, stream, pool, rows, locs, k_scale: float, kv_bytes: int, reps: int = 200):
    """Mean duration of one mla_kv_append launch (HIP events around `reps`
    back-to-back launches on `stream`, after 20 untimed ones) writing rows
    [T, 576] bf16 at flat slots locs into pool, and its HBM roofline."""
    import torch
    import paged_mla_decode_06_amd as mla
    nope, rope = rows[:, :512], rows[:, 512:]
    p = mla.make_append_params(rows.shape[0], pool.shape[1], pool.shape[0],
                               mla.MLA_KV_FP8_E4M3FN if kv_bytes == 1 else mla.MLA_KV_BF16, k_scale,
                               rows.stride(0), rows.stride(0))
    for _ in range(20):
        mla.mla_kv_append(nope, rope, locs, pool, stream=stream, params=p)
    a, b = ev.create(), ev.create()
    ev.record(a, stream)
    for _ in range(reps):
        mla.mla_kv_append(nope, rope, locs, pool, stream=stream, params=p)
    ev.record(b, stream)
    torch.cuda.synchronize()
    us = ev.elapsed_ms(a, b) * 1e3 / reps
    ev.destroy(a)
    ev.destroy(b)
    nbytes = mla.append_work(rows.shape[0], kv_bytes)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"rows": int(rows.shape[0]), "us": round(us, 3), "bytes": nbytes, "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "mla_append_kernel"}


def kernel_sources_sha256() -> str:
    """Hash of the sources the split kernel is built from (counter summaries name it)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_mla_decode_06_amd", "csrc")
    for name in ("mla_kernels.hip", "mla_plan.h", "mla_args.h", "mla_rope.h", "mla_fp8.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, "paged_mla_decode_06_amd", "build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, whole_call: bool = False):
    """HBM bytes per split-kernel launch (whole_call: split and combine kernels
    together) from the committed counter summary of this workload, or None
    when there is none or it was taken on other sources."""
    path = os.path.join(ROOT, "profiles", f"mla_split_kernel.{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    try:
        t = int(fields["traffic_bytes_per_launch"])
        if whole_call:
            t += int(fields["combine_read_bytes_per_launch"]) + int(fields["combine_write_bytes_per_launch"])
        return t
    except (KeyError, ValueError):
        return None


def copy_calibration(nbytes: int, reps: int):
    """A plain copy kernel of known size (torch's elementwise mul by 1 over float32),
    run under rocprofv3 --pmc to scale FETCH_SIZE / WRITE_SIZE to bytes."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n * 4, "bytes_written": n * 4, "reps": reps,
                                           "kernel": "torch elementwise mul (float32, out=)"}}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first; a few hundred let the GPU clocks settle")
    ap.add_argument("--workload", default="deepseek_decode")
    ap.add_argument("--rotate-gib", type=float, default=1.5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0)
    ap.add_argument("--quantize-q-fp8", action="store_true",
                    help="fp8 pool: cast the query to e4m3fn in the kernel and take fp8 score products")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy kernel of known size (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the decode runs on one GPU "
              f"(across GPUs the requests would shard with no exchange between them)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(1 << 30, 3)
        return

    import numpy as np
    import torch
    import paged_mla_decode_06_amd as mla
    from mla_synth import generate, ragged, WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    inp = generate(w)
    kv_bytes = 1 if inp.kv_fp8 else 2
    q8 = bool(args.quantize_q_fp8)
    if q8 and not inp.kv_fp8:
        print("bench.py: --quantize-q-fp8 needs a workload with an fp8 pool", file=sys.stderr)
        sys.exit(2)
    profile_name = w.name + ("_q8" if q8 else "")
    # a ragged batch (per-request query lengths) runs through mla_decode_ragged
    rg = ragged(inp) if w.ragged_q else None
    q_lens = rg.q_lens if rg is not None else np.full(inp.batch, inp.q_len, dtype=np.int32)
    if rg is not None:
        nbytes, flops = mla.algorithmic_work_ragged(inp.seq_lens, q_lens, inp.heads, inp.page_size, kv_bytes)
    else:
        nbytes, flops = mla.algorithmic_work(inp.seq_lens, inp.q_len, inp.heads, inp.page_size, kv_bytes)
    q_rows = int(q_lens.sum())    # query tokens of the step

    # device inputs, rotated over enough copies to exceed the last-level cache
    q0 = torch.from_numpy((rg.q if rg is not None else inp.q).view(np.int16)).view(torch.bfloat16).to(dev)
    if inp.kv_fp8:
        pool0 = torch.from_numpy(inp.pool).view(torch.float8_e4m3fn).to(dev)
    else:
        pool0 = torch.from_numpy(inp.pool.view(np.int16)).view(torch.bfloat16).to(dev)
    per_copy = pool0.numel() * pool0.element_size() + q0.numel() * 2
    copies = max(2, math.ceil(args.rotate_gib * (1 << 30) / per_copy))
    qs = [q0] + [q0.clone() for _ in range(copies - 1)]
    pools = [pool0] + [pool0.clone() for _ in range(copies - 1)]
    bt = torch.from_numpy(inp.block_table).to(dev)
    sl = torch.from_numpy(inp.seq_lens).to(dev)
    out = torch.empty((q_rows, inp.heads, 512) if rg is not None else (inp.batch, inp.q_len, inp.heads, 512),
                      dtype=torch.bfloat16, device=dev)
    lse = torch.empty(out.shape[:-1], dtype=torch.float32, device=dev)
    p = mla.make_params(inp.batch, inp.q_len, inp.heads, inp.page_size, inp.num_pages, inp.block_table.shape[1],
                        inp.max_seq_len, mla.MLA_KV_FP8_E4M3FN if inp.kv_fp8 else mla.MLA_KV_BF16,
                        inp.softmax_scale, inp.k_scale, min_work_units=w.min_work_units, quantize_q_fp8=int(q8))
    ws = mla.alloc_workspace(p, dev)
    stream = torch.cuda.current_stream()
    ind = torch.from_numpy(rg.qo_indptr).to(dev) if rg is not None else None

    # Every fourth timed step (every step when fewer than 8 are timed) records
    # two events on the stream both kernels run on: before the split kernel
    # and after it.  The split kernel's duration is (start, split end) of its
    # own step; the GPU time of a whole call, combine and the gaps included,
    # is (start, next sampled start) over the steps between them.  A ragged
    # call is bracketed as a whole (split kernel and combine).  Event records
    # take GPU time of their own (DeepSeek workload: 71.4 us a step with none,
    # 73.6 with two on every step, 76.9 with a third after the combine), hence
    # the sampling and no event after the combine.
    ev = HipEvents()
    every = 4 if args.steps >= 8 else 1
    sampled = list(range(0, args.steps, every))
    events = {k: (ev.create(), ev.create()) for k in sampled}

    def step(i, e0, e1):
        if rg is None:
            mla.mla_decode_timed(p, qs[i % copies], pools[i % copies], bt, sl, out, lse, ws, stream, e0, e1, None)
            return
        if e0 is not None:
            ev.record(e0, stream)
        mla.mla_decode_ragged(qs[i % copies], ind, pools[i % copies], bt, sl, out, lse, ws, max_q_len=inp.q_len,
                              max_seq_len=inp.max_seq_len, softmax_scale=inp.softmax_scale, stream=stream, params=p)
        if e1 is not None:
            ev.record(e1, stream)

    for i in range(args.warmup):
        step(i, None, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k, *events.get(k, (None, None)))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    split_ms = float(np.mean([ev.elapsed_ms(a, b) for a, b in events.values()]))
    spans = [(ev.elapsed_ms(events[a][0], events[b][0]), b - a) for a, b in zip(sampled, sampled[1:])]
    gpu_step_ms = sum(t for t, _ in spans) / sum(n for _, n in spans) if spans else float("nan")
    # the whole call, split kernel to the next call's start (a single sampled
    # step has no next start: its split kernel alone then)
    call_ms = gpu_step_ms if spans else split_ms
    for e in events.values():
        for x in e:
            ev.destroy(x)
    assert torch.isfinite(out.float()).all().item(), "non-finite output"

    # The KV-cache append that precedes each decode step, timed on its own
    # after the decode: the B*q_len new rows into their slots (the newest
    # tokens of each request), and a prefill-sized append of 32768 rows at
    # scattered slots.  Both write into a rotating pool copy the decode no
    # longer uses.
    P = inp.page_size
    new_locs = [int(inp.block_table[b, t // P]) * P + t % P
                for b in range(inp.batch) for t in range(max(int(inp.seq_lens[b]) - int(q_lens[b]), 0),
                                                        int(inp.seq_lens[b]))]
    step_rows = q0.view(-1, 576)[:len(new_locs)]
    step_locs = torch.tensor(new_locs, dtype=torch.int64, device=dev)
    n_big = min(32768, inp.num_pages * P)
    big_locs = torch.from_numpy(np.random.default_rng(99).permutation(inp.num_pages * P)[:n_big].astype(np.int64)).to(dev)
    big_rows = torch.empty((n_big, 576), dtype=torch.bfloat16, device=dev).normal_()
    append_step = time_kv_append(ev, stream, pools[-1], step_rows, step_locs, inp.k_scale, kv_bytes)
    append_big = time_kv_append(ev, stream, pools[-1], big_rows, big_locs, inp.k_scale, kv_bytes)

    gbs = nbytes / (ms_step * 1e-3) / 1e9
    kv_only = int(inp.seq_lens.astype(np.int64).sum()) * 576 * kv_bytes
    # the split kernel's own algorithmic bytes: everything but the output rows
    # and LSEs, which the combine kernel writes for split requests
    split_bytes = nbytes - q_rows * inp.heads * (512 * 2 + 4) if rg is None else nbytes
    split_gbs = split_bytes / (split_ms * 1e-3) / 1e9
    # The binding roofline of the split kernel: HBM when its algorithmic flops
    # per byte are below the ridge (peak flops / peak bandwidth, 312.5 flop/B),
    # else the dense bf16 MFMA peak; the other fraction is reported beside it.
    split_tflops = flops / (split_ms * 1e-3) / 1e12
    hbm_frac = split_gbs / HBM_PEAK_GBS
    # With the query cast to fp8 the score products (576 of every 1088 flops
    # per row and token) run at the fp8 peak and the P.V products at the bf16
    # one: the peak is the flops over the shortest time the two peaks allow.
    mfma_peak = MFMA_BF16_PEAK_TFLOPS
    if q8:
        qk_share = 576.0 / (576.0 + 512.0)
        mfma_peak = 1.0 / (qk_share / MFMA_FP8_PEAK_TFLOPS + (1.0 - qk_share) / MFMA_BF16_PEAK_TFLOPS)
    mfma_frac = split_tflops / mfma_peak
    mfma_bound = flops / split_bytes > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    roofline = {"bound": "mfma" if mfma_bound else "hbm",
                "achieved": round(split_tflops if mfma_bound else split_gbs, 2),
                "peak": round(mfma_peak, 1) if mfma_bound else HBM_PEAK_GBS,
                "unit": "TFLOP/s" if mfma_bound else "GB/s",
                "frac": round(mfma_frac if mfma_bound else hbm_frac, 4),
                "traffic": measured_traffic(profile_name, whole_call=rg is not None),
                "kernel": "mla_split_kernel" if rg is None else "mla_split_kernel + mla_combine_kernel (one call)",
                "algorithmic_bytes_per_launch": split_bytes, "algorithmic_flops_per_launch": flops,
                "hbm_frac": round(hbm_frac, 4), "mfma_frac": round(mfma_frac, 4),
                # the whole decode call (split kernel, combine and the gaps
                # around it): all its algorithmic bytes, output included, over
                # the GPU time from before one call's split kernel to before
                # the next call's
                "call": {"kernels": "mla_split_kernel + mla_combine_kernel", "ms": round(call_ms, 5),
                         "algorithmic_bytes": nbytes,
                         "achieved": round(nbytes / (call_ms * 1e-3) / 1e9, 2), "unit": "GB/s",
                         "frac": round(nbytes / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8_e4m3fn-kv/fp8-q" if q8 else "fp8_e4m3fn-kv/bf16") if inp.kv_fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": inp.batch,
                   "q_len": f"ragged 1..{inp.q_len}" if rg is not None else inp.q_len, "query_tokens": q_rows,
                   "heads": inp.heads,
                   "page_size": inp.page_size, "kv_dtype": w.kv, "seq_lens": f"{w.lens}", "seed": w.seed,
                   "cached_tokens": int(inp.seq_lens.sum()), "num_pages": inp.num_pages,
                   "query": "e4m3fn, cast in the kernel" if q8 else "bf16",
                   "rotating_copies": copies},
        "tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "kv_gbs": round(kv_only / (ms_step * 1e-3) / 1e9, 2),
        "decode_tokens_per_s": round(q_rows / (ms_step * 1e-3), 1),
        "algorithmic_bytes": nbytes,
        "algorithmic_flops": flops,
        # null where a figure does not exist: no GPU step from a single
        # sampled step, and no separate combine time for a ragged call (its
        # events bracket split kernel and combine together)
        "event_ms": {"split_kernel": round(split_ms, 5), "call": round(call_ms, 5),
                     "gpu_step": round(gpu_step_ms, 5) if spans else None,
                     "combine_and_launch_gaps": round(gpu_step_ms - split_ms, 5) if spans and rg is None else None},
        "roofline": roofline,
        "path_frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
        "kv_append": append_step,
        "kv_append_32k_rows": append_big,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget_s, rg)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
