"""Benchmark of the fused causal RoPE-GQA attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama3_8b] [--no-cpu-baseline]
                    [--interleaved] [--non-causal] [--cold]
    python bench.py --ring N | --decode [--batch B] | --backward   (shard composition / decode / backward)

A step is one attn_fwd call (key-rotation pre-pass + fused attention kernel) over the whole
workload, inputs already resident in HBM.  Prints one JSON line:
  value      causal attention TFLOP/s, FLOPs = 2 * B * Hq * S^2 * d (QK^T and PV over the
             visible half of the score matrix), over wall time of K back-to-back steps;
  roofline   the attention kernel alone, against the MI355X dense bf16 MFMA peak (2516.6
             TFLOP/s), timed in a second pass of K steps with HIP events that the runtime
             records with that kernel's dispatch on its stream (the event packets leave the
             GPU idle for ~10 us around the kernel, so the step time is taken without them);
  cpu_baseline the float64 CPU oracle timed on this host on a bounded sample of the same
             workload, in the same unit.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E

CSRC = os.path.join(ROOT, "transformer_causal_attention_amd", "csrc")

# Per-dispatch HBM counters of the attention kernel, from two rocprofv3 --pmc passes (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch) over `bench.py --steps 3 --warmup 1 --no-cpu-baseline`.
# Each is scaled by what the same counter reads for a plain 256 MiB device copy
# (`bench.py --copy-calibration`): the copy moves 262144 KiB each way.  An entry counts only
# while the kernel sources hash to the value it was taken with; otherwise traffic is null.
PMC_SCALE = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
MEASURED_TRAFFIC = {
    "llama3_8b": {"sources_sha256": "861a4383230c4d82", "FETCH_SIZE_KiB": 16617.41, "WRITE_SIZE_KiB": 24848.0},
    "palm_mqa": {"sources_sha256": "861a4383230c4d82", "FETCH_SIZE_KiB": 7366.23, "WRITE_SIZE_KiB": 10504.0},
    "smollm_mha": {"sources_sha256": "861a4383230c4d82", "FETCH_SIZE_KiB": 41396.72, "WRITE_SIZE_KiB": 49898.07},
    "long_shard": {"sources_sha256": "861a4383230c4d82", "FETCH_SIZE_KiB": 1106943.0, "WRITE_SIZE_KiB": 266242.04},
    "palm540b_d256": {"sources_sha256": "a06e174a962e6ba8", "FETCH_SIZE_KiB": 37831.38, "WRITE_SIZE_KiB": 49615.95},
}


def flops(w, rows=None):
    """Causal: 2 * B * Hq * S^2 * d.  For a subset of rows: 4 * d * sum(visible keys)."""
    if rows is None:
        return 2.0 * w.B * w.Hq * w.S * w.S * w.d if w.causal else 4.0 * w.B * w.Hq * w.S * w.S * w.d
    import numpy as np

    vis = (np.asarray(rows) + 1).sum() if w.causal else len(rows) * w.S
    return 4.0 * w.d * float(vis) * w.B * w.Hq


def algorithmic_bytes(w):
    el = 2 if w.dtype == "bf16" else 4
    return (2 * w.B * w.S * w.Hq * w.d + 2 * w.B * w.S * w.Hkv * w.d) * el + 4 * w.B * w.Hq * w.S


# The sources each attention kernel is compiled from (head_dim 256 has a kernel of its own).
KERNEL_SOURCES = ("attn_device.h", "attn_fwd_bf16.hip", "attn_fwd_f32.hip")
KERNEL_SOURCES_D256 = ("attn_device.h", "attn_fwd_d256.hip")


def sources_sha256(d=128):
    """Hash of the code (comments and blank space left out) of the sources of the attention kernel
    that runs head_dim d, so that stored counter readings expire when that kernel changes."""
    import hashlib
    import re

    h = hashlib.sha256()
    for name in KERNEL_SOURCES_D256 if d == 256 else KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(w, interleaved=False):
    m = MEASURED_TRAFFIC.get(w.name + ("_interleaved" if interleaved else ""))
    if not m or m["sources_sha256"] != sources_sha256(w.d):
        return None
    return int(1024 * (m["FETCH_SIZE_KiB"] * PMC_SCALE["FETCH_SIZE"] + m["WRITE_SIZE_KiB"] * PMC_SCALE["WRITE_SIZE"]))


def copy_calibration(n_bytes=256 << 20, reps=3):
    """A plain device-to-device copy of known size, the scale for the HBM byte counters."""
    import torch

    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n_bytes, "reps": reps}), flush=True)


_ORACLE_STATE = {}


def _oracle_worker_init(wd, interleaved):
    """Worker process of the CPU baseline: regenerate the seeded inputs once (one BLAS thread)."""
    from transformer_causal_attention_amd.workloads import Workload, make_inputs

    w = Workload(**wd)
    _ORACLE_STATE.update(w=w, qkv=make_inputs(w), interleaved=interleaved)


def _oracle_task(task):
    """One (query head, row block) of batch row 0 through the oracle; returns its FLOPs."""
    from oracle import attention

    h, r0, r1 = task
    w, (q, k, v), il = _ORACLE_STATE["w"], _ORACLE_STATE["qkv"], _ORACLE_STATE["interleaved"]
    g = h // (w.Hq // w.Hkv)
    n = r1 if w.causal else w.S  # causal rows below r1 see keys below r1 only
    attention(q[:1, :n, h:h + 1].double().numpy(), k[:1, :n, g:g + 1].double().numpy(),
              v[:1, :n, g:g + 1].double().numpy(), w.rope_theta, w.causal, rows=list(range(r0, r1)),
              interleaved=il)
    vis = sum(i + 1 for i in range(r0, r1)) if w.causal else (r1 - r0) * w.S
    return 4.0 * w.d * vis


def cpu_baseline(w, budget_s=10.0, interleaved=False, rows_per_task=256):
    """Time the oracle as it stands on the host's cores: one worker process per core of the
    affinity mask, one BLAS thread each, tasks of (query head, block of query rows) of batch row
    0 (heads and rows are independent, so each task is the definition restricted to its rows).
    Tasks are handed out (two per worker in flight) until budget_s of wall time has passed,
    cycling over batch row 0; the row blocks are visited in a spread order so that a partial pass
    samples every part of the sequence.  value = FLOPs of the finished tasks / wall time."""
    import dataclasses
    import multiprocessing as mp
    from collections import deque

    cores = len(os.sched_getaffinity(0))
    n_blk = (w.S + rows_per_task - 1) // rows_per_task
    step = max(1, int(round(n_blk * 0.6180339887)))
    while n_blk > 1 and np_gcd(step, n_blk) != 1:
        step += 1
    blocks = [(i * step) % n_blk for i in range(n_blk)]
    tasks = [(h, b * rows_per_task, min(w.S, (b + 1) * rows_per_task)) for b in blocks for h in range(w.Hq)]
    workers = max(1, min(cores, len(tasks)))
    env_keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k_: os.environ.get(k_) for k_ in env_keys}
    for k_ in env_keys:
        os.environ[k_] = "1"  # inherited by the spawned workers only (this process's BLAS is set up)
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers, initializer=_oracle_worker_init,
                      initargs=(dataclasses.asdict(w), interleaved)) as pool:
            pool.map(_oracle_task, [(0, 0, 1)] * (2 * workers), chunksize=1)  # imports, first touch
            pending, fl, done, ti = deque(), 0.0, 0, 0
            t0 = time.perf_counter()
            while True:
                while len(pending) < 2 * workers and time.perf_counter() - t0 < budget_s:
                    pending.append(pool.apply_async(_oracle_task, (tasks[ti % len(tasks)],)))
                    ti += 1
                if not pending:
                    break
                fl += pending.popleft().get()
                done += 1
            elapsed = time.perf_counter() - t0
    finally:
        for k_, v_ in saved.items():
            if v_ is None:
                os.environ.pop(k_, None)
            else:
                os.environ[k_] = v_
    passes, rest = divmod(done, len(tasks))
    sample = f"batch row 0 of {w.name} ({w.Hq} query heads x {w.S} rows in tasks of {rows_per_task} rows): "
    sample += f"{passes} whole passes" + (f" and {rest} of {len(tasks)} tasks of one more" if rest else "")
    return {"value": fl / elapsed / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle", "sample": sample,
            "seconds": round(elapsed, 3), "host_cores": cores, "blas_threads_per_worker": 1,
            "workers": workers}


def np_gcd(a, b):
    while b:
        a, b = b, a % b
    return a


def ring_bench(args):
    """Causal attention over the workload's sequence split into args.ring shards: every query
    shard against every key shard at or before it (attn_fwd with q_pos0 / k_pos0), joined by
    attn_merge, as the ranks of a ring would compute it, here one after another on one GPU.
    Also times the merge kernel alone against the HBM bandwidth."""
    import torch

    from transformer_causal_attention_amd import attn_fwd_into, attn_merge, workspace_bytes
    from transformer_causal_attention_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    n_sh = args.ring
    if w.S % n_sh or not w.causal:
        raise SystemExit("--ring needs a causal workload whose S is a multiple of the shard count")
    n = w.S // n_sh
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_inputs(w))
    qs = [q[:, i * n:(i + 1) * n].contiguous() for i in range(n_sh)]
    ks = [k[:, i * n:(i + 1) * n].contiguous() for i in range(n_sh)]
    vs = [v[:, i * n:(i + 1) * n].contiguous() for i in range(n_sh)]
    acc = [(torch.empty_like(qs[0]), torch.empty((w.B, w.Hq, n), dtype=torch.float32, device=dev)) for _ in range(n_sh)]
    part = (torch.empty_like(qs[0]), torch.empty((w.B, w.Hq, n), dtype=torch.float32, device=dev))
    ws = torch.empty(max(1, workspace_bytes(w.B, n, w.Hkv, w.d, 0 if w.dtype == "bf16" else 1)),
                     dtype=torch.uint8, device=dev)

    def step():
        for s in range(n_sh):
            for t in range(s + 1):  # later key shards would only give empty rows
                dst = acc[s] if t == 0 else part
                attn_fwd_into(qs[s], ks[t], vs[t], w.rope_theta, True, dst[0], dst[1], workspace=ws,
                              q_pos0=s * n, k_pos0=t * n)
                if t:
                    attn_merge(acc[s][0], acc[s][1], part[0], part[1], out=acc[s][0], lse=acc[s][1])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # the merge kernel alone, back to back (in place into one accumulator)
    reps = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        attn_merge(acc[0][0], acc[0][1], part[0], part[1], out=acc[0][0], lse=acc[0][1])
    e1.record()
    torch.cuda.synchronize()
    merge_ms = e0.elapsed_time(e1) / reps
    esz = 2 if w.dtype == "bf16" else 4
    merge_bytes = 3 * w.B * n * w.Hq * w.d * esz + 3 * w.B * w.Hq * n * 4  # read 2 parts, write 1
    fl = flops(w)
    value = fl / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    res = {
        "metric": f"ring-composed causal RoPE-GQA attn fwd TFLOP/s ({n_sh} shards on one GPU)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0, sigma) q/k/v)",
        "config": {"workload": f"{w.name}: B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d} "
                               f"rope_theta={w.rope_theta:g} causal={w.causal}, {n_sh} shards of {n}",
                   "shard_calls_per_step": n_sh * (n_sh + 1) // 2,
                   "merges_per_step": n_sh * (n_sh - 1) // 2,
                   "pct_peak": round(100.0 * value / peak, 2)},
        "merge": {"bound": "hbm", "kernel_ms": round(merge_ms, 5), "bytes": merge_bytes,
                  "achieved": round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                  "unit": "GB/s", "frac": round(merge_bytes / (merge_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
    }
    print(json.dumps(res), flush=True)


def decode_bench(args):
    """Decode steps over a full key/value cache: each step appends the newest key (attn_kv_prepare
    re-prepares its 64-key tile) and attends one query per (batch row, head) at position S - 1 to
    all S cached keys (attn_decode).  HBM-bound: the step reads every cached key and value once.
    The rate is algorithmic bytes (cached K and V of the visible keys, q, out, lse) per second."""
    import torch

    from transformer_causal_attention_amd import attn_decode, decode_workspace_bytes, kv_prepare, new_kv_cache
    from transformer_causal_attention_amd.workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    if args.batch:
        w = w.with_(B=args.batch)
    if w.dtype != "bf16":
        raise SystemExit("the decode path is bf16 only")
    B, S, Hq, Hkv, d = w.B, w.S, w.Hq, w.Hkv, w.d
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(int(w.seed))
    k = (torch.randn((B, S, Hkv, d), generator=g, device=dev) * w.sigma).to(torch.bfloat16)
    v = (torch.randn((B, S, Hkv, d), generator=g, device=dev) * w.sigma).to(torch.bfloat16)
    q = (torch.randn((B, Hq, d), generator=g, device=dev) * w.sigma).to(torch.bfloat16)
    cache = new_kv_cache(B, S, Hkv, d, dev)
    kv_prepare(k, v, w.rope_theta, 0, S, cache)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(decode_workspace_bytes(B, Hq, Hkv, d), dtype=torch.uint8, device=dev)
    pos = S - 1

    def step():
        kv_prepare(k, v, w.rope_theta, pos, pos + 1, cache)
        attn_decode(q, cache, S, Hkv, w.rope_theta, pos, out=out, lse=lse, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # attn_decode alone (split kernel + join kernel), back to back between two events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        attn_decode(q, cache, S, Hkv, w.rope_theta, pos, out=out, lse=lse, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    decode_ms = e0.elapsed_time(e1) / args.steps
    nbytes = 2 * B * Hkv * (pos + 1) * d * 2 + 2 * B * Hq * d * 2 + 4 * B * Hq
    achieved = nbytes / (decode_ms * 1e-3) / 1e9
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": "decode-step attention over a KV cache, algorithmic HBM GB/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, sigma) q/k/v)",
        "config": {"workload": f"decode over a full cache: B={B} S_cap={S} q_pos={pos} Hq={Hq} Hkv={Hkv} d={d} "
                               f"rope_theta={w.rope_theta:g}",
                   "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
                   "step": "attn_kv_prepare of the newest tile + attn_decode"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "attn_decode (attn_decode_kernel + attn_decode_join_kernel)",
                     "kernel_ms": round(decode_ms, 5), "algorithmic_bytes": nbytes},
    }
    print(json.dumps(res), flush=True)


def backward_bench(args):
    """Backward steps: attn_bwd (layout passes + dk/dv kernel + dq kernel) over the workload,
    from one forward's out and lse, with a seeded output gradient.  FLOPs are the usual
    2.5x the forward's (S recomputed, dP, dV, dK, dQ: five products of the forward's size);
    the kernels execute seven, recomputing S and dP in the dq kernel rather than using atomics."""
    import torch

    from transformer_causal_attention_amd import attn_bwd, attn_fwd, bwd_workspace_bytes
    from transformer_causal_attention_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    if w.dtype != "bf16":
        raise SystemExit("the backward is bf16 only")
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_inputs(w))
    g = torch.Generator(device=dev).manual_seed(int(w.seed) + 1000)
    dout = torch.randn(q.shape, generator=g, device=dev).to(torch.bfloat16)
    out, lse = attn_fwd(q, k, v, w.rope_theta, w.causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(bwd_workspace_bytes(w.B, w.S, w.Hq, w.Hkv, w.d), dtype=torch.uint8, device=dev)

    def step():
        attn_bwd(q, k, v, out, lse, dout, w.rope_theta, w.causal, dq=dq, dk=dk, dv=dv, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / args.steps
    fl = 2.5 * flops(w)
    value = fl / (ms_per_step * 1e-3) / 1e12
    achieved = fl / (call_ms * 1e-3) / 1e12
    res = {
        "metric": "causal RoPE-GQA attention backward TFLOP/s (2.5x forward FLOPs)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0, sigma) q/k/v and output gradient)",
        "config": {"workload": f"{w.name}: B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d} "
                               f"rope_theta={w.rope_theta:g} causal={w.causal}",
                   "pct_peak_bf16": round(100.0 * value / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "attn_bwd (all its launches)",
                     "kernel_ms": round(call_ms, 5)},
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 256 MiB device copy (scale for the rocprofv3 byte counters)")
    ap.add_argument("--ring", type=int, default=0,
                    help="split the sequence into this many shards and time one ring-attention pass "
                         "(shard calls with position offsets + lse merges) on this GPU")
    ap.add_argument("--decode", action="store_true",
                    help="time decode steps (one query per head at position S - 1 over a full KV cache)")
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch size (--decode)")
    ap.add_argument("--backward", action="store_true", help="time the backward pass (attn_bwd)")
    ap.add_argument("--non-causal", action="store_true",
                    help="forward without the causal mask (every key visible; FLOPs 4 * B * Hq * S^2 * d)")
    ap.add_argument("--cold", action="store_true",
                    help="also time the attention kernel with a 512 MiB scratch write before every step "
                         "(evicts the 256 MB last-level cache), reported as roofline.cold")
    ap.add_argument("--interleaved", action="store_true",
                    help="forward with the adjacent-pair rotary form (rope_style ATTN_ROPE_INTERLEAVED)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the attention forward is a single-GPU kernel here "
              "(no collectives, no sharding); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    if args.ring:
        ring_bench(args)
        return
    if args.decode:
        decode_bench(args)
        return
    if args.backward:
        backward_bench(args)
        return

    import torch

    from transformer_causal_attention_amd import Event, attn_fwd_into, workspace_bytes
    from transformer_causal_attention_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    if args.non_causal:
        w = w.with_(causal=False)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in make_inputs(w))
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, workspace_bytes(w.B, w.S, w.Hkv, w.d, 0 if w.dtype == "bf16" else 1)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    il = args.interleaved
    for _ in range(args.warmup):
        attn_fwd_into(q, k, v, w.rope_theta, w.causal, out, lse, workspace=ws, interleaved=il)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        attn_fwd_into(q, k, v, w.rope_theta, w.causal, out, lse, workspace=ws, stream=stream, interleaved=il)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # second pass: the same steps, each with events bound to the attention kernel's dispatch
    evs = [(Event(), Event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        attn_fwd_into(q, k, v, w.rope_theta, w.causal, out, lse, workspace=ws, stream=stream, events=evs[i],
                      interleaved=il)
    torch.cuda.synchronize()
    kernel_ms = sum(a.elapsed_ms(b) for a, b in evs) / args.steps
    cold = None
    if args.cold:
        # third pass: before each step a 512 MiB write replaces the last-level cache's contents, so
        # the attention kernel reads q (and whatever the preparation pass did not just write)
        # from HBM
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        evc = [(Event(), Event()) for _ in range(args.steps)]
        for i in range(args.steps):
            scratch.fill_(i & 0xFF)
            attn_fwd_into(q, k, v, w.rope_theta, w.causal, out, lse, workspace=ws, stream=stream, events=evc[i],
                          interleaved=il)
        torch.cuda.synchronize()
        cold_ms = sum(a.elapsed_ms(b) for a, b in evc) / args.steps
        cold = {"kernel_ms": round(cold_ms, 5),
                "achieved_TFLOPs": round(flops(w) / (cold_ms * 1e-3) / 1e12, 2),
                "hbm_GBps_algorithmic": round(algorithmic_bytes(w) / (cold_ms * 1e-3) / 1e9, 1),
                "flush": "512 MiB device write before each step"}

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    fl = flops(w)
    value = fl / (ms_per_step * 1e-3) / 1e12
    achieved = fl / (kernel_ms * 1e-3) / 1e12
    bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_TFLOPS
    res = {
        "metric": "causal RoPE-GQA attn fwd TFLOP/s (Llama-3-8B, S=2048); % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0, sigma) q/k/v)",
        "config": {"workload": f"{w.name}: B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} d={w.d} "
                               f"rope_theta={w.rope_theta:g} causal={w.causal}"
                               + (" rope=interleaved" if il else ""),
                   "global_batch": w.B, "seq_len": w.S, "parallelism": "single GPU",
                   "pct_peak_bf16": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
                   "hbm_GBps_algorithmic": round(algorithmic_bytes(w) / (ms_per_step * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "mfma" if bf16 else "alu", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": measured_traffic(w, il) if w.causal else None,
                     "kernel": ("attn_fwd_d256_kernel" if w.d == 256 else "attn_fwd_bf16_kernel") if bf16
                     else "attn_fwd_f32_kernel",
                     "kernel_ms": round(kernel_ms, 5), "algorithmic_bytes": algorithmic_bytes(w),
                     "sources_sha256": sources_sha256(w.d),
                     "hbm_GBps_algorithmic": round(algorithmic_bytes(w) / (kernel_ms * 1e-3) / 1e9, 1)},
    }
    if cold is not None:
        res["roofline"]["cold"] = cold
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, interleaved=il)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
