"""Throughput of the multi-LoRA adapter execution unit on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

Default workload: decode-shaped q_proj, 4096x4096 fp16 base, 6 adapters of
rank 16 (alpha 32) in an HBM pool, 64 tokens per call with 10% base_only.  A
step is one lora_apply over one batch: routing, shrink, base GEMM with the
fused expand, separate expand.  Inputs are resident in HBM before timing.
To keep the 256 MB last-level cache from serving the 32 MiB base weight,
steps rotate over 16 independent (W, pool, x, idx, y) copies (>= 512 MiB).

Other workloads: sweep<T> (100 adapters r8, Zipf), prefill, stack (the 7B
linear stack), shard_col / shard_row (one GPU's 4096x512 / 512x4096 share of
the decode q_proj under eight-way tensor parallelism).

Prints ONE JSON line: tokens/s over K timed steps (HIP events on the stream
the kernels run on, synchronize on both sides), four more repeats of the same
K steps and their median, the single-call latency of an isolated call, the
roofline of the dominant kernel (its algorithmic bytes or FLOPs over its
average duration, timed by the kernel's own dispatch events in a second pass
of K steps), an achievable-peak calibration (a device copy, a device read and
a large library matmul on the same GPU), and the CPU fp64 oracle timed on the
host cores on a bounded sample of the same workload, plus single-thread oracle
times of the tiny fp32 call and the decode call.
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "multi-LoRA linear tokens/s + % HBM/MFMA roofline, 4096² r=16, batch 1–256"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD published
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}
ESZ = {"f32": 4, "f16": 2, "bf16": 2}
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
CSRC = os.path.join(ROOT, "rank_adapter_gemm_token_amd", "csrc")
# Dominant kernel of each workload and the sources it is compiled from (their
# hash keys the committed counter readings to the code they were taken on).
KERNELS = {
    "decode": ("k_decode_gemm", ["gemm_decode.hip", "epilogue.hpp", "dtype.hpp", "internal.hpp"]),
    "tiled": ("k_gemm_tiled", ["gemm_tiled.hip", "epilogue.hpp", "dtype.hpp", "internal.hpp"]),
    "split": ("k_gemm_lds<64, split>", ["gemm_tiled.hip", "epilogue.hpp", "dtype.hpp", "internal.hpp"]),
    "big": ("k_gemm_lds<256>", ["gemm_tiled.hip", "epilogue.hpp", "dtype.hpp", "internal.hpp"]),
}
REPEATS = 5          # timed repeats of the K steps (the first is `value`)
WARM_S = 0.2         # untimed warm-up before the W warm-up steps, seconds
LATENCY_CALLS = 50   # isolated calls for the single-call latency
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# workload set-up (inputs drawn by the seeded generators, then made resident)
# ----------------------------------------------------------------------------

class Call:
    """One lora_apply of a step, with its algorithmic figures."""

    def __init__(self, pool, x, W, idx, y, T, d_in, d_out, dtype, distinct, ranks, fused_slots):
        self.pool, self.x, self.W, self.idx, self.y = pool, x, W, idx, y
        e = ESZ[dtype]
        self.T, self.d_in, self.d_out = T, d_in, d_out
        r_sum = sum(ranks[s] for s in distinct)
        r_fused = sum(ranks[s] for s in fused_slots)
        # Whole call: W once, x once, y once, A and B of each distinct adapter
        # touched (true rank) once, plus the index array.
        self.call_bytes = d_in * d_out * e + T * (d_in + d_out) * e + r_sum * (d_in + d_out) * e + 4 * T
        # Base GEMM kernel.  Calls of at most 64 tokens (k_decode_gemm, which
        # also runs the shrink; the split sum, the expand and y belong to its
        # epilogue kernel): W, x and the true-rank A rows of every adapter
        # touched.  Larger calls (k_gemm_tiled, whose epilogue adds the fused
        # expand): W, x, y and the B rows of FUSED buckets.
        if T <= 64:
            self.gemm_bytes = d_in * d_out * e + T * d_in * e + r_sum * d_in * e
        else:
            self.gemm_bytes = d_in * d_out * e + T * (d_in + d_out) * e + r_fused * d_out * e
        lora_tokens = int(sum(1 for v in idx.cpu().tolist() if v in ranks))
        self.call_flops = 2 * T * d_in * d_out + 2 * sum(
            ranks.get(int(v), 0) for v in idx.cpu().tolist()) * (d_in + d_out)
        self.gemm_flops = 2 * T * d_in * d_out + 2 * sum(
            ranks[int(v)] for v in idx.cpu().tolist() if int(v) in fused_slots) * d_out
        self.lora_tokens = lora_tokens


def _register(L, pool, lin, stream=None):
    for a in lin.adapters:
        L.lora_set_tenant_quota(pool, a.tenant, 1 << 50)
        L.lora_register(pool, a.slot, a.tenant, a.A.cuda(), a.B.cuda(), a.rank, a.alpha)


def _buckets(idx_cpu, ranks, policy, theta):
    vals, counts = np.unique(idx_cpu.numpy(), return_counts=True)
    distinct = [int(v) for v in vals if int(v) in ranks]
    fused = []
    for v, c in zip(vals, counts):
        v = int(v)
        if v in ranks and (policy == 1 or (policy == 0 and c > theta)):
            fused.append(v)
    return distinct, fused


def build_linear_copies(L, w, lin, copies, policy, theta):
    """`copies` independent (pool, W, x, idx, y) sets for one linear.  theta
    None keeps the library's default policy."""
    out = []
    ranks = {a.slot: a.rank for a in lin.adapters}
    for c in range(copies):
        pool = L.lora_pool_create(lin.d_in, lin.d_out, w.R, w.S, w.T, TDT[w.dtype])
        if theta is not None:
            L.lora_set_policy(pool, policy, theta)
        if c == 0:
            policy, theta = L.lora_get_policy(pool)
            distinct, fused = _buckets(w.idx, ranks, policy, theta)
        _register(L, pool, lin)
        x = w.x[lin.d_in].cuda().contiguous()
        W = lin.W.cuda().contiguous() if c == 0 else out[0].W.clone()
        idx = w.idx.cuda().contiguous()
        y = torch.empty((w.T, lin.d_out), dtype=TDT[w.dtype], device="cuda")
        call = Call(pool, x, W, idx, y, w.T, lin.d_in, lin.d_out, w.dtype, distinct, ranks, fused)
        call.policy, call.theta = policy, theta
        out.append(call)
    return out


def setup(args, L):
    from rank_adapter_gemm_token_amd import workloads as wl
    if args.workload == "decode":
        w = wl.decode()
        calls = build_linear_copies(L, w, w.linears[0], args.copies, args.policy, args.theta)
        steps = [[c] for c in calls]
        desc = ("decode q_proj 4096x4096 fp16, 6 adapters r16 alpha32 in an HBM pool, "
                "64 tokens (10% base_only)")
    elif args.workload.startswith("sweep"):
        T = int(args.workload[len("sweep"):] or 64)
        w = wl.sweep(T)
        calls = build_linear_copies(L, w, w.linears[0], args.copies, args.policy, args.theta)
        steps = [[c] for c in calls]
        desc = "sweep 4096x4096 fp16, 100 adapters r8 alpha16, %d tokens, Zipf(1.1)" % T
    elif args.workload in ("shard_col", "shard_row"):
        kind = args.workload[len("shard_"):]
        w = wl.shard(kind)
        calls = build_linear_copies(L, w, w.linears[0], args.copies, args.policy, args.theta)
        steps = [[c] for c in calls]
        lin = w.linears[0]
        desc = ("shard-%s: one GPU's share of the decode q_proj under 8-way tensor parallelism, "
                "%dx%d fp16, 6 adapters r16 alpha32, 64 tokens (10%% base_only)" % (kind, lin.d_in, lin.d_out))
    elif args.workload == "prefill":
        w = wl.prefill()
        per = [build_linear_copies(L, w, lin, max(1, args.copies // 4), args.policy, args.theta)
               for lin in w.linears]
        steps = [list(s) for s in zip(*per)]
        desc = ("prefill q_proj+v_proj 4096x4096 bf16, 32 adapters r{8,16,32,64} padded to 64, "
                "8 sequences x 512 tokens")
    elif args.workload == "stack":
        w = wl.stack(layers=args.layers)
        step = []
        for lin in w.linears:
            step += build_linear_copies(L, w, lin, 1, args.policy, args.theta)
            lin.W = None
            for a in lin.adapters:
                a.A = a.B = None
        steps = [step]
        desc = ("stack: %d layers x {q,k,v,o 4096x4096; gate,up 4096x11008; down 11008x4096} bf16, "
                "64 adapters r16 alpha32, 256 tokens (Zipf 1.1 + 5%% base_only)" % args.layers)
    else:
        raise SystemExit("unknown workload " + args.workload)
    return w, steps, desc


# ----------------------------------------------------------------------------
# timing
# ----------------------------------------------------------------------------

# Steps of several calls over one batch (prefill's two projections, the
# stack's 224 linears) resolve the token -> adapter routing once per step
# (lora_plan_route) and run every linear on it (lora_apply_routed); a step of
# one call, or calls of at most 64 tokens (whose routing rides the decode
# epilogue), calls lora_apply.  PLAN holds the plan handle when in use.
PLAN = {"handle": None}


def use_plan(steps, per_call):
    return not per_call and len(steps[0]) > 1 and steps[0][0].T > 64


def run_steps(L, steps, n, start=0):
    plan = PLAN["handle"]
    for i in range(start, start + n):
        step = steps[i % len(steps)]
        if plan is not None:
            c0 = step[0]
            L.lora_plan_route(plan, c0.pool, c0.idx, c0.T)
            for c in step:
                L.lora_apply_routed(c.pool, plan, c.x, c.W, c.y)
        else:
            for c in step:
                L.lora_apply(c.pool, c.x, c.W, c.idx, c.T, c.y)


def timed(L, steps, K):
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    run_steps(L, steps, K)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / 1e3


def kernel_profile(L, steps, K):
    """Device time of the dominant kernel per call, from the pair of events
    its own dispatch records (lora_profile_enable), over K more steps."""
    pools = sorted({c.pool for s in steps for c in s})
    per_pool = {}
    for s in steps:
        for c in s:
            per_pool[c.pool] = per_pool.get(c.pool, 0) + 1
    for p in pools:
        L.lora_profile_enable(p, 1, per_pool[p] * (K // len(steps) + 2))
    torch.cuda.synchronize()
    run_steps(L, steps, K)
    torch.cuda.synchronize()
    calls, kernel_ms = 0, 0.0
    for p in pools:
        r = L.lora_profile_read(p)
        calls += r["calls"]
        kernel_ms += r["kernel_ms"]
        L.lora_profile_enable(p, 0)
    return kernel_ms / calls / 1e3


def kernel_hash(kind):
    h = hashlib.sha256()
    for name in KERNELS[kind][1]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def workload_kind(workload):
    """The dominant kernel's kind for a bench workload (the kernel the library
    picks for its call shape, gemm_tiled.hip / gemm_decode.hip)."""
    if workload in ("decode", "shard_col", "shard_row"):
        return "decode"
    if workload.startswith("sweep"):
        return "decode" if int(workload[len("sweep"):] or 64) <= 64 else "split"
    return {"prefill": "big", "stack": "split"}[workload]


def write_counters(workload, fetch_dir, write_dir):
    """profiles/counters.json entry for `workload` from two rocprofv3 --pmc
    runs of its bench command (FETCH_SIZE, WRITE_SIZE; both with
    --copy-calibration-mib 256): the dominant kernel's mean reading per
    dispatch, each scaled by what the same counter reads for the run's 256 MiB
    device copy, as HBM bytes per launch."""
    import csv
    import glob
    kind = workload_kind(workload)
    # k_gemm_lds<dtype, tile width, split, fused shrink>: the split kernel
    # (64-wide tiles, with or without the shrink in its launch) or the
    # 256-wide unsplit one.
    match = {"decode": "k_decode_gemm", "split": "k_gemm_lds<", "big": "k_gemm_lds<"}[kind]
    must = {"decode": "", "split": ", 64, true", "big": ", 256, false"}[kind]

    def read(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit("no counter_collection.csv under " + d)
        vals, copy = [], []
        for f in files:
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"])
                if "copyBuffer" in r["Kernel_Name"]:
                    copy.append(v)
                elif match in r["Kernel_Name"] and must in r["Kernel_Name"]:
                    vals.append(v)
        if not vals or not copy:
            raise SystemExit("no %s readings for the kernel or the copy under %s" % (counter, d))
        # the largest copy is the 256 MiB calibration copy
        return sum(vals) / len(vals), len(vals), max(copy)

    f_kib, n_f, f_copy = read(fetch_dir, "FETCH_SIZE")
    w_kib, n_w, w_copy = read(write_dir, "WRITE_SIZE")
    ff, wf = 262144.0 / f_copy, 262144.0 / w_copy
    entry = {"kernel": KERNELS[kind][0], "kernel_sha": kernel_hash(kind),
             "hbm_bytes_per_launch": (f_kib * ff + w_kib * wf) * 1024,
             "fetch_kib_per_launch": f_kib, "write_kib_per_launch": w_kib,
             "fetch_factor": ff, "write_factor": wf, "dispatches": [n_f, n_w]}
    try:
        with open(COUNTERS) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data[workload] = entry
    with open(COUNTERS, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(json.dumps({workload: entry}))


def traffic_for(workload_key, kind):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter readings, if they were taken on the current kernel sources; else
    None."""
    try:
        with open(COUNTERS) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(workload_key)
    if not ent or ent.get("kernel_sha") != kernel_hash(kind):
        return None
    return ent.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on host cores, bounded sample of the same workload
# ----------------------------------------------------------------------------

def _oracle_rate(oracle, x, W, idx, S, ads, cores, seconds):
    """Full oracle calls of one linear on the given token rows for about
    `seconds`: (calls, elapsed s)."""
    oracle.apply(x[:1], W, idx[:1], S, ads, n_threads=cores)  # load + first touch
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.apply(x, W, idx, S, ads, n_threads=cores)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return reps, el


def cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def single_thread_times():
    """Single-thread oracle time per call of the tiny fp32 call (256x256, 16
    tokens) and the decode call (4096x4096 fp16, 64 tokens), in seconds."""
    import oracle
    from rank_adapter_gemm_token_amd import workloads as wl
    out = {}
    for name, w, reps in (("tiny_256x256_f32_T16", wl.tiny(), 200), ("decode_4096x4096_f16_T64", wl.decode(), 1)):
        lin = w.linears[0]
        x = oracle.to_f64(w.x[lin.d_in])
        W = oracle.to_f64(lin.W)
        ads = {a.slot: (oracle.to_f64(a.A), oracle.to_f64(a.B), a.rank, a.alpha) for a in lin.adapters}
        idx = w.idx.numpy()
        oracle.apply(x[:1], W, idx[:1], w.S, ads, n_threads=1)
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.apply(x, W, idx, w.S, ads, n_threads=1)
        out[name] = (time.perf_counter() - t0) / reps
    return out


def cpu_baseline(w, seconds, workload):
    """The fp64 oracle on this host's cores over a bounded sample of the same
    workload, as tokens/s of one bench step (all the step's linears)."""
    import oracle
    from rank_adapter_gemm_token_amd import workloads as wl
    cores = len(os.sched_getaffinity(0))
    idx_all = w.idx.numpy()

    def prep(lin, rows):
        xt = w.x[lin.d_in]
        x = oracle.to_f64(xt[torch.as_tensor(rows, device=xt.device)])
        ads = {a.slot: (oracle.to_f64(a.A), oracle.to_f64(a.B), a.rank, a.alpha) for a in lin.adapters}
        return x, oracle.to_f64(lin.W), idx_all[rows], ads

    if workload == "prefill":
        # Every 16th token (256 of 4096, all eight sequences and their
        # adapters) through both projections; a step is the q+v pair.
        rows = np.arange(0, w.T, 16)
        per_lin = []
        for lin in w.linears:
            x, W, idx, ads = prep(lin, rows)
            reps, el = _oracle_rate(oracle, x, W, idx, w.S, ads, cores, seconds / len(w.linears))
            per_lin.append(el / (reps * len(rows)))
        value = 1.0 / sum(per_lin)
        sample = ("%d of the %d tokens (every 16th) through q_proj and v_proj, fp64, %.1f s"
                  % (len(rows), w.T, seconds))
    elif workload == "stack":
        # 8 tokens through one linear of each shape (layer 0's q_proj, gate_proj,
        # down_proj); a step is 32 layers x (4 q-shaped + 2 gate-shaped + 1
        # down-shaped) linears, all of the same cost per token as the sample's.
        # The bench setup hands the weights to the pools, so the three linears
        # are drawn again from their seeds.
        rows = np.arange(0, w.T, w.T // 8)
        per_tok = 0.0
        for proj, count in ((0, 4), (4, 2), (6, 1)):  # q_proj, gate_proj, down_proj
            lin = wl.stack_linear(0, proj, w.x[4096].device, w.seed, w.S, w.R)
            x, W, idx, ads = prep(lin, rows)
            del lin
            reps, el = _oracle_rate(oracle, x, W, idx, w.S, ads, cores, seconds / 3)
            per_tok += count * el / (reps * len(rows))
        n_layers = len(w.linears) // 7
        value = 1.0 / (n_layers * per_tok)
        sample = ("%d tokens through one q_proj, gate_proj and down_proj (fp64, %.1f s), scaled to the "
                  "%d-linear step" % (len(rows), seconds, len(w.linears)))
    else:
        lin = w.linears[0]
        rows = np.arange(w.T)
        x, W, idx, ads = prep(lin, rows)
        reps, el = _oracle_rate(oracle, x, W, idx, w.S, ads, cores, seconds)
        value = w.T * reps / el
        what = "linear" if lin.name == "linear" else "%s linear" % lin.name
        sample = "%d full calls of the %s (%d tokens each, fp64, %.1f s)" % (reps, what, w.T, el)
    return {"value": value, "unit": "tokens/s", "cores": cores, "kind": "oracle", "sample": sample,
            "cpu_model": cpu_model(), "single_thread_s_per_call": single_thread_times()}


# ----------------------------------------------------------------------------

def device_info():
    """The GPU's name, architecture, compute units and peak engine clock (from
    rocminfo, run as a child process)."""
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hbm_bytes": props.total_memory,
            "max_clock_mhz": None}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        agent, arch = None, None
        for line in out.splitlines():
            t = line.strip()
            if t.startswith("Name:") and "gfx" in t:
                arch = t.split(":", 1)[1].strip()
            if arch and t.startswith("Max Clock Freq. (MHz):"):
                info["max_clock_mhz"] = int(t.split(":", 1)[1].strip())
                break
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    return info


def calibration(dtype):
    """Achievable peaks on this GPU, from the probes in libcalibrate.so: one
    pass of 16-byte non-temporal loads over a 1 GiB buffer (larger than the
    256 MB last-level cache), a register-only loop of 16x16x32 MFMAs in the
    workload's 16-bit type (fp16 for fp32 workloads), every workgroup
    re-reading one 2 MiB window that stays in L2 (the L2-to-CU rate that
    bounds kernels re-streaming an activation block per column tile), each
    the best of a few grid sizes; plus a 1 GiB device-to-device torch copy
    (read + write bytes)."""
    import ctypes
    path = os.path.join(ROOT, "rank_adapter_gemm_token_amd", "libcalibrate.so")
    if not os.path.exists(path):
        log("calibration skipped: %s is not built" % path)
        return None
    lib = ctypes.CDLL(path)
    lib.calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.calib_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.calib_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.calib_mfma_flops.restype = ctypes.c_double
    lib.calib_l2read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def per_launch(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / reps

    def check(rc):
        if rc != 0:
            raise RuntimeError("calibration launch failed: %d" % rc)

    n = 1 << 30
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    read = {}
    for blocks in (1024, 2048, 4096):
        t = per_launch(lambda: check(lib.calib_read(buf.data_ptr(), n, sink.data_ptr(), blocks, sp)), 10)
        read[blocks] = n / t / 1e9
    dst = torch.empty_like(buf)
    t_copy = per_launch(lambda: dst.copy_(buf), 10)
    del buf, dst
    win, l2reps = 2 << 20, 4
    wbuf = torch.ones(win, dtype=torch.uint8, device="cuda")
    l2 = {}
    for blocks in (256, 512, 1024):
        t = per_launch(lambda: check(lib.calib_l2read(wbuf.data_ptr(), win, l2reps, sink.data_ptr(), blocks, sp)), 10)
        l2[blocks] = blocks * l2reps * win / t / 1e9
    del wbuf
    bf = 1 if dtype == "bf16" else 0
    iters = 2000
    mfma = {}
    for blocks in (1024, 2048, 4096):
        t = per_launch(lambda: check(lib.calib_mfma(bf, iters, sink.data_ptr(), blocks, sp)), 5)
        mfma[blocks] = lib.calib_mfma_flops(iters, blocks) / t / 1e12
    torch.cuda.empty_cache()
    return {"read_GBs": max(read.values()), "read_GBs_by_blocks": read,
            "mfma_TFLOPs": max(mfma.values()), "mfma_TFLOPs_by_blocks": mfma,
            "copy_GBs": 2 * n / t_copy / 1e9,
            "l2_read_GBs": max(l2.values()), "l2_read_GBs_by_blocks": l2,
            "what": "libcalibrate.so: 1 GiB read once (16-byte non-temporal loads, grid-stride), "
                    "register-only 16x16x32 %s MFMA loop (8 chains per wave), every workgroup reading "
                    "one 2 MiB window 4 times (16-byte loads, L2-resident; bytes the CUs take in); "
                    "1 GiB torch copy_ (read+write bytes); 10 (5) timed launches after one untimed"
                    % ("bf16" if bf else "f16")}


def single_call_latency(L, steps, n):
    """Device time of one isolated step (GPU idle before it: synchronize,
    event, the step's launches, event, synchronize), median over n."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    dev, host = [], []
    for i in range(n):
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        e0.record(stream)
        run_steps(L, steps, 1, start=i)
        e1.record(stream)
        torch.cuda.synchronize()
        host.append(time.perf_counter() - h0)
        dev.append(e0.elapsed_time(e1) / 1e3)
    dev.sort()
    host.sort()
    return {"device_us_median": 1e6 * dev[n // 2], "host_us_median": 1e6 * host[n // 2], "calls": n,
            "what": "one step after a device synchronize: device time between events around its "
                    "launches, and host time from before the launches to the end of the synchronize"}


def loader_bench(L, args):
    """Adapter load latency through the async loader (lora_load_async): a
    whole-model adapter (rank 16 on the 224 linears of the 7B stack, bf16,
    from ordinary host memory) switched into every linear's pool, and the
    per-linear load latency (async + wait) distribution.  One JSON line."""
    import time
    from rank_adapter_gemm_token_amd import workloads as wl
    r = 16
    rng = np.random.default_rng(7)
    lins = []
    for layer in range(wl.STACK_LAYERS):
        for name, d_in, d_out in wl.STACK_SHAPES:
            A = torch.from_numpy(rng.standard_normal((r, d_in), dtype=np.float32) / np.sqrt(d_in)).to(torch.bfloat16)
            B = torch.from_numpy(rng.standard_normal((d_out, r), dtype=np.float32) * 0.1).to(torch.bfloat16)
            lins.append((d_in, d_out, A.contiguous(), B.contiguous()))
    pools = []
    for d_in, d_out, _, _ in lins:
        p = L.lora_pool_create(d_in, d_out, r, 2, 1, torch.bfloat16)
        L.lora_set_tenant_quota(p, 0, 1 << 40)
        pools.append(p)
    cap = max(r * (d_in + d_out) * 2 for d_in, d_out, _, _ in lins)
    ld = L.lora_loader_create(cap)
    total_bytes = sum(r * (d_in + d_out) * 2 for d_in, d_out, _, _ in lins)

    def switch(slot):
        # Unload what the slot held, then load the whole adapter into it.
        for p in pools:
            try:
                L.lora_unregister(p, slot)
            except L.LoraError:
                pass
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tickets = [L.lora_load_async(ld, p, slot, 0, A, B, r, 2.0 * r) for p, (_, _, A, B) in zip(pools, lins)]
        for t in tickets:
            L.lora_load_wait(ld, t)
        return time.perf_counter() - t0

    switch(0)  # warm-up
    whole = [switch(k % 2) for k in range(args.loader_rounds)]
    per = []
    for k in range(2):
        for p, (_, _, A, B) in zip(pools, lins):
            L.lora_unregister(p, k)
            t0 = time.perf_counter()
            t = L.lora_load_async(ld, p, k, 0, A, B, r, 2.0 * r)
            L.lora_load_wait(ld, t)
            per.append(time.perf_counter() - t0)
    # Plain pinned host -> device copy of the same byte count (the link's rate).
    src = torch.empty(total_bytes, dtype=torch.uint8).pin_memory()
    dst = torch.empty(total_bytes, dtype=torch.uint8, device="cuda")
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(5):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    h2d = total_bytes * 5 / (time.perf_counter() - t0) / 1e9
    L.lora_loader_destroy(ld)
    for p in pools:
        L.lora_pool_destroy(p)
    whole_ms = sorted(1e3 * v for v in whole)
    per_ms = sorted(1e3 * v for v in per)
    pct = lambda v, q: v[min(len(v) - 1, int(q * len(v)))]
    out = {"loader": "whole-model adapter switch (rank 16 on 224 linears of the 7B stack, bf16) and "
                     "per-linear loads, host memory -> pool slot via lora_load_async",
           "adapter_bytes": total_bytes, "linears": len(lins), "rounds": len(whole),
           "switch_ms": {"p50": pct(whole_ms, 0.5), "p95": pct(whole_ms, 0.95), "max": whole_ms[-1]},
           "switch_GBs": total_bytes / (whole_ms[len(whole_ms) // 2] / 1e3) / 1e9,
           "per_linear_ms": {"p50": pct(per_ms, 0.5), "p95": pct(per_ms, 0.95), "max": per_ms[-1],
                             "n": len(per_ms)},
           "pinned_h2d_copy_GBs": h2d}
    print(json.dumps(out), flush=True)


def theta_sweep(L, args):
    """The fused/separate sweep on the 100-adapter workload: tokens/s of every
    policy at T in {1, 8, 16, 32, 64}; the threshold whose geometric mean over
    T is highest is the device's threshold.  Prints one JSON line."""
    from rank_adapter_gemm_token_amd import workloads as wl
    policies = [("separate", 2, 16), ("fused", 1, 16)] + [("auto%d" % t, 0, t) for t in (0, 1, 2, 4, 8, 16, 32, 64)]
    table = {}
    for T in wl.SWEEP_T:
        w = wl.sweep(T)
        calls = build_linear_copies(L, w, w.linears[0], args.copies, 0, 16)
        steps = [[c] for c in calls]
        row = {}
        for name, pol, th in policies:
            for c in calls:
                L.lora_set_policy(c.pool, pol, th)
            run_steps(L, steps, args.warmup)
            torch.cuda.synchronize()
            sec = timed(L, steps, args.steps)
            row[name] = T * args.steps / sec
        table[T] = row
        log("T=%d" % T, {k: round(v) for k, v in row.items()})
        for c in calls:
            L.lora_pool_destroy(c.pool)
    gm = {name: float(np.exp(np.mean([np.log(table[T][name]) for T in table]))) for name, _, _ in policies}
    best = max((n for n in gm if n.startswith("auto")), key=lambda n: gm[n])
    print(json.dumps({"sweep": "fused/separate threshold, 4096x4096 fp16, 100 adapters r8, Zipf(1.1)",
                      "unit": "tokens/s", "steps": args.steps, "copies": args.copies,
                      "per_T": {str(T): table[T] for T in table}, "geomean": gm,
                      "best_auto": best, "theta_star": int(best[4:])}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode",
                    help="decode (default) | sweep<T> | prefill | stack | shard_col | shard_row")
    ap.add_argument("--copies", type=int, default=16)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--policy", type=int, default=0, help="0 auto, 1 fused, 2 separate (with --theta)")
    ap.add_argument("--theta", type=int, default=None, help="threshold; default: the library's policy")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true", help="skip the kernel-timing pass")
    ap.add_argument("--no-calibration", action="store_true", help="skip the achievable-peak calibration")
    ap.add_argument("--route-per-call", action="store_true",
                    help="route every call (lora_apply) instead of once per step (lora_plan_route)")
    ap.add_argument("--loader", action="store_true",
                    help="measure adapter load latency through the async loader instead of the bench step")
    ap.add_argument("--loader-rounds", type=int, default=20)
    ap.add_argument("--theta-sweep", action="store_true",
                    help="run the fused/separate threshold sweep instead of the bench step")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the workload's profiles/counters.json entry from two rocprofv3 --pmc "
                         "output directories (FETCH_SIZE, WRITE_SIZE) of its bench command; no GPU")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before warm-up, run two plain device-to-device copies of this many MiB "
                         "(the known-size reference for hardware byte counters)")
    args = ap.parse_args()

    if args.write_counters:
        write_counters(args.workload, *args.write_counters)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    from rank_adapter_gemm_token_amd import lora as L
    if args.theta_sweep:
        theta_sweep(L, args)
        return
    if args.loader:
        loader_bench(L, args)
        return

    w, steps, desc = setup(args, L)
    if use_plan(steps, args.route_per_call):
        PLAN["handle"] = L.lora_plan_create(w.T, w.S)
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log("workload:", desc, "| step sets:", len(steps), "| calls/step:", len(steps[0]))
    # Every rotating copy once (first touch), untimed steps for at least
    # WARM_S seconds (clocks settle: with a few short steps the first timed
    # pass of a sub-millisecond step ran ~10% slow), then the warm-up steps.
    run_steps(L, steps, len(steps))
    t_warm, i_warm = time.perf_counter(), 0
    while True:
        run_steps(L, steps, len(steps), start=i_warm)
        i_warm += len(steps)
        torch.cuda.synchronize()
        if time.perf_counter() - t_warm >= WARM_S:
            break
    run_steps(L, steps, args.warmup)
    torch.cuda.synchronize()
    sec = timed(L, steps, args.steps)
    tokens_per_step = w.T
    value = tokens_per_step * args.steps / sec
    ms_per_step = sec * 1e3 / args.steps
    log("timed: %.3f ms/step, %.0f tokens/s" % (ms_per_step, value))
    rep_ms = [ms_per_step] + [timed(L, steps, args.steps) * 1e3 / args.steps for _ in range(REPEATS - 1)]
    log("repeats ms/step:", ["%.4f" % v for v in rep_ms])
    latency = single_call_latency(L, steps, LATENCY_CALLS if len(steps[0]) == 1 else 3)
    log("single-call latency:", latency)

    calls = steps[0]
    step_bytes = sum(c.call_bytes for c in calls)
    step_flops = sum(c.call_flops for c in calls)
    mfma_bound = args.workload == "prefill"
    roof = None
    if not args.no_profile:
        calls_per_step = len(calls)
        # The dominant kernel's own device time (dispatch timestamps recorded
        # by its launch), averaged over the K calls of the profile pass.
        gemm_s = kernel_profile(L, steps, args.steps)
        if mfma_bound:
            achieved = (sum(c.gemm_flops for c in calls) / calls_per_step) / gemm_s / 1e12
            roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK_TFLOPS[w.dtype],
                    "unit": "TFLOP/s", "frac": achieved / MFMA_PEAK_TFLOPS[w.dtype]}
        else:
            per_launch = sum(c.gemm_bytes for c in calls) / calls_per_step
            achieved = per_launch / gemm_s / 1e9
            roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS}
        kind = workload_kind(args.workload)
        roof["kernel"] = KERNELS[kind][0]
        roof["kernel_us"] = gemm_s * 1e6
        roof["traffic"] = traffic_for(args.workload, kind)

    calib = None
    if not args.no_calibration:
        calib = calibration(w.dtype)
        log("calibration:", calib)
        if roof is not None:
            ach = calib["mfma_TFLOPs"] if roof["bound"] == "mfma" else calib["read_GBs"]
            roof["frac_of_achievable"] = roof["achieved"] / ach

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds, args.workload)
        log("cpu baseline:", cpu)

    # The rank-padding share of the batch's LoRA rows (the shrink and expand
    # skip those rank blocks), from one routed call's pool statistics.
    c0 = steps[0][0]
    L.lora_apply(c0.pool, c0.x, c0.W, c0.idx, c0.T, c0.y)
    st = L.lora_pool_stats(c0.pool)
    zero_pad = {"rows_padded": st["last_lora_rows_padded"], "rows_true": st["last_lora_rows_true"],
                "fraction": st["last_zero_pad_fraction"]}
    log("zero pad:", zero_pad)

    step_s = sec / args.steps
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded generators; 7B-decoder shapes, N(0,1) x, N(0,1/d_in) W and A, "
                "N(0,0.01) B)",
        "config": {"workload": desc, "tokens_per_step": tokens_per_step,
                   "calls_per_step": len(calls), "weight_copies": len(steps),
                   "policy": ["auto", "fused", "separate"][calls[0].policy], "theta": calls[0].theta,
                   "routing": "once per step (lora_plan_route)" if PLAN["handle"] is not None else "per call",
                   "step_bytes_alg": step_bytes, "step_flops_alg": step_flops},
        "step_roofline": {"hbm_GBs": step_bytes / step_s / 1e9,
                          "hbm_frac": step_bytes / step_s / 1e9 / HBM_PEAK_GBS,
                          "mfma_TFLOPs": step_flops / step_s / 1e12,
                          "mfma_frac": step_flops / step_s / 1e12 / MFMA_PEAK_TFLOPS[w.dtype]},
        "roofline": roof,
        "repeats": {"ms_per_step": rep_ms, "median_ms_per_step": float(np.median(rep_ms)),
                    "median_value": tokens_per_step / (float(np.median(rep_ms)) / 1e3)},
        "single_call_latency": latency,
        "calibration": calib,
        "device": device_info(),
        "cpu_baseline": cpu,
        "zero_pad": zero_pad,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
