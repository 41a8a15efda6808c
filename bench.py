"""Benchmark of the layerwise QK-Norm hot path on one MI355X.

A step is one fused Q + K launch (sum of squares, 1/rms, gamma scale of both tensors) over one
batch of the OLMo-2-7B-shaped workload: Q and K [8192, 4096] bf16, seeded synthetic inputs
already resident in HBM. Working buffers rotate over >= 1 GiB so that every launch streams
from HBM rather than from the 256 MB Infinity Cache.

Prints ONE JSON line: tokens/s, ms per step, the roofline of the fused kernel (algorithmic
bytes / average launch duration, from HIP events on the launch stream, against 8 TB/s), the
fp64 CPU oracle's rate on a bounded sample of the same workload, and per-workload timings of
the other entry points ("cases").
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 matrix peak, published
METRIC = "fused Q+K QK-Norm tokens/s + achieved HBM GB/s (% of peak), OLMo-7B shape, 1 GPU"
ROTATE_BYTES = 1 << 30
MAX_SETS = 128  # small workloads are latency-bound; their graphs stay a few hundred nodes long
PMC_SUMMARY = os.path.join(ROOT, "profiles", "qknorm_fused_olmo2_7b_T8192_pmc.md")
KERNEL_SOURCES = ["layerwise_qk_norm_amd/csrc/rows_impl.h", "layerwise_qk_norm_amd/csrc/rows_inst.hip",
                  "layerwise_qk_norm_amd/csrc/device.h"]


def rows_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch from the committed counter summary, or None when it is absent or
    was taken on different kernel sources."""
    try:
        text = open(PMC_SUMMARY).read()
    except OSError:
        return None
    m_hash = re.search(r"kernel source hash:\s*`?([0-9a-f]{16})", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != rows_source_hash():
        return None
    return int(m_bytes.group(1))


def fused_bytes(T, dq, dk, es=2, gs=2):
    """Algorithmic bytes of one fused launch: each row read once and written once, gamma once."""
    return T * (dq + dk) * 2 * es + (dq + dk) * gs


class Timer:
    """HIP events recorded on the stream the kernels are launched on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def run(self, fn, iters, warmup, reps=1):
        """ms per call: the median over reps of the mean of iters back-to-back calls."""
        torch = self.torch
        means = []
        with torch.cuda.stream(self.stream):
            for i in range(warmup):
                fn(i)
            torch.cuda.synchronize()
            for _ in range(reps):
                start = torch.cuda.Event(enable_timing=True)
                end = torch.cuda.Event(enable_timing=True)
                start.record(self.stream)
                for i in range(iters):
                    fn(i)
                end.record(self.stream)
                end.synchronize()
                means.append(start.elapsed_time(end) / iters)
        torch.cuda.synchronize()
        return statistics.median(means)

    def run_graph(self, fn, per_graph, replays, warmup, reps=1):
        """The same launches captured into one HIP graph (per_graph calls, one per rotating
        buffer set) and replayed: GPU time per call without the host's launch overhead (the
        median over reps of the mean over replays)."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            for i in range(per_graph):
                fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for i in range(per_graph):
                fn(i)
        means = []
        with torch.cuda.stream(self.stream):
            for _ in range(warmup):
                g.replay()
            torch.cuda.synchronize()
            for _ in range(reps):
                start = torch.cuda.Event(enable_timing=True)
                end = torch.cuda.Event(enable_timing=True)
                start.record(self.stream)
                for _ in range(replays):
                    g.replay()
                end.record(self.stream)
                end.synchronize()
                means.append(start.elapsed_time(end) / (replays * per_graph))
        torch.cuda.synchronize()
        del g
        return statistics.median(means)


def rotation_count(bytes_per_set):
    """Buffer sets so that successive launches sweep >= 1 GiB (capped at MAX_SETS)."""
    return min(MAX_SETS, max(1, -(-ROTATE_BYTES // bytes_per_set)))


def dev(torch, a):
    import numpy as np

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


# ----------------------------------------------------------------------------- workloads
def fused_setup(torch, Q, inputs, workload, T, stream):
    """Rotating buffer sets of one fused workload and a step that launches qknorm_fused on one
    set. The step calls the C entry point with its arguments marshalled once here (the Python
    binding's per-call checks are host work outside the library); the binding is called once
    per set first, so its checks still pass on every argument tuple timed."""
    c = inputs.make_case(workload, T)
    q, k = dev(torch, c["q"]), dev(torch, c["k"])
    gq, gk = dev(torch, c["gamma_q"]), dev(torch, c["gamma_k"])
    es = q.element_size()
    nbytes = fused_bytes(T, q.shape[1], k.shape[1], es, gq.element_size())
    n = rotation_count(2 * T * (q.shape[1] + k.shape[1]) * es)
    sets = [(q.clone(), k.clone(), torch.empty_like(q), torch.empty_like(k)) for _ in range(n)]
    del q, k
    L = Q.lib()
    dt = Q.QKN_BF16 if sets[0][0].dtype == torch.bfloat16 else Q.QKN_F32
    gdt = Q.QKN_BF16 if gq.dtype == torch.bfloat16 else Q.QKN_F32
    dq, dk = sets[0][0].shape[1], sets[0][1].shape[1]
    args = []
    with torch.cuda.stream(stream):
        for qi, ki, qo, ko in sets:
            Q.qknorm_fused(qi, gq, ki, gk, eps=c["eps"], q_out=qo, k_out=ko)
            args.append((T, c["eps"], dt, gdt, qi.data_ptr(), dq, qo.data_ptr(), dq,
                         gq.data_ptr(), dq, ki.data_ptr(), dk, ko.data_ptr(), dk, gk.data_ptr(),
                         dk, stream.cuda_stream))

    def step(i):
        status = L.qknorm_fused(*args[i % n])
        if status:
            raise Q.QknError("qknorm_fused", status, L)

    # the argument tuples hold raw device addresses: the step owns the tensors behind them, so
    # they stay allocated (an emptied allocator cache cannot release them) as long as
    # the step can be called
    step.tensors = (sets, gq, gk)
    step.args = args
    step.sets = n
    return step, nbytes


def shard_setup(torch, Q, inputs, T):
    c = inputs.make_case("tp8-shard", T)
    q, k = dev(torch, c["q"]), dev(torch, c["k"])
    gq, gk = dev(torch, c["gamma_q"]), dev(torch, c["gamma_k"])
    eq, ek = dev(torch, c["ext_q"]), dev(torch, c["ext_k"])
    per_set = 2 * T * 512 * 2 * 2 + 2 * T * 4
    n = rotation_count(per_set)
    sets = []
    for _ in range(n):
        sets.append((q.clone(), k.clone(), torch.empty_like(q), torch.empty_like(k),
                     torch.empty(T, device="cuda"), torch.empty(T, device="cuda")))

    def k1(i):
        qi, ki, _, _, pq, pk = sets[i % n]
        Q.qknorm_partial_sumsq(qi, ki, psq_q=pq, psq_k=pk)

    def k2(i):
        qi, ki, qo, ko, pq, pk = sets[i % n]
        Q.qknorm_apply_with_stats(qi, gq, pq, eq, 4096, ki, gk, pk, ek, 4096, eps=c["eps"],
                                  q_out=qo, k_out=ko)

    # single pass with the mailbox: the peers' partials are published once (epoch 1) before
    # timing, so every pass finds its words tagged and measures the one-pass cost
    mail_q, mail_k = Q.mailbox_words(7, T), Q.mailbox_words(7, T)
    tout = torch.zeros((1,), dtype=torch.int32, device="cuda")
    Q.qknorm_shard_publish(eq, mail_q, 1, ek, mail_k)
    words = [(torch.empty(T, dtype=torch.int64, device="cuda"),
              torch.empty(T, dtype=torch.int64, device="cuda")) for _ in range(n)]

    def k3(i):
        qi, ki, qo, ko, _, _ = sets[i % n]
        wq, wk = words[i % n]
        Q.qknorm_shard_fused(qi, gq, mail_q, 4096, ki, gk, mail_k, 4096, eps=c["eps"], q_out=qo,
                             k_out=ko, psq_q=wq, psq_k=wk, epoch=1, timed_out=tout)

    def k4(i):  # one workgroup per row block: producers on other devices
        qi, ki, qo, ko, _, _ = sets[i % n]
        wq, wk = words[i % n]
        Q.qknorm_shard_fused(qi, gq, mail_q, 4096, ki, gk, mail_k, 4096, eps=c["eps"], q_out=qo,
                             k_out=ko, psq_q=wq, psq_k=wk, epoch=1, timed_out=tout,
                             persistent=False)

    k1.sets = k2.sets = k3.sets = k4.sets = n
    k3.timed_out = k4.timed_out = tout

    b1 = T * 2 * (512 * 2 + 4)
    b2 = T * 2 * (512 * 2 * 2 + 4 + 7 * 4) + 2 * 512 * 2
    b3 = T * 2 * (512 * 2 * 2 + 8 + 7 * 8) + 2 * 512 * 2
    return k1, k2, k3, k4, b1, b2, b3


def normproj_setup(torch, Q, inputs, T, unfused=False):
    c = inputs.make_case("flashnorm-2048", T)
    x, w, g = dev(torch, c["x"]), dev(torch, c["w"]), dev(torch, c["gamma"])
    K, N = w.shape
    wm = w if unfused else Q.normproj_fold_weight(w, g)
    n = rotation_count(T * (K + N) * 2 + K * N * 2 + (T * K * 2 if unfused else 0))
    sets = [(x.clone(), torch.empty((T, N), dtype=torch.bfloat16, device="cuda"),
             torch.empty((T, K), dtype=torch.bfloat16, device="cuda") if unfused else None,
             wm.clone()) for _ in range(n)]

    def deferred(i):
        xi, yi, _, wi = sets[i % n]
        Q.normproj_deferred(xi, wi, eps=c["eps"], y=yi)

    def unf(i):
        xi, yi, xn, wi = sets[i % n]
        Q.normproj_unfused(xi, g, wi, eps=c["eps"], xn=xn, y=yi)

    flops = 2.0 * T * K * N
    nbytes = T * K * 2 + K * N * 2 + T * N * 2
    deferred.sets = unf.sets = n
    return (unf if unfused else deferred), flops, nbytes


def elimination_setup(torch, Q, inputs, T, mode):
    """Pre-norm -> Q/K projection -> QK-Norm at OLMo-2-7B widths (x [T, 4096], Wq, Wk
    [4096, 4096]). mode: 'eliminated' (no pre-norm), 'exact' (pre-norm scale deferred to the
    product) or 'unfused' (qknorm_project_unfused: RMSNorm launch, plain product, QK-Norm
    launch in place, the intermediates kept in the caches as in the eliminated form)."""
    c = inputs.make_elimination_case(T)
    x, w = dev(torch, c["x"]), dev(torch, c["w"])
    g1, gq, gk = dev(torch, c["gamma_pre"]), dev(torch, c["gamma_q"]), dev(torch, c["gamma_k"])
    K, N, nq = c["K"], c["nq"] + c["nk"], c["nq"]
    wm = w if mode == "unfused" else Q.normproj_fold_weight(w, g1)
    del w
    n = rotation_count(T * (K + N) * 2 + K * N * 2 + (T * K * 2 if mode == "unfused" else 0))
    sets = [(x.clone(), torch.empty((T, N), dtype=torch.bfloat16, device="cuda"),
             torch.empty((T, K), dtype=torch.bfloat16, device="cuda") if mode == "unfused"
             else None, wm.clone()) for _ in range(n)]
    del wm

    def fn(i):
        xi, yi, xn, wi = sets[i % n]
        if mode == "unfused":
            Q.qknorm_project_unfused(xi, g1, wi, nq, gq, gk, eps_qk=c["eps_qk"],
                                     eps_pre=c["eps_pre"], xn=xn, y=yi)
        else:
            Q.qknorm_project_eliminated(xi, wi, nq, gq, gk, eps_qk=c["eps_qk"],
                                        eps_pre=c["eps_pre"], exact=(mode == "exact"), y=yi)

    fn.sets = n
    return fn, 2.0 * T * K * N


def layernorm_setup(torch, Q, inputs, T, unfused, in_product=False):
    """LayerNorm -> projection at the FlashNorm shape (x [T, 2048], W [2048, 2048]): deferred
    (row statistics from a streaming pass into a workspace, or with in_product accumulated
    inside the product) or unfused (LayerNorm launch, then the plain product)."""
    c = inputs.make_layernorm_case(T)
    x, w = dev(torch, c["x"]), dev(torch, c["w"])
    g, be = dev(torch, c["gamma"]), dev(torch, c["beta"])
    K, N = c["K"], c["N"]
    if unfused:
        wm, cs, b = w, None, None
    else:
        wm, cs, b = Q.normproj_fold_layernorm(w, g, be)
    n = rotation_count(T * (K + N) * 2 + K * N * 2 + (T * K * 2 if unfused else 0))
    sets = [(x.clone(), torch.empty((T, N), dtype=torch.bfloat16, device="cuda"),
             torch.empty((T, K), dtype=torch.bfloat16, device="cuda") if unfused else None,
             wm.clone()) for _ in range(n)]
    ws = None if in_product else torch.empty((T, 2), dtype=torch.float32, device="cuda")

    def fn(i):
        xi, yi, xn, wi = sets[i % n]
        if unfused:
            Q.normproj_layernorm_unfused(xi, g, be, wi, eps=c["eps"], xn=xn, y=yi)
        else:
            Q.normproj_deferred_layernorm(xi, wi, cs, b, eps=c["eps"], y=yi, row_stats=ws)

    fn.sets = n
    return fn, 2.0 * T * K * N, T * K * 2 + K * N * 2 + T * N * 2


CASE_REPS = 5


def time_case(timer, fn, iters, warmup):
    """(eager ms per call, graph-replay ms per call), each the median of CASE_REPS repeats."""
    eager = timer.run(fn, iters, warmup, CASE_REPS)
    per_graph = max(fn.sets, 8 if fn.sets == 1 else fn.sets)
    graph = timer.run_graph(fn, per_graph, max(2, iters // per_graph), 2, CASE_REPS)
    return eager, graph


# ----------------------------------------------------------------------------- CPU baseline
def host_cores():
    """(threads used, cores in this process's affinity mask). The threads are every core of the
    affinity mask, capped by the host share the machine allots per GPU when it states one in
    OMP_NUM_THREADS (16 on the GPU machines this runs on)."""
    affinity = len(os.sched_getaffinity(0))
    share = os.environ.get("OMP_NUM_THREADS", "")
    cap = int(share) if share.isdigit() and int(share) > 0 else affinity
    return max(1, min(affinity, cap)), affinity


def oracle_timer(fn, rows_total, threads, min_seconds=0.3, reps=3):
    """Seconds per pass of fn over rows [0, rows_total), the rows split into `threads` equal
    chunks run concurrently (the C oracle releases the interpreter lock): the best of `reps`
    passes, or of as many as fit min_seconds when a pass is short."""
    from concurrent.futures import ThreadPoolExecutor

    bounds = [(i * rows_total // threads, (i + 1) * rows_total // threads)
              for i in range(threads)]
    bounds = [b for b in bounds if b[1] > b[0]]
    best, t_all, n = float("inf"), time.perf_counter(), 0
    with ThreadPoolExecutor(max_workers=len(bounds)) as ex:
        while n < reps or time.perf_counter() - t_all < min_seconds:
            t0 = time.perf_counter()
            list(ex.map(lambda b: fn(b[0], b[1]), bounds))
            best = min(best, time.perf_counter() - t0)
            n += 1
            if n >= 50:
                break
    return best


def cpu_oracle_cases(inputs, threads, row_budget_s=1.0):
    """The fp64 oracle, as it stands, on every workload and token count, on one thread and on
    `threads` threads. Row operations run on all T rows; the projection's oracle (about
    2 K N flops per row in naive fp64) runs on a sample of rows sized to about row_budget_s on
    one thread, and its per-call time is scaled per row to T ("extrapolated")."""
    import oracle

    out = []

    def add(cfg, T, nthreads, sec, rows_timed, what):
        rec = {"case": f"oracle {what} {cfg} T={T}", "config": cfg, "T": T, "threads": nthreads,
               "us_per_call": sec * 1e6, "tokens_per_s": T / sec if sec > 0 else None,
               "rows_timed": rows_timed}
        if rows_timed < T:
            rec["extrapolated"] = f"timed on {rows_timed} of {T} rows, scaled per row"
        out.append(rec)

    for cfg, Ts in (("tiny-fp32", (64,)), ("olmo2-7b", (1, 16, 256, 4096, 8192)),
                    ("gqa-olmo2-32b-like", (1, 512, 8192))):
        for T in Ts:
            c = inputs.make_case(cfg, T)

            def fused(lo, hi, c=c):
                oracle.rmsnorm_rows(c["q"][lo:hi], c["gamma_q"], c["eps"])
                oracle.rmsnorm_rows(c["k"][lo:hi], c["gamma_k"], c["eps"])

            for nt in sorted({1, threads}):
                add(cfg, T, nt, oracle_timer(fused, T, min(nt, T)), T, "rmsnorm Q+K")
    c = inputs.make_case("tp8-shard", 131072)
    T = 131072

    def shard(lo, hi):
        pq = oracle.partial_sumsq(c["q"][lo:hi])
        pk = oracle.partial_sumsq(c["k"][lo:hi])
        oracle.apply_with_stats(c["q"][lo:hi], c["gamma_q"], pq, c["ext_q"][:, lo:hi], 4096,
                                c["eps"])
        oracle.apply_with_stats(c["k"][lo:hi], c["gamma_k"], pk, c["ext_k"][:, lo:hi], 4096,
                                c["eps"])

    for nt in sorted({1, threads}):
        add("tp8-shard", T, nt, oracle_timer(shard, T, nt, reps=1), T,
            "partial sums + aggregation and scale")
    c = inputs.make_case("flashnorm-2048", 64)
    wf = oracle.round_bf16(oracle.fold_weight(c["w"], c["gamma"]))
    t0 = time.perf_counter()
    oracle.normproj(c["x"][:1], wf, c["eps"])
    per_row = max(time.perf_counter() - t0, 1e-6)
    for T in inputs.WORKLOADS["flashnorm-2048"]["Ts"]:
        for nt in sorted({1, threads}):
            rows = max(1, min(T, nt * max(1, int(row_budget_s / per_row)), 64 * nt))
            cx = inputs.make_case("flashnorm-2048", rows) if rows > 64 else c

            def proj(lo, hi, cx=cx):
                oracle.normproj(cx["x"][lo:hi], wf, cx["eps"])

            sec = oracle_timer(proj, rows, min(nt, rows), min_seconds=0.0, reps=1)
            add("flashnorm-2048", T, nt, sec * T / rows, rows, "deferred projection")
    return out


def cpu_baseline(cases, threads, T_full):
    """The headline's CPU figure: the oracle of the fused Q+K norm on the whole headline
    workload on `threads` threads (with the one-thread figure beside it)."""
    multi = [c for c in cases if c["config"] == "olmo2-7b" and c["T"] == T_full and
             c["threads"] == threads]
    single = [c for c in cases if c["config"] == "olmo2-7b" and c["T"] == T_full and
              c["threads"] == 1]
    if not multi:
        return None
    _, affinity = host_cores()
    return {"value": multi[0]["tokens_per_s"], "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"all {T_full} tokens of Q and K [{T_full}, 4096] bf16 (the headline "
                      f"workload), fp64 oracle, rows split over {threads} threads, best pass",
            "affinity_cores": affinity,
            "single_thread_value": single[0]["tokens_per_s"] if single else None,
            "cpu_model": cpu_model()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--tokens", type=int, default=8192)
    ap.add_argument("--cases", default="all", help="'all' or 'none': per-workload timings")
    ap.add_argument("--only", default="",
                    help="comma-separated prefixes: time only the cases whose entry point "
                         "starts with one of them (e.g. 'normproj,qknorm_partial')")
    ap.add_argument("--ts", default="",
                    help="comma-separated token counts: per-workload cases at these T only")
    ap.add_argument("--case-iters", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copies", type=int, default=0,
                    help="after the timed region, run this many qkn_device_copy launches of "
                         "half the headline's algorithmic bytes (memory-counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (rows shard with no "
              "exchange; the column-sharded exchange is not built). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import layerwise_qk_norm_amd as Q
    from layerwise_qk_norm_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    Q.lib()
    stream = torch.cuda.Stream()
    timer = Timer(torch, stream)

    T = args.tokens
    step, nbytes = fused_setup(torch, Q, inputs, "olmo2-7b", T, stream)
    torch.cuda.synchronize()
    ms = timer.run(step, args.steps, args.warmup)
    achieved = nbytes / (ms * 1e-3) / 1e9
    print(f"# headline: fused Q+K [{T}, 4096] bf16: {ms * 1e3:.2f} us/call, {achieved:.0f} GB/s",
          file=sys.stderr, flush=True)

    if args.calib_copies > 0:
        half = (nbytes // 2) // 16 * 16
        src = torch.empty(half, dtype=torch.uint8, device="cuda")
        dst = torch.empty(half, dtype=torch.uint8, device="cuda")
        with torch.cuda.stream(stream):
            for _ in range(args.calib_copies):
                Q.qkn_device_copy(dst, src)
        torch.cuda.synchronize()
        print(f"# calibration: {args.calib_copies} copies of {half} B", file=sys.stderr)
        del src, dst

    cases = []
    if args.cases == "all":
        it, wu = args.case_iters, max(5, args.case_iters // 10)

        def want(name):
            return not args.only or any(name.startswith(p) for p in args.only.split(","))

        ts_only = {int(v) for v in args.ts.split(",") if v}

        def want_t(t):
            return not ts_only or t in ts_only

        # empirical copy ceiling over the same bytes (read nbytes/2, write nbytes/2)
        half = (nbytes // 2) // 16 * 16
        n_copy = rotation_count(2 * half)
        bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda"),
                 torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(n_copy)]
        if want("qkn_device_copy"):
            cms = timer.run(lambda i: Q.qkn_device_copy(bufs[i % n_copy][1], bufs[i % n_copy][0]),
                            it, wu)
            cases.append({"case": f"device copy {half} B (same traffic as the headline)",
                          "us_per_call": cms * 1e3, "GB_s": 2 * half / (cms * 1e-3) / 1e9})
        del bufs

        for wl, Ts in (("tiny-fp32", (64,)), ("olmo2-7b", (1, 16, 256, 4096, 8192)),
                       ("gqa-olmo2-32b-like", (1, 512, 8192))):
            for t in Ts:
                if not want("qknorm_fused") or not want_t(t):
                    continue
                fn, b = fused_setup(torch, Q, inputs, wl, t, stream)
                cms, gms = time_case(timer, fn, it, wu)
                cases.append({"case": f"qknorm_fused {wl} T={t}",
                              "us_per_call": cms * 1e3, "us_per_call_graph": gms * 1e3,
                              "GB_s": b / (gms * 1e-3) / 1e9,
                              "frac_hbm": b / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS})
                del fn
                torch.cuda.empty_cache()

        k1, k2, k3, k4, b1, b2, b3 = shard_setup(torch, Q, inputs, 131072)
        for name, label, fn, b in (
                ("qknorm_partial_sumsq", "", k1, b1), ("qknorm_apply_with_stats", "", k2, b2),
                ("qknorm_shard_fused", " persistent", k3, b3),
                ("qknorm_shard_fused", " one workgroup per row block", k4, b3)):
            if not want(name):
                continue
            m, gm = time_case(timer, fn, it, wu)
            cases.append({"case": f"{name}{label} tp8-shard T=131072",
                          "us_per_call": m * 1e3, "us_per_call_graph": gm * 1e3,
                          "GB_s": b / (gm * 1e-3) / 1e9,
                          "frac_hbm": b / (gm * 1e-3) / 1e9 / PEAK_HBM_GBS})
            if name == "qknorm_shard_fused":
                torch.cuda.synchronize()
                cases[-1]["timed_out"] = int(fn.timed_out.item())
        del k1, k2, k3, k4
        torch.cuda.empty_cache()

        for t in (1, 2048, 16384):
            for unfused in (False, True):
                if (unfused and t == 1) or not want_t(t) or not want(
                        "normproj_unfused" if unfused else "normproj_deferred"):
                    continue
                fn, flops, b = normproj_setup(torch, Q, inputs, t, unfused)
                cms, gms = time_case(timer, fn, it, wu)
                name = "normproj_unfused" if unfused else "normproj_deferred"
                entry = {"case": f"{name} flashnorm-2048 T={t}", "us_per_call": cms * 1e3,
                         "us_per_call_graph": gms * 1e3, "TFLOP_s": flops / (gms * 1e-3) / 1e12}
                if t == 1:
                    entry["GB_s"] = b / (gms * 1e-3) / 1e9
                    entry["frac_hbm"] = entry["GB_s"] / PEAK_HBM_GBS
                else:
                    entry["frac_mfma_bf16"] = entry["TFLOP_s"] / PEAK_BF16_TFLOPS
                cases.append(entry)
                del fn
                torch.cuda.empty_cache()

        for t in inputs.ELIMINATION["Ts"]:
            for mode in ("eliminated", "exact", "unfused"):
                name = {"eliminated": "qknorm_project_eliminated",
                        "exact": "qknorm_project_eliminated_exact",
                        "unfused": "unfused_prenorm_chain"}[mode]
                if (t == 16 and mode != "eliminated") or not want(name) or not want_t(t):
                    continue
                fn, flops = elimination_setup(torch, Q, inputs, t, mode)
                cms, gms = time_case(timer, fn, it, wu)
                cases.append({"case": f"{name} {inputs.ELIMINATION['name']} T={t}",
                              "us_per_call": cms * 1e3, "us_per_call_graph": gms * 1e3,
                              "TFLOP_s": flops / (gms * 1e-3) / 1e12,
                              "frac_mfma_bf16": flops / (gms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS})
                del fn
                torch.cuda.empty_cache()

        for t in inputs.LAYERNORM["Ts"]:
            for unfused, in_product in ((False, False), (False, True), (True, False)):
                name = "normproj_layernorm_unfused" if unfused else "normproj_deferred_layernorm"
                if ((unfused or in_product) and t == 1) or not want(name) or not want_t(t):
                    continue
                fn, flops, b = layernorm_setup(torch, Q, inputs, t, unfused, in_product)
                cms, gms = time_case(timer, fn, it, wu)
                label = " (statistics inside the product)" if in_product else ""
                entry = {"case": f"{name}{label} {inputs.LAYERNORM['name']} T={t}",
                         "us_per_call": cms * 1e3, "us_per_call_graph": gms * 1e3,
                         "TFLOP_s": flops / (gms * 1e-3) / 1e12}
                if t == 1:
                    entry["GB_s"] = b / (gms * 1e-3) / 1e9
                    entry["frac_hbm"] = entry["GB_s"] / PEAK_HBM_GBS
                else:
                    entry["frac_mfma_bf16"] = entry["TFLOP_s"] / PEAK_BF16_TFLOPS
                cases.append(entry)
                del fn
                torch.cuda.empty_cache()
        for cs in cases:
            print("# " + json.dumps(cs), file=sys.stderr, flush=True)

    cpu, cpu_cases = None, []
    if not args.no_cpu_baseline:
        threads, _ = host_cores()
        if T == 8192:
            cpu_cases = cpu_oracle_cases(inputs, threads)
        else:
            cpu_cases = []
            c = inputs.make_case("olmo2-7b", T)
            import oracle

            def fused(lo, hi):
                oracle.rmsnorm_rows(c["q"][lo:hi], c["gamma_q"], c["eps"])
                oracle.rmsnorm_rows(c["k"][lo:hi], c["gamma_k"], c["eps"])

            for nt in sorted({1, threads}):
                sec = oracle_timer(fused, T, min(nt, T))
                cpu_cases.append({"case": f"oracle rmsnorm Q+K olmo2-7b T={T}",
                                  "config": "olmo2-7b", "T": T, "threads": nt,
                                  "us_per_call": sec * 1e6, "tokens_per_s": T / sec,
                                  "rows_timed": T})
        cpu = cpu_baseline(cpu_cases, threads, T)

    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"layerwise QK-Norm, OLMo-2-7B shape: Q and K [{T}, 4096] bf16 "
                               f"(32 heads x 128), one fused Q+K launch per step, x~N(0,2), "
                               f"gamma~N(1,0.05), eps=1e-6",
                   "tokens": T, "dq": 4096, "dk": 4096, "parallelism": "none (1 GPU)",
                   "rotating_buffers_bytes": ROTATE_BYTES},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": recorded_traffic(),
                     "algorithmic_bytes_per_launch": nbytes,
                     "kernel": "rows_team_kernel<kFused, bf16, bf16, 3, 3, nt, full> (qknorm_fused)"},
        "cpu_baseline": cpu,
        "cpu_oracle_cases": cpu_cases,
        "cases": cases,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
