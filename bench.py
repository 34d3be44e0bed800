"""Benchmark of one paged split-KV decode step on one MI355X.

Workload (default): the 100K-token long-context decode -- batch 1, context
100000, 32 query heads / 4 KV heads, head_dim 128, block_size 16, bf16 KV with
+8 logit outliers on 0.1% of keys, partition_size 512 (196 partitions).  One
step is one full pass of the decode path over the batch: phase 1 (per-partition
attention) + phase 2 (log-sum-exp merge), exactly what pa_decode enqueues for
this shape, called through the C ABI.

Inputs are resident in HBM before the timed region starts.  The KV pool is
replicated R times and step i reads copy i mod R, so consecutive steps never
find their KV in the 256 MB last-level cache: the figure is an HBM figure.

Prints ONE JSON line.  Value = KV bytes read per step / step time (GB/s).
The float64 oracle is used only in the CPU-baseline leg, which also checks the
first step's GPU output against it.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published peak
MFMA_PEAK_TFLOPS_16BIT = 2500.0  # MI355X dense bf16 / fp16 matrix-core peak
KERNEL_SOURCE = os.path.join(ROOT, "paged_split_kv_pa_amd", "csrc", "pa_kernels.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_mfma_kernel_long_100k_p512.md")


def counted_traffic():
    """HBM bytes per attention launch from the committed counter summary, or None
    when the kernel source has changed since those counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_SUMMARY).read()
        fields = dict(ln.split(": ", 1) for ln in text.splitlines() if ": " in ln
                      and ln.split(": ", 1)[0] in ("traffic_bytes_per_launch",
                                                    "kernel_source_sha256_prefix"))
        digest = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
        if digest.startswith(fields["kernel_source_sha256_prefix"].strip()):
            return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        pass
    return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="2",
                    help="decode workload index (2 = 100K context), or 'all' for one record "
                         "per workload")
    ap.add_argument("--partition-size", type=int, default=512)
    ap.add_argument("--path", choices=("auto", "v1", "v2"), default="auto",
                    help="decode path (auto = the library's rule)")
    ap.add_argument("--copies", type=int, default=0,
                    help="KV pool replicas rotated across steps (0 = enough for >= 1 GiB)")
    ap.add_argument("--variant", type=int, default=-1, help="matrix-core kernel variant")
    ap.add_argument("--split-pieces", type=int, default=-1,
                    help="work split: -1 automatic, 0 off, 2/4/8/16 pieces per item from "
                         "--split-first on")
    ap.add_argument("--split-first", type=int, default=0)
    ap.add_argument("--event-every", type=int, default=8,
                    help="copy_blocks / prefill: record the kernel's start/stop events on "
                         "every N-th timed step")
    ap.add_argument("--no-graph", action="store_true",
                    help="decode: skip the graph-replay measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--sweep-paths", action="store_true",
                    help="time forced V1 against forced V2 over a grid of batch sizes and "
                         "context lengths (32/4 heads, head_dim 128, bf16) and exit")
    ap.add_argument("--op", choices=("decode", "copy_blocks", "prefill"), default="decode",
                    help="decode (the headline), the prefix-caching KV block copy, or paged "
                         "prefix-prefill attention")
    ap.add_argument("--prefill-config", type=int, default=1,
                    help="prefill: workload index (1 = 8192-token chunk after a 65536 prefix)")
    ap.add_argument("--pairs", type=int, default=2048,
                    help="copy_blocks: (src, dst) block pairs per call")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (reference "
                         "kernel for scaling hardware byte counters), then exit")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="only time dense square GEMMs (torch.matmul, bf16 and fp16, N(0,1) "
                         "and all-zero operands): the matrix-core rate this card sustains, "
                         "then exit")
    ap.add_argument("--prefill-zero", choices=("none", "k", "v", "kv"), default="none",
                    help="prefill: zero the cached and new keys and/or values (the same "
                         "kernel and work on operands that draw less power)")
    return ap.parse_args()


def gemm_reference(reps=20):
    """Dense square GEMMs through torch.matmul (hipBLASLt) in bf16 and fp16, on N(0,1) and on
    all-zero operands: the matrix-core rate a vendor GEMM sustains on this card, to read the
    prefill rates against.  The zero operands draw less power, so the clock runs higher:
    the gap between the two is the data-dependent part of the sustained rate."""
    import torch
    rec = {"metric": "dense GEMM TFLOP/s (torch.matmul)", "unit": "TFLOP/s", "n_gpus": 1,
           "peak": MFMA_PEAK_TFLOPS_16BIT, "rates": []}
    gen = torch.Generator(device="cuda").manual_seed(3)
    for dt in (torch.bfloat16, torch.float16):
        for n in (8192, 16384):
            a = torch.randn(n, n, device="cuda", dtype=dt, generator=gen)
            b = torch.randn(n, n, device="cuda", dtype=dt, generator=gen)
            z = torch.zeros_like(a)
            for name, (x, y) in (("randn", (a, b)), ("zeros", (z, z))):
                for _ in range(3):
                    torch.matmul(x, y)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(reps):
                    torch.matmul(x, y)
                torch.cuda.synchronize()
                tf = 2 * n ** 3 / ((time.perf_counter() - t0) / reps) / 1e12
                rec["rates"].append({"dtype": str(dt).split(".")[-1], "n": n, "operands": name,
                                     "tflops": round(tf, 1),
                                     "of_peak": round(tf / MFMA_PEAK_TFLOPS_16BIT, 4)})
                log(f"gemm {dt} n={n} {name}: {tf:.0f} TFLOP/s")
            del a, b, z
    print(json.dumps(rec), flush=True)


def copy_calibration(mib, reps=5):
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters calibrate the
    byte counters read for the decode kernels (bytes expected / bytes counted)."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_dispatch": n, "dispatches": reps}), flush=True)


def to_dev(a, dtype):
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def _host_threads():
    """(threadpool limiter or None, threads used): BLAS threads pinned to every core the
    process may run on."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        ctx = threadpool_limits(limits=len(os.sched_getaffinity(0)))
        return ctx, max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: numpy picks its own thread count
        return None, len(os.sched_getaffinity(0))


def cpu_baseline(w, seconds):
    """Time the float64 oracle (as it stands) on the host cores over a bounded sample of
    the workload: whole decode steps when one step takes less than the budget, else
    sequences of the batch one at a time, longest first (the oracle processes a batch
    sequence by sequence either way)."""
    import oracle
    from paged_split_kv_pa_amd import workloads as wl
    ctx, threads = _host_threads()
    order = np.argsort(-w.context_lens, kind="stable")
    kv_seq = [wl.kv_bytes([n], w.num_kv_heads, w.head_dim, w.dtype) for n in w.context_lens]
    done_bytes, seqs, steps, t0 = 0, 0, 0, time.perf_counter()
    while True:
        b = int(order[seqs % w.num_seqs])
        oracle.decode_attention(w.q[b:b + 1], w.k_cache, w.v_cache, w.block_tables[b:b + 1],
                                w.context_lens[b:b + 1], w.scale, w.dtype)
        done_bytes += kv_seq[b]
        seqs += 1
        if seqs % w.num_seqs == 0:
            steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    if ctx is not None:
        ctx.restore_original_limits()
    sample = (f"{steps} full decode steps" if seqs % w.num_seqs == 0 else
              f"{seqs} sequences of the {w.num_seqs}-sequence batch, longest first") + \
        f" (float64 numpy oracle: gather, upcast, softmax attention), {el:.1f} s wall"
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "sample": sample}


def parity_sample(w, got, max_seqs=8):
    """The first step's GPU output against the oracle on up to max_seqs sequences (the
    longest, the shortest and the first ones): max abs error, max row relative L2 and the
    verdict at the tolerance for fp16/bf16 KV with fp32 accumulation."""
    import oracle
    S = w.num_seqs
    pick = sorted(set([int(np.argmax(w.context_lens)), int(np.argmin(w.context_lens))] +
                      list(range(min(S, max_seqs)))))[:max_seqs]
    ref = oracle.decode_attention(w.q[pick], w.k_cache, w.v_cache, w.block_tables[pick],
                                  w.context_lens[pick], w.scale, w.dtype)
    g = got[pick]
    err = np.abs(g - ref)
    ok = bool(np.all(err <= 2e-3 + 1e-2 * np.abs(ref)))
    num = np.linalg.norm((g - ref).reshape(-1, w.head_dim), axis=1)
    den = np.linalg.norm(ref.reshape(-1, w.head_dim), axis=1)
    rel = float(np.max(np.where(den > 0, num / np.maximum(den, 1e-300), num)))
    return {"sequences_checked": len(pick), "max_abs_err": float(err.max()),
            "max_row_rel_l2": rel, "within_tolerance": ok and rel <= 1e-2}


# The pages' own setting, carried in every decode record as context (not a target):
# the hardware their numbers refer to and the 100K-token partition count.  They publish
# no measured kernel throughput for this path.
PAGES_CONTEXT = {
    "hardware": "BI-V100",
    "compute_units": 16,
    "hbm_GBps": 900,
    "partitions_at_100k_tokens": {
        "pages": "about 195 partitions in parallel with V2, against 1 work item for V1",
        "computed": "196 = ceil(100000 / 512): 195 full partitions and one of 160 tokens"},
    "published_kernel_throughput": None,
    "source": "project_6 commit 96f4baf page (V2 plan); prefix_prefill_patch.py analysis "
              "(BI-V100 figures); GROUND_TRUTH_STATUS_v2.md (compute-unit count)",
}


def stats(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(xs)), 3), "p10": round(float(np.percentile(xs, 10)), 3),
            "p90": round(float(np.percentile(xs, 90)), 3), "n": int(xs.size)}


def sweep_paths(reps=20):
    """Forced V1 vs forced V2 step time over (batch, context); prints JSON lines.

    Each step is timed on the GPU side: a rotation of steps over cold copies of the KV
    pool is captured in a graph and replayed, so the host's per-call cost does not enter
    (the wall-clock rate of eager calls is printed beside it).  Inputs are random bf16
    tensors drawn on the device (the values do not matter for timing; parity is covered
    by the tests).
    """
    import torch
    from paged_split_kv_pa_amd import binding as B
    Hq, Hkv, D, P = 32, 4, 128, 512
    gen = torch.Generator(device="cuda").manual_seed(7)
    rows = []
    for S in (1, 4, 16, 64, 256):
        for n in (256, 512, 1024, 2048, 4096, 8192, 16384, 32768):
            if S * n > (1 << 20):
                continue
            nb = -(-n // 16)
            NB = S * nb + 1
            pool_bytes = 2 * NB * Hkv * 16 * D * 2
            R = max(2, -(-(1 << 30) // pool_bytes))
            q = torch.randn(S, Hq, D, device="cuda", dtype=torch.bfloat16, generator=gen)
            ks = [torch.randn(NB, Hkv, 16, D, device="cuda", dtype=torch.bfloat16, generator=gen)
                  for _ in range(R)]
            vs = [torch.randn_like(k) for k in ks]
            bt = torch.randperm(NB - 1, device="cuda", generator=gen)[:S * nb].view(S, nb)
            bt = bt.to(torch.int32).contiguous()
            ctx = torch.full((S,), n, dtype=torch.int32, device="cuda")
            out = torch.empty_like(q)
            ws = torch.empty(B.pa_workspace_bytes(q, ks[0], bt, 0, P), dtype=torch.uint8,
                             device="cuda")
            res = {}
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.current_stream())
            for name, path in (("v1", B.PA_PATH_V1), ("v2", B.PA_PATH_V2)):
                def steps(count):
                    for i in range(count):
                        B.pa_decode_ex(out, q, ks[i % R], vs[i % R], bt, ctx, 0.088, P,
                                       stream=st, workspace=ws, path=path)
                with torch.cuda.stream(st):
                    steps(R)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=st):
                    steps(R)
                for _ in range(2):
                    g.replay()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(reps):
                    g.replay()
                torch.cuda.synchronize()
                res[name] = (time.perf_counter() - t0) * 1e6 / (reps * R)
                with torch.cuda.stream(st):
                    steps(2)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                with torch.cuda.stream(st):
                    steps(4 * R)
                torch.cuda.synchronize()
                res[name + "_eager"] = (time.perf_counter() - t0) * 1e6 / (4 * R)
                del g
            rec = {"num_seqs": S, "context": n, "us_v1": round(res["v1"], 2),
                   "us_v2": round(res["v2"], 2), "us_v1_eager": round(res["v1_eager"], 2),
                   "us_v2_eager": round(res["v2_eager"], 2),
                   "faster": "v1" if res["v1"] <= res["v2"] else "v2",
                   "auto": "v1" if B.pa_choose_path(B.dims_of(q, ks[0], bt), 0, P) == 1 else "v2"}
            rows.append(rec)
            print(json.dumps(rec), flush=True)
            del q, ks, vs, bt, ctx, out, ws
    return rows


def bench_copy_blocks(args):
    """The prefix-caching block copy (pa_copy_blocks) on the long_100k pool shape: 7500
    blocks of 4 KV heads x 16 x 128 bf16 per pool, `--pairs` disjoint (src, dst) pairs
    drawn with a fixed seed; pool replicas rotate so that the copied blocks are cold."""
    import ctypes
    import torch
    from paged_split_kv_pa_amd import binding as B

    NB, Hkv, D = 7500, 4, 128
    n = args.pairs
    rng = np.random.default_rng(7)
    ids = rng.permutation(NB)[:2 * n]
    pairs_np = np.stack([ids[:n], ids[n:]], axis=1).astype(np.int32)
    pool_bytes = 2 * NB * Hkv * 16 * D * 2
    R = args.copies if args.copies > 0 else max(2, -(-(1 << 30) // pool_bytes))
    gen = torch.Generator(device="cuda").manual_seed(7)
    ks = [torch.randn(NB, Hkv, 16, D, device="cuda", dtype=torch.bfloat16, generator=gen)
          for _ in range(R)]
    vs = [torch.randn(NB, Hkv, 16, D, device="cuda", dtype=torch.bfloat16, generator=gen)
          for _ in range(R)]
    pairs = torch.from_numpy(pairs_np).cuda()
    block_bytes = Hkv * 16 * D * 2
    algo_bytes = 2 * 2 * n * block_bytes  # K and V, read once and written once
    lib = B.lib()
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    call_args = [[ctypes.c_void_p(ks[c].data_ptr()), ctypes.c_void_p(vs[c].data_ptr()),
                  block_bytes, NB, ctypes.c_void_p(pairs.data_ptr()), n, sptr, None, None]
                 for c in range(R)]
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]

    def step(i, e0=None, e1=None):
        a = call_args[i % R]
        a[7], a[8] = e0, e1
        st = lib.pa_copy_blocks_profiled(*a)
        if st != 0:
            raise B.PaError(st, B.pa_last_error())

    # The first call's source blocks are kept for the bitwise check in the CPU leg.
    sample = pairs_np[:64]
    k_src0 = ks[0][torch.from_numpy(sample[:, 0]).long().cuda()].view(torch.int16).cpu().numpy()
    step(0)
    torch.cuda.synchronize()
    k_dst0 = ks[0][torch.from_numpy(sample[:, 1]).long().cuda()].view(torch.int16).cpu().numpy()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % max(1, args.event_every) == 0:
            e0, e1 = ctypes.c_void_p(), ctypes.c_void_p()
            hip.hipEventCreate(ctypes.byref(e0))
            hip.hipEventCreate(ctypes.byref(e1))
            step(i, e0, e1)
            evs.append((e0, e1))
        else:
            step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ctypes.c_float()
    ker = []
    for e0, e1 in evs:
        hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1)
        ker.append(ms.value * 1e3)
        hip.hipEventDestroy(e0)
        hip.hipEventDestroy(e1)
    us = wall * 1e6 / args.steps
    kmean = float(np.mean(ker))
    # Reference: a plain contiguous device-to-device copy of the same byte count (read +
    # write), cold source rotated the same way: what the hardware gives for a copy.
    half = algo_bytes // 2
    srcs = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(R)]
    dst = torch.empty(half, dtype=torch.uint8, device="cuda")
    for i in range(5):
        dst.copy_(srcs[i % R])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(50):
        dst.copy_(srcs[i % R])
    torch.cuda.synchronize()
    plain_us = (time.perf_counter() - t1) * 1e6 / 50
    del srcs, dst
    log(f"copy_blocks: {n} pairs, {algo_bytes / 1e6:.1f} MB moved per call; call {us:.2f} us; "
        f"kernel mean {kmean:.2f} us, median {np.median(ker):.2f}")
    rec = {
        "metric": "KV block copy GB/s (bytes read + written) + us/call, prefix-caching copy",
        "value": round(algo_bytes / (us / 1e6) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "us_per_step": round(us, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"copy_blocks_{n}", "num_blocks": NB, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": 16, "pairs": n, "block_bytes": block_bytes,
                   "bytes_per_call": algo_bytes, "pool_copies": R},
        "roofline": {"bound": "hbm", "achieved": round(algo_bytes / (kmean / 1e6) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(algo_bytes / (kmean / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "kernel": "copy_blocks_kernel",
                     "kernel_mean_us": round(kmean, 3), "kernel_samples": len(ker)},
        "plain_copy_reference": {"bytes": algo_bytes, "us": round(plain_us, 3),
                                 "GBps": round(algo_bytes / (plain_us / 1e6) / 1e9, 2)},
    }
    if not args.no_cpu_baseline:
        import oracle
        # parity of the first call on 64 sampled pairs: the oracle's copy of the kept
        # source blocks against what the kernel wrote
        pool = np.zeros((2 * len(sample),) + k_src0.shape[1:], dtype=np.int16)
        pool[:len(sample)] = k_src0
        want, _ = oracle.copy_blocks(pool, pool.copy(), np.stack(
            [np.arange(len(sample)), np.arange(len(sample)) + len(sample)], axis=1).astype(np.int32))
        rec["parity"] = {"sampled_pairs_bitwise": bool(np.array_equal(want[len(sample):], k_dst0))}
        kc = ks[0].view(torch.int16).cpu().numpy()
        vc = vs[0].view(torch.int16).cpu().numpy()
        reps, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < min(args.cpu_seconds, 10.0):
            oracle.copy_blocks(kc, vc, pairs_np)
            reps += 1
        el = time.perf_counter() - t1
        rec["cpu_baseline"] = {"value": round(algo_bytes * reps / el / 1e9, 3), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{reps} full calls (numpy gather of every block "
                                         f"pair into copies of both pools), {el:.1f} s wall"}
    print(json.dumps(rec), flush=True)


def prefill_flops(w):
    """Algorithmic FLOP of one prefill call: 2 D for q.k and 2 D for p.v per visible
    (query row, key) pair and query head; new token i of sequence b sees c_b + i + 1 keys."""
    total = 0
    for b in range(w.num_seqs):
        c = int(w.context_lens[b])
        L = int(w.query_start[b + 1]) - int(w.query_start[b])
        total += L * c + L * (L + 1) // 2
    return 4 * w.head_dim * w.num_q_heads * total


def bench_prefill(args):
    """Paged prefix-prefill attention (pa_prefill) on a seeded prefill workload; the
    metric is algorithmic TFLOP/s (2 D FLOP for q.k and 2 D for p.v per visible
    (query row, key) pair, per head) against the MI355X dense bf16/fp16 peak."""
    import ctypes
    import torch
    from paged_split_kv_pa_amd import binding as B
    from paged_split_kv_pa_amd import workloads as wl

    w = wl.prefill_config(args.prefill_config)
    log(f"prefill workload {w.name}: S={w.num_seqs} T={w.num_tokens} prefix "
        f"{list(map(int, w.context_lens))} Hq={w.num_q_heads} Hkv={w.num_kv_heads}")
    dev = {n: to_dev(getattr(w, n), w.dtype) for n in ("q", "k_new", "v_new", "k_cache",
                                                        "v_cache")}
    for n in ("block_tables", "context_lens", "query_start"):
        dev[n] = torch.from_numpy(np.ascontiguousarray(getattr(w, n), dtype=np.int32)).cuda()
    zeroed = {"none": (), "k": ("k_new", "k_cache"), "v": ("v_new", "v_cache"),
              "kv": ("k_new", "k_cache", "v_new", "v_cache")}[args.prefill_zero]
    for n in zeroed:
        dev[n].zero_()
    out = torch.empty_like(dev["q"])
    flops = prefill_flops(w)
    lib = B.lib()
    d = B.prefill_dims_of(dev["q"], dev["k_new"], dev["k_cache"], dev["block_tables"],
                          dev["context_lens"], w.max_query_len)
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    call = [ctypes.byref(d), vp(out), vp(dev["q"]), vp(dev["k_new"]), vp(dev["v_new"]),
            vp(dev["k_cache"]), vp(dev["v_cache"]), vp(dev["block_tables"]),
            vp(dev["context_lens"]), vp(dev["query_start"]), ctypes.c_float(w.scale), sptr,
            None, None]
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]

    def step(e0=None, e1=None):
        call[12], call[13] = e0, e1
        st = lib.pa_prefill_profiled(*call)
        if st != 0:
            raise B.PaError(st, B.pa_last_error())

    step()
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()  # the first call's output, checked in the CPU leg
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % max(1, args.event_every) == 0:
            e0, e1 = ctypes.c_void_p(), ctypes.c_void_p()
            hip.hipEventCreate(ctypes.byref(e0))
            hip.hipEventCreate(ctypes.byref(e1))
            step(e0, e1)
            evs.append((e0, e1))
        else:
            step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ctypes.c_float()
    ker = []
    for e0, e1 in evs:
        hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1)
        ker.append(ms.value * 1e3)
        hip.hipEventDestroy(e0)
        hip.hipEventDestroy(e1)
    us = wall * 1e6 / args.steps
    kmean = float(np.mean(ker))
    log(f"prefill: {flops / 1e12:.3f} TFLOP per call; call {us / 1e3:.3f} ms; kernel mean "
        f"{kmean / 1e3:.3f} ms")
    peak = MFMA_PEAK_TFLOPS_16BIT
    rec = {
        "metric": "prefix-prefill attention TFLOP/s (algorithmic, causal) + ms/call",
        "value": round(flops / (us / 1e6) / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic" if not zeroed else "synthetic, zeroed " + "/".join(zeroed),
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_tokens": w.num_tokens,
                   "context_lens": [int(x) for x in w.context_lens],
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": 16, "flops_per_call": flops},
        "roofline": {"bound": "mfma", "achieved": round(flops / (kmean / 1e6) / 1e12, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(flops / (kmean / 1e6) / 1e12 / peak, 4), "traffic": None,
                     "kernel": "prefill_kernel", "kernel_mean_us": round(kmean, 3),
                     "kernel_samples": len(ker)},
    }
    if not args.no_cpu_baseline and not zeroed:  # the oracle sees the workload's inputs
        import oracle
        from oracle.storage import upcast
        # parity of the first call on 16 sampled (row, head) outputs: the oracle computes
        # single causal rows cheaply
        rng = np.random.default_rng(1)
        G = w.num_q_heads // w.num_kv_heads
        worst = 0.0
        s32 = float(np.float32(w.scale))
        for _ in range(16):
            b = int(rng.integers(0, w.num_seqs))
            r0, r1 = int(w.query_start[b]), int(w.query_start[b + 1])
            if r1 == r0:
                continue
            i = int(rng.integers(0, r1 - r0))
            h = int(rng.integers(0, w.num_q_heads))
            c = int(w.context_lens[b])
            kp = upcast(oracle.gather_sequence(w.k_cache, w.block_tables, b, c), w.dtype)[:, h // G]
            vp_ = upcast(oracle.gather_sequence(w.v_cache, w.block_tables, b, c), w.dtype)[:, h // G]
            ka = np.concatenate([kp, upcast(w.k_new[r0:r0 + i + 1, h // G], w.dtype)])
            va = np.concatenate([vp_, upcast(w.v_new[r0:r0 + i + 1, h // G], w.dtype)])
            ref = oracle.prefill_rows(upcast(w.q[r0 + i:r0 + i + 1, h], w.dtype), ka, va, c + i,
                                      s32)[0]
            worst = max(worst, float(np.max(np.abs(got[r0 + i, h] - ref)
                                            / (2e-3 + 1e-2 * np.abs(ref)))))
        rec["parity"] = {"sampled_rows": 16, "worst_tolerance_ratio": round(worst, 4),
                         "within_tolerance": worst <= 1.0}
        # The oracle on a bounded sample: whole causal rows of the chunk, one at a time.
        b = 0
        c = int(w.context_lens[b])
        r0, r1 = int(w.query_start[b]), int(w.query_start[b + 1])
        kp = upcast(oracle.gather_sequence(w.k_cache, w.block_tables, b, c), w.dtype)
        vpc = upcast(oracle.gather_sequence(w.v_cache, w.block_tables, b, c), w.dtype)
        kn, vn = upcast(w.k_new, w.dtype), upcast(w.v_new, w.dtype)
        qq = upcast(w.q, w.dtype)
        try:
            from threadpoolctl import threadpool_info, threadpool_limits
            ctx = threadpool_limits(limits=len(os.sched_getaffinity(0)))
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        except Exception:  # threadpoolctl missing: numpy picks its own thread count
            ctx, threads = None, len(os.sched_getaffinity(0))
        rows, fl, t1 = 0, 0, time.perf_counter()
        while time.perf_counter() - t1 < min(args.cpu_seconds, 10.0) and rows < r1 - r0:
            i = rows
            for h in range(w.num_q_heads):
                g = h // G
                ka = np.concatenate([kp[:, g], kn[r0:r0 + i + 1, g]])
                va = np.concatenate([vpc[:, g], vn[r0:r0 + i + 1, g]])
                oracle.prefill_rows(qq[r0 + i:r0 + i + 1, h], ka, va, c + i, s32)
            fl += 4 * w.num_q_heads * w.head_dim * (c + i + 1)
            rows += 1
        el = time.perf_counter() - t1
        if ctx is not None:
            ctx.restore_original_limits()
        rec["cpu_baseline"] = {"value": round(fl / el / 1e12, 6), "unit": "TFLOP/s",
                               "cores": int(threads), "kind": "oracle",
                               "sample": f"{rows} query rows x {w.num_q_heads} heads of "
                                         f"sequence 0 (float64 numpy oracle), {el:.1f} s wall"}
    print(json.dumps(rec), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode "
              "kernel is measured at one GPU's share of the work", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gemm_reference:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        torch.cuda.set_device(0)
        gemm_reference()
        return
    if args.sweep_paths:
        sweep_paths()
        return
    if args.op == "prefill":
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        torch.cuda.set_device(0)
        bench_prefill(args)
        return
    if args.op == "copy_blocks":
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        torch.cuda.set_device(0)
        bench_copy_blocks(args)
        return

    from paged_split_kv_pa_amd import binding as B

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.variant >= 0:
        B.pa_set_mfma_variant(args.variant)
    if args.split_pieces != -1:
        B.pa_set_work_split(args.split_pieces, args.split_first)
    if args.config == "all":
        # one record per workload (the mixed batch at both partition sizes), the headline
        # long-context one last
        args.cpu_seconds = min(args.cpu_seconds, 6.0)
        for cfg, P in ((0, 512), (1, 512), (3, 512), (4, 512), (4, 256), (2, 512)):
            bench_decode(args, cfg, P)
    else:
        bench_decode(args, int(args.config), args.partition_size)


def bench_decode(args, cfg, P):
    """One decode workload: prints one JSON line."""
    import ctypes
    import torch
    from paged_split_kv_pa_amd import binding as B
    from paged_split_kv_pa_amd import workloads as wl

    log(f"generating workload {wl.CONFIG_NAMES[cfg]} (partition size {P})")
    w = wl.config(cfg)
    kvb = wl.kv_bytes(w.context_lens, w.num_kv_heads, w.head_dim, w.dtype)
    pool_bytes = w.k_cache.nbytes + w.v_cache.nbytes
    R = args.copies if args.copies > 0 else max(2, -(-(1 << 30) // pool_bytes))
    log(f"KV bytes/step {kvb}, pool {pool_bytes / 1e6:.1f} MB x {R} copies")

    q = to_dev(w.q, w.dtype)
    kc0, vc0 = to_dev(w.k_cache, w.dtype), to_dev(w.v_cache, w.dtype)
    ks = [kc0] + [kc0.clone() for _ in range(R - 1)]
    vs = [vc0] + [vc0.clone() for _ in range(R - 1)]
    bt = torch.from_numpy(w.block_tables).cuda()
    ctx = torch.from_numpy(w.context_lens).cuda()
    out = torch.empty_like(q)
    dims = B.dims_of(q, kc0, bt, out, vc0)
    path = {"auto": B.pa_choose_path(dims, 0, P), "v1": B.PA_PATH_V1,
            "v2": B.PA_PATH_V2}[args.path]
    stream = torch.cuda.current_stream()

    # Argument tuples are marshalled once, so a step costs one plain C call on the host:
    # pa_decode_profiled with no caller workspace = pa_decode (the library's workspace, the
    # same path and kernels: V2 as a single launch where it applies) plus optional
    # start/stop timestamps of the attention kernel taken by the runtime.
    lib = B.lib()
    dref = ctypes.byref(dims)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    scale = ctypes.c_float(w.scale)

    def args_for(st):
        sp = ctypes.c_void_p(st.cuda_stream)
        return [[dref, vp(out), vp(q), vp(ks[c]), vp(vs[c]), vp(bt), vp(ctx), scale, P, sp,
                 None, 0, 0, path, None, None] for c in range(R)]
    call_args = args_for(stream)

    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]

    def new_event():
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_us(e0, e1):
        ms = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1)
        return ms.value * 1e3

    def step(i, ev0=None, ev1=None, a=None):
        a = (a or call_args)[i % R]
        a[14], a[15] = ev0, ev1
        st = lib.pa_decode_profiled(*a)
        if st != 0:
            raise B.PaError(st, B.pa_last_error())

    # First step: its output is kept and checked against the oracle in the CPU leg.
    step(0)
    torch.cuda.synchronize()
    first_out = out.to(torch.float64).cpu().numpy()
    first_bits = out.clone()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")

    # (1) The timed region: exactly `steps` steps, nothing else on the stream.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    enqueue_us = (t_enq - t0) * 1e6 / args.steps

    # (2) Step-time distribution: a marker event between consecutive steps (GPU clock).
    n_s = max(args.steps, 20)
    marks = [new_event() for _ in range(n_s + 1)]
    torch.cuda.synchronize()
    for i in range(n_s):
        hip.hipEventRecord(marks[i], ctypes.c_void_p(stream.cuda_stream))
        step(i)
    hip.hipEventRecord(marks[n_s], ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    periods = [elapsed_us(marks[i], marks[i + 1]) for i in range(n_s)]
    for e in marks:
        hip.hipEventDestroy(e)

    # (3) Attention-kernel durations: runtime timestamps at its start and end, every step.
    ev0 = [new_event() for _ in range(n_s)]
    ev1 = [new_event() for _ in range(n_s)]
    torch.cuda.synchronize()
    for i in range(n_s):
        step(i, ev0[i], ev1[i])
    torch.cuda.synchronize()
    k1 = [elapsed_us(a, b) for a, b in zip(ev0, ev1)]
    for e in ev0 + ev1:
        hip.hipEventDestroy(e)

    # (4) Graph replay: one rotation of R steps captured once, replayed; the GPU-side
    # step time without the host's per-call cost.  The replayed output must equal the
    # eager one bitwise.
    graph = None
    if not args.no_graph:
        gs = torch.cuda.Stream()
        gargs = args_for(gs)
        gs.wait_stream(stream)
        with torch.cuda.stream(gs):
            for i in range(R):
                step(i, a=gargs)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            for i in range(R):
                step(i, a=gargs)
        reps = max(2, -(-n_s // R))
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        g_us = (time.perf_counter() - tg) * 1e6 / (reps * R)
        same = bool(torch.equal(out.view(torch.int16) if w.dtype != "f32" else out.view(torch.int32),
                                first_bits.view(torch.int16) if w.dtype != "f32"
                                else first_bits.view(torch.int32)))
        graph = {"us_per_step": round(g_us, 3), "steps_replayed": reps * R,
                 "steps_per_graph": R, "output_bitwise_equal_to_eager": same}
        del g

    k1s = stats(k1)
    k1_mean = float(np.mean(k1))
    log(f"step {ms_per_step * 1e3:.2f} us (host enqueue {enqueue_us:.2f} us/step); GPU step "
        f"period median {np.median(periods):.2f} us; attention kernel median "
        f"{k1s['median']:.2f} us (p10 {k1s['p10']:.2f}, p90 {k1s['p90']:.2f})" +
        (f"; graph replay {graph['us_per_step']:.2f} us/step" if graph else ""))

    mfma = w.dtype != "f32" and w.num_q_heads // w.num_kv_heads >= 4
    single = path == B.PA_PATH_V2 and B.pa_fused_applies(q, kc0, bt, P)
    kernel_name = ("attn_mfma_kernel" if mfma else "attn_valu_kernel") + \
        (" (V1 single pass)" if path == B.PA_PATH_V1 else
         " (V2 phase 1 and merge, one launch)" if single else " (V2 phase 1)")
    value = kvb / (ms_per_step / 1e3) / 1e9
    achieved = kvb / (k1_mean / 1e6) / 1e9
    rec = {
        "metric": "KV-read GB/s (% of HBM peak) + us/decode step, paged attn at 100K ctx",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.CONFIG_NAMES[cfg],
            "num_seqs": w.num_seqs, "context_lens_sum": int(w.context_lens.sum()),
            "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "block_size": wl.BLOCK_SIZE, "partition_size": P,
            "path": "v1" if path == B.PA_PATH_V1 else "v2",
            "kv_bytes_per_step": kvb, "kv_pool_copies": R,
            "mfma_variant": B.pa_get_mfma_variant(),
            "work_split": list(B.pa_get_work_split()),
            "single_launch": bool(single),
        },
        "step_us_gpu": stats(periods),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counted_traffic() if cfg == 2 and P == 512 else None,
            "kernel": kernel_name, "kernel_mean_us": round(k1_mean, 3),
            "kernel_us": k1s, "kernel_samples": len(k1),
        },
        "graph_replay": graph,
        "host_enqueue_us_per_step": round(enqueue_us, 3),
        "pages_context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        rec["parity"] = parity_sample(w, first_out)
        log(f"parity of the first step: {rec['parity']}")
    print(json.dumps(rec), flush=True)

if __name__ == "__main__":
    main()
