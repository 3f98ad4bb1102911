#!/usr/bin/env python3
"""Benchmark of the CSA2 decode step with an FP4 KV cache on one MI355X.

Workload (the 128K-context decode group): 16 sequences, 131,072 cache
entries each (ratio 1), one decoder group of 4 layers run twice on its state:
Full + 3 Reuse, then Reindex + 3 Reuse.  One step = both runs, so every
sequence sends one query token through each of the two groups: 32
query-tokens per step.  Inputs are seeded synthetic tensors resident in HBM;
the FP4 / fp8 caches are encoded before timing.

To keep the 256 MB Infinity Cache from serving the 143 MB indexer-key scan,
the step rotates over `--copies` independent copies of the caches (each with
its own group state): the Full run of step i uses copy 2i mod C, the Reindex
run copy 2i+1 mod C, whose state holds its own earlier Full layer.

Printed: one JSON line with throughput, the roofline of the dominant kernel
(the indexer scan: 68 algorithmic bytes per scanned key) timed with HIP
events on its stream during the timed loop, and the CPU oracle's throughput
on a bounded sample.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
KEY_BYTES = 64 + 4         # fp8 indexer key + float32 scale
ENTRY_BYTES = 256 + 32     # packed E2M1 + E4M3 scales
ROW_BYTES = 512 * 2        # bf16 window row
Q_BYTES, OUT_BYTES, IDX_BYTES, IDXQ_BYTES = 16 * 512 * 2, 16 * 512 * 4, 512 * 4, 4 * 64 + 4 * 4


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=8)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--ctx", type=int, default=131072)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 256 MiB five times (the known-size reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    ap.add_argument("--page-size", type=int, default=256, help="entries per page of --workload paged")
    ap.add_argument("--workload", choices=["decode", "multi", "prefill", "hier", "paged", "full64k", "tiny4k",
                                           "heads64k"],
                    default="decode",
                    help="decode: the 128K decode group (default, the headline); prefill: a 4,096-token "
                         "chunk on a 262,144-token prefix at ratio 2, 1 Full + 5 Reuse layers; hier: the "
                         "hierarchical Full layer at 1M context, batch 4; multi: the decode group with 4 query "
                         "tokens per sequence (speculative decoding); full64k: one Full layer, batch 8, 65,536 "
                         "entries with lognormal channel scales; tiny4k: one Full layer, batch 1, 4,096 entries; "
                         "heads64k: full64k with per-head 4 x 64 indexer keys")
    return ap.parse_args()


def algorithmic_bytes_per_qtok(ctx, nq=1, layers=4, key_bytes=KEY_BYTES):
    """Bytes one query token must move through one group of `layers` layers:
    its share of the key scan of the Full/Reindex layer (the nq query tokens
    of a sequence share one scan), and per layer the 512 gathered entries
    (all of them when fewer are visible), the 128 window rows, its query and
    output, the index list."""
    per_layer = min(512, ctx) * ENTRY_BYTES + 128 * ROW_BYTES + Q_BYTES + OUT_BYTES + IDX_BYTES
    return ctx * key_bytes / nq + IDXQ_BYTES + layers * per_layer


def host_cpu():
    """The host's logical CPUs this process may use, and the CPU model."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return nproc, model


def cpu_baseline(x0, k0, layers_host, ctx, seconds):
    """The oracle, as it stands, on sequence 0 of the first cache copy: every
    group run of a step per iteration (one query-token each), repeated for
    ~`seconds`.  `cores` is the thread count it runs with: numpy's BLAS pool
    (the rest of the oracle is single-threaded numpy)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count()
    nproc, model = host_cpu()
    nib, sc, k8, ks = oracle.quantize_kv(x0, 1, k0)          # setup, untimed
    kv = dict(nib=[nib], scale=[sc], k8=[k8], ks=[ks])
    runs = []
    for run in range(len(layers_host)):
        ls = []
        for j, L in enumerate(layers_host[run]):
            d = dict(mode=L["mode"], q=L["q"][:1], swa=L["swa"][:1])
            if "idx_q" in L:
                d["idx_q"], d["idx_w"] = L["idx_q"][:1], None
            if L["mode"] == oracle.FULL:
                d["kv"] = kv
            ls.append(d)
        runs.append(ls)
    st = oracle.new_state()
    iters, t0 = 0, time.perf_counter()
    while True:
        for ls in runs:
            oracle.run_group(ls, st, [ctx - 1], [ctx], [ctx - 128])
        iters += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    plans = ", ".join("+".join("F" if L["mode"] == oracle.FULL else "R" if L["mode"] == oracle.REINDEX else "U"
                               for L in ls) for ls in runs)
    return {"value": len(runs) * iters / el, "unit": "query-tokens/s", "cores": int(cores), "kind": "oracle",
            "nproc": nproc, "cpu_model": model,
            "sample": f"sequence 0 of the batch, group runs ({plans}) = {len(runs)} query-token(s) per "
                      f"iteration, {iters} iterations in {el:.1f} s; cache encoding excluded"}


MFMA_FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8, published


def prefill(args):
    """The prefill chunk step: encode the chunk's 4,096 tokens into 2,048
    entries (ratio-2 pair mean), index every query row on fp8 MFMA, and run
    the 1 Full + 5 Reuse attention layers over 4,096 query rows."""
    import torch

    import csa2_inputs as gen
    import sparse_attention_decode_fp4_amd as csa2

    dev = "cuda"
    c = gen.CONFIGS[4]
    P, T = c["prefix_tokens"], c["chunk"]
    seed = 1004
    n_prefix, n_ent = P // 2, (P + T) // 2
    nib = torch.empty((n_ent, 256), dtype=torch.uint8, device=dev)
    sc = torch.empty((n_ent, 32), dtype=torch.uint8, device=dev)
    k8 = torch.empty((n_ent, 64), dtype=torch.uint8, device=dev)
    ks = torch.empty((n_ent,), dtype=torch.float32, device=dev)
    x = gen.latent(P + T, seed, device=dev)
    kin = gen.index_key(P + T, seed, device=dev)
    csa2.csa2_quantize_kv(x[:P], ratio=2, k_in=kin[:P],
                          out=[nib[:n_prefix], sc[:n_prefix], k8[:n_prefix], ks[:n_prefix]])
    xc, kc = x[P:].contiguous(), kin[P:].contiguous()
    del x, kin
    kv = csa2.make_kv(nib, sc, k8, ks, n_ent)
    swa_pos0 = P - 127
    layers = []
    for j, m in enumerate(c["plans"][0]):
        d = dict(mode=csa2.MODE_FULL if m == "F" else csa2.MODE_REUSE,
                 q=gen.attn_query((1, T), seed, j, device=dev),
                 swa=gen.window_rows(1, P + T - swa_pos0, seed, j, device=dev),
                 out=torch.empty((1, T, 16, 512), dtype=torch.float32, device=dev))
        if m == "F":
            d["idx_q"], d["kv"] = gen.index_query((1, T), seed, j, device=dev), kv
        layers.append(d)
    ws = csa2.Workspace(1, T, n_ent)
    st = csa2.State(1, T)
    chunk_out = [nib[n_prefix:], sc[n_prefix:], k8[n_prefix:], ks[n_prefix:]]

    def step():
        csa2.csa2_quantize_kv(xc, ratio=2, k_in=kc, out=chunk_out)
        csa2.csa2_run_group(ws, st, layers, [P], [n_ent], [swa_pos0], ratio=2)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    csa2.csa2_profile_reset()
    csa2.csa2_profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    csa2.csa2_profile_enable(False)
    kern = {}
    for kid, name in enumerate(csa2.KERNEL_NAMES):
        ms, n = csa2.csa2_profile_read(kid)
        if n:
            kern[name] = {"avg_us": round(1000.0 * ms / n, 3), "launches_per_step": n / args.steps}
    fms, fn = csa2.csa2_profile_read(csa2.K_PREFILL_FILTER)
    # visible (query, entry) pairs: query i at token P + i sees (P + i + 1) // 2 entries
    pairs = sum((P + i + 1) // 2 for i in range(T))
    flops = 2 * pairs * 4 * 64
    filt_s = fms / 1000.0 / fn
    achieved = flops / filt_s / 1e12
    line = {
        "metric": "CSA2 prefill chunk query-tokens/s (4,096-token chunk, 262,144-token prefix)",
        "value": round(T * args.steps / el, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(1000.0 * el / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "prefill chunk: 4,096 query tokens at ratio 2 on a 262,144-token prefix, "
                               "1 Full + 5 Reuse layers, top-512 + 128-token window",
                   "prefix_tokens": P, "chunk": T, "entries": n_ent, "layers": 6, "timing": "eager"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "k_prefill_mfma (filter pass)", "flops_per_launch": flops,
                     "avg_launch_us": round(filt_s * 1e6, 3)},
        "kernels": kern,
    }
    print(json.dumps(line), flush=True)


def append_timing(csa2, gen, B, dev, launches=200):
    """The write side of a decode step, timed apart from the step: one
    csa2_append per launch puts a new token of each of the B sequences into
    the FP4 cache and indexer keys, updates its block key and writes its
    bf16 window row (HIP events around each launch).  The cache here is a
    small one: the append's cost does not depend on the context."""
    import torch
    stride, ring, pos = 1024, 128, 1005
    nib = torch.zeros((B * stride, 256), dtype=torch.uint8, device=dev)
    sc = torch.zeros((B * stride, 32), dtype=torch.uint8, device=dev)
    k8 = torch.zeros((B * stride, 64), dtype=torch.uint8, device=dev)
    ks = torch.zeros((B * stride,), dtype=torch.float32, device=dev)
    bk8 = torch.zeros((B * stride // 8, 64), dtype=torch.uint8, device=dev)
    bks = torch.zeros((B * stride // 8,), dtype=torch.float32, device=dev)
    swa = torch.zeros((B, ring, 512), dtype=torch.bfloat16, device=dev)
    x = gen.latent(B, 77, device=dev)
    k = gen.index_key(B, 77, device=dev)

    def one():
        csa2.csa2_append(x, k, [pos] * B, nib, sc, k8, ks, stride, bk8=bk8, bkscale=bks, bk_stride=stride // 8,
                         swa=swa, swa_ring=ring)

    for _ in range(10):
        one()
    torch.cuda.synchronize()
    csa2.csa2_profile_reset()
    csa2.csa2_profile_enable(True)
    for _ in range(launches):
        one()
    torch.cuda.synchronize()
    csa2.csa2_profile_enable(False)
    ms, n = csa2.csa2_profile_read(csa2.K_APPEND)
    csa2.csa2_profile_reset()
    # bytes per launch: x and k read, entry (288 + 68 B) and block key (68 B)
    # written, the block's earlier keys re-read (pos % 8 of them), window row
    return {"kernel": "k_append", "sequences": B, "avg_us": round(1000.0 * ms / n, 3),
            "bytes_per_launch": B * (512 * 4 + 64 * 4 + 288 + 68 + 68 + (pos % 8) * 68 + 1024)}


def graph_replay_seconds(torch, step, n_cycle, steps, warmup, per_graph=4):
    """Time `steps` steps replayed from captured HIP graphs.  A cycle of
    n_cycle steps goes through every cache copy once; it is captured as
    graphs of up to per_graph consecutive steps each (as a serving loop
    captures the layer groups of a forward pass), so a graph launch (about
    8 us here) is paid once per graph rather than once per step.  A step
    that does not start a whole graph in the remaining count replays a
    one-step graph.  Returns the seconds of the timed replays (exactly
    `steps` steps)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    groups, singles = [], []
    with torch.cuda.stream(s):
        for g0 in range(0, n_cycle, per_graph):
            n = min(per_graph, n_cycle - g0)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for i in range(g0, g0 + n):
                    step(i)
            groups.append((g, n))
        for i in range(n_cycle):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step(i)
            singles.append(g)
    torch.cuda.current_stream().wait_stream(s)
    at = [0]  # the next step's index in the cycle

    def run(n):
        done = 0
        while done < n:
            k = at[0]
            g, cnt = groups[k // per_graph]
            if k % per_graph == 0 and cnt <= n - done:
                g.replay()
            else:
                cnt = 1
                singles[k].replay()
            done += cnt
            at[0] = (k + cnt) % n_cycle

    # warm up over whole cycles: the timed replays then start a graph, on
    # copies the last warm-up step did not touch
    run(-(-warmup // n_cycle) * n_cycle)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def hier(args):
    """The hierarchical Full layer at 1M context, batch 4: block-key scan and
    top-2,048 blocks, pool scan and top-512, then attention over the 512
    entries and the 128-token window.  The indexer keys and block keys are
    rotated over 8 copies (each 285 MB) so the Infinity Cache cannot hold
    them between steps; the FP4 main cache is one copy (only 512 entries per
    query are gathered)."""
    import torch

    import csa2_inputs as gen
    import sparse_attention_decode_fp4_amd as csa2

    dev = "cuda"
    c = gen.CONFIGS[3]
    B, ctx, C = c["batch"], c["ctx"], 8
    seed = 1003
    chunk = 1 << 17
    nib = torch.empty((B * ctx, 256), dtype=torch.uint8, device=dev)
    sc = torch.empty((B * ctx, 32), dtype=torch.uint8, device=dev)
    copies = []
    zbuf = torch.zeros((chunk, 512), dtype=torch.float32, device=dev)
    scratch = [torch.empty((chunk, 256), dtype=torch.uint8, device=dev),
               torch.empty((chunk, 32), dtype=torch.uint8, device=dev)]
    for ci in range(C):
        k8 = torch.empty((B * ctx, 64), dtype=torch.uint8, device=dev)
        ks = torch.empty((B * ctx,), dtype=torch.float32, device=dev)
        for b in range(B):
            k = gen.index_key(ctx, seed + 100 * ci, seq=b, device=dev)
            for r0 in range(0, ctx, chunk):
                sl = slice(b * ctx + r0, b * ctx + r0 + chunk)
                if ci == 0:  # copy 0 also writes the FP4 main cache
                    xs = gen.normal((chunk, 512), seed, "latent", layer=r0 // chunk, seq=b, device=dev)
                    out_main = [nib[sl], sc[sl]]
                else:  # other copies encode indexer keys only
                    xs, out_main = zbuf, scratch
                csa2.csa2_quantize_kv(xs, k_in=k[r0:r0 + chunk], out=out_main + [k8[sl], ks[sl]])
            del k
        bk8, bks = csa2.csa2_build_block_keys(k8, ks, [ctx] * B, ctx)
        copies.append(csa2.make_kv(nib, sc, k8, ks, ctx, bk8, bks, (ctx + 7) // 8))
    torch.cuda.synchronize()
    q_pos0, n_entries, swa_pos0 = [ctx - 1] * B, [ctx] * B, [ctx - 128] * B
    layer = dict(mode=csa2.MODE_FULL, q=gen.attn_query((B, 1), seed, 0, device=dev),
                 swa=gen.window_rows(B, 128, seed, 0, device=dev),
                 out=torch.empty((B, 1, 16, 512), dtype=torch.float32, device=dev),
                 idx_q=gen.index_query((B, 1), seed, 0, device=dev))
    ws = csa2.Workspace(B, 1, ctx)
    states = [csa2.State(B, 1, with_pool=True) for _ in range(C)]

    def step(i):
        L = dict(layer)
        L["kv"] = copies[i % C]
        csa2.csa2_run_group(ws, states[i % C], [L], q_pos0, n_entries, swa_pos0, index_kind=csa2.INDEX_HIER)

    for i in range(C + args.warmup):
        step(i)
    torch.cuda.synchronize()
    csa2.csa2_profile_reset()
    csa2.csa2_profile_enable(True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0
    csa2.csa2_profile_enable(False)
    kern = {}
    for kid, name in enumerate(csa2.KERNEL_NAMES):
        ms, n = csa2.csa2_profile_read(kid)
        if n:
            kern[name] = {"avg_us": round(1000.0 * ms / n, 3), "launches_per_step": n / args.steps}
    scan_ms, _ = csa2.csa2_profile_read(csa2.K_INDEX_SCAN)
    graph_s = None
    if not args.no_graph:
        graph_s = graph_replay_seconds(torch, step, C, args.steps, args.warmup, per_graph=C)
    best_s = min(eager_s, graph_s) if graph_s is not None else eager_s
    # the two scans of a step: every block key once, then the 16,384-position pool
    scan_bytes = B * ((ctx + 7) // 8) * KEY_BYTES + B * 2048 * 8 * KEY_BYTES
    scan_s = scan_ms / 1000.0 / args.steps
    achieved = scan_bytes / scan_s / 1e9
    line = {
        "metric": "CSA2 hierarchical decode query-tokens/s at 1M ctx (batch 4, one Full layer)",
        "value": round(B * args.steps / best_s, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(1000.0 * best_s / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "hierarchical Full layer: 131,072 block keys, top-2,048 blocks, 16,384-position "
                               "pool, top-512, attention with a 128-token window; batch 4, 1,048,576 entries",
                   "batch": B, "ctx": ctx, "key_copies": C,
                   "timing": "graph replay" if best_s == graph_s else "eager"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_index_scan (block scan + pool scan per step)", "bytes_per_step": scan_bytes,
                     "scan_us_per_step": round(scan_s * 1e6, 3)},
        "eager_ms_per_step": round(1000.0 * eager_s / args.steps, 4),
        "graph_ms_per_step": None if graph_s is None else round(1000.0 * graph_s / args.steps, 4),
        "kernels": kern,
    }
    print(json.dumps(line), flush=True)


COPY_BYTES = 256 << 20


def stream_copy(reps=20):
    """The device's streaming rate: a plain copy of 1 GiB (read + write),
    HIP events around `reps` copies, against the published HBM peak."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    b.synchronize()
    s = a.elapsed_time(b) / 1000.0 / reps
    gbs = 2 * 4 * n / s / 1e9
    del src, dst
    return {"kind": "device copy of 1 GiB (read + write)", "GBs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def calibrate_copy():
    """A plain device-to-device copy of COPY_BYTES, five times: under
    rocprofv3 --pmc FETCH_SIZE (or WRITE_SIZE) each dispatch should read (and
    write) COPY_BYTES; the ratio to the counter's reading scales the counters
    taken on the library's kernels."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "dispatches": 5}), flush=True)


def scan_traffic(path=os.path.join(ROOT, "profiles", "k_index_scan_decode128k_b16_traffic.txt")):
    """HBM bytes per k_index_scan launch from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on other kernel source."""
    import hashlib
    try:
        with open(path) as f:
            fields = dict(line.split(":", 1) for line in f if line.startswith("@"))
    except OSError:
        return None
    src = os.path.join(ROOT, "sparse_attention_decode_fp4_amd", "csrc", "index.hip")
    with open(src, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if fields.get("@index_hip_sha256", "").strip() != digest:
        return None
    return int(fields["@traffic_bytes_per_launch"])


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(sequences are independent: a multi-GPU run would shard them by rank).", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.workload == "prefill":
        prefill(args)
        return
    if args.workload == "hier":
        hier(args)
        return
    import numpy as np
    import torch

    import csa2_inputs as gen
    import sparse_attention_decode_fp4_amd as csa2

    dev = "cuda"
    B, ctx, C = args.batch, args.ctx, args.copies
    lognormal = False
    if args.workload in ("full64k", "tiny4k", "heads64k"):  # the Full-layer decode configurations
        c = gen.CONFIGS[0 if args.workload == "tiny4k" else 1]
        B, ctx, lognormal = c["batch"], c["ctx"], c["lognormal"]
    full_only = args.workload in ("full64k", "tiny4k", "heads64k")
    key_heads = 4 if args.workload == "heads64k" else 1
    key_bytes = 64 * key_heads + 4
    nq = 4 if args.workload == "multi" else 1   # query tokens per sequence per step
    paged, page = args.workload == "paged", args.page_size
    if paged and ctx % page:
        raise SystemExit("--ctx must be a multiple of --page-size")
    if full_only and B * ctx * key_bytes >= (16 << 20):
        # a copy comes back after the other copies' scans: at least 1 GiB of
        # them (64K: 32 copies of 35.7 MB), so the 256 MB Infinity Cache does
        # not serve the scan (the 4K configuration fits it whatever the copies)
        C = max(C, -(-(1 << 30) // (B * ctx * key_bytes)) + 1)
    seed = 1002
    # ---- caches: C copies, each its own draw
    kvs, keep = [], []
    for c in range(C):
        nib = torch.empty((B * ctx, 256), dtype=torch.uint8, device=dev)
        sc = torch.empty((B * ctx, 32), dtype=torch.uint8, device=dev)
        k8 = torch.empty((B * ctx, 64 * key_heads), dtype=torch.uint8, device=dev)
        ks = torch.empty((B * ctx,), dtype=torch.float32, device=dev)
        for b in range(B):
            x = gen.latent(ctx, seed + 100 * c, seq=b, lognormal=lognormal, device=dev)
            sl = slice(b * ctx, (b + 1) * ctx)
            if key_heads == 4:
                k = gen.normal((ctx, 4, 64), seed + 100 * c, "idxk4", seq=b, device=dev)
                csa2.csa2_quantize_kv(x, out=[nib[sl], sc[sl]])
                csa2.csa2_quantize_head_keys(k, out=[k8[sl].view(ctx, 4, 64), ks[sl]])
            else:
                k = gen.index_key(ctx, seed + 100 * c, seq=b, device=dev)
                csa2.csa2_quantize_kv(x, k_in=k, out=[nib[sl], sc[sl], k8[sl], ks[sl]])
            del x, k
        if paged:
            # the same cache as a pool of pages in a random order, with its
            # page table (setup, untimed)
            n_pages = B * ctx // page
            perm = torch.from_numpy(np.random.default_rng(seed + c).permutation(n_pages)).to(dev)
            arrs = []
            for a in (nib, sc, k8, ks):
                pool = torch.empty_like(a)
                pool.view(n_pages, page, -1)[perm] = a.view(n_pages, page, -1)
                arrs.append(pool)
            del nib, sc, k8, ks
            nib, sc, k8, ks = arrs
            table = perm.to(torch.int32).view(B, ctx // page).contiguous()
            kvs.append(csa2.make_kv(nib, sc, k8, ks, 0, pages=csa2.make_pages(table, page, n_pages * page)))
            keep.append((nib, sc, k8, ks, table))
        else:
            kvs.append(csa2.make_kv(nib, sc, k8, ks, ctx, key_heads=key_heads))
            keep.append((nib, sc, k8, ks))
    torch.cuda.synchronize()
    # ---- per-layer inputs of the two runs (shared by the copies)
    q_pos0, n_entries, swa_pos0 = [ctx - nq] * B, [ctx] * B, [ctx - nq - 127] * B
    plans = [["F"]] if full_only else [["F", "U", "U", "U"], ["R", "U", "U", "U"]]
    mode_of = {"F": csa2.MODE_FULL, "R": csa2.MODE_REINDEX, "U": csa2.MODE_REUSE}
    layers = []
    for run, plan in enumerate(plans):
        ls = []
        for j, m in enumerate(plan):
            li = 4 * run + j
            d = dict(mode=mode_of[m], q=gen.attn_query((B, nq), seed, li, device=dev),
                     swa=gen.window_rows(B, 127 + nq, seed, li, device=dev),
                     out=torch.empty((B, nq, 16, 512), dtype=torch.float32, device=dev))
            if m in "FR":
                d["idx_q"] = gen.index_query((B, nq), seed, li, device=dev)
            ls.append(d)
        layers.append(ls)
    ws = csa2.Workspace(B, nq, ctx)
    states = [csa2.State(B, nq) for _ in range(C)]

    def run_full(c):
        ls = [dict(L) for L in layers[0]]
        ls[0]["kv"] = kvs[c]
        csa2.csa2_run_group(ws, states[c], ls, q_pos0, n_entries, swa_pos0)

    def run_reindex(c):
        csa2.csa2_run_group(ws, states[c], layers[1], q_pos0, n_entries, swa_pos0)

    def step(i):
        if full_only:
            run_full(i % C)
            return
        run_full((2 * i) % C)
        run_reindex((2 * i + 1) % C)

    for c in range(C):  # every state gets its own Full layer first
        run_full(c)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed loop (eager), with the library's HIP-event kernel timing on
    csa2.csa2_profile_reset()
    csa2.csa2_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0
    csa2.csa2_profile_enable(False)
    kern = {}
    for kid, name in enumerate(csa2.KERNEL_NAMES):
        ms, n = csa2.csa2_profile_read(kid)
        if n:
            kern[name] = {"avg_us": round(1000.0 * ms / n, 3), "launches_per_step": n / args.steps}
    scan_ms, scan_n = csa2.csa2_profile_read(csa2.K_INDEX_SCAN)
    csa2.csa2_profile_reset()

    # ---- timed loop replaying captured graphs (a cycle over every copy per graph)
    graph_s = None
    if not args.no_graph:
        graph_s = graph_replay_seconds(torch, step, C if full_only else C // 2, args.steps, args.warmup)

    best_s = min(eager_s, graph_s) if graph_s is not None else eager_s
    append = append_timing(csa2, gen, B, dev) if nq == 1 and not paged else None
    copy = stream_copy()
    n_runs, n_layers = len(plans), len(plans[0])
    qtok_per_step = n_runs * B * nq
    value = qtok_per_step * args.steps / best_s
    step_bytes = int(n_runs * B * nq * algorithmic_bytes_per_qtok(ctx, nq, n_layers, key_bytes))
    scan_bytes = B * ctx * key_bytes                       # one launch scans every sequence once
    scan_avg_s = scan_ms / 1000.0 / scan_n
    achieved = scan_bytes / scan_avg_s / 1e9
    line = {
        "metric": (f"CSA2 multi-token decode query-tokens/s at 128K ctx ({nq} query tokens per sequence)" if nq > 1 else
                   f"CSA2 decode query-tokens/s at 128K ctx, paged KV ({page}-entry pages)" if paged else
                   f"CSA2 Full-layer decode query-tokens/s, batch {B} at {ctx} ctx"
                   + (", per-head indexer keys" if key_heads == 4 else "") if full_only else
                   "CSA2 decode query-tokens/s at 128K ctx; % of peak HBM GB/s"),
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1000.0 * best_s / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": (f"one Full layer, batch {B}, {ctx} FP4 entries per sequence"
                                + (" (N(0,1) latents times lognormal(0, 0.5) channel scales)" if lognormal else "")
                                + (", per-head 4 x 64 fp8 indexer keys (260 B per entry)" if key_heads == 4 else "")
                                + ", top-512 + 128-token window") if full_only else
                               (f"decode group of 4 layers run as Full+3 Reuse then Reindex+3 Reuse, "
                                f"batch {B}, {ctx} FP4 entries per sequence, top-512 + 128-token window"
                                + ("" if nq == 1 else f", {nq} query tokens per sequence")
                                + ("" if not paged else f", caches as a pool of {page}-entry pages in random order")),
                   "batch": B, "ctx": ctx, "query_tokens_per_sequence": nq, "layers_per_step": n_runs * n_layers,
                   "query_tokens_per_step": qtok_per_step,
                   "cache_copies": C, "timing": "graph replay" if best_s == graph_s else "eager"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": scan_traffic() if args.workload == "decode" else None,
                     "kernel": "k_index_scan", "bytes_per_launch": scan_bytes,
                     "avg_launch_us": round(scan_avg_s * 1e6, 3),
                     "frac_of_stream_copy": round(achieved / copy["GBs"], 4)},
        "stream_copy": copy,
        "step_hbm": {"algorithmic_bytes": step_bytes,
                     "achieved_GBs": round(step_bytes * args.steps / best_s / 1e9, 1),
                     "frac": round(step_bytes * args.steps / best_s / 1e9 / HBM_PEAK_GBS, 4)},
        "eager_ms_per_step": round(1000.0 * eager_s / args.steps, 4),
        "graph_ms_per_step": None if graph_s is None else round(1000.0 * graph_s / args.steps, 4),
        "kernels": kern,
        "append": append,
    }
    if not args.no_cpu_baseline and nq == 1 and not paged:
        x0 = gen.latent(ctx, seed, seq=0, lognormal=lognormal, device=dev).cpu().numpy()
        k0 = (gen.normal((ctx, 4, 64), seed, "idxk4", seq=0, device=dev) if key_heads == 4 else
              gen.index_key(ctx, seed, seq=0, device=dev)).cpu().numpy()
        host_layers = []
        for run in range(n_runs):
            hl = []
            for L in layers[run]:
                h = dict(mode=L["mode"], q=gen.bf16_bits(L["q"]), swa=gen.bf16_bits(L["swa"]))
                if "idx_q" in L:
                    h["idx_q"] = L["idx_q"].cpu().numpy()
                hl.append(h)
            host_layers.append(hl)
        line["cpu_baseline"] = cpu_baseline(x0, k0, host_layers, ctx, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
