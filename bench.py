"""Benchmark: one decode step of query-aware sparse attention over a paged KV
cache on one MI355X, at 32K context and batch 32 (Llama-3.1-8B-shaped layer:
32 q / 8 KV heads, head_dim 128, pages of 16 tokens; budget 1 sink + 8 local
+ top-119 pages).

A step = append of the current token (K/V write + page-summary update),
score_pages, select_topk, sparse_paged_decode (attention + split merge), all
HIP kernels behind the C ABI, on inputs resident in HBM.  Steps rotate over
independent layer caches so that no step finds the previous step's data in
the 256 MB Infinity Cache.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]

--reuse R measures cross-layer selection reuse instead: a group of R + 1
layers sharing the page table, where the first layer runs the whole step and
the next R layers append their token and attend over its selection
(qasp_decode_step_reuse); one JSON line with the per-layer figures.

--drafts N measures the multi-query step instead (qasp_decode_step_multi):
N draft tokens per sequence appended, one shared selection, causal attention
per draft; value = draft tokens checked per second.

--quant R measures 2-bit quantised pages instead (qasp_decode_step_quant):
every page outside the last R of a sequence read from the quantised pool.

--host-pool measures the host-tier pool instead: K/V pools in pinned host
memory mapped into the GPU (qasp_host_alloc), summaries in HBM; the step's
attention reads the selected pages over the host link.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "llama8b_b32_32k"
METRIC = "decode tokens/s and achieved KV GB/s (% of MI355X HBM peak), 32K ctx, batch 32"


# the sources the one-kernel step is compiled from (its file and every header it includes)
FUSED_STEP_SOURCES = ("query_aware_sparse_paged_amd/csrc/fused_gqa.hip", "query_aware_sparse_paged_amd/csrc/attend_core.h",
                      "query_aware_sparse_paged_amd/csrc/common.h", "query_aware_sparse_paged_amd/csrc/launch.h",
                      "query_aware_sparse_paged_amd/csrc/quant_core.h", "query_aware_sparse_paged_amd/csrc/score_core.h",
                      "query_aware_sparse_paged_amd/csrc/select_core.h", "include/qasp.h")


def kernel_source_hash(files=FUSED_STEP_SOURCES):
    """First 16 hex digits of the sha256 over the named sources (path and
    contents): a counter record taken on other sources is stale."""
    import hashlib
    h = hashlib.sha256()
    for rel in sorted(files):
        h.update(rel.encode())
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter record, or None
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "%s_%s_traffic.json" % (kernel.replace("_kernel", ""), workload))
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bytes(w, msel_counts):
    """Algorithmic bytes of one step (what the method must move), split into
    the scoring side (the 512 B summary of every candidate page-head, and each
    sequence's page-table row once) and the attention side (the K and V tiles
    of every selected page-head, q once, the fp32 output)."""
    s = w.spec
    lens = w.seq_lens.cpu().tolist()
    summ_b = 2 * s.head_dim_k * 2
    kv_b = s.page_size * (s.head_dim_k + (0 if s.v_from_k else s.head_dim_v)) * 2
    score = decode = 0
    for b, L in enumerate(lens):
        P = (L + s.page_size - 1) // s.page_size
        score += P * 4
        for g in range(s.num_kv_heads):
            if not (s.static_heads and s.static_heads[g]):
                score += max(0, P - s.n_sink_pages - s.n_local_pages) * summ_b
            decode += int(msel_counts[b][g]) * kv_b
    decode += s.batch * s.num_q_heads * (s.head_dim_k * 2 + s.head_dim_v * 4)
    return score, decode


def auto_layers(spec):
    """Layer caches to rotate so that at least 512 MB (twice the 256 MB
    last-level cache) is touched between two steps on one cache: the bytes a
    step touches are estimated from the full budget (summaries of every page,
    K/V of the selected pages)."""
    ps = spec.page_size
    P = (spec.seq_len + ps - 1) // ps
    sel = min(P, spec.n_sink_pages + spec.n_local_pages + spec.top_k)
    kv = ps * (spec.head_dim_k + (0 if spec.v_from_k else spec.head_dim_v)) * 2
    per_step = spec.batch * spec.num_kv_heads * (P * 4 * spec.head_dim_k + sel * kv)
    return max(3, min(16, -(-2 * 256 * 2 ** 20 // max(1, per_step)) + 1))


def cpu_info():
    """(CPU model, nproc, CPUs this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    nproc = os.cpu_count() or 1
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = nproc
    return model, nproc, usable


def oracle_threads(usable):
    """All usable CPUs, capped by OMP_NUM_THREADS when it is set."""
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return max(1, min(usable, cap) if cap > 0 else usable)


def _oracle_inputs(w, seqs):
    """The sequences' pages re-packed into a small host pool (bit patterns),
    their summaries computed by the oracle (not timed)."""
    import numpy as np
    import oracle
    from query_aware_sparse_paged_amd import workloads

    s = w.spec
    pt_full = w.page_table[seqs]
    valid = pt_full >= 0
    phys = pt_full[valid].long()
    k = workloads.bits(w.k_pool[phys.to(w.k_pool.device)])
    v = None if w.v_pool is None else workloads.bits(w.v_pool[phys.to(w.v_pool.device)])
    pt = np.full(tuple(pt_full.shape), -1, np.int32)
    pt[valid.cpu().numpy()] = np.arange(phys.numel(), dtype=np.int32)
    sl = w.seq_lens[seqs].cpu().numpy()
    q = workloads.bits(w.q[seqs])
    lay = oracle.Layout(int(phys.numel()), s.page_size, s.num_kv_heads, s.head_dim_k, s.head_dim_v, s.v_from_k)
    pol = oracle.Policy(s.n_sink_pages, s.n_local_pages, s.top_k, s.sink_tokens, s.window_tokens, s.static_heads)
    summ = oracle.summaries(lay, pt, sl, s.num_q_heads, k)
    return lay, pol, pt, sl, q, k, v, summ


def _time_oracle(w, inputs, msel, threads, runs=3):
    """Median wall time of the oracle's decode step (scores + selection +
    attention over the precomputed summaries) and its selection counts."""
    import oracle
    lay, pol, pt, sl, q, k, v, summ = inputs
    times, cnt = [], None
    for _ in range(runs):
        t0 = time.perf_counter()
        _, _, cnt = oracle.decode(lay, pt, sl, q, k, v, summ, pol, w.scale, num_threads=threads, max_sel_n=msel)
        times.append(time.perf_counter() - t0)
    return statistics.median(times), cnt


def cpu_baseline(w, msel, one_thread_seqs=4):
    """The CPU oracle (test infrastructure), timed on this machine's host CPUs
    over the whole workload (every sequence and KV head, one decode step over
    precomputed summaries), with all usable CPUs and with one thread on a
    bounded sample; and the tiny one-sequence workload at both thread counts.
    Rates are tokens/s and GB/s over the same algorithmic bytes as the GPU
    figure."""
    from query_aware_sparse_paged_amd import workloads

    model, nproc, usable = cpu_info()
    threads = oracle_threads(usable)
    s = w.spec
    t_all = time.perf_counter()
    seqs = list(range(s.batch))
    inp = _oracle_inputs(w, seqs)
    msel_all = msel
    dt, cnt = _time_oracle(w, inp, msel_all, threads)
    b_sc, b_dec = step_bytes(w, cnt.tolist())
    one = {}
    sub = list(range(min(one_thread_seqs, s.batch)))
    inp1 = _oracle_inputs(w, sub)
    dt1, cnt1 = _time_oracle(w, inp1, msel_all, 1)
    b1 = sum(step_bytes_of(w, sub, cnt1.tolist()))
    one[s.name] = {"tokens_per_s": round(len(sub) / dt1, 2), "gbps": round(b1 / dt1 / 1e9, 3),
                   "sample": "%d of %d sequences" % (len(sub), s.batch)}
    tiny = workloads.make("tiny_b1_4k", device="cpu")
    from query_aware_sparse_paged_amd import api
    tmsel = api.max_sel(api.layout_of(tiny), api.policy_of(tiny), tiny.max_pages)
    tin = _oracle_inputs(tiny, [0])
    tiny_rates = {}
    for n in (1, threads):
        tdt, tcnt = _time_oracle(tiny, tin, tmsel, n, runs=5)
        tb = sum(step_bytes(tiny, tcnt.tolist()))
        tiny_rates[n] = (round(1 / tdt, 2), round(tb / tdt / 1e9, 3))
    one["tiny_b1_4k"] = {"tokens_per_s": tiny_rates[1][0], "gbps": tiny_rates[1][1], "sample": "the whole workload"}
    total_s = time.perf_counter() - t_all
    return {"value": round(s.batch / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "the whole workload (%d sequences, all %d KV heads): one decode step over precomputed "
                      "summaries, median of 3 runs, %.3f s each; %d threads" % (s.batch, s.num_kv_heads, dt, threads),
            "gbps": round((b_sc + b_dec) / dt / 1e9, 3),
            "nproc": nproc, "usable_cpus": usable, "cpu_model": model,
            "one_thread": one,
            "tiny_b1_4k_all_threads": {"tokens_per_s": tiny_rates[threads][0], "gbps": tiny_rates[threads][1]},
            "wall_s": round(total_s, 1)}


def step_bytes_of(w, seqs, counts):
    """step_bytes restricted to the sequences seqs (counts: their rows)."""
    import copy
    sub = copy.copy(w)
    sub.spec = copy.copy(w.spec)
    sub.spec.batch = len(seqs)
    sub.seq_lens = w.seq_lens[seqs]
    return step_bytes(sub, counts)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--layers", type=int, default=0,
                    help="independent layer caches rotated over (0: enough that at least 512 MB, twice the "
                         "last-level cache, is touched between two visits of a cache; at least 3, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reuse", type=int, default=0,
                    help="cross-layer reuse: per group, 1 selecting layer + this many reusing layers")
    ap.add_argument("--drafts", type=int, default=0,
                    help="multi-query step: this many draft tokens per sequence")
    ap.add_argument("--quant", type=int, default=0,
                    help="2-bit quantised pages outside a residual region of this many pages")
    ap.add_argument("--host-pool", action="store_true",
                    help="K/V pools in pinned host memory mapped into the GPU")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this size first (a known-size kernel for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the per-(sequence, KV head) work would shard by batch or KV head with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from query_aware_sparse_paged_amd import api, workloads

    if args.layers <= 0:
        args.layers = auto_layers(workloads.SPECS[args.workload])
    dev = torch.device("cuda:0")
    if args.reuse > 0:
        return run_reuse(args, torch, api, workloads, dev)
    if args.drafts > 0:
        return run_drafts(args, torch, api, workloads, dev)
    if args.host_pool:
        return run_host_pool(args, torch, api, workloads, dev)
    if args.quant > 0:
        return run_quant(args, torch, api, workloads, dev)
    layers = []
    for i in range(args.layers):
        base = workloads.SPECS[args.workload].seed
        w = workloads.make(args.workload, seed=base + 100 * i, device=dev)
        lay, pol = api.layout_of(w), api.policy_of(w)
        bat = api.Batch(w.page_table, w.seq_lens, w.spec.num_q_heads)
        bat_before = api.Batch(w.page_table, (w.seq_lens - 1).contiguous(), w.spec.num_q_heads)
        msel = api.max_sel(lay, pol, bat.max_pages)
        summ = torch.zeros((w.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16,
                           device=dev)
        api.build_summaries(lay, bat, w.k_pool, summ)
        ws = api.new_workspace(lay, bat, pol, msel, dev)
        B = w.spec.batch
        layers.append(dict(w=w, lay=lay, pol=pol, bat=bat, bat_before=bat_before, msel=msel, summ=summ, ws=ws,
                           scores=torch.empty((B, lay.num_kv_heads, bat.max_pages, 4), dtype=torch.float32,
                                              device=dev),
                           sel=torch.empty((B, lay.num_kv_heads, msel), dtype=torch.int32, device=dev),
                           cnt=torch.empty((B, lay.num_kv_heads), dtype=torch.int32, device=dev),
                           out=torch.empty((B, w.spec.num_q_heads, lay.head_dim_v), dtype=torch.float32,
                                           device=dev)))
        log("layer %d ready: pool %.2f GB" % (i, (w.k_pool.numel() + (0 if w.v_pool is None else w.v_pool.numel()))
                                               * 2 / 1e9))
    torch.cuda.synchronize()
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # one elementwise kernel: n bytes read, n bytes written
        torch.cuda.synchronize()
        log("calibration kernel (neg): %d bytes read, %d bytes written" % (n, n))
        del src, dst
    stream = torch.cuda.current_stream()
    w0 = layers[0]["w"]
    spec = w0.spec

    def step(L):
        w = L["w"]
        api.decode_step(L["lay"], L["bat"], L["pol"], w.q, w.k_pool, w.v_pool, L["summ"], w.scale, L["ws"],
                        L["msel"], k_new=w.k_new, v_new=w.v_new, out=L["out"], sel=L["sel"], sel_count=L["cnt"])

    for i in range(args.warmup):
        step(layers[i % len(layers)])
    torch.cuda.synchronize()

    # the timed region: K steps back to back, a synchronize on both sides;
    # HIP events on the launch stream bracket the same K launches, so their
    # span / K is the average launch duration as the GPU saw it (a kernel
    # trace of back-to-back launches records the same: each one's start is the
    # previous one's end)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(layers[i % len(layers)])
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    launch_ms = ev0.elapsed_time(ev1) / args.steps

    # a second pass of K steps with HIP events on the launch stream around
    # every step, for the spread of single launches (event records add a few
    # microseconds between launches, so they stay out of the timed region)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(layers[i % len(layers)])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    step_ms = sorted(a.elapsed_time(b) for a, b in evs)
    med = statistics.median
    counts = layers[0]["cnt"].cpu().tolist()
    b_score, b_decode = step_bytes(w0, counts)
    total_bytes = b_score + b_decode
    L0 = layers[0]
    one_kernel = api.decode_step_path(L0["lay"], L0["bat"], L0["pol"], L0["msel"]) == api.PATH_ONE_KERNEL
    kernel = "fused_step_gqa_kernel" if one_kernel else "decode_step (several kernels)"
    dom_ms = med(step_ms)
    achieved = total_bytes / (launch_ms * 1e-3) / 1e9
    tokens_per_s = spec.batch / (ms_per_step * 1e-3)
    gbps = total_bytes / (ms_per_step * 1e-3) / 1e9
    log("timed region: %.1f us per launch by events, %.1f us per step by wall clock; single launches: median "
        "%.1f us (p10 %.1f, p90 %.1f)" % (launch_ms * 1e3, ms_per_step * 1e3, dom_ms * 1e3,
                                         step_ms[len(step_ms) // 10] * 1e3, step_ms[(9 * len(step_ms)) // 10] * 1e3))

    stream_ref = stream_read_reference(torch, dev, total_bytes)
    log("streaming-read reference: %.1f us for the step's %d bytes (%.0f GB/s)" % (
        stream_ref["us"], total_bytes, stream_ref["gbps"]))
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w0, layers[0]["msel"])
        log("cpu oracle: %s; %.1f s in all" % (cpu["sample"], cpu["wall_s"]))

    line = {
        "metric": METRIC if spec.name == DEFAULT_WORKLOAD else
                  "decode tokens/s and achieved GB/s (%% of MI355X HBM peak), %s" % spec.name,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch, "seq_len": spec.seq_len,
                   "q_heads": spec.num_q_heads, "kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim_k,
                   "page_size": spec.page_size,
                   "pages_read": "%d sink + %d local + top-%d" % (spec.n_sink_pages, spec.n_local_pages, spec.top_k),
                   "layer_caches_rotated": args.layers},
        "kv_gbps_wall": round(gbps, 1),
        "step_bytes": total_bytes,
        "launch_us_timed_region": round(launch_ms * 1e3, 2),
        "step_us_events": {"median": round(dom_ms * 1e3, 2), "mean": round(statistics.mean(step_ms) * 1e3, 2),
                           "p10": round(step_ms[len(step_ms) // 10] * 1e3, 2),
                           "p90": round(step_ms[(9 * len(step_ms)) // 10] * 1e3, 2)},
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": profiled_traffic(kernel, spec.name) if one_kernel else None,
                     "algorithmic_bytes": total_bytes,
                     "timing": "HIP events on the launch stream around the %d timed launches, span / %d (a "
                               "rocprofv3 kernel trace of back-to-back launches records the same average)"
                               % (args.steps, args.steps)},
        "stream_read_reference": stream_ref,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def stream_read_reference(torch, dev, nbytes, reps=20):
    """What a plain streaming read of the same number of bytes takes on this
    GPU: torch's row sums over fp32 buffers of nbytes (rows of 1024, so the
    written sums are 0.1% of the bytes), three buffers rotated, HIP events
    around each launch, median.  Context for the roofline fraction (what this
    memory delivers to a sequential read), not a result."""
    rows = max(1, -(-nbytes // 4096))
    bufs = [torch.ones((rows, 1024), dtype=torch.float32, device=dev) for _ in range(3)]
    out = torch.empty(rows, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    for i in range(3):
        torch.sum(bufs[i], dim=1, out=out)
    ts = []
    for i in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.sum(bufs[i % 3], dim=1, out=out)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    us = statistics.median(ts)
    del bufs
    read = rows * 4096
    return {"bytes": read, "us": round(us, 2), "gbps": round(read / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(read / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "kernel": "torch.sum over rows of 1024 fp32, three buffers rotated"}


def run_quant(args, torch, api, workloads, dev):
    """One-token steps with 2-bit quantised pages (residual region of R
    pages), rotated over independent layer caches like the default mode."""
    R = args.quant
    layers = []
    for i in range(args.layers):
        base = workloads.SPECS[args.workload].seed
        w = workloads.make(args.workload, seed=base + 100 * i, device=dev)
        lay, pol = api.layout_of(w), api.policy_of(w)
        bat = api.Batch(w.page_table, w.seq_lens, w.spec.num_q_heads)
        msel = api.max_sel(lay, pol, bat.max_pages)
        summ = torch.zeros((w.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16,
                           device=dev)
        api.build_summaries(lay, bat, w.k_pool, summ)
        qpool = api.new_quant_pool(lay, dev)
        api.quantize_pages(lay, bat, R, w.k_pool, w.v_pool, qpool)
        B = w.spec.batch
        layers.append(dict(w=w, lay=lay, pol=pol, bat=bat, msel=msel, summ=summ, qpool=qpool,
                           ws=api.new_workspace(lay, bat, pol, msel, dev),
                           sel=torch.empty((B, lay.num_kv_heads, msel), dtype=torch.int32, device=dev),
                           cnt=torch.empty((B, lay.num_kv_heads), dtype=torch.int32, device=dev),
                           out=torch.empty((B, w.spec.num_q_heads, lay.head_dim_v), dtype=torch.float32,
                                           device=dev)))
        log("layer %d ready" % i)
    torch.cuda.synchronize()

    def step(L):
        w = L["w"]
        api.decode_step_quant(L["lay"], L["bat"], L["pol"], R, w.q, w.k_pool, w.v_pool, L["summ"], L["qpool"],
                              w.scale, L["ws"], L["msel"], k_new=w.k_new, v_new=w.v_new, out=L["out"], sel=L["sel"],
                              sel_count=L["cnt"])

    for i in range(args.warmup):
        step(layers[i % len(layers)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(layers[i % len(layers)])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    w0, spec = layers[0]["w"], layers[0]["w"].spec
    counts = layers[0]["cnt"].cpu().tolist()
    sel = layers[0]["sel"].cpu().tolist()
    lens = w0.seq_lens.cpu().tolist()
    b_score, b_decode = step_bytes(w0, counts)
    qo = spec.batch * spec.num_q_heads * (spec.head_dim_k * 2 + spec.head_dim_v * 4)
    bf16_ph = spec.page_size * (spec.head_dim_k + spec.head_dim_v) * 2
    n_q = n_r = 0
    for b in range(spec.batch):
        P = (lens[b] + spec.page_size - 1) // spec.page_size
        for g in range(spec.num_kv_heads):
            for j in sel[b][g][:counts[b][g]]:
                if j < P - R:
                    n_q += 1
                else:
                    n_r += 1
    attend_bytes = n_q * 1536 + n_r * bf16_ph + qo
    total = b_score + attend_bytes
    gbps = total / (ms_per_step * 1e-3) / 1e9
    log("quantised-page step (R=%d): %.1f us; %d quantised + %d residual page-heads read" %
        (R, ms_per_step * 1e3, n_q, n_r))
    L0 = layers[0]
    one_kernel = api.decode_step_path(L0["lay"], L0["bat"], L0["pol"], L0["msel"]) == api.PATH_ONE_KERNEL
    kernel = "fused_step_gqa_kernel (quantised form)" if one_kernel else "decode_step_quant (several kernels)"
    line = {
        "metric": "decode tokens/s with 2-bit quantised pages (residual %d pages), %s" % (R, spec.name),
        "value": round(spec.batch / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch, "seq_len": spec.seq_len, "residual_pages": R,
                   "layer_caches_rotated": args.layers},
        "step_bytes": total,
        "selected_bytes_quantised_vs_bf16": [attend_bytes - qo, b_decode - qo],
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes": total},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction


def run_host_pool(args, torch, api, workloads, dev):
    """One-token steps with the K/V pools in host-tier memory (one layer
    cache: the link does not cache, so rotation changes nothing)."""
    w = workloads.make(args.workload, device=dev)
    lay, pol, spec = api.layout_of(w), api.policy_of(w), w.spec
    bat = api.Batch(w.page_table, w.seq_lens, spec.num_q_heads)
    msel = api.max_sel(lay, pol, bat.max_pages)
    summ = torch.zeros((w.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16, device=dev)
    api.build_summaries(lay, bat, w.k_pool, summ)
    R = args.quant
    qh = None
    if R > 0:  # 2-bit pages too: the quantised pool built on the device, then moved to host memory
        qpool = api.new_quant_pool(lay, dev)
        api.quantize_pages(lay, bat, R, w.k_pool, w.v_pool, qpool)
        qh = api.host_pool_like(qpool)
        del qpool
    kh = api.host_pool_like(w.k_pool)
    vh = None if w.v_pool is None else api.host_pool_like(w.v_pool)
    w.k_pool = w.v_pool = None
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log("host-tier pools ready: %.2f GB pinned" % ((kh.buf.nbytes + (vh.buf.nbytes if vh else 0) +
                                                    (qh.buf.nbytes if qh else 0)) / 1e9))
    ws = api.new_workspace(lay, bat, pol, msel, dev)
    B = spec.batch
    sel = torch.empty((B, lay.num_kv_heads, msel), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, lay.num_kv_heads), dtype=torch.int32, device=dev)
    out = torch.empty((B, spec.num_q_heads, lay.head_dim_v), dtype=torch.float32, device=dev)

    def step():
        if qh is None:
            api.decode_step(lay, bat, pol, w.q, kh, vh, summ, w.scale, ws, msel, k_new=w.k_new, v_new=w.v_new,
                            out=out, sel=sel, sel_count=cnt)
        else:
            api.decode_step_quant(lay, bat, pol, R, w.q, kh, vh, summ, qh, w.scale, ws, msel, k_new=w.k_new,
                                  v_new=w.v_new, out=out, sel=sel, sel_count=cnt)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    b_score, b_decode = step_bytes(w, cnt.cpu().tolist())
    qo = spec.batch * spec.num_q_heads * (spec.head_dim_k * 2 + spec.head_dim_v * 4)
    kv_link = b_decode - qo  # the selected K/V tiles: read over the host link
    if qh is not None:  # quantised pages: 1536 B per page-head below the residual region
        sl_, cn_ = sel.cpu().tolist(), cnt.cpu().tolist()
        lens = w.seq_lens.cpu().tolist()
        bf16_ph = spec.page_size * (spec.head_dim_k + spec.head_dim_v) * 2
        kv_link = 0
        for b_ in range(B):
            P = (lens[b_] + spec.page_size - 1) // spec.page_size
            for g_ in range(lay.num_kv_heads):
                kv_link += sum(1536 if j < P - R else bf16_ph for j in sl_[b_][g_][:cn_[b_][g_]])
    kv_link += spec.batch * spec.num_kv_heads * (spec.head_dim_k + (0 if spec.v_from_k else spec.head_dim_v)) * 2
    link = kv_link / (ms_per_step * 1e-3) / 1e9
    log("host-tier step: %.1f us, %.1f GB/s over the host link" % (ms_per_step * 1e3, link))
    line = {
        "metric": "decode tokens/s with the K/V pools in host memory (host-tier pool)%s, %s" % (
            ", 2-bit pages outside the last %d" % R if R > 0 else "", spec.name),
        "value": round(B / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": B, "seq_len": spec.seq_len, "pools": "host-tier",
                   "residual_pages": R if R > 0 else None},
        "roofline": {"kernel": "decode step, selected pages over the host link", "bound": "host-link",
                     "achieved": round(link, 2), "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(link / HOST_LINK_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes": kv_link},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def run_drafts(args, torch, api, workloads, dev):
    """Multi-query steps (N draft tokens per sequence) rotated over independent
    layer caches; each step appends the drafts (the same values every step),
    scores and selects once per (sequence, KV head) for all drafts and attends
    causally."""
    n = args.drafts
    layers = []
    for i in range(args.layers):
        base = workloads.SPECS[args.workload].seed
        w = workloads.make(args.workload, seed=base + 100 * i, device=dev)
        lay, pol = api.layout_of(w), api.policy_of(w)
        bat = api.Batch(w.page_table, w.seq_lens, w.spec.num_q_heads)
        msel = api.max_sel_multi(lay, pol, n, bat.max_pages)
        dq, dk, dv = workloads.drafts(w, n, base + 100 * i + 1, device=dev)
        summ = torch.zeros((w.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16,
                           device=dev)
        api.build_summaries(lay, bat, w.k_pool, summ)
        B = w.spec.batch
        layers.append(dict(w=w, lay=lay, pol=pol, bat=bat, msel=msel, dq=dq, dk=dk, dv=dv, summ=summ,
                           ws=api.new_workspace_multi(lay, bat, pol, n, msel, dev),
                           sel=torch.empty((B, lay.num_kv_heads, msel), dtype=torch.int32, device=dev),
                           cnt=torch.empty((B, lay.num_kv_heads), dtype=torch.int32, device=dev),
                           out=torch.empty((B, n, w.spec.num_q_heads, lay.head_dim_v), dtype=torch.float32,
                                           device=dev)))
        log("layer %d ready" % i)
    torch.cuda.synchronize()

    def step(L):
        api.decode_step_multi(L["lay"], L["bat"], L["pol"], L["dq"], L["w"].k_pool, L["w"].v_pool, L["summ"],
                              L["w"].scale, L["ws"], L["msel"], k_new=L["dk"], v_new=L["dv"], out=L["out"],
                              sel=L["sel"], sel_count=L["cnt"])

    for i in range(args.warmup):
        step(layers[i % len(layers)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(layers[i % len(layers)])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(layers[i % len(layers)])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    step_ms = statistics.median(a.elapsed_time(b) for a, b in evs)
    w0, L0 = layers[0]["w"], layers[0]
    spec = w0.spec
    b_score, b_decode = step_bytes(w0, L0["cnt"].cpu().tolist())
    # the other drafts' queries and outputs, and every draft's key and value row written
    extra = (n - 1) * spec.batch * spec.num_q_heads * (spec.head_dim_k * 2 + spec.head_dim_v * 4)
    extra += n * spec.batch * spec.num_kv_heads * (spec.head_dim_k + spec.head_dim_v) * 2
    total = b_score + b_decode + extra
    achieved = total / (step_ms * 1e-3) / 1e9
    log("multi-query step (%d drafts): events median %.1f us, wall %.1f us/step" % (n, step_ms * 1e3,
                                                                                   ms_per_step * 1e3))
    one_kernel = api.decode_step_path(L0["lay"], L0["bat"], L0["pol"], L0["msel"]) == api.PATH_ONE_KERNEL
    kernel = "fused_step_gqa_kernel (multi-query form)" if one_kernel else "decode_step_multi (several kernels)"
    line = {
        "metric": "draft tokens checked per second, multi-query step with %d drafts per sequence, %s" % (n, spec.name),
        "value": round(spec.batch * n / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch, "seq_len": spec.seq_len, "drafts": n,
                   "layer_caches_rotated": args.layers},
        "step_us_events": round(step_ms * 1e3, 2),
        "roofline": {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None, "algorithmic_bytes": total},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def run_reuse(args, torch, api, workloads, dev):
    """Groups of 1 selecting layer + R reusing layers (same page table and
    lengths; the reusing layers' pools are the first layer's with the key
    channels reversed and the values negated, their queries reversed too, so
    every layer reads its own HBM)."""
    R = args.reuse
    w = workloads.make(args.workload, seed=workloads.SPECS[args.workload].seed, device=dev)
    lay, pol, spec = api.layout_of(w), api.policy_of(w), w.spec
    bat = api.Batch(w.page_table, w.seq_lens, spec.num_q_heads)
    msel = api.max_sel(lay, pol, bat.max_pages)
    ws = api.new_workspace(lay, bat, pol, msel, dev)
    B = spec.batch
    sel = torch.empty((B, lay.num_kv_heads, msel), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, lay.num_kv_heads), dtype=torch.int32, device=dev)
    layer = []
    for r in range(R + 1):
        if r == 0:
            kp, vp, q, kn, vn = w.k_pool, w.v_pool, w.q, w.k_new, w.v_new
        else:
            kp, q, kn = w.k_pool.flip(-1).contiguous(), w.q.flip(-1).contiguous(), w.k_new.flip(-1).contiguous()
            vp = None if w.v_pool is None else (-w.v_pool).contiguous()
            vn = None if w.v_new is None else (-w.v_new).contiguous()
        summ = torch.zeros((w.num_pool_pages, lay.num_kv_heads, 2, lay.head_dim_k), dtype=torch.bfloat16,
                           device=dev)
        api.build_summaries(lay, bat, kp, summ)
        out = torch.empty((B, spec.num_q_heads, lay.head_dim_v), dtype=torch.float32, device=dev)
        layer.append(dict(kp=kp, vp=vp, q=q, kn=kn, vn=vn, summ=summ, out=out))
        log("layer %d ready" % r)
    torch.cuda.synchronize()

    def full(L):
        api.decode_step(lay, bat, pol, L["q"], L["kp"], L["vp"], L["summ"], w.scale, ws, msel, k_new=L["kn"],
                        v_new=L["vn"], out=L["out"], sel=sel, sel_count=cnt)

    def reuse(L):
        api.decode_step_reuse(lay, bat, pol, L["q"], L["kp"], L["vp"], L["summ"], w.scale, sel, cnt, ws,
                              k_new=L["kn"], v_new=L["vn"], out=L["out"])

    def group():
        full(layer[0])
        for r in range(1, R + 1):
            reuse(layer[r])

    for _ in range(args.warmup):
        group()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        group()
    torch.cuda.synchronize()
    group_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # HIP events around each layer of a second pass
    stream = torch.cuda.current_stream()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(R + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        for r in range(R + 1):
            ev[i][r][0].record(stream)
            (full if r == 0 else reuse)(layer[r])
            ev[i][r][1].record(stream)
    torch.cuda.synchronize()
    med = statistics.median
    full_ms = med(ev[i][0][0].elapsed_time(ev[i][0][1]) for i in range(args.steps))
    reuse_ms = med(ev[i][r][0].elapsed_time(ev[i][r][1]) for i in range(args.steps) for r in range(1, R + 1))
    b_score, b_decode = step_bytes(w, cnt.cpu().tolist())
    full_bytes, reuse_bytes = b_score + b_decode, b_decode
    layer_ms = group_ms / (R + 1)
    gqa = spec.head_dim_k == spec.head_dim_v and not spec.v_from_k
    rkernel = ("fused_reuse_gqa_kernel" if gqa and B * lay.num_kv_heads >= 200
               else "append + decode kernels")
    log("group of %d layers: %.1f us wall; events: selecting layer %.1f us, reusing layer %.1f us"
        % (R + 1, group_ms * 1e3, full_ms * 1e3, reuse_ms * 1e3))
    line = {
        "metric": "decode tokens/s per layer with cross-layer selection reuse (1 selecting + %d reusing layers), %s"
                  % (R, spec.name),
        "value": round(B / (layer_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(group_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": B, "seq_len": spec.seq_len, "reusing_layers": R},
        "layer_us_events": {"selecting": round(full_ms * 1e3, 2), "reusing": round(reuse_ms * 1e3, 2)},
        "roofline": {"kernel": rkernel, "bound": "hbm", "achieved": round(reuse_bytes / (reuse_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(reuse_bytes / (reuse_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": None, "algorithmic_bytes": reuse_bytes},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
