"""Decode-step benchmark of the DSA indexer on one MI355X.

A step is the whole hot path over one batch: the score kernel (page walk,
weighted-ReLU scores, -inf tail) followed by the top-k kernels, both replayed
from a captured HIP graph. Inputs are seeded synthetic tensors already
resident in HBM; R identical copies at different addresses are used round
robin so that every step reads its keys from HBM, not from the 256 MB
Infinity Cache.

Prints one JSON line. ``value`` is valid positions scored per second over the
timed steps of the headline workload (B=64, 128K-token context, uniform
lengths). ``roofline`` prices the score kernel's valid-page key bytes per
launch against the 8 TB/s HBM peak, with its average launch duration measured
here with HIP events (median of five batches), and against two ceilings
measured in the same run by the HBM read probes (one long contiguous read,
and random 8 KiB pages read like the score kernel reads its keys).
``workloads`` holds the same figures for the all-pages-valid workload and
for the 1M-token and 8K-token row widths at 512-token lengths in both tail
modes, with the stress ratio between them. ``cpu_baseline`` times the float64
CPU oracle, requests spread over the host's cores, on the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak
MALL_BYTES = 256 << 20  # Infinity Cache
METRIC = "valid positions scored/s + µs/step at B=64,128K ctx; % of HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_kernel_traffic.txt")
SCORE_SOURCES = ["sparse_attention_kv_indexer_amd/csrc/score.hip", "sparse_attention_kv_indexer_amd/csrc/common.h"]
BATCHES = 5  # timed batches; the launch averages are their median
# Steps per captured graph (at least; a multiple of the input copies, taken in
# turn): each replay of a graph is followed by a gap of a few microseconds on
# the GPU before the next one starts, so a graph of only the R copies' steps
# (two at c3) adds about 1 us to every step. A decode step's graph holds the
# indexer of many layers.
GRAPH_STEPS = 16


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c3", help="workload name (tiny, c2, c3, stress1m, stress8k, full)")
    ap.add_argument("--rotate", type=int, default=0, help="input copies used round robin (0: enough to exceed 2x the Infinity Cache)")
    ap.add_argument("--hwm", action="store_true", help="incremental -inf tail (row_hwm) instead of the stateless full tail")
    ap.add_argument("--keys", choices=["bf16", "fp8"], default="bf16",
                    help="key format: bfloat16, or e4m3fn codes with a float32 scale per key")
    ap.add_argument("--tokens", type=int, default=1,
                    help="query tokens per request (2..4: a speculative step, every page read once for all of them)")
    ap.add_argument("--stage", choices=["indexer", "attention"], default="indexer",
                    help="indexer: the score + top-k step (default); attention: sparse attention over a "
                         "top-k-shaped selection of the same workload")
    ap.add_argument("--topk", choices=["hist", "sampled"], default="sampled",
                    help="hist: the score kernel counts each row's first-digit histogram and the top-k starts "
                         "from it (score_hist + topk_hist); sampled: the top-k samples its own cut")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only --config (no extra workloads, no stress ratio, no probes)")
    ap.add_argument("--probe", action="store_true",
                    help="only run the HBM read probes and print their JSON line")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall-clock budget of the CPU baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of known size (reference for HBM byte counters)")
    return ap.parse_args()


ATT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_kernel_traffic.txt")
ATT_SOURCES = ["sparse_attention_kv_indexer_amd/csrc/attention.hip", "sparse_attention_kv_indexer_amd/csrc/common.h"]


def source_digest(sources=SCORE_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(key: str, path: str = TRAFFIC_FILE, sources=SCORE_SOURCES):
    """HBM bytes per launch measured with rocprofv3 counters, from the
    summary under profiles/, or None when absent or taken on other source."""
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        line = line.strip()
        if line.startswith(key + " "):
            rec = dict(kv.split("=", 1) for kv in line.split()[1:])
    if rec.get("source_digest") != source_digest(sources):
        return None
    return {"read_bytes": int(rec["read_bytes"]), "write_bytes": int(rec["write_bytes"]),
            "total_bytes": int(rec["read_bytes"]) + int(rec["write_bytes"])}


def copy_calibration():
    """A plain copy of 512 MiB, five times: the reference that scales the HBM
    byte counters (FETCH_SIZE / WRITE_SIZE) to bytes."""
    import torch

    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)


def algorithmic_bytes(inp, hwm: bool, tokens: int = 1, token_lens=None) -> dict:
    """Bytes one score launch must move at minimum: every valid key row (once,
    however many query tokens read it), the logits it writes, the page-table
    entries of valid slots, and q, w and the length of every request and token."""
    import numpy as np

    from sparse_attention_kv_indexer_amd import workloads as wl

    lens = np.clip(inp.seq_lens.astype(np.int64), 0, inp.max_c4)
    if token_lens is not None:
        lens = np.clip(np.asarray(token_lens, dtype=np.int64), 0, inp.max_c4).max(axis=1)
    pages = wl.pages_needed(lens)
    per_key = wl.DIM + 4 if inp.fp8 else wl.DIM * 2  # fp8: 64 codes and a float32 scale
    k_bytes = int(pages.sum()) * wl.PAGE * per_key
    out_positions = tokens * (inp.batch * inp.max_c4 if not hwm else int((pages * wl.PAGE).sum()))
    out_bytes = out_positions * 4
    table_bytes = int(pages.sum()) * 4
    req_bytes = inp.batch * tokens * (wl.HEADS * wl.DIM * 2 + wl.HEADS * 4 + 4)
    return {"k": k_bytes, "logits": out_bytes, "page_table": table_bytes, "q_w_len": req_bytes,
            "total": k_bytes + out_bytes + table_bytes + req_bytes}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, with requests spread over processes
# ---------------------------------------------------------------------------

_CPU_INP = None  # the workload, inherited by the forked workers


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)  # one BLAS thread per worker process
    except Exception:
        pass


def _cpu_rows(rows):
    """Score + top-k of requests `rows` by the oracle (in a worker)."""
    import numpy as np

    import oracle

    inp = _CPU_INP
    r = np.asarray(rows)
    if inp.fp8:
        s = oracle.score_fp8(inp.q_bits[r], inp.w[r], inp.k8, inp.k_scale, inp.page_table[r], inp.seq_lens[r])
    else:
        s = oracle.score(inp.q_bits[r], inp.w[r], inp.k_bits, inp.page_table[r], inp.seq_lens[r])
    oracle.topk(s, inp.seq_lens[r], inp.topk)
    return len(rows)


def cpu_baseline(inp, seconds: float) -> dict:
    """The float64 oracle, unchanged, on the host: the step's requests are
    spread over one worker process per core the process may run on (each with
    one BLAS thread), and whole steps are repeated for about `seconds` of
    wall-clock time; the median step is reported. Called before the GPU is
    touched, so the workers are forked from a process without a GPU context."""
    import multiprocessing as mp

    import numpy as np

    global _CPU_INP
    _CPU_INP = inp
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, inp.batch))
    # longest requests first, dealt round robin, so the workers' shares are even
    order = np.argsort(-np.clip(inp.seq_lens, 0, inp.max_c4), kind="stable")
    chunks = [order[i::workers].tolist() for i in range(workers)]
    ctx = mp.get_context("fork")
    times = []
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_rows, [[c[0]] for c in chunks if c])  # warm the workers up
        t_end = time.perf_counter() + seconds
        while len(times) < 3 or (time.perf_counter() < t_end and len(times) < 200):
            t0 = time.perf_counter()
            pool.map(_cpu_rows, chunks, chunksize=1)
            times.append(time.perf_counter() - t0)
    _CPU_INP = None
    dt = sorted(times)[len(times) // 2]
    valid = int(np.clip(inp.seq_lens, 0, inp.max_c4).sum())
    try:
        cpu = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")][0]
    except Exception:
        cpu = "unknown"
    return {"value": valid / dt, "unit": "valid positions/s", "cores": workers, "kind": "oracle",
            "sample": f"score + top-{inp.topk} of all {inp.batch} requests ({valid} valid positions) per step, "
                      f"float64 numpy oracle, requests spread over {workers} worker processes (one BLAS thread "
                      f"each; {cores} cores available), median of {len(times)} steps, {dt:.3f} s each; cpu {cpu}"}


# ---------------------------------------------------------------------------
# HBM read probes
# ---------------------------------------------------------------------------

def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def timed_batches(launch, n: int, batches: int = BATCHES):
    """Median per-launch ms over `batches` batches of n launches each, queued
    back to back behind a spin kernel (so the host never starves the GPU) and
    bracketed by HIP events on the launching stream."""
    import torch

    out = []
    for _ in range(batches):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(int(2.4e9 * 0.01))  # ~10 ms of queued work ahead of the launches
        s.record()
        for i in range(n):
            launch(i)
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e) / n)
    return _median(out)


def probes(page_counts, cu_count: int, page_sizes=(8192,)) -> dict:
    """Achievable HBM read rates on this GPU: a 1 GiB contiguous read, and
    random pages (8 KiB: bf16 keys; 4 KiB: fp8 codes) from a 1 GiB pool for
    each page count (the valid pages of a workload), on grids of one-wave
    workgroups like the score kernel's (the faster of 8 and 12 per compute
    unit), with disjoint page sets read round robin."""
    import numpy as np
    import torch

    from sparse_attention_kv_indexer_amd import build

    lib = ctypes.CDLL(build.PROBE_LIB_PATH)
    vp = ctypes.c_void_p
    lib.dsa_probe_stream_read.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_int, ctypes.c_int, vp]
    lib.dsa_probe_page_read.argtypes = [vp, ctypes.c_uint64, vp, ctypes.c_int, vp, ctypes.c_int, ctypes.c_int, vp]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    out = torch.empty(cu_count * 16 * 256, dtype=torch.int32, device="cuda")
    best = None
    for per_cu in (4, 8, 16):  # 256-lane workgroups per compute unit
        for variant in range(4):  # 4 or 8 loads in flight per lane, streaming or default cache policy
            grid_s = cu_count * per_cu

            def stream_launch(_):
                rc = lib.dsa_probe_stream_read(src.data_ptr(), nbytes, out.data_ptr(), grid_s, variant, st)
                assert rc == 0, rc

            for _ in range(2):
                stream_launch(0)
            ms = timed_batches(stream_launch, 5)
            if best is None or ms < best[0]:
                best = (ms, per_cu, variant)
    ms, per_cu, variant = best
    res["stream_read"] = {"bytes": nbytes, "us": round(ms * 1e3, 2), "GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                          "best_of": "3 grids x 4 load shapes",
                          "shape": f"{per_cu} x 256 lanes per CU, {8 if variant & 1 else 4} loads in flight per lane, "
                                   f"{'default' if variant >= 2 else 'streaming'} cache policy"}
    del src
    pool_bytes = 1 << 30  # four times the Infinity Cache
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda").fill_(3)
    outp = torch.empty(cu_count * 12 * 64, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(0)
    for page_bytes in page_sizes:
        pool_pages = pool_bytes // page_bytes
        for name, n in page_counts.items():
            # R disjoint random page sets, read round robin (as the bench rotates its
            # input copies), so that no launch finds its pages in the Infinity Cache
            R = min(16, max(2, math.ceil(2 * MALL_BYTES / (n * page_bytes))))
            assert 0 < n and R * n <= pool_pages
            perm = rng.permutation(pool_pages)[:R * n].astype(np.int32)
            assert perm.min() >= 0 and perm.max() < pool_pages
            sets = [torch.from_numpy(perm[r * n:(r + 1) * n].copy()).cuda() for r in range(R)]
            best = None
            for per_cu in (8, 12):
                grid_p = cu_count * per_cu

                def page_launch(i):
                    rc = lib.dsa_probe_page_read(pool.data_ptr(), pool_bytes, sets[i % R].data_ptr(), n,
                                                 outp.data_ptr(), grid_p, page_bytes, st)
                    assert rc == 0, rc

                for i in range(2 * R):
                    page_launch(i)
                ms = timed_batches(page_launch, 20 * R)
                if best is None or ms < best[0]:
                    best = (ms, per_cu)
            ms, per_cu = best
            key = f"page_read_{name}" if page_bytes == 8192 else f"page_read_{page_bytes // 1024}k_{name}"
            res[key] = {"pages": n, "page_bytes": page_bytes, "bytes": n * page_bytes, "page_sets": R,
                        "waves_per_cu": per_cu, "us": round(ms * 1e3, 2),
                        "GBs": round(n * page_bytes / (ms * 1e-3) / 1e9, 1)}
    torch.cuda.synchronize()
    return res


# ---------------------------------------------------------------------------
# The indexer step
# ---------------------------------------------------------------------------

def cu_count() -> int:
    import torch

    return torch.cuda.get_device_properties(0).multi_processor_count


def measure_step(cfg_name: str, steps: int, warmup: int, hwm=False, keys="bf16", T=1, fused=False, rotate=0,
                 inp=None) -> dict:
    """One workload: R input copies and one captured graph of S consecutive
    steps [score; top-k] (S >= GRAPH_STEPS, a multiple of R), the copies in
    turn (as a decode step's graph holds the indexer of consecutive layers,
    each over its own keys), `warmup` untimed steps (rounded up to whole
    graphs), then exactly `steps` timed steps in BATCHES batches (events
    between batches, no synchronization), and the median per-launch duration
    of the score and top-k calls alone. Also times one-step graphs, whose
    replay overhead is reported beside the step."""
    import numpy as np
    import torch

    from sparse_attention_kv_indexer_amd import binding, workloads as wl

    cfg = wl.CONFIGS[cfg_name]
    if inp is None:
        inp = wl.generate(cfg)
    if keys == "fp8":
        inp = wl.to_fp8(inp)
    dev = torch.device("cuda:0")
    base = binding.to_device(inp, dev)
    mt = None
    if T > 1:
        mt = wl.mtp_inputs(inp, T, cfg.seed)
        base["q"] = torch.from_numpy(mt.q_bits.view("int16")).to(dev).view(torch.bfloat16)
        base["w"] = torch.from_numpy(mt.w).to(dev)
        base["seq_lens"] = torch.from_numpy(mt.seq_lens).to(dev)
    B, N, k = inp.batch, inp.max_c4, inp.topk
    set_bytes = (inp.k8.nbytes + inp.k_scale.nbytes if inp.fp8 else inp.k_bits.nbytes) + T * B * N * 4
    R = rotate or min(16, max(2, math.ceil(2 * MALL_BYTES / set_bytes)))
    sets = []
    for r in range(R):
        t = {name: (v if r == 0 else v.clone()) for name, v in base.items()}
        t["logits"] = torch.full((B * T, N), float("-inf"), dtype=torch.float32, device=dev)
        t["hwm"] = torch.zeros(B, dtype=torch.int32, device=dev) if hwm else None
        t["idx"] = torch.empty((B * T, k), dtype=torch.int32, device=dev)
        t["vals"] = torch.empty((B * T, k), dtype=torch.float32, device=dev)
        t["hist"] = binding.hist_buffer(B, dev) if fused else None
        sets.append(t)

    def launch_score(t):
        if T > 1:
            binding.score_mtp(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"],
                              out=t["logits"].view(B, T, N), row_hwm=t["hwm"])
        elif inp.fp8:
            binding.score_fp8(t["q"], t["w"], t["k8"], t["k_scale"], t["page_table"], t["seq_lens"], out=t["logits"],
                              row_hwm=t["hwm"])
        elif fused:
            binding.score_hist(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"], t["hist"],
                               out=t["logits"], row_hwm=t["hwm"])
        else:
            binding.score(t["q"], t["w"], t["k_pool"], t["page_table"], t["seq_lens"], out=t["logits"],
                          row_hwm=t["hwm"])

    def launch_topk(t):
        binding.topk(t["logits"], t["seq_lens"].view(-1), k, out_idx=t["idx"], out_vals=t["vals"], hist=t["hist"])

    def launch_step(t):
        launch_score(t)
        launch_topk(t)

    # warm up eagerly once per set (also brings row_hwm to its steady state)
    for t in sets:
        launch_step(t)
    torch.cuda.synchronize()

    # graphs: S steps over the R input copies in turn, and the first
    # steps % S of them for the remainder of `steps`; one-step graphs for the
    # replay overhead
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())

    def capture(ts):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for t in ts:
                launch_step(t)
        return g

    S = R * -(-GRAPH_STEPS // R)
    g_all = capture([sets[i % R] for i in range(S)])
    rem = steps % S
    g_rem = capture([sets[i % R] for i in range(rem)]) if rem else None
    g_one = [capture([t]) for t in sets]
    torch.cuda.synchronize()

    for _ in range(-(-warmup // S)):
        g_all.replay()
    torch.cuda.synchronize()
    # exactly `steps` steps between one synchronized start and end, with
    # events at the batch boundaries only
    n_rep = steps // S
    cuts = [round(n_rep * j / BATCHES) for j in range(BATCHES + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(BATCHES + 1)]
    evs[0].record()
    i = 0
    for j in range(BATCHES):
        while i < cuts[j + 1]:
            g_all.replay()
            i += 1
        if j == BATCHES - 1 and g_rem is not None:
            g_rem.replay()
        evs[j + 1].record()
    torch.cuda.synchronize()
    total_ms = evs[0].elapsed_time(evs[-1])
    batch_ms = [evs[j].elapsed_time(evs[j + 1]) / ((cuts[j + 1] - cuts[j]) * S) for j in range(BATCHES - 1)
                if cuts[j + 1] > cuts[j]]
    if not batch_ms:
        batch_ms = [total_ms / steps]
    one_ms = timed_batches(lambda i: g_one[i % R].replay(), 20 * R)

    n_kern = 200
    if fused:
        # the top-k consumes (and zeroes) the histogram its score call filled,
        # so it is timed as whole steps minus the score kernel alone; the
        # score kernel's own back-to-back launches leave the histograms dirty,
        # so they go last
        step_avg_ms = timed_batches(lambda i: launch_step(sets[i % R]), n_kern)
        score_avg_ms = timed_batches(lambda i: launch_score(sets[i % R]), n_kern)
        topk_avg_ms = step_avg_ms - score_avg_ms
    else:
        score_avg_ms = timed_batches(lambda i: launch_score(sets[i % R]), n_kern)
        topk_avg_ms = timed_batches(lambda i: launch_topk(sets[i % R]), n_kern)

    valid = int(np.clip(inp.seq_lens if mt is None else mt.seq_lens, 0, N).sum())
    alg = algorithmic_bytes(inp, hwm, T, None if mt is None else mt.seq_lens)
    res = {
        "inp": inp, "cfg": cfg, "R": R, "S": S, "valid": valid, "T": T, "alg": alg,
        "ms_per_step": total_ms / steps, "step_us_median_of_batches": _median(batch_ms) * 1e3,
        "one_step_graph_us": one_ms * 1e3,
        "score_us": score_avg_ms * 1e3, "topk_us": topk_avg_ms * 1e3,
        "k_GBs": alg["k"] / (score_avg_ms * 1e-3) / 1e9,
        "all_GBs": alg["total"] / (score_avg_ms * 1e-3) / 1e9,
    }
    del sets, g_all, g_rem, g_one, base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def summary(r: dict) -> dict:
    """The per-workload figures carried in the JSON line."""
    return {
        "workload": f"{r['cfg'].name}: {r['cfg'].description}",
        "us_per_step": round(r["ms_per_step"] * 1e3, 2),
        "step_us_median_of_batches": round(r["step_us_median_of_batches"], 2),
        "one_step_graph_us": round(r["one_step_graph_us"], 2),
        "valid_positions": r["valid"],
        "valid_positions_per_s": r["valid"] / (r["ms_per_step"] * 1e-3),
        "score_us": round(r["score_us"], 2), "topk_us": round(r["topk_us"], 2),
        "score_key_GBs": round(r["k_GBs"], 1), "score_key_frac": round(r["k_GBs"] / HBM_PEAK_GBS, 4),
        "score_all_bytes_frac": round(r["all_GBs"] / HBM_PEAK_GBS, 4),
        "input_copies": r["R"], "steps_per_graph": r["S"],
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this path runs on one GPU only (no cross-GPU sharding or collectives); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    from sparse_attention_kv_indexer_amd import workloads as wl

    cfg = wl.CONFIGS[args.config]
    T = args.tokens
    if args.stage == "indexer" and not args.probe and not args.copy_calibration:
        if T != 1 and (args.keys == "fp8" or not 1 <= T <= 4):
            print("bench.py: --tokens 2..4 runs bf16 keys", file=sys.stderr)
            sys.exit(2)
        if args.topk == "hist" and (T != 1 or args.keys == "fp8"):
            print("bench.py: --topk hist runs one query token with bf16 keys", file=sys.stderr)
            sys.exit(2)
    inp = wl.generate(cfg) if not (args.probe or args.copy_calibration) else None

    # the CPU baseline runs first, so its worker processes fork from a process
    # that has not touched the GPU
    cpu = None
    if args.stage == "indexer" and inp is not None and not args.no_cpu and T == 1:
        cpu = cpu_baseline(wl.to_fp8(inp) if args.keys == "fp8" else inp, args.cpu_seconds)

    import torch

    from sparse_attention_kv_indexer_amd import binding

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    binding.load()
    if args.probe:
        print(json.dumps({"probe": probes({"c3": 17511, "full": 32768}, cu_count(), (8192, 4096))}), flush=True)
        return
    if args.stage == "attention":
        bench_attention(args, cfg, inp)
        return

    fused = args.topk == "hist"
    head = measure_step(args.config, args.steps, args.warmup, hwm=args.hwm, keys=args.keys, T=T, fused=fused,
                        rotate=args.rotate, inp=inp)
    inp = head["inp"]
    alg = head["alg"]
    traffic = read_traffic(args.config + ("+hwm" if args.hwm else "") + ("+fp8" if inp.fp8 else "")
                           + (f"+tok{T}" if T > 1 else "") + ("+hist" if fused else ""))
    roofline = {
        "bound": "hbm", "kernel": "score_kernel", "numerator": "valid-page key bytes per launch",
        "achieved": round(head["k_GBs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(head["k_GBs"] / HBM_PEAK_GBS, 4),
        "traffic": (traffic or {}).get("total_bytes"), "traffic_bytes": traffic,
        "algorithmic_bytes_per_launch": alg, "launch_avg_us": round(head["score_us"], 3),
        "launch_avg": f"median of {BATCHES} batches of 200 back-to-back launches, HIP events",
        "all_bytes": {"achieved": round(head["all_GBs"], 1), "frac": round(head["all_GBs"] / HBM_PEAK_GBS, 4)},
        "topk_launch_avg_us": round(head["topk_us"], 3),
        "topk_path": "score_hist + topk_hist (histogram from the score kernel)" if fused else "sampled cut",
    }
    result = {
        "metric": METRIC,
        "value": head["valid"] / (head["ms_per_step"] * 1e-3),
        "unit": "valid positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "us_per_step": head["ms_per_step"] * 1e3,
        "step_us_median_of_batches": round(head["step_us_median_of_batches"], 3),
        "one_step_graph_us": round(head["one_step_graph_us"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "batch": inp.batch, "heads": wl.HEADS, "dim": wl.DIM, "page_positions": wl.PAGE,
            "max_pages": inp.max_pages, "max_c4": inp.max_c4, "valid_positions": head["valid"],
            "valid_pages": int(wl.pages_needed(inp.seq_lens).sum()), "topk": inp.topk, "seed": cfg.seed,
            "tail": "incremental (row_hwm)" if args.hwm else "stateless full -inf",
            "input_copies": head["R"], "steps_per_graph": head["S"],
            "timing": f"hipGraph replays of {head['S']} consecutive steps [score; top-k], the {head['R']} input "
                      f"copies in turn; "
                      f"HIP events, {BATCHES} batches; one_step_graph_us: graphs of one step each, whose replay "
                      f"adds a fixed launch cost per step",
            "accumulate": "fp32",
            "keys": "e4m3fn codes + float32 scale per key" if inp.fp8 else "bf16",
            "query_tokens": T,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if T > 1:
        result["metric"] = METRIC + f" ({T} query tokens per request: token-positions scored/s)"
        result["unit"] = "valid token-positions/s"
    fp8 = inp.fp8
    del head, inp
    if not args.no_extra:
        xs = min(args.steps, 200) if args.steps >= 20 else 20
        xw = max(args.warmup, 5)
        full = measure_step("full", xs, xw)
        extra = {"full": summary(full)}
        for name in ("stress8k", "stress1m"):
            for hwm in (False, True):
                r = measure_step(name, xs, xw, hwm=hwm)
                extra[name + ("+hwm" if hwm else "")] = summary(r)
        step = {key: extra[key]["us_per_step"] for key in extra}
        result["workloads"] = extra
        result["stress_ratio"] = {
            "definition": "step time of stress1m / step time of stress8k (1M- vs 8K-token row width, "
                          "every length 512 tokens); target <= 1.2",
            "incremental_tail": round(step["stress1m+hwm"] / step["stress8k+hwm"], 3),
            "incremental_vs_stateless_8k": round(step["stress1m+hwm"] / step["stress8k"], 3),
            "stateless": round(step["stress1m"] / step["stress8k"], 3),
        }
        # (the head workload's pages under the name c3; fp8 pages are 4 KiB)
        pr = probes({"c3": result["config"]["valid_pages"], "full": full["inp"].batch * full["inp"].max_pages},
                    cu_count(), (8192, 4096) if fp8 else (8192,))
        roofline["measured_ceiling"] = pr
        roofline["frac_of_page_read"] = round(
            roofline["achieved"] / pr["page_read_4k_c3" if fp8 else "page_read_c3"]["GBs"], 4)
        roofline["frac_of_stream_read"] = round(roofline["achieved"] / pr["stream_read"]["GBs"], 4)
        extra["full"]["score_key_frac_of_page_read"] = round(full["k_GBs"] / pr["page_read_full"]["GBs"], 4)
    print(json.dumps(result), flush=True)


ATT_METRIC = "selected positions attended/s + µs/step (sparse attention after the indexer); % of HBM roofline"


def attention_bytes(inp, idx) -> dict:
    """Bytes one attention call must move at minimum: the latent of every
    selected entry, the selection itself, the page-table entries of the pages
    it touches, the queries, and the outputs (float32 out and lse)."""
    import numpy as np

    from sparse_attention_kv_indexer_amd import workloads as wl

    valid = idx >= 0
    n = int(valid.sum())
    pages = sum(np.unique(idx[b][valid[b]] // wl.PAGE).size for b in range(inp.batch))
    lat = n * wl.ATT_KD * 2
    q = inp.batch * wl.ATT_HEADS * wl.ATT_KD * 2
    out = inp.batch * wl.ATT_HEADS * (wl.ATT_VD + 1) * 4
    sel = idx.size * 4
    return {"latents": lat, "selection": sel, "page_table": pages * 4, "q": q, "out_lse": out,
            "total": lat + sel + pages * 4 + q + out}


def attention_cpu_baseline(inp, att, idx, total_s: float = 12.0) -> dict:
    """The attention oracle on the host over the first requests of the step
    (as many as fit about 2 s per repetition), repeated at least 3 times and
    until about total_s seconds; the median repetition is reported. numpy's
    BLAS runs each product on its own threads."""
    import oracle
    from sparse_attention_kv_indexer_amd import workloads as wl

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    rows, times, spent = inp.batch, [], 0.0
    while len(times) < 3 or (spent < total_s and len(times) < 200):
        t0 = time.perf_counter()
        oracle.sparse_attention(att.q_bits[:rows], att.kv_bits, inp.page_table[:rows], idx[:rows], att.scale,
                                wl.ATT_VD)
        dt = time.perf_counter() - t0
        spent += dt
        times.append(dt)
        if dt > 2.0 and rows > 1:
            rows = max(1, int(rows * 2.0 / dt))
            times = []
    dt = sorted(times)[len(times) // 2]
    n = int((idx[:rows] >= 0).sum())
    return {"value": n / dt, "unit": "selected positions/s", "cores": int(threads), "kind": "oracle",
            "sample": f"attention of {rows} of {inp.batch} requests ({n} selected positions), float64 numpy "
                      f"oracle (BLAS threads: {threads}), median of {len(times)} repetitions ({spent:.1f} s in all), "
                      f"{dt:.3f} s each"}

def bench_attention(args, cfg, inp):
    """Sparse attention of 32 heads over top-k-shaped selections (k entries,
    ascending, -1 padded) of the workload's pages, timed like the indexer
    step: R distinct selections over the same latent pool, so that two calls'
    worth of selected latents exceed twice the Infinity Cache and every call
    reads its rows from HBM, and one captured graph of R consecutive calls,
    one per selection."""
    import numpy as np
    import torch

    from sparse_attention_kv_indexer_amd import binding, workloads as wl

    dev = torch.device("cuda:0")
    att = wl.attention_inputs(inp, cfg.seed)
    idx = wl.random_selection(inp, inp.topk, cfg.seed)
    B, k = idx.shape
    n_sel = int((idx >= 0).sum())
    sel_bytes = n_sel * wl.ATT_KD * 2
    R = args.rotate or min(16, max(2, math.ceil(2 * MALL_BYTES / sel_bytes)))
    idxs = [idx] + [wl.random_selection(inp, inp.topk, cfg.seed + 1000 + r) for r in range(1, R)]
    base = binding.attention_to_device(att, dev)
    base["page_table"] = torch.from_numpy(inp.page_table).to(dev)
    sets = []
    for r in range(R):
        t = dict(base)
        t["idx"] = torch.from_numpy(idxs[r]).to(dev)
        t["out"] = torch.empty((B, wl.ATT_HEADS, wl.ATT_VD), dtype=torch.float32, device=dev)
        t["lse"] = torch.empty((B, wl.ATT_HEADS), dtype=torch.float32, device=dev)
        sets.append(t)
    need = binding.sparse_attention_workspace_bytes(B, k)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def launch(t):
        binding.sparse_attention(t["q"], t["kv_pool"], t["page_table"], t["idx"], att.scale, out=t["out"],
                                 lse=t["lse"], workspace=ws)

    for t in sets:
        launch(t)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())

    def capture(ts):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for t in ts:
                launch(t)
        return g

    S = R * -(-GRAPH_STEPS // R)
    g_all = capture([sets[i % R] for i in range(S)])
    rem = args.steps % S
    g_rem = capture([sets[i % R] for i in range(rem)]) if rem else None
    g_one = [capture([t]) for t in sets]
    torch.cuda.synchronize()
    for _ in range(-(-args.warmup // S)):
        g_all.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps // S):
        g_all.replay()
    if g_rem is not None:
        g_rem.replay()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    one_ms = timed_batches(lambda i: g_one[i % R].replay(), 20 * R)
    call_ms = timed_batches(lambda i: launch(sets[i % R]), 200)

    # algorithmic bytes of a call: the mean over the selections (they differ
    # only in how many distinct pages they touch)
    algs = [attention_bytes(inp, x) for x in idxs]
    alg = {key: int(round(sum(a_[key] for a_ in algs) / R)) for key in algs[0]}
    achieved = alg["total"] / (call_ms * 1e-3) / 1e9
    nsplit = need // (B * wl.ATT_HEADS * (wl.ATT_VD + 1) * 4) if need else 1
    att_traffic = read_traffic(cfg.name, ATT_TRAFFIC_FILE, ATT_SOURCES)
    roofline = {
        "bound": "hbm", "kernel": "attention_kernel + merge_kernel (one call)", "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": (att_traffic or {}).get("total_bytes"),
        "traffic_bytes": att_traffic,
        "algorithmic_bytes_per_launch": alg, "launch_avg_us": round(call_ms * 1e3, 3),
    }
    result = {
        "metric": ATT_METRIC,
        "value": n_sel / (ms_per_step * 1e-3),
        "unit": "selected positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "us_per_step": ms_per_step * 1e3, "one_step_graph_us": round(one_ms * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": f"attention over {cfg.name}: {cfg.description}",
            "batch": B, "heads": wl.ATT_HEADS, "latent_dims": wl.ATT_KD, "value_dims": wl.ATT_VD, "k": k,
            "selected_positions": n_sel, "splits": int(nsplit), "scale": att.scale, "seed": cfg.seed,
            "selection": "uniform random subset of min(k, L) positions per request, ascending, -1 padded; "
                         "R such subsets, one per call in turn",
            "input_copies": R, "steps_per_graph": S,
            "timing": f"hipGraph replays of {S} consecutive calls, the {R} selections in turn (each its own random "
                      f"subset of the same pages); HIP events; launch_avg_us: median of {BATCHES} batches of 200 "
                      f"back-to-back calls; one_step_graph_us: graphs of one call each",
            "accumulate": "fp32 (softmax weights bf16 into the value product)",
        },
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        result["cpu_baseline"] = attention_cpu_baseline(inp, att, idx)
    print(json.dumps(result), flush=True)




if __name__ == "__main__":
    main()
