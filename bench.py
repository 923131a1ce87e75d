"""Benchmark of the MSA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload (100M-token bank on one GPU): 195,313 documents x 512 tokens,
pool 64 -> 1,562,504 pooled rows.  The pooled router keys (8 heads x 128,
bf16, 3.2 GB) are resident in HBM; the pooled content K/V (8 x 128, bf16,
6.4 GB) are in pinned host memory.  One step is one pass of the whole hot
path on fresh synthetic inputs:
  1. pool: msa_pool_encode of a batch of 64 new documents x 512 tokens
     (document-wise RoPE + chunk means of K/V/Kr);
  2. route: msa_route with one query token - cosine scan of the whole bank,
     head mean, per-document max, top-16, then the device-side copy of the
     16 selected documents' pooled K/V from mapped pinned memory (the
     host-driven hipMemcpyAsync mode is timed beside it for latency);
  3. decode: msa_sparse_decode, GQA 32/8 x 128 over [128 memory rows ;
     4096 local tokens] with the query offset by k = 16.
Inputs are resident before the timed region.  Prints one JSON line.
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_latent_memory_amd as msa  # noqa: E402
from sparse_latent_memory_amd.interleave import InterleavePipeline  # noqa: E402
from sparse_latent_memory_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E peak, GB/s
# the measured scan kernel's own source and the device helpers it includes
SCAN_SOURCES = [os.path.join(ROOT, "sparse_latent_memory_amd", "csrc", f) for f in ("route_scan.hip", "msa_device.h")]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "route_scan_100M_bank.traffic.json")
CALIBRATION_BYTES = 1 << 30


def source_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per scan launch from the committed FETCH_SIZE / WRITE_SIZE
    counter runs (scaled by the copy calibration), or None when the record is
    missing, covers another kernel, or was taken on a different version of
    the scan source."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(SCAN_SOURCES) or kernel not in rec.get("kernel", ""):
        return None
    return rec.get("hbm_bytes_per_launch")


def calibrate_copy():
    """A plain device copy of CALIBRATION_BYTES, three times: reads and
    writes exactly that many bytes per launch, for scaling the counters."""
    n = CALIBRATION_BYTES // 2
    x = torch.randn(n, device="cuda:0").to(torch.bfloat16)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": CALIBRATION_BYTES, "launches": 3}), flush=True)


SCAN_KERNELS = {"tiled": "scan_mfma_kernel<8, 4, 1, true, true>", "rows": "scan_mfma_kernel<8, 4, 1, false, true>"}
SCAN_KERNEL = SCAN_KERNELS["tiled"]     # the headline line's router bank is tiled
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _counter_kib(run_dir, counter, kernel):
    """Average KiB per dispatch of one rocprofv3 --pmc counter over the
    dispatches of `kernel` (and how many there were), from the
    run_counter_collection.csv under run_dir."""
    import csv
    import glob
    per_dispatch = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter and kernel in r["Kernel_Name"]:
                    key = (path, r["Dispatch_Id"])
                    per_dispatch[key] = per_dispatch.get(key, 0.0) + float(r["Counter_Value"])
    if not per_dispatch:
        raise SystemExit(f"no {counter} values for {kernel} under {run_dir}")
    return sum(per_dispatch.values()) / len(per_dispatch), len(per_dispatch)


def write_traffic_record(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    """HBM bytes per scan launch from FETCH_SIZE / WRITE_SIZE counter runs of
    this bench and of --calibrate-copy, each counter scaled by what it reads
    for the 1 GiB copy (which moves exactly that many bytes each way)."""
    cfg = synth.config(4)
    n_pool = int(synth.row_offsets(synth.doc_lengths(cfg), cfg.pool)[-1])
    fetch, n = _counter_kib(fetch_dir, "FETCH_SIZE", SCAN_KERNEL)
    write, _ = _counter_kib(write_dir, "WRITE_SIZE", SCAN_KERNEL)
    cfetch, _ = _counter_kib(copy_fetch_dir, "FETCH_SIZE", COPY_KERNEL)
    cwrite, _ = _counter_kib(copy_write_dir, "WRITE_SIZE", COPY_KERNEL)
    fscale = CALIBRATION_BYTES / (cfetch * 1024)
    wscale = CALIBRATION_BYTES / (cwrite * 1024)
    hbm = fetch * 1024 * fscale + write * 1024 * wscale
    algo = n_pool * cfg.n_router_heads * cfg.router_dim * 2 + cfg.n_router_heads * cfg.router_dim * 2
    rec = {
        "kernel": f"msa::{SCAN_KERNEL} (route bank scan, 100M-token bank, 1 query token)",
        "sources": [os.path.relpath(p, ROOT) for p in SCAN_SOURCES],
        "source_sha256": source_digest(SCAN_SOURCES),
        "fetch_kib_per_launch_raw": fetch,
        "write_kib_per_launch_raw": write,
        "launches": n,
        "copy_calibration": {"bytes": CALIBRATION_BYTES, "kernel": COPY_KERNEL, "fetch_kib_raw": cfetch,
                             "write_kib_raw": cwrite, "fetch_scale": fscale, "write_scale": wscale},
        "hbm_bytes_per_launch": hbm,
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": hbm / algo,
    }
    with open(TRAFFIC_RECORD, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hip_runtime_api.h: timing-only events
EVENT_EVERY = 4


class HipEvents:
    """Plain hipEvent_t pairs from the HIP runtime torch has loaded, created
    for timing only: without the system-scope fence a default event performs
    when it completes (an L2 write-back and invalidate that left a ~5 us gap
    in the stream at every record)."""

    def __init__(self, n):
        lib_dir = os.path.join(os.path.dirname(torch.__file__), "lib")
        self.hip = ctypes.CDLL(os.path.join(lib_dir, "libamdhip64.so"))
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(a), HIP_EVENT_DISABLE_SYSTEM_FENCE) == 0
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(b), HIP_EVENT_DISABLE_SYSTEM_FENCE) == 0
            self.pairs.append((a, b))

    def elapsed_ms(self, i):
        ms = ctypes.c_float()
        a, b = self.pairs[i]
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def read_ceiling(buf, stream, reps=10):
    """The streaming-read ceiling of the tiled bank's access pattern on this
    device and buffer: libmsa_readref's reference read (one wave per 32 KiB
    tile, 1 KiB contiguous non-temporal loads, an XOR fold and nothing else)
    over the bank itself, timed with events on its dispatch; the best median
    over grids of 1, 2, 4 and 8 workgroups per CU."""
    from sparse_latent_memory_amd import readref
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    ev = HipEvents(reps)
    best = None
    n_bytes = 0
    for mult in (1, 2, 4, 8):
        grid = n_cu * mult
        sink = torch.empty(grid * 256 * 4, dtype=torch.int32, device=buf.device)
        readref.read_tiles(buf, grid, True, sink, stream)
        for r in range(reps):
            _, n_bytes = readref.read_tiles(buf, grid, True, sink, stream, ev.pairs[r])
        torch.cuda.synchronize()
        us = float(np.median([ev.elapsed_ms(r) for r in range(reps)])) * 1e3
        if best is None or us < best[1]:
            best = (grid, us)
    return {"GBs": n_bytes / (best[1] * 1e-6) / 1e9, "us": best[1], "bytes": n_bytes, "grid": best[0],
            "kernel": "read_tiles_kernel<true> (libmsa_readref): one wave per 32 KiB tile, 1 KiB contiguous "
                      "non-temporal loads, XOR fold only; best median of 10 over 1-8 workgroups per CU"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--latency-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--write-traffic-record", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the scan's HBM traffic record from four rocprofv3 --pmc output folders "
                         "(this bench with FETCH_SIZE, with WRITE_SIZE; --calibrate-copy with each)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--workload", default="bank-100M", choices=sorted(WORKLOADS),
                    help="bank-100M (default, the headline line); the others print supporting lines")
    ap.add_argument("--reps", type=int, default=10, help="timed repetitions of a supporting workload")
    ap.add_argument("--kr-layout", default="tiled", choices=["tiled", "rows"],
                    help="router-bank layout of the headline workload (tiled: the library's scan order)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.write_traffic_record:
        write_traffic_record(*args.write_traffic_record)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this benchmark runs on one GPU only (the bank is held whole in one GPU's HBM); "
              "multi-GPU runs are not supported", file=sys.stderr)
        sys.exit(2)

    dev = "cuda:0"
    torch.cuda.set_device(0)
    msa.load()
    if args.workload != "bank-100M":
        WORKLOADS[args.workload](args, dev)
        return
    cfg = synth.config(4)
    K, W = args.steps, args.warmup
    n_steps = W + K + args.latency_steps

    # ---------------- resident inputs ----------------
    t_setup = time.time()
    lens = synth.doc_lengths(cfg)
    pool_off = synth.row_offsets(lens, cfg.pool)
    n_docs, n_pool = len(lens), int(pool_off[-1])
    bank_tokens = int(lens.sum())
    log(f"bank: {n_docs} docs, {bank_tokens} tokens, {n_pool} pooled rows")
    kr = synth.pooled_router_bank(cfg, lens, device=dev)
    lay = args.kr_layout
    bank, rkw = _router_bank(kr, pool_off, lay)    # what the scan reads
    host_kv = synth.pooled_content_bank(cfg, lens, device=dev, pin=True)
    pool_off_d = torch.as_tensor(pool_off, device=dev)
    pool_off_h = torch.as_tensor(pool_off)
    enc = synth.config(4, n_docs=64)
    enc_lens = synth.doc_lengths(enc)
    enc_bank = synth.raw_bank(enc, lens=enc_lens, device=dev)
    enc_pool_off = synth.row_offsets(enc_lens, enc.pool)
    enc_pool_off_d = torch.as_tensor(enc_pool_off, device=dev)
    enc_npool = int(enc_pool_off[-1])
    enc_kv = torch.empty((enc_npool, 2, cfg.n_kv_heads, cfg.head_dim), dtype=cfg.torch_dtype, device=dev)
    enc_kr = torch.empty((msa.bank_rows(enc_npool, lay), cfg.n_router_heads, cfg.router_dim), dtype=cfg.torch_dtype,
                         device=dev)
    lk, lv = synth.local_context(cfg, device=dev)
    qrs = [synth.router_queries(cfg, step=i, device=dev) for i in range(n_steps)]
    qs = [synth.decode_queries(cfg, step=i, device=dev) for i in range(n_steps)]
    k = cfg.top_k
    mem_cap = k * (512 // cfg.pool)
    copy_stream = torch.cuda.Stream()
    asm = msa.Assembly.allocate(host_kv, pool_off_h, cfg.batch, k, mem_cap, dev, mode="kernel")
    asm_copies = msa.Assembly.allocate(host_kv, pool_off_h, cfg.batch, k, mem_cap, dev, copy_stream=copy_stream,
                                       mode="copies")
    loc_len = torch.full((cfg.batch,), cfg.local_len, dtype=torch.int32, device=dev)
    pos = torch.full((cfg.batch,), k, dtype=torch.int32, device=dev)
    rws = torch.empty(msa.route_workspace_bytes(cfg.torch_dtype, cfg.batch, 1, cfg.n_router_heads, cfg.router_dim,
                                                n_docs, n_pool, k), dtype=torch.uint8, device=dev)
    dws = torch.empty(msa.decode_workspace_bytes(cfg.batch, cfg.n_q_heads, cfg.head_dim, mem_cap, cfg.local_len),
                      dtype=torch.uint8, device=dev)
    doc_scores = torch.empty((cfg.batch, n_docs), dtype=torch.float32, device=dev)
    topk_idx = torch.empty((cfg.batch, k), dtype=torch.int32, device=dev)
    topk_score = torch.empty((cfg.batch, k), dtype=torch.float32, device=dev)
    out = torch.empty((cfg.batch, cfg.n_q_heads, cfg.head_dim), dtype=cfg.torch_dtype, device=dev)
    lse = torch.empty((cfg.batch, cfg.n_q_heads), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f} s")

    # kernel durations: event pairs attached to the scan and attention
    # dispatches of every EVENT_EVERY-th timed step (each event point still
    # costs the queue a ~4 us marker)
    samples = list(range(0, K, EVENT_EVERY))
    scan_ev = HipEvents(len(samples))
    dec_ev = HipEvents(len(samples))
    stream = torch.cuda.current_stream()

    def step(i, j=None):
        msa.pool_encode(enc_bank["k"], enc_bank["v"], enc_bank["kr"], enc_bank["doc_tok_off"], enc_pool_off_d,
                        enc.pool, enc.rope_theta, enc_npool, enc_kv, enc_kr, stream=stream, kr_layout=lay)
        msa.route(qrs[i], bank, pool_off_d, k, doc_scores, topk_idx, topk_score, rws, assembly=asm, stream=stream,
                  prof_events=None if j is None else scan_ev.pairs[j], **rkw)
        msa.sparse_decode(qs[i], asm.mem_kv, asm.mem_len, lk, lv, loc_len, pos, cfg.rope_theta, out, lse, dws,
                          stream=stream, prof_events=None if j is None else dec_ev.pairs[j])

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    log("warmup done")
    t0 = time.perf_counter()
    for j in range(K):
        step(W + j, j // EVENT_EVERY if j % EVENT_EVERY == 0 else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    log(f"timed {K} steps: {elapsed * 1e3 / K:.3f} ms/step")

    scan_ms = np.array([scan_ev.elapsed_ms(j) for j in range(len(samples))])
    dec_ms = np.array([dec_ev.elapsed_ms(j) for j in range(len(samples))])

    # route + decode latency per step (synchronised each step), both assembly modes
    # as a serving loop calls it (msa.RouteCall: every argument but the
    # query bound once), and with route() marshalling all its arguments
    calls = {name: msa.RouteCall(tuple(qrs[0].shape), qrs[0].dtype, bank, pool_off_d, k, doc_scores, topk_idx,
                                 topk_score, rws, assembly=a, **rkw)
             for name, a in (("kernel", asm), ("copies", asm_copies))}
    # completion observed by polling an event (and, for comparison, by a
    # blocking synchronise)
    poll = CompletionPoll()
    lat = {}
    for name, a, bound, polled in (("kernel", asm, True, True), ("copies", asm_copies, True, True),
                                   ("kernel_route", asm, False, True), ("kernel_sync", asm, True, False)):
        vals = []
        for i in range(W + K, n_steps):
            torch.cuda.synchronize()
            t = time.perf_counter()
            if bound:
                calls[name.split("_")[0]](qrs[i], stream=stream)
            else:
                msa.route(qrs[i], bank, pool_off_d, k, doc_scores, topk_idx, topk_score, rws, assembly=a,
                          stream=stream, **rkw)
            msa.sparse_decode(qs[i], a.mem_kv, a.mem_len, lk, lv, loc_len, pos, cfg.rope_theta, out, lse, dws,
                              stream=stream)
            if polled:
                poll.wait(stream)
            else:
                torch.cuda.synchronize()
            vals.append((time.perf_counter() - t) * 1e3)
        lat[name] = np.array(vals)
    log(f"route+decode p50: kernel gather {np.median(lat['kernel']):.3f} ms "
        f"(route() with every argument: {np.median(lat['kernel_route']):.3f} ms; waiting by synchronise: "
        f"{np.median(lat['kernel_sync']):.3f} ms), copy gather {np.median(lat['copies']):.3f} ms")

    # pipelined steady state: consecutive queries alternate between two
    # streams with their own buffers (device-side assembly never waits on the
    # host), so one query's selection, gather and decode overlap the next
    # query's scan; the interval is the wall time per query
    lanes = []
    for s_ in (stream, torch.cuda.Stream()):
        lanes.append({"s": s_, "asm": asm if s_ is stream else msa.Assembly.allocate(
                          host_kv, pool_off_h, cfg.batch, k, mem_cap, dev, mode="kernel"),
                      "rws": torch.empty_like(rws), "dws": torch.empty_like(dws), "dsc": torch.empty_like(doc_scores),
                      "tki": torch.empty_like(topk_idx), "tks": torch.empty_like(topk_score),
                      "out": torch.empty_like(out), "lse": torch.empty_like(lse)})
    n_pipe = n_steps - (W + K)
    for rep in range(2):                       # the first pass warms the second stream
        torch.cuda.synchronize()
        t = time.perf_counter()
        for n, i in enumerate(range(W + K, n_steps)):
            L = lanes[n % 2]
            msa.route(qrs[i], bank, pool_off_d, k, L["dsc"], L["tki"], L["tks"], L["rws"], assembly=L["asm"],
                      stream=L["s"], **rkw)
            msa.sparse_decode(qs[i], L["asm"].mem_kv, L["asm"].mem_len, lk, lv, loc_len, pos, cfg.rope_theta,
                              L["out"], L["lse"], L["dws"], stream=L["s"])
        torch.cuda.synchronize()
        pipe_ms = (time.perf_counter() - t) * 1e3 / n_pipe
    log(f"route+decode pipelined interval {pipe_ms:.3f} ms")

    # the same with the host-driven hipMemcpyAsync assembly: msa_route without
    # assembly for query i, then msa_assemble (copy mode) for query i - 1,
    # whose top-k has landed by then, so that query's copies cross the host
    # link while query i is scored; msa_assemble blocks this thread only
    # until query i - 1's ids are on the host
    for L in lanes:
        L["asm_c"] = msa.Assembly.allocate(host_kv, pool_off_h, cfg.batch, k, mem_cap, dev, mode="copies",
                                           copy_stream=torch.cuda.Stream())

    def finish(i, L):
        msa.assemble(L["tki"], pool_off_d, L["asm_c"], stream=L["s"])
        msa.sparse_decode(qs[i], L["asm_c"].mem_kv, L["asm_c"].mem_len, lk, lv, loc_len, pos, cfg.rope_theta,
                          L["out"], L["lse"], L["dws"], stream=L["s"])

    for rep in range(2):
        torch.cuda.synchronize()
        t = time.perf_counter()
        prev = None
        for n, i in enumerate(range(W + K, n_steps)):
            L = lanes[n % 2]
            msa.route(qrs[i], bank, pool_off_d, k, L["dsc"], L["tki"], L["tks"], L["rws"], stream=L["s"], **rkw)
            if prev is not None:
                finish(*prev)
            prev = (i, L)
        finish(*prev)
        torch.cuda.synchronize()
        pipe_copy_ms = (time.perf_counter() - t) * 1e3 / n_pipe
    log(f"route+decode pipelined interval, hipMemcpyAsync assembly {pipe_copy_ms:.3f} ms")

    scan_bytes = n_pool * cfg.n_router_heads * cfg.router_dim * 2 + cfg.n_router_heads * cfg.router_dim * 2
    scan_avg_s = scan_ms.mean() / 1e3
    achieved = scan_bytes / scan_avg_s / 1e9
    value = cfg.batch * bank_tokens * K / elapsed
    dec_bytes = (mem_cap + cfg.local_len) * cfg.n_kv_heads * cfg.head_dim * 2 * 2
    # route + decode floor: bank + decode K/V at HBM peak, the 16 documents over a 64 GB/s host link
    t_floor_ms = (scan_bytes + dec_bytes) / (HBM_PEAK_GBS * 1e9) * 1e3 + mem_cap * 4096 / 64e9 * 1e3

    ceiling = read_ceiling(bank, stream) if lay == "tiled" else None
    if ceiling:
        log(f"read ceiling (reference read, tiled pattern): {ceiling['GBs']:.0f} GB/s; scan at "
            f"{achieved / ceiling['GBs']:.1%} of it")

    cpu = None
    if not args.no_cpu_baseline:
        step_in = {"enc_bank": enc_bank, "enc_tok_off": synth.row_offsets(enc_lens, 1), "enc_pool": enc.pool,
                   "rope_theta": cfg.rope_theta, "k": k, "q": qs[W], "mem_kv": asm.mem_kv, "mem_len": asm.mem_len,
                   "local_k": lk, "local_v": lv, "local_len": loc_len, "pos": pos}
        cpu = cpu_baseline(cfg, kr, pool_off, qrs[W], args.cpu_seconds, step_in)

    res = {
        "metric": "bank tokens scored/s (% HBM peak); p50 route+decode step at 100M bank",
        "value": value,
        "unit": "bank tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": elapsed * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "bank-100M-decode: 195,313 docs x 512 tokens, pool 64 -> 1,562,504 pooled rows; "
                        "Kr 8x128 bf16 in HBM (3.2 GB); pooled K/V 8x128 bf16 in pinned host memory (6.4 GB); "
                        "1 query token, top-16, gather, decode GQA 32/8x128 over 128 memory rows + 4096 local "
                        "tokens; plus a 64-doc x 512-token encode batch per step",
            "bank_tokens": bank_tokens,
            "pooled_rows": n_pool,
            "global_batch": cfg.batch,
            "kr_layout": lay,
            "doc_map": "built once with the bank (msa_doc_map) and passed to every route call",
        },
        "roofline": {
            "kernel": f"route bank scan ({SCAN_KERNELS[lay]})",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(SCAN_KERNELS[lay]),
            "scan_us": scan_ms.mean() * 1e3,
            "timed_launches": len(samples),
            "scan_bytes": scan_bytes,
            "read_ceiling": ceiling,
            "frac_of_read_ceiling": achieved / ceiling["GBs"] if ceiling else None,
        },
        "latency_ms": {
            "route_decode_p50": float(np.percentile(lat["kernel"], 50)),
            "route_decode_p90": float(np.percentile(lat["kernel"], 90)),
            "route_decode_p99": float(np.percentile(lat["kernel"], 99)),
            "route_decode_p50_route_every_argument": float(np.percentile(lat["kernel_route"], 50)),
            "route_decode_p50_synchronize": float(np.percentile(lat["kernel_sync"], 50)),
            "route_decode_p50_copy_gather": float(np.percentile(lat["copies"], 50)),
            "route_decode_pipelined_interval": float(pipe_ms),
            "route_decode_pipelined_interval_copy_gather": float(pipe_copy_ms),
            "roofline_floor": float(t_floor_ms),
            "decode_attention_us": float(dec_ms.mean() * 1e3),
            "decode_achieved_GBs": float(dec_bytes / (dec_ms.mean() / 1e3) / 1e9),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


# --------------------------------------------------------------------------
# supporting workloads (one JSON line each; not the headline line)
# --------------------------------------------------------------------------

class CompletionPoll:
    """Waits for the work queued so far on a stream by polling a fence-free
    HIP event (what a latency-bound caller does); a blocking synchronise adds
    its wake-up, ~4 us after a half-millisecond wait."""

    def __init__(self):
        self.ev = HipEvents(1)
        hip = self.ev.hip
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventQuery.argtypes = [ctypes.c_void_p]
        self.hip, self.e = hip, self.ev.pairs[0][0]

    def wait(self, stream):
        assert self.hip.hipEventRecord(self.e, ctypes.c_void_p(stream.cuda_stream)) == 0
        while True:
            st = self.hip.hipEventQuery(self.e)
            if st == 0:
                return
            assert st == 600, f"hipEventQuery returned {st}"     # hipErrorNotReady


class StreamEvents:
    """Event pairs on torch's current stream (the stream the library runs on here)."""

    def __init__(self, n):
        self.pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    def ms(self, i):
        a, b = self.pairs[i]
        return a.elapsed_time(b)


def _router_bank(kr, off, lay):
    """The router bank in the layout the scan reads, and route()'s keywords
    for it: the layout, the row count and the bank's document map, built
    once here (msa_doc_map) as part of the bank, like its layout."""
    n_pool = int(off[-1])
    dmap = msa.doc_map(torch.as_tensor(off, device=kr.device), n_pool)
    return (synth.tile_router_bank(kr) if lay == "tiled" else kr), {"kr_layout": lay, "n_pool": n_pool,
                                                                    "doc_map": dmap}


def _supporting_line(metric, value, unit, workload, roofline, extra, higher=True, kr_layout=None):
    cfg = {"workload": workload}
    if kr_layout:
        cfg["kr_layout"] = kr_layout
    res = {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "higher_is_better": higher,
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": cfg, "roofline": roofline}
    res.update(extra)
    print(json.dumps(res), flush=True)


def workload_interleave(args, dev):
    """Memory interleave at 50M tokens: 64 queries x 3 rounds.  A round routes
    a fresh one-token query per sequence over the whole bank (the wide MFMA
    scan), appends the top-8 documents' pooled K/V from pinned host memory to
    each query's memory (device-side gather), and runs one decode step over
    [memory ; 4096 local tokens] with the query offset by 8 per round so far.
    The memory is reset at the start of every repetition."""
    cfg = synth.config(5)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    n_docs, n_pool = len(lens), int(off[-1])
    log(f"interleave bank: {n_docs} docs, {int(lens.sum())} tokens, {n_pool} pooled rows")
    kr, rkw = _router_bank(synth.pooled_router_bank(cfg, lens, device=dev), off, args.kr_layout)
    host_kv = synth.pooled_content_bank(cfg, lens, device=dev, pin=True)
    off_d = torch.as_tensor(off, device=dev)
    k, B = cfg.top_k, cfg.batch
    mem_cap = cfg.ctx_cap - cfg.local_len
    asm = msa.Assembly.allocate(host_kv, torch.as_tensor(off), B, k, mem_cap, dev)
    lk, lv = synth.local_context(cfg, device=dev)
    loc_len = torch.full((B,), cfg.local_len, dtype=torch.int32, device=dev)
    R = cfg.rounds
    qrs = [synth.router_queries(cfg, step=r, device=dev) for r in range(R)]
    qs = [synth.decode_queries(cfg, step=r, device=dev) for r in range(R)]
    pos = [torch.full((B,), k * (r + 1), dtype=torch.int32, device=dev) for r in range(R)]
    rws = torch.empty(msa.route_workspace_bytes(torch.bfloat16, B, 1, cfg.n_router_heads, cfg.router_dim, n_docs,
                                                n_pool, k), dtype=torch.uint8, device=dev)
    dws = torch.empty(msa.decode_workspace_bytes(B, cfg.n_q_heads, cfg.head_dim, mem_cap, cfg.local_len),
                      dtype=torch.uint8, device=dev)
    dsc = torch.empty((B, n_docs), dtype=torch.float32, device=dev)
    tki = torch.empty((B, k), dtype=torch.int32, device=dev)
    tks = torch.empty((B, k), dtype=torch.float32, device=dev)
    out = torch.empty((B, cfg.n_q_heads, cfg.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, cfg.n_q_heads), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    reps = args.reps
    scan_ev = HipEvents(reps * R)
    route_ev, dec_ev = StreamEvents(reps * R), StreamEvents(reps * R)
    mem_len_log = torch.zeros((reps, R + 1, B), dtype=torch.int32, device=dev)   # read after the timed loop

    def one(rep, timed):
        for r in range(R):
            i = rep * R + r
            asm.append = r > 0
            if timed:
                route_ev.pairs[i][0].record(stream)
            msa.route(qrs[r], kr, off_d, k, dsc, tki, tks, rws, assembly=asm, stream=stream,
                      prof_events=scan_ev.pairs[i] if timed else None, **rkw)
            if timed:
                route_ev.pairs[i][1].record(stream)
                dec_ev.pairs[i][0].record(stream)
            msa.sparse_decode(qs[r], asm.mem_kv, asm.mem_len, lk, lv, loc_len, pos[r], cfg.rope_theta, out, lse,
                              dws, stream=stream)
            if timed:
                dec_ev.pairs[i][1].record(stream)
                mem_len_log[rep, r + 1].copy_(asm.mem_len)         # device copy: no host synchronisation

    for _ in range(2):
        one(0, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for rep in range(reps):
        one(rep, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mem_rows = mem_len_log.to(torch.int64).sum(-1).cpu().numpy()
    scan = np.array([[scan_ev.elapsed_ms(rep * R + r) for r in range(R)] for rep in range(reps)])
    route = np.array([[route_ev.ms(rep * R + r) for r in range(R)] for rep in range(reps)])
    dec = np.array([[dec_ev.ms(rep * R + r) for r in range(R)] for rep in range(reps)])
    kv_row = 2 * cfg.n_kv_heads * cfg.head_dim * 2
    scan_bytes = n_pool * cfg.n_router_heads * cfg.router_dim * 2
    rows_after = mem_rows[:, 1:].mean(0)
    dec_bytes = (rows_after + B * cfg.local_len) * kv_row
    gathered = np.diff(mem_rows, axis=1).mean(0) * kv_row
    per_round = []
    for r in range(R):
        per_round.append({
            "round": r + 1, "scan_us": float(scan[:, r].mean() * 1e3),
            "scan_GBs": float(scan_bytes / (scan[:, r].mean() / 1e3) / 1e9),
            "route_us": float(route[:, r].mean() * 1e3),
            "select_gather_us": float((route[:, r] - scan[:, r]).mean() * 1e3),
            "gathered_bytes": float(gathered[r]), "memory_rows": float(rows_after[r]),
            "decode_us": float(dec[:, r].mean() * 1e3),
            "decode_GBs": float(dec_bytes[r] / (dec[:, r].mean() / 1e3) / 1e9)})
    round_ms = (route + dec).mean()
    achieved = scan_bytes / (scan.mean() / 1e3) / 1e9

    # ---- pipelined rounds (sparse_latent_memory_amd.interleave): round n's
    # assembly crosses the host link while round n + 1 is scored and round
    # n - 1 decoded; one group of R rounds per repetition, memory reset at
    # each group's first round
    pipe = InterleavePipeline(kr, off_d, rkw, host_kv, torch.as_tensor(off), B, k, mem_cap, lk, lv, loc_len,
                              cfg.rope_theta, cfg.n_q_heads)

    def pipelined(n_reps):
        for _ in range(n_reps):
            pipe.run(qrs, qs, pos)

    torch.cuda.synchronize()
    pipelined(1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    pipelined(reps)
    torch.cuda.synchronize()
    pipe_wall = time.perf_counter() - t0
    pipe_round_ms = pipe_wall * 1e3 / (reps * R)
    log(f"interleave: serial {round_ms:.3f} ms per round, pipelined {pipe_round_ms:.3f} ms per round")
    _supporting_line(
        "query-rounds/s (route + gather + decode), memory interleave", B * R * reps / pipe_wall, "query-rounds/s",
        f"interleave-50M: {n_docs} docs, {int(lens.sum())} tokens (lognormal, mean 1024), {n_pool} pooled rows; "
        f"64 queries x {R} rounds of top-{k}, memory <= {mem_cap} rows + {cfg.local_len} local tokens, "
        "GQA 32/8 x 128",
        {"kernel": f"route bank scan, 64 one-token queries (scan_wide_kernel<8, 4, 4>, {args.kr_layout} bank)", "bound": "hbm",
         "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
         "traffic": None},
        {"ms_per_round": float(pipe_round_ms), "ms_per_round_serial": float(round_ms),
         "schedule": "pipelined: round n's assembly overlaps round n+1's routing and round n-1's decode "
                     "(three streams); the per-round figures below are from the serial schedule",
         "rounds": per_round, "reps": reps}, kr_layout=args.kr_layout)


def workload_prefill(args, dev):
    """The 2048-document routing-layer workload: encode the raw 1.31M-token
    bank (document-wise RoPE + chunk means), route one 256-token query
    prefill over it (wide MFMA scan), gather the top-16, run the 256-token
    prefill through [memory ; causal 2048 local tokens] (msa_sparse_attend)
    and one decode step.  The bank is 44.6 MB, so the scan runs out of the
    MALL: reported as warm."""
    cfg = synth.config(2)
    bank = synth.raw_bank(cfg, device=dev)
    lens = bank["lens"]
    off = synth.row_offsets(lens, cfg.pool)
    n_docs, n_pool, n_tok = len(lens), int(off[-1]), int(lens.sum())
    log(f"prefill bank: {n_docs} docs, {n_tok} tokens, {n_pool} pooled rows")
    off_d = torch.as_tensor(off, device=dev)
    kv = torch.empty((n_pool, 2, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device=dev)
    lay = args.kr_layout
    rkw = {"kr_layout": lay, "n_pool": n_pool}
    krp = torch.empty((msa.bank_rows(n_pool, lay), cfg.n_router_heads, cfg.router_dim), dtype=torch.bfloat16,
                      device=dev)
    stream = torch.cuda.current_stream()
    reps = args.reps
    pool_ev = StreamEvents(reps)
    for _ in range(2):
        msa.pool_encode(bank["k"], bank["v"], bank["kr"], bank["doc_tok_off"], off_d, cfg.pool, cfg.rope_theta,
                        n_pool, kv, krp, stream=stream, kr_layout=lay)
    for i in range(reps):
        pool_ev.pairs[i][0].record(stream)
        msa.pool_encode(bank["k"], bank["v"], bank["kr"], bank["doc_tok_off"], off_d, cfg.pool, cfg.rope_theta,
                        n_pool, kv, krp, stream=stream, kr_layout=lay)
        pool_ev.pairs[i][1].record(stream)
    torch.cuda.synchronize()
    pool_ms = np.mean([pool_ev.ms(i) for i in range(reps)])
    elt = 2
    pool_read = n_tok * (2 * cfg.n_kv_heads * cfg.head_dim + cfg.n_router_heads * cfg.router_dim) * elt
    pool_write = n_pool * (2 * cfg.n_kv_heads * cfg.head_dim + cfg.n_router_heads * cfg.router_dim) * elt
    pool_gbs = (pool_read + pool_write) / (pool_ms / 1e3) / 1e9

    host_kv = kv.cpu().pin_memory()
    k = cfg.top_k
    mem_cap = 512
    asm = msa.Assembly.allocate(host_kv, torch.as_tensor(off), 1, k, mem_cap, dev)
    qr = synth.router_queries(cfg, device=dev)
    q = synth.decode_queries(cfg, device=dev)
    lk, lv = synth.local_context(cfg, device=dev)
    loc_len = torch.full((1,), cfg.local_len, dtype=torch.int32, device=dev)
    pos = torch.full((1,), k, dtype=torch.int32, device=dev)
    rws = torch.empty(msa.route_workspace_bytes(torch.bfloat16, 1, cfg.q_tokens, cfg.n_router_heads, cfg.router_dim,
                                                n_docs, n_pool, k), dtype=torch.uint8, device=dev)
    # the prefill itself: the 256 query tokens are the last 256 of the 2048
    # local tokens and attend over [gathered memory ; causal local]
    qp = synth.prefill_queries(cfg, device=dev)
    tq = cfg.q_tokens
    aws = torch.empty(msa.attend_workspace_bytes(1, tq, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, mem_cap,
                                                 cfg.local_len), dtype=torch.uint8, device=dev)
    scan_ev = HipEvents(reps)
    att_ev = HipEvents(reps)
    route_ev, dec_ev, pre_ev = StreamEvents(reps), StreamEvents(reps), StreamEvents(reps)
    for i in range(-2, reps):
        if i >= 0:
            route_ev.pairs[i][0].record(stream)
        msa.route(qr, krp, off_d, k, workspace=rws, assembly=asm, stream=stream,
                  prof_events=scan_ev.pairs[i] if i >= 0 else None, **rkw)
        if i >= 0:
            route_ev.pairs[i][1].record(stream)
            pre_ev.pairs[i][0].record(stream)
        msa.sparse_attend(qp, asm.mem_kv, asm.mem_len, lk, lv, loc_len, pos, cfg.rope_theta, workspace=aws,
                          stream=stream, prof_events=att_ev.pairs[i] if i >= 0 else None)
        if i >= 0:
            pre_ev.pairs[i][1].record(stream)
            dec_ev.pairs[i][0].record(stream)
        msa.sparse_decode(q, asm.mem_kv, asm.mem_len, lk, lv, loc_len, pos, cfg.rope_theta, stream=stream)
        if i >= 0:
            dec_ev.pairs[i][1].record(stream)
    torch.cuda.synchronize()
    scan_ms = np.mean([scan_ev.elapsed_ms(i) for i in range(reps)])
    flops = 2.0 * cfg.q_tokens * n_pool * cfg.n_router_heads * cfg.router_dim
    tfs = flops / (scan_ms / 1e3) / 1e12
    mrows = int(asm.mem_len[0])
    # QK and PV: 4 D flops per (query head, visible key); token t sees mrows + (2048 - 256 + t + 1) keys
    att_flops = 4.0 * cfg.n_q_heads * cfg.head_dim * sum(mrows + cfg.local_len - tq + t + 1 for t in range(tq))
    att_ms = np.mean([att_ev.elapsed_ms(i) for i in range(reps)])
    _supporting_line(
        "pooled tokens/s (encode) and prefill routing", n_tok / (pool_ms / 1e3), "tokens/s",
        f"prefill-1M: {n_docs} docs, lengths U[256,1024], {n_tok} raw tokens -> {n_pool} pooled rows, "
        "K/V 8x128 + Kr 8x128 bf16; 256-token routing query, top-16, decode GQA 32/8x128 over 2048 local tokens",
        {"kernel": "pool_kernel<bf16> (encode)", "bound": "hbm", "achieved": pool_gbs, "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": pool_gbs / HBM_PEAK_GBS, "traffic": None},
        {"encode_us": float(pool_ms * 1e3), "encode_bytes": pool_read + pool_write,
         "routing": {"kernel": f"scan_wide_kernel<8, 4, 4> ({args.kr_layout} bank)", "bound": "mfma", "scan_us": float(scan_ms * 1e3),
                     "achieved_TFs": tfs, "peak_TFs": 2500.0, "frac": tfs / 2500.0, "bank": "MALL-warm (44.6 MB)",
                     "route_us": float(np.mean([route_ev.ms(i) for i in range(reps)]) * 1e3)},
         "prefill_attention": {"kernel": "attend_block_kernel<128, 16> (256 tokens, causal, GQA 32/8; 16 query tiles per workgroup share each key group)", "bound": "mfma",
                               "memory_rows": mrows, "attend_us": float(att_ms * 1e3),
                               "achieved_TFs": att_flops / (att_ms / 1e3) / 1e12,
                               "with_merge_us": float(np.mean([pre_ev.ms(i) for i in range(reps)]) * 1e3)},
         "decode_us": float(np.mean([dec_ev.ms(i) for i in range(reps)]) * 1e3), "reps": reps}, kr_layout=args.kr_layout)


def workload_needles(args, dev):
    """The 16.7M-token bank with 8 one-token queries, each with a planted
    needle (one pooled row at per-head cosine 0.6): scan + top-16, and the
    fraction of queries whose needle document is selected."""
    cfg = synth.config(3)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    n_docs, n_pool = len(lens), int(off[-1])
    log(f"needle bank: {n_docs} docs, {int(lens.sum())} tokens, {n_pool} pooled rows")
    kr = synth.pooled_router_bank(cfg, lens, device=dev)
    qr = synth.router_queries(cfg, device=dev)
    needles = synth.plant_needles(cfg, qr, kr, off)
    kr, rkw = _router_bank(kr, off, args.kr_layout)
    off_d = torch.as_tensor(off, device=dev)
    k = cfg.top_k
    rws = torch.empty(msa.route_workspace_bytes(torch.bfloat16, cfg.batch, 1, cfg.n_router_heads, cfg.router_dim,
                                                n_docs, n_pool, k), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    reps = args.reps
    scan_ev = HipEvents(reps)
    route_ev = StreamEvents(reps)
    for i in range(-2, reps):
        if i >= 0:
            route_ev.pairs[i][0].record(stream)
        idx, _, _ = msa.route(qr, kr, off_d, k, workspace=rws, stream=stream,
                              prof_events=scan_ev.pairs[i] if i >= 0 else None, **rkw)
        if i >= 0:
            route_ev.pairs[i][1].record(stream)
    torch.cuda.synchronize()
    found = float(np.mean([needles[b] in set(idx[b].cpu().tolist()) for b in range(cfg.batch)]))
    scan_ms = np.mean([scan_ev.elapsed_ms(i) for i in range(reps)])
    route_ms = np.mean([route_ev.ms(i) for i in range(reps)])
    scan_bytes = n_pool * cfg.n_router_heads * cfg.router_dim * 2
    achieved = scan_bytes / (scan_ms / 1e3) / 1e9
    _supporting_line(
        "bank tokens scored/s, 8 queries with planted needles", cfg.batch * int(lens.sum()) / (route_ms / 1e3),
        "bank tokens/s",
        f"needles-16M: {n_docs} docs, {int(lens.sum())} tokens (lognormal, mean 512), {n_pool} pooled rows, "
        "8 one-token queries, top-16",
        {"kernel": "route bank scan, 8 one-token queries (scan_mfma_kernel<8, 4, 1, "
                   f"{'true' if args.kr_layout == 'tiled' else 'false'}, true>)", "bound": "hbm",
         "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
         "traffic": None},
        {"scan_us": float(scan_ms * 1e3), "route_us": float(route_ms * 1e3), "needle_recall_top16": found,
         "reps": reps}, kr_layout=args.kr_layout)


def workload_encode(args, dev):
    """Streaming encode of the 100M-token bank (195,313 documents x 512
    tokens) in batches of 2048 documents: each batch's pooled K/V go
    straight into the 6.4 GB pinned host tier and its pooled router keys
    into the 3.2 GB HBM bank, at the batch's row offset.  The raw K/V/Kr of a
    batch (6 GiB) are synthetic and stay resident; every batch reads them
    from HBM again (they are 24x the MALL).  The same stream is also timed
    with the pooled K/V written to HBM."""
    cfg = synth.config(4)
    lens = synth.doc_lengths(cfg)
    off = synth.row_offsets(lens, cfg.pool)
    n_docs, n_pool, n_tok = len(lens), int(off[-1]), int(lens.sum())
    per = 2048
    enc = synth.config(4, n_docs=per)
    bank = synth.raw_bank(enc, device=dev)
    boff = synth.row_offsets(bank["lens"], enc.pool)
    tok_off_h = synth.token_offsets(bank["lens"])
    log(f"encode: {n_docs} docs, {n_tok} tokens -> {n_pool} rows, batches of {per} docs")
    tier = torch.empty((n_pool, 2, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16, pin_memory=True)
    lay = args.kr_layout
    kr_bank = torch.empty((msa.bank_rows(n_pool, lay), cfg.n_router_heads, cfg.router_dim), dtype=torch.bfloat16,
                          device=dev)
    stage = torch.empty((int(boff[-1]), 2, cfg.n_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device=dev)
    batches = []
    for d0 in range(0, n_docs, per):
        nd = min(per, n_docs - d0)
        nt, npb = int(tok_off_h[nd]), int(boff[nd])
        batches.append((int(off[d0]), nd, nt, npb,
                        torch.as_tensor(tok_off_h[:nd + 1], device=dev), torch.as_tensor(boff[:nd + 1], device=dev)))
    stream = torch.cuda.current_stream()

    def run(to_host):
        for r0, nd, nt, npb, toff, poff in batches:
            kv_out = tier[r0:r0 + npb] if to_host else stage[:npb]
            msa.pool_encode(bank["k"][:nt], bank["v"][:nt], bank["kr"][:nt], toff, poff, cfg.pool, cfg.rope_theta,
                            npb, kv_out, kr_bank, stream=stream, kr_layout=lay, kr_row_base=r0)

    res = {}
    for name, to_host in (("host_tier", True), ("hbm", False)):
        run(to_host)
        torch.cuda.synchronize()
        times = []
        for _ in range(max(1, args.reps // 5)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run(to_host)
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        res[name] = float(np.median(times))
    hbm_bytes = n_tok * 6144 + n_pool * 6144
    host_bytes = n_pool * 2 * cfg.n_kv_heads * cfg.head_dim * 2
    t_host = res["host_tier"] / 1e3
    achieved = hbm_bytes / t_host / 1e9
    _supporting_line(
        "bank tokens encoded/s into the host tier (streaming encode)", n_tok / t_host, "tokens/s",
        f"encode-100M: {n_docs} docs x 512 tokens = {n_tok} tokens -> {n_pool} pooled rows in {len(batches)} batches "
        f"of {per} docs; pooled K/V (8x128 bf16, {host_bytes / 1e9:.2f} GB) into pinned host memory, pooled Kr into "
        f"the HBM bank ({lay} layout, each batch at its first row)",
        {"kernel": "pool_kernel<bf16> (encode, K/V written over the host link)", "bound": "hbm",
         "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
         "traffic": None},
        {"ms_total_host_tier": res["host_tier"], "ms_total_kv_to_hbm": res["hbm"],
         "host_link_GBs": host_bytes / t_host / 1e9, "tokens_per_s_kv_to_hbm": n_tok / (res["hbm"] / 1e3),
         "batches": len(batches), "reps": max(1, args.reps // 5)}, kr_layout=args.kr_layout)


WORKLOADS = {"bank-100M": None, "encode-100M": workload_encode, "interleave-50M": workload_interleave, "prefill-1M": workload_prefill,
             "needles-16M": workload_needles}


def cpu_baseline(cfg, kr, pool_off, qr, seconds, step_in=None):
    """The float64 CPU oracle on a bounded sample of the same step, on one
    thread (its elementwise NumPy work is single-threaded anyway; BLAS is
    held to one thread too).  Routing: consecutive blocks of 2048 documents
    from the start of the bank, scored until `seconds` of CPU time have
    passed; the first block is also timed with every thread of the process
    allowed.  With `step_in`, the rest of the step is timed once each: the
    encode batch (oracle.pool), the top-k over the sampled scores, and the
    decode step over the gathered memory and the local context; the
    whole-step rate scales the scoring and the top-k from the sample to the
    full bank (both are linear in the documents) and adds the other two."""
    import oracle
    from threadpoolctl import threadpool_limits

    qn = qr.detach().cpu().float().double().numpy()
    block = 2048
    done_docs, spent = 0, 0.0
    n_docs = len(pool_off) - 1
    parts = []
    with threadpool_limits(limits=1):
        while spent < seconds and done_docs < n_docs:
            d0, d1 = done_docs, min(done_docs + block, n_docs)
            rows = kr[pool_off[d0]:pool_off[d1]].float().cpu().double().numpy()
            t = time.perf_counter()
            parts.append(oracle.doc_scores(qn, rows, pool_off[d0:d1 + 1] - pool_off[d0]))
            spent += time.perf_counter() - t
            done_docs = d1
        step = None
        if step_in is not None:
            f64 = lambda x: x.detach().float().cpu().double().numpy()
            i64 = lambda x: x.detach().cpu().numpy().astype(np.int64)
            dsc = np.concatenate(parts, axis=1)
            t = time.perf_counter()
            oracle.topk(dsc, step_in["k"])
            t_topk = time.perf_counter() - t
            eb = step_in["enc_bank"]
            ek, ev, ekr = f64(eb["k"]), f64(eb["v"]), f64(eb["kr"])
            t = time.perf_counter()
            oracle.pool(ek, ev, ekr, step_in["enc_tok_off"], step_in["enc_pool"], step_in["rope_theta"])
            t_pool = time.perf_counter() - t
            dq, dm, dlk, dlv = f64(step_in["q"]), f64(step_in["mem_kv"]), f64(step_in["local_k"]), f64(step_in["local_v"])
            t = time.perf_counter()
            oracle.decode(dq, dm, i64(step_in["mem_len"]), dlk, dlv, i64(step_in["local_len"]), i64(step_in["pos"]),
                          step_in["rope_theta"])
            t_dec = time.perf_counter() - t
            scale = n_docs / done_docs
            t_step = (spent + t_topk) * scale + t_pool + t_dec
            step = {"step_s": t_step, "scoring_s": spent * scale, "topk_s": t_topk * scale, "encode_batch_s": t_pool,
                    "decode_s": t_dec, "scoring_rate": done_docs * 512 * cfg.batch / spent}
    tokens = done_docs * 512
    allowed = len(os.sched_getaffinity(0))
    b_all = min(block, n_docs)
    rows = kr[pool_off[0]:pool_off[b_all]].float().cpu().double().numpy()
    t = time.perf_counter()
    oracle.doc_scores(qn, rows, pool_off[:b_all + 1])
    t_all = time.perf_counter() - t
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    res = {"value": tokens * cfg.batch / spent, "unit": "bank tokens/s", "cores": 1, "kind": "oracle",
           "sample": f"oracle.doc_scores (NumPy float64, one thread) over the first {done_docs} documents "
                     f"({tokens} bank tokens, {int(pool_off[done_docs])} pooled rows) of the same bank, "
                     f"one query token, in blocks of {block} documents; {spent:.1f} s of compute",
           "all_threads_value": b_all * 512 * cfg.batch / t_all, "all_threads": allowed, "cpu_model": model}
    if step is not None:
        res["value"] = n_docs * 512 * cfg.batch / step["step_s"]
        res["sample"] = (f"the whole step's oracle (NumPy float64, one thread): oracle.doc_scores over the first "
                         f"{done_docs} documents ({tokens} bank tokens, {int(pool_off[done_docs])} pooled rows) of "
                         f"the same bank in blocks of {block} documents ({spent:.1f} s) and oracle.topk over their "
                         f"scores, both scaled to all {n_docs} documents, plus oracle.pool of the 64-document encode "
                         f"batch and oracle.decode of the step's query; value = bank tokens / that step time")
        res["step_components_s"] = {k_: round(v_, 4) for k_, v_ in step.items() if k_.endswith("_s")}
        res["scoring_only_value"] = step["scoring_rate"]
    return res


if __name__ == "__main__":
    main()
