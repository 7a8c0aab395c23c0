"""Benchmark of block-sparse FP8 attention prefill on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sparse16k]

One step is one launch of the whole prefill (compaction, paged gather, both
FP8 MFMA products, online softmax, P quantisation, epilogue) over the full
synthetic workload, with every input already resident in HBM.  Prints one
JSON line.

Throughput counts the algorithmic work of the active tiles only: every
(sequence, q-head, 128-query tile, 128-key tile) pair whose mask byte is on,
that lies below the KV length and inside the causal range, is 2*128*128*128
FLOP for Q.K^T plus the same for P.V, i.e. 8,388,608 FLOP, and reads 32 KiB
of K and V (plus 512 B of K descales with per-token K scales).
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

TILE = 128
FLOP_PER_TILE = 4 * TILE * TILE * TILE          # 8,388,608
KV_BYTES_PER_TILE = 2 * TILE * TILE             # 32,768
PEAK_FP8_TFLOPS = 5000.0                        # MI355X dense FP8 MFMA
PEAK_F16_TFLOPS = 2500.0                        # MI355X dense f16 / bf16 MFMA
PEAK_CLOCK_GHZ = 2.4                            # the clock both peaks are quoted at
PEAK_HBM_GBPS = 8000.0
METRIC = "effective FP8 TFLOPS (active tiles) + prefill tokens/s; % of FP8 MFMA peak"
_CSRC = os.path.join(ROOT, "block_sparse_fp8_amd", "csrc")
# per operation: the kernel source the counters belong to and the kernel's name
KERNELS = {
    "prefill": (os.path.join(_CSRC, "bsa_fp8_prefill.hip"), "bsa_fp8_prefill_kernel"),
    "quantize_append": (os.path.join(_CSRC, "bsa_fp8_quantize.hip"), "bsa_fp8_quantize_kernel"),
    "decode": (os.path.join(_CSRC, "bsa_fp8_decode.hip"), "bsa_fp8_decode_kernel"),
}
KERNEL_SOURCE = KERNELS["prefill"][0]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 256 * 1024 * 1024   # size of the calibration copy (see --ingest-counters)


def kernel_source_hash(op="prefill"):
    with open(KERNELS[op][0], "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _traffic_key(workload, op):
    return workload if op == "prefill" else f"{op}:{workload}"


def traffic_record(workload, op="prefill"):
    """The rocprofv3 FETCH_SIZE / WRITE_SIZE record of this exact kernel source
    for the operation and workload, or None when there is none or the source
    changed since."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[_traffic_key(workload, op)]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash(op):
        return None
    return rec


def recorded_traffic(workload, op="prefill"):
    """HBM bytes (read + written) per launch from the record, or None."""
    rec = traffic_record(workload, op)
    return None if rec is None else rec["hbm_bytes_per_launch"]


WARMUP_MIN_S = 0.1   # default warm-up: at least this long (the clock settles within ~30 ms of work)


def warm_up(step, args):
    """Untimed warm-up: exactly --warmup steps when given, else at least 10
    steps and at least WARMUP_MIN_S of wall time.  Returns the step count,
    which the JSON line reports as "warmup"."""
    import torch
    if args.warmup is not None:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        return args.warmup
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= WARMUP_MIN_S:
            return n


# the library's Q.K^T path when the call leaves qk_precision at its default
DEFAULT_QK = "fp8split"
QK_CODES = {"default": 0, "f16": 1, "fp8": 2, "fp8split": 3}
QK_DTYPES = {
    "f16": "Q.K^T on f16 MFMA (E4M3 codes widened exactly to f16), P.V on fp8_e4m3 MFMA, "
           "fp32 accumulate, bf16 out",
    "fp8": "fp8_e4m3 MFMA for Q.K^T and P.V, fp32 accumulate, bf16 out",
    "fp8split": "fp8_e4m3 MFMA for Q.K^T (two products per K operand, query codes split by "
                "magnitude) and P.V, fp32 accumulate, bf16 out",
}


def qk_path(qk):
    return DEFAULT_QK if qk == "default" else qk


def qk_ceiling_tflops(qk):
    """Matrix-core ceiling of one tile's instruction mix: Q.K^T and P.V carry
    equal FLOP; with Q.K^T at half the FP8 rate (f16 MFMA, or two FP8 products
    per operand) the mix tops out at 1 / (0.5 / 2500 + 0.5 / 5000) = 3333 TFLOP/s."""
    if qk_path(qk) == "fp8":
        return PEAK_FP8_TFLOPS
    return 1.0 / (0.5 / PEAK_F16_TFLOPS + 0.5 / PEAK_FP8_TFLOPS)


def _clock_key(workload, qk):
    return f"clock:{workload}:{qk_path(qk)}"


def clock_record(workload, qk):
    """The shader clock measured for this kernel source and workload, or None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[_clock_key(workload, qk)]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash("prefill"):
        return None
    return rec


def ingest_clock(workload, qk, directory, command):
    """Record the prefill kernel's mean shader clock from a GRBM_GUI_ACTIVE pass:
    the counter sums busy cycles over the XCDs, so one XCD's cycles divided by
    the dispatch's own start-to-end time is the clock it ran at."""
    kname = KERNELS["prefill"][1]
    nxcc = 8
    for path in glob.glob(os.path.join(directory, "**", "*agent_info.csv"), recursive=True):
        for row in csv.DictReader(open(path)):
            if row.get("Name", "").startswith("gfx") and row.get("Num_Xcc"):
                nxcc = int(row["Num_Xcc"])
    ghz, ns = [], []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(path)):
            if kname in row["Kernel_Name"] and row["Counter_Name"] == "GRBM_GUI_ACTIVE":
                dur = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
                ghz.append(float(row["Counter_Value"]) / nxcc / dur)
                ns.append(dur)
    rec = {"kernel_source_sha256": kernel_source_hash("prefill"), "num_xcc": nxcc,
           "dispatches": len(ghz), "clock_ghz_mean": sum(ghz) / len(ghz),
           "clock_ghz_min": min(ghz), "clock_ghz_max": max(ghz),
           "dispatch_ns_mean": sum(ns) / len(ns), "command": command}
    try:
        allrec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        allrec = {}
    allrec[_clock_key(workload, qk)] = rec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(allrec, fh, indent=1, sort_keys=True)
    print(json.dumps(rec))


def _counter_means(directory, kernel_substr):
    vals = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(path)):
            if kernel_substr in row["Kernel_Name"]:
                vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def ingest_counters(workload, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, command, op="prefill"):
    """Record FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the operation's
    kernel, scaled by what the same counters read for a plain copy of
    COPY_BYTES."""
    kname = KERNELS[op][1]
    f = _counter_means(fetch_dir, kname)["FETCH_SIZE"]
    w = _counter_means(write_dir, kname)["WRITE_SIZE"]
    cf = _counter_means(cal_fetch_dir, "copyBuffer")["FETCH_SIZE"]
    cw = _counter_means(cal_write_dir, "copyBuffer")["WRITE_SIZE"]
    fetch_scale = COPY_BYTES / (cf * 1024)
    write_scale = COPY_BYTES / (cw * 1024)
    rec = {"kernel_source_sha256": kernel_source_hash(op),
           "fetch_kib_per_launch": f, "write_kib_per_launch": w,
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "hbm_bytes_per_launch": f * 1024 * fetch_scale + w * 1024 * write_scale,
           "command": command}
    try:
        allrec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        allrec = {}
    allrec[_traffic_key(workload, op)] = rec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(allrec, fh, indent=1, sort_keys=True)
    print(json.dumps(rec))


def active_tiles(p):
    """Per (b, h, m): number of active KV tiles and the number of (query, key)
    pairs they contribute (for the stricter 'useful' FLOP count)."""
    n_act = 0
    pairs = 0
    B = len(p.seqlens_kv)
    Hq = p.q.shape[1]
    for b in range(B):
        t0 = int(p.cu_seqlens_q[b])
        lq = int(p.cu_seqlens_q[b + 1]) - t0
        lkv = int(p.seqlens_kv[b])
        kv_tiles = (lkv + TILE - 1) // TILE
        for m in range((lq + TILE - 1) // TILE):
            rows = np.arange(m * TILE, min(m * TILE + TILE, lq))
            pos = lkv - lq + rows
            n_end = kv_tiles
            if p.causal:
                n_end = min(n_end, int(pos.max()) // TILE + 1)
            if p.block_mask is not None:
                n_end = min(n_end, p.block_mask.shape[3])
                on = p.block_mask[b, :, m, :n_end] != 0          # [Hq, n_end]
            else:
                on = np.ones((Hq, n_end), dtype=bool)
            n_act += int(on.sum())
            # pairs per tile n: sum over rows of clip(min(p_t+1, lkv) - 128n, 0, 128)
            n = np.arange(n_end)
            lim = np.minimum(pos + 1 if p.causal else lkv, lkv)
            cnt = np.clip(lim[None, :] - n[:, None] * TILE, 0, TILE).sum(axis=1)   # [n_end]
            pairs += int((on * cnt[None, :]).sum())
    return n_act, pairs


def cpu_baseline(p, n_act_total, budget_s):
    """Time the oracle, as it stands, on a bounded sample of Q tiles: two thirds
    of the budget in its P-emulating mode (the reported value), one third in its
    exact mode (reported beside it)."""
    from oracle import attention as A
    from synth.workloads import sample_q_tiles
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    tiles = sample_q_tiles(p, 100000, seed=2)
    rng = np.random.default_rng(3)
    rng.shuffle(tiles)
    kw = p.oracle_kwargs()

    def run(mode, todo, budget):
        done, flop = [], 0
        t_start = time.perf_counter()
        for tile in todo:
            A.prefill(**kw, mode=mode, tiles=[tile])
            done.append(tile)
            if time.perf_counter() - t_start > budget:
                break
        elapsed = time.perf_counter() - t_start
        for (b, h, m) in done:
            lq = int(p.cu_seqlens_q[b + 1] - p.cu_seqlens_q[b])
            lkv = int(p.seqlens_kv[b])
            pos_max = lkv - lq + min(m * TILE + TILE - 1, lq - 1)
            n_end = min((lkv + TILE - 1) // TILE, pos_max // TILE + 1)
            flop += FLOP_PER_TILE * int((p.block_mask[b, h, m, :n_end] != 0).sum())
        return flop / elapsed / 1e12, len(done), elapsed

    emu, n_emu, t_emu = run("emulate", tiles, budget_s * 2 / 3)
    exa, n_exa, t_exa = run("exact", tiles[::-1], budget_s / 3)
    return {"value": emu, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{n_emu} of {p.num_q_tiles} Q tiles (seeded random order), "
                      f"P-emulating fp64 NumPy oracle, {t_emu:.1f} s wall; "
                      f"host cpu_count={os.cpu_count()}",
            "exact_value": exa,
            "exact_sample": f"{n_exa} Q tiles from the other end of the same order, exact fp64 mode, "
                            f"{t_exa:.1f} s wall"}


def bench_quantize_append(p, args):
    """Time bsa_fp8_quantize_append over the workload's query chunk: Q to E4M3
    with per-(token, head) descales, the chunk's K and V appended to the paged
    cache.  Algorithmic HBM bytes per row of 128 values: 256 read (bf16) and
    128 written (E4M3), plus a 4-byte descale for Q rows and for K rows of
    quant type 1."""
    import torch
    import block_sparse_fp8_amd as bsa
    from synth import append_inputs

    a = append_inputs(p, seed=0, spread=False)
    d = p.to_device("cuda")
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    q_in, k_in, v_in = (t(a[n]).to(torch.bfloat16) for n in ("q", "k", "v"))
    ks, vs = t(a["kscale"]), t(a["vscale"])
    T, Hq, D = p.q.shape
    Hkv = p.cfg.hkv
    q_out = torch.empty((T, Hq, D), dtype=torch.float8_e4m3fn, device="cuda")
    qs_out = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    kcache_scale = d["kscale"] if p.quant_type == 1 else None

    def step():
        bsa.bsa_fp8_quantize_append(q_in, k_in, v_in, d["cu_seqlens_q"], d["seqlens_kv"],
                                    d["block_table"], ks, vs, p.quant_type, p.page_size,
                                    kcache=d["kcache"], vcache=d["vcache"],
                                    kscale_cache=kcache_scale, kv_layout=p.kv_layout,
                                    q_out=q_out, qscale_out=qs_out,
                                    scale_mode=1 if args.scale_mode == "pow2" else 0)

    warmup = warm_up(step, args)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_, e_ in ev:
        s_.record(stream)
        step()
        e_.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = np.array([s_.elapsed_time(e_) for s_, e_ in ev])
    rows_q, rows_kv = T * Hq, T * Hkv
    nbytes = (rows_q * (256 + 128 + 4) + rows_kv * (256 + 128 + (4 if p.quant_type == 1 else 0))
              + rows_kv * (256 + 128))
    med = float(np.median(kernel_ms)) / 1e3
    res = {
        "metric": "FP8 quantise-and-append HBM GB/s (algorithmic bytes)",
        "value": round(nbytes / (wall / args.steps) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, fp8_e4m3 out (fp32 arithmetic)",
        "data": "synthetic (seeded N(0,1) bfloat16)",
        "config": {"workload": f"{p.cfg.name} query chunk: {T} tokens, Hq {Hq}, Hkv {Hkv}, "
                               f"quant {p.quant_type}", "rows": rows_q + 2 * rows_kv,
                   "bytes_per_launch": nbytes, "scale_mode": args.scale_mode},
        "kernel_ms_min": round(float(kernel_ms.min()), 4),
        "kernel_ms_median": round(float(np.median(kernel_ms)), 4),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / med / 1e9, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(nbytes / med / 1e9 / PEAK_HBM_GBPS, 4),
                     "traffic": (recorded_traffic(p.cfg.name, "quantize_append")
                                 if args.scale_mode == "amax" else None)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_quantize(p, a, args.cpu_budget)
    print(json.dumps(res), flush=True)


def cpu_baseline_quantize(p, a, budget_s):
    """Time the quantise-and-append oracle, as it stands, on growing prefixes of
    the first sequence's chunk (the tokens keep their places at the tail of the
    sequence) until the budget is spent; GB/s over the same algorithmic bytes."""
    from oracle import quantize as Qz
    Hq, Hkv = p.q.shape[1], p.cfg.hkv
    lq0 = int(p.cu_seqlens_q[1] - p.cu_seqlens_q[0])
    n, best, t_total = 64, None, 0.0
    while n <= lq0:
        cu = np.array([0, n], dtype=np.int32)
        lkv = np.array([int(p.seqlens_kv[0]) - lq0 + n], dtype=np.int32)
        t0 = time.perf_counter()
        Qz.quantize_append(a["q"][:n], a["k"][:n], a["v"][:n], cu, lkv, p.block_table[:1], a["kscale"],
                           a["vscale"], p.quant_type, p.page_size, p.kv_layout, p.kcache, p.vcache,
                           p.kscale if p.quant_type == 1 else None)
        dt = time.perf_counter() - t0
        t_total += dt
        nbytes = n * (Hq * (256 + 128 + 4) + Hkv * (256 + 128 + (4 if p.quant_type == 1 else 0)) + Hkv * 384)
        best = (nbytes / dt / 1e9, n, dt)
        if t_total > budget_s or n == lq0:
            break
        n = min(2 * n, lq0)
    return {"value": best[0], "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{best[1]} of {p.q.shape[0]} tokens of the chunk in one call, {best[2]:.1f} s "
                      f"(NumPy, single-threaded elementwise work); host cpu_count={os.cpu_count()}"}


PEAK_BF16_TFLOPS = 2500.0                        # MI355X dense bf16 MFMA


def bench_decode(args):
    """Time bsa_fp8_sparse_decode (bsa_fp8_sparse_decode_ex when the lists are
    split into parts).  Work per query token and head: the selected tokens
    (valid indices) times 2*(576 + 512) FLOP (Q.K over 576 dims, P.V over 512),
    the count the FlashMLA article uses; bytes: 656 per selected token per query
    token (the gathered cache rows), plus Q and O."""
    import torch
    import block_sparse_fp8_amd as bsa
    from synth import make_decode_problem, DECODE_CONFIGS

    name = args.workload if args.workload in DECODE_CONFIGS else "decode_b128"
    p = make_decode_problem(name)
    d = p.to_device("cuda")
    B, s_q, h_q, _ = p.q.shape
    n_rows = p.kv_cache.shape[0] * p.kv_cache.shape[1]
    valid = ((p.indices >= 0) & (p.indices < n_rows)).sum()
    flop = float(valid) * h_q * 2 * (576 + 512)
    nbytes = float(valid) * 656 + B * s_q * h_q * (576 * 2 + 512 * 2)
    out = torch.empty((B, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, h_q, s_q), dtype=torch.float32, device="cuda")
    topk = p.indices.shape[2]
    splits = (bsa.bsa_fp8_sparse_decode_num_splits(B, s_q, h_q, topk) if args.splits == "auto"
              else int(args.splits))
    ws = torch.empty(max(1, bsa.bsa_fp8_sparse_decode_workspace_bytes(B, s_q, h_q, splits)),
                     dtype=torch.uint8, device="cuda")

    def step():
        if splits == 1:
            bsa.bsa_fp8_sparse_decode(d["q"], d["kv_cache"], d["indices"], softmax_scale=p.softmax_scale,
                                      out=out, lse=lse)
        else:
            bsa.bsa_fp8_sparse_decode_ex(d["q"], d["kv_cache"], d["indices"], num_splits=splits, workspace=ws,
                                         softmax_scale=p.softmax_scale, out=out, lse=lse)

    warmup = warm_up(step, args)
    if args.graph:
        # the call captured once and replayed: what a serving loop does to drop launch costs
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
    else:
        run = step
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s_, e_ in ev:
        s_.record(stream)
        run()
        e_.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = np.array([s_.elapsed_time(e_) for s_, e_ in ev])
    med = float(np.median(kernel_ms)) / 1e3
    avg = float(kernel_ms.mean()) / 1e3
    res = {
        "metric": "FP8 sparse decode TFLOPS (selected tokens, 2*(576+512) FLOP per token and head)",
        "value": round(flop / (wall / args.steps) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 (fp8_e4m3 cache dequantised to bf16, fp32 accumulate)",
        "data": "synthetic (seeded N(0,1); power-of-two tile descales)",
        "config": {"workload": f"{p.cfg.name}: {p.cfg.description}", "selected_tokens": int(valid),
                   "query_tokens": B * s_q, "num_splits": splits, "graph": bool(args.graph)},
        "kernel_ms_min": round(float(kernel_ms.min()), 4),
        "kernel_ms_median": round(float(np.median(kernel_ms)), 4),
        "kernel_ms_mean": round(avg * 1e3, 4),
        "kv_gbps_logical": round(nbytes / med / 1e9, 1),
        # achieved over the mean launch; traffic: the rocprofv3 record of this
        # decode source for the single-part launch of this workload, else null
        "roofline": {"bound": "mfma", "achieved": round(flop / avg / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(flop / avg / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(p.cfg.name, "decode") if splits == 1 else None},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(p, args.cpu_budget)
    print(json.dumps(res), flush=True)


def cpu_baseline_decode(p, budget_s):
    """Time the decode oracle, as it stands, one query token at a time over a
    seeded sample of the workload's query tokens until the budget is spent."""
    from oracle import decode as D
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    B, s_q, h_q, _ = p.q.shape
    order = np.random.default_rng(4).permutation(B * s_q)
    flop, done = 0.0, 0
    t0 = time.perf_counter()
    for i in order:
        b, s = divmod(int(i), s_q)
        D.sparse_decode(p.q[b:b + 1, s:s + 1], p.kv_cache, p.indices[b:b + 1, s:s + 1], p.softmax_scale)
        idx = p.indices[b, s]
        flop += float(D.valid_entries(idx, p.kv_cache).size) * h_q * 2 * (576 + 512)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    elapsed = time.perf_counter() - t0
    return {"value": flop / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of {B * s_q} query tokens (seeded order), fp64 NumPy oracle, "
                      f"{elapsed:.1f} s wall; host cpu_count={os.cpu_count()}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 10 and at least 0.1 s of them)")
    ap.add_argument("--workload", default="sparse16k")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--form", choices=("mask", "list"), default="mask",
                    help="sparsity argument: the uint8 block mask, or the same tiles as ascending "
                         "index lists (sparse_indices + sparse_seq_len)")
    ap.add_argument("--op", choices=("prefill", "quantize_append", "decode"), default="prefill",
                    help="prefill (the default, the headline metric); the FP8 quantise-and-append "
                         "step that produces its inputs (GB/s against HBM); or FP8 sparse decode "
                         "(MQA over 656-byte cache rows, TFLOP/s against the bf16 matrix peak; "
                         "workload decode_b128 unless --workload names another decode config)")
    ap.add_argument("--no-flushed", dest="flushed", action="store_false",
                    help="prefill: skip the second timing pass, in which a 512 MiB buffer is written "
                         "before each launch (cold caches; reported as kernel_ms_flushed_median)")
    ap.add_argument("--flushed", dest="flushed", action="store_true",
                    help="prefill: run the cold-cache pass (the default)")
    ap.add_argument("--graph", action="store_true",
                    help="decode only: capture the call in a HIP graph and time its replays")
    ap.add_argument("--splits", default="auto",
                    help="decode only: parts per index list (an integer, or 'auto' for the library's "
                         "choice; 1 is the single-pass kernel)")
    ap.add_argument("--qk", choices=tuple(QK_CODES), default="default",
                    help="matrix path of the prefill's Q.K^T products (bsa_qk_precision)")
    ap.add_argument("--scale-mode", choices=("amax", "pow2"), default="amax",
                    help="quantize_append: descales amax/448 as computed, or rounded up to powers of two")
    ap.add_argument("--q-layout", choices=("tnd", "ntd"), default="tnd",
                    help="prefill: query layout, TND (q [T,Hq,128]) or NTD (q [Hq,T,128], qscale [Hq,T])")
    ap.add_argument("--schedule", action="store_true",
                    help="run the scheduling pre-pass inside every step and launch the prefill "
                         "in its task order")
    ap.add_argument("--ingest-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="record HBM traffic of --op's kernel on --workload from rocprofv3 counter CSV "
                         "directories and exit")
    ap.add_argument("--ingest-clock", metavar="GRBM_DIR",
                    help="record the prefill kernel's shader clock from a rocprofv3 --pmc GRBM_GUI_ACTIVE "
                         "run of the same workload and --qk")
    ap.add_argument("--ingest-command", default="", help="command line recorded with --ingest-counters")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 256 MiB (x3), for calibrating FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        x = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copied_bytes": COPY_BYTES, "copies": 3}))
        return
    if args.ingest_clock:
        ingest_clock(args.workload, args.qk, args.ingest_clock, args.ingest_command)
        return
    if args.ingest_counters:
        ingest_counters(args.workload, *args.ingest_counters, command=args.ingest_command, op=args.op)
        return
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(the prefill shards by kv-head: each GPU takes Hkv/N kv-heads with their q-heads "
              "and needs no communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_fp8_amd as bsa
    from synth import make_problem

    if args.op == "decode":
        bench_decode(args)
        return
    p = make_problem(args.workload)
    if args.op == "quantize_append":
        bench_quantize_append(p, args)
        return
    n_act, pairs = active_tiles(p)
    d = p.to_device("cuda")
    T, Hq, D = p.q.shape
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((Hq, T), dtype=torch.float32, device="cuda")

    si = sl = None
    if args.form == "list":
        from synth import index_form
        idx, slen = index_form(p, "ascending", junk=False)
        si = torch.from_numpy(idx).cuda()
        sl = torch.from_numpy(slen).cuda()
    mask = d["block_mask"] if si is None else None
    q_dev, qs_dev, q_layout = d["q"], d["qscale"], bsa.QLayout.TND
    if args.q_layout == "ntd":
        from synth import to_ntd
        q_ntd, qs_ntd = to_ntd(p)
        q_dev, qs_dev = torch.from_numpy(q_ntd).cuda(), torch.from_numpy(qs_ntd).cuda()
        q_layout = bsa.QLayout.NTD
    sched = ws = None
    if args.schedule:
        ntasks = len(p.seqlens_kv) * Hq * ((p.max_seqlen_q + TILE - 1) // TILE)
        sched = torch.empty(ntasks, dtype=torch.int32, device="cuda")
        ws = torch.empty(bsa.bsa_fp8_schedule_workspace_bytes(len(p.seqlens_kv), Hq, p.max_seqlen_q),
                         dtype=torch.uint8, device="cuda")

    def pre_pass():
        bsa.bsa_fp8_schedule(d["cu_seqlens_q"], d["seqlens_kv"], mask, num_heads_q=Hq,
                             max_seqlen_q=p.max_seqlen_q, causal=p.causal, sparse_indices=si,
                             sparse_seq_len=sl, workspace=ws, schedule=sched)

    qk = QK_CODES[args.qk]

    def step():
        if args.form == "mask" and not args.schedule and qk == 0 and args.q_layout == "tnd":
            bsa.bsa_fp8_prefill(d["q"], d["kcache"], d["vcache"], d["qscale"], d["kscale"],
                                d["vscale"], d["cu_seqlens_q"], d["block_table"], d["seqlens_kv"],
                                d["block_mask"], p.quant_type, p.page_size,
                                max_seqlen_q=p.max_seqlen_q, kv_layout=p.kv_layout,
                                causal=p.causal, softmax_scale=p.softmax_scale, out=out, lse=lse)
            return
        if args.schedule:
            pre_pass()
        bsa.bsa_fp8_prefill_ex(q_dev, d["kcache"], d["vcache"], qs_dev, d["kscale"],
                               d["vscale"], d["cu_seqlens_q"], d["block_table"], d["seqlens_kv"],
                               mask, p.quant_type, p.page_size, max_seqlen_q=p.max_seqlen_q,
                               kv_layout=p.kv_layout, causal=p.causal,
                               softmax_scale=p.softmax_scale, q_layout=q_layout, sparse_indices=si,
                               sparse_seq_len=sl, schedule=sched, qk_precision=qk, out=out, lse=lse)

    warmup = warm_up(step, args)
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = np.array([s.elapsed_time(e) for s, e in ev])
    schedule_ms = None
    if args.schedule:
        pe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for s, e in pe:
            s.record(stream)
            pre_pass()
            e.record(stream)
        torch.cuda.synchronize()
        schedule_ms = round(float(np.mean([s.elapsed_time(e) for s, e in pe])), 4)
    # the same launches with a 512 MiB buffer written before each (caches flushed)
    flushed_ms = None
    if args.flushed:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for s, e in fe:
            flush.fill_(1)
            s.record(stream)
            step()
            e.record(stream)
        torch.cuda.synchronize()
        flushed_ms = round(float(np.median([s.elapsed_time(e) for s, e in fe])), 4)
        del flush
    avg_kernel_s = float(kernel_ms.mean()) / 1e3
    # the traffic record is taken on the default launch (mask form, default Q.K^T path)
    recorded = (args.form == "mask" and not args.schedule and qk_path(args.qk) == DEFAULT_QK
                and args.q_layout == "tnd")
    rec = traffic_record(p.cfg.name) if recorded else None
    dram_read_gbps = None
    if rec is not None:
        dram_read_gbps = round(rec["fetch_kib_per_launch"] * 1024 * rec["fetch_scale"]
                               / (float(np.median(kernel_ms)) / 1e3) / 1e9, 1)
    flop = n_act * FLOP_PER_TILE
    kv_bytes = n_act * (KV_BYTES_PER_TILE + (TILE * 4 if p.quant_type == 1 else 0))
    tflops = flop / (wall / args.steps) / 1e12
    achieved = flop / avg_kernel_s / 1e12
    crec = (clock_record(p.cfg.name, args.qk)
            if args.form == "mask" and not args.schedule and args.q_layout == "tnd" else None)
    clk = None if crec is None else crec["clock_ghz_mean"]
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": QK_DTYPES[qk_path(args.qk)],
        "data": "synthetic (seeded N(0,1) quantised to E4M3, random paging and block mask)",
        "config": {"workload": f"{p.cfg.name}: {p.cfg.description}", "active_tiles": n_act,
                   "q_tokens": T, "causal": bool(p.causal), "sparsity_form": args.form, "q_layout": args.q_layout,
                   "schedule_pre_pass": bool(args.schedule), "qk_precision": args.qk},
        "tokens_per_s": round(T / (wall / args.steps), 1),
        "pct_fp8_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
        # the matrix-core ceiling of this instruction mix, and both peaks scaled
        # to the shader clock measured for this kernel source (GRBM_GUI_ACTIVE)
        "mix_ceiling_tflops": round(qk_ceiling_tflops(args.qk), 1),
        "pct_mix_ceiling": round(100 * achieved / qk_ceiling_tflops(args.qk), 2),
        "measured_clock_ghz": None if clk is None else round(clk, 3),
        "pct_fp8_peak_at_measured_clock": None if clk is None else
            round(100 * achieved / (PEAK_FP8_TFLOPS * clk / PEAK_CLOCK_GHZ), 2),
        "pct_mix_ceiling_at_measured_clock": None if clk is None else
            round(100 * achieved / (qk_ceiling_tflops(args.qk) * clk / PEAK_CLOCK_GHZ), 2),
        "useful_tflops": round(pairs * 4 * TILE / (wall / args.steps) / 1e12, 2),
        "kv_gbps_logical": round(kv_bytes / (wall / args.steps) / 1e9, 1),
        "kernel_ms_min": round(float(kernel_ms.min()), 4),
        "kernel_ms_median": round(float(np.median(kernel_ms)), 4),
        "schedule_pre_pass_ms": schedule_ms,
        "kernel_ms_flushed_median": flushed_ms,
        # HBM read bytes per launch (the FETCH_SIZE record) over the median launch
        "kv_gbps_dram": dram_read_gbps,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": recorded_traffic(p.cfg.name) if recorded else None},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(p, n_act, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
