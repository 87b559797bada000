"""Throughput of the product-key memory forward on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload memplus_16m_bf16]
    python bench.py --workload engram_zipf_2m_bf16     # the hashed n-gram lookup
    python bench.py --workload ma_values_32k_bf16      # Memory Attention token-memory values
    python bench.py --workload engram_zipf_2m_bf16 --tables host   # tables in host memory, prefetched
    python bench.py --backward                         # value-table backward + sparse update
    python bench.py --uniform                          # the gather alone, uniform indices

A step is one whole forward (projection, qk-norm, scoring + per-half top-k,
combine + softmax, weighted EmbeddingBag over the value table, Memory+ gate) over
one batch of synthetic tokens whose inputs are already resident in HBM.  Prints one
JSON line with tokens/s, the roofline of the dominant kernel (the value gather,
HBM-bound) measured with HIP events on the forward's stream, and the oracle's
throughput on the host cores over a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 matrix, published
FP32_MFMA_PEAK_TFLOPS = 157.3
HOST_LINK_PEAK_GBPS = 64.0    # PCIe 5.0 x16 host link, one direction, published
METRIC = "PKM fwd tokens/s + value-gather GB/s (% of HBM peak) at 16M keys, 1 MI355X"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gather_memplus_16m_bf16_counters.json")
ENGRAM_COUNTERS_FILE = os.path.join(ROOT, "profiles", "engram_zipf_2m_bf16_counters.json")
# committed counter runs of the forward's gather, per workload (device-resident tables)
GATHER_COUNTERS = {"memplus_16m_bf16": COUNTERS_FILE,
                   "memplus_64m_bf16": os.path.join(ROOT, "profiles", "gather_memplus_64m_bf16_counters.json")}
# committed counter runs of the backward call and the Memory Attention values, per workload
BACKWARD_COUNTERS = {"memplus_16m_bf16": os.path.join(ROOT, "profiles", "bag_backward_memplus_16m_bf16_counters.json")}
MA_COUNTERS = {"ma_values_32k_bf16": os.path.join(ROOT, "profiles", "ma_values_32k_bf16_counters.json")}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def gather_bytes(cfg, T):
    """Algorithmic bytes one gather launch must move: value rows + (idx, w) + its output --
    with the Memory+ gate, z = x W1 read and g = y * silu(z) written (both in the stored type);
    else y written (stored type)."""
    rows = T * cfg.H * cfg.k * cfg.d_v * cfg.elem_bytes
    sel = T * cfg.H * cfg.k * 8
    out = T * cfg.d_v * 2 * cfg.elem_bytes if cfg.memory_plus else T * cfg.d_v * cfg.elem_bytes
    return rows, rows + sel + out


def flops(cfg, T):
    """Algorithmic FLOPs of the forward's matrix stages, charged to the stage that runs them.

    project: x [W_q | W1] -- with the Memory+ gate, z = x W1 runs in the same GEMM as the query
    projection; score: both halves of every head against all sub-keys (each score once);
    gate: (y * silu(z)) W2.
    """
    proj = 2 * T * cfg.d_model * (cfg.H * cfg.d_q + (cfg.d_v if cfg.memory_plus else 0))
    score = 2 * T * cfg.H * 2 * cfg.n_sub * cfg.d_h
    gate = 2 * T * cfg.d_v * cfg.d_model if cfg.memory_plus else 0
    return proj, score, gate


def stage_rates(cfg, T, stages):
    """TFLOP/s of the matrix stages from their mean times in ms (None for a stage that did
    not run), and the scoring's fraction of the matrix-core peak for the workload's dtype."""
    proj, score, gate = flops(cfg, T)
    ok = lambda ms: ms is not None and ms == ms and ms > 0
    tf = lambda f, ms: f / (ms * 1e-3) / 1e12 if f and ok(ms) else None
    peak = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
    r = {"score_TFLOPs": tf(score, stages.get("score")), "project_TFLOPs": tf(proj, stages.get("project")),
         "gate_TFLOPs": tf(gate, stages.get("gate"))}
    r["score_mfma_frac"] = r["score_TFLOPs"] / peak if r["score_TFLOPs"] else None
    return r


def calibration_copy():
    """A plain copy of 1 GiB (1 GiB read + 1 GiB written) in the measured process: what a profiler
    run's HBM byte counters read for it scales the counters of the other kernels to bytes."""
    import torch

    from synth import device as SD
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    SD.copy(dst, src)
    torch.cuda.synchronize()
    del src, dst


def counter_traffic(counters_file=COUNTERS_FILE):
    """HBM bytes per launch from a committed rocprofv3 counter run, if its kernel source is unchanged.

    The counter file records the kernel's source file and that file's sha256; a source that
    has changed since the counters were taken gives None.
    """
    try:
        rec = json.load(open(counters_file))
        src = os.path.join(ROOT, rec["source"])
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if rec.get("source_sha256") != sha:
            return None
        return rec.get("traffic_bytes_per_launch")
    except (OSError, ValueError, KeyError):
        return None


def source_digest():
    """sha256 (first 16 hex digits) over the library's kernel and header sources, in path order:
    names the code a bench line measured (the GPU run has no git metadata)."""
    h = hashlib.sha256()
    for d in ("sparse_key_value_amd/csrc", "include"):
        for name in sorted(os.listdir(os.path.join(ROOT, d))):
            if name.endswith((".hip", ".hpp", ".h")):
                h.update(f"{d}/{name}\0".encode())
                h.update(open(os.path.join(ROOT, d, name), "rb").read())
    return h.hexdigest()[:16]


def environment(a):
    """Seed, software stack and device of a bench line."""
    env = {"seed": a.seed, "source_sha16": source_digest(), "torch": None, "hip": None, "device": None, "arch": None}
    try:
        import torch
        env["torch"], env["hip"] = torch.__version__, torch.version.hip
        if torch.cuda.is_available():
            p = torch.cuda.get_device_properties(0)
            env["device"], env["arch"] = p.name, getattr(p, "gcnArchName", None)
    except Exception as ex:  # the line still prints without it
        log(f"environment: {ex}")
    return env


def cpu_baseline(wl, cfg, target_s, max_tokens=None):
    """Time the oracle on the first S tokens of the same workload on the host cores."""
    import numpy as np
    import torch

    from oracle import pkm as O

    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = max([p["num_threads"] for p in blas] or [1])
    except Exception:
        cores = 1
    # the oracle reads value rows from a host copy of the table (uint16 bf16 bits / float32)
    table_bytes = cfg.N * cfg.d_v * cfg.elem_bytes
    avail = 0
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemAvailable:"):
                avail = int(line.split()[1]) * 1024
    except OSError:
        pass
    note = ""
    if avail > table_bytes + (24 << 30):
        log(f"copying the {table_bytes / 2**30:.0f} GiB value table to host memory for the oracle")
        t0 = time.perf_counter()
        host = np.empty((cfg.N, cfg.d_v), dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)
        ht = torch.from_numpy(host.view(np.int16) if cfg.dtype == "bf16" else host)
        dv = wl.values.view(torch.int16) if cfg.dtype == "bf16" else wl.values
        step = max(1, (1 << 30) // (cfg.d_v * cfg.elem_bytes))
        for r0 in range(0, cfg.N, step):
            ht[r0:r0 + step].copy_(dv[r0:r0 + step])
        log(f"host table ready in {time.perf_counter() - t0:.1f} s")
        rows_of = O.rows_from_table(host, cfg.dtype)
    else:
        from synth import inputs as S
        note = "; host RAM too small for the table: rows regenerated on the host, inside the timing"
        rows_of = lambda r: O.to_f64(S.value_rows(wl.seed, r, cfg.d_v, cfg.dtype), cfg.dtype)

    def run(n):
        inp = {k: (v[:n] if k == "x" else v) for k, v in wl.inp.items()}
        t0 = time.perf_counter()
        O.forward(inp, cfg, rows_of)
        return time.perf_counter() - t0

    run(4)
    # a call has a fixed part (the sub-keys' normalisation and every step's setup): the
    # per-token cost is taken from two sizes, so that the timing lands near target_s
    t16, t64 = run(16), run(64)
    per_tok = max((t64 - t16) / 48, t64 / 256, 1e-9)
    fixed = max(t16 - 16 * per_tok, 0.0)
    n = int(max(16, min(max_tokens or wl.T, (target_s - fixed) / per_tok)))
    log(f"oracle: {per_tok * 1e3:.1f} ms/token + {fixed:.2f} s per call estimated, timing {n} tokens")
    dt = run(n)
    return {"value": n / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(), **numeric_stack(),
            "sample": f"first {n} of {wl.T} tokens of {cfg.name}, float64 NumPy oracle, {dt:.1f} s" + note}


def host_copy(t):
    """A host copy of a large device tensor (bf16 as uint16 bits), in 1 GiB pieces."""
    import numpy as np
    import torch

    bf16 = t.dtype == torch.bfloat16
    host = np.empty(tuple(t.shape), dtype=np.uint16 if bf16 else np.float32)
    ht = torch.from_numpy(host.view(np.int16) if bf16 else host)
    dv = t.view(torch.int16) if bf16 else t
    step = max(1, (1 << 30) // (t.shape[1] * t.element_size()))
    for r0 in range(0, t.shape[0], step):
        ht[r0:r0 + step].copy_(dv[r0:r0 + step])
    return host


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def numeric_stack():
    """NumPy version and the BLAS library it calls (name, version), for the CPU baseline."""
    import numpy as np
    info = {"numpy": np.__version__}
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
    except Exception:
        pass
    return info


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        return 1


def bench_engram(a):
    """The hashed n-gram lookup: one step = engram_forward over the workload's tokens."""
    import numpy as np
    import torch

    import sparse_key_value_amd as P
    from synth import configs as C
    from synth import device as SD
    from synth import inputs as S
    from tests.gpu_util import TORCH_DT, to_dev

    cfg = C.ENGRAM_CONFIGS[a.workload]
    T, eb = cfg.T, cfg.elem_bytes
    log(f"workload {cfg.name}: T={T}, {cfg.n_tables} tables x {cfg.table_rows} rows x {cfg.head_dim} {cfg.dtype}")
    inp = S.make_engram_inputs(cfg, a.seed)
    tables = torch.empty((cfg.total_rows, cfg.head_dim), dtype=TORCH_DT[cfg.dtype], device="cuda")
    SD.fill_values(tables, a.seed, tid=S.TID_ENGRAM)
    ids = torch.from_numpy(inp["ids"]).cuda()
    h = to_dev(inp["h"], cfg.dtype)
    mult = torch.from_numpy(inp["mult"].view(np.int64)).cuda()
    comp = torch.from_numpy(inp["compress"]).cuda() if inp["compress"] is not None else None
    out = torch.empty((T, cfg.d), dtype=TORCH_DT[cfg.dtype], device="cuda")
    ec = P.make_engram_config(cfg.min_order, cfg.n_orders, cfg.heads, cfg.head_dim, cfg.table_rows, cfg.vocab,
                              cfg.dtype, cfg.residual, cfg.norm_eps)
    stream = torch.cuda.current_stream()
    run = lambda: P.engram_forward(ec, tables, ids, T, cfg.seq_len, comp, mult, h, out, stream=stream)

    # streaming-read ceiling over the tables
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    SD.stream_read(tables, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    SD.stream_read(tables, sink)
    e1.record()
    torch.cuda.synchronize()
    tbytes = tables.numel() * tables.element_size()
    stream_gbps = tbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # the 1 GiB copy that scales a profiler's HBM byte counters
    cal_dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    SD.copy(cal_dst, tables.view(torch.uint8).view(-1)[: 1 << 30])
    torch.cuda.synchronize()
    del cal_dst

    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    # HIP events on the stream the kernel is launched on, around the timed launches
    e0.record(stream)
    t0 = time.perf_counter()
    for _ in range(a.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launch_ms = e0.elapsed_time(e1) / a.steps

    # algorithmic bytes per launch: the table rows, the ids, h and out
    rows_b = T * cfg.n_tables * cfg.head_dim * eb
    alg_b = rows_b + T * 4 + 2 * T * cfg.d * eb
    uniq = None
    try:
        r = torch.empty((T, cfg.heads, cfg.n_orders), dtype=torch.int32, device="cuda")
        P.engram_hash(ec, ids, T, cfg.seq_len, comp, mult, r, stream=stream)
        uniq = int(torch.unique(r).numel())
    except Exception as ex:  # pragma: no cover - reporting only
        log(f"unique-row count failed: {ex}")
    achieved = alg_b / (launch_ms * 1e-3) / 1e9
    traffic = counter_traffic(ENGRAM_COUNTERS_FILE) if cfg.name == "engram_zipf_2m_bf16" else None

    cpu = None
    if not a.no_cpu_baseline:
        from oracle import engram as E
        log(f"copying the {tbytes / 2**30:.1f} GiB tables to host memory for the oracle")
        host = host_copy(tables)
        rows_of = lambda rr: E.to_f64(host[rr], cfg.dtype)

        def orc(n):
            c2 = cfg.with_(T=n)
            t1 = time.perf_counter()
            E.forward(c2, inp["ids"][:n], inp["h"][:n], inp["mult"], rows_of, inp["compress"])
            return time.perf_counter() - t1

        per_tok = orc(64) / 64
        n = int(max(64, min(T, a.cpu_seconds / max(per_tok, 1e-9))))
        dt = orc(n)
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"first {n} of {T} tokens of {cfg.name}, float64 NumPy oracle (Python hash loops), "
                         f"{dt:.1f} s"}
        del host

    res = {
        "metric": "Engram hashed n-gram lookup tokens/s + HBM GB/s, 1 MI355X",
        "value": T * a.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": elapsed / a.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (Zipf(1.1) token ids, Gaussian hidden states, tables generated on the GPU)",
        "config": {"workload": cfg.name, "tokens": T, "seq_len": cfg.seq_len, "vocab": cfg.vocab,
                   "orders": list(range(cfg.min_order, cfg.min_order + cfg.n_orders)), "heads": cfg.heads,
                   "head_dim": cfg.head_dim, "table_rows": cfg.table_rows, "d": cfg.d, "table_GiB": tbytes / 2**30},
        "roofline": {"bound": "hbm", "kernel": "engram_forward (hash + row gather + gate)", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": alg_b, "avg_launch_ms": launch_ms},
        "unique_rows": uniq,
        "unique_row_bytes": uniq * cfg.head_dim * eb if uniq is not None else None,
        "stream_read_GBps": stream_gbps,
        "env": environment(a),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_engram_host(a):
    """Hashed n-gram lookup with the tables in pinned host memory: each step prefetches the
    next batch's rows over the host link on a side stream while the current batch is gated
    from its staged rows (two staging buffers)."""
    import numpy as np
    import torch

    import sparse_key_value_amd as P
    from synth import configs as C
    from synth import device as SD
    from synth import inputs as S
    from tests.gpu_util import TORCH_DT, to_dev

    cfg = C.ENGRAM_CONFIGS[a.workload]
    T, eb = cfg.T, cfg.elem_bytes
    log(f"workload {cfg.name} with host-resident tables: T={T}, {cfg.n_tables} tables x {cfg.table_rows} rows")
    inp = S.make_engram_inputs(cfg, a.seed)
    dev_tables = torch.empty((cfg.total_rows, cfg.head_dim), dtype=TORCH_DT[cfg.dtype], device="cuda")
    SD.fill_values(dev_tables, a.seed, tid=S.TID_ENGRAM)
    tables = torch.empty(dev_tables.shape, dtype=dev_tables.dtype, pin_memory=True)
    tables.copy_(dev_tables)
    torch.cuda.synchronize()
    del dev_tables
    torch.cuda.empty_cache()
    ids = torch.from_numpy(inp["ids"]).cuda()
    h = to_dev(inp["h"], cfg.dtype)
    mult = torch.from_numpy(inp["mult"].view(np.int64)).cuda()
    comp = torch.from_numpy(inp["compress"]).cuda() if inp["compress"] is not None else None
    out = torch.empty((T, cfg.d), dtype=TORCH_DT[cfg.dtype], device="cuda")
    staged = [torch.empty((T, cfg.n_orders, cfg.d), dtype=TORCH_DT[cfg.dtype], device="cuda") for _ in range(2)]
    ec = P.make_engram_config(cfg.min_order, cfg.n_orders, cfg.heads, cfg.head_dim, cfg.table_rows, cfg.vocab,
                              cfg.dtype, cfg.residual, cfg.norm_eps)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    prefetch = lambda buf, st: P.engram_prefetch(ec, tables, ids, T, cfg.seq_len, comp, mult, buf, stream=st)
    gate = lambda buf: P.engram_forward_staged(ec, buf, h, T, out, stream=main)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # each part alone, timed with events on the stream it runs on
    for _ in range(a.warmup):
        prefetch(staged[0], main)
        gate(staged[0])
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    e0.record(main)
    for _ in range(a.steps):
        prefetch(staged[0], main)
    e1.record(main)
    torch.cuda.synchronize()
    pf_ms = e0.elapsed_time(e1) / a.steps
    e0.record(main)
    for _ in range(a.steps):
        gate(staged[0])
    e1.record(main)
    torch.cuda.synchronize()
    gate_ms = e0.elapsed_time(e1) / a.steps

    # the pipeline: prefetch of step i + 1 on the side stream beside the gate of step i
    ready = [torch.cuda.Event(), torch.cuda.Event()]
    free = [torch.cuda.Event(), torch.cuda.Event()]
    with torch.cuda.stream(side):
        prefetch(staged[0], side)
        ready[0].record(side)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        cur, nxt = i % 2, (i + 1) % 2
        side.wait_event(free[nxt]) if i > 0 else None
        prefetch(staged[nxt], side)
        ready[nxt].record(side)
        main.wait_event(ready[cur])
        gate(staged[cur])
        free[cur].record(main)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    link_b = T * cfg.n_orders * cfg.d * eb           # rows read from host memory per step
    achieved = link_b / (pf_ms * 1e-3) / 1e9
    res = {
        "metric": "Engram hashed n-gram lookup tokens/s, tables in host memory + host-link GB/s, 1 MI355X",
        "value": T * a.steps / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": elapsed / a.steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (Zipf(1.1) token ids, Gaussian hidden states, tables generated on the GPU, kept in "
                "pinned host memory)",
        "config": {"workload": cfg.name, "tables": "host (pinned)", "tokens": T, "table_GiB":
                   cfg.total_rows * cfg.head_dim * eb / 2**30, "staging_MiB": link_b / 2**20},
        "roofline": {"bound": "host-link", "kernel": "engram_prefetch (hash + row copy from host memory)",
                     "achieved": achieved, "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HOST_LINK_PEAK_GBPS, "traffic": None, "algorithmic_bytes_per_launch": link_b,
                     "avg_launch_ms": pf_ms},
        "prefetch_ms": pf_ms, "staged_gate_ms": gate_ms,
        "env": environment(a),
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def backward_cpu_baseline(a, cfg, wl, idx, w, dy):
    """The oracle's backward step (dw, ds, the per-row sums and the SGD update of the touched
    rows) on the first n tokens of the workload, taken as a batch of their own, on the host
    cores.  The rows it reads are fetched from the device beforehand (not timed)."""
    import numpy as np
    import torch

    from oracle import backward as B
    from oracle import pkm as O
    from tests.gpu_util import to_host

    bag = cfg.H * cfg.k
    idx_h = idx.cpu().numpy().astype(np.int64)
    w_h = w.cpu().numpy().astype(np.float64)
    dy_h = dy.cpu().numpy().astype(np.float64)

    def step(n):
        ii = idx_h[:n]
        uniq = np.unique(ii[(ii >= 0) & (ii < cfg.N)])
        stored = to_host(wl.values[torch.from_numpy(uniq).cuda()])
        table = O.to_f64(stored, cfg.dtype)
        rows_of = lambda r: table[np.searchsorted(uniq, r)]
        t1 = time.perf_counter()
        dw = B.grad_weights(rows_of, ii, dy_h[:n], cfg.N)
        B.softmax_backward(w_h[:n], dw, cfg.k)
        rows, grad = B.grad_rows(ii, w_h[:n], dy_h[:n], cfg.N)
        B.sgd_rows(stored[np.searchsorted(uniq, rows)], grad, 1e-4, cfg.dtype)
        return time.perf_counter() - t1

    per_tok = step(16) / 16
    n = int(max(16, min(cfg.T, a.cpu_seconds / max(per_tok, 1e-9))))
    dt = step(n)
    return {"value": n / dt, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens ({n * bag} entries) of {cfg.name} as a batch of their own: "
                      f"float64 NumPy oracle dw, ds, per-row sums (Python loop) and SGD step, {dt:.1f} s"}


def bench_backward(a):
    """The sparse training step of the value table behind the forward's gather, as one
    pkm_bag_backward call: dw and the softmax ds for every token, the distinct rows and the
    in-place update of every touched row, on the indices and weights of a real forward.
    With the update asked for, dw comes from the rows the update reads, so each touched row
    is read once and written once; the dw pass on its own (no update) is timed beside it."""
    import numpy as np
    import torch

    import sparse_key_value_amd as P
    from synth import CONFIGS
    from tests.gpu_util import Workload

    cfg = CONFIGS[a.workload]
    T, bag, eb = cfg.T, cfg.H * cfg.k, cfg.elem_bytes
    log(f"backward of {cfg.name}: T={T}, {bag} entries per token, N={cfg.N}, d_v={cfg.d_v}")
    wl = Workload(cfg, seed=a.seed)
    x = wl.dev["x"]
    out = torch.empty((T, cfg.d_out), dtype=x.dtype, device="cuda")
    idx = torch.empty((T, bag), dtype=torch.int32, device="cuda")
    w = torch.empty((T, bag), dtype=torch.float32, device="cuda")
    P.pkm_forward(wl.pkm.handle, x, T, out, idx, w)
    dy = torch.randn((T, cfg.d_v), dtype=torch.float32, device="cuda", generator=torch.Generator("cuda").manual_seed(a.seed))
    dw = torch.empty((T, bag), dtype=torch.float32, device="cuda")
    ds = torch.empty_like(dw)
    rows = torch.empty(T * bag, dtype=torch.int32, device="cuda")
    nu = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws_bytes = P.pkm_bag_backward_workspace_size(T, bag, cfg.N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    common = dict(table=wl.values, n_rows=cfg.N, dim=cfg.d_v, dtype=cfg.dtype, idx=idx, w=w, dy=dy, n_bags=T,
                  bag_size=bag, dw=dw, ds=ds, softmax_group=cfg.k, workspace=ws, stream=stream)
    run_step = lambda: P.pkm_bag_backward(**common, rows=rows, n_unique=nu, update=True, lr=1e-4)
    run_dw = lambda: P.pkm_bag_backward(**common)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(a.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(a.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / a.steps

    calibration_copy()
    dw_ms = timed(run_dw)
    step_ms = timed(run_step)
    U = int(nu.item())
    n = T * bag
    dw_bytes = n * cfg.d_v * eb + T * cfg.d_v * 4 + n * 16            # every entry's row, dy, idx/w/dw/ds
    step_bytes = 2 * U * cfg.d_v * eb + T * cfg.d_v * 4 + n * 16      # touched rows read + written, dy, idx/w/dw/ds
    achieved = step_bytes / (step_ms * 1e-3) / 1e9
    # the committed counters: every kernel of one update call, at the workload's own seed
    traffic = counter_traffic(BACKWARD_COUNTERS[cfg.name]) if cfg.name in BACKWARD_COUNTERS and a.seed == 0 else None
    res = {
        "metric": "PKM value-table backward (dw, ds, sparse update of the touched rows) tokens/s, 1 MI355X",
        "value": T / (step_ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic (indices and weights of a real forward over the generated table; "
                                    "dy ~ N(0, 1))",
        "config": {"workload": cfg.name, "tokens": T, "entries_per_token": bag, "n_keys": cfg.N, "d_value": cfg.d_v,
                   "distinct_rows": U},
        "roofline": {"bound": "hbm",
                     "kernel": "pkm_bag_backward call (sort + bag_update_kernel with dw + ds); the update kernel "
                               "dominates",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": step_bytes, "avg_launch_ms": step_ms},
        "dw_alone": {"kernel": "bag_dw_kernel (dw + ds, no update)", "ms": dw_ms, "algorithmic_bytes": dw_bytes,
                     "GBps": dw_bytes / (dw_ms * 1e-3) / 1e9,
                     "frac_hbm": dw_bytes / (dw_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS},
        "env": environment(a),
        "cpu_baseline": None if a.no_cpu_baseline else backward_cpu_baseline(a, cfg, wl, idx, w, dy),
    }
    print(json.dumps(res), flush=True)


def bench_uniform(a):
    """The gather alone (pkm_embedding_bag) over the workload's table with i.i.d. uniform
    row indices and random normalised weights: the no-reuse floor of the value read."""
    import numpy as np
    import torch

    import sparse_key_value_amd as P
    from synth import CONFIGS
    from synth import inputs as S
    from tests.gpu_util import make_value_table

    cfg = CONFIGS[a.workload]
    T, bag, eb = cfg.T, cfg.H * cfg.k, cfg.elem_bytes
    log(f"uniform-index gather over {cfg.name}'s table: {T} bags of {bag}, N={cfg.N}, d_v={cfg.d_v}")
    values = make_value_table(cfg, a.seed)
    idx, w = S.uniform_bags(a.seed, T, bag, cfg.N)
    uniq = len(np.unique(idx))
    idx_d, w_d = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
    y = torch.empty((T, cfg.d_v), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    run = lambda: P.pkm_embedding_bag(values, cfg.N, cfg.d_v, cfg.dtype, idx_d, w_d, T, bag, y, stream=stream)
    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    rows_b = T * bag * cfg.d_v * eb
    alg_b = rows_b + T * bag * 8 + T * cfg.d_v * 4
    res = {
        "metric": "value-gather GB/s with uniform indices (no-reuse floor), 1 MI355X",
        "value": alg_b / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (i.i.d. uniform row indices, random normalised weights, table generated on the GPU)",
        "config": {"workload": cfg.name + " (uniform indices)", "bags": T, "bag_size": bag, "n_keys": cfg.N,
                   "d_value": cfg.d_v, "unique_rows": uniq, "unique_row_bytes": uniq * cfg.d_v * eb},
        "roofline": {"bound": "hbm", "kernel": "gather (weighted EmbeddingBag)", "achieved": alg_b / (ms * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": alg_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "traffic": None, "algorithmic_bytes_per_launch": alg_b, "avg_launch_ms": ms},
        "value_rows_GBps": rows_b / (ms * 1e-3) / 1e9,
        "env": environment(a),
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def bench_shard(a):
    """One GPU's share of a column-sharded value table: the gather (pkm_embedding_bag) of the
    forward's own indices and weights over a [N, d_v / G] slice, as each of G GPUs would run
    it after the replicated selection.  The exchange between GPUs is not part of it."""
    import numpy as np
    import torch

    import sparse_key_value_amd as P
    from synth import CONFIGS
    from synth import device as SD
    from tests.gpu_util import TORCH_DT, Workload

    cfg = CONFIGS[a.workload]
    G = a.shard_columns
    T, bag, eb = cfg.T, cfg.H * cfg.k, cfg.elem_bytes
    if cfg.d_v % G or (cfg.d_v // G * eb) % 16:
        raise SystemExit(f"d_v = {cfg.d_v} does not split into {G} slices of a multiple of 16 bytes")
    dv = cfg.d_v // G
    log(f"column shard of {cfg.name}: {G} shards, slice [{cfg.N}, {dv}], {T} bags of {bag}")
    wl = Workload(cfg, seed=a.seed)
    out = torch.empty((T, cfg.d_out), dtype=wl.dev["x"].dtype, device="cuda")
    idx = torch.empty((T, bag), dtype=torch.int32, device="cuda")
    w = torch.empty((T, bag), dtype=torch.float32, device="cuda")
    P.pkm_forward(wl.pkm.handle, wl.dev["x"], T, out, idx, w)
    torch.cuda.synchronize()
    uniq = int(torch.unique(idx).numel())
    wl.close()
    del wl, out
    torch.cuda.empty_cache()
    table = torch.empty((cfg.N, dv), dtype=TORCH_DT[cfg.dtype], device="cuda")
    SD.fill_values(table, a.seed)
    y = torch.empty((T, dv), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    run = lambda: P.pkm_embedding_bag(table, cfg.N, dv, cfg.dtype, idx, w, T, bag, y, stream=stream)
    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(a.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    rows_b = T * bag * dv * eb
    alg_b = rows_b + T * bag * 8 + T * dv * 4
    res = {
        "metric": f"value-gather GB/s of one GPU's column shard (d_v / {G}) with the forward's indices, 1 MI355X",
        "value": alg_b / (ms * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (indices and weights of a real forward; slice generated on the GPU)",
        "config": {"workload": f"{cfg.name} column shard 1 of {G}", "bags": T, "bag_size": bag, "n_keys": cfg.N,
                   "d_value_slice": dv, "row_bytes": dv * eb, "unique_rows": uniq},
        "roofline": {"bound": "hbm", "kernel": "gather (weighted EmbeddingBag) over the slice",
                     "achieved": alg_b / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": alg_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, "traffic": None,
                     "algorithmic_bytes_per_launch": alg_b, "avg_launch_ms": ms},
        "value_rows_GBps": rows_b / (ms * 1e-3) / 1e9,
        "env": environment(a),
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def bench_ma(a):
    """Memory Attention token-memory values: one step = ma_values over the workload's tokens
    (the table fold runs once, before the timing)."""
    import numpy as np
    import torch

    import sparse_key_value_amd as P
    from synth import configs as C
    from synth import inputs as S
    from tests.gpu_util import TORCH_DT, to_dev

    cfg = C.MA_CONFIGS[a.workload]
    T, eb = cfg.T, cfg.elem_bytes
    log(f"workload {cfg.name}: T={T}, vocab={cfg.vocab}, d_v={cfg.d_v}, {cfg.n_heads} heads, {cfg.dtype}")
    d = S.make_ma_inputs(cfg, a.seed)
    E = to_dev(d["E"], cfg.dtype)
    gain = torch.from_numpy(d["gain"]).cuda() if d["gain"] is not None else None
    P.ma_fold_table(E, cfg.vocab, cfg.d_v, cfg.n_heads, gain, cfg.norm_eps, cfg.dtype, E)
    ids = torch.from_numpy(d["ids"]).cuda()
    K = to_dev(d["K"], cfg.dtype)
    V = torch.empty((T, cfg.d_v), dtype=TORCH_DT[cfg.dtype], device="cuda")
    stream = torch.cuda.current_stream()
    run = lambda: P.ma_values(E, cfg.vocab, cfg.d_v, cfg.dtype, ids, T, K, V, stream=stream)
    calibration_copy()
    for _ in range(a.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    t0 = time.perf_counter()
    for _ in range(a.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launch_ms = e0.elapsed_time(e1) / a.steps
    alg_b = T * (3 * cfg.d_v * eb + 4)          # K row, table row, V row, id
    uniq = len(np.unique(d["ids"]))
    achieved = alg_b / (launch_ms * 1e-3) / 1e9

    cpu = None
    if not a.no_cpu_baseline:
        from oracle import ma as M
        from oracle import pkm as O
        Eh = d["E"]

        def orc(n):
            t1 = time.perf_counter()
            Eb = M.store(M.fold_table(O.to_f64(Eh, cfg.dtype), cfg.n_heads, d["gain"], cfg.norm_eps), cfg.dtype)
            t2 = time.perf_counter()
            M.values(Eb, d["ids"][:n], d["K"][:n], cfg.dtype)
            return t2 - t1, time.perf_counter() - t2

        fold_s, per = orc(256)
        n = int(max(256, min(T, a.cpu_seconds / max(per / 256, 1e-9))))
        _, dt = orc(n)
        cpu = {"value": n / dt, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"first {n} of {T} tokens of {cfg.name}, float64 NumPy oracle, {dt:.2f} s "
                         f"(the one-off table fold, {fold_s:.1f} s, not counted)"}

    res = {
        "metric": "Memory Attention token-memory values tokens/s + HBM GB/s, 1 MI355X",
        "value": T * a.steps / elapsed, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": elapsed / a.steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (Zipf(1.1) token ids, Gaussian keys and table)",
        "config": {"workload": cfg.name, "tokens": T, "vocab": cfg.vocab, "d_v": cfg.d_v, "heads": cfg.n_heads,
                   "table_MiB": cfg.vocab * cfg.d_v * eb / 2**20},
        # the folded table (vocab x d_v) fits in the 256 MB Infinity Cache, so its repeated rows are
        # served from there: the bound is the last-level cache and HBM together, and the fraction
        # of the HBM peak is a figure of the algorithmic bytes, not of HBM traffic (traffic: the
        # counted bytes that left L2, from either)
        "roofline": {"bound": "llc/hbm", "kernel": "ma_values (k = 1 lookup + add)", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": counter_traffic(MA_COUNTERS[cfg.name]) if cfg.name in MA_COUNTERS and a.seed == 0
                     else None,
                     "algorithmic_bytes_per_launch": alg_b, "avg_launch_ms": launch_ms,
                     "table_MiB_vs_llc_MiB": [cfg.vocab * cfg.d_v * eb / 2**20, 256]},
        "unique_ids": uniq,
        "env": environment(a),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="memplus_16m_bf16")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--uniform", action="store_true",
                    help="time the gather alone with uniform random indices over the workload's table")
    ap.add_argument("--shard-columns", type=int, default=0,
                    help="time one GPU's gather over a d_v / G column slice of the table (G > 1)")
    ap.add_argument("--backward", action="store_true",
                    help="time the value-table backward and sparse update instead of the forward")
    ap.add_argument("--tables", choices=["device", "host"], default="device",
                    help="Engram workloads: keep the tables in HBM or in pinned host memory (prefetched)")
    ap.add_argument("--bound", choices=["auto", "exact"], default="auto",
                    help="the scoring's bound pass: fp8 estimate where built (auto) or exact in the stored type")
    ap.add_argument("--tokens", type=int, default=0,
                    help="product-key forward: a batch of this many tokens instead of the workload's (small batches)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}): the path has no multi-GPU execution; "
              "--shard-columns G times one GPU's share of a column-sharded table", file=sys.stderr)
        sys.exit(2)

    from synth import configs as C
    if a.workload in C.ENGRAM_CONFIGS:
        return bench_engram_host(a) if a.tables == "host" else bench_engram(a)
    if a.workload in C.MA_CONFIGS:
        return bench_ma(a)
    if a.backward:
        return bench_backward(a)
    if a.uniform:
        return bench_uniform(a)
    if a.shard_columns > 1:
        return bench_shard(a)

    import torch

    import sparse_key_value_amd as P
    from synth import CONFIGS
    from synth import device as SD
    from tests.gpu_util import Workload

    cfg = CONFIGS[a.workload]
    if a.tokens > 0:
        cfg = cfg.with_(T=a.tokens)
    T = cfg.T
    log(f"workload {cfg.name}: T={T}, N={cfg.N}, d_v={cfg.d_v}, {cfg.dtype}; filling the value table")
    host = a.tables == "host"
    if host:
        # a host-resident table: generated on the GPU, moved to pinned host memory in 1 GiB pieces
        from tests.gpu_util import TORCH_DT
        hv = torch.empty((cfg.N, cfg.d_v), dtype=TORCH_DT[cfg.dtype], pin_memory=True)
        step = max(1, (1 << 30) // (cfg.d_v * cfg.elem_bytes))
        piece = torch.empty((step, cfg.d_v), dtype=hv.dtype, device="cuda")
        for r0 in range(0, cfg.N, step):
            n = min(step, cfg.N - r0)
            SD.fill_rows(piece, a.seed, r0, n)
            hv[r0:r0 + n].copy_(piece[:n])
        torch.cuda.synchronize()
        del piece
        wl = Workload(cfg, seed=a.seed, values=hv, value_seed=a.seed)
    else:
        wl = Workload(cfg, seed=a.seed)
    h = wl.pkm.handle
    P.pkm_set_score_bound(h, a.bound)
    x = wl.dev["x"]
    out = torch.empty((T, cfg.d_out), dtype=x.dtype, device="cuda")
    stream = torch.cuda.current_stream()

    tbytes = wl.values.numel() * wl.values.element_size()
    stream_gbps = None
    if not host:
        # streaming-read ceiling over the value table itself (one pass, after a warm pass)
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        SD.stream_read(wl.values, sink)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        SD.stream_read(wl.values, sink)
        ev1.record()
        torch.cuda.synchronize()
        stream_gbps = tbytes / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
        log(f"streaming read of the table: {stream_gbps:.0f} GB/s")
        # a plain copy of known size (1 GiB read + 1 GiB written): the reference that scales the
        # HBM byte counters of a profiler run to bytes
        cal_src = wl.values.view(torch.uint8).view(-1)[: 1 << 30]
        cal_dst = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        SD.copy(cal_dst, cal_src)
        torch.cuda.synchronize()
        del cal_dst

    for _ in range(a.warmup):
        P.pkm_forward(h, x, T, out, stream=stream)
    # the timed steps record only the gather's two events (the roofline's kernel time, on
    # the forward's stream); the events of every stage cost a forward about 2%, so the
    # stage breakdown comes from further forwards after the timed region
    P.pkm_enable_stage_timing(h, a.steps)
    P.pkm_set_stage_timing_mask(h, ["gather"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        P.pkm_forward(h, x, T, out, stream=stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed / a.steps * 1e3
    tok_s = T * a.steps / elapsed
    g_ms = sum(P.pkm_stage_times(h, "gather", a.steps)) / a.steps

    n_bd = min(a.steps, 10)
    P.pkm_set_stage_timing_mask(h, P.STAGES)
    for _ in range(n_bd):
        P.pkm_forward(h, x, T, out, stream=stream)
    torch.cuda.synchronize()
    stages = {n: sum(P.pkm_stage_times(h, n, n_bd)) / n_bd for n in P.STAGES}
    stages = {n: (v if v == v else None) for n, v in stages.items()}   # NaN: the stage did not run
    rows_b, alg_b = gather_bytes(cfg, T)
    achieved = alg_b / (g_ms * 1e-3) / 1e9
    log("stages (ms): " + ", ".join(f"{k} {v:.3f}" for k, v in stages.items() if v is not None))

    rr_ms = uniq = None
    if not host:
        # the same rows read with the gather's lane layout and no arithmetic (XOR only): the
        # read rate of this random-row pattern, the gather's own ceiling
        sel = torch.empty((T, cfg.H * cfg.k), dtype=torch.int32, device="cuda")
        P.pkm_forward(h, x, T, out, idx_out=sel, stream=stream)
        rr_out = torch.empty((T, cfg.d_v * cfg.elem_bytes), dtype=torch.uint8, device="cuda")
        SD.row_read(wl.values, sel, rr_out)
        rr = []
        for _ in range(3):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            SD.row_read(wl.values, sel, rr_out)
            ev1.record()
            torch.cuda.synchronize()
            rr.append(ev0.elapsed_time(ev1))
        rr_ms = sorted(rr)[1]
        uniq = int(torch.unique(sel).numel())
        del sel, rr_out
        log(f"row read of the forward's rows (no arithmetic): {rr_ms:.3f} ms against the gather's {g_ms:.3f} ms")

    cpu = None
    if not a.no_cpu_baseline and not host:
        cpu = cpu_baseline(wl, cfg, a.cpu_seconds)
        # the oracle's rate in the gather's algorithmic bytes (the same bytes per token)
        cpu["gather_GBps_equivalent"] = cpu["value"] * alg_b / T / 1e9

    # the committed counters were taken with device-resident tables
    # the counters were taken at the workload's own batch; another batch size has other bytes
    traffic = (counter_traffic(GATHER_COUNTERS[cfg.name]) if (not host and cfg.name in GATHER_COUNTERS and a.tokens <= 0)
               else None)
    res = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian inputs and weights; value table generated on the GPU)",
        "config": {"workload": cfg.name, "tokens": T, "d_model": cfg.d_model, "heads": cfg.H, "d_query": cfg.d_q,
                   "n_sub": cfg.n_sub, "n_keys": cfg.N, "d_value": cfg.d_v, "k": cfg.k, "qk_norm": cfg.qk_norm,
                   "memory_plus": cfg.memory_plus, "score_bound": a.bound, "table_GiB": tbytes / 2**30,
                   "table_memory": "host (pinned)" if host else "device"},
        "roofline": {"bound": "host-link" if host else "hbm", "kernel": "gather (weighted EmbeddingBag)",
                     "achieved": achieved, "peak": HOST_LINK_PEAK_GBPS if host else HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / (HOST_LINK_PEAK_GBPS if host else HBM_PEAK_GBPS),
                     "traffic": traffic, "algorithmic_bytes_per_launch": alg_b, "avg_launch_ms": g_ms},
        "gather_value_GBps": rows_b / (g_ms * 1e-3) / 1e9,
        "gather_value_frac_hbm": rows_b / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "stream_read_GBps": stream_gbps,
        "gather_frac_of_stream_read": achieved / stream_gbps if stream_gbps else None,
        "row_read_ms": rr_ms,
        "row_read_value_GBps": rows_b / (rr_ms * 1e-3) / 1e9 if rr_ms else None,
        "gather_time_over_row_read": g_ms / rr_ms if rr_ms else None,
        # distinct rows among the T * H * k selected (a row picked twice is read twice)
        "unique_rows": uniq,
        "unique_row_GBps": uniq * cfg.d_v * cfg.elem_bytes / (g_ms * 1e-3) / 1e9 if uniq else None,
        "stages_ms": stages,
        "stages_note": f"from {n_bd} forwards after the timed steps with every stage's events recorded (the events "
                       "slow a forward by about 2%; the timed steps record the gather's alone)",
        **stage_rates(cfg, T, stages),
        "env": environment(a),
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
