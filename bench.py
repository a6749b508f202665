"""Benchmark: one hybrid-head prefill layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic inputs
resident in HBM: XA block selection (when the layer has XA heads: scoring +
selector) and the fused prefill (work-list build + attention kernel).  The
default workload is the Llama-3.1-8B-shaped FA-SSA layer at 64K tokens
(3 FA + 5 SSA KV heads, sink 128, window 2048).  Prints one JSON line.

Reported beside the throughput: ms per layer, tokens/s, effective TFLOP/s
(4 B^2 d per computed tile) and pair-level TFLOP/s (4 d per attended pair),
the speedup over the same kernel with every head in FA mode, the roofline of
the attention kernel, the latency of the attention router (ea_route_heads,
off the hot path), one decode step over a batch of caches of the same
length and modes (ea_hybrid_attn_decode, HBM-bound, with its own roofline)
and the fp64 oracle timed on the host cores.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="llama8b-fassa-64k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all-fa", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--oracle-timing", metavar="NAMES",
                    help="comma-separated workloads: time the whole fp64 oracle layer (FA / SSA heads) "
                         "with one thread and with the host's threads, then exit (no GPU needed)")
    ap.add_argument("--decode-batch", type=int, default=8,
                    help="sequences of the decode measurement (0 skips it)")
    ap.add_argument("--decode-only", action="store_true",
                    help="measure only the decode step (for profiling)")
    ap.add_argument("--decode-modes", metavar="DIGITS",
                    help="with --decode-only: one mode digit per KV head (0 FA, 1 SSA, 2 XA) "
                         "in place of the workload's, e.g. 11111111")
    ap.add_argument("--serial-sweep", action="store_true",
                    help="time fused vs serial dispatch over model sparsity 0.125-0.875 and "
                         "lengths 16K-256K (Llama-3.1-8B shape, FA + SSA heads) and exit")
    ap.add_argument("--sweep-lengths", default="16384,32768,65536,131072,262144")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (counter calibration)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE csv output under DIR "
                         "(subfolders fetch, write, cfetch, cwrite) into the traffic record")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy of exactly 1 GiB, so that HBM byte counters read under the
    same profiler can be scaled to bytes (read 1 GiB, write 1 GiB)."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 3}))


def _counter_means(folder, counter):
    """Mean counter value (KiB per dispatch) per kernel name, from the
    *_counter_collection.csv files rocprofv3 wrote under `folder`, over the
    dispatches of each kernel with its largest grid (the whole layer: the
    serial-dispatch leg launches the same kernel on smaller sub-layers)."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(folder, "**", "*_counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                vals.setdefault(r["Kernel_Name"], []).append((int(r.get("Grid_Size") or 0),
                                                             float(r["Counter_Value"])))
    out = {}
    for k, v in vals.items():
        g = max(x[0] for x in v)
        sel = [x[1] for x in v if x[0] == g]
        out[k] = (float(np.mean(sel)), len(sel))
    return out


def write_traffic(base, cfg_name):
    """Scale the attention kernel's FETCH_SIZE / WRITE_SIZE by what the same
    counters read for a 1 GiB device copy (bytes known), and store the result
    keyed to the hash of the attention source it was measured on."""
    import hashlib
    def pick(d, key):
        m = [v for k, v in d.items() if key in k]
        if not m:
            raise SystemExit(f"no dispatch of {key} in the counter output")
        return m[0]
    fetch = pick(_counter_means(os.path.join(base, "fetch"), "FETCH_SIZE"), "k_attn")
    write = pick(_counter_means(os.path.join(base, "write"), "WRITE_SIZE"), "k_attn")
    cf = pick(_counter_means(os.path.join(base, "cfetch"), "FETCH_SIZE"), "copyBuffer")
    cw = pick(_counter_means(os.path.join(base, "cwrite"), "WRITE_SIZE"), "copyBuffer")
    one_gib = float(1 << 30)
    f_scale = one_gib / (cf[0] * 1024.0)
    w_scale = one_gib / (cw[0] * 1024.0)
    read_b = fetch[0] * 1024.0 * f_scale
    write_b = write[0] * 1024.0 * w_scale
    src = os.path.join(ROOT, "hybrid_sparse_full_amd", "csrc", "ea_attn.hip")
    rec = {
        "kernel": "k_attn", "workload": cfg_name,
        "source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest(),
        "fetch_kib_per_dispatch": round(fetch[0], 1), "fetch_dispatches": fetch[1],
        "write_kib_per_dispatch": round(write[0], 1), "write_dispatches": write[1],
        "copy_fetch_kib_per_GiB": round(cf[0], 1), "copy_write_kib_per_GiB": round(cw[0], 1),
        "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
        "read_bytes_per_launch": round(read_b), "write_bytes_per_launch": round(write_b),
        "bytes_per_launch": round(read_b + write_b),
    }
    path = os.path.join(ROOT, "profiles", f"k_attn_{cfg_name}_traffic.json")
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


def traffic_record(cfg_name):
    """Measured HBM bytes per attention launch, if a counter summary for the
    current attention source exists under profiles/ (null otherwise)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"k_attn_{cfg_name}_traffic.json")
    src = os.path.join(ROOT, "hybrid_sparse_full_amd", "csrc", "ea_attn.hip")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec


def attended_pairs(inp, gpu_xa_pairs=None):
    """Attended (i, j) pairs of the layer (all q-heads), from the definitions."""
    cfg = inp["cfg"]
    G = cfg.gqa
    total = 0
    for b, L in enumerate(inp["seqlens"]):
        L = int(L)
        i = np.arange(L, dtype=np.int64)
        causal = L * (L + 1) // 2
        lo = np.maximum(i - cfg.ssa_window + 1, 0)
        ssa = int((np.minimum(i + 1, cfg.ssa_sink) +
                   np.maximum(0, i - np.maximum(lo, cfg.ssa_sink) + 1)).sum())
        for g in range(cfg.num_kv_heads):
            m = int(inp["modes"][b, g])
            if m == 0:
                total += G * causal
            elif m == 1:
                total += G * ssa
            else:
                total += int(gpu_xa_pairs[b, g * G:(g + 1) * G].sum())
    return total


def workspace_counts(layer):
    """(tile-list entries, computed (tile, q-head) pairs) of the last prefill,
    read from the counters its work-list build wrote into the workspace."""
    import torch
    from hybrid_sparse_full_amd import ea as E
    off = E.ea_workspace_offset(layer.desc, E.EA_OP_PREFILL, "scal")
    scal = layer.ws_prefill[off:off + 64].view(torch.int64).cpu().numpy()
    return int(scal[4]), int(scal[3])


def time_steps(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    per = [a.elapsed_time(b) for a, b in ev]
    return wall * 1e3, float(np.mean(per)), per


def _oracle_head_rows(inp, heads, threads, rows_per_task=1024):
    """The fp64 oracle (oracle.attention.head_attention, as it stands) over
    every row of the listed (b, h) FA / SSA heads, the rows of each head split
    into ranges run by `threads` host threads (numpy releases the GIL in its
    products and elementwise loops; BLAS single-threaded in each task)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import attention as OA
    from synth import bf16_bits_to_f64
    cfg = inp["cfg"]
    cu = inp["cu_seqlens"]
    G = cfg.gqa
    tasks = []
    for (b, h) in heads:
        g = h // G
        L = int(cu[b + 1] - cu[b])
        qh = bf16_bits_to_f64(inp["q"][cu[b]:cu[b + 1], h])
        kh = bf16_bits_to_f64(inp["k"][cu[b]:cu[b + 1], g])
        vh = bf16_bits_to_f64(inp["v"][cu[b]:cu[b + 1], g])
        mode = int(inp["modes"][b, g])
        for r0 in range(0, L, rows_per_task):
            tasks.append((qh, kh, vh, mode, r0, min(L, r0 + rows_per_task)))
    tasks.sort(key=lambda t: -t[5])

    def run(t):
        qh, kh, vh, mode, r0, r1 = t
        return OA.head_attention(qh, kh, vh, mode, cfg.softmax_scale, sink=cfg.ssa_sink,
                                 window=cfg.ssa_window, block=cfg.block, chunk=256, row_range=(r0, r1))

    with threadpool_limits(limits=1, user_api="blas"):
        if threads == 1:
            for t in tasks:
                run(t)
        else:
            with ThreadPoolExecutor(max_workers=threads) as ex:
                list(ex.map(run, tasks))


def _head_pairs(cfg, L, mode):
    """Attended (i, j) pairs of one FA / SSA q-head of a sequence of length L."""
    if mode == 0:
        return L * (L + 1) // 2
    i = np.arange(L, dtype=np.int64)
    lo = np.maximum(i - cfg.ssa_window + 1, 0)
    return int((np.minimum(i + 1, cfg.ssa_sink) + np.maximum(0, i - np.maximum(lo, cfg.ssa_sink) + 1)).sum())


def cpu_baseline(inp, seconds, threads=None):
    """The fp64 oracle, as it stands, on whole q-heads of the workload: FA and
    SSA heads in turn (XA heads need the oracle's masks first and are left
    out), until `seconds` of wall time have passed (at least one head)."""
    cfg = inp["cfg"]
    G = cfg.gqa
    threads = threads or max(1, min(16, len(os.sched_getaffinity(0))))
    cand = [(b, h) for b in range(len(inp["seqlens"])) for h in range(cfg.num_q_heads)
            if int(inp["modes"][b, h // G]) in (0, 1) and inp["seqlens"][b] > 0]
    # FA and SSA heads alternate, so a short sample holds both.
    fa = [x for x in cand if int(inp["modes"][x[0], x[1] // G]) == 0]
    ssa = [x for x in cand if int(inp["modes"][x[0], x[1] // G]) == 1]
    order = [x for pair in zip(fa, ssa) for x in pair] + fa[len(ssa):] + ssa[len(fa):]
    flops = 0.0
    done = []
    t0 = time.perf_counter()
    for (b, h) in order:
        _oracle_head_rows(inp, [(b, h)], threads)
        L = int(inp["seqlens"][b])
        flops += 4.0 * cfg.head_dim * _head_pairs(cfg, L, int(inp["modes"][b, h // G]))
        done.append((b, h))
        if time.perf_counter() - t0 >= seconds:
            break
    wall = time.perf_counter() - t0
    kinds = {0: "FA", 1: "SSA"}
    desc = ", ".join(f"seq {b} q-head {h} ({kinds[int(inp['modes'][b, h // G])]})" for b, h in done)
    return dict(value=flops / wall / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"every query row of {len(done)} whole q-head(s) of {cfg.name}: {desc}; fp64 numpy "
                       f"oracle (head_attention over row ranges, {threads} threads, single-threaded BLAS "
                       f"per task); pair-level flops / wall {wall:.1f} s; "
                       f"{len(os.sched_getaffinity(0))} host cores visible")


def oracle_timing(names, threads):
    """The CPU baseline over whole layers: wall time of the fp64 oracle layer
    (every row of every FA / SSA q-head) per workload, with `threads` host
    threads.  Like cpu_baseline, it times the oracle and runs no GPU work."""
    from synth import get_config, make_inputs
    out = []
    for name in names:
        inp = make_inputs(get_config(name))
        cfg = inp["cfg"]
        G = cfg.gqa
        heads = [(b, h) for b in range(len(inp["seqlens"])) for h in range(cfg.num_q_heads)
                 if int(inp["modes"][b, h // G]) in (0, 1) and inp["seqlens"][b] > 0]
        t0 = time.perf_counter()
        _oracle_head_rows(inp, heads, threads)
        wall = time.perf_counter() - t0
        flops = sum(4.0 * cfg.head_dim * _head_pairs(cfg, int(inp["seqlens"][b]), int(inp["modes"][b, h // G]))
                    for b, h in heads)
        rec = {"workload": name, "threads": threads, "heads": len(heads), "wall_s": round(wall, 2),
               "gflops": round(flops / wall / 1e9, 2)}
        print(json.dumps(rec), flush=True)
        out.append(rec)
    return out


def decode_bench(cfg, mode_row, L, batch, steps, warmup):
    """One decode step over `batch` caches of length L with the workload's
    head modes (`mode_row`, one per KV head).
    The cache and queries are seeded N(0, 1) on the device (timing only; the
    parity tests use the oracle's inputs).  Bytes are algorithmic: every kept
    K and V row once, plus q and o."""
    import torch
    from hybrid_sparse_full_amd.layer import HybridDecode, make_desc
    D, Hq, Hkv = cfg.head_dim, cfg.num_q_heads, cfg.num_kv_heads
    modes = np.repeat(np.asarray(mode_row, dtype=np.uint8).reshape(1, -1), batch, axis=0)
    T = L * batch
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(17)
    k = torch.randn((T, Hkv, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((T, Hkv, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q = torch.randn((batch, Hq, D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    cu = np.arange(batch + 1, dtype=np.int32) * L
    desc = make_desc(num_seqs=batch, total_tokens=T, max_seqlen=L, num_q_heads=Hq, num_kv_heads=Hkv,
                     head_dim=D, block=cfg.block, softmax_scale=cfg.softmax_scale, ssa_sink=cfg.ssa_sink,
                     ssa_window=cfg.ssa_window, xa_stride=cfg.xa_stride, xa_tau=(cfg.tau_num, cfg.tau_den))

    def kept(mode):
        if mode == 1:  # SSA: sink plus window of the decoded query
            head = min(cfg.ssa_sink, L)
            return head + max(0, L - max(head, L - cfg.ssa_window))
        return L

    def run(m):
        dec = HybridDecode(desc, cu, m, device=dev)
        _, ms, _ = time_steps(lambda: dec(q, k, v), steps, warmup)
        keys = sum(kept(int(x)) for x in m.reshape(-1))
        nbytes = keys * 2 * D * 2 + 2 * (batch * Hq * D * 2) + batch * Hq * 4
        return ms, nbytes

    ms, nbytes = run(modes)
    fa_ms, fa_bytes = run(np.zeros_like(modes))

    # The same step over the segmented cache, where SSA heads keep only their
    # sink and window keys (filled from the packed cache above).
    from hybrid_sparse_full_amd.layer import SegmentedDecodeCache
    cu_dev = torch.from_numpy(cu.astype(np.int32)).to(dev)
    cache = SegmentedDecodeCache(desc, modes, np.full(batch, L, dtype=np.int32), device=dev)
    cache.fill(desc, k, v, cu_dev)
    o_c = torch.empty((batch, Hq, D), dtype=torch.bfloat16, device=dev)
    lse_c = torch.empty((batch, Hq), dtype=torch.float32, device=dev)
    from hybrid_sparse_full_amd import ea as E
    ws_c = torch.empty(E.ea_workspace_bytes(desc, E.EA_OP_DECODE), dtype=torch.uint8, device=dev)
    _, cached_ms, _ = time_steps(lambda: cache.decode(desc, q, cu_dev, o_c, lse_c, ws_c), steps, warmup)
    packed_cache_bytes = 2 * T * Hkv * D * 2
    cached = {
        "ms_per_step": round(cached_ms, 5),
        "cache_bytes": cache.nbytes(),
        "packed_cache_bytes": packed_cache_bytes,
        "cache_fraction": round(cache.nbytes() / packed_cache_bytes, 4),
        "hbm_gbs": round(nbytes / (cached_ms * 1e-3) / 1e9, 1),
    }
    del k, v, cache
    torch.cuda.synchronize()
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": f"{cfg.name} decode, {batch} sequences x {L} cached tokens",
        "ms_per_step": round(ms, 5),
        "tokens_per_s": round(batch / (ms * 1e-3), 1),
        "algorithmic_bytes": nbytes,
        "roofline": {"kernel": "k_decode + k_decode_combine", "bound": "hbm", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)},
        "all_fa_ms_per_step": round(fa_ms, 5),
        "all_fa_gbs": round(fa_bytes / (fa_ms * 1e-3) / 1e9, 1),
        "speedup_vs_all_fa": round(fa_ms / ms, 4),
        "segmented_cache": cached,
        "data": "seeded N(0,1) cache on the device",
    }


class SerialLayer:
    """Buffers of the serial-dispatch baseline (ea_hybrid_attn_prefill_serial)
    for one descriptor and one mode row shared by every sequence."""

    def __init__(self, desc, cu_seqlens_dev, layer_modes, device):
        import torch
        from hybrid_sparse_full_amd import ea as E
        self.E = E
        self.desc = desc
        self.cu = cu_seqlens_dev
        self.modes = np.ascontiguousarray(layer_modes, dtype=np.uint8)
        T, Hq, D = desc.total_tokens, desc.num_q_heads, desc.head_dim
        self.o = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((Hq, T), dtype=torch.float32, device=device)
        self.ws = torch.empty(E.ea_workspace_bytes(desc, E.EA_OP_PREFILL_SERIAL), dtype=torch.uint8,
                              device=device)

    def __call__(self, q, k, v):
        self.E.ea_hybrid_attn_prefill_serial(self.desc, q, k, v, self.cu, self.modes, self.o, self.lse,
                                             self.ws)


def serial_sweep(lengths, steps, warmup):
    """Fused kernel vs serial dispatch (split, one single-mode layer per group,
    write back) over model sparsity n/8 and sequence length, one sequence of
    seeded N(0, 1) q, k, v generated on the device (timing only)."""
    import torch
    from hybrid_sparse_full_amd.layer import HybridPrefill, make_desc
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Hq, Hkv, D, B = 32, 8, 128, 128
    rows = []
    for L in lengths:
        gen = torch.Generator(device=dev)
        gen.manual_seed(L)
        q = torch.randn((L, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((L, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((L, Hkv, D), generator=gen, device=dev).to(torch.bfloat16)
        desc = make_desc(num_seqs=1, total_tokens=L, max_seqlen=L, num_q_heads=Hq, num_kv_heads=Hkv,
                         head_dim=D, block=B, ssa_sink=128, ssa_window=2048)
        cu = np.array([0, L], dtype=np.int32)
        for n_sparse in range(1, Hkv):
            row = np.zeros(Hkv, dtype=np.uint8)
            row[np.random.default_rng(n_sparse).permutation(Hkv)[:n_sparse]] = 1
            fused = HybridPrefill(desc, cu, row.reshape(1, -1), device=dev)
            _, f_ms, _ = time_steps(lambda: fused(q, k, v), steps, warmup)
            serial = SerialLayer(desc, fused.cu, row, dev)
            _, s_ms, _ = time_steps(lambda: serial(q, k, v), steps, warmup)
            rec = {"seq_len": L, "omega_msr": n_sparse / Hkv, "sparse_kv_heads": int(n_sparse),
                   "fused_ms": round(f_ms, 4), "serial_ms": round(s_ms, 4),
                   "speedup_fused_over_serial": round(s_ms / f_ms, 4)}
            rows.append(rec)
            print(json.dumps(rec), flush=True)
            del fused, serial
        del q, k, v
        torch.cuda.empty_cache()
    return rows


def main():
    a = parse()
    if a.calibrate_copy:
        calibrate_copy()
        return
    if a.traffic_from:
        write_traffic(a.traffic_from, a.config)
        return
    if a.oracle_timing:
        names = a.oracle_timing.split(",")
        oracle_timing(names, 1)
        oracle_timing(names, max(1, min(16, len(os.sched_getaffinity(0)))))
        return
    if a.serial_sweep:
        if a.gpus != 1:
            raise SystemExit("the sweep runs on one GPU")
        rows = serial_sweep([int(x) for x in a.sweep_lengths.split(",")], max(a.steps, 1), a.warmup)
        print(json.dumps({"serial_dispatch_sweep": rows, "workload": "one sequence, 32/8 heads, d 128, "
                          "FA + SSA (sink 128, window 2048), seeded N(0,1) on the device"}), flush=True)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU only; sharding over several GPUs is "
                                   "described, not implemented", "n_gpus": a.gpus}))
        sys.exit(2)
    import torch
    from hybrid_sparse_full_amd.layer import HybridPrefill, bf16_tensor, desc_for
    from synth import get_config, make_inputs

    cfg = get_config(a.config)
    if a.decode_only:
        meta = make_inputs(cfg, with_values=False)
        row = meta["modes"][0]
        if a.decode_modes:
            row = [int(c) for c in a.decode_modes if c.isdigit()]
            if len(row) != len(a.decode_modes) or len(row) != cfg.num_kv_heads or max(row) > 2:
                raise SystemExit(f"--decode-modes needs {cfg.num_kv_heads} digits in 0..2")
        torch.cuda.set_device(0)
        r = decode_bench(cfg, row, int(np.max(meta["seqlens"])), max(a.decode_batch, 1),
                         max(a.steps, 20), a.warmup)
        print(json.dumps({"metric": "decode step HBM GB/s (kept K/V, q, o)", "value": r["roofline"]["achieved"],
                          "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "decode": r}), flush=True)
        return
    inp = make_inputs(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    desc = desc_for(cfg, inp["seqlens"])
    q = bf16_tensor(inp["q"], dev)
    k = bf16_tensor(inp["k"], dev)
    v = bf16_tensor(inp["v"], dev)
    layer = HybridPrefill(desc, inp["cu_seqlens"], inp["modes"], device=dev)

    wall_ms, ev_ms, per = time_steps(lambda: layer(q, k, v), a.steps, a.warmup)
    # Attention kernel (dominant) timed alone: one plan call (work list and
    # K/V packing), then ea_hybrid_attn_run launches only the attention
    # kernel; events on the stream the kernels run on.
    if layer.has_xa:
        layer.select(q, k)
    layer.plan(k, v)
    _, attn_ms, _ = time_steps(lambda: layer.run(q), a.steps, 1)
    tiles, head_tiles = workspace_counts(layer)
    xa_pairs = layer.xa_pairs.cpu().numpy().reshape(len(inp["seqlens"]), -1) if layer.has_xa else None
    pairs = attended_pairs(inp, xa_pairs)
    D, B = cfg.head_dim, cfg.block
    tile_flops = 4.0 * B * B * D * head_tiles
    pair_flops = 4.0 * D * pairs
    T = int(inp["cu_seqlens"][-1])
    ms = ev_ms
    eff_tflops = tile_flops / (ms * 1e-3) / 1e12
    pair_tflops = pair_flops / (ms * 1e-3) / 1e12
    attn_pair_tflops = pair_flops / (attn_ms * 1e-3) / 1e12
    rat = layer.ratios(cfg.sparse_mode)
    traffic = traffic_record(cfg.name)

    # The attention router (off the hot path, reported beside it): modes for
    # every (sequence, KV head) from the boundary-pooled keys, seeded random
    # weights of the pages' shape (hidden 4 d), into a buffer of its own.
    from hybrid_sparse_full_amd.layer import Router
    from synth.router_weights import make_router_weights
    router = Router(make_router_weights(D, 4 * D, seed=1), device=dev)
    routed = torch.empty(desc.num_seqs * desc.num_kv_heads, dtype=torch.uint8, device=dev)
    _, router_ms, _ = time_steps(lambda: router(desc, k, layer.cu, 0, cfg.sparse_mode, routed),
                                 max(a.steps, 20), a.warmup)

    # End to end with routing on the device: the router writes the modes into
    # device memory, XA selection (when the mode set has XA) and the prefill
    # read them there, with no host round trip.  The retrieval mode of the
    # set is the workload's most common mode other than its sparse mode.  The
    # random weights choose their own modes, so the same layer with those
    # modes passed in is timed beside it.
    other = inp["modes"][inp["modes"] != cfg.sparse_mode]
    rmode = int(np.bincount(other, minlength=3).argmax()) if other.size else 0
    rlayer = HybridPrefill(desc, inp["cu_seqlens"], None, device=dev, mode_set=(rmode, cfg.sparse_mode))
    _, routed_ms, _ = time_steps(lambda: (rlayer.route(router, k), rlayer(q, k, v)), a.steps, a.warmup)
    rmodes = rlayer.device_modes()
    del rlayer
    plain = HybridPrefill(desc, inp["cu_seqlens"], rmodes, device=dev)
    _, plain_ms, _ = time_steps(lambda: plain(q, k, v), a.steps, a.warmup)
    del plain
    routed_layer = {
        "ms_per_layer": round(routed_ms, 4),
        "same_modes_passed_in_ms": round(plain_ms, 4),
        "mode_set": [rmode, int(cfg.sparse_mode)],
        "modes_chosen": np.bincount(rmodes.reshape(-1), minlength=3).tolist(),
        "weights": "seeded random (no trained router weights)",
    }

    decode = None
    if a.decode_batch > 0:
        decode = decode_bench(cfg, inp["modes"][0], int(np.max(inp["seqlens"])), a.decode_batch,
                              max(a.steps, 20), a.warmup)
        if a.decode_batch != 1:
            decode["batch_1"] = decode_bench(cfg, inp["modes"][0], int(np.max(inp["seqlens"])), 1,
                                             max(a.steps, 20), a.warmup)

    # Serial dispatch of the same layer (split by mode, one single-mode layer
    # per group, write back), when every sequence shares one mode row without
    # XA heads: the baseline the fused kernel is compared with.
    serial = None
    mrow = inp["modes"][0]
    if (inp["modes"] == mrow).all() and not (mrow == 2).any():
        sl = SerialLayer(desc, layer.cu, mrow, dev)
        _, serial_ms, _ = time_steps(lambda: sl(q, k, v), a.steps, a.warmup)
        serial = {"ms_per_layer": round(serial_ms, 4), "fused_ms_per_layer": round(ms, 4),
                  "speedup_fused_over_serial": round(serial_ms / ms, 4)}
        del sl

    speedup = None
    allfa_ms = None
    if not a.no_all_fa:
        fa_layer = HybridPrefill(desc, inp["cu_seqlens"], np.zeros_like(inp["modes"]), device=dev)
        _, allfa_ms, _ = time_steps(lambda: fa_layer(q, k, v), a.steps, a.warmup)
        speedup = allfa_ms / ms
        del fa_layer
    torch.cuda.synchronize()

    out = {
        "metric": "hybrid-head prefill effective TFLOP/s (computed tiles) per layer",
        "value": round(eff_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            "description": cfg.description,
            "tokens": T,
            "seqlens": [int(x) for x in inp["seqlens"]],
            "heads_q_kv": [cfg.num_q_heads, cfg.num_kv_heads],
            "head_dim": D,
            "block": B,
            "modes": inp["modes"].tolist() if len(inp["seqlens"]) <= 8 else "drawn",
        },
        "ms_per_layer": round(ms, 4),
        "wall_ms_per_layer": round(wall_ms, 4),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "effective_tflops": round(eff_tflops, 2),
        "effective_frac_of_peak": round(eff_tflops / PEAK_BF16_TFLOPS, 4),
        "pair_level_tflops": round(pair_tflops, 2),
        "computed_tiles": head_tiles,
        "tile_list_entries": tiles,
        "attended_pairs": pairs,
        "all_fa_ms_per_layer": None if allfa_ms is None else round(allfa_ms, 4),
        "speedup_vs_all_fa": None if speedup is None else round(speedup, 4),
        "speedup_bar": round(0.7 / (1.0 - rat["esr"][-1]), 4),
        "omega_msr": round(float(rat["msr"][-1]), 6),
        "omega_esr": round(float(rat["esr"][-1]), 6),
        "omega_esr_pair_weighted": round(rat["esr_pairs"], 6),
        "serial_dispatch": serial,
        "decode": decode,
        "router": {
            "ms": round(router_ms, 4),
            "heads_routed": desc.num_seqs * desc.num_kv_heads,
            "pooled_tokens_per_sequence": 200,
            "hidden": 4 * D,
            "weights": "seeded random (no trained router weights)",
        },
        "routed_layer": routed_layer,
        "roofline": {
            "kernel": "k_attn (fused hybrid attention)",
            "bound": "mfma",
            "achieved": round(attn_pair_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_pair_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            "per_launch_ms": round(attn_ms, 4),
            "algorithmic_flops_per_launch": pair_flops,
        },
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
