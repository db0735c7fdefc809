"""Benchmark: paged decode attention on one MI355X, Llama-3-8B-shaped GQA layer.

One step = the append of 256 new tokens (one per sequence, its newest) and the decode
over all 256 sequences, on one stream, with every input already resident in HBM: one
pa_decode_append call (decode kernel + merge kernel, whose last workgroups store the new
rows); ``--two-call`` runs it as pa_write_kv followed by pa_decode instead (bit-identical).
Workload: 256 sequences, 32 query / 8 KV heads, head_dim 128, bf16 KV and q, fp32
accumulation, block size 16, lengths uniform in [512, 4096] (seed 0), 70,000-block
pool with random block placement.
--workload picks one of the other workloads instead (its step also runs its block
copies, if any, before the write).

Prints ONE JSON line.  ``value`` is the K/V bytes the decode step must read
(each (token, KV head) row of K and V once) divided by the wall time per step of K
back-to-back steps, timed with no event between them; ``step_us`` gives the median / p10 /
p90 of K steps from HIP events around each one, run before them (``events_ms_per_step`` is
their wall time: an event record costs GPU time of its own).  ``roofline`` reports the decode call alone: K further calls, each preceded by
an untimed read of a 1 GiB buffer that evicts the caches (L2 and the 256 MiB Infinity
Cache; a read leaves no dirty lines to write back), timed with HIP events on the stream
it runs on; ``achieved`` uses the median.  ``cache_ops`` times pa_write_kv (the step's
new tokens) and pa_copy_blocks (224 copy-on-write pairs of OPT-13B-shaped blocks) the
same way.  ``cpu_baseline`` times the float64 CPU oracle on the host.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME [--block-size B]]
    python bench.py --two-call           # the step as pa_write_kv + pa_decode
    python bench.py --workload opt13b_shared --shared-prefix   # shared-prefix decode
    python bench.py --workload llama3_8b_spec                  # multi-query (also llama3_8b_chunk)
    python bench.py --swap               # pa_swap_blocks HBM <-> pinned host throughput
    python bench.py --copy-calibration   # a block copy of known size, for counter scaling
    python bench.py --record-traffic DEC_FETCH.csv DEC_WRITE.csv COPY_FETCH.csv COPY_WRITE.csv
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_kv_cache_351_amd as pk  # noqa: E402
import workloads  # noqa: E402

METRIC = "paged-decode KV GB/s read (% of HBM peak) and seqs/s, Llama-3-8B-shaped, 1 GPU"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, vendor figure
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama3_8b_traffic.json")
# the files that define the decode kernels and their launch (traffic is re-recorded when they change)
KERNEL_SOURCES = ["decode_kernel.h", "split.h", "decode_bf16.hip", "decode_params.h", "decode_api.hip",
                  "host_util.h", "common.h"]
DECODE_KERNELS = ["pagedkv::decode_kernel", "pagedkv::reduce_kernel"]   # kernels one pa_decode call launches


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


FLUSH_BYTES = 1 << 30            # > 8 x 4 MiB L2 + 256 MiB Infinity Cache


class CacheFlush:
    """Evicts the GPU caches by reading (not writing) a 1 GiB buffer: a write would leave
    dirty lines whose write-back lands in the next timed call."""

    def __init__(self, dev):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.sink = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        torch.sum(self.buf, dim=0, out=self.sink)


def pct(ms):
    """median / p10 / p90 of event timings in ms, as microseconds."""
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean()), "n": int(a.size)}


class HipEvent:
    """A HIP timing event created with hipEventDisableSystemFence, recorded on a torch stream.

    A default event (torch.cuda.Event included) performs a system-scope fence when it is
    recorded: the L2 is written back and invalidated, which costs the timed interval a few
    µs and slows the work after it.  HIP documents this flag for events used only to
    measure time; every reading here follows a device synchronisation, so nothing needs
    the fence.  The events come from the HIP runtime torch has loaded."""

    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            with open("/proc/self/maps") as f:
                path = next((ln.split()[-1] for ln in f if "libamdhip64" in ln), "libamdhip64.so.7")
            L = ctypes.CDLL(path)
            vp = ctypes.c_void_p
            L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            L.hipEventRecord.argtypes = [vp, vp]
            L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            L.hipEventDestroy.argtypes = [vp]
            cls._hip = L
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        e = self._lib().hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if e != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({e})")

    def record(self, stream):
        e = self._lib().hipEventRecord(self.h, self._ct.c_void_p(stream.cuda_stream))
        if e != 0:
            raise RuntimeError(f"hipEventRecord failed ({e})")

    def elapsed_time(self, end):
        """ms from this event to `end` (both recorded and complete)."""
        ms = self._ct.c_float()
        e = self._lib().hipEventElapsedTime(self._ct.byref(ms), self.h, end.h)
        if e != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({e})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


def timed_calls(fn, n, stream, flush=None):
    """Event timings (ms) of n calls of fn on stream, each after an untimed flush."""
    ev = [(HipEvent(), HipEvent()) for _ in range(n)]
    for a, z in ev:
        if flush is not None:
            flush()
        a.record(stream)
        fn()
        z.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(z) for a, z in ev]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def kernel_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_351_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode call from the committed counter runs, or None when they
    were taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("hbm_bytes_per_call")


def _pmc_per_dispatch(csv_path, counter, kernel_substr):
    """Mean value of ``counter`` over the dispatches of kernels whose name contains
    ``kernel_substr`` in a rocprofv3 ``--pmc ... -f csv`` counter_collection file (one row per
    dispatch and counter; the value is the sum over hardware instances)."""
    import csv
    per = {}
    with open(csv_path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter or kernel_substr not in row.get("Kernel_Name", ""):
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"{csv_path}: no {counter} rows for kernels matching {kernel_substr!r}")
    return sum(per.values()) / len(per), len(per)


def record_traffic(paths):
    """Turn four rocprofv3 counter files into HBM bytes per decode call and write them to
    the traffic file, tagged with the hash of the kernel sources they were taken on.

    paths: decode FETCH_SIZE csv, decode WRITE_SIZE csv, calibration-copy FETCH_SIZE csv,
    calibration-copy WRITE_SIZE csv.  FETCH_SIZE and WRITE_SIZE are in KiB per dispatch;
    each is scaled by (known bytes / counter bytes) of the calibration copy, which reads
    and writes exactly 1 GiB per launch."""
    dec_f, dec_w, cal_f, cal_w = paths
    known = 16384 * 16 * 8 * 128 * 2 * 2
    cf, _ = _pmc_per_dispatch(cal_f, "FETCH_SIZE", "copy_blocks_kernel")
    cw, _ = _pmc_per_dispatch(cal_w, "WRITE_SIZE", "copy_blocks_kernel")
    fetch_scale, write_scale = known / (cf * 1024), known / (cw * 1024)
    per_kernel = {}
    total = 0.0
    for name in DECODE_KERNELS:
        f, nf = _pmc_per_dispatch(dec_f, "FETCH_SIZE", name)
        w, nw = _pmc_per_dispatch(dec_w, "WRITE_SIZE", name)
        rb, wb = f * 1024 * fetch_scale, w * 1024 * write_scale
        per_kernel[name] = {"fetch_kib": f, "write_kib": w, "dispatches": [nf, nw],
                            "read_bytes": rb, "write_bytes": wb}
        total += rb + wb
    out = {"kernel_sha": kernel_sha(), "hbm_bytes_per_call": total,
           "fetch_scale": fetch_scale, "write_scale": write_scale,
           "calibration_counter_kib": {"fetch": cf, "write": cw, "known_bytes_each": known},
           "per_kernel": per_kernel}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def copy_calibration(steps):
    """pa_copy_blocks of 2 x 16384 blocks x 32 KiB: 1 GiB read and 1 GiB written per launch."""
    dev = torch.device("cuda:0")
    nb, B, H, D = 32768, 16, 8, 128
    kc = torch.zeros(nb, B, H, D, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    half = nb // 2
    pairs = torch.stack([torch.arange(half), torch.arange(half) + half], 1).int().to(dev)
    for _ in range(steps):
        pk.pa_copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    per = half * B * H * D * 2 * 2
    print(json.dumps({"copy_calibration": True, "launches": steps, "read_bytes_per_launch": per,
                      "write_bytes_per_launch": per}))


PCIE_PEAK_GBS = 64.0             # PCIe 5.0 x16 host link, per direction, vendor figure


def swap_bench(steps, warmup, with_cpu):
    """pa_swap_blocks of 4096 Llama-3-8B blocks (16 tokens x 8 KV heads x 128, bf16; K and V,
    64 KiB a block, 256 MiB a call) from the HBM pool to a pinned host pool and back, random
    block ids on both sides.  A plain contiguous copy of the same byte count (the runtime's
    DMA engines) is timed beside it as the host link's practical ceiling."""
    dev = torch.device("cuda:0")
    B, H, D, NG, NC, N = 16, 8, 128, 16384, 8192, 4096
    g = torch.Generator(device=dev).manual_seed(0)
    gk = torch.randn((NG, B, H, D), device=dev, generator=g).to(torch.bfloat16)
    gv = torch.randn((NG, B, H, D), device=dev, generator=g).to(torch.bfloat16)
    hk = torch.zeros((NC, B, H, D), dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros((NC, B, H, D), dtype=torch.bfloat16).pin_memory()
    rng = np.random.default_rng(0)
    out_pairs = np.stack([rng.choice(NG, N, replace=False), rng.choice(NC, N, replace=False)], 1)
    po = torch.from_numpy(out_pairs.astype(np.int32)).to(dev)
    pi = torch.from_numpy(out_pairs[:, ::-1].astype(np.int32).copy()).to(dev)
    nbytes = N * B * H * D * 2 * 2
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, z in ev:
            a.record(stream)
            fn()
            z.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(z) for a, z in ev])) * 1e-3

    log(f"swap out / in: {N} blocks, {nbytes / 2**20:.0f} MiB per call, {steps} calls each")
    t_out = timed(lambda: pk.pa_swap_blocks(gk, gv, hk, hv, po))
    t_in = timed(lambda: pk.pa_swap_blocks(hk, hv, gk, gv, pi))
    flat_g, flat_h = gk[:2 * N].reshape(-1), hk[:2 * N].reshape(-1)
    t_d2h = timed(lambda: flat_h.copy_(flat_g, non_blocking=True))
    t_h2d = timed(lambda: flat_g.copy_(flat_h, non_blocking=True))
    res = {"metric": "pa_swap_blocks host-link GB/s (swap-out and swap-in of 4096 scattered blocks)",
           "value": 2 * nbytes / (t_out + t_in) / 1e9, "unit": "GB/s", "n_gpus": 1,
           "steps": steps, "warmup": warmup, "higher_is_better": True, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": "Llama-3-8B blocks, HBM <-> pinned host", "blocks_per_call": N,
                      "block_bytes_kv": B * H * D * 2 * 2, "gpu_pool_blocks": NG, "host_pool_blocks": NC},
           "swap_out_gbs": nbytes / t_out / 1e9, "swap_in_gbs": nbytes / t_in / 1e9,
           "swap_out_us": t_out * 1e6, "swap_in_us": t_in * 1e6,
           "contiguous_copy_gbs": {"d2h": nbytes / t_d2h / 1e9, "h2d": nbytes / t_h2d / 1e9},
           "roofline": {"kernel": "copy_blocks_kernel (two pools)", "bound": "host link",
                        "achieved": 2 * nbytes / (t_out + t_in) / 1e9, "peak": PCIE_PEAK_GBS,
                        "unit": "GB/s", "frac": 2 * nbytes / (t_out + t_in) / 1e9 / PCIE_PEAK_GBS,
                        "traffic": None},
           "cpu_baseline": None}
    if with_cpu:
        import oracle
        n = 512                                   # a bounded sample of the same copy
        hk_np = hk.view(torch.int16).numpy().view(np.uint16)
        src = gk[:n].cpu().view(torch.int16).numpy().view(np.uint16)
        pairs = np.stack([np.arange(n), out_pairs[:n, 1]], 1)
        t0 = time.perf_counter()
        oracle.swap_blocks(src, src, hk_np, hk_np, pairs)
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": n * B * H * D * 2 * 2 / dt / 1e9, "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"{n} blocks of oracle.swap_blocks "
                               "between host arrays (includes its copy of the 8192-block target pool)"}
    print(json.dumps(res))


TOL = {"f32": 1e-5, "f16": 4e-3, "bf16": 8e-3}   # max-abs bounds of the attention output


class ErrSplit:
    """GPU-vs-oracle error split by output magnitude: below 4 the dtype's max-abs bound
    applies; from 4 on, rounding a bf16 output alone can exceed it, so those errors are
    reported against half a bf16 ulp of the reference (plus 1e-5), as the parity tests do."""

    def __init__(self):
        self.small, self.big, self.big_ratio, self.n_big = 0.0, 0.0, 0.0, 0

    def add(self, got, ref):
        err = np.abs(got - ref)
        a = np.abs(ref)
        big = a >= 4
        if (~big).any():
            self.small = max(self.small, float(err[~big].max()))
        if big.any():
            half_ulp = np.exp2(np.floor(np.log2(a[big])) - 8)
            self.big_ratio = max(self.big_ratio, float((err[big] / (half_ulp + 1e-5)).max()))
            self.big = max(self.big, float(err[big].max()))
            self.n_big += int(big.sum())

    def report(self, dtype):
        r = {"max_abs_err_where_ref_below_4": self.small, "tolerance": TOL[dtype],
             "outputs_with_ref_at_least_4": self.n_big}
        if self.n_big and dtype == "bf16":
            r["max_err_over_half_bf16_ulp_where_ref_at_least_4"] = self.big_ratio
            big_ok = self.big_ratio <= 1.0
        else:
            r["max_abs_err_where_ref_at_least_4"] = self.big
            big_ok = self.big <= TOL[dtype]
        r["within_tolerance"] = self.small <= TOL[dtype] and big_ok
        return r


def cpu_baseline(b, gpu_out, time_cap=25.0):
    """The float64 oracle on the host: the step's block copies and write, then decode over the
    workload's sequences in order until all are done or the time cap is reached.  Also reports
    its max abs difference from the GPU output on those sequences."""
    import oracle
    from workloads import as_numpy
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = 1
    q, bt, lens = as_numpy(b.q), as_numpy(b.block_tables), as_numpy(b.seq_lens)
    done, err = 0, 0.0
    t0, c0 = time.time(), time.process_time()
    kc, vc = as_numpy(b.k_cache), as_numpy(b.v_cache)
    if b.cow_pairs is not None:
        kc, vc = oracle.copy_blocks(kc, vc, as_numpy(b.cow_pairs))
    if b.slot_mapping is not None:
        kc, vc = oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), as_numpy(b.slot_mapping), kc, vc)
    split = ErrSplit()
    while done < b.num_seqs and time.time() - t0 < time_cap:
        ref = oracle.paged_decode(q, kc, vc, bt, lens, b.scale, b.dtype, seqs=[done])
        err = max(err, float(np.abs(gpu_out[done] - ref[0]).max()))
        split.add(gpu_out[done], ref[0])
        done += 1
    wall, cpu = time.time() - t0, time.process_time() - c0
    esize = 4 if b.dtype == "f32" else 2
    kv = int(lens[:done].astype(np.int64).sum()) * b.num_kv_heads * b.head_dim * 2 * esize
    steps = ("block copies, " if b.cow_pairs is not None else "") + \
            (f"write of all {len(b.slot_mapping)} new tokens, " if b.slot_mapping is not None else "")
    steps = steps + "then decode" if steps else "decode"
    return {"value": kv / wall / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} of the first {done} of {b.num_seqs} sequences of the "
                      f"same workload (numpy float64, {kv / 1e9:.3f} GB of K/V)",
            "seqs_per_s": done / wall, "wall_s": wall, "cpu_s": cpu,
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "max_abs_err_gpu_vs_oracle": err, **split.report(b.dtype)}


def cpu_baseline_multi_query(b, gpu_out, flops_unit=False, time_cap=25.0):
    """The float64 oracle on the host for a multi-query step: the write of the new tokens, then
    attention for the workload's sequences in order until done or the time cap is reached.  The
    rate is in the workload's metric: GB/s of K/V, or (flops_unit) causal TFLOP/s, 4 x pairs x
    heads x head_dim over the sequences done."""
    import oracle
    from workloads import as_numpy
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = 1
    q, bt, lens, qs = as_numpy(b.q), as_numpy(b.block_tables), as_numpy(b.seq_lens), b.q_start.tolist()
    t0 = time.time()
    kc, vc = oracle.write_kv(as_numpy(b.new_k), as_numpy(b.new_v), as_numpy(b.slot_mapping),
                             as_numpy(b.k_cache), as_numpy(b.v_cache))
    done, err, kv, pairs = 0, 0.0, 0, 0
    split = ErrSplit()
    while done < b.num_seqs and time.time() - t0 < time_cap:
        a, z = qs[done], qs[done + 1]
        n, L = z - a, int(lens[done])
        pairs += n * (L - n) + n * (n + 1) // 2
        ref = oracle.paged_multi_query(q[a:z], kc, vc, bt[done:done + 1], lens[done:done + 1],
                                       np.array([0, z - a]), b.scale, b.dtype)
        err = max(err, float(np.abs(gpu_out[a:z] - ref).max()))
        split.add(gpu_out[a:z], ref)
        kv += int(lens[done]) * b.num_kv_heads * b.head_dim * 2 * 2
        done += 1
    wall = time.time() - t0
    if flops_unit:
        rate = {"value": 4.0 * pairs * b.num_heads * b.head_dim / wall / 1e12, "unit": "TFLOP/s"}
    else:
        rate = {"value": kv / wall / 1e9, "unit": "GB/s"}
    return {**rate, "cores": threads, "kind": "oracle",
            "sample": f"write of all {len(b.slot_mapping)} new tokens, then the queries of the first "
                      f"{done} of {b.num_seqs} sequences of the same workload (numpy float64)",
            "seqs_per_s": done / wall, "wall_s": wall, "host_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(), "max_abs_err_gpu_vs_oracle": err, **split.report(b.dtype)}


def unique_kv_bytes(b):
    """K/V bytes of the distinct pool slots the step's sequences read (shared blocks once)."""
    B = b.block_size
    seen = set()
    for s, L in enumerate(b.seq_lens.tolist()):
        row = b.block_tables[s].tolist()
        for j in range(-(-L // B)):
            seen.add((row[j], min(B, L - j * B)))
    slots = {}
    for blk, fill in seen:
        slots[blk] = max(slots.get(blk, 0), fill)
    esize = 4 if b.dtype == "f32" else 2
    return sum(slots.values()) * b.num_kv_heads * b.head_dim * 2 * esize


def write_is_newest(b):
    """True when the step's write stores one token per sequence, at its position L - 1 (the
    slot the block table gives that position), so write and decode can run as one call."""
    if b.slot_mapping is None or len(b.slot_mapping) != b.num_seqs:
        return False
    B = b.block_size
    for s, L in enumerate(b.seq_lens.tolist()):
        if L < 1 or int(b.slot_mapping[s]) != int(b.block_tables[s, (L - 1) // B]) * B + (L - 1) % B:
            return False
    return True


def cache_op_lines(dev, stream, K, flush, nk, nv, slots, kc, vc):
    """pa_write_kv of the step's new tokens, and pa_copy_blocks of 224 copy-on-write pairs of
    OPT-13B-shaped blocks (16 tokens x 40 KV heads x 128, fp16: 160 KiB per block per pool),
    each call after a cache flush; GB/s on the bytes each call must read plus write."""
    res = {}
    # the write is idempotent (the same rows to the same slots)
    w_ms = timed_calls(lambda: pk.pa_write_kv(nk, nv, slots, kc, vc), K, stream, flush)
    wb = 2 * 2 * nk.numel() * nk.element_size()              # K and V rows, read + written
    w = pct(w_ms)
    res["pa_write_kv"] = {"workload": f"{nk.shape[0]} new tokens of the Llama-3-8B shape",
                          "bytes_read_plus_written": wb, "us": w,
                          "gbs": wb / (w["median"] * 1e-6) / 1e9,
                          "frac_of_hbm_peak": wb / (w["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS}
    # 32 prompts x 7 copying samples: sources are the prompts' last blocks, destinations
    # fresh blocks; a pool of 32 + 224 blocks plus slack, on the device
    nb, B, H, D = 320, 16, 40, 128
    g = torch.Generator(device=dev).manual_seed(0)
    ck = torch.randn((nb, B, H, D), device=dev, generator=g).to(torch.float16)
    cv = torch.randn((nb, B, H, D), device=dev, generator=g).to(torch.float16)
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(0))
    src = perm[:32].repeat_interleave(7)
    dst = perm[32:32 + 224]
    pairs = torch.stack([src, dst], 1).int().to(dev)
    c_ms = timed_calls(lambda: pk.pa_copy_blocks(ck, cv, pairs), K, stream, flush)
    cb = 224 * 2 * 2 * B * H * D * 2                         # K and V blocks, read + written
    c = pct(c_ms)
    res["pa_copy_blocks"] = {"workload": "224 copy-on-write pairs of OPT-13B-shaped fp16 blocks "
                                         "(32 prompts x 7 copying samples)",
                             "bytes_read_plus_written": cb, "us": c,
                             "gbs": cb / (c["median"] * 1e-6) / 1e9,
                             "frac_of_hbm_peak": cb / (c["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS}
    return res


WORKLOADS = {
    # name: (builder, shape description)
    "llama3_8b": (lambda a: workloads.llama3_8b(seed=0),
                  {"num_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 16,
                   "seq_len_range": [512, 4096], "num_blocks": 70000}),
    "llama7b": (lambda a: workloads.llama7b(seed=0),
                {"num_heads": 32, "num_kv_heads": 32, "head_dim": 128, "block_size": 16,
                 "seq_len_range": [1, 2048]}),
    "opt13b_shared": (lambda a: workloads.opt13b_shared(seed=0),
                      {"num_heads": 40, "num_kv_heads": 40, "head_dim": 128, "block_size": 16,
                       "prompts": 32, "samples": 8, "prompt_len": 1024, "tail_range": [0, 256]}),
    "opt13b_cow": (lambda a: workloads.opt13b_cow(seed=0),
                   {"num_heads": 40, "num_kv_heads": 40, "head_dim": 128, "block_size": 16,
                    "prompts": 32, "samples": 8, "prompt_len": 1000, "cow_pairs": 224}),
    "llama2_70b": (lambda a: workloads.llama2_70b(seed=0, block_size=a.block_size),
                   {"num_heads": 64, "num_kv_heads": 8, "head_dim": 128,
                    "seq_len_range": [8192, 32768], "key_outliers": 0.01}),
    "llama3_8b_spec": (lambda a: workloads.llama3_8b_spec(seed=0),
                       {"num_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 16,
                        "seq_len_range": [512, 4096], "queries_per_seq": 4, "num_blocks": 70000}),
    "llama3_8b_chunk": (lambda a: workloads.llama3_8b_chunk(seed=0),
                        {"num_heads": 32, "num_kv_heads": 8, "head_dim": 128, "block_size": 16,
                         "prior_range": [0, 3584], "chunk": 512}),
}
WORKLOAD_NAMES = {"llama3_8b": "llama3_8b_gqa_decode", "llama7b": "llama7b_mha_decode",
                  "opt13b_shared": "opt13b_shared_prefix_decode", "opt13b_cow": "opt13b_cow_decode",
                  "llama2_70b": "llama2_70b_long_context_decode",
                  "llama3_8b_spec": "llama3_8b_speculative_verify_4_tokens",
                  "llama3_8b_chunk": "llama3_8b_chunked_prefill_512"}
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, vendor figure
DTYPE_NAME = {"f32": "f32", "f16": "fp16", "bf16": "bf16"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--swap", action="store_true",
                    help="measure pa_swap_blocks (HBM <-> pinned host) instead of the decode step")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="opt13b_* workloads: decode with pa_decode_shared_prefix (each group's "
                         "shared prompt blocks read once) instead of pa_decode")
    ap.add_argument("--workload", default="llama3_8b", choices=sorted(WORKLOADS),
                    help="the benchmark line is llama3_8b; the others are the remaining workloads "
                         "of the same study, measured the same way")
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32],
                    help="block size of the llama2_70b workload")
    ap.add_argument("--fused", action="store_true",
                    help="run the step's write and decode as one pa_decode_append (the default "
                         "wherever the write stores each sequence's newest token and the batch "
                         "shares no blocks); an error where it cannot")
    ap.add_argument("--two-call", action="store_true",
                    help="run the step's write and decode as two calls, pa_write_kv then pa_decode")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as replays of a HIP graph captured once (the roofline "
                         "still times the eager decode call)")
    ap.add_argument("--record-traffic", nargs=4, metavar="CSV",
                    help="decode FETCH_SIZE, decode WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE "
                         "counter files from rocprofv3 --pmc -f csv")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    pk.lib()
    if args.copy_calibration:
        copy_calibration(max(1, args.steps))
        return
    if args.swap:
        swap_bench(max(1, min(args.steps, 20)), max(1, min(args.warmup, 3)), not args.no_cpu_baseline)
        return

    dev = torch.device("cuda:0")
    build, shape = WORKLOADS[args.workload]
    log(f"building the {args.workload} workload (seed 0)")
    b = build(args)
    q, kc, vc = b.q.to(dev), b.k_cache.to(dev), b.v_cache.to(dev)
    bt, lens = b.block_tables.to(dev), b.seq_lens.to(dev)
    has_write = b.slot_mapping is not None
    if has_write:
        nk, nv, slots = b.new_k.to(dev), b.new_v.to(dev), b.slot_mapping.to(dev)
    pairs = b.cow_pairs.to(dev) if b.cow_pairs is not None else None
    out = torch.empty_like(q)
    max_len = b.max_seq_len
    kv_bytes = b.kv_bytes()
    stream = torch.cuda.current_stream()
    multi = b.q_start is not None
    shared = args.shared_prefix
    if shared and b.group_start is None:
        raise SystemExit("--shared-prefix needs a workload with shared-prefix groups (opt13b_*)")
    if multi:
        qs = b.q_start.to(dev)
        need = pk.pa_multi_query_workspace_size(b.num_seqs, q.shape[0], b.num_heads, b.num_kv_heads,
                                                b.head_dim, b.max_q_len, max_len)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

        def attend():
            pk.pa_multi_query(q, kc, vc, bt, lens, qs, b.num_kv_heads, b.scale, out,
                              max_q_len=b.max_q_len, max_seq_len=max_len, workspace=ws)
    elif shared:
        gs, pre = b.group_start.to(dev), b.prefix_lens.to(dev)
        max_group = int((b.group_start[1:] - b.group_start[:-1]).max())
        need = pk.pa_decode_shared_prefix_workspace_size(b.num_seqs, len(b.prefix_lens), b.num_heads,
                                                         b.num_kv_heads, b.head_dim, max_group, max_len)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

        def attend():
            pk.pa_decode_shared_prefix(q, kc, vc, bt, lens, gs, pre, b.num_kv_heads, b.scale, out,
                                       max_group_size=max_group, max_seq_len=max_len, workspace=ws)
    else:
        ws = pk.decode_workspace(q, b.num_kv_heads, max_len)
        # batches whose sequences share blocks read them with the default cache policy
        decode_fn = pk.pa_decode_cached if b.group_start is not None else pk.pa_decode

        def decode():
            decode_fn(q, kc, vc, bt, lens, b.num_kv_heads, b.scale, out, max_seq_len=max_len,
                      workspace=ws)

        def decode_append():
            pk.pa_decode_append(q, nk, nv, kc, vc, bt, lens, b.num_kv_heads, b.scale, out,
                                max_seq_len=max_len, workspace=ws)
        attend = decode
    # A step whose write stores exactly each sequence's newest token (position L - 1), in a
    # batch that shares no blocks, runs write and decode as one pa_decode_append unless
    # --two-call asks for pa_write_kv + pa_decode.
    can_fuse = (not multi and not shared and has_write and b.group_start is None
                and write_is_newest(b))
    if args.fused and (args.two_call or not can_fuse):
        raise SystemExit("--fused needs a decode workload whose write stores each sequence's "
                         "newest token, in a batch that shares no blocks (and no --two-call)")
    fused = can_fuse and not args.two_call
    if fused:
        attend = decode_append

    def step(ev0=None, ev1=None):
        # copies and writes are idempotent, so every step repeats the same state change
        if pairs is not None:
            pk.pa_copy_blocks(kc, vc, pairs)
        if has_write and not fused:
            pk.pa_write_kv(nk, nv, slots, kc, vc)
        if ev0 is not None:
            ev0.record(stream)
        attend()
        if ev1 is not None:
            ev1.record(stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    # The per-step spread first: K steps with HIP events around each step and its attention
    # call.  They also carry the GPU past its first ~20 ms of this kernel, which run slower
    # than the steady state (the first 20 steps after 5 warm-up steps take about 7 µs more
    # each than every later 20).  An event record takes GPU time of its own, so the
    # wall-clock steps below run without them.
    ev = [(HipEvent(), HipEvent(), HipEvent()) for _ in range(K)]
    log(f"timing {K} steps with events")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        step(ev[i][1], ev[i][2])
    torch.cuda.synchronize()
    events_total = time.perf_counter() - t0
    step_ms = [a.elapsed_time(z) for a, _, z in ev]          # whole step, back to back
    call_ms_warm = [a.elapsed_time(z) for _, a, z in ev]     # its attention call

    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    eager_total = total

    # the roofline leg: the attention call alone, K times, each after an untimed read of
    # 1 GiB that evicts L2 and the Infinity Cache (the step's write and copies are done,
    # and repeating the call changes nothing)
    log(f"timing {K} calls, each after a cache flush")
    flush = CacheFlush(dev)
    call_ms = timed_calls(attend, K, stream, flush)
    call = pct(call_ms)
    dec_avg = call["median"] * 1e-3                          # ms
    if args.graph:
        # a serving loop records its step once and replays it; inputs stay where they were
        # captured, and the copies and writes are idempotent, so replays repeat the step
        log("capturing the step in a HIP graph")
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(max(1, args.warmup)):
            graph.replay()
        torch.cuda.synchronize()
        log(f"timing {K} graph replays")
        t0 = time.perf_counter()
        for _ in range(K):
            graph.replay()
        torch.cuda.synchronize()
        total = time.perf_counter() - t0

    ms_per_step = total * 1e3 / K
    value = kv_bytes / (total / K) / 1e9
    achieved = kv_bytes / (dec_avg * 1e-3) / 1e9
    traffic = measured_traffic()
    cache_ops = None
    if args.workload == "llama3_8b":
        cache_ops = cache_op_lines(dev, stream, K, flush, nk, nv, slots, kc, vc)
    res = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAME[b.dtype], "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "num_seqs": b.num_seqs, **shape,
                   "block_size": b.block_size, "num_blocks": b.num_blocks,
                   "write_tokens": len(b.slot_mapping) if has_write else 0,
                   "seed": 0, "kv_bytes_per_step": kv_bytes},
        "pct_of_hbm_peak": 100.0 * value / HBM_PEAK_GBS,
        "step_mode": "graph" if args.graph else "eager",
        "eager_ms_per_step": eager_total * 1e3 / K,
        "events_ms_per_step": events_total * 1e3 / K,
        "timing_order": (f"{args.warmup} warm-up steps; {K} steps with events (step_us); {K} "
                         f"wall-clock steps (value); {K} flushed calls (roofline)"),
        "step_calls": ("pa_decode_append" if fused else
                       ("pa_copy_blocks + " if pairs is not None else "") +
                       ("pa_write_kv + " if has_write else "") + ("pa_multi_query" if multi else
                       "pa_decode_shared_prefix" if shared else
                       "pa_decode_cached" if b.group_start is not None else "pa_decode")),
        "seqs_per_s": b.num_seqs / (total / K),
        "step_us": pct(step_ms),
        "roofline": {"kernel": ("pa_decode_append" if fused else "pa_decode_cached"
                                if b.group_start is not None else "pa_decode") +
                               " (decode_kernel + reduce_kernel)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": kv_bytes,
                     "timing": "median of K calls, each after a 1 GiB read that evicts the caches; "
                               "HIP events without the system-scope fence",
                     "call_us": call, "call_us_back_to_back": pct(call_ms_warm),
                     "avg_launch_us": call["mean"], "p10_us": call["p10"], "p90_us": call["p90"]},
        "cache_ops": cache_ops,
        "cpu_baseline": None,
    }
    if args.workload != "llama3_8b":
        # counters are recorded for the benchmark line's kernel only
        res["roofline"]["traffic"] = None
    if args.workload.startswith("opt13b"):
        # samples share their prompt's blocks: logical bytes count them once per sample
        ub = unique_kv_bytes(b)
        res["config"]["unique_kv_bytes_per_step"] = ub
        res["roofline"]["achieved_unique"] = ub / (dec_avg * 1e-3) / 1e9
        res["metric"] = "paged-decode KV GB/s read (logical, each sample's prompt counted), OPT-13B-shaped, 1 GPU"
        if shared:
            # the shared-prefix call reads each distinct block once: its algorithmic bytes
            # are the unique bytes, and so is the step's rate
            res["metric"] = "shared-prefix paged-decode KV GB/s read (distinct blocks), OPT-13B-shaped, 1 GPU"
            res["config"]["workload"] = WORKLOAD_NAMES[args.workload] + "_grouped"
            res["value"] = ub / (total / K) / 1e9
            res["pct_of_hbm_peak"] = 100.0 * res["value"] / HBM_PEAK_GBS
            res["logical_kv_gbs"] = kv_bytes / (total / K) / 1e9
            split = os.environ.get("PA_SHARED_PREFIX_ROWS") == "0"
            res["roofline"].update({"kernel": "pa_decode_shared_prefix (multi_query_kernel, shared layout)"
                                    if split else
                                    "pa_decode_shared_prefix (decode_kernel rows mode over laid-out group "
                                    "tables, + shared_layout_kernel and reduce_kernel)",
                                    "achieved": res["roofline"]["achieved_unique"],
                                    "frac": res["roofline"]["achieved_unique"] / HBM_PEAK_GBS,
                                    "algorithmic_bytes_per_launch": ub})
    if args.workload in ("llama7b", "llama2_70b"):
        res["metric"] = f"paged-decode KV GB/s read (% of HBM peak), {WORKLOAD_NAMES[args.workload]}, 1 GPU"
    if multi:
        res["metric"] = ("paged multi-query attention, Llama-3-8B-shaped, 1 GPU: KV GB/s read"
                         if args.workload.endswith("spec") else
                         "paged multi-query attention, Llama-3-8B-shaped, 1 GPU: causal TFLOP/s")
        flops = 4.0 * b.causal_pairs() * b.num_heads * b.head_dim
        res["config"]["query_rows"] = int(q.shape[0])
        res["config"]["causal_flops_per_step"] = flops
        res["roofline"]["kernel"] = ("pa_multi_query (decode_kernel rows mode + reduce_kernel)"
                                     if args.workload.endswith("spec") and
                                     os.environ.get("PA_MULTI_QUERY_ROWS") != "0" else
                                     "pa_multi_query (multi_query_kernel)")
        if args.workload.endswith("chunk"):
            tf = flops / (dec_avg * 1e-3) / 1e12
            res.update({"value": flops / (total / K) / 1e12, "unit": "TFLOP/s"})
            res["roofline"].update({"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS,
                                    "algorithmic_flops_per_launch": flops})
            res.pop("pct_of_hbm_peak", None)
    if not args.no_cpu_baseline:
        log("cpu baseline: float64 oracle on the host")
        torch.cuda.synchronize()
        gpu_out = out.float().cpu().double().numpy()
        res["cpu_baseline"] = (cpu_baseline_multi_query(b, gpu_out, flops_unit=args.workload.endswith("chunk"))
                               if multi else cpu_baseline(b, gpu_out))
    print(json.dumps(res))


if __name__ == "__main__":
    main()
