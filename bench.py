"""Benchmark of the FP8 ASH + DS compression path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input, the
Qwen2.5-7B-shaped tensor-parallel activation workload: P = 8 simulated rank shards of
bfloat16 [8, 4096, 3584], block 128, target 1.0.

  1. compress   all 8 shards in one call (8 x 117,440,512 elements) -> codes + alpha + s
  2. reduce_fp8 the 8 contributions -> one requantised tensor (codes + alpha + s)
  3. decompress the reduced tensor to bfloat16

Inputs are generated on the host (seeded, see workloads/) and are resident in HBM before the
timed region starts.  Before the timed region a settle phase runs steps for a fixed span of
wall time (the GPU's clocks take about that long to reach their loaded level), whatever the
--warmup count.  `value` is the metric: the compress kernel's throughput in GB/s of bfloat16
input (8 x 117,440,512 x 2 bytes per launch) over its mean duration in the K timed steps, from
HIP events on the kernels' stream around every kernel of those steps; the whole step's rate is
reported beside it (`pipeline_gbps_bf16_in`, from the wall clock around exactly K steps).
`roofline` describes the same compress launches; `cpu_baseline` is the FP64 CPU oracle's
compress timed on this host over a bounded sample of the same shards (the whole pipeline's
oracle rate beside it).  After the timed steps
each kernel is also timed over K back-to-back launches, and so is the local gradient
accumulation on its own workload (GPT-13B-shaped gradients [4, 4096, 5120], block 128: main
gradient = compressed shard 0, local gradient = shard 1); those figures are reported beside
the step and are not part of `value`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --copy-calibrate   (plain 1 GiB device copy, for HBM counter scaling)
       python bench.py --all-workloads      (every operation on every workload, warm and with the
                                           caches flushed, beside same-byte references)
       python bench.py --size-curve         (compress, decompress and the reduce from 2^19 to
                                           2^31 elements, flushed and rotating)
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

METRIC = "fused FP8 ASH+DS compress GB/s (bf16 in) and % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
STEP_WORKLOAD = "qwen2.5-7b-act"  # Qwen2.5-7B-shaped activations, 8 shards: the timed step
ACC_WORKLOAD = "gpt13b-grad"  # GPT-13B-shaped gradients, for the local gradient accumulation
TARGET = 1.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "compress_qwen7b_8shards_hbm_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(csrc: str | None = None) -> str:
    """SHA-256 of the kernel sources with comments and whitespace removed, so that the counter
    record is tied to the code it measured and not to its comments."""
    import re

    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "fp8_compression_tensor_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        text = re.sub(r"\s+", " ", text).strip()
        h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()


def measured_traffic(path: str = TRAFFIC_FILE, csrc: str | None = None):
    """HBM bytes per compress launch from the committed rocprofv3 counter summary, scaled by
    the copy-kernel calibration it records; None if absent or taken on other kernel source."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash(csrc):
        return None
    return float(rec["fetch_bytes_per_launch"]) + float(rec["write_bytes_per_launch"])


def copy_calibrate(steps: int):
    import torch

    n = 1 << 29  # 1 GiB of bfloat16
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy-calibrate: {steps} copies of {2 * n} bytes (read {2 * n}, write {2 * n} per copy)")
    print(json.dumps({"copy_bytes_read": 2 * n, "copy_bytes_written": 2 * n, "copies": steps}))


def cpu_baseline(xs, block: int, model: str, budget_s: float = 8.0):
    """Time the oracle on bounded prefix samples of every shard, all cores and one core:
    compress alone (the metric's operation, `value`), and the whole pipeline.  `model` is the
    host CPU's description, taken (by cpu_model) before the process touched the GPU."""
    import numpy as np

    import oracle

    P = xs.shape[0]
    cores = len(os.sched_getaffinity(0))
    xs = xs.reshape(P, -1)
    n_full = xs.shape[1]

    def sample(m):  # the first m blocks of each shard, stacked
        return np.ascontiguousarray(xs[:, :m * block]).reshape(-1)

    def run_compress(m):
        x = sample(m)
        t0 = time.perf_counter()
        oracle.compress(x, block, TARGET)
        return time.perf_counter() - t0

    def run_pipeline(m):
        x = sample(m)
        t0 = time.perf_counter()
        q, a, s = oracle.compress(x, block, TARGET)
        qr, ar, sr = oracle.reduce_fp8(q.reshape(P, -1), a.reshape(P, -1), s.reshape(P, -1), block,
                                       TARGET)
        oracle.decompress(qr, ar, sr, block, np.uint16)
        return time.perf_counter() - t0

    def timed(run, threads, budget, m0):
        # scale a first short sample so the timed one takes about `budget`, capped at the shards
        oracle.set_threads(threads)
        t = run(m0)
        m = int(min(n_full // block, max(m0, m0 * budget / max(t, 1e-3))))
        t = run(m)
        return m, t, P * m * block * 2 / t / 1e9

    mc, tc, gc = timed(run_compress, cores, budget_s, 4096)
    m1, t1, g1 = timed(run_compress, 1, budget_s / 2, 512)
    mp, tp, gp = timed(run_pipeline, cores, budget_s / 2, 2048)
    oracle.set_threads(cores)
    return {"value": gc, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"compress of the first {mc} blocks ({mc * block} elements) of each of the "
                      f"{P} shards (bf16 in), float64 oracle on {cores} threads, {tc:.1f} s wall",
            "single_thread_value": g1,
            "single_thread_sample": f"compress of the first {m1} blocks of each shard, 1 thread, "
                                    f"{t1:.1f} s wall",
            "pipeline_value": gp,
            "pipeline_sample": f"compress -> reduce_fp8 -> decompress(bf16) of the first {mp} "
                               f"blocks of each shard, {cores} threads, {tp:.1f} s wall",
            "cpu_model": model}


def cpu_model() -> str:
    """lscpu's model name and family / model / stepping, else /proc/cpuinfo's model name.  Runs
    lscpu as a child process, so it must be called before this process initialises the GPU."""
    import subprocess

    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        f = {k.strip(): v.strip() for k, v in (l.split(":", 1) for l in out.splitlines() if ":" in l)}
        if "Model name" in f:
            return (f"{f['Model name']} (lscpu: vendor {f.get('Vendor ID', '?')}, family "
                    f"{f.get('CPU family', '?')}, model {f.get('Model', '?')}, stepping "
                    f"{f.get('Stepping', '?')}, {f.get('Socket(s)', '?')} socket(s), "
                    f"{f.get('Thread(s) per core', '?')} thread(s) per core)")
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _event():
    import torch

    return torch.cuda.Event(enable_timing=True)


def _timed(fn, flushed, reps, stream, flush):
    """Median and minimum duration (us) of single launches fn(), after 3 untimed ones, each
    bracketed by events on `stream`; with `flushed`, a read of `flush` before each launch."""
    import statistics

    ts = []
    for i in range(reps + 3):
        if flushed:
            flush.sum()  # reads the buffer: evicts the caches without leaving dirty lines
        a, b = _event(), _event()
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        if i >= 3:
            ts.append(a.elapsed_time(b) * 1e3)
    return statistics.median(ts), min(ts)


def _rotating(setup, set_bytes, stream, rot_bytes=3 << 30):
    """Steady-state duration (us) of back-to-back launches cycling through distinct buffer sets:
    setup(i) -> launch closure on set i, with enough sets (2 to 256) to total rot_bytes, timed
    over whole cycles after a 0.4 s settle; median of 5 runs of 4 cycles.  Returns (us, sets)."""
    import statistics

    import torch

    R = min(256, max(2, -(-rot_bytes // int(set_bytes))))
    fns = [setup(i) for i in range(R)]
    # settle: the timed cycles then run at the loaded clock level (right after single-launch
    # protocols the clocks are measurably lower)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.4:
        for f in fns:
            f()
        torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a, b = _event(), _event()
        a.record(stream)
        for k in range(4 * R):
            fns[k % R]()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / (4 * R))
    del fns
    torch.cuda.empty_cache()
    return statistics.median(ts), R


def all_workloads(reps: int):
    """Every operation on every workload, three ways: warm, flushed, and rotating (see below),
    beside same-byte references; one JSON object on stdout, a table on stderr.

    warm      one launch at a time, back to back on the same buffers, a synchronisation each.
    flushed   one launch at a time with a 1 GiB read between launches (evicts the L2 and the
              256 MB MALL).  Plain stores can look fast here: their output waits in the MALL
              and its write to HBM falls into the next flush, outside the launch.
    rotating  back-to-back launches that cycle through distinct buffer sets (inputs and
              outputs) totalling at least 3 GiB (at most 256 sets), timed over whole cycles:
              nothing stays cached between a set's uses and every write-back is paid inside
              the sequence.  The steady-state rate of a stream of such calls."""
    import numpy as np
    import torch

    from workloads import WORKLOADS, make_shards

    host = {}
    for key, wl in WORKLOADS.items():
        host[key] = make_shards(key, count=max(wl.shards, 2 if key == ACC_WORKLOAD else 1))
    log("inputs generated")

    import fp8_compression_tensor_amd as tfp8

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, > L2 + MALL
    rot_bytes = 3 << 30

    def check(st):
        if st != 0:
            raise RuntimeError(tfp8.status_string(st))

    def timed(fn, flushed):
        return _timed(fn, flushed, reps, stream, flush)

    def rotating(setup, set_bytes):
        # at most 256 sets (the small workloads: still more than 1.5x the 256 MB MALL)
        return _rotating(setup, set_bytes, stream, rot_bytes)

    rows = []

    def gbps(nbytes, us):
        return nbytes / (us * 1e-6) / 1e9

    def measure(key, op, setup, alg_bytes, set_bytes, elements, B, P, bf16_in=None, ref=None,
                rotate=True):
        fn = setup(0)
        wm, wn = timed(fn, False)
        fm, fn_ = timed(fn, True)
        row = {"workload": key, "op": op, "elements": elements, "block": B, "P": P,
               "bytes_algorithmic": int(alg_bytes), "warm_us_median": round(wm, 2),
               "warm_us_min": round(wn, 2), "flushed_us_median": round(fm, 2),
               "flushed_us_min": round(fn_, 2),
               "flushed_GBps": round(gbps(alg_bytes, fm), 1),
               "flushed_frac_of_peak": round(gbps(alg_bytes, fm) / HBM_PEAK_GBS, 4)}
        if rotate:
            rm, R = rotating(setup, set_bytes)
            row.update({"rotating_us": round(rm, 2), "rotating_sets": R,
                        "rotating_GBps": round(gbps(alg_bytes, rm), 1),
                        "rotating_frac_of_peak": round(gbps(alg_bytes, rm) / HBM_PEAK_GBS, 4)})
        if bf16_in is not None:
            row["bf16_in_GBps_flushed"] = round(gbps(bf16_in, fm), 1)
        if ref is not None:
            rsetup, rbytes, rname = ref
            rfm, _ = timed(rsetup(0), True)
            row.update({"ref": rname, "ref_bytes": int(rbytes), "ref_flushed_us_median": round(rfm, 2),
                        "ref_GBps_flushed": round(gbps(rbytes, rfm), 1)})
            row["ratio_to_ref_flushed"] = round(row["flushed_GBps"] / row["ref_GBps_flushed"], 4)
            if rotate:
                rrm, _ = rotating(rsetup, rbytes)
                row.update({"ref_rotating_us": round(rrm, 2),
                            "ref_GBps_rotating": round(gbps(rbytes, rrm), 1)})
                row["ratio_to_ref_rotating"] = round(row["rotating_GBps"] / row["ref_GBps_rotating"],
                                                     4)
        rows.append(row)
        log(f"{key:15s} {op:44s} n={elements:>10d} B={B} P={P}: warm {wm:8.1f}, flushed {fm:8.1f} us "
            f"({100 * row['flushed_frac_of_peak']:.1f}%)"
            + (f", rotating {row['rotating_us']:8.1f} us ({100 * row['rotating_frac_of_peak']:.1f}%)"
               if rotate else "")
            + (f"; {row['ref']}: flushed {row['ref_flushed_us_median']:.1f} us"
               + (f", rotating {row['ref_rotating_us']:.1f} us" if rotate else "")
               if ref is not None else ""))

    def own(t, i):  # set 0 uses the tensor itself, other sets a copy of it
        return t if i == 0 else t.clone()

    for key, wl in WORKLOADS.items():
        B, P, n = wl.block, wl.shards, wl.n
        nb = n // B
        xs = host[key]
        x = torch.from_numpy(xs.reshape(-1).view(np.int16)).to(dev)
        ntot = P * n

        def compress_setup(m):
            def setup(i):
                xi = own(x[:m], i)
                q = torch.empty(m, dtype=torch.uint8, device=dev)
                a = torch.empty(m // B, dtype=torch.float32, device=dev)
                s_ = torch.empty_like(a)
                return lambda: check(tfp8.compress_raw(xi.data_ptr(), tfp8.BF16, m, B, TARGET,
                                                       q.data_ptr(), a.data_ptr(), s_.data_ptr(),
                                                       sh))
            return setup

        # Same-byte references, torch kernels that move the operation's bytes with no other
        # work: compress reads 2 bytes and writes 1 per element, as an element-wise maximum of
        # the two halves of the input's bytes (uint8) does; the reduce reads P bytes and writes
        # 1, as a maximum over P uint8 rows does.  (torch's dtype-converting copies are not
        # vectorised and reach only ~2 TB/s, so they bound nothing.)
        def narrow_ref(m):
            def setup(i):
                x8 = own(x[:m], i).view(torch.uint8)
                y8 = torch.empty(m, dtype=torch.uint8, device=dev)
                return lambda: torch.maximum(x8[:m], x8[m:2 * m], out=y8)
            return setup, 3 * m, "uint8 max of two halves"

        measure(key, "compress", compress_setup(n), n * (3 + 8 / B), 3 * n, n, B, 1, 2 * n,
                narrow_ref(n))

        # float32 input: the same values widened (exactly), 4 bytes read and 1 written per
        # element; its same-byte reference is a maximum over the input's four uint8 rows
        x32 = x[:n].view(torch.bfloat16).float()

        def compress32_setup(i):
            xi = own(x32, i)
            q32 = torch.empty(n, dtype=torch.uint8, device=dev)
            a32 = torch.empty(nb, dtype=torch.float32, device=dev)
            s32 = torch.empty_like(a32)
            return lambda: check(tfp8.compress_raw(xi.data_ptr(), tfp8.F32, n, B, TARGET,
                                                   q32.data_ptr(), a32.data_ptr(), s32.data_ptr(),
                                                   sh))

        def quarters_ref(i):
            x8 = own(x32, i).view(torch.uint8).view(4, n)
            y8 = torch.empty(n, dtype=torch.uint8, device=dev)
            return lambda: torch.amax(x8, dim=0, out=y8)

        measure(key, "compress fp32 in", compress32_setup, n * (5 + 8 / B), 5 * n, n, B, 1,
                ref=(quarters_ref, 5 * n, "max of 4 uint8 rows"))
        del x32
        if P > 1:
            measure(key, f"compress {P} stacked shards", compress_setup(ntot), ntot * (3 + 8 / B),
                    3 * ntot, ntot, B, P, 2 * ntot, narrow_ref(ntot))
        # codes of every shard, for the stages below
        q = torch.empty(ntot, dtype=torch.uint8, device=dev)
        al = torch.empty(ntot // B, dtype=torch.float32, device=dev)
        sc = torch.empty_like(al)
        check(tfp8.compress_raw(x.data_ptr(), tfp8.BF16, ntot, B, TARGET, q.data_ptr(),
                                al.data_ptr(), sc.data_ptr(), sh))
        for dt, name, ob in ((torch.bfloat16, "decompress bf16", 2),
                             (torch.float32, "decompress fp32", 4)):
            code = tfp8.BF16 if dt == torch.bfloat16 else tfp8.F32

            def setup(i, dt=dt, code=code):
                qi, ai, si = own(q[:n], i), own(al[:nb], i), own(sc[:nb], i)
                out = torch.empty(n, dtype=dt, device=dev)
                return lambda: check(tfp8.decompress_raw(qi.data_ptr(), ai.data_ptr(),
                                                         si.data_ptr(), n, B, out.data_ptr(), code,
                                                         sh))
            measure(key, name, setup, n * (1 + 8 / B + ob), n * (1 + ob), n, B, 1)
        if P > 1:
            def reduce_setup(c, stacked):
                # P contributions of c codes each: the whole shards (c = n) or chunk 0 of each
                # shard, one rank's share in a P-way reduce-scatter (c = n / P), contiguous
                cb = c // B

                def setup(i):
                    qi = q.view(P, n)[:, :c].contiguous() if (i > 0 or not stacked) else q
                    ai = al.view(P, nb)[:, :cb].contiguous() if (i > 0 or not stacked) else al
                    si = sc.view(P, nb)[:, :cb].contiguous() if (i > 0 or not stacked) else sc
                    oq = torch.empty(c, dtype=torch.uint8, device=dev)
                    oa = torch.empty(cb, dtype=torch.float32, device=dev)
                    os_ = torch.empty_like(oa)
                    return lambda: check(tfp8.reduce_fp8_raw(qi.data_ptr(), ai.data_ptr(),
                                                             si.data_ptr(), P, c, B, TARGET,
                                                             oq.data_ptr(), oa.data_ptr(),
                                                             os_.data_ptr(), sh))
                return setup

            def rows_ref(c):
                def setup(i):
                    rows_q = q.view(P, n)[:, :c] if c == n and i == 0 else \
                        q.view(P, n)[:, :c].contiguous()
                    y8 = torch.empty(c, dtype=torch.uint8, device=dev)
                    return lambda: torch.amax(rows_q, dim=0, out=y8)
                return setup, (P + 1) * c, f"max of {P} uint8 rows"

            measure(key, f"reduce P={P}, {P} x n", reduce_setup(n, True),
                    (P + 1) * n * (1 + 8 / B), (P + 1) * n, n, B, P, ref=rows_ref(n))
            c = n // P
            measure(key, f"reduce P={P}, {P} x n/{P} (one rank)", reduce_setup(c, False),
                    (P + 1) * c * (1 + 8 / B), (P + 1) * c, c, B, P, ref=rows_ref(c))
            # the same share read in place from the stacked shards (row stride n), and from one
            # buffer of [codes | alpha | scale] messages, one per peer, as one all-to-all would
            # leave them, packed and with 65 KiB between messages (warm and flushed only)
            rq = torch.empty(c, dtype=torch.uint8, device=dev)
            ra = torch.empty(c // B, dtype=torch.float32, device=dev)
            rs = torch.empty_like(ra)
            fn = lambda: check(tfp8.reduce_strided_raw(q.data_ptr(), n, al.data_ptr(), nb,
                                                       sc.data_ptr(), nb, P, c, B, TARGET,
                                                       rq.data_ptr(), ra.data_ptr(), rs.data_ptr(),
                                                       sh))
            measure(key, f"reduce P={P}, {P} x n/{P} in place (stride n)", lambda i: fn,
                    (P + 1) * c * (1 + 8 / B), 0, c, B, P, rotate=False)
            cb = c // B
            for pad in (0, 65536 + 1024):
                M = (c + 8 * cb + pad + 15) // 16 * 16
                msg = torch.zeros(P, M, dtype=torch.uint8, device=dev)
                msg[:, :c].copy_(q.view(P, n)[:, :c])
                msg[:, c:c + 4 * cb].view(torch.float32).copy_(al.view(P, nb)[:, :cb])
                msg[:, c + 4 * cb:c + 8 * cb].view(torch.float32).copy_(sc.view(P, nb)[:, :cb])
                mp = msg.data_ptr()
                fn = (lambda mp=mp, M=M: check(tfp8.reduce_strided_raw(
                    mp, M, mp + c, M // 4, mp + c + 4 * cb, M // 4, P, c, B, TARGET,
                    rq.data_ptr(), ra.data_ptr(), rs.data_ptr(), sh)))
                measure(key, f"reduce P={P}, {P} x n/{P} from messages {M} B apart",
                        lambda i, fn=fn: fn, (P + 1) * c * (1 + 8 / B), 0, c, B, P, rotate=False)
                del msg
            del rq, ra, rs
        if key == ACC_WORKLOAD:
            # gradient accumulation: main = compressed shard 0, local = shard 1, out of place
            g = x[n:2 * n]

            def setup(i):
                qi, ai, si, gi = own(q[:n], i), own(al[:nb], i), own(sc[:nb], i), own(g, i)
                oq = torch.empty(n, dtype=torch.uint8, device=dev)
                oa = torch.empty(nb, dtype=torch.float32, device=dev)
                os_ = torch.empty_like(oa)
                return lambda: check(tfp8.accumulate_raw(qi.data_ptr(), ai.data_ptr(),
                                                         si.data_ptr(), gi.data_ptr(), tfp8.BF16,
                                                         n, B, TARGET, oq.data_ptr(),
                                                         oa.data_ptr(), os_.data_ptr(), sh))
            measure(key, "accumulate (main + local)", setup, n * (4 + 16 / B), 4 * n, n, B, 1)
            # the same with the local gradient in float32 (its values widened exactly)
            g32 = g.view(torch.bfloat16).float()

            def setup32(i):
                qi, ai, si, gi = own(q[:n], i), own(al[:nb], i), own(sc[:nb], i), own(g32, i)
                oq = torch.empty(n, dtype=torch.uint8, device=dev)
                oa = torch.empty(nb, dtype=torch.float32, device=dev)
                os_ = torch.empty_like(oa)
                return lambda: check(tfp8.accumulate_raw(qi.data_ptr(), ai.data_ptr(),
                                                         si.data_ptr(), gi.data_ptr(), tfp8.F32,
                                                         n, B, TARGET, oq.data_ptr(),
                                                         oa.data_ptr(), os_.data_ptr(), sh))
            measure(key, "accumulate, fp32 local gradient", setup32, n * (6 + 16 / B), 6 * n, n, B,
                    1)
            del g32
        del x, q, al, sc
        torch.cuda.empty_cache()
    print(json.dumps({"mode": "all-workloads", "reps": reps, "peak_GBps": HBM_PEAK_GBS,
                      "protocols": {"warm": "single launches back to back on the same buffers",
                                    "flushed": "a 1 GiB read (sum) between single launches",
                                    "rotating": "back-to-back launches cycling through distinct "
                                                "buffer sets of >= 3 GiB in total"},
                      "ref": "same-byte torch reference: compress vs a uint8 maximum of the two "
                             "halves of the input's bytes (2 bytes read, 1 written per element), "
                             "reduce vs a maximum over P uint8 rows; ratio = GB/s over its GB/s",
                      "rows": rows}), flush=True)


def size_curve(reps: int):
    """Compress (bfloat16 in), decompress (bfloat16 out) and the P = 8 reduce at B = 128 over
    sizes from 2^19 to 2^31 elements (the reduce: 2^16 to 2^28 per contribution), flushed and
    rotating as in --all-workloads, beside the same-byte references; one JSON object on stdout, a
    table on stderr.  The values are the Qwen2.5-7B-shaped activation shard's, repeated past its
    117 M elements; the reduce's P contributions are consecutive chunks of their codes."""
    import numpy as np
    import torch

    from workloads import WORKLOADS, make_shard

    wl = WORKLOADS[STEP_WORKLOAD]
    B, P = wl.block, wl.shards
    xs = make_shard(STEP_WORKLOAD, 0).reshape(-1)
    log("input generated")

    import fp8_compression_tensor_amd as tfp8

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, > L2 + MALL

    def check(st):
        if st != 0:
            raise RuntimeError(tfp8.status_string(st))

    nmax = 1 << 31
    x = torch.empty(nmax, dtype=torch.int16, device=dev)
    src = torch.from_numpy(xs.view(np.int16)).to(dev)
    for off in range(0, nmax, src.numel()):
        k = min(src.numel(), nmax - off)
        x[off:off + k].copy_(src[:k])
    del src
    q = torch.empty(nmax, dtype=torch.uint8, device=dev)
    al = torch.empty(nmax // B, dtype=torch.float32, device=dev)
    sc = torch.empty_like(al)
    check(tfp8.compress_raw(x.data_ptr(), tfp8.BF16, nmax, B, TARGET, q.data_ptr(), al.data_ptr(),
                            sc.data_ptr(), sh))

    def own(t, i):  # set 0 uses the tensor itself, other sets a copy of it
        return t if i == 0 else t.clone()

    rows = []

    def frac(nbytes, us):
        return nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS

    def measure(op, m, setup, alg_bytes, ref=None):
        fm, _ = _timed(setup(0), True, reps, stream, flush)
        rm, R = _rotating(setup, alg_bytes, stream)
        row = {"op": op, "elements": m, "block": B, "bytes_algorithmic": int(alg_bytes),
               "flushed_us": round(fm, 2), "flushed_frac_of_peak": round(frac(alg_bytes, fm), 4),
               "rotating_us": round(rm, 3), "rotating_sets": R,
               "rotating_frac_of_peak": round(frac(alg_bytes, rm), 4)}
        if ref is not None:
            rsetup, rbytes, rname = ref
            rfm, _ = _timed(rsetup(0), True, reps, stream, flush)
            rrm, _ = _rotating(rsetup, rbytes, stream)
            row.update({"ref": rname, "ref_bytes": int(rbytes), "ref_flushed_us": round(rfm, 2),
                        "ref_rotating_us": round(rrm, 3),
                        "ratio_rotating": round(frac(alg_bytes, rm) / frac(rbytes, rrm), 4)})
        rows.append(row)
        log(f"{op:24s} n={m:>11d}: flushed {fm:9.1f} us ({100 * row['flushed_frac_of_peak']:.1f}%), "
            f"rotating {rm:9.2f} us ({100 * row['rotating_frac_of_peak']:.1f}%)"
            + (f"; {row['ref']}: rotating {row['ref_rotating_us']:.2f} us, ratio "
               f"{row['ratio_rotating']:.3f}" if ref is not None else ""))

    for e in range(19, 32):
        m = 1 << e
        mb = m // B

        def compress_setup(i, m=m, mb=mb):
            xi = own(x[:m], i)
            oq = torch.empty(m, dtype=torch.uint8, device=dev)
            oa = torch.empty(mb, dtype=torch.float32, device=dev)
            os_ = torch.empty_like(oa)
            return lambda: check(tfp8.compress_raw(xi.data_ptr(), tfp8.BF16, m, B, TARGET,
                                                   oq.data_ptr(), oa.data_ptr(), os_.data_ptr(),
                                                   sh))

        def halves_ref(i, m=m):
            x8 = own(x[:m], i).view(torch.uint8)
            y8 = torch.empty(m, dtype=torch.uint8, device=dev)
            return lambda: torch.maximum(x8[:m], x8[m:], out=y8)

        measure("compress", m, compress_setup, m * (3 + 8 / B),
                (halves_ref, 3 * m, "uint8 max of two halves"))

        def decompress_setup(i, m=m, mb=mb):
            qi, ai, si = own(q[:m], i), own(al[:mb], i), own(sc[:mb], i)
            out = torch.empty(m, dtype=torch.bfloat16, device=dev)
            return lambda: check(tfp8.decompress_raw(qi.data_ptr(), ai.data_ptr(), si.data_ptr(),
                                                     m, B, out.data_ptr(), tfp8.BF16, sh))

        measure("decompress bf16", m, decompress_setup, m * (3 + 8 / B))

    for e in range(16, 29):
        c = 1 << e
        cb = c // B

        def reduce_setup(i, c=c, cb=cb):
            qi, ai, si = own(q[:P * c], i), own(al[:P * cb], i), own(sc[:P * cb], i)
            oq = torch.empty(c, dtype=torch.uint8, device=dev)
            oa = torch.empty(cb, dtype=torch.float32, device=dev)
            os_ = torch.empty_like(oa)
            return lambda: check(tfp8.reduce_fp8_raw(qi.data_ptr(), ai.data_ptr(), si.data_ptr(),
                                                     P, c, B, TARGET, oq.data_ptr(),
                                                     oa.data_ptr(), os_.data_ptr(), sh))

        def rows_ref(i, c=c):
            rq = own(q[:P * c], i).view(P, c)
            y8 = torch.empty(c, dtype=torch.uint8, device=dev)
            return lambda: torch.amax(rq, dim=0, out=y8)

        measure(f"reduce P={P}", c, reduce_setup, (P + 1) * c * (1 + 8 / B),
                (rows_ref, (P + 1) * c, f"max of {P} uint8 rows"))
    print(json.dumps({"mode": "size-curve", "reps": reps, "peak_GBps": HBM_PEAK_GBS,
                      "protocols": {"flushed": "a 1 GiB read (sum) between single launches",
                                    "rotating": "back-to-back launches cycling through distinct "
                                                "buffer sets of >= 3 GiB in total"},
                      "rows": rows}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # The GPU's clocks reach their loaded level only after some tens of milliseconds of steady
    # work (measured: with 5 warm-up steps the first timed compress launches ran up to 25%
    # longer), so after the warm-up steps the bench keeps stepping for this much wall time
    # before the timed region, whatever --warmup is.
    ap.add_argument("--settle-seconds", type=float, default=2.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibrate", action="store_true")
    ap.add_argument("--all-workloads", action="store_true",
                    help="time every operation on every workload, warm and flushed (own JSON)")
    ap.add_argument("--size-curve", action="store_true",
                    help="time compress, decompress and the reduce over a range of sizes (own JSON)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the reduce's contributions are simulated shards in one HBM).", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibrate:
        copy_calibrate(max(args.steps, 1))
        return
    if args.all_workloads:
        all_workloads(max(min(args.steps, 50), 5))
        return
    if args.size_curve:
        size_curve(max(min(args.steps, 50), 5))
        return

    from workloads import WORKLOADS, make_shards

    host_cpu = cpu_model()  # runs lscpu: before anything touches the GPU
    wl = WORKLOADS[STEP_WORKLOAD]
    B, P, n = wl.block, wl.shards, wl.n
    log(f"generating {P} shards of {wl.label} (seeded) ...")
    t0 = time.perf_counter()
    xs = make_shards(STEP_WORKLOAD)  # host generation before the GPU is touched
    log(f"  done in {time.perf_counter() - t0:.1f} s")
    # the local gradient accumulation's own workload: GPT-13B-shaped gradients, shard 0 as the
    # main gradient (compressed on the GPU below) and shard 1 as the local gradient
    gcfg = WORKLOADS[ACC_WORKLOAD]
    gs = make_shards(ACC_WORKLOAD, count=2)

    import numpy as np
    import torch

    import fp8_compression_tensor_amd as tfp8

    dev = torch.device("cuda:0")
    x = torch.from_numpy(xs.reshape(-1).view(np.int16)).to(dev).view(torch.bfloat16)
    nb = n // B
    codes = torch.empty(P * n, dtype=torch.uint8, device=dev)
    alpha = torch.empty(P * nb, dtype=torch.float32, device=dev)
    scale = torch.empty(P * nb, dtype=torch.float32, device=dev)
    rcodes = torch.empty(n, dtype=torch.uint8, device=dev)
    ralpha = torch.empty(nb, dtype=torch.float32, device=dev)
    rscale = torch.empty(nb, dtype=torch.float32, device=dev)
    out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def check(st):
        if st != 0:
            raise RuntimeError(tfp8.status_string(st))

    def k_compress():
        check(tfp8.compress_raw(x.data_ptr(), tfp8.BF16, P * n, B, TARGET, codes.data_ptr(),
                                alpha.data_ptr(), scale.data_ptr(), sh))

    def k_reduce():
        check(tfp8.reduce_fp8_raw(codes.data_ptr(), alpha.data_ptr(), scale.data_ptr(), P, n, B,
                                  TARGET, rcodes.data_ptr(), ralpha.data_ptr(), rscale.data_ptr(),
                                  sh))

    def k_decompress():
        check(tfp8.decompress_raw(rcodes.data_ptr(), ralpha.data_ptr(), rscale.data_ptr(), n, B,
                                  out.data_ptr(), tfp8.BF16, sh))

    def step():
        k_compress()
        k_reduce()
        k_decompress()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Settle: keep the GPU busy for a fixed span of wall time so that the timed steps run at the
    # loaded clock level (the queue is refilled every 16 steps; the GPU idles only for the
    # launch of the next batch).
    settle_steps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < args.settle_seconds:
        for _ in range(16):
            step()
        settle_steps += 16
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t0
    # Timed region: exactly K steps.  Events on the kernels' stream bracket every kernel, so the
    # per-kernel durations are those of the launches inside the timed steps (an event packet
    # between kernels was measured to change the step time by about 1%).
    log(f"settled for {settle_s:.2f} s ({settle_steps} steps); timing {args.steps} steps ...")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record(stream)
        k_compress()
        ev[k][1].record(stream)
        k_reduce()
        ev[k][2].record(stream)
        k_decompress()
        ev[k][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_step_events = ev[0][0].elapsed_time(ev[-1][3]) / args.steps
    d_c = sorted(e[0].elapsed_time(e[1]) for e in ev)  # compress durations, ms
    t_c = sum(d_c) / args.steps
    med_c = d_c[args.steps // 2] if args.steps % 2 else 0.5 * (d_c[args.steps // 2 - 1] +
                                                               d_c[args.steps // 2])
    t_r = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    t_d = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps

    # For reference: each kernel launched K times back to back (no other kernel in between).
    def per_launch_ms(fn):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    b2b = {"compress": round(per_launch_ms(k_compress), 4),
           "reduce_fp8": round(per_launch_ms(k_reduce), 4),
           "decompress": round(per_launch_ms(k_decompress), 4)}

    # Local gradient accumulation, measured on its own (not part of the step): main gradient =
    # the compressed shard 0 of the gradient workload, local gradient = its shard 1 (bfloat16),
    # sum requantised out of place.
    gn, gB = gcfg.n, gcfg.block
    g = torch.from_numpy(gs.reshape(-1).view(np.int16)).to(dev).view(torch.bfloat16)
    gq = torch.empty(2 * gn, dtype=torch.uint8, device=dev)
    ga = torch.empty(2 * gn // gB, dtype=torch.float32, device=dev)
    gsc = torch.empty(2 * gn // gB, dtype=torch.float32, device=dev)
    check(tfp8.compress_raw(g.data_ptr(), tfp8.BF16, gn, gB, TARGET, gq.data_ptr(), ga.data_ptr(),
                            gsc.data_ptr(), sh))

    def k_accumulate():
        check(tfp8.accumulate_raw(gq.data_ptr(), ga.data_ptr(), gsc.data_ptr(),
                                  g.data_ptr() + 2 * gn, tfp8.BF16, gn, gB, TARGET,
                                  gq.data_ptr() + gn, ga.data_ptr() + 4 * (gn // gB),
                                  gsc.data_ptr() + 4 * (gn // gB), sh))

    t_a = per_launch_ms(k_accumulate)
    alg_a = gn * (2 + 2 * (1 + 8.0 / gB))        # grad in, codes + scales in and out

    bytes_in = P * n * 2
    value = bytes_in / (t_c * 1e-3) / 1e9       # the metric: compress, bf16-in GB/s
    pipeline = bytes_in / (ms_step * 1e-3) / 1e9  # the whole step, wall clock
    alg_c = P * n * (2 + 1 + 8.0 / B)            # compress: bf16 in, codes out, 2 fp32 per block
    alg_r = (P + 1) * n * (1 + 8.0 / B)          # reduce: P code sets in, one out
    alg_d = n * (1 + 8.0 / B + 2)                # decompress: codes in, bf16 out
    ach_c = alg_c / (t_c * 1e-3) / 1e9
    traffic = measured_traffic()
    roofline = {"bound": "hbm", "achieved": round(ach_c, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach_c / HBM_PEAK_GBS, 4),
                "traffic": (round(traffic / (t_c * 1e-3) / 1e9, 1) if traffic else None),
                "kernel": "tfp8::k_compress<128, false, 0, false>",
                "bytes_per_launch_algorithmic": int(alg_c),
                "launch_us_mean": round(t_c * 1e3, 2), "launch_us_median": round(med_c * 1e3, 2),
                "launch_us_min": round(d_c[0] * 1e3, 2), "launch_us_max": round(d_c[-1] * 1e3, 2),
                "frac_at_median": round(alg_c / (med_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "traffic_bytes_per_launch": (int(traffic) if traffic else None)}
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "qwen2.5-7b tp activation [8,4096,3584] bf16 x 8 shards, block 128, "
                               "target 1: compress(8 stacked shards) -> reduce_fp8(P=8) -> "
                               "decompress(bf16); value = the compress launch",
                   "shape": list(wl.shape), "shards": P, "block": B, "target": TARGET},
        "value_hbm_frac": round(ach_c / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "settle": {"seconds": round(settle_s, 3), "steps": settle_steps},
        "pipeline_gbps_bf16_in": round(pipeline, 1),
        "kernels_ms": {"compress": round(t_c, 4), "reduce_fp8": round(t_r, 4),
                       "decompress": round(t_d, 4)},
        "kernels_ms_back_to_back": b2b,
        "ms_per_step_gpu_events": round(ms_step_events, 4),
        "reduce_hbm_frac_algorithmic": round(alg_r / (t_r * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "decompress_hbm_frac_algorithmic": round(alg_d / (t_d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "accumulate": {"kernel": "tfp8::k_accumulate<128, false, 0> + k_accumulate_fix",
                       "workload": f"gpt-13b gradients {list(gcfg.shape)} bf16, block {gB}: "
                                   "main gradient = compressed shard 0, local = shard 1, "
                                   "out of place",
                       "ms_per_launch": round(t_a, 4),
                       "bytes_per_launch_algorithmic": int(alg_a),
                       "gbps_algorithmic": round(alg_a / (t_a * 1e-3) / 1e9, 1),
                       "hbm_frac_algorithmic": round(alg_a / (t_a * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    del x, codes, out, g, gq
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(xs, B, host_cpu)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
