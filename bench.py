#!/usr/bin/env python3
"""Paged decode attention throughput on one MI355X.

One step = one decode step of a model's attention over every rotated layer:
  host   the native allocator reserves one new slot per sequence (taking a
         block when a sequence's last block is full) and rebuilds the block
         tables; slots and tables go to the GPU (pinned host buffers, async);
  GPU    per layer: copy-on-write copies (if any), the cache-write kernel
         appends the new token's K/V, then paged_attention_decode (main
         kernel; the partition merge runs in the same launch) attends over the whole cache.
Every layer has its own pool, so the K/V read each step is far larger than
the 256 MB Infinity Cache (reads come from HBM).

value    = KV tokens attended per second = sum over timed steps and layers of
           sum_b L_b, divided by the timed wall time.
roofline = the decode call's algorithmic bytes (K/V [+ fp8 scales] of every
           attended token, q, out, block-table entries, lengths, and the
           appended K/V row) divided by the whole call's average duration
           (attention kernel + partition merge), from HIP events on the launch
           stream around each step's run of consecutive layer calls (from its
           second call on, so that the GPU is already busy when the first
           event fires); the attention kernel alone is reported beside it.
cpu_baseline = the fp64 oracle (test infrastructure) timed on the host over a
           bounded sample of the same workload: single-sequence decodes
           through the oracle's paged pool, block-table gather and widening
           to fp64 inside the timed region.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention KV tokens/s and achieved HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 * 2 ** 20
ES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1}
# cache format -> (bytes per K element, bytes per V element, float32 scales per (token, head) and tensor)
KV_BYTES = {"f32": (4, 4, 0), "f16": (2, 2, 0), "bf16": (2, 2, 0), "fp8_e4m3": (1, 1, 1), "fp8_e5m2": (1, 1, 1),
            "int8_int4": (1, 0.5, 1)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2: Llama-3-8B shape, bf16)")
    ap.add_argument("--layers", type=int, default=0, help="pools to rotate (0 = 32, or at least 4 and enough for 4x the MALL)")
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (counter calibration) and exit")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV", "CAL_WRITE_CSV"),
                    help="from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of this bench and of "
                         "--calibrate-copy, write profiles/decode_<workload>_traffic.json and exit")
    ap.add_argument("--probe-read", action="store_true",
                    help="only measure a cold HBM reference (device-to-device copies of 128 MiB, 256 MiB of "
                         "traffic per launch, rotating through 16 slices of a 2 GiB source) and exit")
    ap.add_argument("--unfused", action="store_true",
                    help="write the step's rows with kv_cache_append, then attend (default: the write is fused "
                         "into the attention kernel)")
    ap.add_argument("--row", choices=["decode", "prefix", "prefill", "swap"], default="decode",
                    help="decode (default): the hot path; prefix: host prefix-cache replay of agent sessions; "
                         "prefill: multi-token append + chunked prefill attention; swap: sequences to host "
                         "memory and back")
    ap.add_argument("--cache", default=None,
                    help="decode and prefill rows: cache format to run with instead of the workload's own "
                         "(fp8_e4m3, fp8_e5m2, int8_int4, ...; K/V rows stay in the workload's dtype)")
    ap.add_argument("--block-size", type=int, choices=[16, 32], default=16,
                    help="decode row: tokens per block (32: the same workload on 32-token blocks)")
    ap.add_argument("--swap-mode", choices=["overlapped", "sequential"], default="overlapped",
                    help="swap row: out and in on two streams at once (PagedKVCache.swap), or one after the other")
    ap.add_argument("--swap-ahead", type=int, default=1,
                    help="swap row, overlapped mode: the host waits for the GPU after every N steps (default 1: "
                         "after each step, as a scheduler does; 0: never inside the timed loop)")
    ap.add_argument("--cached", type=int, default=3584, help="prefill row: cached tokens per sequence")
    ap.add_argument("--chunk", type=int, default=512, help="prefill row: chunk tokens per sequence")
    ap.add_argument("--split", action="store_true",
                    help="time the split form (paged_attention_decode_append_partials, then "
                         "paged_attention_merge_partials: the merge as a second launch) instead of the one-call "
                         "paged_attention_decode_append (one launch; the last partition of a sequence merges)")
    return ap.parse_args()


def source_digest() -> str:
    """Digest of the decode kernel's code (line comments and blank lines
    dropped, so that editing a comment keeps a counter record valid)."""
    h = hashlib.sha256()
    for name in ("decode.hip", "device_common.h", "launch.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_160_amd", "csrc", name), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def percentiles(times_us):
    t = sorted(times_us)
    n = len(t)
    return {"median_us": t[n // 2], "p10_us": t[n // 10], "p90_us": t[min(n - 1, (9 * n) // 10)], "n": n}


def load_traffic(workload_name: str):
    """HBM bytes per decode launch from a committed rocprofv3 counter summary,
    if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"decode_{workload_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def write_traffic(args):
    """HBM bytes per decode call from counter CSVs, each counter scaled by what
    it reads for a 1 GiB device copy (reads 1 GiB, writes 1 GiB)."""
    import csv
    import statistics

    import workloads as wl

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    def per_kernel(path, key):
        vals = [float(r["Counter_Value"]) for r in rows(path) if key in r["Kernel_Name"]]
        return statistics.median(vals) if vals else 0.0, len(vals)

    fetch_csv, write_csv, cal_fetch_csv, cal_write_csv = args.write_traffic
    gib_kib = float(2 ** 20)
    # the device-to-device copy runs as the runtime's copyBuffer kernel
    cal_f = statistics.median(float(r["Counter_Value"]) for r in rows(cal_fetch_csv)
                              if "copyBuffer" in r["Kernel_Name"])
    cal_w = statistics.median(float(r["Counter_Value"]) for r in rows(cal_write_csv)
                              if "copyBuffer" in r["Kernel_Name"])
    f_scale, w_scale = gib_kib / cal_f, gib_kib / cal_w
    rec = {"workload": wl.make_workload(args.config).name, "source_digest": source_digest(),
           "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    total = 0.0
    for key in ("paged_decode_kernel", "partition_merge_kernel"):
        fk, n = per_kernel(fetch_csv, key)
        wk, _ = per_kernel(write_csv, key)
        b = (fk * f_scale + wk * w_scale) * 1024.0
        rec["kernels"][key] = {"dispatches": n, "fetch_kib_raw": fk, "write_kib_raw": wk, "hbm_bytes": b}
        total += b
    rec["bytes_per_launch"] = total
    out = os.path.join(ROOT, "profiles", f"decode_{rec['workload']}_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=2)
    print(json.dumps(rec))


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(sharding by sequence or KV head needs no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    if args.row == "prefix":
        run_prefix_row(args)
        return
    if args.row == "prefill":
        run_prefill_row(args)
        return
    if args.row == "swap":
        run_swap_row(args)
        return

    import numpy as np
    import torch

    if args.calibrate_copy:
        # HBM-counter calibration: a copy of known size (reads and writes
        # 1 GiB per launch); FETCH_SIZE / WRITE_SIZE per dispatch of this
        # kernel divided by 1 GiB gives the counters' scale.
        src = torch.ones(2 ** 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copies done: 5 x 1 GiB")
        return

    if args.probe_read:
        # Reference for the per-launch cold HBM rate of this GPU at the size of
        # one 8B-shape decode layer: device-to-device copies of 128 MiB
        # (256 MiB of traffic per launch) rotating through 16 slices of a
        # 2 GiB source, so no slice is cache-resident.
        n = 2 ** 27
        src = torch.ones(16 * n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        res = []
        for r in range(48):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src[(r % 16) * n:(r % 16 + 1) * n])
            e1.record()
            res.append((e0, e1))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) * 1e3 for a, b in res[16:])
        med = t[len(t) // 2]
        log(f"[bench] cold 128 MiB copy (256 MiB traffic): median {med:.1f} us -> {2 * n / med / 1e3:.0f} GB/s")
        print(json.dumps({"probe": "cold_copy_128MiB", "median_us": med, "gbps": 2 * n / med / 1e3}))
        return

    import workloads as wl
    import paged_kv_cache_160_amd as pkv
    from paged_kv_cache_160_amd.cache import PagedKVCache
    from paged_kv_cache_160_amd.workload_runner import TORCH_DTYPES, to_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.with_block_size(wl.make_workload(args.config), args.block_size)
    bs = w.block_size
    B, hq, hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    if args.cache:
        if args.cache not in KV_BYTES:
            raise SystemExit(f"unknown cache format {args.cache}")
        w.cache_dtype = args.cache
        if args.cache not in ("f32", "f16", "bf16"):
            w.q_dtype = "bf16" if w.q_dtype == "f32" else w.q_dtype
        else:
            w.src_dtype = w.q_dtype = args.cache
        w.name = f"{w.name}-{args.cache}"
    kb_el, vb_el, nscale = KV_BYTES[w.cache_dtype]
    per_layer_bytes = int(w.num_blocks * hkv * bs * (D * (kb_el + vb_el) + 8 * nscale))
    layers = args.layers or (32 if args.config == 2 else max(4, math.ceil(4 * MALL_BYTES / per_layer_bytes)))
    log(f"[bench] workload {args.config} {w.name}: B={B} Hq={hq} Hkv={hkv} D={D} cache={w.cache_dtype} "
        f"layers={layers} pool={w.num_blocks} blocks/layer ({per_layer_bytes / 2**30:.2f} GiB/layer)")

    cache = PagedKVCache(layers, w.num_blocks, hkv, D, w.cache_dtype, w.max_blocks_per_seq,
                         device=dev, block_size=bs)
    gen = torch.Generator(device=dev)
    src_t = TORCH_DTYPES[w.src_dtype]

    def gpu_rows(n, seed):
        gen.manual_seed(seed)
        return torch.randn((n, hkv, D), generator=gen, device=dev, dtype=torch.float32).to(src_t)

    # ---- setup: the workload's allocator script; layer 0 holds the seeded
    # workload rows, the other layers seeded device-generated rows of the same
    # distribution
    t0 = time.perf_counter()
    for op in wl.setup_ops(w):
        kind = op[0]
        if kind == "free_order":
            cache.set_free_order(op[1])
        elif kind == "create":
            cache.create(op[1])
        elif kind == "fork":
            cache.fork(op[1], op[2])
        elif kind == "free":
            cache.free(op[1])
        elif kind == "append":
            seq, n = op[1], op[2]
            if seq >= wl.CHURN_ID_BASE:
                cache.alloc.append_slots(seq, n)
                continue
            start = cache.seq_len(seq)
            k0 = to_device(wl.kv_rows(w, seq, "k")[start:start + n], w.src_dtype, dev)
            v0 = to_device(wl.kv_rows(w, seq, "v")[start:start + n], w.src_dtype, dev)
            ks = [k0] + [gpu_rows(n, 7919 * (l + 1) + 2 * seq) for l in range(1, layers)]
            vs = [v0] + [gpu_rows(n, 7919 * (l + 1) + 2 * seq + 1) for l in range(1, layers)]
            cache.append(seq, ks, vs)
    torch.cuda.synchronize()
    log(f"[bench] setup {time.perf_counter() - t0:.1f}s; stats {cache.alloc.stats()}")

    seqs = list(range(B))
    n_steps = args.warmup + args.steps
    qt = TORCH_DTYPES[w.q_dtype]
    gen.manual_seed(12345)
    qs = torch.randn((n_steps, layers, B, hq, D), generator=gen, device=dev).to(qt)
    knew = torch.randn((n_steps, layers, B, hkv, D), generator=gen, device=dev).to(src_t)
    vnew = torch.randn((n_steps, layers, B, hkv, D), generator=gen, device=dev).to(src_t)
    outs = torch.empty((layers, B, hq, D), dtype=qt, device=dev)

    mb = w.max_blocks_per_seq
    # one set of pinned host buffers per step: an async copy may still be
    # queued behind the previous step's kernels when the host moves on
    h_tables = [torch.zeros((B, mb), dtype=torch.int32).pin_memory() for _ in range(n_steps)]
    h_lens = [torch.zeros(B, dtype=torch.int32).pin_memory() for _ in range(n_steps)]
    h_slots = [torch.zeros(B, dtype=torch.int64).pin_memory() for _ in range(n_steps)]
    d_tables = torch.zeros((B, mb), dtype=torch.int32, device=dev)
    d_lens = torch.zeros(B, dtype=torch.int32, device=dev)
    d_slots = torch.zeros(B, dtype=torch.int64, device=dev)
    max_possible = max(w.context_lens) + n_steps
    ws = torch.zeros(max(1, pkv.workspace_size(B, hq, hkv, D, max_possible, args.partition_size,
                                               cache.cache_code)), dtype=torch.uint8, device=dev)
    ps_used, np_used = pkv.decode_partition_size(B, hq, hkv, D, max(w.context_lens) + 1,
                                                 cache.cache_code)
    if args.partition_size:
        ps_used = args.partition_size
    stream = torch.cuda.current_stream()
    # One event pair per timed step, around its calls 1 .. layers-1 (the first
    # is queued ahead of the first event): per-call times are the span divided
    # by the calls in it, so no event sits between two calls of the run.
    step_ev = {s_: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for s_ in range(args.warmup, n_steps)}
    tokens_timed = 0
    bytes_timed = 0

    # Raw C-ABI calls with precomputed arguments: the timed loop enqueues
    # 2 * layers launches per step and Python must stay ahead of the GPU.
    lib = pkv._lib.lib()
    sp = stream.cuda_stream
    src_code = pkv.dtype_code(src_t)
    cache_code = cache.cache_code
    q_code = pkv.dtype_code(qt)
    scale = 1.0 / math.sqrt(D)
    kv_stride = knew[0, 0].numel() * knew.element_size()
    q_stride = qs[0, 0].numel() * qs.element_size()
    out_stride = outs[0].numel() * outs.element_size()
    ptr = lambda t: None if t is None else t.data_ptr()
    pools = [(ptr(cache.k[l]), ptr(cache.v[l]), ptr(cache.k_scale[l]), ptr(cache.v_scale[l]))
             for l in range(layers)]
    ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()

    def attend(s, l, max_len):
        """Layer l's attention kernel of step s: the one-call form (cache write
        fused, partitions merged in the same launch) by default; the split
        form's first launch with --split, without the cache write with
        --unfused (kv_cache_append wrote the rows already)."""
        kp, vp, ksp, vsp = pools[l]
        kl = knew.data_ptr() + (s * layers + l) * kv_stride
        vl = vnew.data_ptr() + (s * layers + l) * kv_stride
        o_ptr = outs.data_ptr() + l * out_stride
        q_ptr = qs.data_ptr() + (s * layers + l) * q_stride
        if not args.split and not args.unfused:
            rc = lib.paged_attention_decode_append_bs(o_ptr, q_ptr, kl, vl, kp, vp, ksp, vsp,
                                                      d_slots.data_ptr(), d_tables.data_ptr(), d_lens.data_ptr(),
                                                      B, hq, hkv, D, w.num_blocks, bs, mb, max_len, scale,
                                                      q_code, src_code, cache_code, args.partition_size,
                                                      ws_ptr, ws_bytes, sp)
            if rc:
                raise pkv.PagedKVError(rc, "paged_attention_decode_append")
            return
        slot_ptr = None if args.unfused else d_slots.data_ptr()
        rc = lib.paged_attention_decode_append_partials_bs(o_ptr, q_ptr, kl, vl, kp, vp, ksp, vsp, slot_ptr,
                                                           d_tables.data_ptr(), d_lens.data_ptr(), B, hq, hkv,
                                                           D, w.num_blocks, bs, mb, max_len, scale, q_code,
                                                           src_code, cache_code, args.partition_size, ws_ptr,
                                                           ws_bytes, sp)
        if rc:
            raise pkv.PagedKVError(rc, "paged_attention_decode_append_partials")

    def merge(l, max_len):
        """Layer l's partition merge, split form only (nothing is launched when
        no sequence is split)."""
        if not args.split and not args.unfused:
            return
        o_ptr = outs.data_ptr() + l * out_stride
        rc = lib.paged_attention_merge_partials_bs(o_ptr, d_lens.data_ptr(), B, hq, hkv, D, bs, mb, max_len,
                                                   q_code, cache_code, args.partition_size, ws_ptr, ws_bytes, sp)
        if rc:
            raise pkv.PagedKVError(rc, "paged_attention_merge_partials")

    def step(s, timed):
        nonlocal tokens_timed, bytes_timed
        slots, pairs = cache.alloc.batch_append_one(seqs)
        h_slots[s].copy_(torch.tensor(slots, dtype=torch.int64))
        cache.alloc.block_tables(seqs, mb, out_tables=h_tables[s], out_lens=h_lens[s])
        d_slots.copy_(h_slots[s], non_blocking=True)
        d_tables.copy_(h_tables[s], non_blocking=True)
        d_lens.copy_(h_lens[s], non_blocking=True)
        if pairs:
            cache._apply_cow(pairs)
        lens = h_lens[s].tolist()
        max_len = max(lens)
        sum_l = sum(lens)
        if args.unfused:
            for l in range(layers):
                kp, vp, ksp, vsp = pools[l]
                kl = knew.data_ptr() + (s * layers + l) * kv_stride
                vl = vnew.data_ptr() + (s * layers + l) * kv_stride
                rc = lib.kv_cache_append_bs(kl, vl, kp, vp, ksp, vsp, d_slots.data_ptr(), B, hkv, D,
                                            w.num_blocks, bs, src_code, cache_code, sp)
                if rc:
                    raise pkv.PagedKVError(rc, "kv_cache_append")
        e = step_ev.get(s) if timed else None
        for l in range(layers):
            if e and l == 1:
                # the events bracket calls 1 .. layers-1: the step's first call
                # is queued ahead, so the GPU is busy when the first event
                # fires and no host-side launch latency enters the span
                e[0].record(stream)
            attend(s, l, max_len)
            merge(l, max_len)
        if e:
            e[1].record(stream)
        if timed:
            tokens_timed += sum_l * layers
            kv_bytes = sum_l * hkv * (D * (kb_el + vb_el) + 8 * nscale)
            qo_bytes = 2 * B * hq * D * ES[w.q_dtype]
            table_bytes = sum(-(-L // bs) for L in lens) * 4 + B * 4
            # the fused call also reads the new rows and slots (its writes are
            # inside the K/V bytes already counted)
            new_bytes = 0 if args.unfused else B * hkv * D * 2 * ES[w.src_dtype] + B * 8
            bytes_timed += (kv_bytes + qo_bytes + table_bytes + new_bytes) * layers
        return max_len

    for s in range(args.warmup):
        step(s, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.warmup, n_steps):
        last_max_len = step(s, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_call_us = [a.elapsed_time(b) * 1e3 / (layers - 1) for a, b in step_ev.values()]
    call_s = sum(per_call_us) / len(per_call_us) / 1e6
    calls = args.steps * layers
    bytes_per_call = bytes_timed / calls
    achieved = bytes_per_call / call_s / 1e9
    value = tokens_timed / elapsed
    call_pct = percentiles(per_call_us)
    log(f"[bench] {args.steps} steps in {elapsed * 1e3:.2f} ms; whole decode call {call_s * 1e6:.2f} us "
        f"(runs of {layers} consecutive calls, {achieved:.0f} GB/s algorithmic, "
        f"{100 * achieved / HBM_PEAK_GBPS:.1f}% of peak); {value / 1e9:.3f} G KV tokens/s")

    # The two kernels of the call apart (after the timed region, last step's
    # arguments): runs of `layers` consecutive attention kernels, then of
    # merges, one event pair around each run's calls after its first.
    def time_runs(fn, reps=10):
        spans = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            fn(0)
            e0.record(stream)
            for l in range(1, layers):
                fn(l)
            e1.record(stream)
            spans.append((e0, e1))
        torch.cuda.synchronize()
        return percentiles([a.elapsed_time(b) * 1e3 / (layers - 1) for a, b in spans])

    last_s = n_steps - 1
    kern_pct = time_runs(lambda l: attend(last_s, l, last_max_len))
    split = (args.split or args.unfused) and ps_used < last_max_len
    merge_pct = time_runs(lambda l: merge(l, last_max_len)) if split else None
    kern_s = kern_pct["median_us"] / 1e6
    log(f"[bench] attention kernel alone: median {kern_pct['median_us']:.2f} us per call "
        f"({bytes_per_call / kern_s / 1e9:.0f} GB/s)"
        + (f"; merge kernel alone: median {merge_pct['median_us']:.2f} us" if merge_pct else ""))
    traffic = load_traffic(w.name)

    # Side measurements after the timed region (not part of the value): the
    # decode step's cache write on its own (B rows into layer 0, the slots of
    # the last step) and a copy-on-write copy of up to 8 used blocks into
    # free blocks, 100 calls each, HIP events around every call.
    def time_calls(fn, n=100):
        evs_ = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc_ = fn()
            e1.record(stream)
            if rc_:
                raise pkv.PagedKVError(rc_, "side measurement")
            evs_.append((e0, e1))
        torch.cuda.synchronize()
        return percentiles([a.elapsed_time(b) * 1e3 for a, b in evs_])

    kp0, vp0, ksp0, vsp0 = pools[0]
    side = {"append_b_rows": time_calls(lambda: lib.kv_cache_append_bs(
        knew.data_ptr(), vnew.data_ptr(), kp0, vp0, ksp0, vsp0, d_slots.data_ptr(), B, hkv, D, w.num_blocks, bs,
        src_code, cache_code, sp))}
    used_tables, used_lens = cache.alloc.block_tables(seqs, mb)
    used = sorted(set(int(used_tables[b_, i]) for b_ in range(B) for i in range(-(-int(used_lens[b_]) // bs))))
    free_blocks = [blk for blk in range(w.num_blocks) if blk not in set(used)]
    n_pairs = min(8, len(used), len(free_blocks))
    if n_pairs:
        pairs_t = torch.tensor([[used[i], free_blocks[i]] for i in range(n_pairs)], dtype=torch.int32, device=dev)
        side[f"cow_copy_{n_pairs}_blocks"] = time_calls(lambda: lib.pkv_copy_blocks_bs(
            kp0, vp0, ksp0, vsp0, pairs_t.data_ptr(), n_pairs, hkv, D, w.num_blocks, bs, cache_code, sp))
    for k_, v_ in side.items():
        log(f"[bench] {k_}: median {v_['median_us']:.2f} us (p10 {v_['p10_us']:.2f}, p90 {v_['p90_us']:.2f}), "
            f"events around each call")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.cache_dtype,
        "data": "synthetic (seeded N(0,1) K/V/q; no weights or datasets)",
        "config": {
            "workload": f"{w.name} (paged decode, one layer per call)",
            "batch": B, "context_len_first_timed_step": max(w.context_lens) + args.warmup + 1,
            "q_heads": hq, "kv_heads": hkv, "head_dim": D, "block_size": bs, "kv_dtype": w.cache_dtype,
            "q_dtype": w.q_dtype, "layers_rotated": layers, "pool_blocks_per_layer": w.num_blocks,
            "partition_size": ps_used, "parallelism": "none (1 GPU)",
        },
        "achieved_hbm_gbps": achieved,
        "pct_of_peak": 100.0 * achieved / HBM_PEAK_GBPS,
        "decode_call_us": call_s * 1e6,
        "decode_call_us_percentiles": call_pct,
        "attention_kernel_us_percentiles": kern_pct,
        "attention_kernel_hbm_gbps": bytes_per_call / kern_s / 1e9,
        "merge_kernel_us_percentiles": merge_pct,
        "side_kernels_us": side,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
            "kernel": ("whole decode call: paged_decode_kernel" + ("" if args.unfused else " (cache write fused)")
                       + (" + partition_merge_kernel" if split else
                          (", partitions merged in the same launch" if ps_used < last_max_len else ""))),
            "timing": f"HIP events around calls 2..{layers} of each step's {layers} consecutive calls on the "
                      f"launch stream (the first queued ahead), {args.steps} runs; per-call time = span / "
                      f"{layers - 1}",
            "bytes_per_launch": bytes_per_call,
            "attention_kernel_alone": {"us": kern_s * 1e6, "achieved": bytes_per_call / kern_s / 1e9,
                                       "frac": bytes_per_call / kern_s / 1e9 / HBM_PEAK_GBPS},
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(w, budget_s: float):
    """The fp64 oracle on the host, decoding through its own paged pool: the
    workload's setup script builds the oracle's allocator and pool (not
    timed); then single-sequence decodes of layer 0, cycling over the batch,
    are timed until the budget is spent.  Each decode gathers the sequence's
    K/V through its block table, widens (dequantises) them to fp64 and
    attends - the paged work the GPU call does."""
    import numpy as np
    import psutil
    from threadpoolctl import threadpool_info, threadpool_limits

    import workloads as wl
    from oracle import attention, scenario

    scale = 1.0 / math.sqrt(w.head_dim)
    q = wl.queries(w, 0)
    # the sample: the first sequences up to 65536 tokens (32768 for quantised
    # caches, whose rows the oracle quantises one by one while building)
    cap = 32768 if w.cache_dtype not in ("f32", "f16", "bf16") else 65536
    seqs = []
    for b in range(w.num_seqs):
        if seqs and sum(w.context_lens[x] for x in seqs) + w.context_lens[b] > cap:
            break
        seqs.append(b)
    t_setup = time.perf_counter()
    st = scenario.OracleState(w, build_pool=True, pool_seqs=set(seqs)).run(wl.setup_ops(w))
    tables, lens = st.tables(seqs)
    log(f"[cpu] oracle pool built in {time.perf_counter() - t_setup:.1f}s (not timed)")

    def run(limit_s):
        t0_ = time.perf_counter()
        tokens_, done_ = 0, 0
        while True:
            i = done_ % len(seqs)
            b = seqs[i]
            attention.decode_paged(q[b:b + 1], st.pool, tables[i:i + 1], lens[i:i + 1], scale)
            tokens_ += int(lens[i])
            done_ += 1
            if time.perf_counter() - t0_ >= limit_s and done_ >= 1:
                return tokens_, done_, time.perf_counter() - t0_

    proc = psutil.Process()
    c0 = proc.cpu_times()
    tokens, seqs_done, wall = run(budget_s)
    c1 = proc.cpu_times()
    busy = (c1.user - c0.user + c1.system - c0.system) / wall
    blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
    allowed = len(os.sched_getaffinity(0))
    log(f"[cpu] oracle: {seqs_done} sequence decodes, {tokens} KV tokens in {wall:.1f}s "
        f"({tokens / wall / 1e6:.2f} M KV tokens/s), {busy:.1f} cores busy on average")
    with threadpool_limits(limits=1):
        tokens1, done1, wall1 = run(min(3.0, budget_s))
    log(f"[cpu] oracle on one thread: {done1} sequence decodes, {tokens1 / wall1 / 1e6:.2f} M KV tokens/s")
    return {
        "value": tokens / wall, "unit": "KV tokens/s", "cores": max(1, round(busy)),
        "kind": "oracle",
        "sample": (f"{seqs_done} single-sequence decodes (all {w.num_q_heads} query heads) of layer 0 of "
                   f"{w.name}, cycling over its first {len(seqs)} sequences ({sum(int(x) for x in lens)} tokens), through the oracle's paged pool: "
                   f"block-table gather, widening to fp64 and attention timed; fp64 numpy; "
                   f"{busy:.2f} cores busy on average, {allowed} allowed, BLAS threads {blas}"),
        "single_thread_value": tokens1 / wall1,
        "single_thread_sample": f"{done1} of the same decodes with BLAS limited to one thread",
    }


# ---- chunked prefill row ------------------------------------------------------------

MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_flops(cached, chunk, hq, d):
    """Algorithmic flops of one prefill call: query i of a chunk at position
    p = cached + i meets p + 1 keys, 2*d flops each for q.k and for p*v."""
    total = 0
    for c, n in zip(cached, chunk):
        keys = n * c + n * (n + 1) // 2
        total += 4 * d * hq * keys
    return total


def run_prefill_row(args, lib=None):
    """Multi-token append + chunked prefill on the Llama-3-8B layer shape
    (32 query heads, 8 KV heads, D=128, bf16): 16 sequences, each holding
    ``--cached`` tokens and appending a chunk of ``--chunk`` more (3584 + 512
    = 4096 by default).  One step = for every layer: kv_cache_append of the
    chunks' K/V rows (one multi-token append), then paged_attention_prefill.
    Pools hold seeded device-generated N(0,1) rows; several layers rotate so
    that K/V are read from HBM."""
    import numpy as np
    import torch

    import paged_kv_cache_160_amd as pkv
    from paged_kv_cache_160_amd.cache import PagedKVCache

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = lib or pkv._lib.lib()
    B, hq, hkv, D = 16, 32, 8, 128
    fmt = args.cache or "bf16"
    if fmt not in KV_BYTES or fmt in ("f32", "f16"):
        raise SystemExit(f"prefill row: cache format {fmt} not taken (bf16 queries)")
    kb_el, vb_el, nscale = KV_BYTES[fmt]
    cached, chunk = [args.cached] * B, [args.chunk] * B
    L = args.cached + args.chunk
    nb = int(math.ceil(1.1 * B * -(-L // 16)))
    mb = -(-L // 16) + 1
    layer_bytes = int(nb * hkv * 16 * (D * (kb_el + vb_el) + 8 * nscale))
    layers = args.layers or max(2, math.ceil(4 * MALL_BYTES / layer_bytes))
    log(f"[prefill] B={B} cached={args.cached} chunk={args.chunk} Hq={hq} Hkv={hkv} D={D} q bf16, cache {fmt}, "
        f"{layers} layers x {layer_bytes / 2**30:.2f} GiB")
    cache = PagedKVCache(layers, nb, hkv, D, fmt, mb, device=dev)
    cache.set_free_order(np.random.default_rng(2025).permutation(nb).astype(np.int32))
    gen = torch.Generator(device=dev)
    gen.manual_seed(99)
    ctx_slots, chunk_slots = [], []
    for b in range(B):
        cache.create(b)
        slots, _ = cache.alloc.append_slots(b, args.cached)  # the cached context, written once below
        ctx_slots += slots
        slots, _ = cache.alloc.append_slots(b, args.chunk)  # the chunk: its rows are written every step
        chunk_slots += slots
    # the cached context: seeded N(0,1) rows through the cache write (quantised for quantised formats)
    ctx_t = torch.tensor(ctx_slots, dtype=torch.int64, device=dev)
    for l in range(layers):
        krow = torch.randn((len(ctx_slots), hkv, D), generator=gen, device=dev).to(torch.bfloat16)
        vrow = torch.randn((len(ctx_slots), hkv, D), generator=gen, device=dev).to(torch.bfloat16)
        pkv.kv_cache_append(krow, vrow, cache.k[l], cache.v[l], ctx_t, cache.k_scale[l], cache.v_scale[l])
        del krow, vrow
    torch.cuda.synchronize()
    seqs = list(range(B))
    tables, lens, max_len = cache.block_tables(seqs)
    T = sum(chunk)
    slot_t = torch.tensor(chunk_slots, dtype=torch.int64, device=dev)
    qs_t = torch.tensor(np.concatenate([[0], np.cumsum(chunk)]), dtype=torch.int32, device=dev)
    n_steps = args.warmup + args.steps
    q = torch.randn((layers, T, hq, D), generator=gen, device=dev).to(torch.bfloat16)
    knew = torch.randn((layers, T, hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    vnew = torch.randn((layers, T, hkv, D), generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty((layers, T, hq, D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    code = pkv.dtype_code(torch.bfloat16)
    ccode = cache.cache_code
    ptr = lambda t: None if t is None else t.data_ptr()
    scale = 1.0 / math.sqrt(D)
    flops = prefill_flops(cached, chunk, hq, D)
    ev = {(s_, l): tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
          for s_ in range(args.warmup, n_steps) for l in range(layers)}

    def step(s, timed):
        for l in range(layers):
            e = ev.get((s, l)) if timed else None
            if e:
                e[0].record(stream)
            rc = lib.kv_cache_append(knew[l].data_ptr(), vnew[l].data_ptr(), cache.k[l].data_ptr(),
                                     cache.v[l].data_ptr(), ptr(cache.k_scale[l]), ptr(cache.v_scale[l]),
                                     slot_t.data_ptr(), T, hkv, D, nb, code, ccode, sp)
            if rc:
                raise pkv.PagedKVError(rc, "kv_cache_append")
            if e:
                e[1].record(stream)
            rc = lib.paged_attention_prefill(out[l].data_ptr(), q[l].data_ptr(), cache.k[l].data_ptr(),
                                             cache.v[l].data_ptr(), ptr(cache.k_scale[l]), ptr(cache.v_scale[l]),
                                             tables.data_ptr(), lens.data_ptr(), qs_t.data_ptr(), B, T, hq, hkv, D,
                                             nb, mb, max_len, max(chunk), scale, code, ccode, sp)
            if rc:
                raise pkv.PagedKVError(rc, "paged_attention_prefill")
            if e:
                e[2].record(stream)

    for s in range(args.warmup):
        step(s, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.warmup, n_steps):
        step(s, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    app_s = sum(a.elapsed_time(b) for a, b, _ in ev.values()) / len(ev) / 1e3
    pf_s = sum(b.elapsed_time(c) for _, b, c in ev.values()) / len(ev) / 1e3
    calls = args.steps * layers
    achieved = flops / pf_s / 1e12
    value = flops * calls / elapsed / 1e12
    kv_bytes = B * L * hkv * (D * (kb_el + vb_el) + 8 * nscale)
    log(f"[prefill] {args.steps} steps x {layers} layers in {elapsed * 1e3:.2f} ms; append {app_s * 1e6:.1f} us, "
        f"prefill {pf_s * 1e6:.1f} us = {achieved:.1f} TFLOP/s ({100 * achieved / MFMA_BF16_PEAK_TFLOPS:.1f}% of "
        f"bf16 MFMA peak); K/V read {kv_bytes / pf_s / 1e9:.0f} GB/s")
    rec = {
        "metric": "chunked prefill attention over the paged cache, TFLOP/s (algorithmic, causal), 1 GPU",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": fmt, "data": "synthetic (seeded N(0,1) K/V/q)",
        "config": {"workload": f"llama3-8b-shape chunked prefill: 16 x ({args.cached} cached + {args.chunk} new)"
                               + ("" if fmt == "bf16" else f", {fmt} cache"),
                   "q_heads": hq, "kv_heads": hkv, "head_dim": D, "block_size": 16, "layers_rotated": layers},
        "append_us": app_s * 1e6, "prefill_kernel_us": pf_s * 1e6,
        "chunk_tokens_per_s": T * calls / elapsed,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None, "kernel": "paged_prefill_kernel",
                     "flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = prefill_cpu_baseline(args, hq, hkv, D, args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return rec


def prefill_cpu_baseline(args, hq, hkv, D, budget_s):
    """The fp64 oracle (test infrastructure): chunk rows of one sequence with
    the same context length, timed until the budget is spent."""
    import numpy as np

    from oracle import prefill

    import psutil

    rng = np.random.default_rng(5)
    L = args.cached + args.chunk
    K = rng.standard_normal((L, hkv, D))
    V = rng.standard_normal((L, hkv, D))
    q = rng.standard_normal((args.chunk, hq, D))
    proc = psutil.Process()
    c0 = proc.cpu_times()
    t0 = time.perf_counter()
    done = flops = 0
    step = 8
    while True:
        i0 = (done * step) % args.chunk
        n = min(step, args.chunk - i0)
        # rows i0 .. i0+n-1 of the chunk: pass the rows up to the last one's position
        prefill.prefill_rows(q[i0:i0 + n], K[:args.cached + i0 + n], V[:args.cached + i0 + n], 1.0 / math.sqrt(D))
        flops += prefill_flops([args.cached + i0], [n], hq, D)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    wall = time.perf_counter() - t0
    c1 = proc.cpu_times()
    busy = (c1.user - c0.user + c1.system - c0.system) / wall
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": max(1, round(busy)), "kind": "oracle",
            "sample": f"{done} slices of {step} chunk rows (all {hq} heads, contexts {args.cached}..{L}), "
                      f"fp64 numpy, {busy:.2f} cores busy on average"}


# ---- swap row --------------------------------------------------------------------------

def run_swap_row(args):
    """Sequence swap on the Llama-3-8B layer shape ("KV Cache 和 vLLM" §6.2):
    32 layers of bf16 pools holding 16 sequences of 4096 tokens (the decode
    workload's state); one step swaps 4 sequences out (per sequence: 64
    gathers - 32 layers x K/V - into one device staging buffer, then one
    device -> pinned-host copy) and back in (one host -> staging copy, 64
    scatters into fresh blocks).  Each leg is timed with HIP events."""
    import numpy as np
    import torch

    import paged_kv_cache_160_amd as pkv
    import workloads as wl
    from paged_kv_cache_160_amd.cache import PagedKVCache

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = pkv._lib.lib()
    w = wl.make_workload(2)
    B, hkv, D = w.num_seqs, w.num_kv_heads, w.head_dim
    layers = args.layers or 32
    n_swap = 4
    cache = PagedKVCache(layers, w.num_blocks, hkv, D, "bf16", w.max_blocks_per_seq, device=dev)
    cache.set_free_order(w.free_order)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    for l in range(layers):
        cache.k[l].normal_(generator=gen)
        cache.v[l].normal_(generator=gen)
    for b in range(B):
        cache.create(b)
        cache.alloc.append_slots(b, w.context_lens[b])
    nblk = -(-w.context_lens[0] // 16)
    tensors = cache._tensors()
    block_bytes = tensors[0][0].numel() * tensors[0].element_size()
    seq_bytes = nblk * block_bytes * len(tensors)
    staging = torch.empty(seq_bytes, dtype=torch.uint8, device=dev)
    host = [torch.empty(seq_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(n_swap)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    log(f"[swap] {layers} layers, {B} x {w.context_lens[0]} tokens, swapping {n_swap} sequences of "
        f"{seq_bytes / 2**20:.0f} MiB ({len(tensors)} pool tensors x {nblk} blocks x {block_bytes} B)")

    def leg_out(b, h, ev):
        blocks = cache.alloc.swap_out(b)
        bt = torch.tensor(blocks, dtype=torch.int32).to(dev)
        ev[0].record(stream)
        for t_i, t in enumerate(tensors):
            rc = lib.pkv_gather_blocks(staging.data_ptr() + t_i * nblk * block_bytes, t.data_ptr(), bt.data_ptr(),
                                       nblk, block_bytes, w.num_blocks, sp)
            if rc:
                raise pkv.PagedKVError(rc, "pkv_gather_blocks")
        ev[1].record(stream)
        h.copy_(staging, non_blocking=True)
        ev[2].record(stream)

    def leg_in(b, h, ev):
        blocks = cache.alloc.swap_in(b)
        bt = torch.tensor(blocks, dtype=torch.int32).to(dev)
        ev[0].record(stream)
        staging.copy_(h, non_blocking=True)
        ev[1].record(stream)
        for t_i, t in enumerate(tensors):
            rc = lib.pkv_scatter_blocks(t.data_ptr(), staging.data_ptr() + t_i * nblk * block_bytes, bt.data_ptr(),
                                        nblk, block_bytes, w.num_blocks, sp)
            if rc:
                raise pkv.PagedKVError(rc, "pkv_scatter_blocks")
        ev[2].record(stream)

    n_steps = args.warmup + args.steps
    if args.swap_mode == "overlapped":
        return run_swap_overlapped(args, cache, w, n_swap, seq_bytes, layers)
    evs = {(s_, i, d): tuple(torch.cuda.Event(enable_timing=True) for _ in range(3))
           for s_ in range(n_steps) for i in range(n_swap) for d in (0, 1)}
    t_start = None
    for s_ in range(n_steps):
        if s_ == args.warmup:
            torch.cuda.synchronize()
            t_start = time.perf_counter()
        for i in range(n_swap):
            leg_out(i, host[i], evs[(s_, i, 0)])
            # the staging buffer is reused: the copy to the host must finish first
            torch.cuda.current_stream().synchronize()
        for i in range(n_swap):
            leg_in(i, host[i], evs[(s_, i, 1)])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    timed = [(s_, i) for s_ in range(args.warmup, n_steps) for i in range(n_swap)]
    avg = lambda d, a, b: sum(evs[(s_, i, d)][a].elapsed_time(evs[(s_, i, d)][b]) for s_, i in timed) / len(timed) / 1e3
    log("[swap] step times (ms): " + " ".join(
        f"{evs[(s_, 0, 0)][0].elapsed_time(evs[(s_, n_swap - 1, 1)][2]):.1f}" for s_ in range(args.warmup, n_steps)))
    gather_s, d2h_s = avg(0, 0, 1), avg(0, 1, 2)
    h2d_s, scatter_s = avg(1, 0, 1), avg(1, 1, 2)
    gb = seq_bytes / 1e9
    log(f"[swap] per sequence ({gb:.3f} GB): gather {gather_s * 1e3:.2f} ms ({2 * gb / gather_s:.0f} GB/s HBM), "
        f"D2H {d2h_s * 1e3:.2f} ms ({gb / d2h_s:.1f} GB/s), H2D {h2d_s * 1e3:.2f} ms ({gb / h2d_s:.1f} GB/s), "
        f"scatter {scatter_s * 1e3:.2f} ms ({2 * gb / scatter_s:.0f} GB/s HBM)")
    swapped_tokens = args.steps * n_swap * w.context_lens[0]
    rec = {
        "metric": "sequence swap to host memory and back: KV tokens per second (round trip), 1 GPU",
        "value": swapped_tokens / elapsed, "unit": "KV tokens/s (out + in)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"llama3-8b-shape: {layers} layers x 16 x 4096 tokens, {n_swap} sequences "
                               f"swapped per step", "bytes_per_sequence": seq_bytes},
        "gather_ms": gather_s * 1e3, "d2h_ms": d2h_s * 1e3, "h2d_ms": h2d_s * 1e3, "scatter_ms": scatter_s * 1e3,
        "gather_hbm_gbps": 2 * gb / gather_s, "scatter_hbm_gbps": 2 * gb / scatter_s,
        "d2h_gbps": gb / d2h_s, "h2d_gbps": gb / h2d_s,
        "roofline": {"bound": "hbm", "achieved": 2 * gb / gather_s, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": 2 * gb / gather_s / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "swap_blocks_kernel (gather, 64 launches per sequence)",
                     "bytes_per_launch": 2 * seq_bytes / len(tensors)},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = swap_cpu_baseline(args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def run_swap_overlapped(args, cache, w, n_swap, seq_bytes, layers):
    """Steady-state swapping with both directions of the host link in use:
    the 16 sequences form 4 groups of ``n_swap``; step s swaps group s % 4
    out while the group swapped out one step earlier comes back in
    (PagedKVCache.swap: gathers and device -> host copies on one stream,
    host -> device copies and scatters on another).  One step moves
    ``n_swap`` sequences each way, the same bytes as one sequential step.
    The host waits for each step before it queues the next."""
    import torch

    B = w.num_seqs
    groups = [list(range(g * n_swap, (g + 1) * n_swap)) for g in range(B // n_swap)]
    held = {}
    # pinned buffers reused across steps: n_swap travelling out, n_swap held out
    free_bufs = [torch.empty(seq_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(2 * n_swap)]
    n_steps = args.warmup + args.steps
    stream = torch.cuda.current_stream()
    evs = []
    host_ms = []        # host time to queue each timed step (the runtime may block the caller)
    t_start = None
    for s_ in range(n_steps):
        if s_ == args.warmup:
            torch.cuda.synchronize()
            t_start = time.perf_counter()
        t_q = time.perf_counter()
        back = {x: held.pop(x) for x in groups[(s_ - 1) % len(groups)]} if s_ > 0 else {}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        outs = {x: free_bufs.pop() for x in groups[s_ % len(groups)]}
        held.update(cache.swap(groups[s_ % len(groups)], back, out_host=outs))
        e1.record(stream)
        if s_ >= args.warmup:
            host_ms.append((time.perf_counter() - t_q) * 1e3)
        # a scheduler step ends when its swaps are done (--swap-ahead N: the
        # host waits only after every N steps; a pinned buffer handed back is
        # reused only after the current stream has passed its copy, which
        # the stream order guarantees)
        if args.swap_ahead > 0 and (s_ + 1) % args.swap_ahead == 0:
            stream.synchronize()
        free_bufs += [buf for buf, _ in back.values()]
        if s_ >= args.warmup:
            evs.append((e0, e1))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    step_s = sum(a.elapsed_time(b) for a, b in evs) / len(evs) / 1e3
    log("[swap] step times (ms): " + " ".join(f"{a.elapsed_time(b):.1f}" for a, b in evs))
    log("[swap] host time to queue each step (ms): " + " ".join(f"{t:.1f}" for t in host_ms))
    gb = seq_bytes / 1e9
    link = 2 * n_swap * gb / step_s             # bytes over the host link per second, both directions
    log(f"[swap] overlapped: {args.steps} steps in {elapsed * 1e3:.1f} ms; per step {n_swap} sequences out and "
        f"{n_swap} in ({2 * n_swap * gb:.2f} GB over the host link) in {step_s * 1e3:.2f} ms = {link:.1f} GB/s")
    swapped_tokens = args.steps * n_swap * w.context_lens[0]
    rec = {
        "metric": "sequence swap to host memory and back: KV tokens per second (round trip), 1 GPU",
        "value": swapped_tokens / elapsed, "unit": "KV tokens/s (out + in)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"llama3-8b-shape: {layers} layers x 16 x 4096 tokens, {n_swap} sequences out and "
                               f"{n_swap} in per step, both directions at once", "bytes_per_sequence": seq_bytes},
        "step_ms_events": step_s * 1e3, "host_link_gbps_both_directions": link,
        "roofline": {"bound": "host link", "achieved": link, "peak": None, "unit": "GB/s", "frac": None,
                     "traffic": None, "kernel": "hipMemcpyAsync D2H + H2D (gathers and scatters beside them)"},
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = swap_cpu_baseline(args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return rec


def swap_cpu_baseline(budget_s: float):
    """The allocator model (test infrastructure) swapping the same sequences
    out and in: swap operations per second (the model moves no data)."""
    import workloads as wl
    from oracle.allocator import BlockAllocatorModel

    w = wl.make_workload(2)
    m = BlockAllocatorModel(w.num_blocks, w.max_blocks_per_seq)
    m.set_free_order(w.free_order)
    for b in range(w.num_seqs):
        m.create(b)
        m.append_slots(b, w.context_lens[b])
    t0 = time.perf_counter()
    ops = 0
    while time.perf_counter() - t0 < budget_s:
        for b in range(4):
            m.swap_out(b)
        for b in range(4):
            m.swap_in(b)
        ops += 8
    wall = time.perf_counter() - t0
    return {"value": ops / wall, "unit": "swap operations/s (allocator state only)", "cores": 1, "kind": "oracle",
            "sample": f"{ops} swap-outs and swap-ins of 4096-token sequences in the pure-Python allocator model"}


# ---- prefix caching row --------------------------------------------------------------

PREFIX_SHAPE = dict(n_sessions=32, turns=11, system_len=1000, user_len=400, output_len=100, vocab=32000)


def run_prefix_row(args):
    """Host prefix cache on agent sessions ("KV Cache优化实战" §5.1, §5.3).

    32 sessions on one 1000-token system prompt; every turn appends 400 user
    tokens to the session's history and generates 100, so the eleventh turn's
    prompt is 6400 tokens of which 5900 were seen the turn before (the pages'
    log: 6000-token requests, 5500 seen before).  Each turn: every session's
    request goes through the cache (lookup, then the missed prompt tokens are
    appended and indexed), then 100 decode steps append one token to every
    session at once; the turn's requests then finish.  Times are of the
    library calls alone (token buffers built beforehand).  The same stream is
    replayed with 8 tokens of per-request content after the first block (an
    unstable template, §5.3) for its hit fraction.  The pool holds 1.1x the
    last turn's live blocks."""
    import ctypes
    import numpy as np

    import paged_kv_cache_160_amd as pkv
    import workloads as wl
    from paged_kv_cache_160_amd import _lib

    lib = _lib.lib()
    res = {}
    for label, dyn in (("stable", 0), ("dynamic_head", 8)):
        turns = wl.agent_sessions(2024, dynamic_head=dyn, **PREFIX_SHAPE)
        last = max(len(t.prompt) + len(t.output) for t in turns)
        nb = int(1.1 * PREFIX_SHAPE["n_sessions"] * -(-last // 16))
        mbps = -(-last // 16) + 1
        a = pkv.BlockAllocator(nb, mbps)
        a.enable_prefix_cache(model_key=1)
        h = a._h
        slots = np.empty(last, np.int64)
        pair = np.empty(2, np.int32)
        bslots = np.empty(PREFIX_SHAPE["n_sessions"], np.int64)
        bpairs = np.empty(2 * PREFIX_SHAPE["n_sessions"], np.int32)
        ncow = ctypes.c_int()
        got = ctypes.c_int()
        P32, P64 = _lib.P_i32, _lib.P_i64
        row = np.empty(PREFIX_SHAPE["n_sessions"], np.int32)
        p_got, p_ncow = ctypes.byref(got), ctypes.byref(ncow)
        p_slots, p_pair = slots.ctypes.data_as(P64), pair.ctypes.data_as(P32)
        t_lookup = t_append = t_step = 0.0
        n_req = n_steps = 0
        prompt_tok = hit_tok = 0
        late_prompt = late_hit = 0
        for turn in range(PREFIX_SHAPE["turns"]):
            group = [t for t in turns if t.turn == turn]
            ids = np.array([1000 * turn + t.session for t in group], np.int64)
            prompts = [np.asarray(t.prompt, np.int32) for t in group]
            outs = np.stack([np.asarray(t.output, np.int32) for t in group], axis=1)   # [steps, sessions]
            # ctypes pointers are built before timing: making one costs more
            # than a whole batch step of the library
            p_ids, p_row, p_bs, p_bp = (ids.ctypes.data_as(P64), row.ctypes.data_as(P32),
                                        bslots.ctypes.data_as(P64), bpairs.ctypes.data_as(P32))
            p_prompts = [p.ctypes.data_as(P32) for p in prompts]
            for sid, p, pp in zip(ids, prompts, p_prompts):
                t0 = time.perf_counter()
                rc = lib.pkv_seq_create_cached(h, int(sid), pp, p.size, p_got)
                t1 = time.perf_counter()
                n = got.value
                p_rest = ctypes.cast(ctypes.addressof(pp.contents) + 4 * n, P32)
                t2 = time.perf_counter()
                rc |= lib.pkv_seq_append_tokens(h, int(sid), p_rest, p.size - n, p_slots, p_pair, p_ncow)
                t3 = time.perf_counter()
                if rc:
                    raise RuntimeError(f"allocator error {rc}")
                t_lookup += t1 - t0
                t_append += t3 - t2
                n_req += 1
                prompt_tok += p.size
                hit_tok += n
                if turn == PREFIX_SHAPE["turns"] - 1:
                    late_prompt += p.size
                    late_hit += n
            for j in range(outs.shape[0]):
                row[:] = outs[j]
                t0 = time.perf_counter()
                rc = lib.pkv_batch_append_tokens(h, p_ids, p_row, ids.size, p_bs, p_bp, p_ncow)
                t_step += time.perf_counter() - t0
                if rc:
                    raise RuntimeError(f"allocator error {rc}")
                n_steps += 1
            for sid in ids:
                a.free(int(sid))
        st = a.prefix_stats()
        res[label] = {
            "hit_fraction_all_turns": hit_tok / prompt_tok,
            "hit_fraction_last_turn": late_hit / late_prompt,
            "last_turn_prompt_tokens": late_prompt // len(ids),
            "last_turn_cached_tokens": late_hit // len(ids),
            "lookup_us_per_request": 1e6 * t_lookup / n_req,
            "append_us_per_request": 1e6 * t_append / n_req,
            "batch_step_us": 1e6 * t_step / n_steps,
            "pool_blocks": nb, **st,
        }
        log(f"[prefix] {label}: {json.dumps(res[label])}")
    s = res["stable"]
    rec = {
        "metric": "prefix cache: fraction of prompt tokens served from cache (agent sessions, last turn)",
        "value": s["hit_fraction_last_turn"], "unit": "fraction", "higher_is_better": True,
        "n_gpus": 0, "data": "synthetic", "dtype": "int32 token ids",
        "config": {"workload": "agent sessions 32 x 11 turns, system 1000 + 400 user + 100 out per turn",
                   **PREFIX_SHAPE},
        "stable": s, "dynamic_head": res["dynamic_head"],
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = prefix_cpu_baseline(args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def prefix_cpu_baseline(budget_s: float):
    """The prefix-cache model (test infrastructure) replaying the first turns
    of the same stream until the budget is spent: requests per second."""
    import workloads as wl
    from oracle.allocator import PrefixCachingAllocatorModel

    turns = wl.agent_sessions(2024, dynamic_head=0, **PREFIX_SHAPE)
    last = max(len(t.prompt) + len(t.output) for t in turns)
    m = PrefixCachingAllocatorModel(int(1.1 * PREFIX_SHAPE["n_sessions"] * -(-last // 16)), -(-last // 16) + 1,
                                    model_key=1)
    t0 = time.perf_counter()
    n_req = 0
    for turn in range(PREFIX_SHAPE["turns"]):
        group = [t for t in turns if t.turn == turn]
        ids = [1000 * turn + t.session for t in group]
        for sid, t in zip(ids, group):
            n = m.create_cached(sid, t.prompt)
            m.append_tokens(sid, t.prompt[n:])
            n_req += 1
        for j in range(len(group[0].output)):
            m.batch_append_tokens(ids, [t.output[j] for t in group])
        for sid in ids:
            m.free_seq(sid)
        if time.perf_counter() - t0 >= budget_s:
            break
    wall = time.perf_counter() - t0
    return {"value": n_req / wall, "unit": "requests/s (with their decode steps)", "cores": 1, "kind": "oracle",
            "sample": f"first {turn + 1} turns ({n_req} requests) of the same stream, pure Python, one thread"}


if __name__ == "__main__":
    main()
