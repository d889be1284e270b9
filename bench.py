#!/usr/bin/env python3
"""Benchmark of the R-SWA hot path on one MI355X.

A step is one decode step of the whole batch: K1 append of one new K/V row per sequence and head,
then K2 split-K decode attention over prefix u window, fused in one launch. The headline workload
is the multi-page decode (8 sequences of 20 pages, m = 5155, n = 128, bf16, T = 20000 steps):
346 MB of K/V rows per step, more than the 256 MB Infinity Cache holds, so the rows stream from
HBM. The cache is built untimed first (t = 1 .. T - K - W, timed in 64-step blocks for the
latency-vs-t curve), then W warmup steps and the K timed steps, the workload's last ones: the
window is full and the figure is the per-step cost that R-SWA keeps constant. Inputs for every
step are resident in HBM before timing.

Also reported: the decode kernel's algorithmic HBM GB/s against the 8 TB/s peak, latency vs t and
its flatness, the same workload in full-causal mode (the growth curve), the batched single-page
decode (64 sequences; its 211 MB working set fits the Infinity Cache, so its GB/s are effective),
the single-page fp32 decode (B = 1, latency-bound), the ragged batch, the masked prefill in
TFLOP/s against the bf16 MFMA peak, the teacher-forced training pass on the same 32K sequence,
shared-document decode with the prefixes in a token pool vs copied per sequence, and the fp64
oracle timed on bounded samples on the host cores with one thread and with all (cpu_baseline).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "R-SWA decode tok/s + HBM GB/s vs T (1 GPU); masked prefill TFLOP/s"
LEGS = ("growth", "batched", "single", "ragged", "shared", "graph", "prefill", "backward", "cpu")
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
H, D = 16, 128
DECODE_SOURCES = ["windowed_attention_amd/csrc/decode.hip", "windowed_attention_amd/csrc/device.h",
                  "windowed_attention_amd/csrc/kernels.h", "windowed_attention_amd/csrc/plan.h",
                  "windowed_attention_amd/_build.py"]
PREFILL_SOURCES = ["windowed_attention_amd/csrc/prefill.hip", "windowed_attention_amd/csrc/mfma.h",
                   "windowed_attention_amd/csrc/device.h", "windowed_attention_amd/csrc/kernels.h",
                   "windowed_attention_amd/_build.py"]  # the build script carries per-source flags
BACKWARD_SOURCES = ["windowed_attention_amd/csrc/prefill_bwd.hip",
                    "windowed_attention_amd/csrc/mfma.h", "windowed_attention_amd/csrc/device.h",
                    "windowed_attention_amd/csrc/kernels.h"]
KIND_SOURCES = {"decode": DECODE_SOURCES, "prefill": PREFILL_SOURCES,
                "backward": BACKWARD_SOURCES}
KIND_KERNELS = {"decode": ("decode_kernel",), "prefill": ("prefill_kernel",),
                "backward": ("delta_kernel", "dkdv_kernel", "dq_kernel")}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    """Hash of the sources a kernel is compiled from, comments and blank space left out, so that a
    traffic record stays valid across edits that do not change the code."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        if p.endswith(".py"):
            text = re.sub(r"#[^\n]*", "", text)
        else:
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", choices=["batched", "single", "multipage"],
                    default="multipage")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline decode (for counter runs of its kernel)")
    ap.add_argument("--legs", default="all",
                    help="comma list of the other measurements to run: growth, batched, single, "
                         "ragged, shared, graph, prefill, backward, cpu (default all)")
    ap.add_argument("--mode", choices=["rswa", "full"], default="rswa")
    ap.add_argument("--chunk", type=int, default=0, help="decode rows per split (0 = automatic)")
    ap.add_argument("--grid", type=int, default=0, help="decode workgroups (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-shared", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the headline decode")
    ap.add_argument("--kernel-events", action="store_true",
                    help="diagnostic: record HIP events around every launch (adds GPU time)")
    ap.add_argument("--unfused", action="store_true",
                    help="time rswa_append_kv + rswa_decode_attn instead of rswa_decode_step")
    ap.add_argument("--no-growth", action="store_true",
                    help="skip the multi-page R-SWA vs full-causal growth curve")
    ap.add_argument("--no-ragged", action="store_true", help="skip the ragged-batch decode")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also time a plain 1 GiB device copy (bandwidth reference, PMC scale)")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "KIND"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs of the decode or "
                         "prefill kernel (KIND) into profiles/<KIND>_traffic.json and exit "
                         "(no GPU use)")
    ap.add_argument("--prefill-runs", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="oracle decode seconds per leg (1 thread, all cores)")
    return ap.parse_args()


# ------------------------------------------------------------------------------------------------
# decode
# ------------------------------------------------------------------------------------------------
def decode_workload(name: str):
    import workloads as W
    return {"single": lambda: W.decode_config(1), "batched": lambda: W.decode_config(2),
            "multipage": lambda: W.decode_config(3), "ragged": lambda: W.varlen_config(0)}[name]()


def upload(arr, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def decode_bytes(wl, t: int, full: bool, out_elem: int) -> int:
    """Algorithmic HBM bytes of one decode launch at step t: every live K and V row once, q read,
    output written (the append's own traffic is counted separately)."""
    e = 2 if wl.dtype == "bf16" else 4
    act = wl.steps >= t
    live = wl.prefix_len.astype(np.int64) + (np.minimum(t, wl.steps) if full else
                                             np.minimum(wl.window, t))
    rows = int(live[act].sum())
    nb = int(act.sum())
    return rows * 2 * H * D * e + nb * H * D * (e + out_elem)


def append_bytes(wl, t: int) -> int:
    e = 2 if wl.dtype == "bf16" else 4
    return int((wl.steps >= t).sum()) * H * D * e * 4  # k, v read; k, v written


def run_decode(args, wl, mode_full: bool, steps: int, warmup: int, kernel_events: bool = False,
               paged=None, setup: int = 0, block: int = 64, series_block: int = 0):
    """Run decode steps t = 1 .. setup + warmup + steps of one workload through the C ABI.

    Steps 1 .. setup build the cache state (the ring fills, the full-causal cache grows); they are
    timed in blocks of `block` steps with events between blocks, which gives the latency-vs-t
    curve. After a synchronization, `warmup` untimed steps, another synchronization, then the
    `steps` timed steps between two events (nothing recorded in between) and a synchronization.
    `paged` (workloads.PagedPrefix): the cache reads the prefixes from the shared token pool
    through the page table instead of holding copies. `series_block` > 0 also records an event
    every that many timed steps (a per-block latency series of the timed region)."""
    import torch
    import windowed_attention_amd as wa
    lib = wa._lib
    dev_q, dev_k, dev_v = upload(wl.q, wl.dtype), upload(wl.k, wl.dtype), upload(wl.v, wl.dtype)
    kvdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    if paged is None:
        pk, pv = upload(wl.prefix_k, wl.dtype), upload(wl.prefix_v, wl.dtype)
        pool = {}
    else:
        pk = pv = None
        pool = dict(pool_k=upload(paged.pool_k, wl.dtype), pool_v=upload(paged.pool_v, wl.dtype),
                    prefix_table=torch.from_numpy(paged.table).cuda())
    mode = wa.MODE_FULL_CAUSAL if mode_full else wa.MODE_RSWA
    ragged = bool((wl.steps != wl.steps.max()).any())
    total = setup + warmup + steps
    if total > wl.T:
        raise SystemExit(f"setup + warmup + steps = {total} exceeds the workload's T = {wl.T}")
    cache = wa.RswaCache(pk, pv, wl.prefix_len, None if mode_full else wl.window, mode=mode,
                         max_steps=wl.steps if mode_full else None, kv_dtype=kvdt, **pool)
    del pk, pv
    cache.set_decode_split(args.chunk, args.grid)
    out_dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    out = torch.empty((wl.batch, H, D), dtype=out_dt, device="cuda")
    out_code = wa.BF16 if out_dt == torch.bfloat16 else wa.F32
    act = None
    if ragged:
        act = torch.from_numpy(np.stack([wl.active(t) for t in range(1, wl.T + 1)])).cuda()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    h = cache.handle
    step_bytes = wl.batch * H * D * dev_q.element_size()
    qb, kb, vb = dev_q.data_ptr(), dev_k.data_ptr(), dev_v.data_ptr()
    ob = out.data_ptr()
    ab = act.data_ptr() if act is not None else None

    fused = not args.unfused

    def step(t):  # t is 1-based; the separate path's append (the fused path appends in decode)
        o = (t - 1) * step_bytes
        a = None if ab is None else ab + (t - 1) * wl.batch
        if not fused:
            r = lib.rswa_append_kv(h, kb + o, vb + o, a, sp)
            if r:
                raise RuntimeError(f"append failed: {r} {lib.rswa_last_error()}")
        return o, a

    def decode(o, a):
        if fused:
            r = lib.rswa_decode_step(h, qb + o, kb + o, vb + o, ob, out_code, ctypes.c_float(0.0),
                                     a, sp)
        else:
            r = lib.rswa_decode_attn(h, qb + o, ob, out_code, ctypes.c_float(0.0), a, sp)
        if r:
            raise RuntimeError(f"decode failed: {r} {lib.rswa_last_error()}")

    # state set-up, timed in blocks (the latency-vs-t curve)
    nblk = (setup + block - 1) // block
    ev_blk = [torch.cuda.Event(enable_timing=True) for _ in range(nblk + 1)]
    torch.cuda.synchronize()
    for t in range(1, setup + 1):
        if (t - 1) % block == 0:
            ev_blk[(t - 1) // block].record()
        decode(*step(t))
    if setup:
        ev_blk[nblk].record()
    torch.cuda.synchronize()
    lat = []
    for j in range(nblk):
        t_lo = 1 + j * block
        n_in = min(block, setup - t_lo + 1)
        lat.append((t_lo + n_in // 2, ev_blk[j].elapsed_time(ev_blk[j + 1]) * 1e3 / n_in))

    for t in range(setup + 1, setup + warmup + 1):
        decode(*step(t))
    torch.cuda.synchronize()
    grid_blocks, launches = cache.decode_plan(appending=fused)
    if not fused:
        launches += 1  # the separate append launch

    t_first = setup + warmup + 1
    ev_k = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(steps)] if kernel_events else []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_ser = []
    start.record()
    for i in range(steps):
        if series_block and i % series_block == 0 and i:
            ev_ser.append((i, torch.cuda.Event(enable_timing=True)))
            ev_ser[-1][1].record()
        o, a = step(t_first + i)
        if kernel_events:
            ev_k[i][0].record()
            decode(o, a)
            ev_k[i][1].record()
        else:
            decode(o, a)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    elapsed_ms = start.elapsed_time(end) if steps else 0.0
    steps_done = cache.steps()
    cache.close()

    kern_ms = np.array([a.elapsed_time(b) for a, b in ev_k]) if kernel_events else None
    series = []
    if ev_ser:
        marks = [(0, start)] + ev_ser + [(steps, end)]
        for (i0, e0), (i1, e1) in zip(marks[:-1], marks[1:]):
            series.append((t_first + i0, t_first + i1 - 1, e0.elapsed_time(e1) * 1e3 / (i1 - i0)))
    if steps:
        lat.append((t_first + steps // 2, elapsed_ms * 1e3 / steps))
    out_elem = out.element_size()
    ts = range(t_first, t_first + steps)
    dec_bytes = np.array([decode_bytes(wl, t, mode_full, out_elem) for t in ts], dtype=np.float64)
    app_bytes = np.array([append_bytes(wl, t) for t in ts], dtype=np.float64)
    tokens = int(sum(int((wl.steps >= t).sum()) for t in ts))
    # bytes of the launch the events bracket: the fused step also moves the append's rows
    launch_bytes = dec_bytes + app_bytes if fused else dec_bytes
    return dict(elapsed_ms=elapsed_ms, wall_s=wall, kern_ms=kern_ms, lat=lat,
                dec_bytes=dec_bytes, app_bytes=app_bytes, launch_bytes=launch_bytes,
                tokens=tokens, fused=fused, steps_done=steps_done.tolist(),
                launches_per_step=launches, grid_blocks=grid_blocks,
                timed_t=[t_first, t_first + steps - 1], series=series)


def flatness(lat, n, T):
    """Median step latency over the last w steps / over the first w steps once the ring is full
    (t > n), w = max(500, T / 10) capped at half of the steps after the ring fills, so that the
    late window holds the timed region's sample."""
    ts = np.array([t for t, _ in lat])
    us = np.array([u for _, u in lat])
    w = min(max(500, T // 10), max(1, (T - n) // 2))
    late = us[(ts >= T - w) & (ts <= T)]
    early = us[(ts >= n + 1) & (ts <= n + w)]
    if late.size == 0 or early.size == 0:
        return None
    return float(np.median(late) / np.median(early))


def traffic_from_profile(kind: str, src_hash: str, per_launch_units: float | None = None):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE summaries, scaled by
    the same counters' reading for a plain copy of known size; None if the kernel source changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kind}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device-to-device copy of `nbytes` (torch's copy kernel): the practical bandwidth
    reference, and the known-size dispatch the PMC byte counters are scaled by."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    ms = float(np.median(ts))
    return dict(bytes_moved=2 * nbytes, ms=ms, gbs=2 * nbytes / (ms * 1e-3) / 1e9)


def pmc_summary(fetch_csv: str, write_csv: str, kind: str):
    """Scale the decode/prefill kernels' FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the same
    counters read for the 1 GiB calibration copy (1 GiB read, 1 GiB written)."""
    import csv
    def per_kernel(path, counter):
        rows = list(csv.DictReader(open(path)))
        out = {}
        for r in rows:
            if r.get("Counter_Name", counter) != counter:
                continue
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out
    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    # torch's copy_ of the calibration buffers dispatches the runtime's blit kernel; its largest
    # dispatch is the 1 GiB copy (1 GiB read, 1 GiB written)
    copy_k = [k for k in fetch if k.startswith("__amd_rocclr_copyBuffer")]
    if not copy_k:
        raise SystemExit("no calibration copy dispatch in the counter CSV (run with --copy-calibration)")
    cf = (1 << 30) / (max(fetch[copy_k[0]]) * 1024.0)
    cw = (1 << 30) / (max(write[copy_k[0]]) * 1024.0)
    names = [k for k in fetch if any(f"::{n}<" in k for n in KIND_KERNELS[kind])]
    rec = dict(kernel_names=names, copy_kernel=copy_k[0], fetch_scale=cf, write_scale=cw)
    for k in names:
        f = np.array(fetch[k]) * 1024.0 * cf
        w = np.array(write.get(k, [0.0])) * 1024.0 * cw
        rec[k] = dict(dispatches=int(f.size), fetch_bytes_median=float(np.median(f)),
                      write_bytes_median=float(np.median(w)))
    if kind == "backward":  # the backward call: its three launches together
        rec["bytes_per_launch"] = sum(rec[k]["fetch_bytes_median"] + rec[k]["write_bytes_median"]
                                      for k in names)
    else:
        main = max(names, key=lambda k: rec[k]["fetch_bytes_median"])
        rec["bytes_per_launch"] = rec[main]["fetch_bytes_median"] + rec[main]["write_bytes_median"]
    rec["source_hash"] = source_hash(KIND_SOURCES[kind])
    return rec


def shared_documents(args, warmup=128, steps=1024):
    """Several sequences decoding over the same documents: prefixes held once in a token pool
    (paged) vs a copy per sequence. Both read the same rows per step; the paged cache's distinct
    prefix bytes are those of the documents only."""
    import workloads as W
    import torch
    wl, pp = W.shared_document_config(seed=0)
    res = dict(workload=wl.name)
    for kind in ("paged", "copied"):
        r = run_decode(args, wl, False, steps, warmup, False, paged=pp if kind == "paged" else None)
        torch.cuda.empty_cache()
        ms = r["elapsed_ms"] / steps
        res[kind] = dict(us_per_step=ms * 1e3, tok_s=r["tokens"] / (r["elapsed_ms"] * 1e-3),
                         requested_gbs=float(r["launch_bytes"].mean()) / (ms * 1e-3) / 1e9)
    e = 2
    t_mid = warmup + steps // 2
    live = int(wl.prefix_len[0]) + 128
    res["rows_per_step"] = int(wl.batch * live)
    res["requested_bytes_per_step"] = float(wl.batch * live * 2 * H * D * e)
    res["distinct_prefix_bytes"] = float(pp.pool_k.nbytes + pp.pool_v.nbytes)
    res["copied_prefix_bytes"] = float(wl.prefix_k.nbytes + wl.prefix_v.nbytes)
    res["speedup"] = res["copied"]["us_per_step"] / res["paged"]["us_per_step"]
    res["t_mid"] = t_mid
    return res


def graph_loop(args, G=64, replays=6):
    """Fused decode steps launched one by one vs replayed from a captured HIP graph of G steps
    (input slots filled once; timing only). Same workloads as the single-page fp32 (B = 1) and
    the headline batched decode."""
    import torch
    import windowed_attention_amd as wa
    import workloads as W
    res = {}
    for name, wl in (("single", W.decode_config(1)), ("batched", W.decode_config(2, T=1200))):
        kvdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        q, k, v = upload(wl.q, wl.dtype), upload(wl.k, wl.dtype), upload(wl.v, wl.dtype)
        out = torch.empty((wl.batch, H, D), dtype=torch.float32, device="cuda")
        times = {}
        for kind in ("eager", "graph"):
            pk, pv = upload(wl.prefix_k, wl.dtype), upload(wl.prefix_v, wl.dtype)
            cache = wa.RswaCache(pk, pv, wl.prefix_len, wl.window, kv_dtype=kvdt)
            if kind == "graph":
                g = wa.StepGraph(cache, G)
                g.q.copy_(q[:G])
                g.k.copy_(k[:G])
                g.v.copy_(v[:G])
                g.launch()  # warmup
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(replays):
                    g.launch()
                b.record()
                torch.cuda.synchronize()
                times[kind] = a.elapsed_time(b) * 1e3 / (G * replays)
                g.close()
            else:  # raw C-ABI calls, as in the headline measurement
                lib, h = wa._lib, cache.handle
                sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                sb = wl.batch * H * D * q.element_size()
                qb, kb, vb, ob = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr()
                zero = ctypes.c_float(0.0)

                def step(t):
                    o = t * sb
                    if lib.rswa_decode_step(h, qb + o, kb + o, vb + o, ob, wa.F32, zero, None, sp):
                        raise RuntimeError(lib.rswa_last_error())
                for t in range(G):
                    step(t)
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for t in range(G, G + G * replays):
                    step(t)
                b.record()
                torch.cuda.synchronize()
                times[kind] = a.elapsed_time(b) * 1e3 / (G * replays)
            cache.close()
        res[name] = dict(workload=wl.name, eager_us_per_step=times["eager"],
                         graph_us_per_step=times["graph"], graph_steps=G)
    return res


# ------------------------------------------------------------------------------------------------
# prefill
# ------------------------------------------------------------------------------------------------
def visible_pairs(S: int, m: int, n: int, prefix_causal: bool = False) -> int:
    """Visible (query, key) pairs of one sequence under the R-SWA prefill mask (closed form)."""
    pre = m * (m + 1) // 2 if prefix_causal else m * m
    outs = S - m
    win = 0
    for i in range(outs):  # output i sees min(n, i + 1) outputs
        win += min(n, i + 1)
    return pre + outs * m + win


def tile_issued_pairs(S: int, m: int, n: int, prefix_causal: bool = False, bm: int = 256,
                      bn: int = 64) -> int:
    """(query, key) pairs the prefill kernel's MFMAs compute for one sequence and head: every
    workgroup of bm queries visits the bn-key tiles over the prefix [0, m) (over [0, q_end) for a
    causal prefix tile that ends inside it) and over the window [max(m, max(q0, m) - n + 1),
    q_end), all bm x bn pairs of each, masked ones included."""
    pairs = 0
    for q0 in range(0, S, bm):
        q1 = min(q0 + bm, S)
        pre_end = q1 if (prefix_causal and q1 <= m) else m
        tiles = (pre_end + bn - 1) // bn
        if q1 > m:
            ws = max(m, max(q0, m) - n + 1)
            tiles += (q1 - ws + bn - 1) // bn
        pairs += bm * bn * tiles
    return pairs


def run_prefill(args):
    import torch
    import windowed_attention_amd as wa
    import workloads as W
    pw = W.prefill_config()
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    cu = torch.tensor(pw.cu_seqlens, dtype=torch.int32, device="cuda")
    m = torch.tensor(pw.prefix_len, dtype=torch.int32, device="cuda")
    n = torch.tensor(pw.window, dtype=torch.int32, device="cuda")
    S = int(pw.cu_seqlens[-1])
    out = torch.empty((S, H, D), dtype=torch.bfloat16, device="cuda")
    try:
        wa.rswa_prefill_attn(q, k, v, cu, m, n, out=out, max_seqlen=S)
    except wa.RswaError as e:
        if e.status == -2:
            return None
        raise
    for _ in range(3):
        wa.rswa_prefill_attn(q, k, v, cu, m, n, out=out, max_seqlen=S)
    torch.cuda.synchronize()
    times = []
    for _ in range(args.prefill_runs):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        wa.rswa_prefill_attn(q, k, v, cu, m, n, out=out, max_seqlen=S)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    med_ms = float(np.median(times))
    pairs = visible_pairs(S, int(pw.prefix_len[0]), int(pw.window[0]))
    issued = tile_issued_pairs(S, int(pw.prefix_len[0]), int(pw.window[0]))
    flops = 4.0 * D * H * pairs
    tflops = flops / (med_ms * 1e-3) / 1e12
    return dict(workload=pw.name, ms=med_ms, runs=args.prefill_runs, warmup_runs=3,
                tflops=tflops, flop=flops, visible_pairs_per_head=pairs,
                tile_issued_flop=4.0 * D * H * issued, tile_issued_over_algorithmic=issued / pairs,
                exp_count=H * pairs,
                roofline=dict(bound="mfma", achieved=tflops, peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                              frac=tflops / PEAK_BF16_TFLOPS,
                              traffic=traffic_from_profile("prefill",
                                                           source_hash(PREFILL_SOURCES))))


def run_backward(args):
    """Training pass on the 32K prefill workload: forward with log-sum-exp, then the backward
    (delta, dK/dV, dQ launches). Algorithmic FLOPs: 4 D per visible (query, key) pair and head
    for the forward, 10 D for the backward (S = Q K^T, dP = dO V^T, dV, dK, dQ)."""
    import torch
    import windowed_attention_amd as wa
    import workloads as W
    pw = W.prefill_config()
    g = W.make_output_grad(pw, seed=0)
    q, k, v = upload(pw.q, "bf16"), upload(pw.k, "bf16"), upload(pw.v, "bf16")
    dout = upload(g, "bf16")
    cu = torch.tensor(pw.cu_seqlens, dtype=torch.int32, device="cuda")
    m = torch.tensor(pw.prefix_len, dtype=torch.int32, device="cuda")
    n = torch.tensor(pw.window, dtype=torch.int32, device="cuda")
    S = int(pw.cu_seqlens[-1])
    out = torch.empty((S, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((S, H), dtype=torch.float32, device="cuda")
    work = torch.empty((2, H, S), dtype=torch.float32, device="cuda")
    grads = [torch.empty((S, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(3)]

    def fwd():
        wa.rswa_prefill_fwd(q, k, v, cu, m, n, out=out, lse=lse, max_seqlen=S)

    def bwd():
        wa.rswa_prefill_bwd(q, k, v, out, dout, lse, cu, m, n, dq=grads[0], dk=grads[1],
                            dv=grads[2], work=work, max_seqlen=S)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(args.prefill_runs):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        return float(np.median(times))

    fwd()
    fwd_ms = timed(fwd)
    bwd_ms = timed(bwd)
    pairs = visible_pairs(S, int(pw.prefix_len[0]), int(pw.window[0]))
    bflop = 10.0 * D * H * pairs
    tflops = bflop / (bwd_ms * 1e-3) / 1e12
    train = (bflop + 4.0 * D * H * pairs) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12
    return dict(workload=pw.name + ", forward + backward, bf16 gradients", fwd_ms=fwd_ms,
                bwd_ms=bwd_ms, bwd_tflops=tflops, train_tflops=train, bwd_flop=bflop,
                roofline=dict(bound="mfma", achieved=tflops, peak=PEAK_BF16_TFLOPS,
                              unit="TFLOP/s", frac=tflops / PEAK_BF16_TFLOPS,
                              traffic=traffic_from_profile("backward",
                                                           source_hash(BACKWARD_SOURCES)),
                              kernel="backward call (delta + dK/dV + dQ launches)"))


# ------------------------------------------------------------------------------------------------
# cpu baseline: the fp64 oracle on a bounded sample
# ------------------------------------------------------------------------------------------------
def oracle_step_sample(wl, extra: int = 16, seed: int = 0):
    """Sampled decode steps: {1, 2, n-1, n, n+1, 2n, 1000, T-1, T}, the steps where the live row
    count m + min(n, t) crosses a multiple of 64, and `extra` seeded random steps."""
    n, m, T = int(wl.window[0]), int(wl.prefix_len[0]), int(wl.T)
    s = {1, 2, n - 1, n, n + 1, 2 * n, 1000, T - 1, T}
    s |= {t for t in range(1, min(T, n) + 1) if (m + t - 1) // 64 != (m + t) // 64}
    s |= set(np.random.default_rng(seed).integers(1, T + 1, size=extra).tolist())
    return sorted(t for t in s if 1 <= t <= T)


def _oracle_decode_leg(wl, steps, seconds, O, to_f64):
    rng = np.random.default_rng(1)
    pre = {}
    done, per_step = 0, []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        t = steps[done % len(steps)]
        b = int(rng.integers(0, wl.batch))
        if wl.steps[b] < t:
            continue
        if b not in pre:
            pk, pv = wl.prefix(b)
            pre[b] = (to_f64(pk, wl.dtype), to_f64(pv, wl.dtype))
        a = time.perf_counter()
        O.decode_step(to_f64(wl.q[t - 1, b], wl.dtype), pre[b][0], pre[b][1],
                      to_f64(wl.k[:t, b], wl.dtype), to_f64(wl.v[:t, b], wl.dtype), t,
                      int(wl.window[b]))
        per_step.append(time.perf_counter() - a)
        done += 1
    el = time.perf_counter() - t0
    return dict(tok_s=done / el, outputs=done, seconds=el,
                median_ms_per_step=float(np.median(per_step)) * 1e3 if per_step else None)


def _oracle_prefill_leg(pw, qkv, blocks, O):
    """The oracle's prefill on the given query blocks of the 32K sequence (its own 512-row
    blocking); algorithmic FLOPs of those rows: 4 D H per visible (query, key) pair."""
    S, m, n = int(pw.cu_seqlens[-1]), int(pw.prefix_len[0]), int(pw.window[0])
    q, k, v = qkv
    pairs = 0
    t0 = time.perf_counter()
    for b0 in blocks:
        rows = np.arange(b0, min(S, b0 + 512))
        O.prefill(q, k, v, m, n, rows=rows)
        for p in rows:  # visible keys of query p (prefix, then its output window)
            pairs += m if p < m else m + min(n, p - m + 1)
    el = time.perf_counter() - t0
    flops = 4.0 * D * H * pairs
    return dict(seconds=el, rows=int(sum(min(S, b + 512) - b for b in blocks)),
                gflops=flops / el / 1e9, flop=flops)


def cpu_baseline(wl, seconds: float):
    """The fp64 oracle as it stands, on the host cores of this run: decode on sampled steps of the
    headline workload (each computed independently from the growing cache) and the masked
    prefill on sampled 512-query blocks of the 32K sequence, each with one BLAS thread and with
    every thread the BLAS pool has. Reported only; never a target."""
    import oracle as O
    import workloads as W
    from workloads import to_f64
    from threadpoolctl import threadpool_info, threadpool_limits
    aff = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    pools = threadpool_info()
    blas_threads = max([p.get("num_threads", 1) for p in pools] or [1])
    steps = oracle_step_sample(wl)
    pw = W.prefill_config()
    S, m = int(pw.cu_seqlens[-1]), int(pw.prefix_len[0])
    blocks = [(m // 512 + 1) * 512]  # the first 512-row block of outputs (prefix + window keys)
    qkv = tuple(to_f64(x, "bf16") for x in (pw.q, pw.k, pw.v))
    legs = {}
    for name, lim in (("1_thread", 1), ("all_cores", blas_threads)):
        with threadpool_limits(limits=lim):
            dec = _oracle_decode_leg(wl, steps, seconds, O, to_f64)
            pre = _oracle_prefill_leg(pw, qkv, blocks, O)
        total_pairs = visible_pairs(S, m, int(pw.window[0]))
        pre["full_prefill_seconds_extrapolated"] = 4.0 * D * H * total_pairs / (pre["gflops"] * 1e9)
        legs[name] = dict(threads=lim, decode=dec, prefill=pre)
        log(f"[bench] oracle {name}: decode {dec['tok_s']:.2f} tok/s, prefill "
            f"{pre['gflops']:.1f} GFLOP/s")
    best = legs["all_cores"]
    return dict(value=best["decode"]["tok_s"], unit="tok/s", cores=blas_threads, kind="oracle",
                sample=(f"{best['decode']['outputs']} (sequence, step) decode outputs of the "
                        f"headline workload at steps {{1,2,n-1,n,n+1,2n,1000,T-1,T}} + the "
                        f"64-row crossings + 16 seeded random steps, each from the growing cache "
                        f"in fp64 ({seconds:.0f} s per leg); prefill: "
                        f"{best['prefill']['rows']} of the {S} query rows of the 32K sequence "
                        f"(the first 512-row block of output queries)"),
                cpu_count=os.cpu_count(), affinity=aff, blas_threads=blas_threads, legs=legs)


# ------------------------------------------------------------------------------------------------
def growth_curve(args, wl, rswa_lat):
    """Multi-page decode (B=8, m=5155, n=128, T=20000): per-step latency vs t for R-SWA (flat;
    the headline run's curve) and for the full-causal mode (cache m + t, growing), same inputs
    and launch path."""
    import types
    out = {}
    for mode in ("rswa", "full"):
        if mode == "rswa":
            lat = rswa_lat
        else:
            a = types.SimpleNamespace(chunk=args.chunk, grid=args.grid, unfused=args.unfused)
            lat = run_decode(a, wl, True, 0, 0, setup=wl.T)["lat"]
        ts = np.array([t for t, _ in lat], dtype=np.float64)
        us = np.array([u for _, u in lat])
        byt = np.array([decode_bytes(wl, int(t), mode == "full", 2) + append_bytes(wl, int(t))
                        for t in ts])
        keep = np.linspace(0, len(lat) - 1, 40).round().astype(int)
        rec = dict(us_per_step_vs_t=[[int(ts[i]), round(float(us[i]), 2)] for i in keep],
                   gbs_vs_t=[[int(ts[i]), round(float(byt[i] / (us[i] * 1e-6) / 1e9))]
                             for i in keep],
                   median_us=float(np.median(us)))
        if mode == "full":
            rows = int(wl.prefix_len[0]) + ts
            rec["slope_us_per_1k_rows"] = float(np.polyfit(rows, us, 1)[0] * 1000.0)
        else:
            rec["flatness"] = flatness(lat, int(wl.window[0]), int(wl.T))
        rec["jumps_over_10pct"] = [[int(ts[i]), round(float(us[i] / us[i - 1]), 3)]
                                   for i in range(1, len(us)) if abs(us[i] / us[i - 1] - 1) > 0.10]
        out[mode] = rec
        log(f"[bench] growth {mode}: median {rec['median_us']:.1f} us/step")
    out["workload"] = wl.name
    return out


def steady_leg(args, name: str, steps: int, warmup: int):
    """Another decode workload at steady state: the cache is built untimed (block-timed for the
    latency curve), then `warmup` steps, then `steps` timed steps ending at its last step."""
    import types
    wl = decode_workload(name)
    a = types.SimpleNamespace(chunk=args.chunk, grid=args.grid, unfused=args.unfused)
    setup = int(wl.T) - steps - warmup
    r = run_decode(a, wl, False, steps, warmup, setup=setup, series_block=250)
    ms = r["elapsed_ms"] / steps
    gbs = float((r["dec_bytes"] + r["app_bytes"]).mean()) / (ms * 1e-3) / 1e9
    lat = r["lat"]
    if r["series"]:  # the timed steps by blocks instead of one point at their middle
        lat = lat[:-1] + [((lo + hi) // 2, us) for lo, hi, us in r["series"]]
    keep = np.linspace(0, len(lat) - 1, min(len(lat), 24)).round().astype(int)
    return dict(workload=wl.name, timed_t=r["timed_t"], steps=steps,
                tok_s=r["tokens"] / (r["elapsed_ms"] * 1e-3), us_per_step=ms * 1e3,
                step_bytes=float((r["dec_bytes"] + r["app_bytes"]).mean()), step_gbs=gbs,
                frac=gbs / PEAK_HBM_GBS, launches_per_step=r["launches_per_step"],
                latency_vs_t=[[int(lat[i][0]), round(float(lat[i][1]), 3)] for i in keep],
                flatness=flatness(lat, int(wl.window[0]), int(wl.T)))


def ragged_decode(args, steps=3000):
    import types
    wl = decode_workload("ragged")
    a = types.SimpleNamespace(chunk=args.chunk, grid=args.grid, unfused=args.unfused)
    warm = 300
    r = run_decode(a, wl, False, steps, warm, False, series_block=250)
    ms = r["elapsed_ms"] / steps
    gbs = float((r["dec_bytes"] + r["app_bytes"]).mean()) / (ms * 1e-3) / 1e9
    # per block of 250 timed steps: first t, last t, us/step, sequences still decoding at the
    # block's middle step, GB/s over the block's algorithmic bytes
    byts = r["dec_bytes"] + r["app_bytes"]
    t0 = r["timed_t"][0]
    vs_t = []
    for lo, hi, us in r["series"]:
        mid = (lo + hi) // 2
        active = int((wl.steps >= mid).sum())
        blk_gbs = float(byts[lo - t0:hi - t0 + 1].mean()) / (us * 1e-6) / 1e9
        vs_t.append([lo, hi, round(us, 2), active, round(blk_gbs)])
    return dict(workload=wl.name, steps=steps, timed_t=[warm + 1, warm + steps],
                tok_s=r["tokens"] / (r["elapsed_ms"] * 1e-3), us_per_step=ms * 1e3,
                step_gbs=gbs, frac=gbs / PEAK_HBM_GBS, launches_per_step=r["launches_per_step"],
                vs_t=vs_t, vs_t_columns=["t_first", "t_last", "us_per_step", "active_sequences",
                                         "gbs"])


def main():
    args = parse()
    if args.pmc_summary:
        rec = pmc_summary(*args.pmc_summary)
        path = os.path.join(ROOT, "profiles", f"{args.pmc_summary[2]}_traffic.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    import windowed_attention_amd  # noqa: F401  (fails loudly if the HIP library is missing)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    res = dict(metric=METRIC, n_gpus=1, higher_is_better=True, scaling="weak", vs_baseline=None,
               data="synthetic")
    wanted = set(LEGS if args.legs == "all" else args.legs.split(","))
    unknown = wanted - set(LEGS)
    if unknown:
        raise SystemExit(f"unknown legs: {sorted(unknown)}")
    on = {leg: (not args.headline_only) and leg in wanted for leg in LEGS}
    wl = None
    if not args.no_decode:
        t0 = time.perf_counter()
        wl = decode_workload(args.workload)
        log(f"[bench] generated {wl.name} in {time.perf_counter() - t0:.1f} s")
        full = args.mode == "full"
        n = int(wl.window.max())
        warmup = args.warmup
        steps = args.steps
        # Whatever --steps / --warmup say, the timed steps are the workload's last ones: the cache
        # is first built untimed (ring full, steady state), so the figure is the per-step cost
        # the method keeps constant, not the fill transient.
        setup = int(wl.T) - steps - warmup
        if setup < n and not full:
            raise SystemExit(f"--steps + --warmup = {steps + warmup} leave fewer than n = {n} "
                             f"set-up steps of T = {wl.T}: the timed steps would fill the ring")
        r = run_decode(args, wl, full, steps, warmup, args.kernel_events, setup=setup)
        log(f"[bench] decode: {steps} steps (t = {r['timed_t'][0]}..{r['timed_t'][1]}) in "
            f"{r['elapsed_ms']:.3f} ms (host wall {r['wall_s']:.3f} s)")
        ms_step = r["elapsed_ms"] / steps
        tok_s = r["tokens"] / (r["elapsed_ms"] * 1e-3)
        step_bytes = float((r["dec_bytes"] + r["app_bytes"]).mean())
        res.update(value=tok_s, unit="tok/s", steps=steps, warmup=warmup, ms_per_step=ms_step,
                   dtype="bf16" if wl.dtype == "bf16" else "f32",
                   math="fp32 (scores, softmax, accumulation)",
                   config=dict(workload=wl.name, batch=wl.batch, prefix_len=int(wl.prefix_len[0]),
                               window=int(wl.window[0]), T=int(wl.T), kv_dtype=wl.dtype,
                               mode=args.mode, timed_t=r["timed_t"], setup_steps=setup,
                               state="ring full (steady state)" if not full else "full causal"))
        res["hbm_gbs_step"] = step_bytes / (ms_step * 1e-3) / 1e9
        # The dominant kernel is the fused append + decode launch. When it is the step's only
        # launch, its average duration is the event-bracketed timed region over the number of
        # steps (no events between launches: recording one per launch costs several microseconds
        # of GPU time per step and would inflate the figure).
        one_launch = r["launches_per_step"] == 1
        per_launch_ms = ms_step if one_launch else None
        if r["kern_ms"] is not None:  # --kernel-events: bracket every launch (diagnostic)
            per_launch_ms = float(r["kern_ms"].mean())
        if per_launch_ms is not None:
            ach = float(r["launch_bytes"].mean()) / (per_launch_ms * 1e-3) / 1e9
        else:  # separate append and decode launches per step: the step is the unit
            ach = step_bytes / (ms_step * 1e-3) / 1e9
        res["roofline"] = dict(bound="hbm", achieved=ach, peak=PEAK_HBM_GBS, unit="GB/s",
                               frac=ach / PEAK_HBM_GBS,
                               traffic=traffic_from_profile("decode", source_hash(DECODE_SOURCES)),
                               kernel=("fused append + decode step" if r["fused"] else
                                       "decode (separate append)")
                               + ("" if one_launch else " (append + decode launches)"),
                               launches_per_step=r["launches_per_step"],
                               workgroups=r["grid_blocks"],
                               avg_launch_us=(per_launch_ms or ms_step) * 1e3,
                               bytes_per_launch=float(r["launch_bytes"].mean()))
        lat = r["lat"]
        keep = np.linspace(0, len(lat) - 1, min(len(lat), 40)).round().astype(int)
        res["latency_vs_t"] = [[int(lat[i][0]), round(float(lat[i][1]), 3)] for i in keep]
        res["flatness"] = flatness(lat, n, int(wl.T))
        if on["growth"] and not args.no_growth and args.workload == "multipage" and not full:
            res["growth"] = growth_curve(args, wl, lat)
    if args.copy_calibration:
        res["copy_calibration"] = copy_calibration()
        log(f"[bench] 1 GiB copy: {res['copy_calibration']['gbs']:.0f} GB/s")
    if on["batched"]:
        res["batched_mall_resident"] = b = steady_leg(args, "batched", 2000, 100)
        b["note"] = ("effective GB/s: the 211 MB step working set fits the 256 MB Infinity Cache, "
                     "so rows are partly served from it rather than from HBM")
        log(f"[bench] batched (MALL-resident): {b['us_per_step']:.2f} us/step, "
            f"{b['step_gbs']:.0f} GB/s effective")
    if on["single"]:
        res["single_fp32"] = s1 = steady_leg(args, "single", 64, 64)
        s1["note"] = "latency-bound (6.6 MB per step, cache-resident); GB/s effective"
        log(f"[bench] single-page fp32 B=1: {s1['us_per_step']:.2f} us/step")
    if on["ragged"] and not args.no_ragged:
        res["ragged"] = ragged_decode(args)
        log(f"[bench] ragged: {res['ragged']['us_per_step']:.1f} us/step, "
            f"{res['ragged']['step_gbs']:.0f} GB/s")
    if on["shared"] and not args.no_shared:
        res["shared_documents"] = sd = shared_documents(args)
        log(f"[bench] shared documents: paged {sd['paged']['us_per_step']:.1f} us/step, "
            f"copied {sd['copied']['us_per_step']:.1f} us/step ({sd['speedup']:.2f}x)")
    if on["graph"] and not args.no_graph:
        res["graph_loop"] = gl = graph_loop(args)
        for k2, r2 in gl.items():
            log(f"[bench] graph loop {k2}: eager {r2['eager_us_per_step']:.2f} us/step, "
                f"graph {r2['graph_us_per_step']:.2f} us/step")
    if on["prefill"] and not args.no_prefill:
        p = run_prefill(args)
        if p is not None:
            res["prefill"] = p
            log(f"[bench] prefill: {p['ms']:.3f} ms, {p['tflops']:.1f} TFLOP/s")
    if on["backward"] and not args.no_backward:
        bw = run_backward(args)
        res["backward"] = bw
        log(f"[bench] training pass: forward {bw['fwd_ms']:.3f} ms, backward {bw['bwd_ms']:.3f} ms "
            f"({bw['bwd_tflops']:.1f} TFLOP/s), fwd+bwd {bw['train_tflops']:.1f} TFLOP/s")
    if wl is not None and on["cpu"] and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
