#!/usr/bin/env python3
"""Benchmark of the paged KV hot path on one MI355X.

A step is one decode step of the whole batch through every layer:
    paged_attn_decode_plan (the batch state's work list: which pages each
    block reads for which query columns, shared prefix pages once), then for
    each layer: the append of one new token per sequence into its page
    through the block table, and the decode (split-K over pages and the
    cross-split combine).  Where the matrix-core page streams cover the pool
    (every closed profile at the configs' shapes) both are one call,
    paged_attn_decode_append_run; otherwise kv_append + paged_attn_decode_run.
Inputs are resident in HBM before timing; the step is idempotent (the same
positions are re-appended, the same contexts decoded).

Default workload: 8 sequences, 32 layers, 32 query / 8 KV heads, head_dim 128,
BF16 pages, contexts U[1, 32768] with a 4096-token prefix shared by sequences
0-3.  `value` is whole-step KV throughput in GB/s: algorithmic bytes (unique
KV bytes read by decode, plus append rows, queries and outputs) over the
measured step time.

Prints one JSON line.  Progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PCIE5_X16_GBS = 63.0
METRIC = "paged decode KV GB/s (% of HBM peak) + decode steps/s at C=8, 32K ctx"
PROFILES = os.path.join(ROOT, "profiles")
# sources of the decode kernel; the traffic summary is valid for this exact text
DECODE_SRC = [os.path.join(ROOT, "paged_kv_cache_03_amd", "csrc", f)
              for f in ("decode.hip", "decode_common.h", "qstream.hip", "codec_write.h", "stream_common.h",
                        "stream_plan.h", "stream_plan.hip")]


# sources of one paged_attn_verify call: the tile kernel and the page stream in chunk mode
VERIFY_SRC = [os.path.join(ROOT, "paged_kv_cache_03_amd", "csrc", "verify.hip")] + DECODE_SRC



def fused_append(wl) -> bool:
    """paged_attn_decode_append_run covers the pool: the page streams' shapes
    (at most 8 entries, Hq / H in {1, 2, 4, 8}; NVFP4 sides at D 128 / 256)."""
    gq = wl.Hq // wl.H
    fp4 = wl.profile in ("NVFP4_G16", "K8V4")
    dims = wl.D in ((128, 256) if fp4 else (64, 128, 256))
    return dims and wl.B <= 8 and wl.Hq % wl.H == 0 and gq in (1, 2, 4, 8)


def step_append_fused(wl) -> bool:
    """The step appends inside the run: that call writes one row per entry, at
    seq_len - 1, so it stands for the step's append only where every entry
    appends exactly one row; several rows per entry (config 3: 1-64, page
    crossings included) go through kv_append."""
    return fused_append(wl) and all(int(t) == 1 for t in wl.step)


def source_sha256(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def decode_source_sha256() -> str:
    return source_sha256(DECODE_SRC)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class KernelEvents:
    """HIP event pairs that the library records around the dominant kernel of
    an attention call (kv_trace_next_kernel): the kernel's own time on the
    stream it runs on, without the combine launch or launch gaps."""

    def __init__(self, n: int):
        import torch
        self.pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(n)]
        for a, b in self.pairs:              # torch creates the HIP event at its first record
            a.record()
            b.record()
        torch.cuda.synchronize()
        self.used = 0

    def arm(self) -> None:
        from paged_kv_cache_03_amd import _abi as abi
        a, b = self.pairs[self.used]
        abi.kv_trace_next_kernel(a.cuda_event, b.cuda_event)
        self.used += 1

    def mean_ms(self) -> float:
        import torch
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in self.pairs[:self.used]) / max(1, self.used)


def host_threads() -> dict:
    """The host the oracle runs on: CPUs the process may use, and the BLAS
    threads NumPy's matrix products use (the oracle's only parallel part)."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return {"cores": int(blas), "blas_threads": int(blas), "host_cpus": int(os.cpu_count() or 1),
            "cpus_available": int(avail)}


def bytes_per_token_head(profile: str, D: int, scale_bytes: int = 4) -> int:
    from paged_kv_cache_03_amd import _abi as abi
    dt = abi.KV_DT_F16 if scale_bytes == 2 else abi.KV_DT_F32
    return sum(p.x_extent * p.elem_bytes for p in abi.kv_profile_planes(abi.KV_PROFILE[profile], D, dt))


def kv_read_bytes(table, wl) -> tuple[int, int]:
    """(unique, logical) KV bytes decode reads: every valid (page, column) of every
    entry; a page shared by several entries counts once in `unique`."""
    import numpy as np
    bpth = bytes_per_token_head(wl.profile, wl.D, wl.scale_bytes)
    cols = {}
    logical = 0
    for b, ctx in enumerate(wl.seq_lens):
        row = table[wl.table_rows[b]]
        for p in range((ctx + 63) // 64):
            c = min(64, ctx - 64 * p)
            g = int(row[p])
            cols[g] = max(cols.get(g, 0), c)
            logical += c
    unique = int(np.sum(list(cols.values())))
    return unique * wl.H * bpth, logical * wl.H * bpth


def decode_kernel_name(wl) -> str:
    """The kernel that carries paged_attn_decode for this workload (as rocprofv3 names it)."""
    gq = wl.Hq // wl.H
    if gq in (1, 2, 4, 8) and wl.B <= 8:
        if wl.profile == "BF16" and wl.D in (64, 128, 256):
            return f"paged_vstream_kernel<{wl.D}, {gq}, 1, false>"
        # codec numbers of the page-stream instances: INT8-G64 1, FP8-row 2, NVFP4-G16 3
        sides = {"INT8_G64": (1, 1), "FP8_E4M3FN_ROW256": (2, 2), "NVFP4_G16": (3, 3), "K8V4": (2, 3)}
        if wl.profile in sides and (wl.D in (128, 256) or (wl.D == 64 and 3 not in sides[wl.profile])):
            kc, vc = sides[wl.profile]
            # last argument: bytes of an INT8-G64 / FP8-row scale
            sb = 2 if wl.scale_bytes == 2 and wl.profile != "NVFP4_G16" else 4
            return f"paged_qstream_kernel<{wl.D}, {kc}, {vc}, {sb}>"
    return "decode_split_kernel + decode_combine_kernel"


def measured_traffic(wl, kind: str = "decode", field: str = "traffic_bytes_per_dispatch") -> int | None:
    """HBM bytes per launch of the dominant kernel of a decode (kind "decode")
    or a verify call (kind "verify"; field "call_traffic_bytes": every kernel
    of the call) from the committed rocprofv3 counter summary (FETCH_SIZE +
    WRITE_SIZE, each scaled by what the same counter reads for a plain device
    copy of known size), or None when there is none for this workload or the
    sources have changed since it was taken."""
    path = os.path.join(PROFILES, f"{kind}_traffic_{wl.name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kind == "decode":
        sha, kernel = decode_source_sha256(), decode_kernel_name(wl)
    else:
        sha, kernel = source_sha256(VERIFY_SRC), verify_kernel_names(wl)
    if kv.get("source_sha256") != sha or kv.get("kernel") != kernel:
        return None
    try:
        return int(float(kv[field]))
    except (KeyError, ValueError):
        return None


def copy_calibration(n_bytes: int = 1 << 30, reps: int = 4) -> int:
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters of the decode kernel (run under rocprofv3 --pmc)."""
    import torch
    src = torch.ones(n_bytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n_bytes, "reps": reps}), flush=True)
    return 0


def cpu_baseline(wl, seconds_hint: float = 20.0) -> dict:
    """The oracle, as it stands, on a bounded sample of the same step: layer 0 of
    the workload (append of the step rows + paged decode of every entry and head)."""
    import numpy as np
    from oracle import attention as A
    from oracle.pool import OraclePool
    from oracle.store import OracleStore
    threads = host_threads()
    log("cpu baseline: building the oracle's pool for layer 0")
    pool = OraclePool(wl.S, wl.C, wl.M, free_order=wl.free_order)
    st = OracleStore(pool, wl.profile, wl.H, wl.D, 1, scale_bytes=wl.scale_bytes)
    sids = {}
    for b in wl.order():
        row = wl.table_rows[b]
        if wl.fork[b] is None:
            sids[b] = pool.open(row)
            n_inh = 0
        else:
            sids[b] = pool.fork(sids[wl.fork[b][0]], wl.fork[b][1], row)
            n_inh = wl.fork[b][1]
            if wl.hist[b] > n_inh and n_inh % 64:
                st.cow_copy(*pool.cow_tail(sids[b])[1])
        pool.ensure_mapped(sids[b], wl.hist[b])
        if wl.hist[b] > n_inh:
            k, v = wl.hist_kv(0, b)
            st.append(0, row, n_inh, k, v)
        pool.commit(sids[b], wl.hist[b])
    for b in range(wl.B):
        if wl.cow[b]:
            _, info = pool.cow_tail(sids[b])
            if info is not None:
                st.cow_copy(*info)
        pool.ensure_mapped(sids[b], wl.hist[b] + wl.step[b])
    steps = [wl.step_kv(0, b) for b in range(wl.B)]
    q = wl.q(0)
    log("cpu baseline: timing the oracle")
    reps, elapsed = 0, 0.0
    while reps == 0 or (elapsed < seconds_hint * 0.5 and reps < 3):
        t0 = time.perf_counter()
        for b in range(wl.B):
            st.append(0, wl.table_rows[b], wl.hist[b], *steps[b])
        A.paged_decode(st, 0, wl.table_rows, wl.seq_lens, q, wl.sm_scale)
        elapsed += time.perf_counter() - t0
        reps += 1
    unique, _ = kv_read_bytes(pool.table, wl)
    per_layer = elapsed / reps
    return {"value": round(unique / per_layer / 1e9, 4), "unit": "GB/s", **threads, "kind": "oracle",
            "sample": f"layer 0 of {wl.layers}: append of the step rows + decode of all {wl.B} entries x {wl.Hq} "
                      f"heads, {reps} rep(s), {per_layer:.2f} s per layer (KV bytes read / time)"}


def cpu_baseline_verify(wl, seconds_hint: float = 20.0) -> dict:
    """The oracle, as it stands, on a bounded sample of the verify workload: the
    first entry with a short chunk (a speculative verify, T = 5) over its whole
    history, layer 0.  Reported as TFLOP/s of the same algorithmic work."""
    import numpy as np
    from oracle import attention as A
    from oracle.pool import OraclePool
    from oracle.store import OracleStore
    threads = host_threads()
    sample = [b for b in range(wl.B) if wl.step[b] <= 8 and wl.fork[b] is None][:1]
    log(f"cpu baseline: the oracle's pool for entries {sample}")
    pool = OraclePool(wl.S, wl.C, wl.M, free_order=wl.free_order)
    st = OracleStore(pool, wl.profile, wl.H, wl.D, 1, scale_bytes=wl.scale_bytes)
    for b in sample:
        row = wl.table_rows[b]
        sid = pool.open(row)
        pool.ensure_mapped(sid, wl.hist[b] + wl.step[b])
        k, v = wl.hist_kv(0, b)
        st.append(0, row, 0, k, v)
        pool.commit(sid, wl.hist[b])
        st.append(0, row, wl.hist[b], *wl.step_kv(0, b))
    q_all = wl.q(0)
    rows = [wl.table_rows[b] for b in sample]
    n0s = [wl.hist[b] for b in sample]
    cu = [0]
    for b in sample:
        cu.append(cu[-1] + wl.step[b])
    q = np.concatenate([q_all[wl.cu_q[b]:wl.cu_q[b + 1]] for b in sample])
    log("cpu baseline: timing the oracle")
    reps, elapsed = 0, 0.0
    while reps == 0 or (elapsed < seconds_hint * 0.5 and reps < 3):
        t0 = time.perf_counter()
        A.paged_verify(st, 0, rows, n0s, cu, q, wl.sm_scale)
        elapsed += time.perf_counter() - t0
        reps += 1
    pairs = sum(n0 * T + T * (T + 1) // 2 for n0, T in ((wl.hist[b], wl.step[b]) for b in sample))
    flops = 4.0 * wl.D * wl.Hq * pairs
    per = elapsed / reps
    return {"value": round(flops / per / 1e12, 6), "unit": "TFLOP/s", **threads, "kind": "oracle",
            "sample": f"layer 0: one verify chunk of {wl.step[sample[0]]} tokens over its {n0s[0]}-token history, "
                      f"all {wl.Hq} heads, {reps} rep(s), {per:.2f} s each"}


MFMA_BF16_PEAK_TFLOPS = 2500.0


# codec numbers of the kernel instances: BF16 0, INT8-G64 1, FP8-row 2, NVFP4-G16 3
CODECS = {"BF16": (0, 0), "INT8_G64": (1, 1), "FP8_E4M3FN_ROW256": (2, 2), "NVFP4_G16": (3, 3), "K8V4": (2, 3)}


def gtile_name(wl) -> str:
    kc, vc = CODECS[wl.profile]
    sb = 2 if wl.scale_bytes == 2 and wl.profile in ("INT8_G64", "FP8_E4M3FN_ROW256", "K8V4") else 4
    return f"verify_gtile_kernel<{wl.D}, {wl.Hq // wl.H}, {kc}, {vc}, {sb}>"


def bf16_tiles(wl) -> bool:
    return wl.profile == "BF16" and wl.D in (64, 128) and wl.Hq // wl.H in (1, 2, 4, 8)


def verify_dominant_kernel(wl) -> str:
    """The kernel that carries most of a paged_attn_verify call (rocprofv3 name)."""
    gq = wl.Hq // wl.H
    if bf16_tiles(wl):
        if max(wl.step) * gq > 32:
            return f"verify_tile_kernel<{wl.D}, {gq}>"
        return f"paged_vstream_kernel<{wl.D}, {gq}, 2, true>"
    return gtile_name(wl)


def verify_kernel_names(wl) -> str:
    gq = wl.Hq // wl.H
    if bf16_tiles(wl):
        return f"verify_tile_kernel<{wl.D}, {gq}> + paged_vstream_kernel<{wl.D}, {gq}, 2, true>"
    return gtile_name(wl) + " (+ gtile_combine_kernel when its tiles are split)"


def bench_verify(wl, args) -> int:
    """Verify / chunked-prefill step (the mixed batch of the workload): per layer,
    kv_append of every chunk's rows, then paged_attn_verify.  The verify launch
    is bound by the matrix cores (prefill chunks) and HBM (short chunks); the
    roofline is reported on the algorithmic FLOPs 4*D*Hq*sum(n0*T + T(T+1)/2)."""
    import numpy as np
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    from workloads.device_driver import _dev, build_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    log(f"workload {wl.name}: filling {wl.layers} layer(s) of history")
    dp, _, step_inputs = build_device(wl, zero=False, head_major=args.head_major)
    log(f"history resident after {time.time() - t0:.1f} s")
    rows_t, pos0_t, cu_t = i32(wl.table_rows, dev), i32(wl.hist, dev), i32(wl.cu_q, dev)
    total = int(wl.cu_q[-1])
    msl, mql = max(wl.seq_lens), max(wl.step)
    qs = [_dev(wl.q(layer), dev) for layer in range(wl.layers)]
    out = torch.empty((total, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    ws = dp.workspace(wl.B, wl.Hq, msl, mql)

    def step(events=None, kern=None):
        for layer in range(wl.layers):
            kd, vd = step_inputs[layer]
            dp.append(layer, rows_t, pos0_t, cu_t, total, kd, vd)
            if events is not None:
                events[layer][0].record()
            if kern is not None:
                kern.arm()
            dp.verify(layer, wl.Hq, rows_t, pos0_t, cu_t, total, mql, msl, qs[layer], wl.sm_scale, out, ws)
            if events is not None:
                events[layer][1].record()

    steps = max(1, min(args.steps, 10))
    for _ in range(min(args.warmup, 2)):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / steps
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(wl.layers)] for _ in range(steps)]
    kern = KernelEvents(wl.layers * steps)
    for s_ in range(steps):
        step(evs[s_], kern)
    torch.cuda.synchronize()
    ver_ms = float(np.mean([a.elapsed_time(b) for row in evs for (a, b) in row]))
    kern_ms = kern.mean_ms()

    pairs = sum(n0 * T + T * (T + 1) // 2 for n0, T in zip(wl.hist, wl.step))
    flops = 4.0 * wl.D * wl.Hq * pairs                      # per layer
    # the dominant kernel: the prefill tiles take the chunks wider than 32
    # query columns (tokens x query heads per KV head); the rest go through
    # the page stream in chunk mode before them
    gq = wl.Hq // wl.H
    wide = [(n0, T) for n0, T in zip(wl.hist, wl.step) if T * gq > 32] if bf16_tiles(wl) else []
    kern_flops = 4.0 * wl.D * wl.Hq * sum(n0 * T + T * (T + 1) // 2 for n0, T in (wide or zip(wl.hist, wl.step)))
    kern_tflops = kern_flops / (kern_ms * 1e-3) / 1e12
    table = dp.table.cpu().numpy()
    bpth = bytes_per_token_head(wl.profile, wl.D, wl.scale_bytes)
    kv_bytes = sum(len({int(table[wl.table_rows[b], p]) for p in range((c + 63) // 64)}) * 64 * wl.H * bpth
                   for b, c in enumerate(wl.seq_lens))
    tflops = flops / (ver_ms * 1e-3) / 1e12
    line = {
        "metric": f"paged verify/prefill TFLOP/s (mixed batch: verify T=5 + prefill T=512, C=4, "
                  f"{wl.S // 1024}K ctx, {wl.profile} pages)",
        "value": round(flops * wl.layers / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": min(args.warmup, 2), "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name, "profile": wl.profile, "batch": wl.B, "layers": wl.layers,
                   "q_heads": wl.Hq, "kv_heads": wl.H, "head_dim": wl.D, "chunk_tokens": list(wl.step),
                   "frontiers": list(wl.hist), "page_size": 64, "pool_pages": wl.M},
        "roofline": {"kernel": verify_dominant_kernel(wl), "bound": "mfma", "achieved": round(kern_tflops, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(wl, "verify"), "flops_per_launch": kern_flops,
                     "launch_ms": round(kern_ms, 5),
                     "call": {"kernels": verify_kernel_names(wl), "flops": flops, "kv_bytes": kv_bytes,
                              "traffic": measured_traffic(wl, "verify", "call_traffic_bytes"),
                              "ms": round(ver_ms, 5), "tflops": round(tflops, 2),
                              "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_verify(wl),
    }
    print(json.dumps(line), flush=True)
    dp.close()
    return 0


def bench_spec(wl, args) -> int:
    """Speculative rounds on the histories of the verify workload: per round and
    entry, map T = 5 draft rows (from the entry's reservation first), append
    them, one paged_attn_verify call for the batch (5-token chunks: the page
    stream, bound by HBM), then commit a seeded accepted prefix (1..5 rows)
    and trim the trailing pages into the entry's reservation.  The frontiers
    advance by the accepted rows, so each round reads a slightly longer
    history.  `value` is rounds per second; the roofline covers the verify
    call (KV bytes of the four histories per launch)."""
    import numpy as np
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    from workloads.device_driver import _dev, build_device
    from workloads.gen import bf16_normal, rng_for

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    log(f"workload {wl.name}: filling the history for speculative rounds")
    dp, seqs, _ = build_device(wl, zero=False, step_append=False)
    log(f"history resident after {time.time() - t0:.1f} s")
    T, B = 5, wl.B
    rounds = max(1, min(args.steps, 40))
    warm = min(args.warmup, 3)
    total_rounds = warm + 2 * rounds
    r = rng_for(7700, 0)
    acc = r.integers(1, T + 1, size=(total_rounds, B))
    if max(wl.hist) + int(acc.sum(axis=0).max()) + T > wl.S:
        raise SystemExit("speculative rounds would pass the maximum context")
    kd = _dev(bf16_normal(r, (B * T, wl.H, wl.D)), dev)
    vd = _dev(bf16_normal(r, (B * T, wl.H, wl.D)), dev)
    qd = _dev(bf16_normal(r, (B * T, wl.Hq, wl.D)), dev)
    rows_t, cu_t = i32(wl.table_rows, dev), i32([T * b for b in range(B + 1)], dev)
    out = torch.empty((B * T, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    max_ctx = wl.S
    ws = dp.workspace(B, wl.Hq, max_ctx, T)
    front = list(wl.hist)
    # one pinned host buffer of frontiers per round, copied to the device in order
    pos_host = torch.empty((total_rounds, B), dtype=torch.int32, pin_memory=True)
    pos_dev = torch.empty((total_rounds, B), dtype=torch.int32, device=dev)
    host_s = [0.0]

    def one(k, events=None):
        h0 = time.perf_counter()
        for b in range(B):
            dp.ensure_mapped(seqs[b], front[b] + T)
        pos_host[k] = torch.tensor(front, dtype=torch.int32)
        host_s[0] += time.perf_counter() - h0
        pos_dev[k].copy_(pos_host[k], non_blocking=True)
        dp.append(0, rows_t, pos_dev[k], cu_t, B * T, kd, vd)
        if events is not None:
            events[0].record()
            kern.arm()
        dp.verify(0, wl.Hq, rows_t, pos_dev[k], cu_t, B * T, T, max_ctx, qd, wl.sm_scale, out, ws)
        if events is not None:
            events[1].record()
        h0 = time.perf_counter()
        for b in range(B):
            dp.commit_accepted(seqs[b], T, int(acc[k, b]))
            front[b] += int(acc[k, b])
        host_s[0] += time.perf_counter() - h0

    for k in range(warm):
        one(k)
    torch.cuda.synchronize()
    host_s[0] = 0.0
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(warm, warm + rounds):
        one(k)
    end.record()
    torch.cuda.synchronize()
    ms_round = start.elapsed_time(end) / rounds
    host_us = host_s[0] / rounds * 1e6
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(rounds)]
    kern = KernelEvents(rounds)
    for i, k in enumerate(range(warm + rounds, warm + 2 * rounds)):
        one(k, evs[i])
    torch.cuda.synchronize()
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    ver_ms = kern.mean_ms()
    a_, res_, v_ = dp.stats()
    reserved = [dp.reservation(seqs[b]) for b in range(B)]
    bpth = bytes_per_token_head(wl.profile, wl.D, wl.scale_bytes)
    kv_bytes = sum(front) * wl.H * bpth          # the last round's histories, about those of every round
    achieved = kv_bytes / (ver_ms * 1e-3) / 1e9
    line = {
        "metric": "speculative verify rounds/s (C=4, T=5 drafts, commit accepted + trim, 128K ctx)",
        "value": round(1000.0 / ms_round, 2), "unit": "rounds/s", "n_gpus": 1, "steps": rounds, "warmup": warm,
        "ms_per_step": round(ms_round, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + "_spec_rounds", "profile": wl.profile, "batch": B, "layers": 1,
                   "q_heads": wl.Hq, "kv_heads": wl.H, "head_dim": wl.D, "draft_tokens": T,
                   "accepted_mean": round(float(acc.mean()), 3), "frontiers_start": list(wl.hist),
                   "page_size": 64, "pool_pages": wl.M},
        "host_us_per_round": round(host_us, 1),
        "pool_after": {"allocated": a_, "reserved": res_, "available": v_, "reserved_per_entry": reserved},
        "roofline": {"kernel": "paged_vstream_kernel<%d, %d, 2, true>" % (wl.D, wl.Hq // wl.H), "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": kv_bytes,
                     "launch_ms": round(ver_ms, 5), "call_ms": round(call_ms, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    dp.close()
    return 0


def bench_replica(wl, args) -> int:
    """Host replica of the longest entry of a decode workload, every layer:
    kv_seq_offload into pinned host memory (device to host), release, then
    kv_seq_restore into the same row (host to device).  Reports the bytes of
    full page payloads moved per second each way; a decode of the restored
    row is checked against the original bit for bit."""
    import numpy as np
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    from workloads.device_driver import _dev, build_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    log(f"workload {wl.name}: filling {wl.layers} layer(s) of history")
    dp, seqs, _ = build_device(wl, zero=False)
    log(f"history resident after {time.time() - t0:.1f} s")
    # the longest entry that shares no pages (no fork source or fork)
    private = [x for x in range(wl.B)
               if wl.fork[x] is None and not any(fk is not None and fk[0] == x for fk in wl.fork)]
    b = max(private, key=lambda x: wl.hist[x])
    row, f = wl.table_rows[b], wl.hist[b]
    n = -(-f // 64)
    pb = dp.replica_page_bytes()
    host = torch.empty(n * pb, dtype=torch.uint8, pin_memory=True)
    q = _dev(wl.q(0)[b:b + 1], dev)
    ws = dp.workspace(1, wl.Hq, f)

    def decode(r_):
        out = torch.empty((1, wl.Hq, wl.D), dtype=torch.float32, device=dev)
        dp.decode(0, wl.Hq, i32([r_], dev), i32([f], dev), f, q, wl.sm_scale, out, ws)
        return out

    ref = decode(row)
    reps = max(1, min(args.steps, 5))
    d2h, h2d = [], []
    seq = seqs[b]
    for _ in range(reps + 1):
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        torch.cuda.synchronize()
        e0.record()
        dp.offload(seq, host)
        e1.record()
        torch.cuda.synchronize()
        dp.release(seq)
        e1b = torch.cuda.Event(enable_timing=True)
        e1b.record()
        seq = dp.restore(row, host, f)
        e2.record()
        torch.cuda.synchronize()
        d2h.append(e0.elapsed_time(e1))
        h2d.append(e1b.elapsed_time(e2))
    d2h, h2d = d2h[1:], h2d[1:]                   # the first round trip is warm-up
    same = bool(torch.equal(decode(row), ref))
    total = n * pb
    line = {
        "metric": "host replica GB/s (offload D2H / restore H2D of full page payloads, every layer)",
        "value": round(total / (np.mean(d2h) * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": reps,
        "warmup": 1, "ms_per_step": round(float(np.mean(d2h) + np.mean(h2d)), 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bytes", "data": "synthetic",
        "config": {"workload": wl.name + "_replica", "profile": wl.profile, "layers": wl.layers,
                   "kv_heads": wl.H, "head_dim": wl.D, "entry_tokens": f, "pages": n, "page_bytes": pb},
        "offload_gbs": round(total / (np.mean(d2h) * 1e-3) / 1e9, 2),
        "restore_gbs": round(total / (np.mean(h2d) * 1e-3) / 1e9, 2),
        "offload_ms": round(float(np.mean(d2h)), 4), "restore_ms": round(float(np.mean(h2d)), 4),
        "restored_decode_bitwise_equal": same,
        # the host link: PCIe 5.0 x16, 32 GT/s x 16 lanes with 128b/130b coding = 63.0 GB/s each way
        "roofline": {"kernel": "replica_copy_kernel", "bound": "pcie",
                     "achieved": round(total / (np.mean(d2h) * 1e-3) / 1e9, 2), "peak": PCIE5_X16_GBS,
                     "unit": "GB/s", "frac": round(total / (np.mean(d2h) * 1e-3) / 1e9 / PCIE5_X16_GBS, 4),
                     "traffic": None, "bytes_per_launch": total, "launch_ms": round(float(np.mean(d2h)), 4)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    dp.close()
    return 0 if same else 1


def bench_read_ceiling(args) -> int:
    """The HBM read ceiling of the decode's access pattern (kv_read_probe): per
    launch, 22,300 distinct random 16 KiB slices (365 MB, the BF16 K and V
    slices one decode of the 8-sequence 32K workload reads) out of an 8 GiB
    buffer, 32 different slice lists in rotation as the 32 layers of a step
    rotate, so the launches stream from HBM rather than the 256 MB
    Infinity Cache.  Sweeps blocks per compute unit (4 waves each); `value` is
    the best mean rate.  A secondary denominator for the decode kernel."""
    import numpy as np
    import torch
    from paged_kv_cache_03_amd import _abi as abi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    slice_bytes, n, lists = 16384, 22300, 32
    buf_bytes = 8 << 30
    buf = torch.empty(buf_bytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    r = np.random.default_rng(31)
    ids = [torch.from_numpy(r.choice(buf_bytes // slice_bytes, n, replace=False).astype(np.int32)).to(dev)
           for _ in range(lists)]
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    reps = max(1, min(args.steps, 20))
    results = {}
    for bpc in (1, 2, 4, 8):
        def launch(i):
            abi.kv_read_probe(buf.data_ptr(), ids[i % lists].data_ptr(), n, slice_bytes, bpc, sink.data_ptr(), stream)
        for i in range(lists):
            launch(i)
        torch.cuda.synchronize()
        # back-to-back launches of all 32 lists between one event pair (an
        # event pair around each launch would add its own packets' time)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            for i in range(lists):
                launch(i)
            b.record()
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in ev]) / lists
        results[bpc] = {"mean_gbs": round(n * slice_bytes / (ms.mean() * 1e-3) / 1e9, 1),
                        "best_gbs": round(n * slice_bytes / (ms.min() * 1e-3) / 1e9, 1),
                        "mean_us": round(float(ms.mean()) * 1e3, 2)}
        log(f"blocks per CU {bpc}: {results[bpc]}")
    best = max(results, key=lambda k: results[k]["mean_gbs"])
    value = results[best]["mean_gbs"]
    line = {
        "metric": "HBM read ceiling of the decode access pattern (random 16 KiB slices, read once)",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": round(results[best]["mean_us"] * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bytes", "data": "synthetic",
        "config": {"workload": "read_probe_16k_slices_365MB", "slice_bytes": slice_bytes, "slices_per_launch": n,
                   "slice_lists": lists, "buffer_bytes": buf_bytes},
        "by_blocks_per_cu": results, "best_blocks_per_cu": best,
        "roofline": {"kernel": f"read_probe_kernel<16>", "bound": "hbm", "achieved": value, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": n * slice_bytes, "launch_ms": round(results[best]["mean_us"] * 1e-3, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_advance(wl, args) -> int:
    """Advancing decode: K steps in which every entry's frontier moves by one
    token.  Per step, on the host: commit the previous token and map the next
    one (a new page group at each page crossing, published on the stream);
    then the device step as in the default run -- the plan of the new batch
    state and, per layer, the append of the new rows with the decode.  The
    rows and queries are those of the workload's step (their values do not
    change the work).  Reports the step rate next to the host time per step."""
    import numpy as np
    import torch
    from paged_kv_cache_03_amd.device_pool import i32
    from workloads.device_driver import _dev, build_device

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if any(t != 1 for t in wl.step):
        raise SystemExit("--advance takes a workload with one new token per entry")
    t0 = time.time()
    log(f"workload {wl.name}: filling {wl.layers} layer(s) of history")
    dp, seqs, step_inputs = build_device(wl, zero=False)
    log(f"history resident after {time.time() - t0:.1f} s")
    steps = max(1, min(args.steps, 64))
    warm = min(args.warmup, 5)
    lens = list(wl.seq_lens)
    if max(lens) + warm + steps > wl.S:
        raise SystemExit("the advancing run would pass the maximum context")
    bound = max(lens) + warm + steps               # grid bound for every step of the run
    rows_t = i32(wl.table_rows, dev)
    # per step, pinned host rows of (lengths, append positions) copied in stream order
    lp_host = torch.empty((warm + steps, 2, wl.B), dtype=torch.int32, pin_memory=True)
    lp_dev = torch.empty((warm + steps, 2, wl.B), dtype=torch.int32, device=dev)
    cu_t = i32(list(range(wl.B + 1)), dev)
    qs = [_dev(wl.q(layer), dev) for layer in range(wl.layers)]
    out = torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    ws = dp.workspace(wl.B, wl.Hq, bound)
    fused = fused_append(wl)
    host_s = [0.0]
    crossings = [0]

    def step(k):
        h0 = time.perf_counter()
        for b in range(wl.B):
            dp.commit(seqs[b], lens[b])            # the previous step's token is committed
            lens[b] += 1
            if lens[b] % 64 == 1:
                crossings[0] += 1
            dp.ensure_mapped(seqs[b], lens[b])     # a new group only at a page crossing
        lp_host[k] = torch.tensor([lens, [n - 1 for n in lens]], dtype=torch.int32)
        host_s[0] += time.perf_counter() - h0
        lp_dev[k].copy_(lp_host[k], non_blocking=True)
        lens_k, pos_k = lp_dev[k, 0], lp_dev[k, 1]
        dp.decode_plan(wl.Hq, rows_t, lens_k, bound, ws)
        for layer in range(wl.layers):
            kd, vd = step_inputs[layer]
            if fused:
                dp.decode_append_run(layer, wl.B, wl.Hq, bound, kd, vd, qs[layer], wl.sm_scale, out, ws)
            else:
                dp.append(layer, rows_t, pos_k, cu_t, wl.B, kd, vd)
                dp.decode_run(layer, wl.B, wl.Hq, bound, qs[layer], wl.sm_scale, out, ws)

    for k in range(warm):
        step(k)
    torch.cuda.synchronize()
    host_s[0], crossings[0] = 0.0, 0
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(warm, warm + steps):
        step(k)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    table = dp.table.cpu().numpy()
    unique, _ = kv_read_bytes(table, wl)          # the histories at the start: within steps/ctx of every step's
    bpth = bytes_per_token_head(wl.profile, wl.D, wl.scale_bytes)
    per_step = wl.layers * (unique + wl.B * wl.Hq * wl.D * 6 + wl.B * wl.H * (bpth + 4 * wl.D))
    line = {
        "metric": METRIC + " (advancing: frontiers grow every step)", "value": round(per_step / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.profile == "BF16" else wl.profile.lower(), "data": "synthetic",
        "config": {"workload": wl.name + "_advancing", "profile": wl.profile, "batch": wl.B, "layers": wl.layers,
                   "ctx_sum_start": int(sum(wl.seq_lens)), "page_crossings": crossings[0]},
        "steps_per_s": round(1000.0 / ms, 2),
        "host_us_per_step": round(host_s[0] / steps * 1e6, 1),
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    dp.close()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2,
                    help="workload number (1-4: decode, 5: verify/prefill; 6, 7: BF16 at head_dim 256; "
                         "8, 9: verify/prefill on INT8-G64 and K8V4 pools)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--scale-bytes", type=int, choices=(2, 4), default=4,
                    help="INT8-G64 / FP8-row scale planes: 4 (fp32) or 2 (binary16, the page's D256 byte table)")
    ap.add_argument("--head-major", action="store_true",
                    help="decode and verify configs: planes in the head-major order [X, P, N, H]")
    ap.add_argument("--graph", action="store_true",
                    help="decode configs: time replays of the step captured as one HIP graph")
    ap.add_argument("--advance", action="store_true",
                    help="decode configs with one token per entry: frontiers grow every step (host mapping timed in)")
    ap.add_argument("--replica", action="store_true",
                    help="decode configs: offload / restore of the longest entry's pages (host replica)")
    ap.add_argument("--spec", action="store_true",
                    help="with --config 5: speculative rounds (draft, verify, commit the accepted prefix, trim)")
    ap.add_argument("--read-ceiling", action="store_true",
                    help="only measure the HBM read ceiling of the decode's access pattern (kv_read_probe)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration under rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("one GPU only: --gpus must be 1 (the path runs on one GPU's share; no collectives)",
              file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration()
    if args.read_ceiling:
        return bench_read_ceiling(args)

    import numpy as np
    import torch

    import workloads
    from paged_kv_cache_03_amd.device_pool import i32
    from workloads.device_driver import _dev, build_device

    wl = workloads.get(args.config)
    if args.scale_bytes != 4:
        wl.scale_bytes = args.scale_bytes
        wl.name += f"_scales{8 * args.scale_bytes}bit"
    if args.head_major:
        if wl.mode not in ("decode", "verify") or args.spec or args.replica or args.advance:
            print("--head-major applies to the plain decode and verify runs", file=sys.stderr)
            return 2
        wl.name += "_headmajor"
    if args.spec:
        if wl.mode != "verify":
            print("--spec needs the verify workload (--config 5)", file=sys.stderr)
            return 2
        return bench_spec(wl, args)
    if wl.mode != "decode":
        return bench_verify(wl, args)
    if args.replica:
        return bench_replica(wl, args)
    if args.advance:
        return bench_advance(wl, args)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    log(f"workload {wl.name}: filling {wl.layers} layer(s) of history")
    dp, _, step_inputs = build_device(wl, zero=False, head_major=args.head_major)
    log(f"history resident after {time.time() - t0:.1f} s")

    rows_t, pos0_t, cu_t = i32(wl.table_rows, dev), i32(wl.hist, dev), i32(wl.cu_q, dev)
    lens_t = i32(wl.seq_lens, dev)
    total = int(wl.cu_q[-1])
    max_ctx = max(wl.seq_lens)
    qs = [_dev(wl.q(layer), dev) for layer in range(wl.layers)]
    out = torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device=dev)
    ws = dp.workspace(wl.B, wl.Hq, max_ctx)

    # one step: the work list of the batch state once (it depends only on the
    # block table and the lengths), then per layer the append of the step's
    # rows and the decode run -- one launch on the page streams, which
    # append the rows themselves
    fused = step_append_fused(wl)

    def step(events=None, kern=None):
        dp.decode_plan(wl.Hq, rows_t, lens_t, max_ctx, ws)
        for layer in range(wl.layers):
            kd, vd = step_inputs[layer]
            if not fused:
                dp.append(layer, rows_t, pos0_t, cu_t, total, kd, vd)
            if events is not None:
                events[layer][0].record()
            if kern is not None:
                kern.arm()
            if fused:
                dp.decode_append_run(layer, wl.B, wl.Hq, max_ctx, kd, vd, qs[layer], wl.sm_scale, out, ws)
            else:
                dp.decode_run(layer, wl.B, wl.Hq, max_ctx, qs[layer], wl.sm_scale, out, ws)
            if events is not None:
                events[layer][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        # the same step as one HIP graph: plan, then per layer the append and the run
        outs = [out] * wl.layers
        ks = [step_inputs[layer][0] for layer in range(wl.layers)]
        vs = [step_inputs[layer][1] for layer in range(wl.layers)]
        # the fused form (no positions: one row per entry at seq_len - 1) where the eager step uses it
        graph = dp.step_graph(wl.B, wl.Hq, rows_t, lens_t, max_ctx, qs, wl.sm_scale, outs, ws, ks=ks, vs=vs,
                              pos0=None if fused else pos0_t, cu=None if fused else cu_t, total_tokens=total)
        eager_step = step

        def step(events=None, kern=None):
            if events is not None or kern is not None:
                eager_step(events, kern)
            else:
                dp.graph_launch(graph)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()

    # timed region: K whole steps, no probes inside
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    log(f"{ms_per_step:.4f} ms per step")

    # the same K steps again, with HIP events around every decode call (the
    # call: page stream, combine and their launches) and, recorded by the
    # library on the stream it launches on, around the page-stream kernel alone
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(wl.layers)] for _ in range(args.steps)]
    kern = KernelEvents(wl.layers * args.steps)
    for s in range(args.steps):
        step(evs[s], kern)
    torch.cuda.synchronize()
    call_ms = float(np.mean([a.elapsed_time(b) for row in evs for (a, b) in row]))
    dec_ms = kern.mean_ms()

    table = dp.table.cpu().numpy()
    unique, logical = kv_read_bytes(table, wl)
    bpth = bytes_per_token_head(wl.profile, wl.D, wl.scale_bytes)
    qo_bytes = wl.B * wl.Hq * wl.D * (2 + 4)
    append_bytes = total * wl.H * (bpth + 2 * 2 * wl.D)
    per_decode = unique + qo_bytes
    per_step = wl.layers * (per_decode + append_bytes)
    value = per_step / (ms_per_step * 1e-3) / 1e9
    achieved = per_decode / (dec_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if wl.profile == "BF16" else wl.profile.lower(), "data": "synthetic",
        "config": {"workload": wl.name, "profile": wl.profile, "batch": wl.B, "layers": wl.layers, "q_heads": wl.Hq,
                   "kv_heads": wl.H, "head_dim": wl.D, "ctx_sum": int(sum(wl.seq_lens)), "ctx_max": int(max_ctx),
                   "page_size": 64, "pool_pages": wl.M, "scale_bytes": wl.scale_bytes,
                   "plane_order": "head_major" if args.head_major else "page_major"},
        "steps_per_s": round(1000.0 / ms_per_step, 2),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "step_form": "hip_graph" if graph is not None else "eager",
        "kv_bytes_per_step": {"unique": wl.layers * unique, "logical": wl.layers * logical},
        "roofline": {"kernel": decode_kernel_name(wl), "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl),
                     "bytes_per_launch": per_decode, "launch_ms": round(dec_ms, 5),
                     "call_ms": round(call_ms, 5),
                     "call_frac": round(per_decode / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if graph is not None:
        dp.graph_destroy(graph)
    dp.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
