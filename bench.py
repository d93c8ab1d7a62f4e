#!/usr/bin/env python3
"""Decode-step benchmark of the INT2 paged KV cache on one MI355X.

Workload: a Qwen3-8B-shaped model's attention, 36 layers x (32 query heads, 8 KV heads,
head_dim 128), batch 32, 100000-token context per sequence, INT2 history with a BF16 sink
(64) and recent window (256), 64-token pages in a shuffled physical order.  Keys and values
are synthetic (seeded, drawn on the GPU); rotations are calibrated per (layer, KV head) from
seeded queries.

One step = for every layer one decode-step call: the decode-step write (evict the oldest window
token of each sequence into INT2, append one new token per sequence), sharing its launch with the
query preparation, then decode attention for all 32 query heads.  Prints one JSON line (stdout);
progress goes to stderr.
"""
import argparse
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0
METRIC = "INT2 paged decode-attn achieved HBM GB/s (% peak) + steps/s @100K ctx, B=32"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def split_kernel_bytes(lens, n2s, hkv):
    """Algorithmic bytes of one launch of the decode split kernel: per (sequence, KV head) the
    INT2 tokens (32 B key codes + 32 B value codes + 16 B scales/minimums) and the BF16 sink and
    window tokens (256 B key + 256 B value row), plus each sequence's page ids."""
    b = 0
    for L, n2 in zip(lens, n2s):
        b += hkv * (80 * n2 + 512 * (L - n2))
        b += 4 * (-(-n2 // 64))
    return b


def decode_bytes(lens, n2s, hq, hkv):
    """Algorithmic bytes of one decode_attn call (per layer): the split kernel's, the bf16
    queries read, the fp32 outputs written and the fp32 rotations read once."""
    return split_kernel_bytes(lens, n2s, hkv) + len(lens) * hq * 128 * (2 + 4) + hkv * 128 * 128 * 4


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "k_decode_mfma_g4_100k_b32_traffic.txt")
KERNEL_SOURCES = ["decode_mfma.hip", "common.h", "launch.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "decode_attention_write_amd", "csrc",
                               name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per split-kernel launch from the committed counter summary, or None when the
    kernel sources changed since the counters were taken (or no summary exists)."""
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE) if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != kernel_source_hash():
        return None
    return int(kv["hbm_bytes_per_launch"])


def evict_bytes(n_seqs, hkv):
    return n_seqs * (hkv * (512 + 80) + 4)


def append_bytes(n_seqs, hkv):
    return n_seqs * hkv * (512 + 512) + hkv * 128 * 128 * 4


CPU_UNITS = [(s, (5 * s + 3) % 8) for s in range(32)]     # (seq, kv head): one per sequence


def export_units(st, seqs_kv):
    """Host copies of the store state of (seq, kv head) units: their pages, ring slots, lengths."""
    import numpy as np
    import torch
    torch.cuda.synchronize()
    table = st.page_table()
    out = []
    for s, kv in seqs_kv:
        L, n2 = st.seq_info(s)
        n_pages = -(-n2 // 64)
        pages = torch.from_numpy(table[s, :n_pages].astype(np.int64)).cuda()
        pool_u = st.pool_view()[pages, kv].cpu().numpy()[:, None, :]          # [n_pages, 1, 5120]
        ring_u = st.ring_view()[s, kv].cpu().numpy().view(np.uint16)[None, None]  # [1, 1, 2, 320, 128]
        out.append((s, kv, L, n2, pool_u, ring_u))
    return out


def _cpu_job(job):
    """One sampled unit of CPU-oracle work in a worker process (no GPU use), single-threaded BLAS.
    Returns (seconds of the timed part, output or None).  Jobs:
      ("warm",)                                        imports only
      ("decode", L, n2, pool_u, ring_u, rot, q, g)     decode attention of one (seq, KV head)
                                                       unit on its exported store state
      ("write", cfg, layer, seq, kv, n, rot1)          first write of n tokens into an empty
                                                       one-head store (inputs drawn untimed)
      ("appends", cfg, layer, seq, kv, L, n, rot1)     n single-token decode-step writes (evict
                                                       when the window is full, append) after an
                                                       untimed first write of L tokens
    """
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass
    import synth
    from oracle import attention, store as ostore
    kind = job[0]
    if kind == "warm":
        return 0.0, None
    if kind == "decode":
        _, L, n2, pool_u, ring_u, rot, q, g = job
        table_u = np.arange(pool_u.shape[0], dtype=np.int32)[None, :]
        t1 = time.perf_counter()
        out = attention.decode(pool_u, ring_u, table_u, np.array([L]), np.array([n2]), rot, q, [0],
                               1 / math.sqrt(128), g)
        return time.perf_counter() - t1, out
    if kind == "write":
        _, cfg, layer, seq, kv, n, rot1 = job
        kb, vb = synth.unit_kv(cfg, layer, seq, kv, n)
        pages = -(-max(0, n - 320) // 64) + 1
        st = ostore.OracleStore(1, 1, pages, pages, range(pages), rot1)
        t1 = time.perf_counter()
        st.write([0], kb[None, :, None, :], vb[None, :, None, :])
        return time.perf_counter() - t1, None
    if kind == "appends":
        _, cfg, layer, seq, kv, L, n, rot1 = job
        kb, vb = synth.unit_kv(cfg, layer, seq, kv, L + n)
        pages = -(-(L + n) // 64) + 1
        st = ostore.OracleStore(1, 1, pages, pages, range(pages), rot1)
        st.write([0], kb[None, :L, None, :], vb[None, :L, None, :])
        t1 = time.perf_counter()
        for i in range(L, L + n):
            if st.window_count(0) == 256:
                st.evict([0], 1)
            st.write([0], kb[None, i:i + 1, None, :], vb[None, i:i + 1, None, :])
        return time.perf_counter() - t1, None
    raise ValueError(kind)


def host_info():
    """CPU model and the NumPy/BLAS thread settings of this process."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [{k: d.get(k) for k in ("internal_api", "version", "num_threads")} for d in threadpool_info()]
    except Exception:  # pragma: no cover
        pass
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    return model, blas, env


def cpu_baseline(legs):
    """Time the oracle, as it stands, on sampled units of each workload on the host's cores.

    legs: {name: (jobs, extrapolate)}; extrapolate(times, outputs, P) returns the leg's report.
    All jobs run on P spawned worker processes (P = min(16, cores available), one BLAS thread
    each; each job's time is measured inside its worker).  The leg "c2_decode" (decode attention
    of the 100000-token x 32-sequence step on the GPU's exported store of each sampled unit) is
    the reported `value`; the others go under "legs".
    """
    import multiprocessing as mp
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        raise RuntimeError("the CPU-oracle leg spawns worker processes: run it outside the profiler "
                           "(profiled runs take --no-cpu-baseline)")
    P = max(1, min(16, len(os.sched_getaffinity(0))))
    names = list(legs)
    flat = [(n, j) for n in names for j in legs[n][0]]
    with mp.get_context("spawn").Pool(P) as pool:
        pool.map(_cpu_job, [("warm",)] * P, chunksize=1)   # start-up, not timed
        w0 = time.perf_counter()
        res = pool.map(_cpu_job, [j for _, j in flat], chunksize=1)
        wall = time.perf_counter() - w0
    by = {n: ([], []) for n in names}
    for (n, _), (t, out) in zip(flat, res):
        by[n][0].append(t)
        by[n][1].append(out)
    reports = {n: legs[n][1](by[n][0], by[n][1], P) for n in names}
    head = reports.pop("c2_decode")
    model, blas, env = host_info()
    cpu_s = float(sum(t for n in names for t in by[n][0]))
    log(f"cpu oracle: {len(flat)} sampled jobs on {P} worker processes in {wall:.1f} s wall ({cpu_s:.1f} s CPU); "
        f"step attention {head['value']:.3f} GB/s; max rel-l2 vs gpu {head['sample_rel_l2_vs_gpu']:.2e}")
    head.update({"cores": P, "kind": "oracle", "cpu_model": model, "blas": blas, "blas_env": env,
                 "worker_blas_threads": 1, "cpu_seconds_all_legs": round(cpu_s, 2),
                 "wall_seconds_all_legs": round(wall, 2), "legs": reports})
    return head


def decode_leg(st, seqs_kv, rot, q_host, gpu_out, hq, hkv, label, n_layers=1):
    """CPU-oracle leg of decode attention: jobs for the sampled (seq, KV head) units on their
    exported store state, and the report builder.  The workload (n_layers layers of this store's
    state) takes the sampled units' time scaled by its split-kernel bytes over the sampled units'
    bytes, run on P cores; its rate counts the decode call's algorithmic bytes.  The sampled
    outputs are compared with the GPU's (gpu_out: the store's decode output on the same state)."""
    import numpy as np
    g = hq // hkv
    units = export_units(st, seqs_kv)
    jobs = [("decode", L, n2, pool_u, ring_u, rot[kv:kv + 1], q_host[s:s + 1, kv * g:(kv + 1) * g], g)
            for s, kv, L, n2, pool_u, ring_u in units]
    info = [st.seq_info(s) for s in range(len(gpu_out))]
    lens, n2s = [L for L, _ in info], [n2 for _, n2 in info]
    scale_total = n_layers * split_kernel_bytes(lens, n2s, hkv)
    value_total = n_layers * decode_bytes(lens, n2s, hq, hkv)
    sample = sum(split_kernel_bytes([L], [n2], 1) for _, _, L, n2, _, _ in units)
    n_units = n_layers * len(lens) * hkv

    def rep(times, outs, P):
        cpu_total = float(np.sum(times)) * scale_total / sample
        errs = [float(np.linalg.norm(gpu_out[s, kv * g:(kv + 1) * g] - o[0]) / np.linalg.norm(o[0]))
                for (s, kv), o in zip(seqs_kv, outs)]
        return {"value": value_total / (cpu_total / P) / 1e9, "unit": "GB/s", "workload": label,
                "sample": f"{len(times)} of {n_units} (seq, kv-head) units, decode attention on the GPU's "
                          f"exported store state, scaled by bytes ({scale_total / sample:.1f}x) over {P} cores",
                "seconds_sampled": round(float(np.sum(times)), 3), "seconds_on_P_cores": round(cpu_total / P, 3),
                "value_one_core": value_total / cpu_total / 1e9, "sample_rel_l2_vs_gpu": max(errs)}
    return jobs, rep


PREFILL_TOKENS, PREFILL_APPENDS = 131072, 1024


def prefill_bytes(n_tokens, hkv):
    """Algorithmic bytes of a first write of n_tokens: bf16 K and V read (512 B per token-head),
    INT2 written (80 B per INT2 token-head), BF16 written (512 B per sink/window token-head),
    page ids written."""
    n_bf16 = min(n_tokens, 320)
    n_int2 = n_tokens - n_bf16
    return hkv * (512 * n_tokens + 80 * n_int2 + 512 * n_bf16) + 4 * (-(-n_int2 // 64))


CPU_APPEND_SAMPLE = (4096, 256)    # oracle appends: 256 per KV head after a 4096-token first write


def prefill_leg(reps=5, cpu=True):
    """One 131072-token sequence x 8 KV heads: the multi-token write (rotation on the matrix cores,
    clip, INT2, pack), then 1024 sequential single-token appends each evicting one window token.
    Returns (report, CPU-oracle legs or {})."""
    import numpy as np
    import torch

    import decode_attention_write_amd as oscar
    import synth
    from synth import gpu as sgpu

    cfg, hkv, hq, L = synth.CFG_PREFILL, 8, 32, PREFILL_TOKENS
    rots = np.stack([oscar.oscar_calibrate_host(synth.bf16_bits_to_f32(synth.calibration_queries(cfg, 0, h)))[0]
                     for h in range(hkv)])
    max_pages = -(-(L + PREFILL_APPENDS) // 64) + 1
    st = oscar.KVStore(hq, hkv, 1, max_pages, max_pages, free_pages=synth.page_permutation(cfg, 0, max_pages))
    st.set_rotation(rots)
    prm = sgpu.HeadParams(cfg, 0, hkv)
    kbuf = torch.empty((1, L + PREFILL_APPENDS, hkv, 128), dtype=torch.int16, device="cuda")
    vbuf = torch.empty_like(kbuf)
    sgpu.draw_kv(prm, 0, 0, L + PREFILL_APPENDS, kbuf[0], vbuf[0])
    kpre, vpre = kbuf[:, :L], vbuf[:, :L]
    st.set_timing(True)
    call_ms = []
    for r in range(reps + 1):
        st.reset_seq(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        st.write([0], kpre, vpre)
        e1.record()
        torch.cuda.synchronize()
        if r > 0:
            call_ms.append(e0.elapsed_time(e1))
    n, k_ms = st.read_timing(oscar.TIMED_WRITE)
    assert n == reps + 1, n
    kernel_us = k_ms * 1e3 / n
    nbytes = prefill_bytes(L, hkv)
    # algorithmic matrix-core work: k . R_K per token-head (2 * 128 * 128 flop); the kernel runs
    # it twice (bf16 terms r0 + r1 of R_K)
    flop = 2 * 128 * 128 * L * hkv
    # appends: evict the oldest window token into INT2, then write one token, per step (the
    # per-call input views are made before the timed loop: a caller holds its new token's tensor)
    kviews = [kbuf[:, L + i] for i in range(PREFILL_APPENDS)]
    vviews = [vbuf[:, L + i] for i in range(PREFILL_APPENDS)]
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for i in range(PREFILL_APPENDS):
        st.decode_write([0], kviews[i], vviews[i])
    a1.record()
    torch.cuda.synchronize()
    st.set_timing(False)
    append_us = a0.elapsed_time(a1) * 1e3 / PREFILL_APPENDS
    assert st.seq_info(0) == (L + PREFILL_APPENDS, L + PREFILL_APPENDS - 320)
    res = {
        "workload": f"prefill write: 1 sequence x {L} tokens x {hkv} KV heads (bf16 K/V in, INT2 pages + "
                    f"BF16 sink/window out), then {PREFILL_APPENDS} single-token appends each evicting one",
        "call_us": round(float(np.median(call_ms)) * 1e3, 2),
        "kernel_us": round(kernel_us, 2),
        "bytes": nbytes,
        "gbps_kernel": round(nbytes / kernel_us / 1e3, 1),
        "gbps_call": round(nbytes / (float(np.median(call_ms)) * 1e3) / 1e3, 1),
        "pct_peak_kernel": round(100 * nbytes / kernel_us / 1e3 / PEAK_GBPS, 2),
        "rotation_tflops_algorithmic": round(flop / kernel_us / 1e6, 1),
        "rotation_mfma_frac_executed": round(2 * flop / kernel_us / 1e6 / 2500.0, 4),
        "append_step_us": round(append_us, 2),
    }
    log(f"prefill: call {res['call_us']} us, write kernel {res['kernel_us']} us = {res['gbps_kernel']} GB/s "
        f"({res['pct_peak_kernel']}% of 8 TB/s); rotation {res['rotation_tflops_algorithmic']} TFLOP/s algorithmic; "
        f"evict+append step {res['append_step_us']} us")
    del kbuf, vbuf, st
    if not cpu:
        return res, {}
    rot1 = [rots[h:h + 1] for h in range(hkv)]

    def write_rep(times, outs, P):
        par = min(P, hkv)
        t = float(np.sum(times)) / par
        return {"value": nbytes / t / 1e9, "unit": "GB/s", "workload": res["workload"].split(", then")[0],
                "sample": f"all {hkv} KV heads (one job each; inputs drawn untimed) on {par} cores",
                "seconds_sampled": round(float(np.sum(times)), 3), "seconds_on_P_cores": round(t, 3),
                "gpu_kernel_over_cpu": round(t * 1e6 / kernel_us, 1)}

    L0, n_app = CPU_APPEND_SAMPLE

    def append_rep(times, outs, P):
        par = min(P, hkv)
        per_step = float(np.sum(times)) / n_app / par
        return {"value": round(per_step * 1e6, 1), "unit": "us per evict+append step (8 KV heads)",
                "workload": f"{PREFILL_APPENDS} single-token appends each evicting one window token, 8 KV heads",
                "sample": f"{n_app} appends per KV head after an untimed {L0}-token first write (the oracle's "
                          f"append cost does not depend on the length), one job per head on {par} cores",
                "seconds_sampled": round(float(np.sum(times)), 3),
                "gpu_step_over_cpu": round(per_step * 1e6 / append_us, 1)}

    legs = {"c4_prefill_write": ([("write", cfg, 0, 0, h, L, rot1[h]) for h in range(hkv)], write_rep),
            "c4_appends": ([("appends", cfg, 0, 0, h, L0, n_app, rot1[h]) for h in range(hkv)], append_rep)}
    return res, legs


def layer_leg(cfg, hq, hkv, lengths, reps, label, cpu_units=None):
    """One attention layer over sequences of the given lengths (one R_K per KV head, pages in a
    seeded shuffled order): prefill writes, one untimed decode step (the decode-step write of one
    token per sequence, then decode attention), `reps` steps with the library's events around
    the split kernel, then `reps` steps without them, timed as whole steps (an event pair inside a
    step adds its own gaps).  Returns the split kernel's mean launch time, the whole step's time,
    their difference and rates, and with cpu_units ((seq, KV head) list) the CPU-oracle decode
    leg on the final state (or None)."""
    import numpy as np
    import torch

    import decode_attention_write_amd as oscar
    import synth
    from synth import gpu as sgpu

    B = len(lengths)
    rots = np.stack([oscar.oscar_calibrate_host(synth.bf16_bits_to_f32(synth.calibration_queries(cfg, 0, h)))[0]
                     for h in range(hkv)])
    n_new = 2 * reps + 1
    max_pages = -(-(max(lengths) + n_new + 1) // 64) + 1
    num_pages = sum(-(-(L + n_new + 1) // 64) for L in lengths) + B
    st = oscar.KVStore(hq, hkv, B, max_pages, num_pages, free_pages=synth.page_permutation(cfg, 0, num_pages))
    st.set_rotation(rots)
    prm = sgpu.HeadParams(cfg, 0, hkv)
    kbuf = torch.empty((1, max(lengths) + n_new, hkv, 128), dtype=torch.int16, device="cuda")
    vbuf = torch.empty_like(kbuf)
    newk = torch.empty((n_new, B, hkv, 128), dtype=torch.int16, device="cuda")
    newv = torch.empty_like(newk)
    for s, L in enumerate(lengths):
        sgpu.draw_kv(prm, s, 0, L + n_new, kbuf[0, :L + n_new], vbuf[0, :L + n_new])
        st.write([s], kbuf[:, :L], vbuf[:, :L])
        newk[:, s] = kbuf[0, L:L + n_new]
        newv[:, s] = vbuf[0, L:L + n_new]
    del kbuf, vbuf
    seqs = list(range(B))
    q = torch.from_numpy(synth.decode_queries(cfg, 0, B, hq, hkv).view(np.int16)).cuda()
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(st.workspace_bytes(seqs) // 4 + (1 << 18), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(128)

    def step(i):
        st.decode_step(seqs, newk[i], newv[i], q, scale, out=out, ws=ws)

    # the layer's cache may fit the 256 MB last-level cache: stream a larger buffer through it
    # before every timed step so that each one reads its pages from HBM.  The buffer is read, not
    # written ("read"): a fill leaves up to 256 MB of dirty lines whose write-back then competes
    # with the timed kernel's reads (measured: 8 x 32768 layer 51.9 -> 48.4 us, ragged GQA-8
    # layer 223 -> 198 us, whose 763 MB cannot be served from the cache in either mode)
    flush = torch.empty(1 << 28, dtype=torch.int32, device="cuda")
    st.set_timing(True)
    step(0)
    torch.cuda.synchronize()
    st.read_timing(oscar.TIMED_DECODE)
    info = [st.seq_info(s) for s in seqs]
    flush.fill_(1)
    for i in range(reps):
        flush.sum()
        step(1 + i)
    torch.cuda.synchronize()
    n, k_ms, each = st.read_timing(oscar.TIMED_DECODE, each=True)
    st.set_timing(False)
    assert n == reps * -(-B // 64), n
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        flush.sum()
        evs[i][0].record()
        step(1 + reps + i)
        evs[i][1].record()
    torch.cuda.synchronize()
    step_us = np.array([e0.elapsed_time(e1) for e0, e1 in evs]) * 1e3
    kbytes = float(np.mean([split_kernel_bytes([L + i + 1 for L, _ in info], [n2 + i + 1 for _, n2 in info], hkv)
                            for i in range(reps)]))
    kernel_us = k_ms * 1e3 / n
    res = {
        "workload": label,
        "split_kernel_us": round(kernel_us, 2),
        "split_kernel_us_median": round(float(np.median(each)) * 1e3, 2),
        "split_kernel_bytes": int(kbytes),
        "split_kernel_gbps": round(kbytes / kernel_us / 1e3, 1),
        "split_kernel_pct_peak": round(100 * kbytes / kernel_us / 1e3 / PEAK_GBPS, 2),
        "step_us_median": round(float(np.median(step_us)), 2),
        "step_overhead_us": round(float(np.median(step_us)) - float(np.median(each)) * 1e3, 2),
        "steps": reps,
    }
    log(f"{label}: split kernel {res['split_kernel_us']} us = {res['split_kernel_gbps']} GB/s "
        f"({res['split_kernel_pct_peak']}% of 8 TB/s); step (write + attention) {res['step_us_median']} us, "
        f"{res['step_overhead_us']} us above the split kernel")
    leg = None
    if cpu_units:
        st.decode(seqs, q, scale, out=out, ws=ws)
        torch.cuda.synchronize()
        leg = decode_leg(st, cpu_units, rots, q.cpu().numpy().view(np.uint16), out.cpu().numpy(), hq, hkv, label)
    del st, newk, newv, ws, flush
    return res, leg


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=36,
                    help="layers of the step (36; fewer only for short profiled runs, reported as such)")
    ap.add_argument("--attn-reps", type=int, default=3)
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run a plain device copy of this size at the end (scales the memory counters of a "
                         "profiled run)")
    ap.add_argument("--cpu-units", type=int, default=16, help="sampled (seq, kv head) units of the CPU-oracle decode leg of the step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 131072-token prefill-write leg")
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the single-layer legs (32K x 8 GQA 4; ragged 8K-128K x 16 GQA 8)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the decode step shards by sequence or KV head with no exchange between GPUs).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import decode_attention_write_amd as oscar
    import synth
    from synth import gpu as sgpu

    oscar.load()
    torch.cuda.set_device(0)
    cfg = synth.CFG_QWEN3_8B
    n_layers, B, ctx = args.layers, 32, 100000
    hq, hkv = 32, 8
    # warmup, the timed steps, then warmup and the kernel-timed steps again
    n_steps_total = 2 * args.warmup + 2 * args.steps
    max_pages = -(-(ctx + n_steps_total + 64) // 64)
    num_pages = B * max_pages
    full = (n_layers, B, ctx) == (36, 32, 100000)

    # ---- calibration (host, fp64), one R_K per (layer, kv head)
    t0 = time.time()

    def calib(lh):
        l, h = lh
        q = synth.bf16_bits_to_f32(synth.calibration_queries(cfg, l, h))
        return oscar.oscar_calibrate_host(q)[0]

    with ThreadPoolExecutor(16) as ex:
        flat = list(ex.map(calib, [(l, h) for l in range(n_layers) for h in range(hkv)]))
    rots = [np.stack(flat[l * hkv:(l + 1) * hkv]) for l in range(n_layers)]
    log(f"calibrated {n_layers * hkv} rotations in {time.time() - t0:.1f}s")

    # ---- stores and prefill
    t0 = time.time()
    stores = []
    kbuf = torch.empty((1, ctx, hkv, 128), dtype=torch.int16, device="cuda")
    vbuf = torch.empty_like(kbuf)
    for l in range(n_layers):
        st = oscar.KVStore(hq, hkv, B, max_pages, num_pages, free_pages=synth.page_permutation(cfg, l, num_pages))
        st.set_rotation(rots[l])
        prm = sgpu.HeadParams(cfg, l, hkv)
        for s in range(B):
            sgpu.draw_kv(prm, s, 0, ctx, kbuf[0], vbuf[0])
            st.write([s], kbuf, vbuf)
        stores.append(st)
        if l % 6 == 5 or l == n_layers - 1:
            torch.cuda.synchronize()
            log(f"prefilled layer {l + 1}/{n_layers} ({time.time() - t0:.1f}s)")
    del kbuf, vbuf
    # per-step new tokens, drawn on the GPU up front: [layer][step] -> [B, 1, hkv, 128]
    newk = torch.empty((n_layers, n_steps_total, B, 1, hkv, 128), dtype=torch.int16, device="cuda")
    newv = torch.empty_like(newk)
    tmpk = torch.empty((n_steps_total, hkv, 128), dtype=torch.int16, device="cuda")
    tmpv = torch.empty_like(tmpk)
    for l in range(n_layers):
        prm = sgpu.HeadParams(cfg, l, hkv)
        for s in range(B):
            sgpu.draw_kv(prm, s, ctx, n_steps_total, tmpk, tmpv)
            newk[l, :, s, 0] = tmpk
            newv[l, :, s, 0] = tmpv
    qs = [torch.from_numpy(synth.decode_queries(cfg, l, B, hq, hkv).view(np.int16)).cuda() for l in range(n_layers)]
    seqs = list(range(B))
    outs = [torch.empty((B, hq, 128), dtype=torch.float32, device="cuda") for _ in range(n_layers)]
    # sized for both decode modes (the deterministic one plans its own split size)
    ws_bytes = max(st.workspace_bytes(seqs) for st in stores)
    for st in stores:
        st.set_decode_deterministic(True)
    ws_bytes = max(ws_bytes, max(st.workspace_bytes(seqs) for st in stores)) + (1 << 20)
    for st in stores:
        st.set_decode_deterministic(False)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(128)

    # layer-0 decode on the prefill state, kept for the CPU-oracle sample check
    stores[0].decode(seqs, qs[0], scale, out=outs[0], ws=ws)
    torch.cuda.synchronize()
    legs = {}
    if not args.no_cpu_baseline:
        legs["c2_decode"] = decode_leg(stores[0], CPU_UNITS[:args.cpu_units], rots[0],
                                       qs[0].cpu().numpy().view(np.uint16), outs[0].cpu().numpy(), hq, hkv,
                                       "decode attention of the step (all layers) on the prefill state", n_layers)

    def step(i):
        for l in range(n_layers):
            stores[l].decode_step(seqs, newk[l, i, :, 0], newv[l, i, :, 0], qs[l], scale, out=outs[l], ws=ws)

    def step_bytes():
        tot = 0
        for st in stores:
            info = [st.seq_info(s) for s in seqs]
            # state after evict + append of this step: n_int2 + 1, len + 1
            tot += decode_bytes([L + 1 for L, _ in info], [n2 + 1 for _, n2 in info], hq, hkv)
            tot += evict_bytes(B, hkv) + append_bytes(B, hkv)
        return tot

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    bytes_per_step = []
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    step_ev[0].record()
    for i in range(args.steps):
        bytes_per_step.append(step_bytes())
        step(args.warmup + i)
        step_ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = step_ev[0].elapsed_time(step_ev[-1])
    step_ms = np.array([step_ev[i].elapsed_time(step_ev[i + 1]) for i in range(args.steps)])
    ms_per_step = gpu_ms / args.steps
    step_gbps = sum(bytes_per_step) / (gpu_ms / 1e3) / 1e9
    log(f"timed {args.steps} steps: {ms_per_step:.2f} ms/step (wall {wall / args.steps * 1e3:.2f} ms/step), {step_gbps:.0f} GB/s")

    # ---- the same decode steps again, with the library's fence-free HIP events around every
    # split-kernel launch (on the launch stream): the roofline's kernel durations.  Like the
    # block above it starts with untimed warmup steps, here with the events already in use
    # (without them the block's first step measured ~15 % slower launches)
    for st in stores:
        st.set_timing(True)
    for i in range(args.warmup):
        step(args.warmup + args.steps + i)
    torch.cuda.synchronize()
    for st in stores:
        st.read_timing(oscar.TIMED_DECODE)      # discards the warmup launches
    info0 = [[st.seq_info(s) for s in seqs] for st in stores]
    kt0, kt1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    kt0.record()
    for i in range(args.steps):
        step(2 * args.warmup + args.steps + i)
    kt1.record()
    torch.cuda.synchronize()
    ms_per_step_kt = kt0.elapsed_time(kt1) / args.steps
    k_launches, k_ms, k_each = 0, 0.0, []
    for st in stores:
        n, ms, each = st.read_timing(oscar.TIMED_DECODE, each=True)
        k_launches += n
        k_ms += ms
        k_each.append(each)
        st.set_timing(False)
    k_each = np.concatenate(k_each) * 1e3  # us
    n_chunks = -(-B // 64)
    assert k_launches == args.steps * n_layers * n_chunks, k_launches
    # bytes of each timed launch: step i attends over the state after its evict + append
    kbytes_steps = [split_kernel_bytes([L + i + 1 for L, _ in info], [n2 + i + 1 for _, n2 in info], hkv)
                    for info in info0 for i in range(args.steps)]
    kernel_us = k_ms * 1e3 / k_launches
    kernel_bytes = float(np.mean(kbytes_steps)) / n_chunks
    kernel_gbps = kernel_bytes / (kernel_us / 1e6) / 1e9
    log(f"split kernel over {args.steps} timed steps: {kernel_us:.1f} us/launch (median {np.median(k_each):.1f}), "
        f"{kernel_gbps:.0f} GB/s ({100 * kernel_gbps / PEAK_GBPS:.1f}% of 8 TB/s); "
        f"those steps took {ms_per_step_kt:.2f} ms each")

    # ---- attention-only passes over the frozen cache, default mode (a unit's INT2 splits share
    # page groups at run time) and deterministic mode (fixed page range per split): per-call HIP
    # events on the launch stream, and the library's events around each split-kernel launch
    attn_bytes = []
    for st in stores:
        info = [st.seq_info(s) for s in seqs]
        attn_bytes.append(decode_bytes([L for L, _ in info], [n2 for _, n2 in info], hq, hkv))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_layers)]

    def attn_pass(deterministic):
        per_call, repeat = [], None
        for st in stores:
            st.set_decode_deterministic(deterministic)
            st.set_timing(True)
        for r in range(args.attn_reps + 1):
            for l, st in enumerate(stores):
                evs[l][0].record()
                st.decode(seqs, qs[l], scale, out=outs[l], ws=ws)
                evs[l][1].record()
            torch.cuda.synchronize()
            if r == 0:                       # untimed pass; keep layer 0's output
                first = outs[0].clone()
                for st in stores:
                    st.read_timing(oscar.TIMED_DECODE)
                continue
            per_call.extend(a.elapsed_time(b) for a, b in evs)
            repeat = bool(torch.equal(first, outs[0]))
        n_k, ms_k = 0, 0.0
        for st in stores:
            n, ms = st.read_timing(oscar.TIMED_DECODE)
            n_k += n
            ms_k += ms
            st.set_timing(False)
            st.set_decode_deterministic(False)
        call_ms = float(np.mean(per_call))
        gbps = float(np.mean(attn_bytes)) / (call_ms / 1e3) / 1e9
        return {"us_per_layer": round(call_ms * 1e3, 2), "gbps": round(gbps, 1),
                "pct_peak": round(100 * gbps / PEAK_GBPS, 2), "bytes_per_layer": int(np.mean(attn_bytes)),
                "split_kernel_us": round(ms_k * 1e3 / n_k, 2),
                "split_kernel_pct_peak": round(100 * kernel_bytes / (ms_k * 1e3 / n_k) / 1e3 / PEAK_GBPS, 2),
                "layer0_output_bitwise_repeats": repeat}

    attn = attn_pass(False)
    attn_det = attn_pass(True)
    for name, a in (("attention-only", attn), ("attention-only, deterministic", attn_det)):
        log(f"{name}: {a['us_per_layer']} us/layer, {a['gbps']} GB/s ({a['pct_peak']}% of 8 TB/s); split kernel "
            f"{a['split_kernel_us']} us ({a['split_kernel_pct_peak']}%); layer-0 output repeats bitwise: "
            f"{a['layer0_output_bitwise_repeats']}")
    if not attn_det["layer0_output_bitwise_repeats"]:
        raise RuntimeError("deterministic decode did not repeat bitwise")
    result = {
        "metric": METRIC,
        "value": round(step_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "steps_per_s": round(1e3 / ms_per_step, 3),
        "pct_peak": round(100 * step_gbps / PEAK_GBPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2 KV (fp16 scale/min per 64) + bf16 ring; Q.K on i8 MFMA with q' as two int8 terms, "
                 "P.V on f16 MFMA with P as an f16 hi+lo pair; f32 accumulate, f32 output",
        "data": "synthetic (seeded; keys/values drawn on the GPU, Philox4x32-10)",
        "config": {
            "workload": (f"qwen3-8b-shaped decode step: {n_layers} layers x (write: evict 1 + append 1, "
                         f"then GQA decode attention), {hq} q / {hkv} kv heads, head_dim 128, batch {B}, {ctx}-token context, "
                         "INT2 KV in 64-token pages (shuffled), BF16 sink 64 + window 256"),
            "layers": n_layers, "batch": B, "context": ctx, "q_heads": hq, "kv_heads": hkv,
            "headline_config": full,
            "write_calls": "one decode-step call per layer (write + attention)",
        },
        "attn_only": attn,
        "attn_only_deterministic": attn_det,
        "roofline": {
            "bound": "hbm",
            "achieved": round(kernel_gbps, 1),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(kernel_gbps / PEAK_GBPS, 4),
            "traffic": measured_traffic() if full else None,
            "kernel": f"k_decode_mfma<{hq // hkv}> (split-K decode attention over the INT2 pages and BF16 ring), "
                      f"{args.steps} timed decode steps x {n_layers} layers",
            "us_per_launch": round(kernel_us, 2),
            "us_median": round(float(np.median(k_each)), 2),
            "us_p10": round(float(np.percentile(k_each, 10)), 2),
            "us_p90": round(float(np.percentile(k_each, 90)), 2),
            "launches": int(k_launches),
            "bytes_per_launch": int(kernel_bytes),
        },
        "step_ms": {"median": round(float(np.median(step_ms)), 4), "p10": round(float(np.percentile(step_ms, 10)), 4),
                    "p90": round(float(np.percentile(step_ms, 90)), 4),
                    "mean_with_kernel_events": round(ms_per_step_kt, 4)},
    }
    cpu = not args.no_cpu_baseline
    if not args.no_prefill:
        result["prefill"], pl = prefill_leg(cpu=cpu)
        legs.update(pl)
    if not args.no_layers:
        c1_units = [(s, (3 * s + 1) % 8) for s in range(8)] + [(s, (3 * s + 5) % 8) for s in range(8)]
        result["layer_qwen3_4b_32k_b8"], legs["c1_decode"] = layer_leg(
            synth.CFG_QWEN3_4B, 32, 8, [32768] * 8, 20,
            "qwen3-4b-shaped layer: 32 q / 8 kv heads, batch 8, 32768-token context",
            c1_units if cpu else None)
        result["layer_qwen3_32b_ragged_b16"], legs["c3_decode"] = layer_leg(
            synth.CFG_QWEN3_32B, 64, 8, [int(x) for x in synth.ragged_lengths(synth.CFG_QWEN3_32B, 16, 8192, 131072)],
            20, "qwen3-32b-shaped layer: 64 q / 8 kv heads (GQA 8), batch 16, lengths U[8192, 131072]",
            [(s, (5 * s + 2) % 8) for s in range(16)] if cpu else None)
    if args.copy_calib_mib:
        # a plain copy of known size, for scaling the memory counters of a profiled run
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calib_mib} MiB read + {args.copy_calib_mib} MiB written")
    if cpu:
        result["cpu_baseline"] = cpu_baseline({k: v for k, v in legs.items() if v is not None})
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
