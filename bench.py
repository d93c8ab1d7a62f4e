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


def _cpu_unit(job):
    """One (seq, kv head) unit of the oracle's decode attention in a worker process (no GPU use):
    returns its decode time and output."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass
    from oracle import attention
    L, n2, pool_u, ring_u, rot, q, g = job
    if pool_u is None:
        return 0.0, None          # warm-up task: imports only
    table_u = np.arange(pool_u.shape[0], dtype=np.int32)[None, :]
    t1 = time.perf_counter()
    out = attention.decode(pool_u, ring_u, table_u, np.array([L]), np.array([n2]), rot, q, [0], 1 / math.sqrt(128), g)
    return time.perf_counter() - t1, out


def cpu_baseline(units, rots, q_layer0, out_layer0, hq, hkv, total_units, step_bytes_attn):
    """Time the oracle's decode attention on sampled (layer 0, seq, kv head) units on the host's
    cores: P worker processes (spawned, one BLAS thread each, P = min(16, cores available)) run
    the units concurrently; each unit's decode time is measured inside its worker.  The step's
    CPU time is extrapolated as total units x mean unit time / P.

    The oracle runs on the GPU's exported store state of each unit (identical inputs), so the
    reported rel-L2 is the decode parity figure.
    """
    import multiprocessing as mp
    import numpy as np
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        raise RuntimeError("the CPU-oracle leg spawns worker processes: run it outside the profiler "
                           "(profiled runs take --no-cpu-baseline)")
    g = hq // hkv
    P = max(1, min(16, len(os.sched_getaffinity(0)), len(units)))
    jobs = [(L, n2, pool_u, ring_u, rots[0][kv:kv + 1], q_layer0[s:s + 1, kv * g:(kv + 1) * g], g)
            for s, kv, L, n2, pool_u, ring_u in units]
    with mp.get_context("spawn").Pool(P) as pool:
        pool.map(_cpu_unit, [(0, 0, None, None, None, None, g)] * P, chunksize=1)   # start-up, not timed
        w0 = time.perf_counter()
        res = pool.map(_cpu_unit, jobs, chunksize=1)
        wall = time.perf_counter() - w0
    times = [t for t, _ in res]
    errs = []
    for (s, kv, L, n2, _, _), (t, out) in zip(units, res):
        gpu = out_layer0[s, kv * g:(kv + 1) * g]
        errs.append(float(np.linalg.norm(gpu - out[0]) / np.linalg.norm(out[0])))
    per_unit = float(np.mean(times))
    cpu_step_s = per_unit * total_units / P
    log(f"cpu oracle: {len(units)} units on {P} worker processes in {wall:.1f} s wall, "
        f"{per_unit:.2f} s per unit, max rel-l2 vs gpu {max(errs):.2e}")
    return {
        "value": step_bytes_attn / cpu_step_s / 1e9,
        "unit": "GB/s",
        "cores": P,
        "kind": "oracle",
        "sample": (f"{len(units)} of {total_units} (layer, seq, kv-head) units of the attention pass "
                   f"(oracle on the GPU's exported store of each unit, 100000-token context), decode "
                   f"attention only, on {P} concurrent single-threaded worker processes, "
                   f"extrapolated x{total_units}/{P}"),
        "seconds_per_unit": per_unit,
        "cpu_seconds_sampled": float(np.sum(times)),
        "value_one_core": step_bytes_attn / (per_unit * total_units) / 1e9,
        "sample_rel_l2_vs_gpu": max(errs),
    }


PREFILL_TOKENS, PREFILL_APPENDS = 131072, 1024


def prefill_bytes(n_tokens, hkv):
    """Algorithmic bytes of a first write of n_tokens: bf16 K and V read (512 B per token-head),
    INT2 written (80 B per INT2 token-head), BF16 written (512 B per sink/window token-head),
    page ids written."""
    n_bf16 = min(n_tokens, 320)
    n_int2 = n_tokens - n_bf16
    return hkv * (512 * n_tokens + 80 * n_int2 + 512 * n_bf16) + 4 * (-(-n_int2 // 64))


def prefill_leg(reps=5):
    """One 131072-token sequence x 8 KV heads: the multi-token write (rotation on the matrix cores,
    clip, INT2, pack), then 1024 sequential single-token appends each evicting one window token."""
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
    # appends: evict the oldest window token into INT2, then write one token, per step
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    for i in range(PREFILL_APPENDS):
        st.decode_write([0], kbuf[:, L + i], vbuf[:, L + i])
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
    return res


def layer_leg(cfg, hq, hkv, lengths, reps, label, pps=0, flush_mode="read"):
    """One attention layer over sequences of the given lengths (one R_K per KV head, pages in a
    seeded shuffled order): prefill writes, then `reps` decode steps (the decode-step write of
    one token per sequence, then decode attention), each after one untimed step.  Returns the
    split kernel's mean launch time (library events), the whole step's time and their rates."""
    import numpy as np
    import torch

    import decode_attention_write_amd as oscar
    import synth
    from synth import gpu as sgpu

    B = len(lengths)
    rots = np.stack([oscar.oscar_calibrate_host(synth.bf16_bits_to_f32(synth.calibration_queries(cfg, 0, h)))[0]
                     for h in range(hkv)])
    max_pages = -(-(max(lengths) + reps + 2) // 64) + 1
    num_pages = sum(-(-(L + reps + 2) // 64) for L in lengths) + B
    st = oscar.KVStore(hq, hkv, B, max_pages, num_pages, free_pages=synth.page_permutation(cfg, 0, num_pages))
    st.set_rotation(rots)
    st.set_decode_split(pps)
    prm = sgpu.HeadParams(cfg, 0, hkv)
    n_new = reps + 1
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
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    flush.fill_(1)
    for i in range(reps):
        if flush_mode == "write":
            flush.fill_(i)
        else:
            flush.sum()
        evs[i][0].record()
        step(1 + i)
        evs[i][1].record()
    torch.cuda.synchronize()
    n, k_ms, each = st.read_timing(oscar.TIMED_DECODE, each=True)
    st.set_timing(False)
    assert n == reps * -(-B // 64), n
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
        "steps": reps,
    }
    log(f"{label}: split kernel {res['split_kernel_us']} us = {res['split_kernel_gbps']} GB/s "
        f"({res['split_kernel_pct_peak']}% of 8 TB/s); step (write + attention) {res['step_us_median']} us")
    del st, newk, newv, ws, flush
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=36, help="development only: fewer layers")
    ap.add_argument("--context", type=int, default=100000, help="development only")
    ap.add_argument("--batch", type=int, default=32, help="development only")
    ap.add_argument("--attn-reps", type=int, default=3)
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="run a plain device copy of this size at the end (counter scaling in profiled runs)")
    ap.add_argument("--cpu-units", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 131072-token prefill-write leg")
    ap.add_argument("--no-layers", action="store_true",
                    help="skip the single-layer legs (32K x 8 GQA 4; ragged 8K-128K x 16 GQA 8)")
    ap.add_argument("--pps", type=int, default=0, help="pages per decode split (0 = library choice)")
    ap.add_argument("--sweep-pps", default="", help="development: comma list of split sizes to time")
    ap.add_argument("--deterministic", action="store_true",
                    help="fixed page range per split (no page sharing between the splits of a unit)")
    ap.add_argument("--kernel", type=int, default=0, help="decode kernel: 0 matrix-core, 1 reference")
    ap.add_argument("--layer-pps", type=int, default=0,
                    help="development: pages per decode split in the single-layer legs (0 = library choice)")
    ap.add_argument("--layer-flush", choices=["write", "read"], default="read",
                    help="development: how the single-layer legs push their cache out of the last-level cache")
    ap.add_argument("--two-call", action="store_true",
                    help="development: the decode-step write and the attention as two calls")
    ap.add_argument("--separate-write", action="store_true",
                    help="write each step with the eviction and the append as two calls (comparison)")
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
    n_layers, B, ctx = args.layers, args.batch, args.context
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
        st.set_decode_split(args.pps)
        st.set_decode_kernel(args.kernel)
        st.set_decode_deterministic(args.deterministic)
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
    ws_bytes = max(st.workspace_bytes(seqs) for st in stores) + (1 << 20)
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(128)

    # layer-0 decode on the prefill state, kept for the CPU-oracle sample check
    stores[0].decode(seqs, qs[0], scale, out=outs[0], ws=ws)
    torch.cuda.synchronize()
    out_layer0 = outs[0].cpu().numpy()
    q_layer0 = qs[0].cpu().numpy().view(np.uint16)
    units0 = [] if args.no_cpu_baseline else export_units(stores[0], CPU_UNITS[:args.cpu_units])

    def step(i):
        for l in range(n_layers):
            st = stores[l]
            if args.separate_write:
                st.evict(seqs, 1)
                st.write(seqs, newk[l, i], newv[l, i])
                st.decode(seqs, qs[l], scale, out=outs[l], ws=ws)
            elif args.two_call:
                st.decode_write(seqs, newk[l, i, :, 0], newv[l, i, :, 0])
                st.decode(seqs, qs[l], scale, out=outs[l], ws=ws)
            else:
                st.decode_step(seqs, newk[l, i, :, 0], newv[l, i, :, 0], qs[l], scale, out=outs[l], ws=ws)

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

    # ---- development sweep of the split size (attention only)
    for pps in [int(x) for x in args.sweep_pps.split(",") if x]:
        for st in stores:
            st.set_decode_split(pps)
        need = max(st.workspace_bytes(seqs) for st in stores)
        if need > ws.numel() * 4:
            ws = torch.empty(need // 4 + 1, dtype=torch.float32, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for st in stores:
            st.decode(seqs, qs[0], scale, out=outs[0], ws=ws)
            st.set_timing(True)
        e0.record()
        for r in range(2):
            for l, st in enumerate(stores):
                st.decode(seqs, qs[l], scale, out=outs[l], ws=ws)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (2 * n_layers)
        k_n, k_ms = 0, 0.0
        for st in stores:
            n, ms = st.read_timing(oscar.TIMED_DECODE)
            k_n, k_ms = k_n + n, k_ms + ms
            st.set_timing(False)
        log(f"sweep pps={pps}: split kernel {k_ms * 1e3 / max(k_n, 1):.1f} us, call {us:.1f} us/layer")
    for st in stores:
        st.set_decode_split(args.pps)

    # ---- attention-only pass over the frozen cache: per-call HIP events on the launch stream
    per_call = []
    attn_bytes = []
    for st in stores:
        info = [st.seq_info(s) for s in seqs]
        attn_bytes.append(decode_bytes([L for L, _ in info], [n2 for _, n2 in info], hq, hkv))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_layers)]
    for r in range(args.attn_reps):
        for l, st in enumerate(stores):
            evs[l][0].record()
            st.decode(seqs, qs[l], scale, out=outs[l], ws=ws)
            evs[l][1].record()
        torch.cuda.synchronize()
        per_call.extend(a.elapsed_time(b) for a, b in evs)
    attn_ms = float(np.mean(per_call))
    attn_gbps = float(np.mean(attn_bytes)) / (attn_ms / 1e3) / 1e9
    log(f"attention-only: {attn_ms * 1e3:.1f} us/layer, {attn_gbps:.0f} GB/s ({100 * attn_gbps / PEAK_GBPS:.1f}% of 8 TB/s)")

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
        "dtype": "f32",
        "data": "synthetic (seeded; keys/values drawn on the GPU, Philox4x32-10)",
        "config": {
            "workload": (f"qwen3-8b-shaped decode step: {n_layers} layers x (write: evict 1 + append 1, "
                         f"then GQA decode attention), {hq} q / {hkv} kv heads, head_dim 128, batch {B}, {ctx}-token context, "
                         "INT2 KV in 64-token pages (shuffled), BF16 sink 64 + window 256"),
            "layers": n_layers, "batch": B, "context": ctx, "q_heads": hq, "kv_heads": hkv,
            "headline_config": full,
            "write_calls": ("evict + append, then attention" if args.separate_write else
                            "decode-step write, then attention" if args.two_call else
                            "one decode-step call (write + attention)"),
        },
        "attn_only": {"us_per_layer": round(attn_ms * 1e3, 2), "gbps": round(attn_gbps, 1),
                      "pct_peak": round(100 * attn_gbps / PEAK_GBPS, 2),
                      "bytes_per_layer": int(np.mean(attn_bytes))},
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
    if not args.no_prefill:
        result["prefill"] = prefill_leg()
    if not args.no_layers:
        result["layer_qwen3_4b_32k_b8"] = layer_leg(
            synth.CFG_QWEN3_4B, 32, 8, [32768] * 8, 20,
            "qwen3-4b-shaped layer: 32 q / 8 kv heads, batch 8, 32768-token context", pps=args.layer_pps,
            flush_mode=args.layer_flush)
        result["layer_qwen3_32b_ragged_b16"] = layer_leg(
            synth.CFG_QWEN3_32B, 64, 8, [int(x) for x in synth.ragged_lengths(synth.CFG_QWEN3_32B, 16, 8192, 131072)],
            20, "qwen3-32b-shaped layer: 64 q / 8 kv heads (GQA 8), batch 16, lengths U[8192, 131072]",
            pps=args.layer_pps, flush_mode=args.layer_flush)
    if args.copy_calib_mib:
        # a plain copy of known size, for scaling the memory counters of a profiled run
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calib_mib} MiB read + {args.copy_calib_mib} MiB written")
    if not args.no_cpu_baseline:
        total_units = n_layers * B * hkv
        step_attn_bytes = float(np.sum(attn_bytes))
        result["cpu_baseline"] = cpu_baseline(units0, rots, q_layer0, out_layer0, hq, hkv, total_units,
                                              step_attn_bytes)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
