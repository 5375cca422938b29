#!/usr/bin/env python3
"""Paged decode-attention throughput on one MI355X (gfx950).

Workload: OPT-13B-shaped decode of 7 texts x 2,048 tokens (40 heads x 128, fp16,
block 16, 983-block pools with randomly placed blocks). One step is the whole hot
path for the batch:
  host allocator step (one slot per text, copy-on-write pairs) -> table/slot upload
  -> for every layer: pa_copy_blocks (when pairs exist), the write of the new token
     and decode attention over the cache, in one launch (pa_decode_attention_write;
     `--separate-write`, and E4M3 pools: pa_kv_write then pa_decode_attention).
Kernels are launched one by one (the host runs ahead of the GPU; the slots and lengths
of a step arrive in one upload). `--graph` replays each step's launches from HIP graphs
captured for that step instead (measured slower here: tens of us per step go to the
hand-over between graph launches).
`--layers` pools share one allocator, as the layers of one model do; reading a
different layer's pools on every launch keeps repeat reads out of the 256 MB
Infinity Cache, so every launch streams its keys and values from HBM.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value      algorithmic decode bytes (K and V of every attended token, q, out,
             table entries) per second over the timed steps, inputs resident in HBM
  roofline   the decode launch: algorithmic bytes per launch / its average duration
             from HIP events around each launch on the launch stream, vs 8 TB/s
  cpu_baseline  the fp64 CPU oracle on the same step (one layer), one thread
"""
from __future__ import annotations

import argparse
import dataclasses
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CSRC = os.path.join(ROOT, "paged_kv_cache_320_amd", "csrc")
DECODE_SRCS = [os.path.join(CSRC, f) for f in ("decode.hip", "decode_kernels.hpp",
                                               "decode_inst.hip")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_opt13b_7x2048.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def quiet_gc():
    """Collect once and pause Python's cyclic garbage collector for the timed steps: a
    full collection over the setup's objects stalls the host for milliseconds at random
    steps (measured: one 6 ms step among 12 of the Llama-shaped decode)."""
    gc.collect()
    gc.freeze()
    gc.disable()


def decode_bytes(lens, H, D, B, elt, Hkv=None, kv_elt=None) -> int:
    """Algorithmic bytes of one decode launch: K+V of attended tokens (each key/value head
    once, kv_elt bytes a number), q and out (elt bytes a number), table entries."""
    S = len(lens)
    kv = sum(int(L) for L in lens) * 2 * (Hkv or H) * D * (kv_elt or elt)
    qo = 2 * S * H * D * elt
    tab = sum((int(L) + B - 1) // B for L in lens) * 4
    return kv + qo + tab


def src_hash() -> str:
    """Hash of the decode source files' code (comments and blank space left out): counter
    figures are tied to one kernel build."""
    import re
    h = hashlib.sha256()
    for f in DECODE_SRCS:
        text = open(f).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(fused: bool):
    """The committed counter record of the decode launch (HBM bytes per launch and the run they
    come from), if the kernel is unchanged (same sources, and the same variant: with or
    without the fused new-token write); else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("decode_src_sha256_16") != src_hash() or rec.get("fused_write", False) != fused:
        return None
    return rec


def traffic_note(rec):
    """Where roofline.traffic comes from: the counter runs' steps and their own algorithmic
    bytes per launch (the ratio is taken within those runs)."""
    if not rec:
        return None
    alg = rec.get("algorithmic_bytes_per_launch")
    note = (f"rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE of `bench.py --steps "
            f"{rec.get('steps')} --warmup {rec.get('warmup')}`, copy-calibrated")
    if alg:
        note += (f"; that run's algorithmic bytes per launch {alg}, HBM / algorithmic "
                 f"{rec['hbm_bytes_per_launch'] / alg:.4f}")
    return note


COPY_CAL_BYTES = 512 << 20
ELT = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def _counter_rows(d, name):
    """(kernel name, value) per dispatch of counter `name` from a rocprofv3 --pmc output
    folder: CSV output (*counter_collection.csv) or the default database (*_results.db)."""
    import csv
    import glob
    import sqlite3
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") == name:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    for f in glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True):
        db = sqlite3.connect(f)
        out += [(k, float(v)) for k, v in db.execute(
            "select kernel_name, value from counters_collection where counter_name = ?", (name,))]
        db.close()
    if not out:
        raise SystemExit(f"no {name} records under {d}")
    return out


def traffic_from_counters(fetch_dir: str, write_dir: str) -> None:
    """HBM bytes per decode launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for pa_copy_probe moving COPY_CAL_BYTES."""
    import numpy as np
    res = {}
    fused = set()
    for key, d, name in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d, name)
        ours = [(k, v) for k, v in rows if k.startswith("pagedkv::") or "pagedkv::" in k[:40]]
        copy = [v for k, v in ours if "copy_kernel" in k]
        part = [v for k, v in ours if "decode_partition" in k]
        # the fused variant's template arguments end in "true>"
        fused |= {"true>" in k for k, v in ours if "decode_partition" in k}
        merge = [v for k, v in ours if "decode_merge" in k]
        if not copy or not part:
            raise SystemExit(f"{name}: need copy_kernel and decode_partition dispatches in {d}")
        scale = COPY_CAL_BYTES / (float(np.median(copy)) * 1024)
        res[key] = {"counter": name, "copy_kib_median": float(np.median(copy)),
                    "scale": scale, "partition_kib_median": float(np.median(part)),
                    "merge_kib_median": float(np.median(merge)) if merge else 0.0,
                    "bytes_per_launch": (float(np.median(part)) +
                                         (float(np.median(merge)) if merge else 0.0)) * 1024 * scale}
    if len(fused) != 1:
        raise SystemExit("counter runs mix the decode kernel with and without the fused write")
    # the profiled runs' own JSON lines (--line-out DIR/line.json): their algorithmic bytes
    lines = []
    for d in (fetch_dir, write_dir):
        try:
            lines.append(json.load(open(os.path.join(d, "line.json"))))
        except (OSError, ValueError):
            raise SystemExit(f"{d}/line.json missing: profile `bench.py --copy-calibration "
                             f"--line-out {d}/line.json`")
    alg = float(np.mean([ln["roofline"]["bytes_per_launch"] for ln in lines]))
    hbm = int(res["fetch"]["bytes_per_launch"] + res["write"]["bytes_per_launch"])
    rec = {"decode_src_sha256_16": src_hash(), "workload": lines[0]["config"]["workload"],
           "fused_write": fused.pop(),
           "steps": lines[0]["steps"], "warmup": lines[0]["warmup"],
           "layers": lines[0]["config"]["layers_per_step"],
           "hbm_bytes_per_launch": hbm,
           "algorithmic_bytes_per_launch": int(alg),
           "hbm_over_algorithmic": round(hbm / alg, 5),
           "fetch": res["fetch"], "write": res["write"],
           "calibration": f"pa_copy_probe reading and writing {COPY_CAL_BYTES} bytes"}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(rec, indent=1))


def run_copy_calibration(L, torch):
    src = torch.empty(COPY_CAL_BYTES // 2, dtype=torch.float16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        L.pa_copy_probe(dst, src)
    torch.cuda.synchronize()


def run_probe(L, torch, gib=4):
    n = gib << 30
    buf = torch.empty(n // 2, dtype=torch.float16, device="cuda").normal_()
    sink = torch.empty(L.pa_probe_sink_bytes(0), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        L.pa_stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        L.pa_stream_read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbps = n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    return gbps


def run_volume_probe(L, torch, bytes_per_launch: int):
    """A plain contiguous read of the decode's own volume per launch: each launch streams
    the next disjoint range of a buffer of at least 4 GiB and 4 launches' worth, so the
    launch's fixed costs (its ramp, the first loads' latency, the tail) weigh as they do in
    the decode. Mean GB/s."""
    per = (int(bytes_per_launch) + 4095) // 4096 * 4096
    n = max(4 << 30, (4 * per + (1 << 30) - 1) >> 30 << 30)
    buf = torch.empty(n // 2, dtype=torch.float16, device="cuda").normal_()
    sink = torch.empty(L.pa_probe_sink_bytes(0), dtype=torch.uint8, device="cuda")
    L.pa_stream_read_probe(buf[: per // 2], sink)  # checked call through the binding
    torch.cuda.synchronize()
    fn, stream = L.lib().pa_stream_read_probe, torch.cuda.current_stream().cuda_stream
    calls = [(buf.data_ptr() + k * per, per, sink.data_ptr(), 0, stream) for k in range(n // per)]
    for c in calls:  # first touch of every page outside the timed region
        assert fn(*c) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for c in calls[1:]:
        fn(*c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (len(calls) - 1)
    del buf
    return per / (ms * 1e-3) / 1e9


def run_tile_probe(L, torch, tile_bytes: int, bytes_per_launch: int):
    """The decode's own read volume in randomly placed tiles of its (block, head) tile size:
    each launch reads a disjoint random set of tiles of a buffer of at least 4 GiB and 4
    launches' worth (more than the 256 MB Infinity Cache holds between two uses of a
    set). Mean GB/s."""
    n = max(4 << 30, (4 * bytes_per_launch + (1 << 30) - 1) >> 30 << 30)  # >= 4 sets
    buf = torch.empty(n // 2, dtype=torch.float16, device="cuda").normal_()
    sink = torch.empty(L.pa_probe_sink_bytes(4), dtype=torch.uint8, device="cuda")
    per = max(1, bytes_per_launch // tile_bytes)
    g = torch.Generator().manual_seed(0)
    perm = torch.randperm(n // tile_bytes, generator=g).to(torch.int32)
    sets = [perm[k * per:(k + 1) * per].cuda() for k in range(len(perm) // per)]
    L.pa_tile_read_probe(buf, tile_bytes, sets[0], sink)  # checked call through the binding
    torch.cuda.synchronize()
    # then the raw entry point with the pointers taken once (the binding's per-call work
    # would otherwise starve the GPU between 50 us launches), and one launch ahead of the
    # first event so no host time falls inside the timed region
    fn, stream = L.lib().pa_tile_read_probe, torch.cuda.current_stream().cuda_stream
    calls = [(buf.data_ptr(), n, tile_bytes, ids.data_ptr(), ids.numel(), sink.data_ptr(), stream)
             for ids in sets]
    # one untimed pass over every set first: the decode steps run over pools they have
    # touched before, and the first touch of a page costs address-translation misses
    for c in calls:
        assert fn(*c) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for c in calls[1:]:
        fn(*c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (len(sets) - 1)
    del buf
    return per * tile_bytes / (ms * 1e-3) / 1e9


def run_swap_probe(cache, seqs, torch, reps: int = 3):
    """Texts given way and brought back («The KV Cache and PagedAttention», "When Memory
    Runs Out"): every layer's blocks of two texts moved to pinned host pools by
    pa_swap_blocks and back (the allocator's pairs). Returns (out GB/s, in GB/s, bytes
    each way) over the host link, HIP events around each direction."""
    chosen = list(seqs[:2])
    nblk = sum(cache.alloc.info(s)[1] for s in chosen)
    cache.host_pool(nblk)
    per_block = 2 * cache.num_kv_heads * cache.block_size * cache.head_dim * \
        cache.k[0].element_size() * len(cache.k)
    t_out, t_in = [], []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        pairs = cache.swap_out(chosen)
        e[1].record()
        e[2].record()
        cache.swap_in(chosen)
        e[3].record()
        torch.cuda.synchronize()
        t_out.append(e[0].elapsed_time(e[1]))
        t_in.append(e[2].elapsed_time(e[3]))
    nbytes = len(pairs) * per_block
    return (nbytes / (min(t_out) * 1e-3) / 1e9, nbytes / (min(t_in) * 1e-3) / 1e9, nbytes)


def host_cores() -> dict:
    """The host the CPU baseline ran on: logical CPUs, the ones this process may use, and the
    BLAS threads numpy would use by default (the baseline itself is limited to one)."""
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 0) for p in threadpool_info()), default=None)
    except Exception:
        blas = None
    return {"nproc": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "blas_threads_default": blas, "baseline_threads": 1}


def cpu_baseline(w, d0, seconds: float, gpu_out0):
    """The oracle as it stands, on one layer's step-0 batch, one thread, about `seconds` long."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import workloads as wl
    from oracle.attention import decode_attention
    from oracle.replay import Replay

    cpu = dataclasses.replace(
        d0, prefill_k=[t.cpu() for t in d0.prefill_k], prefill_v=[t.cpu() for t in d0.prefill_v],
        step_k=[d0.step_k[0].cpu()], step_v=[d0.step_v[0].cpu()], step_q=[d0.step_q[0].cpu()])
    w1 = w.scaled(steps=1)
    # the oracle allocator and cache writes build the step-0 pools and tables
    # (attention skipped there: decode_pairs -> []); the attention itself is timed below
    rp = Replay(w1, cpu, pool=True)
    res = rp.run(wl.script(w1, cpu), decode_pairs=lambda t: [])[0]
    q = cpu.step_q[0]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        reps = 0
        out = None
        while True:
            out = decode_attention(q, rp.k, rp.v, res.tables, res.lens, w.block_size,
                                   k_scale=w.k_scale, v_scale=w.v_scale)
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    nbytes = decode_bytes(res.lens, w.num_heads, w.head_dim, w.block_size, ELT[w.dtype],
                          w.num_kv_heads, ELT[w.pool_dtype])
    err = None
    if gpu_out0 is not None:
        err = float(np.max(np.abs(gpu_out0.astype(np.float64) - out)))
    return {
        "value": round(nbytes * reps / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "host": host_cores(),
        "sample": f"{w.name} one layer, step 0: all {w.num_seqs * w.num_heads} (text, head) pairs "
                  f"x {reps} repetitions in {dt:.1f} s (fp64 numpy, BLAS limited to 1 thread)",
        "seq_layers_per_s": round(w.num_seqs * reps / dt, 3),
    }, err


def unique_kv_bytes(tables, lens, B, Hkv, D, kv_elt) -> int:
    """K and V bytes of the physical blocks a decode launch reads, each block once (blocks
    shared by several texts counted once, with the most places any of them attends)."""
    filled = {}
    for t, L in zip(tables, lens):
        for j in range((int(L) + B - 1) // B):
            b = int(t[j])
            filled[b] = max(filled.get(b, 0), min(B, int(L) - j * B))
    return sum(filled.values()) * 2 * Hkv * D * kv_elt


def bench_sharing(args, base, K: int, W: int) -> dict:
    """Parallel sampling / beam search: groups of texts share their prompt's blocks. Every
    step each odd sample is replaced by a fork of its even partner (the pair then shares a
    partly filled last block), one token is appended to every text (copy-on-write copies
    for the first writer of a shared partial block) and every layer runs its block copies
    and the fused write + decode. Reported on the unique physical bytes read (shared blocks
    once) and, beside it, on the logical bytes (every text's tokens)."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_320_amd import PagedKVCache, _lib as L, torch_dtype

    w = base.scaled(steps=K + W)
    S, H, Hkv, D, B = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    NL = args.layers or 8
    elt, kv_elt = ELT[w.dtype], ELT[w.pool_dtype]
    log(f"setup: {w.name}, {NL} layers, drawing inputs on the GPU")
    # one draw for every layer: the layers' pools are separate buffers; their values do
    # not change what is read
    d = wl.draw(w, device="cuda")
    cache = PagedKVCache(w.num_blocks, B, Hkv, D, w.pool_dtype, layers=NL, device="cuda",
                         free_order=d.free_order, fill=float("nan"))
    ops = wl.script(w, d)
    first_step = ops.index(("step", 0))
    slot_of = {}

    def host_op(op):
        kind = op[0]
        if kind == "add":
            slot_of[op[1]] = cache.add()
        elif kind == "fork":
            slot_of[op[1]] = cache.fork(slot_of[op[2]])
        elif kind == "free":
            cache.free(slot_of.pop(op[1]))
        elif kind in ("prefill", "suffix"):
            ks = d.prefill_k if kind == "prefill" else d.suffix_k
            vs = d.prefill_v if kind == "prefill" else d.suffix_v
            if ks[op[2]].shape[0] == 0:
                return
            slots, pair = cache.alloc.append(slot_of[op[1]], int(ks[op[2]].shape[0]))
            if pair[0] >= 0:
                cache.copy([pair])
            for li in range(NL):
                cache.write(slots, ks[op[2]], vs[op[2]], layer=li)
        else:
            raise ValueError(kind)

    for op in ops[:first_step]:
        host_op(op)
    step_ops, cur = [], []
    for op in ops[first_step:]:
        if op[0] == "step":
            step_ops.append(cur)
            cur = []
        else:
            cur.append(op)
    torch.cuda.synchronize()

    att0 = wl.attended_at_step0(w, d)
    max_ctx_bound = max(att0) + K + W
    max_blocks = (max_ctx_bound + B - 1) // B
    ws = L.decode_workspace(S, H, D, max_ctx_bound, 0)
    R = K + W
    d_slots = torch.empty(S, dtype=torch.int64, device="cuda")
    d_lens = torch.empty(S, dtype=torch.int32, device="cuda")
    d_tables = torch.empty((S, max_blocks), dtype=torch.int32, device="cuda")
    d_pairs = torch.empty((S, 2), dtype=torch.int32, device="cuda")
    p_slots = [torch.empty(S, dtype=torch.int64, pin_memory=True) for _ in range(R)]
    p_lens = [torch.empty(S, dtype=torch.int32, pin_memory=True) for _ in range(R)]
    p_tables = [torch.empty((S, max_blocks), dtype=torch.int32, pin_memory=True) for _ in range(R)]
    p_pairs = [torch.empty((S, 2), dtype=torch.int32, pin_memory=True) for _ in range(R)]
    outs = [torch.empty((S, H, D), dtype=torch_dtype(w.dtype), device="cuda") for _ in range(NL)]
    ev, logical, unique, copies, cev = [], [], [], [], []
    mode = args.sharing_decode
    per_text = mode == "per-text"
    if not per_text:
        # the share groups are read off the block tables every step (pa_share_groups): a
        # request's samples hold its prompt's blocks in common; each forked pair of beams
        # also holds the blocks written before the pair split (up to the last block the
        # step's copy-on-write split), so the groups' promise holds by construction
        J = w.samples
        GMAX = S // 2
        d_groups = torch.empty((6, GMAX), dtype=torch.int32, device="cuda")
        p_groups = [torch.empty((6, GMAX), dtype=torch.int32, pin_memory=True) for _ in range(R)]
        if mode == "nested":
            pws = torch.empty(L.pa_decode_prefix2_workspace_bytes(
                S, H, Hkv, D, B, max_ctx_bound, GMAX, max_ctx_bound, GMAX, max_ctx_bound, 2,
                L.dtype_code(outs[0])), dtype=torch.uint8, device="cuda")
        else:
            pws = torch.empty(L.pa_decode_prefix_workspace_bytes(
                S, H, Hkv, D, B, max_ctx_bound, GMAX, max_ctx_bound, L.dtype_code(outs[0])),
                dtype=torch.uint8, device="cuda")
    ngroups = [0, 0]
    nfused = [0]  # timed steps whose new-token writes ran inside the nested decode
    planned_any = mode == "nested" and not args.per_layer_setup

    def step(i: int, timed: bool):
        for op in step_ops[i]:
            host_op(op)
        seqs = [slot_of[s] for s in range(S)]
        slots, pairs, done = cache.alloc.step_append(seqs)
        p_slots[i].numpy()[:] = slots
        L.pa_export_tables(cache.alloc.h, seqs, max_blocks, p_tables[i].numpy(),
                           p_lens[i].numpy())
        d_slots.copy_(p_slots[i], non_blocking=True)
        d_lens.copy_(p_lens[i], non_blocking=True)
        d_tables.copy_(p_tables[i], non_blocking=True)
        if not per_text:
            outer, inner = cache.alloc.share_groups(seqs, J, inner_members=2)
            pg = p_groups[i].numpy()
            for k, a in enumerate(outer + inner):
                pg[k, :len(a)] = a
            ngroups[0], ngroups[1] = len(outer[0]), len(inner[0])
            assert ngroups[0] > 0, "every request's samples share its prompt"
            d_groups.copy_(p_groups[i], non_blocking=True)
        if pairs:
            p_pairs[i].numpy()[:len(pairs)] = np.asarray(pairs, dtype=np.int32)
            d_pairs.copy_(p_pairs[i], non_blocking=True)
            if timed:
                c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                c0.record()
            for li in range(NL):
                L.pa_copy_blocks(cache.k[li], cache.v[li], d_pairs[:len(pairs)])
            if timed:
                c1.record()
                cev.append((c0, c1, len(pairs)))
        if timed:
            lens = p_lens[i].numpy()
            logical.append(decode_bytes(lens, H, D, B, elt, Hkv, kv_elt))
            unique.append(unique_kv_bytes(p_tables[i].numpy(), lens, B, Hkv, D, kv_elt) +
                          2 * S * H * D * elt + 4 * sum((int(x) + B - 1) // B for x in lens))
            copies.append(len(pairs))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        mctx = max_ctx_bound
        if per_text:
            for li in range(NL):
                L.pa_decode_attention_write(outs[li], d.step_q[i], cache.k[li], cache.v[li],
                                            d.step_k[i], d.step_v[i], d_slots, d_tables, d_lens,
                                            mctx, ws)
        else:
            no, ni = ngroups
            og = [d_groups[k, :no] for k in range(3)]
            ig = [d_groups[3 + k, :ni] for k in range(3)]
            nested = mode == "nested" and ni > 0
            # the nested decode stores the new rows itself (its texts' own pass) unless
            # --separate-write; otherwise pa_kv_write first
            fuse = nested and not args.separate_write
            nfused[0] += int(fuse and timed)
            if not fuse:
                for li in range(NL):
                    L.pa_kv_write(cache.k[li], cache.v[li], d.step_k[i], d.step_v[i], d_slots)
            planned = nested and not args.per_layer_setup
            if planned:
                # the set-up once per step: every layer attends with these tables, lengths
                # and groups
                L.pa_decode_prefix2_plan(d.step_q[i], cache.k[0], d_tables, d_lens, mctx, *og,
                                         max_ctx_bound, *ig, max_ctx_bound, 2, pws)
            counts = (no, max_ctx_bound, ni, max_ctx_bound, 2)
            rows = ({"k_new": d.step_k[i], "v_new": d.step_v[i], "slots": d_slots} if fuse
                    else {})
            for li in range(NL):
                if planned:
                    L.pa_decode_attention_prefix2_run(outs[li], d.step_q[i], cache.k[li],
                                                      cache.v[li], d_tables, d_lens, mctx,
                                                      *counts, pws, **rows)
                elif fuse:
                    L.pa_decode_attention_prefix2_write(
                        outs[li], d.step_q[i], cache.k[li], cache.v[li], d.step_k[i],
                        d.step_v[i], d_slots, d_tables, d_lens, mctx, *og, max_ctx_bound, *ig,
                        max_ctx_bound, 2, pws)
                elif nested:
                    L.pa_decode_attention_prefix2(outs[li], d.step_q[i], cache.k[li],
                                                  cache.v[li], d_tables, d_lens, mctx, *og,
                                                  max_ctx_bound, *ig, max_ctx_bound, 2, pws)
                else:
                    L.pa_decode_attention_prefix(outs[li], d.step_q[i], cache.k[li],
                                                 cache.v[li], d_tables, d_lens, mctx, *og,
                                                 max_ctx_bound, pws)
        if timed:
            e1.record()
            ev.append((e0, e1))

    log(f"warmup {W} steps")
    for i in range(W):
        step(i, False)
    torch.cuda.synchronize()
    log(f"timing {K} steps")
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    quiet_gc()
    t0.record()
    for i in range(W, W + K):
        step(i, True)
    t1.record()
    torch.cuda.synchronize()
    gc.enable()
    total_ms = t0.elapsed_time(t1)
    launch_ms = [a.elapsed_time(b) / NL for a, b in ev]
    avg = float(np.mean(launch_ms))
    u_launch, l_launch = float(np.mean(unique)), float(np.mean(logical))
    achieved = u_launch / (avg * 1e-3) / 1e9
    value = sum(unique) * NL / (total_ms * 1e-3) / 1e9
    copy_us = [a.elapsed_time(b) / NL * 1e3 for a, b, _ in cev]
    copy_bytes = [2 * 2 * n * Hkv * B * D * kv_elt for _, _, n in cev]  # K and V, read + write
    copy_gbps = (sum(copy_bytes) / (sum(copy_us) * 1e-6) / 1e9) if cev else None
    if cev:
        log(f"block copies: {np.mean(copy_us):.1f} us per layer ({np.mean(copy_bytes) / 1e6:.1f} MB "
            f"read + written, {copy_gbps:.0f} GB/s)")
    used_blocks, filled = cache.alloc.stats()
    util = filled / (used_blocks * B) if used_blocks else None
    fused_nested = nfused[0] == K
    if per_text:
        kernel_desc = "pa_decode_attention_write = decode_partition (new-token write fused) + " \
                      "decode_merge"
    elif mode != "nested":
        kernel_desc = "pa_kv_write + pa_decode_attention_prefix (set-up, prompt blocks once " \
                      "per group, each text's own blocks, merges)"
    else:
        kernel_desc = (("" if fused_nested else "pa_kv_write + ") +
                       ("pa_decode_prefix2_plan once per step (set-up) + "
                        "pa_decode_attention_prefix2_run per layer" if planned_any else
                        "pa_decode_attention_prefix2" + ("_write" if fused_nested else "") +
                        " per layer (set-up,") +
                       (" (" if planned_any else " ") +
                       "shared blocks once per group, each text's own blocks" +
                       (" with the new-token write" if fused_nested else "") + ", merges)")
    log(f"step {total_ms / K * 1e3:.1f} us ({NL} layers, {np.mean(copies):.0f} block copies "
        f"per layer), decode launch {avg * 1e3:.1f} us: unique {u_launch / 1e9:.2f} GB -> "
        f"{achieved:.0f} GB/s = {achieved / HBM_PEAK_GBPS:.1%} of 8 TB/s; logical "
        f"{l_launch / 1e9:.2f} GB -> {l_launch / (avg * 1e-3) / 1e9:.0f} GB/s")
    line = {
        "metric": "paged decode attention with shared prompt blocks: unique KV GB/s and % of HBM peak",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(total_ms / K, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded keys, values and queries; random block placement)",
        "config": {"workload": w.name, "seqs": S, "groups": w.groups, "samples": w.samples,
                   "prompt_len": w.prompt_len, "heads": H, "kv_heads": Hkv, "head_dim": D,
                   "block_size": B, "pool_blocks": w.num_blocks, "layers_per_step": NL,
                   "parallelism": "single GPU",
                   "new_token_write": "fused into decode" if (per_text or fused_nested)
                                      else ("pa_kv_write per layer" if nfused[0] == 0 else
                                            f"fused into decode on {nfused[0]} of {K} steps"),
                   "shared_blocks": {"per-text": "read once per text",
                                     "prefix": "prompt read once per group",
                                     "nested": "prompt once per group, a pair's blocks once "
                                               "per pair"}[mode]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": kernel_desc,
                     "avg_launch_us": round(avg * 1e3, 2),
                     "median_launch_us": round(float(np.median(launch_ms)) * 1e3, 2),
                     "min_launch_us": round(float(min(launch_ms)) * 1e3, 2),
                     "bytes_per_launch": int(u_launch)},
        "seq_layers_per_s": round(S * NL * K / (total_ms * 1e-3), 1),
        "cache_holding_tokens": round(util, 4) if util is not None else None,
        "logical_gbps": round(l_launch / (avg * 1e-3) / 1e9, 1),
        "logical_bytes_per_launch": int(l_launch),
        "block_copies_per_layer_per_step": float(np.mean(copies)),
        "copy_blocks_us_per_layer": round(float(np.mean(copy_us)), 2) if cev else None,
        "copy_blocks_gbps": round(copy_gbps, 1) if cev else None,
        "cpu_baseline": None,
    }
    return line


MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}   # dense fp16/bf16 matrix-core peak


def prompt_flops(prompt_lens, prefix_len, H, D) -> int:
    """Algorithmic flops of one prompt-phase launch: the query at position p takes
    2*D flops per attended key for q.k and 2*D for the weighted sum of values."""
    keys = sum(n * prefix_len + n * (n + 1) // 2 for n in prompt_lens)
    return 4 * D * H * keys


def bench_prompt(args, w) -> dict:
    """The prompt phase: per step, every text is added (after the shared cached prefix,
    if any), its prompt's keys and values are written, and pa_prefill_attention runs."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_320_amd import PagedKVCache, _lib as L, torch_dtype

    K, W = args.steps, args.warmup
    S, H, Hkv, D, B = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size
    NL = args.layers or 4
    log(f"setup: {w.name}, {NL} layers, drawing inputs on the GPU")
    d = wl.draw_prompt(w, device="cuda")
    lens = d.prompt_lens
    T = sum(lens)
    cache = PagedKVCache(w.num_blocks, B, Hkv, D, w.dtype, layers=NL, device="cuda",
                         free_order=d.free_order, fill=float("nan"))
    prefix_seq = None
    if w.prefix_len:
        prefix_seq = cache.add()
        slots, _ = cache.alloc.append(prefix_seq, w.prefix_len)
        for li in range(NL):
            cache.write(slots, d.prefix_k, d.prefix_v, layer=li)
    pk = torch.cat(d.prompt_k).contiguous()
    pv = torch.cat(d.prompt_v).contiguous()
    q = d.q
    q_start = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32,
                           device="cuda")
    max_blocks = (w.prefix_len + max(lens) + B - 1) // B
    d_slots = torch.empty(T, dtype=torch.int64, device="cuda")
    d_tables = torch.empty((S, max_blocks), dtype=torch.int32, device="cuda")
    d_lens = torch.empty(S, dtype=torch.int32, device="cuda")
    outs = [torch.empty((T, H, D), dtype=torch_dtype(w.dtype), device="cuda") for _ in range(NL)]
    R = K + W  # one pinned staging buffer per step: the host never waits on an upload
    p_slots = [torch.empty(T, dtype=torch.int64, pin_memory=True) for _ in range(R)]
    p_tables = [torch.empty((S, max_blocks), dtype=torch.int32, pin_memory=True) for _ in range(R)]
    p_lens = [torch.empty(S, dtype=torch.int32, pin_memory=True) for _ in range(R)]
    up_done = [torch.cuda.Event() for _ in range(R)]
    ev = []
    tables0 = {}

    def step(i: int, timed: bool):
        seqs = [cache.fork(prefix_seq) if prefix_seq is not None else cache.add() for _ in lens]
        r = i % R
        up_done[r].synchronize()
        off = 0
        for sid, n in zip(seqs, lens):
            slots, pair = cache.alloc.append(sid, n)
            assert pair == (-1, -1), "the cached prefix ends on a block boundary"
            p_slots[r].numpy()[off:off + n] = slots
            off += n
        L.pa_export_tables(cache.alloc.h, seqs, max_blocks, p_tables[r].numpy(), p_lens[r].numpy())
        if i == 0:
            tables0["tables"] = p_tables[r].numpy().copy()
            tables0["lens"] = p_lens[r].numpy().copy()
        d_slots.copy_(p_slots[r], non_blocking=True)
        d_tables.copy_(p_tables[r], non_blocking=True)
        d_lens.copy_(p_lens[r], non_blocking=True)
        up_done[r].record()
        for li in range(NL):
            cache.write(d_slots, pk, pv, layer=li)
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        for li in range(NL):
            L.pa_prefill_attention(outs[li], q, cache.k[li], cache.v[li], d_tables, d_lens,
                                   q_start, max(lens))
        if timed:
            e1.record()
            ev.append((e0, e1))
        for sid in seqs:
            cache.free(sid)

    log(f"warmup {W} steps")
    for i in range(W):
        step(i, False)
        if i == 0:
            torch.cuda.synchronize()
            out0 = outs[0].float().cpu().numpy()
    torch.cuda.synchronize()
    log(f"timing {K} steps")
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    quiet_gc()
    wall0 = time.perf_counter()
    t0.record()
    for i in range(W, W + K):
        step(i, True)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gc.enable()
    total_ms = t0.elapsed_time(t1)
    flops = prompt_flops(lens, w.prefix_len, H, D)
    launch_ms = [a.elapsed_time(b) / NL for a, b in ev]
    avg = float(np.mean(launch_ms))
    achieved = flops / (avg * 1e-3) / 1e12
    value = flops * NL * K / (total_ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    log(f"step {total_ms / K * 1e3:.1f} us ({NL} layers), prefill launch {avg * 1e3:.1f} us "
        f"(min {min(launch_ms) * 1e3:.1f}), {achieved:.1f} TFLOP/s = {achieved / peak:.1%} of "
        f"{peak:.0f}")

    cpu, err0 = None, None
    if not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle, sampled query rows of one layer, one thread")
        cpu, err0 = cpu_baseline_prompt(w, d, tables0, args.cpu_seconds, out0)
        log(f"cpu baseline {cpu['value']} GFLOP/s; sampled max abs error vs oracle {err0:.3e}")
    line = {
        "metric": "prompt-phase paged attention: TFLOP/s and % of the fp16/bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": f"synthetic (seeded N(0,1)*{w.kv_std:.4g} keys/values, N(0,{w.q_std:g}) queries; "
                "random block placement)",
        "config": {"workload": w.name, "seqs": S, "prompt_tokens": T, "prefix_len": w.prefix_len,
                   "heads": H, "kv_heads": Hkv, "head_dim": D, "block_size": B,
                   "pool_blocks": w.num_blocks, "layers_per_step": NL,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "pa_prefill_attention (prefill_kernel)",
                     "avg_launch_us": round(avg * 1e3, 2), "flops_per_launch": flops},
        "cpu_baseline": cpu,
        "sampled_max_abs_err_vs_oracle": err0,
        "wall_s_timed": round(wall, 4),
    }
    return line


def cpu_baseline_prompt(w, d, tables0, seconds: float, gpu_out0):
    """The prompt oracle on seeded sampled (row, head) pairs of step 0, one layer, one thread,
    about `seconds` long; also the GPU's error on those pairs."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    from oracle.prefill import prefill_attention

    lens = d.prompt_lens
    B, Hkv, D = w.block_size, w.num_kv_heads, w.head_dim
    tables, ctx = tables0["tables"], tables0["lens"]
    # the pools as the step-0 writes left them, built on the host from the same draws
    N = w.num_blocks
    kc = torch.full((N, Hkv, B, D), float("nan"), dtype=d.q.dtype)
    vc = torch.full((N, Hkv, B, D), float("nan"), dtype=d.q.dtype)
    for s in range(len(lens)):
        ks = torch.cat([d.prefix_k.cpu(), d.prompt_k[s].cpu()])
        vs = torch.cat([d.prefix_v.cpu(), d.prompt_v[s].cpu()])
        t = torch.arange(ks.shape[0])
        blk = torch.from_numpy(tables[s].astype(np.int64))[t // B]
        kc[blk, :, t % B] = ks
        vc[blk, :, t % B] = vs
    q = d.q.cpu()
    q_start = np.concatenate([[0], np.cumsum(lens)])
    rng = np.random.default_rng(0)
    rows = [(int(rng.integers(q.shape[0])), int(rng.integers(w.num_heads))) for _ in range(4096)]
    rows += [(int(q_start[s + 1] - 1), 0) for s in range(len(lens))]  # every text's last row
    done, got, t0 = [], {}, time.perf_counter()
    with threadpool_limits(limits=1):
        for i in range(0, len(rows), 512):
            part = rows[i:i + 512]
            o = prefill_attention(q, kc, vc, tables, ctx, q_start, B, rows=part)
            for r, h in part:
                got[(r, h)] = o[r, h].copy()
            del o
            done += part
            if time.perf_counter() - t0 >= seconds:
                break
    dt = time.perf_counter() - t0
    where = {}
    for s in range(len(lens)):
        for i in range(lens[s]):
            where[int(q_start[s] + i)] = w.prefix_len + i
    keys = sum(where[r] + 1 for r, _ in done)
    flops = 4 * D * keys
    err = float(max(np.abs(gpu_out0[r, h].astype(np.float64) - got[(r, h)]).max() for r, h in done))
    return {"value": round(flops / dt / 1e9, 4), "unit": "GFLOP/s", "cores": 1, "kind": "oracle",
            "host": host_cores(),
            "sample": f"{w.name} one layer, step 0: {len(done)} seeded (query row, head) pairs "
                      f"in {dt:.1f} s (fp64 numpy, BLAS limited to 1 thread)"}, err


def bench_decode(args, base, K: int, W: int, layers: int = 0, placement: str = "random",
                 probes: bool = True, cpu: bool = True) -> dict:
    """Decode steps of a workload whose texts each decode one token per step: the JSON line.

    layers: pools per step (0: --layers, else enough for >= 2 GB of pools); placement
    "random" (the workload's seeded free-list permutation) or "identity" (blocks handed out
    in id order); probes / cpu: also run the read probes and swap probe / the CPU oracle."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_320_amd import PagedKVCache, _lib as L, torch_dtype

    kv_elt = ELT[base.pool_dtype]
    fp8 = base.pool_dtype == "fp8"
    w = base.scaled(steps=K + W)
    S, H, Hkv, D, B = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.block_size

    log(f"setup: {w.name}, drawing inputs on the GPU")
    draws = [wl.draw(w, device="cuda")]
    lens0 = [n + 1 for n in draws[0].prefill_lens]  # attended at step 0
    per_layer = sum(lens0) * 2 * Hkv * D * kv_elt
    NL = layers or args.layers or min(16, max(8, -(-2_000_000_000 // per_layer)))
    need = sum((n + K + W + B - 1) // B for n in draws[0].prefill_lens)
    assert need <= w.num_blocks, f"the pool holds {w.num_blocks} blocks; {K + W} steps need {need}"
    log(f"{NL} layers")
    for li in range(1, NL):
        # every layer holds the same texts (lengths), with its own keys, values and queries
        draws.append(wl.draw(w.scaled(seed=w.seed * 1000 + li, length_kind="list",
                                      ctx_list=tuple(lens0)), device="cuda"))
    # random placement: the workload's seeded permutation of the free list; identity: the
    # free list in block order, so that every text's blocks are consecutive ids
    free_order = draws[0].free_order if placement == "random" else \
        np.arange(w.num_blocks, dtype=np.int32)
    cache = PagedKVCache(w.num_blocks, B, Hkv, D, w.pool_dtype, layers=NL, device="cuda",
                         free_order=free_order, fill=float("nan"),
                         k_scale=w.k_scale, v_scale=w.v_scale)
    seqs = []
    for s in range(S):
        sid = cache.add()
        slots, pair = cache.alloc.append(sid, draws[0].prefill_lens[s])
        assert pair == (-1, -1)
        for li in range(NL):
            cache.write(slots, draws[li].prefill_k[s], draws[li].prefill_v[s], layer=li)
        seqs.append(sid)
    torch.cuda.synchronize()

    max_blocks = (max(lens0) + K + W + B - 1) // B
    max_ctx_bound = max(lens0) + K + W
    T = args.partition_tokens
    ws = L.decode_workspace(S, H, D, max_ctx_bound, T)
    # a step's slots (int64) and lengths (int32) share one buffer: one upload per step
    meta_bytes = 12 * S
    d_meta = torch.empty(meta_bytes, dtype=torch.uint8, device="cuda")
    d_slots = d_meta[:8 * S].view(torch.int64)
    d_lens = d_meta[8 * S:].view(torch.int32)
    d_tables = torch.empty((S, max_blocks), dtype=torch.int32, device="cuda")
    d_pairs = torch.empty((S, 2), dtype=torch.int32, device="cuda")
    # one pinned staging buffer per step: the host allocator runs ahead of the GPU and never
    # waits on an upload event (waiting on a ring slot let the host sleep for milliseconds
    # past the event and the GPU run dry)
    R = K + W
    p_meta = [torch.empty(meta_bytes, dtype=torch.uint8, pin_memory=True) for _ in range(R)]
    p_slots = [m[:8 * S].view(torch.int64) for m in p_meta]
    p_lens = [m[8 * S:].view(torch.int32) for m in p_meta]
    p_tables = [torch.empty((S, max_blocks), dtype=torch.int32, pin_memory=True) for _ in range(R)]
    p_pairs = [torch.empty((S, 2), dtype=torch.int32, pin_memory=True) for _ in range(R)]
    up_done = [torch.cuda.Event() for _ in range(R)]
    outs = [torch.empty((S, H, D), dtype=torch_dtype(w.dtype), device="cuda") for _ in range(NL)]
    newk = [[dl.step_k[i] for i in range(K + W)] for dl in draws]
    newv = [[dl.step_v[i] for i in range(K + W)] for dl in draws]
    qs = [[dl.step_q[i] for i in range(K + W)] for dl in draws]
    step_lens = []
    ev = []  # (start, end) events around every timed decode launch
    wev = []  # the same around the separate new-token writes
    graphs = {}

    # 16- and 32-bit pools: each layer's new-token write runs inside its decode launch
    # (pa_decode_attention_write); E4M3 pools quantize the new rows in pa_kv_write_fp8 first
    fused = not fp8 and not args.separate_write

    def write_all(i):
        for li in range(NL):
            cache.write(d_slots, newk[li][i], newv[li][i], layer=li)

    def decode_all(i, mctx):
        for li in range(NL):
            if fp8:
                L.pa_decode_attention_fp8(outs[li], qs[li][i], cache.k[li], cache.v[li], d_tables,
                                          d_lens, mctx, ws, w.k_scale, w.v_scale, partition_tokens=T)
            elif fused:
                L.pa_decode_attention_write(outs[li], qs[li][i], cache.k[li], cache.v[li],
                                            newk[li][i], newv[li][i], d_slots, d_tables, d_lens,
                                            mctx, ws, partition_tokens=T)
            else:
                L.pa_decode_attention(outs[li], qs[li][i], cache.k[li], cache.v[li], d_tables,
                                      d_lens, mctx, ws, partition_tokens=T)

    def capture():
        """HIP graphs for every step from the second on, over that step's own inputs: its
        NL new-token writes (unless fused), then its NL decode launches (max_context_len =
        the bound the workspace was sized for; the kernels read the true lengths from d_lens)."""
        torch.cuda.synchronize()
        for i in range(1, K + W):
            g_write, g_dec = None, torch.cuda.CUDAGraph()
            if not fused:
                g_write = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g_write):
                    write_all(i)
            with torch.cuda.graph(g_dec):
                decode_all(i, max_ctx_bound)
            graphs[i] = (g_write, g_dec)
        torch.cuda.synchronize()

    last_tables = None

    def step(i: int, timed: bool):
        nonlocal last_tables
        slots, pairs, done = cache.alloc.step_append(seqs)
        r = i % R
        up_done[r].synchronize()
        p_slots[r].numpy()[:] = slots
        L.pa_export_tables(cache.alloc.h, seqs, max_blocks, p_tables[r].numpy(), p_lens[r].numpy())
        lens = p_lens[r].numpy().copy()
        step_lens.append(lens)
        d_meta.copy_(p_meta[r], non_blocking=True)
        # the tables change only when a text opens a new block (every block_size steps):
        # upload them only then (an upload of the unchanged 33 KB tables of the 32-text
        # workloads stalled the host for ~6 ms every ten-odd steps)
        if last_tables is None or not np.array_equal(last_tables, p_tables[r].numpy()):
            d_tables.copy_(p_tables[r], non_blocking=True)
            last_tables = p_tables[r].numpy().copy()
        if pairs:
            p_pairs[r].numpy()[:len(pairs)] = np.asarray(pairs, dtype=np.int32)
            d_pairs.copy_(p_pairs[r], non_blocking=True)
        up_done[r].record()
        mctx = int(lens.max())
        # every layer's copies and new-token writes, then every layer's attention back to
        # back: one event pair brackets the NL decode launches of the step
        if pairs:
            for li in range(NL):
                L.pa_copy_blocks(cache.k[li], cache.v[li], d_pairs[:len(pairs)])
        if not fused:
            if timed:
                w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                w0.record()
            if i in graphs:
                graphs[i][0].replay()
            else:
                write_all(i)
            if timed:
                w1.record()
                wev.append((w0, w1))
        if timed:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        if i in graphs:
            graphs[i][1].replay()
        else:
            decode_all(i, mctx)
        if timed:
            e1.record()
            ev.append((e0, e1))

    if args.copy_calibration and probes:
        run_copy_calibration(L, torch)

    log(f"warmup {W} steps")
    for i in range(W):
        if i == 1 and args.graph:
            capture()
        step(i, False)
        if i == 0:
            torch.cuda.synchronize()
            out0 = outs[0].float().cpu().numpy()
    torch.cuda.synchronize()

    log(f"timing {K} steps ({'HIP graph replay' if graphs else 'eager launches'})")
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    quiet_gc()
    wall0 = time.perf_counter()
    t_start.record()
    host_s = 0.0
    for i in range(W, W + K):
        h0 = time.perf_counter()
        step(i, True)
        host_s += time.perf_counter() - h0
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gc.enable()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K

    timed_lens = step_lens[W:]
    elt = ELT[w.dtype]
    bytes_per_step = [decode_bytes(l, H, D, B, elt, Hkv, kv_elt) * NL for l in timed_lens]
    value = sum(bytes_per_step) / (total_ms * 1e-3) / 1e9
    launch_ms = [a.elapsed_time(b) / NL for a, b in ev]   # per decode launch, per step
    avg_launch_ms = float(np.mean(launch_ms))
    bytes_per_launch = float(np.mean([decode_bytes(l, H, D, B, elt, Hkv, kv_elt)
                                      for l in timed_lens]))
    achieved = bytes_per_launch / (avg_launch_ms * 1e-3) / 1e9
    traffic = measured_traffic(fused) if (base.name == "opt13b_7x2048_f16_b16" and
                                          placement == "random") else None
    log(f"host time per step (allocator, uploads, launches) {host_s / K * 1e6:.1f} us")
    write_us = float(np.mean([a.elapsed_time(b) / NL * 1e3 for a, b in wev])) if wev else None
    if wev:
        log(f"separate new-token write: {write_us:.1f} us per layer")
    used_blocks, filled = cache.alloc.stats()
    util = filled / (used_blocks * B) if used_blocks else None
    log(f"step {ms_per_step * 1e3:.1f} us ({NL} layers), decode launch {avg_launch_ms * 1e3:.1f} us "
        f"(median {np.median(launch_ms) * 1e3:.1f}, min {min(launch_ms) * 1e3:.1f}), "
        f"{achieved:.0f} GB/s = {achieved / HBM_PEAK_GBPS:.1%} of 8 TB/s; {placement} placement; "
        f"cache holding tokens {util:.2%}")

    probe = tprobe = vprobe = swap = None
    if probes and not args.no_probe:
        probe = run_probe(L, torch)
        log(f"stream-read probe: {probe:.0f} GB/s")
        vprobe = run_volume_probe(L, torch, int(bytes_per_launch))
        log(f"same-volume stream probe ({int(bytes_per_launch) >> 20} MiB per launch, "
            f"contiguous): {vprobe:.0f} GB/s")
        tprobe = run_tile_probe(L, torch, B * D * kv_elt, int(bytes_per_launch))
        log(f"same-pattern probe ({int(bytes_per_launch) >> 20} MiB per launch in random "
            f"{B * D * kv_elt} B tiles): {tprobe:.0f} GB/s")
        swap = run_swap_probe(cache, seqs, torch)
        log(f"swap of two texts ({NL} layers, {swap[2] / 1e6:.0f} MB each way): out to pinned "
            f"host memory {swap[0]:.1f} GB/s, back in {swap[1]:.1f} GB/s")

    cpu_line = None
    err0 = None
    if cpu and not args.no_cpu_baseline:
        log("cpu baseline: fp64 oracle, one layer, one thread")
        cpu_line, err0 = cpu_baseline(base, draws[0], args.cpu_seconds, out0)
        log(f"cpu baseline {cpu_line['value']} GB/s; step-0 max abs error vs oracle {err0:.3e}")

    line = {
        "metric": "paged decode attention: KV GB/s and % of HBM peak; sequences·layers/sec",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": f"synthetic (seeded N(0,1)*{w.kv_std:.4g} keys/values, N(0,{w.q_std:g}) queries; "
                f"{placement} block placement)",
        "config": {"workload": base.name, "seqs": S,
                   "context_at_step0": (lens0[0] if len(set(lens0)) == 1 else
                                        f"{min(lens0)}..{max(lens0)}, mean {np.mean(lens0):.0f}"),
                   "heads": H, "kv_heads": Hkv, "head_dim": D, "block_size": B,
                   "kv_cache_dtype": "fp8_e4m3" if fp8 else w.dtype,
                   "pool_blocks": w.num_blocks, "layers_per_step": NL,
                   "partition_tokens": T, "parallelism": "single GPU",
                   "launch": "HIP graph replay" if graphs else "eager",
                   "new_token_write": "fused into decode" if fused else "pa_kv_write"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "seq_layers_per_s": round(S * NL * K / (total_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
                     "traffic_source": traffic_note(traffic),
                     "kernel": ("pa_decode_attention_write = decode_partition (new-token write "
                                "fused) + decode_merge") if fused else
                               "pa_decode_attention = decode_partition + decode_merge",
                     "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                     "median_launch_us": round(float(np.median(launch_ms)) * 1e3, 2),
                     "min_launch_us": round(float(min(launch_ms)) * 1e3, 2),
                     "bytes_per_launch": int(bytes_per_launch)},
        "cache_holding_tokens": round(util, 4) if util is not None else None,
        "placement": placement,
        "kv_write_us_per_layer": round(write_us, 2) if wev else None,
        "swap_out_gbps": round(swap[0], 2) if swap else None,
        "swap_in_gbps": round(swap[1], 2) if swap else None,
        "swap_bytes": int(swap[2]) if swap else None,
        "probe_read_gbps": round(probe, 1) if probe else None,
        "probe_same_volume_gbps": round(vprobe, 1) if vprobe else None,
        "probe_same_pattern_gbps": round(tprobe, 1) if tprobe else None,
        "cpu_baseline": cpu_line,
        "step0_max_abs_err_vs_oracle": err0,
        "wall_s_timed": round(wall, 4),
        "decode_src_sha256_16": src_hash(),
    }
    return line


CONFIG_RUNS = (
    # (workload, steps, warmup, layers): the other decode configurations, each far beyond the
    # 256 MB Infinity Cache per launch, timed after the headline one and reported beside it
    ("opt13b_mixed256_f16_b16", 10, 3, 2),
    ("long_16x32k_f16_b16", 6, 2, 2),
    ("sharing_32x8_bf16_b16", 8, 2, 8),
)


def config_summary(line: dict) -> dict:
    """The figures of one configuration's JSON line that go into the headline line."""
    r = line["roofline"]
    out = {"op_us_mean": r["avg_launch_us"], "op_us_median": r.get("median_launch_us"),
           "op_us_min": r.get("min_launch_us"), "bytes_per_op": r["bytes_per_launch"],
           "gbps": r["achieved"], "frac_of_hbm_peak": r["frac"],
           "ms_per_step": line["ms_per_step"], "layers_per_step": line["config"]["layers_per_step"],
           "steps": line["steps"], "kernel": r["kernel"]}
    for k in ("seq_layers_per_s", "cache_holding_tokens", "logical_gbps",
              "logical_bytes_per_launch", "copy_blocks_us_per_layer", "copy_blocks_gbps",
              "placement"):
        if k in line:
            out[k] = line[k]
    if "logical_gbps" in line:
        out["bytes"] = "unique physical blocks (shared blocks once); logical beside it"
    return out


def free_gpu():
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="opt13b_7x2048_f16_b16",
                    help="workload from workloads.BY_NAME")
    ap.add_argument("--layers", type=int, default=0,
                    help="pools (model layers) per step; 0 = enough for >= 2 GB of pools")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--placement", choices=["random", "identity"], default="random",
                    help="block placement of the decode workloads: the seeded random free list, "
                         "or blocks handed out in id order")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the headline workload (not the other configurations, nor "
                         "the identity-placement run)")
    ap.add_argument("--separate-write", action="store_true",
                    help="write each layer's new token with pa_kv_write before its decode launch "
                         "instead of inside it (pa_decode_attention_write, and "
                         "pa_decode_attention_prefix2_write for the nested shared-block decode)")
    ap.add_argument("--per-layer-setup", action="store_true",
                    help="nested shared-block decode: the set-up in every layer's call "
                         "(pa_decode_attention_prefix2_write) instead of once per step "
                         "(pa_decode_prefix2_plan, then pa_decode_attention_prefix2_run per "
                         "layer)")
    ap.add_argument("--sharing-decode", choices=["nested", "prefix", "per-text"],
                    default="nested",
                    help="shared-prompt workloads: every shared block read once (the prompt per "
                         "group, each forked pair's blocks per pair: pa_decode_attention_prefix2)"
                         ", the prompt once per group (pa_decode_attention_prefix), or every "
                         "text its whole table (pa_decode_attention_write)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each decode step's writes and decode launches from HIP graphs "
                         "captured for that step instead of launching them one by one")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run pa_copy_probe over 512 MiB (reference for memory counters)")
    ap.add_argument("--line-out", metavar="PATH",
                    help="also write the JSON line to PATH (for the counter runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --copy-calibration --line-out DIR/line.json` into " +
                         os.path.relpath(TRAFFIC_FILE, ROOT))
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from_counters(*args.traffic_from)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (the decode "
              "path would shard by text, with no exchange between GPUs). "
              f"Got --gpus {args.gpus}, WORLD_SIZE {world}.", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as wl
    from paged_kv_cache_320_amd import _lib as L

    L.lib()  # fails loudly when libpagedkv.so has not been built
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    base = wl.BY_NAME[args.workload]
    if isinstance(base, wl.PromptWorkload):
        line = bench_prompt(args, base)
    elif base.length_kind == "sharing":
        line = bench_sharing(args, base, args.steps, args.warmup)
    else:
        assert base.length_kind in ("fixed", "uniform", "list"), \
            "bench.py times batches whose texts each decode one token per step (no forks)"
        line = bench_decode(args, base, args.steps, args.warmup, placement=args.placement)
        if args.workload == "opt13b_7x2048_f16_b16" and not args.no_configs:
            free_gpu()
            # the paging cost: the same step with every text's blocks in id order
            log("identity placement run")
            ident = bench_decode(args, base, args.steps, args.warmup, placement="identity",
                                 probes=False, cpu=False)
            r_op, i_op = line["roofline"]["avg_launch_us"], ident["roofline"]["avg_launch_us"]
            line["placement_cost"] = {
                "random_op_us": r_op, "identity_op_us": i_op,
                "random_over_identity": round(r_op / i_op, 4),
                "identity_op_us_median": ident["roofline"]["median_launch_us"],
                "random_op_us_median": line["roofline"]["median_launch_us"]}
            del ident
            configs = {}
            for name, k, w_, nl in CONFIG_RUNS:
                free_gpu()
                cw = wl.BY_NAME[name]
                log(f"configuration {name}: {k} steps, {w_} warmup, {nl} layers")
                sub = argparse.Namespace(**{**vars(args), "layers": nl, "partition_tokens": 0})
                if cw.length_kind == "sharing":
                    c = bench_sharing(sub, cw, k, w_)
                else:
                    c = bench_decode(sub, cw, k, w_, layers=nl, probes=False, cpu=False)
                configs[name] = config_summary(c)
            line["configs"] = configs
    if args.line_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.line_out)), exist_ok=True)
        with open(args.line_out, "w") as f:
            f.write(json.dumps(line) + "\n")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
