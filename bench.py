#!/usr/bin/env python3
"""Benchmark of one paged-KV decode step on one MI355X.

A step is the whole hot path for one decode layer: slot resolution for the new
tokens and the scatter-write of their K/V into the paged cache (one call,
paged_kv_write_positions), then decode attention (plus the log-sum-exp merge when
the context is split).  Inputs are synthetic and
seeded, resident in HBM before timing starts.

Prints ONE JSON line on stdout:
  value        effective KV GB/s of the step = algorithmic bytes of a step / step time,
               on the headline workload (the Llama-3-8B-shaped layer unless --config)
  roofline     the decode call (its dominant kernel) against the 8 TB/s HBM peak: its
               average duration over back-to-back calls on 4 copies of the layer's cache
               taken in turn (each call reads cold data, as consecutive layers do), HIP
               events on the stream it runs on; single launches after an L2/MALL flush
               are reported beside it.  Bytes are the algorithmic bytes; where sequences
               share blocks (prefix caching) the unique bytes, each shared block once
  read_ceiling the same tiles read by a streaming-read probe, timed the same way
  cpu_baseline the fp64 oracle timed on this host's cores on a bounded sample
  configs      every one of the five decode-layer workloads measured the same way (the
               headline's entry is the headline's measurement), each with its own
               roofline fraction, read ceiling, single-launch percentiles and oracle
               baseline; --only skips them
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0
METRIC = "effective KV GB/s (% of HBM peak) and seq-heads/s per decode layer"
DT_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
CSRC = "paged_kv_cache_27_amd/csrc"
KERNEL_SOURCES = [f"{CSRC}/{n}" for n in (
    "decode.hip", "decode_sk.hip", "decode_sk_kernel.h", "decode_sk_bf16.hip", "decode_sk_f16.hip",
    "decode_sk_pre.hip", "decode_sk_pre_fp8.hip", "mfma_rows.hip",
    "decode_sk_f32.hip", "decode_sk_fp8_qbf16.hip", "decode_sk_fp8_qf16.hip", "decode_common.h",
    "pkv_device.h", "pkv_launch.h", "api.cpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama3-8b-shaped-bf16-64seq",
                    help="workload name or 1-based index (default: the 8B-shaped layer)")
    ap.add_argument("--reps", type=int, default=30, help="cold-cache reps of the roofline leg (>= 1)")
    ap.add_argument("--all", action="store_true",
                    help="also the windowed workload, block moves and prefill (stderr + --json-out)")
    ap.add_argument("--only", action="store_true",
                    help="measure the headline workload only (no configs array; e.g. under a profiler)")
    ap.add_argument("--config-cpu-seconds", type=float, default=3.0,
                    help="wall budget of the oracle leg of each non-headline workload")
    ap.add_argument("--json-out", default=None, help="write per-workload results here")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall budget of the oracle leg")
    ap.add_argument("--partition", type=int, default=None, help="override the partition size")
    ap.add_argument("--no-shared-prefix", action="store_true",
                    help="prefix-sharing workloads: plain decode instead of the shared-prefix entry point")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy --steps times (counter calibration)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run the chunked-prefill leg (--reps calls) and print its result")
    ap.add_argument("--blocks-only", action="store_true",
                    help="only run the block-moves leg (--reps calls each) and print its result")
    return ap.parse_args()


def pick_config(spec):
    from workloads import CONFIGS, EXTRA_CONFIGS
    if str(spec).isdigit():
        return CONFIGS[int(spec) - 1]
    for c in CONFIGS + EXTRA_CONFIGS:
        if c.name == spec:
            return c
    raise SystemExit(f"unknown workload {spec}; known: {[c.name for c in CONFIGS + EXTRA_CONFIGS]}")


def window_tokens(ctx, window, sinks):
    """Positions a decode over a sliding window attends to: the last `window` of a
    ctx-token context plus its first `sinks` (every position when window is 0)."""
    import numpy as np
    t = np.arange(int(ctx))
    return t if window == 0 else t[(t >= ctx - window) | (t < sinks)]


def algorithmic_bytes(w):
    """Bytes the method must move: decode reads each sequence's whole context once per KV
    head plus q, out, its block-table entries and context length; the write reads the new
    K/V and writes the cache rows; slot resolution, inside the write, reads each token's
    sequence ID, position and table entry."""
    c = w.cfg
    n, hq, hkv, d, B = c.num_seqs, c.num_q_heads, c.num_kv_heads, c.head_dim, c.block_size
    ctx = w.context_lens.astype("int64")
    if c.window:  # only the attended tokens and the table entries of their blocks
        att = [window_tokens(x, c.window, c.sinks) for x in ctx]
        kv = sum(len(a) for a in att) * hkv * d * 2 * DT_BYTES[c.kv_dtype]
        table = sum(len(set((a // B).tolist())) for a in att) * 4 + 4 * n
    else:
        kv = int(ctx.sum()) * hkv * d * 2 * DT_BYTES[c.kv_dtype]
        table = int(((ctx + B - 1) // B).sum()) * 4 + 4 * n
    qo = n * hq * d * (DT_BYTES[c.q_dtype] + DT_BYTES[c.out_dtype])
    decode = kv + table + qo
    write = n * hkv * d * 2 * (DT_BYTES[c.src_dtype] + DT_BYTES[c.kv_dtype])
    slots = n * (4 + 4 + 4)
    unique_kv = w.kv_bytes_unique()
    return {"decode": decode, "kv": kv, "kv_unique": unique_kv, "decode_unique": decode - kv + unique_kv,
            "write": write, "slots": slots, "step": decode + write + slots}


def roofline_bytes(nbytes, w):
    """Bytes of one decode call priced against HBM: each shared physical block once when
    sequences share blocks (the logical bytes, every sequence's whole context, would count
    a shared prefix once per sequence and could exceed the peak), else the algorithmic
    bytes."""
    return nbytes["decode_unique"] if w.shared_blocks else nbytes["decode"]


class Step:
    """Device-resident inputs of one decode step and the two ABI calls that run it (the
    write with its slot resolution, then the decode)."""

    def __init__(self, w, partition=None, shared_prefix=True):
        import numpy as np
        import torch
        import paged_kv_cache_27_amd as pkv
        from workloads import POISON_BITS, cache_shape

        self.pkv, self.torch, self.w = pkv, torch, w
        c = w.cfg
        dev = "cuda"
        tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

        def up(x, dt):
            if dt == "bf16":
                return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

        bits = POISON_BITS[c.kv_dtype]
        store = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16, "fp8": torch.uint8}[c.kv_dtype]
        view = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.uint8}[c.kv_dtype]
        self.k_cache = torch.full(cache_shape(w), bits, dtype=store, device=dev).view(view)
        self.v_cache = torch.full(cache_shape(w), bits, dtype=store, device=dev).view(view)
        self.kv_dtype = "fp8" if c.kv_dtype == "fp8" else None
        self.block_tables = torch.from_numpy(w.block_tables).to(dev)
        self.context_lens = torch.from_numpy(w.context_lens).to(dev)
        self.q = up(w.q, c.q_dtype)
        self.new_k = up(w.new_k, c.src_dtype)
        self.new_v = up(w.new_v, c.src_dtype)
        self.new_seq = torch.from_numpy(w.new_seq).to(dev)
        self.new_pos = torch.from_numpy(w.new_pos).to(dev)
        self.slots = torch.empty(c.num_seqs, dtype=torch.int64, device=dev)
        self.out = torch.empty((c.num_seqs, c.num_q_heads, c.head_dim), dtype=tdt[c.out_dtype], device=dev)
        self.partition = c.partition_size if partition is None else partition
        # prefix sharing maps many sequences to one physical block: say so (cache policy)
        self.shared = bool(w.shared_blocks)
        self.desc = pkv.cache_desc(self.k_cache, self.kv_dtype, w.k_scale, w.v_scale, self.shared)
        need = pkv.paged_attention_workspace_size(self.desc, c.q_dtype, c.num_seqs, c.num_q_heads,
                                                  w.max_context_len, self.partition)
        self.schedule = pkv.paged_attention_schedule(self.desc, c.q_dtype, c.num_seqs,
                                                     c.num_q_heads, w.max_context_len,
                                                     self.partition)
        self.workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
        # Prefix sharing: the shared-prefix entry point with the workload's own grouping
        # (every group's prefix read once), unless a partition was asked for.
        self.prefix = None
        if self.shared and c.ctx_kind == "prefix" and self.partition == 0 and shared_prefix:
            starts = w.prefix_group_starts()
            plens = np.full(c.num_seqs, int(c.ctx_params[0]), np.int32)
            gmax, pmax = int(np.diff(starts).max()), int(plens.max())
            self.prefix = (torch.from_numpy(starts).to(dev), torch.from_numpy(plens).to(dev), gmax, pmax)
            pneed = pkv.paged_attention_shared_prefix_workspace_size(
                self.desc, c.q_dtype, c.num_seqs, c.num_q_heads, w.max_context_len, len(starts) - 1,
                gmax, pmax)
            self.pworkspace = torch.zeros(pneed, dtype=torch.uint8, device=dev)
            self.schedule = {"schedule": "shared-prefix", "partition": 0,
                             "workers": self.schedule.get("workers", 0), "groups": len(starts) - 1}
        # history: every cached token written once through the same write kernel
        if w.hist_seq.size:
            hs = torch.from_numpy(w.hist_seq).to(dev)
            hp = torch.from_numpy(w.hist_pos).to(dev)
            hslots = pkv.paged_kv_slot_mapping(hs, hp, self.block_tables, c.block_size)
            hk, hv = up(w.hist_k, c.src_dtype), up(w.hist_v, c.src_dtype)
            pkv.paged_kv_write(hslots, hk, hv, self.k_cache, self.v_cache, self.kv_dtype,
                               w.k_scale, w.v_scale)
            torch.cuda.synchronize()
            del hk, hv, hs, hp, hslots
        # A sliding window: the engine frees every block holding no attended token; its
        # table entries then name a NaN-filled block the decode must never let in.
        if c.window:
            bt = w.block_tables.copy()
            for s, x in enumerate(w.context_lens):
                used = set((window_tokens(x, c.window, c.sinks) // c.block_size).tolist())
                for j in range((int(x) + c.block_size - 1) // c.block_size):
                    if j not in used:
                        bt[s, j] = w.sentinel_block
            self.block_tables = torch.from_numpy(bt).to(dev)
            self.schedule = dict(self.schedule, window=c.window, sinks=c.sinks)

    def slot_map(self):
        self.pkv.paged_kv_slot_mapping(self.new_seq, self.new_pos, self.block_tables,
                                       self.w.cfg.block_size, slot_mapping=self.slots)

    def write(self):
        w = self.w
        self.pkv.paged_kv_write(self.slots, self.new_k, self.new_v, self.k_cache, self.v_cache,
                                self.kv_dtype, w.k_scale, w.v_scale)

    def decode(self):
        w = self.w
        if self.prefix is not None:
            starts, plens, gmax, pmax = self.prefix
            self.pkv.paged_attention_decode_shared_prefix(
                self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens, w.scale,
                self.out, w.max_context_len, starts, plens, gmax, pmax, workspace=self.pworkspace)
            return
        if w.cfg.window:
            self.pkv.paged_attention_decode_window(
                self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens, w.scale,
                self.out, w.max_context_len, w.cfg.window, w.cfg.sinks, partition_size=self.partition,
                workspace=self.workspace, kv_dtype=self.kv_dtype, k_scale=w.k_scale,
                v_scale=w.v_scale, shared_blocks=self.shared)
            return
        self.pkv.paged_attention_decode(self.q, self.k_cache, self.v_cache, self.block_tables,
                                        self.context_lens, w.scale, self.out, w.max_context_len,
                                        partition_size=self.partition, workspace=self.workspace,
                                        kv_dtype=self.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale,
                                        shared_blocks=self.shared)

    def write_positions(self):
        w = self.w
        self.pkv.paged_kv_write_positions(self.new_seq, self.new_pos, self.block_tables, self.new_k, self.new_v,
                                          self.k_cache, self.v_cache, self.kv_dtype, w.k_scale, w.v_scale)

    def step(self):
        self.write_positions()
        self.decode()


KERNEL_LABEL = {
    "balanced": "paged_attention_decode call (decode_sk_kernel, merges in-kernel)",
    "fixed-partitions": "paged_attention_decode call (decode_kernel + merge_kernel)",
    "single-pass": "paged_attention_decode call (decode_kernel)",
    "shared-prefix": "paged_attention_decode_shared_prefix call (prefix_kernel + decode_sk_kernel suffix pass)",
}


def kernel_label(schedule):
    label = KERNEL_LABEL.get(schedule["schedule"], "?")
    if schedule.get("window"):
        label = label.replace("paged_attention_decode call", "paged_attention_decode_window call")
    return label


def traffic_for(cfg_name):
    """HBM bytes per decode call from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; else None."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    data = json.loads(f.read_text())
    h = hashlib.sha256()
    for src in KERNEL_SOURCES:
        h.update((ROOT / src).read_bytes())
    entry = data.get(cfg_name)
    if not entry or entry.get("kernel_sources_sha256") != h.hexdigest():
        return None
    return entry.get("bytes_per_call")


def decode_tiles(w):
    """The 16-token K/V tiles a decode reads, as indices in units of tile bytes into each
    cache, in the balanced schedule's order (KV head, then sequence, then chunk); only
    attended chunks under a window; a tile shared by several sequences (a shared prefix)
    listed once, where it is first met (the bytes HBM must deliver)."""
    import numpy as np
    c = w.cfg
    B, hkv = c.block_size, c.num_kv_heads
    per_head = []
    for s in range(c.num_seqs):
        ctx = int(w.context_lens[s])
        if ctx == 0:
            continue
        chunks = np.unique(window_tokens(ctx, c.window, c.sinks) // 16)
        blk = w.block_tables[s][(16 * chunks) // B].astype(np.int64)
        per_head.append(blk * B + (16 * chunks) % B)  # rows of head 0, in units of token rows
    rows = np.concatenate(per_head)
    out = []
    for g in range(hkv):
        t = ((rows // B) * hkv + g) * B + rows % B
        _, first = np.unique(t, return_index=True)
        out.append(t[np.sort(first)] // 16)
    return np.concatenate(out).astype(np.int32)


LAYERS = 4  # cache copies decoded in turn by the layered leg


def layered_ms(run, copies, reps):
    """Average duration of run(k_cache, v_cache) launched back to back over copies of a
    layer's cache, taken in turn as a model's layers are decoded: between two uses of a
    copy the others are read, which evicts it from L2/MALL, so every call reads cold data.
    HIP events around the whole sequence (on the current stream), divided by the calls."""
    import torch
    for k, v in copies:  # warm-up pass: code, tables, workspaces
        run(k, v)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        for k, v in copies:
            run(k, v)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(copies))


def read_ceiling(w, st, reps, copies):
    """Achievable read rate of the decode's K/V access pattern: the streaming-read probe
    (libpkv_probe.so, loads as the decode kernel issues them, no arithmetic) over
    decode_tiles(w); single launches after an L2/MALL flush (HIP events on the current
    stream), and the layered form over the same cache copies as the decode."""
    import ctypes
    import numpy as np
    import torch
    from paged_kv_cache_27_amd._binding import LIB_PATH

    lib = ctypes.CDLL(str(Path(LIB_PATH).with_name("libpkv_probe.so")))
    f = lib.pkv_probe_read_tiles
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    c = w.cfg
    tb = 16 * c.head_dim * DT_BYTES[c.kv_dtype]
    tiles = torch.from_numpy(decode_tiles(w)).cuda()
    n = tiles.numel()
    assert int(tiles.max()) < st.k_cache.numel() * st.k_cache.element_size() // tb
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = lambda: f(st.k_cache.data_ptr(), st.v_cache.data_ptr(), tiles.data_ptr(), n, tb, sink.data_ptr(),
                     stream)
    assert call() == 0
    flush = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
    fsink = torch.empty((), dtype=torch.float32, device="cuda")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        fsink.copy_(flush.sum())
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    lay = layered_ms(lambda k, v: f(k.data_ptr(), v.data_ptr(), tiles.data_ptr(), n, tb, sink.data_ptr(), stream),
                     copies, reps)
    return {"kernel": "pkv_probe_read_tiles", "tiles": n, "tile_bytes": tb, "bytes": 2 * n * tb,
            "ms_cold_mean": ms, "ms_layered": lay, "GBps": 2 * n * tb / (lay * 1e-3) / 1e9}


def measure(cfg, args, partition=None, steps=None, warmup=None):
    import numpy as np
    import torch
    from workloads import make_workload

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    t0 = time.time()
    w = make_workload(cfg)
    log(f"[{cfg.name}] inputs generated in {time.time() - t0:.1f}s")
    st = Step(w, partition if partition is not None else args.partition,
              shared_prefix=not args.no_shared_prefix)
    nbytes = algorithmic_bytes(w)
    rbytes = roofline_bytes(nbytes, w)

    for _ in range(warmup):
        st.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        st.step()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    ms_step = (t2 - t1) * 1e3 / steps

    # Cold-cache leg: L2 and MALL flushed before each rep by reading 1 GiB (a read leaves
    # no dirty lines to write back during the timed call); HIP events on the stream the
    # library launches on (torch's current stream, which the binding passes down).
    flush = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.reps)]
    for r in range(args.reps):
        sink.copy_(flush.sum())
        e = ev[r]
        e[0].record()
        st.write_positions()
        e[1].record()
        st.decode()
        e[2].record()
    torch.cuda.synchronize()
    t_write = np.array([e[0].elapsed_time(e[1]) for e in ev])
    t_dec = np.array([e[1].elapsed_time(e[2]) for e in ev])
    del flush
    dec_ms = float(np.mean(t_dec))
    achieved = nbytes["decode"] / (dec_ms * 1e-3) / 1e9
    res = {
        "workload": cfg.name, "ms_per_step": ms_step,
        "step_GBps": nbytes["step"] / (ms_step * 1e-3) / 1e9,
        "seq_heads_per_s": cfg.num_seqs * cfg.num_q_heads / (ms_step * 1e-3),
        "decode_ms_cold_mean": dec_ms, "decode_ms_cold_median": float(np.median(t_dec)),
        "decode_ms_cold_p10": float(np.percentile(t_dec, 10)),
        "decode_ms_cold_p90": float(np.percentile(t_dec, 90)),
        "write_ms_cold_mean": float(np.mean(t_write)),
        "decode_GBps_cold": achieved, "decode_frac_hbm_peak": achieved / HBM_PEAK_GBS,
        "decode_unique_GBps_cold": (nbytes["decode"] - nbytes["kv"] + nbytes["kv_unique"]) / (dec_ms * 1e-3) / 1e9,
        "bytes": nbytes, "roofline_bytes": rbytes, "schedule": st.schedule,
        "max_context_len": w.max_context_len, "sum_context": int(w.context_lens.sum()),
    }
    # layered leg: LAYERS copies of this layer's cache decoded in turn, back to back
    copies = [(st.k_cache, st.v_cache)] + [(st.k_cache.clone(), st.v_cache.clone()) for _ in range(LAYERS - 1)]
    k0, v0 = st.k_cache, st.v_cache

    def run_decode(k, v):
        st.k_cache, st.v_cache = k, v
        st.decode()
    lay_ms = layered_ms(run_decode, copies, max(4, args.reps // LAYERS))
    st.k_cache, st.v_cache = k0, v0
    res["decode_ms_layered"] = lay_ms
    res["decode_GBps_layered"] = nbytes["decode"] / (lay_ms * 1e-3) / 1e9
    res["roofline_GBps_layered"] = rbytes / (lay_ms * 1e-3) / 1e9
    ceil = read_ceiling(w, st, max(4, args.reps // LAYERS), copies)
    del copies
    torch.cuda.empty_cache()
    # the same tiles read by the probe alone vs by the decode (which also reads q and the
    # tables and computes), both layered: the decode's fraction of the pattern's rate
    ceil["decode_frac"] = ceil["ms_layered"] / lay_ms
    res["read_ceiling"] = ceil
    log(f"[{cfg.name}] step {ms_step * 1e3:.1f} us ({res['step_GBps']:.0f} GB/s), decode cold "
        f"{dec_ms * 1e3:.1f} us ({achieved:.0f} GB/s), "
        f"write {res['write_ms_cold_mean'] * 1e3:.1f} us, schedule {res['schedule']}; layered decode "
        f"{lay_ms * 1e3:.1f} us ({res['decode_GBps_layered']:.0f} GB/s; roofline "
        f"{100 * res['roofline_GBps_layered'] / HBM_PEAK_GBS:.1f}% of peak); read ceiling of its tiles "
        f"{ceil['GBps']:.0f} GB/s ({ceil['ms_layered'] * 1e3:.1f} us layered), decode at "
        f"{100 * ceil['decode_frac']:.1f}% of it")
    return w, st, res


def measure_block_moves(args):
    """Copy-on-write copies and swap-outs of whole blocks on the 8B-shaped layer's cache:
    algorithmic bytes = blocks x block bytes x (K, V) x (read + write), cold L2/MALL."""
    import numpy as np
    import torch
    import paged_kv_cache_27_amd as pkv
    from workloads import LLAMA8B, cache_shape, make_workload

    w = make_workload(LLAMA8B)
    shape = cache_shape(w)
    k = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    block_bytes = k[0].numel() * 2
    rng = np.random.default_rng(0)
    perm = rng.permutation(w.num_blocks).astype(np.int32)
    n = min(2048, w.num_blocks // 2)
    src = torch.from_numpy(perm[:n].copy()).cuda()
    dst = torch.from_numpy(perm[n:2 * n].copy()).cuda()
    kb = torch.empty((n,) + tuple(shape[1:]), dtype=torch.bfloat16, device="cuda")
    vb = torch.empty_like(kb)
    # pinned host buffers: the swap kernel itself moves the blocks across the host link
    kh = torch.empty((n,) + tuple(shape[1:]), dtype=torch.bfloat16, pin_memory=True)
    vh = torch.empty((n,) + tuple(shape[1:]), dtype=torch.bfloat16, pin_memory=True)
    flush = torch.ones(256 << 20, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    # the practical ceiling of a move: one contiguous device copy of the same bytes (2n
    # whole blocks), no block lookup
    csrc = k[:2 * n]
    cdst = torch.empty_like(csrc)
    out = {}
    for name, call in (("copy_blocks", lambda: pkv.paged_kv_copy_blocks(src, dst, k, v)),
                       ("swap_out_to_device", lambda: pkv.paged_kv_swap_out(src, k, v, kb, vb)),
                       ("contiguous_device_copy", lambda: cdst.copy_(csrc)),
                       ("swap_out_to_pinned_host", lambda: pkv.paged_kv_swap_out(src, k, v, kh, vh)),
                       ("swap_in_from_pinned_host", lambda: pkv.paged_kv_swap_in(dst, kh, vh, k, v))):
        for _ in range(3):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.reps)]
        for e0, e1 in ev:
            sink.copy_(flush.sum())
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        if "host" in name:  # one direction across the host link: K and V blocks
            nbytes = n * block_bytes * 2
            out[name] = {"blocks": n, "block_bytes": block_bytes, "bytes_over_link": nbytes, "ms_cold_mean": ms,
                         "GBps_link": nbytes / (ms * 1e-3) / 1e9}
            log(f"[block moves] {name}: {n} blocks of {block_bytes} B (K and V), {ms * 1e3:.1f} us, "
                f"{out[name]['GBps_link']:.1f} GB/s across the host link")
            continue
        nbytes = n * block_bytes * 2 * 2
        out[name] = {"blocks": n, "block_bytes": block_bytes, "bytes": nbytes, "ms_cold_mean": ms,
                     "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        log(f"[block moves] {name}: {n} blocks of {block_bytes} B (K and V), {ms * 1e3:.1f} us, "
            f"{out[name]['GBps']:.0f} GB/s read+write ({100 * out[name]['frac_hbm_peak']:.1f}% of peak)")
    for name in ("copy_blocks", "swap_out_to_device"):
        out[name]["frac_of_contiguous_copy"] = out[name]["GBps"] / out["contiguous_device_copy"]["GBps"]
    return out


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def measure_prefill(args, kv="bf16"):
    """Chunked prefill: 8 sequences, each a 512-token chunk ending a 4096-token context
    (Llama-3-8B-shaped heads, bf16 queries; a bf16 or an fp8 e4m3fn cache).  Algorithmic
    flops: per query head and attended (query, token) pair, 2 d for q.k and 2 d for p v;
    MFMA-bound (the fp8 tiles are converted to bf16 for bf16 MFMAs)."""
    import numpy as np
    import torch
    import paged_kv_cache_27_amd as pkv
    from workloads import LLAMA8B, POISON_BITS, cache_shape, make_workload, prefill_queries

    name = "prefill-8x512-at-4096-bf16" if kv == "bf16" else "prefill-8x512-at-4096-fp8kv"
    cfg = LLAMA8B.replace(name=name, num_seqs=8, ctx_kind="fixed", ctx_params=(4096,) * 8, kv_dtype=kv)
    w = make_workload(cfg)
    c = cfg
    n = np.full(c.num_seqs, 512, np.int32)
    q_np, cu_np = prefill_queries(w, n)
    dev = "cuda"
    store = torch.int16 if kv == "bf16" else torch.uint8
    k = torch.full(cache_shape(w), POISON_BITS[kv], dtype=store, device=dev)
    v = torch.full(cache_shape(w), POISON_BITS[kv], dtype=store, device=dev)
    if kv == "bf16":
        k, v = k.view(torch.bfloat16), v.view(torch.bfloat16)
    kvd = None if kv == "bf16" else "fp8"
    bt = torch.from_numpy(w.block_tables).to(dev)
    ctx = torch.from_numpy(w.context_lens).to(dev)
    up = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    hs = torch.from_numpy(w.hist_seq).to(dev)
    hp = torch.from_numpy(w.hist_pos).to(dev)
    slots = pkv.paged_kv_slot_mapping(hs, hp, bt, c.block_size)
    pkv.paged_kv_write(slots, up(w.hist_k), up(w.hist_v), k, v, kvd, w.k_scale, w.v_scale)
    ns = pkv.paged_kv_slot_mapping(torch.from_numpy(w.new_seq).to(dev), torch.from_numpy(w.new_pos).to(dev), bt,
                                   c.block_size)
    pkv.paged_kv_write(ns, up(w.new_k), up(w.new_v), k, v, kvd, w.k_scale, w.v_scale)
    q = up(q_np)
    cu = torch.from_numpy(cu_np).to(dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    call = lambda: pkv.paged_attention_prefill(q, cu, 512, k, v, bt, ctx, w.scale, out, w.max_context_len,
                                               kv_dtype=kvd, k_scale=w.k_scale, v_scale=w.v_scale)
    for _ in range(3):
        call()
    flush = torch.ones(256 << 20, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.reps)]
    for e0, e1 in ev:
        sink.copy_(flush.sum())
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    pairs = sum(int(x) - 512 + i + 1 for x in w.context_lens for i in range(512))
    flops = pairs * c.num_q_heads * c.head_dim * 4
    tflops = flops / (ms * 1e-3) / 1e12
    res = {"workload": cfg.name, "flops": flops, "ms_cold_mean": ms, "TFLOPs": tflops,
           "frac_mfma_bf16_peak": tflops / MFMA_BF16_PEAK_TFLOPS}
    log(f"[{cfg.name}] {ms * 1e3:.1f} us, {tflops:.1f} TFLOP/s ({100 * tflops / MFMA_BF16_PEAK_TFLOPS:.1f}% of "
        f"the bf16 MFMA peak), {flops / 1e9:.1f} GFLOP")
    return res


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        for ln in Path("/proc/cpuinfo").read_text().splitlines():
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# Oracle threads: the host CPUs this process may run on, at most 16, the CPU share one GPU
# of a shared MI355X host gets (its affinity mask can list more CPUs than the share).
CPU_SHARE = 16


def cpu_baseline(w, budget_s):
    """The fp64 oracle on this host's cores (its affinity, at most CPU_SHARE threads) over
    whole sequences (all query heads), taken in order until the wall budget is spent; then
    the same on one thread for a third of the budget (`single_thread`)."""
    import numpy as np
    from oracle.oracle import Oracle
    from workloads import poisoned_cache

    orc = Oracle()
    c = w.cfg
    kc, vc = poisoned_cache(w), poisoned_cache(w)
    hs = orc.slot_mapping(w.hist_seq, w.hist_pos, w.block_tables, c.block_size)
    orc.kv_write(hs, w.hist_k, w.hist_v, c.src_dtype, kc, vc, c.kv_dtype, w.k_scale, w.v_scale)
    ns = orc.slot_mapping(w.new_seq, w.new_pos, w.block_tables, c.block_size)
    orc.kv_write(ns, w.new_k, w.new_v, c.src_dtype, kc, vc, c.kv_dtype, w.k_scale, w.v_scale)
    affinity = len(os.sched_getaffinity(0))
    threads = min(CPU_SHARE, affinity)
    res = _oracle_rate(orc, w, kc, vc, threads, budget_s)
    one = _oracle_rate(orc, w, kc, vc, 1, budget_s / 3)
    res["single_thread"] = {"value": one["value"], "unit": "GB/s", "cores": 1, "sample": one["sample"]}
    res["affinity_cpus"] = affinity
    res["cpu_model"] = cpu_model()
    res["threads_note"] = f"threads = min(affinity {affinity}, the {CPU_SHARE}-CPU share of one GPU)"
    return res


def _oracle_rate(orc, w, kc, vc, threads, budget_s):
    """Whole passes of the oracle's decode over the workload (all sequences, all query
    heads) on `threads` threads until the budget is spent; the last pass may stop early
    at a sequence boundary."""
    import numpy as np
    c = w.cfg
    passes, elapsed, tokens, seq_heads = 0, 0.0, 0, 0
    per = max(1, threads // 2)
    while elapsed < budget_s:
        s0 = 0
        while s0 < c.num_seqs and elapsed < budget_s:
            seqs = range(s0, min(c.num_seqs, s0 + per))
            pairs = np.array([(s, h) for s in seqs for h in range(c.num_q_heads)], np.int32)
            t0 = time.perf_counter()
            orc.decode(w.q, c.q_dtype, kc, vc, c.kv_dtype, w.block_tables, w.context_lens,
                       w.scale, w.k_scale, w.v_scale, pairs=pairs, threads=threads,
                       window=c.window, sinks=c.sinks)
            elapsed += time.perf_counter() - t0
            tokens += sum(len(window_tokens(w.context_lens[s], c.window, c.sinks)) for s in seqs)
            seq_heads += len(seqs) * c.num_q_heads
            s0 = seqs[-1] + 1
        passes += s0 / c.num_seqs
    kv_bytes = tokens * c.num_kv_heads * c.head_dim * 2 * DT_BYTES[c.kv_dtype]
    return {"value": kv_bytes / elapsed / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "seq_heads_per_s": seq_heads / elapsed,
            "sample": f"{passes:.2f} passes of the decode over all {c.num_seqs} sequences x "
                      f"{c.num_q_heads} query heads ({tokens} context tokens in total), fp64, "
                      f"{elapsed:.1f}s wall on {threads} threads"}


def config_entry(res, cpu):
    """One workload's entry of the `configs` array: the decode call against the HBM
    roofline (layered mean), its single-launch percentiles, HBM traffic, read ceiling and
    the oracle's rate on this host."""
    r = lambda x, n=2: None if x is None else round(x, n)
    rb, logical = res["roofline_bytes"], res["bytes"]["decode"]
    ceil = res["read_ceiling"]
    e = {"workload": res["workload"], "schedule": res["schedule"],
         "kernel": kernel_label(res["schedule"]),
         "decode_us_layered": r(res["decode_ms_layered"] * 1e3),
         "bytes_per_launch": rb,
         "bytes_basis": "unique (each shared block once)" if rb != logical else "algorithmic",
         "GBps": r(res["roofline_GBps_layered"], 1),
         "frac_hbm_peak": r(res["roofline_GBps_layered"] / HBM_PEAK_GBS, 4),
         "decode_us_single_launch": {"mean": r(res["decode_ms_cold_mean"] * 1e3),
                                     "p10": r(res["decode_ms_cold_p10"] * 1e3),
                                     "median": r(res["decode_ms_cold_median"] * 1e3),
                                     "p90": r(res["decode_ms_cold_p90"] * 1e3)},
         "traffic": traffic_for(res["workload"]),
         "read_ceiling": {"us_layered": r(ceil["ms_layered"] * 1e3), "GBps": r(ceil["GBps"], 1),
                          "decode_frac": r(ceil["decode_frac"], 4)},
         "step_us": r(res["ms_per_step"] * 1e3), "write_us_single_launch": r(res["write_ms_cold_mean"] * 1e3),
         "seq_heads_per_s": r(res["seq_heads_per_s"], 1),
         "cpu_baseline": None if cpu is None else {
             "value": r(cpu["value"], 4), "unit": cpu["unit"], "cores": cpu["cores"], "kind": cpu["kind"],
             "single_thread_value": r(cpu["single_thread"]["value"], 4), "affinity_cpus": cpu["affinity_cpus"],
             "cpu_model": cpu["cpu_model"], "sample": cpu["sample"]}}
    if rb != logical:  # prefix sharing: the logical bytes (every sequence's whole context) too
        e["logical_bytes"] = logical
        e["GBps_logical"] = r(res["decode_GBps_layered"], 1)
        e["frac_logical"] = r(res["decode_GBps_layered"] / HBM_PEAK_GBS, 4)
    if res["bytes"]["decode"] < 1 << 20:
        e["note"] = "parity-only size: its whole budget at 6 TB/s is far below a launch's latency"
    return e


def gpu_clocks():
    """Current clocks as rocm-smi reports them (a child process, started before this
    process touches the GPU), or None."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
    except Exception:  # tool missing or stuck: the record just goes without clocks
        return None
    lines = [(ln.split(":", 1)[1] if ln.lstrip().startswith("GPU[") else ln).strip()
             for ln in r.stdout.splitlines() if any(x in ln for x in ("sclk", "mclk", "fclk"))]
    return "; ".join(lines[:6]) or None


def main():
    args = parse_args()
    args.reps = max(1, args.reps)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): this path has "
              "no multi-GPU leg (a decode step shards by KV head or by sequence, with no collective "
              "inside the step)", file=sys.stderr)
        sys.exit(2)
    clocks = gpu_clocks() if not (args.copy_calibration or args.prefill_only or args.blocks_only) else None
    import torch
    import paged_kv_cache_27_amd as pkv

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    pkv.load_library()  # raises if the HIP library is missing: there is no fallback
    props = torch.cuda.get_device_properties(0)
    env = {"gpu": props.name, "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
           "clocks": clocks, "torch": torch.__version__, "hip": torch.version.hip}
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.steps} x {src.numel() * 4} bytes")
        return
    if args.prefill_only:
        print(json.dumps(measure_prefill(args)))
        return
    if args.blocks_only:
        print(json.dumps(measure_block_moves(args)))
        return
    from workloads import CONFIGS, EXTRA_CONFIGS
    cfg = pick_config(args.config)
    w, st, res = measure(cfg, args)
    del st
    torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)
        log(f"[cpu oracle] {cpu['value']:.3f} GB/s on {cpu['cores']} threads: {cpu['sample']}; "
            f"{cpu['single_thread']['value']:.3f} GB/s on one thread")
    del w
    # every decode-layer workload, measured the same way (the headline's entry is its own
    # measurement); fewer steps, a smaller oracle budget
    configs = []
    if not args.only:
        for c2 in CONFIGS:
            if c2.name == cfg.name:
                configs.append(config_entry(res, cpu))
                continue
            w2, s2, r2 = measure(c2, args, steps=min(args.steps, 20), warmup=min(args.warmup, 5))
            del s2
            torch.cuda.empty_cache()
            cpu2 = None
            if not args.no_cpu_baseline:
                cpu2 = cpu_baseline(w2, args.config_cpu_seconds)
                log(f"[cpu oracle, {c2.name}] {cpu2['value']:.3f} GB/s on {cpu2['cores']} threads")
            del w2
            configs.append(config_entry(r2, cpu2))
    others = []
    if args.all:
        for c in EXTRA_CONFIGS:
            _, s2, r2 = measure(c, args)
            others.append(r2)
            del s2
            torch.cuda.empty_cache()
    blocks = measure_block_moves(args) if args.all else None
    prefill = measure_prefill(args) if args.all else None
    prefill_fp8 = measure_prefill(args, "fp8") if args.all else None
    traffic = traffic_for(cfg.name)
    c = cfg
    line = {
        "metric": METRIC, "value": round(res["step_GBps"], 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": c.kv_dtype, "data": "synthetic",
        "config": {"workload": c.name, "num_seqs": c.num_seqs, "num_q_heads": c.num_q_heads,
                   "num_kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
                   "block_size": c.block_size, "q_dtype": c.q_dtype, "kv_dtype": c.kv_dtype,
                   "context_lens": f"{c.ctx_kind}{tuple(c.ctx_params)}",
                   "sum_context": res["sum_context"], "schedule": res["schedule"],
                   "seed": c.seed, **({"window": c.window, "sinks": c.sinks} if c.window else {})},
        "pct_hbm_peak": round(100 * res["step_GBps"] / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(res["seq_heads_per_s"], 1),
        # achieved: the decode call's average duration over back-to-back calls on cold
        # per-layer cache copies (the layered leg); the single-launch figure beside it
        "roofline": {"bound": "hbm", "achieved": round(res["roofline_GBps_layered"], 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(res["roofline_GBps_layered"] / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": kernel_label(res["schedule"]),
                     "bytes_per_launch": res["roofline_bytes"],
                     "mean_launch_ms": round(res["decode_ms_layered"], 6),
                     "timing": f"mean over back-to-back calls on {LAYERS} cold per-layer cache copies",
                     "single_launch_ms": round(res["decode_ms_cold_mean"], 6),
                     "single_launch_GBps": round(res["decode_GBps_cold"], 2)},
        "cpu_baseline": cpu,
        "read_ceiling": {k: (round(v, 4) if isinstance(v, float) else v)
                         for k, v in res["read_ceiling"].items()},
        "configs": configs,
        "env": env,
    }
    if args.json_out:
        Path(args.json_out).parent.mkdir(parents=True, exist_ok=True)
        Path(args.json_out).write_text(json.dumps({"headline": res, "configs": configs, "others": others,
                                                   "block_moves": blocks,
                                                   "prefill": prefill, "prefill_fp8kv": prefill_fp8,
                                                   "cpu": cpu}, indent=1))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
