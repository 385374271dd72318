"""Decode-step benchmark of the paged KV-cache hot path on one MI355X.

One step = one decode iteration of a batch, all inside one call of libpkv's native step
driver (pkv_stepper_step):
  1. host block manager: append one slot per sequence (new block on a block boundary,
     copy-on-write pairs for shared blocks), export the block tables and lengths;
  2. one packed copy of tables / lengths / slots / pairs to the device (pinned,
     double-buffered, asynchronous);
  3. copy_blocks for any copy-on-write pairs;
  4. reshape_and_cache: write each sequence's new K/V token into its slot;
  5. paged_attention_decode over every sequence's context (new token included).

Default workload: a LLaMA-13B-shaped layer in fp16 -- 64 sequences, 40 heads, head_dim 128,
16-token blocks, context lengths uniform in [128, 2048], physical blocks from a seeded random
permutation of a pool 1.2x the need.  Sequences grow by one token per step; a sequence that has
grown by 64 tokens finishes and a new one of its starting length takes its place (so the
batch stays the same size and shape however many steps run).

Printed: one JSON line.  ``value`` is logical KV bytes read by decode attention per second of
whole-step time (inputs resident in HBM); ``roofline`` is for the decode attention launch,
timed with events on the stream it runs on; ``cpu_baseline`` times the float64 oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode-attn KV GB/s (frac of HBM peak) and seq·layer/s, LLaMA-13B shape"
HBM_PEAK_GBS = 8000.0
# rocprofv3 counter summaries (see each one's header for the commands); a traffic figure is
# used only while the kernel sources it was taken on are unchanged.
CSRC = os.path.join(ROOT, "paged_kv_cache_306_amd", "csrc")
COUNTER_PROFILE = os.path.join(ROOT, "profiles", "decode_llama13b_layer_fp16_counters.md")
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("pkv_decode.hip", "pkv_device.h", "pkv_xcd.h")]
MQ_COUNTER_PROFILE = os.path.join(ROOT, "profiles", "multi_query_prefix_hit_fp16_counters.md")
MQ_KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("pkv_multi_query.hip", "pkv_device.h")]


def kernel_source_hash(sources=None) -> str:
    """SHA-256 of the kernel sources' code: comments and whitespace are dropped first, so a
    change to the comments alone leaves a counter profile valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(profile=COUNTER_PROFILE, sources=None):
    """Scaled HBM bytes per launch from a committed counter profile, with the counter scale
    factors and what they were calibrated on, or None when there is no profile or it was
    taken on different kernel sources."""
    try:
        with open(profile) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    fields = {}
    for ln in lines:
        if ln.startswith("- ") and ": " in ln:
            k, v = ln[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    try:
        out = {"bytes": int(fields["traffic_bytes_per_launch"])}
    except (KeyError, ValueError):
        return None
    for k in ("fetch_scale", "write_scale"):
        if k in fields:
            out[k] = float(fields[k])
    if "calibration" in fields:
        out["calibration"] = fields["calibration"]
    return out


GROWTH = 64   # tokens a sequence grows before it is replaced


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--placement", choices=["permuted", "contiguous"], default="permuted")
    ap.add_argument("--workload", choices=WORKLOADS, default="llama13b_layer")
    ap.add_argument("--block-size", type=int, default=16, choices=(8, 16, 32),
                    help="block size of the llama13b_layer / long_context workloads")
    ap.add_argument("--swap", action="store_true",
                    help="swap-out / swap-in bandwidth between HBM and a pinned host pool for "
                         "block sizes 8, 16, 32: one JSON line per configuration")
    ap.add_argument("--prefix-cache", action="store_true",
                    help="host-only: KV blocks saved by the prefix cache on a chat workload")
    ap.add_argument("--sweep", action="store_true",
                    help="block size x placement sweep of the llama13b_layer and long_context "
                         "workloads, 3 interleaved rounds: one JSON line per configuration")
    ap.add_argument("--user-turns", default="16,512", metavar="LO,HI",
                    help="prefix_hit: new tokens per request, uniform in [LO, HI]")
    ap.add_argument("--mq-schedule", choices=("packed", "grouped"), default="packed",
                    help="prefix_hit: full tiles packed across the requests that share a "
                         "prompt's blocks, or one tile list per request grouped by prompt")
    ap.add_argument("--dtype", choices=("f16", "bf16"), default="f16",
                    help="storage type of the prefix_hit workload")
    ap.add_argument("--flush-mall", action="store_true",
                    help="decode workloads: read a 1 GiB buffer before every timed step (outside "
                         "the decode launch's events) so the 256 MB MALL holds none of the "
                         "previous step's K/V; the step time then includes that read")
    ap.add_argument("--event-every", type=int, default=10, metavar="K",
                    help="decode workloads: the attention launches of every K-th step carry the "
                         "HIP timing events that roofline.avg_launch_us averages (the events "
                         "lengthen a step by ~4 us, so the other steps run without them)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=2560,
                    help="most (sequence, head) units the oracle baseline computes")
    ap.add_argument("--cpu-bytes", type=float, default=1.6e9,
                    help="most K+V bytes the oracle baseline reads (about 10 s of CPU work)")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the achievable HBM read rate (libpkv_probe.so): a "
                         "contiguous stream and whole 2/4/8 KiB tiles in random order")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only measure the sustained 16x16x32 fp16 matrix-core rate "
                         "(libpkv_probe.so): products alone, each fed by a 1 KiB LDS read per "
                         "wave as the multi-query kernel's K/V fragments are, and each followed "
                         "by independent vector instructions")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (to scale HBM counters)")
    ap.add_argument("--calibrate-read", type=int, default=0, metavar="MIB",
                    help="only run 5 plain nontemporal reads of MIB MiB with the probe library "
                         "(to scale the FETCH_SIZE counter)")
    return ap.parse_args()


@contextlib.contextmanager
def gc_paused():
    """Python's cyclic garbage collector off while steps are timed, as timeit does: a full
    collection walks every object torch has created and takes tens of milliseconds, which
    would otherwise land inside one timed step."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def hip_runtime():
    """The HIP runtime this process already uses (torch's), found among the loaded objects, so
    that events created here are valid in torch's and libpkv's calls."""
    import ctypes
    import torch
    torch.cuda.init()
    with open("/proc/self/maps") as f:
        paths = sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln})
    if not paths:
        raise RuntimeError("no HIP runtime loaded")
    hip = ctypes.CDLL(paths[0])
    hip.hipEventCreateWithFlags.argtypes = [ctypes.c_void_p, ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return hip


# hipEventDisableSystemFence: the event's completion does not write back and invalidate the
# caches for the host's sake -- timing needs none of that, and the flush would otherwise sit
# between the timed kernel and the next one.
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class TimingEvents:
    """steps x pairs of HIP timing events (start, stop) for the step driver's attention
    launches, which record them themselves (their own start and end).  ``fence`` False creates
    them with hipEventDisableSystemFence."""

    def __init__(self, steps: int, pairs: int, fence: bool = False):
        import ctypes
        self.hip = hip_runtime()
        flags = 0 if fence else HIP_EVENT_DISABLE_SYSTEM_FENCE
        self.handles = []
        for _ in range(steps):
            arr = (ctypes.c_void_p * (2 * pairs))()
            for e in range(2 * pairs):
                ev = ctypes.c_void_p()
                if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), flags) != 0:
                    raise RuntimeError("hipEventCreateWithFlags failed")
                arr[e] = ev.value
            self.handles.append(arr)
        self.pairs = pairs
        # record every event once so that a pair is never read before it was taken
        import torch
        stream = torch.cuda.current_stream().cuda_stream
        for arr in self.handles:
            for e in range(2 * pairs):
                self.hip.hipEventRecord(ctypes.c_void_p(arr[e]), ctypes.c_void_p(stream))

    def elapsed_ms(self):
        """Every pair's duration in ms (after the work has finished), step-major."""
        import ctypes
        out = []
        ms = ctypes.c_float()
        for arr in self.handles:
            for l in range(self.pairs):
                if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(arr[2 * l]),
                                                ctypes.c_void_p(arr[2 * l + 1])) != 0:
                    raise RuntimeError("hipEventElapsedTime failed")
                out.append(ms.value)
        return out

    def destroy(self):
        import ctypes
        for arr in self.handles:
            for e in range(2 * self.pairs):
                self.hip.hipEventDestroy(ctypes.c_void_p(arr[e]))
        self.handles = []


def calibrate_read(mib: int):
    """Five plain nontemporal reads of a device buffer of MIB MiB by the probe library (the
    decode kernel's load form, each byte once): FETCH_SIZE of this run over the bytes read
    gives the counter's scale factor for reads."""
    import torch
    probe = load_probe()
    if probe is None:
        raise RuntimeError("libpkv_probe.so is not built")
    n = mib << 20
    buf = torch.ones(n // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(5):
        if probe(buf.data_ptr(), n, 0, None, 0, 1, 0, sink.data_ptr(), 4096, stream) != 0:
            raise RuntimeError("pkv_probe_read failed")
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_read_bytes": n, "reads": 5}), flush=True)


def calibrate_copy(mib: int):
    """Five plain device-to-device copies of a known size: FETCH_SIZE / WRITE_SIZE of this
    run divided by the bytes moved gives the scale factor for the counters."""
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)


def decode_tile_list(workload, seed):
    """The 4 KiB (block, head) tiles one decode layer of `workload` reads (start lengths + the
    appended token, seeded placement), as indices into a buffer holding the K pool and then
    the V pool: sequences longest first, then logical block, then head, K before V.
    Returns (tile indices, tiles in the buffer, tile bytes, spec)."""
    import paged_kv_cache_306_amd as pkv
    sp = workload_spec(workload, seed, 16, "permuted")
    H, NB = sp["H"], sp["NB"]
    tile = sp["BS"] * sp["D"] * 2
    alloc = pkv.BlockAllocator(NB, sp["BS"], free_order=sp["order"])
    lens = sp["lens"] + 1
    for s, L in enumerate(lens.tolist()):
        alloc.add_seq(s, int(L))
    heads = np.arange(H, dtype=np.int64)
    parts = []
    for s in np.argsort(-lens, kind="stable").tolist():
        blk = np.asarray(alloc.block_table(s), np.int64)
        k_tiles = (blk[:, None] * H + heads[None, :]).reshape(-1)
        parts.append(np.stack([k_tiles, NB * H + k_tiles], axis=1).reshape(-1))
    return np.concatenate(parts), 2 * NB * H, tile, sp


def decode_tiles_ceiling(probe, workload, seed, wgs, sink, stream, split=0):
    """Plain nontemporal read of exactly the K/V tiles one decode layer of `workload` reads;
    with `split` (of 1024) the even XCDs read that share of them, as the decode deals its
    units."""
    import torch
    idx, n_buf_tiles, tile, _ = decode_tile_list(workload, seed)
    nbytes = n_buf_tiles * tile
    assert tile == 4096 and idx.max() < n_buf_tiles
    dev = torch.device("cuda:0")
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    order = torch.from_numpy(idx.astype(np.int32)).to(dev)
    read = len(idx) * tile

    def launch():
        st = probe(buf.data_ptr(), nbytes, tile, order.data_ptr(), len(idx), 1, split,
                   sink.data_ptr(), wgs, stream)
        if st != 0:
            raise RuntimeError(f"pkv_probe_read returned {st}")
    for _ in range(3):
        launch()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(20)]
    for a, z in evs:
        a.record()
        launch()
        z.record()
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(z) for a, z in evs])) / 1e3
    return {"pattern": f"decode_tiles_{workload}", "tile_bytes": tile, "nontemporal": True,
            "xcd_split": split,
            "bytes": int(read), "us": round(t * 1e6, 1), "GB/s": round(read / t / 1e9, 1),
            "frac_of_peak": round(read / t / 1e9 / HBM_PEAK_GBS, 4)}


def load_probe():
    """pkv_probe_read from the in-tree probe library (include/pkv_probe.h), or None if it is
    not built."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_306_amd",
                        "libpkv_probe.so")
    if not os.path.exists(path):
        return None
    probe = ctypes.CDLL(path).pkv_probe_read
    probe.restype = ctypes.c_int32
    probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                      ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                      ctypes.c_int32, ctypes.c_void_p]
    return probe


def load_probe_lib():
    """The in-tree probe library (include/pkv_probe.h) with the matrix-core probe's signature
    set, or None if it is not built."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_306_amd",
                        "libpkv_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.pkv_probe_mfma.restype = ctypes.c_int32
    lib.pkv_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p, ctypes.c_void_p]
    return lib


def mfma_ceiling(args):
    """Sustained 16x16x32 fp16 matrix-core rate on all CUs (16 waves per CU, eight independent
    accumulators per wave): products alone; each product's A operand read from LDS (1 KiB per
    wave and product, the multi-query kernel's ratio of K/V fragment bytes to products); and
    each product followed by 2, 4 or 8 independent v_fma_f32 or by 1 or 2 (v_mul_f32, v_exp_f32)
    pairs, which shows how much vector work the SIMD overlaps with its products.  HIP events, median of 5
    launches after one warm-up."""
    import torch
    lib = load_probe_lib()
    if lib is None:
        raise RuntimeError("libpkv_probe.so is not built (run __graft_entry__.build())")
    wgs, iters = 256 * 4, 20000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    flops = wgs * 4 * iters * 8 * 2.0 * 16 * 16 * 32
    names = ["mfma_f16_16x16x32", "mfma_f16_16x16x32+lds_1KiB", "mfma+2_fma", "mfma+4_fma",
             "mfma+8_fma", "mfma+1_mul_exp", "mfma+2_mul_exp"]
    for mode, name in enumerate(names):
        def launch():
            if lib.pkv_probe_mfma(mode, iters, wgs, out.data_ptr(), stream) != 0:
                raise RuntimeError("pkv_probe_mfma failed")
        launch()
        ts = []
        for _ in range(5):
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            launch()
            z.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(z) / 1e3)
        t = float(np.median(ts))
        tf = flops / t / 1e12
        print(json.dumps({"pattern": name, "us": round(t * 1e6, 1), "TFLOP/s": round(tf, 1),
                          "frac_of_peak": round(tf / MFMA_PEAK_TFLOPS["f16"], 4)}), flush=True)


def own_tiles_read_rate(workload, seed, split=0):
    """GB/s of a plain nontemporal read of exactly the K/V tiles one decode launch of
    `workload` reads, in one launch of that size (the decode launch's practical ceiling): with
    the tiles dealt evenly to the XCDs, and with the decode's `split` when it has one.  Returns
    (even, with the split or None), or None when the probe library is missing."""
    import torch
    probe = load_probe()
    if probe is None:
        return None
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    even = decode_tiles_ceiling(probe, workload, seed, 4096, sink, stream)["GB/s"]
    weighted = (decode_tiles_ceiling(probe, workload, seed, 4096, sink, stream, split)["GB/s"]
                if split > 0 else None)
    torch.cuda.empty_cache()
    return even, weighted


def ceiling_bench(args):
    """Achievable HBM read rate on this GPU for the decode kernel's access patterns: one
    contiguous stream, and whole tiles visited in a seeded random order (a paged gather reads
    whole (block, head) tiles: 2, 4 and 8 KiB at fp16, head_dim 128, block size 8, 16, 32),
    plus the same 4 KiB tiles in address order (4 GiB buffer), and exactly the tiles one decode
    launch of the LLaMA-13B-shaped layer, of the 40-layer step and of the long-context batch
    reads.  HIP events, median of 20."""
    import torch
    probe = load_probe()
    if probe is None:
        raise RuntimeError("libpkv_probe.so is not built (run __graft_entry__.build())")
    dev = torch.device("cuda:0")
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    g = np.random.default_rng(args.seed)
    wgs = 4096
    cases = [("stream", 0, 1), ("stream", 0, 0)]
    cases += [("tiles_random", tb, 1) for tb in (2048, 4096, 8192)]
    cases += [("tiles_random", 4096, 0), ("tiles_in_order", 4096, 1)]
    rows = []
    for pattern, tb, nt in cases:
        order = None
        n_tiles = nbytes // tb if tb else 0
        if tb:
            idx = np.arange(n_tiles) if pattern == "tiles_in_order" else g.permutation(n_tiles)
            order = torch.from_numpy(idx.astype(np.int32)).to(dev)

        def launch():
            st = probe(buf.data_ptr(), nbytes, tb, order.data_ptr() if order is not None else None,
                       n_tiles, nt, 0, sink.data_ptr(), wgs, stream)
            if st != 0:
                raise RuntimeError(f"pkv_probe_read returned {st}")
        for _ in range(3):
            launch()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(20)]
        for a, z in evs:
            a.record()
            launch()
            z.record()
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(z) for a, z in evs])) / 1e3
        rows.append({"pattern": pattern, "tile_bytes": tb, "nontemporal": bool(nt),
                     "us": round(t * 1e6, 1), "GB/s": round(nbytes / t / 1e9, 1),
                     "frac_of_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)})
        print(json.dumps(rows[-1]), flush=True)

    # The decode launch's own bytes: every K and V (block, head) tile that one decode layer of
    # the LLaMA-13B-shaped layer, of the 40-layer step and of the long-context batch reads
    # (start lengths + the appended token), at their seeded physical places, in one launch of
    # that size -- sequences longest first, then logical block, then head, K before V.  Each
    # workload's two pools sit back to back in a buffer of their own.
    del buf
    for wl in ("llama13b_layer", "full_step_40", "long_context"):
        rows.append(decode_tiles_ceiling(probe, wl, args.seed, wgs, sink, stream))
        print(json.dumps(rows[-1]), flush=True)
    print(json.dumps({"ceiling_bytes_per_launch": nbytes, "workgroups": wgs,
                      "peak_GB/s": HBM_PEAK_GBS, "cases": len(rows)}), flush=True)


WORKLOADS = ("llama13b_layer", "long_context", "shared_prefix", "fork_step", "full_step_40",
             "prefix_hit")
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}   # MI355X dense fp16 / bf16 matrix peak


def workload_spec(name: str, seed: int, block_size: int, placement: str):
    """Shapes, start lengths, pool and block-manager set-up of one benchmark workload."""
    import workloads as W
    if name == "llama13b_layer":
        w = W.llama13b_layer(seed)
        need = sum(W.nblocks_for(int(L), block_size) for L in w.lens)
        spec = dict(S=w.S, H=w.H, D=w.D, BS=block_size, dtype=w.dtype, scale=w.scale, layers=1,
                    lens=w.lens.astype(np.int64), NB=int(math.ceil(1.2 * need)), growth=64,
                    groups=0, desc=f"64 seqs, 40 heads, head_dim 128, BS {block_size}, lengths "
                                   "U[128,2048], fp16")
    elif name == "long_context":
        w = W.long_context(seed=4, block_size=block_size)
        spec = dict(S=w.S, H=w.H, D=w.D, BS=w.BS, dtype=w.dtype, scale=w.scale, layers=1,
                    lens=w.lens.astype(np.int64), NB=w.num_blocks, growth=64, groups=0,
                    desc=f"8 seqs, 40 heads, head_dim 128, BS {block_size}, lengths "
                         "U[16384,32768], bf16")
    elif name == "shared_prefix":
        w = W.shared_prefix(seed=3)
        # the block manager holds one root per group (the shared 512-token prefix) that is
        # not stepped; the 8 members are forks of it plus their own tails
        NB = w.num_blocks + 32 * 8 * 8
        spec = dict(S=w.S, H=w.H, D=w.D, BS=w.BS, dtype=w.dtype, scale=w.scale, layers=1,
                    lens=w.lens.astype(np.int64), NB=NB, growth=64, groups=32, prefix=512,
                    desc="32 groups x 8 seqs sharing a 512-token prefix, tails U[0,256], fp16")
    elif name == "fork_step":
        # every step re-forks each group: member 0 takes the group's prompt of 512 + r_g tokens
        # (r_g uniform in [1, 15], so the last prompt block is shared and partly filled), the
        # other 7 fork from it, and the step's append copies that block for 7 of the 8
        g = W.rng(seed * 31 + 3)
        r = W.uniform_lens(g, 32, 1, 15)
        prompts = (512 + r).astype(np.int64)
        lens = np.repeat(prompts, 8)
        NB = 2 * 32 * (W.nblocks_for(512 + 15, 16) + 8)
        spec = dict(S=256, H=40, D=128, BS=16, dtype="f16",
                    scale=float(np.float32(1 / math.sqrt(128))), layers=1, lens=lens, NB=NB,
                    growth=1, groups=32, refork=True, prompts=prompts,
                    desc="32 groups x 8 seqs forked from a prompt of 512 + U[1,15] tokens every "
                         "step: 224 copy-on-write block copies, then the append and decode, fp16")
    elif name == "full_step_40":
        lens, nb, _ = W.full_step(seed=5)
        spec = dict(S=len(lens), H=40, D=128, BS=16, dtype="f16",
                    scale=float(np.float32(1 / math.sqrt(128))), layers=40,
                    lens=lens.astype(np.int64), NB=nb, growth=16, groups=0,
                    desc="512 seqs, 40 layers, 40 heads, head_dim 128, BS 16, lognormal "
                         "lengths (mean 600, sigma 0.8) in [1,2048], fp16")
    else:
        raise ValueError(name)
    spec["name"] = name
    g = W.rng(seed * 7919 + 1)
    spec["order"] = (np.arange(spec["NB"]) if placement == "contiguous"
                     else g.permutation(spec["NB"]))
    return spec


class DecodeBatch:
    """The synthetic decode batch, its block manager and the native step driver."""

    def __init__(self, args, dev):
        import torch
        import paged_kv_cache_306_amd as pkv
        import workloads as W
        sp = workload_spec(args.workload, args.seed, args.block_size, args.placement)
        self.sp = sp
        self.S, self.H, self.D, self.BS = sp["S"], sp["H"], sp["D"], sp["BS"]
        self.dtype, self.scale, self.layers = sp["dtype"], sp["scale"], sp["layers"]
        self.e = W.ELEM_BYTES[self.dtype]
        self.init_lens = sp["lens"]
        self.growth = sp["growth"]
        self.NB = sp["NB"]
        self.max_ctx = int(self.init_lens.max()) + self.growth + 1
        self.MB = -(-self.max_ctx // self.BS)
        self.alloc = pkv.BlockAllocator(self.NB, self.BS, free_order=sp["order"])
        self.seq_ids = np.arange(self.S, dtype=np.int64)
        self.next_id = self.S
        self.roots = []
        if sp.get("refork"):
            self._fork_groups()
        elif sp["groups"]:
            per = self.S // sp["groups"]
            for gi in range(sp["groups"]):
                root = 1_000_000 + gi
                self.alloc.add_seq(root, sp["prefix"])
                self.roots.append(root)
            for s in range(self.S):
                self._fork_member(s, int(self.seq_ids[s]))
        else:
            for s in range(self.S):
                self.alloc.add_seq(int(self.seq_ids[s]), int(self.init_lens[s]))
        # Every sequence of a batch grows one token per step and all are replaced together, so
        # one counter (tokens grown since the last replacement) describes every length; the
        # per-step byte counts are tabulated by it once, outside the timed steps.
        self.grown = 0
        g = np.arange(self.growth + 2)[:, None]
        lens_by_grown = self.init_lens[None, :] + g
        self.tot_by_grown = lens_by_grown.sum(axis=1)
        self.nblk_by_grown = ((lens_by_grown + self.BS - 1) // self.BS).sum(axis=1)

        shape = (self.NB, self.H, self.BS, self.D)
        tensors = {k: [] for k in ("kp", "vp", "q", "kn", "vn", "out")}
        for l in range(self.layers):
            base = args.seed * 1000 + l * 10
            tensors["kp"].append(W.device_normal(shape, self.dtype, base + 1, dev))
            tensors["vp"].append(W.device_normal(shape, self.dtype, base + 2, dev))
            for j, k in enumerate(("q", "kn", "vn")):
                tensors[k].append(W.device_normal((self.S, self.H, self.D), self.dtype,
                                                  base + 3 + j, dev))
            tensors["out"].append(torch.empty_like(tensors["q"][-1]))
        self.t = tensors
        self.k_pool, self.v_pool, self.q = tensors["kp"][0], tensors["vp"][0], tensors["q"][0]
        self.stepper = pkv.DecodeStepper(self.alloc, tensors["kp"], tensors["vp"], tensors["q"],
                                         tensors["kn"], tensors["vn"], tensors["out"],
                                         self.scale, self.S, self.MB, self.max_ctx)
        self.cow_pairs = []      # copy-on-write block copies per step
        self.kv_bytes = []       # logical K+V bytes read by attention, per step (all layers)
        self.alg_bytes = []      # algorithmic bytes of one attention launch, per step
        self.last = None

    def _fork_groups(self):
        """Every group afresh: member 0 holds the group's prompt, the other members fork it
        (one batched block-manager call for the prompts and one for the forks)."""
        per = self.S // self.sp["groups"]
        self.seq_ids[:] = np.arange(self.next_id, self.next_id + self.S, dtype=np.int64)
        self.next_id += self.S
        firsts = self.seq_ids[::per]
        self.alloc.add_seqs(firsts, self.sp["prompts"])
        members = self.seq_ids.reshape(-1, per)
        self.alloc.fork_many(np.repeat(firsts, per - 1), members[:, 1:].reshape(-1))

    def _fork_member(self, s, sid):
        """Member s of its group: a fork of the group's prefix root plus its own tail."""
        per = self.S // self.sp["groups"]
        self.alloc.fork(self.roots[s // per], sid)
        tail = int(self.init_lens[s]) - self.sp["prefix"]
        if tail:
            self.alloc.append_slots(np.full(tail, sid, np.int64))

    @property
    def cur_len(self):
        return self.init_lens + self.grown

    def recycle(self):
        """Replace sequences that grew `growth` tokens by fresh ones of their start length
        (the fork step replaces every group after each step)."""
        if self.sp.get("refork"):
            if self.grown:
                self.alloc.free_seqs(self.seq_ids)
                self._fork_groups()
                self.grown = 0
            return
        if self.grown < self.growth:
            return
        for s in range(self.S):
            self.alloc.free_seq(int(self.seq_ids[s]))
            self.seq_ids[s] = self.next_id
            self.next_id += 1
            if self.sp["groups"]:
                self._fork_member(s, int(self.seq_ids[s]))
            else:
                self.alloc.add_seq(int(self.seq_ids[s]), int(self.init_lens[s]))
        self.grown = 0

    def step(self, events=None):
        self.recycle()
        max_len, ncow = self.stepper.step(self.seq_ids, events)
        self.cow_pairs.append(ncow)
        self.grown += 1
        self.last = (max_len, ncow)
        kv = 2 * int(self.tot_by_grown[self.grown]) * self.H * self.D * self.e
        nblk = int(self.nblk_by_grown[self.grown])
        self.kv_bytes.append(kv * self.layers)
        self.alg_bytes.append(kv + 2 * self.S * self.H * self.D * self.e + 4 * nblk + 4 * self.S)


def host_cpu() -> dict:
    """The host CPU the oracle baseline ran on: model name and the cores this process may use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "cores_available": len(os.sched_getaffinity(0))}


def cpu_baseline(batch, units_wanted, bytes_wanted):
    """Time the float64 oracle on (sequence, head) units of the same workload: layer 0, or for
    a multi-layer batch the first and the last layer (half of the budget each)."""
    import torch
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W
    tables, lens = batch.alloc.export(batch.seq_ids, batch.MB)
    layers = [0] if batch.layers == 1 else [0, batch.layers - 1]
    units, kv = [], 0
    prepared = {}
    for li, l in enumerate(layers):
        share_units = units_wanted * (li + 1) // len(layers)
        share_bytes = bytes_wanted * (li + 1) / len(layers)
        kp, vp = batch.t["kp"][l], batch.t["vp"][l]
        q = W.from_torch(batch.t["q"][l], batch.dtype)
        for s in range(batch.S):
            if len(units) >= share_units or kv >= share_bytes:
                break
            n = -(-int(lens[s]) // batch.BS)
            idx = torch.from_numpy(tables[s, :n].astype(np.int64)).to(kp.device)
            prepared[(l, s)] = (q, W.from_torch(kp.index_select(0, idx), batch.dtype),
                                W.from_torch(vp.index_select(0, idx), batch.dtype),
                                np.arange(n, dtype=np.int32)[None, :])
            for h in range(batch.H):
                if len(units) < share_units and kv < share_bytes:
                    units.append((l, s, h))
                    kv += 2 * int(lens[s]) * batch.D * batch.e

    def unit(u):
        l, s, h = u
        q, kc, vc, tab = prepared[(l, s)]
        oracle.decode_unit(q[s:s + 1], kc, vc, tab, lens[s:s + 1], batch.scale, batch.dtype,
                           0, h)

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for u in units:
            unit(u)
        dt = time.perf_counter() - t0
        # the same calls over every host core this process may use (at most 16, the host
        # share of one GPU): one thread per core, each running whole units, BLAS single-threaded
        from concurrent.futures import ThreadPoolExecutor
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        with ThreadPoolExecutor(threads) as ex:
            t0 = time.perf_counter()
            list(ex.map(unit, units))
            dt_all = time.perf_counter() - t0
    per_layer = {l: sum(1 for u in units if u[0] == l) for l in layers}
    where = ", ".join(f"layer {l}: {n} units" for l, n in per_layer.items())
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(units)} (sequence, head) units of the same batch ({where}), "
                      f"{kv / 1e6:.1f} MB of K+V, float64 numpy, {dt:.2f} s",
            "seq_layer_per_s": len(units) / batch.H / dt,
            "all_cores": {"value": kv / dt_all / 1e9, "threads": threads,
                          "seq_layer_per_s": len(units) / batch.H / dt_all,
                          "seconds": round(dt_all, 2)},
            "host_cpu": host_cpu()}


def sweep(args, reps: int = 3):
    """Block-size x placement microbenchmark: the decode launch and whole step of the
    LLaMA-13B-shaped layer and of the long-context batch at block sizes 8, 16, 32, with
    seeded random (scattered) and contiguous block placement, plus the KV waste.  Every
    configuration is built once; then ``reps`` rounds time each in turn (the order rotating
    from round to round), so every cell gets ``reps`` interleaved readings in one process.
    One JSON line per configuration: the median and the spread (min, max) of its readings."""
    import torch
    dev = device_or_die()
    cells = []
    for wl in ("llama13b_layer", "long_context"):
        for bs in (8, 16, 32):
            for placement in ("permuted", "contiguous"):
                args.workload, args.block_size, args.placement = wl, bs, placement
                b = DecodeBatch(args, dev)
                for _ in range(max(args.warmup, 50)):
                    b.step()
                cells.append({"wl": wl, "bs": bs, "placement": placement, "batch": b,
                              "launch_us": [], "step_ms": [], "alg_GBs": []})
    torch.cuda.synchronize()
    for rep in range(reps):
        order = cells[rep % len(cells):] + cells[:rep % len(cells)]
        if rep % 2:
            order = order[::-1]
        for c in order:
            b = c["batch"]
            warm = TimingEvents(10, 1)
            for i in range(10):                 # re-warm after the other configurations
                b.step(warm.handles[i])
            events = TimingEvents(args.steps, 1)
            torch.cuda.synchronize()
            with gc_paused():
                t0 = time.perf_counter()
                for i in range(args.steps):
                    b.step(events.handles[i])
                torch.cuda.synchronize()
                wall = time.perf_counter() - t0
            launch = float(np.mean(events.elapsed_ms())) / 1e3
            events.destroy()
            warm.destroy()
            c["launch_us"].append(launch * 1e6)
            c["step_ms"].append(wall / args.steps * 1e3)
            c["alg_GBs"].append(float(np.mean(b.alg_bytes[-args.steps:])) / launch / 1e9)
    for c in cells:
        b = c["batch"]
        used = int(sum(len(b.alloc.block_table(int(x))) for x in b.seq_ids))
        waste = b.alloc.wasted_slots()
        stat = lambda v, nd: {"median": round(float(np.median(v)), nd),
                              "min": round(float(np.min(v)), nd), "max": round(float(np.max(v)), nd)}
        print(json.dumps({
            "sweep": "block_size x placement", "workload": f"{c['wl']}_{b.dtype}",
            "block_size": c["bs"], "placement": c["placement"], "reps": reps,
            "steps_per_rep": args.steps,
            "decode_launch_us": stat(c["launch_us"], 1), "ms_per_step": stat(c["step_ms"], 4),
            "decode_alg_GBs": stat(c["alg_GBs"], 1),
            "allocated_slots": used * c["bs"], "wasted_slots": int(waste),
            "waste_frac": round(waste / max(1, used * c["bs"]), 5),
            "xcd_split": b.stepper.xcd_split}), flush=True)


def device_or_die():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    return torch.device("cuda:0")


def swap_bench(args, layers: int = 8, tokens: int = 16384):
    """Preemption by swapping: move `tokens` tokens per layer of LLaMA-13B-shaped fp16 K/V
    (scattered blocks) to a pinned host pool and back with one pkv_swap_blocks call each way;
    a single contiguous copy of the same byte count gives the PCIe reference."""
    import torch
    import paged_kv_cache_306_amd as pkv
    import workloads as W
    dev = torch.device("cuda:0")
    H, D = 40, 128
    for bs in (8, 16, 32):
        n = tokens // bs
        nb_dev, nb_host = n * 2, n
        g = W.rng(77 + bs)
        dk = [W.device_normal((nb_dev, H, bs, D), "f16", 10 * l + 1, dev) for l in range(layers)]
        dv = [W.device_normal((nb_dev, H, bs, D), "f16", 10 * l + 2, dev) for l in range(layers)]
        hk = [torch.empty((nb_host, H, bs, D), dtype=torch.float16).pin_memory() for _ in range(layers)]
        hv = [torch.empty((nb_host, H, bs, D), dtype=torch.float16).pin_memory() for _ in range(layers)]
        src = g.permutation(nb_dev)[:n].astype(np.int32)
        out_pairs = torch.from_numpy(np.stack([src, g.permutation(n).astype(np.int32)], 1)).to(dev)
        in_pairs = torch.from_numpy(np.stack([np.arange(n, dtype=np.int32),
                                              g.permutation(nb_dev)[:n].astype(np.int32)], 1)).to(dev)
        nbytes = 2 * layers * n * H * bs * D * 2
        res = {"swap": "HBM <-> pinned host", "block_size": bs, "layers": layers,
               "blocks_per_layer": n, "bytes_each_way": nbytes}
        for name, fn in (("out", lambda: pkv.swap_blocks(dk, dv, hk, hv, out_pairs)),
                         ("in", lambda: pkv.swap_blocks(hk, hv, dk, dv, in_pairs))):
            fn()
            torch.cuda.synchronize()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            times = []
            for _ in range(5):
                a.record()
                fn()
                z.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(z) / 1e3)
            t = float(np.median(times))
            res[f"swap_{name}_ms"] = round(t * 1e3, 3)
            res[f"swap_{name}_GBs"] = round(nbytes / t / 1e9, 2)
        # the same swap-out done block by block (one async copy per K or V block of layer 0):
        # the per-transfer cost that one batched launch avoids
        lb = 2 * n * H * bs * D * 2
        srcs, dsts = out_pairs[:, 0].tolist(), out_pairs[:, 1].tolist()

        def per_block():
            for sb, db in zip(srcs, dsts):
                hk[0][db].copy_(dk[0][sb], non_blocking=True)
                hv[0][db].copy_(dv[0][sb], non_blocking=True)
        per_block()
        torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record()
        per_block()
        z.record()
        torch.cuda.synchronize()
        res["per_block_copies_out"] = 2 * n
        res["per_block_copy_out_GBs"] = round(lb / (a.elapsed_time(z) / 1e3) / 1e9, 2)
        res["per_block_copy_out_wall_GBs"] = round(lb / (time.perf_counter() - t0) / 1e9, 2)
        # one contiguous copy of the same size each way (the PCIe reference)
        flat_d = torch.empty(nbytes // 2, dtype=torch.float16, device=dev)
        flat_h = torch.empty(nbytes // 2, dtype=torch.float16).pin_memory()
        for name, (dst, srct) in (("d2h", (flat_h, flat_d)), ("h2d", (flat_d, flat_h))):
            dst.copy_(srct, non_blocking=True)
            torch.cuda.synchronize()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dst.copy_(srct, non_blocking=True)
            z.record()
            torch.cuda.synchronize()
            res[f"contiguous_{name}_GBs"] = round(nbytes / (a.elapsed_time(z) / 1e3) / 1e9, 2)
        print(json.dumps(res), flush=True)
        del dk, dv, hk, hv, flat_d, flat_h
        torch.cuda.empty_cache()


def prefix_cache_bench(args, requests: int = 512, prompts: int = 4, system_len: int = 1024):
    """Prefix caching ("Advanced Features" -> "Prefix Caching"): chat requests whose prompt is
    one of a few system prompts plus a user message of 16-512 tokens.  Compares the KV blocks
    the block manager holds with and without the prefix cache, and times the cached admission
    (host C++, one call per request)."""
    import paged_kv_cache_306_amd as pkv
    import workloads as W
    g = W.rng(args.seed + 99)
    BS = 16
    systems = [g.integers(0, 32000, size=system_len).astype(np.int32) for _ in range(prompts)]
    reqs = [np.concatenate([systems[int(g.integers(prompts))],
                            g.integers(0, 32000, size=int(g.integers(16, 513))).astype(np.int32)])
            for _ in range(requests)]
    need_plain = sum(W.nblocks_for(len(r), BS) for r in reqs)
    NB = need_plain + 16
    plain = pkv.BlockAllocator(NB, BS)
    for i, r in enumerate(reqs):
        plain.add_seq(i, len(r))
    cached = pkv.BlockAllocator(NB, BS)
    hit_tokens = 0
    t0 = time.perf_counter()
    for i, r in enumerate(reqs):
        hit_tokens += cached.add_seq_cached(i, r)
    dt = time.perf_counter() - t0
    used_plain = NB - plain.num_free()
    used_cached = NB - cached.num_free()
    total_tokens = int(sum(len(r) for r in reqs))
    print(json.dumps({
        "prefix_cache": "chat requests", "requests": requests, "system_prompts": prompts,
        "system_len": system_len, "user_len": "U[16,512]", "block_size": BS,
        "blocks_without_cache": used_plain, "blocks_with_cache": used_cached,
        "kv_memory_saved_frac": round(1 - used_cached / used_plain, 4),
        "prompt_tokens_served_from_cache_frac": round(hit_tokens / total_tokens, 4),
        "admission_us_per_request": round(dt / requests * 1e6, 2),
        "host": "the machine bench.py ran on"}), flush=True)


def multi_query_bench(args):
    """Chat requests after a prefix-cache hit: per step, the user turns' new K/V are appended
    in one pkv_reshape_and_cache call, then every new token attends (one
    pkv_paged_attention_multi_query launch on a host-built schedule)."""
    import torch
    import paged_kv_cache_306_amd as pkv
    import workloads as W
    dev = torch.device("cuda:0")
    lo, hi = (int(x) for x in args.user_turns.split(","))
    w = W.prefix_hit(dtype=args.dtype, user_lo=lo, user_hi=hi)
    qs = w.extra["query_start"]
    T, H, D, BS, dt = int(qs[-1]), w.H, w.D, w.BS, w.dtype
    new = np.diff(qs).astype(np.int64)
    # slots of the new tokens: the last n_s positions of each context
    slots = np.concatenate([
        w.tables[s, (np.arange(w.lens[s] - new[s], w.lens[s]) // BS)].astype(np.int64) * BS
        + np.arange(w.lens[s] - new[s], w.lens[s]) % BS for s in range(w.S)]).astype(np.int32)
    kp = W.device_normal((w.num_blocks, H, BS, D), dt, 71, dev)
    vp = W.device_normal((w.num_blocks, H, BS, D), dt, 72, dev)
    q = W.device_normal((T, H, D), dt, 73, dev)
    kn = W.device_normal((T, H, D), dt, 74, dev)
    vn = W.device_normal((T, H, D), dt, 75, dev)
    out = torch.empty_like(q)
    bt = torch.from_numpy(w.tables).to(dev)
    cl = torch.from_numpy(w.lens).to(dev)
    qsd = torch.from_numpy(qs).to(dev)
    sl = torch.from_numpy(slots).to(dev)
    packed = args.mq_schedule == "packed"
    if packed:
        # the new tokens of the requests that share a prompt's blocks fill whole tiles
        items = torch.from_numpy(pkv.multi_query_schedule_packed(qs, w.lens, w.tables, BS,
                                                                 w.max_len)).to(dev)
    else:
        # requests that share a system prompt (the same first physical block) side by side
        items = torch.from_numpy(pkv.multi_query_schedule(qs, w.lens, w.max_len,
                                                          group_keys=w.tables[:, 0])).to(dev)
    maxq = int(new.max())

    def attend():
        if packed:
            pkv.paged_attention_multi_query_packed(out, q, kp, vp, bt, cl, qsd, w.scale, maxq,
                                                   w.max_len, items)
        else:
            pkv.paged_attention_multi_query(out, q, kp, vp, bt, cl, qsd, w.scale, maxq,
                                            w.max_len, work_items=items)
    # algorithmic work: token i of sequence s sees P + 1 = L_s - n_s + i + 1 keys; per key and
    # head 2 D flops for the score and 2 D for the output
    keys = int(sum(int(new[s]) * (int(w.lens[s]) - int(new[s])) + int(new[s]) * (int(new[s]) + 1) // 2
                   for s in range(w.S)))
    flops = 4.0 * D * H * keys

    def step():
        pkv.reshape_and_cache(kn, vn, kp, vp, sl)
        attend()

    for _ in range(args.warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    with gc_paused():
        t0 = time.perf_counter()
        for a, z in evs:
            pkv.reshape_and_cache(kn, vn, kp, vp, sl)
            a.record()
            attend()
            z.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    launch_s = float(np.mean([a.elapsed_time(z) for a, z in evs])) / 1e3
    peak = MFMA_PEAK_TFLOPS[dt]
    achieved = flops / launch_s / 1e12
    value = flops * args.steps / wall / 1e12
    res = {
        "metric": "multi-query paged attention TFLOP/s after a prefix-cache hit, LLaMA-13B "
                  "shape", "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dt, "data": "synthetic",
        "config": {"workload": f"prefix_hit_{dt}" + ("" if (lo, hi) == (16, 512)
                                                     else f"_turns{lo}-{hi}"),
                   "description": f"{w.S} requests, {w.extra['prompts']} shared system prompts "
                                  f"of {w.extra['system_len']} cached tokens, user turns "
                                  f"U{list(w.extra['user_range'])} new tokens, 40 heads, "
                                  "head_dim 128, BS 16",
                   "requests": w.S, "new_tokens": T, "keys_seen": keys, "heads": H,
                   "head_dim": D, "block_size": BS, "pool_blocks": w.num_blocks,
                   "schedule": args.mq_schedule, "tiles_per_head": int(items.shape[0])},
        "new_tokens_per_s": round(T * args.steps / wall, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": ((measured_traffic(MQ_COUNTER_PROFILE, MQ_KERNEL_SOURCES) or {})
                                 .get("bytes") if dt == "f16" else None),
                     "kernel": f"multi_query_kernel<{dt.upper()},{D},{BS}>",
                     "avg_launch_us": round(launch_s * 1e6, 2),
                     "alg_flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = multi_query_cpu_baseline(w, q, kp, vp, dt)
    print(json.dumps(res), flush=True)


def multi_query_cpu_baseline(w, q, kp, vp, dt, seconds: float = 8.0):
    """The float64 oracle on (request, new token, head) units of the same batch, one thread,
    for about ``seconds``: rows of the first requests, all heads."""
    import torch
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W
    qs = w.extra["query_start"]
    q_np = W.from_torch(q, dt)
    done, flops, units = 0.0, 0.0, 0
    with threadpool_limits(limits=1):
        for s in range(w.S):
            n = int(qs[s + 1] - qs[s])
            nbk = W.nblocks_for(int(w.lens[s]), w.BS)
            idx = torch.from_numpy(w.tables[s, :nbk].astype(np.int64)).to(kp.device)
            kc = W.from_torch(kp.index_select(0, idx), dt)
            vc = W.from_torch(vp.index_select(0, idx), dt)
            tab = np.arange(nbk, dtype=np.int32)[None, :]
            qsub = q_np[qs[s]:qs[s + 1]]
            for i in range(n):
                t0 = time.perf_counter()
                for h in range(w.H):
                    oracle.multi_query_unit(qsub, kc, vc, tab, w.lens[s:s + 1],
                                            np.array([0, n]), w.scale, dt, 0, i, h)
                done += time.perf_counter() - t0
                units += w.H
                flops += 4.0 * w.D * w.H * (int(w.lens[s]) - n + i + 1)
                if done >= seconds:
                    break
            if done >= seconds:
                break
    return {"value": flops / done / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{units} (new token, head) units of the first requests of the same "
                      f"batch, float64 numpy, {done:.2f} s",
            "host_cpu": host_cpu()}


def main():
    args = parse()
    if args.prefix_cache:
        prefix_cache_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the paged "
              "attention path here has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.calibrate_read:
        calibrate_read(args.calibrate_read)
        return
    if args.mfma_ceiling:
        mfma_ceiling(args)
        return
    if args.ceiling:
        ceiling_bench(args)
        return
    if args.sweep:
        sweep(args)
        return
    if args.swap:
        swap_bench(args)
        return
    if args.workload == "prefix_hit":
        multi_query_bench(args)
        return
    import torch
    dev = torch.device("cuda:0")
    b = DecodeBatch(args, dev)
    L = b.layers
    # The step driver's attention launches take these events themselves (start and end), on
    # the last step of every K: a launch that carries them is preceded and followed by a few
    # idle microseconds more (≈ 4 us per step on the LLaMA-13B layer), which the other steps
    # do not pay, and the first step after the region's synchronization (an idle GPU, a
    # slower launch) is not one of them.  The warm-up steps follow the same pattern.
    every = max(1, args.event_every)

    def carries(i, n):
        return i % every == every - 1 or (n < every and i == n - 1)
    timed = [i for i in range(args.steps) if carries(i, args.steps)]
    warm_idx = {i: k for k, i in enumerate(i for i in range(args.warmup) if carries(i, args.warmup))}
    warm_events = TimingEvents(max(1, len(warm_idx)), L)
    events = TimingEvents(len(timed), L)
    ev_idx = {i: k for k, i in enumerate(timed)}
    for i in range(args.warmup):
        b.step(warm_events.handles[warm_idx[i]] if i in warm_idx else None)
    torch.cuda.synchronize()
    warm_events.destroy()
    b.kv_bytes.clear()
    b.alg_bytes.clear()
    import paged_kv_cache_306_amd as pkv
    flush = (torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
             if args.flush_mall else None)
    torch.cuda.synchronize()
    host = 0.0
    with gc_paused():
        t0 = time.perf_counter()
        for i in range(args.steps):
            if flush is not None:
                flush.view(torch.int64).sum()   # reads 1 GiB: evicts the MALL, no dirty lines
            h0 = time.perf_counter()
            b.step(events.handles[ev_idx[i]] if i in ev_idx else None)
            host += time.perf_counter() - h0
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    attn_ms = events.elapsed_ms()
    events.destroy()
    attn_avg_s = float(np.mean(attn_ms)) / 1e3
    attn_med_s = float(np.median(attn_ms)) / 1e3
    kv_total = float(np.sum(b.kv_bytes))
    value = kv_total / wall / 1e9
    alg_per_launch = float(np.mean([b.alg_bytes[i] for i in timed]))   # the timed launches'
    achieved = alg_per_launch / attn_avg_s / 1e9
    desc = pkv.desc_for_pool(b.k_pool)
    split = pkv.decode_partition_tokens(desc, b.S, b.max_ctx) > 0
    dt_name = {"f16": "F16", "bf16": "BF16", "f32": "F32"}[b.dtype]
    kname = f"decode_partition_kernel<{dt_name},{b.D},{b.BS}>"
    kname += " + decode_reduce_kernel (split context)" if split else " (single pass: one launch)"
    if b.stepper.last_attention == pkv.PKV_STEP_ATTN_MULTI_QUERY:
        # groups sharing their first blocks: the step driver attends through packed tiles
        kname = (f"multi_query_kernel<{dt_name},{b.D},{b.BS}> over packed tiles (sequences "
                 "sharing their first blocks, one new token each)")
    default = args.workload == "llama13b_layer" and args.placement == "permuted"
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": b.dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}_{b.dtype}", "description": b.sp["desc"],
                   "seqs": b.S, "heads": b.H, "head_dim": b.D, "block_size": b.BS,
                   "layers": L, "pool_blocks": b.NB, "placement": args.placement,
                   "growth_tokens_before_replacement": b.growth,
                   "flush_mall_bytes_per_step": (1 << 30) if args.flush_mall else 0},
        "seq_layer_per_s": round(b.S * L * args.steps / wall, 1),
        "cow_pairs_per_step": round(float(np.mean(b.cow_pairs[-args.steps:])), 2),
        "host_ms_per_step": round(host / args.steps * 1e3, 4),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": kname, "avg_launch_us": round(attn_avg_s * 1e6, 2),
                     "median_launch_us": round(attn_med_s * 1e6, 2),
                     "achieved_at_median": round(alg_per_launch / attn_med_s / 1e9, 1),
                     "launches": len(attn_ms), "launch_events_every_k_steps": every,
                     "alg_bytes_per_launch": int(alg_per_launch),
                     # share (of 1024) of the units dealt to the even XCDs, as the stepper
                     # measured it on its first step (0: dealt evenly), and the halves' tokens
                     # per 100 MHz tick of workgroup time in that measurement
                     "xcd_split": b.stepper.xcd_split,
                     "xcd_rates_even_odd": [round(x, 5) for x in b.stepper.xcd_rates()[:2]]},
    }
    traffic = measured_traffic() if default else None
    if traffic:
        res["roofline"]["traffic"] = traffic["bytes"]
        res["roofline"]["traffic_counter_scale"] = {
            "FETCH_SIZE": traffic.get("fetch_scale"), "WRITE_SIZE": traffic.get("write_scale"),
            "calibrated_on": traffic.get("calibration")}
    # the decode launch against a plain read of exactly its own tiles (measured here, after the
    # timed steps; 16-token blocks at the seeded placement, pools small enough for a copy)
    if (args.workload in ("llama13b_layer", "long_context") and args.block_size == 16
            and args.placement == "permuted"):
        own = own_tiles_read_rate(args.workload, args.seed, b.stepper.xcd_split)
        if own:
            # the ceiling is the better of the two reads: evenly dealt, or weighted like the
            # decode launches
            best = max(x for x in own if x)
            res["roofline"]["own_tiles_read_GBs"] = best
            res["roofline"]["own_tiles_read_even_deal_GBs"] = own[0]
            res["roofline"]["own_tiles_read_weighted_GBs"] = own[1]
            res["roofline"]["frac_of_own_tiles_read"] = round(achieved / best, 4)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(b, args.cpu_units, args.cpu_bytes)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
