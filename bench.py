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
GROWTH = 64   # tokens a sequence grows before it is replaced


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--placement", choices=["permuted", "contiguous"], default="permuted")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=320,
                    help="(sequence, head) units the oracle baseline computes")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (to scale HBM counters)")
    return ap.parse_args()


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


class DecodeBatch:
    """The synthetic decode batch, its block manager and the native step driver."""

    def __init__(self, args, dev):
        import torch
        import paged_kv_cache_306_amd as pkv
        import workloads as W
        w = W.llama13b_layer(args.seed)
        self.w = w
        self.S, self.H, self.D, self.BS = w.S, w.H, w.D, w.BS
        self.dtype = w.dtype
        self.scale = w.scale
        self.init_lens = w.lens.astype(np.int64)
        # pool 1.2x the need at the start lengths, as in the workload recipe
        self.NB = w.num_blocks
        self.max_ctx = int(self.init_lens.max()) + GROWTH + 1
        self.MB = -(-self.max_ctx // self.BS)
        g = W.rng(args.seed * 7919 + 1)
        order = (np.arange(self.NB) if args.placement == "contiguous"
                 else g.permutation(self.NB))
        self.alloc = pkv.BlockAllocator(self.NB, self.BS, free_order=order)
        self.seq_ids = np.arange(self.S, dtype=np.int64)
        self.next_id = self.S
        for s in range(self.S):
            self.alloc.add_seq(int(self.seq_ids[s]), int(self.init_lens[s]))
        self.cur_len = self.init_lens.copy()

        shape = (self.NB, self.H, self.BS, self.D)
        self.k_pool = W.device_normal(shape, self.dtype, args.seed * 10 + 1, dev)
        self.v_pool = W.device_normal(shape, self.dtype, args.seed * 10 + 2, dev)
        self.q = W.device_normal((self.S, self.H, self.D), self.dtype, args.seed * 10 + 3, dev)
        self.k_new = W.device_normal((self.S, self.H, self.D), self.dtype, args.seed * 10 + 4, dev)
        self.v_new = W.device_normal((self.S, self.H, self.D), self.dtype, args.seed * 10 + 5, dev)
        self.out = torch.empty_like(self.q)
        self.stepper = pkv.DecodeStepper(self.alloc, [self.k_pool], [self.v_pool], [self.q],
                                         [self.k_new], [self.v_new], [self.out], self.scale,
                                         self.S, self.MB, self.max_ctx)
        self.kv_bytes = []       # logical K+V bytes read by attention, per step
        self.alg_bytes = []      # algorithmic bytes of the attention launch, per step
        self.last = None

    def recycle(self):
        """Replace sequences that grew GROWTH tokens by fresh ones of their start length."""
        done = np.nonzero(self.cur_len - self.init_lens >= GROWTH)[0]
        for s in done:
            self.alloc.free_seq(int(self.seq_ids[s]))
            self.seq_ids[s] = self.next_id
            self.next_id += 1
            self.alloc.add_seq(int(self.seq_ids[s]), int(self.init_lens[s]))
            self.cur_len[s] = self.init_lens[s]

    def step(self, events=None):
        self.recycle()
        max_len, ncow = self.stepper.step(self.seq_ids, events)
        self.cur_len += 1
        self.last = (max_len, ncow)
        tot = int(self.cur_len.sum())
        kv = 2 * tot * self.H * self.D * 2
        nblk = int(((self.cur_len + self.BS - 1) // self.BS).sum())
        self.kv_bytes.append(kv)
        self.alg_bytes.append(kv + 2 * self.S * self.H * self.D * 2 + 4 * nblk + 4 * self.S)


def cpu_baseline(batch, units_wanted):
    """Time the float64 oracle on (sequence, head) units of the same workload."""
    import torch
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W
    tables, lens = batch.alloc.export(batch.seq_ids, batch.MB)
    q = W.from_torch(batch.q, batch.dtype)
    units, seqs, kv = [], [], 0
    for s in range(batch.S):
        if len(units) >= units_wanted:
            break
        seqs.append(s)
        for h in range(batch.H):
            if len(units) < units_wanted:
                units.append((s, h))
                kv += 2 * int(lens[s]) * batch.D * 2
    prepared = {}
    for s in seqs:
        n = -(-int(lens[s]) // batch.BS)
        idx = torch.from_numpy(tables[s, :n].astype(np.int64)).to(batch.k_pool.device)
        prepared[s] = (W.from_torch(batch.k_pool.index_select(0, idx), batch.dtype),
                       W.from_torch(batch.v_pool.index_select(0, idx), batch.dtype),
                       np.arange(n, dtype=np.int32)[None, :])
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for s, h in units:
            kc, vc, tab = prepared[s]
            oracle.decode_unit(q[s:s + 1], kc, vc, tab, lens[s:s + 1], batch.scale, batch.dtype,
                               0, h)
        dt = time.perf_counter() - t0
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(units)} (sequence, head) units = first {len(seqs)} sequences x "
                      f"40 heads of the same batch, {kv / 1e6:.1f} MB of K+V, float64 numpy, "
                      f"{dt:.2f} s",
            "seq_layer_per_s": len(units) / batch.H / dt}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no "
              "multi-GPU mode in this build", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    import torch
    dev = torch.device("cuda:0")
    b = DecodeBatch(args, dev)
    for _ in range(args.warmup):
        b.step()
    torch.cuda.synchronize()
    b.kv_bytes.clear()
    b.alg_bytes.clear()
    import ctypes
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, z in evs:          # create the events; the step driver re-records them
        a.record()
        z.record()
    handles = [(ctypes.c_void_p * 2)(a.cuda_event, z.cuda_event) for a, z in evs]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        b.step(handles[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = [a.elapsed_time(z) for a, z in evs]
    attn_avg_s = float(np.mean(attn_ms)) / 1e3
    kv_total = float(np.sum(b.kv_bytes))
    value = kv_total / wall / 1e9
    alg_per_launch = float(np.mean(b.alg_bytes))
    achieved = alg_per_launch / attn_avg_s / 1e9
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama13b_layer_fp16", "seqs": b.S, "heads": b.H,
                   "head_dim": b.D, "block_size": b.BS, "context_lens": "uniform[128,2048] + growth",
                   "pool_blocks": b.NB, "placement": args.placement, "layers": 1},
        "seq_layer_per_s": round(b.S * args.steps / wall, 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "paged_attention_decode (partition + reduce launches)",
                     "avg_launch_us": round(attn_avg_s * 1e6, 2),
                     "alg_bytes_per_launch": int(alg_per_launch)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(b, args.cpu_units)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
