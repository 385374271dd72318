"""Decode-step benchmark of the paged KV-cache hot path on one MI355X.

One step = one decode iteration of a batch, all through libpkv:
  1. host block manager: append one slot per sequence (new block on a block boundary,
     copy-on-write pairs for shared blocks), export the block tables and lengths;
  2. copy tables / lengths / slots to the device (pinned, double-buffered, asynchronous);
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
    return ap.parse_args()


class DecodeBatch:
    """The synthetic decode batch and its device buffers."""

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
        self.MB = -(-(int(w.lens.max()) + GROWTH + 1) // self.BS)
        g = W.rng(args.seed * 7919 + 1)
        order = (np.arange(self.NB) if args.placement == "contiguous"
                 else g.permutation(self.NB))
        self.alloc = pkv.BlockAllocator(self.NB, self.BS, free_order=order)
        self.seq_ids = np.arange(self.S, dtype=np.int64)
        self.next_id = self.S
        for s in range(self.S):
            self.alloc.add_seq(int(self.seq_ids[s]), int(self.init_lens[s]))
        self.grown = np.zeros(self.S, np.int64)

        shape = (self.NB, self.H, self.BS, self.D)
        self.k_pool = W.device_normal(shape, self.dtype, args.seed * 10 + 1, dev)
        self.v_pool = W.device_normal(shape, self.dtype, args.seed * 10 + 2, dev)
        self.q = W.device_normal((self.S, self.H, self.D), self.dtype, args.seed * 10 + 3, dev)
        self.k_new = W.device_normal((self.S, self.H, self.D), self.dtype, args.seed * 10 + 4, dev)
        self.v_new = W.device_normal((self.S, self.H, self.D), self.dtype, args.seed * 10 + 5, dev)
        self.out = torch.empty_like(self.q)

        # device index buffers and two pinned host staging sets
        self.d_tables = torch.empty((self.S, self.MB), dtype=torch.int32, device=dev)
        self.d_lens = torch.empty(self.S, dtype=torch.int32, device=dev)
        self.d_slots = torch.empty(self.S, dtype=torch.int32, device=dev)
        self.d_pairs = torch.empty((self.S, 2), dtype=torch.int32, device=dev)
        self.stage = []
        for _ in range(2):
            t = torch.empty((self.S, self.MB), dtype=torch.int32, pin_memory=True)
            L = torch.empty(self.S, dtype=torch.int32, pin_memory=True)
            sl = torch.empty(self.S, dtype=torch.int32, pin_memory=True)
            pr = torch.empty((self.S, 2), dtype=torch.int32, pin_memory=True)
            self.stage.append({"t": t, "L": L, "sl": sl, "pr": pr, "ev": torch.cuda.Event()})
        max_ctx = int(self.init_lens.max()) + GROWTH + 1
        desc = pkv.desc_for_pool(self.k_pool)
        self.workspace = torch.empty(max(16, pkv.decode_workspace_bytes(desc, self.S, max_ctx)),
                                     dtype=torch.uint8, device=dev)
        self.step_i = 0
        self.kv_bytes = []       # logical K+V bytes read by attention, per step
        self.alg_bytes = []      # algorithmic bytes of the attention launch, per step

    def recycle(self):
        """Replace sequences that grew GROWTH tokens by fresh ones of their start length."""
        for s in np.nonzero(self.grown >= GROWTH)[0]:
            self.alloc.free_seq(int(self.seq_ids[s]))
            self.seq_ids[s] = self.next_id
            self.next_id += 1
            self.alloc.add_seq(int(self.seq_ids[s]), int(self.init_lens[s]))
            self.grown[s] = 0

    def step(self, ev_pair=None):
        import paged_kv_cache_306_amd as pkv
        st = self.stage[self.step_i % 2]
        self.step_i += 1
        st["ev"].synchronize()             # its previous copies have left the buffers
        self.recycle()
        sl, pr = st["sl"].numpy(), st["pr"].numpy()
        ncow = self.alloc.append_slots_into(self.seq_ids, sl, pr)
        self.grown += 1
        tables, lens = st["t"].numpy(), st["L"].numpy()
        self.alloc.export_into(self.seq_ids, tables, lens)
        max_len = int(lens.max())
        self.d_tables.copy_(st["t"], non_blocking=True)
        self.d_lens.copy_(st["L"], non_blocking=True)
        self.d_slots.copy_(st["sl"], non_blocking=True)
        if ncow:
            self.d_pairs[:ncow].copy_(st["pr"][:ncow], non_blocking=True)
        st["ev"].record()
        if ncow:
            pkv.copy_blocks([self.k_pool], [self.v_pool], self.d_pairs[:ncow])
        pkv.reshape_and_cache(self.k_new, self.v_new, self.k_pool, self.v_pool, self.d_slots)
        if ev_pair is not None:
            ev_pair[0].record()
        pkv.paged_attention_decode(self.out, self.q, self.k_pool, self.v_pool, self.d_tables,
                                   self.d_lens, self.scale, max_len, workspace=self.workspace)
        if ev_pair is not None:
            ev_pair[1].record()
        tot = int(lens.astype(np.int64).sum())
        e = 2
        kv = 2 * tot * self.H * self.D * e
        nblk = int(sum(-(-int(L) // self.BS) for L in lens))
        self.kv_bytes.append(kv)
        self.alg_bytes.append(kv + 2 * self.S * self.H * self.D * e + 4 * nblk + 4 * self.S)
        return lens


def cpu_baseline(batch, units_wanted):
    """Time the float64 oracle on (sequence, head) units of the same workload."""
    import torch
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W
    lens = batch.stage[(batch.step_i - 1) % 2]["L"].numpy().copy()
    tables = batch.stage[(batch.step_i - 1) % 2]["t"].numpy().copy()
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
    import torch
    dev = torch.device("cuda:0")
    b = DecodeBatch(args, dev)
    for _ in range(args.warmup):
        b.step()
    torch.cuda.synchronize()
    b.kv_bytes.clear()
    b.alg_bytes.clear()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        b.step(evs[i])
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
