"""XCD-weighted dealing of the attention units in the decode-step driver: outputs bit-identical
under every split and matching the oracle, and the split the stepper measures on its first
step with enough units."""
import math

import numpy as np
import pytest

import oracle
import paged_kv_cache_306_amd as pkv
import workloads as W
from gpu_util import check_close, device, to_dev

pytestmark = pytest.mark.gpu

D, BS, DT = 128, 16, "f16"
STEPS = 2


def _lengths(seed, full=False):
    g = W.rng(seed)
    if full:
        # the LLaMA-13B layer's shape: 64 sequences x 40 heads = 2560 units, more than the
        # chip holds at once, so the stepper measures its XCD halves under load
        return g.integers(128, 2049, 64).astype(np.int64)
    # single-pass lengths and a few sequences long enough to be split into partitions
    return np.concatenate([g.integers(1, 2049, 36), g.integers(4097, 6001, 4)]).astype(np.int64)


def _run(split, seed=77, full=False):
    """One stepper over a fresh copy of the same batch (8 heads; the full batch: 40); `split`
    None: the stepper measures it.  Returns (outputs per step, the split in use after the last
    step, the measurement's rates and outcome, oracle inputs)."""
    import torch
    dev = device()
    H = 40 if full else 8
    start = _lengths(seed, full)
    S = len(start)
    MB = int((start.max() + STEPS + BS - 1) // BS)
    NB = int(sum((L + STEPS + BS - 1) // BS for L in start) * 1.3) + 8
    g = W.rng(seed + 1)
    order = g.permutation(NB)
    a = pkv.BlockAllocator(NB, BS, free_order=order)
    m = oracle.BlockManager(NB, BS, free_order=order)
    for sid, L in enumerate(start):
        a.add_seq(sid, int(L))
        m.add_seq(sid, int(L))
    kp = W.normal_values(g, (NB, H, BS, D), DT)
    vp = W.normal_values(g, (NB, H, BS, D), DT)
    qs = [W.normal_values(g, (S, H, D), DT) for _ in range(STEPS)]
    kn = [W.normal_values(g, (S, H, D), DT) for _ in range(STEPS)]
    vn = [W.normal_values(g, (S, H, D), DT) for _ in range(STEPS)]
    kpt, vpt = to_dev(kp, DT, dev), to_dev(vp, DT, dev)
    q_t, kn_t, vn_t = (to_dev(x[0], DT, dev) for x in (qs, kn, vn))
    out_t = torch.empty_like(q_t)
    scale = 1 / math.sqrt(D)
    st = pkv.DecodeStepper(a, [kpt], [vpt], [q_t], [kn_t], [vn_t], [out_t], scale, S, MB,
                           int(start.max()) + STEPS)
    if split is not None:
        st.set_xcd_split(split)
    seqs = np.arange(S, dtype=np.int64)
    outs = []
    for i in range(STEPS):
        q_t.copy_(to_dev(qs[i], DT, dev))
        kn_t.copy_(to_dev(kn[i], DT, dev))
        vn_t.copy_(to_dev(vn[i], DT, dev))
        st.step(seqs)
        torch.cuda.synchronize()      # the measurement is read at the next step's start
        outs.append(W.from_torch(out_t, DT).copy())
    used = st.xcd_split
    rates = st.xcd_rates()
    del st
    return outs, used, rates, (m, kp, vp, qs, kn, vn, seqs, MB, scale)


def _oracle_outputs(m, kp, vp, qs, kn, vn, seqs, MB, scale):
    S = len(seqs)
    ek, ev = kp, vp
    refs = []
    for i in range(STEPS):
        mslots, mpairs, _ = m.append_slots(seqs.tolist())
        assert not mpairs
        ek, ev = oracle.reshape_and_cache(kn[i], vn[i], ek, ev, np.array(mslots))
        lens = np.array([m.seq_len(int(s)) for s in seqs], np.int32)
        tables = np.full((S, MB), -1, np.int32)
        for j, s in enumerate(seqs):
            row = m.block_table(int(s))
            tables[j, :len(row)] = row
        refs.append(oracle.paged_attention_decode(qs[i], ek, ev, tables, lens, scale, DT))
    return refs


def test_outputs_do_not_depend_on_the_split():
    print(f"[xcd] batch lengths {_lengths(77).tolist()}", flush=True)
    base, used0, _, inputs = _run(0)
    assert used0 == 0
    refs = _oracle_outputs(*inputs)
    for i in range(STEPS):
        check_close(oracle.decode(base[i], DT), refs[i], DT, f"split 0 step {i}")
    for split in (384, 460, 600, 640, 1, 1023):
        print(f"[xcd] split {split}", flush=True)
        outs, used, _, _ = _run(split)
        assert used == split
        for i in range(STEPS):
            assert np.array_equal(outs[i].view(np.uint16), base[i].view(np.uint16)), (split, i)


def test_small_batch_is_not_measured():
    # 320 units fit on the chip at once: no measurement, the units stay evenly dealt
    _, used, (even, odd, outcome), _ = _run(None)
    assert used == 0 and outcome == pkv.PKV_XCD_NONE and even == 0 and odd == 0


def test_stepper_measures_the_split():
    outs, used, (even, odd, outcome), inputs = _run(None, seed=78, full=True)
    print(f"[xcd] measured split {used} of 1024 for the even XCDs; tokens per tick "
          f"even {even:.4f} odd {odd:.4f}; outcome {outcome}", flush=True)
    assert outcome in (pkv.PKV_XCD_MEASURED, pkv.PKV_XCD_UNMAPPED)
    assert used == 0 or 384 <= used <= 640
    if outcome == pkv.PKV_XCD_MEASURED:
        assert even > 0 and odd > 0
        expect = round(1024 * even / (even + odd))
        assert used == 0 or used == min(max(expect, 384), 640)
    refs = _oracle_outputs(*inputs)
    for i in range(STEPS):
        check_close(oracle.decode(outs[i], DT), refs[i], DT, f"measured split, step {i}")


def test_set_split_arguments():
    import torch
    dev = device()
    H, NB, MB = 8, 64, 4
    a = pkv.BlockAllocator(NB, BS)
    a.add_seq(0, 5)
    kp = torch.zeros((NB, H, BS, D), dtype=torch.float16, device=dev)
    vp = torch.zeros_like(kp)
    t = torch.zeros((1, H, D), dtype=torch.float16, device=dev)
    st = pkv.DecodeStepper(a, [kp], [vp], [t], [t.clone()], [t.clone()], [t.clone()], 0.1, 1,
                           MB, 64)
    assert st.xcd_split == 0
    for bad in (-2, 1024, 5000):
        with pytest.raises(pkv.PkvError):
            st.set_xcd_split(bad)
    st.set_xcd_split(700)
    assert st.xcd_split == 700
    st.set_xcd_split(-1)              # measure again: a one-unit batch is too small to tell
    st.step(np.zeros(1, np.int64))
    torch.cuda.synchronize()
    assert st.xcd_split == 700


def test_stand_alone_decode_takes_the_device_split():
    """pkv_paged_attention_decode (and _noalloc) deal their units by the device's split, and
    their outputs do not depend on it."""
    import torch
    dev = device()
    g = W.rng(91)
    H, S, MB = 40, 48, 128
    lens = g.integers(1, 2049, S).astype(np.int32)
    NB = int(sum(-(-int(L) // BS) for L in lens)) + 8
    kp = to_dev(W.normal_values(g, (NB, H, BS, D), DT), DT, dev)
    vp = to_dev(W.normal_values(g, (NB, H, BS, D), DT), DT, dev)
    q = to_dev(W.normal_values(g, (S, H, D), DT), DT, dev)
    tables = np.full((S, MB), 0, np.int32)
    perm = g.permutation(NB)
    used = 0
    for s, L in enumerate(lens.tolist()):
        nb = -(-L // BS)
        tables[s, :nb] = perm[used:used + nb]
        used += nb
    bt = torch.from_numpy(tables).to(dev)
    cl = torch.from_numpy(lens).to(dev)
    before = pkv.decode_xcd_split()
    assert 0 <= before < 1024
    outs = {}
    try:
        for split in (0, 600, 400):
            pkv.decode_set_xcd_split(split)
            assert pkv.decode_xcd_split() == split
            out = torch.empty_like(q)
            pkv.paged_attention_decode(out, q, kp, vp, bt, cl, 1 / math.sqrt(D), 2048)
            out2 = torch.empty_like(q)
            pkv.paged_attention_decode_noalloc(out2, q, kp, vp, bt, cl, 1 / math.sqrt(D), 2048)
            torch.cuda.synchronize()
            outs[split] = (W.from_torch(out, DT).copy(), W.from_torch(out2, DT).copy())
        with pytest.raises(pkv.PkvError):
            pkv.decode_set_xcd_split(1024)
    finally:
        pkv.decode_set_xcd_split(before)
    for split in (600, 400):
        for a, b in zip(outs[split], outs[0]):
            assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), split
    ref = oracle.paged_attention_decode(W.from_torch(q, DT), W.from_torch(kp, DT),
                                        W.from_torch(vp, DT), tables, lens, 1 / math.sqrt(D), DT)
    check_close(oracle.decode(outs[600][0], DT), ref, DT, "stand-alone decode, split 600")


def test_scheduled_shared_prefix_decode_takes_the_device_split():
    """The scheduled entry point with cache-allocating loads (shared prefixes, grouped work list,
    a few sequences split into partitions) deals its units by the device's split as well, with
    outputs that do not depend on it."""
    import torch
    dev = device()
    g = W.rng(93)
    H, groups, per = 40, 12, 4
    prefix = 32                                   # shared blocks of each group (512 tokens)
    S = groups * per
    tails = g.integers(0, 257, S)
    tails[:3] = g.integers(4000, 5000, 3)         # long enough to be split into partitions
    lens = (prefix * BS + tails).astype(np.int32)
    MB = int(-(-int(lens.max()) // BS))
    NB = groups * prefix + int(sum(-(-int(t) // BS) for t in tails)) + 8
    perm = g.permutation(NB)
    tables = np.zeros((S, MB), np.int32)
    used = 0
    for k in range(groups):
        shared = perm[used:used + prefix]
        used += prefix
        for j in range(per):
            s = k * per + j
            nb = -(-int(tails[s]) // BS)
            tables[s, :prefix] = shared
            tables[s, prefix:prefix + nb] = perm[used:used + nb]
            used += nb
    kp = to_dev(W.normal_values(g, (NB, H, BS, D), DT), DT, dev)
    vp = to_dev(W.normal_values(g, (NB, H, BS, D), DT), DT, dev)
    q = to_dev(W.normal_values(g, (S, H, D), DT), DT, dev)
    bt = torch.from_numpy(tables).to(dev)
    cl = torch.from_numpy(lens).to(dev)
    maxlen = int(lens.max())
    desc = pkv.desc_for_pool(kp)
    items = torch.from_numpy(pkv.decode_schedule(desc, lens, maxlen,
                                                 group_keys=np.arange(S) // per)).to(dev)
    scale = 1 / math.sqrt(D)
    before = pkv.decode_xcd_split()
    outs = {}
    try:
        for split in (0, 600, 400):
            print(f"[xcd] scheduled shared-prefix decode, split {split}", flush=True)
            pkv.decode_set_xcd_split(split)
            out = torch.empty_like(q)
            pkv.paged_attention_decode(out, q, kp, vp, bt, cl, scale, maxlen, work_items=items,
                                       shared_kv=True)
            torch.cuda.synchronize()
            outs[split] = W.from_torch(out, DT).copy()
    finally:
        pkv.decode_set_xcd_split(before)
    for split in (600, 400):
        assert np.array_equal(outs[split].view(np.uint16), outs[0].view(np.uint16)), split
    ref = oracle.paged_attention_decode(W.from_torch(q, DT), W.from_torch(kp, DT),
                                        W.from_torch(vp, DT), tables, lens, scale, DT)
    check_close(oracle.decode(outs[400], DT), ref, DT, "scheduled shared-prefix decode, split 400")
