"""Pins for the float64 oracle: each check ties it to something other than itself.

* the pages' worked examples (tests/golden/, each with its citation);
* the IEEE binary16 / bfloat16 field definitions and numpy's own float16;
* a library reduction: with a contiguous (identity) block table paged attention is plain
  attention, so torch's scaled_dot_product_attention in float64 on the CPU must agree;
* closed forms (one token, two tokens as a logistic weight, q = 0, a dominant key);
* invariances the pages state (placement anywhere, block-size choice, shared prefix, poison
  in slots no sequence uses);
* planted mistakes: mutated copies of the oracle must fail at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ============================================================================ storage
def test_storage_golden_values():
    g = golden("storage_formats.json")
    for hexbits, val in g["f16"]:
        got = oracle.decode_bits_f16(np.array([int(hexbits, 16)], np.uint16))[0]
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), hexbits
    for hexbits, val in g["bf16"]:
        got = oracle.decode_bits_bf16(np.array([int(hexbits, 16)], np.uint16))[0]
        assert got == float(val), hexbits


def test_f16_decode_matches_numpy_on_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bits_f16(bits)
    ref = bits.view(np.float16).astype(np.float64)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_decode_matches_field_formula_on_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32)
    ours = oracle.decode_bits_bf16(bits.astype(np.uint16))
    sign = np.where(bits >> 15, -1.0, 1.0)
    e = ((bits >> 7) & 0xFF).astype(np.int64)
    f = (bits & 0x7F).astype(np.float64)
    with np.errstate(over="ignore"):
        ref = np.where(e == 0, sign * np.ldexp(f, -133),
                       sign * np.ldexp(1 + f / 128.0, e - 127))
    ref = np.where(e == 255, np.where(f == 0, sign * np.inf, np.nan), ref)
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_generator_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125 -> even (1.0);
    # 1 + 3*2^-8 is halfway between 1.0078125 and 1.015625 -> even (1.015625).
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20], np.float32)
    got = oracle.decode_bits_bf16(W.f32_to_storage(x, "bf16"))
    assert got.tolist() == [1.0, 1.015625, 1.0078125]


# ============================================================================ gather
def test_gather_follows_page_table_worked_example():
    g = golden("page_table_47_123.json")
    BS = g["block_size"]
    H, D, NB = 2, 3, 200
    # every element records (block, head, slot, dim) so a wrong index shows up
    pool = np.zeros((NB, H, BS, D), np.float32)
    b, h, o, d = np.indices(pool.shape)
    pool[...] = b * 1e4 + h * 1e3 + o * 10 + d
    table = np.array(g["table"], np.int32)
    rows = oracle.gather_sequence(pool, table, 2 * BS, 1, BS)
    for t, blk, slot in g["token_block_slot"]:
        assert rows[t].tolist() == [blk * 1e4 + 1e3 + slot * 10 + dd for dd in range(D)]


# ============================================================================ attention pins
def _random_case(seed, S=3, H=2, D=8, BS=4, lens=(1, 5, 13), dtype="f32", contiguous=False):
    g = W.rng(seed)
    lens = np.array(lens, np.int32)
    if contiguous:
        tables, nb = W.identity_block_tables(lens, BS)
    else:
        tables, nb = W.permuted_block_tables(g, lens, BS, pool_factor=2.0)
    q = W.normal_values(g, (S, H, D), dtype)
    kp = W.normal_values(g, (nb, H, BS, D), dtype)
    vp = W.normal_values(g, (nb, H, BS, D), dtype)
    return q, kp, vp, tables, lens


def pin_library_reduction(impl):
    """Identity block table -> torch SDPA (float64, CPU) on the contiguous K/V."""
    import torch
    S, H, D, BS = 3, 5, 16, 4
    lens = (7, 1, 22)
    q, kp, vp, tables, lens = _random_case(11, S, H, D, BS, lens, contiguous=True)
    scale = 0.3
    out = impl(q, kp, vp, tables, lens, scale, "f32")
    for s in range(S):
        L = int(lens[s])
        nb = -(-L // BS)
        blocks = tables[s, :nb]
        K = kp[blocks].transpose(1, 0, 2, 3).reshape(H, nb * BS, D)[:, :L]
        V = vp[blocks].transpose(1, 0, 2, 3).reshape(H, nb * BS, D)[:, :L]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[s].astype(np.float64))[:, None, :],
            torch.from_numpy(K.astype(np.float64)),
            torch.from_numpy(V.astype(np.float64)), scale=float(np.float32(scale)))
        np.testing.assert_allclose(out[s], ref[:, 0, :].numpy(), rtol=0, atol=1e-12)


def pin_closed_forms(impl):
    D, BS, H = 6, 4, 1
    g = W.rng(5)
    # one token -> out = v0 exactly
    q, kp, vp, tables, lens = _random_case(3, 1, H, D, BS, (1,))
    out = impl(q, kp, vp, tables, lens, 0.7, "f32")
    assert np.array_equal(out[0, 0], vp[tables[0, 0], 0, 0].astype(np.float64))
    # two tokens -> out = v1 + (v0 - v1) * logistic(z0 - z1)
    q, kp, vp, tables, lens = _random_case(4, 1, H, D, BS, (2,))
    sc = float(np.float32(0.9))
    qq = q[0, 0].astype(np.float64)
    b0 = tables[0, 0]
    k0, k1 = kp[b0, 0, 0].astype(np.float64), kp[b0, 0, 1].astype(np.float64)
    v0, v1 = vp[b0, 0, 0].astype(np.float64), vp[b0, 0, 1].astype(np.float64)
    dz = sc * (sum(qq[i] * (k0[i] - k1[i]) for i in range(D)))
    want = v1 + (v0 - v1) / (1.0 + math.exp(-dz))
    out = impl(q, kp, vp, tables, lens, 0.9, "f32")
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-12)
    # q = 0 -> uniform weights -> mean of the V rows
    q, kp, vp, tables, lens = _random_case(6, 1, H, D, BS, (11,))
    q[:] = 0
    out = impl(q, kp, vp, tables, lens, 1.0, "f32")
    rows = [vp[tables[0, t // BS], 0, t % BS].astype(np.float64) for t in range(11)]
    np.testing.assert_allclose(out[0, 0], np.mean(rows, axis=0), rtol=0, atol=1e-12)
    # a dominant key (score gap > 40) -> out = its value row within e^-40
    q, kp, vp, tables, lens = _random_case(7, 1, H, D, BS, (9,))
    q[0, 0] = 0
    q[0, 0, 0] = 1
    kp[...] = 0
    t_dom = 6
    kp[tables[0, t_dom // BS], 0, t_dom % BS, 0] = 50.0
    out = impl(q, kp, vp, tables, lens, 1.0, "f32")
    want = vp[tables[0, t_dom // BS], 0, t_dom % BS].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-15)


def pin_shift_and_scale_of_v(impl):
    """out(a*V + c) = a*out(V) + c: the weights are a normalised distribution."""
    q, kp, vp, tables, lens = _random_case(8, 2, 2, 8, 4, (6, 10))
    # V on a grid of eighths so that 2 V + 3 is exact in binary32
    vp = (np.rint(vp * 8) / 8).astype(np.float32)
    out = impl(q, kp, vp, tables, lens, 0.5, "f32")
    vp2 = vp * np.float32(2.0) + np.float32(3.0)
    out2 = impl(q, kp, vp2, tables, lens, 0.5, "f32")
    np.testing.assert_allclose(out2, 2.0 * out + 3.0, rtol=0, atol=1e-12)


def pin_placement_invariance(impl):
    """The same logical KV placed anywhere in the pool gives bit-identical outputs."""
    S, H, D, BS = 3, 2, 8, 4
    lens = np.array([3, 9, 16], np.int32)
    g = W.rng(9)
    q = W.normal_values(g, (S, H, D), "f32")
    logical_k = [W.normal_values(g, (int(L), H, D), "f32") for L in lens]
    logical_v = [W.normal_values(g, (int(L), H, D), "f32") for L in lens]
    outs = []
    for seed in (1, 2, 3):
        tables, nb = W.permuted_block_tables(W.rng(seed), lens, BS, pool_factor=3.0)
        kp = np.zeros((nb, H, BS, D), np.float32)
        vp = np.zeros((nb, H, BS, D), np.float32)
        for s, L in enumerate(lens):
            for t in range(L):
                kp[tables[s, t // BS], :, t % BS] = logical_k[s][t]
                vp[tables[s, t // BS], :, t % BS] = logical_v[s][t]
        outs.append(impl(q, kp, vp, tables, lens, 0.35, "f32"))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # and equals attention over the logical rows directly
    for s, L in enumerate(lens):
        for h in range(H):
            want = oracle.attend(q[s, h].astype(np.float64), logical_k[s][:, h].astype(np.float64),
                                 logical_v[s][:, h].astype(np.float64), float(np.float32(0.35)))
            assert np.array_equal(outs[0][s, h], want)


def pin_block_size_invariance(impl):
    """The same logical KV stored with block sizes 8, 16, 32 gives bit-identical outputs."""
    S, H, D = 2, 2, 8
    lens = np.array([37, 70], np.int32)
    g = W.rng(10)
    q = W.normal_values(g, (S, H, D), "f16")
    lk = [W.normal_values(g, (int(L), H, D), "f16") for L in lens]
    lv = [W.normal_values(g, (int(L), H, D), "f16") for L in lens]
    outs = []
    for BS in (8, 16, 32):
        tables, nb = W.permuted_block_tables(W.rng(BS), lens, BS)
        kp = np.zeros((nb, H, BS, D), np.float16)
        vp = np.zeros((nb, H, BS, D), np.float16)
        for s, L in enumerate(lens):
            for t in range(L):
                kp[tables[s, t // BS], :, t % BS] = lk[s][t]
                vp[tables[s, t // BS], :, t % BS] = lv[s][t]
        outs.append(impl(q, kp, vp, tables, lens, 0.25, "f16"))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def pin_poison_is_never_read(impl):
    """NaN in blocks no table references and in slots past each length changes nothing."""
    q, kp, vp, tables, lens = _random_case(12, 3, 2, 8, 4, (2, 7, 12))
    out = impl(q, kp, vp, tables, lens, 0.5, "f32")
    kp2, vp2 = kp.copy(), vp.copy()
    W.poison_unused(kp2, tables, lens, 4, "f32")
    W.poison_unused(vp2, tables, lens, 4, "f32")
    assert np.isnan(kp2).any()
    out2 = impl(q, kp2, vp2, tables, lens, 0.5, "f32")
    assert np.array_equal(out, out2)


PINS = [pin_library_reduction, pin_closed_forms, pin_shift_and_scale_of_v,
        pin_placement_invariance, pin_block_size_invariance, pin_poison_is_never_read]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_attention_pins(pin):
    pin(oracle.paged_attention_decode)


def test_zero_length_is_zero_vector():
    q, kp, vp, tables, lens = _random_case(13, 2, 2, 8, 4, (0, 3))
    out = oracle.paged_attention_decode(q, kp, vp, tables, lens, 1.0, "f32")
    assert np.array_equal(out[0], np.zeros((2, 8)))


def test_bf16_and_f16_read_stored_values():
    """The oracle reads the stored (rounded) values: a one-token sequence returns the stored
    V row exactly in every storage type."""
    for dt in ("f16", "bf16"):
        q, kp, vp, tables, lens = _random_case(14, 1, 1, 8, 4, (1,), dtype=dt)
        out = oracle.paged_attention_decode(q, kp, vp, tables, lens, 1.0, dt)
        assert np.array_equal(out[0, 0], oracle.decode(vp[tables[0, 0], 0, 0], dt))


# ============================================================================ planted mistakes
def _mutant(kind):
    """A copy of the oracle's decode with one plausible mistake planted in it."""
    def impl(q, k_pool, v_pool, block_tables, context_lens, scale, dtype, units=None):
        S, H, D = q.shape
        BS = k_pool.shape[2]
        out = np.zeros((S, H, D))
        for s in range(S):
            L = int(context_lens[s])
            for h in range(H):
                t = np.arange(L)
                if kind == "block_index_off_by_one":
                    blk = block_tables[s][np.minimum((t + 1) // BS, max(0, (L - 1) // BS))]
                else:
                    blk = block_tables[s][t // BS]
                off = t % BS
                if kind == "slot_from_block_count":
                    off = (t // BS) % BS
                K = oracle.decode(k_pool[blk, h, off, :], dtype)
                V = oracle.decode(v_pool[blk, h, off, :], dtype)
                if kind == "k_for_v":
                    V = K
                qq = oracle.decode(q[s, h], dtype)
                sc = float(np.float32(scale))
                if kind == "no_scale":
                    sc = 1.0
                if L == 0:
                    continue
                z = sc * (K @ qq)
                if kind == "drop_last_token":
                    z, V = z[:-1] if L > 1 else z, V[:-1] if L > 1 else V
                w = np.exp(z - z.max())
                if kind == "no_normalise":
                    out[s, h] = w @ V
                else:
                    out[s, h] = (w @ V) / w.sum()
        return out
    return impl


@pytest.mark.parametrize("kind", ["block_index_off_by_one", "slot_from_block_count", "k_for_v",
                                  "no_scale", "drop_last_token", "no_normalise"])
def test_planted_mistakes_fail_a_pin(kind):
    impl = _mutant(kind)
    caught = 0
    for pin in PINS:
        try:
            pin(impl)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin catches {kind}"


def test_unplanted_mutant_copy_passes_every_pin():
    # the mutation harness itself is sound: with no mistake planted, every pin passes
    for pin in PINS:
        pin(_mutant("none"))


# ============================================================================ cache ops
def test_reshape_and_cache_writes_only_its_slots():
    g = W.rng(20)
    NB, H, BS, D, N = 9, 3, 4, 8, 5
    kp = W.normal_values(g, (NB, H, BS, D), "bf16")
    vp = W.normal_values(g, (NB, H, BS, D), "bf16")
    k = W.normal_values(g, (N, H, D), "bf16")
    v = W.normal_values(g, (N, H, D), "bf16")
    slots = np.array([5, -1, 35, 0, 17], np.int32)
    kp2, vp2 = oracle.reshape_and_cache(k, v, kp, vp, slots)
    changed = {(int(s) // BS, int(s) % BS) for s in slots if s >= 0}
    for b in range(NB):
        for o in range(BS):
            if (b, o) in changed:
                continue
            assert np.array_equal(kp2[b, :, o], kp[b, :, o])
            assert np.array_equal(vp2[b, :, o], vp[b, :, o])
    # the written token reads back through a table that points at its block
    for i, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kp2[s // BS, :, s % BS], k[i])
        assert np.array_equal(vp2[s // BS, :, s % BS], v[i])
    # the worked page-table example: token 16 lands in block 123, slot 0
    g2 = golden("page_table_47_123.json")
    big = np.zeros((130, 1, 16, 2), np.float16)
    kk = np.ones((1, 1, 2), np.float16)
    slot = g2["table"][1] * 16 + 0
    kb, _ = oracle.reshape_and_cache(kk, kk, big, big, np.array([slot]))
    rows = oracle.gather_sequence(kb, np.array(g2["table"]), 17, 0, 16)
    assert rows[16].tolist() == [1.0, 1.0] and not rows[:16].any()


def test_reshape_and_cache_keeps_nan_payloads():
    kp = np.zeros((2, 1, 2, 2), np.float16)
    k = np.array([[[0x7E01, 0xFC01]]], np.uint16).view(np.float16)
    kp2, _ = oracle.reshape_and_cache(k, k, kp, kp, np.array([3]))
    assert kp2.view(np.uint16)[1, 0, 1].tolist() == [0x7E01, 0xFC01]


def test_copy_blocks_copies_bits_in_every_layer():
    g = W.rng(21)
    pools = [W.normal_values(g, (6, 2, 4, 8), "f16") for _ in range(3)]
    pairs = np.array([[1, 4], [2, 5]], np.int32)
    out = oracle.copy_blocks(pools, pairs)
    for p, o in zip(pools, out):
        assert np.array_equal(o[4], p[1]) and np.array_equal(o[5], p[2])
        for b in (0, 1, 2, 3):
            assert np.array_equal(o[b], p[b])
    with pytest.raises(AssertionError):
        oracle.copy_blocks(pools, np.array([[1, 2], [2, 3]]))


def test_shared_prefix_outputs_equal_before_and_after_copy():
    """Sequences sharing prefix blocks, with the same q and tail, attend identically; copying a
    shared block to a fresh one and repointing one table changes nothing."""
    g = W.rng(22)
    H, D, BS = 2, 8, 4
    tables, lens, nb = W.shared_prefix_tables(g, 1, 3, 10, np.array([0, 0, 0]), BS)
    kp = W.normal_values(g, (nb + 2, H, BS, D), "f16")
    vp = W.normal_values(g, (nb + 2, H, BS, D), "f16")
    # make the private last blocks identical across the three sequences
    last = tables[:, 2]
    kp[last[1:]] = kp[last[0]]
    vp[last[1:]] = vp[last[0]]
    q = np.repeat(W.normal_values(g, (1, H, D), "f16"), 3, axis=0)
    out = oracle.paged_attention_decode(q, kp, vp, tables, lens, 0.5, "f16")
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])
    src = int(tables[1, 0])
    dst = nb  # an unused block
    kc, vc = oracle.copy_blocks([kp, vp], [[src, dst]])
    t2 = tables.copy()
    t2[1, 0] = dst
    out2 = oracle.paged_attention_decode(q, kc, vc, t2, lens, 0.5, "f16")
    assert np.array_equal(out, out2)


# ============================================================================ block manager
def test_block_manager_memory_efficiency_example():
    g = golden("memory_efficiency_100_tokens.json")
    bm = oracle.BlockManager(64, g["block_size"], free_order=W.rng(1).permutation(64))
    bm.add_seq(0, 0)
    for _ in range(g["tokens"]):
        bm.append_slot(0)
    assert len(bm.block_table(0)) == g["blocks"]
    assert len(bm.block_table(0)) * g["block_size"] == g["allocated_slots"]
    assert bm.wasted_slots() == g["wasted_slots"]
    bm2 = oracle.BlockManager(64, g["block_size"])
    bm2.add_seq(7, g["tokens"])
    assert len(bm2.block_table(7)) == g["blocks"] and bm2.wasted_slots() == g["wasted_slots"]


def test_block_manager_page_table_example():
    g = golden("page_table_47_123.json")
    order = list(g["table"]) + [b for b in range(200) if b not in g["table"]]
    bm = oracle.BlockManager(200, g["block_size"], free_order=order)
    bm.add_seq(0, 0)
    slots = [bm.append_slot(0)[0] for _ in range(32)]
    assert bm.block_table(0) == g["table"]
    for t, blk, slot in g["token_block_slot"]:
        assert slots[t] == blk * g["block_size"] + slot


def _invariants(bm):
    refs = [0] * bm.num_blocks
    for t in bm.tables.values():
        for b in t:
            refs[b] += 1
    assert refs == bm.ref
    used = sum(1 for r in bm.ref if r > 0)
    assert used + bm.num_free() == bm.num_blocks


def test_block_manager_fork_and_copy_on_write():
    BS = 4
    bm = oracle.BlockManager(32, BS)
    bm.add_seq(0, 10)            # blocks 0,1,2 ; last block holds 2 of 4
    for c in (1, 2, 3):
        bm.fork(0, c)
    _invariants(bm)
    assert [bm.ref[b] for b in bm.block_table(0)] == [4, 4, 4]
    # first three writers into the shared partial block copy it; the last writes in place
    pairs = []
    for s in (1, 2, 3, 0):
        slot, cow = bm.append_slot(s)
        pairs.append(cow)
        _invariants(bm)
        assert slot % BS == 2
    assert [p is not None for p in pairs] == [True, True, True, False]
    assert {p[0] for p in pairs[:3]} == {2}
    assert bm.block_table(0)[2] == 2 and bm.ref[2] == 1
    # the full prefix blocks stay shared
    assert bm.ref[0] == 4 and bm.ref[1] == 4


def test_block_manager_aligned_prefix_needs_no_copy():
    bm = oracle.BlockManager(64, 16)
    bm.add_seq(0, 512 - 480)     # 2 full blocks
    for c in range(1, 8):
        bm.fork(0, c)
    slots, pairs, n = bm.append_slots(list(range(8)))
    assert n == 8 and pairs == []
    assert len(set(slots)) == 8
    _invariants(bm)


def test_block_manager_free_and_out_of_blocks():
    bm = oracle.BlockManager(4, 2)
    bm.add_seq(0, 5)             # 3 blocks
    with pytest.raises(oracle.OutOfBlocks):
        bm.add_seq(1, 3)
    assert 1 not in bm.tables and bm.num_free() == 1
    bm.append_slot(0)            # token 5 fills block 2
    bm.append_slot(0)            # token 6 takes the last free block
    bm.append_slot(0)            # token 7 fills it
    with pytest.raises(oracle.OutOfBlocks):
        bm.append_slot(0)        # token 8 would need a fifth block
    assert bm.seq_len(0) == 8 and bm.num_free() == 0
    bm.free_seq(0)
    assert bm.num_free() == 4 and bm.wasted_slots() == 0
    # freed blocks come back in logical order
    bm.add_seq(5, 8)
    assert bm.block_table(5) == [0, 1, 2, 3]
    with pytest.raises(ValueError):
        bm.free_seq(99)


# ============================================================================ prefix cache
def test_prefix_cache_model_follows_the_pages_pattern():
    """"Prefix Caching": the first request with a system prompt computes and caches its KV
    blocks; later requests with the same prompt reuse them and skip recomputing; another
    prompt shares nothing; only full blocks are cached."""
    BS = 4
    bm = oracle.BlockManager(40, BS)
    system = list(range(100, 112))                     # 3 full blocks
    assert bm.add_seq_cached(1, system + [7, 8]) == 0  # first request: nothing cached yet
    assert bm.num_cached() == 3                        # the partial 4th block is not cached
    assert bm.add_seq_cached(2, system + [9]) == 12    # second request reuses 3 blocks
    assert bm.block_table(2)[:3] == bm.block_table(1)[:3]
    assert bm.block_table(2)[3] != bm.block_table(1)[3]
    assert [bm.ref[b] for b in bm.block_table(1)[:3]] == [2, 2, 2]
    # same tokens after a different first block are a different prefix
    other = [555, 556, 557, 558] + system[4:]
    assert bm.add_seq_cached(3, other) == 0
    # a prompt diverging inside block 2 reuses blocks 0 and 1 only
    assert bm.add_seq_cached(4, system[:8] + [0, 0, 0, 0]) == 8
    _invariants(bm)


def test_prefix_cache_parks_then_evicts_oldest():
    BS = 2
    bm = oracle.BlockManager(6, BS)
    bm.add_seq_cached(1, [1, 2, 3, 4])        # blocks cached: (1,2), (3,4)
    bm.add_seq_cached(2, [5, 6])              # (5,6)
    bm.free_seq(1)                            # parks (3,4) then (1,2) (reverse logical order)
    bm.free_seq(2)                            # parks (5,6)
    assert bm.num_free() == 6 and bm.num_cached() == 3
    assert bm.add_seq_cached(3, [1, 2, 3, 4]) == 4   # hit on parked blocks revives them
    assert bm.num_cached() == 3 and list(bm.parked) == [bm.cache[(0, (5, 6))]]
    bm.add_seq(4, 6)   # 3 plain free blocks are used first: nothing evicted
    assert bm.num_cached() == 3
    bm.add_seq(5, 1)   # now the parked (5,6) block is evicted
    assert bm.num_cached() == 2 and (0, (5, 6)) not in bm.cache
    with pytest.raises(oracle.OutOfBlocks):
        bm.add_seq(6, 1)
    _invariants(bm)


# ============================================================================ swapping
def test_swap_model_moves_groups_and_keeps_sharing():
    """Preemption by swapping ("vLLM: The Serving Engine": swap KV to CPU when the GPU is
    full, resume later): a group moved out and back keeps its token-to-slot structure, its
    shared blocks stay shared, and a partial group is refused."""
    BS = 4
    gpu = oracle.BlockManager(20, BS, free_order=W.rng(3).permutation(20))
    cpu = oracle.BlockManager(12, BS)
    gpu.add_seq(1, 10)
    gpu.fork(1, 2)
    gpu.append_slot(2)                         # copy-on-write of the shared partial block
    gpu.add_seq(3, 5)
    with pytest.raises(ValueError):
        gpu.move_seqs(cpu, [1])                # block 0/1 still shared with seq 2
    before = {s: gpu.block_table(s) for s in (1, 2)}
    out = gpu.move_seqs(cpu, [1, 2])
    assert len(out) == 4                       # 2 shared + 2 private last blocks
    assert [cpu.ref[d] for _, d in out[:2]] == [2, 2]
    assert gpu.num_free() == 20 - len(gpu.block_table(3)) and 1 not in gpu.tables
    fwd = dict(out)
    for s in (1, 2):
        assert cpu.block_table(s) == [fwd[b] for b in before[s]]
        assert cpu.seq_len(s) == (10 if s == 1 else 11)
    back = cpu.move_seqs(gpu, [1, 2])
    bwd = dict(back)
    # the composite map old gpu block -> new gpu block is one-to-one on the moved blocks
    composite = {b: bwd[fwd[b]] for b in fwd}
    assert len(set(composite.values())) == len(composite)
    for s in (1, 2):
        assert gpu.block_table(s) == [composite[b] for b in before[s]]
    _invariants(gpu)
    _invariants(cpu)
    assert cpu.num_free() == 12


def test_swap_blocks_copies_across_pools():
    g = W.rng(33)
    src = [W.normal_values(g, (6, 2, 4, 8), "bf16") for _ in range(2)]
    dst = [W.normal_values(g, (3, 2, 4, 8), "bf16") for _ in range(2)]
    out = oracle.swap_blocks(src, dst, [[5, 0], [1, 2]])
    for s, d, o in zip(src, dst, out):
        assert np.array_equal(o[0], s[5]) and np.array_equal(o[2], s[1])
        assert np.array_equal(o[1], d[1])
