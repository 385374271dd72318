"""Pins for the multi-query oracle (several new tokens of a sequence attend at once).

* a library reduction: with a contiguous block table every sequence is plain attention with
  the new tokens at the end of the context, so torch's scaled_dot_product_attention in
  float64 with an explicit position mask (token i sees positions 0 .. L-n+i) must agree;
* closed form: q = 0 gives uniform weights, so new token i returns the mean of V rows
  0 .. L-n+i -- the running means pin every query's extent;
* the last new token of a sequence sees the whole context, so it equals single-query decode
  (itself pinned in test_oracle_pins.py); a batch with one new token per sequence is decode;
* invariances: K/V of tokens after a query's position never change that query's output,
  NaN in slots no sequence uses is never read, placement in the pool does not matter;
* planted mistakes (no causal mask, a position off by one, top-left alignment of the mask,
  a wrong query row) each fail at least one pin.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _case(seed, H, D, BS, ctx, new, dtype="f32", contiguous=False, poison=True):
    g = W.rng(seed)
    ctx = np.asarray(ctx, np.int32)
    new = np.asarray(new, np.int32)
    assert (new <= ctx).all()
    qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    if contiguous:
        tables, nb = W.identity_block_tables(ctx, BS)
    else:
        tables, nb = W.permuted_block_tables(g, ctx, BS, pool_factor=1.5)
    q = W.normal_values(g, (int(qs[-1]), H, D), dtype)
    kp = W.normal_values(g, (nb, H, BS, D), dtype)
    vp = W.normal_values(g, (nb, H, BS, D), dtype)
    if poison:
        W.poison_unused(kp, tables, ctx, BS, dtype)
        W.poison_unused(vp, tables, ctx, BS, dtype)
    return q, kp, vp, tables, ctx, qs


def pin_mq_library_reduction(impl):
    """Contiguous table -> torch SDPA (float64, CPU) with a bottom-right aligned mask."""
    H, D, BS = 3, 16, 4
    ctx, new = (9, 5, 13, 4), (4, 5, 1, 0)
    q, kp, vp, tables, ctx, qs = _case(21, H, D, BS, ctx, new, contiguous=True)
    scale = 0.4
    out = impl(q, kp, vp, tables, ctx, qs, scale, "f32")
    for s in range(len(ctx)):
        L, n = int(ctx[s]), int(qs[s + 1] - qs[s])
        if n == 0:
            continue
        nb = -(-L // BS)
        blocks = tables[s, :nb]
        K = kp[blocks].transpose(1, 0, 2, 3).reshape(H, nb * BS, D)[:, :L]
        V = vp[blocks].transpose(1, 0, 2, 3).reshape(H, nb * BS, D)[:, :L]
        mask = np.arange(L)[None, :] <= (L - n + np.arange(n))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[qs[s]:qs[s + 1]].transpose(1, 0, 2).astype(np.float64)),
            torch.from_numpy(K.astype(np.float64)), torch.from_numpy(V.astype(np.float64)),
            attn_mask=torch.from_numpy(mask), scale=float(np.float32(scale)))
        np.testing.assert_allclose(out[qs[s]:qs[s + 1]], ref.numpy().transpose(1, 0, 2),
                                   rtol=0, atol=1e-12)


def pin_mq_running_means(impl):
    """q = 0: new token i returns the mean of V rows 0 .. L-n+i (read through the table)."""
    H, D, BS = 2, 6, 4
    ctx, new = (11, 6, 3), (3, 6, 1)
    q, kp, vp, tables, ctx, qs = _case(22, H, D, BS, ctx, new)
    q[:] = 0
    out = impl(q, kp, vp, tables, ctx, qs, 1.0, "f32")
    for s in range(len(ctx)):
        L, n = int(ctx[s]), int(qs[s + 1] - qs[s])
        rows = np.stack([vp[tables[s, t // BS], :, t % BS].astype(np.float64) for t in range(L)])
        for i in range(n):
            want = rows[:L - n + i + 1].mean(axis=0)
            np.testing.assert_allclose(out[qs[s] + i], want, rtol=0, atol=1e-12)


def pin_mq_last_token_is_decode(impl):
    """The last new token sees the whole context: single-query decode at length L.  With one
    new token per sequence the whole batch is decode."""
    H, D, BS = 2, 8, 4
    ctx, new = (7, 12, 5), (3, 12, 2)
    q, kp, vp, tables, ctx, qs = _case(23, H, D, BS, ctx, new)
    out = impl(q, kp, vp, tables, ctx, qs, 0.6, "f32")
    last = q[qs[1:] - 1]
    dec = oracle.paged_attention_decode(last, kp, vp, tables, ctx, 0.6, "f32")
    np.testing.assert_allclose(out[qs[1:] - 1], dec, rtol=0, atol=1e-12)
    ones = np.ones(len(ctx), np.int32)
    q1, kp1, vp1, tables1, ctx1, qs1 = _case(24, H, D, BS, ctx, ones)
    out1 = impl(q1, kp1, vp1, tables1, ctx1, qs1, 0.6, "f32")
    dec1 = oracle.paged_attention_decode(q1, kp1, vp1, tables1, ctx1, 0.6, "f32")
    np.testing.assert_allclose(out1, dec1, rtol=0, atol=1e-12)


def pin_mq_future_is_never_seen(impl):
    """Changing the K/V of positions after a query's own changes nothing for that query and
    does change the queries that see them."""
    H, D, BS = 2, 8, 4
    ctx, new = (10,), (6,)
    q, kp, vp, tables, ctx, qs = _case(25, H, D, BS, ctx, new, poison=False)
    out = impl(q, kp, vp, tables, ctx, qs, 0.5, "f32")
    t = 7                                   # position of new token 3 is 10 - 6 + 3 = 7
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[tables[0, t // BS], :, t % BS] += 1.5
    vp2[tables[0, t // BS], :, t % BS] -= 2.0
    out2 = impl(q, kp2, vp2, tables, ctx, qs, 0.5, "f32")
    assert np.array_equal(out[:3], out2[:3])
    assert not np.allclose(out[3:], out2[3:], rtol=0, atol=1e-6)


def pin_mq_poison_and_placement(impl):
    """NaN in unused slots is never read; the same logical KV placed twice gives identical
    outputs."""
    H, D, BS = 2, 8, 4
    ctx = np.array([6, 13], np.int32)
    new = np.array([2, 5], np.int32)
    qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    g = W.rng(26)
    q = W.normal_values(g, (int(qs[-1]), H, D), "f32")
    lk = [W.normal_values(g, (int(L), H, D), "f32") for L in ctx]
    lv = [W.normal_values(g, (int(L), H, D), "f32") for L in ctx]
    outs = []
    for seed in (1, 2):
        tables, nb = W.permuted_block_tables(W.rng(seed), ctx, BS, pool_factor=3.0)
        kp = np.zeros((nb, H, BS, D), np.float32)
        vp = np.zeros((nb, H, BS, D), np.float32)
        for s, L in enumerate(ctx):
            for t in range(L):
                kp[tables[s, t // BS], :, t % BS] = lk[s][t]
                vp[tables[s, t // BS], :, t % BS] = lv[s][t]
        W.poison_unused(kp, tables, ctx, BS, "f32")
        W.poison_unused(vp, tables, ctx, BS, "f32")
        outs.append(impl(q, kp, vp, tables, ctx, qs, 0.45, "f32"))
    assert np.isfinite(outs[0]).all()
    assert np.array_equal(outs[0], outs[1])


MQ_PINS = [pin_mq_library_reduction, pin_mq_running_means, pin_mq_last_token_is_decode,
           pin_mq_future_is_never_seen, pin_mq_poison_and_placement]


@pytest.mark.parametrize("pin", MQ_PINS, ids=lambda p: p.__name__)
def test_multi_query_oracle_pins(pin):
    pin(oracle.paged_attention_multi_query)


def test_multi_query_rows_and_empty_sequences():
    H, D, BS = 1, 4, 4
    q, kp, vp, tables, ctx, qs = _case(27, H, D, BS, (5, 0, 3), (2, 0, 3))
    out = oracle.paged_attention_multi_query(q, kp, vp, tables, ctx, qs, 1.0, "f32")
    assert out.shape == (5, H, D) and np.isfinite(out).all()
    assert [oracle.query_position(ctx, qs, 0, i) for i in range(2)] == [3, 4]
    assert [oracle.query_position(ctx, qs, 2, i) for i in range(3)] == [0, 1, 2]
    with pytest.raises(AssertionError):
        oracle.query_position(ctx, qs, 1, 0)


# ============================================================================ planted mistakes
def _mq_mutant(kind):
    """A copy of the multi-query oracle with one plausible mistake planted in it."""
    def impl(q, k_pool, v_pool, block_tables, context_lens, query_start, scale, dtype):
        T, H, D = q.shape
        BS = k_pool.shape[2]
        out = np.zeros((T, H, D))
        for s in range(len(context_lens)):
            L = int(context_lens[s])
            n = int(query_start[s + 1] - query_start[s])
            for i in range(n):
                P = L - n + i
                if kind == "no_causal_mask":
                    P = L - 1
                elif kind == "position_low":
                    P = max(L - n + i - 1, 0)
                elif kind == "position_high":
                    P = min(L - n + i + 1, L - 1)
                elif kind == "top_left_mask":
                    P = i
                row = int(query_start[s]) + i
                if kind == "query_row_unpacked":
                    row = min(s * n + i, T - 1)
                t = np.arange(P + 1)
                blk = block_tables[s][t // BS]
                for h in range(H):
                    K = oracle.decode(k_pool[blk, h, t % BS, :], dtype)
                    V = oracle.decode(v_pool[blk, h, t % BS, :], dtype)
                    z = float(np.float32(scale)) * (K @ oracle.decode(q[row, h], dtype))
                    w = np.exp(z - z.max())
                    out[int(query_start[s]) + i, h] = (w @ V) / w.sum()
        return out
    return impl


@pytest.mark.parametrize("kind", ["no_causal_mask", "position_low", "position_high",
                                  "top_left_mask", "query_row_unpacked"])
def test_multi_query_planted_mistakes_fail_a_pin(kind):
    impl = _mq_mutant(kind)
    caught = 0
    for pin in MQ_PINS:
        try:
            pin(impl)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"no pin catches {kind}"


def test_multi_query_unplanted_mutant_passes_every_pin():
    for pin in MQ_PINS:
        pin(_mq_mutant("none"))
