"""Helpers for the GPU parity tests: move seeded inputs to the device, call the HIP path
through the binding, and evaluate the oracle on the stored values."""
import os

import numpy as np

import oracle
import workloads as W

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}


def device():
    import pytest
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def to_dev(arr, dtype, dev):
    return W.to_torch(arr, dtype).to(dev)


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (x float64)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 7)


# mantissa bits and smallest normal exponent of each output type
_FORMAT = {"f32": (23, -126), "f16": (10, -14), "bf16": (7, -126)}


def ulp(x, dtype):
    """Spacing of the output type's numbers at |x| (x float64); subnormal spacing below the
    smallest normal."""
    bits, emin = _FORMAT[dtype]
    ax = np.maximum(np.abs(x), 2.0 ** emin)
    return np.exp2(np.floor(np.log2(ax)) - bits)


def round_to(x, dtype):
    """x (float64) rounded to the nearest number of the output type, ties to even: exact,
    since x / ulp(x) is an exact float64 and numpy's round takes ties to even (|x| stays far
    below the output types' overflow thresholds here)."""
    x = np.asarray(x, np.float64)
    u = ulp(x, dtype)
    return np.round(x / u) * u


def kernel_error(got64, ref64, dtype):
    """Per element: how far the oracle lies from the set of reals that round to the GPU's
    output, i.e. the error of the kernel's result before its final rounding to the output
    type (0 when the output is the correctly rounded oracle)."""
    g = np.abs(got64)
    above = ulp(g, dtype) / 2                      # half the spacing above |g|
    below = ulp(g * (1 - 2.0 ** -30), dtype) / 2   # half the spacing below |g| (a binade edge halves it)
    below = np.where(g == 0, above, below)
    lo = np.where(got64 >= 0, got64 - below, got64 - above)
    hi = np.where(got64 >= 0, got64 + above, got64 + below)
    return np.maximum(0.0, np.maximum(lo - ref64, ref64 - hi))


# (test, dtype, elements, max abs error, max error in output ulps, max kernel error, fraction
# equal to the rounded oracle) of every check_close in the session; tests/conftest.py prints
# them per test at the end of the run.  The ulp is taken at the larger of |ref| and the checked
# outputs' RMS, so outputs near zero (where any absolute error is many of their own ulps) are
# measured at the outputs' scale.
REPORT = []


def check_close(got64, ref64, dtype, what=""):
    """|got - ref| <= the stated bound: 1e-5 (f32) or 2e-3 (f16 / bf16).  Where a bfloat16
    output's own spacing exceeds 2e-3 (|ref| >= 0.5) the bound is one bfloat16 ulp, since
    rounding to the output type alone can exceed 2e-3 there; the kernel's error before that
    rounding (kernel_error) must stay within the stated bound everywhere."""
    assert got64.shape == ref64.shape
    assert np.isfinite(ref64).all()
    assert np.isfinite(got64).all(), f"{what}: non-finite output"
    err = np.abs(got64 - ref64)
    bound = np.full_like(ref64, TOL[dtype])
    if dtype == "bf16":
        bound = np.maximum(bound, bf16_ulp(ref64))
    kerr = kernel_error(got64, ref64, dtype)
    exact = float(np.mean(got64 == round_to(ref64, dtype)))
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    scale = max(float(np.sqrt(np.mean(ref64 * ref64))), 1e-30)
    test = os.environ.get("PYTEST_CURRENT_TEST", what or "-").split(" ")[0]
    REPORT.append((test, dtype, int(err.size), float(err.max()),
                   float((err / ulp(np.maximum(np.abs(ref64), scale), dtype)).max()),
                   float(kerr.max()), exact))
    assert (err <= bound).all(), (
        f"{what}: max err {err.max():.3g} at {worst} (got {got64[worst]}, ref {ref64[worst]})")
    assert (kerr <= TOL[dtype]).all(), f"{what}: kernel error {kerr.max():.3g}"
    return float(err.max())


def full_oracle(q_np, k_pool_t, v_pool_t, tables, lens, dtype, scale, threads=16):
    """Oracle outputs [S][H][D] of every (sequence, head) unit, reading each sequence's blocks
    back from the device pools (the stored values); sequences run on a thread pool (numpy
    releases the GIL in the heavy parts)."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    S, H, D = q_np.shape
    BS = k_pool_t.shape[2]
    out = np.full((S, H, D), np.nan)

    def one(s):
        L = int(lens[s])
        n = W.nblocks_for(L, BS)
        if n:
            idx = torch.from_numpy(np.asarray(tables[s, :n], np.int64)).to(k_pool_t.device)
            kc = W.from_torch(k_pool_t.index_select(0, idx), dtype)
            vc = W.from_torch(v_pool_t.index_select(0, idx), dtype)
        else:
            kc = W.from_torch(k_pool_t[:1], dtype)
            vc = W.from_torch(v_pool_t[:1], dtype)
        tab = np.arange(max(n, 1), dtype=np.int32)[None, :]
        for h in range(H):
            out[s, h] = oracle.decode_unit(q_np[s:s + 1], kc, vc, tab, np.array([L]), scale,
                                           dtype, 0, h)

    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(S)))
    return out


def sampled_oracle(q_np, k_pool_t, v_pool_t, tables, lens, units, dtype, scale):
    """Oracle outputs for (s, h) in ``units``, reading each sampled sequence's blocks back
    from the device pools (the stored values)."""
    import torch
    out = {}
    by_seq = {}
    for s, h in units:
        by_seq.setdefault(int(s), []).append(int(h))
    BS = k_pool_t.shape[2]
    for s, heads in by_seq.items():
        L = int(lens[s])
        n = W.nblocks_for(L, BS)
        if n:
            idx = torch.from_numpy(np.asarray(tables[s, :n], np.int64)).to(k_pool_t.device)
            kc = W.from_torch(k_pool_t.index_select(0, idx), dtype)
            vc = W.from_torch(v_pool_t.index_select(0, idx), dtype)
        else:
            kc = W.from_torch(k_pool_t[:1], dtype)
            vc = W.from_torch(v_pool_t[:1], dtype)
        tab = np.arange(max(n, 1), dtype=np.int32)[None, :]
        for h in heads:
            out[(s, h)] = oracle.decode_unit(q_np[s:s + 1], kc, vc, tab, np.array([L]), scale,
                                             dtype, 0, h)
    return out
