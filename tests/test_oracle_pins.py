"""Pins for the CPU fp64 oracle (runs without a GPU).

The pages print no worked input/output pair for the execution unit, so the
oracle is pinned to things other than itself:
  * hand-worked examples (tests/golden/*.json, each with its citation);
  * closed forms: selection-matrix bases, one-hot adapters;
  * special cases that reduce to library routines: all-base_only == a numpy
    matrix product; routing == numpy's stable argsort + bincount + cumsum;
  * the exact result: integer inputs, checked against Python Fractions;
  * invariants: zero padding, linearity in alpha, B = 0, token permutation,
    thread count.
A dropped term, a wrong sign, a transposed operand, a wrong scale or a wrong
slot index each fails at least one of these.
"""
import json
import os
import zlib
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# apply: hand-worked example and closed forms
# --------------------------------------------------------------------------

def test_apply_worked_example():
    g = _golden("apply_worked_example.json")
    ads = {int(s): (np.array(a["A"], float), np.array(a["B"], float), a["rank"], a["alpha"])
           for s, a in g["adapters"].items()}
    y, inv = oracle.apply(np.array(g["x"], float), np.array(g["W"], float),
                          np.array(g["idx"]), g["n_slots"], ads)
    assert inv.tolist() == g["invalid"]
    for t, row in enumerate(g["y"]):
        if g["invalid"][t]:
            assert np.all(np.isnan(y[t]))
        else:
            assert y[t].tolist() == row  # exact: integers and halves


def test_apply_selection_matrix_base():
    # W[n][k] = 1 iff k == sigma(n), d_in != d_out: base[t][n] = x[t][sigma(n)].
    rng = np.random.default_rng(11)
    d_in, d_out, T = 7, 5, 6
    sigma = rng.permutation(d_in)[:d_out]
    W = np.zeros((d_out, d_in))
    W[np.arange(d_out), sigma] = 1.0
    x = rng.standard_normal((T, d_in))
    y, inv = oracle.apply(x, W, np.full(T, -1), 2, {})
    assert not inv.any()
    assert np.array_equal(y, x[:, sigma])


def test_apply_one_hot_adapter_closed_form():
    # A[j0][k0] = 1 and B[n0][j0] = 1: delta = (alpha/r) * x[t][k0] at column n0 only.
    rng = np.random.default_rng(12)
    d_in, d_out, r, alpha = 6, 9, 3, 6.0   # s = 2
    j0, k0, n0 = 2, 4, 7
    A = np.zeros((r, d_in))
    A[j0, k0] = 1.0
    B = np.zeros((d_out, r))
    B[n0, j0] = 1.0
    x = rng.integers(-4, 5, size=(5, d_in)).astype(float)
    W = rng.integers(-2, 3, size=(d_out, d_in)).astype(float)
    y_ad, _ = oracle.apply(x, W, np.zeros(5, int), 1, {0: (A, B, r, alpha)})
    y_base, _ = oracle.apply(x, W, np.full(5, -1), 1, {0: (A, B, r, alpha)})
    delta = y_ad - y_base
    expect = np.zeros_like(delta)
    expect[:, n0] = 2.0 * x[:, k0]
    assert np.array_equal(delta, expect)


def test_apply_base_only_is_library_matmul():
    rng = np.random.default_rng(13)
    T, d_in, d_out = 9, 33, 17
    x = rng.standard_normal((T, d_in))
    W = rng.standard_normal((d_out, d_in))
    y, inv = oracle.apply(x, W, np.full(T, -1), 3, {})
    ref = np.matmul(x, W.T)
    assert not inv.any()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_apply_exact_rational_small_integers():
    # With small integer inputs every fp64 operation is exact, so the oracle must
    # equal exact rational arithmetic of the per-token definition.
    rng = np.random.default_rng(14)
    T, d_in, d_out, S = 7, 5, 4, 3
    x = rng.integers(-3, 4, size=(T, d_in))
    W = rng.integers(-2, 3, size=(d_out, d_in))
    ads = {}
    for s, (r, alpha) in enumerate([(1, 3.0), (2, 1.0), (4, 2.0)]):
        ads[s] = (rng.integers(-2, 3, size=(r, d_in)).astype(float),
                  rng.integers(-2, 3, size=(d_out, r)).astype(float), r, alpha)
    idx = np.array([0, 1, 2, -1, 2, 0, 1])
    y, inv = oracle.apply(x.astype(float), W.astype(float), idx, S, ads)
    assert not inv.any()
    for t in range(T):
        for n in range(d_out):
            v = sum(Fraction(int(x[t, k])) * int(W[n, k]) for k in range(d_in))
            if idx[t] >= 0:
                A, B, r, alpha = ads[int(idx[t])]
                h = [sum(Fraction(int(x[t, k])) * int(A[j, k]) for k in range(d_in))
                     for j in range(r)]
                v += Fraction(alpha) / r * sum(h[j] * int(B[n, j]) for j in range(r))
            assert Fraction(y[t, n]) == v


# --------------------------------------------------------------------------
# apply: invariants
# --------------------------------------------------------------------------

def _rand_case(seed, T=12, d_in=24, d_out=20, S=4, r=4, alpha=8.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d_in))
    W = rng.standard_normal((d_out, d_in)) / np.sqrt(d_in)
    ads = {s: (rng.standard_normal((r, d_in)) / np.sqrt(d_in),
               rng.standard_normal((d_out, r)) * 0.1, r, alpha) for s in range(S)}
    idx = rng.integers(-1, S, size=T)
    return x, W, ads, idx


def test_zero_padding_keeps_result():
    # rank r padded with zero rows/columns to R, alpha scaled by R/r: identical.
    x, W, ads, idx = _rand_case(21, r=8, alpha=16.0)
    R = 64
    padded = {}
    for s, (A, B, r, alpha) in ads.items():
        Ap = np.zeros((R, A.shape[1]))
        Ap[:r] = A
        Bp = np.zeros((B.shape[0], R))
        Bp[:, :r] = B
        padded[s] = (Ap, Bp, R, alpha * R / r)
    y1, _ = oracle.apply(x, W, idx, 4, ads)
    y2, _ = oracle.apply(x, W, idx, 4, padded)
    assert np.array_equal(y1, y2)


def test_linear_in_alpha_and_base_untouched():
    x, W, ads, idx = _rand_case(22)
    ads2 = {s: (A, B, r, 2.0 * a) for s, (A, B, r, a) in ads.items()}
    y1, _ = oracle.apply(x, W, idx, 4, ads)
    y2, _ = oracle.apply(x, W, idx, 4, ads2)
    yb, _ = oracle.apply(x, W, np.full_like(idx, -1), 4, ads)
    lora = idx >= 0
    np.testing.assert_allclose(y2[lora] - yb[lora], 2.0 * (y1[lora] - yb[lora]),
                               rtol=1e-12, atol=1e-12)
    assert np.array_equal(y1[~lora], yb[~lora])


def test_b_zero_is_noop():
    x, W, ads, idx = _rand_case(23)
    zero = {s: (A, np.zeros_like(B), r, a) for s, (A, B, r, a) in ads.items()}
    y, _ = oracle.apply(x, W, idx, 4, zero)
    yb, _ = oracle.apply(x, W, np.full_like(idx, -1), 4, zero)
    assert np.array_equal(y, yb)


def test_token_permutation_permutes_rows():
    x, W, ads, idx = _rand_case(24)
    p = np.random.default_rng(5).permutation(x.shape[0])
    y, _ = oracle.apply(x, W, idx, 4, ads)
    yp, _ = oracle.apply(x[p], W, idx[p], 4, ads)
    assert np.array_equal(yp, y[p])


def test_thread_count_does_not_change_result():
    x, W, ads, idx = _rand_case(25, T=40)
    y1, _ = oracle.apply(x, W, idx, 4, ads, n_threads=1)
    y8, _ = oracle.apply(x, W, idx, 4, ads, n_threads=8)
    assert np.array_equal(y1, y8)


def test_invalid_tokens_are_nan_and_counted():
    x, W, ads, _ = _rand_case(26)
    del ads[2]
    idx = np.array([0, 2, -1, 5, -2, 1, 3, 0, 2, -1, 1, 3])
    y, inv = oracle.apply(x, W, idx, 4, ads)
    bad = np.array([i in (2, 5, -2) for i in idx])
    assert np.array_equal(inv.astype(bool), bad)
    assert np.all(np.isnan(y[bad]))
    assert not np.any(np.isnan(y[~bad]))


# --------------------------------------------------------------------------
# route
# --------------------------------------------------------------------------

def test_route_worked_example():
    g = _golden("route_worked_example.json")
    r = oracle.route(g["idx"], g["n_slots"], g["active"], g["policy"], g["theta"])
    assert r["counts"].tolist() == g["counts"]
    assert r["offsets"].tolist() == g["offsets"]
    assert r["perm"].tolist() == g["perm"]
    assert r["segs"].tolist() == g["segs"]
    assert r["n_seg"] == g["n_seg"]


def _numpy_route(idx, S, active, policy, theta):
    idx = np.asarray(idx, np.int64)
    ok = (idx >= 0) & (idx < S)
    act = np.zeros(idx.shape, bool)
    act[ok] = np.asarray(active)[idx[ok]] != 0
    keys = np.where(idx == -1, S, np.where(ok & act, idx, S + 1))
    counts = np.bincount(keys, minlength=S + 2)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.argsort(keys, kind="stable")
    return counts, offsets, perm


EDGE_IDX = {
    "all_same": [3] * 50,
    "all_base_only": [-1] * 33,
    "sorted": sorted([0, 0, 1, 2, 2, 2, 5, 7, 7, -1, -1]),
    "reversed": sorted([0, 0, 1, 2, 2, 2, 5, 7, 7, -1, -1], reverse=True),
    "all_invalid": [9, 100, -5, 8, 8],
    "single": [4],
    "empty": [],
}


@pytest.mark.parametrize("case", list(EDGE_IDX) + ["random%d" % i for i in range(6)])
def test_route_matches_numpy_stable_sort(case):
    S = 8
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    if case in EDGE_IDX:
        idx = np.array(EDGE_IDX[case], np.int32)
        active = np.ones(S, np.int32)
    else:
        T = int(rng.integers(1, 3000))
        idx = rng.integers(-3, S + 2, size=T).astype(np.int32)
        active = (rng.random(S) < 0.7).astype(np.int32)
    r = oracle.route(idx, S, active, oracle.POLICY_AUTO, 16)
    counts, offsets, perm = _numpy_route(idx, S, active, 0, 16)
    assert r["counts"].tolist() == counts.tolist()
    assert r["offsets"].tolist() == offsets.tolist()
    assert r["perm"].tolist() == perm.tolist()
    nz = [k for k in range(S + 2) if counts[k] > 0]
    assert r["n_seg"] == len(nz)
    for rec, k in zip(r["segs"].tolist(), nz):
        assert rec[:3] == [k, offsets[k], counts[k]]


@pytest.mark.parametrize("policy,theta,expect", [
    (0, 4, [2, 1, 0]),      # AUTO: len 4 is not > 4 -> SEPARATE; len 5 -> FUSED
    (0, 3, [1, 1, 0]),
    (1, 100, [1, 1, 0]),    # forced FUSED
    (2, 0, [2, 2, 0]),      # forced SEPARATE
])
def test_route_modes(policy, theta, expect):
    idx = [0] * 4 + [1] * 5 + [-1] * 3
    r = oracle.route(idx, 2, [1, 1], policy, theta)
    assert r["segs"][:, 3].tolist() == expect
