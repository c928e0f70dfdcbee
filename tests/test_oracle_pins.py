"""Pins for the CPU oracle: each check is independent of the oracle's own code.

Sources of truth used here (none re-types an oracle formula):
* hand-worked examples in tests/golden/hand_worked.json (derivations inside),
* brute force in pure Python on tiny inputs,
* library routines the oracle does not itself use (searchsorted, lexsort,
  bincount, cumsum, stable argsort, torch's bf16 conversion),
* closed forms (two-way softmax = logistic function; K=1 reduces to a plain
  single-adapter LoRA),
* invariants (sum of counts = N*k, perm is a permutation of the routed pairs,
  inv o perm = id, gate weights sum to 1, applications N*k versus K*N).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import (apply, apply_masked_passes, bf16_to_f64, dispatch, route_topk, route_vocab,
                    router_logits)

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))


def f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------- golden

def test_golden_vocab_k1():
    g = GOLDEN["vocab_k1"]
    idx, w = route_vocab(np.array(g["ids"], np.int32), np.array(g["bounds"], np.int32))
    assert idx.tolist() == g["expect_idx"]
    assert w.tolist() == g["expect_w"]
    counts, offsets, perm, perm_w, inv = dispatch(idx, w, 2)
    assert counts.tolist() == g["expect_counts"]
    assert offsets.tolist() == g["expect_offsets"]
    assert perm.tolist() == g["expect_perm"]
    assert inv.tolist() == g["expect_inv"]
    y = apply(f64(g["y0"]), f64(g["x"]), f64(g["A"]), f64(g["B"]), g["scale"], perm, perm_w, offsets, 1)
    assert y.tolist() == g["expect_y"]


def test_golden_topk_k2():
    g = GOLDEN["topk_k2"]
    idx, w, flags = route_topk(f64(g["logits"]), g["k"])
    assert idx.tolist() == g["expect_idx"]
    np.testing.assert_allclose(w, g["expect_w"], rtol=0, atol=1e-15)
    assert flags.tolist() == g["expect_flags"]
    counts, offsets, perm, perm_w, inv = dispatch(idx, w, 3)
    assert counts.tolist() == g["expect_counts"]
    assert offsets.tolist() == g["expect_offsets"]
    assert perm.tolist() == g["expect_perm"]
    assert inv.tolist() == g["expect_inv"]
    np.testing.assert_allclose(perm_w, g["expect_perm_w"], rtol=0, atol=1e-15)
    y = apply(f64(g["y0"]), f64(g["x"]), f64(g["A"]), f64(g["B"]), g["scale"], perm, perm_w, offsets, 2)
    np.testing.assert_allclose(y, g["expect_y"], rtol=0, atol=1e-14)
    y2 = apply_masked_passes(f64(g["y0"]), f64(g["x"]), f64(g["A"]), f64(g["B"]), g["scale"], idx, w)
    np.testing.assert_allclose(y2, g["expect_y"], rtol=0, atol=1e-14)


def test_golden_router():
    g = GOLDEN["router_mlp"]
    lg = router_logits(f64(g["x"]), f64(g["W1"]), f64(g["b1"]), f64(g["W2"]), f64(g["b2"]))
    assert lg.tolist() == g["expect_logits"]


# --------------------------------------------------------------------------- bf16 widening

def test_bf16_widening_against_torch_and_hand_values():
    assert bf16_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert bf16_to_f64(np.array([0xC000], np.uint16))[0] == -2.0
    assert bf16_to_f64(np.array([0x3F81], np.uint16))[0] == 1.0078125
    assert bf16_to_f64(np.array([0x0000], np.uint16))[0] == 0.0
    bits = np.random.default_rng(0).integers(0, 0x7F80, size=4096).astype(np.uint16)  # finite positives
    bits = np.concatenate([bits, bits | 0x8000])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_to_f64(bits), ref)


def test_synth_bf16_rounding_matches_torch_rne():
    v = np.random.default_rng(1).standard_normal(20000).astype(np.float32) * 10
    # include exact ties (lower 16 bits = 0x8000) to check ties-to-even
    ties = (np.arange(1, 200, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties])
    ours = synth.to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


# --------------------------------------------------------------------------- route_vocab

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_route_vocab_matches_searchsorted(seed):
    g = np.random.default_rng(seed)
    K = int(g.integers(1, 9))
    widths = g.integers(0, 50, size=K)  # empty ranges allowed
    bounds = np.concatenate([[int(g.integers(-20, 20))], widths]).cumsum().astype(np.int32)
    ids = g.integers(int(bounds[0]) - 30, int(bounds[-1]) + 30, size=3000).astype(np.int32)
    ids[:K + 1] = bounds  # every boundary value itself
    idx, w = route_vocab(ids, bounds)
    pos = np.searchsorted(bounds, ids, side="right") - 1
    inside = (ids >= bounds[0]) & (ids < bounds[-1])
    expect = np.where(inside, pos, -1)
    np.testing.assert_array_equal(idx, expect)
    np.testing.assert_array_equal(w, np.where(expect >= 0, 1.0, 0.0))


def test_route_vocab_uniform_ranges_is_integer_division():
    ids = np.random.default_rng(3).integers(0, 32768, size=10000).astype(np.int32)
    ids[:6] = [0, 8191, 8192, 16383, 16384, 32767]
    idx, _ = route_vocab(ids, synth.vocab_bounds(4))
    np.testing.assert_array_equal(idx, ids // 8192)
    edge, _ = route_vocab(np.array([-1, 32768, 40000], np.int32), synth.vocab_bounds(4))
    assert edge.tolist() == [-1, -1, -1]


# --------------------------------------------------------------------------- route_topk

def brute_topk(row, k):
    """All k-subsets; keep the one whose members all beat every non-member under
    the order (larger logit first, then lower index)."""
    K = len(row)
    better = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)  # noqa: E731
    found = []
    for S in itertools.combinations(range(K), k):
        rest = [j for j in range(K) if j not in S]
        if all(better(a, b) for a in S for b in rest):
            found.append(S)
    assert len(found) == 1
    return list(found[0])


@pytest.mark.parametrize("K,k", [(2, 1), (3, 1), (3, 2), (4, 2), (5, 3), (6, 1), (6, 4), (4, 4)])
def test_topk_brute_force_with_ties(K, k):
    g = np.random.default_rng(K * 10 + k)
    lg = g.integers(-3, 4, size=(400, K)).astype(np.float64)  # many exact ties
    idx, w, flags = route_topk(lg, k)
    for t in range(lg.shape[0]):
        row = lg[t].tolist()
        assert idx[t].tolist() == brute_topk(row, k)
        desc = sorted(row, reverse=True)
        assert bool(flags[t]) == (k < K and desc[k - 1] - desc[k] < 1e-4)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_topk_matches_lexsort_on_continuous_logits():
    g = np.random.default_rng(11)
    lg = g.standard_normal((2000, 16))
    for k in (1, 2, 3, 4):
        idx, w, _ = route_topk(lg, k)
        order = np.lexsort((np.broadcast_to(np.arange(16), lg.shape), -lg), axis=1)
        expect = np.sort(order[:, :k], axis=1)
        np.testing.assert_array_equal(idx, expect)


def test_topk_weights_closed_forms():
    g = np.random.default_rng(5)
    lg = g.standard_normal((500, 8)) * 3
    idx, w, _ = route_topk(lg, 1)
    assert np.all(w == 1.0)  # k=1: the single selected adapter gets weight exactly 1
    idx, w, _ = route_topk(lg, 2)
    l0 = np.take_along_axis(lg, idx[:, :1], axis=1)[:, 0]
    l1 = np.take_along_axis(lg, idx[:, 1:], axis=1)[:, 0]
    logistic = np.array([1.0 / (1.0 + math.exp(b - a)) for a, b in zip(l0, l1)])
    np.testing.assert_allclose(w[:, 0], logistic, rtol=0, atol=1e-14)
    np.testing.assert_allclose(w[:, 1], 1.0 - logistic, rtol=0, atol=1e-14)
    # softmax over all K, renormalised over the selected set, gives the same weights
    idx, w, _ = route_topk(lg, 3)
    full = np.exp(lg - lg.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(full, idx, axis=1)
    np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=0, atol=1e-13)


def test_topk_margin_flags():
    lg = np.array([[1.0, 1.0 + 5e-5, 0.0],   # top-1 margin 5e-5 < 1e-4 -> flag
                   [1.0, 1.0 + 2e-4, 0.0],   # margin 2e-4 -> no flag
                   [2.0, 1.0, 1.0 - 1e-5]])  # top-2: 2nd vs 3rd margin 1e-5 -> flag for k=2
    _, _, f1 = route_topk(lg, 1)
    assert f1.tolist() == [True, False, False]
    _, _, f2 = route_topk(lg, 2)
    assert f2.tolist() == [False, False, True]
    _, _, f3 = route_topk(lg, 3)
    assert f3.tolist() == [False, False, False]  # k == K: nothing left to confuse


# --------------------------------------------------------------------------- router MLP

def test_router_matches_triple_loop():
    g = np.random.default_rng(9)
    N, d, H, K = 5, 7, 4, 3
    x, W1, b1 = g.standard_normal((N, d)), g.standard_normal((d, H)), g.standard_normal(H)
    W2, b2 = g.standard_normal((H, K)), g.standard_normal(K)
    lg = router_logits(x, W1, b1, W2, b2)
    for t in range(N):
        hid = []
        for j in range(H):
            s = b1[j]
            for i in range(d):
                s += x[t, i] * W1[i, j]
            hid.append(s if s > 0 else 0.0)
        for e in range(K):
            s = b2[e]
            for j in range(H):
                s += hid[j] * W2[j, e]
            assert abs(lg[t, e] - s) < 1e-12


# --------------------------------------------------------------------------- dispatch

@pytest.mark.parametrize("N,k,K", [(1, 1, 1), (37, 1, 4), (300, 2, 4), (257, 3, 16), (1000, 4, 64), (0, 1, 3)])
def test_dispatch_matches_library_routines(N, k, K):
    g = np.random.default_rng(N + 7 * k + K)
    idx = g.integers(-1, K + 1, size=(N, k)).astype(np.int32)  # includes unrouted -1 and K
    w = g.random((N, k))
    counts, offsets, perm, perm_w, inv = dispatch(idx, w, K)
    e = idx.reshape(-1)
    valid = (e >= 0) & (e < K)
    np.testing.assert_array_equal(counts, np.bincount(e[valid], minlength=K))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(e[valid], minlength=K))]))
    key = np.where(valid, e, K)  # unrouted pairs sort past the last adapter
    order = np.argsort(key, kind="stable")[: int(valid.sum())]
    np.testing.assert_array_equal(perm, order)
    np.testing.assert_array_equal(perm_w, w.reshape(-1)[order])
    # invariants
    assert counts.sum() == valid.sum()
    assert sorted(perm.tolist()) == np.nonzero(valid)[0].tolist()
    for q, p in enumerate(perm):
        assert inv[p] == q
    assert np.all(inv[~valid] == -1)


def test_dispatch_all_routed_sums_to_Nk():
    g = np.random.default_rng(21)
    for k in (1, 2, 3, 4):
        idx, _, _ = route_topk(g.standard_normal((512, 16)), k)
        counts, offsets, perm, _, _ = dispatch(idx, np.ones(idx.shape), 16)
        assert counts.sum() == 512 * k and offsets[-1] == 512 * k
        assert np.array_equal(np.sort(perm), np.arange(512 * k))


# --------------------------------------------------------------------------- apply

def brute_apply(y0, x, A, B, scale, idx, w):
    N, d_out = len(y0), len(y0[0])
    d_in, r = len(A[0]), len(A[0][0])
    y = [list(map(float, row)) for row in y0]
    for t in range(N):
        for s in range(len(idx[t])):
            e = int(idx[t][s])
            if e < 0 or e >= len(A):
                continue
            h = [sum(x[t][i] * A[e][i][j] for i in range(d_in)) for j in range(r)]
            for c in range(d_out):
                y[t][c] += w[t][s] * scale * sum(h[j] * B[e][j][c] for j in range(r))
    return np.array(y)


@pytest.mark.parametrize("N,d_in,d_out,K,r,k", [(4, 8, 5, 3, 2, 1), (6, 5, 9, 3, 3, 2), (7, 6, 4, 5, 2, 3)])
def test_apply_brute_force(N, d_in, d_out, K, r, k):
    g = np.random.default_rng(N * d_in)
    x, A, B = g.standard_normal((N, d_in)), g.standard_normal((K, d_in, r)), g.standard_normal((K, r, d_out))
    y0 = g.standard_normal((N, d_out))
    idx, w, _ = route_topk(g.standard_normal((N, K)), k)
    idx = idx.copy()
    idx[0, 0] = -1  # one unrouted slot
    counts, offsets, perm, perm_w, _ = dispatch(idx, w, K)
    y = apply(y0, x, A, B, 1.7, perm, perm_w, offsets, k)
    ref = brute_apply(y0.tolist(), x.tolist(), A.tolist(), B.tolist(), 1.7, idx.tolist(), w.tolist())
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_apply_small_integers_exact():
    xb, Ab, Bb, yb = synth.small_int_case(N=9, d_in=16, d_out=12, K=3, r=4)
    x, A, B, y0 = (bf16_to_f64(v) for v in (xb, Ab, Bb, yb))
    idx = np.array([0, 1, 2, 0, 1, 2, 2, 2, -1], np.int32)
    counts, offsets, perm, perm_w, _ = dispatch(idx, np.where(idx >= 0, 1.0, 0.0), 3)
    y = apply(y0, x, A, B, 2.0, perm, perm_w, offsets, 1)
    ref = brute_apply(y0.tolist(), x.tolist(), A.tolist(), B.tolist(), 2.0, idx[:, None].tolist(),
                      np.ones((9, 1)).tolist())
    np.testing.assert_array_equal(y, ref)  # integers: exact


def test_apply_single_adapter_is_plain_lora():
    g = np.random.default_rng(4)
    N, d_in, d_out, r = 33, 40, 24, 8
    x, A, B, y0 = (g.standard_normal((N, d_in)), g.standard_normal((1, d_in, r)),
                   g.standard_normal((1, r, d_out)), g.standard_normal((N, d_out)))
    idx = np.zeros(N, np.int32)
    counts, offsets, perm, perm_w, _ = dispatch(idx, np.ones(N), 1)
    y = apply(y0, x, A, B, 2.0, perm, perm_w, offsets, 1)
    lora = y0 + 2.0 * np.matmul(np.matmul(x, A[0]), B[0])
    np.testing.assert_allclose(y, lora, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("k", [1, 2, 4])
def test_apply_equals_masked_passes_and_work_counts(k):
    g = np.random.default_rng(100 + k)
    N, d, K, r = 300, 64, 8, 16
    x, A, B, y0 = (g.standard_normal((N, d)), g.standard_normal((K, d, r)) / 8,
                   g.standard_normal((K, r, d)) / 4, g.standard_normal((N, d)))
    idx, w, _ = route_topk(g.standard_normal((N, K)), k)
    counts, offsets, perm, perm_w, _ = dispatch(idx, w, K)
    y = apply(y0, x, A, B, 2.0, perm, perm_w, offsets, k)
    y2 = apply_masked_passes(y0, x, A, B, 2.0, idx, w)
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)
    # work: per-token routing applies N*k (token, adapter) pairs; K masked passes apply K*N
    assert int(offsets[-1]) == N * k
    assert K * N > N * k


def test_vocab_pipeline_equals_masked_passes_on_modality_runs():
    case = synth.modality4(N=512, d=128, r=16)
    t = case.targets[0]
    x, A, B, y0 = (bf16_to_f64(v) for v in (t.x, t.A, t.B, t.y0))
    idx, w = route_vocab(case.ids, case.bounds)
    counts, offsets, perm, perm_w, _ = dispatch(idx, w, case.K)
    y = apply(y0, x, A, B, case.scale, perm, perm_w, offsets, 1)
    y2 = apply_masked_passes(y0, x, A, B, case.scale, idx, w)
    np.testing.assert_allclose(y, y2, rtol=1e-12, atol=1e-12)
    assert counts.sum() == 512
