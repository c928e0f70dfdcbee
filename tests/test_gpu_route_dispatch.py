"""GPU parity: routing decisions and dispatch against the CPU oracle (bit-exact)."""
import numpy as np
import pytest
import torch

import synth
from oracle import dispatch, route_topk, route_vocab, router_logits
from tests.gpu_util import W_TOL, dev, dev_bf16, f64, host, need_gpu

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------- route_vocab

@pytest.mark.parametrize("case", ["tiny", "modality4"])
def test_route_vocab_configs(case):
    m = need_gpu()
    c = synth.tiny_vocab() if case == "tiny" else synth.modality4()
    idx, w = m.molora_route_vocab(dev(c.ids), c.bounds.tolist())
    ri, rw = route_vocab(c.ids, c.bounds)
    np.testing.assert_array_equal(host(idx), ri)
    np.testing.assert_array_equal(host(w), rw.astype(np.float32))


def test_route_vocab_edges_and_uneven_ranges():
    m = need_gpu()
    bounds = [-5, 0, 0, 17, 300, 300, 4096]  # empty ranges included
    ids = np.array([-6, -5, -1, 0, 1, 16, 17, 299, 300, 301, 4095, 4096, 10**9, -10**9], np.int32)
    ids = np.concatenate([ids, np.random.default_rng(3).integers(-50, 4200, 5000).astype(np.int32)])
    idx, w = m.molora_route_vocab(dev(ids), bounds)
    ri, rw = route_vocab(ids, np.array(bounds))
    np.testing.assert_array_equal(host(idx), ri)
    np.testing.assert_array_equal(host(w), rw.astype(np.float32))


# ----------------------------------------------------------------------------- route_topk

def _check_selection(gpu_logits, idx, w, flags, k):
    """The GPU's selection equals the oracle's selection on the GPU's own fp32 logits."""
    oi, ow, of = route_topk(gpu_logits.astype(np.float64), k)
    np.testing.assert_array_equal(idx, oi)
    np.testing.assert_array_equal(flags.astype(bool), of)
    assert np.max(np.abs(w - ow)) <= W_TOL
    np.testing.assert_allclose(w.astype(np.float64).sum(axis=1), 1.0, rtol=0, atol=4 * W_TOL)
    if k == 1:
        assert np.all(w == 1.0)


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_route_topk_logits_mode_stress(k):
    m = need_gpu()
    lg = synth.zipf_logits(4, 16384, 16)
    logits, idx, w, flags = m.molora_route_topk(k, 16, logits=dev(lg))
    _check_selection(lg, host(idx), host(w), host(flags), k)
    np.testing.assert_array_equal(host(logits), lg)  # input untouched


@pytest.mark.parametrize("K,k", [(3, 2), (8, 1), (8, 8), (64, 8), (64, 1), (5, 5)])
def test_route_topk_ties_and_shapes(K, k):
    m = need_gpu()
    g = np.random.default_rng(K * 100 + k)
    N = 1000 + K  # ragged in the 16-token workgroup tiles
    lg = g.integers(-2, 3, size=(N, K)).astype(np.float32)  # many exact ties
    lg[::7] += (g.random((len(lg[::7]), K)) * 1e-5).astype(np.float32)  # near ties
    logits, idx, w, flags = m.molora_route_topk(k, K, logits=dev(lg))
    _check_selection(lg, host(idx), host(w), host(flags), k)


def test_route_topk_router_mode_qwen_layer():
    m = need_gpu()
    c = synth.qwen_layer()
    r = c.router
    x = c.targets[0].x
    W1t = np.ascontiguousarray(r["W1"].T)  # nn.Linear layout [64][d]
    W2t = np.ascontiguousarray(r["W2"].T)  # [K][64]
    logits, idx, w, flags = m.molora_route_topk(c.k, c.K, x=dev_bf16(x), W1=dev_bf16(W1t), b1=dev(r["b1"]),
                                               W2=dev_bf16(W2t), b2=dev(r["b2"]))
    gl = host(logits)
    ref = router_logits(f64(x), f64(r["W1"]), r["b1"].astype(np.float64), f64(r["W2"]), r["b2"].astype(np.float64))
    assert np.max(np.abs(gl - ref)) <= 1e-4, np.max(np.abs(gl - ref))
    gi, gw, gf = host(idx), host(w), host(flags)
    _check_selection(gl, gi, gw, gf, c.k)
    oi, _, of = route_topk(ref, c.k)
    sure = ~(of | gf.astype(bool))
    np.testing.assert_array_equal(gi[sure], oi[sure])
    assert sure.mean() > 0.99


def test_route_topk_router_ragged_small():
    m = need_gpu()
    g = np.random.default_rng(5)
    N, d, K, k = 37, 256, 6, 3
    xb = synth.to_bf16_bits(g.standard_normal((N, d)).astype(np.float32))
    W1 = synth.to_bf16_bits((g.standard_normal((d, 64)) / 16).astype(np.float32))
    W2 = synth.to_bf16_bits((g.standard_normal((64, K)) / 8).astype(np.float32))
    b1 = (g.standard_normal(64) / 10).astype(np.float32)
    logits, idx, w, flags = m.molora_route_topk(k, K, x=dev_bf16(xb), W1=dev_bf16(np.ascontiguousarray(W1.T)),
                                               b1=dev(b1), W2=dev_bf16(np.ascontiguousarray(W2.T)), b2=None)
    ref = router_logits(f64(xb), f64(W1), b1.astype(np.float64), f64(W2), None)
    assert np.max(np.abs(host(logits) - ref)) <= 1e-4
    _check_selection(host(logits), host(idx), host(w), host(flags), k)


@pytest.mark.parametrize("N,d,K,k,bias", [(4096, 2048, 4, 2, True), (37, 256, 6, 3, True), (129, 128, 4, 1, False),
                                          (300, 640, 8, 2, True), (1000, 4096, 16, 4, True), (64, 4224, 4, 2, True)])
def test_route_topk_workspace_same_bits(N, d, K, k, bias):
    """The first layer split over eighths of d (a workspace) gives the one-launch path's bits:
    logits, idx, w and flags; d above 4096 ignores the workspace.  The workspace starts as NaN
    bytes, so a chunk read before it is written would show.  Logits against the oracle too."""
    m = need_gpu()
    g = np.random.default_rng(N + d + K)
    xb = synth.to_bf16_bits(g.standard_normal((N, d)).astype(np.float32))
    W1 = synth.to_bf16_bits((g.standard_normal((d, 64)) / np.sqrt(d)).astype(np.float32))
    W2 = synth.to_bf16_bits((g.standard_normal((64, K)) / 8).astype(np.float32))
    b1 = (g.standard_normal(64) / 10).astype(np.float32) if bias else None
    b2 = (g.standard_normal(K) / 10).astype(np.float32) if bias else None
    args = dict(x=dev_bf16(xb), W1=dev_bf16(np.ascontiguousarray(W1.T)), b1=dev(b1) if bias else None,
                W2=dev_bf16(np.ascontiguousarray(W2.T)), b2=dev(b2) if bias else None)
    one = [host(t) for t in m.molora_route_topk(k, K, **args)]
    need = m.molora_route_topk_workspace(N, d)
    assert need == (8 * N * 64 * 4 if d <= 4096 else 0)
    ws = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        two = [host(t) for t in m.molora_route_topk(k, K, ws=ws, **args)]
        for a, b in zip(one, two):
            np.testing.assert_array_equal(a, b)
    ref = router_logits(f64(xb), f64(W1), b1.astype(np.float64) if bias else None, f64(W2),
                        b2.astype(np.float64) if bias else None)
    assert np.max(np.abs(two[0] - ref)) <= 1e-4
    _check_selection(two[0], two[1], two[2], two[3], k)


# ----------------------------------------------------------------------------- dispatch

def _check_dispatch(idx_np, w_np, K, k, out):
    counts, offsets, perm, perm_w, inv = (host(t) for t in out)
    oc, oo, op, opw, oinv = dispatch(idx_np, w_np, K)
    n = int(oo[-1])
    np.testing.assert_array_equal(counts, oc)
    np.testing.assert_array_equal(offsets, oo)
    np.testing.assert_array_equal(perm[:n], op)
    np.testing.assert_array_equal(perm_w[:n], opw.astype(np.float32))
    np.testing.assert_array_equal(inv, oinv)


@pytest.mark.parametrize("N,k,K", [(1, 1, 1), (256, 1, 4), (2048, 1, 4), (1000, 2, 4), (4096, 2, 4),
                                   (333, 3, 7), (2048, 1, 64), (5000, 8, 64), (16384, 4, 16), (16384, 1, 16),
                                   (40000, 2, 2), (8192, 1, 3), (8193, 1, 3), (1048579, 1, 64),
                                   (2049, 1, 4), (1025, 2, 64), (3000, 2, 5), (1365, 6, 16), (1537, 1, 16),
                                   (2730, 3, 11), (1024, 1, 4), (4097, 1, 16), (2731, 3, 9)])
def test_dispatch_random(N, k, K):
    m = need_gpu()
    g = np.random.default_rng(N + k * 7 + K)
    idx = g.integers(0, K, size=(N, k)).astype(np.int32)
    w = g.random((N, k)).astype(np.float32)
    out = m.molora_dispatch(dev(idx), dev(w), K, k)
    _check_dispatch(idx, w, K, k, out)


@pytest.mark.parametrize("N", [3001, 30001])
def test_dispatch_unrouted_and_out_of_range(N):
    """Unrouted pairs (adapter outside [0, K)) in the one-workgroup sort and in the chip-wide one."""
    m = need_gpu()
    g = np.random.default_rng(17)
    k, K = 2, 5
    idx = g.integers(-3, K + 3, size=(N, k)).astype(np.int32)
    w = g.random((N, k)).astype(np.float32)
    out = m.molora_dispatch(dev(idx), dev(w), K, k)
    _check_dispatch(idx, w, K, k, out)


def test_dispatch_of_gpu_routing_stress():
    m = need_gpu()
    lg = synth.zipf_logits(4, 16384, 16)
    for k in (1, 2, 3, 4):
        _, idx, w, _ = m.molora_route_topk(k, 16, logits=dev(lg))
        out = m.molora_dispatch(idx, w, 16, k)
        _check_dispatch(host(idx), host(w), 16, k, out)
        assert int(host(out[1])[-1]) == 16384 * k  # every pair routed: work N*k


def test_dispatch_deterministic():
    m = need_gpu()
    g = np.random.default_rng(2)
    idx = dev(g.integers(0, 16, size=(20000, 2)).astype(np.int32))
    w = dev(g.random((20000, 2)).astype(np.float32))
    a = [host(t) for t in m.molora_dispatch(idx, w, 16, 2)]
    b = [host(t) for t in m.molora_dispatch(idx, w, 16, 2)]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
