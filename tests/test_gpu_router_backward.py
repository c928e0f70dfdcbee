"""Router gradient on the GPU against the oracle: molora_route_topk_backward (softmax over the
selected logits) and molora_router_backward (the ReLU MLP d -> 64 -> K), plus the whole chain
dL/dw -> dL/dlogits -> router parameters on the Qwen-shaped layer.

The ReLU's mask is an integer decision taken from floating point: the GPU takes it on its fp32
pre-activation, the oracle on fp64.  The exact test uses small-integer inputs whose
pre-activations are exact in fp32 (both sides decide identically).  The realistic tests allow,
per output element, exactly what flipping the entries with |pre-activation| < AMBIG could
change, and nothing else.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev, dev_bf16, f64, host, need_gpu
from oracle import (apply_backward, dispatch, route_topk, route_topk_backward, router_backward,
                    router_logits)

pytestmark = pytest.mark.gpu

REL = 1e-4     # fp32 sums of exact bf16 products; hi/lo-carried fp32 gradients
AMBIG = 1e-4   # pre-activations this close to 0 may take either side of the ReLU


def _close(got, ref, name, allow=None):
    scale = max(float(np.max(np.abs(ref))) if ref.size else 0.0, 1e-30)
    bound = REL * scale + (allow if allow is not None else 0.0)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{name}: {int(bad.sum())} elements off; max err {float(np.max(np.abs(got - ref))):.3e}"


@pytest.mark.parametrize("K,k", [(2, 1), (4, 2), (16, 4), (64, 8), (8, 8)])
def test_route_topk_backward_matches_oracle(K, k):
    m = need_gpu()
    N = 1000
    g = np.random.default_rng(70 + K + k)
    logits = (g.standard_normal((N, K)) * 2).astype(np.float32)
    idx, w, _ = route_topk(logits.astype(np.float64), k)
    w32 = w.astype(np.float32)
    dw = g.standard_normal((N, k)).astype(np.float32)
    dl = m.molora_route_topk_backward(dev(idx.astype(np.int32)), dev(w32), dev(dw), K)
    ref = route_topk_backward(w32.astype(np.float64), idx, dw.astype(np.float64), K)
    got = host(dl)
    _close(got, ref, "dlogits")
    sel = np.zeros((N, K), bool)
    np.put_along_axis(sel, idx.astype(np.int64), True, axis=1)
    assert np.all(got[~sel] == 0.0)


def _router_case(cid, N, d, K, exact=False):
    if exact:
        g = np.random.default_rng(cid)
        x = synth.to_bf16_bits(g.integers(-2, 3, size=(N, d)).astype(np.float32))
        W1 = synth.to_bf16_bits((g.integers(-1, 2, size=(d, 64)) / 8.0).astype(np.float32))
        W2 = synth.to_bf16_bits((g.integers(-2, 3, size=(64, K)) / 4.0).astype(np.float32))
        b1 = (g.integers(-4, 4, size=64) / 8.0 + 1.0 / 16.0).astype(np.float32)  # pre is never 0
    else:
        r = synth.router_mlp(cid, d, 64, K)
        x, _ = synth.clustered_x(cid, N, d)
        W1, W2, b1 = r["W1"], r["W2"], r["b1"]
    dl = np.random.default_rng(cid + 1).standard_normal((N, K)).astype(np.float32)
    return x, W1, W2, b1, dl


def _allowances(x, W1, W2, b1, dl):
    """Per-output bounds on what flipping the ambiguous ReLU entries can change."""
    pre = x @ W1 + (b1 if b1 is not None else 0.0)
    amb = np.abs(pre) < AMBIG
    dh = np.abs(dl @ W2.T) * amb  # |dL/dhidden| on ambiguous entries
    return {"dW1": np.abs(x).T @ dh, "db1": dh.sum(axis=0), "dW2": (amb * AMBIG).T @ np.abs(dl),
            "dx": dh @ np.abs(W1).T}, int(amb.sum())


CASES = [  # N, d, K, case id, with b1, exact
    (1, 128, 4, 80, True, True),
    (100, 128, 4, 62, True, False),
    (1000, 512, 16, 61, False, False),
    (777, 1024, 64, 63, True, False),
    (4096, 2048, 4, 2, True, False),
    (333, 256, 8, 81, True, True),
]


@pytest.mark.parametrize("N,d,K,cid,with_b1,exact", CASES)
def test_router_backward_matches_oracle(N, d, K, cid, with_b1, exact):
    m = need_gpu()
    x, W1, W2, b1, dl = _router_case(cid, N, d, K, exact)
    b1 = b1 if with_b1 else None
    dx0 = np.random.default_rng(cid + 2).standard_normal((N, d)).astype(np.float32)
    out = m.molora_router_backward(dev_bf16(x), dev_bf16(np.ascontiguousarray(W1.T)),
                                   dev(b1) if b1 is not None else None, dev_bf16(np.ascontiguousarray(W2.T)),
                                   dev(dl), dx0=dev(dx0))
    torch.cuda.synchronize()
    xf, W1f, W2f = f64(x), f64(W1), f64(W2)
    b1f = b1.astype(np.float64) if b1 is not None else None
    dW1, db1, dW2, db2, dx = router_backward(xf, W1f, b1f, W2f, dl.astype(np.float64))
    allow, n_amb = _allowances(xf, W1f, W2f, b1f, dl.astype(np.float64))
    if exact:
        assert n_amb == 0
    _close(host(out["dW1"]), dW1.T, "dW1", allow["dW1"].T)
    _close(host(out["db1"]), db1, "db1", allow["db1"])
    _close(host(out["dW2"]), dW2.T, "dW2", allow["dW2"].T)
    _close(host(out["db2"]), db2, "db2")
    _close(host(out["dx"]), dx0 + dx, "dx", allow["dx"])


def test_router_backward_empty_batch_gives_zero_gradients():
    m = need_gpu()
    d, K = 256, 4
    W1 = torch.zeros(64, d, dtype=torch.bfloat16, device="cuda")
    W2 = torch.zeros(K, 64, dtype=torch.bfloat16, device="cuda")
    out = {n: torch.full(s, 5.0, device="cuda") for n, s in (("dW1", (64, d)), ("db1", (64,)), ("dW2", (K, 64)),
                                                           ("db2", (K,)))}
    m.molora_router_backward(torch.empty(0, d, dtype=torch.bfloat16, device="cuda"), W1, None, W2,
                             torch.empty(0, K, device="cuda"), want=(), out=out)
    torch.cuda.synchronize()
    for t in out.values():
        assert not t.any()


def test_router_backward_graph_replays_equal_eager():
    m = need_gpu()
    N, d, K = 512, 512, 8
    x, W1, W2, b1, dl = _router_case(82, N, d, K)
    xs, W1s, W2s, b1s, dls = (dev_bf16(x), dev_bf16(np.ascontiguousarray(W1.T)), dev_bf16(np.ascontiguousarray(W2.T)),
                              dev(b1), dev(dl))
    out = {n: torch.empty(s, device="cuda") for n, s in (("dW1", (64, d)), ("db1", (64,)), ("dW2", (K, 64)),
                                                         ("db2", (K,)), ("dx", (N, d)))}
    ws = torch.zeros(m.molora_router_backward_workspace(N, d, K), dtype=torch.uint8, device="cuda")

    def call():
        m.molora_router_backward(xs, W1s, b1s, W2s, dls, want=(), out=out, ws=ws)

    call()
    torch.cuda.synchronize()
    eager = {n: t.clone() for n, t in out.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(3):
        for t in out.values():
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in out:
            assert torch.equal(out[n], eager[n]), f"{n} replay {rep}"


def test_router_training_chain_on_qwen_layer():
    """One target of the Qwen-shaped layer (4096 tokens, d = 2048, K = 4, k = 2): the routing
    from the oracle's fp64 router, then on the GPU dw (molora_backward) -> dlogits ->
    router gradients, against the oracle chain apply_backward -> route_topk_backward ->
    router_backward."""
    m = need_gpu()
    c = synth.qwen_layer()
    r, t = c.router, c.targets[0]
    N, K, k = c.N, c.K, c.k
    xf = f64(t.x)
    logits = router_logits(xf, f64(r["W1"]), r["b1"].astype(np.float64), f64(r["W2"]), r["b2"].astype(np.float64))
    idx, w, _ = route_topk(logits, k)
    w32 = w.astype(np.float32)
    gy, _ = synth.grad_case(c.case_id, N, t.d_in, t.d_out)
    A, B = dev_bf16(t.A), dev_bf16(t.B)
    hs = m.molora_hotset_init([(A, B)], c.scale)
    hs_t = m.molora_hotset_init_transposed([(A, B)], c.scale)
    idx_d = dev(idx.reshape(-1).astype(np.int32))
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(idx_d, dev(w32.reshape(-1)), K, k)
    _, _, _, dw = m.molora_backward(hs, hs_t, dev_bf16(t.x), dev_bf16(gy), offsets, perm, perm_w, inv, k=k,
                                    want=("dw",))
    dl = m.molora_route_topk_backward(idx_d.view(N, k), dev(w32), dw.view(N, k), K)
    out = m.molora_router_backward(dev_bf16(t.x), dev_bf16(np.ascontiguousarray(r["W1"].T)), dev(r["b1"]),
                                   dev_bf16(np.ascontiguousarray(r["W2"].T)), dl, want=("dW1", "db1", "dW2", "db2"))
    torch.cuda.synchronize()
    _, o_o, p_o, pw_o, _ = dispatch(idx, w32.astype(np.float64), K)
    _, _, _, rdw = apply_backward(xf, f64(gy), f64(t.A), f64(t.B), c.scale, p_o, pw_o, o_o, k)
    _close(host(dw), rdw, "dw")
    rdl = route_topk_backward(w32.astype(np.float64), idx, rdw.reshape(N, k), K)
    _close(host(dl), rdl, "dlogits")
    dW1, db1, dW2, db2, _ = router_backward(xf, f64(r["W1"]), r["b1"].astype(np.float64), f64(r["W2"]), rdl)
    allow, _ = _allowances(xf, f64(r["W1"]), f64(r["W2"]), r["b1"].astype(np.float64), rdl)
    _close(host(out["dW1"]), dW1.T, "dW1", allow["dW1"].T)
    _close(host(out["db1"]), db1, "db1", allow["db1"])
    _close(host(out["dW2"]), dW2.T, "dW2", allow["dW2"].T)
    _close(host(out["db2"]), db2, "db2")
