"""Pins for the oracle's synthetic decoder (oracle/transformer.py), independent of its code.

* torch (fp64, CPU) with its own library routines -- F.rms_norm, F.scaled_dot_product_attention
  with is_causal=True, F.silu -- and the LoRA deltas written per token slot (Figure 2's
  weighted sum), on the same weights: the exact-definition oracle (store = identity) must agree
  to rounding.
* brute-force attention in pure Python loops on a tiny case;
* causality (changing later tokens leaves earlier outputs unchanged) and sequence independence
  (permuting the batch's sequences permutes the outputs);
* with every LoRA B zero the routing has no effect;
* the bf16 storage rounding against torch's own bf16 conversion.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import bf16_to_f64, route_vocab
from oracle import transformer as T


def f64(b):
    return bf16_to_f64(b)


def _model(cid, d, L, K, r, n_seq, seq_len):
    layers_b = synth.xf_layers(cid, d, L, K, r)
    layers = []
    for lb in layers_b:
        lay = {n: f64(v) for n, v in lb.items() if n not in ("A", "B")}
        lay["A"] = [f64(a) for a in lb["A"]]
        lay["B"] = [f64(b) for b in lb["B"]]
        layers.append(lay)
    xb, ids, bounds, labels = synth.xf_batch(cid, n_seq, seq_len, d, K, mean_run=8.0)
    idx, w = route_vocab(ids, bounds)
    return layers, f64(xb), idx, w


def _torch_forward(x, layers, scale, idx, w, n_seq, seq_len):
    """The decoder written with torch's library routines (a different implementation)."""
    N, d = x.shape
    H = d // 128
    t = torch.tensor(x)
    idx_t = torch.tensor(np.asarray(idx).reshape(N, -1).astype(np.int64))
    w_t = torch.tensor(np.asarray(w, np.float64).reshape(N, -1))

    def lin(inp, W, A, B):
        base = inp @ torch.tensor(W).T
        delta = torch.zeros_like(base)
        for tok in range(N):
            for s in range(idx_t.shape[1]):
                e = int(idx_t[tok, s])
                if e >= 0:
                    delta[tok] += w_t[tok, s] * scale * ((inp[tok] @ torch.tensor(A[e])) @ torch.tensor(B[e]))
        return base + delta

    for L in layers:
        h = F.rms_norm(t, (d,), torch.tensor(L["norm1"]), eps=1e-6)
        q, k, v = (lin(h, L[n], L["A"][i], L["B"][i]) for i, n in enumerate(("Wq", "Wk", "Wv")))

        def heads(a):
            return a.view(n_seq, seq_len, H, 128).transpose(1, 2)

        att = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=True)
        att = att.transpose(1, 2).reshape(N, d)
        t = t + lin(att, L["Wo"], L["A"][3], L["B"][3])
        h2 = F.rms_norm(t, (d,), torch.tensor(L["norm2"]), eps=1e-6)
        g = lin(h2, L["Wgate"], L["A"][4], L["B"][4])
        u = lin(h2, L["Wup"], L["A"][5], L["B"][5])
        t = t + lin(F.silu(g) * u, L["Wdown"], L["A"][6], L["B"][6])
    return t.numpy()


@pytest.mark.parametrize("d,L,K,r,n_seq,seq_len", [(256, 1, 2, 4, 2, 16), (384, 2, 3, 8, 1, 24)])
def test_forward_matches_torch_library_routines(d, L, K, r, n_seq, seq_len):
    layers, x, idx, w = _model(11 + d, d, L, K, r, n_seq, seq_len)
    got = T.forward(x, layers, 0.5, idx, w, K, n_seq, seq_len)
    ref = _torch_forward(x, layers, 0.5, idx, w, n_seq, seq_len)
    np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-9)


def test_causal_attention_brute_force():
    rng = np.random.default_rng(5)
    n_seq, S, d = 2, 5, 256
    q, k, v = (rng.standard_normal((n_seq * S, d)) for _ in range(3))
    got = T.causal_attention(q, k, v, n_seq, S)
    for b in range(n_seq):
        for h in range(2):
            for i in range(S):
                ti = b * S + i
                sc = []
                for j in range(i + 1):
                    tj = b * S + j
                    sc.append(sum(q[ti, h * 128 + c] * k[tj, h * 128 + c] for c in range(128)) / math.sqrt(128))
                m = max(sc)
                ex = [math.exp(s - m) for s in sc]
                z = sum(ex)
                for c in (0, 63, 127):
                    ref = sum(ex[j] / z * v[b * S + j, h * 128 + c] for j in range(i + 1))
                    assert abs(got[ti, h * 128 + c] - ref) < 1e-12


def test_causality_and_sequence_independence():
    d, L, K, r, n_seq, S = 256, 2, 2, 4, 3, 12
    layers, x, idx, w = _model(21, d, L, K, r, n_seq, S)
    y = T.forward(x, layers, 0.5, idx, w, K, n_seq, S)
    # change tokens 7.. of sequence 1: its tokens 0..6 and the other sequences are unchanged
    x2 = x.copy()
    x2[S + 7:2 * S] += 1.0
    y2 = T.forward(x2, layers, 0.5, idx, w, K, n_seq, S)
    np.testing.assert_array_equal(y2[:S + 7], y[:S + 7])
    np.testing.assert_array_equal(y2[2 * S:], y[2 * S:])
    assert np.abs(y2[S + 7:2 * S] - y[S + 7:2 * S]).max() > 1e-3
    # permute the sequences
    order = [2, 0, 1]
    rows = np.concatenate([np.arange(b * S, (b + 1) * S) for b in order])
    y3 = T.forward(x[rows], layers, 0.5, idx[rows], w[rows], K, n_seq, S)
    np.testing.assert_allclose(y3, y[rows], rtol=1e-12, atol=1e-12)


def test_zero_lora_makes_routing_irrelevant():
    d, L, K, r, n_seq, S = 256, 1, 3, 4, 2, 10
    layers, x, idx, w = _model(31, d, L, K, r, n_seq, S)
    for lay in layers:
        lay["B"] = [np.zeros_like(b) for b in lay["B"]]
    y1 = T.forward(x, layers, 0.5, idx, w, K, n_seq, S)
    y2 = T.forward(x, layers, 0.5, np.zeros_like(idx), np.ones_like(w), K, n_seq, S)
    np.testing.assert_allclose(y1, y2, rtol=1e-13, atol=1e-13)


def test_bf16_store_matches_torch_rounding():
    rng = np.random.default_rng(2)
    a = rng.standard_normal(10000) * 10.0 ** rng.integers(-6, 6, size=10000)
    ref = torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(T.bf16_store(a), ref)
