"""The synthetic decoder with per-token LoRA (molora_xf_forward) against the oracle's decoder.

The GPU keeps every intermediate in bf16 (unit roundoff 2^-9) and accumulates products in
fp32; the oracle takes the same storage points (oracle/transformer.py, store = bf16 rounding)
with exact fp64 arithmetic between them.  The two then differ where an fp32 sum lands on the
other side of a bf16 rounding boundary: a one-ulp (2^-8 relative) difference in a few
elements, which the following layers carry along.  Bars: relative Frobenius error
<= XF_FROB (about 2^-8 x sqrt(storage points per layer x layers)) and, per element,
|gpu - ref| <= XF_ELEM x rms(ref).  A lost LoRA term, a wrong head or mask, a misrouted token
or a transposed projection moves the output by O(1) of its scale and fails both.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import dev, dev_bf16, host, need_gpu
from oracle import bf16_to_f64, route_topk, route_vocab
from oracle import transformer as T

pytestmark = pytest.mark.gpu

XF_FROB = 1e-2
XF_ELEM = 0.1


def f64(b):
    return bf16_to_f64(b)


def _model(m, layers_b, d, f, scale, with_lora, layout=0):
    layers = []
    for lb in layers_b:
        W = [dev_bf16(lb[n]) for n in ("Wq", "Wk", "Wv", "Wo", "Wgate", "Wup", "Wdown")]
        hs = None
        if with_lora:
            hs = m.molora_hotset_init([(dev_bf16(a), dev_bf16(b)) for a, b in zip(lb["A"], lb["B"])], scale,
                                      layout=layout)
        layers.append({"norm1": dev_bf16(lb["norm1"]), "norm2": dev_bf16(lb["norm2"]), "W": W, "lora": hs})
    return m.XfModel(d, f, layers)


def _oracle_layers(layers_b, with_lora):
    out = []
    for lb in layers_b:
        lay = {n: f64(v) for n, v in lb.items() if n not in ("A", "B")}
        lay["A"] = [f64(a) for a in lb["A"]]
        lay["B"] = [f64(b) if with_lora else np.zeros(b.shape) for b in lb["B"]]
        out.append(lay)
    return out


def _compare(got, ref, exact=None):
    err = got - ref
    frob = np.linalg.norm(err) / np.linalg.norm(ref)
    rms = np.sqrt(np.mean(ref * ref))
    mx = float(np.max(np.abs(err)))
    msg = f"frob {frob:.2e}, max {mx:.2e} (rms {rms:.2e})"
    if exact is not None:
        msg += f", vs the exact fp64 definition {np.linalg.norm(got - exact) / np.linalg.norm(exact):.2e}"
    print(msg)
    assert frob <= XF_FROB, msg
    assert mx <= XF_ELEM * rms, msg


def _run(m, cid, d, L, K, r, n_seq, seq_len, k=1, with_lora=True, layout=0, idx=None, w=None, scale=0.5):
    f = synth.xf_mlp_width(d)
    layers_b = synth.xf_layers(cid, d, L, K, r)
    xb, ids, bounds, labels = synth.xf_batch(cid, n_seq, seq_len, d, K, mean_run=16.0)
    if idx is None:
        if k == 1:
            idx, w = route_vocab(ids, bounds)
            w = w.astype(np.float32)
        else:
            logits = np.random.default_rng(cid).standard_normal((n_seq * seq_len, K))
            i2, w2, _ = route_topk(logits, k)
            idx, w = i2.reshape(-1).astype(np.int32), w2.reshape(-1).astype(np.float32)
    model = _model(m, layers_b, d, f, scale, with_lora, layout)
    N = n_seq * seq_len
    route = None
    if with_lora:
        _, offsets, perm, perm_w, inv = m.molora_dispatch(dev(np.asarray(idx, np.int32)), dev(np.asarray(w, np.float32)),
                                                          K, k)
        route = (offsets, perm, perm_w, inv)
    x = dev_bf16(xb)
    y = m.molora_xf_forward(model, x, n_seq, seq_len, route=route, k=k)
    torch.cuda.synchronize()
    lay = _oracle_layers(layers_b, with_lora)
    idx_o = np.asarray(idx).reshape(N, k) if k > 1 else np.asarray(idx)
    w_o = np.asarray(w, np.float64).reshape(N, k) if k > 1 else np.asarray(w, np.float64)
    ref = T.forward(f64(xb), lay, scale, idx_o, w_o, K, n_seq, seq_len, store=T.bf16_store)
    exact = T.forward(f64(xb), lay, scale, idx_o, w_o, K, n_seq, seq_len)
    _compare(host(y), ref, exact)
    return model, x, y


@pytest.mark.parametrize("d,L,K,r,n_seq,seq_len,layout", [
    (256, 2, 4, 8, 2, 64, 0),
    (256, 1, 2, 16, 3, 37, 1),
    (512, 2, 3, 16, 1, 100, 0),
    (1024, 2, 4, 16, 2, 128, 0),
])
def test_decoder_vocab_routing_matches_oracle(d, L, K, r, n_seq, seq_len, layout):
    m = need_gpu()
    _run(m, 90 + d + L, d, L, K, r, n_seq, seq_len, layout=layout)


def test_decoder_top2_routing_matches_oracle():
    m = need_gpu()
    _run(m, 95, 256, 2, 4, 16, 2, 48, k=2)


def test_decoder_without_lora_matches_oracle():
    m = need_gpu()
    _run(m, 96, 384, 2, 2, 8, 2, 40, with_lora=False)


def test_per_sequence_pass_routing_matches_oracle():
    """A per-sequence pass: every token on adapter 1 with weight 1 (the comparator's routing)."""
    m = need_gpu()
    n_seq, seq_len = 2, 50
    N = n_seq * seq_len
    _run(m, 97, 256, 2, 3, 8, n_seq, seq_len, idx=np.ones(N, np.int32), w=np.ones(N, np.float32))


def test_decoder_in_place_and_repeatable():
    m = need_gpu()
    model, x, y = _run(m, 98, 256, 1, 2, 8, 2, 32)
    # in place: x_out == x_in gives the same bits as the out-of-place call
    xb, ids, bounds, _ = synth.xf_batch(98, 2, 32, 256, 2, mean_run=16.0)
    idx, w = route_vocab(ids, bounds)
    _, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx.astype(np.int32)), dev(w.astype(np.float32)), 2, 1)
    xi = dev_bf16(xb)
    m.molora_xf_forward(model, xi, 2, 32, route=(offsets, perm, perm_w, inv), out=xi)
    torch.cuda.synchronize()
    assert torch.equal(xi, y)
