"""Backward of the routed LoRA on the GPU against the oracle's apply_backward.

molora_backward (dx through the transposed twin hot set, dA, dB, dw through the pair shrinks,
the pair pass and the chunked weight-gradient reduction) on seeded inputs: ragged sizes,
unrouted tokens, K up to 64, ranks 8..64, k up to 4, both layouts, bf16 and fp32 dx, the
4-modality shape and the full 16384-token Zipf stress routing.  Bars: dx as every apply output
(one bf16 ulp, or the fp32 bars); dA, dB and dw (fp32) within GRAD_REL of their largest
magnitude -- fp32 accumulation of exact bf16 products, with the per-pair vectors carried as
bf16 hi + lo, leaves errors near 1e-6 of that scale, so 1e-4 flags any lost or misplaced term.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import check_bf16_output, check_float_output, dev, dev_bf16, f64, host, need_gpu
from oracle import apply_backward, dispatch, route_topk, route_vocab

pytestmark = pytest.mark.gpu

GRAD_REL = 1e-4


def check_grad(got: np.ndarray, ref: np.ndarray, name: str):
    scale = max(float(np.max(np.abs(ref))) if ref.size else 0.0, 1e-30)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= GRAD_REL * scale, f"{name}: max-abs error {err:.3e} > {GRAD_REL} x {scale:.3e}"


def _routing(case_id, N, K, k, unrouted):
    """Top-k routing from seeded logits (fp32 weights, as the GPU receives them); a fraction of
    the tokens' first slot unrouted (-1)."""
    g = np.random.default_rng(1000 + case_id)
    logits = g.standard_normal((N, K)).astype(np.float32)
    idx, w, _ = route_topk(logits.astype(np.float64), k)
    idx = idx.copy()
    if unrouted > 0:
        drop = g.random(N) < unrouted
        idx[drop, 0] = -1
    return idx.reshape(-1).astype(np.int32), w.reshape(-1).astype(np.float32)


def _run(m, case_id, N, d_in, d_out, K, r, k, layout=0, dx_f32=False, unrouted=0.1, idx=None, w=None,
         want=("dx", "dA", "dB", "dw")):
    A = synth.normal_bf16(case_id, synth.T_A, (K, d_in, r), std=1.0 / np.sqrt(d_in))
    B = synth.normal_bf16(case_id, synth.T_B, (K, r, d_out), std=1.0 / np.sqrt(r))
    x = synth.normal_bf16(case_id, synth.T_X, (N, d_in))
    gy, dx0 = synth.grad_case(case_id, N, d_in, d_out)
    if idx is None:
        idx, w = _routing(case_id, N, K, k, unrouted)
    scale = 2.0
    Ad, Bd = dev_bf16(A), dev_bf16(B)
    hs = m.molora_hotset_init([(Ad, Bd)], scale, layout=layout)
    hs_t = m.molora_hotset_init_transposed([(Ad, Bd)], scale, layout=layout)
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    dx0_t = dev_bf16(dx0)
    if dx_f32:
        dx0_t = dx0_t.float()
    dx, dA, dB, dw = m.molora_backward(hs, hs_t, dev_bf16(x), dev_bf16(gy), offsets, perm, perm_w, inv, k=k,
                                       dx0=dx0_t if "dx" in want else None, want=want)
    torch.cuda.synchronize()
    c_o, o_o, p_o, pw_o, inv_o = dispatch(idx, w.astype(np.float64), K)
    rdx, rdA, rdB, rdw = apply_backward(f64(x), f64(gy), f64(A), f64(B), scale, p_o, pw_o, o_o, k)
    out = {}
    if "dx" in want:
        ref = f64(dx0) + rdx
        if dx_f32:
            check_float_output(host(dx), ref, f64(dx0))
        else:
            check_bf16_output(host(dx), ref)
        out["dx"] = dx
    if "dA" in want:
        check_grad(host(dA), rdA, "dA")
    if "dB" in want:
        check_grad(host(dB), rdB, "dB")
    if "dw" in want:
        got = host(dw)
        check_grad(got, rdw, "dw")
        assert np.all(got[np.asarray(inv_o) < 0] == 0.0)  # unrouted pairs: exactly 0
    return hs, hs_t, (dx, dA, dB, dw)


SHAPES = [  # N, d_in, d_out, K, r, k
    (256, 512, 256, 4, 8, 1),
    (300, 256, 640, 5, 16, 2),
    (777, 1024, 512, 8, 48, 3),
    (1000, 512, 512, 64, 16, 2),
    (513, 384, 128, 16, 64, 4),
    (1, 256, 256, 4, 16, 1),
    (65, 128, 256, 3, 32, 2),
]


@pytest.mark.parametrize("N,d_in,d_out,K,r,k", SHAPES)
@pytest.mark.parametrize("layout", [0, 1])
def test_backward_matches_oracle(N, d_in, d_out, K, r, k, layout):
    m = need_gpu()
    _run(m, 40 + N % 97, N, d_in, d_out, K, r, k, layout=layout)


@pytest.mark.parametrize("dx_f32", [False, True])
def test_backward_dx_dtypes_and_in_place(dx_f32):
    m = need_gpu()
    _run(m, 51, 640, 512, 384, 4, 16, 2, dx_f32=dx_f32)


@pytest.mark.parametrize("want", [("dA",), ("dB",), ("dw",), ("dx",), ("dA", "dw"), ("dx", "dB")])
def test_backward_subsets_of_outputs(want):
    m = need_gpu()
    _run(m, 52, 300, 256, 512, 4, 16, 1, want=want)


def test_backward_vocab_routing_with_empty_adapter():
    """k = 1 vocabulary routing (ids outside every range stay unrouted); adapter 2 owns no
    token, so its dA and dB are zero."""
    m = need_gpu()
    c = synth.vocab_case(N=512, d=512, K=4, r=8, case_id=53)
    ids = c.ids.copy()
    b = c.bounds
    ids[(ids >= b[2]) & (ids < b[3])] = b[0]  # adapter 2 gets nothing
    idx, w = route_vocab(ids, b)
    _, _, (dx, dA, dB, dw) = _run(m, 53, 512, 512, 512, 4, 8, 1, idx=idx.astype(np.int32), w=w.astype(np.float32))
    assert not host(dA)[2].any() and not host(dB)[2].any()


def test_backward_modality4_shape():
    """The 4-modality shape: 2048 tokens, d = 4096, K = 4, rank 16, one adapter per token."""
    m = need_gpu()
    _run(m, 54, 2048, 4096, 4096, 4, 16, 1, unrouted=0.0)


@pytest.mark.parametrize("k", [1, 2])
def test_backward_stress_full_size(k):
    """16384 tokens, K = 16 adapters of rank 64, d = 4096, Zipf-skewed top-k routing: every
    output element against the oracle."""
    m = need_gpu()
    c = synth.stress(k)
    idx, w, _ = route_topk(c.logits.astype(np.float64), k)
    _run(m, 4, c.N, 4096, 4096, 16, 64, k, idx=idx.reshape(-1).astype(np.int32),
         w=w.reshape(-1).astype(np.float32))


def test_backward_empty_batch_zeroes_weight_gradients():
    m = need_gpu()
    K, d_in, d_out, r = 3, 256, 128, 16
    A = torch.zeros(K, d_in, r, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(K, r, d_out, dtype=torch.bfloat16, device="cuda")
    hs = m.molora_hotset_init([(A, B)], 1.0)
    hs_t = m.molora_hotset_init_transposed([(A, B)], 1.0)
    offsets = torch.zeros(K + 1, dtype=torch.int32, device="cuda")
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    dA = torch.full((K, d_in, r), 7.0, device="cuda")
    dB = torch.full((K, r, d_out), 7.0, device="cuda")
    m.molora_backward(hs, hs_t, torch.empty(0, d_in, dtype=torch.bfloat16, device="cuda"),
                      torch.empty(0, d_out, dtype=torch.bfloat16, device="cuda"), offsets, e,
                      torch.empty(0, device="cuda"), e, dA=dA, dB=dB, want=("dA", "dB"))
    torch.cuda.synchronize()
    assert not dA.any() and not dB.any()


def test_backward_graph_replays_and_determinism():
    """Captured once, replayed three times with eager work in between: every replay equals
    the eager call bit for bit (the sums run in a fixed order)."""
    m = need_gpu()
    N, d_in, d_out, K, r, k = 1024, 512, 512, 8, 16, 2
    hs, hs_t, (dx, dA, dB, dw) = _run(m, 55, N, d_in, d_out, K, r, k)
    x = dev_bf16(synth.normal_bf16(55, synth.T_X, (N, d_in)))
    gy_b, dx0_b = synth.grad_case(55, N, d_in, d_out)
    gy, dx0 = dev_bf16(gy_b), dev_bf16(dx0_b)
    idx, w = _routing(55, N, K, k, 0.1)
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    outs = [torch.empty_like(dx), torch.empty_like(dA), torch.empty_like(dB), torch.empty_like(dw)]
    ws = torch.zeros(m.molora_backward_workspace(hs, hs_t, N, k), dtype=torch.uint8, device="cuda")

    def call():
        m.molora_backward(hs, hs_t, x, gy, offsets, perm, perm_w, inv, k=k, dx0=dx0, dx=outs[0], dA=outs[1],
                          dB=outs[2], dw=outs[3], ws=ws)

    call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    for a, b in zip(eager, (dx, dA, dB, dw)):
        assert torch.equal(a, b)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    for rep in range(3):
        for t in outs:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, outs):
            assert torch.equal(a, b), f"replay {rep}"
        y = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")  # unrelated eager work
        del y
