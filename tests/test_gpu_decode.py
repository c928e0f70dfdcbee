"""GPU parity of the decode expand: the skinny path with k = 2..4 at most 1024 tokens and
K * r_pad <= 1024 (one h-sum launch, then one launch over (target, 32-column slice) that keeps
every adapter's B^T slice in LDS and sums a token's routed pairs in registers).  Covered: the
28-layer stack's projection shapes (K = 16, r = 64, k = 2) and k = 3, 4, K = 64 at rank 16 (the
LDS bound), ranks 8 and 48 (rank blocks 1 and 3), 1 .. 1024 tokens with ragged row blocks,
unrouted slots and tokens, a token routed twice to one adapter, bf16 and fp32 y, in place, the
indirect slab layout; the same bits on a second run and from molora_apply per target; every
output against the oracle (MoLoRA pages, thelatestinai.com: Figure 2, the routed pairs'
weighted LoRA deltas added to the base output)."""
import numpy as np
import pytest
import torch

import synth
from oracle import apply, dispatch
from tests.gpu_util import check_bf16_output, check_float_output, dev, dev_bf16, f64, host, need_gpu

pytestmark = pytest.mark.gpu

DIMS = [(1024, 512), (512, 1536), (1536, 256)]


def _targets(g, N, K, r, dims):
    tgs = []
    for di, do in dims:
        xb = synth.to_bf16_bits(g.standard_normal((N, di)).astype(np.float32))
        Ab = synth.to_bf16_bits((g.standard_normal((K, di, r)) / np.sqrt(di)).astype(np.float32))
        Bb = synth.to_bf16_bits((g.standard_normal((K, r, do)) / np.sqrt(r)).astype(np.float32))
        yb = synth.to_bf16_bits(g.standard_normal((N, do)).astype(np.float32))
        tgs.append(synth.Target("p", di, do, Ab, Bb, xb, yb))
    return tgs


def _routing(g, N, K, k, dup=True):
    idx = np.stack([g.permutation(K)[:k] for _ in range(N)]).astype(np.int32)
    w = g.uniform(0.1, 1.0, (N, k)).astype(np.float32)
    idx[::5, k - 1] = -1      # fewer routed pairs than slots
    idx[1::7, 0] = -1         # a gap before the routed pairs
    idx[::13, :] = -1         # no routed pair at all
    if dup:
        idx[3::11, 1] = idx[3::11, 0]  # one adapter twice in a token's slots
    return idx.reshape(-1), w.reshape(-1)


def _oracle(t, scale, idx, w, K, k):
    _, offsets, perm, perm_w, _ = dispatch(idx, w.astype(np.float64), K)
    return apply(f64(t.y0), f64(t.x), f64(t.A), f64(t.B), scale, perm, perm_w, offsets, k)


CASES = [
    # N, K, r, k, layout
    (256, 16, 64, 2, 0),     # the stack's decode batch
    (256, 16, 64, 4, 1),
    (100, 16, 64, 3, 0),     # ragged last row block
    (1, 4, 64, 2, 0),
    (1024, 16, 64, 2, 0),    # the token bound: 8 row blocks per wave
    (333, 64, 16, 2, 1),     # K r_pad = 1024: 64 KB of B^T slices
    (200, 8, 8, 4, 0),       # rank 8 padded to 16 (one rank block)
    (160, 16, 48, 2, 0),     # rank block 3 (plain LDS placement)
]


@pytest.mark.parametrize("N,K,r,k,layout", CASES)
def test_decode_multi(N, K, r, k, layout):
    m = need_gpu()
    g = np.random.default_rng(7 * N + K + r + 3 * k + layout)
    tgs = _targets(g, N, K, r, DIMS)
    idx, w = _routing(g, N, K, k, dup=k >= 2 and K > 1)
    scale = 2.0
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B)) for t in tgs], scale, layout=layout)
    _, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    xs = [dev_bf16(t.x) for t in tgs]
    refs = [_oracle(t, scale, idx, w, K, k) for t in tgs]
    for y_dtype in (torch.bfloat16, torch.float32):
        y0s = [dev_bf16(t.y0).to(y_dtype) for t in tgs]
        ys = m.molora_apply_multi(hs, xs, y0s, offsets, perm, perm_w, inv, k=k, y_dtype=y_dtype,
                                  path=m.PATH_SKINNY)
        again = m.molora_apply_multi(hs, xs, y0s, offsets, perm, perm_w, inv, k=k, y_dtype=y_dtype,
                                     path=m.PATH_SKINNY)
        for i, t in enumerate(tgs):
            y = host(ys[i])
            np.testing.assert_array_equal(y, host(again[i]))
            single = m.molora_apply(hs, xs[i], y0s[i], offsets, perm, perm_w, inv, k=k, target=i,
                                    y_dtype=y_dtype, path=m.PATH_SKINNY)
            np.testing.assert_array_equal(y, host(single))
            if y_dtype == torch.float32:
                check_float_output(y, refs[i], f64(t.y0))
            else:
                check_bf16_output(y, refs[i])
        yin = [v.clone() for v in y0s]
        m.molora_apply_multi(hs, xs, yin, offsets, perm, perm_w, inv, k=k, ys=yin, path=m.PATH_SKINNY)
        for i in range(len(tgs)):
            np.testing.assert_array_equal(host(yin[i]), host(ys[i]))


def test_decode_stack_layer_auto():
    """The 28-layer stack's layer (7 Qwen3-1.7B projections, 256 tokens, K = 16, r = 64, top-2
    of Zipf logits): AUTO takes the decode expand; every target against the oracle."""
    m = need_gpu()
    N, K, r, k = 256, 16, 64, 2
    g = np.random.default_rng(2026)
    dims = [(d_in, d_out) for (_, d_in, d_out) in synth.QWEN3_1P7B_TARGETS]
    tgs = _targets(g, N, K, r, dims)
    logits = torch.from_numpy(synth.zipf_logits(5, N, K, sub=3)).to("cuda")
    _, idx, w, _ = m.molora_route_topk(k, K, logits=logits, want_flags=False)
    idx, w = idx.reshape(-1), w.reshape(-1)
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B)) for t in tgs], 2.0)
    assert m.molora_apply_path(hs, N, k, 0, target=0) == m.PATH_SKINNY
    _, offsets, perm, perm_w, inv = m.molora_dispatch(idx, w, K, k)
    xs = [dev_bf16(t.x) for t in tgs]
    y0s = [dev_bf16(t.y0) for t in tgs]
    ys = m.molora_apply_multi(hs, xs, y0s, offsets, perm, perm_w, inv, k=k)
    hi, hw = host(idx).astype(np.int32), host(w).astype(np.float32)
    for i, t in enumerate(tgs):
        check_bf16_output(host(ys[i]), _oracle(t, 2.0, hi, hw, K, k))


def test_decode_none_routed():
    """Every slot unrouted: y = y0 bit for bit (bf16 and fp32), on the decode expand."""
    m = need_gpu()
    N, K, r, k = 256, 16, 64, 2
    g = np.random.default_rng(5)
    tgs = _targets(g, N, K, r, DIMS[:1])
    idx = np.full(N * k, -1, np.int32)
    w = np.ones(N * k, np.float32)
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B)) for t in tgs], 1.0)
    _, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    for y_dtype in (torch.bfloat16, torch.float32):
        y0 = dev_bf16(tgs[0].y0).to(y_dtype)
        y = m.molora_apply(hs, dev_bf16(tgs[0].x), y0, offsets, perm, perm_w, inv, k=k, y_dtype=y_dtype,
                           path=m.PATH_SKINNY)
        np.testing.assert_array_equal(host(y), host(y0))


def test_decode_graph_replays():
    """The decode path captured in a HIP graph (h rows, then the expand of 3 targets): every
    replay, with eager calls and synchronisations between them, gives the eager bits."""
    m = need_gpu()
    N, K, r, k = 256, 16, 64, 3
    g = np.random.default_rng(77)
    tgs = _targets(g, N, K, r, DIMS)
    idx, w = _routing(g, N, K, k)
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B)) for t in tgs], 2.0)
    _, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    xs = [dev_bf16(t.x) for t in tgs]
    y0s = [dev_bf16(t.y0) for t in tgs]
    tids = list(range(len(tgs)))
    ws = torch.zeros(m.molora_apply_multi_workspace(hs, tids, N, k, m.PATH_SKINNY, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    eager = [host(v) for v in m.molora_apply_multi(hs, xs, y0s, offsets, perm, perm_w, inv, k=k,
                                                   path=m.PATH_SKINNY, ws=ws)]
    outs = [torch.empty_like(v) for v in y0s]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.molora_apply_multi(hs, xs, y0s, offsets, perm, perm_w, inv, k=k, ys=outs, path=m.PATH_SKINNY, ws=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        m.molora_apply_multi(hs, xs, y0s, offsets, perm, perm_w, inv, k=k, ys=outs, path=m.PATH_SKINNY, ws=ws)
    for rep in range(3):
        for v in outs:
            v.zero_()
        m.molora_apply_multi(hs, xs, y0s, offsets, perm, perm_w, inv, k=k, path=m.PATH_SKINNY)  # eager work between
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            graph.replay()
        torch.cuda.synchronize()
        for i in range(len(tgs)):
            np.testing.assert_array_equal(host(outs[i]), eager[i])


@pytest.mark.parametrize("N,K,r,k", [(1025, 16, 64, 2), (1025, 64, 16, 2), (256, 64, 32, 2), (256, 8, 64, 5)])
def test_decode_bounds_fall_back(N, K, r, k):
    """Just past the decode path's bounds (1025 tokens; K r_pad = 2048; k = 5) the skinny path
    runs its rank passes or token expand: multi-target equals per-target calls and the oracle."""
    m = need_gpu()
    g = np.random.default_rng(N + K + r + k)
    tgs = _targets(g, N, K, r, DIMS[:2])
    idx, w = _routing(g, N, K, k)
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B)) for t in tgs], 2.0)
    _, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    xs = [dev_bf16(t.x) for t in tgs]
    y0s = [dev_bf16(t.y0) for t in tgs]
    ys = m.molora_apply_multi(hs, xs, y0s, offsets, perm, perm_w, inv, k=k, path=m.PATH_SKINNY)
    for i, t in enumerate(tgs):
        single = m.molora_apply(hs, xs[i], y0s[i], offsets, perm, perm_w, inv, k=k, target=i, path=m.PATH_SKINNY)
        np.testing.assert_array_equal(host(ys[i]), host(single))
        check_bf16_output(host(ys[i]), _oracle(t, 2.0, idx, w, K, k))
