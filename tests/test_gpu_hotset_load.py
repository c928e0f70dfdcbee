"""GPU parity of molora_hotset_load (paging one adapter into its fixed hot-set slot):
the slab it leaves is byte for byte the slab molora_hotset_init builds from the same
weights, and a step over paged adapters matches the CPU oracle, eagerly and from a graph
replayed while the paged weights change."""
import numpy as np
import pytest
import torch

import synth
from oracle import apply, dispatch, route_vocab
from tests.gpu_util import check_float_output, dev, dev_bf16, f64, host, need_gpu

pytestmark = pytest.mark.gpu


def hotset(m, targets, scale, layout=0, slab=None):
    return m.molora_hotset_init([(dev_bf16(A), dev_bf16(B)) for A, B in targets], scale, layout=layout, slab=slab)


def oracle_step(c, A, B):
    """Oracle route + dispatch + apply of target 0 of a vocab case with adapter weights A, B."""
    t = c.targets[0]
    idx, w = route_vocab(c.ids, c.bounds)
    counts, offsets, perm, perm_w, inv = dispatch(idx, w.astype(np.float64), c.K)
    return apply(f64(t.y0), f64(t.x), f64(A), f64(B), c.scale, perm, perm_w, offsets, 1)


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("r", [8, 16, 64])
def test_load_equals_init_bytes(layout, r):
    """Two targets of different shapes; every adapter of both paged over an old hot set."""
    m = need_gpu()
    K = 5
    dims = [(512, 384), (256, 640)]
    old = [synth._lora_weights(11, i, K, a, b, r) for i, (a, b) in enumerate(dims)]
    new = [synth._lora_weights(12, i, K, a, b, r) for i, (a, b) in enumerate(dims)]
    # one zero-filled slab for both, so alignment padding and the indirect layout's pointer
    # tables (absolute slot addresses) are the same on both sides
    slab = torch.zeros(m.molora_hotset_bytes(K, r, dims, layout), dtype=torch.uint8, device="cuda")
    hs = hotset(m, old, 2.0, layout, slab)
    before = slab.clone()
    for t, (A, B) in enumerate(new):
        for e in range(K):
            m.molora_hotset_load(hs, t, e, dev_bf16(A[e]), dev_bf16(B[e]))
    torch.cuda.synchronize()
    paged = slab.clone()
    hotset(m, new, 2.0, layout, slab)  # init over the same slab
    assert not torch.equal(before, slab)
    assert torch.equal(paged, slab)


def test_partial_paging_step_matches_oracle():
    """Adapters 1 and 3 paged in; 0 and 2 keep the hot set's original weights."""
    m = need_gpu()
    c = synth.modality4()
    t = c.targets[0]
    oldA, oldB = synth._lora_weights(13, 0, c.K, t.d_in, t.d_out, c.r)
    hs = hotset(m, [(oldA, oldB)], c.scale)
    A, B = oldA.copy(), oldB.copy()
    for e in (1, 3):
        A[e], B[e] = t.A[e], t.B[e]
        m.molora_hotset_load(hs, 0, e, dev_bf16(t.A[e]), dev_bf16(t.B[e]))
    ws = torch.zeros(max(m.molora_step_workspace(hs, 0, c.N), 1), dtype=torch.uint8, device="cuda")
    y, (idx, w), _ = m.molora_step_vocab(hs, dev(c.ids), c.bounds.tolist(), dev_bf16(t.x), dev_bf16(t.y0).float(),
                                         y_dtype=torch.float32, ws=ws)
    np.testing.assert_array_equal(host(idx), route_vocab(c.ids, c.bounds)[0])
    check_float_output(host(y), oracle_step(c, A, B), f64(t.y0))


@pytest.mark.parametrize("layout", [0, 1])
def test_paged_step_in_graph(layout):
    """Loads of all K adapters from a device staging buffer plus the split step, captured
    once and replayed after the staged weights change (copied in from pinned host memory
    between replays): every replay equals the eager step on the weights staged at the time,
    and the first matches the oracle."""
    m = need_gpu()
    c = synth.modality4()
    t = c.targets[0]
    hs = hotset(m, [synth._lora_weights(14, 0, c.K, t.d_in, t.d_out, c.r)], c.scale, layout)
    ids, x, y0 = dev(c.ids), dev_bf16(t.x), dev_bf16(t.y0).float()
    y = torch.empty(c.N, t.d_out, dtype=torch.float32, device="cuda")
    route = (torch.empty(c.N, dtype=torch.int32, device="cuda"), torch.empty(c.N, dtype=torch.float32, device="cuda"))
    meta = (torch.empty(c.K, dtype=torch.int32, device="cuda"), torch.empty(c.K + 1, dtype=torch.int32, device="cuda"),
            torch.empty(c.N, dtype=torch.int32, device="cuda"), torch.empty(c.N, dtype=torch.float32, device="cuda"),
            torch.empty(c.N, dtype=torch.int32, device="cuda"))
    ws = torch.zeros(max(m.molora_step_workspace(hs, 0, c.N), 1), dtype=torch.uint8, device="cuda")
    hostA = torch.empty(c.K, t.d_in, c.r, dtype=torch.bfloat16).pin_memory()
    hostB = torch.empty(c.K, c.r, t.d_out, dtype=torch.bfloat16).pin_memory()
    stA = torch.empty(c.K, t.d_in, c.r, dtype=torch.bfloat16, device="cuda")
    stB = torch.empty(c.K, c.r, t.d_out, dtype=torch.bfloat16, device="cuda")
    weights = [(t.A, t.B), synth._lora_weights(15, 0, c.K, t.d_in, t.d_out, c.r)]

    def stage(i):
        A, B = weights[i]
        hostA.copy_(torch.from_numpy(A.view(np.int16)).view(torch.bfloat16))
        hostB.copy_(torch.from_numpy(B.view(np.int16)).view(torch.bfloat16))
        stA.copy_(hostA, non_blocking=True)
        stB.copy_(hostB, non_blocking=True)
        torch.cuda.synchronize()

    def step():
        for e in range(c.K):
            m.molora_hotset_load(hs, 0, e, stA[e], stB[e])
        m.molora_step_vocab(hs, ids, c.bounds.tolist(), x, y0, y=y, route=route, meta=meta, ws=ws)

    eager = []
    for i in range(2):
        stage(i)
        step()
        torch.cuda.synchronize()
        eager.append(host(y).copy())
    check_float_output(eager[0], oracle_step(c, t.A, t.B), f64(t.y0))
    assert not np.array_equal(eager[0], eager[1])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        i = rep % 2
        stage(i)
        y.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), eager[i])


def test_load_rejects_bad_arguments():
    m = need_gpu()
    c = synth.tiny_vocab()
    t = c.targets[0]
    hs = hotset(m, [(t.A, t.B)], c.scale)
    A, B = dev_bf16(t.A[0]), dev_bf16(t.B[0])
    for target, e in ((1, 0), (-1, 0), (0, c.K), (0, -1)):
        with pytest.raises(m.MoloraError) as ei:
            m.molora_hotset_load(hs, target, e, A, B)
        assert ei.value.code == 1
    with pytest.raises(ValueError):
        m.molora_hotset_load(hs, 0, 0, dev_bf16(t.A[0][:128]), B)
