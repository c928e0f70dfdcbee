"""GPU parity of the 64-token block path's dense-slot kernels (hot sets whose adapters' 512-wide
slices fit in LDS together: K * r_pad <= 64): every rank block (r = 16 .. 64), k from 1 to K
with repeated adapters in a token's slots, unrouted pairs and tokens, ragged N (an odd number
of 64-token blocks, a partial last block), ragged d_in / d_out (a last slice of one step, a
last column slice of one 128-column block), the direct and indirect slab layouts, bf16 and
fp32 y, in place; several targets of which some read the same x, in one call, bit for bit
equal to one call per target and within the bars of the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import apply, dispatch
from tests.gpu_util import check_bf16_output, check_float_output, dev, dev_bf16, f64, host, need_gpu

pytestmark = pytest.mark.gpu


def _routing(g, N, K, k):
    """Random adapters per slot (repeats allowed), gate weights, some unrouted pairs/tokens."""
    idx = g.integers(0, K, (N, k)).astype(np.int32)
    w = g.uniform(0.1, 1.0, (N, k)).astype(np.float32)
    idx[::7, 0] = -1
    idx[::11, :] = -1
    return idx.reshape(-1), w.reshape(-1)


def _target(g, N, di, do, K, r, x=None):
    xb = x if x is not None else synth.to_bf16_bits(g.standard_normal((N, di)).astype(np.float32))
    Ab = synth.to_bf16_bits((g.standard_normal((K, di, r)) / np.sqrt(di)).astype(np.float32))
    Bb = synth.to_bf16_bits((g.standard_normal((K, r, do)) / np.sqrt(r)).astype(np.float32))
    yb = synth.to_bf16_bits(g.standard_normal((N, do)).astype(np.float32))
    return synth.Target("p", di, do, Ab, Bb, xb, yb)


def _oracle(t, scale, idx, w, K, k):
    counts, offsets, perm, perm_w, inv = dispatch(idx, w.astype(np.float64), K)
    return apply(f64(t.y0), f64(t.x), f64(t.A), f64(t.B), scale, perm, perm_w, offsets, k)


CASES = [
    # N, K, r, k, layout
    (4100, 4, 16, 2, 0),  # 65 blocks: the last 128-token workgroup holds one block
    (300, 2, 32, 2, 1),
    (77, 1, 64, 1, 0),
    (129, 1, 48, 1, 1),   # rank block 3
    (1000, 4, 16, 4, 0),
    (1, 3, 16, 1, 0),
    (640, 4, 8, 3, 1),    # r = 8 padded to 16
]


@pytest.mark.parametrize("N,K,r,k,layout", CASES)
def test_dense_block_multi_targets(N, K, r, k, layout):
    m = need_gpu()
    g = np.random.default_rng(7 * N + 13 * K + r + k + layout)
    # q-, k- and up-like targets read the same x; the last reads its own (d_in 640: a last
    # slice of one step); d_out 384 leaves a last column slice of three 128-column blocks
    t0 = _target(g, N, 512, 640, K, r)
    t1 = _target(g, N, 512, 384, K, r, x=t0.x)
    t2 = _target(g, N, 512, 1536, K, r, x=t0.x)
    t3 = _target(g, N, 640, 512, K, r)
    tgs = [t0, t1, t2, t3]
    idx, w = _routing(g, N, K, k)
    scale = 2.0
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B)) for t in tgs], scale, layout=layout)
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    xs = [dev_bf16(t.x) for t in tgs]
    xs[1] = xs[0]
    xs[2] = xs[0]  # the same device rows: one x group
    order = [2, 0, 3, 1]
    for y_dtype in (torch.bfloat16, torch.float32):
        y0s = [dev_bf16(t.y0).to(y_dtype) for t in tgs]
        ys = m.molora_apply_multi(hs, [xs[i] for i in order], [y0s[i] for i in order], offsets, perm, perm_w, inv,
                                  k=k, targets=order, y_dtype=y_dtype, path=m.PATH_BLOCK)
        torch.cuda.synchronize()
        for j, i in enumerate(order):
            single = m.molora_apply(hs, xs[i], y0s[i], offsets, perm, perm_w, inv, k=k, target=i, y_dtype=y_dtype,
                                    path=m.PATH_BLOCK)
            np.testing.assert_array_equal(host(ys[j]), host(single))
            ref = _oracle(tgs[i], scale, idx, w, K, k)
            if y_dtype == torch.float32:
                check_float_output(host(ys[j]), ref, f64(tgs[i].y0))
            else:
                check_bf16_output(host(ys[j]), ref)
        # in place, twice in a row on the same workspace
        for _ in range(2):
            yin = [v.clone() for v in y0s]
            m.molora_apply_multi(hs, xs, yin, offsets, perm, perm_w, inv, k=k, ys=yin, path=m.PATH_BLOCK)
            torch.cuda.synchronize()
            for i in range(len(tgs)):
                np.testing.assert_array_equal(host(yin[i]), host(ys[order.index(i)]))


def test_dense_block_deterministic_and_repeat_routing():
    """Two runs give the same bits; a token routed twice to one adapter equals weight w1 + w2
    on it once (the oracle's sum over pairs), to the bars."""
    m = need_gpu()
    g = np.random.default_rng(5)
    N, K, r, k = 700, 4, 16, 2
    t = _target(g, N, 1024, 1024, K, r)
    e = g.integers(0, K, N).astype(np.int32)
    w1 = g.uniform(0.1, 0.6, N).astype(np.float32)
    w2 = g.uniform(0.1, 0.4, N).astype(np.float32)
    idx2 = np.stack([e, e], 1).reshape(-1)
    wk2 = np.stack([w1, w2], 1).reshape(-1)
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B))], 1.5)
    x, y0 = dev_bf16(t.x), dev_bf16(t.y0).float()
    outs = []
    for _ in range(2):
        _, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx2), dev(wk2), K, 2)
        outs.append(host(m.molora_apply(hs, x, y0, offsets, perm, perm_w, inv, k=2, y_dtype=torch.float32,
                                        path=m.PATH_BLOCK)))
    np.testing.assert_array_equal(outs[0], outs[1])
    ref = _oracle(t, 1.5, e, (w1.astype(np.float64) + w2), K, 1)
    check_float_output(outs[0], ref, f64(t.y0))


@pytest.mark.parametrize("N,K,r,k,path,layout", [
    (4096, 4, 16, 2, 0, 0),    # the Qwen-layer shape: dispatch inside the shrink launch
    (300, 3, 16, 2, 4, 1),
    (1, 2, 32, 1, 4, 0),
    (5000, 4, 16, 2, 4, 0),    # 10000 pairs: dispatch first, then the dense kernels
    (700, 16, 16, 2, 4, 0),    # no dense kernels: dispatch, then the general block path
    (513, 4, 16, 3, 1, 1),     # grouped path
])
def test_dispatch_apply_multi_equals_two_calls(N, K, r, k, path, layout):
    """molora_dispatch_apply_multi = molora_dispatch + molora_apply_multi bit for bit (every
    dispatch output and every y), with unrouted and out-of-range adapters, in place too;
    and within the oracle's bars."""
    m = need_gpu()
    g = np.random.default_rng(N + 3 * K + r + k + path)
    t0 = _target(g, N, 512, 640, K, r)
    t1 = _target(g, N, 512, 384, K, r, x=t0.x)
    t2 = _target(g, N, 1024, 512, K, r)
    tgs = [t0, t1, t2]
    idx, w = _routing(g, N, K, k)
    idx[5::17] = K + 2  # outside [0, K): unrouted
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B)) for t in tgs], 1.5, layout=layout)
    xs = [dev_bf16(t.x) for t in tgs]
    xs[1] = xs[0]
    y0s = [dev_bf16(t.y0) for t in tgs]
    di, dw = dev(idx), dev(w)
    meta2 = m.molora_dispatch(di, dw, K, k)
    ref_ys = m.molora_apply_multi(hs, xs, y0s, meta2[1], meta2[2], meta2[3], meta2[4], k=k, path=path)
    ws = torch.full((max(1, m.molora_dispatch_apply_multi_workspace(hs, [0, 1, 2], N, k, path, torch.bfloat16)),),
                    0xFF, dtype=torch.uint8, device="cuda")
    for _ in range(2):
        ys, meta1 = m.molora_dispatch_apply_multi(hs, xs, y0s, di, dw, K, k, path=path, ws=ws)
        torch.cuda.synchronize()
        n_routed = int(host(meta2[1])[-1])
        for a, b, full in zip(meta1, meta2, (True, True, False, False, True)):
            if full:
                np.testing.assert_array_equal(host(a), host(b))
            else:
                np.testing.assert_array_equal(host(a)[:n_routed], host(b)[:n_routed])
        for a, b in zip(ys, ref_ys):
            np.testing.assert_array_equal(host(a), host(b))
    yin = [v.clone() for v in y0s]
    m.molora_dispatch_apply_multi(hs, xs, yin, di, dw, K, k, ys=yin, path=path, ws=ws)
    torch.cuda.synchronize()
    for a, b in zip(yin, ref_ys):
        np.testing.assert_array_equal(host(a), host(b))
    for i, t in enumerate(tgs):
        check_bf16_output(host(ys[i]), _oracle(t, 1.5, idx, w, K, k))
