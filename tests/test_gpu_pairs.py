"""GPU parity of the grouped path's pair passes (k > 1 on the 64-row grouped tiles once the
adapter pairs (a, b) hold 32 rows on average: N >= 32 K (K + 1)): each pass applies a token's
routed pairs of rank 2m and 2m + 1 together.  Covered: k = 2 .. 8 (one to four passes, an odd
k leaving a last pass of single pairs), tokens whose routed pairs stop short of the last pass
or are all unrouted, a token routed twice to one adapter, ranks 16 .. 64 (rank block 3, the
padded rank 8), a last 256-wide column slice of one 128-column block, bf16 and fp32 y, in place,
the direct and indirect slab layouts, the fixed-tiling comparator; the same bits on a second
run (the tuple sort is not stable, a row's result does not depend on its position) and within
the oracle's bars."""
import numpy as np
import pytest
import torch

import synth
from oracle import apply, dispatch
from tests.gpu_util import check_bf16_output, check_float_output, dev, dev_bf16, f64, host, need_gpu

pytestmark = pytest.mark.gpu


def _case(g, N, di, do, K, r, k):
    xb = synth.to_bf16_bits(g.standard_normal((N, di)).astype(np.float32))
    Ab = synth.to_bf16_bits((g.standard_normal((K, di, r)) / np.sqrt(di)).astype(np.float32))
    Bb = synth.to_bf16_bits((g.standard_normal((K, r, do)) / np.sqrt(r)).astype(np.float32))
    yb = synth.to_bf16_bits(g.standard_normal((N, do)).astype(np.float32))
    idx = np.stack([g.permutation(K)[:k] for _ in range(N)]).astype(np.int32)
    w = g.uniform(0.1, 1.0, (N, k)).astype(np.float32)
    idx[::5, k - 1] = -1        # the last slot unrouted: fewer routed pairs than slots
    idx[1::7, 0] = -1           # a gap before the routed pairs
    idx[::13, :] = -1           # no routed pair at all
    if k >= 2:
        idx[3::11, 1] = idx[3::11, 0]  # one adapter twice in a token's slots
    return synth.Target("p", di, do, Ab, Bb, xb, yb), idx.reshape(-1), w.reshape(-1)


def _oracle(t, scale, idx, w, K, k):
    counts, offsets, perm, perm_w, inv = dispatch(idx, w.astype(np.float64), K)
    return apply(f64(t.y0), f64(t.x), f64(t.A), f64(t.B), scale, perm, perm_w, offsets, k)


CASES = [
    # N, K, r, k, d_in, d_out, layout, path
    (700, 4, 64, 2, 512, 640, 0, 1),     # one pass; d_out 640: a last slice of one 128 block
    (1000, 4, 48, 3, 1024, 512, 1, 1),   # a pass of pairs, then one of single pairs
    (2304, 8, 64, 4, 640, 384, 0, 1),    # 72 keys per pass, two passes
    (2304, 8, 16, 8, 512, 512, 1, 1),    # four passes
    (3000, 4, 8, 4, 512, 1024, 0, 5),    # rank 8 padded to 16; fixed 64-row tiles
    (4097, 3, 32, 2, 2048, 256, 0, 1),
]


@pytest.mark.parametrize("N,K,r,k,di,do,layout,path", CASES)
def test_pair_passes(N, K, r, k, di, do, layout, path):
    m = need_gpu()
    assert N >= 32 * K * (K + 1), "shape outside the pair-pass rule"
    g = np.random.default_rng(N + 7 * K + r + 3 * k + layout)
    t, idx, w = _case(g, N, di, do, K, r, k)
    scale = 1.25
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B))], scale, layout=layout)
    _, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    x = dev_bf16(t.x)
    ref = _oracle(t, scale, idx, w, K, k)
    for y_dtype in (torch.bfloat16, torch.float32):
        y0 = dev_bf16(t.y0).to(y_dtype)
        outs = []
        for _ in range(2):
            outs.append(host(m.molora_apply(hs, x, y0, offsets, perm, perm_w, inv, k=k, y_dtype=y_dtype,
                                            path=path)))
        np.testing.assert_array_equal(outs[0], outs[1])
        if y_dtype == torch.float32:
            check_float_output(outs[0], ref, f64(t.y0))
        else:
            check_bf16_output(outs[0], ref)
        yin = y0.clone()
        m.molora_apply(hs, x, yin, offsets, perm, perm_w, inv, k=k, y=yin, path=path)
        np.testing.assert_array_equal(host(yin), outs[0])


@pytest.mark.parametrize("mode", ["none_routed", "one_routed"])
def test_pair_passes_sparse_routing(mode):
    """Pair-pass sizes (N = 2304, K = 8, k = 4: two passes) where no token has a routed pair (y
    = y0; every pass empty) or every token has exactly one (pass 0 holds only single pairs,
    pass 1 nothing: the tokens' sums come from the carry), bf16 and fp32 y, in place."""
    m = need_gpu()
    N, K, r, k = 2304, 8, 64, 4
    g = np.random.default_rng(11 if mode == "none_routed" else 12)
    t, idx, w = _case(g, N, 512, 640, K, r, k)
    idx = idx.reshape(N, k)
    if mode == "none_routed":
        idx[:] = -1
    else:
        keep = g.integers(0, k, N)
        for j in range(k):
            idx[keep != j, j] = -1
        idx[np.arange(N), keep] = g.integers(0, K, N)
    idx = idx.reshape(-1)
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B))], 1.0)
    _, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    x = dev_bf16(t.x)
    ref = _oracle(t, 1.0, idx, w, K, k)
    for y_dtype in (torch.bfloat16, torch.float32):
        y0 = dev_bf16(t.y0).to(y_dtype)
        y = host(m.molora_apply(hs, x, y0, offsets, perm, perm_w, inv, k=k, y_dtype=y_dtype, path=m.PATH_GROUPED))
        if mode == "none_routed":
            np.testing.assert_array_equal(y, host(y0))
        elif y_dtype == torch.float32:
            check_float_output(y, ref, f64(t.y0))
        else:
            check_bf16_output(y, ref)
        yin = y0.clone()
        m.molora_apply(hs, x, yin, offsets, perm, perm_w, inv, k=k, y=yin, path=m.PATH_GROUPED)
        np.testing.assert_array_equal(host(yin), y)
