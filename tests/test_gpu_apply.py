"""GPU parity: hot set + grouped apply (all paths and layouts) against the CPU oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import apply, apply_masked_passes, dispatch, route_topk, route_vocab, router_logits
from tests.gpu_util import (DESIGN_MAXABS, check_bf16_output, check_float_output, dev, dev_bf16, f64, host,
                            need_gpu)

pytestmark = pytest.mark.gpu


def make_hotset(m, targets, scale, layout=0):
    return m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B)) for t in targets], scale, layout=layout)


def oracle_from_gpu_routing(tgt, scale, idx, w, K, k):
    """Oracle dispatch + apply on the routing the GPU produced (fp64)."""
    counts, offsets, perm, perm_w, inv = dispatch(idx, w.astype(np.float64), K)
    return apply(f64(tgt.y0), f64(tgt.x), f64(tgt.A), f64(tgt.B), scale, perm, perm_w, offsets, k)


def run_pipeline_vocab(m, case, hs, y_dtype, path=0, y=None, in_place=False):
    t = case.targets[0]
    idx, w = m.molora_route_vocab(dev(case.ids), case.bounds.tolist())
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(idx, w, case.K, 1)
    x = dev_bf16(t.x)
    y0 = dev_bf16(t.y0)
    if y_dtype == torch.float32:
        y0 = y0.float()
    out = m.molora_apply(hs, x, y0, offsets, perm, perm_w, inv, k=1, y=y0 if in_place else y, y_dtype=y_dtype,
                         path=path)
    return out, idx, w


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16])
def test_tiny_vocab_pipeline(layout, y_dtype):
    m = need_gpu()
    c = synth.tiny_vocab()
    hs = make_hotset(m, c.targets, c.scale, layout)
    y, idx, w = run_pipeline_vocab(m, c, hs, y_dtype)
    ref = oracle_from_gpu_routing(c.targets[0], c.scale, host(idx), host(w), c.K, 1)
    if y_dtype == torch.float32:
        check_float_output(host(y), ref, f64(c.targets[0].y0))
    else:
        check_bf16_output(host(y), ref)


@pytest.mark.parametrize("path", [1, 2, 3, 4])
def test_modality4_full_size(path):
    m = need_gpu()
    c = synth.modality4()
    hs = make_hotset(m, c.targets, c.scale)
    y, idx, w = run_pipeline_vocab(m, c, hs, torch.float32, path=path)
    ri, rw = route_vocab(c.ids, c.bounds)
    np.testing.assert_array_equal(host(idx), ri)
    t = c.targets[0]
    ref = oracle_from_gpu_routing(t, c.scale, ri, rw, c.K, 1)
    check_float_output(host(y), ref, f64(t.y0))
    yb, _, _ = run_pipeline_vocab(m, c, hs, torch.bfloat16, path=path)
    check_bf16_output(host(yb), ref)


def test_modality4_per_sequence_comparator():
    """K masked dense passes (per-sequence routing) give the per-token result with K*N work."""
    m = need_gpu()
    c = synth.modality4()
    t = c.targets[0]
    hs = make_hotset(m, c.targets, c.scale)
    idx, w = m.molora_route_vocab(dev(c.ids), c.bounds.tolist())
    offs, perm, pw = m.molora_seqpass_meta(idx, c.K)
    ho = host(offs)
    for e in range(c.K):
        assert ho[e, e] == 0 and ho[e, e + 1] == c.N  # pass e applies adapter e to all N tokens
    x = dev_bf16(t.x)
    y = dev_bf16(t.y0).float()
    inv = perm  # identity
    for e in range(c.K):
        m.molora_apply(hs, x, y, offs[e].contiguous(), perm, pw[e].contiguous(), inv, k=1, y=y, path=1)
    ri, rw = route_vocab(c.ids, c.bounds)
    ref = apply_masked_passes(f64(t.y0), f64(t.x), f64(t.A), f64(t.B), c.scale, ri, rw)
    check_float_output(host(y), ref, f64(t.y0))


@pytest.mark.parametrize("case", ["tiny", "modality4"])
def test_k1_paths_deterministic_and_close(case):
    """The grouped and the tile paths split the reductions differently, so they agree to the
    rounding of the bf16 output, not bit for bit; each is deterministic (same bits on a repeat)."""
    m = need_gpu()
    c = synth.tiny_vocab() if case == "tiny" else synth.modality4()
    hs = make_hotset(m, c.targets, c.scale)
    outs = {p: [host(run_pipeline_vocab(m, c, hs, torch.float32, path=p)[0]) for _ in range(2)] for p in (1, 3)}
    for p in (1, 3):
        np.testing.assert_array_equal(outs[p][0], outs[p][1])
    assert np.abs(outs[1][0] - outs[3][0]).max() <= DESIGN_MAXABS


def test_small_integers_bit_exact():
    m = need_gpu()
    N, d_in, d_out, K, r = 50, 256, 384, 3, 8
    xb, Ab, Bb, yb = synth.small_int_case(N, d_in, d_out, K, r, lo=-2, hi=3)
    tg = synth.Target("p", d_in, d_out, Ab, Bb, xb, yb)
    idx = np.random.default_rng(1).integers(0, K, N).astype(np.int32)
    w = np.ones(N, np.float32)
    for layout in (0, 1):
        hs = m.molora_hotset_init([(dev_bf16(Ab), dev_bf16(Bb))], 2.0, layout=layout)
        counts, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, 1)
        for path in (1, 2, 3, 4):
            y = m.molora_apply(hs, dev_bf16(xb), dev_bf16(yb).float(), offsets, perm, perm_w, inv, k=1,
                               y_dtype=torch.float32, path=path)
            ref = oracle_from_gpu_routing(tg, 2.0, idx, w, K, 1)
            assert np.abs(ref).max() < 2 ** 24
            np.testing.assert_array_equal(host(y), ref)


SHAPES = [
    # N, d_in, d_out, K, r, k
    (1, 128, 128, 1, 8, 1),
    (3, 512, 256, 4, 16, 1),
    (37, 256, 512, 5, 32, 1),
    (300, 384, 640, 7, 64, 1),
    (1000, 1024, 1024, 64, 16, 1),
    (17, 256, 256, 4, 16, 2),
    (301, 512, 384, 6, 24, 3),
    (1000, 256, 1024, 16, 64, 4),
    (2500, 640, 512, 8, 16, 8),
    (700, 512, 512, 64, 64, 1),   # 64-row grouped tiles over 64 adapters
    (90, 256, 2048, 16, 48, 2),   # few tiles: output columns split over workgroups
    (4100, 128, 256, 2, 16, 2),   # one reduction step, long segments
    (256, 2048, 6144, 16, 64, 2), # decode batch of the 28-layer stack, down-projection shape
]


@pytest.mark.parametrize("N,d_in,d_out,K,r,k", SHAPES)
@pytest.mark.parametrize("path", [1, 2, 3, 4])
def test_apply_shapes_paths(N, d_in, d_out, K, r, k, path):
    m = need_gpu()
    if path in (3, 4) and K > 16:
        pytest.skip("the tile and block paths take K <= 16")
    g = np.random.default_rng(N * 31 + d_in + K * 7 + r + k)
    xb = synth.to_bf16_bits(g.standard_normal((N, d_in)).astype(np.float32))
    Ab = synth.to_bf16_bits((g.standard_normal((K, d_in, r)) / np.sqrt(d_in)).astype(np.float32))
    Bb = synth.to_bf16_bits((g.standard_normal((K, r, d_out)) / np.sqrt(r)).astype(np.float32))
    yb = synth.to_bf16_bits(g.standard_normal((N, d_out)).astype(np.float32))
    tg = synth.Target("p", d_in, d_out, Ab, Bb, xb, yb)
    lg = g.standard_normal((N, K)).astype(np.float32)
    oi, ow, _ = route_topk(lg.astype(np.float64), k)
    idx = oi.astype(np.int32)
    w = ow.astype(np.float32)
    if N > 5:
        idx[N // 3, 0] = -1  # an unrouted pair
        idx[N // 4, :] = -1  # a token with no routed pair
        if k > 1:
            idx[N // 2, k - 1] = -1  # last slot unrouted
    hs = m.molora_hotset_init([(dev_bf16(Ab), dev_bf16(Bb))], 2.0)
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    ref = oracle_from_gpu_routing(tg, 2.0, idx, w, K, k)
    y = m.molora_apply(hs, dev_bf16(xb), dev_bf16(yb), offsets, perm, perm_w, inv, k=k, y_dtype=torch.float32,
                       path=path)
    check_float_output(host(y), ref, f64(yb))
    yb16 = m.molora_apply(hs, dev_bf16(xb), dev_bf16(yb), offsets, perm, perm_w, inv, k=k, y_dtype=torch.bfloat16,
                          path=path)
    check_bf16_output(host(yb16), ref)


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("k,r", [(2, 16), (3, 64), (1, 64)])
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16])
def test_grouped_in_place_multi_slot(k, r, y_dtype, path):
    """In-place grouped apply (y0 is y) on the 64-row tiles (path 1) and the split-shrink
    grouped expand (path 2): per-rank passes and the fp32 carry must leave unrouted tokens
    untouched and give the out-of-place result bit for bit."""
    m = need_gpu()
    N, d_in, d_out, K = 333, 384, 768, 8
    g = np.random.default_rng(7 * k + r)
    xb = synth.to_bf16_bits(g.standard_normal((N, d_in)).astype(np.float32))
    Ab = synth.to_bf16_bits((g.standard_normal((K, d_in, r)) / np.sqrt(d_in)).astype(np.float32))
    Bb = synth.to_bf16_bits((g.standard_normal((K, r, d_out)) / np.sqrt(r)).astype(np.float32))
    yb = synth.to_bf16_bits(g.standard_normal((N, d_out)).astype(np.float32))
    tg = synth.Target("p", d_in, d_out, Ab, Bb, xb, yb)
    oi, ow, _ = route_topk(g.standard_normal((N, K)), k)
    idx, w = oi.astype(np.int32), ow.astype(np.float32)
    idx[::7, 0] = -1
    idx[::11, :] = -1
    hs = m.molora_hotset_init([(dev_bf16(Ab), dev_bf16(Bb))], 2.0)
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    ref = oracle_from_gpu_routing(tg, 2.0, idx, w, K, k)
    y0 = dev_bf16(yb).to(y_dtype)
    out = m.molora_apply(hs, dev_bf16(xb), y0, offsets, perm, perm_w, inv, k=k, y_dtype=y_dtype, path=path)
    yin = y0.clone()
    m.molora_apply(hs, dev_bf16(xb), yin, offsets, perm, perm_w, inv, k=k, y=yin, path=path)
    np.testing.assert_array_equal(host(yin), host(out))
    np.testing.assert_array_equal(host(yin)[::11], f64(yb)[::11])
    if y_dtype == torch.float32:
        check_float_output(host(out), ref, f64(yb))
    else:
        check_bf16_output(host(out), ref)


def test_in_place_and_unrouted_rows():
    m = need_gpu()
    c = synth.tiny_vocab()
    ids = c.ids.copy()
    ids[::5] = 40000  # outside every range: unrouted
    c.ids = ids
    t = c.targets[0]
    hs = make_hotset(m, c.targets, c.scale)
    y_out, idx, w = run_pipeline_vocab(m, c, hs, torch.float32)
    ri, rw = route_vocab(ids, c.bounds)
    ref = oracle_from_gpu_routing(t, c.scale, ri, rw, c.K, 1)
    check_float_output(host(y_out), ref, f64(t.y0))
    np.testing.assert_array_equal(host(y_out)[::5], f64(t.y0)[::5])  # untouched rows copied exactly
    y_in, _, _ = run_pipeline_vocab(m, c, hs, torch.float32, in_place=True)
    np.testing.assert_array_equal(host(y_in), host(y_out))


@pytest.mark.parametrize("B", [1, 16, 64, 160, 512, 2048])
def test_decode_sweep(B):
    m = need_gpu()
    c = synth.decode_batch(B)
    t = c.targets[0]
    hs_d = make_hotset(m, c.targets, c.scale, 0)
    hs_i = make_hotset(m, c.targets, c.scale, 1)
    w = np.ones(B, np.float32)
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(dev(c.idx), dev(w), c.K, 1)
    ref = oracle_from_gpu_routing(t, c.scale, c.idx, w, c.K, 1)
    outs = []
    for hs in (hs_d, hs_i):
        for path in (1, 2):
            y = m.molora_apply(hs, dev_bf16(t.x), dev_bf16(t.y0), offsets, perm, perm_w, inv, k=1,
                               y_dtype=torch.float32, path=path)
            check_float_output(host(y), ref, f64(t.y0))
            outs.append(host(y))
    np.testing.assert_array_equal(outs[0], outs[2])  # direct == indirect, bit for bit
    np.testing.assert_array_equal(outs[1], outs[3])


def test_qwen_layer_all_targets():
    m = need_gpu()
    c = synth.qwen_layer()
    r = c.router
    x0 = c.targets[0].x
    logits, idx, w, flags = m.molora_route_topk(
        c.k, c.K, x=dev_bf16(x0), W1=dev_bf16(np.ascontiguousarray(r["W1"].T)), b1=dev(r["b1"]),
        W2=dev_bf16(np.ascontiguousarray(r["W2"].T)), b2=dev(r["b2"]))
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(idx, w, c.K, c.k)
    gi, gw = host(idx), host(w)
    hs = make_hotset(m, c.targets, c.scale)
    for ti, t in enumerate(c.targets):
        y = m.molora_apply(hs, dev_bf16(t.x), dev_bf16(t.y0), offsets, perm, perm_w, inv, k=c.k, target=ti,
                           y_dtype=torch.float32)
        ref = oracle_from_gpu_routing(t, c.scale, gi, gw, c.K, c.k)
        check_float_output(host(y), ref, f64(t.y0))


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_stress_full_size(k):
    """The stress workload at full size (N=16384, d=4096, K=16, r=64, Zipf logits), k = 1..4, on
    the AUTO path the bench times: every one of the 16384 rows against the oracle, for an fp32
    and a bf16 y (the bf16 y goes through the fp32 carry of the k > 1 passes)."""
    m = need_gpu()
    c = synth.stress(k)
    t = c.targets[0]
    _, idx, w, _ = m.molora_route_topk(k, c.K, logits=dev(c.logits))
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(idx, w, c.K, k)
    hs = make_hotset(m, c.targets, c.scale)
    x, y0 = dev_bf16(t.x), dev_bf16(t.y0)
    y32 = m.molora_apply(hs, x, y0, offsets, perm, perm_w, inv, k=k, y_dtype=torch.float32)
    y16 = m.molora_apply(hs, x, y0, offsets, perm, perm_w, inv, k=k, y_dtype=torch.bfloat16)
    gi, gw = host(idx), host(w)
    oi, _, _ = route_topk(c.logits.astype(np.float64), k)
    np.testing.assert_array_equal(gi, oi)
    ref = oracle_from_gpu_routing(t, c.scale, gi, gw, c.K, k)
    check_float_output(host(y32), ref, f64(t.y0))
    check_bf16_output(host(y16), ref)


def test_qwen_layer_multi_auto_all_targets():
    """The Qwen3-1.7B-shaped layer as the bench runs it: router MLP, top-2, dispatch, then one
    molora_apply_multi over all 7 targets on AUTO (which resolves to the 64-token block path for
    several targets with k > 1), bf16 and fp32 y; every target against the oracle.  Then the
    row's fused line (router with a workspace, molora_dispatch_apply_multi): the same bits."""
    m = need_gpu()
    c = synth.qwen_layer()
    r = c.router
    logits, idx, w, flags = m.molora_route_topk(
        c.k, c.K, x=dev_bf16(c.targets[0].x), W1=dev_bf16(np.ascontiguousarray(r["W1"].T)), b1=dev(r["b1"]),
        W2=dev_bf16(np.ascontiguousarray(r["W2"].T)), b2=dev(r["b2"]))
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(idx, w, c.K, c.k)
    gi, gw = host(idx), host(w)
    hs = make_hotset(m, c.targets, c.scale)
    xs = [dev_bf16(t.x) for t in c.targets]
    y0s = [dev_bf16(t.y0) for t in c.targets]
    assert m.molora_apply_multi_workspace(hs, list(range(7)), c.N, c.k, m.PATH_AUTO, torch.bfloat16) == \
        m.molora_apply_multi_workspace(hs, list(range(7)), c.N, c.k, m.PATH_BLOCK, torch.bfloat16)
    y16 = m.molora_apply_multi(hs, xs, y0s, offsets, perm, perm_w, inv, k=c.k, y_dtype=torch.bfloat16)
    y32 = m.molora_apply_multi(hs, xs, y0s, offsets, perm, perm_w, inv, k=c.k, y_dtype=torch.float32)
    # the bench row's fastest line: the router with a workspace, then dispatch and the 7 applies
    # in one call (the dispatch inside the block shrink's launch) -- the same routing bits, the
    # same dispatch outputs and the same y bits
    rws = torch.empty(m.molora_route_topk_workspace(c.N, c.targets[0].d_in), dtype=torch.uint8, device="cuda")
    l2, i2, w2, f2 = m.molora_route_topk(
        c.k, c.K, x=xs[0], W1=dev_bf16(np.ascontiguousarray(r["W1"].T)), b1=dev(r["b1"]),
        W2=dev_bf16(np.ascontiguousarray(r["W2"].T)), b2=dev(r["b2"]), ws=rws)
    for a, b in ((l2, logits), (i2, idx), (w2, w), (f2, flags)):
        np.testing.assert_array_equal(host(a), host(b))
    yf, meta = m.molora_dispatch_apply_multi(hs, xs, y0s, i2.reshape(-1), w2.reshape(-1), c.K, c.k,
                                             y_dtype=torch.bfloat16)
    n_routed = int(host(offsets)[-1])
    for a, b, full in zip(meta, (counts, offsets, perm, perm_w, inv), (True, True, False, False, True)):
        np.testing.assert_array_equal(host(a) if full else host(a)[:n_routed], host(b) if full else host(b)[:n_routed])
    for ti, t in enumerate(c.targets):
        ref = oracle_from_gpu_routing(t, c.scale, gi, gw, c.K, c.k)
        check_bf16_output(host(y16[ti]), ref)
        check_float_output(host(y32[ti]), ref, f64(t.y0))
        np.testing.assert_array_equal(host(yf[ti]), host(y16[ti]))


@pytest.mark.parametrize("path", [0, 4])
def test_graph_replay_matches_eager(path):
    """The vocab step captured in a HIP graph, replayed with eager work in between."""
    m = need_gpu()
    c = synth.modality4()
    t = c.targets[0]
    hs = make_hotset(m, c.targets, c.scale)
    ids = dev(c.ids)
    x, y0 = dev_bf16(t.x), dev_bf16(t.y0)
    idx = torch.empty(c.N, dtype=torch.int32, device="cuda")
    w = torch.empty(c.N, dtype=torch.float32, device="cuda")
    meta = (torch.empty(c.K, dtype=torch.int32, device="cuda"), torch.empty(c.K + 1, dtype=torch.int32, device="cuda"),
            torch.empty(c.N, dtype=torch.int32, device="cuda"), torch.empty(c.N, dtype=torch.float32, device="cuda"),
            torch.empty(c.N, dtype=torch.int32, device="cuda"))
    y = torch.empty(c.N, t.d_out, dtype=torch.bfloat16, device="cuda")
    need = m.molora_apply_workspace(hs, 0, c.N, 1, path, torch.bfloat16)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")

    def step():
        m.molora_route_vocab(ids, c.bounds.tolist(), idx=idx, w=w)
        m.molora_dispatch(idx, w, c.K, 1, out=meta)
        m.molora_apply(hs, x, y0, meta[1], meta[2], meta[3], meta[4], k=1, y=y, path=path, ws=ws)

    step()
    torch.cuda.synchronize()
    eager = host(y).copy()
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
        y.zero_()
        meta[2].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), eager)


def test_zero_tokens_is_noop():
    m = need_gpu()
    c = synth.tiny_vocab()
    hs = make_hotset(m, c.targets, c.scale)
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    idx, w = m.molora_route_vocab(empty, c.bounds.tolist())
    assert idx.numel() == 0
    x = torch.empty(0, 512, dtype=torch.bfloat16, device="cuda")
    y = m.molora_apply(hs, x, x.clone(), torch.zeros(5, dtype=torch.int32, device="cuda"), empty, empty.float(),
                       empty, k=1)
    assert y.shape == (0, 512)


@pytest.mark.parametrize("k,r,path", [(2, 64, 0), (1, 64, 0), (2, 16, 0), (2, 16, 2), (3, 32, 1), (2, 16, 3), (2, 16, 4),
                                      (1, 64, 4)])
@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16])
def test_apply_multi_equals_single_calls(k, r, path, y_dtype):
    """Several projections sharing one routing in one call (the skinny path fuses the phases
    over the targets; other paths loop): bit-identical to one molora_apply per target, and
    within the bars of the oracle."""
    m = need_gpu()
    N, K = 256, 16
    dims = [(512, 512), (512, 256), (512, 1536), (1536, 512)]
    g = np.random.default_rng(100 + 10 * k + r + path)
    tgs = []
    for di, do in dims:
        xb = synth.to_bf16_bits(g.standard_normal((N, di)).astype(np.float32))
        Ab = synth.to_bf16_bits((g.standard_normal((K, di, r)) / np.sqrt(di)).astype(np.float32))
        Bb = synth.to_bf16_bits((g.standard_normal((K, r, do)) / np.sqrt(r)).astype(np.float32))
        yb = synth.to_bf16_bits(g.standard_normal((N, do)).astype(np.float32))
        tgs.append(synth.Target("p", di, do, Ab, Bb, xb, yb))
    oi, ow, _ = route_topk(g.standard_normal((N, K)), k)
    idx, w = oi.astype(np.int32), ow.astype(np.float32)
    idx[::9, 0] = -1
    idx[::13, :] = -1
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B)) for t in tgs], 2.0)
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), K, k)
    xs = [dev_bf16(t.x) for t in tgs]
    y0s = [dev_bf16(t.y0).to(y_dtype) for t in tgs]
    order = [2, 0, 3, 1]  # targets in any order
    ys = m.molora_apply_multi(hs, [xs[i] for i in order], [y0s[i] for i in order], offsets, perm, perm_w, inv, k=k,
                              targets=order, y_dtype=y_dtype, path=path)
    # the documented AUTO rule (blocks instead of tiles for several targets with k > 1)
    single_path = path
    if path == 0:
        if r <= 32 and k > 1:
            single_path = 4 if (K <= 16 and N * k >= 192) else 1  # tile, then blocks for several targets
        elif r <= 32:
            single_path = 3 if (N >= 1024 and K <= 4) else 1
        else:
            single_path = 1 if N * k >= 1024 else 2
        assert m.molora_apply_path(hs, N, k, 0, target=0) == (3 if single_path == 4 else single_path)
    for j, i in enumerate(order):
        single = m.molora_apply(hs, xs[i], y0s[i], offsets, perm, perm_w, inv, k=k, target=i, y_dtype=y_dtype,
                                path=single_path)
        np.testing.assert_array_equal(host(ys[j]), host(single))
    t = tgs[3]
    ref = oracle_from_gpu_routing(t, 2.0, idx, w, K, k)
    if y_dtype == torch.float32:
        check_float_output(host(ys[2]), ref, f64(t.y0))
    else:
        check_bf16_output(host(ys[2]), ref)
    # in place: y0 is y for every target
    yin = [v.clone() for v in y0s]
    m.molora_apply_multi(hs, xs, yin, offsets, perm, perm_w, inv, k=k, ys=yin, path=path)
    for i in range(len(dims)):
        np.testing.assert_array_equal(host(yin[i]), host(ys[order.index(i)]))
