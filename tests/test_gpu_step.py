"""GPU parity: the one-launch vocabulary step against the three separate calls and the oracle."""
import numpy as np
import pytest
import torch

import synth
from oracle import apply, dispatch, route_vocab
from tests.gpu_util import check_bf16_output, check_float_output, dev, dev_bf16, f64, host, need_gpu

pytestmark = pytest.mark.gpu


def three_calls(m, hs, ids, bounds, K, x, y0, y_dtype, path):
    idx, w = m.molora_route_vocab(ids, bounds)
    meta = m.molora_dispatch(idx, w, K, 1)
    counts, offsets, perm, perm_w, inv = meta
    y = m.molora_apply(hs, x, y0, offsets, perm, perm_w, inv, k=1, y_dtype=y_dtype, path=path)
    return y, (idx, w), meta


def step_ws(m, hs, N, block):
    """A step workspace (split step), or None (tile step).  It needs no initial contents, so it
    starts as 0xFF bytes (NaN floats): a partial read before it is written would show."""
    if not block:
        return None
    return torch.full((max(1, m.molora_step_workspace(hs, 0, N)),), 0xFF, dtype=torch.uint8, device="cuda")


def cases():
    tiny = synth.tiny_vocab()
    mod = synth.modality4()
    odd = synth.vocab_case(N=1000, d=640, K=7, r=24, case_id=11, runs=True, probs=(0.3, 0.2, 0.1, 0.1, 0.1, 0.1, 0.1))
    odd.ids = odd.ids.copy()
    odd.ids[::37] = -5        # unrouted
    odd.ids[5::41] = 10 ** 6  # unrouted
    # whole tiles of unrouted tokens (they apply no adapter and copy y0 to y), two 256-column
    # units per wave, rank blocks 1 and 2, and tiles with up to four adapters
    holes = []
    for r in (16, 32):
        h = synth.vocab_case(N=520, d=4096, K=4, r=r, case_id=12, runs=False)
        h.ids = h.ids.copy()
        h.ids[16:40] = -5
        h.ids[500:] = 10 ** 6
        holes.append((f"unrouted_tiles_r{r}", h))
    dead = synth.vocab_case(N=100, d=4096, K=4, r=32, case_id=13, runs=False)
    dead.ids = np.full_like(dead.ids, -1)
    # rank blocks 3 and 4, and more adapters than the split expand stages at once (groups)
    wide = [
        ("k16_r64", synth.vocab_case(N=300, d=1024, K=16, r=64, case_id=14, runs=True, probs=(1 / 16,) * 16)),
        ("k9_r16", synth.vocab_case(N=777, d=2048, K=9, r=16, case_id=15, runs=True, probs=(1 / 9,) * 9)),
        ("k3_r48", synth.vocab_case(N=200, d=1536, K=3, r=48, case_id=16, runs=False)),
    ]
    return [("tiny", tiny), ("modality4", mod), ("ragged_unrouted", odd), *holes, ("all_unrouted", dead), *wide]


@pytest.mark.parametrize("block", [False, True])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("y_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("name,case", cases())
def test_step_equals_three_calls_and_oracle(name, case, y_dtype, layout, block):
    m = need_gpu()
    t = case.targets[0]
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B))], case.scale, layout=layout)
    ids = dev(case.ids)
    bounds = case.bounds.tolist()
    x, y0 = dev_bf16(t.x), dev_bf16(t.y0)
    y1, r1, m1 = m.molora_step_vocab(hs, ids, bounds, x, y0, y_dtype=y_dtype, ws=step_ws(m, hs, case.N, block))
    y3, r3, m3 = three_calls(m, hs, ids, bounds, case.K, x, y0, y_dtype, m.PATH_BLOCK if block else m.PATH_TILE)
    N = case.N
    np.testing.assert_array_equal(host(r1[0])[:N], host(r3[0]))
    np.testing.assert_array_equal(host(r1[1])[:N], host(r3[1]))
    n_routed = int(host(m3[1])[-1])
    for a, b, full in zip(m1, m3, (True, True, False, False, True)):
        ha, hb = host(a), host(b)
        if full:
            np.testing.assert_array_equal(ha, hb)
        else:
            np.testing.assert_array_equal(ha[:n_routed], hb[:n_routed])
    np.testing.assert_array_equal(host(y1), host(y3))
    # against the oracle
    ri, rw = route_vocab(case.ids, case.bounds)
    np.testing.assert_array_equal(host(r1[0])[:N], ri)
    oc, oo, op, opw, oinv = dispatch(ri, rw, case.K)
    np.testing.assert_array_equal(host(m1[0]), oc)
    np.testing.assert_array_equal(host(m1[1]), oo)
    np.testing.assert_array_equal(host(m1[2])[:oo[-1]], op)
    np.testing.assert_array_equal(host(m1[4])[:N], oinv)
    ref = apply(f64(t.y0), f64(t.x), f64(t.A), f64(t.B), case.scale, op, opw, oo, 1)
    if y_dtype == torch.float32:
        check_float_output(host(y1), ref, f64(t.y0))
    else:
        check_bf16_output(host(y1), ref)


def test_step_in_place_and_graph_replay():
    m = need_gpu()
    c = synth.modality4()
    t = c.targets[0]
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B))], c.scale)
    ids = dev(c.ids)
    bounds = c.bounds.tolist()
    x = dev_bf16(t.x)
    y_ref, _, _ = m.molora_step_vocab(hs, ids, bounds, x, dev_bf16(t.y0))
    y = dev_bf16(t.y0)
    m.molora_step_vocab(hs, ids, bounds, x, y, y=y)  # in place
    np.testing.assert_array_equal(host(y), host(y_ref))
    # graph capture of the one-launch step, replayed with eager work in between
    y0 = dev_bf16(t.y0)
    out = torch.empty_like(y0)
    route = (torch.empty(c.N, dtype=torch.int32, device="cuda"), torch.empty(c.N, dtype=torch.float32, device="cuda"))
    meta = (torch.empty(c.K, dtype=torch.int32, device="cuda"), torch.empty(c.K + 1, dtype=torch.int32, device="cuda"),
            torch.empty(c.N, dtype=torch.int32, device="cuda"), torch.empty(c.N, dtype=torch.float32, device="cuda"),
            torch.empty(c.N, dtype=torch.int32, device="cuda"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        m.molora_step_vocab(hs, ids, bounds, x, y0, y=out, route=route, meta=meta)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.molora_step_vocab(hs, ids, bounds, x, y0, y=out, route=route, meta=meta)
    for _ in range(3):
        out.zero_()
        meta[2].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), host(y_ref))
        ri, rw = route_vocab(c.ids, c.bounds)
        np.testing.assert_array_equal(host(meta[2]), dispatch(ri, rw, c.K)[2])


def test_block_step_reuses_workspace_across_inputs_and_graph_replays():
    """One step workspace across different batches and across graph replays: every result
    matches the oracle (no partial sums left over from an earlier call)."""
    m = need_gpu()
    cases_ = [synth.modality4(),
              synth.vocab_case(N=2048, d=4096, K=4, r=16, case_id=23, runs=True, probs=(0.25, 0.25, 0.25, 0.25))]
    t0 = cases_[0].targets[0]
    hs = m.molora_hotset_init([(dev_bf16(t0.A), dev_bf16(t0.B))], cases_[0].scale)
    ws = step_ws(m, hs, 2048, True)
    for case in cases_:
        t = case.targets[0]
        ids = dev(case.ids)
        y, r, meta = m.molora_step_vocab(hs, ids, case.bounds.tolist(), dev_bf16(t.x), dev_bf16(t.y0),
                                         y_dtype=torch.float32, ws=ws)
        torch.cuda.synchronize()
        ri, rw = route_vocab(case.ids, case.bounds)
        oc, oo, op, opw, oinv = dispatch(ri, rw, case.K)
        ref = apply(f64(t.y0), f64(t.x), f64(t0.A), f64(t0.B), case.scale, op, opw, oo, 1)
        check_float_output(host(y), ref, f64(t.y0))
    # graph replays, eager work between them
    case = cases_[0]
    t = case.targets[0]
    ids, x, y0 = dev(case.ids), dev_bf16(t.x), dev_bf16(t.y0)
    y = torch.empty(case.N, t.d_out, dtype=torch.bfloat16, device="cuda")
    route = (torch.empty(case.N, dtype=torch.int32, device="cuda"), torch.empty(case.N, dtype=torch.float32, device="cuda"))
    meta = (torch.empty(case.K, dtype=torch.int32, device="cuda"), torch.empty(case.K + 1, dtype=torch.int32, device="cuda"),
            torch.empty(case.N, dtype=torch.int32, device="cuda"), torch.empty(case.N, dtype=torch.float32, device="cuda"),
            torch.empty(case.N, dtype=torch.int32, device="cuda"))

    def step():
        m.molora_step_vocab(hs, ids, case.bounds.tolist(), x, y0, y=y, route=route, meta=meta, ws=ws)

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
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), eager)


def large_cases():
    # above 4096 tokens: route, the chip-wide dispatch (8193 pairs and more) and the split launches
    out = []
    for N, cid in ((4097, 31), (8192, 32), (8193, 33)):
        c = synth.vocab_case(N=N, d=4096, K=4, r=16, case_id=cid, runs=True, probs=(0.4, 0.3, 0.15, 0.15))
        c.ids = c.ids.copy()
        c.ids[7::1001] = -3  # a few unrouted tokens
        out.append((f"n{N}", c))
    out.append(("n5000_k16_r64", synth.vocab_case(N=5000, d=1024, K=16, r=64, case_id=34, runs=True,
                                                  probs=(1 / 16,) * 16)))
    return out


@pytest.mark.parametrize("block", [False, True])
@pytest.mark.parametrize("name,case", large_cases())
def test_step_above_4096_tokens(name, case, block):
    """molora_step_vocab above 4096 tokens, with and without a workspace: routing and dispatch
    bit-exact against the oracle, y within the output bars, and (with a workspace) y bit-identical
    to the block path on the same dispatch, as the header states."""
    m = need_gpu()
    t = case.targets[0]
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B))], case.scale)
    ids = dev(case.ids)
    bounds = case.bounds.tolist()
    x, y0 = dev_bf16(t.x), dev_bf16(t.y0)
    ws = step_ws(m, hs, case.N, block)
    y, r, meta = m.molora_step_vocab(hs, ids, bounds, x, y0, y_dtype=torch.float32, ws=ws)
    torch.cuda.synchronize()
    N = case.N
    ri, rw = route_vocab(case.ids, case.bounds)
    np.testing.assert_array_equal(host(r[0])[:N], ri)
    np.testing.assert_array_equal(host(r[1])[:N], rw.astype(np.float32))
    oc, oo, op, opw, oinv = dispatch(ri, rw, case.K)
    np.testing.assert_array_equal(host(meta[0]), oc)
    np.testing.assert_array_equal(host(meta[1]), oo)
    np.testing.assert_array_equal(host(meta[2])[:oo[-1]], op)
    np.testing.assert_array_equal(host(meta[3])[:oo[-1]], opw.astype(np.float32))
    np.testing.assert_array_equal(host(meta[4])[:N], oinv)
    ref = apply(f64(t.y0), f64(t.x), f64(t.A), f64(t.B), case.scale, op, opw, oo, 1)
    check_float_output(host(y), ref, f64(t.y0))
    if block:
        yb = m.molora_apply(hs, x, y0, meta[1], meta[2], meta[3], meta[4], k=1, y_dtype=torch.float32,
                            path=m.PATH_BLOCK)
        np.testing.assert_array_equal(host(y), host(yb))
        # the same workspace again, after a smaller batch used it: same bits
        n_small = 1000
        m.molora_step_vocab(hs, ids[:n_small].contiguous(), bounds, x[:n_small].contiguous(),
                            torch.flip(y0[:n_small], dims=[0]).contiguous(), ws=ws)
        y2, _, _ = m.molora_step_vocab(hs, ids, bounds, x, y0, y_dtype=torch.float32, ws=ws)
        np.testing.assert_array_equal(host(y2), host(y))
