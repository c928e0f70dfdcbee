"""GPU parity of the 64-row grouped kernel's tile choice (thelatestinai.com, Table 9: fixed
versus adaptive tiling under skewed adapter usage): the adaptive tiles (MOLORA_PATH_GROUPED,
tile heights per segment from the offsets) and the fixed 64-row tiles (MOLORA_PATH_GROUPED_FIXED)
against the oracle on the table's three mixes, with empty and one-row segments, k = 1 and 2,
ranks 16 and 64; the two tilings split only the rows, never a reduction, so they agree bit for
bit."""
import numpy as np
import pytest
import torch

import synth
from oracle import apply, dispatch, route_topk
from tests.gpu_util import check_bf16_output, check_float_output, dev, dev_bf16, f64, host, need_gpu

pytestmark = pytest.mark.gpu

MIXES = {"uniform": (0.25, 0.25, 0.25, 0.25), "80_10_5_5": (0.8, 0.1, 0.05, 0.05), "95_2_2_1": (0.95, 0.02, 0.02, 0.01)}


def _run(m, c, idx, w, k, path, y_dtype):
    t = c.targets[0]
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B))], c.scale)
    counts, offsets, perm, perm_w, inv = m.molora_dispatch(dev(idx), dev(w), c.K, k)
    y = m.molora_apply(hs, dev_bf16(t.x), dev_bf16(t.y0), offsets, perm, perm_w, inv, k=k, path=path, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return host(y)


@pytest.mark.parametrize("r", [64, 16])
@pytest.mark.parametrize("mix", list(MIXES))
@pytest.mark.parametrize("N", [2048, 777])
def test_tiling_mixes_k1(mix, N, r):
    m = need_gpu()
    c = synth.mixed_batch(N, MIXES[mix], d=1024, r=r, case_id=60, sub=N)
    idx = c.idx.copy()
    idx[5] = 3          # at least one row of the rarest adapter ...
    idx[idx == 2] = 1   # ... and an empty segment
    idx[::101] = -1     # unrouted tokens
    w = np.ones(N, dtype=np.float32)
    t = c.targets[0]
    oc, oo, op, opw, _ = dispatch(idx, w, c.K)
    ref = apply(f64(t.y0), f64(t.x), f64(t.A), f64(t.B), c.scale, op, opw, oo, 1)
    ya = _run(m, c, idx, w, 1, m.PATH_GROUPED, torch.float32)
    yf = _run(m, c, idx, w, 1, m.PATH_GROUPED_FIXED, torch.float32)
    check_float_output(ya, ref, f64(t.y0))
    check_float_output(yf, ref, f64(t.y0))
    if r > 32:  # the same 64-row kernel on both tilings (rank 16 GROUPED takes the 16-row kernel)
        np.testing.assert_array_equal(ya, yf)
    yb = _run(m, c, idx, w, 1, m.PATH_GROUPED_FIXED, torch.bfloat16)
    check_bf16_output(yb, ref)


@pytest.mark.parametrize("path_name", ["GROUPED", "GROUPED_FIXED"])
def test_tiling_zipf_k2(path_name):
    """Top-2 over Zipf-skewed logits (the stress workload's router, 16 adapters of rank 64): the
    rank passes run on either tiling."""
    m = need_gpu()
    N, K, k = 1500, 16, 2
    logits = synth.zipf_logits(61, N, K)
    oi, ow, _ = route_topk(logits.astype(np.float64), k)
    idx, w = oi.astype(np.int32), ow.astype(np.float32)
    A, B = synth._lora_weights(61, 0, K, 1024, 512, 64)
    x = synth.normal_bf16(61, synth.T_X, (N, 1024))
    y0 = synth.normal_bf16(61, synth.T_Y0, (N, 512))
    c = synth.Case("zipf2", 61, N, K, 64, k, 2.0, [synth.Target("p", 1024, 512, A, B, x, y0)])
    oc, oo, op, opw, _ = dispatch(idx, w, K)
    ref = apply(f64(y0), f64(x), f64(A), f64(B), 2.0, op, opw, oo, k)
    y = _run(m, c, idx, w, k, getattr(m, "PATH_" + path_name), torch.bfloat16)
    check_bf16_output(y, ref)
