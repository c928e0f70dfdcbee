"""The allocation-free step (molora_step_vocab_noalloc) against molora_step_vocab with a
caller workspace: the same bits for y and every dispatch output, on two calls in a row (the
second with a smaller batch, so scratch left by the first would show), at sizes that take the
fused two-launch step and the route + dispatch + split step; and the size limit."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import dev, dev_bf16, host, need_gpu

pytestmark = pytest.mark.gpu


def _case(N, cid):
    c = synth.vocab_case(N=N, d=4096, K=4, r=16, case_id=cid, runs=True, probs=(0.4, 0.3, 0.15, 0.15))
    c.ids = c.ids.copy()
    c.ids[3::517] = -2  # a few unrouted tokens
    return c


@pytest.mark.parametrize("sizes", [(2048, 700), (8192, 4097)])
def test_noalloc_step_equals_workspace_step(sizes):
    m = need_gpu()
    first = _case(sizes[0], 41)
    t0 = first.targets[0]
    hs = m.molora_hotset_init([(dev_bf16(t0.A), dev_bf16(t0.B))], first.scale)
    bounds = first.bounds.tolist()
    for i, N in enumerate(sizes):
        c = first if i == 0 else _case(N, 42)
        t = c.targets[0]
        ids, x, y0 = dev(c.ids), dev_bf16(t.x), dev_bf16(t.y0)
        ws = torch.full((m.molora_step_workspace(hs, 0, N),), 0xFF, dtype=torch.uint8, device="cuda")
        y_ref, r_ref, meta_ref = m.molora_step_vocab(hs, ids, bounds, x, y0, ws=ws)
        y, r, meta = m.molora_step_vocab_noalloc(hs, ids, bounds, x, y0)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(y), host(y_ref))
        n_routed = int(host(meta_ref[1])[-1])
        assert n_routed < N  # the unrouted tokens are there
        for j, (a, b) in enumerate(zip(r + meta, r_ref + meta_ref)):
            ha, hb = host(a), host(b)
            if j in (4, 5):  # perm, perm_w: entries past offsets[K] are left untouched
                ha, hb = ha[:n_routed], hb[:n_routed]
            np.testing.assert_array_equal(ha, hb)


def test_noalloc_rejects_steps_above_the_scratch_size():
    m = need_gpu()
    c = _case(2048, 43)
    t = c.targets[0]
    hs = m.molora_hotset_init([(dev_bf16(t.A), dev_bf16(t.B))], c.scale)
    N = 16384  # 256 blocks x 8 slices x 64 x 16 fp32 partials = 8 MiB, plus the dispatch counts
    assert m.molora_step_workspace(hs, 0, N) > m.NOALLOC_SCRATCH_BYTES
    ids = torch.zeros(N, dtype=torch.int32, device="cuda")
    x = torch.zeros(N, 4096, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MoloraError) as ei:
        m.molora_step_vocab_noalloc(hs, ids, c.bounds.tolist(), x, x)
    assert ei.value.code == m.MOLORA_ENOSPC
