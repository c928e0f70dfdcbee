"""CPU checks of the C ABI: the library loads, exports every declared entry point, and its
host-side validation / size arithmetic behaves as include/molora.h states.  No kernel is
launched here (no GPU)."""
import ctypes
import os
import re

import pytest

import token_adapter_routing_amd as m
from token_adapter_routing_amd.binding import MoloraTarget

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "molora.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(molora_\w+)\s*\(", text)))


def lib():
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("library not built")
    return m.load_library()


def test_every_declared_symbol_is_exported_and_bound():
    L = lib()
    names = declared_functions()
    assert len(names) == 29, names
    for n in names:
        assert hasattr(L, n), n
    assert sorted(m.exported_symbols()) == names


def test_hotset_bytes_arithmetic():
    # direct: K * (r_pad*d_in + d_out*r_pad) * 2 bytes per target (all multiples of 256 here)
    assert m.molora_hotset_bytes(4, 16, [(4096, 4096)]) == 4 * (16 * 4096 + 4096 * 16) * 2
    assert m.molora_hotset_bytes(4, 8, [(512, 512)]) == 4 * (16 * 512 + 512 * 16) * 2  # rank padded to 16
    qwen = [(2048, 2048), (2048, 1024), (2048, 1024), (2048, 2048), (2048, 6144), (2048, 6144), (6144, 2048)]
    assert m.molora_hotset_bytes(4, 16, qwen) == sum(4 * 16 * (a + b) * 2 for a, b in qwen)
    ind = m.molora_hotset_bytes(4, 16, [(4096, 4096)], layout=1)
    assert ind == 4 * (16 * 4096 + 4096 * 16) * 2 + 2 * 256  # plus two 256-byte pointer tables


@pytest.mark.parametrize("K,r,dims,code", [(0, 16, [(128, 128)], 2), (65, 16, [(128, 128)], 2),
                                          (4, 0, [(128, 128)], 2), (4, 65, [(128, 128)], 2),
                                          (4, 16, [(100, 128)], 2), (4, 16, [(128, 0)], 2)])
def test_hotset_bytes_rejects(K, r, dims, code):
    lib()
    with pytest.raises(m.MoloraError) as ei:
        m.molora_hotset_bytes(K, r, dims)
    assert ei.value.code == code


def test_host_validation_without_launch():
    L = lib()
    nul = None
    # route_vocab: K out of range, decreasing bounds, negative N
    b = (ctypes.c_int32 * 3)(0, 10, 5)
    assert L.molora_route_vocab(nul, 4, ctypes.cast(b, ctypes.c_void_p), 2, nul, nul, nul) == 1
    assert b"non-decreasing" in L.molora_last_error()
    assert L.molora_route_vocab(nul, 4, ctypes.cast(b, ctypes.c_void_p), 0, nul, nul, nul) == 2
    assert b"K=0" in L.molora_last_error()
    assert L.molora_route_vocab(nul, -1, ctypes.cast(b, ctypes.c_void_p), 2, nul, nul, nul) == 1
    assert b"N=-1" in L.molora_last_error()
    ok = (ctypes.c_int32 * 3)(0, 5, 10)
    assert L.molora_route_vocab(nul, 0, ctypes.cast(ok, ctypes.c_void_p), 2, nul, nul, nul) == 0  # N=0 no-op
    assert L.molora_route_vocab(nul, 3, ctypes.cast(ok, ctypes.c_void_p), 2, nul, nul, nul) == 1  # NULL buffers
    # route_topk: k > K, k > 8, router mode with d not a multiple of 128
    assert L.molora_route_topk(nul, 4, 0, nul, nul, nul, nul, nul, 4, 5, nul, nul, nul, nul, 0, nul) == 2
    assert L.molora_route_topk(nul, 4, 0, nul, nul, nul, nul, nul, 16, 9, nul, nul, nul, nul, 0, nul) == 2
    assert L.molora_route_topk(nul, 4, 100, ctypes.c_void_p(256), nul, ctypes.c_void_p(256), nul, nul, 4, 2,
                               nul, nul, nul, nul, 0, nul) == 2
    # route_topk workspace: eighths of d in fp32 per token up to d = 4096, none above
    sz = ctypes.c_size_t(0)
    assert L.molora_route_topk_workspace(4096, 2048, ctypes.byref(sz)) == 0 and sz.value == 8 * 4096 * 64 * 4
    assert L.molora_route_topk_workspace(100, 8192, ctypes.byref(sz)) == 0 and sz.value == 0
    assert L.molora_route_topk_workspace(100, 100, ctypes.byref(sz)) == 2
    # dispatch: k out of range, K out of range, N=0 no-op, NULL outputs
    assert L.molora_dispatch(nul, nul, 4, 0, 4, nul, nul, nul, nul, nul, nul, 0, nul) == 2
    assert L.molora_dispatch(nul, nul, 4, 1, 65, nul, nul, nul, nul, nul, nul, 0, nul) == 2
    assert L.molora_dispatch(nul, nul, 0, 1, 4, nul, nul, nul, nul, nul, nul, 0, nul) == 0
    assert L.molora_dispatch(nul, nul, 4, 1, 4, nul, nul, nul, nul, nul, nul, 0, nul) == 1
    # apply: NULL hot set
    assert L.molora_apply(nul, 0, nul, nul, 0, nul, 0, 4, 1, nul, nul, nul, nul, 0, nul, 0, nul) == 1
    sz = ctypes.c_size_t()
    assert L.molora_dispatch_workspace(2048, 4, 16, ctypes.byref(sz)) == 0 and sz.value == 0  # 8192 pairs: one workgroup
    # 65536 pairs: 64 workgroups of 1024 pairs, 16 counts each
    assert L.molora_dispatch_workspace(16384, 4, 16, ctypes.byref(sz)) == 0 and sz.value == 64 * 16 * 4
    # 1M pairs: 128 workgroups of 8192 pairs
    assert L.molora_dispatch_workspace(262144, 4, 16, ctypes.byref(sz)) == 0 and sz.value == 128 * 16 * 4
    assert L.molora_apply_workspace(nul, 0, 4, 1, 0, 0, ctypes.byref(sz)) == 1
    # multi-target apply: NULL hot set
    assert L.molora_apply_multi_workspace(nul, 2, nul, 4, 1, 0, 0, ctypes.byref(sz)) == 1
    assert L.molora_apply_multi(nul, 2, nul, nul, nul, 0, nul, 0, 4, 1, nul, nul, nul, nul, 0, nul, 0, nul) == 1
    # hotset_init: unaligned slab is rejected before any launch
    tg = (MoloraTarget * 1)(MoloraTarget(128, 128, 2, 2))
    h = ctypes.c_void_p()
    assert L.molora_hotset_init(ctypes.byref(h), 4, 16, 2.0, 1, tg, 0, ctypes.c_void_p(16), 1 << 20, nul) == 1
    assert L.molora_hotset_init(ctypes.byref(h), 4, 16, 2.0, 1, tg, 0, ctypes.c_void_p(256), 16, nul) == 3
    assert L.molora_hotset_destroy(nul) == 0
    # hotset_load: NULL hot set is rejected before any launch
    assert L.molora_hotset_load(nul, 0, 0, ctypes.c_void_p(256), ctypes.c_void_p(256), nul) == 1
    assert L.molora_seqpass_meta(nul, 0, 4, nul, nul, nul, nul) == 0
    # backward: NULL hot sets; the transposed init refuses a misaligned slab before any launch
    assert L.molora_backward_workspace(nul, nul, 0, 4, 1, 0, ctypes.byref(sz)) == 1
    assert b"hot set is NULL" in L.molora_last_error()
    assert L.molora_backward(nul, nul, 0, nul, nul, nul, 0, nul, 0, 4, 1, nul, nul, nul, nul, nul, nul, nul, nul, 0,
                             nul) == 1
    assert L.molora_hotset_init_transposed(ctypes.byref(h), 4, 16, 2.0, 1, tg, 0, ctypes.c_void_p(16), 1 << 20,
                                           nul) == 1
    assert b"256-byte" in L.molora_last_error()


def test_binding_refuses_cpu_tensors():
    lib()
    import torch
    with pytest.raises(ValueError):
        m.molora_route_vocab(torch.zeros(4, dtype=torch.int32), [0, 1, 2])
