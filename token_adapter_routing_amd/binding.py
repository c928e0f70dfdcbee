"""ctypes binding of libmolora.so with the C entry points' names.

Argument marshalling only: every function checks tensor placement, dtype and contiguity,
allocates missing outputs with torch (device memory is torch's; the work is the library's),
passes raw pointers and the current HIP stream, and turns a non-OK status into
``MoloraError``.  Nothing here computes any part of the routing path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmolora.so")

MOLORA_OK, MOLORA_EINVAL, MOLORA_ENOTSUP, MOLORA_ENOSPC, MOLORA_EHIP = range(5)
LAYOUT_DIRECT, LAYOUT_INDIRECT = 0, 1
PATH_AUTO, PATH_GROUPED, PATH_SKINNY, PATH_TILE, PATH_BLOCK, PATH_GROUPED_FIXED = 0, 1, 2, 3, 4, 5
BF16, F32 = 0, 1

_c_p = ctypes.c_void_p
_c_i = ctypes.c_int
_c_f = ctypes.c_float
_c_sz = ctypes.c_size_t


class MoloraError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"molora error {code}: {msg}")
        self.code = code


class MoloraTarget(ctypes.Structure):
    _fields_ = [("d_in", _c_i), ("d_out", _c_i), ("A", _c_p), ("B", _c_p)]


class MoloraXfLayer(ctypes.Structure):
    _fields_ = [("norm1", _c_p), ("norm2", _c_p), ("W", _c_p * 7), ("lora", _c_p)]


_SIGS = {
    "molora_last_error": (ctypes.c_char_p, []),
    "molora_hotset_bytes": (_c_i, [_c_i, _c_i, _c_i, ctypes.POINTER(MoloraTarget), _c_i, ctypes.POINTER(_c_sz)]),
    "molora_hotset_init": (_c_i, [ctypes.POINTER(_c_p), _c_i, _c_i, _c_f, _c_i, ctypes.POINTER(MoloraTarget), _c_i,
                                  _c_p, _c_sz, _c_p]),
    "molora_hotset_load": (_c_i, [_c_p, _c_i, _c_i, _c_p, _c_p, _c_p]),
    "molora_hotset_destroy": (_c_i, [_c_p]),
    "molora_route_vocab": (_c_i, [_c_p, _c_i, _c_p, _c_i, _c_p, _c_p, _c_p]),
    "molora_route_topk_workspace": (_c_i, [_c_i, _c_i, _c_p]),
    "molora_route_topk": (_c_i, [_c_p, _c_i, _c_i, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i, _c_i, _c_p, _c_p, _c_p, _c_p,
                                 _c_sz, _c_p]),
    "molora_dispatch_workspace": (_c_i, [_c_i, _c_i, _c_i, ctypes.POINTER(_c_sz)]),
    "molora_dispatch": (_c_i, [_c_p, _c_p, _c_i, _c_i, _c_i, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "molora_apply_workspace": (_c_i, [_c_p, _c_i, _c_i, _c_i, _c_i, _c_i, ctypes.POINTER(_c_sz)]),
    "molora_apply_path": (_c_i, [_c_p, _c_i, _c_i, _c_i, _c_i, ctypes.POINTER(_c_i)]),
    "molora_apply": (_c_i, [_c_p, _c_i, _c_p, _c_p, _c_i, _c_p, _c_i, _c_i, _c_i, _c_p, _c_p, _c_p, _c_p, _c_i,
                            _c_p, _c_sz, _c_p]),
    "molora_apply_multi_workspace": (_c_i, [_c_p, _c_i, _c_p, _c_i, _c_i, _c_i, _c_i, ctypes.POINTER(_c_sz)]),
    "molora_apply_multi": (_c_i, [_c_p, _c_i, _c_p, _c_p, _c_p, _c_i, _c_p, _c_i, _c_i, _c_i,  # hs .. k
                                  _c_p, _c_p, _c_p, _c_p, _c_i, _c_p, _c_sz, _c_p]),
    "molora_dispatch_apply_multi_workspace": (_c_i, [_c_p, _c_i, _c_p, _c_i, _c_i, _c_i, _c_i,
                                                     ctypes.POINTER(_c_sz)]),
    "molora_dispatch_apply_multi": (_c_i, [_c_p, _c_i, _c_p, _c_p, _c_p, _c_i, _c_p, _c_i, _c_i, _c_i,  # hs .. k
                                           _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,  # idx, w, counts .. inv
                                           _c_i, _c_p, _c_sz, _c_p]),
    "molora_seqpass_meta": (_c_i, [_c_p, _c_i, _c_i, _c_p, _c_p, _c_p, _c_p]),
    "molora_step_vocab": (_c_i, [_c_p, _c_i, _c_p, _c_i, _c_p, _c_p, _c_p, _c_i, _c_p, _c_i,  # hs .. y_dtype
                                 _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,  # idx, w, counts, offsets, perm, perm_w, inv
                                 _c_p, _c_sz, _c_p]),  # ws, ws_bytes, stream
    "molora_step_workspace": (_c_i, [_c_p, _c_i, _c_i, ctypes.POINTER(_c_sz)]),
    "molora_hotset_init_transposed": (_c_i, [ctypes.POINTER(_c_p), _c_i, _c_i, _c_f, _c_i, ctypes.POINTER(MoloraTarget),
                                             _c_i, _c_p, _c_sz, _c_p]),
    "molora_backward_workspace": (_c_i, [_c_p, _c_p, _c_i, _c_i, _c_i, _c_i, ctypes.POINTER(_c_sz)]),
    "molora_route_topk_backward": (_c_i, [_c_p, _c_p, _c_p, _c_i, _c_i, _c_i, _c_p, _c_p]),
    "molora_xf_workspace": (_c_i, [_c_i, _c_i, _c_i, ctypes.POINTER(MoloraXfLayer), _c_i, _c_i, _c_i,
                                   ctypes.POINTER(_c_sz)]),
    "molora_xf_forward": (_c_i, [_c_i, _c_i, _c_i, ctypes.POINTER(MoloraXfLayer), _c_i, _c_i, _c_p, _c_p, _c_i,
                                 _c_p, _c_p, _c_p, _c_p, _c_p, _c_sz, _c_p]),
    "molora_router_backward_workspace": (_c_i, [_c_i, _c_i, _c_i, ctypes.POINTER(_c_sz)]),
    "molora_router_backward": (_c_i, [_c_p, _c_i, _c_i, _c_p, _c_p, _c_p, _c_i, _c_p,  # x .. dlogits
                                      _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,  # dW1, db1, dW2, db2, dx0, dx
                                      _c_p, _c_sz, _c_p]),
    "molora_backward": (_c_i, [_c_p, _c_p, _c_i, _c_p, _c_p, _c_p, _c_i, _c_p, _c_i, _c_i, _c_i,  # hs .. k
                               _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,  # offsets .. dw
                               _c_p, _c_sz, _c_p]),  # ws, ws_bytes, stream
    "molora_step_vocab_noalloc": (_c_i, [_c_p, _c_i, _c_p, _c_i, _c_p, _c_p, _c_p, _c_i, _c_p, _c_i,  # hs .. y_dtype
                                         _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,  # idx .. inv
                                         _c_p]),  # stream
}
NOALLOC_SCRATCH_BYTES = 8 << 20

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                          f"(python -m token_adapter_routing_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols() -> Sequence[str]:
    return tuple(_SIGS)


def _check(rc: int):
    if rc != MOLORA_OK:
        raise MoloraError(rc, load_library().molora_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ----------------------------------------------------------------------------------- hot set

class HotSet:
    """Owns a molora_hotset descriptor and the torch slab it points into."""

    def __init__(self, handle: int, slab: torch.Tensor, K: int, r: int, scale: float, dims, layout: int,
                 transposed: bool = False):
        self.handle = handle
        self.slab = slab
        self.K, self.r, self.scale, self.dims, self.layout = K, r, scale, list(dims), layout
        self.transposed = transposed  # dims are the forward (d_in, d_out); the twin maps d_out -> d_in

    def close(self):
        if self.handle:
            _check(load_library().molora_hotset_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _targets(targets) -> Tuple[ctypes.Array, list]:
    arr = (MoloraTarget * len(targets))()
    dims = []
    for i, t in enumerate(targets):
        A, B = t
        K, d_in, r = A.shape
        K2, r2, d_out = B.shape
        if K2 != K or r2 != r:
            raise ValueError("A must be [K][d_in][r] and B [K][r][d_out]")
        arr[i] = MoloraTarget(int(d_in), int(d_out), _ptr(A, torch.bfloat16, "A"), _ptr(B, torch.bfloat16, "B"))
        dims.append((int(d_in), int(d_out)))
    return arr, dims


def molora_hotset_bytes(K: int, r: int, dims, layout: int = LAYOUT_DIRECT) -> int:
    arr = (MoloraTarget * len(dims))()
    for i, (d_in, d_out) in enumerate(dims):
        arr[i] = MoloraTarget(int(d_in), int(d_out), None, None)
    out = _c_sz()
    _check(load_library().molora_hotset_bytes(K, r, len(dims), arr, layout, ctypes.byref(out)))
    return out.value


def molora_hotset_init(targets, scale: float, layout: int = LAYOUT_DIRECT, slab: Optional[torch.Tensor] = None,
                       stream=None) -> HotSet:
    """targets: list of (A [K][d_in][r] bf16, B [K][r][d_out] bf16) device tensors."""
    lib = load_library()
    arr, dims = _targets(targets)
    K, _, r = targets[0][0].shape
    nbytes = molora_hotset_bytes(int(K), int(r), dims, layout)
    if slab is None:
        slab = torch.empty(nbytes, dtype=torch.uint8, device=targets[0][0].device)
    h = _c_p()
    _check(lib.molora_hotset_init(ctypes.byref(h), int(K), int(r), float(scale), len(dims), arr, layout,
                                  _ptr(slab, torch.uint8, "slab"), slab.numel(), _stream(stream)))
    return HotSet(h.value, slab, int(K), int(r), float(scale), dims, layout)


def molora_hotset_init_transposed(targets, scale: float, layout: int = LAYOUT_DIRECT,
                                  slab: Optional[torch.Tensor] = None, stream=None) -> HotSet:
    """The transposed twin of molora_hotset_init(targets): adapter e = (B_e^T, A_e^T), target t
    mapping d_out -> d_in (the adapters' part of dL/dx is molora_apply on it with x = dL/dy)."""
    lib = load_library()
    arr, dims = _targets(targets)
    K, _, r = targets[0][0].shape
    nbytes = molora_hotset_bytes(int(K), int(r), dims, layout)
    if slab is None:
        slab = torch.empty(nbytes, dtype=torch.uint8, device=targets[0][0].device)
    h = _c_p()
    _check(lib.molora_hotset_init_transposed(ctypes.byref(h), int(K), int(r), float(scale), len(dims), arr, layout,
                                             _ptr(slab, torch.uint8, "slab"), slab.numel(), _stream(stream)))
    return HotSet(h.value, slab, int(K), int(r), float(scale), dims, layout, transposed=True)


def molora_hotset_load(hs: HotSet, target: int, e: int, A: torch.Tensor, B: torch.Tensor, stream=None):
    """Write adapter e of `target` into its slot: A bf16 [d_in][r], B bf16 [r][d_out], device tensors.
    Only enqueues on `stream`; A and B must stay alive until the copy kernels have run."""
    d_in, d_out = hs.dims[target] if 0 <= target < len(hs.dims) else (None, None)
    if d_in is not None and (tuple(A.shape) != (d_in, hs.r) or tuple(B.shape) != (hs.r, d_out)):
        raise ValueError(f"A must be [{d_in}][{hs.r}] and B [{hs.r}][{d_out}]")
    _check(load_library().molora_hotset_load(hs.handle, int(target), int(e), _ptr(A, torch.bfloat16, "A"),
                                             _ptr(B, torch.bfloat16, "B"), _stream(stream)))


def molora_hotset_destroy(hs: HotSet):
    hs.close()


# ----------------------------------------------------------------------------------- routing

def molora_route_vocab(ids: torch.Tensor, bounds: Sequence[int], idx: Optional[torch.Tensor] = None,
                       w: Optional[torch.Tensor] = None, stream=None):
    N = ids.numel()
    K = len(bounds) - 1
    if idx is None:
        idx = torch.empty(N, dtype=torch.int32, device=ids.device)
    if w is None:
        w = torch.empty(N, dtype=torch.float32, device=ids.device)
    b = (ctypes.c_int32 * len(bounds))(*[int(v) for v in bounds])
    _check(load_library().molora_route_vocab(_ptr(ids, torch.int32, "ids"), N, ctypes.cast(b, _c_p), K,
                                             _ptr(idx, torch.int32, "idx"), _ptr(w, torch.float32, "w"),
                                             _stream(stream)))
    return idx, w


def molora_route_topk_workspace(N: int, d: int) -> int:
    out = _c_sz()
    _check(load_library().molora_route_topk_workspace(N, d, ctypes.byref(out)))
    return out.value


def molora_route_topk(k: int, K: int, x: Optional[torch.Tensor] = None, W1: Optional[torch.Tensor] = None,
                      b1: Optional[torch.Tensor] = None, W2: Optional[torch.Tensor] = None,
                      b2: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                      idx: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
                      flags: Optional[torch.Tensor] = None, want_flags: bool = True,
                      ws: Optional[torch.Tensor] = None, stream=None):
    """Router mode when W1 is given (W1 [64][d], W2 [K][64], nn.Linear layout), else logits mode.
    ``ws`` (uint8, molora_route_topk_workspace bytes) selects the two-launch first layer."""
    router = W1 is not None
    if router:
        N, d = x.shape
        dev = x.device
    else:
        N = logits.shape[0]
        d = 0
        dev = logits.device
    if logits is None:
        logits = torch.empty(N, K, dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(N, k, dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty(N, k, dtype=torch.float32, device=dev)
    if flags is None and want_flags:
        flags = torch.empty(N, dtype=torch.uint8, device=dev)
    _check(load_library().molora_route_topk(
        _ptr(x, torch.bfloat16, "x") if router else None, N, d,
        _ptr(W1, torch.bfloat16, "W1") if router else None, _ptr(b1, torch.float32, "b1") if router else None,
        _ptr(W2, torch.bfloat16, "W2") if router else None, _ptr(b2, torch.float32, "b2") if router else None,
        _ptr(logits, torch.float32, "logits"), K, k, _ptr(idx, torch.int32, "idx"), _ptr(w, torch.float32, "w"),
        _ptr(flags, torch.uint8, "flags"), _ptr(ws, None, "ws") if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream(stream)))
    return logits, idx, w, flags


# ----------------------------------------------------------------------------------- dispatch

def molora_dispatch_workspace(N: int, k: int, K: int) -> int:
    out = _c_sz()
    _check(load_library().molora_dispatch_workspace(N, k, K, ctypes.byref(out)))
    return out.value


def molora_dispatch(idx: torch.Tensor, w: torch.Tensor, K: int, k: int = 1, out=None, ws=None, stream=None):
    """Returns (counts, offsets, perm, perm_w, inv); ``out`` may supply those five tensors."""
    P = idx.numel()
    N = P // k
    dev = idx.device
    if out is None:
        out = (torch.empty(K, dtype=torch.int32, device=dev), torch.empty(K + 1, dtype=torch.int32, device=dev),
               torch.empty(max(P, 1), dtype=torch.int32, device=dev), torch.empty(max(P, 1), dtype=torch.float32, device=dev),
               torch.empty(max(P, 1), dtype=torch.int32, device=dev))
    counts, offsets, perm, perm_w, inv = out
    nws = molora_dispatch_workspace(N, k, K)
    if nws and ws is None:
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    _check(load_library().molora_dispatch(
        _ptr(idx, torch.int32, "idx"), _ptr(w, torch.float32, "w"), N, k, K, _ptr(counts, torch.int32, "counts"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(perm, torch.int32, "perm"), _ptr(perm_w, torch.float32, "perm_w"),
        _ptr(inv, torch.int32, "inv"), _ptr(ws, None, "ws") if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream(stream)))
    return counts, offsets, perm, perm_w, inv


# ----------------------------------------------------------------------------------- apply

def molora_apply_workspace(hs: HotSet, target: int, N: int, k: int, path: int = PATH_AUTO,
                           y_dtype=torch.float32) -> int:
    out = _c_sz()
    code = F32 if y_dtype == torch.float32 else BF16
    _check(load_library().molora_apply_workspace(hs.handle, target, N, k, code, path, ctypes.byref(out)))
    return out.value


def molora_apply_path(hs: HotSet, N: int, k: int = 1, path: int = PATH_AUTO, target: int = 0) -> int:
    """The path molora_apply runs for these arguments (AUTO resolved by the library's rule)."""
    out = _c_i()
    _check(load_library().molora_apply_path(hs.handle, target, N, k, path, ctypes.byref(out)))
    return out.value


def molora_apply(hs: HotSet, x: torch.Tensor, y0: torch.Tensor, offsets: torch.Tensor, perm: torch.Tensor,
                 perm_w: torch.Tensor, inv: torch.Tensor, k: int = 1, target: int = 0, y: Optional[torch.Tensor] = None,
                 y_dtype=None, path: int = PATH_AUTO, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    N = x.shape[0]
    d_out = hs.dims[target][1]
    if y is None:
        y = torch.empty(N, d_out, dtype=y_dtype or y0.dtype, device=x.device)
    need = molora_apply_workspace(hs, target, N, k, path, y.dtype)
    if need and (ws is None or ws.numel() < need):
        # a fresh workspace for this call (zero-filled, so that its contents are defined)
        ws = torch.zeros(need, dtype=torch.uint8, device=x.device)
    _check(load_library().molora_apply(
        hs.handle, target, _ptr(x, torch.bfloat16, "x"), _ptr(y0, None, "y0"), _dtype_code(y0), _ptr(y, None, "y"),
        _dtype_code(y), N, k, _ptr(offsets, torch.int32, "offsets"), _ptr(perm, torch.int32, "perm"),
        _ptr(perm_w, torch.float32, "perm_w"), _ptr(inv, torch.int32, "inv"), path,
        _ptr(ws, None, "ws") if ws is not None else None, ws.numel() if ws is not None else 0, _stream(stream)))
    return y


def molora_apply_multi_workspace(hs: HotSet, targets: Sequence[int], N: int, k: int, path: int = PATH_AUTO,
                                 y_dtype=torch.float32) -> int:
    out = _c_sz()
    tg = (ctypes.c_int * len(targets))(*targets)
    code = F32 if y_dtype == torch.float32 else BF16
    _check(load_library().molora_apply_multi_workspace(hs.handle, len(targets), tg, N, k, code, path,
                                                       ctypes.byref(out)))
    return out.value


def molora_apply_multi(hs: HotSet, xs: Sequence[torch.Tensor], y0s: Sequence[torch.Tensor], offsets: torch.Tensor,
                       perm: torch.Tensor, perm_w: torch.Tensor, inv: torch.Tensor, k: int = 1,
                       targets: Optional[Sequence[int]] = None, ys: Optional[Sequence[torch.Tensor]] = None,
                       y_dtype=None, path: int = PATH_AUTO, ws: Optional[torch.Tensor] = None, stream=None):
    """molora_apply for several targets that share one routing (one launch per phase)."""
    n = len(xs)
    targets = list(range(n)) if targets is None else list(targets)
    N = xs[0].shape[0]
    if ys is None:
        ys = [torch.empty(N, hs.dims[t][1], dtype=y_dtype or y0s[i].dtype, device=xs[0].device)
              for i, t in enumerate(targets)]
    need = molora_apply_multi_workspace(hs, targets, N, k, path, ys[0].dtype)
    if need and (ws is None or ws.numel() < need):
        ws = torch.zeros(need, dtype=torch.uint8, device=xs[0].device)
    tg = (ctypes.c_int * n)(*targets)
    xp = (_c_p * n)(*[_ptr(x, torch.bfloat16, "x") for x in xs])
    y0p = (_c_p * n)(*[_ptr(v, None, "y0") for v in y0s])
    yp = (_c_p * n)(*[_ptr(v, None, "y") for v in ys])
    _check(load_library().molora_apply_multi(
        hs.handle, n, tg, xp, y0p, _dtype_code(y0s[0]), yp, _dtype_code(ys[0]), N, k,
        _ptr(offsets, torch.int32, "offsets"), _ptr(perm, torch.int32, "perm"), _ptr(perm_w, torch.float32, "perm_w"),
        _ptr(inv, torch.int32, "inv"), path, _ptr(ws, None, "ws") if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream(stream)))
    return ys


def molora_dispatch_apply_multi_workspace(hs: HotSet, targets: Sequence[int], N: int, k: int, path: int = PATH_AUTO,
                                          y_dtype=torch.float32) -> int:
    out = _c_sz()
    tg = (ctypes.c_int * len(targets))(*targets)
    code = F32 if y_dtype == torch.float32 else BF16
    _check(load_library().molora_dispatch_apply_multi_workspace(hs.handle, len(targets), tg, N, k, code, path,
                                                                ctypes.byref(out)))
    return out.value


def molora_dispatch_apply_multi(hs: HotSet, xs: Sequence[torch.Tensor], y0s: Sequence[torch.Tensor], idx: torch.Tensor,
                                w: torch.Tensor, K: int, k: int = 1, targets: Optional[Sequence[int]] = None,
                                ys: Optional[Sequence[torch.Tensor]] = None, y_dtype=None, path: int = PATH_AUTO,
                                meta=None, ws: Optional[torch.Tensor] = None, stream=None):
    """molora_dispatch of (idx, w) then molora_apply_multi on its outputs, in one call.
    Returns (ys, (counts, offsets, perm, perm_w, inv)); ``meta`` may supply those five."""
    n = len(xs)
    targets = list(range(n)) if targets is None else list(targets)
    N = xs[0].shape[0]
    dev = xs[0].device
    if ys is None:
        ys = [torch.empty(N, hs.dims[t][1], dtype=y_dtype or y0s[i].dtype, device=dev) for i, t in enumerate(targets)]
    if meta is None:
        P = N * k
        meta = (torch.empty(K, dtype=torch.int32, device=dev), torch.empty(K + 1, dtype=torch.int32, device=dev),
                torch.empty(P, dtype=torch.int32, device=dev), torch.empty(P, dtype=torch.float32, device=dev),
                torch.empty(P, dtype=torch.int32, device=dev))
    counts, offsets, perm, perm_w, inv = meta
    need = molora_dispatch_apply_multi_workspace(hs, targets, N, k, path, ys[0].dtype)
    if need and (ws is None or ws.numel() < need):
        ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    tg = (ctypes.c_int * n)(*targets)
    xp = (_c_p * n)(*[_ptr(x, torch.bfloat16, "x") for x in xs])
    y0p = (_c_p * n)(*[_ptr(v, None, "y0") for v in y0s])
    yp = (_c_p * n)(*[_ptr(v, None, "y") for v in ys])
    _check(load_library().molora_dispatch_apply_multi(
        hs.handle, n, tg, xp, y0p, _dtype_code(y0s[0]), yp, _dtype_code(ys[0]), N, k,
        _ptr(idx, torch.int32, "idx"), _ptr(w, torch.float32, "w"), _ptr(counts, torch.int32, "counts"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(perm, torch.int32, "perm"), _ptr(perm_w, torch.float32, "perm_w"),
        _ptr(inv, torch.int32, "inv"), path, _ptr(ws, None, "ws") if ws is not None else None,
        ws.numel() if ws is not None else 0, _stream(stream)))
    return ys, meta


def molora_step_workspace(hs: HotSet, target: int, N: int) -> int:
    out = _c_sz()
    _check(load_library().molora_step_workspace(hs.handle, target, N, ctypes.byref(out)))
    return out.value


def molora_step_vocab(hs: HotSet, ids: torch.Tensor, bounds: Sequence[int], x: torch.Tensor, y0: torch.Tensor,
                      target: int = 0, y: Optional[torch.Tensor] = None, y_dtype=None, route=None, meta=None,
                      ws: Optional[torch.Tensor] = None, stream=None):
    """route_vocab + dispatch + apply (k = 1) in one call.  Returns (y, (idx, w),
    (counts, offsets, perm, perm_w, inv)); `route` and `meta` may supply those buffers.
    `ws` (uint8, 256-byte aligned, at least molora_step_workspace bytes, no initial contents
    needed) selects the split step over 512-wide slices (two launches); without it the
    one-launch tile step runs.  Above 4096 tokens routing and dispatch run as launches of their
    own first.
    """
    N = ids.numel()
    K = len(bounds) - 1
    dev = ids.device
    d_out = hs.dims[target][1]
    if y is None:
        y = torch.empty(N, d_out, dtype=y_dtype or y0.dtype, device=dev)
    if route is None:
        route = (torch.empty(max(N, 1), dtype=torch.int32, device=dev), torch.empty(max(N, 1), dtype=torch.float32, device=dev))
    if meta is None:
        meta = (torch.empty(K, dtype=torch.int32, device=dev), torch.empty(K + 1, dtype=torch.int32, device=dev),
                torch.empty(max(N, 1), dtype=torch.int32, device=dev), torch.empty(max(N, 1), dtype=torch.float32, device=dev),
                torch.empty(max(N, 1), dtype=torch.int32, device=dev))
    b = (ctypes.c_int32 * len(bounds))(*[int(v) for v in bounds])
    idx, w = route
    counts, offsets, perm, perm_w, inv = meta
    _check(load_library().molora_step_vocab(
        hs.handle, target, _ptr(ids, torch.int32, "ids"), N, ctypes.cast(b, _c_p), _ptr(x, torch.bfloat16, "x"),
        _ptr(y0, None, "y0"), _dtype_code(y0), _ptr(y, None, "y"), _dtype_code(y), _ptr(idx, torch.int32, "idx"),
        _ptr(w, torch.float32, "w"), _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(perm, torch.int32, "perm"), _ptr(perm_w, torch.float32, "perm_w"), _ptr(inv, torch.int32, "inv"),
        _ptr(ws, None, "ws") if ws is not None else None, ws.numel() if ws is not None else 0, _stream(stream)))
    return y, route, meta


def molora_step_vocab_noalloc(hs: HotSet, ids: torch.Tensor, bounds: Sequence[int], x: torch.Tensor,
                              y0: torch.Tensor, target: int = 0, y: Optional[torch.Tensor] = None, y_dtype=None,
                              route=None, meta=None, stream=None):
    """molora_step_vocab with the library's own device scratch instead of a caller workspace
    (the entry point allocates nothing).  Outputs that are not supplied are allocated here, by
    torch, before the call; pass all of them to keep the call allocation-free."""
    N = ids.numel()
    K = len(bounds) - 1
    dev = ids.device
    d_out = hs.dims[target][1]
    if y is None:
        y = torch.empty(N, d_out, dtype=y_dtype or y0.dtype, device=dev)
    if route is None:
        route = (torch.empty(max(N, 1), dtype=torch.int32, device=dev), torch.empty(max(N, 1), dtype=torch.float32, device=dev))
    if meta is None:
        meta = (torch.empty(K, dtype=torch.int32, device=dev), torch.empty(K + 1, dtype=torch.int32, device=dev),
                torch.empty(max(N, 1), dtype=torch.int32, device=dev), torch.empty(max(N, 1), dtype=torch.float32, device=dev),
                torch.empty(max(N, 1), dtype=torch.int32, device=dev))
    b = (ctypes.c_int32 * len(bounds))(*[int(v) for v in bounds])
    idx, w = route
    counts, offsets, perm, perm_w, inv = meta
    _check(load_library().molora_step_vocab_noalloc(
        hs.handle, target, _ptr(ids, torch.int32, "ids"), N, ctypes.cast(b, _c_p), _ptr(x, torch.bfloat16, "x"),
        _ptr(y0, None, "y0"), _dtype_code(y0), _ptr(y, None, "y"), _dtype_code(y), _ptr(idx, torch.int32, "idx"),
        _ptr(w, torch.float32, "w"), _ptr(counts, torch.int32, "counts"), _ptr(offsets, torch.int32, "offsets"),
        _ptr(perm, torch.int32, "perm"), _ptr(perm_w, torch.float32, "perm_w"), _ptr(inv, torch.int32, "inv"),
        _stream(stream)))
    return y, route, meta


def molora_seqpass_meta(idx: torch.Tensor, K: int, stream=None):
    """Returns (offsets [K][K+1], perm [N], perm_w [K][N]) for K one-hot passes."""
    N = idx.numel()
    dev = idx.device
    offsets = torch.empty(K, K + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(N, 1), dtype=torch.int32, device=dev)
    perm_w = torch.empty(K, max(N, 1), dtype=torch.float32, device=dev)
    _check(load_library().molora_seqpass_meta(_ptr(idx, torch.int32, "idx"), N, K, _ptr(offsets, torch.int32, "offsets"),
                                              _ptr(perm, torch.int32, "perm"), _ptr(perm_w, torch.float32, "perm_w"),
                                              _stream(stream)))
    return offsets, perm, perm_w


# ----------------------------------------------------------------------------------- backward

def molora_backward_workspace(hs: HotSet, hs_t: HotSet, N: int, k: int = 1, target: int = 0,
                              dx_dtype=torch.bfloat16) -> int:
    n = _c_sz()
    _check(load_library().molora_backward_workspace(hs.handle, hs_t.handle, int(target), int(N), int(k),
                                                    BF16 if dx_dtype == torch.bfloat16 else F32, ctypes.byref(n)))
    return n.value


def molora_backward(hs: HotSet, hs_t: HotSet, x: torch.Tensor, gy: torch.Tensor, offsets: torch.Tensor,
                    perm: torch.Tensor, perm_w: torch.Tensor, inv: torch.Tensor, k: int = 1, target: int = 0,
                    dx0: Optional[torch.Tensor] = None, dx: Optional[torch.Tensor] = None,
                    dA: Optional[torch.Tensor] = None, dB: Optional[torch.Tensor] = None,
                    dw: Optional[torch.Tensor] = None, want=("dx", "dA", "dB", "dw"),
                    ws: Optional[torch.Tensor] = None, stream=None):
    """Gradients of molora_apply for one target: dx = dx0 + the adapters' part of dL/dx (dx0
    defaults to zeros of gy's dtype), dA fp32 [K][d_in][r], dB fp32 [K][r][d_out], dw fp32 [N*k].
    Outputs named in `want` and not given are allocated; the others are skipped."""
    N = x.shape[0]
    d_in, d_out = hs.dims[target]
    dev = x.device
    if "dx" in want and dx is None:
        dx = torch.empty(N, d_in, dtype=dx0.dtype if dx0 is not None else gy.dtype, device=dev)
    if dx is not None and dx0 is None:
        dx0 = torch.zeros(N, d_in, dtype=dx.dtype, device=dev)
    if "dA" in want and dA is None:
        dA = torch.empty(hs.K, d_in, hs.r, dtype=torch.float32, device=dev)
    if "dB" in want and dB is None:
        dB = torch.empty(hs.K, hs.r, d_out, dtype=torch.float32, device=dev)
    if "dw" in want and dw is None:
        dw = torch.empty(N * k, dtype=torch.float32, device=dev)
    dx_dtype = dx.dtype if dx is not None else torch.bfloat16
    need = molora_backward_workspace(hs, hs_t, N, k, target, dx_dtype)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(load_library().molora_backward(
        hs.handle, hs_t.handle, int(target), _ptr(x, torch.bfloat16, "x"), _ptr(gy, torch.bfloat16, "gy"),
        _ptr(dx0, None, "dx0"), _dtype_code(dx0) if dx0 is not None else BF16, _ptr(dx, None, "dx"),
        _dtype_code(dx) if dx is not None else BF16, N, int(k), _ptr(offsets, torch.int32, "offsets"),
        _ptr(perm, torch.int32, "perm"), _ptr(perm_w, torch.float32, "perm_w"), _ptr(inv, torch.int32, "inv"),
        _ptr(dA, torch.float32, "dA"), _ptr(dB, torch.float32, "dB"), _ptr(dw, torch.float32, "dw"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))
    return dx, dA, dB, dw


def molora_route_topk_backward(idx: torch.Tensor, w: torch.Tensor, dw: torch.Tensor, K: int,
                               dlogits: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """dL/dlogits [N][K] fp32 through the softmax over the selected logits (idx, w, dw [N][k])."""
    N, k = idx.shape if idx.dim() == 2 else (idx.numel(), 1)
    if dlogits is None:
        dlogits = torch.empty(N, K, dtype=torch.float32, device=idx.device)
    _check(load_library().molora_route_topk_backward(
        _ptr(idx, torch.int32, "idx"), _ptr(w, torch.float32, "w"), _ptr(dw, torch.float32, "dw"), int(N), int(K),
        int(k), _ptr(dlogits, torch.float32, "dlogits"), _stream(stream)))
    return dlogits


def molora_router_backward_workspace(N: int, d: int, K: int) -> int:
    n = _c_sz()
    _check(load_library().molora_router_backward_workspace(int(N), int(d), int(K), ctypes.byref(n)))
    return n.value


def molora_router_backward(x: torch.Tensor, W1: torch.Tensor, b1: Optional[torch.Tensor], W2: torch.Tensor,
                           dlogits: torch.Tensor, dx0: Optional[torch.Tensor] = None,
                           want=("dW1", "db1", "dW2", "db2", "dx"), out=None, ws: Optional[torch.Tensor] = None,
                           stream=None):
    """Router MLP gradients (W1 [64][d], W2 [K][64] bf16): returns dict of the requested fp32
    outputs dW1 [64][d], db1 [64], dW2 [K][64], db2 [K], dx [N][d] (= dx0 + router part)."""
    N, d = x.shape
    K = W2.shape[0]
    o = dict(out or {})
    shapes = {"dW1": (64, d), "db1": (64,), "dW2": (K, 64), "db2": (K,), "dx": (N, d)}
    for name in want:
        if name not in o:
            o[name] = torch.empty(*shapes[name], dtype=torch.float32, device=x.device)
    need = molora_router_backward_workspace(N, d, K)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    g = o.get
    _check(load_library().molora_router_backward(
        _ptr(x, torch.bfloat16, "x"), int(N), int(d), _ptr(W1, torch.bfloat16, "W1"), _ptr(b1, torch.float32, "b1"),
        _ptr(W2, torch.bfloat16, "W2"), int(K), _ptr(dlogits, torch.float32, "dlogits"),
        _ptr(g("dW1"), torch.float32, "dW1"), _ptr(g("db1"), torch.float32, "db1"), _ptr(g("dW2"), torch.float32, "dW2"),
        _ptr(g("db2"), torch.float32, "db2"), _ptr(dx0, torch.float32, "dx0"), _ptr(g("dx"), torch.float32, "dx"),
        _ptr(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)))
    return o


# ----------------------------------------------------------------------------------- decoder

XF_TARGETS = ("q", "k", "v", "o", "gate", "up", "down")


class XfModel:
    """Device weights of the synthetic decoder: per layer norm1, norm2 (bf16 [d]), the seven
    base projections (bf16, nn.Linear layout) and an optional 7-target LoRA hot set."""

    def __init__(self, d: int, f: int, layers):
        self.d, self.f = d, f
        self.layers = layers  # list of dicts: norm1, norm2, W (list of 7), lora (HotSet or None)
        arr = (MoloraXfLayer * len(layers))()
        for i, L in enumerate(layers):
            arr[i].norm1 = _ptr(L["norm1"], torch.bfloat16, "norm1")
            arr[i].norm2 = _ptr(L["norm2"], torch.bfloat16, "norm2")
            for t in range(7):
                arr[i].W[t] = _ptr(L["W"][t], torch.bfloat16, f"W[{t}]")
            arr[i].lora = L["lora"].handle if L.get("lora") is not None else None
        self._arr = arr


def molora_xf_workspace(model: XfModel, n_seq: int, seq_len: int, k: int = 1) -> int:
    n = _c_sz()
    _check(load_library().molora_xf_workspace(model.d, model.f, len(model.layers), model._arr, int(n_seq),
                                              int(seq_len), int(k), ctypes.byref(n)))
    return n.value


def molora_xf_forward(model: XfModel, x: torch.Tensor, n_seq: int, seq_len: int, route=None, k: int = 1,
                      out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """Decoder forward; route = (offsets, perm, perm_w, inv) of molora_dispatch (None when no
    layer has LoRA)."""
    if out is None:
        out = torch.empty_like(x)
    need = molora_xf_workspace(model, n_seq, seq_len, k)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    offsets, perm, perm_w, inv = route if route is not None else (None, None, None, None)
    _check(load_library().molora_xf_forward(
        model.d, model.f, len(model.layers), model._arr, int(n_seq), int(seq_len), _ptr(x, torch.bfloat16, "x"),
        _ptr(out, torch.bfloat16, "out"), int(k), _ptr(offsets, torch.int32, "offsets"), _ptr(perm, torch.int32, "perm"),
        _ptr(perm_w, torch.float32, "perm_w"), _ptr(inv, torch.int32, "inv"), _ptr(ws, torch.uint8, "ws"), ws.numel(),
        _stream(stream)))
    return out
