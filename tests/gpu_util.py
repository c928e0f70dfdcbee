"""Helpers for the GPU parity tests: device copies of synthetic inputs and the comparison
bars.  Comparisons always run the oracle (fp64) on the same bits the GPU received."""
import numpy as np
import pytest
import torch

import synth
from oracle import bf16_to_f64

# Output bars for floating point (the tolerance fixed for this path): relative Frobenius
# error <= 5e-3 and max-abs error <= 2e-2 on unit-scale data.  The design bound is tighter:
# fp32 accumulation of exact bf16 products and h carried as a bf16 hi/lo pair leave errors
# around 1e-5 of the output scale, so 2e-3 max-abs would already flag a lost term.
FROB_TOL = 5e-3
MAXABS_TOL = 2e-2
DESIGN_MAXABS = 2e-3
W_TOL = 2.0 ** -20


def gpu_available():
    return torch.cuda.is_available()


def need_gpu():
    if not gpu_available():
        pytest.skip("no GPU visible")
    import token_adapter_routing_amd as m
    m.load_library()  # raises if the HIP library is missing: no fallback
    return m


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return bf16_to_f64(t.cpu().view(torch.int16).numpy().view(np.uint16))
    return t.cpu().numpy()


def f64(bits):
    return bf16_to_f64(bits)


def check_float_output(y_gpu: np.ndarray, y_ref: np.ndarray, y0: np.ndarray = None, design=True):
    """fp32 outputs: Frobenius and max-abs bars on y and, when y0 is given, on delta = y - y0."""
    pairs = [(y_gpu, y_ref)]
    if y0 is not None:
        pairs.append((y_gpu - y0, y_ref - y0))
    for g, r in pairs:
        if r.size == 0:
            continue
        err = g - r
        nref = np.linalg.norm(r)
        frob = np.linalg.norm(err) / (nref if nref > 0 else 1.0)
        mx = float(np.max(np.abs(err)))
        assert frob <= FROB_TOL, f"relative Frobenius error {frob:.3e} > {FROB_TOL}"
        assert mx <= MAXABS_TOL, f"max-abs error {mx:.3e} > {MAXABS_TOL}"
        if design:
            assert mx <= DESIGN_MAXABS, f"max-abs error {mx:.3e} above the design bound {DESIGN_MAXABS}"


def bf16_round(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def check_bf16_output(y_gpu: np.ndarray, y_ref: np.ndarray):
    """bf16 outputs: every element within one bf16 ulp of the rounded reference -- or, for
    values so small that one bf16 ulp is below the fp32 path's own error, within that error
    (DESIGN_MAXABS) of the exact value -- plus the Frobenius bar."""
    rr = bf16_round(y_ref)
    mag = np.maximum(np.abs(rr), np.finfo(np.float32).tiny)
    ulp = np.exp2(np.floor(np.log2(mag)) - 7)
    bad = (np.abs(y_gpu - rr) > ulp) & (np.abs(y_gpu - y_ref) > DESIGN_MAXABS)
    if bad.any():
        where = np.argwhere(bad)[:3]
        vals = [(float(y_gpu[tuple(i)]), float(y_ref[tuple(i)])) for i in where]
        raise AssertionError(f"{int(bad.sum())} elements beyond 1 bf16 ulp; (gpu, ref) = {vals}")
    err = np.linalg.norm(y_gpu - y_ref) / max(np.linalg.norm(y_ref), 1e-30)
    assert err <= FROB_TOL
