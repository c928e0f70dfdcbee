"""Seeded synthetic inputs for the per-token adapter-routing workloads.

This module only draws random numbers and rounds them to the storage formats
the path consumes (bf16 bit patterns, fp32, int32).  It holds none of the
method's arithmetic: no routing, no dispatch, no LoRA contraction.  Both the
CPU oracle's tests and the GPU path's tests/benchmark take their inputs from
here, so the two sides always see identical bits.

Every generator is keyed by ``SeedSequence([20260316, case_id, tensor_id])``
so that any tensor can be regenerated alone.

Workload recipes (MoLoRA pages: thelatestinai.com, Tables 1, 3, 10 and 16;
the Figure 1 caption for interleaved modalities; the value distributions are
our readings, listed in the design notes):

* vocab routing: token ids uniform over the union of the adapters' vocabulary
  ranges; adapter ``e`` owns ``[8192 e, 8192 (e+1))``.
* 4-modality benchmark: modality runs with geometric lengths (mean 64) and
  mixing proportions 0.4/0.3/0.15/0.15, ids uniform inside the run's range.
* learned top-k: x drawn as N(mu_c, 1) around 4 cluster means with
  per-component magnitude 0.5 and mix 0.4/0.3/0.2/0.1; router MLP d->64->K
  initialised like ``nn.Linear`` (U(+-1/sqrt(fan_in))).
* decode sweep: one uniformly random adapter per token.
* stress: a biased random router whose logits are ``ln p_e + Gumbel`` with
  Zipf(s=1.1) popularity ``p_e ~ (e+1)^-1.1``.
* LoRA weights: A_e ~ N(0, 1/d_in), B_e ~ N(0, 1/r); base output y0 ~ N(0,1).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

BASE_SEED = 20260316

# tensor ids inside one case (stable: changing them changes every input)
T_IDS, T_X, T_Y0, T_A, T_B, T_W1, T_B1, T_W2, T_B2, T_LOGITS, T_IDX, T_RUNS, T_CLUSTER, T_GY, T_DX0, T_BASE, T_NORM = range(17)


def rng_for(case_id: int, tensor_id: int, sub: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED, case_id, tensor_id, sub]))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return the uint16 bit patterns."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def normal_bf16(case_id: int, tensor_id: int, shape, std: float = 1.0, mean=0.0, sub: int = 0) -> np.ndarray:
    g = rng_for(case_id, tensor_id, sub)
    v = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    if not (isinstance(mean, float) and mean == 0.0):
        v += np.asarray(mean, dtype=np.float32)
    return to_bf16_bits(v)


@dataclass
class Target:
    """One LoRA target (projection): A [K][d_in][r], B [K][r][d_out] as bf16 bits."""
    name: str
    d_in: int
    d_out: int
    A: np.ndarray
    B: np.ndarray
    x: np.ndarray      # bf16 bits [N][d_in]: the input this target reads
    y0: np.ndarray     # bf16 bits [N][d_out]: base output


@dataclass
class Case:
    name: str
    case_id: int
    N: int
    K: int
    r: int
    k: int
    scale: float                       # alpha / r
    targets: List[Target]
    ids: Optional[np.ndarray] = None   # int32 [N] token ids (vocab routing)
    bounds: Optional[np.ndarray] = None  # int32 [K+1] vocabulary range bounds
    idx: Optional[np.ndarray] = None   # int32 [N] given routing (decode sweep)
    logits: Optional[np.ndarray] = None  # fp32 [N][K] given logits (stress case)
    router: Optional[Dict[str, np.ndarray]] = None  # W1,b1,W2,b2 (bf16 bits / fp32)
    info: Dict[str, object] = field(default_factory=dict)


def _lora_weights(case_id: int, t: int, K: int, d_in: int, d_out: int, r: int):
    A = normal_bf16(case_id, T_A, (K, d_in, r), std=1.0 / np.sqrt(d_in), sub=t)
    B = normal_bf16(case_id, T_B, (K, r, d_out), std=1.0 / np.sqrt(r), sub=t)
    return A, B


def vocab_bounds(K: int, width: int = 8192) -> np.ndarray:
    return (np.arange(K + 1, dtype=np.int64) * width).astype(np.int32)


def modality_runs(case_id: int, N: int, probs, mean_len: float = 64.0) -> np.ndarray:
    """Per-token modality labels in contiguous runs: run lengths ~ Geometric(1/mean_len)
    on {1, 2, ...}; each run's modality drawn i.i.d. from ``probs``."""
    g = rng_for(case_id, T_RUNS)
    labels = np.empty(N, dtype=np.int32)
    pos = 0
    probs = np.asarray(probs, dtype=np.float64)
    while pos < N:
        L = int(g.geometric(1.0 / mean_len))
        m = int(g.choice(len(probs), p=probs))
        labels[pos:pos + L] = m
        pos += L
    return labels


def ids_for_labels(case_id: int, labels: np.ndarray, bounds: np.ndarray) -> np.ndarray:
    g = rng_for(case_id, T_IDS)
    lo = bounds[labels].astype(np.int64)
    hi = bounds[labels + 1].astype(np.int64)
    return (lo + np.floor(g.random(labels.shape[0]) * (hi - lo)).astype(np.int64)).astype(np.int32)


def vocab_case(N: int = 256, d: int = 512, K: int = 4, r: int = 8, case_id: int = 0,
               runs: bool = False, probs=(0.4, 0.3, 0.15, 0.15), name: Optional[str] = None,
               scale: float = 2.0) -> Case:
    """Vocabulary-routed case.  ``runs=False``: ids uniform in [0, 8192 K).
    ``runs=True``: interleaved modality runs (the 4-modality benchmark)."""
    bounds = vocab_bounds(K)
    if runs:
        labels = modality_runs(case_id, N, probs)
        ids = ids_for_labels(case_id, labels, bounds)
    else:
        g = rng_for(case_id, T_IDS)
        ids = g.integers(0, int(bounds[-1]), size=N, dtype=np.int64).astype(np.int32)
    x = normal_bf16(case_id, T_X, (N, d))
    y0 = normal_bf16(case_id, T_Y0, (N, d))
    A, B = _lora_weights(case_id, 0, K, d, d, r)
    tgt = Target("proj", d, d, A, B, x, y0)
    return Case(name or ("vocab_runs" if runs else "vocab"), case_id, N, K, r, 1, scale, [tgt],
                ids=ids, bounds=bounds)


def tiny_vocab() -> Case:
    """N=256, d=512, K=4, r=8, k=1; ids uniform in [0, 32768)."""
    return vocab_case(256, 512, 4, 8, case_id=0, runs=False, name="tiny_vocab")


def modality4(N: int = 2048, d: int = 4096, r: int = 16) -> Case:
    """4-modality kernel benchmark: N=2048, d=4096, K=4 (text/image/audio/video), r=16."""
    return vocab_case(N, d, 4, r, case_id=1, runs=True, name="modality4")


QWEN3_1P7B_TARGETS = (("q", 2048, 2048), ("k", 2048, 1024), ("v", 2048, 1024), ("o", 2048, 2048),
                      ("gate", 2048, 6144), ("up", 2048, 6144), ("down", 6144, 2048))


def router_mlp(case_id: int, d: int, H: int, K: int) -> Dict[str, np.ndarray]:
    """Router weights initialised like nn.Linear: U(-1/sqrt(fan_in), 1/sqrt(fan_in)).
    W1 [d][H] and W2 [H][K] as bf16 bits; b1 [H], b2 [K] fp32."""
    g1 = rng_for(case_id, T_W1)
    g2 = rng_for(case_id, T_W2)
    gb1 = rng_for(case_id, T_B1)
    gb2 = rng_for(case_id, T_B2)
    a1 = 1.0 / np.sqrt(d)
    a2 = 1.0 / np.sqrt(H)
    W1 = to_bf16_bits(g1.uniform(-a1, a1, size=(d, H)).astype(np.float32))
    W2 = to_bf16_bits(g2.uniform(-a2, a2, size=(H, K)).astype(np.float32))
    b1 = gb1.uniform(-a1, a1, size=H).astype(np.float32)
    b2 = gb2.uniform(-a2, a2, size=K).astype(np.float32)
    return {"W1": W1, "b1": b1, "W2": W2, "b2": b2, "H": H}


def clustered_x(case_id: int, N: int, d: int, mix=(0.4, 0.3, 0.2, 0.1), mu: float = 0.5):
    g = rng_for(case_id, T_CLUSTER)
    signs = np.where(g.random((len(mix), d)) < 0.5, -1.0, 1.0).astype(np.float32)
    means = (mu * signs).astype(np.float32)
    labels = g.choice(len(mix), size=N, p=np.asarray(mix, dtype=np.float64)).astype(np.int32)
    gx = rng_for(case_id, T_X)
    v = gx.standard_normal(size=(N, d), dtype=np.float32)
    v += means[labels]
    return to_bf16_bits(v), labels


def qwen_layer(N: int = 4096, K: int = 4, r: int = 16, k: int = 2, case_id: int = 2,
               targets=QWEN3_1P7B_TARGETS, H: int = 64) -> Case:
    """Learned top-k MoLoRA on one Qwen3-1.7B-shaped layer (d=2048, 7 targets, k=2).
    q/k/v/gate/up read the clustered x; o and down read their own N(0,1) inputs."""
    d = targets[0][1]
    x, labels = clustered_x(case_id, N, d)
    tg = []
    for t, (name, d_in, d_out) in enumerate(targets):
        # o and down take their own inputs (no attention / MLP is computed here)
        xin = normal_bf16(case_id, T_X, (N, d_in), sub=100 + t) if name in ("o", "down") else x
        y0 = normal_bf16(case_id, T_Y0, (N, d_out), sub=t)
        A, B = _lora_weights(case_id, t, K, d_in, d_out, r)
        tg.append(Target(name, d_in, d_out, A, B, xin, y0))
    router = router_mlp(case_id, d, H, K)
    return Case("qwen_layer", case_id, N, K, r, k, 2.0, tg, router=router, info={"cluster": labels})


def decode_batch(B: int, K: int = 64, d: int = 4096, r: int = 16, case_id: int = 3) -> Case:
    """Decode sweep: B tokens, K hot-set adapters, one uniformly random adapter per token."""
    g = rng_for(case_id, T_IDX, B)
    idx = g.integers(0, K, size=B, dtype=np.int64).astype(np.int32)
    x = normal_bf16(case_id, T_X, (B, d), sub=B)
    y0 = normal_bf16(case_id, T_Y0, (B, d), sub=B)
    A, B_ = _lora_weights(case_id, 0, K, d, d, r)
    return Case(f"decode_B{B}", case_id, B, K, r, 1, 2.0, [Target("proj", d, d, A, B_, x, y0)], idx=idx)


def mixed_batch(N: int, probs, d: int = 4096, r: int = 64, case_id: int = 6, sub: int = 0) -> Case:
    """Adapter-usage mix of the tiling comparison (thelatestinai.com, Table 9: 25% each,
    80/10/5/5, 95/2/2/1): one adapter per token drawn i.i.d. from `probs` (K = len(probs))."""
    K = len(probs)
    g = rng_for(case_id, T_IDX, sub)
    p = np.asarray(probs, dtype=np.float64)
    idx = g.choice(K, size=N, p=p / p.sum()).astype(np.int32)
    x = normal_bf16(case_id, T_X, (N, d), sub=sub)
    y0 = normal_bf16(case_id, T_Y0, (N, d), sub=sub)
    A, B = _lora_weights(case_id, 0, K, d, d, r)
    return Case(f"mix_{K}_{N}", case_id, N, K, r, 1, 2.0, [Target("proj", d, d, A, B, x, y0)], idx=idx)


def zipf_logits(case_id: int, N: int, K: int, s: float = 1.1, sub: int = 0) -> np.ndarray:
    """Biased random router: logits ln p_e + G with G ~ Gumbel(0,1) and p_e ~ (e+1)^-s."""
    p = (np.arange(1, K + 1, dtype=np.float64) ** -s)
    p /= p.sum()
    g = rng_for(case_id, T_LOGITS, sub)
    u = g.random((N, K))
    u = np.clip(u, 1e-300, None)
    gumbel = -np.log(-np.log(u))
    return (np.log(p)[None, :] + gumbel).astype(np.float32)


def stress(k: int, N: int = 16384, K: int = 16, r: int = 64, d: int = 4096, case_id: int = 4) -> Case:
    """Stress case: K=16 adapters of rank 64, d=4096, Zipf(1.1)-skewed biased random router."""
    logits = zipf_logits(case_id, N, K)
    x = normal_bf16(case_id, T_X, (N, d))
    y0 = normal_bf16(case_id, T_Y0, (N, d))
    A, B = _lora_weights(case_id, 0, K, d, d, r)
    return Case(f"stress_k{k}", case_id, N, K, r, k, 2.0, [Target("proj", d, d, A, B, x, y0)], logits=logits)


def small_int_case(N: int, d_in: int, d_out: int, K: int, r: int, seed: int = 7, k: int = 1, lo: int = -3, hi: int = 4):
    """Inputs made of small integers, exact in bf16 and with every intermediate sum exact in fp32."""
    g = rng_for(90, seed)
    x = g.integers(lo, hi, size=(N, d_in)).astype(np.float32)
    A = g.integers(lo, hi, size=(K, d_in, r)).astype(np.float32)
    B = g.integers(lo, hi, size=(K, r, d_out)).astype(np.float32)
    y0 = g.integers(-8, 9, size=(N, d_out)).astype(np.float32)
    return to_bf16_bits(x), to_bf16_bits(A), to_bf16_bits(B), to_bf16_bits(y0)


def grad_case(case_id: int, N: int, d_in: int, d_out: int, sub: int = 0):
    """Upstream gradient dL/dy [N][d_out] and the rest of dL/dx [N][d_in] of a backward case,
    bf16 bits, N(0, 1)."""
    return (normal_bf16(case_id, T_GY, (N, d_out), sub=sub), normal_bf16(case_id, T_DX0, (N, d_in), sub=sub))


XF_TARGETS = ("q", "k", "v", "o", "gate", "up", "down")


def xf_mlp_width(d: int) -> int:
    """MLP width of the synthetic decoder: 8d/3 rounded up to a multiple of 128."""
    return -(-(8 * d) // (3 * 128)) * 128


def xf_dims(d: int, f: int):
    """(d_in, d_out) of the seven LoRA targets, in XF_TARGETS order."""
    return [(d, d), (d, d), (d, d), (d, d), (d, f), (d, f), (f, d)]


def xf_layers(case_id: int, d: int, L: int, K: int, r: int, f: int = None):
    """Random decoder weights as bf16 bits: RMSNorm weights 1 + N(0, 0.1^2); base projections
    N(0, 1/fan_in) in nn.Linear layout [out][in]; per target K LoRA adapters
    A [K][d_in][r] ~ N(0, 1/d_in), B [K][r][d_out] ~ N(0, 1/(16 r)) (deltas about a quarter of
    the base output)."""
    f = f or xf_mlp_width(d)
    layers = []
    for l in range(L):
        sub = 1000 * (l + 1)
        lay = {"norm1": normal_bf16(case_id, T_NORM, (d,), std=0.1, mean=1.0, sub=sub),
               "norm2": normal_bf16(case_id, T_NORM, (d,), std=0.1, mean=1.0, sub=sub + 1)}
        for i, (name, (din, dout)) in enumerate(zip(("Wq", "Wk", "Wv", "Wo", "Wgate", "Wup", "Wdown"),
                                                    xf_dims(d, f))):
            lay[name] = normal_bf16(case_id, T_BASE, (dout, din), std=1.0 / np.sqrt(din), sub=sub + i)
        lay["A"], lay["B"] = [], []
        for i, (din, dout) in enumerate(xf_dims(d, f)):
            lay["A"].append(normal_bf16(case_id, T_A, (K, din, r), std=1.0 / np.sqrt(din), sub=sub + i))
            lay["B"].append(normal_bf16(case_id, T_B, (K, r, dout), std=0.25 / np.sqrt(r), sub=sub + i))
        layers.append(lay)
    return layers


def xf_batch(case_id: int, n_seq: int, seq_len: int, d: int, K: int, mean_run: float = 64.0, probs=None):
    """Interleaved mixed-modality batch (Tables 7 and 8): per-token modality labels in runs of
    mean length `mean_run` (uniform over the K modalities unless `probs`), the token ids of
    those labels under vocabulary ranges of 8192 ids each, and N(0, 1) input activations
    [N][d] (the embedding lookup is not part of the measured path)."""
    N = n_seq * seq_len
    p = probs if probs is not None else [1.0 / K] * K
    labels = modality_runs(case_id, N, p, mean_run)
    bounds = vocab_bounds(K)
    ids = ids_for_labels(case_id, labels, bounds)
    x = normal_bf16(case_id, T_X, (N, d), sub=7)
    return x, ids, bounds, labels
