"""Plain fp64 CPU oracle of a synthetic decoder with per-token LoRA.  TEST INFRASTRUCTURE ONLY.

Source: the MoLoRA pages (thelatestinai.com), Table 7 (an end-to-end transformer with per-token
routing, d = 1024/2048/4096, L = 2/4 layers, against a per-sequence simulation that runs one
forward pass per adapter) and Table 8 (a Chameleon-style interleaved batch, d = 2048, L = 4,
K = 2 modalities).  The pages name only d, L, K and the batch; everything else here is a
reading, each listed in the design notes:

* a pre-norm decoder layer:  x += o(attn(norm1(x)));  x += down(silu(gate(h)) * up(h)) with
  h = norm2(x); RMSNorm with a learned weight, eps 1e-6; no biases;
* causal softmax attention inside each sequence, heads of width 128, scores scaled by
  1/sqrt(128), no positional encoding;
* the MLP width f = 8d/3 rounded up to a multiple of 128 (given by the weights' shapes);
* per-token LoRA on all seven projections (q, k, v, o, gate, up, down), every projection's
  delta from the same routing: the grouped apply of ``molora_oracle.apply``.

``store`` is applied wherever the GPU keeps an intermediate in memory: identity gives the
exact fp64 definition; a bf16 rounding gives the same arithmetic with the storage precision
of the GPU's tensors (the reading used for parity; see ``bf16_store``).
"""
from __future__ import annotations

import numpy as np

from .molora_oracle import apply, dispatch

TARGETS = ("q", "k", "v", "o", "gate", "up", "down")
HEAD_DIM = 128


def identity(a):
    return a


def bf16_store(a):
    """Round fp64 values to bf16 (round to nearest, ties to even), returned as fp64."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def rms_norm(x, w, eps: float = 1e-6):
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def causal_attention(q, k, v, n_seq: int, seq_len: int, store=identity):
    """Softmax attention of every token over the earlier tokens of its own sequence (itself
    included), per head of width 128; scores scaled by 1/sqrt(128).  q, k, v [N][d]."""
    N, d = q.shape
    H = d // HEAD_DIM
    out = np.zeros_like(q)
    mask = np.tril(np.ones((seq_len, seq_len), dtype=bool))
    for b in range(n_seq):
        rows = slice(b * seq_len, (b + 1) * seq_len)
        for h in range(H):
            cols = slice(h * HEAD_DIM, (h + 1) * HEAD_DIM)
            s = (q[rows, cols] @ k[rows, cols].T) / np.sqrt(HEAD_DIM)
            s = np.where(mask, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p = store(p / p.sum(axis=1, keepdims=True))
            out[rows, cols] = p @ v[rows, cols]
    return store(out)


def silu(a):
    return a / (1.0 + np.exp(-a))


def lora_linear(x, W, A, B, scale, route, k, store=identity):
    """store(store(x W^T) + routed LoRA delta): the base projection (nn.Linear layout [out][in])
    stored, then the per-token delta of the grouped apply added and stored."""
    counts, offsets, perm, perm_w, inv = route
    base = store(x @ W.T)
    return store(apply(base, x, A, B, scale, perm, perm_w, offsets, k))


def layer_forward(x, L, scale, route, k, n_seq, seq_len, eps=1e-6, store=identity):
    """One decoder layer.  L: dict with norm1, norm2 [d]; Wq, Wk, Wv, Wo [d][d]; Wgate, Wup
    [f][d]; Wdown [d][f]; A, B: per target (TARGETS order) [K][d_in][r] and [K][r][d_out]."""
    h = store(rms_norm(x, L["norm1"], eps))
    q = lora_linear(h, L["Wq"], L["A"][0], L["B"][0], scale, route, k, store)
    kk = lora_linear(h, L["Wk"], L["A"][1], L["B"][1], scale, route, k, store)
    v = lora_linear(h, L["Wv"], L["A"][2], L["B"][2], scale, route, k, store)
    att = causal_attention(q, kk, v, n_seq, seq_len, store)
    o = lora_linear(att, L["Wo"], L["A"][3], L["B"][3], scale, route, k, store)
    x = store(x + o)
    h2 = store(rms_norm(x, L["norm2"], eps))
    g = lora_linear(h2, L["Wgate"], L["A"][4], L["B"][4], scale, route, k, store)
    u = lora_linear(h2, L["Wup"], L["A"][5], L["B"][5], scale, route, k, store)
    a = store(silu(g) * u)
    dn = lora_linear(a, L["Wdown"], L["A"][6], L["B"][6], scale, route, k, store)
    return store(x + dn)


def forward(x, layers, scale, idx, w, K, n_seq, seq_len, eps=1e-6, store=identity):
    """The whole decoder: every layer with the same per-token routing (idx, w: [N] or [N][k];
    -1 = unrouted), which is dispatched once."""
    idx = np.asarray(idx)
    k = 1 if idx.ndim == 1 else idx.shape[1]
    route = dispatch(idx, w, K)
    for L in layers:
        x = layer_forward(x, L, scale, route, k, n_seq, seq_len, eps, store)
    return x
