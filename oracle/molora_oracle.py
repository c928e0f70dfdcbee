"""Plain fp64 CPU oracle for per-token adapter routing.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
module.  It shares no code with the GPU library: inputs arrive as the same
bf16 bit patterns / fp32 / int32 arrays the GPU receives, are widened exactly
to fp64 here, and every step below is computed in fp64 with no intermediate
rounding.

Sources (all on the MoLoRA pages, "MoLoRA: Composable Specialization via
Per-Token Adapter Routing"):

* thelatestinai.com, Table 1: the routing decision is either the vocabulary
  range function R_vocab(v) or TopK(g_theta(x)); after it, both routers share
  the same histogram, pointer arrays and grouped GEMM dispatch.
* thelatestinai.com, Figure 2: a router picks top-k adapters per token and
  their outputs are combined by a weighted sum; physically the tokens are
  grouped by selected adapter and processed by a grouped GEMM.
* thelatestinai.com, Table 10: adapter weights A have shape (K, d, r) and B
  shape (K, r, d); the multi-adapter "capacity" is a memory budget (so no
  token is ever dropped).
* thelatestinai.com, Table 1 (routing cost O(64d + 64K)): the learned router
  is read as an MLP d -> 64 -> K.
* the abstract (all pages): per-token routing does work N for N tokens,
  per-sequence routing does K * N for K adapter types (one masked pass per
  adapter), giving the second formulation ``apply_masked_passes``.
* thelatestinai.com, Figure 2 read backwards and Table 13 (the router is
  trained without labels, so gradients reach the adapters, the gate weights
  and the router): ``apply_backward``, ``route_topk_backward`` and
  ``router_backward`` are the exact derivatives of ``apply``, of the
  renormalised softmax of ``route_topk`` (selection held fixed) and of
  ``router_logits``.

Readings where the pages are silent (each is also listed in the design notes):
half-open vocabulary ranges and unrouted ids outside them; ReLU in the router;
softmax renormalised over the selected adapters; top-k ties broken toward the
lower adapter index; slots of a token stored in ascending adapter order; each
adapter segment ordered by ascending pair id; LoRA scale alpha/r applied to
every delta.

Every function here is pinned by tests that do not re-type it (brute force,
closed forms, invariants, a hand-worked example, library routines the oracle
does not use).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to fp64: a bf16 value is the
    upper half of the fp32 with the same sign/exponent/leading mantissa bits."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        b = b.view(np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def route_vocab(ids: np.ndarray, bounds: np.ndarray):
    """Vocabulary routing R_vocab(v) (thelatestinai.com, Table 1).

    Adapter ``e`` owns the half-open id range ``[bounds[e], bounds[e+1])``.
    An id outside ``[bounds[0], bounds[K])`` belongs to no adapter: its index
    is -1 (unrouted) and its weight 0.  A routed token has exactly one
    adapter and gate weight 1.
    Returns ``idx`` int32 [N] and ``w`` fp64 [N].
    """
    v = np.asarray(ids, dtype=np.int64)
    b = np.asarray(bounds, dtype=np.int64)
    K = b.shape[0] - 1
    idx = np.full(v.shape, -1, dtype=np.int32)
    for e in range(K):
        owned = (v >= b[e]) & (v < b[e + 1])
        idx[owned] = e
    w = np.where(idx >= 0, 1.0, 0.0)
    return idx, w


def router_logits(x, W1, b1, W2, b2):
    """Learned gate g_theta(x) read as the MLP d -> H -> K of Table 1's routing
    cost O(64d + 64K) (thelatestinai.com): logits = ReLU(x W1 + b1) W2 + b2,
    in fp64.  ``x`` [N][d], ``W1`` [d][H], ``W2`` [H][K]; biases may be None.
    Inputs are fp64 arrays (already widened from bf16/fp32)."""
    a = x @ W1
    if b1 is not None:
        a = a + b1
    hdn = np.maximum(a, 0.0)
    logits = hdn @ W2
    if b2 is not None:
        logits = logits + b2
    return logits


def route_topk(logits: np.ndarray, k: int, margin: float = 1e-4):
    """TopK over the gate's logits, then a softmax over the selected ones
    (thelatestinai.com, Table 1 and Figure 2: top-k adapters combined by a
    weighted sum).

    Selection: k rounds, each taking the largest logit not yet taken; among
    equal logits the lower adapter index is taken first.  A token's slots are
    then listed in ascending adapter index.  Weights: softmax over the k
    selected logits (the same numbers as a softmax over all K renormalised to
    the selected set).  Flag: set when k < K and the k-th largest logit
    exceeds the (k+1)-th by less than ``margin``.
    Returns ``idx`` int32 [N][k], ``w`` fp64 [N][k], ``flags`` bool [N].
    """
    lg = np.asarray(logits, dtype=np.float64)
    N, K = lg.shape
    if not (1 <= k <= K):
        raise ValueError("need 1 <= k <= K")
    rows = np.arange(N)
    taken = np.zeros((N, K), dtype=bool)
    chosen = np.empty((N, k), dtype=np.int64)
    for s in range(k):
        remaining = np.where(taken, -np.inf, lg)
        j = np.argmax(remaining, axis=1)  # first maximum = lowest index among ties
        chosen[:, s] = j
        taken[rows, j] = True
    idx = np.sort(chosen, axis=1)
    sel = np.take_along_axis(lg, idx, axis=1)
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    w = ex / ex.sum(axis=1, keepdims=True)
    if k < K:
        desc = -np.sort(-lg, axis=1)
        flags = (desc[:, k - 1] - desc[:, k]) < margin
    else:
        flags = np.zeros(N, dtype=bool)
    return idx.astype(np.int32), w, flags


def pairs_of(idx: np.ndarray, w: np.ndarray):
    """Flatten per-token slots into pairs p = t*k + s (adapter e_p, weight w_p)."""
    e = np.asarray(idx).reshape(-1).astype(np.int64)
    wp = np.asarray(w, dtype=np.float64).reshape(-1)
    return e, wp


def dispatch(idx: np.ndarray, w: np.ndarray, K: int):
    """Histogram, offsets ("pointer arrays") and the grouping permutation
    (thelatestinai.com, Table 1 rows "Histogram computation" and "Pointer
    arrays"; Figure 2 right: tokens grouped by their selected adapter).

    ``idx``/``w`` are [N] or [N][k]; pair p = t*k + s.  Pairs whose adapter is
    outside [0, K) are unrouted and appear nowhere.
      counts[e]   = number of pairs with adapter e
      offsets     = [0, counts[0], counts[0]+counts[1], ...]  (K+1 entries)
      perm[q]     = pair id at grouped position q; within adapter e's segment
                    the pair ids ascend
      perm_w[q]   = gate weight of pair perm[q]
      inv[p]      = grouped position of pair p, -1 if unrouted
    """
    e_p, w_p = pairs_of(idx, w)
    P = e_p.shape[0]
    counts = np.zeros(K, dtype=np.int64)
    for e in range(K):
        counts[e] = np.count_nonzero(e_p == e)
    offsets = np.zeros(K + 1, dtype=np.int64)
    for e in range(K):
        offsets[e + 1] = offsets[e] + counts[e]
    perm = np.empty(offsets[K], dtype=np.int64)
    for e in range(K):
        perm[offsets[e]:offsets[e + 1]] = np.nonzero(e_p == e)[0]
    perm_w = w_p[perm]
    inv = np.full(P, -1, dtype=np.int64)
    inv[perm] = np.arange(offsets[K])
    return (counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32),
            perm_w, inv.astype(np.int32))


def apply(y0, x, A, B, scale: float, perm, perm_w, offsets, k: int):
    """Grouped LoRA application (thelatestinai.com, Figure 2 right; Table 10
    shapes A (K, d_in, r), B (K, r, d_out)).

    For every adapter e, the pairs of its segment are gathered (token
    t = pair // k), shrunk ``h = x_t A_e`` (d_in -> r), expanded
    ``delta = h B_e`` (r -> d_out), and ``perm_w * scale * delta`` is added to
    ``y[t]`` (the weighted sum of Figure 2, with the LoRA scale alpha/r).
    All arrays fp64; returns a new ``y`` [N][d_out].
    """
    y = np.array(y0, dtype=np.float64, copy=True)
    K = len(offsets) - 1
    for e in range(K):
        q0, q1 = int(offsets[e]), int(offsets[e + 1])
        if q1 == q0:
            continue
        t = np.asarray(perm[q0:q1], dtype=np.int64) // k
        h = x[t] @ A[e]
        delta = h @ B[e]
        contrib = (np.asarray(perm_w[q0:q1], dtype=np.float64) * scale)[:, None] * delta
        if np.unique(t).shape[0] == t.shape[0]:
            y[t] += contrib
        else:  # a token listed twice under one adapter: accumulate both
            np.add.at(y, t, contrib)
    return y


def apply_masked_passes(y0, x, A, B, scale: float, idx, w):
    """The same result as K masked dense passes, one per adapter (the
    per-sequence comparator of the abstract's work K*N versus N, and of
    thelatestinai.com Table 3): pass e computes ``(x A_e) B_e`` for every
    token and adds it with the token's gate mass on e (0 for tokens not routed
    to e).  Work: K*N token-adapter applications."""
    y = np.array(y0, dtype=np.float64, copy=True)
    K = A.shape[0]
    N = y.shape[0]
    idx2 = np.asarray(idx).reshape(N, -1)
    w2 = np.asarray(w, dtype=np.float64).reshape(N, -1)
    for e in range(K):
        mass = np.where(idx2 == e, w2, 0.0).sum(axis=1)
        y += (mass * scale)[:, None] * ((x @ A[e]) @ B[e])
    return y


# --------------------------------------------------------------------------- backward

def apply_backward(x, gy, A, B, scale: float, perm, perm_w, offsets, k: int):
    """Derivatives of ``apply`` given dL/dy = ``gy`` (thelatestinai.com, Figure 2
    with the grouping reused backwards; Table 13: adapters and router learn
    from the loss).

    For a routed pair p = (token t, adapter e, gate weight w_p) with
    c_p = w_p * scale, the forward adds c_p * (x_t A_e) B_e to y_t.  With
    h_p = x_t A_e and g_p = gy_t B_e^T (both [r]):
      dL/dA_e  = sum over e's pairs of  outer(x_t, c_p g_p)      [d_in][r]
      dL/dB_e  = sum over e's pairs of  outer(c_p h_p, gy_t)     [r][d_out]
      dL/dx_t  = sum over t's pairs of  c_p g_p A_e^T            [d_in]
                 (the adapters' part only; y0's own path is the caller's)
      dL/dw_p  = scale * (h_p . g_p)
    Unrouted pairs get dL/dw_p = 0.  All fp64.  Returns (dx [N][d_in],
    dA [K][d_in][r], dB [K][r][d_out], dw [N*k] in pair order)."""
    x = np.asarray(x, dtype=np.float64)
    gy = np.asarray(gy, dtype=np.float64)
    N = x.shape[0]
    K = len(offsets) - 1
    dx = np.zeros_like(x)
    dA = np.zeros(np.shape(A), dtype=np.float64)
    dB = np.zeros(np.shape(B), dtype=np.float64)
    dw = np.zeros(N * k, dtype=np.float64)
    for e in range(K):
        q0, q1 = int(offsets[e]), int(offsets[e + 1])
        if q1 == q0:
            continue
        pid = np.asarray(perm[q0:q1], dtype=np.int64)
        t = pid // k
        c = np.asarray(perm_w[q0:q1], dtype=np.float64) * scale
        h = x[t] @ A[e]
        g = gy[t] @ B[e].T
        dB[e] = (c[:, None] * h).T @ gy[t]
        dA[e] = x[t].T @ (c[:, None] * g)
        np.add.at(dx, t, (c[:, None] * g) @ A[e].T)
        dw[pid] = scale * np.sum(h * g, axis=1)
    return dx, dA, dB, dw


def route_topk_backward(w, idx, dw, K: int):
    """dL/dlogits through the softmax over the k selected logits of
    ``route_topk`` (thelatestinai.com, Table 1 TopK(g_theta(x)) and Figure 2's
    weighted sum), with the selection held fixed (it is piecewise constant in
    the logits).  For a token with selected weights w_j and incoming dL/dw_j,
    the selected logit of slot j receives w_j * (dL/dw_j - sum_i w_i dL/dw_i);
    unselected logits receive 0.  ``w``/``dw`` [N][k] fp64, ``idx`` [N][k].
    Returns [N][K] fp64."""
    w = np.asarray(w, dtype=np.float64)
    dw = np.asarray(dw, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    N = w.shape[0]
    mean = np.sum(w * dw, axis=1, keepdims=True)
    dl = np.zeros((N, K), dtype=np.float64)
    np.put_along_axis(dl, idx, w * (dw - mean), axis=1)
    return dl


def router_backward(x, W1, b1, W2, dlogits):
    """Derivatives of ``router_logits`` (logits = ReLU(x W1 + b1) W2 + b2, the
    MLP d -> H -> K read from Table 1's routing cost) given dL/dlogits.
    ``x`` [N][d], ``W1`` [d][H], ``W2`` [H][K], fp64; ``b1`` may be None.  The
    ReLU's derivative is taken as 1 where its input is > 0, else 0.
    Returns (dW1 [d][H], db1 [H], dW2 [H][K], db2 [K], dx [N][d])."""
    x = np.asarray(x, dtype=np.float64)
    dl = np.asarray(dlogits, dtype=np.float64)
    a = x @ W1
    if b1 is not None:
        a = a + b1
    hdn = np.maximum(a, 0.0)
    dW2 = hdn.T @ dl
    db2 = dl.sum(axis=0)
    da = (dl @ W2.T) * (a > 0.0)
    dW1 = x.T @ da
    db1 = da.sum(axis=0)
    dx = da @ W1.T
    return dW1, db1, dW2, db2, dx
