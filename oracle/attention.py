"""Plain, slow fp64 CPU oracle for scaled dot-product attention and its gradients.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import or call this module. The HIP library never uses it, and it uses
nothing from the HIP library: the two share no code.

What it computes (untiled, everything materialised, float64 throughout):

  forward, for each (b, h):    S = (Q K^T) * scale
                               causal: key j is visible to query i iff j <= i (top-left)
                               P = softmax over the visible keys of each row of S
                               L_i = logsumexp of the visible S_ij      (natural log)
                               O = P V
  backward (analytic gradient of O = softmax(S) V with upstream gradient dO):
                               dV = P^T dO
                               dP = dO V^T
                               D_i = sum_j P_ij dP_ij
                               dS = P o (dP - D)
                               dQ = scale * dS K
                               dK = scale * dS^T Q

Sources, "Systems and Parallelism" (CS336 field map, A2), section 1.2-1.3:
  * problem flash_forward: L = m + log(l) is the row logsumexp, and O and L are compared
    with a reference attention plus torch.logsumexp; causal masking compares query
    positions against key positions.
  * problem flash_backward: P = exp(S - L), D = rowsum(dO o O), dS = P o (dP - D); the
    1/sqrt(d) scale appears in dQ and dK.
The tiling, online softmax and recomputation that the pages describe are how the GPU reaches
this same result faster; none of them appears here.

Readings of points the pages leave open (each is also listed in the design notes):
  * Masked keys are excluded from the softmax (set to -inf before the row max). The pages add
    -1e6 instead; with at least one visible key per row (always true for top-left causal and
    Nk >= 1) exp(-1e6 + O(10)) is exactly 0 in float64, so both give the same P.
  * Causal alignment with Nq != Nk is top-left: visible iff j <= i, indices from 0.
  * scale is an argument; the callers pass float32(1/sqrt(d)), upcast exactly.

Row-block evaluation (``head_blocked``) computes every output of one head with the query
rows taken a block of whole rows at a time, so that only one block's scores exist at once
(for the long-context workload, whose full N x N score matrix would not fit comfortably).
Each row's softmax is still over all of its visible keys, so this is the same definition,
not an online softmax; dK and dV add up the blocks' contributions, and D is the same
sum_j P_ij dP_ij as in head_backward.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "visible",
    "head_forward",
    "head_backward",
    "forward",
    "backward",
    "head_blocked",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible(nq: int, nk: int, is_causal: bool) -> np.ndarray:
    """Boolean [nq, nk]: True where key j is visible to query i (top-left causal: j <= i)."""
    if not is_causal:
        return np.ones((nq, nk), dtype=bool)
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    return j <= i


def _softmax_rows(s: np.ndarray, vis: np.ndarray):
    """Row softmax over the visible entries; returns (P, L) with L the natural logsumexp."""
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)  # masked entries give exp(-inf) = 0
    z = np.sum(e, axis=-1, keepdims=True)
    p = e / z
    lse = (m + np.log(z))[..., 0]
    return p, lse


def head_forward(q, k, v, is_causal: bool, scale: float):
    """One head: q [Nq,d], k and v [Nk,d] -> (O [Nq,d], L [Nq], P [Nq,Nk])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = (q @ k.T) * np.float64(scale)
    p, lse = _softmax_rows(s, visible(q.shape[0], k.shape[0], is_causal))
    o = p @ v
    return o, lse, p


def head_backward(q, k, v, do, is_causal: bool, scale: float):
    """One head: analytic gradients (dQ, dK, dV, D) of O = softmax(Q K^T scale) V."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    _, _, p = head_forward(q, k, v, is_causal, scale)
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.sum(p * dp, axis=-1)
    ds = p * (dp - dsum[:, None])
    dq = np.float64(scale) * (ds @ k)
    dk = np.float64(scale) * (ds.T @ q)
    return dq, dk, dv, dsum


def forward(q, k, v, is_causal: bool, scale: float):
    """[B,H,Nq,d], [B,H,Nk,d] x2 -> (O [B,H,Nq,d], L [B,H,Nq]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    o = np.empty((B, H, Nq, v.shape[-1]))
    lse = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h], _ = head_forward(q[b, h], k[b, h], v[b, h], is_causal, scale)
    return o, lse


def backward(q, k, v, do, is_causal: bool, scale: float):
    """[B,H,N,d] tensors -> (dQ, dK, dV, D) in float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H = q.shape[:2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dsum = np.empty(q.shape[:3])
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h], dsum[b, h] = head_backward(
                q[b, h], k[b, h], v[b, h], do[b, h], is_causal, scale)
    return dq, dk, dv, dsum


def head_blocked(q, k, v, do, is_causal: bool, scale: float, row_block: int = 1024,
                 grads: bool = True):
    """One head, every output, a block of whole query rows at a time.

    q and do are [Nq, d], k and v [Nk, d]. Returns (O, L, dQ, dK, dV, D); with
    grads=False only O and L are formed and the rest are None.

    Same definitions as head_forward and head_backward. Under causal masking the rows
    [r0, r1) of a block see no key at or past r1, so their scores are formed against keys
    [0, min(Nk, r1)) only: every other key's P is exactly 0 and adds nothing to any sum.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    nq, nk = q.shape[0], k.shape[0]
    sc = np.float64(scale)
    o = np.empty((nq, v.shape[1]))
    lse = np.empty(nq)
    if grads:
        do = _f64(do)
        dq = np.empty_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        dsum = np.empty(nq)
    for r0 in range(0, nq, row_block):
        r1 = min(nq, r0 + row_block)
        kn = min(nk, r1) if is_causal else nk  # the keys any row of the block can see
        s = (q[r0:r1] @ k[:kn].T) * sc
        if is_causal:
            vis = np.arange(kn)[None, :] <= np.arange(r0, r1)[:, None]
        else:
            vis = np.ones((r1 - r0, kn), dtype=bool)
        p, lse[r0:r1] = _softmax_rows(s, vis)
        del s, vis
        o[r0:r1] = p @ v[:kn]
        if grads:
            g = do[r0:r1]
            dp = g @ v[:kn].T
            dsum[r0:r1] = np.sum(p * dp, axis=-1)
            ds = p * (dp - dsum[r0:r1, None])
            del dp
            dq[r0:r1] = sc * (ds @ k[:kn])
            dk[:kn] += sc * (ds.T @ q[r0:r1])
            dv[:kn] += p.T @ g
    if not grads:
        return o, lse, None, None, None, None
    return o, lse, dq, dk, dv, dsum
