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

Sampled evaluation (``head_sampled``) computes O, L, dQ for chosen query rows and dK, dV for
chosen key rows of one head, with every sum complete; it needs L and D for every query row,
which it takes from the full forward evaluated one block of whole rows at a time, and it
uses D_i = sum_k dO_ik O_ik (equal to sum_j P_ij dP_ij; the pins check this identity).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "visible",
    "head_forward",
    "head_backward",
    "forward",
    "backward",
    "head_sampled",
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


def head_sampled(q, k, v, do, is_causal: bool, scale: float, q_rows, k_rows,
                 row_block: int = 1024):
    """One head, selected outputs only, every sum complete.

    Returns a dict with O and L and dQ at ``q_rows`` and dK and dV at ``k_rows``.
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    nq, nk = q.shape[0], k.shape[0]
    sc = np.float64(scale)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)

    # L and O for every query row, a block of whole rows at a time.
    lse = np.empty(nq)
    o = np.empty((nq, v.shape[1]))
    for r0 in range(0, nq, row_block):
        r1 = min(nq, r0 + row_block)
        s = (q[r0:r1] @ k.T) * sc
        if is_causal:
            vis = np.arange(nk)[None, :] <= np.arange(r0, r1)[:, None]
        else:
            vis = np.ones((r1 - r0, nk), dtype=bool)
        p, lse[r0:r1] = _softmax_rows(s, vis)
        o[r0:r1] = p @ v
    dsum = np.sum(do * o, axis=-1)

    # Query rows: dQ_i = scale * sum_j P_ij (dP_ij - D_i) K_j.
    s = (q[q_rows] @ k.T) * sc
    vis_q = np.arange(nk)[None, :] <= q_rows[:, None] if is_causal else np.ones(s.shape, bool)
    p = np.where(vis_q, np.exp(np.where(vis_q, s, 0.0) - lse[q_rows][:, None]), 0.0)
    dp = do[q_rows] @ v.T
    ds = p * (dp - dsum[q_rows][:, None])
    dq = sc * (ds @ k)

    # Key rows: dV_j = sum_i P_ij dO_i, dK_j = scale * sum_i dS_ij Q_i.
    s = (q @ k[k_rows].T) * sc  # [nq, len(k_rows)]
    vis_k = k_rows[None, :] <= np.arange(nq)[:, None] if is_causal else np.ones(s.shape, bool)
    p = np.where(vis_k, np.exp(np.where(vis_k, s, 0.0) - lse[:, None]), 0.0)
    dv = p.T @ do
    dp = do @ v[k_rows].T
    ds = p * (dp - dsum[:, None])
    dk = sc * (ds.T @ q)
    return {"O": o[q_rows], "L": lse[q_rows], "dQ": dq, "dK": dk, "dV": dv,
            "D": dsum[q_rows]}
