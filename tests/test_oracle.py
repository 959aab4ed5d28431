"""Pins for the fp64 oracle, against facts fixed by the mathematics (CPU only).

Every check here comes from somewhere other than the oracle itself: closed forms, an
independent pure-Python brute force, central finite differences, torch's own fp64 autograd
and SDPA, invariants of softmax attention, and metamorphic relations. The last test plants
plausible mistakes in copies of the oracle and checks that these pins catch each one.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa


def rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# ----------------------------------------------------------------------------- pin functions
# Each takes (fwd, bwd) with the signatures of oracle.head_forward / head_backward and raises
# AssertionError when the pin does not hold.

def pin_rows_sum_to_one(fwd, bwd):
    for causal in (False, True):
        q, k, v = rand((9, 4), 1), rand((9, 4), 2), rand((9, 4), 3)
        _, _, p = fwd(q, k, v, causal, 0.5)
        assert np.all(p >= 0.0)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def pin_causal_zeros(fwd, bwd):
    q, k, v = rand((7, 3), 4), rand((7, 3), 5), rand((7, 3), 6)
    _, _, p = fwd(q, k, v, True, 0.7)
    iu = np.triu_indices(7, k=1)
    assert np.all(p[iu] == 0.0)
    assert np.all(p[np.tril_indices(7)] > 0.0)


def _brute_lse(q, k, scale, causal):
    """Pure-Python logsumexp of the visible scores, fsum-accumulated."""
    out = []
    for i in range(q.shape[0]):
        ss = [scale * math.fsum(float(q[i, t]) * float(k[j, t]) for t in range(q.shape[1]))
              for j in range(k.shape[0]) if (not causal or j <= i)]
        m = max(ss)
        out.append(m + math.log(math.fsum(math.exp(s - m) for s in ss)))
    return np.array(out)


def pin_lse_bruteforce(fwd, bwd):
    for causal in (False, True):
        q, k, v = rand((6, 5), 7), rand((6, 5), 8), rand((6, 5), 9)
        _, lse, _ = fwd(q, k, v, causal, 0.45)
        np.testing.assert_allclose(lse, _brute_lse(q, k, 0.45, causal), rtol=0, atol=1e-13)


def pin_lse_bounds(fwd, bwd):
    q, k, v = rand((12, 4), 10), rand((12, 4), 11), rand((12, 4), 12)
    _, lse, _ = fwd(q, k, v, True, 1.0)
    s = q @ k.T
    for i in range(12):
        mx = s[i, : i + 1].max()
        assert mx - 1e-12 <= lse[i] <= mx + math.log(i + 1) + 1e-12


def pin_closed_forms(fwd, bwd):
    # One key: O = V and L = scale * q.k for every query.
    q, k, v = rand((5, 3), 13), rand((1, 3), 14), rand((1, 3), 15)
    o, lse, _ = fwd(q, k, v, False, 0.3)
    np.testing.assert_allclose(o, np.repeat(v, 5, axis=0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, 0.3 * (q @ k[0]), rtol=0, atol=1e-14)
    # Q = 0: uniform weights over the visible keys.
    n = 6
    z = np.zeros((n, 4))
    k, v = rand((n, 4), 16), rand((n, 4), 17)
    o, lse, _ = fwd(z, k, v, True, 0.5)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None],
                               rtol=0, atol=1e-14)
    o, lse, _ = fwd(z, k, v, False, 0.5)
    np.testing.assert_allclose(lse, np.full(n, math.log(n)), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), rtol=0, atol=1e-14)
    # Causal row 0 sees only key 0.
    q = rand((n, 4), 18)
    o, lse, _ = fwd(q, k, v, True, 0.5)
    np.testing.assert_array_equal(o[0], v[0])
    assert abs(lse[0] - 0.5 * float(q[0] @ k[0])) < 1e-14
    # Q = 0 backward: dV_j = sum_{i >= j} dO_i / (i + 1).
    g = rand((n, 4), 19)
    _, _, dv, _ = bwd(z, k, v, g, True, 0.5)
    want = np.stack([sum(g[i] / (i + 1) for i in range(j, n)) for j in range(n)])
    np.testing.assert_allclose(dv, want, rtol=0, atol=1e-14)


def pin_sdpa_forward(fwd, bwd):
    for causal in (False, True):
        q, k, v = rand((2, 3, 10, 8), 20), rand((2, 3, 10, 8), 21), rand((2, 3, 10, 8), 22)
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            is_causal=causal, scale=0.35).numpy()
        for b in range(2):
            for h in range(3):
                o, _, _ = fwd(q[b, h], k[b, h], v[b, h], causal, 0.35)
                np.testing.assert_allclose(o, want[b, h], rtol=0, atol=1e-13)


def pin_torch_autograd(fwd, bwd):
    for causal in (False, True):
        for nq, nk in ((9, 9), (6, 11), (11, 6)):
            q, k, v, g = rand((nq, 5), 23), rand((nk, 5), 24), rand((nk, 5), 25), rand((nq, 5), 26)
            tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
            s = (tq @ tk.T) * 0.4
            if causal:
                mask = torch.ones(nq, nk, dtype=torch.bool).tril()
                s = s.masked_fill(~mask, float("-inf"))
            out = torch.softmax(s, dim=-1) @ tv
            out.backward(torch.tensor(g))
            o, lse, _ = fwd(q, k, v, causal, 0.4)
            np.testing.assert_allclose(o, out.detach().numpy(), rtol=0, atol=1e-13)
            np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).detach().numpy(),
                                       rtol=0, atol=1e-13)
            dq, dk, dv, _ = bwd(q, k, v, g, causal, 0.4)
            np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def pin_finite_differences(fwd, bwd):
    """Central differences of f = sum(O o dO) against every element of Q, K and V."""
    h = 1e-6
    cases = [(1, 1, 1, True), (2, 2, 2, True), (3, 3, 4, False), (5, 5, 2, True),
             (8, 8, 4, True), (4, 6, 3, False), (16, 16, 1, True)]
    for n_q, n_k, d, causal in cases:
        seed = 100 * n_q + 10 * d + causal
        q, k, v = rand((n_q, d), seed), rand((n_k, d), seed + 1), rand((n_k, d), seed + 2)
        g = rand((n_q, d), seed + 3)
        sc = 1.0 / math.sqrt(d)
        grads = dict(zip("qkv", bwd(q, k, v, g, causal, sc)[:3]))
        for name in "qkv":
            x = {"q": q, "k": k, "v": v}[name]
            for idx in np.ndindex(x.shape):
                args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
                args[name][idx] += h
                fp = np.sum(fwd(args["q"], args["k"], args["v"], causal, sc)[0] * g)
                args[name][idx] -= 2 * h
                fm = np.sum(fwd(args["q"], args["k"], args["v"], causal, sc)[0] * g)
                num = (fp - fm) / (2 * h)
                assert abs(num - grads[name][idx]) <= 1e-6 * (1.0 + abs(num)), (name, idx)


def pin_invariants(fwd, bwd):
    for causal in (False, True):
        q, k, v, g = rand((10, 6), 30), rand((10, 6), 31), rand((10, 6), 32), rand((10, 6), 33)
        o, _, p = fwd(q, k, v, causal, 0.4)
        dq, dk, dv, dsum = bwd(q, k, v, g, causal, 0.4)
        # D = rowsum(dO o O) = rowsum(P o dP)
        np.testing.assert_allclose(dsum, np.sum(g * o, axis=1), rtol=0, atol=1e-12)
        # rows of dS sum to zero, so the keys' gradients sum to zero per feature
        np.testing.assert_allclose(dk.sum(axis=0), 0.0, rtol=0, atol=1e-12)
        if causal:
            assert np.all(dq[0] == 0.0)


def pin_metamorphic(fwd, bwd):
    q, k, v, g = rand((8, 4), 40), rand((8, 4), 41), rand((8, 4), 42), rand((8, 4), 43)
    c = rand((4,), 44)
    for causal in (False, True):
        o, lse, _ = fwd(q, k, v, causal, 0.5)
        base = bwd(q, k, v, g, causal, 0.5)[:3]
        # K_j -> K_j + c: P, O and all gradients unchanged; L_i shifts by scale q_i.c
        o2, lse2, _ = fwd(q, k + c, v, causal, 0.5)
        np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse2, lse + 0.5 * (q @ c), rtol=0, atol=1e-12)
        for a, b in zip(bwd(q, k + c, v, g, causal, 0.5)[:3], base):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
        # V_j -> V_j + c: O shifts by c, gradients unchanged
        o3, _, _ = fwd(q, k, v + c, causal, 0.5)
        np.testing.assert_allclose(o3, o + c, rtol=0, atol=1e-12)
        for a, b in zip(bwd(q, k, v + c, g, causal, 0.5)[:3], base):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # non-causal: permuting keys and values together permutes dK, dV; O and dQ unchanged
    perm = np.array([3, 0, 7, 1, 6, 2, 5, 4])
    o, _, _ = fwd(q, k, v, False, 0.5)
    dq, dk, dv, _ = bwd(q, k, v, g, False, 0.5)
    o4, _, _ = fwd(q, k[perm], v[perm], False, 0.5)
    dq4, dk4, dv4, _ = bwd(q, k[perm], v[perm], g, False, 0.5)
    np.testing.assert_allclose(o4, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq4, dq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk4, dk[perm], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv4, dv[perm], rtol=0, atol=1e-12)


PINS = [pin_rows_sum_to_one, pin_causal_zeros, pin_lse_bruteforce, pin_lse_bounds,
        pin_closed_forms, pin_sdpa_forward, pin_torch_autograd, pin_finite_differences,
        pin_invariants, pin_metamorphic]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.head_forward, oracle.head_backward)


# ------------------------------------------------------------------ batched and sampled forms

def test_batched_matches_heads():
    q, k, v, g = (rand((2, 3, 12, 4), s) for s in (50, 51, 52, 53))
    o, lse = oracle.forward(q, k, v, True, 0.5)
    dq, dk, dv, dsum = oracle.backward(q, k, v, g, True, 0.5)
    for b in range(2):
        for h in range(3):
            o1, l1, _ = oracle.head_forward(q[b, h], k[b, h], v[b, h], True, 0.5)
            np.testing.assert_array_equal(o[b, h], o1)
            np.testing.assert_array_equal(lse[b, h], l1)
            r = oracle.head_backward(q[b, h], k[b, h], v[b, h], g[b, h], True, 0.5)
            for a, c in zip((dq[b, h], dk[b, h], dv[b, h], dsum[b, h]), r):
                np.testing.assert_array_equal(a, c)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", [(40, 40), (37, 53), (53, 37), (1, 9), (9, 1)])
@pytest.mark.parametrize("row_block", [1, 7, 16, 64])
def test_blocked_matches_full(causal, nq, nk, row_block):
    """The row-block form gives the whole-matrix form's outputs, for blocks that divide Nq,
    leave a ragged last block, or exceed Nq."""
    q, k, v, g = rand((nq, 8), 60), rand((nk, 8), 61), rand((nk, 8), 62), rand((nq, 8), 63)
    o, lse, _ = oracle.head_forward(q, k, v, causal, 0.3)
    dq, dk, dv, dsum = oracle.head_backward(q, k, v, g, causal, 0.3)
    got = oracle.head_blocked(q, k, v, g, causal, 0.3, row_block=row_block)
    for name, a, b in zip(("O", "L", "dQ", "dK", "dV", "D"), got, (o, lse, dq, dk, dv, dsum)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12, err_msg=name)
    o2, l2, *rest = oracle.head_blocked(q, k, v, None, causal, 0.3, row_block=row_block,
                                        grads=False)
    np.testing.assert_array_equal(o2, got[0])
    np.testing.assert_array_equal(l2, got[1])
    assert rest == [None] * 4


def _blocked_pair(row_block, blocked=None):
    """(fwd, bwd) with the signatures of head_forward / head_backward, computed by the
    row-block form; fwd has no P to return."""
    blocked = blocked or oracle.head_blocked

    def fwd(q, k, v, causal, scale):
        o, lse, *_ = blocked(q, k, v, None, causal, scale, row_block=row_block, grads=False)
        return o, lse, None

    def bwd(q, k, v, do, causal, scale):
        _, _, dq, dk, dv, dsum = blocked(q, k, v, do, causal, scale, row_block=row_block)
        return dq, dk, dv, dsum

    return fwd, bwd


# Every pin that reads only O, L and the gradients (the row-block form keeps no P).
BLOCKED_PINS = [p for p in PINS if p not in (pin_rows_sum_to_one, pin_causal_zeros)]


@pytest.mark.parametrize("row_block", [2, 3])
@pytest.mark.parametrize("pin", BLOCKED_PINS, ids=lambda f: f.__name__)
def test_blocked_oracle_pin(pin, row_block):
    pin(*_blocked_pair(row_block))


def _mut_blocked(kind):
    """head_blocked with one planted mistake in its blocking."""
    def blocked(q, k, v, do, causal, scale, row_block=1024, grads=True):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        nq, nk = q.shape[0], k.shape[0]
        o, lse = np.empty((nq, v.shape[1])), np.empty(nq)
        if grads:
            do = np.asarray(do, np.float64)
            dq, dk, dv, dsum = np.empty_like(q), np.zeros_like(k), np.zeros_like(v), np.empty(nq)
        for r0 in range(0, nq, row_block):
            r1 = min(nq, r0 + row_block)
            kn = min(nk, r1) if causal else nk
            if kind == "keys_short" and causal and kn > 1:
                kn -= 1
            s = (q[r0:r1] @ k[:kn].T) * scale
            rows = np.arange(r0, r1) + (1 if kind == "rows_shifted" else 0)
            vis = (np.arange(kn)[None, :] <= rows[:, None]) if causal else np.ones(s.shape, bool)
            p, lse[r0:r1] = oa._softmax_rows(s, vis)
            o[r0:r1] = p @ v[:kn]
            if grads:
                g = do[r0:r1]
                dp = g @ v[:kn].T
                dsum[r0:r1] = np.sum(p * dp, axis=-1)
                ds = p * (dp - dsum[r0:r1, None])
                dq[r0:r1] = scale * (ds @ k[:kn])
                if kind == "dk_overwritten":
                    dk[:kn] = scale * (ds.T @ q[r0:r1])
                else:
                    dk[:kn] += scale * (ds.T @ q[r0:r1])
                if kind == "dv_first_block_only":
                    if r0 == 0:
                        dv[:kn] += p.T @ g
                else:
                    dv[:kn] += p.T @ g
        if not grads:
            return o, lse, None, None, None, None
        return o, lse, dq, dk, dv, dsum
    return blocked


@pytest.mark.parametrize("kind", ["keys_short", "rows_shifted", "dk_overwritten",
                                  "dv_first_block_only"])
def test_blocked_pins_catch_planted_mistake(kind):
    fwd, bwd = _blocked_pair(3, _mut_blocked(kind))
    caught = []
    for pin in BLOCKED_PINS:
        try:
            pin(fwd, bwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted blocking mistake {kind}"


def test_blocked_mutant_harness_without_mistake_passes():
    """The copy the mistakes are planted in passes every pin when no mistake is planted."""
    fwd, bwd = _blocked_pair(3, _mut_blocked("none"))
    for pin in BLOCKED_PINS:
        pin(fwd, bwd)


def test_minus_1e6_mask_reading():
    """Adding -1e6 to masked scores (the pages' rule) gives exactly the oracle's P."""
    q, k, v = rand((9, 4), 70), rand((9, 4), 71), rand((9, 4), 72)
    s = (q @ k.T) * 0.5
    s = s + np.where(oracle.visible(9, 9, True), 0.0, -1e6)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p_add = e / e.sum(axis=1, keepdims=True)
    _, _, p = oracle.head_forward(q, k, v, True, 0.5)
    np.testing.assert_array_equal(p_add == 0.0, p == 0.0)
    np.testing.assert_allclose(p_add, p, rtol=1e-15, atol=0)


def test_golden_fixture():
    """Regression fixture written by tests/golden/make_golden.py from the oracle."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_causal.json")
    with open(path) as f:
        fx = json.load(f)
    inp = {n: np.array(fx["inputs"][n]) for n in ("q", "k", "v", "do")}
    o, lse, _ = oracle.head_forward(inp["q"], inp["k"], inp["v"], fx["causal"], fx["scale"])
    dq, dk, dv, _ = oracle.head_backward(inp["q"], inp["k"], inp["v"], inp["do"],
                                         fx["causal"], fx["scale"])
    for name, got in (("O", o), ("L", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        np.testing.assert_allclose(got, np.array(fx["outputs"][name]), rtol=0, atol=1e-14)


# ---------------------------------------------------------------------- planted mistakes

def _mut_forward(kind):
    def fwd(q, k, v, causal, scale):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        s = q @ k.T * (1.0 if kind == "no_scale" else scale)
        nq, nk = s.shape
        vis = oa.visible(nq, nk, causal)
        if kind == "strict_mask" and causal:
            vis = np.arange(nk)[None, :] < np.arange(nq)[:, None]
            vis[0, 0] = True
        if kind == "mask_ignored":
            vis = np.ones_like(vis)
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        lse = (np.log(z) if kind == "lse_drops_max" else m + np.log(z))[:, 0]
        p = e / z
        o = (p @ v[::-1]) if kind == "v_reversed" else p @ v
        return o, lse, p
    return fwd


def _mut_backward(kind):
    def bwd(q, k, v, do, causal, scale):
        q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
        _, _, p = oracle.head_forward(q, k, v, causal, scale)
        dv = p @ do if kind == "dv_untransposed" else p.T @ do
        dp = do @ v.T
        dsum = np.sum(p * dp, axis=1)
        if kind == "d_dropped":
            dsum = np.zeros_like(dsum)
        if kind == "d_wrong_axis":
            dsum = np.sum(p * dp, axis=0)
        ds = p * (dp - dsum[:, None])
        if kind == "ds_sign":
            ds = -ds
        dq = (ds @ k) * (1.0 if kind == "dq_no_scale" else scale)
        dk = (ds.T @ q) * (scale * scale if kind == "dk_scale_twice" else scale)
        if kind == "dk_wrong_operand":
            dk = scale * (ds.T @ do)
        return dq, dk, dv, dsum
    return bwd


MUTANTS = ([("fwd", k) for k in ("no_scale", "strict_mask", "mask_ignored", "lse_drops_max",
                                 "v_reversed")]
           + [("bwd", k) for k in ("dv_untransposed", "d_dropped", "d_wrong_axis", "ds_sign",
                                   "dq_no_scale", "dk_scale_twice", "dk_wrong_operand")])


@pytest.mark.parametrize("side,kind", MUTANTS)
def test_pins_catch_planted_mistake(side, kind):
    fwd = _mut_forward(kind) if side == "fwd" else oracle.head_forward
    bwd = _mut_backward(kind) if side == "bwd" else oracle.head_backward
    caught = []
    for pin in PINS:
        try:
            pin(fwd, bwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {side}:{kind}"
