"""The GPU parity cases reach every attention kernel the library's dispatch can choose.

Host logic only: fa_forward_kernel_name and fa_backward_kernel_name answer from the same
dispatch code the launchers run (kernel choice depends on the shape, the dtype, the mask and
the workspace), and return before anything touches the GPU. A kernel that the dispatch can
choose but that no parity case launches would only ever be checked against the oracle by
chance; this test names it.
"""
import itertools
import os

import pytest

import test_parity as tp
from seeded_inputs import WORKLOADS

DT = {"f32": 0, "bf16": 1}


@pytest.fixture(scope="module")
def lib():
    from tiled_attention_causal_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfa.so is not built; run `python -m tiled_attention_causal_amd.build`")
    return _lib.load()


def names(lib, dt, B, H, Nq, Nk, d, causal, fws=None, bws=None):
    """(forward, backward) kernel names for these arguments; the workspaces default to what
    fa_forward and fa_backward use (the sizes the library asks for)."""
    if fws is None:
        fws = lib.fa_forward_workspace_bytes(DT[dt], B, H, Nq, Nk, d, int(causal))
    if bws is None:
        bws = lib.fa_backward_workspace_bytes(DT[dt], B, H, Nq, Nk, d)
    return (lib.fa_forward_kernel_name(DT[dt], B, H, Nq, Nk, d, int(causal), fws).decode(),
            lib.fa_backward_kernel_name(DT[dt], B, H, Nq, Nk, d, int(causal), bws).decode())


def parity_launches(lib):
    """Kernel names that the GPU tests comparing with the oracle launch, from their own case
    lists (the tests that compare two HIP runs with each other are left out)."""
    cases = [(dt, B, H, Nq, Nk, d, c) for (B, H, Nq, Nk, d, dt, c) in tp.SMALL]
    for n in tp.FULL + ["long_n16384_d128"]:
        w = WORKLOADS[n]
        cases.append((w.dtype, w.B, w.H, w.Nq, w.Nk, w.d, w.causal))
    square_causal = tp.PAIRED + tp.WIDE_T + tp.SPLIT_WG + tp.GROWING + tp.MID + tp.ONE_SHARE
    cases += [("bf16", B, H, N, N, d, True) for (B, H, N, d) in square_causal]
    cases += [("bf16", B, H, N, N, d, c) for (B, H, N, d, c) in tp.SPLIT_BWD]
    cases += [("f32", B, H, N, N, d, c) for (B, H, N, d, c) in tp.SPLIT_F32]
    cases += [("f32", B, H, Nq, Nk, d, True) for (B, H, Nq, Nk, d) in tp.F32_RAGGED_SPLIT]
    seen = set()
    for c in cases:
        seen.update(names(lib, *c))
    return seen


def reachable(lib):
    """Every kernel name the dispatch gives over a spread of square grids (one head to far
    more tiles than CUs), both dtypes, every head dim, both masks, and the three workspace
    choices (the library's size, the per-row terms only, none for the forward)."""
    out = set()
    grid = itertools.product(["f32", "bf16"], [16, 32, 64, 128], [False, True],
                             [1, 2, 4, 8, 16], [1, 3, 12, 25, 64],
                             [64, 128, 256, 512, 1024, 2048, 4096, 8192])
    for dt, d, causal, B, H, N in grid:
        out.update(names(lib, dt, B, H, N, N, d, causal))
        out.update(names(lib, dt, B, H, N, N, d, causal, 0, B * H * N * 8))
    out.discard("")
    return out


def test_parity_cases_reach_every_kernel(lib):
    want = reachable(lib)
    assert len(want) >= 40  # both kernel families, four head dims, both masks, both dtypes
    missing = sorted(want - parity_launches(lib))
    assert not missing, f"kernels no GPU parity case launches: {missing}"
