"""fa_backward_noalloc (the backward with the library's static device workspace, for callers
that cannot allocate) against fa_backward on the same inputs, through the C ABI: two calls in
a row, the second on smaller inputs, so the second reuses the array the first left behind."""
import ctypes
import sys

import numpy as np
import pytest
import torch

from seeded_inputs import make_inputs, to_f64

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _noalloc(q, k, v, o, lse, do, causal, scale, dq, dk, dv):
    """One call of the C entry point, arguments marshalled by hand."""
    from tiled_attention_causal_amd import _lib
    lib = _lib.load()
    B, H, Nq, d = q.shape
    dt = _lib.FA_DTYPE_BF16 if q.dtype == torch.bfloat16 else _lib.FA_DTYPE_F32
    st = lib.fa_backward_noalloc(dt, B, H, Nq, k.shape[2], d, q.data_ptr(), k.data_ptr(),
                                 v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                                 int(causal), ctypes.c_float(scale), dq.data_ptr(),
                                 dk.data_ptr(), dv.data_ptr(),
                                 torch.cuda.current_stream(q.device).cuda_stream)
    assert st == _lib.FA_SUCCESS, _lib.status_string(st)


def _check_pair(a, b, dtype):
    """The method's bar: fp32 max abs 1e-4; bf16 2e-2 + 1e-2 |reference|."""
    a, b = to_f64(a.cpu()), to_f64(b.cpu())
    bound = 1e-4 if dtype == "f32" else 2e-2 + 1e-2 * np.abs(b)
    assert np.all(np.abs(a - b) <= bound)


# Per dtype, the first call's shape and a smaller second one (fewer heads, shorter rows,
# another head dim, a ragged length, the other mask).
CALLS = {
    "bf16": [(2, 3, 1024, 64, True), (1, 2, 300, 32, False)],
    "f32": [(1, 2, 640, 64, True), (1, 1, 200, 16, True)],
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_backward_matches_backward_twice(gpu, dtype):
    from tiled_attention_causal_amd import fa_backward, fa_forward
    for i, (B, H, N, d, causal) in enumerate(CALLS[dtype]):
        note(f"noalloc backward call {i}: {dtype} B={B} H={H} N={N} d={d} causal={causal}")
        inp = make_inputs(B, H, N, N, d, dtype, index=9600 + 10 * i + d)
        q, k, v, do = (inp[n].to(gpu) for n in ("q", "k", "v", "do"))
        scale = float(np.float32(1.0 / np.sqrt(d)))
        o, lse = fa_forward(q, k, v, causal, scale)
        want = fa_backward(q, k, v, o, lse, do, causal, scale)
        got = tuple(torch.full_like(t, 7.0) for t in want)
        _noalloc(q, k, v, o, lse, do, causal, scale, *got)
        torch.cuda.synchronize(gpu)
        for name, a, b in zip(("dQ", "dK", "dV"), got, want):
            _check_pair(a, b, dtype)
            note(f"  {name}: max |noalloc - fa_backward| = "
                 f"{float((a.double() - b.double()).abs().max()):.3g}, "
                 f"bitwise equal: {torch.equal(a, b)}")
