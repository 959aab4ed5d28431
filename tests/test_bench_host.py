"""Host-side checks of bench.py: the plain-attention baseline of the sweep computes attention
(checked against the oracle on the CPU in float64), the kernel names it reports are the
library's dispatch choices for the workloads, and more than one GPU is refused."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import oracle
from seeded_inputs import WORKLOADS, Workload, make_inputs, to_f64

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n,d", [(1, 16), (37, 32), (96, 64)])
def test_plain_attention_matches_oracle(n, d):
    inp = make_inputs(2, 1, n, n, d, "f32", index=9100 + n)
    q, k, v, do = (torch.from_numpy(to_f64(inp[x])) for x in ("q", "k", "v", "do"))
    scale = 1.0 / d ** 0.5
    mask = torch.ones(n, n, dtype=torch.bool).triu_(1)
    o, p = bench.plain_attention_forward(q, k, v, True, scale, mask)
    dq, dk, dv = bench.plain_attention_backward(q, k, v, p, do, scale)
    want_o, _ = oracle.forward(q.numpy(), k.numpy(), v.numpy(), True, scale)
    want = oracle.backward(q.numpy(), k.numpy(), v.numpy(), do.numpy(), True, scale)
    np.testing.assert_allclose(o.numpy(), want_o, rtol=0, atol=1e-12)
    for got, ref in zip((dq, dk, dv), want[:3]):
        np.testing.assert_allclose(got.numpy(), ref, rtol=0, atol=1e-12)


def test_kernel_names_follow_dispatch():
    assert bench.kernel_names(WORKLOADS["b8_n4096_d64"]) == (
        "fwd_causal_wide_kernel<64>", "bwd_causal_paired_kernel<64>")
    assert bench.kernel_names(WORKLOADS["xl_noncausal"]) == (
        "fwd_kernel<64, false>", "bwd_kernel<64, false>")
    assert bench.kernel_names(WORKLOADS["long_n16384_d128"]) == (
        "fwd_kernel<128, true>", "bwd_kernel<128, true>")
    assert bench.kernel_names(WORKLOADS["gpt_small"]) == (
        "fwd_causal_paired_kernel<64>", "bwd_causal_paired_lean_kernel<64>")
    assert bench.kernel_names(WORKLOADS["xl_causal"]) == (
        "fwd_kernel<64, true>", "bwd_kernel<64, true>")
    assert bench.kernel_names(WORKLOADS["tiny_f32"]) == (
        "fwd_f32_kernel<16, true>", "bwd_f32_kernel<16, true>")
    one_head_d16 = Workload("one_head_d16", 99, 1, 1, 8192, 8192, 16, "bf16", True)
    assert bench.kernel_names(one_head_d16) == (
        "fwd_causal_split_kernel<16>", "bwd_kernel<16, true>")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
