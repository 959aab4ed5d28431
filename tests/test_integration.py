"""The drop-in path: integration.scaled_dot_product_attention monkey-patched into a model.

CPU tests cover the patch mechanics and argument checks (they fail before any kernel call);
GPU tests train-step a small decoder with plain attention and with the flash kernels patched
in, and compare the loss and every parameter gradient."""
import types

import pytest
import torch

import bench
from tiled_attention_causal_amd import integration


def test_patched_replaces_and_restores():
    mod = types.SimpleNamespace(scaled_dot_product_attention="orig")
    with integration.patched(mod, "scaled_dot_product_attention"):
        assert mod.scaled_dot_product_attention is integration.scaled_dot_product_attention
    assert mod.scaled_dot_product_attention == "orig"
    with pytest.raises(RuntimeError):
        with integration.patched(mod, "scaled_dot_product_attention", fn="other"):
            assert mod.scaled_dot_product_attention == "other"
            raise RuntimeError("inside")
    assert mod.scaled_dot_product_attention == "orig"
    with pytest.raises(AttributeError):
        with integration.patched(mod, "missing"):
            pass


def test_causal_mask_detection():
    keep = torch.ones(5, 7, dtype=torch.bool).tril_()
    assert integration._is_causal_mask(keep, 5, 7)
    assert integration._is_causal_mask(keep.expand(2, 3, 5, 7), 5, 7)
    assert not integration._is_causal_mask(keep.float(), 5, 7)
    assert not integration._is_causal_mask(torch.ones(5, 7, dtype=torch.bool), 5, 7)
    shifted = keep.clone()
    shifted[0, 1] = True
    assert not integration._is_causal_mask(shifted, 5, 7)


def test_unsupported_arguments_raise_before_any_kernel():
    q = torch.zeros(2, 3, 8, 64)
    with pytest.raises(NotImplementedError):
        integration.scaled_dot_product_attention(q, q, q, torch.ones(8, 8, dtype=torch.bool))
    with pytest.raises(NotImplementedError):
        integration.scaled_dot_product_attention(torch.zeros(2, 8, 48), torch.zeros(2, 8, 48),
                                                 torch.zeros(2, 8, 48))
    with pytest.raises(ValueError):
        integration.scaled_dot_product_attention(q, torch.zeros(2, 4, 8, 64), q)


def _train_grads(model, x):
    for p in model.parameters():
        p.grad = None
    loss = model(x).float().pow(2).mean()
    loss.backward()
    return loss.detach(), [p.grad.detach().clone() for p in model.parameters()]


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,rtol", [(torch.float32, 2e-4), (torch.bfloat16, 3e-2)])
def test_patched_model_matches_plain_attention(gpu, dtype, rtol):
    model = bench.toy_model(128, 2, 256, 2, dtype, gpu, seed=3)
    x = torch.randn(2, 192, 128, generator=torch.Generator().manual_seed(4)).to(gpu, dtype)
    loss_p, g_p = _train_grads(model, x)
    with integration.patched(bench, "scaled_dot_product_attention"):
        loss_f, g_f = _train_grads(model, x)
    torch.cuda.synchronize(gpu)
    assert torch.allclose(loss_f, loss_p, rtol=rtol, atol=0)
    for a, b in zip(g_f, g_p):
        a, b = a.float(), b.float()
        assert (a - b).norm() <= rtol * b.norm() + 1e-6


# (leading dims, N, d, how causality is given): [2, 3, N, d] as a model passes (batch,
# heads); a single leading dim; the boolean keep-mask path, is_causal, and no mask at all.
DROP_IN = [((2, 3), 200, 64, "mask"), ((2, 3), 200, 64, "is_causal"), ((6,), 130, 32, "mask"),
           ((2, 3), 96, 64, "none")]


@pytest.mark.gpu
@pytest.mark.parametrize("case", DROP_IN, ids=lambda c: "lead{}-N{}-d{}-{}".format(
    "x".join(map(str, c[0])), c[1], c[2], c[3]))
def test_drop_in_matches_oracle(gpu, case):
    """The patched-in function's output and its q, k, v gradients, element by element against
    the fp64 oracle on every (batch, head), at the bf16 bar 2e-2 + 1e-2 |oracle|."""
    import numpy as np

    import oracle
    from seeded_inputs import draw, to_f64
    lead, n, d, how = case
    shape = (*lead, n, d)
    q, k, v, do = (torch.from_numpy(draw(shape, 4200 + t)).to(torch.bfloat16)
                   for t in range(4))
    causal = how != "none"
    qg, kg, vg = (t.to(gpu).requires_grad_(True) for t in (q, k, v))
    if how == "mask":
        keep = torch.ones(n, n, dtype=torch.bool, device=gpu).tril_()
        out = integration.scaled_dot_product_attention(qg, kg, vg, keep)
    else:
        out = integration.scaled_dot_product_attention(qg, kg, vg, is_causal=causal)
    out.backward(do.to(gpu))
    torch.cuda.synchronize(gpu)
    assert out.shape == shape and out.dtype == torch.bfloat16
    scale = float(np.float32(1.0 / np.sqrt(d)))
    got = {"O": out, "dQ": qg.grad, "dK": kg.grad, "dV": vg.grad}
    got = {name: to_f64(t.detach().cpu()).reshape(-1, n, d) for name, t in got.items()}
    flat = [to_f64(t).reshape(-1, n, d) for t in (q, k, v, do)]
    for i in range(flat[0].shape[0]):
        a = [x[i] for x in flat]
        o, _, _ = oracle.head_forward(a[0], a[1], a[2], causal, scale)
        dq, dk, dv, _ = oracle.head_backward(*a, causal, scale)
        for name, want in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv)):
            err = np.abs(got[name][i] - want)
            assert np.all(err <= 2e-2 + 1e-2 * np.abs(want)), (name, i, float(err.max()))
