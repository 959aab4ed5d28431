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
