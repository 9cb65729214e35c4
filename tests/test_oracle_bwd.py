"""Pins of the backward (gradient) oracle against things other than itself:
torch autograd through scaled_dot_product_attention in fp64 on the CPU (an
independent library routine), central finite differences of a numpy forward,
and two identities of the softmax gradient."""
import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits


def _rand(shape, gen, scale=1.0):
    return (torch.randn(shape, generator=gen, dtype=torch.float32) * scale).to(torch.bfloat16)


def _case(B, H, Hkv, N, d, seed, qscale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (_rand((B, H, N, d), g, qscale), _rand((B, Hkv, N, d), g), _rand((B, Hkv, N, d), g),
            _rand((B, H, N, d), g))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 4), (2, 4, 2, 19, 16), (1, 6, 3, 33, 8),
                                   (1, 8, 1, 40, 32)])
def test_against_torch_autograd(oracle_lib, causal, shape):
    B, H, Hkv, N, d = shape
    q, k, v, do = _case(B, H, Hkv, N, d, seed=N + H, qscale=2.0)
    scale = 0.7 / np.sqrt(d)
    dq, dk, dv = oracle.attn_bwd(bf16_bits(q), bf16_bits(k), bf16_bits(v), bf16_bits(do),
                                 causal=causal, scale=scale)
    G = H // Hkv
    qt = q.double().requires_grad_()
    kt = k.double().requires_grad_()
    vt = v.double().requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1), is_causal=causal,
        scale=scale)
    o.backward(do.double())
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-10)


def _forward_np(q, k, v, causal, scale, G):
    B, H, N, d = q.shape
    o = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            S = q[b, h] @ k[b, h // G].T * scale
            if causal:
                S = np.where(np.tril(np.ones((N, N), dtype=bool)), S, -np.inf)
            P = np.exp(S - S.max(1, keepdims=True))
            o[b, h] = (P / P.sum(1, keepdims=True)) @ v[b, h // G]
    return o


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(oracle_lib, causal):
    B, H, Hkv, N, d = 1, 2, 1, 5, 3
    q, k, v, do = _case(B, H, Hkv, N, d, seed=3, qscale=1.5)
    scale = 0.9
    dq, dk, dv = oracle.attn_bwd(bf16_bits(q), bf16_bits(k), bf16_bits(v), bf16_bits(do),
                                 causal=causal, scale=scale)
    base = [x.double().numpy() for x in (q, k, v)]
    dod = do.double().numpy()
    loss = lambda xs: float((_forward_np(*xs, causal, scale, H // Hkv) * dod).sum())
    eps = 1e-6
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for idx in np.ndindex(*base[which].shape):
            xs = [x.copy() for x in base]
            xs[which][idx] += eps
            up = loss(xs)
            xs[which][idx] -= 2 * eps
            fd = (up - loss(xs)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7, (which, idx, fd, grad[idx])


def test_gradient_identities(oracle_lib):
    """Rows of dS sum to zero, so sum_j dK_j = 0 per head; rows of P sum to one,
    so sum_j dV_j = sum_i dO_i (summed over the group's heads)."""
    B, H, Hkv, N, d = 2, 4, 2, 37, 16
    q, k, v, do = _case(B, H, Hkv, N, d, seed=11)
    for causal in (False, True):
        dq, dk, dv = oracle.attn_bwd(bf16_bits(q), bf16_bits(k), bf16_bits(v), bf16_bits(do),
                                     causal=causal, scale=0.25)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-11)
        dos = do.double().numpy().reshape(B, Hkv, H // Hkv, N, d).sum(axis=(2, 3))
        np.testing.assert_allclose(dv.sum(axis=2), dos, atol=1e-10)
