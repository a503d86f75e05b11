"""GPU parity of the linear layer Y = X W^T (+ bias) (the nn.Linear
projections around the latent attention) against a float64 matmul of the
same bf16 inputs, in every layout mode."""

import numpy as np
import pytest
import torch

from tests.gpu_util import f64, say

# a plain import: a missing or stale libmla.so must fail these tests, not skip them
import head_latent_attention_rmsnorm_amd as M  # noqa: E402

pytestmark = pytest.mark.gpu
api = M.api


def bf16(shape, gen, std=1.0):
    return (torch.randn(*shape, generator=gen) * std).to(torch.bfloat16)


def check(got, x, w, bias=None):
    """One bf16 rounding after an fp32 sum: |err| <= |ref| 2^-8 + K 2^-24 sum|x||w|."""
    X, W = f64(x), f64(w)
    ref = X @ W.T
    if bias is not None:
        ref = ref + f64(bias)
    mag = np.abs(X) @ np.abs(W).T
    K = X.shape[1]
    d = np.abs(f64(got) - ref)
    bound = np.abs(ref) * 2.0 ** -8 + K * 2.0 ** -24 * mag + 1e-30
    assert np.all(d <= bound), float((d / bound).max())
    return float(d.max())


@pytest.mark.parametrize("M,N,K", [(300, 200, 192), (1, 576, 512), (1024, 1536, 7168), (513, 264, 1536)])
def test_linear_rows(M, N, K):
    g = torch.Generator().manual_seed(M + N + K)
    x, w = bf16((M, K), g), bf16((N, K), g, K ** -0.5)
    say(f"[linear] rows M={M} N={N} K={K}")
    got = api.mla_linear(x.cuda(), w.cuda()).cpu()
    check(got, x, w)


def test_linear_bias():
    g = torch.Generator().manual_seed(3)
    x, w, b = bf16((257, 512), g), bf16((72, 512), g, 512 ** -0.5), bf16((72,), g)
    say("[linear] bias")
    check(api.mla_linear(x.cuda(), w.cuda(), b.cuda()).cpu(), x, w, b)


@pytest.mark.parametrize("H,D", [(4, 32), (3, 128)])
def test_linear_heads_in(H, D):
    # X head-major [B, H, T, D] read as [B*T, H*D] (the o_proj input)
    g = torch.Generator().manual_seed(H * D)
    B, T, N = 2, 50, 96
    x4 = bf16((B, H, T, D), g)
    w = bf16((N, H * D), g, (H * D) ** -0.5)
    say(f"[linear] head-major X H={H} D={D}")
    got = api.mla_linear(x4.cuda(), w.cuda(), x_heads=True).cpu()  # [B*T, N]
    x2 = x4.permute(0, 2, 1, 3).reshape(B * T, H * D)
    check(got.reshape(B * T, N), x2, w)


def test_linear_heads_out():
    # Y head-major [B, H, T, D] (the q_b_proj output feeding the attention)
    g = torch.Generator().manual_seed(11)
    B, T, K, H, D = 2, 70, 192, 3, 24
    x = bf16((B, T, K), g)
    w = bf16((H * D, K), g, K ** -0.5)
    say("[linear] head-major Y")
    got = api.mla_linear(x.cuda(), w.cuda(), out_heads=(H, D)).cpu()  # [B, H, T, D]
    assert got.shape == (B, H, T, D)
    check(got.permute(0, 2, 1, 3).reshape(B * T, H * D), x.reshape(B * T, K), w)


def test_linear_split():
    # Y split at a column (kv_a_proj_with_mqa: latent | rotary key)
    g = torch.Generator().manual_seed(12)
    x = bf16((2, 33, 512), g)
    w = bf16((576, 512), g, 512 ** -0.5)
    b = bf16((576,), g)
    say("[linear] split")
    y0, y1 = api.mla_linear(x.cuda(), w.cuda(), b.cuda(), split=512)
    assert y0.shape == (2, 33, 512) and y1.shape == (2, 33, 64)
    got = torch.cat([y0.cpu(), y1.cpu()], -1).reshape(66, 576)
    check(got, x.reshape(66, 512), w, b)
