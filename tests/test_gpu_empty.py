"""Empty batches and zero-length inputs on the GPU: every entry point returns
cleanly, launches nothing that fails, leaves no stale HIP error behind (a
normal call right after still succeeds), and returns outputs of the empty
shape the call implies."""

import pytest
import torch

import workloads
from tests.gpu_util import say

import head_latent_attention_rmsnorm_amd as M  # noqa: E402

pytestmark = pytest.mark.gpu
api, pipeline = M.api, M.pipeline
DEV = "cuda"
BF, F16, I32 = torch.bfloat16, torch.float16, torch.int32
H, R, Dn, Dr, Dv = 4, 512, 128, 64, 128  # a compiled head shape (Kimi-K2 widths)


def rnd(*shape, dtype=BF, seed=0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV) * 0.1).to(dtype)


def table(n):
    return pipeline.build_table(api.params_from(workloads.YARN_KIMI, Dr), n, Dn + Dr)


def still_works():
    # a normal call after the empty ones: no stale error is reported
    x = rnd(3, R)
    y = api.mla_latent_rmsnorm(x, torch.ones(R, dtype=BF, device=DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()


def test_empty_norms_linear_expand():
    say("[empty] rmsnorm, linear, kv_expand")
    g = torch.ones(R, dtype=BF, device=DEV)
    x0 = torch.empty((0, R), dtype=BF, device=DEV)
    assert api.mla_latent_rmsnorm(x0, g).shape == (0, R)
    assert api.mla_rmsnorm(x0, g).shape == (0, R)
    assert api.mla_linear(x0, rnd(96, R)).shape == (0, 96)
    c0 = torch.empty((2, 0, R), dtype=F16, device=DEV)
    k, v = api.mla_kv_expand(c0, rnd(H * (Dn + Dv), R), H, Dn, Dv)
    assert k.shape == (2, H, 0, Dn) and v.shape == (2, H, 0, Dv)
    torch.cuda.synchronize()
    still_works()


def test_empty_chunk_and_rotation():
    say("[empty] rotate_rope_key T=0, prefill_attention_cached T=0")
    B, Tcap, past = 2, 32, 16
    tab = table(Tcap)
    dst = torch.zeros((B, Tcap, Dr), dtype=F16, device=DEV)
    api.mla_rotate_rope_key(torch.empty((B, 0, Dr), dtype=BF, device=DEV), tab.cos, tab.sin, dst, past)
    assert torch.count_nonzero(dst) == 0
    q = torch.empty((B, H, 0, Dn + Dr), dtype=BF, device=DEV)
    kn = rnd(B, H, Tcap, Dn, dtype=F16)
    vt = rnd(B, H, Dv, Tcap, dtype=F16)
    out = api.mla_prefill_attention_cached(q, kn, dst, vt, past, tab.cos, tab.sin, tab.scale)
    assert out.shape == (B, H, 0, Dv)
    torch.cuda.synchronize()
    still_works()


def test_empty_decode_batches():
    say("[empty] decode_attention, latent_cache_append, decode_absorbed, decode_latent_expanded with B=0")
    L = 40
    tab = table(L)
    e32 = torch.empty((0,), dtype=I32, device=DEV)
    q = torch.empty((0, H, 1, Dn + Dr), dtype=BF, device=DEV)
    out = api.mla_decode_attention(q, torch.empty((0, H, L, Dn + Dr), dtype=BF, device=DEV),
                                   torch.empty((0, H, L, Dv), dtype=BF, device=DEV), e32, e32, tab.cos, tab.sin,
                                   tab.scale, Dn)
    assert out.shape == (0, H, 1, Dv)
    cache = torch.empty((0, L, R + Dr), dtype=F16, device=DEV)
    api.mla_latent_cache_append(torch.empty((0, R), dtype=BF, device=DEV), torch.ones(R, dtype=BF, device=DEV),
                                torch.empty((0, Dr), dtype=BF, device=DEV), tab.cos, tab.sin, e32, cache)
    W = rnd(H * (Dn + Dv), R)
    wt = api.mla_absorb_prepare(W, H, Dn, Dv)
    out = api.mla_decode_absorbed(q, W, wt, cache, e32, e32, tab.cos, tab.sin, tab.scale, Dn, Dv)
    assert out.shape == (0, H, 1, Dv)
    out = api.mla_decode_latent_expanded(q, W, cache, e32, e32, tab.cos, tab.sin, tab.scale, Dn, Dv)
    assert out.shape == (0, H, 1, Dv)
    torch.cuda.synchronize()
    still_works()
