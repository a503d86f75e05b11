"""A decode step recorded as a HIP graph and replayed: every replay, with new
inputs copied into the captured buffers and eager work and synchronisations
in between, gives the same bits as the same step run eagerly on the same
inputs (the latent-cache step: append + absorbed decode; the expanded-cache
step: RMSNorm + append + decode attention)."""

import pytest
import torch

import workloads
from tests.gpu_util import say

import head_latent_attention_rmsnorm_amd as M  # noqa: E402

pytestmark = pytest.mark.gpu
api, pipeline = M.api, M.pipeline


def _bits(t):
    return t.view(torch.int16)


def test_latent_decode_step_graph_replays():
    w = workloads.custom(name="graph-latent", B=4, T=1, H=8, R=512, Dn=128, Dr=64, Dv=128, seed=60, decode=True,
                         cache_len=300, q_pos=299, rope=workloads.YARN_KIMI, latent_cache=True)
    say("[graph] latent-cache decode step: capture, 3 replays against eager")
    base = {k: v.cuda() for k, v in workloads.make_inputs(w).items()}
    tab = pipeline.build_table(api.params_from(w.rope, w.Dr), w.cache_len, w.Dqk)
    wt = api.mla_absorb_prepare(base["W"], w.H, w.Dn, w.Dv)
    qpos = torch.full((w.B,), w.q_pos, dtype=torch.int32, device="cuda")
    seq = qpos + 1
    # static buffers the graph reads
    q, latent, k_pe = base["q"].clone(), base["latent"].clone(), base["k_pe"].clone()
    cache = base["latent_cache"].clone()
    ws = torch.empty((16 << 20,), dtype=torch.uint8, device="cuda")

    def step():
        return pipeline.decode_latent_step(q, latent, k_pe, base["gain"], base["W"], wt, cache, seq, qpos, tab, w.Dn,
                                           w.Dv, w.pairing, w.eps, workspace=ws)
    g = pipeline.StepGraph(step)
    gen = torch.Generator(device="cuda").manual_seed(61)
    for r in range(3):
        # new token data; the cache row the step appends is rewritten each time
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        latent.copy_(torch.randn(latent.shape, generator=gen, device="cuda").to(torch.bfloat16))
        k_pe.copy_(torch.randn(k_pe.shape, generator=gen, device="cuda").to(torch.bfloat16))
        got = g.replay().clone()
        cache_after = cache.clone()
        torch.cuda.synchronize()
        # eager on the same inputs, into fresh buffers
        ref_cache = cache.clone()
        ref = pipeline.decode_latent_step(q, latent, k_pe, base["gain"], base["W"], wt, ref_cache, seq, qpos, tab,
                                          w.Dn, w.Dv, w.pairing, w.eps)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(ref)), r
        assert torch.equal(_bits(cache_after), _bits(ref_cache)), r
        torch.cuda.synchronize()


def test_expanded_decode_step_graph_replays():
    w = workloads.custom(name="graph-decode", B=4, T=1, H=8, R=512, Dn=128, Dr=64, Dv=128, seed=62, decode=True,
                         cache_len=300, q_pos=299, rope=workloads.YARN_KIMI)
    say("[graph] expanded-cache decode step: capture, 3 replays against eager")
    base = {k: v.cuda() for k, v in workloads.make_inputs(w).items()}
    tab = pipeline.build_table(api.params_from(w.rope, w.Dr), w.cache_len, w.Dqk)
    qpos = torch.full((w.B,), w.q_pos, dtype=torch.int32, device="cuda")
    seq = qpos + 1
    q, latent, k_pe = base["q"].clone(), base["latent"].clone(), base["k_pe"].clone()
    kc, vc = base["k_cache"].clone(), base["v_cache"].clone()
    ws = torch.empty((16 << 20,), dtype=torch.uint8, device="cuda")

    def step():
        return pipeline.decode_step(q, latent, k_pe, base["gain"], base["W"], kc, vc, seq, qpos, w.q_pos, tab, w.Dn,
                                    w.pairing, w.eps, workspace=ws)
    g = pipeline.StepGraph(step)
    gen = torch.Generator(device="cuda").manual_seed(63)
    for r in range(3):
        q.copy_(torch.randn(q.shape, generator=gen, device="cuda").to(torch.bfloat16))
        latent.copy_(torch.randn(latent.shape, generator=gen, device="cuda").to(torch.bfloat16))
        k_pe.copy_(torch.randn(k_pe.shape, generator=gen, device="cuda").to(torch.bfloat16))
        got = g.replay().clone()
        torch.cuda.synchronize()
        kr, vr = kc.clone(), vc.clone()
        ref = pipeline.decode_step(q, latent, k_pe, base["gain"], base["W"], kr, vr, seq, qpos, w.q_pos, tab, w.Dn,
                                   w.pairing, w.eps)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(ref)), r
        assert torch.equal(_bits(kc), _bits(kr)) and torch.equal(_bits(vc), _bits(vr)), r
