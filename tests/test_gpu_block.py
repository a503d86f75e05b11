"""GPU parity of the whole attention block around the path: q_a_proj ->
query RMSNorm -> q_b_proj (head-major), kv_a_proj_with_mqa (latent and
rotary key apart), the prefill path, o_proj on its head-major output,
against the fp64 oracle's block_forward."""

import numpy as np
import pytest
import torch

import workloads
from oracle import mla_oracle as O
from tests.gpu_util import errors, f64, say

# a plain import: a missing or stale libmla.so must fail these tests, not skip them
import head_latent_attention_rmsnorm_amd as M  # noqa: E402

pytestmark = pytest.mark.gpu
api, pipeline = M.api, M.pipeline

# The path's tolerance. The bf16 rounding of the intermediate projections
# (q_a, the normalised query, q, the latent and rotary key, the attention
# output) adds to the path's own error: measured rel-L2 3.5e-3 / 3.6e-3 and
# max-abs 1.4e-2 / 8.5e-3 (Kimi-K2 1k sampled rows / tiny) on outputs of unit
# scale.
BLOCK_MAX_ABS, BLOCK_REL_L2 = 2e-2, 5e-3


def run_block(w, inp):
    g = {k: v.cuda() for k, v in inp.items()}
    tab = pipeline.build_table(api.params_from(w.rope, w.Dr), w.T, w.Dqk)
    out = pipeline.block_forward(g["hidden"], g["W_qa"], g["gain_q"], g["W_qb"], g["W_kva"], g["gain"], g["W"],
                                 g["W_o"], tab, w.H, w.Dn, w.Dr, w.Dv, w.pairing, w.eps)
    torch.cuda.synchronize()
    return out.cpu()


def test_rmsnorm_bf16_out():
    g = torch.Generator().manual_seed(4)
    x = torch.randn(37, 1536, generator=g).to(torch.bfloat16)
    w = (1 + 0.3 * torch.randn(1536, generator=g)).to(torch.bfloat16)
    say("[block] rmsnorm bf16")
    got = f64(api.mla_rmsnorm(x.cuda(), w.cuda(), 1e-6, dtype=torch.bfloat16).cpu())
    ref = O.rmsnorm(f64(x), f64(w), 1e-6)
    # fp32 arithmetic, one bf16 rounding
    assert np.all(np.abs(got - ref) <= np.abs(ref) * (2.0 ** -8 + 1544 * 2.0 ** -24) + 1e-30)


def test_block_tiny():
    w = workloads.WORKLOADS["tiny_block"]
    say("[block] tiny")
    inp = workloads.make_inputs(w)
    got = run_block(w, inp)
    ma, rl = errors(f64(got), O.block_forward(w, inp))
    say(f"  max-abs {ma:.3e} rel-L2 {rl:.3e}")
    assert ma <= BLOCK_MAX_ABS and rl <= BLOCK_REL_L2


def test_block_kimi_1k_sampled_rows():
    w = workloads.WORKLOADS["kimi_k2_block_1k"]
    say("[block] kimi_k2_block_1k, sampled rows")
    inp = workloads.make_inputs(w)
    got = run_block(w, inp)
    assert got.shape == (w.B, w.T, w.hidden)
    rows = [0, 1, 255, 512, 1023]
    ma, rl = errors(f64(got[:, rows]), O.block_forward(w, inp, rows=rows))
    say(f"  max-abs {ma:.3e} rel-L2 {rl:.3e}")
    assert ma <= BLOCK_MAX_ABS and rl <= BLOCK_REL_L2
    assert np.all(np.isfinite(f64(got)))
