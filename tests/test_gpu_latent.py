"""GPU parity of the decode against a compressed-latent cache: the weight
preparation, the cache append and the absorbed attention, against the fp64
oracle's definition (every cached latent expanded into per-head keys and
values, then plain attention), on the Kimi-K2-shape workload and on small,
ragged and edge shapes."""

import numpy as np
import pytest
import torch

import workloads
from oracle import mla_oracle as O
from tests.gpu_util import MAX_ABS, REL_L2, assert_close, errors, f64, say

# a plain import: a missing or stale libmla.so must fail these tests, not skip them
import head_latent_attention_rmsnorm_amd as M  # noqa: E402

pytestmark = pytest.mark.gpu
api, pipeline = M.api, M.pipeline


def table(w, n_pos):
    return pipeline.build_table(api.params_from(w.rope, w.Dr), n_pos, w.Dqk)


def small(seed=41, B=3, H=8, Dn=64, Dv=64, L=150, pairing="half", rope=workloads.YARN_KIMI):
    return workloads.custom(name="latent_small", B=B, T=1, H=H, R=512, Dn=Dn, Dr=64, Dv=Dv, seed=seed,
                            decode=True, cache_len=L, q_pos=L - 1, pairing=pairing, rope=rope, latent_cache=True)


def run(w, inp, q_pos, num_splits=0, cache=None):
    """Append + absorbed decode on the GPU; returns (out [B,H,1,Dv], cache)."""
    g = {k: v.cuda() for k, v in inp.items()}
    qp = torch.tensor(q_pos, dtype=torch.int32, device="cuda")
    seq = qp + 1
    tab = table(w, w.cache_len)
    wt = api.mla_absorb_prepare(g["W"], w.H, w.Dn, w.Dv)
    cache = (g["latent_cache"] if cache is None else cache.cuda()).clone()
    out = pipeline.decode_latent_step(g["q"], g["latent"], g["k_pe"], g["gain"], g["W"], wt, cache, seq, qp, tab,
                                      w.Dn, w.Dv, w.pairing, w.eps, num_splits)
    torch.cuda.synchronize()
    return out.cpu(), cache.cpu()


def test_absorb_prepare_is_a_transpose():
    say("[latent] absorb_prepare")
    H, R, Dn, Dv = 3, 100, 40, 24
    W = torch.randn(H * (Dn + Dv), R, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    got = api.mla_absorb_prepare(W.cuda(), H, Dn, Dv).cpu()
    ref = W.view(H, Dn + Dv, R)[:, :Dn, :].transpose(1, 2).contiguous()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_latent_cache_append(pairing):
    w = small(seed=42, pairing=pairing)
    say(f"[latent] append {pairing}")
    inp = workloads.make_inputs(w)
    q_pos = [149, 0, 77]
    g = {k: v.cuda() for k, v in inp.items()}
    qp = torch.tensor(q_pos, dtype=torch.int32, device="cuda")
    tab = table(w, w.cache_len)
    cache = g["latent_cache"].clone()
    api.mla_latent_cache_append(g["latent"].view(w.B, w.R), g["gain"], g["k_pe"].view(w.B, w.Dr), tab.cos, tab.sin,
                                qp, cache, w.eps, pairing)
    got = cache.cpu()
    before = inp["latent_cache"]
    c_ref = O.rmsnorm(f64(inp["latent"]), f64(inp["gain"]), w.eps)[:, 0]  # [B, R]
    cos, sin = O.rope_table(w.rope, w.Dr, w.cache_len)
    u = 2.0 ** -24
    for b, p in enumerate(q_pos):
        # RMSNorm in fp32, one fp16 rounding
        r = c_ref[b]
        d = np.abs(f64(got[b, p, :w.R]) - r)
        assert np.all(d <= np.abs(r) * (2.0 ** -11 + (w.R + 8) * u) + 2.0 ** -25), (b, d.max())
        # rotation in fp32 from the fp32 table (angle error about p * 2^-24), one fp16 rounding
        x = f64(inp["k_pe"][b, 0])
        k = O.rotate(x, cos[p], sin[p], pairing)
        mag = np.abs(x) + np.abs(x[(np.arange(w.Dr) + w.Dr // 2) % w.Dr] if pairing == "half"
                                  else x.reshape(-1, 2)[:, ::-1].reshape(-1))
        d = np.abs(f64(got[b, p, w.R:]) - k)
        assert np.all(d <= np.abs(k) * 2.0 ** -11 + mag * (p + 64) * 8 * u), (b, d.max())
        # every other row is untouched
        mask = torch.ones(w.cache_len, dtype=torch.bool)
        mask[p] = False
        assert torch.equal(got[b][mask].view(torch.int16), before[b][mask].view(torch.int16))


@pytest.mark.parametrize("q_pos", [[149, 149, 149], [149, 0, 77]], ids=["uniform", "ragged"])
def test_decode_absorbed_small(q_pos):
    w = small(seed=43)
    inp = workloads.make_inputs(w)
    ref = O.decode_latent(w, inp, q_pos=q_pos)
    for S in (0, 1, 2, 3):
        say(f"[latent] small q_pos={q_pos} splits={S}")
        out, _ = run(w, inp, q_pos, S)
        assert_close(f64(out), ref, f"absorbed small splits={S}")


def test_decode_absorbed_heads_dims_pairing():
    # H = 70: a second, partial group of 64 heads; Dn 128 / Dv 96; default
    # RoPE with interleaved pairing
    w = small(seed=44, B=2, H=70, Dn=128, Dv=96, L=300, pairing="interleaved",
              rope=workloads.RopeSpec(kind="default", base=10000.0))
    inp = workloads.make_inputs(w)
    q_pos = [299, 130]
    ref = O.decode_latent(w, inp, q_pos=q_pos)
    for S in (0, 4):
        say(f"[latent] H=70 Dn=128 Dv=96 interleaved splits={S}")
        out, _ = run(w, inp, q_pos, S)
        assert_close(f64(out), ref, f"absorbed H70 splits={S}")


def test_decode_absorbed_single_row_and_padding():
    # q_pos 0: the new row alone (softmax of one score); cache rows past
    # seq_len hold large finite garbage, which must not reach the output
    w = small(seed=45, B=2, L=200)
    inp = workloads.make_inputs(w)
    q_pos = [0, 63]
    cache = inp["latent_cache"].clone()
    cache[0, 1:] = 3.0e4
    cache[1, 64:] = -3.0e4
    inp2 = dict(inp, latent_cache=cache)
    ref = O.decode_latent(w, inp2, q_pos=q_pos)
    for S in (0, 1, 4):
        say(f"[latent] single row / padding splits={S}")
        out, _ = run(w, inp2, q_pos, S)
        assert np.all(np.isfinite(f64(out)))
        assert_close(f64(out), ref, f"absorbed single-row splits={S}")


@pytest.mark.parametrize("qmul", [3.0, 4.5])
def test_decode_absorbed_sharp_softmax(qmul):
    # the query scaled up: scores span many powers of two, so later key tiles
    # overtake the per-head reference (the lazy rescale path)
    w = small(seed=46, B=2, L=400)
    inp = workloads.make_inputs(w)
    inp["q"] = (inp["q"].float() * qmul).to(torch.bfloat16)
    q_pos = [399, 250]
    ref = O.decode_latent(w, inp, q_pos=q_pos)
    for S in (0, 1, 3):
        say(f"[latent] sharp softmax q x {qmul} splits={S}")
        out, _ = run(w, inp, q_pos, S)
        assert np.all(np.isfinite(f64(out)))
        assert_close(f64(out), ref, f"absorbed sharp x{qmul} splits={S}")


def test_decode_absorbed_kimi():
    w = workloads.WORKLOADS["kimi_k2_decode_latent"]
    say("[latent] kimi_k2_decode_latent B=32 L=1001 H=64")
    inp = workloads.make_inputs(w)
    q_pos = [w.q_pos] * w.B
    picks = [0, 13, 31]
    ref = O.decode_latent(w, inp, b_idx=picks)
    outs = {}
    for S in (0, 1, 5, 16):
        out, cache = run(w, inp, q_pos, S)
        outs[S] = out
        ma, rl = errors(f64(out[picks]), ref)
        say(f"  splits={S or 'auto'}: max-abs {ma:.3e} rel-L2 {rl:.3e}")
        assert ma <= MAX_ABS and rl <= REL_L2, (S, ma, rl)
    # every sequence, not only the sampled ones: the split counts agree
    for S in (1, 5, 16):
        d = np.abs(f64(outs[S]) - f64(outs[0]))
        assert np.all(d <= np.abs(f64(outs[0])) * 2.0 ** -7 + 2e-3), (S, d.max())


# ---- the same outputs by re-expanding the latent cache on every call

def run_expand(w, inp, q_pos, num_splits=0):
    g = {k: v.cuda() for k, v in inp.items()}
    qp = torch.tensor(q_pos, dtype=torch.int32, device="cuda")
    tab = table(w, w.cache_len)
    cache = g["latent_cache"].clone()
    out = pipeline.decode_latent_step(g["q"], g["latent"], g["k_pe"], g["gain"], g["W"], None, cache, qp + 1, qp, tab,
                                      w.Dn, w.Dv, w.pairing, w.eps, num_splits, method="expand")
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("q_pos", [[36, 36, 36], [36, 0, 20]], ids=["uniform", "ragged"])
def test_decode_latent_expanded_tiny(q_pos):
    w = workloads.WORKLOADS["tiny_decode_latent"]
    inp = workloads.make_inputs(w)
    ref = O.decode_latent(w, inp, q_pos=q_pos)
    for S in (0, 1, 2):
        say(f"[latent expand] tiny q_pos={q_pos} splits={S}")
        assert_close(f64(run_expand(w, inp, q_pos, S)), ref, f"re-expansion tiny splits={S}")


def test_decode_latent_expanded_kimi_agrees_with_absorbed():
    w = workloads.WORKLOADS["kimi_k2_decode_latent"]
    say("[latent expand] kimi_k2_decode_latent B=32 L=1001")
    inp = workloads.make_inputs(w)
    q_pos = [w.q_pos] * w.B
    picks = [0, 31]
    ref = O.decode_latent(w, inp, b_idx=picks)
    out = run_expand(w, inp, q_pos)
    ma, rl = errors(f64(out[picks]), ref)
    say(f"  re-expansion: max-abs {ma:.3e} rel-L2 {rl:.3e}")
    assert ma <= MAX_ABS and rl <= REL_L2
    absorbed, _ = run(w, inp, q_pos)
    ma, rl = errors(f64(out), f64(absorbed))  # every sequence: the two evaluations agree
    say(f"  re-expansion vs absorbed, all sequences: max-abs {ma:.3e} rel-L2 {rl:.3e}")
    assert ma <= MAX_ABS and rl <= REL_L2
