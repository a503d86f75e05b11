"""GPU parity of chunked prefill (prefill against a past cache): a sequence
processed in chunks, each appended to an expanded cache and attending to all
earlier rows, must give the rows of the one-shot causal prefill that the
fp64 oracle computes (Kimi-K2 "Query content heads", section "Join query
parts": with past key values the cache is updated first and the causal mask
is offset by the cached length)."""

import numpy as np
import pytest
import torch

import workloads
from oracle import mla_oracle as O
from tests.gpu_util import assert_close, errors, f64, say

# a plain import: a missing or stale libmla.so must fail these tests, not skip them
import head_latent_attention_rmsnorm_amd as M  # noqa: E402

pytestmark = pytest.mark.gpu
api, pipeline = M.api, M.pipeline


def table(w, n_pos):
    return pipeline.build_table(api.params_from(w.rope, w.Dr), n_pos, w.Dqk)


SHAPES = [
    dict(name="k2", B=2, T=600, H=4, R=512, Dn=128, Dr=64, Dv=128, rope=workloads.YARN_KIMI, pairing="half",
         chunks=[256, 144, 200]),
    dict(name="glm", B=1, T=333, H=3, R=512, Dn=192, Dr=64, Dv=256,
         rope=workloads.RopeSpec(kind="default", base=10000.0), pairing="interleaved", chunks=[100, 1, 232]),
    dict(name="tiny", B=3, T=150, H=2, R=64, Dn=32, Dr=16, Dv=32,
         rope=workloads.RopeSpec(kind="default", base=10000.0), pairing="half", chunks=[64, 13, 73]),
]


def run_chunks(w, inp, chunks, Tcap, return_lse=True):
    g = {k: v.cuda() for k, v in inp.items()}
    tab = table(w, Tcap)
    cache = pipeline.alloc_chunk_cache(w.B, w.H, Tcap, w.Dn, w.Dr, w.Dv)
    outs, lses, past = [], [], 0
    for n in chunks:
        sl = slice(past, past + n)
        o, l = pipeline.prefill_chunk(g["q"][:, :, sl].contiguous(), g["latent"][:, sl].contiguous(),
                                      g["k_pe"][:, sl].contiguous(), g["gain"], g["W"], cache, past, tab, w.pairing,
                                      w.eps, return_lse=True)
        outs.append(o)
        lses.append(l)
        past += n
    torch.cuda.synchronize()
    return torch.cat(outs, 2).cpu(), torch.cat(lses, 2).cpu()


@pytest.mark.parametrize("spec", SHAPES, ids=[s["name"] for s in SHAPES])
def test_chunked_prefill_matches_oracle(spec):
    spec = dict(spec)
    name, chunks = spec.pop("name"), spec.pop("chunks")
    w = workloads.custom(name=f"chunked_{name}", seed=50 + len(name), **spec)
    assert sum(chunks) == w.T
    say(f"[chunked] {name} chunks={chunks}")
    inp = workloads.make_inputs(w)
    out, lse = run_chunks(w, inp, chunks, Tcap=w.T + 37)  # cache capacity past the last row
    parts = O.prefill_parts(w, inp)
    ref = np.empty((w.B, w.H, w.T, w.Dv))
    ref_lse = np.empty((w.B, w.H, w.T))
    for b in range(w.B):
        for h in range(w.H):
            ref[b, h], ref_lse[b, h] = O.prefill_head(w, parts, b, h, return_lse=True)
    assert_close(f64(out), ref, f"chunked {name}")
    np.testing.assert_allclose(f64(lse), ref_lse, atol=2e-2, rtol=0)


def test_chunked_single_chunk_equals_plain_prefill():
    # past = 0 and one chunk covering the sequence: the same kernel on the
    # same prepared operands as mla_prefill_attention, so the bits agree
    w = workloads.custom(name="chunked_eq", B=2, T=300, H=4, R=512, Dn=128, Dr=64, Dv=128, seed=58,
                         rope=workloads.YARN_KIMI, pairing="half")
    say("[chunked] single chunk vs plain prefill")
    inp = workloads.make_inputs(w)
    out, _ = run_chunks(w, inp, [w.T], Tcap=w.T)
    g = {k: v.cuda() for k, v in inp.items()}
    tab = table(w, w.T)
    c = api.mla_latent_rmsnorm(g["latent"], g["gain"], w.eps)
    kn, vt = api.mla_kv_expand(c, g["W"], w.H, w.Dn, w.Dv, v_layout="cols")
    plain = api.mla_prefill_attention(g["q"], kn, g["k_pe"], vt, tab.cos, tab.sin, tab.scale, w.pairing,
                                      v_layout="cols").cpu()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))


def test_chunked_one_token_chunks():
    # single-token chunks at several depths: each is a decode step against
    # the expanded cache (keys 0..past)
    w = workloads.custom(name="chunked_tok", B=2, T=70, H=3, R=512, Dn=128, Dr=64, Dv=128, seed=59,
                         rope=workloads.YARN_KIMI, pairing="half")
    say("[chunked] one-token chunks")
    inp = workloads.make_inputs(w)
    chunks = [64, 1, 1, 1, 1, 1, 1]
    out, _ = run_chunks(w, inp, chunks, Tcap=80)
    parts = O.prefill_parts(w, inp)
    rows = np.arange(64, 70)
    for b in range(w.B):
        for h in range(w.H):
            ref = O.prefill_head(w, parts, b, h, rows=rows)
            ma, rl = errors(f64(out[b, h, 64:]), ref)
            assert ma <= 2e-2 and rl <= 5e-3, (b, h, ma, rl)
