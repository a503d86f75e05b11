"""GPU parity of the two-block prefill kernel (192/128 heads, each wave two
32-row query blocks sharing every key and value fragment it reads), which
the library runs when the grid has more than one round of 256-row work
items (B * H * ceil(T / 256) > 256). The shapes here get there with many
heads at small T, so that the fp64 oracle checks every output element in
seconds: ragged tails inside a wave's two blocks, every tile kind (the first
pipelined tile, steady state, the drain, diagonal tiles), both pairings,
explicit positions, a peaked softmax, causality, LSE and chunked prefill
(Kimi-K2 "Query content heads", section "Join query parts")."""

import numpy as np
import pytest
import torch

import workloads
from oracle import mla_oracle as O
from tests.gpu_util import assert_close, errors, f64, say, to_gpu

# a plain import: a missing or stale libmla.so must fail these tests, not skip them
import head_latent_attention_rmsnorm_amd as M  # noqa: E402

pytestmark = pytest.mark.gpu
api, pipeline = M.api, M.pipeline


def table(w, n_pos=None):
    return pipeline.build_table(api.params_from(w.rope, w.Dr), n_pos or w.T, w.Dqk)


def work_items(w):
    return w.B * w.H * ((w.T + 255) // 256)


def run(w, inp, return_lse=False):
    g = to_gpu(inp)
    res = pipeline.prefill_forward(g["q"], g["latent"], g["k_pe"], g["gain"], g["W"], table(w), w.Dn, w.Dv,
                                   w.pairing, w.eps, return_lse=return_lse)
    torch.cuda.synchronize()
    return res


def k2(name, B, T, H, seed, **kw):
    return workloads.custom(name=name, B=B, T=T, H=H, R=512, Dn=128, Dr=64, Dv=128, seed=seed,
                            rope=workloads.YARN_KIMI, **kw)


CASES = [
    k2("dual-ragged", B=2, T=301, H=130, seed=61),          # last work item: 45 rows, one block partly empty
    k2("dual-three-items", B=1, T=700, H=100, seed=62),     # 3 work items per head, 188-row tail
    k2("dual-interleaved", B=1, T=257, H=300, seed=63, pairing="interleaved"),  # one row past a work item
    k2("dual-exact", B=3, T=512, H=44, seed=64),            # whole work items, no tail
]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_dual_matches_oracle(w):
    assert work_items(w) > 256, "shape must take the two-block kernel"
    say(f"[dual] {w.name} B={w.B} T={w.T} H={w.H} ({work_items(w)} work items)")
    inp = workloads.make_inputs(w)
    out, lse = run(w, inp, return_lse=True)
    parts = O.prefill_parts(w, inp)
    ref = np.empty((w.B, w.H, w.T, w.Dv))
    ref_lse = np.empty((w.B, w.H, w.T))
    for b in range(w.B):
        for h in range(w.H):
            ref[b, h], ref_lse[b, h] = O.prefill_head(w, parts, b, h, return_lse=True)
    assert_close(f64(out), ref, f"{w.name} output")
    ma, _ = errors(f64(lse), ref_lse)
    say(f"  lse max_abs={ma:.3e}")
    assert ma < 2e-2


def test_dual_explicit_positions():
    """Positions passed in: sequence b starts at offset 37 b, so the rotation
    angles differ from the row index while the causal mask follows it."""
    w = k2("dual-pos", B=2, T=260, H=130, seed=65)
    assert work_items(w) > 256
    say("[dual] explicit positions")
    inp = workloads.make_inputs(w)
    pos = np.arange(w.T)[None, :] + 37 * np.arange(w.B)[:, None]
    n_pos = int(pos.max()) + 1
    g = to_gpu(inp)
    tab = table(w, n_pos)
    c = api.mla_latent_rmsnorm(g["latent"], g["gain"], w.eps)
    kn, vt = api.mla_kv_expand(c, g["W"], w.H, w.Dn, w.Dv, v_layout="cols")
    out = api.mla_prefill_attention(g["q"], kn, g["k_pe"], vt, tab.cos, tab.sin, tab.scale, w.pairing,
                                    pos=torch.tensor(pos, dtype=torch.int32, device="cuda"), v_layout="cols")
    torch.cuda.synchronize()
    got = f64(out.cpu())
    cn = O.rmsnorm(f64(inp["latent"]), f64(inp["gain"]), w.eps)
    k_nope, vv = O.kv_expand(cn, f64(inp["W"]), w.H, w.Dn, w.Dv)
    cos, sin = O.rope_table(w.rope, w.Dr, n_pos)
    q = f64(inp["q"])
    scale = O.softmax_scale(w.rope, w.Dqk)
    ref = np.empty_like(got)
    for b in range(w.B):
        cb, sb = cos[pos[b]], sin[pos[b]]
        q_pe = O.rotate(q[b, :, :, w.Dn:], cb[None], sb[None], w.pairing)
        k_pe = O.rotate(f64(inp["k_pe"])[b], cb, sb, w.pairing)
        for h in range(w.H):
            Q = np.concatenate([q[b, h, :, :w.Dn], q_pe[h]], axis=-1)
            K = np.concatenate([k_nope[b, h], k_pe], axis=-1)
            ref[b, h] = O.attention(Q, K, vv[b, h], scale, pos[b], pos[b])
    assert_close(got, ref, "dual explicit positions")


@pytest.mark.parametrize("qmul", [3.0, 4.5])
def test_dual_sharp_softmax(qmul):
    """A peaked softmax (query scaled up): later key tiles keep overtaking the
    running reference, so the rare rescaling path runs inside the pipeline,
    with the next sub-tile's scores already accumulated on the old one."""
    w = k2("dual-sharp", B=1, T=600, H=100, seed=66)
    assert work_items(w) > 256
    say(f"[dual] sharp softmax q x {qmul}")
    inp = workloads.make_inputs(w)
    inp["q"] = (inp["q"].float() * qmul).to(torch.bfloat16)
    out = run(w, inp)
    assert torch.isfinite(out.float()).all()
    assert_close(f64(out.cpu()), O.prefill(w, inp), f"dual sharp softmax q x {qmul}")


def test_dual_causality_bitwise():
    """Perturbing every input after row t0 leaves rows 0..t0 bit-identical,
    and the kernel is deterministic run to run."""
    w = k2("dual-causal", B=1, T=600, H=120, seed=67)
    assert work_items(w) > 256
    inp = workloads.make_inputs(w)
    a = run(w, inp)
    t0 = 300
    pert = {k: v.clone() for k, v in inp.items()}
    pert["q"][:, :, t0 + 1:] = -pert["q"][:, :, t0 + 1:]
    pert["latent"][:, t0 + 1:] *= 3
    pert["k_pe"][:, t0 + 1:] += 1
    b = run(w, pert)
    assert torch.equal(a[:, :, :t0 + 1], b[:, :, :t0 + 1])
    assert not torch.equal(a[:, :, t0 + 1:], b[:, :, t0 + 1:])
    assert torch.equal(a, run(w, inp))


def test_dual_chunked():
    """Chunked prefill through the two-block kernel: chunks of 512 and 388
    rows (130 heads: 260 work items each) after 0 and 513 cached rows, and a
    one-row chunk between them (a single round: the 8-wave kernel), against
    the oracle's one-shot rows and LSE."""
    w = k2("dual-chunked", B=1, T=901, H=130, seed=68)
    chunks = [512, 1, 388]
    say(f"[dual] chunked {chunks}")
    inp = workloads.make_inputs(w)
    g = to_gpu(inp)
    tab = table(w)
    cache = pipeline.alloc_chunk_cache(w.B, w.H, w.T, w.Dn, w.Dr, w.Dv)
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
    out, lse = torch.cat(outs, 2).cpu(), torch.cat(lses, 2).cpu()
    parts = O.prefill_parts(w, inp)
    ref = np.empty((w.B, w.H, w.T, w.Dv))
    ref_lse = np.empty((w.B, w.H, w.T))
    for h in range(w.H):
        ref[0, h], ref_lse[0, h] = O.prefill_head(w, parts, 0, h, return_lse=True)
    assert_close(f64(out), ref, "dual chunked output")
    ma, _ = errors(f64(lse), ref_lse)
    assert ma < 2e-2
