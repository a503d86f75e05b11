"""Pins for the oracle's RMSNorm, kv_b_proj expansion, attention and whole
path: invariants, closed forms, an independent library routine (scipy), the
absorbed form the equation page contrasts with the eager one, and scalar
brute force on tiny shapes."""

import dataclasses

import numpy as np
import pytest
import scipy.special
import torch

import workloads
from oracle import brute
from oracle import mla_oracle as O


# ---------------------------------------------------------------- RMSNorm

def test_rmsnorm_unit_mean_square():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 512)) * rng.uniform(0.1, 10, size=(7, 1))
    y = O.rmsnorm(x, np.ones(512), eps=0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)


def test_rmsnorm_closed_forms():
    # constant row c: y = g * c / sqrt(c^2 + eps)
    g = np.linspace(0.5, 1.5, 64)
    for c in (0.3, -2.0, 1e-4):
        y = O.rmsnorm(np.full((1, 64), c), g, eps=1e-6)
        np.testing.assert_allclose(y[0], g * c / np.sqrt(c * c + 1e-6), rtol=1e-14)
    # one non-zero entry a at index k in a row of n: y_k = g_k * a / sqrt(a^2/n + eps)
    x = np.zeros((1, 64))
    x[0, 5] = 3.0
    y = O.rmsnorm(x, g, eps=1e-6)
    assert y[0, 5] == pytest.approx(g[5] * 3.0 / np.sqrt(9.0 / 64 + 1e-6), rel=1e-14)
    assert np.count_nonzero(y) == 1
    # scale invariance as eps/alpha^2 -> 0
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 64))
    np.testing.assert_allclose(O.rmsnorm(1e4 * x, g, 1e-6), O.rmsnorm(x, g, 0.0), rtol=1e-12)


# ---------------------------------------------------------------- expansion

def test_kv_expand_index_map():
    # W row n = h*(Dn+Dv)+j holds the value n*1000 + r in column r. With a
    # one-hot latent e_r at token t, k_nope[b,h,t,j] = W[h*(Dn+Dv)+j, r] and
    # v[b,h,t,j] = W[h*(Dn+Dv)+Dn+j, r]: the view-into-heads then split of
    # the equation page, checked element by element.
    B, T, H, R, Dn, Dv = 2, 3, 3, 5, 4, 2
    W = np.array([[n * 1000 + r for r in range(R)] for n in range(H * (Dn + Dv))], dtype=np.float64)
    c = np.zeros((B, T, R))
    for b in range(B):
        for t in range(T):
            c[b, t, (b * T + t) % R] = 1.0
    kn, v = O.kv_expand(c, W, H, Dn, Dv)
    assert kn.shape == (B, H, T, Dn) and v.shape == (B, H, T, Dv)
    for b in range(B):
        for t in range(T):
            r = (b * T + t) % R
            for h in range(H):
                for j in range(Dn):
                    assert kn[b, h, t, j] == (h * (Dn + Dv) + j) * 1000 + r
                for j in range(Dv):
                    assert v[b, h, t, j] == (h * (Dn + Dv) + Dn + j) * 1000 + r


# ---------------------------------------------------------------- attention

def _rand_qkv(seed, T=40, D=24, Dv=12):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, D)), rng.standard_normal((T, D)), rng.standard_normal((T, Dv))


def test_attention_matches_scipy_softmax():
    Q, K, V = _rand_qkv(0)
    pos = np.arange(40)
    S = 0.3 * Q @ K.T
    S[np.triu_indices(40, 1)] = -np.inf
    expect = scipy.special.softmax(S, axis=1) @ V
    np.testing.assert_allclose(O.attention(Q, K, V, 0.3, pos, pos, block=7), expect, rtol=1e-12, atol=1e-13)


def test_attention_invariants():
    Q, K, V = _rand_qkv(1)
    pos = np.arange(40)
    out = O.attention(Q, K, V, 0.5, pos, pos)
    # row 0 sees only key 0
    np.testing.assert_allclose(out[0], V[0], rtol=1e-15)
    # rows of P sum to one: V = 1 gives 1
    ones = O.attention(Q, K, np.ones_like(V), 0.5, pos, pos)
    np.testing.assert_allclose(ones, 1.0, rtol=1e-13)
    # q = 0: uniform weights over the visible prefix -> prefix mean
    z = O.attention(np.zeros_like(Q), K, V, 0.5, pos, pos)
    np.testing.assert_allclose(z, np.cumsum(V, 0) / np.arange(1, 41)[:, None], rtol=1e-12, atol=1e-14)
    # a shift u added to every key changes row t's scores by a constant
    u = np.random.default_rng(9).standard_normal(24)
    np.testing.assert_allclose(O.attention(Q, K + u, V, 0.5, pos, pos), out, rtol=1e-10, atol=1e-12)


def test_attention_causality_exact():
    Q, K, V = _rand_qkv(2)
    pos = np.arange(40)
    out = O.attention(Q, K, V, 0.5, pos, pos)
    t = 17
    K2, V2, Q2 = K.copy(), V.copy(), Q.copy()
    K2[t + 1:] += 5.0
    V2[t + 1:] -= 3.0
    Q2[t + 1:] *= 2.0
    out2 = O.attention(Q2, K2, V2, 0.5, pos, pos)
    np.testing.assert_array_equal(out2[:t + 1], out[:t + 1])
    assert not np.allclose(out2[t + 1:], out[t + 1:])


# ---------------------------------------------------------------- whole path

TINY_CASES = [
    workloads.WORKLOADS["tiny"],
    workloads.custom(B=2, T=7, H=2, R=16, Dn=8, Dr=4, Dv=6, seed=5),
    workloads.custom(B=1, T=5, H=2, R=8, Dn=4, Dr=6, Dv=4, seed=6, pairing="interleaved"),
    workloads.custom(B=1, T=8, H=1, R=8, Dn=4, Dr=8, Dv=4, seed=7, rope=workloads.YARN_KIMI),
    workloads.custom(B=2, T=6, H=2, R=8, Dn=2, Dr=8, Dv=2, seed=8, pairing="interleaved",
                     rope=workloads.RopeSpec(kind="yarn", base=10000.0, factor=8.0, original_max_pos=16,
                                             beta_fast=4.0, beta_slow=0.5, mscale=0.7, mscale_all_dim=0.9)),
]


@pytest.mark.parametrize("w", TINY_CASES, ids=lambda w: f"{w.name}-T{w.T}-{w.pairing}-{w.rope.kind}")
def test_prefill_matches_brute_force(w):
    inp = workloads.make_inputs(w)
    ref = np.array(brute.prefill(w, inp))
    np.testing.assert_allclose(O.prefill(w, inp), ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("w", TINY_CASES, ids=lambda w: f"{w.name}-T{w.T}-{w.pairing}-{w.rope.kind}")
def test_eager_equals_absorbed_tiny(w):
    inp = workloads.make_inputs(w)
    e = O.prefill(w, inp)
    a = O.prefill_absorbed(w, inp)
    np.testing.assert_allclose(a, e, rtol=1e-10, atol=1e-11)


def test_eager_equals_absorbed_kimi_1k_heads():
    # the 1k-token Kimi-K2 workload, restricted to 4 heads to keep it quick
    w = dataclasses.replace(workloads.WORKLOADS["kimi_k2_1k"], H=4)
    inp = workloads.make_inputs(w)
    e = O.prefill(w, inp)
    a = O.prefill_absorbed(w, inp)
    rel = np.linalg.norm(a - e) / np.linalg.norm(e)
    assert rel < 1e-10


def _tiny_decode(seed, L=9, q_pos=8, pairing="half", rope=workloads.YARN_KIMI):
    return workloads.custom(name="tinydec", B=2, T=1, H=2, R=16, Dn=8, Dr=4, Dv=6, seed=seed,
                            decode=True, cache_len=L, q_pos=q_pos, pairing=pairing, rope=rope)


@pytest.mark.parametrize("args", [dict(seed=11), dict(seed=12, L=12, q_pos=7, pairing="interleaved")])
def test_decode_matches_brute_force(args):
    w = _tiny_decode(**args)
    inp = workloads.make_inputs(w)
    np.testing.assert_allclose(O.decode(w, inp), np.array(brute.decode(w, inp)), rtol=1e-11, atol=1e-12)


def test_decode_equals_prefill_last_row():
    # When the cache holds exactly what a prefill over the same tokens would
    # produce, the decode step at the last position equals the prefill's last
    # row: the expanded-cache append composes with full attention.
    T = 10
    wp = workloads.custom(B=1, T=T, H=2, R=16, Dn=8, Dr=4, Dv=6, seed=21, rope=workloads.YARN_KIMI)
    inp = workloads.make_inputs(wp)
    ref = O.prefill(wp, inp)
    parts = O.prefill_parts(wp, inp)
    wd = dataclasses.replace(wp, T=1, decode=True, cache_len=T, q_pos=T - 1)
    k_cache = np.concatenate([parts["k_nope"], np.broadcast_to(parts["k_pe"][:, None], (1, 2, T, 4))], -1)
    dinp = {
        "q": inp["q"][:, :, T - 1:T], "latent": inp["latent"][:, T - 1:T], "k_pe": inp["k_pe"][:, T - 1:T],
        "gain": inp["gain"], "W": inp["W"],
        "k_cache": torch.from_numpy(k_cache.copy()), "v_cache": torch.from_numpy(parts["v"].copy()),
    }
    # cache rows 0..T-2 come from the prefill; slot T-1 is overwritten by the step
    dinp["k_cache"][:, :, T - 1] = 123.0
    dinp["v_cache"][:, :, T - 1] = -7.0
    out = O.decode(wd, dinp)
    np.testing.assert_allclose(out[:, :, 0], ref[:, :, T - 1], rtol=1e-12, atol=1e-13)


def test_generator_reproducible():
    w = workloads.WORKLOADS["tiny"]
    a = workloads.make_inputs(w)
    b = workloads.make_inputs(w)
    for k in a:
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16))
        assert a[k].dtype == torch.bfloat16
    # distribution sanity: W std ~ 1/sqrt(R), gain mean ~ 1
    w2 = workloads.WORKLOADS["kimi_k2_1k"]
    x = workloads.make_inputs(w2)
    assert abs(float(x["W"].float().std()) - 512 ** -0.5) < 1e-3
    assert abs(float(x["gain"].float().mean()) - 1.0) < 0.05
    assert abs(float(x["gain"].float().std()) - 0.1 ** 0.5) < 0.03


# ---- decode against a compressed-latent cache (normalised latent + rotated
# rotary key per token, re-expanded on every call)

def _tiny_latent(seed, L=9, q_pos=8, pairing="half", rope=workloads.YARN_KIMI, B=2):
    return workloads.custom(name="tinylat", B=B, T=1, H=2, R=16, Dn=8, Dr=4, Dv=6, seed=seed, decode=True,
                            cache_len=L, q_pos=q_pos, pairing=pairing, rope=rope, latent_cache=True)


@pytest.mark.parametrize("args,q_pos", [
    (dict(seed=31), None),
    (dict(seed=32, L=12, q_pos=11, pairing="interleaved"), None),
    (dict(seed=33, L=10, q_pos=9, B=3), [0, 4, 9]),  # ragged: one sequence sees only its new row
])
def test_decode_latent_matches_brute_force(args, q_pos):
    w = _tiny_latent(**args)
    inp = workloads.make_inputs(w)
    assert inp["latent_cache"].dtype == torch.float16
    np.testing.assert_allclose(O.decode_latent(w, inp, q_pos=q_pos), np.array(brute.decode_latent(w, inp, q_pos)),
                               rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("q_pos", [None, [36, 0, 17]])
def test_decode_latent_equals_absorbed(q_pos):
    w = workloads.WORKLOADS["tiny_decode_latent"]
    inp = workloads.make_inputs(w)
    e = O.decode_latent(w, inp, q_pos=q_pos)
    a = O.decode_latent_absorbed(w, inp, q_pos=q_pos)
    np.testing.assert_allclose(a, e, rtol=1e-10, atol=1e-12)


def test_decode_latent_single_row_closed_form():
    # A query at position 0 sees only its own row: softmax of one score is 1,
    # so the output is that row's value, W_uv times the normalised latent.
    w = _tiny_latent(seed=34, L=5, q_pos=4)
    inp = workloads.make_inputs(w)
    out = O.decode_latent(w, inp, q_pos=[0, 0])
    c = O.rmsnorm(inp["latent"].double().numpy(), inp["gain"].double().numpy(), w.eps)[:, 0]  # [B,R]
    Wv = inp["W"].double().numpy().reshape(w.H, w.Dn + w.Dv, w.R)[:, w.Dn:]  # [H,Dv,R]
    ref = np.einsum("hjr,br->bhj", Wv, c)
    np.testing.assert_allclose(out[:, :, 0], ref, rtol=1e-12, atol=1e-13)


def test_decode_latent_equals_expanded_cache_decode():
    # Expanding every cached latent row into per-head keys/values (with the
    # shared rotated rotary key broadcast) and running the expanded-cache
    # decode gives the same output.
    w = _tiny_latent(seed=35, L=11, q_pos=10)
    inp = workloads.make_inputs(w)
    cache = inp["latent_cache"].double().numpy()
    k_nope, v = O.kv_expand(cache[:, :, :w.R], inp["W"].double().numpy(), w.H, w.Dn, w.Dv)
    k_cache = np.concatenate([k_nope, np.broadcast_to(cache[:, None, :, w.R:], k_nope.shape[:3] + (w.Dr,))], -1)
    wd = dataclasses.replace(w, latent_cache=False)
    dinp = {k: inp[k] for k in ("q", "latent", "k_pe", "gain", "W")}
    dinp["k_cache"] = torch.from_numpy(k_cache.copy())
    dinp["v_cache"] = torch.from_numpy(v.copy())
    np.testing.assert_allclose(O.decode_latent(w, inp), O.decode(wd, dinp), rtol=1e-12, atol=1e-13)


def test_decode_latent_equals_prefill_last_row():
    # A latent cache filled with what a prefill over the same tokens
    # normalises and rotates gives, at the last position, the prefill's last
    # output row.
    T = 9
    wp = workloads.custom(B=2, T=T, H=2, R=16, Dn=8, Dr=4, Dv=6, seed=36, rope=workloads.YARN_KIMI)
    inp = workloads.make_inputs(wp)
    ref = O.prefill(wp, inp)
    parts = O.prefill_parts(wp, inp)
    wd = dataclasses.replace(wp, T=1, decode=True, cache_len=T, q_pos=T - 1, latent_cache=True)
    cache = np.concatenate([parts["c_norm"], parts["k_pe"]], -1)
    cache[:, T - 1] = 99.0  # slot T-1 is overwritten by the step
    dinp = {"q": inp["q"][:, :, T - 1:T], "latent": inp["latent"][:, T - 1:T], "k_pe": inp["k_pe"][:, T - 1:T],
            "gain": inp["gain"], "W": inp["W"], "latent_cache": torch.from_numpy(cache)}
    out = O.decode_latent(wd, dinp)
    np.testing.assert_allclose(out[:, :, 0], ref[:, :, T - 1], rtol=1e-12, atol=1e-13)


# ---- the whole attention block (projections around the path)

def test_block_matches_brute_force():
    w = dataclasses.replace(workloads.WORKLOADS["tiny_block"], T=9, B=2)
    inp = workloads.make_inputs(w)
    assert inp["hidden"].dtype == torch.bfloat16 and "q" not in inp
    np.testing.assert_allclose(O.block_forward(w, inp), np.array(brute.block_forward(w, inp)), rtol=1e-10,
                               atol=1e-12)


def test_block_rows_and_inputs():
    w = workloads.WORKLOADS["tiny_block"]
    inp = workloads.make_inputs(w)
    full = O.block_forward(w, inp)
    assert full.shape == (w.B, w.T, w.hidden)
    rows = [0, 7, 39]
    np.testing.assert_allclose(O.block_forward(w, inp, rows=rows), full[:, rows], rtol=1e-13, atol=1e-14)
    # the path's inputs come out at the scales the other workloads draw
    bi = O.block_inputs(w, inp)
    assert bi["q"].shape == (w.B, w.H, w.T, w.Dqk) and bi["latent"].shape == (w.B, w.T, w.R)
    assert 0.5 < np.std(bi["q"]) < 2.0 and 0.5 < np.std(bi["latent"]) < 2.0
