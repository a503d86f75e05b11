"""Scalar pure-Python evaluation of the whole prefill/decode path, for tiny
shapes only.

TEST INFRASTRUCTURE ONLY. It uses nothing but the standard library (no
numpy) and loops over every index, so that the vectorised oracle's reshapes,
transposes and broadcasts can be checked against an index-by-index
evaluation of the same definitions (equation page "Read the equation";
Kimi-K2 "Query content heads", section "Join query parts"; Kimi-K2 "RoPE
coefficients", section "Generate RoPE coefficients").
"""

from __future__ import annotations

import math


def _flat(t):
    """bf16/fp32 torch tensor -> nested Python lists of floats (exact); nested
    lists pass through unchanged."""
    if isinstance(t, list):
        return t
    return t.detach().float().tolist()


def inv_freq(spec, dim):
    out = []
    half = dim // 2
    if spec.kind == "yarn":
        def cdim(nrot):
            return dim * math.log(spec.original_max_pos / (nrot * 2 * math.pi)) / (2 * math.log(spec.base))
        lo = max(math.floor(cdim(spec.beta_fast)), 0)
        hi = min(math.ceil(cdim(spec.beta_slow)), dim - 1)
        lo, hi = float(lo), float(hi)
        if lo == hi:
            hi += 0.001
    for i in range(half):
        theta = spec.base ** (-(2.0 * i) / dim)
        if spec.kind == "default":
            out.append(theta)
        else:
            r = min(max((i - lo) / (hi - lo), 0.0), 1.0)
            # r = 0: keep theta (extrapolate); r = 1: theta / factor (interpolate)
            out.append(theta * (1.0 - r) + (theta / spec.factor) * r)
    return out


def mscale_ratio(spec):
    if spec.kind == "default":
        return 1.0

    def g(s, m):
        return 1.0 if s <= 1 else 0.1 * m * math.log(s) + 1.0
    return g(spec.factor, spec.mscale) / g(spec.factor, spec.mscale_all_dim)


def scale_of(spec, dqk):
    s = 1.0 / math.sqrt(dqk)
    if spec.kind != "default" and spec.mscale_all_dim:
        g = 0.1 * spec.mscale_all_dim * math.log(spec.factor) + 1.0 if spec.factor > 1 else 1.0
        s *= g * g
    return s


def rot(x, p, freqs, m, pairing):
    d = len(x)
    h = d // 2
    y = [0.0] * d
    for i in range(h):
        c = m * math.cos(p * freqs[i])
        s = m * math.sin(p * freqs[i])
        if pairing == "half":
            ia, ib = i, i + h
        else:
            ia, ib = 2 * i, 2 * i + 1
        y[ia] = x[ia] * c - x[ib] * s
        y[ib] = x[ib] * c + x[ia] * s
    return y


def _norm_row(row, gain, eps):
    ms = sum(v * v for v in row) / len(row)
    r = 1.0 / math.sqrt(ms + eps)
    return [gain[i] * row[i] * r for i in range(len(row))]


def _expand_token(cn, Wl, H, Dn, Dv):
    """k_nope[h][j], v[h][j] for one token: row h*(Dn+Dv)+j of W dotted with cn."""
    R = len(cn)
    kn, vv = [], []
    for h in range(H):
        krow, vrow = [], []
        for j in range(Dn + Dv):
            wr = Wl[h * (Dn + Dv) + j]
            acc = 0.0
            for r in range(R):
                acc += wr[r] * cn[r]
            (krow if j < Dn else vrow).append(acc)
        kn.append(krow)
        vv.append(vrow)
    return kn, vv


def _attend(qrow, keys, vals, scale):
    scores = []
    for k in keys:
        scores.append(scale * sum(qrow[d] * k[d] for d in range(len(qrow))))
    mx = max(scores)
    e = [math.exp(s - mx) for s in scores]
    z = sum(e)
    dv = len(vals[0])
    return [sum(e[s] * vals[s][j] for s in range(len(vals))) / z for j in range(dv)]


def prefill(w, inp):
    """O[b][h][t][j] for a tiny prefill workload, by scalar loops."""
    q, lat, kpe = _flat(inp["q"]), _flat(inp["latent"]), _flat(inp["k_pe"])
    gain, Wl = _flat(inp["gain"]), _flat(inp["W"])
    freqs = inv_freq(w.rope, w.Dr)
    m = mscale_ratio(w.rope)
    scale = scale_of(w.rope, w.Dqk)
    out = []
    for b in range(w.B):
        kn_t, v_t, kpe_t = [], [], []
        for t in range(w.T):
            cn = _norm_row(lat[b][t], gain, w.eps)
            kn, vv = _expand_token(cn, Wl, w.H, w.Dn, w.Dv)
            kn_t.append(kn)
            v_t.append(vv)
            kpe_t.append(rot(kpe[b][t], t, freqs, m, w.pairing))
        ob = []
        for h in range(w.H):
            oh = []
            for t in range(w.T):
                qrow = q[b][h][t][:w.Dn] + rot(q[b][h][t][w.Dn:], t, freqs, m, w.pairing)
                keys = [kn_t[s][h] + kpe_t[s] for s in range(t + 1)]
                vals = [v_t[s][h] for s in range(t + 1)]
                oh.append(_attend(qrow, keys, vals, scale))
            ob.append(oh)
        out.append(ob)
    return out


def decode(w, inp):
    """O[b][h][0][j] for a tiny decode workload, by scalar loops."""
    q, lat, kpe = _flat(inp["q"]), _flat(inp["latent"]), _flat(inp["k_pe"])
    gain, Wl = _flat(inp["gain"]), _flat(inp["W"])
    kc, vc = _flat(inp["k_cache"]), _flat(inp["v_cache"])
    freqs = inv_freq(w.rope, w.Dr)
    m = mscale_ratio(w.rope)
    scale = scale_of(w.rope, w.Dqk)
    p = w.q_pos
    out = []
    for b in range(w.B):
        cn = _norm_row(lat[b][0], gain, w.eps)
        kn, vv = _expand_token(cn, Wl, w.H, w.Dn, w.Dv)
        kr = rot(kpe[b][0], p, freqs, m, w.pairing)
        ob = []
        for h in range(w.H):
            keys = [list(kc[b][h][s]) for s in range(w.cache_len)]
            vals = [list(vc[b][h][s]) for s in range(w.cache_len)]
            keys[p] = kn[h] + kr
            vals[p] = vv[h]
            visible = [s for s in range(w.cache_len) if s <= p]
            qrow = q[b][h][0][:w.Dn] + rot(q[b][h][0][w.Dn:], p, freqs, m, w.pairing)
            ob.append([_attend(qrow, [keys[s] for s in visible], [vals[s] for s in visible], scale)])
        out.append(ob)
    return out


def decode_latent(w, inp, q_pos=None):
    """O[b][h][0][j] for a tiny decode workload with a compressed-latent
    cache, by scalar loops: the new token's row q_pos[b] of the cache takes
    its normalised latent and rotated rotary key, every row 0..q_pos[b] is
    expanded by kv_b_proj, and the query attends to those rows."""
    q, lat, kpe = _flat(inp["q"]), _flat(inp["latent"]), _flat(inp["k_pe"])
    gain, Wl = _flat(inp["gain"]), _flat(inp["W"])
    cache = _flat(inp["latent_cache"])
    freqs = inv_freq(w.rope, w.Dr)
    m = mscale_ratio(w.rope)
    scale = scale_of(w.rope, w.Dqk)
    out = []
    for b in range(w.B):
        p = w.q_pos if q_pos is None else int(q_pos[b])
        rows = [list(cache[b][s]) for s in range(p + 1)]
        rows[p] = _norm_row(lat[b][0], gain, w.eps) + rot(kpe[b][0], p, freqs, m, w.pairing)
        expanded = [_expand_token(r[:w.R], Wl, w.H, w.Dn, w.Dv) for r in rows]
        ob = []
        for h in range(w.H):
            keys = [expanded[s][0][h] + rows[s][w.R:] for s in range(p + 1)]
            vals = [expanded[s][1][h] for s in range(p + 1)]
            qrow = q[b][h][0][:w.Dn] + rot(q[b][h][0][w.Dn:], p, freqs, m, w.pairing)
            ob.append([_attend(qrow, keys, vals, scale)])
        out.append(ob)
    return out


def _matvec(row, Wl):
    """[sum_k row[k] * Wl[n][k] for each n] (nn.Linear on one row)."""
    return [sum(row[k] * wn[k] for k in range(len(row))) for wn in Wl]


def block_forward(w, inp):
    """out[b][t][j] for a tiny block workload, by scalar loops: the
    projections of every token, then `prefill` on them, then o_proj."""
    h = _flat(inp["hidden"])
    Wqa, gq, Wqb = _flat(inp["W_qa"]), _flat(inp["gain_q"]), _flat(inp["W_qb"])
    Wkva, Wo = _flat(inp["W_kva"]), _flat(inp["W_o"])
    q = [[[None] * w.T for _ in range(w.H)] for _ in range(w.B)]
    lat, kpe = [], []
    for b in range(w.B):
        lb, kb = [], []
        for t in range(w.T):
            qa = _norm_row(_matvec(h[b][t], Wqa), gq, w.eps)
            qt = _matvec(qa, Wqb)
            for hh in range(w.H):
                q[b][hh][t] = qt[hh * w.Dqk:(hh + 1) * w.Dqk]
            kv = _matvec(h[b][t], Wkva)
            lb.append(kv[:w.R])
            kb.append(kv[w.R:])
        lat.append(lb)
        kpe.append(kb)
    O = prefill(w, {"q": q, "latent": lat, "k_pe": kpe, "gain": _flat(inp["gain"]), "W": _flat(inp["W"])})
    out = []
    for b in range(w.B):
        ob = []
        for t in range(w.T):
            x = [O[b][hh][t][j] for hh in range(w.H) for j in range(w.Dv)]
            ob.append(_matvec(x, Wo))
        out.append(ob)
    return out
