"""fp64 numpy oracle of the eager multi-head latent attention forward path.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Every function takes and returns numpy float64 arrays (inputs are the bf16
tensors the GPU receives, widened exactly). There is no intermediate
rounding anywhere. Citations name the page and the section or code excerpt
each step follows:

  [K2-rope]   Kimi-K2 "RoPE coefficients", section "Generate RoPE
              coefficients" (the yarn helper functions, the YaRN cache
              builder, the YaRN class defaults, the softmax-scale rule and the
              RoPE dispatch).
  [K2-query]  Kimi-K2 "Query content heads", sections "Split content heads"
              and "Join query parts" (query view/split, rotary application,
              nope|rope concatenation, scaled scores, causal mask, fp32
              softmax, value mix, cache update).
  [eq]        The equation page "Read the equation" with its "Original
              context" (latent RMSNorm, kv_b_proj, view into heads, split
              into non-rotary key and value; contrast with the absorbed path).
  [GLM-kv]    GLM-5 "Normalized key-value latent", section "Key-value
              compression" (RMSNorm default epsilon 1e-6, kv_b_proj shape,
              expand_kv, shared rotary key broadcast to all heads, softmax
              scale 1/sqrt(256) under default RoPE) and section "KV cache"
              (per token the cache keeps the normalised latent and the
              rotated rotary key, and re-expands them on every call).

Readings of points the pages leave open are listed beside the functions that
take them (RMSNorm body, rotation pairing and sign, default RoPE body).
"""

from __future__ import annotations

import math
from typing import Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Rotary coefficients [K2-rope]
# ---------------------------------------------------------------------------


def yarn_correction_dim(num_rotations: float, dim: int, base: float, max_pos: int) -> float:
    """Rotary dimension index at which a pair turns `num_rotations` times over
    `max_pos` positions [K2-rope, yarn_find_correction_dim]."""
    return (dim * math.log(max_pos / (num_rotations * 2.0 * math.pi))) / (2.0 * math.log(base))


def yarn_correction_range(beta_fast: float, beta_slow: float, dim: int, base: float,
                          max_pos: int) -> Tuple[int, int]:
    """Integer band [low, high] of pairs that YaRN interpolates, floor of the
    fast bound and ceiling of the slow bound, clamped to [0, dim-1]
    [K2-rope, yarn_find_correction_range]. The clamp uses the full rotary
    width dim-1 as printed, although the ramp only has dim/2 entries."""
    low = math.floor(yarn_correction_dim(beta_fast, dim, base, max_pos))
    high = math.ceil(yarn_correction_dim(beta_slow, dim, base, max_pos))
    return max(low, 0), min(high, dim - 1)


def yarn_get_mscale(scale: float, mscale: float) -> float:
    """Attention magnitude correction: 1 when not scaled, else
    0.1*mscale*ln(scale)+1 [K2-rope, yarn_get_mscale; GLM-kv mla-init]."""
    if scale <= 1:
        return 1.0
    return 0.1 * mscale * math.log(scale) + 1.0


def yarn_linear_ramp(low: float, high: float, n: int) -> np.ndarray:
    """Ramp over pair indices 0..n-1, rising linearly from 0 at `low` to 1 at
    `high` and clamped to [0, 1]; a degenerate band is widened by 0.001
    [K2-rope, yarn_linear_ramp_mask]."""
    low = float(low)
    high = float(high)
    if low == high:
        high += 0.001
    r = (np.arange(n, dtype=np.float64) - low) / (high - low)
    return np.clip(r, 0.0, 1.0)


def rope_base_freqs(base: float, dim: int) -> np.ndarray:
    """theta_i = base^(-2i/dim) for pair i = 0..dim/2-1: the unscaled rotary
    frequencies (freq_extra of [K2-rope, _set_cos_sin_cache]; the body of the
    plain rotary class is elided on the pages and is read as these)."""
    i = np.arange(0, dim, 2, dtype=np.float64)
    return 1.0 / (base ** (i / dim))


def rope_inv_freq(spec, dim: int) -> np.ndarray:
    """Per-pair angular frequency [dim/2].

    Default RoPE: theta_i. YaRN [K2-rope, _set_cos_sin_cache]: each pair's
    frequency moves from the unscaled theta_i towards the interpolated
    theta_i/factor by the fraction r_i = ramp(low, high) of the way:
    theta_i + (theta_i/factor - theta_i) * r_i. Pairs below the band
    (r = 0) keep theta_i, pairs above it (r = 1) take theta_i/factor."""
    theta = rope_base_freqs(spec.base, dim)
    if spec.kind == "default":
        return theta
    if spec.kind != "yarn":
        raise ValueError(f"Unknown RoPE scaling type {spec.kind}")
    low, high = yarn_correction_range(spec.beta_fast, spec.beta_slow, dim, spec.base,
                                      spec.original_max_pos)
    r = yarn_linear_ramp(low, high, dim // 2)
    return theta + (theta / spec.factor - theta) * r


def rope_table_mscale(spec) -> float:
    """Multiplier applied to the cos/sin table: the ratio of the two YaRN
    corrections (mscale over mscale_all_dim) [K2-rope, _set_cos_sin_cache];
    1 for default RoPE."""
    if spec.kind == "default":
        return 1.0
    if spec.kind != "yarn":
        raise ValueError(f"Unknown RoPE scaling type {spec.kind}")
    return yarn_get_mscale(spec.factor, spec.mscale) / yarn_get_mscale(spec.factor, spec.mscale_all_dim)


def rope_table(spec, dim: int, n_pos: int) -> Tuple[np.ndarray, np.ndarray]:
    """cos, sin tables [n_pos, dim/2]: m*cos(p*inv_freq_i), m*sin(p*inv_freq_i)
    for positions p = 0..n_pos-1 [K2-rope, _set_cos_sin_cache]. The pages store
    each pair's value twice (cat(freqs, freqs)); one copy per pair is kept."""
    inv = rope_inv_freq(spec, dim)
    m = rope_table_mscale(spec)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return m * np.cos(ang), m * np.sin(ang)


def softmax_scale(spec, qk_head_dim: int) -> float:
    """qk_head_dim^-0.5, times mscale(factor, mscale_all_dim)^2 when the RoPE is
    scaled and mscale_all_dim is non-zero [K2-rope softmax-scale rule;
    GLM-kv yarn_apply_mscale]."""
    s = qk_head_dim ** (-0.5)
    if spec.kind != "default" and spec.mscale_all_dim:
        g = yarn_get_mscale(spec.factor, spec.mscale_all_dim)
        s = s * g * g
    return s


# ---------------------------------------------------------------------------
# Latent RMSNorm and kv_b_proj [eq, GLM-kv]
# ---------------------------------------------------------------------------


def rmsnorm(x: np.ndarray, gain: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """gain * x / sqrt(mean(x^2) + eps) over the last axis. The module body is
    not printed; this is the standard RMSNorm with eps inside the root and
    default eps 1e-6 [GLM-kv, section text]."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return gain * (x / np.sqrt(ms + eps))


def kv_expand(c_norm: np.ndarray, W: np.ndarray, H: int, Dn: int, Dv: int
              ) -> Tuple[np.ndarray, np.ndarray]:
    """kv = c_norm @ W^T viewed [B, T, H, Dn+Dv], moved to head-major
    [B, H, T, Dn+Dv] and split into k_nope [.., Dn] and v [.., Dv] [eq,
    Original context; GLM-kv expand_kv]."""
    B, T, R = c_norm.shape
    kv = c_norm.reshape(B * T, R) @ W.T
    kv = kv.reshape(B, T, H, Dn + Dv).transpose(0, 2, 1, 3)
    return np.ascontiguousarray(kv[..., :Dn]), np.ascontiguousarray(kv[..., Dn:])


# ---------------------------------------------------------------------------
# Rotation [K2-query]
# ---------------------------------------------------------------------------


def rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, pairing: str) -> np.ndarray:
    """Rotate each pair (a, b) of the rotary part by the pair's angle:
    (a*cos - b*sin, b*cos + a*sin). `cos`/`sin` broadcast against x[..., :dim/2].

    pairing "half": pair i is (x[i], x[i + dim/2]) (rotate-half form, matching
    the cat(freqs, freqs) table layout of [K2-rope]); "interleaved": pair i is
    (x[2i], x[2i+1]) (GLM-5 calls an interleaved variant, GLM-kv "KV cache").
    The output keeps the input's element order."""
    d = x.shape[-1]
    h = d // 2
    out = np.empty_like(x)
    if pairing == "half":
        a, b = x[..., :h], x[..., h:]
        out[..., :h] = a * cos - b * sin
        out[..., h:] = b * cos + a * sin
    elif pairing == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * cos - b * sin
        out[..., 1::2] = b * cos + a * sin
    else:
        raise ValueError(f"unknown pairing {pairing}")
    return out


# ---------------------------------------------------------------------------
# Attention [K2-query]
# ---------------------------------------------------------------------------


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
              q_pos: np.ndarray, k_pos: np.ndarray, block: int = 1024,
              return_lse: bool = False):
    """Scaled, masked softmax attention for one (batch, head).

    Q [Tq, Dqk], K [Tk, Dqk], V [Tk, Dv]; q_pos [Tq], k_pos [Tk].
    S = scale * Q K^T, key s visible to query t iff k_pos[s] <= q_pos[t]
    (the additive causal mask with -inf for hidden keys), P = row softmax,
    O = P V [K2-query, Join query parts]. Queries are processed in blocks of
    `block` rows to bound memory; each block is the plain definition."""
    Tq = Q.shape[0]
    O = np.empty((Tq, V.shape[1]), dtype=np.float64)
    lse = np.empty((Tq,), dtype=np.float64)
    for t0 in range(0, Tq, block):
        t1 = min(Tq, t0 + block)
        S = scale * (Q[t0:t1] @ K.T)
        visible = k_pos[None, :] <= q_pos[t0:t1, None]
        S = np.where(visible, S, -np.inf)
        m = np.max(S, axis=1, keepdims=True)
        E = np.exp(S - m)
        z = np.sum(E, axis=1, keepdims=True)
        O[t0:t1] = (E / z) @ V
        lse[t0:t1] = (m + np.log(z))[:, 0]
    return (O, lse) if return_lse else O


# ---------------------------------------------------------------------------
# Whole path
# ---------------------------------------------------------------------------


def _f64(t) -> np.ndarray:
    """Widen a bf16/fp32 torch tensor or array exactly to float64."""
    if hasattr(t, "detach"):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def prefill_parts(w, inp: dict) -> dict:
    """Steps before attention for a prefill workload: normalised latent,
    k_nope, v, rotated q and rotated shared k_pe (all fp64)."""
    c = rmsnorm(_f64(inp["latent"]), _f64(inp["gain"]), w.eps)
    k_nope, v = kv_expand(c, _f64(inp["W"]), w.H, w.Dn, w.Dv)
    cos, sin = rope_table(w.rope, w.Dr, w.T)
    q = _f64(inp["q"])
    q_pe = rotate(q[..., w.Dn:], cos[None, None], sin[None, None], w.pairing)
    k_pe = rotate(_f64(inp["k_pe"]), cos[None], sin[None], w.pairing)
    return dict(c_norm=c, k_nope=k_nope, v=v, q_nope=q[..., :w.Dn], q_pe=q_pe, k_pe=k_pe,
                cos=cos, sin=sin)


def prefill_head(w, parts: dict, b: int, h: int, rows=None, return_lse: bool = False):
    """Attention output [len(rows), Dv] of head h of sequence b for the given
    query rows (default all), from `prefill_parts`. Positions are 0..T-1."""
    Q = np.concatenate([parts["q_nope"][b, h], parts["q_pe"][b, h]], axis=-1)
    K = np.concatenate([parts["k_nope"][b, h], parts["k_pe"][b]], axis=-1)
    V = parts["v"][b, h]
    pos = np.arange(w.T)
    if rows is None:
        rows = pos
    rows = np.asarray(rows)
    return attention(Q[rows], K, V, softmax_scale(w.rope, w.Dqk), pos[rows], pos,
                     return_lse=return_lse)


def prefill(w, inp: dict) -> np.ndarray:
    """Full prefill output O [B, H, T, Dv] in fp64."""
    parts = prefill_parts(w, inp)
    O = np.empty((w.B, w.H, w.T, w.Dv), dtype=np.float64)
    for b in range(w.B):
        for h in range(w.H):
            O[b, h] = prefill_head(w, parts, b, h)
    return O


def prefill_absorbed(w, inp: dict) -> np.ndarray:
    """The absorbed form the equation page contrasts with the eager one:
    W_uk folded into the non-rotary query, scores taken against the
    normalised latent, and W_uv applied to the latent aggregate [eq]. It is
    algebraically equal to `prefill`."""
    c = rmsnorm(_f64(inp["latent"]), _f64(inp["gain"]), w.eps)  # [B,T,R]
    W = _f64(inp["W"]).reshape(w.H, w.Dn + w.Dv, w.R)
    W_uk, W_uv = W[:, :w.Dn, :], W[:, w.Dn:, :]
    cos, sin = rope_table(w.rope, w.Dr, w.T)
    q = _f64(inp["q"])
    q_pe = rotate(q[..., w.Dn:], cos[None, None], sin[None, None], w.pairing)
    k_pe = rotate(_f64(inp["k_pe"]), cos[None], sin[None], w.pairing)
    scale = softmax_scale(w.rope, w.Dqk)
    pos = np.arange(w.T)
    visible = pos[None, :] <= pos[:, None]
    O = np.empty((w.B, w.H, w.T, w.Dv), dtype=np.float64)
    for b in range(w.B):
        for h in range(w.H):
            q_lat = q[b, h, :, :w.Dn] @ W_uk[h]  # [T, R]
            S = scale * (q_lat @ c[b].T + q_pe[b, h] @ k_pe[b].T)
            S = np.where(visible, S, -np.inf)
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            O[b, h] = (P @ c[b]) @ W_uv[h].T
    return O


def decode_parts(w, inp: dict, b_idx=None) -> dict:
    """Steps before attention for a decode workload: the new token's
    normalised latent, its expanded k_nope/v, the rotated q and k_pe at
    position q_pos. `b_idx` restricts to some sequences."""
    bs = slice(None) if b_idx is None else np.asarray(b_idx)
    c = rmsnorm(_f64(inp["latent"][bs]), _f64(inp["gain"]), w.eps)  # [b,1,R]
    k_nope, v = kv_expand(c, _f64(inp["W"]), w.H, w.Dn, w.Dv)  # [b,H,1,*]
    cos, sin = rope_table(w.rope, w.Dr, w.q_pos + 1)
    cp, sp = cos[w.q_pos], sin[w.q_pos]
    q = _f64(inp["q"][bs])
    q_pe = rotate(q[..., w.Dn:], cp, sp, w.pairing)
    k_pe = rotate(_f64(inp["k_pe"][bs]), cp, sp, w.pairing)  # [b,1,Dr]
    return dict(c_norm=c, k_nope=k_nope, v=v, q_nope=q[..., :w.Dn], q_pe=q_pe, k_pe=k_pe)


def decode_head(w, inp: dict, parts: dict, b: int, h: int, bi: int = None) -> np.ndarray:
    """Decode output [1, Dv] for sequence b, head h. The cache rows 0..L-1 are
    used as given except slot q_pos, which takes the new token's expanded key
    (non-rotary part from kv_b_proj, rotary part the rotated shared k_pe) and
    value, as the expanded-cache update appends them [K2-query, Join query
    parts]. Rows at positions <= q_pos are visible. `bi` indexes `parts` when
    it was built for a subset of sequences."""
    bi = b if bi is None else bi
    K = _f64(inp["k_cache"][b, h])
    V = _f64(inp["v_cache"][b, h])
    K[w.q_pos, :w.Dn] = parts["k_nope"][bi, h, 0]
    K[w.q_pos, w.Dn:] = parts["k_pe"][bi, 0]
    V[w.q_pos] = parts["v"][bi, h, 0]
    Q = np.concatenate([parts["q_nope"][bi, h], parts["q_pe"][bi, h]], axis=-1)  # [1,Dqk]
    k_pos = np.arange(w.cache_len)
    return attention(Q, K, V, softmax_scale(w.rope, w.Dqk), np.array([w.q_pos]), k_pos)


def decode(w, inp: dict) -> np.ndarray:
    """Full decode output O [B, H, 1, Dv] in fp64."""
    parts = decode_parts(w, inp)
    O = np.empty((w.B, w.H, 1, w.Dv), dtype=np.float64)
    for b in range(w.B):
        for h in range(w.H):
            O[b, h] = decode_head(w, inp, parts, b, h)
    return O


# ---------------------------------------------------------------------------
# Decode against a compressed-latent cache [eq], [GLM-kv]
# ---------------------------------------------------------------------------


def _latent_decode_setup(w, inp: dict, b_idx=None, q_pos=None):
    """The latent cache [b, L, R+Dr] after the decode step's update, the
    non-rotary query, the rotated rotary query and the query positions.

    The cache row of a token holds its normalised latent (R values) followed
    by its rotated shared rotary key (Dr values): what the GLM-5 page's
    "KV cache" section keeps per token instead of expanded keys and values.
    Rows other than the new token's are used as given. The new token of
    sequence b sits at position q_pos[b]: its latent is normalised and its
    rotary key rotated at that position, and both replace row q_pos[b]."""
    bs = slice(None) if b_idx is None else np.asarray(b_idx)
    cache = _f64(inp["latent_cache"][bs]).copy()
    nb = cache.shape[0]
    qp = np.full(nb, w.q_pos, dtype=np.int64) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    c_new = rmsnorm(_f64(inp["latent"][bs]), _f64(inp["gain"]), w.eps)  # [b,1,R]
    cos, sin = rope_table(w.rope, w.Dr, int(qp.max()) + 1)
    q = _f64(inp["q"][bs])
    q_pe = np.empty_like(q[..., w.Dn:])
    kpe = _f64(inp["k_pe"][bs])
    for i in range(nb):
        p = int(qp[i])
        q_pe[i] = rotate(q[i, :, :, w.Dn:], cos[p], sin[p], w.pairing)
        cache[i, p, :w.R] = c_new[i, 0]
        cache[i, p, w.R:] = rotate(kpe[i, 0], cos[p], sin[p], w.pairing)
    return cache, q[..., :w.Dn], q_pe, qp


def decode_latent(w, inp: dict, b_idx=None, q_pos=None) -> np.ndarray:
    """Decode output O [b, H, 1, Dv] against a compressed-latent cache, by
    the definition: every cached latent is expanded by kv_b_proj into
    per-head non-rotary keys and values [eq], each head's key is joined with
    the shared rotated rotary key [GLM-kv, expand_kv], and the query at
    position q_pos[b] attends to rows 0..q_pos[b] [K2-query]."""
    cache, q_nope, q_pe, qp = _latent_decode_setup(w, inp, b_idx, q_pos)
    W = _f64(inp["W"])
    scale = softmax_scale(w.rope, w.Dqk)
    O = np.empty((cache.shape[0], w.H, 1, w.Dv), dtype=np.float64)
    for i in range(cache.shape[0]):
        p = int(qp[i])
        rows = cache[i, :p + 1]
        k_nope, v = kv_expand(rows[None, :, :w.R], W, w.H, w.Dn, w.Dv)  # [1,H,p+1,*]
        pos = np.arange(p + 1)
        for h in range(w.H):
            K = np.concatenate([k_nope[0, h], rows[:, w.R:]], axis=-1)
            Q = np.concatenate([q_nope[i, h], q_pe[i, h]], axis=-1)
            O[i, h] = attention(Q, K, v[0, h], scale, np.array([p]), pos)
    return O


def decode_latent_absorbed(w, inp: dict, b_idx=None, q_pos=None) -> np.ndarray:
    """The same output by the absorbed form [eq]: W_uk folded into the
    non-rotary query, scores against the cached latent and rotary key, W_uv
    applied to the probability-weighted latent. Algebraically equal to
    `decode_latent`."""
    cache, q_nope, q_pe, qp = _latent_decode_setup(w, inp, b_idx, q_pos)
    W = _f64(inp["W"]).reshape(w.H, w.Dn + w.Dv, w.R)
    W_uk, W_uv = W[:, :w.Dn, :], W[:, w.Dn:, :]
    scale = softmax_scale(w.rope, w.Dqk)
    O = np.empty((cache.shape[0], w.H, 1, w.Dv), dtype=np.float64)
    for i in range(cache.shape[0]):
        p = int(qp[i])
        rows = cache[i, :p + 1]
        for h in range(w.H):
            q_lat = q_nope[i, h] @ W_uk[h]  # [1, R]
            s = scale * (q_lat @ rows[:, :w.R].T + q_pe[i, h] @ rows[:, w.R:].T)
            e = np.exp(s - s.max())
            P = e / e.sum()
            O[i, h] = (P @ rows[:, :w.R]) @ W_uv[h].T
    return O


# ---------------------------------------------------------------------------
# The whole attention block around the path [K2-query], [GLM-kv]
# ---------------------------------------------------------------------------


def block_inputs(w, inp: dict) -> dict:
    """The path's inputs from the block's hidden states: q =
    q_b_proj(q_a_layernorm(q_a_proj(h))) viewed [B, H, T, Dqk]; latent and
    shared rotary key = the two parts of kv_a_proj_with_mqa(h) [K2-query,
    "Split content heads" and the MLA constructor; GLM-kv, "Key-value
    compression"]. nn.Linear: y = x W^T; no biases."""
    h = _f64(inp["hidden"])
    kva = h @ _f64(inp["W_kva"]).T
    qa = rmsnorm(h @ _f64(inp["W_qa"]).T, _f64(inp["gain_q"]), w.eps)
    q = (qa @ _f64(inp["W_qb"]).T).reshape(w.B, w.T, w.H, w.Dqk).transpose(0, 2, 1, 3)
    return {"q": q, "latent": kva[..., :w.R], "k_pe": kva[..., w.R:], "gain": _f64(inp["gain"]),
            "W": _f64(inp["W"])}


def block_forward(w, inp: dict, rows=None) -> np.ndarray:
    """Block output [B, len(rows), hidden] (default all rows): the eager
    path on `block_inputs`, then o_proj on the heads' outputs concatenated
    per token (attn_output transposed to [B, T, H*Dv], then y = x W_o^T)."""
    parts = prefill_parts(w, block_inputs(w, inp))
    rows = np.arange(w.T) if rows is None else np.asarray(rows)
    O = np.empty((w.B, w.H, len(rows), w.Dv))
    for b in range(w.B):
        for h in range(w.H):
            O[b, h] = prefill_head(w, parts, b, h, rows=rows)
    x = O.transpose(0, 2, 1, 3).reshape(w.B, len(rows), w.H * w.Dv)
    return x @ _f64(inp["W_o"]).T
