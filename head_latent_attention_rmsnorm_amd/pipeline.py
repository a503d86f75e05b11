"""The whole forward path as a sequence of library calls (no arithmetic here).

prefill_forward: latent RMSNorm with the shared rotary key's rotation ->
kv_b_proj expansion -> causal attention with the query's rotation fused in
(Kimi-K2 "Query content heads", "Join query parts"; equation page "Read the
equation"); the cos/sin table is built once per length (build_table).
decode_step: latent RMSNorm of the new token -> kv_b_proj expansion appended
into the expanded cache with its rotated shared key -> split-K decode
attention (same sections, with the expanded-cache update).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import api


@dataclass
class RopeTable:
    cos: torch.Tensor
    sin: torch.Tensor
    scale: float  # softmax scale for the head width it was built for


def build_table(rope: api.RopeParams, n_pos: int, qk_head_dim: int, device="cuda") -> RopeTable:
    cos, sin, _ = api.mla_rope_table_build(rope, n_pos, device)
    return RopeTable(cos, sin, api.mla_softmax_scale(rope, qk_head_dim))


@dataclass
class PrefillBuffers:
    c_norm: torch.Tensor  # [B, T, R] fp16
    k_rot: torch.Tensor   # [B, T, Dr] fp16, the rotated shared rotary key
    k_nope: torch.Tensor  # [B, H, T, Dn] fp16
    v: torch.Tensor       # V^T [B, H, Dv, round8(T)] fp16
    out: torch.Tensor     # [B, H, T, Dv] bf16


def alloc_prefill(B, T, H, R, Dn, Dr, Dv, device="cuda") -> PrefillBuffers:
    """Intermediate buffers; the normalised latent, the rotated key, k_nope and
    v in fp16 (same size and MFMA rate as bf16 on gfx950, three more
    significant bits). The values are kept transposed (V^T), the layout the
    attention reads."""
    return PrefillBuffers(
        c_norm=torch.empty((B, T, R), dtype=torch.float16, device=device),
        k_rot=torch.empty((B, T, Dr), dtype=torch.float16, device=device),
        k_nope=torch.empty((B, H, T, Dn), dtype=torch.float16, device=device),
        v=torch.empty((B, H, Dv, api.round8(T)), dtype=torch.float16, device=device),
        out=torch.empty((B, H, T, Dv), dtype=torch.bfloat16, device=device),
    )


def prefill_forward(q, latent, k_pe, gain, W, table: RopeTable, Dn: int, Dv: int, pairing="half", eps: float = 1e-6,
                    bufs: Optional[PrefillBuffers] = None, return_lse: bool = False):
    """q [B,H,T,Dn+Dr], latent [B,T,R], k_pe [B,T,Dr], gain [R], W [H*(Dn+Dv),R]
    (all bf16 on the GPU) -> out [B,H,T,Dv] bf16. Three launches and the
    attention: latent RMSNorm with the key rotation, the two expansion
    launches, then the causal attention over the prepared operands."""
    B, H, T, _ = q.shape
    R = latent.shape[-1]
    Dr = k_pe.shape[-1]
    if bufs is None:
        bufs = alloc_prefill(B, T, H, R, Dn, Dr, Dv, q.device)
    api.mla_latent_prepare(latent, gain, eps, k_pe, table.cos, table.sin, pairing, c_norm=bufs.c_norm,
                           k_rot=bufs.k_rot)
    api.mla_kv_expand(bufs.c_norm, W, H, Dn, Dv, k=bufs.k_nope, v=bufs.v, v_layout="cols")
    return api.mla_prefill_attention_cached(q, bufs.k_nope, bufs.k_rot, bufs.v, 0, table.cos, table.sin, table.scale,
                                            pairing, return_lse=return_lse, out=bufs.out)


def decode_step(q, latent, k_pe, gain, W, k_cache, v_cache, seq_len, q_pos, slot: int, table: RopeTable, Dn: int,
                pairing="half", eps: float = 1e-6, num_splits: int = 0, c_norm=None, out=None, workspace=None):
    """One decode step: the new token (q [B,H,1,Dqk], latent [B,1,R], k_pe
    [B,1,Dr]) is normalised, expanded and appended at cache row `slot`
    (rotated at q_pos), then attends over seq_len[b] cached rows."""
    c_norm = api.mla_latent_rmsnorm(latent, gain, eps, out=c_norm)
    H = k_cache.shape[1]
    Dv = v_cache.shape[-1]
    api.mla_kv_expand(c_norm, W, H, Dn, Dv, k=k_cache, v=v_cache, t_off=slot, k_pe=k_pe, cos=table.cos,
                      sin=table.sin, pos=q_pos.view(-1, 1) if q_pos is not None else None, pairing=pairing)
    return api.mla_decode_attention(q, k_cache, v_cache, seq_len, q_pos, table.cos, table.sin, table.scale, Dn,
                                    pairing, num_splits, out=out, workspace=workspace)


def decode_latent_step(q, latent, k_pe, gain, W, w_ukt, cache, seq_len, q_pos, table: RopeTable, Dn: int, Dv: int,
                       pairing="half", eps: float = 1e-6, num_splits: int = 0, out=None, workspace=None,
                       method: str = "absorbed"):
    """One decode step against a latent cache [B, Lcap, R+Dr] fp16: the new
    token (q [B,H,1,Dqk], latent [B,1,R], k_pe [B,1,Dr]) is normalised and
    its rotary key rotated into cache row q_pos[b], then it attends over
    seq_len[b] rows, by the absorbed form (w_ukt from
    api.mla_absorb_prepare, once per weight) or, with method="expand", by
    re-expanding every cached row (w_ukt unused)."""
    B = latent.shape[0]
    api.mla_latent_cache_append(latent.view(B, -1), gain, k_pe.view(B, -1), table.cos, table.sin, q_pos, cache,
                                eps, pairing)
    if method == "expand":
        return api.mla_decode_latent_expanded(q, W, cache, seq_len, q_pos, table.cos, table.sin, table.scale, Dn, Dv,
                                              pairing, num_splits, out=out, workspace=workspace)
    if method != "absorbed":
        raise ValueError(f"method must be 'absorbed' or 'expand', not {method!r}")
    return api.mla_decode_absorbed(q, W, w_ukt, cache, seq_len, q_pos, table.cos, table.sin, table.scale, Dn, Dv,
                                   pairing, num_splits, out=out, workspace=workspace)


@dataclass
class ChunkCache:
    """Expanded cache for chunked prefill: k_nope [B, H, Tcap, Dn], the shared
    rotated rotary key [B, Tcap, Dr] and V^T [B, H, Dv, Tcap] (zero-filled,
    so columns past the filled rows stay finite)."""
    k_nope: torch.Tensor
    k_rot: torch.Tensor
    vt: torch.Tensor


def alloc_chunk_cache(B, H, Tcap, Dn, Dr, Dv, device="cuda", kv_dtype=torch.float16) -> ChunkCache:
    Tv = (Tcap + 7) // 8 * 8
    return ChunkCache(torch.zeros((B, H, Tcap, Dn), dtype=kv_dtype, device=device),
                      torch.zeros((B, Tcap, Dr), dtype=kv_dtype, device=device),
                      torch.zeros((B, H, Dv, Tv), dtype=kv_dtype, device=device))


def prefill_chunk(q, latent, k_pe, gain, W, cache: ChunkCache, past: int, table: RopeTable, pairing="half",
                  eps: float = 1e-6, return_lse: bool = False, out=None):
    """One chunk of a chunked prefill: the chunk's tokens (q [B,H,T,Dqk],
    latent [B,T,R], k_pe [B,T,Dr], positions past..past+T-1) are normalised,
    expanded and appended to the cache at row `past`, then attend causally
    to rows 0..past+T-1."""
    H, Dn = cache.k_nope.shape[1], cache.k_nope.shape[3]
    Dv = cache.vt.shape[2]
    c_norm = api.mla_latent_rmsnorm(latent, gain, eps)
    api.mla_kv_expand(c_norm, W, H, Dn, Dv, k=cache.k_nope, v=cache.vt, v_layout="cols", t_off=past)
    api.mla_rotate_rope_key(k_pe, table.cos, table.sin, cache.k_rot, past, pairing)
    return api.mla_prefill_attention_cached(q, cache.k_nope, cache.k_rot, cache.vt, past, table.cos, table.sin,
                                            table.scale, pairing, return_lse=return_lse, out=out)


def block_forward(hidden, W_qa, gain_q, W_qb, W_kva, gain, W, W_o, table: RopeTable, H: int, Dn: int, Dr: int,
                  Dv: int, pairing="half", eps: float = 1e-6):
    """The attention block around the path, from hidden states [B, T, hid]:
    q = q_b_proj(q_a_layernorm(q_a_proj(h))) written head-major, (latent,
    rotary key) = kv_a_proj_with_mqa(h) written apart, the prefill path, then
    o_proj on its head-major output. Returns [B, T, hid] bf16."""
    B, T, _ = hidden.shape
    R = W.shape[1]
    qa = api.mla_linear(hidden, W_qa)
    qn = api.mla_rmsnorm(qa, gain_q, eps, dtype=torch.bfloat16)
    q = api.mla_linear(qn, W_qb, out_heads=(H, Dn + Dr))
    latent, k_pe = api.mla_linear(hidden, W_kva, split=R)
    o = prefill_forward(q, latent, k_pe, gain, W, table, Dn, Dv, pairing, eps)
    return api.mla_linear(o, W_o, x_heads=True).view(B, T, W_o.shape[0])


class StepGraph:
    """A step recorded once as a HIP graph (torch.cuda.CUDAGraph) and replayed:
    for launch-bound steps such as a decode step, whose kernels are short and
    serially dependent. `step` is a callable that issues the library's calls
    on the current stream and returns its output tensor; every tensor it
    reads or writes must stay allocated and at the same address (fill new
    inputs into them before `replay`), and its output (allocated during
    capture from the graph's private pool) is overwritten by each replay. The
    library queues no memset and no host synchronisation, so its calls can
    be recorded."""

    def __init__(self, step, warmup: int = 2):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.output = step()

    def replay(self):
        self.graph.replay()
        return self.output
