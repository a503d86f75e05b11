"""Thin PyTorch binding of libmla (include/mla.h), one function per C entry
point and with the same names. Argument marshalling only: device buffers are
torch tensors, the stream is torch's current HIP stream, and every step of the
path runs in the library's HIP kernels. Outputs not supplied by the caller are
allocated with torch (the library itself never allocates).
"""

from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import DTYPE_BF16, DTYPE_FP16, PAIR_HALF, PAIR_INTERLEAVED, ROPE_DEFAULT, ROPE_YARN, RopeParams, check

__all__ = [
    "RopeParams", "rope_params", "mla_rope_table_build", "mla_softmax_scale", "mla_latent_rmsnorm",
    "mla_kv_expand", "mla_prefill_attention", "mla_decode_attention", "mla_absorb_prepare",
    "mla_latent_cache_append", "mla_decode_absorbed", "mla_rotate_rope_key", "mla_prefill_attention_cached",
    "mla_decode_latent_expanded", "mla_linear", "mla_rmsnorm", "mla_decode_attention_noalloc", "mla_latent_prepare",
    "pairing_code",
    "PAIR_HALF", "PAIR_INTERLEAVED", "ROPE_DEFAULT", "ROPE_YARN",
]


def rope_params(kind: str, rope_dim: int, base: float, factor: float = 1.0, original_max_pos: int = 4096,
                beta_fast: float = 32.0, beta_slow: float = 1.0, mscale: float = 1.0,
                mscale_all_dim: float = 0.0) -> RopeParams:
    """`mla_rope_params` from plain values; kind is "default" or "yarn"
    (any other kind is passed as an unknown type and rejected by the library)."""
    t = {"default": ROPE_DEFAULT, "yarn": ROPE_YARN}.get(kind, 99)
    return RopeParams(int(rope_dim), t, float(base), float(factor), int(original_max_pos), float(beta_fast),
                      float(beta_slow), float(mscale), float(mscale_all_dim))


def params_from(spec, rope_dim: int) -> RopeParams:
    """`mla_rope_params` from any object with the RopeSpec attributes."""
    return rope_params(spec.kind, rope_dim, spec.base, spec.factor, spec.original_max_pos, spec.beta_fast,
                       spec.beta_slow, spec.mscale, spec.mscale_all_dim)


def pairing_code(pairing) -> int:
    if isinstance(pairing, int):
        return pairing
    return {"half": PAIR_HALF, "interleaved": PAIR_INTERLEAVED}.get(pairing, 99)


_DTYPE_CODE = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_FP16}


def _kv_code(t: torch.Tensor, name: str) -> int:
    """mla_dtype of a key/value tensor (bf16 or fp16)."""
    if t.dtype not in _DTYPE_CODE:
        raise TypeError(f"{name} must be bfloat16 or float16 (got {t.dtype})")
    return _DTYPE_CODE[t.dtype]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} should be of size {tuple(shape)}, but is {tuple(t.shape)}")


def _need(t: torch.Tensor, name: str, dtype=torch.bfloat16) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def mla_softmax_scale(rope: RopeParams, qk_head_dim: int) -> float:
    out = ctypes.c_double()
    check("mla_softmax_scale", _lib.load().mla_softmax_scale(ctypes.byref(rope), int(qk_head_dim), ctypes.byref(out)))
    return out.value


def mla_rope_table_build(rope: RopeParams, n_pos: int, device="cuda") -> Tuple[torch.Tensor, torch.Tensor, float]:
    """cos, sin fp32 [n_pos, rope_dim/2] on `device`, and the softmax-scale
    multiplier mscale(factor, mscale_all_dim)^2 (1 when not applicable)."""
    lib = _lib.load()
    half = rope.rope_dim // 2
    cos = torch.empty((n_pos, half), dtype=torch.float32, device=device)
    sin = torch.empty((n_pos, half), dtype=torch.float32, device=device)
    m2 = ctypes.c_double()
    check("mla_rope_table_build",
          lib.mla_rope_table_build(ctypes.byref(rope), int(n_pos), _ptr(cos), _ptr(sin), ctypes.byref(m2),
                                   _stream(cos)))
    return cos, sin, m2.value


def mla_latent_rmsnorm(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """RMSNorm over the last dim of x (bf16 [..., R]) with weight w (bf16 [R]);
    returns the normalised latent in fp16 [..., R]."""
    _need(x, "x")
    _need(w, "w")
    R = x.shape[-1]
    if w.numel() != R:
        raise ValueError("weight size does not match the latent width")
    y = torch.empty(x.shape, dtype=torch.float16, device=x.device) if out is None else out
    _need(y, "out", torch.float16)
    _shape(y, "out", x.shape)
    n = x.numel() // R if R else 0
    check("mla_latent_rmsnorm",
          _lib.load().mla_latent_rmsnorm(_ptr(x), _ptr(w), float(eps), _ptr(y), n, R, _stream(x)))
    return y


def mla_latent_prepare(latent: torch.Tensor, gain: torch.Tensor, eps: float, k_pe: torch.Tensor, cos: torch.Tensor,
                       sin: torch.Tensor, pairing="half", pos: Optional[torch.Tensor] = None,
                       c_norm: Optional[torch.Tensor] = None,
                       k_rot: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Latent RMSNorm (latent bf16 [B, T, R] -> c_norm fp16) and the rotated
    shared rotary key (k_pe bf16 [B, T, Dr] -> k_rot fp16) in one launch."""
    _need(latent, "latent")
    _need(gain, "gain")
    _need(k_pe, "k_pe")
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32)
    B, T, R = latent.shape
    Dr = k_pe.shape[-1]
    _shape(k_pe, "k_pe", (B, T, Dr))
    _shape(gain, "gain", (R,))
    _shape(sin, "sin", cos.shape)
    if cos.dim() != 2 or cos.shape[1] != Dr // 2:
        raise ValueError(f"cos should be [table_len, {Dr // 2}], but is {tuple(cos.shape)}")
    if c_norm is None:
        c_norm = torch.empty((B, T, R), dtype=torch.float16, device=latent.device)
    if k_rot is None:
        k_rot = torch.empty((B, T, Dr), dtype=torch.float16, device=latent.device)
    _need(c_norm, "c_norm", torch.float16)
    _need(k_rot, "k_rot", torch.float16)
    _shape(c_norm, "c_norm", (B, T, R))
    _shape(k_rot, "k_rot", (B, T, Dr))
    if pos is not None:
        _need(pos, "pos", torch.int32)
        _shape(pos, "pos", (B, T))
    check("mla_latent_prepare",
          _lib.load().mla_latent_prepare(_ptr(latent), _ptr(gain), float(eps), _ptr(k_pe), _ptr(cos), _ptr(sin),
                                         cos.shape[0], _ptr(pos), B, T, R, Dr, pairing_code(pairing), _ptr(c_norm),
                                         _ptr(k_rot), _stream(latent)))
    return c_norm, k_rot


def _layout_code(v_layout: str) -> int:
    if v_layout == "rows":
        return _lib.V_ROWS
    if v_layout == "cols":
        return _lib.V_COLS
    raise ValueError(f"v_layout must be 'rows' or 'cols', not {v_layout!r}")


def round8(n: int) -> int:
    return (n + 7) // 8 * 8


def mla_kv_expand(c_norm: torch.Tensor, W: torch.Tensor, H: int, Dn: int, Dv: int,
                  k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None, t_off: int = 0,
                  k_pe: Optional[torch.Tensor] = None, cos: Optional[torch.Tensor] = None,
                  sin: Optional[torch.Tensor] = None, pos: Optional[torch.Tensor] = None,
                  pairing="half", kv_dtype=torch.float16, v_layout: str = "rows") -> Tuple[torch.Tensor, torch.Tensor]:
    """kv_b_proj of c_norm (fp16 [B, T, R]) by W (bf16 [H*(Dn+Dv), R]).

    Without k/v: returns new k_nope [B, H, T, Dn] and v, [B, H, T, Dv] for
    v_layout "rows" or V^T [B, H, Dv, round8(T)] for "cols" (padding columns
    zeroed). New tensors take `kv_dtype` (bf16 or fp16); given k and v must
    share one of those element types.
    With k [B, H, Tcap, k_ld] and v [B, H, Tcap, Dv] (or V^T [B, H, Dv, v_ld]):
    writes rows (columns) t_off .. t_off+T-1; with k_pe [B, T, Dr] also writes
    the rotated shared key into k[..., Dn:Dn+Dr] of every head (append mode)."""
    _need(c_norm, "c_norm", torch.float16)
    _need(W, "W")
    lcode = _layout_code(v_layout)
    B, T, R = c_norm.shape
    if k is None:
        k = torch.empty((B, H, T, Dn), dtype=kv_dtype, device=c_norm.device)
    Tcap = k.shape[2]
    if v is None:
        shape = (B, H, Tcap, Dv) if lcode == _lib.V_ROWS else (B, H, Dv, round8(Tcap))
        v = torch.empty(shape, dtype=k.dtype, device=c_norm.device)
    code = _kv_code(k, "k")
    _need(k, "k", k.dtype)
    _need(v, "v", k.dtype)
    _shape(W, "W", (H * (Dn + Dv), R))
    if k.dim() != 4 or tuple(k.shape[:2]) != (B, H):
        raise ValueError(f"k should be [B={B}, H={H}, Tcap, k_ld], but is {tuple(k.shape)}")
    if lcode == _lib.V_ROWS:
        _shape(v, "v", (B, H, Tcap, Dv))
    elif v.dim() != 4 or tuple(v.shape[:3]) != (B, H, Dv):
        raise ValueError(f"v (V^T) should be [B={B}, H={H}, Dv={Dv}, v_ld], but is {tuple(v.shape)}")
    Dr = 0
    table_len = 0
    if k_pe is not None:
        _need(k_pe, "k_pe")
        _need(cos, "cos", torch.float32)
        _need(sin, "sin", torch.float32)
        Dr = k_pe.shape[-1]
        _shape(k_pe, "k_pe", (B, T, Dr))
        _shape(sin, "sin", cos.shape)
        if cos.dim() != 2 or cos.shape[1] != Dr // 2:
            raise ValueError(f"cos should be [table_len, {Dr // 2}], but is {tuple(cos.shape)}")
        table_len = cos.shape[0]
    if pos is not None:
        _need(pos, "pos", torch.int32)
        _shape(pos, "pos", (B, T))
    check("mla_kv_expand",
          _lib.load().mla_kv_expand(_ptr(c_norm), _ptr(W), B, T, R, H, Dn, Dv, _ptr(k), k.shape[-1], _ptr(v), lcode,
                                    v.shape[-1], Tcap, int(t_off), code, _ptr(k_pe), _ptr(cos), _ptr(sin),
                                    table_len, _ptr(pos), Dr, pairing_code(pairing), _stream(c_norm)))
    return k, v


def mla_prefill_attention(q: torch.Tensor, k_nope: torch.Tensor, k_pe: torch.Tensor, v: torch.Tensor,
                          cos: torch.Tensor, sin: torch.Tensor, scale: float, pairing="half",
                          pos: Optional[torch.Tensor] = None, return_lse: bool = False,
                          out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          v_layout: str = "rows"):
    """Causal attention out [B, H, T, Dv] bf16 (and lse [B, H, T] fp32).

    q [B, H, T, Dn+Dr] bf16, k_nope [B, H, T, Dn] and v (both bf16 or both
    fp16; v [B, H, T, Dv] for v_layout "rows", V^T [B, H, Dv, v_ld] for
    "cols"), k_pe [B, T, Dr] bf16 (not rotated), cos/sin [table_len, Dr/2]
    fp32."""
    for t, n in ((q, "q"), (k_pe, "k_pe")):
        _need(t, n)
    lcode = _layout_code(v_layout)
    code = _kv_code(k_nope, "k_nope")
    _need(k_nope, "k_nope", k_nope.dtype)
    _need(v, "v", k_nope.dtype)
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32)
    B, H, T, Dqk = q.shape
    Dn = k_nope.shape[-1]
    Dr = k_pe.shape[-1]
    _shape(k_nope, "k_nope", (B, H, T, Dqk - Dr))
    _shape(k_pe, "k_pe", (B, T, Dr))
    if lcode == _lib.V_ROWS:
        Dv, v_ld = v.shape[-1], 0
        _shape(v, "v", (B, H, T, Dv))
    else:
        if v.dim() != 4 or tuple(v.shape[:2]) != (B, H):
            raise ValueError(f"v (V^T) should be [B={B}, H={H}, Dv, v_ld], but is {tuple(v.shape)}")
        Dv, v_ld = v.shape[2], v.shape[3]
    _shape(sin, "sin", cos.shape)
    if cos.dim() != 2 or cos.shape[1] != Dr // 2:
        raise ValueError(f"cos should be [table_len, {Dr // 2}], but is {tuple(cos.shape)}")
    lib = _lib.load()
    if out is None:
        out = torch.empty((B, H, T, Dv), dtype=torch.bfloat16, device=q.device)
    _need(out, "out")
    _shape(out, "out", (B, H, T, Dv))
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if return_lse else None
    if pos is not None:
        _need(pos, "pos", torch.int32)
        _shape(pos, "pos", (B, T))
    need = ctypes.c_size_t(0)
    args_head = (_ptr(q), _ptr(k_nope), _ptr(k_pe), _ptr(v), lcode, v_ld, code, _ptr(cos), _ptr(sin), cos.shape[0],
                 _ptr(pos), B, H, T, Dn, Dr, Dv, float(scale), pairing_code(pairing), _ptr(out), _ptr(lse))
    check("mla_prefill_attention", lib.mla_prefill_attention(*args_head, None, ctypes.byref(need), _stream(q)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty((max(need.value, 1),), dtype=torch.uint8, device=q.device)
    have = ctypes.c_size_t(workspace.numel())
    check("mla_prefill_attention",
          lib.mla_prefill_attention(*args_head, _ptr(workspace), ctypes.byref(have), _stream(q)))
    return (out, lse) if return_lse else out


def mla_rotate_rope_key(k_pe: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, dst: torch.Tensor, t_off: int = 0,
                        pairing="half", pos: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rotate k_pe [B, T, Dr] bf16 (at pos [B, T], default t_off + t) into
    rows t_off.. of the shared rotated-key buffer dst [B, Tcap, Dr] (bf16 or
    fp16)."""
    _need(k_pe, "k_pe")
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32)
    code = _kv_code(dst, "dst")
    _need(dst, "dst", dst.dtype)
    B, T, Dr = k_pe.shape
    if dst.dim() != 3 or dst.shape[0] != B or dst.shape[2] != Dr:
        raise ValueError(f"dst should be [{B}, Tcap, {Dr}], but is {tuple(dst.shape)}")
    _shape(sin, "sin", cos.shape)
    if pos is not None:
        _need(pos, "pos", torch.int32)
        _shape(pos, "pos", (B, T))
    check("mla_rotate_rope_key",
          _lib.load().mla_rotate_rope_key(_ptr(k_pe), _ptr(cos), _ptr(sin), cos.shape[0], _ptr(pos), B, T, Dr,
                                          pairing_code(pairing), _ptr(dst), dst.shape[1], int(t_off), code,
                                          _stream(k_pe)))
    return dst


def mla_prefill_attention_cached(q: torch.Tensor, k_nope: torch.Tensor, k_rot: torch.Tensor, vt: torch.Tensor,
                                 past: int, cos: torch.Tensor, sin: torch.Tensor, scale: float, pairing="half",
                                 pos: Optional[torch.Tensor] = None, return_lse: bool = False,
                                 out: Optional[torch.Tensor] = None):
    """Causal attention of the T query tokens q [B, H, T, Dn+Dr] (positions
    past..past+T-1) against the cache k_nope [B, H, Tcap, Dn], k_rot
    [B, Tcap, Dr] (rotated) and V^T [B, H, Dv, v_ld], whose rows
    0..past+T-1 already hold the earlier tokens and the chunk. Returns
    out [B, H, T, Dv] bf16 (and lse [B, H, T])."""
    _need(q, "q")
    code = _kv_code(k_nope, "k_nope")
    _need(k_nope, "k_nope", k_nope.dtype)
    _need(k_rot, "k_rot", k_nope.dtype)
    _need(vt, "vt", k_nope.dtype)
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32)
    B, H, T, Dqk = q.shape
    Tcap, Dn = k_nope.shape[2], k_nope.shape[3]
    Dr = Dqk - Dn
    _shape(k_nope, "k_nope", (B, H, Tcap, Dn))
    _shape(k_rot, "k_rot", (B, Tcap, Dr))
    if vt.dim() != 4 or tuple(vt.shape[:2]) != (B, H):
        raise ValueError(f"vt should be [B={B}, H={H}, Dv, v_ld], but is {tuple(vt.shape)}")
    Dv, v_ld = vt.shape[2], vt.shape[3]
    _shape(sin, "sin", cos.shape)
    if out is None:
        out = torch.empty((B, H, T, Dv), dtype=torch.bfloat16, device=q.device)
    _need(out, "out")
    _shape(out, "out", (B, H, T, Dv))
    lse = torch.empty((B, H, T), dtype=torch.float32, device=q.device) if return_lse else None
    if pos is not None:
        _need(pos, "pos", torch.int32)
        _shape(pos, "pos", (B, T))
    check("mla_prefill_attention_cached",
          _lib.load().mla_prefill_attention_cached(_ptr(q), _ptr(k_nope), _ptr(k_rot), _ptr(vt), v_ld, code,
                                                   _ptr(cos), _ptr(sin), cos.shape[0], _ptr(pos), B, H, T,
                                                   int(past), Tcap, Dn, Dr, Dv, float(scale),
                                                   pairing_code(pairing), _ptr(out), _ptr(lse), _stream(q)))
    return (out, lse) if return_lse else out


def mla_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_len: torch.Tensor,
                         q_pos: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, scale: float, Dn: int,
                         pairing="half", num_splits: int = 0, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention out [B, H, 1, Dv] bf16 of q [B, H, 1, Dn+Dr] over the
    expanded caches k_cache [B, H, Tcap, Dn+Dr], v_cache [B, H, Tcap, Dv]."""
    _need(q, "q")
    code = _kv_code(k_cache, "k_cache")
    _need(k_cache, "k_cache", k_cache.dtype)
    _need(v_cache, "v_cache", k_cache.dtype)
    _need(seq_len, "seq_len", torch.int32)
    _need(q_pos, "q_pos", torch.int32)
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32)
    B, H, Tcap, Dqk = k_cache.shape
    Dv = v_cache.shape[-1]
    Dr = Dqk - Dn
    _shape(q, "q", (B, H, 1, Dqk))
    _shape(v_cache, "v_cache", (B, H, Tcap, Dv))
    _shape(seq_len, "seq_len", (B,))
    _shape(q_pos, "q_pos", (B,))
    _shape(sin, "sin", cos.shape)
    if cos.dim() != 2 or cos.shape[1] != Dr // 2:
        raise ValueError(f"cos should be [table_len, {Dr // 2}], but is {tuple(cos.shape)}")
    if out is None:
        out = torch.empty((B, H, 1, Dv), dtype=torch.bfloat16, device=q.device)
    _need(out, "out")
    _shape(out, "out", (B, H, 1, Dv))
    lib = _lib.load()
    head = (_ptr(q), _ptr(k_cache), _ptr(v_cache), code, _ptr(seq_len), _ptr(q_pos), _ptr(cos), _ptr(sin),
            cos.shape[0], B, H, Tcap, Dn, Dr, Dv, float(scale), pairing_code(pairing), int(num_splits))
    need = ctypes.c_size_t(0)
    check("mla_decode_attention", lib.mla_decode_attention(*head, None, ctypes.byref(need), _ptr(out), _stream(q)))
    if need.value == 0:
        check("mla_decode_attention", lib.mla_decode_attention(*head, None, None, _ptr(out), _stream(q)))
        return out
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty((need.value,), dtype=torch.uint8, device=q.device)
    have = ctypes.c_size_t(workspace.numel())
    check("mla_decode_attention",
          lib.mla_decode_attention(*head, _ptr(workspace), ctypes.byref(have), _ptr(out), _stream(q)))
    return out


# ---- decode against a compressed-latent cache (absorbed form)


def mla_decode_attention_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 seq_len: torch.Tensor, q_pos: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                                 scale: float, Dn: int, pairing="half", num_splits: int = 0,
                                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mla_decode_attention without a workspace: the split partials live in
    the library's static per-GPU scratch (MLA_DECODE_SCRATCH_BYTES). Give
    `out` to allocate nothing at all."""
    _need(q, "q")
    code = _kv_code(k_cache, "k_cache")
    _need(k_cache, "k_cache", k_cache.dtype)
    _need(v_cache, "v_cache", k_cache.dtype)
    _need(seq_len, "seq_len", torch.int32)
    _need(q_pos, "q_pos", torch.int32)
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32)
    B, H, Tcap, Dqk = k_cache.shape
    Dv = v_cache.shape[-1]
    Dr = Dqk - Dn
    _shape(q, "q", (B, H, 1, Dqk))
    _shape(v_cache, "v_cache", (B, H, Tcap, Dv))
    _shape(seq_len, "seq_len", (B,))
    _shape(q_pos, "q_pos", (B,))
    _shape(sin, "sin", cos.shape)
    if cos.dim() != 2 or cos.shape[1] != Dr // 2:
        raise ValueError(f"cos should be [table_len, {Dr // 2}], but is {tuple(cos.shape)}")
    if out is None:
        out = torch.empty((B, H, 1, Dv), dtype=torch.bfloat16, device=q.device)
    _need(out, "out")
    _shape(out, "out", (B, H, 1, Dv))
    check("mla_decode_attention_noalloc",
          _lib.load().mla_decode_attention_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), code, _ptr(seq_len),
                                                   _ptr(q_pos), _ptr(cos), _ptr(sin), cos.shape[0], B, H, Tcap, Dn,
                                                   Dr, Dv, float(scale), pairing_code(pairing), int(num_splits),
                                                   _ptr(out), _stream(q)))
    return out

def mla_absorb_prepare(W: torch.Tensor, H: int, Dn: int, Dv: int,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """W_uk transposed per head, [H, R, Dn] bf16, from the kv_b_proj weight
    W [H*(Dn+Dv), R] (one-time weight preparation for mla_decode_absorbed)."""
    _need(W, "W")
    R = W.shape[1]
    _shape(W, "W", (H * (Dn + Dv), R))
    if out is None:
        out = torch.empty((H, R, Dn), dtype=torch.bfloat16, device=W.device)
    _need(out, "out")
    _shape(out, "out", (H, R, Dn))
    check("mla_absorb_prepare", _lib.load().mla_absorb_prepare(_ptr(W), H, R, Dn, Dv, _ptr(out), _stream(W)))
    return out


def mla_latent_cache_append(latent: torch.Tensor, gain: torch.Tensor, k_pe: torch.Tensor, cos: torch.Tensor,
                            sin: torch.Tensor, t_pos: torch.Tensor, cache: torch.Tensor, eps: float = 1e-6,
                            pairing="half") -> torch.Tensor:
    """Write each sequence's new token into row t_pos[b] of the latent cache
    [B, Lcap, R+Dr] fp16: its normalised latent, then its rotary key rotated
    at that position. latent [B, R] and k_pe [B, Dr] are bf16."""
    _need(latent, "latent")
    _need(gain, "gain")
    _need(k_pe, "k_pe")
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32)
    _need(t_pos, "t_pos", torch.int32)
    _need(cache, "cache", torch.float16)
    B, R = latent.shape
    Dr = k_pe.shape[-1]
    _shape(gain, "gain", (R,))
    _shape(k_pe, "k_pe", (B, Dr))
    _shape(t_pos, "t_pos", (B,))
    _shape(sin, "sin", cos.shape)
    if cache.dim() != 3 or cache.shape[0] != B or cache.shape[2] != R + Dr:
        raise ValueError(f"cache should be [{B}, Lcap, {R + Dr}], but is {tuple(cache.shape)}")
    if cos.dim() != 2 or cos.shape[1] != Dr // 2:
        raise ValueError(f"cos should be [table_len, {Dr // 2}], but is {tuple(cos.shape)}")
    check("mla_latent_cache_append",
          _lib.load().mla_latent_cache_append(_ptr(latent), _ptr(gain), float(eps), _ptr(k_pe), _ptr(cos), _ptr(sin),
                                              cos.shape[0], _ptr(t_pos), pairing_code(pairing), B, R, Dr,
                                              _ptr(cache), cache.shape[1], _stream(latent)))
    return cache


def mla_decode_absorbed(q: torch.Tensor, W: torch.Tensor, w_ukt: torch.Tensor, cache: torch.Tensor,
                        seq_len: torch.Tensor, q_pos: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor,
                        scale: float, Dn: int, Dv: int, pairing="half", num_splits: int = 0,
                        out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention out [B, H, 1, Dv] bf16 of q [B, H, 1, Dn+Dr] against
    the latent cache [B, Lcap, R+Dr] fp16, by the absorbed form (W_uk folded
    into the query, W_uv applied to the attention-weighted latent)."""
    _need(q, "q")
    _need(W, "W")
    _need(w_ukt, "w_ukt")
    _need(cache, "cache", torch.float16)
    _need(seq_len, "seq_len", torch.int32)
    _need(q_pos, "q_pos", torch.int32)
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32)
    B, H, _, Dqk = q.shape
    Dr = Dqk - Dn
    Lcap, RW = cache.shape[1], cache.shape[2]
    R = RW - Dr
    _shape(q, "q", (B, H, 1, Dqk))
    _shape(W, "W", (H * (Dn + Dv), R))
    _shape(w_ukt, "w_ukt", (H, R, Dn))
    _shape(cache, "cache", (B, Lcap, R + Dr))
    _shape(seq_len, "seq_len", (B,))
    _shape(q_pos, "q_pos", (B,))
    _shape(sin, "sin", cos.shape)
    if cos.dim() != 2 or cos.shape[1] != Dr // 2:
        raise ValueError(f"cos should be [table_len, {Dr // 2}], but is {tuple(cos.shape)}")
    if out is None:
        out = torch.empty((B, H, 1, Dv), dtype=torch.bfloat16, device=q.device)
    _need(out, "out")
    _shape(out, "out", (B, H, 1, Dv))
    lib = _lib.load()
    head = (_ptr(q), _ptr(W), _ptr(w_ukt), _ptr(cache), _ptr(seq_len), _ptr(q_pos), _ptr(cos), _ptr(sin),
            cos.shape[0], B, H, Lcap, R, Dn, Dr, Dv, float(scale), pairing_code(pairing), int(num_splits))
    need = ctypes.c_size_t(0)
    check("mla_decode_absorbed", lib.mla_decode_absorbed(*head, None, ctypes.byref(need), _ptr(out), _stream(q)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty((need.value,), dtype=torch.uint8, device=q.device)
    have = ctypes.c_size_t(workspace.numel())
    check("mla_decode_absorbed",
          lib.mla_decode_absorbed(*head, _ptr(workspace), ctypes.byref(have), _ptr(out), _stream(q)))
    return out


def mla_decode_latent_expanded(q: torch.Tensor, W: torch.Tensor, cache: torch.Tensor, seq_len: torch.Tensor,
                               q_pos: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, scale: float, Dn: int,
                               Dv: int, pairing="half", num_splits: int = 0, out: Optional[torch.Tensor] = None,
                               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The same output as mla_decode_absorbed, by re-expanding every cached
    latent row into per-head keys and values on each call."""
    _need(q, "q")
    _need(W, "W")
    _need(cache, "cache", torch.float16)
    _need(seq_len, "seq_len", torch.int32)
    _need(q_pos, "q_pos", torch.int32)
    _need(cos, "cos", torch.float32)
    _need(sin, "sin", torch.float32)
    B, H, _, Dqk = q.shape
    Dr = Dqk - Dn
    Lcap, RW = cache.shape[1], cache.shape[2]
    R = RW - Dr
    _shape(W, "W", (H * (Dn + Dv), R))
    _shape(cache, "cache", (B, Lcap, R + Dr))
    _shape(seq_len, "seq_len", (B,))
    _shape(q_pos, "q_pos", (B,))
    _shape(sin, "sin", cos.shape)
    if out is None:
        out = torch.empty((B, H, 1, Dv), dtype=torch.bfloat16, device=q.device)
    _need(out, "out")
    _shape(out, "out", (B, H, 1, Dv))
    lib = _lib.load()
    head = (_ptr(q), _ptr(W), _ptr(cache), _ptr(seq_len), _ptr(q_pos), _ptr(cos), _ptr(sin), cos.shape[0], B, H,
            Lcap, R, Dn, Dr, Dv, float(scale), pairing_code(pairing), int(num_splits))
    need = ctypes.c_size_t(0)
    check("mla_decode_latent_expanded",
          lib.mla_decode_latent_expanded(*head, None, ctypes.byref(need), _ptr(out), _stream(q)))
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty((need.value,), dtype=torch.uint8, device=q.device)
    have = ctypes.c_size_t(workspace.numel())
    check("mla_decode_latent_expanded",
          lib.mla_decode_latent_expanded(*head, _ptr(workspace), ctypes.byref(have), _ptr(out), _stream(q)))
    return out


def mla_linear(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, x_heads: bool = False,
               out_heads: Optional[Tuple[int, int]] = None, split: Optional[int] = None,
               out: Optional[torch.Tensor] = None):
    """Y = X W^T (+ bias) in bf16 with fp32 accumulation. w [N, K].

    X: [M, K], or with x_heads=True the head-major [B, Hx, T, Dx] tensor read
    as [B*T, Hx*Dx]. Y: [M, N] (for a head-major X: [B, T, N]); with
    out_heads=(H, D) the head-major [B, H, T, D] (N = H*D; B, T from X's
    leading dimensions); with split=s the pair ([..., s], [..., N-s])."""
    _need(x, "x")
    _need(w, "w")
    N, K = w.shape
    if x_heads:
        if x.dim() != 4:
            raise ValueError(f"a head-major x should be [B, H, T, D], but is {tuple(x.shape)}")
        B, Hx, T, Dx = x.shape
        if Hx * Dx != K:
            raise ValueError(f"x heads {Hx} x {Dx} do not match w's K = {K}")
        M, lead, xl, xT, xD = B * T, (B, T), _lib.LIN_HEADS, T, Dx
    else:
        if x.shape[-1] != K:
            raise ValueError(f"x's last dimension {x.shape[-1]} does not match w's K = {K}")
        lead = tuple(x.shape[:-1])
        M = int(torch.tensor(lead).prod()) if lead else 1
        xl, xT, xD = _lib.LIN_ROWS, 0, 0
        B = lead[0] if len(lead) >= 2 else 1
        T = M // B
    if bias is not None:
        _need(bias, "bias")
        _shape(bias, "bias", (N,))
    y1 = None
    yT = yD = ys = 0
    if out_heads is not None:
        Hy, Dy = out_heads
        if Hy * Dy != N:
            raise ValueError(f"out_heads {out_heads} do not match N = {N}")
        yl, yT, yD = _lib.LIN_HEADS, (lead[-1] if len(lead) >= 2 else M), Dy
        Bo = M // yT
        if out is None:
            out = torch.empty((Bo, Hy, yT, Dy), dtype=torch.bfloat16, device=x.device)
        _shape(out, "out", (Bo, Hy, yT, Dy))
    elif split is not None:
        yl, ys = _lib.LIN_SPLIT, int(split)
        y0 = torch.empty(lead + (ys,), dtype=torch.bfloat16, device=x.device)
        y1 = torch.empty(lead + (N - ys,), dtype=torch.bfloat16, device=x.device)
        out = y0
    else:
        yl = _lib.LIN_ROWS
        if out is None:
            out = torch.empty(lead + (N,), dtype=torch.bfloat16, device=x.device)
        _shape(out, "out", lead + (N,))
    _need(out, "out")
    check("mla_linear", _lib.load().mla_linear(_ptr(x), xl, xT, xD, _ptr(w), _ptr(bias), M, N, K, _ptr(out),
                                               _ptr(y1), yl, yT, yD, ys, _stream(x)))
    return (out, y1) if split is not None else out


def mla_rmsnorm(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6, dtype=torch.bfloat16,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """RMSNorm of the rows of x [..., R] (bf16) with gain w [R], written in
    `dtype` (bf16 or fp16)."""
    _need(x, "x")
    _need(w, "w")
    R = x.shape[-1]
    _shape(w, "w", (R,))
    if out is None:
        out = torch.empty(x.shape, dtype=dtype, device=x.device)
    code = _kv_code(out, "out")
    _need(out, "out", out.dtype)
    _shape(out, "out", x.shape)
    check("mla_rmsnorm", _lib.load().mla_rmsnorm(_ptr(x), _ptr(w), float(eps), _ptr(out), x.numel() // R, R, code,
                                                 _stream(x)))
    return out


# ---- measurement aids (mla_ceiling.h): sustained ceilings of the chip

def mla_ceiling_hbm_read(buf: torch.Tensor, sink: torch.Tensor) -> int:
    """Queue one streaming read of every byte of `buf` (device, contiguous,
    16-byte aligned, a multiple of 16 bytes); `sink` is a 4-byte device
    tensor. Returns the bytes read."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if not sink.is_cuda or sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must be a device tensor of at least 4 bytes")
    n = buf.numel() * buf.element_size()
    check("mla_ceiling_hbm_read", _lib.load().mla_ceiling_hbm_read(_ptr(buf), n, _ptr(sink), _stream(buf)))
    return n


def mla_ceiling_mfma(operands: torch.Tensor, iters: int, lds_operands: bool, sink: torch.Tensor) -> float:
    """Queue one dense fp16 MFMA loop over `operands` (fp16 device tensor of
    24576 values, e.g. random ones); returns the launch's flop count."""
    _need(operands, "operands", torch.float16)
    if operands.numel() * 2 != _lib.CEILING_MFMA_OPERAND_BYTES:
        raise ValueError(f"operands must hold {_lib.CEILING_MFMA_OPERAND_BYTES // 2} fp16 values")
    if not sink.is_cuda or sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must be a device tensor of at least 4 bytes")
    flops = ctypes.c_double()
    check("mla_ceiling_mfma", _lib.load().mla_ceiling_mfma(_ptr(operands), int(iters), int(bool(lds_operands)),
                                                           _ptr(sink), ctypes.byref(flops), _stream(operands)))
    return flops.value


def mla_device_info(device: int = 0) -> dict:
    """Compute units and peak shader / memory clocks (MHz) of a device."""
    cu, sclk, mclk = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    check("mla_device_info", _lib.load().mla_device_info(int(device), ctypes.byref(cu), ctypes.byref(sclk),
                                                         ctypes.byref(mclk)))
    return {"compute_units": cu.value, "peak_sclk_mhz": sclk.value / 1000.0, "peak_mclk_mhz": mclk.value / 1000.0}
