"""C-ABI checks that need no GPU: libmla.so loads, exports every function
include/mla.h declares, and rejects invalid arguments with the documented
status codes before any device call (every call here fails validation, so no
HIP work is queued)."""

import ctypes
import os
import re

import pytest

from head_latent_attention_rmsnorm_amd import _lib
from head_latent_attention_rmsnorm_amd._lib import RopeParams

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

OK, NULL, SHAPE, UNSUP, ROPE, WS = 0, -1, -2, -3, -4, -5
FAKE = 0x100000  # a non-null, 16-byte-aligned address that is never dereferenced


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mla_status|const char\*)\s+(mla_\w+)\s*\(", txt, re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared()
    assert len(names) == 17
    assert sorted(_lib.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.mla_status_string(code)
    assert lib.mla_status_string(12345) == b"unknown status"


def yarn(**kw):
    p = dict(rope_dim=64, type=1, base=50000.0, factor=32.0, original_max_pos=4096, beta_fast=32.0, beta_slow=1.0,
             mscale=1.0, mscale_all_dim=1.0)
    p.update(kw)
    return RopeParams(**p)


def test_softmax_scale_host_rule(lib):
    out = ctypes.c_double()
    assert lib.mla_softmax_scale(ctypes.byref(yarn()), 192, ctypes.byref(out)) == OK
    assert out.value == pytest.approx(0.13086079996295005, rel=1e-15)
    assert lib.mla_softmax_scale(ctypes.byref(yarn(type=0)), 256, ctypes.byref(out)) == OK
    assert out.value == 0.0625
    assert lib.mla_softmax_scale(ctypes.byref(yarn(type=7)), 192, ctypes.byref(out)) == ROPE
    assert lib.mla_softmax_scale(None, 192, ctypes.byref(out)) == NULL
    assert lib.mla_softmax_scale(ctypes.byref(yarn()), 0, ctypes.byref(out)) == SHAPE


def test_rope_table_validation(lib):
    p = ctypes.byref(yarn())
    m2 = ctypes.c_double()
    assert lib.mla_rope_table_build(None, 10, FAKE, FAKE, None, None) == NULL
    assert lib.mla_rope_table_build(p, 10, None, FAKE, None, None) == NULL
    assert lib.mla_rope_table_build(p, 0, FAKE, FAKE, None, None) == SHAPE
    assert lib.mla_rope_table_build(ctypes.byref(yarn(type=2)), 10, FAKE, FAKE, None, None) == ROPE
    assert lib.mla_rope_table_build(ctypes.byref(yarn(rope_dim=63)), 10, FAKE, FAKE, None, None) == SHAPE
    assert lib.mla_rope_table_build(ctypes.byref(yarn(base=1.0)), 10, FAKE, FAKE, None, None) == SHAPE
    assert lib.mla_rope_table_build(ctypes.byref(yarn(factor=-1.0)), 10, FAKE, FAKE, ctypes.byref(m2), None) == SHAPE


def test_rmsnorm_validation(lib):
    assert lib.mla_latent_rmsnorm(None, FAKE, 1e-6, FAKE, 4, 512, None) == NULL
    assert lib.mla_latent_rmsnorm(FAKE, FAKE, 1e-6, FAKE, -1, 512, None) == SHAPE
    assert lib.mla_latent_rmsnorm(FAKE, FAKE, 1e-6, FAKE, 4, 0, None) == SHAPE
    assert lib.mla_latent_rmsnorm(FAKE, FAKE, -1.0, FAKE, 4, 512, None) == SHAPE
    assert lib.mla_latent_rmsnorm(FAKE, FAKE, float("nan"), FAKE, 4, 512, None) == SHAPE
    assert lib.mla_latent_rmsnorm(FAKE, FAKE, 1e-6, FAKE, 0, 512, None) == OK  # empty: no-op
    assert lib.mla_latent_rmsnorm(None, None, 1e-6, None, 0, 512, None) == OK


def prepare(lib, **kw):
    a = dict(latent=FAKE, gain=FAKE, eps=1e-6, k_pe=FAKE, cos=FAKE, sin=FAKE, table_len=8192, pos=None, B=2, T=8192,
             R=512, Dr=64, pairing=0, c_norm=FAKE, k_rot=FAKE)
    a.update(kw)
    return lib.mla_latent_prepare(a["latent"], a["gain"], ctypes.c_float(a["eps"]), a["k_pe"], a["cos"], a["sin"],
                                  a["table_len"], a["pos"], a["B"], a["T"], a["R"], a["Dr"], a["pairing"],
                                  a["c_norm"], a["k_rot"], None)


def test_latent_prepare_validation(lib):
    assert prepare(lib, latent=None) == NULL
    assert prepare(lib, k_rot=None) == NULL
    assert prepare(lib, cos=None) == NULL
    assert prepare(lib, R=100) == SHAPE      # not a multiple of 8
    assert prepare(lib, R=8192) == SHAPE     # wider than 4096
    assert prepare(lib, Dr=63) == SHAPE
    assert prepare(lib, eps=-1.0) == SHAPE
    assert prepare(lib, table_len=100) == SHAPE  # positions 0..T-1 need T table rows
    assert prepare(lib, pairing=7) == ROPE
    assert prepare(lib, latent=FAKE + 8) == SHAPE  # 16-byte alignment
    assert prepare(lib, B=0) == OK
    assert prepare(lib, T=0, latent=None) == OK


def expand(lib, **kw):
    a = dict(c=FAKE, W=FAKE, B=1, T=4, R=512, H=2, Dn=128, Dv=128, k=FAKE, k_ld=128, v=FAKE, v_layout=0, v_ld=0,
             Tcap=4, t_off=0, kv_dtype=1, k_pe=None, cos=None, sin=None, table_len=0, pos=None, Dr=0, pairing=0)
    a.update(kw)
    return lib.mla_kv_expand(*a.values(), None)


def test_kv_expand_validation(lib):
    assert expand(lib, c=None) == NULL
    assert expand(lib, R=500) == SHAPE  # not a multiple of 8
    assert expand(lib, Dn=100) == SHAPE
    assert expand(lib, t_off=1) == SHAPE  # t_off + T > Tcap
    assert expand(lib, k_ld=64) == SHAPE
    assert expand(lib, c=FAKE + 2) == SHAPE  # misaligned
    # append mode needs the table and a wide enough key row
    assert expand(lib, k_pe=FAKE, Dr=64, k_ld=192) == NULL
    assert expand(lib, k_pe=FAKE, cos=FAKE, sin=FAKE, table_len=4, Dr=64, k_ld=128) == SHAPE
    assert expand(lib, k_pe=FAKE, cos=FAKE, sin=FAKE, table_len=4, Dr=64, k_ld=192, pairing=5) == ROPE
    assert expand(lib, k_pe=FAKE, cos=FAKE, sin=FAKE, table_len=2, Dr=64, k_ld=192) == SHAPE  # table too short
    assert expand(lib, kv_dtype=2) == UNSUP
    # transposed values: row stride >= Tcap and a multiple of 8
    assert expand(lib, v_layout=1, v_ld=2) == SHAPE
    assert expand(lib, v_layout=1, v_ld=12) == SHAPE
    assert expand(lib, v_layout=2, v_ld=8) == SHAPE
    assert expand(lib, B=0) == OK  # empty: no-op
    assert expand(lib, T=0, c=None, k=None) == OK  # empty tensors may have null data


def prefill(lib, ws=FAKE, ws_bytes=None, **kw):
    a = dict(q=FAKE, kn=FAKE, kpe=FAKE, v=FAKE, v_layout=1, v_ld=4096, kv_dtype=1, cos=FAKE, sin=FAKE,
             table_len=4096, pos=None, B=1, H=64, T=4096, Dn=128, Dr=64, Dv=128, scale=0.13, pairing=0, out=FAKE,
             lse=None)
    a.update(kw)
    return lib.mla_prefill_attention(*a.values(), ws, ws_bytes, None)


def test_prefill_validation(lib):
    need = ctypes.c_size_t(0)
    assert prefill(lib, ws=None, ws_bytes=ctypes.byref(need)) == OK
    assert need.value == 4096 * 64 * 2
    # row-major values are transposed into the workspace: [B, H, Dv, round8(T)] more
    assert prefill(lib, ws=None, ws_bytes=ctypes.byref(need), v_layout=0, T=4095, table_len=4095) == OK
    assert need.value == (4095 * 64 * 2 + 255) // 256 * 256 + 64 * 128 * 4096 * 2
    assert prefill(lib, v_ld=4090) == SHAPE  # below T
    assert prefill(lib, v_ld=4100) == SHAPE  # not a multiple of 8
    assert prefill(lib, v_layout=3) == SHAPE
    assert prefill(lib, v_ld=1 << 30) == SHAPE  # one V^T slice beyond 2 GiB
    assert prefill(lib, q=None) == NULL
    assert prefill(lib, Dn=100) == UNSUP
    assert prefill(lib, Dv=64) == UNSUP
    assert prefill(lib, pairing=3) == ROPE
    assert prefill(lib, scale=0.0) == SHAPE
    assert prefill(lib, table_len=100) == SHAPE  # implicit positions 0..T-1 exceed the table
    assert prefill(lib, ws=None) == WS
    small = ctypes.c_size_t(16)
    assert prefill(lib, ws_bytes=ctypes.byref(small)) == WS
    assert prefill(lib, kv_dtype=-1) == UNSUP
    assert prefill(lib, T=0) == OK  # empty: no-op
    assert prefill(lib, T=0, q=None, out=None) == OK
    assert prefill(lib, T=-1) == SHAPE


def decode(lib, ws=FAKE, ws_bytes=None, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, dtype=0, seq=FAKE, qpos=FAKE, cos=FAKE, sin=FAKE, table_len=1001, B=32,
             H=64, Tcap=1001, Dn=128, Dr=64, Dv=128, scale=0.13, pairing=0, splits=4)
    a.update(kw)
    return lib.mla_decode_attention(*a.values(), ws, ws_bytes, FAKE, None)


def test_decode_validation(lib):
    need = ctypes.c_size_t(0)
    assert decode(lib, ws=None, ws_bytes=ctypes.byref(need)) == OK
    assert need.value >= 32 * 64 * 4 * (128 + 2) * 4
    assert decode(lib, splits=1, ws=None, ws_bytes=ctypes.byref(need)) == OK
    assert need.value == 0
    assert decode(lib, kc=None) == NULL
    assert decode(lib, Dn=96) == UNSUP
    assert decode(lib, pairing=-1) == ROPE
    assert decode(lib, splits=-2) == SHAPE
    assert decode(lib, splits=300) == SHAPE
    assert decode(lib, ws=None) == WS
    assert decode(lib, dtype=3) == UNSUP
    assert decode(lib, B=0) == OK
    assert decode(lib, B=0, splits=0) == OK  # automatic split count of an empty batch


def decode_noalloc(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, dtype=0, seq=FAKE, qpos=FAKE, cos=FAKE, sin=FAKE, table_len=1001, B=32, H=64,
             Tcap=1001, Dn=128, Dr=64, Dv=128, scale=0.13, pairing=0, splits=0, out=FAKE)
    a.update(kw)
    return lib.mla_decode_attention_noalloc(a["q"], a["kc"], a["vc"], a["dtype"], a["seq"], a["qpos"], a["cos"],
                                            a["sin"], a["table_len"], a["B"], a["H"], a["Tcap"], a["Dn"], a["Dr"],
                                            a["Dv"], ctypes.c_float(a["scale"]), a["pairing"], a["splits"], a["out"],
                                            None)


def test_decode_noalloc_validation(lib):
    """Rejections happen on the host before any HIP call: the same argument
    checks as the workspace entry point, and split partials beyond the static
    scratch (B*H*S*(Dv+2)*4 bytes > 16 MiB) are refused with
    MLA_ERR_WORKSPACE."""
    assert _lib.DECODE_SCRATCH_BYTES == 16 << 20
    assert re.search(r"#define MLA_DECODE_SCRATCH_BYTES \(\(size_t\)16 << 20\)", open(HEADER).read())
    assert decode_noalloc(lib, kc=None) == NULL
    assert decode_noalloc(lib, out=None) == NULL
    assert decode_noalloc(lib, Dn=96) == UNSUP
    assert decode_noalloc(lib, dtype=3) == UNSUP
    assert decode_noalloc(lib, pairing=-1) == ROPE
    assert decode_noalloc(lib, splits=-2) == SHAPE
    assert decode_noalloc(lib, splits=300) == SHAPE
    assert decode_noalloc(lib, scale=0.0) == SHAPE
    assert decode_noalloc(lib, table_len=0) == SHAPE
    assert decode_noalloc(lib, B=0) == OK
    # 32 x 64 x 8 splits: 32*64*8*130*4 = 8.5 MB fits; 16 splits (17 MB) and
    # 256 sequences x 64 heads x 4 splits (34 MB) do not
    assert 32 * 64 * 16 * (128 + 2) * 4 > _lib.DECODE_SCRATCH_BYTES
    assert decode_noalloc(lib, splits=16) == WS
    assert decode_noalloc(lib, B=256, splits=4) == WS


def test_absorb_prepare_validation(lib):
    def call(W=FAKE, H=64, R=512, Dn=128, Dv=128, out=FAKE):
        return lib.mla_absorb_prepare(W, H, R, Dn, Dv, out, None)
    assert call(W=None) == NULL
    assert call(out=None) == NULL
    assert call(H=0) == SHAPE
    assert call(R=0) == SHAPE
    assert call(Dn=0) == SHAPE
    assert call(Dv=-1) == SHAPE
    assert call(R=9000) == SHAPE


def latent_append(lib, **kw):
    a = dict(lat=FAKE, gain=FAKE, eps=1e-6, kpe=FAKE, cos=FAKE, sin=FAKE, table_len=1001, tpos=FAKE, pairing=0,
             B=32, R=512, Dr=64, cache=FAKE, Lcap=1001)
    a.update(kw)
    return lib.mla_latent_cache_append(*a.values(), None)


def test_latent_append_validation(lib):
    assert latent_append(lib, B=0) == OK  # empty: no-op
    assert latent_append(lib, B=0, lat=None, cache=None) == OK
    assert latent_append(lib, cache=None) == NULL
    assert latent_append(lib, tpos=None) == NULL
    assert latent_append(lib, B=-1) == SHAPE
    assert latent_append(lib, Dr=63) == SHAPE
    assert latent_append(lib, Lcap=0) == SHAPE
    assert latent_append(lib, eps=-1.0) == SHAPE
    assert latent_append(lib, eps=float("nan")) == SHAPE
    assert latent_append(lib, table_len=0) == SHAPE
    assert latent_append(lib, pairing=2) == ROPE


def absorbed(lib, ws=FAKE, ws_bytes=None, **kw):
    a = dict(q=FAKE, W=FAKE, wt=FAKE, cache=FAKE, seq=FAKE, qpos=FAKE, cos=FAKE, sin=FAKE, table_len=1001, B=32,
             H=64, Lcap=1001, R=512, Dn=128, Dr=64, Dv=128, scale=0.13, pairing=0, splits=0)
    a.update(kw)
    return lib.mla_decode_absorbed(*a.values(), ws, ws_bytes, FAKE, None)


def test_decode_absorbed_validation(lib):
    need = ctypes.c_size_t(0)
    assert absorbed(lib, ws=None, ws_bytes=ctypes.byref(need)) == OK
    # absorbed query [B,H,576] fp16 + (B, split, H) partial latent rows fp16 + lse
    assert need.value >= 32 * 64 * 576 * 2 + 32 * 64 * (512 * 2 + 4)
    small = ctypes.c_size_t(need.value - 256)
    assert absorbed(lib, ws_bytes=ctypes.byref(small)) == WS
    assert absorbed(lib, ws=None) == WS
    assert absorbed(lib, B=0) == OK
    assert absorbed(lib, cache=None) == NULL
    assert absorbed(lib, wt=None) == NULL
    assert absorbed(lib, R=256) == UNSUP
    assert absorbed(lib, Dr=32) == UNSUP
    assert absorbed(lib, Dn=100) == UNSUP
    assert absorbed(lib, Dv=48) == UNSUP
    assert absorbed(lib, pairing=5) == ROPE
    assert absorbed(lib, splits=65) == SHAPE
    assert absorbed(lib, splits=-1) == SHAPE
    assert absorbed(lib, Lcap=0) == SHAPE
    assert absorbed(lib, Lcap=4_000_000) == SHAPE  # one sequence's cache >= 2 GiB
    assert absorbed(lib, scale=0.0) == SHAPE
    assert absorbed(lib, table_len=0) == SHAPE
    assert absorbed(lib, cache=FAKE + 8) == SHAPE  # not 16-byte aligned


def test_rotate_rope_key_validation(lib):
    def call(kpe=FAKE, cos=FAKE, sin=FAKE, table_len=4096, pos=None, B=2, T=100, Dr=64, pairing=0, dst=FAKE,
             Tcap=4096, t_off=0, dtype=1):
        return lib.mla_rotate_rope_key(kpe, cos, sin, table_len, pos, B, T, Dr, pairing, dst, Tcap, t_off, dtype,
                                       None)
    assert call(T=0) == OK
    assert call(T=0, kpe=None, dst=None) == OK
    assert call(dst=None) == NULL
    assert call(Dr=7) == SHAPE
    assert call(t_off=4000) == SHAPE  # t_off + T > Tcap
    assert call(t_off=-1) == SHAPE
    assert call(table_len=50) == SHAPE  # positions t_off..t_off+T-1 need the table
    assert call(dtype=7) == UNSUP
    assert call(pairing=3) == ROPE


def cached(lib, **kw):
    a = dict(q=FAKE, kn=FAKE, kr=FAKE, vt=FAKE, v_ld=4096, dtype=1, cos=FAKE, sin=FAKE, table_len=4096, pos=None,
             B=2, H=64, T=512, past=1024, Tcap=4096, Dn=128, Dr=64, Dv=128, scale=0.13, pairing=0, out=FAKE,
             lse=None)
    a.update(kw)
    return lib.mla_prefill_attention_cached(*a.values(), None)


def test_prefill_cached_validation(lib):
    assert cached(lib, T=0) == OK
    assert cached(lib, T=0, q=None) == OK
    assert cached(lib, kr=None) == NULL
    assert cached(lib, past=-1) == SHAPE
    assert cached(lib, past=3700) == SHAPE  # past + T > Tcap
    assert cached(lib, v_ld=1500) == SHAPE  # v_ld < past + T
    assert cached(lib, v_ld=4092) == SHAPE  # not a multiple of 8
    assert cached(lib, Dn=96) == UNSUP
    assert cached(lib, dtype=4) == UNSUP
    assert cached(lib, pairing=2) == ROPE
    assert cached(lib, scale=-1.0) == SHAPE
    assert cached(lib, table_len=1000) == SHAPE
    assert cached(lib, vt=FAKE + 4) == SHAPE


def reexpand(lib, ws=FAKE, ws_bytes=None, **kw):
    a = dict(q=FAKE, W=FAKE, cache=FAKE, seq=FAKE, qpos=FAKE, cos=FAKE, sin=FAKE, table_len=1001, B=32, H=64,
             Lcap=1001, R=512, Dn=128, Dr=64, Dv=128, scale=0.13, pairing=0, splits=0)
    a.update(kw)
    return lib.mla_decode_latent_expanded(*a.values(), ws, ws_bytes, FAKE, None)


def test_decode_latent_expanded_validation(lib):
    need = ctypes.c_size_t(0)
    assert reexpand(lib, ws=None, ws_bytes=ctypes.byref(need)) == OK
    assert need.value >= 32 * 64 * 1001 * (192 + 128) * 2  # the expanded keys and values
    assert reexpand(lib, ws=None) == WS
    assert reexpand(lib, B=0) == OK
    assert reexpand(lib, cache=None) == NULL
    assert reexpand(lib, Dn=96) == UNSUP
    assert reexpand(lib, R=100) == SHAPE
    assert reexpand(lib, Dr=12, Dn=180) == SHAPE
    assert reexpand(lib, pairing=4) == ROPE
    assert reexpand(lib, splits=300) == SHAPE
    assert reexpand(lib, cache=FAKE + 8) == SHAPE


def linear(lib, **kw):
    a = dict(x=FAKE, xl=0, xT=0, xD=0, w=FAKE, bias=None, M=1024, N=1536, K=7168, y0=FAKE, y1=None, yl=0, yT=0, yD=0,
             ys=0)
    a.update(kw)
    return lib.mla_linear(*a.values(), None)


def test_linear_validation(lib):
    assert linear(lib, M=0) == OK
    assert linear(lib, M=0, x=None) == OK
    assert linear(lib, x=None) == NULL
    assert linear(lib, y0=None) == NULL
    assert linear(lib, yl=2, ys=512, N=576) == NULL  # split needs y1
    assert linear(lib, K=100) == SHAPE  # K not a multiple of 64
    assert linear(lib, N=100) == SHAPE  # N not a multiple of 8
    assert linear(lib, M=-1) == SHAPE
    assert linear(lib, xl=1, xT=1000, xD=128, K=8192) == SHAPE  # x_T does not divide M
    assert linear(lib, xl=1, xT=512, xD=96, K=7680) == SHAPE  # x_D not a power of two
    assert linear(lib, yl=1, yT=1024, yD=100, N=1500) == SHAPE  # y_D not a multiple of 8
    assert linear(lib, yl=2, ys=516, N=576, y1=FAKE) == SHAPE
    assert linear(lib, yl=3) == SHAPE
    assert linear(lib, xl=2) == SHAPE
    assert linear(lib, M=300000, K=8192) == SHAPE  # M*K >= 2^31
    assert linear(lib, x=FAKE + 8) == SHAPE
    assert linear(lib, bias=FAKE + 2) == SHAPE


def test_rmsnorm_dtype_validation(lib):
    def call(x=FAKE, w=FAKE, eps=1e-6, y=FAKE, n=16, R=1536, dt=0):
        return lib.mla_rmsnorm(x, w, eps, y, n, R, dt, None)
    assert call(n=0) == OK
    assert call(y=None) == NULL
    assert call(dt=5) == UNSUP
    assert call(R=0) == SHAPE
    assert call(R=9000) == SHAPE
    assert call(eps=-1.0) == SHAPE


CEILING_HEADER = os.path.join(ROOT, "include", "mla_ceiling.h")


def test_ceiling_exports_every_declared_symbol(lib):
    txt = open(CEILING_HEADER).read()
    names = sorted(set(re.findall(r"^\s*mla_status\s+(mla_\w+)\s*\(", txt, re.M)))
    assert names == sorted(_lib.CEILING_EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    m = re.search(r"#define MLA_CEILING_MFMA_OPERAND_BYTES (\d+)", txt)
    assert m and int(m.group(1)) == _lib.CEILING_MFMA_OPERAND_BYTES


def test_ceiling_validation(lib):
    # every call fails validation: nothing is launched
    assert lib.mla_ceiling_hbm_read(None, 16, FAKE, None) == NULL
    assert lib.mla_ceiling_hbm_read(FAKE, 16, None, None) == NULL
    assert lib.mla_ceiling_hbm_read(FAKE, 0, FAKE, None) == SHAPE
    assert lib.mla_ceiling_hbm_read(FAKE, 24, FAKE, None) == SHAPE
    assert lib.mla_ceiling_hbm_read(FAKE + 8, 32, FAKE, None) == SHAPE
    flops = ctypes.c_double(-1.0)
    assert lib.mla_ceiling_mfma(None, 1, 0, FAKE, ctypes.byref(flops), None) == NULL
    assert lib.mla_ceiling_mfma(FAKE, 1, 0, None, ctypes.byref(flops), None) == NULL
    assert lib.mla_ceiling_mfma(FAKE, 0, 0, FAKE, ctypes.byref(flops), None) == SHAPE
    assert lib.mla_ceiling_mfma(FAKE, 1, 2, FAKE, ctypes.byref(flops), None) == SHAPE
    assert lib.mla_ceiling_mfma(FAKE + 8, 1, 0, FAKE, ctypes.byref(flops), None) == SHAPE
    assert flops.value == -1.0
    v = ctypes.c_int32()
    assert lib.mla_device_info(0, None, ctypes.byref(v), ctypes.byref(v)) == NULL
