"""GPU test of the allocation-free decode entry point: mla_decode_attention_noalloc
(split partials in the library's static per-GPU scratch) must give the bits of
mla_decode_attention (partials in a caller workspace) with the same split
count, on consecutive calls of decreasing size that share the scratch, and
agree with the fp64 oracle's decode attention (Kimi-K2 "Query content heads",
section "Join query parts")."""

import numpy as np
import pytest
import torch

import workloads
from oracle import mla_oracle as O
from tests.gpu_util import assert_close, f64, say

# a plain import: a missing or stale libmla.so must fail these tests, not skip them
import head_latent_attention_rmsnorm_amd as M  # noqa: E402

pytestmark = pytest.mark.gpu
api, pipeline = M.api, M.pipeline


def case(B, H, Tcap, Dn, Dr, Dv, seed, lengths, cache_dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, 1, Dn + Dr, generator=g).to(torch.bfloat16)
    kc = torch.randn(B, H, Tcap, Dn + Dr, generator=g).to(cache_dtype)
    vc = torch.randn(B, H, Tcap, Dv, generator=g).to(cache_dtype)
    seq = torch.tensor(lengths, dtype=torch.int32)
    return q, kc, vc, seq, seq - 1


def oracle(q, kc, vc, seq, qpos, Dn, spec, pairing):
    Dr = q.shape[-1] - Dn
    Tcap = kc.shape[2]
    cos, sin = O.rope_table(spec, Dr, Tcap)
    scale = O.softmax_scale(spec, Dn + Dr)
    B, H = q.shape[:2]
    ref = np.empty((B, H, 1, vc.shape[-1]))
    for b in range(B):
        L, p = int(seq[b]), int(qpos[b])
        for h in range(H):
            qf = f64(q[b, h, 0])
            Q = np.concatenate([qf[:Dn], O.rotate(qf[Dn:], cos[p], sin[p], pairing)])[None]
            ref[b, h] = O.attention(Q, f64(kc[b, h, :L]), f64(vc[b, h, :L]), scale, np.array([p]), np.arange(L))
    return ref


def test_noalloc_decode_matches_workspace_entry_point():
    spec = workloads.YARN_KIMI
    runs = [
        # (B, H, Tcap, Dn, Dr, Dv, seed, lengths, splits): the automatic split
        # count is 8 for the first call and 3 for the second, smaller one
        (4, 16, 2000, 128, 64, 128, 71, [2000, 1, 777, 1500], 0),
        (2, 8, 700, 128, 64, 128, 72, [700, 300], 0),
        # 256/256 heads, explicit split counts, then one split (no scratch)
        (3, 4, 900, 192, 64, 256, 73, [900, 33, 512], 5),
        (3, 4, 900, 192, 64, 256, 73, [900, 33, 512], 1),
    ]
    for (B, H, Tcap, Dn, Dr, Dv, seed, lengths, splits) in runs:
        pairing = "interleaved" if Dv == 256 else "half"
        say(f"[noalloc] B={B} H={H} Tcap={Tcap} {Dn + Dr}/{Dv} splits={splits or 'auto'}")
        q, kc, vc, seq, qpos = case(B, H, Tcap, Dn, Dr, Dv, seed, lengths)
        g = [t.cuda() for t in (q, kc, vc, seq, qpos)]
        tab = pipeline.build_table(api.params_from(spec, Dr), Tcap, Dn + Dr)
        ref_ws = api.mla_decode_attention(*g, tab.cos, tab.sin, tab.scale, Dn, pairing, splits)
        out = torch.empty((B, H, 1, Dv), dtype=torch.bfloat16, device="cuda")
        got = api.mla_decode_attention_noalloc(*g, tab.cos, tab.sin, tab.scale, Dn, pairing, splits, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref_ws), "no-alloc decode differs from the workspace entry point"
        assert_close(f64(got.cpu()), oracle(q, kc, vc, seq, qpos, Dn, spec, pairing), "no-alloc decode vs oracle")


def test_noalloc_decode_rejects_oversized_partials():
    """Partials beyond the 16 MiB scratch are refused before anything is
    queued: the output is left untouched."""
    B, H, Tcap, Dn, Dr, Dv = 32, 64, 1100, 128, 64, 128
    spec = workloads.YARN_KIMI
    assert B * H * 16 * (Dv + 2) * 4 > M._lib.DECODE_SCRATCH_BYTES
    q = torch.zeros((B, H, 1, Dn + Dr), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, H, Tcap, Dn + Dr), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros((B, H, Tcap, Dv), dtype=torch.bfloat16, device="cuda")
    seq = torch.full((B,), Tcap, dtype=torch.int32, device="cuda")
    tab = pipeline.build_table(api.params_from(spec, Dr), Tcap, Dn + Dr)
    out = torch.full((B, H, 1, Dv), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M._lib.MlaError):
        api.mla_decode_attention_noalloc(q, kc, vc, seq, seq - 1, tab.cos, tab.sin, tab.scale, Dn, "half", 16,
                                         out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)
