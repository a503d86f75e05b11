"""Helpers shared by the GPU tests: upload of seeded inputs, the end-to-end
tolerance, and per-head slicing of a workload for the oracle."""

import dataclasses
import sys

import numpy as np
import torch

import workloads

# Tolerance of the whole path against the fp64 oracle (bf16 inputs, fp32
# accumulation; bf16 rounding of the normalised latent, of k_nope/v, of the
# rotated rotary parts and of P dominate).
MAX_ABS = 2e-2
REL_L2 = 5e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_gpu(inp: dict) -> dict:
    return {k: v.cuda() for k, v in inp.items()}


def f64(t) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def errors(got, ref) -> tuple:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    return float(np.max(np.abs(d))), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, what: str, max_abs=MAX_ABS, rel_l2=REL_L2):
    ma, rl = errors(got, ref)
    say(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert np.all(np.isfinite(np.asarray(got))), f"{what}: non-finite values"
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max_abs={ma:.3e} rel_l2={rl:.3e}"


def head_view(w: workloads.Workload, inp: dict, h: int):
    """The workload restricted to head h (heads are independent): q of that
    head and the kv_b_proj rows of that head."""
    n = w.Dn + w.Dv
    sub = {
        "q": inp["q"][:, h:h + 1].contiguous(),
        "latent": inp["latent"], "k_pe": inp["k_pe"], "gain": inp["gain"],
        "W": inp["W"][h * n:(h + 1) * n].contiguous(),
    }
    return dataclasses.replace(w, H=1), sub
