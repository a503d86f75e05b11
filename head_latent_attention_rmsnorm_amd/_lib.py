"""ctypes loader and signatures of libmla.so (the C ABI declared in
include/mla.h). No arithmetic of the method lives here.

The library is loaded from this package's directory. If it is missing the
import fails loudly: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

# torch ships its own HIP runtime (same soname as ROCm's). It must be loaded
# before libmla.so so that the library binds to that one runtime: two HIP
# runtimes in one process would not share streams or allocations.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

MLA_OK = 0
STATUS = {
    0: "MLA_OK", -1: "MLA_ERR_NULL", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_UNSUPPORTED",
    -4: "MLA_ERR_ROPE_TYPE", -5: "MLA_ERR_WORKSPACE", -6: "MLA_ERR_HIP",
}
ROPE_DEFAULT, ROPE_YARN = 0, 1
PAIR_HALF, PAIR_INTERLEAVED = 0, 1
DTYPE_BF16, DTYPE_FP16 = 0, 1
V_ROWS, V_COLS = 0, 1
LIN_ROWS, LIN_HEADS, LIN_SPLIT = 0, 1, 2

# every symbol the header declares
EXPORTS = [
    "mla_rope_table_build", "mla_softmax_scale", "mla_latent_rmsnorm", "mla_kv_expand",
    "mla_prefill_attention", "mla_decode_attention", "mla_absorb_prepare", "mla_latent_cache_append",
    "mla_decode_absorbed", "mla_rotate_rope_key", "mla_prefill_attention_cached", "mla_decode_latent_expanded",
    "mla_linear", "mla_rmsnorm", "mla_decode_attention_noalloc", "mla_latent_prepare", "mla_status_string",
]
DECODE_SCRATCH_BYTES = 16 << 20  # MLA_DECODE_SCRATCH_BYTES
# the measurement aids mla_ceiling.h declares
CEILING_EXPORTS = ["mla_ceiling_hbm_read", "mla_ceiling_mfma", "mla_device_info"]
CEILING_MFMA_OPERAND_BYTES = 49152


class RopeParams(ctypes.Structure):
    """Mirror of `mla_rope_params`."""

    _fields_ = [
        ("rope_dim", ctypes.c_int32),
        ("type", ctypes.c_int32),
        ("base", ctypes.c_double),
        ("factor", ctypes.c_double),
        ("original_max_pos", ctypes.c_int32),
        ("beta_fast", ctypes.c_double),
        ("beta_slow", ctypes.c_double),
        ("mscale", ctypes.c_double),
        ("mscale_all_dim", ctypes.c_double),
    ]


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


_lib = None

P = ctypes.c_void_p
I32 = ctypes.c_int32
F32 = ctypes.c_float
SZ = ctypes.POINTER(ctypes.c_size_t)


def load() -> ctypes.CDLL:
    """Load libmla.so once; raise ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m head_latent_attention_rmsnorm_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.mla_rope_table_build.argtypes = [ctypes.POINTER(RopeParams), I32, P, P, ctypes.POINTER(ctypes.c_double), P]
    lib.mla_softmax_scale.argtypes = [ctypes.POINTER(RopeParams), I32, ctypes.POINTER(ctypes.c_double)]
    lib.mla_latent_rmsnorm.argtypes = [P, P, F32, P, I32, I32, P]
    lib.mla_kv_expand.argtypes = [P, P, I32, I32, I32, I32, I32, I32, P, I32, P, I32, I32, I32, I32, I32, P, P, P,
                                  I32, P, I32, I32, P]
    lib.mla_prefill_attention.argtypes = [P, P, P, P, I32, I32, I32, P, P, I32, P, I32, I32, I32, I32, I32, I32, F32,
                                          I32, P, P, P, SZ, P]
    lib.mla_decode_attention.argtypes = [P, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F32, I32, I32,
                                         P, SZ, P, P]
    lib.mla_decode_attention_noalloc.argtypes = [P, P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F32,
                                                 I32, I32, P, P]
    lib.mla_latent_prepare.argtypes = [P, P, F32, P, P, P, I32, P, I32, I32, I32, I32, I32, P, P, P]
    lib.mla_absorb_prepare.argtypes = [P, I32, I32, I32, I32, P, P]
    lib.mla_latent_cache_append.argtypes = [P, P, F32, P, P, P, I32, P, I32, I32, I32, I32, P, I32, P]
    lib.mla_decode_absorbed.argtypes = [P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, F32, I32,
                                        I32, P, SZ, P, P]
    lib.mla_rotate_rope_key.argtypes = [P, P, P, I32, P, I32, I32, I32, I32, P, I32, I32, I32, P]
    lib.mla_prefill_attention_cached.argtypes = [P, P, P, P, I32, I32, P, P, I32, P, I32, I32, I32, I32, I32, I32,
                                                 I32, I32, F32, I32, P, P, P]
    lib.mla_decode_latent_expanded.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, F32, I32,
                                               I32, P, SZ, P, P]
    lib.mla_rmsnorm.argtypes = [P, P, F32, P, I32, I32, I32, P]
    lib.mla_linear.argtypes = [P, I32, I32, I32, P, P, I32, I32, I32, P, P, I32, I32, I32, I32, P]
    for name in EXPORTS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    lib.mla_ceiling_hbm_read.argtypes = [P, ctypes.c_size_t, P, P]
    lib.mla_ceiling_mfma.argtypes = [P, I32, I32, P, ctypes.POINTER(ctypes.c_double), P]
    lib.mla_device_info.argtypes = [I32, ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32)]
    for name in CEILING_EXPORTS:
        getattr(lib, name).restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != MLA_OK:
        raise MlaError(fn, status)
