"""ctypes binding of the C ABI declared in include/fa.h.

Argument marshalling only: every step of the attention forward, the merge and
the backward runs in the HIP kernels of libfa_mi355x.so.  There is no fallback of any kind: if the library
is missing or cannot be loaded, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libfa_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

# Mirrors enum fa_status in include/fa.h.
FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_SHAPE = 2
FA_ERR_HEADDIM = 3
FA_ERR_SCALE = 4
FA_ERR_CAUSAL = 5
FA_ERR_ALIGN = 6
FA_ERR_ALIAS = 7
FA_ERR_LAUNCH = 8
FA_ERR_SCRATCH = 9
FA_BWD_SCRATCH_ROWS = 1 << 21

EXPORTS = ("fa_fwd", "fa_fwd_f32", "fa_fwd_kv", "fa_merge", "fa_bwd", "fa_bwd_noalloc",
           "fa_fwd_plan", "fa_fwd_kv_plan", "fa_status_str", "fa_abi_version")
ABI_VERSION = 1

# Pipeline-study builds of the same library: the bf16 forward's K/V tile
# pipeline in another mode (FA_PIPE at build time; see the pipeline modes in
# csrc/fa_fwd.hip).  Everything else is the same code.
PIPE_VARIANTS = {"noprefetch": 1, "ksplit": 2, "ring3": 3, "ring4": 4, "mfma_only": 5,
                 "ring256": 6}

_lock = threading.Lock()
_lib = None
_variants = {}


def variant_path(name: str) -> str:
    if name not in PIPE_VARIANTS:
        raise ValueError(f"unknown pipeline variant {name!r} (one of {sorted(PIPE_VARIANTS)})")
    return os.path.join(PKG, f"libfa_mi355x_pipe_{name}.so")


def load_variant(name: str) -> ctypes.CDLL:
    """Load (once) a pipeline-study build; raises if it is not built."""
    p = variant_path(name)
    with _lock:
        if name in _variants:
            return _variants[name]
    lib = load(p)
    with _lock:
        _variants[name] = lib
    return lib


class FAError(RuntimeError):
    """A non-zero fa_status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_str(status)})")


def _declare(lib: ctypes.CDLL) -> None:
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sig = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.fa_fwd.argtypes = sig
    lib.fa_fwd.restype = i
    lib.fa_fwd_f32.argtypes = sig
    lib.fa_fwd_f32.restype = i
    lib.fa_fwd_kv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    lib.fa_fwd_kv.restype = i
    lib.fa_merge.argtypes = [vp, vp, i, i, i, i, i, vp, vp, vp]
    lib.fa_merge.restype = i
    lib.fa_bwd.argtypes = [vp] * 10 + [i, i, i, i, i, f, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + [i, i, i, i, i, f, vp]
    lib.fa_bwd_noalloc.restype = i
    ip = ctypes.POINTER(i)
    lib.fa_fwd_plan.argtypes = [i, i, i, i, i, i, ip, ip, ip, ip]
    lib.fa_fwd_plan.restype = i
    lib.fa_fwd_kv_plan.argtypes = [i, i, i, i, i, i, ip, ip, ip, ip]
    lib.fa_fwd_kv_plan.restype = i
    lib.fa_status_str.argtypes = [i]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (once) and return the HIP library; raises if it is not built."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"{p} is not built; run `python -m exact_attention_67_amd.build` "
                "(there is no fallback path)")
        lib = ctypes.CDLL(p)
        _declare(lib)
        if lib.fa_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{p}: ABI version {lib.fa_abi_version()} != {ABI_VERSION}")
        if path is None:
            _lib = lib
        return lib


def status_str(status: int) -> str:
    return load().fa_status_str(int(status)).decode()


def fa_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, D: int,
           causal: int, scale: float, stream: int | None) -> int:
    """Raw C call on device addresses (ints).  Returns the fa_status."""
    return load().fa_fwd(q, k, v, o, lse, B, H, S, D, causal, scale, stream)


def fa_fwd_f32(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, S: int, D: int,
               causal: int, scale: float, stream: int | None) -> int:
    """Raw C call on device addresses (ints).  Returns the fa_status."""
    return load().fa_fwd_f32(q, k, v, o, lse, B, H, S, D, causal, scale, stream)


def fa_fwd_kv(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Sq: int, Sk: int,
              D: int, causal: int, scale: float, stream: int | None) -> int:
    """Raw C call on device addresses (ints).  Returns the fa_status."""
    return load().fa_fwd_kv(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, stream)


def fa_merge(o_parts: int, lse_parts: int, G: int, B: int, H: int, S: int, D: int, o: int,
             lse: int, stream: int | None) -> int:
    """Raw C call on device addresses (ints).  Returns the fa_status."""
    return load().fa_merge(o_parts, lse_parts, G, B, H, S, D, o, lse, stream)


def fa_bwd(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int, dv: int,
           delta: int, B: int, H: int, S: int, D: int, causal: int, scale: float,
           stream: int | None) -> int:
    """Raw C call on device addresses (ints).  Returns the fa_status."""
    return load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, S, D, causal, scale,
                         stream)


def fa_bwd_noalloc(q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int,
                   dv: int, B: int, H: int, S: int, D: int, causal: int, scale: float,
                   stream: int | None) -> int:
    """Raw C call on device addresses (ints); Delta in the library's fixed
    scratch array (no allocation).  Returns the fa_status."""
    return load().fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, B, H, S, D, causal, scale,
                                 stream)


def fa_fwd_plan(B: int, H: int, S: int, D: int, causal: int, elem_bytes: int) -> dict:
    """Launch shape the library uses for this problem (host-only query).
    Returns {rows_per_group, keys_per_tile, threads, groups}; raises FAError."""
    out = [ctypes.c_int(-1) for _ in range(4)]
    st = load().fa_fwd_plan(B, H, S, D, causal, elem_bytes, *[ctypes.byref(x) for x in out])
    if st != FA_OK:
        raise FAError(st, "fa_fwd_plan")
    return dict(zip(("rows_per_group", "keys_per_tile", "threads", "groups"),
                    (x.value for x in out)))


def fa_fwd_kv_plan(B: int, H: int, Sq: int, Sk: int, D: int, causal: int) -> dict:
    """Launch shape fa_fwd_kv uses for Sq queries against Sk keys (host-only
    query).  Returns {rows_per_group, keys_per_tile, threads, groups}; raises
    FAError."""
    out = [ctypes.c_int(-1) for _ in range(4)]
    st = load().fa_fwd_kv_plan(B, H, Sq, Sk, D, causal, *[ctypes.byref(x) for x in out])
    if st != FA_OK:
        raise FAError(st, "fa_fwd_kv_plan")
    return dict(zip(("rows_per_group", "keys_per_tile", "threads", "groups"),
                    (x.value for x in out)))
