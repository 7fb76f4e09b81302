"""ctypes loader and signatures of libmla.so (see include/mla.h).

Importing this module loads the in-tree library and fails loudly when it has
not been built: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")

MLA_DTYPE_F32 = 0
MLA_DTYPE_BF16 = 1

STATUS_NAMES = {
    0: "MLA_OK", -1: "MLA_ERR_ARG", -2: "MLA_ERR_SHAPE", -3: "MLA_ERR_ROPE", -4: "MLA_ERR_SELECTION",
    -5: "MLA_ERR_WORKSPACE", -6: "MLA_ERR_DEVICE", -7: "MLA_ERR_UNSUPPORTED",
}

EXPORTS = (
    "mla_last_error", "mla_version", "mla_rope_partial_interleaved", "mla_absorb_q", "mla_decode_latent_attn",
    "mla_decode_combine", "mla_absorb_v", "mla_prefill_reconstructed", "mla_dsa_topk_select",
    "mla_append_compressed", "mla_o_proj_workspace_bytes", "mla_o_proj", "mla_decode_query",
    "mla_decode_combine_v", "mla_decode_stream_probe", "mla_dsa_topk_select_noalloc",
)

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_f64 = ctypes.c_double
_pi32 = ctypes.POINTER(ctypes.c_int32)
_pi64 = ctypes.POINTER(ctypes.c_int64)
_psz = ctypes.POINTER(ctypes.c_size_t)

_SIGNATURES = {
    "mla_last_error": (ctypes.c_char_p, []),
    "mla_version": (ctypes.c_int, []),
    "mla_rope_partial_interleaved": (ctypes.c_int, [
        _i32, _p, _p, _i32, _i32, _i32, _i32, _i64, _i64, _i64, _i32, _f64, _pi64, _i32, _p]),
    "mla_absorb_q": (ctypes.c_int, [_i32, _p, _i64, _i64, _p, _p, _i32, _i32, _i32, _i32, _i32, _p]),
    "mla_decode_query": (ctypes.c_int, [
        _i32, _p, _i64, _i64, _p, _p, _i64, _i64, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _pi64, _f64, _p]),
    "mla_decode_latent_attn": (ctypes.c_int, [
        _i32, _p, _p, _i64, _i64, _p, _i64, _i64, _p, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
        _pi32, _p, _pi32, _f32, _i32, _i32, _p, _p, _i32, _p, _p]),
    "mla_decode_combine": (ctypes.c_int, [_i32, _p, _p, _i32, _i32, _i32, _i32, _pi32, _p, _p, _p]),
    "mla_absorb_v": (ctypes.c_int, [_i32, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p]),
    "mla_decode_stream_probe": (ctypes.c_int, [
        _i32, _p, _i64, _i64, _p, _i64, _i64, _i32, _i32, _i32, _i32, _pi32, _i32, _p]),
    "mla_decode_combine_v": (ctypes.c_int, [
        _i32, _i32, _p, _p, _i32, _i32, _i32, _i32, _pi32, _p, _i32, _i32, _p, _p, _p, _p]),
    "mla_dsa_topk_select": (ctypes.c_int, [_p, _i64, _i32, _pi32, _i32, _p, _pi32, _p, _psz, _p]),
    "mla_dsa_topk_select_noalloc": (ctypes.c_int, [_p, _i64, _i32, _pi32, _i32, _p, _pi32, _p]),
    "mla_o_proj_workspace_bytes": (ctypes.c_int, [_i32, _i64, _i32, _i32, _psz]),
    "mla_o_proj": (ctypes.c_int, [_i32, _p, _i64, _i32, _p, _i32, _p, _p, ctypes.c_size_t, _p]),
    "mla_append_compressed": (ctypes.c_int, [
        _i32, _p, _i64, _i64, _i32, _i32, _i32, _i32, _p, _f32, _pi64, _f64, _p, _i64, _i64, _p, _i64, _i64, _i32, _p]),
    "mla_prefill_reconstructed": (ctypes.c_int, [
        _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p, _pi64, _f64, _pi32, _f32,
        _p, _psz, _p, _p]),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libmla.so not found at {LIB_PATH}: build it with `python mla_latent_kv_partial_amd/build.py` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.mla_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")


def check(status: int, where: str) -> None:
    if status != 0:
        raise MlaError(status, where)


def i32_array(values):
    vals = [int(v) for v in values]
    return (ctypes.c_int32 * max(1, len(vals)))(*vals)


def i64_array(values):
    vals = [int(v) for v in values]
    return (ctypes.c_int64 * max(1, len(vals)))(*vals)
