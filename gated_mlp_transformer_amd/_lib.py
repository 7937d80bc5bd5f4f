"""ctypes loader for libmoeffn.so (the HIP kernels behind the C ABI in moeffn.h).

There is no fallback: if the library is missing, importing the binding fails.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoeffn.so")

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_size = ctypes.c_size_t

_SIGNATURES = {
    "mf_status_string": (ctypes.c_char_p, [_i32]),
    "mf_version": (ctypes.c_char_p, []),
    "rmsnorm": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _i32, _f32, _i32, _c_void_p]),
    "rmsnorm_quantize_fp8": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                    _i64, _i32, _f32, _c_void_p]),
    "packed_weights_bytes": (_size, [_i64, _i32, _i32, _i32]),
    "pack_weights": (_i32, [_c_void_p, _c_void_p, _i64, _i32, _i32, _i32, _c_void_p]),
    "pack_weights_kn": (_i32, [_c_void_p, _c_void_p, _i64, _i32, _i32, _i32, _c_void_p]),
    "moe_route_workspace_size": (_size, [_i64, _i32, _i32]),
    "moe_route": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _i32, _c_void_p,
                         _c_void_p, _c_void_p, _size, _c_void_p]),
    "moe_permute_workspace_size": (_size, [_i64, _i32, _i32]),
    "moe_permute": (_i32, [_c_void_p, _i64, _i32, _i32, _i32, _c_void_p, _i32, _i32, _c_void_p,
                           _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size,
                           _c_void_p]),
    "grouped_swiglu": (_i32, [_c_void_p, _c_void_p, _i64, _c_void_p, _i32, _i64, _i32, _i32,
                              _c_void_p, _c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p,
                              _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "grouped_gate_up": (_i32, [_c_void_p, _c_void_p, _i64, _c_void_p, _i32, _i64, _i32, _i32,
                               _c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p, _c_void_p,
                               _c_void_p]),
    "grouped_down": (_i32, [_c_void_p, _c_void_p, _i32, _i64, _i32, _i32, _c_void_p, _i32,
                            _c_void_p, _c_void_p, _c_void_p]),
    "moe_combine": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _i64, _c_void_p,
                           _c_void_p, _i32, _c_void_p]),
    "moe_permute_noalloc": (_i32, [_c_void_p, _i64, _i32, _i32, _i32, _c_void_p, _i32, _i32,
                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p]),
    "moe_dispatch_masked": (_i32, [_c_void_p, _i64, _i32, _i32, _i32, _i32, _c_void_p,
                                   _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
    "grouped_gate_up_masked": (_i32, [_c_void_p, _c_void_p, _i64, _c_void_p, _i32, _i32, _i32,
                                      _i32, _c_void_p, _c_void_p, _i32, _c_void_p, _c_void_p,
                                      _c_void_p, _c_void_p]),
    "grouped_down_masked": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _c_void_p,
                                   _i32, _c_void_p, _c_void_p, _c_void_p]),
    "quantize_fp8_rows": (_i32, [_c_void_p, _i64, _c_void_p, _i32, _c_void_p, _c_void_p,
                                 _c_void_p]),
    "grouped_gate_up_a8": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p, _i32, _i64,
                                  _i32, _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                  _c_void_p, _c_void_p]),
    "grouped_down_a8": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i32, _i32,
                               _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "mf_probe_mfma_bf16": (_i32, [_i32, _i32, _c_void_p, _c_void_p]),
    "mf_probe_hbm_read": (_i32, [_c_void_p, _i64, _i32, _c_void_p, _c_void_p]),
    "mf_probe_hbm_copy": (_i32, [_c_void_p, _c_void_p, _i64, _i32, _c_void_p]),
    "tp_shard_mlp": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32, _i32, _i32,
                            _c_void_p, _c_void_p, _c_void_p]),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


def load() -> ctypes.CDLL:
    """Load libmoeffn.so once and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; build it with `python gated_mlp_transformer_amd/build.py` "
            "(hipcc, gfx950). There is no non-HIP fallback.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
