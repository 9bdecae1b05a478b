"""ctypes loader for libpa.so: one prototype per entry point of include/pa.h.

Argument marshalling only; the library does all the work.  Importing fails
loudly when the built library is missing (there is no fallback path).
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_OK = 0
PA_ERR_NULL = 1
PA_ERR_INVALID = 2
PA_ERR_UNSUPPORTED = 3
PA_ERR_WORKSPACE = 4
PA_ERR_HIP = 5

PA_F32 = 0
PA_BF16 = 1
PA_BLOCK_SIZE = 16
PA_MAX_SPLITS = 256
PA_NOALLOC_SCRATCH_BYTES = 16 << 20

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in the order of include/pa.h
PROTOTYPES = {
    "pa_kv_write": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _i32, _vp]),
    "pa_attention_fwd": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                _i32, _i32, _i32, _i32, _i64, _f32, _i32, _vp, _vp, _vp, _sz,
                                _i32, _vp]),
    "pa_decode_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                              _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32, _i32, _vp, _vp,
                              _vp, _sz, _i32, _vp]),
    "pa_decode_step_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                      _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32,
                                      _i32, _vp, _vp, _i32, _vp]),
    "pa_attention_fwd_cascade": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _i32, _i32, _i64, _f32, _i32, _vp,
                                        _i32, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "pa_cascade_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_step_cascade": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                      _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32,
                                      _i32, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _sz, _vp]),
    "pa_rope_kv_write": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                _i32, _i32, _i64, _i32, _vp]),
    "pa_kv_write_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64,
                               _i32, _vp]),
    "pa_attention_fwd_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                    _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32, _i32, _vp,
                                    _vp, _vp, _sz, _vp]),
    "pa_decode_step_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                  _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i64, _f32,
                                  _i32, _vp, _vp, _vp, _sz, _i32, _vp]),
    "pa_attention_workspace_init": (_i32, [_vp, _sz, _vp]),
    "pa_split_combine": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp]),
    "pa_attention_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_choose_num_splits": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_capture_size": (_i32, [_i32, _i32]),
    "pa_status_string": (ctypes.c_char_p, [_i32]),
    "pa_version": (_i32, []),
    "pa_set_unshared_blocks": (_i32, [_i32]),
    "pa_trace_begin": (_i32, [_i32]),
    "pa_trace_end": (_i32, []),
    "pa_trace_read": (_i32, [ctypes.POINTER(_i32), ctypes.POINTER(_f32), _i32]),
    "pa_kernel_name": (ctypes.c_char_p, [_i32]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first "
            "(python paged_attention_flat_amd/build.py)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in PROTOTYPES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = load()
