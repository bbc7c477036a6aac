"""ctypes loader for libsala.so.  No compute happens here."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# SALA_LIB_PATH selects another build of the library (the sanitizer build of the ABI checks)
LIB_PATH = os.environ.get("SALA_LIB_PATH") or os.path.join(_HERE, "libsala.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "sala.h")

SALA_F32 = 0
SALA_BF16 = 1
STATUS = {0: "SALA_OK", -1: "SALA_ERR_INVALID_ARG", -2: "SALA_ERR_UNSUPPORTED", -3: "SALA_ERR_WORKSPACE",
          -4: "SALA_ERR_HIP"}

_i, _p, _f, _z, _ll = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t, ctypes.c_longlong

_SIGS = {
    "sala_linear_prefill": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _z, _p]),
    "sala_linear_prefill_workspace": (_z, [_i, _i, _i, _i, _i, _i]),
    "sala_linear_prefill_backward": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _z,
                                          _p]),
    "sala_linear_decode": (_i, [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]),
    "sala_linear_prefill_fused": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _f, _f, _ll,
                                       _p, _p, _z, _p]),
    "sala_linear_decode_fused": (_i, [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _f, _f, _p, _p, _p]),
    "sala_qk_norm_rope": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _f, _f, _ll, _p]),
    "sala_output_gate": (_i, [_i, _z, _p, _p, _p, _p]),
    "sala_sparse_prefill_chunk_workspace": (_z, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "sala_sparse_prefill_chunk": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p,
                                       _p, _p, _p, _z, _p]),
    "sala_sparse_decode_step_workspace": (_z, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "sala_sparse_decode_step": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p,
                                     _p, _p, _z, _p]),
    "sala_sparse_decode_step_noalloc": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p,
                                             _p, _p, _p]),
    "sala_sparse_select": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _z, _p]),
    "sala_sparse_select_workspace": (_z, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _i, _i]),
    "sala_sparse_prefill": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _z, _p]),
    "sala_sparse_prefill_workspace": (_z, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "sala_sparse_decode": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _z, _p]),
    "sala_sparse_decode_workspace": (_z, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "sala_sparse_prefill_backward": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p, _p, _p, _z,
                                          _p]),
    "sala_sparse_prefill_backward_workspace": (_z, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "sala_dense_prefill": (_i, [_i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p]),
    "sala_ceiling_mfma": (_i, [_i, _i, _p, _p]),
    "sala_ceiling_copy": (_i, [_p, _p, _z, _p]),
    "sala_ceiling_read": (_i, [_p, _z, _p, _p]),
    "sala_workspace_bytes": (_z, [_i, ctypes.POINTER(ctypes.c_int64), _i]),
    "sala_status_string": (ctypes.c_char_p, [_i]),
    "sala_last_error": (ctypes.c_char_p, []),
    "sala_version": (ctypes.c_char_p, []),
}

_lib = None


class SalaError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}: {detail}")
        self.status = status


def lib():
    """The loaded library.  Raises if libsala.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m hybrid_sparse_linear_amd.build` "
                               "(or __graft_entry__.build()); there is no fallback path")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def call(name, *args):
    """Call an entry point; raise SalaError on a negative status."""
    status = getattr(lib(), name)(*args)
    if status != 0:
        raise SalaError(name, status, lib().sala_last_error().decode())
    return status
