"""ctypes loader for libmxfp4moe.so (built in-tree by build.py).

Loading fails loudly: there is no fallback implementation behind this
package; if the library is missing, every call raises."""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmxfp4moe.so")

_c_int, _c_i64, _c_size, _p = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/mxfp4moe.h
SIGNATURES = {
    "mxm_version": (_c_int, []),
    "mxm_status_string": (ctypes.c_char_p, [_c_int]),
    "mxfp4_pack": (_c_int, [_p, _c_int, _c_i64, _c_i64, _p, _p, _p]),
    "mxfp4_unpack": (_c_int, [_p, _p, _c_i64, _c_i64, _p, _c_int, _p]),
    "moe_route_topk": (_c_int, [_p, _c_int, _c_int, _c_int, _p, _p, _p]),
    "moe_router_topk": (_c_int, [_p, _p, _p, _c_int, _c_int, _c_int, _c_int, _p, _p, _p, _p]),
    "dflash_verify_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "dflash_verify_accept": (_c_int, [_p, _p, _p, _p, _c_int, _c_int, _c_int, _p, _p, _p, _c_size,
                                      _p]),
    "moe_permute_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "moe_permute": (_c_int, [_p, _c_int, _c_int, _c_int, _p, _p, _p, _p, _p, _c_size, _p]),
    "moe_route_permute": (_c_int, [_p, _c_int, _c_int, _c_int, _p, _p, _p, _p, _p, _p, _p,
                                   _c_size, _p]),
    "moe_mxfp4_gate_up_swiglu": (_c_int, [_p, _p, _p, _c_int, _c_int, _c_int, _c_int, _c_int,
                                          _p, _p, _p, _p]),
    "moe_mxfp4_down": (_c_int, [_p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _p, _p, _p, _p]),
    "moe_combine": (_c_int, [_p, _p, _p, _c_int, _c_int, _c_int, _p, _p]),
    "mxm_stream_xor": (_c_int, [_p, _c_i64, _c_int, _p, _p]),
    "moe_mxfp4_decode_layer_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "moe_mxfp4_decode_layer": (_c_int, [_p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _p, _p,
                                        _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_size,
                                        _p]),
    "moe_mxfp4_layer_noalloc": (_c_int, [_p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _p, _p,
                                         _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_mxfp4_layer": (_c_int, [_p, _p, _c_int, _c_int, _c_int, _c_int, _c_int, _p, _p, _p, _p,
                                 _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _c_size, _p]),
}

_lib = None


class MxmError(RuntimeError):
    def __init__(self, status, name):
        self.status = status
        super().__init__("%s failed: %s" % (name, status_string(status)))


def lib():
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmxfp4moe.so is not built (%s); run "
                               "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_string(status):
    return lib().mxm_status_string(int(status)).decode()


def check(status, name):
    if status != 0:
        raise MxmError(status, name)
    return status
