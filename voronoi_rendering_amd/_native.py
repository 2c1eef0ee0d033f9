"""ctypes loader for libsad.so (the HIP library behind the SAD C ABI).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes as C
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libsad.so"

SAD_OK = 0
SAD_EINVAL = -1
SAD_EUNSUPPORTED = -2
SAD_EHIP = -3



class PassMaps(C.Structure):
    """struct sad_pass_maps of include/sad.h (device addresses, 0 for NULL)."""
    _fields_ = [("topk_prev", C.c_void_p), ("scores_prev", C.c_void_p), ("thr_prev", C.c_void_p),
                ("probe_prev", C.c_void_p), ("topk_next", C.c_void_p), ("scores_next", C.c_void_p),
                ("thr_next", C.c_void_p), ("probe_next", C.c_void_p), ("prev_bits", C.c_int32),
                ("next_bits", C.c_int32)]


# every symbol include/sad.h declares, with (restype, argtypes); a
# PassMaps argument is passed as C.byref(...) to a c_void_p slot
_f32p = C.c_void_p
_SIGS = {
    "sad_abi_version": (C.c_int, []),
    "sad_status_string": (C.c_char_p, [C.c_int]),
    "sad_prepare_sites": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]),
    "sad_propagate_topk": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_void_p, C.c_int32, C.c_uint64, C.c_uint32, C.c_int32,
                                     C.c_void_p]),
    "sad_propagate_pass": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_int32,
                                     C.c_uint64, C.c_uint32, C.c_int32, C.c_void_p]),
    "sad_step_fused_pass": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_int32,
                                      C.c_uint64, C.c_uint32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_void_p]),
    "sad_render_fwd": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                 C.c_void_p]),
    "sad_render_bwd": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "sad_site_stats_workspace_bytes": (C.c_size_t, [C.c_int32, C.c_int32]),
    "sad_site_stats_noalloc": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                         C.c_void_p, C.c_void_p]),
    "sad_site_stats": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "sad_budget_workspace_bytes": (C.c_size_t, [C.c_int32]),
    "sad_densify_prune": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                    C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_float, C.c_float, C.c_float,
                                    C.c_float, C.c_float, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "sad_init_workspace_bytes": (C.c_size_t, [C.c_int32, C.c_int32]),
    "sad_init_sites": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_float, C.c_uint64, C.c_float,
                                 C.c_float, C.c_float, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "sad_pack_sites": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                 C.c_void_p]),
    "sad_query_packed": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                   C.c_int64, C.c_void_p, C.c_void_p]),
    "sad_jfa_seed": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "sad_jfa_flood": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32,
                                C.c_int32, C.c_void_p]),
    "sad_step_fused": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                 C.c_void_p, C.c_void_p, C.c_int32, C.c_uint64, C.c_uint32, C.c_int32,
                                 C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "sad_adam_step": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                C.POINTER(C.c_float), C.c_float, C.c_float, C.c_float, C.c_float, C.c_float,
                                C.c_void_p, C.c_void_p]),
    "sad_widen_map": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "sad_adam_step_probe": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32,
                                      C.c_int32, C.POINTER(C.c_float), C.c_float, C.c_float, C.c_float, C.c_float,
                                      C.c_float, C.c_void_p, C.c_void_p, C.c_void_p]),
    "sad_query_points": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                   C.c_int64, C.c_void_p, C.c_void_p]),
}

_lib: C.CDLL | None = None


class SadError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {status}: {status_string(status)}")


def lib() -> C.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m voronoi_rendering_amd.build` "
                               "(or __graft_entry__.build()); there is no non-HIP implementation")
        L = C.CDLL(str(LIB_PATH))
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def symbols() -> list[str]:
    return list(_SIGS)


def status_string(status: int) -> str:
    return lib().sad_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != SAD_OK:
        raise SadError(fn, status)
