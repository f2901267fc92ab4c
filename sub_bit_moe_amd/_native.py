"""ctypes binding of libsbm.so (include/sbm.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsbm.so")

SBM_DICT_ENTRIES = 65536
SBM_DICT_WORDS = 131072
SBM_BLOCK = 1024
SBM_CODE_ALIGN = 8
SBM_F_RELU = 1
SBM_F_OUT_F32 = 2
SBM_F_IN_RMS = 4
SBM_F_MFMA = 8
SBM_F_MINMAX = 16
SBM_F_IMAGE4 = 32
SBM_F_DETERMINISTIC = 64
SBM_F_IN_BF16 = 128

STATUS = {0: "SBM_OK", -1: "SBM_EINVAL", -2: "SBM_EODD_WIDTH", -3: "SBM_ECORRUPT",
          -4: "SBM_EDICT", -5: "SBM_ERANGE", -6: "SBM_ENOSPACE", -7: "SBM_EHIP"}


class SbmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class MatrixDesc(C.Structure):
    _fields_ = [("code_base", C.c_uint64), ("off_base", C.c_uint64), ("scale_base", C.c_uint64),
                ("blk_base", C.c_uint64), ("n_codes", C.c_uint32), ("rows", C.c_int32),
                ("cols", C.c_int32), ("dict_tag", C.c_uint32)]


class Projection(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("row_off", C.c_void_p), ("bstart", C.c_void_p), ("scales", C.c_void_p),
                ("experts", C.c_void_p), ("n_experts", C.c_int32), ("rows", C.c_int32), ("cols", C.c_int32)]


P = C.c_void_p
_SIGS = {
    "sbm_last_error": (C.c_char_p, []),
    "sbm_version": (C.c_char_p, []),
    "sbm_build_dictionary": (C.c_int, [C.c_double, P, P]),
    "sbm_dictionary_checksum": (C.c_int, [P, P]),
    "sbm_dict_image_bytes": (C.c_size_t, []),
    "sbm_dict_image": (C.c_int, [P, P, C.c_size_t]),
    "sbm_dict_image4_bytes": (C.c_size_t, []),
    "sbm_dict_image4": (C.c_int, [P, P, C.c_size_t]),
    "sbm_encode_size": (C.c_int, [P, C.c_int32, C.c_int32, P, P]),
    "sbm_encode_matrix": (C.c_int, [P, C.c_int32, C.c_int32, P, P, C.c_uint64, P, P, P]),
    "sbm_encode_experts": (C.c_int, [C.c_int32, P, C.c_int32, C.c_int32, P, P, C.c_uint64, P, P, C.c_uint64,
                                     P, P, P]),
    "sbm_block_starts": (C.c_int, [P, C.c_uint64, P, P]),
    "sbm_validate_stream": (C.c_int, [P, C.c_uint64, P, C.c_int32, C.c_int32, P]),
    "sbm_decode_ref": (C.c_int, [P, P, C.c_int32, C.c_int32, P, P, P, P]),
    "sbm_decode_dense": (C.c_int, [P, C.c_uint64, P, C.c_int32, C.c_int32, P, C.c_uint32, P, P, P]),
    "sbm_workspace_bytes": (C.c_size_t, [C.c_int32, C.c_int32]),
    "sbm_moe_fused_decode_matvec": (C.c_int, [P, P, P, P, P, C.c_int32, C.c_int32, C.c_int32, P,
                                              P, P, C.c_int32, P, C.c_uint32, P, C.c_size_t, P]),
    "sbm_moe_fused_decode_matvec_noalloc": (C.c_int, [P, P, P, P, P, C.c_int32, C.c_int32, C.c_int32, P,
                                                      P, P, C.c_int32, P, C.c_uint32, P, P]),
    "sbm_ffn_workspace_bytes": (C.c_size_t, [C.c_int32, C.c_int32]),
    "sbm_moe_fused_ffn": (C.c_int, [P, P, P, P, P, C.c_int32, P, P, C.c_uint32, P, C.c_size_t, P]),
    "sbm_layers_workspace_bytes": (C.c_size_t, [C.c_int32, C.c_int32, C.c_int32]),
    "sbm_moe_fused_layers": (C.c_int, [P, P, C.c_int32, P, P, P, C.c_int32, P, P, C.c_uint32, P, C.c_size_t, P]),
    "sbm_stream_read": (C.c_int, [P, C.c_uint64, P, C.c_uint32, P]),
    "sbm_workspace_error": (C.c_int, [P, P, P]),
    "sbm_rms_glue": (C.c_int, [P, C.c_int32, C.c_int32, P, P]),
    "sbm_trie_words": (C.c_size_t, []),
    "sbm_build_trie": (C.c_int, [P, P]),
    "sbm_gen_count": (C.c_int, [C.c_uint64, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                C.c_uint32, P, P, P]),
    "sbm_gen_layout": (C.c_int, [P, C.c_int32, C.c_int32, C.c_int32, P, P, P, C.c_uint64, P]),
    "sbm_gen_write": (C.c_int, [C.c_uint64, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                C.c_uint32, P, P, P, P, P, P, P, P]),
}

_lib = None


def lib():
    """Load libsbm.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m sub_bit_moe_amd.build")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def check(status: int) -> None:
    if status != 0:
        raise SbmError(status, lib().sbm_last_error().decode(errors="replace"))
