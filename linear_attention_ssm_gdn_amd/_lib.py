"""ctypes mirror of include/gdn.h and the loader of libgdn.so.

The library is loaded after torch so that it binds to the HIP runtime torch
already holds (both answer to the soname libamdhip64.so.7).  There is no
fallback: a missing library or symbol raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdn.so")

ABI_VERSION = 2

GDN_OK, GDN_ERR_ARG, GDN_ERR_UNSUPPORTED, GDN_ERR_LAUNCH = 0, 1, 2, 3
GDN_F32, GDN_BF16 = 0, 1
GDN_SPEC_ONEPAGE, GDN_SPEC_SLOTS = 0, 1
GDN_DEVERR_PAGE, GDN_DEVERR_BATCH, GDN_DEVERR_ACCEPTED, GDN_DEVERR_PARITY, GDN_DEVERR_CACHE = 1, 2, 4, 8, 16
GDN_PATH_TOKEN, GDN_PATH_CHUNKED = 0, 1
GDN_PREFILL_MAX_DEFAULT = -1
GDN_MIXED_AUTO, GDN_MIXED_ONE_LAUNCH, GDN_MIXED_TWO_LAUNCHES = 0, 1, 2
GDN_NOALLOC_SYNC_WORDS = 65536

SYMBOLS = ("gdn_abi_version", "gdn_status_str", "gdn_spec_page_layout", "gdn_chunked_workspace_bytes",
           "gdn_conv_update", "gdn_recurrent_seq", "gdn_recurrent_seq_noalloc", "gdn_chunked_prefill", "gdn_prefill_path", "gdn_prefill",
           "gdn_spec_verify", "gdn_spec_verify_cached", "gdn_prefix_restore", "gdn_mixed_step",
           "gdn_mixed_launches", "gdn_mixed_step_launches")

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class GdnDims(ctypes.Structure):
    _fields_ = [("h_k", _i32), ("h_v", _i32), ("d_k", _i32), ("d_v", _i32), ("conv_w", _i32),
                ("n_spec", _i32), ("act_dtype", _i32), ("state_dtype", _i32),
                ("scale", ctypes.c_float), ("l2_eps", ctypes.c_float)]


class GdnParams(ctypes.Structure):
    _fields_ = [("conv_w", _vp), ("a_log", _vp), ("dt_bias", _vp)]


class GdnBatch(ctypes.Structure):
    _fields_ = [("cu_seqlens", _vp), ("page_idx", _vp), ("has_init", _vp), ("n_seqs", _i32),
                ("max_seqlen", _i32), ("n_rows", _i64)]


class GdnConvPool(ctypes.Structure):
    _fields_ = [("base", _vp), ("page_stride", _i64), ("rows", _i32), ("n_pages", _i32), ("sync", _vp)]


class GdnStatePool(ctypes.Structure):
    _fields_ = [("base", _vp), ("page_stride", _i64), ("n_pages", _i32)]


class GdnSpecLayout(ctypes.Structure):
    _fields_ = [("page_bytes", ctypes.c_size_t), ("header_off", ctypes.c_size_t),
                ("state_off", ctypes.c_size_t), ("record_off", ctypes.c_size_t),
                ("record_row_bytes", ctypes.c_size_t)]


class GdnPrefixCache(ctypes.Structure):
    _fields_ = [("entry", _vp), ("row", _vp), ("state", GdnStatePool), ("conv", GdnConvPool)]


class GdnSeqPart(ctypes.Structure):
    _fields_ = [("x", _vp), ("x_stride", _i64), ("a", _vp), ("b", _vp), ("ab_stride", _i64),
                ("batch", ctypes.POINTER(GdnBatch)), ("conv", GdnConvPool), ("state", GdnStatePool), ("o", _vp),
                ("spec_pages", _vp), ("spec_page_bytes", _i64), ("spec_n_pages", _i32)]


class GdnVerifyPart(ctypes.Structure):
    _fields_ = [("layout", _i32), ("x", _vp), ("x_stride", _i64), ("a", _vp), ("b", _vp), ("ab_stride", _i64),
                ("n_req", _i32), ("n_cand", _i32), ("req_page", _vp), ("num_accepted", _vp),
                ("step_parity", _vp), ("pages", _vp), ("page_bytes", _i64), ("n_pages", _i32),
                ("conv", GdnConvPool), ("o", _vp)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libgdn.so (after torch) and bind every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- the HIP runtime must come from torch's process image
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_LOCAL)
    missing = [s for s in SYMBOLS if not hasattr(L, s)]
    if missing:
        raise ImportError(f"libgdn.so lacks {missing}")
    L.gdn_abi_version.restype = _i32
    L.gdn_abi_version.argtypes = []
    if L.gdn_abi_version() != ABI_VERSION:
        raise ImportError(f"libgdn ABI {L.gdn_abi_version()} != {ABI_VERSION}")
    L.gdn_status_str.restype = ctypes.c_char_p
    L.gdn_status_str.argtypes = [_i32]
    L.gdn_spec_page_layout.restype = _i32
    L.gdn_spec_page_layout.argtypes = [ctypes.POINTER(GdnDims), _i32, ctypes.POINTER(GdnSpecLayout)]
    L.gdn_chunked_workspace_bytes.restype = _i32
    L.gdn_chunked_workspace_bytes.argtypes = [ctypes.POINTER(GdnDims), _i32, _i64, _i32,
                                              ctypes.POINTER(ctypes.c_size_t)]
    L.gdn_conv_update.restype = _i32
    L.gdn_conv_update.argtypes = [ctypes.POINTER(GdnDims), _vp, _vp, _i64, ctypes.POINTER(GdnBatch),
                                  GdnConvPool, _i32, _vp, _i32, _i64, _vp, _vp]
    L.gdn_recurrent_seq.restype = _i32
    L.gdn_recurrent_seq.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(GdnParams), _vp, _i64, _vp, _vp,
                                    _i64, ctypes.POINTER(GdnBatch), GdnConvPool, GdnStatePool, _vp, _vp, _vp]
    L.gdn_recurrent_seq_noalloc.restype = _i32
    L.gdn_recurrent_seq_noalloc.argtypes = L.gdn_recurrent_seq.argtypes
    L.gdn_chunked_prefill.restype = _i32
    L.gdn_chunked_prefill.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(GdnParams), _vp, _i64, _vp, _vp,
                                      _i64, ctypes.POINTER(GdnBatch), GdnConvPool, GdnStatePool, _vp, _i32,
                                      _vp, ctypes.c_size_t, _vp, _vp]
    L.gdn_prefill_path.restype = _i32
    L.gdn_prefill_path.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(GdnBatch), _i32,
                                   ctypes.POINTER(_i32)]
    L.gdn_prefill.restype = _i32
    L.gdn_prefill.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(GdnParams), _vp, _i64, _vp, _vp, _i64,
                              ctypes.POINTER(GdnBatch), GdnConvPool, GdnStatePool, _vp, _i32, _vp,
                              ctypes.c_size_t, ctypes.POINTER(_i32), _vp, _vp]
    L.gdn_spec_verify.restype = _i32
    L.gdn_spec_verify.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(GdnParams), _i32, _vp, _i64, _vp,
                                  _vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _i32, GdnConvPool, _vp,
                                  _vp, _vp]
    L.gdn_spec_verify_cached.restype = _i32
    L.gdn_spec_verify_cached.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(GdnParams), _i32, _vp, _i64, _vp,
                                         _vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _i64, _i32, GdnConvPool,
                                         ctypes.POINTER(GdnPrefixCache), _vp, _vp, _vp]
    L.gdn_prefix_restore.restype = _i32
    L.gdn_prefix_restore.argtypes = [ctypes.POINTER(GdnDims), _i32, _i32, _vp, _vp, ctypes.POINTER(GdnPrefixCache),
                                     _vp, _i64, _i32, GdnConvPool, _vp, _vp]
    L.gdn_mixed_step.restype = _i32
    L.gdn_mixed_step.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(GdnParams), ctypes.POINTER(GdnSeqPart),
                                 ctypes.POINTER(GdnVerifyPart), _vp, _vp]
    L.gdn_mixed_launches.restype = _i32
    L.gdn_mixed_launches.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(GdnSeqPart),
                                     ctypes.POINTER(GdnVerifyPart), ctypes.POINTER(_i32)]
    L.gdn_mixed_step_launches.restype = _i32
    L.gdn_mixed_step_launches.argtypes = [ctypes.POINTER(GdnDims), ctypes.POINTER(GdnParams),
                                          ctypes.POINTER(GdnSeqPart), ctypes.POINTER(GdnVerifyPart), _i32, _vp, _vp]
    _lib = L
    return L
