"""ctypes declarations of the C ABI in include/bs.h (argument marshalling only).

The library is ``libbs.so`` next to this file, built for gfx950 by
``lossless_entropy_coding_amd.build``.  Loading fails loudly when it is
missing: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbs.so")

BS_OK = 0
BS_E_INVAL = -1
BS_E_FORMAT = -2
BS_E_VERSION = -3
BS_E_NOSPACE = -4
BS_E_NOMEM = -5
BS_E_HIP = -6
BS_E_CORRUPT = -7
BS_E_MISMATCH = -8
BS_E_EXISTS = -9
FIXED_MANY_MAX = 16          # blobs per bs_fixed_decode_many_async call
NOALLOC_MAX_WEIGHTS = 1 << 36   # words per bs_build_tables_noalloc call

KIND_BF16 = 1
KIND_RAW = 2

VERIFY_STATUS = 1
VERIFY_COMPARE = 2
VERIFY_SHA256 = 4


class Params(C.Structure):
    _fields_ = [("chunk_weights", C.c_uint32), ("lanes", C.c_uint32), ("m_s", C.c_uint32),
                ("m_f", C.c_uint32), ("max_tables", C.c_uint32), ("threads", C.c_uint32),
                ("stream_lanes", C.c_uint32), ("layout", C.c_uint32)]


class Tensor(C.Structure):
    _fields_ = [("kind", C.c_uint32), ("reserved", C.c_uint32), ("h_data", C.c_void_p), ("n", C.c_uint64),
                ("tables", C.c_void_p), ("sha256", C.c_void_p)]


class DTensor(C.Structure):
    _fields_ = [("kind", C.c_uint32), ("reserved", C.c_uint32), ("d_data", C.c_void_p), ("n", C.c_uint64),
                ("tables", C.c_void_p), ("sha256", C.c_void_p)]


class ContainerInfo(C.Structure):
    _fields_ = [("version", C.c_uint32), ("n_records", C.c_uint32), ("total_len", C.c_uint64),
                ("out_len", C.c_uint64), ("n_chunks", C.c_uint64), ("bf16_weights", C.c_uint64),
                ("bf16_bytes", C.c_uint64), ("raw_bytes", C.c_uint64), ("n_streams", C.c_uint64)]


class SizeBreakdown(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in ("weights", "container_bits", "fixed_bits", "table_bits", "index_bits",
                                          "code_bits", "plane_bits", "state_bits", "word_bits", "pad_bits")]


class RecordInfo(C.Structure):
    _fields_ = [("kind", C.c_uint32), ("chunk_weights", C.c_uint32), ("lanes", C.c_uint32),
                ("n_chunks", C.c_uint32), ("m_s", C.c_uint32), ("m_f", C.c_uint32), ("n_tables", C.c_uint32),
                ("n_sym", C.c_uint32), ("n", C.c_uint64), ("out_offset", C.c_uint64), ("rec_offset", C.c_uint64),
                ("rec_len", C.c_uint64), ("chunk_base", C.c_uint64), ("sha256", C.c_uint8 * 32),
                ("stream_base", C.c_uint64), ("streams", C.c_uint32), ("layout", C.c_uint32)]


class Report(C.Structure):
    _fields_ = [("chunks_checked", C.c_uint64), ("chunks_bad", C.c_uint64), ("first_bad_chunk", C.c_uint64),
                ("bytes_compared", C.c_uint64), ("bytes_mismatched", C.c_uint64), ("first_mismatch", C.c_uint64),
                ("records_hashed", C.c_uint32), ("records_hash_bad", C.c_uint32), ("first_hash_bad", C.c_uint32),
                ("reserved", C.c_uint32)]


class FixedInfo(C.Structure):
    _fields_ = [("n", C.c_uint64), ("n_blocks", C.c_uint64), ("n_esc", C.c_uint64), ("esc_off", C.c_uint64),
                ("bytes", C.c_uint64), ("table", C.c_uint16 * 16)]


class StreamerStats(C.Structure):
    _fields_ = [("n_layers", C.c_uint32), ("n_slots", C.c_uint32), ("slot_bytes", C.c_uint64),
                ("staging_bytes", C.c_uint64), ("plan_bytes", C.c_uint64), ("hits", C.c_uint64),
                ("misses", C.c_uint64), ("evictions", C.c_uint64), ("h2d_bytes", C.c_uint64)]


# every symbol declared in include/bs.h, with (restype, argtypes)
SIGNATURES = {
    "bs_params_default": (None, [C.POINTER(Params)]),
    "bs_build_tables": (C.c_int, [C.c_void_p, C.c_uint64, C.POINTER(Params), C.c_void_p, C.POINTER(C.c_void_p)]),
    "bs_tables_get_layout": (C.c_int, [C.c_void_p, C.POINTER(C.c_uint32), C.c_void_p]),
    "bs_tables_get_joint": (C.c_int, [C.c_void_p, C.c_void_p]),
    "bs_build_tables_host": (C.c_int, [C.c_void_p, C.c_uint64, C.POINTER(Params), C.POINTER(C.c_void_p)]),
    "bs_build_tables_noalloc": (C.c_int, [C.c_void_p, C.c_uint64, C.POINTER(Params), C.c_void_p, C.c_void_p]),
    "bs_tables_free": (None, [C.c_void_p]),
    "bs_tables_get": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.POINTER(C.c_uint32),
                                C.POINTER(C.c_uint32), C.POINTER(C.c_uint32), C.POINTER(C.c_uint64)]),
    "bs_encode_host": (C.c_int, [C.POINTER(Tensor), C.c_uint32, C.POINTER(Params), C.POINTER(C.c_void_p)]),
    "bs_encode_device_begin": (C.c_int, [C.POINTER(DTensor), C.c_uint32, C.POINTER(Params), C.c_void_p,
                                         C.POINTER(C.c_void_p)]),
    "bs_encode_device_size": (C.c_uint64, [C.c_void_p]),
    "bs_encode_device_finish": (C.c_int, [C.c_void_p, C.c_void_p, C.c_uint64, C.c_void_p]),
    "bs_encode_device_free": (None, [C.c_void_p]),
    "bs_blob_data": (C.c_void_p, [C.c_void_p]),
    "bs_blob_size": (C.c_uint64, [C.c_void_p]),
    "bs_blob_free": (None, [C.c_void_p]),
    "bs_container_info_get": (C.c_int, [C.c_void_p, C.c_uint64, C.POINTER(ContainerInfo)]),
    "bs_record_info_get": (C.c_int, [C.c_void_p, C.c_uint64, C.c_uint32, C.POINTER(RecordInfo)]),
    "bs_container_sizes_get": (C.c_int, [C.c_void_p, C.c_uint64, C.POINTER(SizeBreakdown)]),
    "bs_plan_create": (C.c_int, [C.c_void_p, C.c_uint64, C.c_void_p, C.c_void_p, C.POINTER(C.c_void_p)]),
    "bs_plan_destroy": (None, [C.c_void_p]),
    "bs_plan_rebind": (C.c_int, [C.c_void_p, C.c_void_p]),
    "bs_plan_container_bytes": (C.c_uint64, [C.c_void_p]),
    "bs_streamer_create": (C.c_int, [C.POINTER(C.c_void_p), C.POINTER(C.c_uint64), C.c_uint32, C.c_uint64, C.c_void_p,
                                     C.POINTER(C.c_void_p)]),
    "bs_streamer_destroy": (None, [C.c_void_p]),
    "bs_streamer_acquire": (C.c_int, [C.c_void_p, C.c_uint32, C.c_void_p, C.POINTER(C.c_void_p)]),
    "bs_streamer_release": (C.c_int, [C.c_void_p, C.c_uint32, C.c_void_p]),
    "bs_streamer_prefetch": (C.c_int, [C.c_void_p, C.c_uint32, C.c_void_p]),
    "bs_streamer_get_stats": (C.c_int, [C.c_void_p, C.POINTER(StreamerStats)]),
    "bs_decode_async": (C.c_int, [C.c_void_p, C.c_uint32, C.c_uint32, C.c_void_p, C.c_uint64, C.c_void_p,
                                  C.c_void_p]),
    "bs_plan_out_bytes": (C.c_uint64, [C.c_void_p, C.c_uint32, C.c_uint32]),
    "bs_gemv_async": (C.c_int, [C.c_void_p, C.c_uint32, C.c_uint64, C.c_uint64, C.c_void_p, C.c_void_p, C.c_void_p,
                                C.c_void_p]),
    "bs_fixed_encode_host": (C.c_int, [C.c_void_p, C.c_uint64, C.c_uint32, C.POINTER(C.c_void_p)]),
    "bs_fixed_max_bytes": (C.c_uint64, [C.c_uint64]),
    "bs_fixed_encode_device": (C.c_int, [C.c_void_p, C.c_uint64, C.c_void_p, C.c_uint64, C.POINTER(C.c_uint64),
                                         C.c_void_p]),
    "bs_fixed_info_get": (C.c_int, [C.c_void_p, C.c_uint64, C.c_uint64, C.POINTER(FixedInfo)]),
    "bs_fixed_decode_async": (C.c_int, [C.POINTER(FixedInfo), C.c_void_p, C.c_void_p, C.c_uint64, C.c_void_p,
                                        C.c_void_p]),
    "bs_fixed_decode_many_async": (C.c_int, [C.POINTER(FixedInfo), C.POINTER(C.c_void_p), C.POINTER(C.c_void_p),
                                             C.POINTER(C.c_uint64), C.POINTER(C.c_void_p), C.c_uint32, C.c_void_p]),
    "bs_fixed_gemv_async": (C.c_int, [C.POINTER(FixedInfo), C.c_void_p, C.c_uint64, C.c_uint64, C.c_void_p,
                                      C.c_void_p, C.c_void_p, C.c_void_p]),
    "bs_fixed_gemm_async": (C.c_int, [C.POINTER(FixedInfo), C.c_void_p, C.c_uint64, C.c_uint64, C.c_uint32,
                                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_uint64, C.c_void_p]),
    "bs_fixed_gemm_work_bytes": (C.c_uint64, [C.c_uint64, C.c_uint64, C.c_uint32]),
    "bs_plan_waves_per_block": (C.c_uint32, [C.c_void_p]),
    "bs_plan_packs": (C.c_uint32, [C.c_void_p, C.c_uint32, C.c_uint32]),
    "bs_verify": (C.c_int, [C.c_void_p, C.c_uint32, C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_uint32,
                            C.c_void_p, C.POINTER(Report)]),
    "bs_sha256": (None, [C.c_void_p, C.c_uint64, C.c_void_p]),
    "bs_write_file_new": (C.c_int, [C.c_char_p, C.c_void_p, C.c_uint64]),
    "bs_strerror": (C.c_char_p, [C.c_int]),
    "bs_last_error": (C.c_char_p, []),
    "bs_version": (C.c_char_p, []),
}

_lib = None


class LibraryMissing(RuntimeError):
    pass


def lib():
    """Load libbs.so (raises LibraryMissing if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(f"{LIB_PATH} is missing: build it with "
                                 "`python -m lossless_entropy_coding_amd.build` (no fallback exists)")
        l = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


class BSError(RuntimeError):
    def __init__(self, rc: int, where: str):
        l = lib()
        msg = l.bs_last_error().decode(errors="replace")
        super().__init__(f"{where}: {l.bs_strerror(rc).decode()} ({rc}): {msg}")
        self.rc = rc


def check(rc: int, where: str) -> None:
    if rc != BS_OK:
        raise BSError(rc, where)
