"""Python face of the CPU oracle (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It loads ``oracle/libbs_oracle.so`` (plain C, built with
gcc by :func:`build`), which shares no code with the HIP library.

The per-tensor sha256 digests that the container stores are computed here
with :mod:`hashlib` and handed to the C encoder; the pages ask for a hash per
tensor checked at decompression [Gemma 2 9B Instruct -- Lossless Compressed
card, "What lossless means"; Qwen3.8-27B-BF16-NVLC-Lossless card, SHA256SUMS
verification block].
"""
from __future__ import annotations

import ctypes as C
import hashlib
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bs_oracle.c")
_LIB = os.path.join(_HERE, "libbs_oracle.so")

KIND_BF16 = 1
KIND_RAW = 2
L = 65536

ERRORS = {0: "ok", -1: "invalid argument", -2: "format", -3: "version", -4: "no space",
          -5: "no memory", -7: "corrupt"}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C11 + the __int128 extension)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-Wall", "-Wextra", "-fPIC", "-shared",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        # BSO_ORACLE_LIB lets the mutation tests load a deliberately broken copy
        path = os.environ.get("BSO_ORACLE_LIB") or build()
        l = C.CDLL(path)
        u32p, u64p = C.POINTER(C.c_uint32), C.POINTER(C.c_uint64)
        l.bso_symbol_s.argtypes = [C.c_uint16]; l.bso_symbol_s.restype = C.c_uint32
        l.bso_symbol_f.argtypes = [C.c_uint16]; l.bso_symbol_f.restype = C.c_uint32
        l.bso_combine.argtypes = [C.c_uint32, C.c_uint32]; l.bso_combine.restype = C.c_uint16
        l.bso_histogram.argtypes = [C.c_void_p, C.c_uint64, u64p, u64p]; l.bso_histogram.restype = None
        l.bso_fixed_encode.argtypes = [C.c_void_p, C.c_uint64, C.POINTER(C.c_void_p), u64p]
        l.bso_fixed_encode.restype = C.c_int
        l.bso_fixed_decode.argtypes = [C.c_void_p, C.c_uint64, C.c_void_p, C.c_uint64]
        l.bso_fixed_decode.restype = C.c_int
        l.bso_normalise.argtypes = [u64p, C.c_uint32, C.c_uint32, u32p]; l.bso_normalise.restype = C.c_int
        l.bso_select_tables.argtypes = [u64p, u64p, C.c_uint32, C.c_uint32, u32p, u32p, u32p]
        l.bso_select_tables.restype = C.c_int
        l.bso_record_shape.argtypes = [C.c_uint64, C.c_uint32, C.c_uint32, u32p, u32p]
        l.bso_record_shape.restype = C.c_int
        l.bso_sched_encode.argtypes = [C.c_uint32, C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p, C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_uint64, u64p]
        l.bso_sched_encode.restype = C.c_int
        l.bso_sched_decode.argtypes = [C.c_uint32, C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p, C.c_uint32, C.c_void_p, C.c_void_p,
                                       C.c_uint64, C.c_void_p, C.c_void_p]
        l.bso_sched_decode.restype = C.c_int
        l.bso_encode_container.argtypes = [C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32,
                                           C.POINTER(C.POINTER(C.c_uint8)), u64p]
        l.bso_encode_container.restype = C.c_int
        l.bso_encode_container2.argtypes = [C.c_uint32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                            C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32,
                                            C.c_uint32, C.POINTER(C.POINTER(C.c_uint8)), u64p]
        l.bso_encode_container2.restype = C.c_int
        l.bso_log2_q16.argtypes = [C.c_uint32]; l.bso_log2_q16.restype = C.c_uint32
        l.bso_select_htables.argtypes = [u64p, u64p, C.c_uint32, C.c_uint32, u32p, u32p, u32p]
        l.bso_select_htables.restype = C.c_int
        l.bso_share_hroutes.argtypes = [u64p, u64p, C.c_uint32, C.c_uint32, u32p, u32p]
        l.bso_share_hroutes.restype = C.c_int
        l.bso_decode_container.argtypes = [C.c_void_p, C.c_uint64, C.c_void_p, C.c_uint64, C.c_void_p]
        l.bso_decode_container.restype = C.c_int
        l.bso_free.argtypes = [C.c_void_p]; l.bso_free.restype = None
        l.bso_decode_chunk.argtypes = [C.c_void_p, C.c_uint64, C.c_uint32, C.c_uint64, C.c_void_p, C.c_uint64, u64p]
        l.bso_decode_chunk.restype = C.c_int
        _lib = l
    return _lib


class OracleError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"{what}: oracle error {rc} ({ERRORS.get(rc, '?')})")
        self.rc = rc


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _u32p(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_uint32))


def _u64p(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_uint64))


# --------------------------------------------------------------------------- fields
def symbol_s(w: int) -> int:
    return int(lib().bso_symbol_s(w))


def symbol_f(w: int) -> int:
    return int(lib().bso_symbol_f(w))


def combine(s: int, f: int) -> int:
    return int(lib().bso_combine(s, f))


# --------------------------------------------------------------------------- model
def histogram(words: np.ndarray):
    """(cs[512], cf[512,128]) as uint64 from a uint16 array."""
    w = np.ascontiguousarray(words, dtype=np.uint16)
    cs = np.zeros(512, np.uint64)
    cf = np.zeros((512, 128), np.uint64)
    lib().bso_histogram(_ptr(w), w.size, _u64p(cs), _u64p(cf))
    return cs, cf


def normalise(counts, M: int) -> np.ndarray:
    c = np.ascontiguousarray(counts, dtype=np.uint64)
    q = np.zeros(c.size, np.uint32)
    rc = lib().bso_normalise(_u64p(c), c.size, M, _u32p(q))
    if rc:
        raise OracleError(rc, "normalise")
    return q


def select_tables(cs, cf, M_f: int = 10, cmax: int = 6):
    """(route[512], n_tables, qf[n_tables,128])."""
    cs = np.ascontiguousarray(cs, dtype=np.uint64)
    cf = np.ascontiguousarray(cf, dtype=np.uint64).reshape(512, 128)
    route = np.zeros(512, np.uint32)
    nt = np.zeros(1, np.uint32)
    qf = np.zeros((max(cmax, 1), 128), np.uint32)
    rc = lib().bso_select_tables(_u64p(cs), _u64p(cf), M_f, cmax, _u32p(route), _u32p(nt), _u32p(qf))
    if rc:
        raise OracleError(rc, "select_tables")
    return route, int(nt[0]), qf[: int(nt[0])].copy()


def log2_q16(q: int) -> int:
    """floor(65536 log2 q) as the container's layout-2 rule computes it."""
    return int(lib().bso_log2_q16(q))


def select_htables(cs, cf, M_h: int = 5, cmax: int = 31):
    """Layout-2 coded tables of h = f >> 4: (route[512], n_tables, qh[cmax, 8])."""
    cs = np.ascontiguousarray(cs, np.uint64)
    cf = np.ascontiguousarray(cf, np.uint64).reshape(-1)
    route = np.zeros(512, np.uint32)
    nt = np.zeros(1, np.uint32)
    qh = np.zeros(max(cmax, 1) * 8, np.uint32)
    rc = lib().bso_select_htables(_u64p(cs), _u64p(cf), M_h, cmax, _u32p(route), _u32p(nt), _u32p(qh))
    if rc:
        raise OracleError(rc, "select_htables")
    return route, int(nt[0]), qh.reshape(max(cmax, 1), 8)


def share_hroutes(cs, cf, qh, route, M_h: int = 5):
    """Layout-2 shared routing: route[] after every exponent without a table
    of its own is sent to the cheapest of the flat and the coded tables qh
    (n_tables rows of 8)."""
    cs = np.ascontiguousarray(cs, np.uint64)
    cf = np.ascontiguousarray(cf, np.uint64).reshape(-1)
    qh = np.ascontiguousarray(qh, np.uint32).reshape(-1, 8)
    r = np.ascontiguousarray(route, np.uint32).copy()
    rc = lib().bso_share_hroutes(_u64p(cs), _u64p(cf), M_h, qh.shape[0], _u32p(qh.reshape(-1)), _u32p(r))
    if rc:
        raise OracleError(rc, "share_hroutes")
    return r


def record_shape(n: int, Wmax: int, Kmax: int):
    W = np.zeros(1, np.uint32)
    K = np.zeros(1, np.uint32)
    rc = lib().bso_record_shape(n, Wmax, Kmax, _u32p(W), _u32p(K))
    if rc:
        raise OracleError(rc, "record_shape")
    return int(W[0]), int(K[0])


# --------------------------------------------------------------------------- raw coder
@dataclass
class Table:
    M: int
    q: list


def _tables(tables):
    M = np.array([t.M for t in tables], np.uint32)
    A = np.array([len(t.q) for t in tables], np.uint32)
    q = np.concatenate([np.asarray(t.q, np.uint32) for t in tables]) if tables else np.zeros(1, np.uint32)
    return M, A, np.ascontiguousarray(q, np.uint32)


def sched_encode(K: int, syms, tab_of, tables, init=None):
    """Interleaved rANS over an explicit schedule.

    syms, tab_of: int arrays of shape (nsteps, K); syms = -1 where a lane is idle.
    init: the lanes' initial states (default: all L).
    Returns (states[K] uint32, words uint16).
    """
    syms = np.ascontiguousarray(syms, np.int32).reshape(-1, K)
    tab_of = np.ascontiguousarray(tab_of, np.uint32).reshape(-1, K)
    nsteps = syms.shape[0]
    M, A, q = _tables(tables)
    cap = 2 * syms.size + 16
    words = np.zeros(cap, np.uint16)
    states = np.zeros(K, np.uint32)
    nw = np.zeros(1, np.uint64)
    ini = None if init is None else np.ascontiguousarray(init, np.uint32)
    rc = lib().bso_sched_encode(K, nsteps, _ptr(syms), _ptr(tab_of), _ptr(M), _ptr(A), _ptr(q), len(tables),
                                None if ini is None else _ptr(ini), _ptr(states), _ptr(words), cap, _u64p(nw))
    if rc:
        raise OracleError(rc, "sched_encode")
    return states, words[: int(nw[0])].copy()


def sched_decode(K: int, active, tab_of, tables, states, words):
    """Inverse of :func:`sched_encode`: returns (syms (nsteps,K) int32, final states)."""
    active = np.ascontiguousarray(active, np.int32).reshape(-1, K)
    tab_of = np.ascontiguousarray(tab_of, np.uint32).reshape(-1, K)
    nsteps = active.shape[0]
    M, A, q = _tables(tables)
    st = np.ascontiguousarray(states, np.uint32)
    w = np.ascontiguousarray(words, np.uint16)
    if w.size == 0:
        w = np.zeros(1, np.uint16)
        nw = 0
    else:
        nw = w.size
    out = np.zeros((nsteps, K), np.int32)
    fin = np.zeros(K, np.uint32)
    rc = lib().bso_sched_decode(K, nsteps, _ptr(active), _ptr(tab_of), _ptr(M), _ptr(A), _ptr(q), len(tables),
                                _ptr(st), _ptr(w), nw, _ptr(out), _ptr(fin))
    if rc:
        raise OracleError(rc, "sched_decode")
    return out, fin


# --------------------------------------------------------------------------- container
@dataclass
class Tensor:
    """One tensor to encode: kind 1 = BF16 words (uint16 array), 2 = RAW bytes."""
    kind: int
    data: np.ndarray

    @property
    def nbytes(self) -> int:
        return int(self.data.nbytes)


def bf16(words) -> Tensor:
    return Tensor(KIND_BF16, np.ascontiguousarray(words, np.uint16).reshape(-1))


def raw(b) -> Tensor:
    return Tensor(KIND_RAW, np.frombuffer(bytes(b), np.uint8).copy())


def sha256(t: Tensor) -> bytes:
    return hashlib.sha256(t.data.tobytes()).digest()


def encode(tensors, W: int = 65536, K: int = 64, M_s: int = 12, M_f: int = 10, cmax: int = 6,
           P: int | None = None, layout: int = 1) -> bytes:
    """Container of the tensors: chunks of W weights with K lanes, split into
    streams of P lanes (default: one stream of all K lanes).  layout 1 gives a
    version-1 container; layout 2 a version-2 one, with M_s 11 or 12, M_f
    the precision of the h tables (16 - M_s) and cmax up to 31; layout 3 a
    version-3 one, with M_s 11 or 12 and M_f the precision of the joint
    (s, h) table (13)."""
    n = len(tensors)
    P = K if P is None else P
    kinds = np.array([t.kind for t in tensors] or [0], np.uint32)
    counts = np.array([t.data.size for t in tensors] or [0], np.uint64)
    keep = [np.ascontiguousarray(t.data) for t in tensors]
    ptrs = (C.c_void_p * max(n, 1))(*[a.ctypes.data for a in keep])
    sha = np.frombuffer(b"".join(sha256(t) for t in tensors) or b"\0" * 32, np.uint8).copy()
    out = C.POINTER(C.c_uint8)()
    out_len = C.c_uint64(0)
    rc = lib().bso_encode_container2(n, _ptr(kinds), ptrs, _ptr(counts), _ptr(sha), W, K, P, M_s, M_f, cmax,
                                     layout, C.byref(out), C.byref(out_len))
    if rc:
        raise OracleError(rc, "encode")
    try:
        return C.string_at(out, out_len.value)
    finally:
        lib().bso_free(out)


def out_len(container: bytes) -> int:
    return int.from_bytes(container[32:40], "little")


def _n_rec(container: bytes) -> int:
    # the C decoder checks the directory against the length before writing any
    # status, so a corrupt count never needs more than len/96 entries
    if len(container) < 16:
        return 0
    return min(int.from_bytes(container[12:16], "little"), len(container) // 96 + 1)


def decode(container: bytes, out_cap: int | None = None):
    """Returns (output bytes, per-record status list)."""
    buf = np.frombuffer(container, np.uint8)
    cap = out_len(container) if out_cap is None else out_cap
    out = np.zeros(max(cap, 1), np.uint8)
    n_rec = _n_rec(container)
    st = np.zeros(max(n_rec, 1), np.int32)
    rc = lib().bso_decode_container(_ptr(buf), buf.size, _ptr(out), cap, _ptr(st))
    if rc:
        raise OracleError(rc, "decode")
    return out[:cap].tobytes(), [int(v) for v in st[:n_rec]]


def decode_status(container: bytes, out_cap: int | None = None):
    """Like :func:`decode` but returns (rc, out, statuses) instead of raising."""
    buf = np.frombuffer(container, np.uint8)
    cap = out_len(container) if out_cap is None and len(container) >= 40 else (out_cap or 0)
    out = np.zeros(max(cap, 1), np.uint8)
    n_rec = _n_rec(container)
    st = np.zeros(max(n_rec, 1), np.int32)
    rc = lib().bso_decode_container(_ptr(buf), buf.size, _ptr(out), cap, _ptr(st))
    return rc, out[:cap].tobytes(), [int(v) for v in st[:n_rec]]


def decode_chunk(container, record: int, chunk: int, max_weights: int = 1 << 20) -> np.ndarray:
    """The words of one chunk of one BF16 record, decoded by the oracle."""
    buf = np.frombuffer(container, np.uint8)
    out = np.zeros(max_weights, np.uint16)
    n_c = np.zeros(1, np.uint64)
    rc = lib().bso_decode_chunk(_ptr(buf), buf.size, record, chunk, _ptr(out), max_weights, _u64p(n_c))
    if rc:
        raise OracleError(rc, "decode_chunk")
    return out[: int(n_c[0])].copy()


# --------------------------------------------------------------------------- fixed-width lane streams
def fixed_encode(words) -> bytes:
    """The fixed-width lane-stream form of one BF16 tensor (see the C source)."""
    w = np.ascontiguousarray(np.asarray(words, np.uint16))
    out = C.c_void_p()
    n = np.zeros(1, np.uint64)
    rc = lib().bso_fixed_encode(_ptr(w), w.size, C.byref(out), _u64p(n))
    if rc:
        raise OracleError(rc, "fixed_encode")
    try:
        return C.string_at(out, int(n[0]))
    finally:
        lib().bso_free(out)


def fixed_decode(blob: bytes, cap: int | None = None) -> np.ndarray:
    """Decode a fixed-width blob; `cap` is the output capacity in weights
    (default: the header's count, bounded by what the blob can hold)."""
    buf = np.frombuffer(blob, np.uint8)
    n = int.from_bytes(blob[16:24], "little") if len(blob) >= 24 else 0
    n = min(n, (len(blob) // 2816 + 1) * 2048)
    cap = n if cap is None else cap
    out = np.zeros(max(cap, 1), np.uint16)
    rc = lib().bso_fixed_decode(_ptr(buf), buf.size, _ptr(out), cap)
    if rc:
        raise OracleError(rc, "fixed_decode")
    return out[:n].copy()
