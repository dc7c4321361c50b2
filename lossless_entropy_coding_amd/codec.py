"""Python face of the codec: thin wrappers over the C ABI (include/bs.h).

PyTorch provides device memory and streams only; every step of building
tables, encoding, decoding and verifying runs in the library (host C++ for
the encoder, HIP kernels on gfx950 for histograms, lookup tables, decoding,
residual copies and compares).

The codec [Qwen3.8-27B-BF16-NVLC-Lossless model card, codec paragraph]: each
BF16 word is split into [sign:1 | exponent:8 | fraction:7]; the joint
(sign, exponent) symbol is rANS-coded with a per-tensor model and selects the
distribution of the fraction; the decoder recombines the fields bitwise and
copies non-BF16 spans verbatim.
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import numpy as np
import torch

from . import _lib as L


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def params(chunk_weights: int = 65536, lanes: int = 128, m_s: int = 12, m_f: int = 10, max_tables: int = 6,
           threads: int = 0, stream_lanes: int = 0, layout: int = 1) -> L.Params:
    """Encoder parameters; stream_lanes 0 keeps each chunk one word stream.
    layout 2 (one renormalisation per weight) takes m_s 11 or 12, m_f =
    16 - m_s and up to 31 tables: see params2."""
    p = L.Params()
    L.lib().bs_params_default(C.byref(p))
    p.chunk_weights, p.lanes, p.m_s, p.m_f, p.max_tables, p.threads = (chunk_weights, lanes, m_s, m_f,
                                                                       max_tables, threads)
    p.stream_lanes = stream_lanes
    p.layout = layout
    return p


def params2(chunk_weights: int = 65536, lanes: int = 128, m_s: int = 11, threads: int = 0,
            stream_lanes: int = 0, max_tables: int = 31) -> L.Params:
    """Layout-2 encoder parameters (two steps, one renormalisation per weight)."""
    return params(chunk_weights, lanes, m_s, 16 - m_s, max_tables, threads, stream_lanes, layout=2)


JOINT_BITS = 13   # precision of a layout-3 record's joint (s, h) table


def params3(chunk_weights: int = 65536, lanes: int = 128, m_s: int = 11, threads: int = 0,
            stream_lanes: int = 0) -> L.Params:
    """Layout-3 encoder parameters (the library's default layout): s and h
    coded as one joint symbol."""
    return params(chunk_weights, lanes, m_s, JOINT_BITS, 0, threads, stream_lanes, layout=3)


class Tables:
    """A per-tensor model (opaque bs_tables), freed with the object."""

    def __init__(self, handle: int):
        self.handle = C.c_void_p(handle)

    def __del__(self):
        if getattr(self, "handle", None) and self.handle.value:
            L.lib().bs_tables_free(self.handle)
            self.handle = C.c_void_p(0)

    def get(self) -> dict:
        cs = np.zeros(512, np.uint64)
        qs = np.zeros(512, np.uint32)
        route = np.zeros(512, np.uint32)
        qf = np.zeros((6, 128), np.uint32)
        nt, ms, mf = C.c_uint32(), C.c_uint32(), C.c_uint32()
        n = C.c_uint64()
        L.check(L.lib().bs_tables_get(self.handle, cs.ctypes.data, qs.ctypes.data, route.ctypes.data,
                                      qf.ctypes.data, C.byref(nt), C.byref(ms), C.byref(mf), C.byref(n)),
                "bs_tables_get")
        layout = C.c_uint32()
        qh = np.zeros((31, 8), np.uint32)
        L.check(L.lib().bs_tables_get_layout(self.handle, C.byref(layout), qh.ctypes.data), "bs_tables_get_layout")
        d = {"counts_s": cs, "q_s": qs, "route": route, "n_tables": nt.value, "m_s": ms.value, "m_f": mf.value,
             "n": n.value, "layout": layout.value}
        if layout.value == 1:
            d["q_f"] = qf[: nt.value].copy()
        elif layout.value == 2:
            d["q_h"] = qh[: nt.value].copy()
        else:
            qt = np.zeros(512 * 8, np.uint32)
            L.check(L.lib().bs_tables_get_joint(self.handle, qt.ctypes.data), "bs_tables_get_joint")
            d["q_t"] = qt
        return d


def build_tables(words: torch.Tensor, p: L.Params | None = None, stream=None) -> Tables:
    """Model of a device-resident BF16 (or int16-viewed) tensor, built by the HIP histogram kernels."""
    p = p or params()
    t = words.contiguous()
    assert t.is_cuda and t.element_size() == 2
    out = C.c_void_p()
    L.check(L.lib().bs_build_tables(C.c_void_p(t.data_ptr()), t.numel(), C.byref(p), C.c_void_p(_stream_handle(stream)),
                                    C.byref(out)), "bs_build_tables")
    return Tables(out.value)


def build_tables_noalloc(words: torch.Tensor, into: Tables, p: L.Params | None = None, stream=None) -> Tables:
    """bs_build_tables_noalloc: the model of a device-resident tensor written
    over an existing Tables, with nothing allocated by the library."""
    p = p or params()
    assert words.is_cuda and words.is_contiguous() and words.element_size() == 2
    L.check(L.lib().bs_build_tables_noalloc(C.c_void_p(words.data_ptr()), words.numel(), C.byref(p),
                                            C.c_void_p(_stream_handle(stream)), into.handle), "bs_build_tables_noalloc")
    return into


def build_tables_host(words: np.ndarray, p: L.Params | None = None) -> Tables:
    p = p or params()
    w = np.ascontiguousarray(words, np.uint16)
    out = C.c_void_p()
    L.check(L.lib().bs_build_tables_host(w.ctypes.data, w.size, C.byref(p), C.byref(out)), "bs_build_tables_host")
    return Tables(out.value)


@dataclass
class HostTensor:
    """A tensor to encode: kind 1 = BF16 words (uint16 ndarray), 2 = raw bytes (uint8 ndarray)."""
    kind: int
    data: np.ndarray
    tables: Tables | None = None
    sha256: bytes | None = None


def bf16(words, tables: Tables | None = None) -> HostTensor:
    return HostTensor(L.KIND_BF16, np.ascontiguousarray(words, np.uint16).reshape(-1), tables)


def raw(b) -> HostTensor:
    a = b if isinstance(b, np.ndarray) else np.frombuffer(bytes(b), np.uint8)
    return HostTensor(L.KIND_RAW, np.ascontiguousarray(a).view(np.uint8).reshape(-1))


def encode(tensors, p: L.Params | None = None) -> bytes:
    """Encode host tensors into one container (host C++ encoder, multithreaded)."""
    p = p or params()
    arr = (L.Tensor * max(len(tensors), 1))()
    keep = []
    for i, t in enumerate(tensors):
        d = np.ascontiguousarray(t.data)
        keep.append(d)
        arr[i].kind = t.kind
        arr[i].h_data = d.ctypes.data if d.size else None
        arr[i].n = d.size
        arr[i].tables = t.tables.handle if t.tables is not None else None
        if t.sha256 is not None:
            sb = C.create_string_buffer(t.sha256, 32)
            keep.append(sb)
            arr[i].sha256 = C.addressof(sb)
    blob = C.c_void_p()
    L.check(L.lib().bs_encode_host(arr, len(tensors), C.byref(p), C.byref(blob)), "bs_encode_host")
    try:
        n = L.lib().bs_blob_size(blob)
        return C.string_at(L.lib().bs_blob_data(blob), n)
    finally:
        L.lib().bs_blob_free(blob)


def encode_device(tensors, p: L.Params | None = None, stream=None, tables=None, digests=None) -> torch.Tensor:
    """Encode device tensors into one container on the GPU (bs_encode_device_*):
    tensors is a list of ("bf16", int16/bfloat16 cuda tensor) or ("raw", uint8
    cuda tensor); tables an optional list of Tables (None entries are built on
    the device); digests an optional list of 32-byte sha256 values (None: the
    library hashes a host copy).  Returns the container as a uint8 cuda tensor."""
    p = p or params()
    n = len(tensors)
    arr = (L.DTensor * max(n, 1))()
    keep = []
    for i, (kind, t) in enumerate(tensors):
        t = t.contiguous()
        keep.append(t)
        arr[i].kind = L.KIND_BF16 if kind == "bf16" else L.KIND_RAW
        arr[i].d_data = t.data_ptr() if t.numel() else None
        arr[i].n = t.numel() if kind == "bf16" else t.numel() * t.element_size()
        if tables is not None and tables[i] is not None:
            arr[i].tables = tables[i].handle
        if digests is not None and digests[i] is not None:
            sb = C.create_string_buffer(bytes(digests[i]), 32)
            keep.append(sb)
            arr[i].sha256 = C.addressof(sb)
    h = _stream_handle(stream)
    enc = C.c_void_p()
    L.check(L.lib().bs_encode_device_begin(arr, n, C.byref(p), C.c_void_p(h), C.byref(enc)), "bs_encode_device_begin")
    try:
        size = L.lib().bs_encode_device_size(enc)
        out = torch.empty(max(size, 16), dtype=torch.uint8, device="cuda")
        L.check(L.lib().bs_encode_device_finish(enc, C.c_void_p(out.data_ptr()), out.numel(), C.c_void_p(h)),
                "bs_encode_device_finish")
    finally:
        L.lib().bs_encode_device_free(enc)
    return out[:size]


def _host_bytes(container):
    """(pointer argument, length) of a host container given as bytes or as a
    uint8 numpy array."""
    if isinstance(container, np.ndarray):
        assert container.dtype == np.uint8 and container.flags.c_contiguous
        return C.c_void_p(container.ctypes.data), container.size
    return container, len(container)


def container_info(container) -> L.ContainerInfo:
    info = L.ContainerInfo()
    ptr, n = _host_bytes(container)
    L.check(L.lib().bs_container_info_get(ptr, n, C.byref(info)), "bs_container_info_get")
    return info


def container_sizes(container) -> dict:
    """bs_container_sizes_get: where the container's BF16 bits go, as a dict
    of bit counts (and the weight count)."""
    sz = L.SizeBreakdown()
    ptr, n = _host_bytes(container)
    L.check(L.lib().bs_container_sizes_get(ptr, n, C.byref(sz)), "bs_container_sizes_get")
    return {name: int(getattr(sz, name)) for name, _ in L.SizeBreakdown._fields_}


def size_breakdown_bits_per_weight(sizes: dict) -> dict:
    """A sum of container_sizes dicts as bits per weight by part."""
    w = max(sizes["weights"], 1)
    return {k[:-5] if k.endswith("_bits") else k: round(v / w, 5) for k, v in sizes.items() if k != "weights"}


def record_info(container, i: int) -> L.RecordInfo:
    info = L.RecordInfo()
    ptr, n = _host_bytes(container)
    L.check(L.lib().bs_record_info_get(ptr, n, i, C.byref(info)), "bs_record_info_get")
    return info


class Plan:
    """A container resident in HBM plus its decode plan (opaque bs_plan)."""

    def __init__(self, container: bytes, device: str = "cuda", stream=None, dev: torch.Tensor | None = None):
        """container: host bytes (header, tables and index are read from it);
        dev: a device copy of the same bytes to decode from (uint8, 16-B
        aligned), or None to upload `container`."""
        self.host = container
        self.info = container_info(container)
        self.n_records = self.info.n_records
        if dev is None:
            # 16-byte aligned device copy (torch allocations are 256-B aligned)
            dev = torch.frombuffer(bytearray(container), dtype=torch.uint8).to(device)
        assert dev.dtype == torch.uint8 and dev.numel() == len(container) and dev.data_ptr() % 16 == 0
        self.dev = dev
        out = C.c_void_p()
        L.check(L.lib().bs_plan_create(container, len(container), C.c_void_p(self.dev.data_ptr()),
                                       C.c_void_p(_stream_handle(stream)), C.byref(out)), "bs_plan_create")
        self.handle = out
        # one status word per chunk stream
        self.status = torch.zeros(max(self.info.n_streams, 1), dtype=torch.int32, device=device)

    def __del__(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            L.lib().bs_plan_destroy(self.handle)
            self.handle = C.c_void_p(0)

    def out_bytes(self, first: int = 0, count: int | None = None) -> int:
        count = self.n_records - first if count is None else count
        return int(L.lib().bs_plan_out_bytes(self.handle, first, count))

    @property
    def waves_per_block(self) -> int:
        return int(L.lib().bs_plan_waves_per_block(self.handle))

    def packs(self, first: int = 0, count: int | None = None) -> int:
        """Workgroups that decode packs of small records when records
        [first, first + count) are decoded (0: none)."""
        if count is None:
            count = self.n_records - first
        return int(L.lib().bs_plan_packs(self.handle, first, count))

    def new_output(self, first: int = 0, count: int | None = None) -> torch.Tensor:
        """A zero-filled output buffer for records [first, first+count) (gaps stay zero)."""
        n = self.out_bytes(first, count)
        return torch.zeros(max(n, 16), dtype=torch.uint8, device=self.dev.device)

    def decode_into(self, out: torch.Tensor, first: int = 0, count: int | None = None, stream=None) -> None:
        """Enqueue the decode of records [first, first+count) into `out` (no sync)."""
        count = self.n_records - first if count is None else count
        rc = L.lib().bs_decode_async(self.handle, first, count, C.c_void_p(out.data_ptr()),
                                     out.numel() * out.element_size(), C.c_void_p(self.status.data_ptr()),
                                     C.c_void_p(_stream_handle(stream)))
        L.check(rc, "bs_decode_async")

    def bound_decode(self, out: torch.Tensor, first: int = 0, count: int | None = None, stream=None):
        """decode_into with its ctypes arguments converted once: returns a
        callable that enqueues the same decode each time it is called."""
        count = self.n_records - first if count is None else count
        f = L.lib().bs_decode_async
        args = (self.handle, C.c_uint32(first), C.c_uint32(count), C.c_void_p(out.data_ptr()),
                C.c_uint64(out.numel() * out.element_size()), C.c_void_p(self.status.data_ptr()),
                C.c_void_p(_stream_handle(stream)))
        keep = (out, self.status)

        def run():
            rc = f(*args)
            if rc:
                L.check(rc, "bs_decode_async")
            return keep
        return run

    def decode(self, first: int = 0, count: int | None = None, stream=None) -> torch.Tensor:
        out = self.new_output(first, count)
        self.decode_into(out, first, count, stream)
        return out

    def gemv_into(self, y: torch.Tensor, x: torch.Tensor, rows: int, cols: int, record: int = 0, stream=None) -> None:
        """Enqueue y = W x for BF16 record `record` read as a rows x cols matrix,
        decoding W on the fly (bs_gemv_async): x a bfloat16 (or int16) tensor of
        cols elements, y a float32 tensor of rows elements (overwritten)."""
        assert x.dtype in (torch.bfloat16, torch.int16) and x.numel() == cols and x.is_contiguous()
        assert y.dtype == torch.float32 and y.numel() == rows and y.is_contiguous()
        rc = L.lib().bs_gemv_async(self.handle, record, rows, cols, C.c_void_p(x.data_ptr()), C.c_void_p(y.data_ptr()),
                                   C.c_void_p(self.status.data_ptr()), C.c_void_p(_stream_handle(stream)))
        L.check(rc, "bs_gemv_async")

    def bound_gemv(self, y: torch.Tensor, x: torch.Tensor, rows: int, cols: int, record: int = 0, stream=None):
        """gemv_into with its ctypes arguments converted once (for timing loops)."""
        f = L.lib().bs_gemv_async
        args = (self.handle, C.c_uint32(record), C.c_uint64(rows), C.c_uint64(cols), C.c_void_p(x.data_ptr()),
                C.c_void_p(y.data_ptr()), C.c_void_p(self.status.data_ptr()), C.c_void_p(_stream_handle(stream)))
        keep = (x, y, self.status)

        def run():
            rc = f(*args)
            if rc:
                L.check(rc, "bs_gemv_async")
            return keep
        return run

    def gemv(self, x: torch.Tensor, rows: int, cols: int, record: int = 0, stream=None) -> torch.Tensor:
        y = torch.empty(rows, dtype=torch.float32, device=self.dev.device)
        self.gemv_into(y, x, rows, cols, record, stream)
        return y

    def verify(self, out: torch.Tensor, ref: torch.Tensor | None = None, flags: int = L.VERIFY_STATUS,
               first: int = 0, count: int | None = None, stream=None):
        """Returns (status code, report dict); synchronises the stream."""
        count = self.n_records - first if count is None else count
        rep = L.Report()
        rc = L.lib().bs_verify(self.handle, first, count, C.c_void_p(out.data_ptr()),
                               C.c_void_p(ref.data_ptr()) if ref is not None else None,
                               C.c_void_p(self.status.data_ptr()), flags, C.c_void_p(_stream_handle(stream)),
                               C.byref(rep))
        return rc, {k: getattr(rep, k) for k, _ in L.Report._fields_}


def sha256(data) -> bytes:
    a = np.ascontiguousarray(np.frombuffer(data, np.uint8) if isinstance(data, (bytes, bytearray)) else data)
    out = (C.c_uint8 * 32)()
    L.lib().bs_sha256(a.ctypes.data if a.size else None, a.nbytes, out)
    return bytes(out)


def write_new(path: str, data: bytes) -> None:
    L.check(L.lib().bs_write_file_new(path.encode(), data, len(data)), "bs_write_file_new")


def record_output(out: torch.Tensor, plan: Plan, i: int, first: int = 0) -> torch.Tensor:
    """View of record i's decoded bytes inside an output buffer decoded from `first`."""
    ri = record_info(plan.host, i)
    base = record_info(plan.host, first).out_offset
    nb = 2 * ri.n if ri.kind == L.KIND_BF16 else ri.n
    return out[ri.out_offset - base: ri.out_offset - base + nb]


# --------------------------------------------------------------------------- fixed-width lane streams
def fixed_encode(words, threads: int = 0) -> bytes:
    """Fixed-width lane-stream form of one BF16 tensor (host uint16 words),
    built by the library's host transcoder (bs_fixed_encode_host)."""
    w = np.ascontiguousarray(np.asarray(words).view(np.uint16).reshape(-1))
    blob = C.c_void_p()
    L.check(L.lib().bs_fixed_encode_host(w.ctypes.data if w.size else None, w.size, threads, C.byref(blob)),
            "bs_fixed_encode_host")
    try:
        return C.string_at(L.lib().bs_blob_data(blob), L.lib().bs_blob_size(blob))
    finally:
        L.lib().bs_blob_free(blob)


def fixed_encode_device(words: torch.Tensor, stream=None) -> torch.Tensor:
    """The fixed-width form of device-resident BF16 words (int16 or bfloat16
    cuda tensor), built on the GPU (bs_fixed_encode_device); returns the blob
    as a uint8 cuda tensor."""
    w = words.contiguous().reshape(-1)
    n = w.numel()
    out = torch.empty(max(L.lib().bs_fixed_max_bytes(n), 16), dtype=torch.uint8, device=w.device)
    ln = C.c_uint64()
    L.check(L.lib().bs_fixed_encode_device(C.c_void_p(w.data_ptr()) if n else None, n, C.c_void_p(out.data_ptr()),
                                           out.numel(), C.byref(ln), C.c_void_p(_stream_handle(stream))),
            "bs_fixed_encode_device")
    return out[: ln.value]


def fixed_info(blob: bytes, blob_len: int | None = None) -> L.FixedInfo:
    info = L.FixedInfo()
    L.check(L.lib().bs_fixed_info_get(blob, len(blob), len(blob) if blob_len is None else blob_len, C.byref(info)),
            "bs_fixed_info_get")
    return info


class FixedPlan:
    """A fixed-width blob resident in HBM and its validated header."""

    def __init__(self, blob, device: str = "cuda"):
        if isinstance(blob, torch.Tensor):          # a blob already in device memory
            self.dev = blob
            self.info = fixed_info(blob[:96].cpu().numpy().tobytes(), blob.numel())
        else:
            self.info = fixed_info(blob)
            self.dev = torch.frombuffer(bytearray(blob), dtype=torch.uint8).to(device)
        self.n = self.info.n
        self.bytes = self.info.bytes
        self.status = torch.zeros(max(self.info.n_blocks, 1), dtype=torch.int32, device=self.dev.device)

    def new_output(self) -> torch.Tensor:
        return torch.empty(max(self.n, 8), dtype=torch.int16, device=self.dev.device)

    def decode_into(self, out: torch.Tensor, status: bool = True, stream=None) -> None:
        """Enqueue the decode of all n weights into `out` (bs_fixed_decode_async)."""
        rc = L.lib().bs_fixed_decode_async(C.byref(self.info), C.c_void_p(self.dev.data_ptr()),
                                           C.c_void_p(out.data_ptr()), C.c_uint64(out.numel() * out.element_size()),
                                           C.c_void_p(self.status.data_ptr()) if status else None,
                                           C.c_void_p(_stream_handle(stream)))
        L.check(rc, "bs_fixed_decode_async")

    def bound_decode(self, out: torch.Tensor, status: bool = True, stream=None):
        """decode_into with its ctypes arguments converted once."""
        f = L.lib().bs_fixed_decode_async
        args = (C.byref(self.info), C.c_void_p(self.dev.data_ptr()), C.c_void_p(out.data_ptr()),
                C.c_uint64(out.numel() * out.element_size()),
                C.c_void_p(self.status.data_ptr()) if status else None, C.c_void_p(_stream_handle(stream)))
        keep = (out, self.status, self.dev)

        def run():
            rc = f(*args)
            if rc:
                L.check(rc, "bs_fixed_decode_async")
            return keep
        return run

    def decode(self, stream=None) -> torch.Tensor:
        out = self.new_output()
        self.decode_into(out, stream=stream)
        return out[: self.n]

    def gemv_into(self, y: torch.Tensor, x: torch.Tensor, rows: int, cols: int, status: bool = True,
                  stream=None) -> None:
        """Enqueue y = W x with W the blob's weights as a rows x cols matrix,
        decoded in registers (bs_fixed_gemv_async): x bfloat16 (or int16) of
        cols elements, y float32 of rows elements (overwritten)."""
        assert x.dtype in (torch.bfloat16, torch.int16) and x.numel() == cols and x.is_contiguous()
        assert y.dtype == torch.float32 and y.numel() == rows and y.is_contiguous()
        rc = L.lib().bs_fixed_gemv_async(C.byref(self.info), C.c_void_p(self.dev.data_ptr()), rows, cols,
                                         C.c_void_p(x.data_ptr()), C.c_void_p(y.data_ptr()),
                                         C.c_void_p(self.status.data_ptr()) if status else None,
                                         C.c_void_p(_stream_handle(stream)))
        L.check(rc, "bs_fixed_gemv_async")

    def bound_gemv(self, y: torch.Tensor, x: torch.Tensor, rows: int, cols: int, status: bool = False,
                   stream=None):
        """gemv_into with its ctypes arguments converted once."""
        f = L.lib().bs_fixed_gemv_async
        args = (C.byref(self.info), C.c_void_p(self.dev.data_ptr()), C.c_uint64(rows), C.c_uint64(cols),
                C.c_void_p(x.data_ptr()), C.c_void_p(y.data_ptr()),
                C.c_void_p(self.status.data_ptr()) if status else None, C.c_void_p(_stream_handle(stream)))
        keep = (x, y, self.status, self.dev)

        def run():
            rc = f(*args)
            if rc:
                L.check(rc, "bs_fixed_gemv_async")
            return keep
        return run

    def gemv(self, x: torch.Tensor, rows: int, cols: int, stream=None) -> torch.Tensor:
        y = torch.empty(rows, dtype=torch.float32, device=self.dev.device)
        self.gemv_into(y, x, rows, cols, stream=stream)
        return y

    def gemm_work(self, rows: int, cols: int, batch: int, work="auto"):
        """The workspace (tensor, bytes) a product of this shape is given:
        work="auto" takes the size bs_fixed_gemm_work_bytes asks for (none
        where it asks for 0), work=None none, and a device tensor is passed as
        it is.  One buffer per plan, grown when a shape needs more; products
        that share it must be enqueued on one stream."""
        if work is None:
            return None, 0
        if isinstance(work, torch.Tensor):                # a caller's own workspace
            return work, work.numel() * work.element_size()
        need = int(L.lib().bs_fixed_gemm_work_bytes(rows, cols, batch))
        if need == 0:
            return None, 0
        if getattr(self, "_work", None) is None or self._work.numel() < need:
            self._work = torch.empty(need, dtype=torch.uint8, device=self.dev.device)
        return self._work, need

    def gemm_into(self, y: torch.Tensor, x: torch.Tensor, rows: int, cols: int, status: bool = True,
                  stream=None, work="auto") -> None:
        """Enqueue Y = X W^T on the matrix cores (bs_fixed_gemm_async): x a
        (batch, cols) bfloat16 (or int16) tensor, y a (batch, rows) float32
        tensor (overwritten), batch 1..64; work as for gemm_work."""
        assert x.dtype in (torch.bfloat16, torch.int16) and x.dim() == 2 and x.shape[1] == cols and x.is_contiguous()
        assert y.dtype == torch.float32 and tuple(y.shape) == (x.shape[0], rows) and y.is_contiguous()
        wt, wb = self.gemm_work(rows, cols, x.shape[0], work)
        rc = L.lib().bs_fixed_gemm_async(C.byref(self.info), C.c_void_p(self.dev.data_ptr()), rows, cols, x.shape[0],
                                         C.c_void_p(x.data_ptr()), C.c_void_p(y.data_ptr()),
                                         C.c_void_p(self.status.data_ptr()) if status else None,
                                         C.c_void_p(wt.data_ptr()) if wt is not None else None, C.c_uint64(wb),
                                         C.c_void_p(_stream_handle(stream)))
        L.check(rc, "bs_fixed_gemm_async")

    def bound_gemm(self, y: torch.Tensor, x: torch.Tensor, rows: int, cols: int, stream=None, work="auto"):
        """gemm_into with its ctypes arguments converted once."""
        f = L.lib().bs_fixed_gemm_async
        wt, wb = self.gemm_work(rows, cols, x.shape[0], work)
        args = (C.byref(self.info), C.c_void_p(self.dev.data_ptr()), C.c_uint64(rows), C.c_uint64(cols),
                C.c_uint32(x.shape[0]), C.c_void_p(x.data_ptr()), C.c_void_p(y.data_ptr()), None,
                C.c_void_p(wt.data_ptr()) if wt is not None else None, C.c_uint64(wb),
                C.c_void_p(_stream_handle(stream)))
        keep = (x, y, self.dev, wt)

        def run():
            rc = f(*args)
            if rc:
                L.check(rc, "bs_fixed_gemm_async")
            return keep
        return run

    def gemm(self, x: torch.Tensor, rows: int, cols: int, stream=None) -> torch.Tensor:
        y = torch.empty(x.shape[0], rows, dtype=torch.float32, device=self.dev.device)
        self.gemm_into(y, x, rows, cols, stream=stream)
        return y

    def block_status(self) -> np.ndarray:
        return self.status[: self.info.n_blocks].cpu().numpy().view(np.uint32)


# --------------------------------------------------------------------------- layer streaming
def _many_args(plans, outs, status, stream):
    k = len(plans)
    if len(outs) != k:
        raise ValueError("one output per blob")
    infos = (L.FixedInfo * max(k, 1))(*[p.info for p in plans])
    blobs = (C.c_void_p * max(k, 1))(*[p.dev.data_ptr() for p in plans])
    dst = (C.c_void_p * max(k, 1))(*[o.data_ptr() for o in outs])
    caps = (C.c_uint64 * max(k, 1))(*[o.numel() * o.element_size() for o in outs])
    st = (C.c_void_p * max(k, 1))(*[p.status.data_ptr() for p in plans]) if status else None
    args = (infos, blobs, dst, caps, st, C.c_uint32(k), C.c_void_p(_stream_handle(stream)))
    return args, (infos, blobs, dst, caps, st, list(outs), [(p.dev, p.status) for p in plans])


def fixed_decode_many(plans, outs, status: bool = True, stream=None) -> None:
    """Enqueue the decode of up to FIXED_MANY_MAX fixed-width blobs (FixedPlan
    objects) into their outputs in one launch (bs_fixed_decode_many_async)."""
    args, _ = _many_args(plans, outs, status, stream)
    L.check(L.lib().bs_fixed_decode_many_async(*args), "bs_fixed_decode_many_async")


def bound_fixed_decode_many(plans, outs, status: bool = False, stream=None):
    """fixed_decode_many with its ctypes arguments converted once."""
    f = L.lib().bs_fixed_decode_many_async
    args, keep = _many_args(plans, outs, status, stream)

    def run():
        rc = f(*args)
        if rc:
            L.check(rc, "bs_fixed_decode_many_async")
        return keep
    return run


class Streamer:
    """Layers streamed on demand under a device-memory budget (bs_streamer_*):
    the containers live in the streamer's pinned host memory; acquire()
    returns a uint8 view of the layer's decoded bytes in a device slot."""

    def __init__(self, containers, vram_budget: int, stream=None):
        n = len(containers)
        self._keep = [bytes(c) for c in containers]
        ptrs = (C.c_void_p * max(n, 1))(*[C.cast(C.c_char_p(c), C.c_void_p) for c in self._keep])
        lens = (C.c_uint64 * max(n, 1))(*[len(c) for c in self._keep])
        out = C.c_void_p()
        L.check(L.lib().bs_streamer_create(ptrs, lens, n, vram_budget, C.c_void_p(_stream_handle(stream)),
                                           C.byref(out)), "bs_streamer_create")
        self.handle = out
        self._keep = None                  # copied into pinned memory
        self.out_bytes = [int(container_info(c).out_len) for c in containers]

    def __del__(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            L.lib().bs_streamer_destroy(self.handle)
            self.handle = C.c_void_p(0)

    def acquire_ptr(self, layer: int, stream=None) -> int:
        p = C.c_void_p()
        L.check(L.lib().bs_streamer_acquire(self.handle, layer, C.c_void_p(_stream_handle(stream)), C.byref(p)),
                "bs_streamer_acquire")
        return int(p.value)

    def acquire(self, layer: int, stream=None) -> torch.Tensor:
        """The layer's decoded bytes (a view of its slot; valid until release)."""
        ptr = self.acquire_ptr(layer, stream)
        return _device_view(ptr, self.out_bytes[layer])

    def release(self, layer: int, stream=None) -> None:
        L.check(L.lib().bs_streamer_release(self.handle, layer, C.c_void_p(_stream_handle(stream))),
                "bs_streamer_release")

    def prefetch(self, layer: int, stream=None) -> None:
        L.check(L.lib().bs_streamer_prefetch(self.handle, layer, C.c_void_p(_stream_handle(stream))),
                "bs_streamer_prefetch")

    def stats(self) -> dict:
        st = L.StreamerStats()
        L.check(L.lib().bs_streamer_get_stats(self.handle, C.byref(st)), "bs_streamer_get_stats")
        return {k: getattr(st, k) for k, _ in L.StreamerStats._fields_}


def _device_view(ptr: int, nbytes: int) -> torch.Tensor:
    """A uint8 tensor over nbytes of library-owned device memory at ptr (no copy)."""
    class _Mem:
        __cuda_array_interface__ = {"shape": (nbytes,), "typestr": "|u1", "data": (ptr, False), "version": 3,
                                    "strides": None}
    return torch.as_tensor(_Mem(), device="cuda")
