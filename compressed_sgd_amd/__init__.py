"""compressed_sgd_amd -- Python binding of libsgc (MI355X / gfx950).

Thin ctypes marshalling over the C ABI declared in include/sgc.h: every step
of the path runs in the library's HIP kernels; this module only allocates
device tensors (torch), passes their pointers and the current stream, and
turns return codes into exceptions.  There is no CPU fallback: if libsgc.so
is missing or no GPU is present, the calls raise.

The entry points keep the C names without the ``sgc_`` prefix:
``compress``, ``binarize``, ``encode``, ``decode_accumulate``, plus the
``Layout`` of segment sizes shared by both ends of the exchange.
"""
from __future__ import annotations

import contextlib
import ctypes as C
import os
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import torch  # loads the HIP runtime first; libsgc binds to that same runtime

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsgc.so")

OK, EINVAL, ENOSPC, EHIP, EUNSUPPORTED, ENOTREADY = 0, -1, -2, -3, -4, -5
STATUS_TRUNCATED, STATUS_CORRUPT, STATUS_DENSE_PATH, STATUS_BAD_INPUT = 1, 2, 4, 8
EXACT, SAMPLED, ACCUMULATE_ONLY = 0, 1, 2
HOLD_KEPT = 0x10
# compress pipelines (same result; AUTO picks by kept fraction and vector size)
PATH_AUTO, PATH_GATHER, PATH_WINDOW = 0, 1, 2
GLOBAL, PER_SEGMENT = 0, 1
BIN_SBC, BIN_2BIT = 0, 1
BIN_HELD = 0x10
MSG_RAW_F32, MSG_RAW_2BIT, MSG_GOLOMB_F32, MSG_GOLOMB_SBC, MSG_GOLOMB_2BIT = 0, 1, 2, 3, 4
INIT_ZERO, INIT_BASE, INIT_INPLACE = 0, 1, 2
CHUNK_CODES = 256

EXPORTED = (
    "sgc_layout_create", "sgc_layout_upload", "sgc_layout_destroy", "sgc_layout_numel", "sgc_layout_nseg",
    "sgc_keep_count", "sgc_rice_param", "sgc_warmup_ppm", "sgc_strerror", "sgc_abi_version",
    "sgc_compress_workspace", "sgc_compress", "sgc_compress_noalloc",
    "sgc_compress_momentum_workspace", "sgc_compress_momentum",
    "sgc_binarize_workspace", "sgc_binarize",
    "sgc_encode_word_bound", "sgc_encode_chunk_bound", "sgc_encode_workspace", "sgc_encode",
    "sgc_decode_accumulate_workspace", "sgc_decode_accumulate", "sgc_set_pass_events",
)


class SGCError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {lib().sgc_strerror(code).decode()} ({code})")


class CompressOpts(C.Structure):
    _fields_ = [("mode", C.c_int32), ("scope", C.c_int32), ("keep_ppm", C.c_uint32),
                ("sample_div", C.c_uint32), ("sample_min", C.c_uint32), ("path", C.c_uint32)]


class MessageDesc(C.Structure):
    _fields_ = [("format", C.c_int32), ("scope", C.c_int32), ("rice_b", C.c_int32), ("reserved", C.c_int32),
                ("cap", C.c_int64), ("counts", C.c_void_p), ("idx", C.c_void_p), ("val", C.c_void_p),
                ("codes", C.c_void_p), ("means", C.c_void_p), ("words", C.c_void_p), ("word_off", C.c_void_p),
                ("nbits", C.c_void_p), ("chunk_off", C.c_void_p)]


_lib = None


def lib():
    """The loaded libsgc (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "'python compressed_sgd_amd/build.py' (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        P, i32, i64, u32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_size_t
        L.sgc_layout_create.argtypes = [P, i32, C.POINTER(P)]
        L.sgc_layout_create.restype = C.c_int
        L.sgc_layout_upload.argtypes = [P]
        L.sgc_layout_upload.restype = C.c_int
        L.sgc_layout_destroy.argtypes = [P]
        L.sgc_layout_destroy.restype = None
        L.sgc_layout_numel.argtypes = [P]
        L.sgc_layout_numel.restype = i64
        L.sgc_layout_nseg.argtypes = [P]
        L.sgc_layout_nseg.restype = i32
        L.sgc_keep_count.argtypes = [i64, u32]
        L.sgc_keep_count.restype = i64
        L.sgc_rice_param.argtypes = [C.c_double]
        L.sgc_rice_param.restype = i32
        L.sgc_warmup_ppm.argtypes = [i64, i64, u32, u32]
        L.sgc_warmup_ppm.restype = i64
        L.sgc_strerror.argtypes = [C.c_int]
        L.sgc_strerror.restype = C.c_char_p
        L.sgc_abi_version.argtypes = []
        L.sgc_abi_version.restype = i32
        L.sgc_compress_workspace.argtypes = [P, P, i64]
        L.sgc_compress_workspace.restype = sz
        L.sgc_compress.argtypes = [P, P, P, P, P, P, i64, P, P, P, sz, P]
        L.sgc_compress.restype = C.c_int
        L.sgc_compress_noalloc.argtypes = [P, P, P, P, P, P, i64, P, P, P]
        L.sgc_compress_noalloc.restype = C.c_int
        L.sgc_compress_momentum_workspace.argtypes = [P, P, i64]
        L.sgc_compress_momentum_workspace.restype = sz
        L.sgc_compress_momentum.argtypes = [P, P, C.c_float, P, P, P, P, P, i64, P, P, P, sz, P]
        L.sgc_compress_momentum.restype = C.c_int
        L.sgc_binarize_workspace.argtypes = [P, i64]
        L.sgc_binarize_workspace.restype = sz
        L.sgc_binarize.argtypes = [P, i32, P, P, P, i64, P, P, P, P, P, P, sz, P]
        L.sgc_binarize.restype = C.c_int
        L.sgc_encode_word_bound.argtypes = [P, i32, i32, i64]
        L.sgc_encode_word_bound.restype = i64
        L.sgc_encode_chunk_bound.argtypes = [P, i32, i64]
        L.sgc_encode_chunk_bound.restype = i64
        L.sgc_encode_workspace.argtypes = [P, i32, i64]
        L.sgc_encode_workspace.restype = sz
        L.sgc_encode.argtypes = [P, i32, i32, P, P, i64, P, i64, P, P, P, i64, P, P, sz, P]
        L.sgc_encode.restype = C.c_int
        L.sgc_decode_accumulate_workspace.argtypes = [P, P, i32]
        L.sgc_decode_accumulate_workspace.restype = sz
        L.sgc_decode_accumulate.argtypes = [P, P, i32, i32, P, P, P, P, sz, P]
        L.sgc_decode_accumulate.restype = C.c_int
        L.sgc_set_pass_events.argtypes = [P, P]
        L.sgc_set_pass_events.restype = C.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise SGCError(rc, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return C.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocate (and zero-fill) under the stream the call's kernels run on:
    torch's caching allocator then ties the memory to that stream, and fills
    run in order with the kernels that use the result."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _zeros(stream, *shape, **kw) -> torch.Tensor:
    with _on(stream):
        return torch.zeros(*shape, **kw)


def _empty(stream, *shape, **kw) -> torch.Tensor:
    with _on(stream):
        return torch.empty(*shape, **kw)


def _require_gpu(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ------------------------------------------------------------------ helpers
def keep_count(n: int, keep_ppm: int) -> int:
    return int(lib().sgc_keep_count(n, keep_ppm))


def rice_param(p: float) -> int:
    return int(lib().sgc_rice_param(p))


def warmup_ppm(step: int, steps: int, start_ppm: int = 250000, end_ppm: int = 1000) -> int:
    """Kept parts per million at step `step` of an exponential warm-up (sgc_warmup_ppm)."""
    v = int(lib().sgc_warmup_ppm(step, steps, start_ppm, end_ppm))
    if v < 0:
        raise ValueError("bad warm-up arguments")
    return v


def abi_version() -> int:
    return int(lib().sgc_abi_version())


class Layout:
    """Segment sizes of the flat parameter vector (one per tensor, in order).

    The tables go to the current device at creation (when a GPU is present)
    and to any other device on its first use there; the compute calls never
    upload (the C library returns ENOTREADY for a device without them).
    """

    def __init__(self, seg_numel: Sequence[int], device: Optional[torch.device] = None):
        self.seg_numel = [int(x) for x in seg_numel]
        arr = (C.c_int64 * max(len(self.seg_numel), 1))(*self.seg_numel)
        h = C.c_void_p()
        _check(lib().sgc_layout_create(arr, len(self.seg_numel), C.byref(h)), "sgc_layout_create")
        self._h = h
        self._devices = set()
        self.n = sum(self.seg_numel)
        self.nseg = len(self.seg_numel)
        off = [0]
        for m in self.seg_numel:
            off.append(off[-1] + m)
        self.seg_off = off
        if device is not None or torch.cuda.is_available():
            self.upload(device)

    @property
    def handle(self):
        return self._h

    def upload(self, device: Optional[torch.device] = None) -> None:
        """Put the tables on `device` (default: the current one); set-up, not capturable."""
        d = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        index = d.index if d.index is not None else torch.cuda.current_device()
        if index in self._devices:
            return
        with torch.cuda.device(index):
            _check(lib().sgc_layout_upload(self._h), "sgc_layout_upload")
        self._devices.add(index)

    def _ready(self, device: torch.device) -> None:
        index = device.index if device.index is not None else torch.cuda.current_device()
        if index not in self._devices:
            self.upload(torch.device("cuda", index))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.sgc_layout_destroy(h)
            self._h = None

    def group_sizes(self, scope: int) -> List[int]:
        return [self.n] if scope == GLOBAL else list(self.seg_numel)

    def keep_total(self, scope: int, keep_ppm: int) -> int:
        return sum(keep_count(m, keep_ppm) for m in self.group_sizes(scope))


_ws_cache: Dict[Tuple[int, int, str], torch.Tensor] = {}


def workspace(nbytes: int, device: torch.device, slot: str = "default", stream=None) -> torch.Tensor:
    """A cached uint8 device buffer of at least nbytes, one per (device, stream, slot).

    It is allocated under the stream the calls run on, so the caching
    allocator hands a replaced buffer to nothing else until that stream has
    passed every call that used it; calls on one stream run in order, and
    calls on two streams get two buffers.  A call captured into a HIP graph
    must be given a workspace of its own (``ws=``): a cached buffer could be
    replaced, and freed, while the graph still points at it.
    """
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("a call captured into a graph needs its own workspace: pass ws= "
                           "(sized with the *_workspace_bytes helpers)")
    index = device.index if device.index is not None else torch.cuda.current_device()
    s = stream if stream is not None else torch.cuda.current_stream(index)
    key = (index, int(s.cuda_stream), slot)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        _ws_cache.pop(key, None)
        buf = _empty(stream, max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def compress_workspace_bytes(layout: "Layout", *, mode: int = EXACT, scope: int = GLOBAL, keep_ppm: int = 10000,
                             sample_div: int = 1000, sample_min: int = 65536, cap: Optional[int] = None,
                             hold: bool = False, momentum: bool = False, path: int = 0) -> int:
    """Workspace bytes of one compress (or compress_momentum) call with these options."""
    opts = CompressOpts(mode | (HOLD_KEPT if hold else 0), scope, keep_ppm, sample_div, sample_min, path)
    cap = _default_cap(layout, mode, scope, keep_ppm) if cap is None else cap
    f = lib().sgc_compress_momentum_workspace if momentum else lib().sgc_compress_workspace
    return int(f(layout.handle, C.byref(opts), cap))


def binarize_workspace_bytes(layout: "Layout", cap: int) -> int:
    return int(lib().sgc_binarize_workspace(layout.handle, cap))


def encode_workspace_bytes(layout: "Layout", scope: int, cap: int) -> int:
    return int(lib().sgc_encode_workspace(layout.handle, scope, cap))


def decode_accumulate_workspace_bytes(layout: "Layout", msgs: Sequence["Message"]) -> int:
    arr = (MessageDesc * max(len(msgs), 1))(*[m.desc() for m in msgs])
    return int(lib().sgc_decode_accumulate_workspace(layout.handle, arr, len(msgs)))


def _default_cap(layout: "Layout", mode: int, scope: int, keep_ppm: int) -> int:
    k = layout.keep_total(scope, keep_ppm)
    return k if mode == EXACT else min(layout.n, 2 * k + 4096)


def _compress_out(layout: "Layout", out: Optional["Compressed"], cap: Optional[int], mode: int, scope: int,
                  keep_ppm: int, dev: torch.device, stream) -> Tuple["Compressed", int]:
    """The output buffers and the capacity of a compress call: new ones, or
    `out` reused after checking that it fits this call (cap defaults to its own)."""
    if out is None:
        cap = _default_cap(layout, mode, scope, keep_ppm) if cap is None else cap
        out = Compressed(_empty(stream, max(cap, 1), dtype=torch.int32, device=dev),
                         _empty(stream, max(cap, 1), dtype=torch.float32, device=dev),
                         _empty(stream, layout.nseg + 1, dtype=torch.int64, device=dev),
                         _zeros(stream, 1, dtype=torch.int32, device=dev), cap)
        return out, cap
    cap = out.cap if cap is None else cap
    if cap > out.idx.numel() or cap > out.val.numel():
        raise ValueError(f"out holds {min(out.idx.numel(), out.val.numel())} entries, this call needs cap {cap}")
    if out.counts.numel() != layout.nseg + 1:
        raise ValueError(f"out.counts has {out.counts.numel()} entries, the layout needs {layout.nseg + 1}")
    for t, name in ((out.idx, "out.idx"), (out.val, "out.val"), (out.counts, "out.counts")):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the call runs on {dev}")
    out.cap = cap
    return out, cap


# ----------------------------------------------------------------- compress
@dataclass
class Compressed:
    idx: torch.Tensor      # int32 [cap], first counts[-1] valid
    val: torch.Tensor      # float32 [cap]
    counts: torch.Tensor   # int64 [nseg+1]
    status: torch.Tensor   # uint32 [1] (stored as int32)
    cap: int

    def total(self) -> int:
        return int(self.counts[-1].item())


def compress(layout: Layout, grad: torch.Tensor, residual: torch.Tensor, *, mode: int = EXACT,
             scope: int = GLOBAL, keep_ppm: int = 10000, sample_div: int = 1000, sample_min: int = 65536,
             cap: Optional[int] = None, out: Optional[Compressed] = None, ws: Optional[torch.Tensor] = None,
             hold: bool = False, stream=None, path: int = 0) -> Optional[Compressed]:
    """One step: residual += grad, select, emit, zero the residual at kept entries.

    mode ACCUMULATE_ONLY only adds (communication delay) and returns None.
    hold: the kept entries keep acc in the residual (for binarize(..., held=True) next).
    """
    for t, name in ((grad, "grad"), (residual, "residual")):
        _require_gpu(t, name)
        if t.dtype != torch.float32 or t.numel() != layout.n:
            raise ValueError(f"{name} must be float32 with {layout.n} elements")
    dev = grad.device
    layout._ready(dev)
    opts = CompressOpts(mode | (HOLD_KEPT if hold else 0), scope, keep_ppm, sample_div, sample_min, path)
    st = _stream(dev, stream)
    if mode == ACCUMULATE_ONLY:
        _check(lib().sgc_compress(layout.handle, C.byref(opts), _ptr(grad), _ptr(residual), None, None, 0, None,
                                  None, None, 0, st), "sgc_compress")
        return None
    out, cap = _compress_out(layout, out, cap, mode, scope, keep_ppm, dev, stream)
    nbytes = lib().sgc_compress_workspace(layout.handle, C.byref(opts), cap)
    if ws is None:
        ws = workspace(nbytes, dev, "compress", stream)
    _check(lib().sgc_compress(layout.handle, C.byref(opts), _ptr(grad), _ptr(residual), _ptr(out.idx),
                              _ptr(out.val), cap, _ptr(out.counts), _ptr(out.status), _ptr(ws), ws.numel(), st),
           "sgc_compress")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # SGC_NOALLOC_SCRATCH_BYTES


def compress_noalloc(layout: Layout, grad: torch.Tensor, residual: torch.Tensor, *, mode: int = EXACT,
                     scope: int = GLOBAL, keep_ppm: int = 10000, sample_div: int = 1000, sample_min: int = 65536,
                     cap: Optional[int] = None, out: Optional[Compressed] = None, hold: bool = False,
                     stream=None, path: int = 0) -> Optional[Compressed]:
    """compress() through sgc_compress_noalloc: the library's own scratch buffer
    instead of a workspace.  The library allocates nothing; pass `out` to keep
    this function from allocating the output buffers either.  Calls that may
    overlap on one GPU share that buffer and must be serialised."""
    for t, name in ((grad, "grad"), (residual, "residual")):
        _require_gpu(t, name)
        if t.dtype != torch.float32 or t.numel() != layout.n:
            raise ValueError(f"{name} must be float32 with {layout.n} elements")
    dev = grad.device
    layout._ready(dev)
    opts = CompressOpts(mode | (HOLD_KEPT if hold else 0), scope, keep_ppm, sample_div, sample_min, path)
    st = _stream(dev, stream)
    if mode == ACCUMULATE_ONLY:
        _check(lib().sgc_compress_noalloc(layout.handle, C.byref(opts), _ptr(grad), _ptr(residual), None, None, 0,
                                          None, None, st), "sgc_compress_noalloc")
        return None
    out, cap = _compress_out(layout, out, cap, mode, scope, keep_ppm, dev, stream)
    rc = lib().sgc_compress_noalloc(layout.handle, C.byref(opts), _ptr(grad), _ptr(residual), _ptr(out.idx),
                                    _ptr(out.val), cap, _ptr(out.counts), _ptr(out.status), st)
    if rc == ENOSPC:
        need = lib().sgc_compress_workspace(layout.handle, C.byref(opts), cap)
        raise SGCError(rc, f"sgc_compress_noalloc (this call needs {need} bytes of workspace, the scratch "
                           f"buffer holds {NOALLOC_SCRATCH_BYTES})")
    _check(rc, "sgc_compress_noalloc")
    return out


def compress_momentum(layout: Layout, grad: torch.Tensor, momentum: torch.Tensor, residual: torch.Tensor,
                      beta: float, *, mode: int = EXACT, scope: int = GLOBAL, keep_ppm: int = 10000,
                      sample_div: int = 1000, sample_min: int = 65536, cap: Optional[int] = None,
                      out: Optional[Compressed] = None, ws: Optional[torch.Tensor] = None,
                      stream=None, path: int = 0) -> Optional[Compressed]:
    """One step with momentum correction: momentum = beta*momentum + grad, residual += momentum,
    select, emit, zero residual and momentum at the sent entries.

    mode ACCUMULATE_ONLY only updates momentum and residual and returns None.
    """
    for t, name in ((grad, "grad"), (momentum, "momentum"), (residual, "residual")):
        _require_gpu(t, name)
        if t.dtype != torch.float32 or t.numel() != layout.n:
            raise ValueError(f"{name} must be float32 with {layout.n} elements")
    dev = grad.device
    layout._ready(dev)
    opts = CompressOpts(mode, scope, keep_ppm, sample_div, sample_min, path)
    st = _stream(dev, stream)
    if mode == ACCUMULATE_ONLY:
        _check(lib().sgc_compress_momentum(layout.handle, C.byref(opts), float(beta), _ptr(grad), _ptr(momentum),
                                           _ptr(residual), None, None, 0, None, None, None, 0, st),
               "sgc_compress_momentum")
        return None
    out, cap = _compress_out(layout, out, cap, mode, scope, keep_ppm, dev, stream)
    nbytes = lib().sgc_compress_momentum_workspace(layout.handle, C.byref(opts), cap)
    if ws is None:
        ws = workspace(nbytes, dev, "compress_momentum", stream)
    _check(lib().sgc_compress_momentum(layout.handle, C.byref(opts), float(beta), _ptr(grad), _ptr(momentum),
                                       _ptr(residual), _ptr(out.idx), _ptr(out.val), cap, _ptr(out.counts),
                                       _ptr(out.status), _ptr(ws), ws.numel(), st), "sgc_compress_momentum")
    return out


# ----------------------------------------------------------------- binarize
@dataclass
class Binarized:
    idx: Optional[torch.Tensor]    # SBC: sent indices (int32 [cap]); 2-bit: copy of the input indices
    counts: torch.Tensor           # int64 [nseg+1]
    means: torch.Tensor            # SBC: [nseg] signed means; 2-bit: [2*nseg] (+mean_pos, -mean_neg)
    codes: Optional[torch.Tensor]  # 2-bit: int32 view of uint32 words [ceil(cap/16)]
    mode: int
    cap: int


def binarize(layout: Layout, comp: Compressed, residual: torch.Tensor, mode: int = BIN_SBC, *,
             ws: Optional[torch.Tensor] = None, held: bool = False, stream=None) -> Binarized:
    """Sparse binarization (SBC) or 2-bit quantization of a compress result.

    held: the residual holds acc at the kept entries (compress(..., hold=True)); same result,
    fewer writes.
    """
    _require_gpu(residual, "residual")
    dev = residual.device
    cap = comp.cap
    out = Binarized(_empty(stream, max(cap, 1), dtype=torch.int32, device=dev),
                    _empty(stream, layout.nseg + 1, dtype=torch.int64, device=dev),
                    _empty(stream, layout.nseg if mode == BIN_SBC else 2 * layout.nseg, dtype=torch.float32,
                           device=dev),
                    _zeros(stream, max((cap + 15) // 16, 1), dtype=torch.int32, device=dev) if mode == BIN_2BIT
                    else None, mode, cap)
    nbytes = lib().sgc_binarize_workspace(layout.handle, cap)
    if ws is None:
        ws = workspace(nbytes, dev, "binarize", stream)
    _check(lib().sgc_binarize(layout.handle, mode | (BIN_HELD if held else 0), _ptr(comp.idx), _ptr(comp.val),
                              _ptr(comp.counts), cap,
                              _ptr(residual), _ptr(out.idx), _ptr(out.counts), _ptr(out.means), _ptr(out.codes),
                              _ptr(ws), ws.numel(), _stream(dev, stream)), "sgc_binarize")
    return out


# ------------------------------------------------------------------- encode
@dataclass
class Encoded:
    words: torch.Tensor      # int32 view of the uint32 stream words
    word_off: torch.Tensor   # int64 view of uint64 [nstreams+1]
    nbits: torch.Tensor      # int64 view of uint64 [nstreams]
    chunk_off: torch.Tensor  # int64 view of uint64 chunk table
    status: torch.Tensor
    scope: int
    b: int
    cap: int


def _encode_out(out: Optional[Encoded], scope: int, b: int, cap: int, wcap: int, ccap: int, nstreams: int,
                dev: torch.device, stream) -> Encoded:
    """`out` when every buffer of it fits this call (words, offsets and bit
    counts of nstreams streams, the chunk table), else new buffers."""
    if (out is None or out.words.numel() < wcap or out.chunk_off.numel() < ccap
            or out.word_off.numel() < nstreams + 1 or out.nbits.numel() < nstreams or out.words.device != dev):
        out = Encoded(_empty(stream, max(wcap, 1), dtype=torch.int32, device=dev),
                      _empty(stream, nstreams + 1, dtype=torch.int64, device=dev),
                      _empty(stream, nstreams, dtype=torch.int64, device=dev),
                      _empty(stream, max(ccap, 1), dtype=torch.int64, device=dev),
                      _zeros(stream, 1, dtype=torch.int32, device=dev), scope, b, cap)
    out.scope, out.b, out.cap = scope, b, cap
    return out


def encode(layout: Layout, idx: torch.Tensor, counts: torch.Tensor, cap: int, *, scope: int = GLOBAL,
           b: Optional[int] = None, keep_ppm: Optional[int] = None, out: Optional[Encoded] = None,
           ws: Optional[torch.Tensor] = None, stream=None) -> Encoded:
    """Rice-code the index gaps of a sparse message.

    b defaults to the parameter that minimises the mean code length at the
    nominal density keep_ppm / 1e6.
    """
    _require_gpu(idx, "idx")
    dev = idx.device
    layout._ready(dev)
    if b is None:
        if keep_ppm is None:
            raise ValueError("give b or keep_ppm")
        b = rice_param(keep_ppm / 1e6)
    nstreams = 1 if scope == GLOBAL else layout.nseg
    wcap = int(lib().sgc_encode_word_bound(layout.handle, scope, b, cap))
    ccap = int(lib().sgc_encode_chunk_bound(layout.handle, scope, cap))
    if wcap < 0 or ccap < 0:
        raise ValueError("bad encode arguments")
    out = _encode_out(out, scope, b, cap, wcap, ccap, nstreams, dev, stream)
    nbytes = lib().sgc_encode_workspace(layout.handle, scope, cap)
    if ws is None:
        ws = workspace(nbytes, dev, "encode", stream)
    _check(lib().sgc_encode(layout.handle, scope, b, _ptr(idx), _ptr(counts), cap, _ptr(out.words),
                            out.words.numel(), _ptr(out.word_off), _ptr(out.nbits), _ptr(out.chunk_off),
                            out.chunk_off.numel(), _ptr(out.status), _ptr(ws), ws.numel(), _stream(dev, stream)),
           "sgc_encode")
    return out


# -------------------------------------------------------- decode + accumulate
@dataclass
class Message:
    """One received message: device tensors + format (see sgc_message)."""
    format: int
    counts: torch.Tensor
    cap: int
    scope: int = GLOBAL
    b: int = 0
    idx: Optional[torch.Tensor] = None
    val: Optional[torch.Tensor] = None
    codes: Optional[torch.Tensor] = None
    means: Optional[torch.Tensor] = None
    enc: Optional[Encoded] = None

    def desc(self) -> MessageDesc:
        e = self.enc
        return MessageDesc(self.format, self.scope, self.b, 0, self.cap, _ptr(self.counts), _ptr(self.idx),
                           _ptr(self.val), _ptr(self.codes), _ptr(self.means),
                           None if e is None else _ptr(e.words), None if e is None else _ptr(e.word_off),
                           None if e is None else _ptr(e.nbits), None if e is None else _ptr(e.chunk_off))


def raw_message(comp: Compressed) -> Message:
    return Message(MSG_RAW_F32, comp.counts, comp.cap, idx=comp.idx, val=comp.val)


def golomb_message(comp_or_bin, enc: Encoded) -> Message:
    """A Rice-coded message from an encode result and the values it carries."""
    if isinstance(comp_or_bin, Compressed):
        return Message(MSG_GOLOMB_F32, comp_or_bin.counts, enc.cap, scope=enc.scope, b=enc.b,
                       val=comp_or_bin.val, enc=enc)
    bn = comp_or_bin
    if bn.mode == BIN_SBC:
        return Message(MSG_GOLOMB_SBC, bn.counts, enc.cap, scope=enc.scope, b=enc.b, means=bn.means, enc=enc)
    return Message(MSG_GOLOMB_2BIT, bn.counts, enc.cap, scope=enc.scope, b=enc.b, codes=bn.codes,
                   means=bn.means, enc=enc)


def decode_accumulate(layout: Layout, msgs: Sequence[Message], out: torch.Tensor, *, init: int = INIT_ZERO,
                      base: Optional[torch.Tensor] = None, status: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """out = init; then add every message in order (present entries only)."""
    _require_gpu(out, "out")
    dev = out.device
    layout._ready(dev)
    W = len(msgs)
    arr = (MessageDesc * max(W, 1))(*[m.desc() for m in msgs])
    nbytes = lib().sgc_decode_accumulate_workspace(layout.handle, arr, W)
    if W > 0 and nbytes == 0:
        raise SGCError(EINVAL, "sgc_decode_accumulate_workspace")
    if ws is None:
        ws = workspace(nbytes, dev, "decode", stream)
    if status is None:
        status = _zeros(stream, 1, dtype=torch.int32, device=dev)
    _check(lib().sgc_decode_accumulate(layout.handle, arr, W, init, _ptr(base), _ptr(out), _ptr(status), _ptr(ws),
                                       ws.numel(), _stream(dev, stream)), "sgc_decode_accumulate")
    return status


def set_pass_events(start: Optional["torch.cuda.Event"], stop: Optional["torch.cuda.Event"]) -> None:
    """Time the fused pass of later compress calls with these (already recorded once) events."""
    if start is None:
        _check(lib().sgc_set_pass_events(None, None), "sgc_set_pass_events")
    else:
        _check(lib().sgc_set_pass_events(C.c_void_p(start.cuda_event), C.c_void_p(stop.cuda_event)),
               "sgc_set_pass_events")
