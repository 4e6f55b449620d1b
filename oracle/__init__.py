"""CPU oracle of the sparse-gradient compression path -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  It wraps the plain C oracle (``sgc_oracle.c``) with
numpy marshalling; the C file states, step by step, which passage of the
pages each function follows and which reading it takes where they are silent.

Every function works on host numpy arrays, returns fresh arrays and never
touches a GPU.  ``compress_*`` and ``binarize`` update the residual passed in
place (like the method does).

The sampled-threshold mode follows a reading (its defining page is cut
short), pinned by hand-worked literal examples of that reading.  Parity
unpinned: the reading that the local node's own message is summed as well as
its dense gradient in the global+local combination (pinned by linearity only).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from .build import LIB, build_oracle

GLOBAL, PER_SEGMENT = 0, 1
BIN_SBC, BIN_2BIT = 0, 1
VAL_F32, VAL_SBC, VAL_2BIT = 0, 1, 2
STATUS_TRUNCATED, STATUS_CORRUPT = 1, 2
CHUNK_CODES = 256

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build_oracle()
        L = C.CDLL(LIB)
        i64, i32, u32, f64 = C.c_int64, C.c_int32, C.c_uint32, C.c_double
        P = C.c_void_p
        L.orc_keep_count.restype = i64
        L.orc_keep_count.argtypes = [i64, u32]
        L.orc_sample_count.restype = i64
        L.orc_sample_count.argtypes = [i64, u32, u32]
        L.orc_warmup_ppm.restype = i64
        L.orc_warmup_ppm.argtypes = [i64, i64, u32, u32]
        L.orc_rice_expected_bits.restype = f64
        L.orc_rice_expected_bits.argtypes = [i32, f64]
        L.orc_rice_param.restype = i32
        L.orc_rice_param.argtypes = [f64]
        L.orc_accumulate.restype = None
        L.orc_accumulate.argtypes = [P, P, i64]
        L.orc_momentum_correct.restype = None
        L.orc_momentum_correct.argtypes = [C.c_float, P, P, i64]
        L.orc_momentum_mask.restype = None
        L.orc_momentum_mask.argtypes = [P, P, i64]
        L.orc_compress_exact.restype = i64
        L.orc_compress_exact.argtypes = [P, P, P, i32, i32, u32, P, P, i64, P]
        L.orc_compress_sampled.restype = i64
        L.orc_compress_sampled.argtypes = [P, P, P, i32, i32, u32, u32, u32, P, P, i64, P, P]
        L.orc_binarize.restype = i64
        L.orc_binarize.argtypes = [P, P, P, i32, i32, P, P, P, P, P]
        L.orc_encode.restype = i32
        L.orc_encode.argtypes = [P, P, P, i32, i32, i32, P, i64, P, P, P, i64]
        L.orc_decode_stream.restype = i32
        L.orc_decode_stream.argtypes = [P, C.c_uint64, i64, i32, i64, P, P, P]
        L.orc_accumulate_message.restype = i32
        L.orc_accumulate_message.argtypes = [P, P, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def seg_offsets(seg_numel: Sequence[int]) -> np.ndarray:
    off = np.zeros(len(seg_numel) + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(seg_numel, dtype=np.int64))
    return off


def keep_count(n: int, ppm: int) -> int:
    return int(lib().orc_keep_count(n, ppm))


def sample_count(n: int, sample_div: int = 1000, sample_min: int = 65536) -> int:
    return int(lib().orc_sample_count(n, sample_div, sample_min))


def warmup_ppm(t: int, steps: int, start: int = 250000, end: int = 1000) -> int:
    return int(lib().orc_warmup_ppm(t, steps, start, end))


def rice_expected_bits(b: int, p: float) -> float:
    return float(lib().orc_rice_expected_bits(b, p))


def rice_param(p: float) -> int:
    return int(lib().orc_rice_param(p))


def accumulate(g: np.ndarray, r: np.ndarray) -> None:
    """Communication delay: r <- fp32(r + g) in place."""
    assert g.dtype == np.float32 and r.dtype == np.float32 and r.flags.c_contiguous
    lib().orc_accumulate(_p(_f32(g)), _p(r), r.size)


def momentum_correct(beta: float, g: np.ndarray, u: np.ndarray) -> None:
    """Momentum correction ([SBC] appendix A): u <- fp32(fp32(beta*u) + g) in place."""
    assert u.dtype == np.float32 and u.flags.c_contiguous
    lib().orc_momentum_correct(float(beta), _p(_f32(g)), _p(u), u.size)


def momentum_mask(u: np.ndarray, sent_idx: np.ndarray) -> None:
    """Momentum masking ([SBC] appendix A): u[sent] <- +0 in place."""
    assert u.dtype == np.float32 and u.flags.c_contiguous
    idx = np.ascontiguousarray(sent_idx, dtype=np.int32)
    lib().orc_momentum_mask(_p(u), _p(idx), idx.size)


def _groups_need(seg_off: np.ndarray, scope: int, ppm: int) -> int:
    if scope == GLOBAL:
        return keep_count(int(seg_off[-1]), ppm)
    return sum(keep_count(int(seg_off[t + 1] - seg_off[t]), ppm) for t in range(len(seg_off) - 1))


@dataclass
class Sparse:
    idx: np.ndarray      # int32 global flat indices, ascending
    val: np.ndarray      # fp32 values (raw bits of acc)
    counts: np.ndarray   # int64 [nseg+1]: per-segment entries, then the total
    status: int = 0


def hold_kept(sp: Sparse, r: np.ndarray) -> None:
    """The residual as a compress with the hold flag leaves it: the sent entries keep acc."""
    r[sp.idx] = sp.val


def compress_exact(g, r: np.ndarray, seg_off, scope: int, ppm: int, cap: Optional[int] = None) -> Sparse:
    g = _f32(g)
    seg_off = np.ascontiguousarray(seg_off, dtype=np.int64)
    nseg = len(seg_off) - 1
    need = _groups_need(seg_off, scope, ppm)
    cap = need if cap is None else cap
    idx = np.zeros(max(cap, 1), np.int32)
    val = np.zeros(max(cap, 1), np.float32)
    counts = np.zeros(nseg + 1, np.int64)
    rc = lib().orc_compress_exact(_p(g), _p(r), _p(seg_off), nseg, scope, ppm, _p(idx), _p(val), cap, _p(counts))
    if rc < 0:
        raise ValueError(f"orc_compress_exact failed: {rc}")
    return Sparse(idx[:rc].copy(), val[:rc].copy(), counts)


def compress_sampled(g, r: np.ndarray, seg_off, scope: int, ppm: int, cap: int,
                     sample_div: int = 1000, sample_min: int = 65536) -> Sparse:
    g = _f32(g)
    seg_off = np.ascontiguousarray(seg_off, dtype=np.int64)
    nseg = len(seg_off) - 1
    idx = np.zeros(max(cap, 1), np.int32)
    val = np.zeros(max(cap, 1), np.float32)
    counts = np.zeros(nseg + 1, np.int64)
    st = np.zeros(1, np.uint32)
    rc = lib().orc_compress_sampled(_p(g), _p(r), _p(seg_off), nseg, scope, ppm, sample_div, sample_min,
                                    _p(idx), _p(val), cap, _p(counts), _p(st))
    if rc < 0:
        raise ValueError(f"orc_compress_sampled failed: {rc}")
    return Sparse(idx[:rc].copy(), val[:rc].copy(), counts, int(st[0]))


def compress_momentum(g, u: np.ndarray, r: np.ndarray, beta: float, seg_off, scope: int, ppm: int,
                      sampled: bool = False, cap: Optional[int] = None, sample_div: int = 1000,
                      sample_min: int = 65536) -> Sparse:
    """One compress step with momentum correction and masking ([SBC] appendix A), in the pages'
    order: correct the momentum, compress with it in place of the gradient, mask the sent entries."""
    momentum_correct(beta, g, u)
    if sampled:
        sp = compress_sampled(u, r, seg_off, scope, ppm, cap, sample_div, sample_min)
    else:
        sp = compress_exact(u, r, seg_off, scope, ppm, cap)
    momentum_mask(u, sp.idx)
    return sp


@dataclass
class Binarized:
    idx: np.ndarray
    counts: np.ndarray
    means: np.ndarray
    codes: Optional[np.ndarray]


def binarize_held(sp: Sparse, nseg: int, mode: int, r: np.ndarray) -> Binarized:
    """Binarize when the residual holds acc (= val) at the kept entries: by definition the same as
    zeroing them first and binarizing as usual."""
    r[sp.idx] = 0.0
    return binarize(sp, nseg, mode, r)


def binarize(sp: Sparse, nseg: int, mode: int, r: np.ndarray) -> Binarized:
    total = int(sp.counts[nseg])
    out_idx = np.zeros(max(total, 1), np.int32)
    out_counts = np.zeros(nseg + 1, np.int64)
    means = np.zeros(nseg if mode == BIN_SBC else 2 * nseg, np.float32)
    codes = np.zeros(max((total + 15) // 16, 1), np.uint32) if mode == BIN_2BIT else None
    rc = lib().orc_binarize(_p(np.ascontiguousarray(sp.idx, np.int32)), _p(_f32(sp.val)),
                            _p(np.ascontiguousarray(sp.counts, np.int64)), nseg, mode, _p(r),
                            _p(out_idx), _p(out_counts), _p(means), _p(codes))
    if rc < 0:
        raise ValueError(f"orc_binarize failed: {rc}")
    return Binarized(out_idx[:rc].copy(), out_counts, means,
                     None if codes is None else codes[:(total + 15) // 16].copy())


@dataclass
class Encoded:
    words: np.ndarray      # uint32
    word_off: np.ndarray   # uint64 [nstreams+1]
    nbits: np.ndarray      # uint64 [nstreams]
    chunk_off: np.ndarray  # uint64 pairs: (bit offset, position reached) per 256 codes


def encode_bound_words(seg_off, counts, scope: int, b: int) -> int:
    """Host bound on the words a message can need (each stream padded)."""
    seg_off = np.asarray(seg_off, np.int64)
    nseg = len(seg_off) - 1
    streams = [(int(seg_off[-1]), int(counts[nseg]))] if scope == GLOBAL else \
        [(int(seg_off[t + 1] - seg_off[t]), int(counts[t])) for t in range(nseg)]
    words = 0
    for m, k in streams:
        bits = k * (b + 1) + ((m - k) >> b)
        words += (bits + 31) // 32
    return words


def encode(idx, counts, seg_off, scope: int, b: int) -> Encoded:
    seg_off = np.ascontiguousarray(seg_off, dtype=np.int64)
    counts = np.ascontiguousarray(counts, dtype=np.int64)
    nseg = len(seg_off) - 1
    nstreams = 1 if scope == GLOBAL else nseg
    word_cap = encode_bound_words(seg_off, counts, scope, b) + 1
    if scope == GLOBAL:
        chunk_cap = 2 * ((int(counts[nseg]) + CHUNK_CODES - 1) // CHUNK_CODES)
    else:
        chunk_cap = 2 * sum((int(c) + CHUNK_CODES - 1) // CHUNK_CODES for c in counts[:nseg])
    words = np.zeros(word_cap, np.uint32)
    word_off = np.zeros(nstreams + 1, np.uint64)
    nbits = np.zeros(nstreams, np.uint64)
    chunk_off = np.zeros(max(chunk_cap, 1), np.uint64)
    rc = lib().orc_encode(_p(np.ascontiguousarray(idx, np.int32)), _p(counts), _p(seg_off), nseg, scope, b,
                          _p(words), word_cap, _p(word_off), _p(nbits), _p(chunk_off), chunk_cap)
    if rc != 0:
        raise ValueError(f"orc_encode failed: {rc}")
    return Encoded(words[:int(word_off[-1])].copy(), word_off, nbits, chunk_off[:chunk_cap].copy())


def decode_stream(words, nbits: int, count: int, b: int, numel: int, chunk_off=None):
    """Positions of one Rice stream; returns (positions int64, status)."""
    words = np.ascontiguousarray(words, np.uint32)
    if words.size == 0:
        words = np.zeros(1, np.uint32)
    pos = np.zeros(max(count, 1), np.int64)
    st = np.zeros(1, np.uint32)
    co = None if chunk_off is None else np.ascontiguousarray(chunk_off, np.uint64)
    lib().orc_decode_stream(_p(words), nbits, count, b, numel, _p(co), _p(pos), _p(st))
    return pos[:count].copy(), int(st[0])


@dataclass
class Message:
    """One received worker message (host arrays).

    golomb: positions are Rice coded (enc) instead of given as idx.
    vkind:  VAL_F32 (val per entry), VAL_SBC (means[t]), VAL_2BIT (codes+means).
    """
    counts: np.ndarray
    vkind: int = VAL_F32
    golomb: bool = False
    scope: int = GLOBAL
    b: int = 0
    idx: Optional[np.ndarray] = None
    val: Optional[np.ndarray] = None
    codes: Optional[np.ndarray] = None
    means: Optional[np.ndarray] = None
    enc: Optional[Encoded] = None


def decode_accumulate(msgs: List[Message], seg_off, out: np.ndarray) -> int:
    """Add the messages into out (fp32, in place) in list order; returns status.

    The caller initialises out: zeros, the local dense gradient (global+local
    combination) or the buffer's previous contents.
    """
    seg_off = np.ascontiguousarray(seg_off, dtype=np.int64)
    nseg = len(seg_off) - 1
    st = np.zeros(1, np.uint32)
    for m in msgs:
        counts = np.ascontiguousarray(m.counts, np.int64)
        enc = m.enc
        words = None if enc is None else np.ascontiguousarray(enc.words if enc.words.size else np.zeros(1, np.uint32))
        rc = lib().orc_accumulate_message(
            _p(out), _p(seg_off), nseg, int(bool(m.golomb)), m.scope, m.b, m.vkind, _p(counts),
            _p(None if m.idx is None else np.ascontiguousarray(m.idx, np.int32)),
            _p(None if m.val is None else _f32(m.val)),
            _p(None if m.codes is None else np.ascontiguousarray(m.codes, np.uint32)),
            _p(None if m.means is None else _f32(m.means)),
            _p(words), _p(None if enc is None else enc.word_off), _p(None if enc is None else enc.nbits),
            _p(None if enc is None else (enc.chunk_off if enc.chunk_off.size else np.zeros(1, np.uint64))),
            _p(st))
        if rc != 0:
            raise ValueError(f"orc_accumulate_message failed: {rc}")
    return int(st[0])
