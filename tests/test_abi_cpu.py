"""The C-ABI library on a host without a GPU: it loads, exports every symbol
include/sgc.h declares, its host helpers agree with the oracle, and every
argument error is reported by its return code before any GPU work.
"""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

import compressed_sgd_amd as sgc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgc.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgc_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 18
    out = subprocess.run(["nm", "-D", "--defined-only", sgc.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT\s+(sgc_\w+)", out.stdout))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    assert sorted(sgc.EXPORTED) == names
    lib = sgc.lib()
    for n in names:
        getattr(lib, n)


def test_abi_version_and_strerror():
    assert sgc.abi_version() == 3
    for code in (0, -1, -2, -3, -4, -5, 99):
        assert sgc.lib().sgc_strerror(code)
    assert b"upload" in sgc.lib().sgc_strerror(sgc.ENOTREADY)


def test_layout_upload_arguments():
    lib = sgc.lib()
    assert lib.sgc_layout_upload(None) == sgc.EINVAL
    lay = sgc.Layout([10, 20])    # no GPU here: nothing uploaded
    assert not lay._devices
    assert lib.sgc_layout_upload(lay.handle) in (sgc.OK, sgc.EHIP)   # EHIP: no device to upload to


def test_reused_compress_output_is_checked():
    import torch
    lay = sgc.Layout([1000, 24])
    cpu = torch.device("cpu")
    k = lay.keep_total(sgc.GLOBAL, 10000)
    out, cap = sgc._compress_out(lay, None, None, sgc.EXACT, sgc.GLOBAL, 10000, cpu, None)
    assert cap == k and out.cap == k and out.idx.numel() == k and out.counts.numel() == lay.nseg + 1
    # reused: cap defaults to the buffer's own
    again, cap2 = sgc._compress_out(lay, out, None, sgc.EXACT, sgc.GLOBAL, 50000, cpu, None)
    assert again is out and cap2 == k
    # a larger kept fraction, or sampled mode's larger default cap, does not fit
    with pytest.raises(ValueError):
        sgc._compress_out(lay, out, lay.keep_total(sgc.GLOBAL, 50000), sgc.EXACT, sgc.GLOBAL, 50000, cpu, None)
    with pytest.raises(ValueError):
        sgc._compress_out(lay, out, sgc._default_cap(lay, sgc.SAMPLED, sgc.GLOBAL, 10000), sgc.SAMPLED,
                          sgc.GLOBAL, 10000, cpu, None)
    # a buffer made for another layout
    other = sgc.Layout([1000, 20, 4])
    with pytest.raises(ValueError):
        sgc._compress_out(other, out, None, sgc.EXACT, sgc.GLOBAL, 10000, cpu, None)
    # a smaller cap is accepted and becomes the buffer's cap
    _, cap3 = sgc._compress_out(lay, out, k - 1, sgc.SAMPLED, sgc.GLOBAL, 10000, cpu, None)
    assert cap3 == k - 1 and out.cap == k - 1


def test_reused_encode_output_is_checked():
    import torch
    cpu = torch.device("cpu")
    g = sgc._encode_out(None, sgc.GLOBAL, 6, 100, 40, 4, 1, cpu, None)
    assert g.word_off.numel() == 2 and g.nbits.numel() == 1
    assert sgc._encode_out(g, sgc.GLOBAL, 6, 100, 40, 4, 1, cpu, None) is g
    # per-tensor streams need nstreams + 1 offsets: a global buffer is replaced
    p = sgc._encode_out(g, sgc.PER_SEGMENT, 6, 100, 40, 4, 5, cpu, None)
    assert p is not g and p.word_off.numel() == 6 and p.nbits.numel() == 5 and p.scope == sgc.PER_SEGMENT
    assert sgc._encode_out(p, sgc.GLOBAL, 6, 100, 41, 4, 1, cpu, None) is not p   # words too small


def test_keep_count_matches_oracle(orc):
    for n in (0, 1, 7, 64, 100, 1 << 20, 2359296, (1 << 31) - 1):
        for ppm in (0, 1, 1000, 10000, 999999, 1000000):
            assert sgc.keep_count(n, ppm) == orc.keep_count(n, ppm)
    assert sgc.keep_count(-1, 10) == -1
    assert sgc.keep_count(10, 1000001) == -1


def test_rice_param_matches_oracle(orc):
    for p in (1.0, 0.5, 0.1, 0.03, 0.01, 0.001, 1e-4, 1e-6):
        assert sgc.rice_param(p) == orc.rice_param(p)
    assert sgc.rice_param(0.0) == -1 and sgc.rice_param(1.5) == -1


def test_warmup_ppm_matches_oracle(orc):
    for T in (1, 2, 6, 20, 37, 100):
        for t in range(0, T + 3):
            for a, b in ((250000, 1000), (1000000, 1), (10000, 10000), (1000, 250000)):
                assert sgc.lib().sgc_warmup_ppm(t, T, a, b) == orc.warmup_ppm(t, T, a, b)
    assert sgc.warmup_ppm(0, 20) == 250000 and sgc.warmup_ppm(19, 20) == 1000
    for bad in ((-1, 6, 1, 1), (0, 0, 1, 1), (0, 6, 0, 1), (0, 6, 1, 0), (0, 6, 1000001, 1)):
        assert sgc.lib().sgc_warmup_ppm(*bad) == -1
        assert orc.warmup_ppm(*bad) == -1


def test_layout_validation():
    lib = sgc.lib()
    h = C.c_void_p()
    arr = (C.c_int64 * 3)(5, -1, 3)
    assert lib.sgc_layout_create(arr, 3, C.byref(h)) == sgc.EINVAL
    assert lib.sgc_layout_create(arr, 0, C.byref(h)) == sgc.EINVAL
    big = (C.c_int64 * 2)(1 << 30, 1 << 30)
    assert lib.sgc_layout_create(big, 2, C.byref(h)) == sgc.EINVAL
    ok = (C.c_int64 * 2)((1 << 30), (1 << 30) - 1)
    assert lib.sgc_layout_create(ok, 2, C.byref(h)) == sgc.OK
    assert lib.sgc_layout_numel(h) == (1 << 31) - 1 and lib.sgc_layout_nseg(h) == 2
    lib.sgc_layout_destroy(h)


P = C.c_void_p
A = P(4096)      # stand-in device pointers: never dereferenced, validation fails first
MIS = P(4100)    # misaligned for fp32 vector access


def test_compress_validation():
    lib = sgc.lib()
    lay = sgc.Layout([1000, 24])
    k = lay.keep_total(sgc.GLOBAL, 10000)
    o = sgc.CompressOpts(sgc.EXACT, sgc.GLOBAL, 10000, 1000, 65536)
    ws_need = lib.sgc_compress_workspace(lay.handle, C.byref(o), k)
    assert ws_need > 0
    call = lambda opt, g=A, r=A, oi=A, ov=A, cap=k, oc=A, ws=A, wsb=ws_need: \
        lib.sgc_compress(lay.handle, C.byref(opt) if opt is not None else None, g, r, oi, ov, cap, oc, None, ws, wsb, None)
    assert call(None) == sgc.EINVAL
    assert call(sgc.CompressOpts(7, 0, 10000, 1000, 1)) == sgc.EINVAL
    assert call(sgc.CompressOpts(0, 5, 10000, 1000, 1)) == sgc.EINVAL
    assert call(sgc.CompressOpts(0, 0, 1000001, 1000, 1)) == sgc.EINVAL
    assert call(sgc.CompressOpts(1, 0, 10000, 0, 1)) == sgc.EINVAL       # sample_div 0
    assert call(o, g=None) == sgc.EINVAL
    assert call(o, r=MIS) == sgc.EINVAL
    assert call(o, cap=k - 1) == sgc.EINVAL                              # exact needs cap >= k
    assert call(o, oc=None) == sgc.EINVAL
    assert call(o, oi=None) == sgc.EINVAL
    assert call(o, ws=None) == sgc.ENOSPC
    assert call(o, wsb=ws_need - 1) == sgc.ENOSPC
    assert lib.sgc_compress_workspace(lay.handle, C.byref(sgc.CompressOpts(9, 0, 1, 1, 1)), 5) == 0
    assert call(sgc.CompressOpts(0, 0, 10000, 1000, 1, 3)) == sgc.EINVAL   # no such pipeline
    assert lib.sgc_compress_workspace(lay.handle, C.byref(sgc.CompressOpts(0, 0, 10000, 1000, 1, 3)), k) == 0


@pytest.mark.parametrize("sizes,ppm,auto", [([1 << 20, 4097], 10000, sgc.PATH_GATHER),
                                            ([1 << 20, 4097], 25000, sgc.PATH_GATHER),
                                            ([1 << 20, 4097], 30000, sgc.PATH_WINDOW),
                                            ([1 << 20, 4097], 250000, sgc.PATH_WINDOW),
                                            ([(1 << 29) - 1], 10000, sgc.PATH_GATHER),
                                            ([1 << 28, 1 << 28], 10000, sgc.PATH_WINDOW)])
def test_compress_path_choice(sizes, ppm, auto):
    # each pipeline sizes its own workspace; by default the gather pipeline takes the
    # kept fractions whose candidate regions are the smallest (256 slots) on vectors
    # below 2^29 elements, window the rest
    lib = sgc.lib()
    lay = sgc.Layout(sizes)
    ws = {p: lib.sgc_compress_workspace(lay.handle, C.byref(sgc.CompressOpts(sgc.EXACT, 0, ppm, 1000, 65536, p)),
                                        lay.keep_total(0, ppm))
          for p in (sgc.PATH_AUTO, sgc.PATH_GATHER, sgc.PATH_WINDOW)}
    assert ws[sgc.PATH_GATHER] > 0 and ws[sgc.PATH_WINDOW] > 0
    assert ws[sgc.PATH_GATHER] != ws[sgc.PATH_WINDOW]
    assert ws[sgc.PATH_AUTO] == ws[auto]
    assert sgc.compress_workspace_bytes(lay, keep_ppm=ppm) == ws[auto]
    assert sgc.compress_workspace_bytes(lay, keep_ppm=ppm, path=sgc.PATH_WINDOW) == ws[sgc.PATH_WINDOW]


def test_compress_momentum_validation():
    lib = sgc.lib()
    lay = sgc.Layout([1000, 24])
    k = lay.keep_total(sgc.GLOBAL, 10000)
    o = sgc.CompressOpts(sgc.EXACT, sgc.GLOBAL, 10000, 1000, 65536)
    need = lib.sgc_compress_momentum_workspace(lay.handle, C.byref(o), k)
    assert need > lib.sgc_compress_workspace(lay.handle, C.byref(o), k) > 0
    call = lambda beta=0.9, u=A, wsb=need, opt=o: lib.sgc_compress_momentum(
        lay.handle, C.byref(opt), beta, A, u, A, A, A, k, A, None, A, wsb, None)
    assert call(beta=float("nan")) == sgc.EINVAL
    assert call(beta=float("-inf")) == sgc.EINVAL
    assert call(u=None) == sgc.EINVAL
    assert call(u=MIS) == sgc.EINVAL
    assert call(opt=sgc.CompressOpts(7, 0, 10000, 1000, 1)) == sgc.EINVAL
    assert call(wsb=need - 1) == sgc.ENOSPC
    assert lib.sgc_compress_momentum_workspace(lay.handle, C.byref(sgc.CompressOpts(9, 0, 1, 1, 1)), 5) == 0
    held = sgc.CompressOpts(sgc.EXACT | sgc.HOLD_KEPT, sgc.GLOBAL, 10000, 1000, 65536)
    assert call(opt=held) == sgc.EUNSUPPORTED
    assert lib.sgc_compress_momentum_workspace(lay.handle, C.byref(held), k) == 0


def test_hold_flag_validation():
    lib = sgc.lib()
    lay = sgc.Layout([1000, 24])
    k = lay.keep_total(sgc.GLOBAL, 10000)
    plain = sgc.CompressOpts(sgc.EXACT, sgc.GLOBAL, 10000, 1000, 65536)
    held = sgc.CompressOpts(sgc.EXACT | sgc.HOLD_KEPT, sgc.GLOBAL, 10000, 1000, 65536)
    held_s = sgc.CompressOpts(sgc.SAMPLED | sgc.HOLD_KEPT, sgc.GLOBAL, 10000, 1000, 65536)
    bad = sgc.CompressOpts(sgc.ACCUMULATE_ONLY | sgc.HOLD_KEPT, sgc.GLOBAL, 10000, 1000, 65536)
    need = lib.sgc_compress_workspace(lay.handle, C.byref(plain), k)
    assert lib.sgc_compress_workspace(lay.handle, C.byref(held), k) == need
    assert lib.sgc_compress_workspace(lay.handle, C.byref(held_s), k) > 0
    assert lib.sgc_compress_workspace(lay.handle, C.byref(bad), k) == 0
    assert lib.sgc_compress(lay.handle, C.byref(bad), A, A, A, A, k, A, None, A, need, None) == sgc.EINVAL
    bneed = lib.sgc_binarize_workspace(lay.handle, 10)
    assert lib.sgc_binarize(lay.handle, 2 | sgc.BIN_HELD, A, A, A, 10, A, A, A, A, A, A, bneed, None) == sgc.EINVAL


def test_binarize_validation():
    lib = sgc.lib()
    lay = sgc.Layout([100, 100])
    need = lib.sgc_binarize_workspace(lay.handle, 10)
    call = lambda mode=0, cap=10, res=A, oidx=A, cnt=A, means=A, codes=A, ws=A, wsb=need: \
        lib.sgc_binarize(lay.handle, mode, A, A, cnt, cap, res, oidx, A, means, codes, ws, wsb, None)
    assert call(mode=3) == sgc.EINVAL
    assert call(cap=-1) == sgc.EINVAL
    assert call(cnt=None) == sgc.EINVAL
    assert call(res=None) == sgc.EINVAL
    assert call(oidx=None) == sgc.EINVAL            # SBC needs out_idx
    assert call(mode=1, codes=None) == sgc.EINVAL   # 2-bit needs codes
    assert call(ws=None) == sgc.ENOSPC
    assert call(wsb=need - 1) == sgc.ENOSPC


def test_encode_validation_and_bounds():
    lib = sgc.lib()
    lay = sgc.Layout([5000, 3000])
    cap = 100
    wb = lib.sgc_encode_word_bound(lay.handle, 0, 6, cap)
    cb = lib.sgc_encode_chunk_bound(lay.handle, 1, cap)
    assert wb == -(-(cap * 7 + (8000 >> 6)) // 32) + 1
    assert cb == 2 * (1 + 2)   # (bit offset, position reached) per chunk; one chunk per stream + ceil(cap/256)
    assert lib.sgc_encode_word_bound(lay.handle, 0, 31, cap) == -1
    need = lib.sgc_encode_workspace(lay.handle, 0, cap)
    call = lambda scope=0, b=6, wcap=wb, ccap=cb, ws=A, wsb=need, idx=A: \
        lib.sgc_encode(lay.handle, scope, b, idx, A, cap, A, wcap, A, A, A, ccap, None, ws, wsb, None)
    assert call(scope=2) == sgc.EINVAL
    assert call(b=-1) == sgc.EINVAL
    assert call(idx=None) == sgc.EINVAL
    assert call(wcap=wb - 1) == sgc.ENOSPC
    assert call(ccap=0) == sgc.ENOSPC
    assert call(wsb=need - 1) == sgc.ENOSPC


def test_encode_word_bound_holds_for_oracle_streams(orc):
    # the host bound must cover any message with at most cap entries
    rng = np.random.default_rng(3)
    sizes = [7000, 0, 13, 20000]
    lay = sgc.Layout(sizes)
    seg_off = np.array(lay.seg_off, np.int64)
    for b in (0, 2, 6, 9):
        for scope in (0, 1):
            for dens in (0.0005, 0.05, 0.9):
                sel = np.flatnonzero(rng.random(lay.n) < dens).astype(np.int32)
                counts = np.array([((sel >= seg_off[t]) & (sel < seg_off[t + 1])).sum() for t in range(4)]
                                  + [sel.size], np.int64)
                enc = orc.encode(sel, counts, seg_off, scope, b)
                assert int(enc.word_off[-1]) <= sgc.lib().sgc_encode_word_bound(lay.handle, scope, b, sel.size)
                assert enc.chunk_off.size <= sgc.lib().sgc_encode_chunk_bound(lay.handle, scope, sel.size)


def test_decode_accumulate_validation():
    lib = sgc.lib()
    lay = sgc.Layout([100])
    m = sgc.MessageDesc(sgc.MSG_RAW_F32, 0, 0, 0, 10, A, A, A, None, None, None, None, None, None)
    arr = (sgc.MessageDesc * 1)(m)
    need = lib.sgc_decode_accumulate_workspace(lay.handle, arr, 1)
    assert need > 0
    call = lambda a=arr, W=1, init=0, base=A, out=A, ws=A, wsb=need: \
        lib.sgc_decode_accumulate(lay.handle, a, W, init, base, out, None, ws, wsb, None)
    assert call(init=5) == sgc.EINVAL
    assert call(out=MIS) == sgc.EINVAL
    assert call(init=1, base=None) == sgc.EINVAL
    assert call(wsb=need - 1) == sgc.ENOSPC
    bad = (sgc.MessageDesc * 1)(sgc.MessageDesc(9, 0, 0, 0, 10, A, A, A, None, None, None, None, None, None))
    assert call(a=bad) == sgc.EINVAL
    nov = (sgc.MessageDesc * 1)(sgc.MessageDesc(sgc.MSG_RAW_F32, 0, 0, 0, 10, A, A, None, None, None, None, None,
                                                None, None))
    assert call(a=nov) == sgc.EINVAL
    gol = (sgc.MessageDesc * 1)(sgc.MessageDesc(sgc.MSG_GOLOMB_F32, 0, 40, 0, 10, A, None, A, None, None, A, A, A, A))
    assert call(a=gol) == sgc.EINVAL   # rice_b out of range
    assert lib.sgc_decode_accumulate_workspace(lay.handle, bad, 1) == 0


def test_binding_refuses_host_tensors():
    import torch
    lay = sgc.Layout([10])
    with pytest.raises(ValueError):
        sgc.compress(lay, torch.zeros(10), torch.zeros(10))
