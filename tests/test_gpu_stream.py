"""The whole path on a caller's stream (the binding's stream argument, not
torch's current stream): compress, SBC binarize, per-tensor Rice encode and
decode-accumulate queued on a side stream of default priority must give
the same bytes as on the default stream, and the compress step the oracle's.
"""
import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu


def run_path(layout, g, r0, base, stream):
    gd, rd, bd = dev(g), dev(r0), dev(base)
    out = torch.empty(layout.n, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()  # inputs in place before another stream reads them
    comp = sgc.compress(layout, gd, rd, scope=sgc.PER_SEGMENT, keep_ppm=20000, stream=stream)
    bn = sgc.binarize(layout, comp, rd, sgc.BIN_SBC, stream=stream)
    enc = sgc.encode(layout, bn.idx, bn.counts, bn.cap, scope=sgc.PER_SEGMENT, b=5, stream=stream)
    st = sgc.decode_accumulate(layout, [sgc.raw_message(comp), sgc.golomb_message(bn, enc)], out,
                               init=sgc.INIT_BASE, base=bd, stream=stream)
    torch.cuda.synchronize()
    return comp, bn, enc, rd, out, st


def test_side_stream_whole_path(orc):
    rng = np.random.default_rng(91)
    layout = sgc.Layout([70000, 0, 17, 130000, 4096])
    n = layout.n
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    r0 = (rng.normal(0, 3e-4, n) * (rng.random(n) < 0.5)).astype(np.float32)
    base = rng.normal(0, 1e-3, n).astype(np.float32)
    side = torch.cuda.Stream()
    announce("whole path on a side stream")
    cs, bs, es, rs, os_, ss = run_path(layout, g, r0, base, side)
    announce("whole path on the default stream")
    cd, bd, ed, rd, od, sd = run_path(layout, g, r0, base, None)
    ref = orc.compress_exact(g, r0.copy(), np.array(layout.seg_off, np.int64), sgc.PER_SEGMENT, 20000, cap=cs.cap)
    total = int(ref.counts[-1])
    assert_bitwise(host(cs.counts), ref.counts, "side stream counts")
    assert_bitwise(host(cs.idx)[:total], ref.idx, "side stream idx")
    assert_bitwise(host(cs.val)[:total], ref.val, "side stream val")
    assert int(host(ss)[0]) == 0 and int(host(sd)[0]) == 0
    for what, a, b in (("SBC counts", bs.counts, bd.counts), ("SBC means", bs.means, bd.means),
                       ("word offsets", es.word_off, ed.word_off), ("residual", rs, rd), ("dense sum", os_, od)):
        assert_bitwise(host(a), host(b), f"side vs default stream: {what}")
    nw = int(host(ed.word_off)[-1])
    assert_bitwise(host(es.words)[:nw], host(ed.words)[:nw], "side vs default stream: words")


def test_two_streams_overlapping_calls(orc):
    # Two side streams each run three compress steps back to back, with no
    # synchronization between the calls and a kept fraction that grows from
    # step to step (each call needs a larger workspace than the one before,
    # so the binding replaces its cached buffer while earlier calls may still
    # be queued).  Each stream has its own cached workspace and its own
    # residual; every step must equal the oracle's.
    rng = np.random.default_rng(17)
    layout = sgc.Layout([300000, 5000, 123457])
    n = layout.n
    seg_off = np.array(layout.seg_off, np.int64)
    ppms = (2000, 20000, 120000)
    gs = [[rng.laplace(0, 1e-3, n).astype(np.float32) for _ in ppms] for _ in range(2)]
    gd = [[dev(g) for g in row] for row in gs]
    rd = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    announce("two side streams, three growing compress steps each, no sync between calls")
    outs = [[], []]
    for step, ppm in enumerate(ppms):
        for w in range(2):
            outs[w].append(sgc.compress(layout, gd[w][step], rd[w], keep_ppm=ppm, stream=streams[w]))
    torch.cuda.synchronize()
    for w in range(2):
        r = np.zeros(n, np.float32)
        for step, ppm in enumerate(ppms):
            ref = orc.compress_exact(gs[w][step], r, seg_off, sgc.GLOBAL, ppm, cap=outs[w][step].cap)
            total = int(ref.counts[-1])
            c = outs[w][step]
            assert_bitwise(host(c.counts), ref.counts, f"stream {w} step {step} counts")
            assert_bitwise(host(c.idx)[:total], ref.idx, f"stream {w} step {step} idx")
            assert_bitwise(host(c.val)[:total], ref.val, f"stream {w} step {step} val")
        assert_bitwise(host(rd[w]), r, f"stream {w} residual")


def test_layout_without_upload_is_refused():
    # The compute calls never upload a layout's tables: a layout that was not
    # uploaded to the device is refused (ENOTREADY) before any GPU work, and
    # works once sgc_layout_upload has run.
    import ctypes as C
    lib = sgc.lib()
    sizes = (C.c_int64 * 2)(5000, 3000)
    h = C.c_void_p()
    assert lib.sgc_layout_create(sizes, 2, C.byref(h)) == sgc.OK
    try:
        n = 8000
        o = sgc.CompressOpts(sgc.EXACT, sgc.GLOBAL, 10000, 1000, 65536)
        k = sgc.keep_count(n, 10000)
        need = lib.sgc_compress_workspace(h, C.byref(o), k)
        g = torch.randn(n, device="cuda") * 1e-3
        r = torch.zeros(n, device="cuda")
        idx = torch.empty(k, dtype=torch.int32, device="cuda")
        val = torch.empty(k, dtype=torch.float32, device="cuda")
        cnt = torch.empty(3, dtype=torch.int64, device="cuda")
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        P = lambda t: C.c_void_p(t.data_ptr())
        args = (C.byref(o), P(g), P(r), P(idx), P(val), k, P(cnt), None, P(ws), need, None)
        assert lib.sgc_compress(h, *args) == sgc.ENOTREADY
        assert lib.sgc_layout_upload(h) == sgc.OK
        assert lib.sgc_layout_upload(h) == sgc.OK   # a second upload does nothing
        assert lib.sgc_compress(h, *args) == sgc.OK
        torch.cuda.synchronize()
        assert int(cnt[-1]) == k
        acc = g.cpu().numpy()
        top = np.sort(np.abs(acc))[::-1][k - 1]
        assert np.abs(host(val)).min() == top
    finally:
        lib.sgc_layout_destroy(h)
