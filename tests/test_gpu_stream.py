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
