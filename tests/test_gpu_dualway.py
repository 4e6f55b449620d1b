"""Dual-way sparsification on one GPU: the aggregated update is compressed again.

Each of W simulated workers compresses its gradient (exact top-k with its own
residual) and Rice-codes the indices; a server sums the W messages in worker
order ([SBC] §I: the server aggregates the updates), compresses that sum with a
residual of its own and Rice-codes it, and every worker adds the downstream
message to its copy of the model.  The same four calls serve both directions
(compress, encode, decode_accumulate); every stage is compared with the oracle
bitwise, over two rounds so that every residual is carried.
"""
import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("scope", [0, 1])
def test_dual_way_two_rounds(orc, scope):
    rng = np.random.default_rng(31)
    layout = sgc.Layout([1 << 20, 300001, 4096, 77777])
    n = layout.n
    seg_off = np.array(layout.seg_off, np.int64)
    W, up_ppm, down_ppm = 4, 10000, 10000
    b_up, b_down = sgc.rice_param(up_ppm / 1e6), sgc.rice_param(down_ppm / 1e6)
    res_w = [np.zeros(n, np.float32) for _ in range(W)]
    res_wd = [dev(r) for r in res_w]
    res_s = np.zeros(n, np.float32)
    res_sd = dev(res_s)
    model = rng.normal(0, 1e-2, n).astype(np.float32)
    models_d = [dev(model) for _ in range(W)]
    for rnd in range(2):
        # upstream: every worker compresses and encodes
        gmsgs, omsgs = [], []
        for k in range(W):
            announce(f"dual-way round {rnd} worker {k} scope={scope}")
            g = rng.laplace(0, 1e-3, n).astype(np.float32)
            comp = sgc.compress(layout, dev(g), res_wd[k], scope=scope, keep_ppm=up_ppm)
            enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, scope=scope, b=b_up)
            ref = orc.compress_exact(g, res_w[k], seg_off, scope, up_ppm, cap=comp.cap)
            oenc = orc.encode(ref.idx, ref.counts, seg_off, scope, b_up)
            torch.cuda.synchronize()
            nw = int(oenc.word_off[-1])
            assert_bitwise(host(enc.words).view(np.uint32)[:nw], oenc.words, f"worker {k} words")
            assert_bitwise(host(res_wd[k]), res_w[k], f"worker {k} residual")
            gmsgs.append(sgc.golomb_message(comp, enc))
            omsgs.append(orc.Message(ref.counts, golomb=True, scope=scope, b=b_up, val=ref.val, enc=oenc))
        # server: sum in worker order, then compress the sum with its own residual
        announce(f"dual-way round {rnd} server")
        agg_d = torch.empty(n, dtype=torch.float32, device="cuda")
        st = sgc.decode_accumulate(layout, gmsgs, agg_d)
        agg = np.zeros(n, np.float32)
        assert orc.decode_accumulate(omsgs, seg_off, agg) == 0
        torch.cuda.synchronize()
        assert int(host(st)[0]) == 0
        assert_bitwise(host(agg_d), agg, "aggregate")
        down = sgc.compress(layout, agg_d, res_sd, scope=scope, keep_ppm=down_ppm)
        denc = sgc.encode(layout, down.idx, down.counts, down.cap, scope=scope, b=b_down)
        dref = orc.compress_exact(agg, res_s, seg_off, scope, down_ppm, cap=down.cap)
        doenc = orc.encode(dref.idx, dref.counts, seg_off, scope, b_down)
        torch.cuda.synchronize()
        total = int(dref.counts[-1])
        assert_bitwise(host(down.idx)[:total], dref.idx, "downstream idx")
        assert_bitwise(host(down.val)[:total], dref.val, "downstream val")
        assert_bitwise(host(res_sd), res_s, "server residual")
        nw = int(doenc.word_off[-1])
        assert_bitwise(host(denc.words).view(np.uint32)[:nw], doenc.words, "downstream words")
        # downstream: every worker adds the server's message to its model copy
        dmsg = sgc.golomb_message(down, denc)
        domsg = orc.Message(dref.counts, golomb=True, scope=scope, b=b_down, val=dref.val, enc=doenc)
        assert orc.decode_accumulate([domsg], seg_off, model) == 0
        for k in range(W):
            out = torch.empty(n, dtype=torch.float32, device="cuda")
            sgc.decode_accumulate(layout, [dmsg], out, init=sgc.INIT_BASE, base=models_d[k])
            models_d[k] = out
        torch.cuda.synchronize()
        for k in range(W):
            assert_bitwise(host(models_d[k]), model, f"round {rnd} worker {k} model")
