"""Worker steps captured in a HIP graph (torch's graph API) and replayed.

The library allocates nothing and queues no memset or synchronous call once
a layout's tables are on the device, so a whole step can be captured after
one eager warm-up call.  Each test replays its graph several times, with
eager work (a new gradient copied into the captured input) and a
synchronization between replays, and checks every replay against the CPU
oracle run on the same inputs.
"""
import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
import workloads as W
from gpu_util import announce, assert_bitwise, host

pytestmark = pytest.mark.gpu


def test_graph_compress_encode_flat(orc):
    w = W.FLAT_1M
    layout = sgc.Layout(w.seg_numel)
    n = w.numel
    seg_off = np.array(layout.seg_off, np.int64)
    ppm, b = w.keep_ppm, sgc.rice_param(w.keep_ppm / 1e6)
    g_in = torch.zeros(n, dtype=torch.float32, device="cuda")
    r = torch.zeros(n, dtype=torch.float32, device="cuda")
    comp = sgc.compress(layout, g_in, r, keep_ppm=ppm)  # warm-up: tables, workspace, outputs
    enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=b)
    torch.cuda.synchronize()
    r.zero_()

    def step():
        sgc.compress(layout, g_in, r, keep_ppm=ppm, out=comp)
        sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=b, out=enc)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    r_host = np.zeros(n, np.float32)
    for it in range(4):
        g = W.gradient(w, 0, it).numpy()
        g_in.copy_(torch.from_numpy(g))
        torch.cuda.synchronize()
        announce(f"graph replay {it}: flat-1M compress + encode")
        graph.replay()
        torch.cuda.synchronize()
        ref = orc.compress_exact(g, r_host, seg_off, sgc.GLOBAL, ppm, cap=comp.cap)
        total = int(ref.counts[-1])
        assert_bitwise(host(comp.counts), ref.counts, f"replay {it} counts")
        assert_bitwise(host(comp.idx)[:total], ref.idx, f"replay {it} idx")
        assert_bitwise(host(comp.val)[:total], ref.val, f"replay {it} val")
        assert_bitwise(host(r), r_host, f"replay {it} residual")
        oenc = orc.encode(ref.idx, ref.counts, seg_off, sgc.GLOBAL, b)
        nw = int(oenc.word_off[-1])
        assert_bitwise(host(enc.words).view(np.uint32)[:nw], oenc.words, f"replay {it} words")
        assert_bitwise(host(enc.chunk_off).view(np.uint64)[:oenc.chunk_off.size], oenc.chunk_off,
                       f"replay {it} chunk table")


def test_graph_per_tensor_sbc_round():
    # per-tensor top-0.1% + SBC + per-tensor Rice on the ResNet-50 layout, captured
    # once and replayed; every replay must equal the same step run eagerly from
    # the same state (the SBC means make the oracle comparison tolerance-based, the
    # graph-versus-eager one is bitwise)
    w = W.RESNET50
    layout = sgc.Layout(w.seg_numel)
    n = w.numel
    b = sgc.rice_param(w.keep_ppm / 1e6)
    g_in = torch.zeros(n, dtype=torch.float32, device="cuda")
    r = torch.zeros(n, dtype=torch.float32, device="cuda")
    comp = sgc.compress(layout, g_in, r, scope=sgc.PER_SEGMENT, keep_ppm=w.keep_ppm)
    bn = sgc.binarize(layout, comp, r, sgc.BIN_SBC)
    enc = sgc.encode(layout, bn.idx, bn.counts, bn.cap, scope=sgc.PER_SEGMENT, b=b)
    torch.cuda.synchronize()
    r.zero_()
    box = {}

    def step():
        sgc.compress(layout, g_in, r, scope=sgc.PER_SEGMENT, keep_ppm=w.keep_ppm, out=comp)
        box["bn"] = sgc.binarize(layout, comp, r, sgc.BIN_SBC)
        sgc.encode(layout, box["bn"].idx, box["bn"].counts, box["bn"].cap, scope=sgc.PER_SEGMENT, b=b, out=enc)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    r_eager = torch.zeros(n, dtype=torch.float32, device="cuda")
    for it in range(3):
        g_in.copy_(W.gradient(w, 0, it, device="cuda"))
        torch.cuda.synchronize()
        # eager reference from the same state
        ce = sgc.compress(layout, g_in, r_eager, scope=sgc.PER_SEGMENT, keep_ppm=w.keep_ppm)
        be = sgc.binarize(layout, ce, r_eager, sgc.BIN_SBC)
        ee = sgc.encode(layout, be.idx, be.counts, be.cap, scope=sgc.PER_SEGMENT, b=b)
        torch.cuda.synchronize()
        announce(f"graph replay {it}: resnet50 per-tensor compress + SBC + Rice")
        graph.replay()
        torch.cuda.synchronize()
        bg = box["bn"]
        total = int(host(be.counts)[-1])
        assert_bitwise(host(bg.counts), host(be.counts), f"replay {it} SBC counts")
        assert_bitwise(host(bg.means), host(be.means), f"replay {it} SBC means")
        assert_bitwise(host(bg.idx)[:total], host(be.idx)[:total], f"replay {it} SBC idx")
        assert_bitwise(host(r), host(r_eager), f"replay {it} residual")
        nw = int(host(ee.word_off)[-1])
        assert_bitwise(host(enc.words)[:nw], host(ee.words)[:nw], f"replay {it} words")
        assert_bitwise(host(enc.word_off), host(ee.word_off), f"replay {it} word offsets")
