"""Worker steps and the receive side captured in a HIP graph (torch's graph
API) and replayed.

The library allocates nothing and queues no memset or synchronous call once
a layout's tables are on the device, so a whole step can be captured after
one eager warm-up call.  Captured calls get workspaces of their own (the
binding's cached ones could be replaced while a graph points at them).  Each test replays its graph several times, with
eager work (a new gradient copied into the captured input) and a
synchronization between replays, and checks every replay against the CPU
oracle run on the same inputs.
"""
import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
import workloads as W
from codec_util import make_messages
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("path", [sgc.PATH_GATHER, sgc.PATH_WINDOW], ids=["gather", "window"])
def test_graph_compress_encode_flat(orc, path):
    # flat-1M top-1% compress + Rice, through either compress pipeline
    w = W.FLAT_1M
    layout = sgc.Layout(w.seg_numel)
    n = w.numel
    seg_off = np.array(layout.seg_off, np.int64)
    ppm, b = w.keep_ppm, sgc.rice_param(w.keep_ppm / 1e6)
    g_in = torch.zeros(n, dtype=torch.float32, device="cuda")
    r = torch.zeros(n, dtype=torch.float32, device="cuda")
    comp = sgc.compress(layout, g_in, r, keep_ppm=ppm, path=path)  # warm-up: outputs
    enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=b)
    ws_c = torch.empty(sgc.compress_workspace_bytes(layout, keep_ppm=ppm, path=path), dtype=torch.uint8,
                       device="cuda")
    ws_e = torch.empty(sgc.encode_workspace_bytes(layout, sgc.GLOBAL, comp.cap), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    r.zero_()

    def step():
        sgc.compress(layout, g_in, r, keep_ppm=ppm, out=comp, ws=ws_c, path=path)
        sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=b, out=enc, ws=ws_e)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    r_host = np.zeros(n, np.float32)
    for it in range(4):
        g = W.gradient(w, 0, it).numpy()
        g_in.copy_(torch.from_numpy(g))
        torch.cuda.synchronize()
        announce(f"graph replay {it}: flat-1M compress + encode, path {path}")
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
    u8 = dict(dtype=torch.uint8, device="cuda")
    ws_c = torch.empty(sgc.compress_workspace_bytes(layout, scope=sgc.PER_SEGMENT, keep_ppm=w.keep_ppm), **u8)
    ws_b = torch.empty(sgc.binarize_workspace_bytes(layout, comp.cap), **u8)
    ws_e = torch.empty(sgc.encode_workspace_bytes(layout, sgc.PER_SEGMENT, bn.cap), **u8)
    torch.cuda.synchronize()
    r.zero_()
    box = {}

    def step():
        sgc.compress(layout, g_in, r, scope=sgc.PER_SEGMENT, keep_ppm=w.keep_ppm, out=comp, ws=ws_c)
        box["bn"] = sgc.binarize(layout, comp, r, sgc.BIN_SBC, ws=ws_b)
        sgc.encode(layout, box["bn"].idx, box["bn"].counts, box["bn"].cap, scope=sgc.PER_SEGMENT, b=b, out=enc,
                   ws=ws_e)

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


def _tensors(m):
    """The device tensors a message reads, in a fixed order."""
    e = m.enc
    ts = [m.counts, m.idx, m.val, m.codes, m.means]
    if e is not None:
        ts += [e.words, e.word_off, e.nbits, e.chunk_off]
    return [t for t in ts if t is not None]


def test_graph_receive(orc):
    # decode + ordered sum of four message kinds onto a local gradient,
    # captured once; before each replay a new set of messages (same shapes:
    # exact selection keeps the counts' totals and so the capacities) is
    # copied into the captured buffers; the workspace and status are the
    # test's own, so no later call can reallocate what the graph points at
    rng = np.random.default_rng(77)
    layout = sgc.Layout([300000, 7, 120000, 0, 65536, 1000])
    n = layout.n
    seg_off = np.array(layout.seg_off, np.int64)
    kinds = ["raw_f32", "golomb_f32_seg", "golomb_sbc", "golomb_2bit"]
    sets = [make_messages(orc, layout, rng, kinds) for _ in range(4)]
    cap_msgs = sets[0][0]
    for gm, _ in sets[1:]:
        for a, b in zip(cap_msgs, gm):
            assert [t.shape for t in _tensors(a)] == [t.shape for t in _tensors(b)]
    base_h = rng.normal(0, 1e-3, n).astype(np.float32)
    base = dev(base_h)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    arr = (sgc.MessageDesc * len(cap_msgs))(*[m.desc() for m in cap_msgs])
    ws = torch.empty(max(int(sgc.lib().sgc_decode_accumulate_workspace(layout.handle, arr, len(cap_msgs))), 256),
                     dtype=torch.uint8, device="cuda")
    sgc.decode_accumulate(layout, cap_msgs, out, init=sgc.INIT_BASE, base=base, status=status, ws=ws)  # eager
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sgc.decode_accumulate(layout, cap_msgs, out, init=sgc.INIT_BASE, base=base, status=status, ws=ws)
    torch.cuda.synchronize()
    for it, (gm, om) in enumerate(sets[1:]):
        for a, b in zip(cap_msgs, gm):
            for dst, src in zip(_tensors(a), _tensors(b)):
                dst.copy_(src)
        status.zero_()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        announce(f"graph replay {it}: receive of {len(gm)} messages ({', '.join(kinds)})")
        graph.replay()
        torch.cuda.synchronize()
        ref = base_h.copy()
        ost = orc.decode_accumulate(om, seg_off, ref)
        assert ost == 0 and int(host(status)[0]) == 0, f"replay {it}: status {ost} / {int(host(status)[0])}"
        assert_bitwise(host(out), ref, f"replay {it}: dense sum")
