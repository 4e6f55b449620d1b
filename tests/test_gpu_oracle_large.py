"""Exact selection at large sizes, bit for bit against the CPU oracle.

The oracle's exact top-k is a full sort (tens of seconds at 10^8 elements on
one core), so each case here keeps to one or two steps, and the oracle runs
of a carried sequence overlap in threads: step s+1 of the oracle starts from
the residual the GPU left after step s, which the test has compared with the
oracle's own step-s residual bit for bit -- the same as running the oracle's
steps one after the other.

Cases (the kernel paths the benchmark's full-size step takes):
* a 2^28-element gradient of the flat-1G recipe, exact global top-1%, two
  carried steps, with the Rice streams (b = 6) of both steps, through the
  window pipeline (the one the 2^30 step takes) and the gather pipeline;
* the NMT-shaped gradient (97.8M elements, clustered embedding rows), exact
  global top-1%, two carried steps;
* 2^27 elements at 55% kept, which takes the gather pipeline's chunk-count
  scan split over workgroups (more than 16,384 chunks of kept entries), and
  the window pipeline on the same input.
Every output is compared: indices, values, per-segment counts, status and
the whole residual.
"""
import threading

import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
import workloads as W
from gpu_util import announce, assert_bitwise, host

pytestmark = pytest.mark.gpu


class OracleThread(threading.Thread):
    """One oracle compress_exact call in a thread (ctypes releases the GIL)."""

    def __init__(self, orc, g, r, seg_off, scope, ppm, cap):
        super().__init__(daemon=True)
        self.args_ = (orc, g, r, seg_off, scope, ppm, cap)
        self.result, self.error = None, None

    def run(self):
        orc, g, r, seg_off, scope, ppm, cap = self.args_
        try:
            self.result = orc.compress_exact(g, r, seg_off, scope, ppm, cap=cap)
        except BaseException as e:  # re-raised in the test thread
            self.error = e

    def get(self):
        self.join()
        if self.error is not None:
            raise self.error
        return self.result


def gpu_steps(layout, grads, ppm, scope=sgc.GLOBAL, b=None, path=sgc.PATH_AUTO):
    """Run the carried steps on the GPU; host copies of every output, the
    residual before each step, and (with b) the Rice streams."""
    n = layout.n
    rd = torch.zeros(n, dtype=torch.float32, device="cuda")
    steps = []
    for s, g in enumerate(grads):
        announce(f"GPU step {s}: n={n} ppm={ppm} path={path}")
        r_in = host(rd).copy()
        gd = torch.from_numpy(g).cuda()
        comp = sgc.compress(layout, gd, rd, keep_ppm=ppm, scope=scope, path=path)
        enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=b, scope=scope) if b is not None else None
        torch.cuda.synchronize()
        del gd
        counts = host(comp.counts)
        total = int(counts[-1])
        out = dict(r_in=r_in, counts=counts, idx=host(comp.idx)[:total].copy(), val=host(comp.val)[:total].copy(),
                   status=int(host(comp.status)[0]), r_out=host(rd).copy(), cap=comp.cap)
        if enc is not None:
            nw = int(host(enc.word_off)[-1])
            out["enc"] = dict(words=host(enc.words)[:nw].view(np.uint32).copy(),
                              word_off=host(enc.word_off).view(np.uint64).copy(),
                              nbits=host(enc.nbits).view(np.uint64).copy(),
                              chunk_off=host(enc.chunk_off).view(np.uint64).copy())
        steps.append(out)
        del comp, enc
    return steps


def check_against_oracle(orc, layout, grads, steps, ppm, scope=sgc.GLOBAL, b=None, what=""):
    seg_off = np.array(layout.seg_off, np.int64)
    # every oracle step at once, each from the residual the GPU started that step with
    threads = []
    for s, g in enumerate(grads):
        t = OracleThread(orc, g, steps[s]["r_in"].copy(), seg_off, scope, ppm, steps[s]["cap"])
        t.r = t.args_[2]
        t.start()
        threads.append(t)
    for s, t in enumerate(threads):
        ref = t.get()
        st = steps[s]
        announce(f"oracle step {s} {what}: compare")
        if s > 0:  # the residual this step started from is the oracle's own step-(s-1) residual
            assert_bitwise(st["r_in"], threads[s - 1].r, f"{what} step {s} input residual")
        assert_bitwise(st["counts"], ref.counts, f"{what} step {s} counts")
        assert_bitwise(st["idx"], ref.idx, f"{what} step {s} idx")
        assert_bitwise(st["val"], ref.val, f"{what} step {s} val")
        assert st["status"] & ~sgc.STATUS_DENSE_PATH == 0, f"{what} step {s} status {st['status']}"
        assert_bitwise(st["r_out"], t.r, f"{what} step {s} residual")
        if b is not None:
            oenc = orc.encode(ref.idx, ref.counts, seg_off, scope, b)
            e = st["enc"]
            nw = int(oenc.word_off[-1])
            assert_bitwise(e["word_off"][:oenc.word_off.size], oenc.word_off, f"{what} step {s} word offsets")
            assert_bitwise(e["words"][:nw], oenc.words, f"{what} step {s} words")
            assert_bitwise(e["nbits"][:oenc.nbits.size], oenc.nbits, f"{what} step {s} nbits")
            assert_bitwise(e["chunk_off"][:oenc.chunk_off.size], oenc.chunk_off, f"{what} step {s} chunk table")


def test_flat_2e28_exact_two_steps_with_rice(orc):
    # the headline step's kernels (exact global top-1% + Rice b = 6) on a
    # 2^28-element draw of the flat-1G recipe, two carried steps, through both
    # compress pipelines (the 2^30 step takes the window pipeline): the two
    # runs must agree bit for bit, and the window run with the oracle
    w = W.FLAT_1G
    n = 1 << 28
    layout = sgc.Layout([n])
    ppm = 10000
    b = sgc.rice_param(ppm / 1e6)
    grads = [host(W.gradient(w, 0, s, device="cuda", numel=n)) for s in range(2)]
    steps = gpu_steps(layout, grads, ppm, b=b, path=sgc.PATH_WINDOW)
    other = gpu_steps(layout, grads, ppm, b=b, path=sgc.PATH_GATHER)
    for s, (a, o) in enumerate(zip(steps, other)):
        for key in ("counts", "idx", "val", "r_out"):
            assert_bitwise(o[key], a[key], f"step {s} {key}: gather against window")
        nch = 2 * ((int(a["counts"][-1]) + 255) // 256)  # the chunk table's valid part (the rest is unused)
        for key, m in (("words", a["enc"]["words"].size), ("word_off", None), ("nbits", None), ("chunk_off", nch)):
            assert_bitwise(o["enc"][key][:m], a["enc"][key][:m], f"step {s} {key}: gather against window")
    del other
    assert all(int(st["counts"][-1]) == layout.keep_total(sgc.GLOBAL, ppm) for st in steps)
    check_against_oracle(orc, layout, grads, steps, ppm, b=b, what="flat 2^28 top-1%")


def test_nmt_exact_two_steps_carried(orc):
    # 97.8M elements whose embedding rows are clustered (Zipf-drawn rows,
    # zero elsewhere): exact global top-1% over two carried steps
    w = W.NMT_RNN
    layout = sgc.Layout(w.seg_numel)
    grads = [host(W.gradient(w, 0, s, device="cuda")) for s in range(2)]
    steps = gpu_steps(layout, grads, w.keep_ppm)
    check_against_oracle(orc, layout, grads, steps, w.keep_ppm, what="nmt-rnn")


def test_split_chunk_scan_2e27_55pct(orc):
    # 55% of 2^27 kept: 73.8M entries in more than 16,384 chunks, so the
    # gather pipeline's chunk-count scan is split over workgroups; the window
    # pipeline (the default at this density: whole-tile regions, one wave per
    # tile in the write) must agree with it bit for bit
    w = W.FLAT_1G
    n = 1 << 27
    layout = sgc.Layout([n])
    ppm = 550000
    k = layout.keep_total(sgc.GLOBAL, ppm)
    assert (k + 4095) // 4096 > 16384
    grads = [host(W.gradient(w, 0, 0, device="cuda", numel=n))]
    steps = gpu_steps(layout, grads, ppm, path=sgc.PATH_GATHER)
    other = gpu_steps(layout, grads, ppm, path=sgc.PATH_WINDOW)
    for key in ("counts", "idx", "val", "r_out"):
        assert_bitwise(other[0][key], steps[0][key], f"{key}: window against gather")
    del other
    assert int(steps[0]["counts"][-1]) == k
    check_against_oracle(orc, layout, grads, steps, ppm, what="2^27 at 55%")
