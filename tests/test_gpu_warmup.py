"""Warm-up training as a carried sequence of steps ([SBC] appendix A, Warm-up
Training: the kept fraction falls exponentially, from 25% to 0.1%, over the
first epochs).  Each step takes its kept fraction from sgc_warmup_ppm (checked
against the oracle's own schedule), compresses with the residual carried from
the step before, and Rice-codes the result with the parameter that suits its
density; every output of every step is compared with the oracle bit for bit.
"""
import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
import workloads as W
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu


def run_schedule(orc, layout, grads, steps, mode, scope, what):
    seg_off = np.array(layout.seg_off, np.int64)
    n = layout.n
    rd = torch.zeros(n, dtype=torch.float32, device="cuda")
    r = np.zeros(n, np.float32)
    bs = []
    for t in range(steps):
        ppm = sgc.warmup_ppm(t, steps)
        assert ppm == orc.warmup_ppm(t, steps)
        b = sgc.rice_param(ppm / 1e6)
        bs.append(b)
        g = grads[t]
        announce(f"{what}: warm-up step {t} ppm={ppm} b={b}")
        comp = sgc.compress(layout, dev(g), rd, mode=mode, scope=scope, keep_ppm=ppm)
        enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, scope=scope, b=b)
        torch.cuda.synchronize()
        if mode == sgc.EXACT:
            ref = orc.compress_exact(g, r, seg_off, scope, ppm, cap=comp.cap)
        else:
            ref = orc.compress_sampled(g, r, seg_off, scope, ppm, comp.cap)
            assert (int(host(comp.status)[0]) & sgc.STATUS_TRUNCATED) == (ref.status & sgc.STATUS_TRUNCATED)
        total = int(ref.counts[-1])
        assert_bitwise(host(comp.counts), ref.counts, f"{what} step {t} counts")
        assert_bitwise(host(comp.idx)[:total], ref.idx, f"{what} step {t} idx")
        assert_bitwise(host(comp.val)[:total], ref.val, f"{what} step {t} val")
        assert_bitwise(host(rd), r, f"{what} step {t} residual")
        oenc = orc.encode(ref.idx, ref.counts, seg_off, scope, b)
        nw = int(oenc.word_off[-1])
        assert_bitwise(host(enc.word_off).view(np.uint64)[:oenc.word_off.size], oenc.word_off,
                       f"{what} step {t} word offsets")
        assert_bitwise(host(enc.words).view(np.uint32)[:nw], oenc.words, f"{what} step {t} words")
        assert_bitwise(host(enc.nbits).view(np.uint64)[:oenc.nbits.size], oenc.nbits, f"{what} step {t} nbits")
        assert_bitwise(host(enc.chunk_off).view(np.uint64)[:oenc.chunk_off.size], oenc.chunk_off,
                       f"{what} step {t} chunk table")
    return bs


def test_warmup_flat_1m_exact_six_steps(orc):
    # the flat 2^20 recipe, exact global selection, 25% -> 0.1% in six steps
    w = W.FLAT_1M
    layout = sgc.Layout(w.seg_numel)
    grads = [W.gradient(w, 0, t).numpy() for t in range(6)]
    bs = run_schedule(orc, layout, grads, 6, sgc.EXACT, sgc.GLOBAL, "flat-1M exact")
    assert bs[0] < bs[-1]   # the code parameter follows the falling density


def test_warmup_ragged_per_tensor_sampled(orc):
    # a ragged layout (empty and tiny tensors), per-tensor sampled selection
    # and per-tensor Rice streams, 25% -> 0.1% in eight steps
    rng = np.random.default_rng(404)
    layout = sgc.Layout([200003, 0, 7, 65536, 300000, 1, 90000])
    grads = [rng.laplace(0, 1e-3, layout.n).astype(np.float32) for _ in range(8)]
    run_schedule(orc, layout, grads, 8, sgc.SAMPLED, sgc.PER_SEGMENT, "ragged sampled")
