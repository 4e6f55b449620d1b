"""Randomised multi-step parity of the carried state: residual (and momentum)
over a sequence of worker steps, bitwise against the CPU oracle.

Each case fixes a layout, whether momentum correction is on (and its
coefficient), then runs 4 to 7 steps.  A step is either a communication-
delay accumulation or an exchange: exact or sampled selection at a random
kept fraction and scope (through either compress pipeline, in turn), with
or without the hold flag, followed (plain path only) by no binarization,
SBC or 2-bit, held or not.  After every step
the GPU residual and momentum must equal the oracle's bit for bit, and the
sent indices and values likewise.  Binarize means must agree to 1e-6
relative; where they are bit-equal (the usual case) the sent set, codes and
residual must match exactly, and where one rounding apart (a different fixed
summation order) the sequence ends, since the residuals then part ways.
"""
import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu

REL = 1e-6
PPMS = [0, 500, 3000, 10000, 60000, 300000, 1000000]


def check_sparse(comp, ref, what):
    counts = host(comp.counts)
    total = int(counts[-1])
    assert_bitwise(counts, ref.counts, f"{what} counts")
    assert_bitwise(host(comp.idx)[:total], ref.idx, f"{what} idx")
    assert_bitwise(host(comp.val)[:total], ref.val, f"{what} val")


@pytest.mark.parametrize("seed", range(45))
def test_random_steps(orc, seed):
    rng = np.random.default_rng(8100 + seed)
    nseg = int(rng.integers(1, 8))
    sizes = [int(x) for x in rng.integers(0, 90000, nseg)]
    if sum(sizes) == 0:
        sizes[0] = 3000
    run_sequence(orc, rng, sgc.Layout(sizes), seed)


@pytest.mark.parametrize("seed", range(4))
def test_random_steps_many_segments(orc, seed):
    # 1500 segments: the per-segment bookkeeping in several rounds, under every kind of step
    rng = np.random.default_rng(8300 + seed)
    sizes = [int(x) for x in rng.integers(0, 2500, 1500)]
    for t in range(0, len(sizes), 5):
        sizes[t] = 0
    run_sequence(orc, rng, sgc.Layout(sizes), seed)


def run_sequence(orc, rng, layout, seed):
    n = layout.n
    seg_off = np.array(layout.seg_off, np.int64)
    mom = rng.random() < 0.4
    beta = float(rng.choice([0.0, 0.5, 0.9, -0.3])) if mom else 0.0
    r = np.zeros(n, np.float32)
    u = np.zeros(n, np.float32)
    rd, ud = dev(r), dev(u)
    steps = int(rng.integers(4, 8))
    for step in range(steps):
        g = rng.laplace(0, 1e-3, n).astype(np.float32)
        if rng.random() < 0.25:
            g = (np.round(g * 2e3) / 2e3).astype(np.float32)  # ties
        what = f"seed {seed} step {step}"
        if rng.random() < 0.3:  # communication delay: accumulate only
            announce(f"{what}: accumulate momentum={mom}")
            if mom:
                sgc.compress_momentum(layout, dev(g), ud, rd, beta, mode=sgc.ACCUMULATE_ONLY)
                orc.momentum_correct(beta, g, u)
                orc.accumulate(u, r)
            else:
                sgc.compress(layout, dev(g), rd, mode=sgc.ACCUMULATE_ONLY)
                orc.accumulate(g, r)
            torch.cuda.synchronize()
            assert_bitwise(host(rd), r, f"{what} residual")
            if mom:
                assert_bitwise(host(ud), u, f"{what} momentum")
            continue
        ppm = int(rng.choice(PPMS))
        scope = int(rng.integers(0, 2))
        mode = sgc.SAMPLED if rng.random() < 0.3 else sgc.EXACT
        path = (sgc.PATH_AUTO, sgc.PATH_GATHER, sgc.PATH_WINDOW)[(seed + step) % 3]
        if mom:
            announce(f"{what}: momentum beta={beta} ppm={ppm} scope={scope} mode={mode} path={path}")
            comp = sgc.compress_momentum(layout, dev(g), ud, rd, beta, mode=mode, scope=scope, keep_ppm=ppm,
                                         path=path)
            torch.cuda.synchronize()
            ref = orc.compress_momentum(g, u, r, beta, seg_off, scope, ppm, sampled=mode == sgc.SAMPLED,
                                        cap=comp.cap)
            check_sparse(comp, ref, what)
            assert_bitwise(host(rd), r, f"{what} residual")
            assert_bitwise(host(ud), u, f"{what} momentum")
            continue
        hold = bool(rng.random() < 0.5)
        bmode = [None, sgc.BIN_SBC, sgc.BIN_2BIT][int(rng.integers(0, 3))]
        if bmode is None:
            hold = False  # a held residual is completed by the binarize step
        announce(f"{what}: ppm={ppm} scope={scope} mode={mode} hold={hold} binarize={bmode} path={path}")
        comp = sgc.compress(layout, dev(g), rd, mode=mode, scope=scope, keep_ppm=ppm, hold=hold, path=path)
        torch.cuda.synchronize()
        if mode == sgc.EXACT:
            ref = orc.compress_exact(g, r, seg_off, scope, ppm, cap=comp.cap)
        else:
            ref = orc.compress_sampled(g, r, seg_off, scope, ppm, comp.cap)
        check_sparse(comp, ref, what)
        if hold:
            orc.hold_kept(ref, r)
        assert_bitwise(host(rd), r, f"{what} residual after compress")
        if bmode is None:
            continue
        bn = sgc.binarize(layout, comp, rd, bmode, held=hold)
        torch.cuda.synchronize()
        ob = orc.binarize_held(ref, layout.nseg, bmode, r) if hold else orc.binarize(ref, layout.nseg, bmode, r)
        gm, om = host(bn.means), ob.means
        assert np.all(np.abs(gm - om) <= REL * np.abs(om) + 1e-30), f"{what}: means"
        if np.array_equal(gm.view(np.uint32), om.view(np.uint32)):
            # equal means: every output and the residual are determined bit for bit
            assert_bitwise(host(bn.counts), ob.counts, f"{what} binarize counts")
            if bmode == sgc.BIN_SBC:
                assert_bitwise(host(bn.idx)[:int(ob.counts[-1])], ob.idx, f"{what} SBC idx")
            else:
                nw = (int(ref.counts[-1]) + 15) // 16
                assert_bitwise(host(bn.codes).view(np.uint32)[:nw], ob.codes[:nw], f"{what} 2-bit codes")
            assert_bitwise(host(rd), r, f"{what} residual after binarize")
        else:
            # a mean one rounding apart (different fixed summation order): the residuals part
            # ways at the sent entries, so the sequence ends here (the codec tests check such a
            # step's self-consistency)
            return
