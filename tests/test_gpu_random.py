"""Randomised whole-path parity: compress -> (binarize) -> (Rice) -> decode-
accumulate, every stage bitwise against the CPU oracle.

Each case draws its own layout (ragged segments, empty ones included), and
per worker message: the kept fraction, the selection mode and scope, the
message format and the Rice parameter b (0..14, so the decoder's LDS column
sizes all occur, mixed inside one batch, and chunks longer than a column
take the global-memory path).  Values are coarsely quantised in some cases
so that ties at the threshold are common.  Binarize means are checked to
1e-6 relative (a different, fixed summation order); the oracle then decodes
the GPU's own message bytes and sums the messages in order, which must match
the GPU's dense result bit for bit.
"""
import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
from codec_util import check_binarize
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu

KINDS = ["raw_f32", "golomb_f32", "golomb_sbc", "raw_2bit", "golomb_2bit"]
PPMS = [0, 137, 1000, 5000, 20000, 100000, 400000, 1000000]


def random_layout(rng):
    nseg = int(rng.integers(1, 12))
    sizes = [int(x) for x in rng.integers(0, 150000, nseg)]
    for t in range(nseg):
        u = rng.random()
        if u < 0.15:
            sizes[t] = 0
        elif u < 0.25:
            sizes[t] = int(rng.integers(1, 40))
    if sum(sizes) == 0:
        sizes[0] = 5000
    return sgc.Layout(sizes)


def random_values(rng, n):
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    if rng.random() < 0.3:  # coarse quantisation: many equal magnitudes
        g = (np.round(g * 4e3) / 4e3).astype(np.float32)
    if rng.random() < 0.2:  # a sparse gradient (embedding-like zero rows)
        g[rng.random(n) < 0.7] = 0.0
    return g


def one_message(orc, layout, rng, what, **fixed):
    """One worker step on both sides; returns the GPU and oracle messages.
    fixed: any of ppm, scope, mode, kind, b, enc_scope, instead of a random draw, and the
    compress pipeline (path, default: chosen by the library)."""
    n = layout.n
    seg_off = np.array(layout.seg_off, np.int64)
    ppm = int(rng.choice(PPMS))
    scope = int(rng.integers(0, 2))
    mode = sgc.SAMPLED if rng.random() < 0.3 else sgc.EXACT
    kind = KINDS[int(rng.integers(0, len(KINDS)))]
    b = int(rng.integers(0, 15))
    enc_scope = int(rng.integers(0, 2))
    ppm = fixed.get("ppm", ppm)
    scope = fixed.get("scope", scope)
    mode = fixed.get("mode", mode)
    kind = fixed.get("kind", kind)
    b = fixed.get("b", b)
    enc_scope = fixed.get("enc_scope", enc_scope)
    g = random_values(rng, n)
    r = (rng.normal(0, 3e-4, n) * (rng.random(n) < 0.5)).astype(np.float32)
    path = fixed.get("path", sgc.PATH_AUTO)
    announce(f"{what}: n={n} nseg={layout.nseg} ppm={ppm} scope={scope} mode={mode} kind={kind} b={b} "
             f"enc_scope={enc_scope} path={path}")
    rd = dev(r)
    comp = sgc.compress(layout, dev(g), rd, mode=mode, scope=scope, keep_ppm=ppm, path=path)
    torch.cuda.synchronize()
    if mode == sgc.EXACT:
        ref = orc.compress_exact(g, r, seg_off, scope, ppm, cap=comp.cap)
    else:
        ref = orc.compress_sampled(g, r, seg_off, scope, ppm, comp.cap)
    counts = host(comp.counts)
    total = int(counts[-1])
    assert_bitwise(counts, ref.counts, f"{what} counts")
    assert_bitwise(host(comp.idx)[:total], ref.idx, f"{what} idx")
    assert_bitwise(host(comp.val)[:total], ref.val, f"{what} val")
    assert_bitwise(host(rd), r, f"{what} residual")

    if kind == "raw_f32":
        return sgc.raw_message(comp), orc.Message(ref.counts, idx=ref.idx, val=ref.val)
    if kind == "golomb_f32":
        enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, scope=enc_scope, b=b)
        oenc = orc.encode(ref.idx, ref.counts, seg_off, enc_scope, b)
        torch.cuda.synchronize()
        nw = int(oenc.word_off[-1])
        assert_bitwise(host(enc.words).view(np.uint32)[:nw], oenc.words, f"{what} words")
        return (sgc.golomb_message(comp, enc),
                orc.Message(ref.counts, golomb=True, scope=enc_scope, b=b, val=ref.val, enc=oenc))
    bmode = sgc.BIN_SBC if kind == "golomb_sbc" else sgc.BIN_2BIT
    bn, _ = check_binarize(orc, layout, comp, ref, rd, r, bmode, what)
    bcnt = host(bn.counts)
    means = host(bn.means)
    if kind == "golomb_sbc":
        sidx = host(bn.idx)[:int(bcnt[-1])]
        enc = sgc.encode(layout, bn.idx, bn.counts, bn.cap, scope=enc_scope, b=b)
        oenc = orc.encode(sidx, bcnt, seg_off, enc_scope, b)
        torch.cuda.synchronize()
        nw = int(oenc.word_off[-1])
        assert_bitwise(host(enc.words).view(np.uint32)[:nw], oenc.words, f"{what} SBC words")
        return (sgc.golomb_message(bn, enc),
                orc.Message(bcnt, vkind=orc.VAL_SBC, golomb=True, scope=enc_scope, b=b, means=means, enc=oenc))
    codes = host(bn.codes).view(np.uint32)
    if kind == "raw_2bit":
        return (sgc.Message(sgc.MSG_RAW_2BIT, bn.counts, bn.cap, idx=comp.idx, codes=bn.codes, means=bn.means),
                orc.Message(bcnt, vkind=orc.VAL_2BIT, idx=ref.idx, codes=codes, means=means))
    enc = sgc.encode(layout, comp.idx, bn.counts, bn.cap, scope=enc_scope, b=b)
    oenc = orc.encode(ref.idx, bcnt, seg_off, enc_scope, b)
    return (sgc.golomb_message(bn, enc),
            orc.Message(bcnt, vkind=orc.VAL_2BIT, golomb=True, scope=enc_scope, b=b, codes=codes, means=means,
                        enc=oenc))


@pytest.mark.parametrize("seed", range(60))
def test_random_pipeline(orc, seed):
    rng = np.random.default_rng(7000 + seed)
    layout = random_layout(rng)
    n = layout.n
    W = int(rng.integers(1, 13))
    gm, om = [], []
    for wk in range(W):
        path = (sgc.PATH_AUTO, sgc.PATH_GATHER, sgc.PATH_WINDOW)[(seed + wk) % 3]
        a, o = one_message(orc, layout, rng, f"seed {seed} worker {wk}", path=path)
        gm.append(a)
        om.append(o)
    init = int(rng.integers(0, 3))
    start = rng.normal(0, 1e-3, n).astype(np.float32)
    base = rng.normal(0, 1e-3, n).astype(np.float32)
    out = dev(start)
    announce(f"seed {seed}: decode_accumulate W={W} init={init}")
    st = sgc.decode_accumulate(layout, gm, out, init=init, base=dev(base))
    torch.cuda.synchronize()
    ref = np.zeros(n, np.float32) if init == 0 else base.copy() if init == 1 else start.copy()
    ost = orc.decode_accumulate(om, np.array(layout.seg_off, np.int64), ref)
    assert ost == 0 and int(host(st)[0]) == 0, f"seed {seed}: status {ost} / {int(host(st)[0])}"
    assert_bitwise(host(out), ref, f"seed {seed}: dense sum")


@pytest.mark.parametrize("nseg", [300, 1500, 2100])
def test_many_segments(orc, nseg):
    # more segments than one round of the per-segment bookkeeping (256 or
    # 1024 threads, one segment each): prefixes carried across rounds in the
    # compress set-up and tile scan, binarize set-up, encode set-up and
    # stream offsets, and the message set-up; every stage against the oracle
    rng = np.random.default_rng(9100 + nseg)
    sizes = [int(x) for x in rng.integers(0, 3000, nseg)]
    for t in range(0, nseg, 7):
        sizes[t] = 0
    layout = sgc.Layout(sizes)
    n = layout.n
    combos = [
        dict(scope=1, mode=sgc.EXACT, kind="golomb_sbc", enc_scope=1, ppm=20000),
        dict(scope=1, mode=sgc.SAMPLED, kind="golomb_f32", enc_scope=1, ppm=5000),
        dict(scope=0, mode=sgc.EXACT, kind="golomb_2bit", enc_scope=1, ppm=100000),
        dict(scope=1, mode=sgc.EXACT, kind="raw_2bit", ppm=1000),
        dict(scope=0, mode=sgc.SAMPLED, kind="raw_f32", ppm=20000),
        dict(scope=1, mode=sgc.EXACT, kind="golomb_f32", enc_scope=0, ppm=400000),
        dict(scope=1, mode=sgc.EXACT, kind="golomb_sbc", enc_scope=0, ppm=50000),
    ]
    gm, om = [], []
    for wk, fixed in enumerate(combos):
        path = (sgc.PATH_GATHER, sgc.PATH_WINDOW)[(nseg + wk) % 2]
        a, o = one_message(orc, layout, rng, f"nseg {nseg} worker {wk}", path=path, **fixed)
        gm.append(a)
        om.append(o)
    out = torch.zeros(n, dtype=torch.float32, device="cuda")
    announce(f"nseg {nseg}: decode_accumulate W={len(gm)}")
    st = sgc.decode_accumulate(layout, gm, out)
    torch.cuda.synchronize()
    ref = np.zeros(n, np.float32)
    ost = orc.decode_accumulate(om, np.array(layout.seg_off, np.int64), ref)
    assert ost == 0 and int(host(st)[0]) == 0
    assert_bitwise(host(out), ref, f"nseg {nseg}: dense sum")
