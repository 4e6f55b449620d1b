"""GPU parity of sgc_binarize, sgc_encode and sgc_decode_accumulate.

Bitstreams, chunk tables, indices, 2-bit codes and dense accumulations must
match the oracle bit for bit.  Binarization means must match within 1e-6
relative (the GPU sums in a different, fixed order); the GPU residual must
then equal fp32(v - mean_gpu) exactly, and the sent index set must match
the oracle's except on a segment whose two means are a near-tie.
"""
import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
import workloads as W
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu

REL = 1e-6


def compress_both(orc, layout, g, r_host, scope, ppm):
    gd, rd = dev(g), dev(r_host)
    comp = sgc.compress(layout, gd, rd, scope=scope, keep_ppm=ppm)
    ref = orc.compress_exact(g, r_host, np.array(layout.seg_off, np.int64), scope, ppm, cap=comp.cap)
    torch.cuda.synchronize()
    assert_bitwise(host(comp.counts), ref.counts, "compress counts")
    return comp, ref, rd


def check_binarize(orc, layout, comp, ref, rd, r_host, mode, what):
    announce(f"binarize {what} mode={mode}")
    nseg = layout.nseg
    bn = sgc.binarize(layout, comp, rd, mode)
    torch.cuda.synchronize()
    ob = orc.binarize(ref, nseg, mode, r_host)
    gm, om = host(bn.means), ob.means
    assert np.all(np.abs(gm - om) <= REL * np.abs(om) + 1e-30), f"{what}: means differ beyond 1e-6"
    res_gpu = host(rd)
    total_in = int(ref.counts[-1])
    idx_in, val_in = ref.idx, ref.val
    e0 = 0
    exact_segments = 0
    gcounts = host(bn.counts)
    if mode == sgc.BIN_SBC:
        g_idx = host(bn.idx)
        ge0 = oe0 = 0
        for t in range(nseg):
            c = int(ref.counts[t])
            ids, vs = idx_in[e0:e0 + c], val_in[e0:e0 + c]
            e0 += c
            gc, oc = int(gcounts[t]), int(ob.counts[t])
            mean = np.float32(gm[t])
            sent = (vs > 0) if mean > 0 else (vs < 0) if mean < 0 else np.zeros(c, bool)
            # GPU self-consistency: sent side and residuals follow its own mean
            assert g_idx[ge0:ge0 + gc].tolist() == ids[sent].tolist(), f"{what} seg {t}: sent set"
            want_r = np.where(sent, (vs - mean).astype(np.float32), vs)
            assert_bitwise(res_gpu[ids], want_r.astype(np.float32), f"{what} seg {t} residual")
            if gm[t].view(np.uint32) == om[t].view(np.uint32):
                exact_segments += 1
                assert gc == oc
            else:  # the side may differ only on a near-tie of the two means
                mp, mn = np.float32(abs(gm[t])), np.float32(abs(om[t]))
                if gc != oc:
                    assert abs(mp - mn) <= 2e-6 * max(mp, mn)
            ge0 += gc
            oe0 += oc
        assert int(gcounts[-1]) == ge0
    else:
        codes = host(bn.codes).view(np.uint32)
        assert_bitwise(codes[:(total_in + 15) // 16], ob.codes, f"{what} 2-bit codes")
        assert_bitwise(gcounts, ob.counts, f"{what} 2-bit counts")
        for t in range(nseg):
            c = int(ref.counts[t])
            ids, vs = idx_in[e0:e0 + c], val_in[e0:e0 + c]
            e0 += c
            q = np.where(vs > 0, np.float32(gm[2 * t]), np.where(vs < 0, np.float32(gm[2 * t + 1]), np.float32(0)))
            assert_bitwise(res_gpu[ids], (vs - q).astype(np.float32), f"{what} seg {t} 2-bit residual")
            exact_segments += int(np.array_equal(gm[2 * t:2 * t + 2].view(np.uint32), om[2 * t:2 * t + 2].view(np.uint32)))
    # untouched residual entries equal the oracle's
    mask = np.ones(layout.n, bool)
    mask[idx_in] = False
    assert_bitwise(res_gpu[mask], r_host[mask], f"{what} residual outside kept set")
    return bn, ob


@pytest.mark.parametrize("mode", [0, 1])
def test_binarize_ragged(orc, mode):
    rng = np.random.default_rng(21)
    sizes = [64, 0, 1000, 4097, 9408, 1, 70000, 2048]
    layout = sgc.Layout(sizes)
    g = rng.laplace(0, 1e-3, layout.n).astype(np.float32)
    g[1064:1100] = -0.0
    for scope in (0, 1):
        r = np.zeros(layout.n, np.float32)
        comp, ref, rd = compress_both(orc, layout, g, r, scope, 20000)
        check_binarize(orc, layout, comp, ref, rd, r, mode, f"ragged scope{scope}")


def test_binarize_resnet50_sbc(orc):
    w = W.RESNET50
    layout = sgc.Layout(w.seg_numel)
    g = W.gradient(w, 0, 0).numpy()
    r = np.zeros(w.numel, np.float32)
    comp, ref, rd = compress_both(orc, layout, g, r, w.scope, w.keep_ppm)
    check_binarize(orc, layout, comp, ref, rd, r, sgc.BIN_SBC, "resnet50")


def test_binarize_mlp_2bit(orc):
    w = W.MLP_MNIST
    layout = sgc.Layout(w.seg_numel)
    g = W.gradient(w, 0, 0).numpy()
    r = np.zeros(w.numel, np.float32)
    comp, ref, rd = compress_both(orc, layout, g, r, w.scope, w.keep_ppm)
    check_binarize(orc, layout, comp, ref, rd, r, sgc.BIN_2BIT, "mlp")


def test_binarize_equal_means_positive(orc):
    layout = sgc.Layout([8])
    g = np.array([0.5, -0.25, -0.75, 0.5, 0, 0, 0, 0], np.float32)
    r = np.zeros(8, np.float32)
    comp, ref, rd = compress_both(orc, layout, g, r, 0, 500000)
    bn, ob = check_binarize(orc, layout, comp, ref, rd, r, sgc.BIN_SBC, "tie")
    assert host(bn.means).tolist() == [0.5]


# ------------------------------------------------------------------ encode
def check_encode(orc, layout, idx_np, counts_np, scope, b, what):
    announce(f"encode {what} scope={scope} b={b} k={int(counts_np[-1])}")
    cap = max(int(counts_np[-1]), 1)
    idx_d = dev(np.concatenate([idx_np, np.zeros(cap - idx_np.size, np.int32)]).astype(np.int32))
    enc = sgc.encode(layout, idx_d, dev(counts_np.astype(np.int64)), cap, scope=scope, b=b)
    torch.cuda.synchronize()
    ref = orc.encode(idx_np, counts_np, np.array(layout.seg_off, np.int64), scope, b)
    wo = host(enc.word_off).view(np.uint64)
    assert_bitwise(wo, ref.word_off, f"{what} word_off")
    assert_bitwise(host(enc.nbits).view(np.uint64), ref.nbits, f"{what} nbits")
    nw = int(wo[-1])
    assert_bitwise(host(enc.words).view(np.uint32)[:nw], ref.words, f"{what} words")
    nc = ref.chunk_off.size
    assert_bitwise(host(enc.chunk_off).view(np.uint64)[:nc], ref.chunk_off, f"{what} chunk table")
    assert int(host(enc.status)[0]) == 0
    return enc, ref


def _random_sets(rng, sizes, density):
    idx, counts = [], []
    off = 0
    for m in sizes:
        sel = np.flatnonzero(rng.random(m) < density) + off
        idx.append(sel)
        counts.append(sel.size)
        off += m
    idx = np.concatenate(idx).astype(np.int32) if idx else np.zeros(0, np.int32)
    counts = np.array(counts + [sum(counts)], np.int64)
    return idx, counts


@pytest.mark.parametrize("b", [0, 1, 3, 6, 9, 13])
@pytest.mark.parametrize("scope", [0, 1])
def test_encode_ragged(orc, b, scope):
    rng = np.random.default_rng(31 + b)
    sizes = [0, 5, 100000, 1, 0, 33333, 4096, 250000]
    layout = sgc.Layout(sizes)
    for density in (0.001, 0.01, 0.3):
        idx, counts = _random_sets(rng, sizes, density)
        check_encode(orc, layout, idx, counts, scope, b, f"ragged d={density}")


def test_encode_long_runs(orc):
    # embedding-like clusters: gaps of up to millions of elements (long unary runs)
    rng = np.random.default_rng(41)
    n = 8_000_000
    layout = sgc.Layout([n])
    rows = np.sort(rng.choice(n // 512, 300, replace=False))
    idx = np.concatenate([r * 512 + np.flatnonzero(rng.random(512) < 0.3) for r in rows]).astype(np.int32)
    counts = np.array([idx.size, idx.size], np.int64)
    for b in (0, 2, 6):
        check_encode(orc, layout, idx, counts, 0, b, "long runs")
    one = np.array([n - 1], np.int32)
    check_encode(orc, layout, one, np.array([1, 1], np.int64), 0, 0, "single far entry")


def test_encode_empty_and_dense(orc):
    layout = sgc.Layout([1000, 3000])
    check_encode(orc, layout, np.zeros(0, np.int32), np.array([0, 0, 0], np.int64), 1, 4, "empty")
    idx = np.arange(4000, dtype=np.int32)
    check_encode(orc, layout, idx, np.array([1000, 3000, 4000], np.int64), 1, 0, "dense b=0")


# ------------------------------------------------------ decode + accumulate
def make_messages(orc, layout, rng, kinds, ppm=20000):
    """Build W messages of the given kinds on both sides; returns (gpu msgs, oracle msgs)."""
    seg_off = np.array(layout.seg_off, np.int64)
    n, nseg = layout.n, layout.nseg
    gm, om = [], []
    for kind in kinds:
        g = rng.laplace(0, 1e-3, n).astype(np.float32)
        r = np.zeros(n, np.float32)
        scope = 1 if kind in ("golomb_sbc", "golomb_f32_seg") else 0
        comp, ref, rd = compress_both(orc, layout, g, r, scope, ppm)
        if kind == "raw_f32":
            gm.append(sgc.raw_message(comp))
            om.append(orc.Message(ref.counts, idx=ref.idx, val=ref.val))
        elif kind in ("golomb_f32", "golomb_f32_seg"):
            b = 4
            enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, scope=scope, b=b)
            oenc = orc.encode(ref.idx, ref.counts, seg_off, scope, b)
            gm.append(sgc.golomb_message(comp, enc))
            om.append(orc.Message(ref.counts, golomb=True, scope=scope, b=b, val=ref.val, enc=oenc))
        elif kind == "golomb_sbc":
            bn = sgc.binarize(layout, comp, rd, sgc.BIN_SBC)
            b = 5
            enc = sgc.encode(layout, bn.idx, bn.counts, bn.cap, scope=1, b=b)
            torch.cuda.synchronize()
            # the oracle side decodes the GPU's message bytes independently
            cnt = host(bn.counts)
            sidx = host(bn.idx)[:int(cnt[-1])]
            oenc = orc.encode(sidx, cnt, seg_off, 1, b)
            gm.append(sgc.golomb_message(bn, enc))
            om.append(orc.Message(cnt, vkind=orc.VAL_SBC, golomb=True, scope=1, b=b, means=host(bn.means),
                                  enc=oenc))
        elif kind in ("raw_2bit", "golomb_2bit"):
            bn = sgc.binarize(layout, comp, rd, sgc.BIN_2BIT)
            torch.cuda.synchronize()
            cnt = host(bn.counts)
            codes = host(bn.codes).view(np.uint32)
            means = host(bn.means)
            if kind == "raw_2bit":
                gm.append(sgc.Message(sgc.MSG_RAW_2BIT, bn.counts, bn.cap, idx=comp.idx, codes=bn.codes,
                                      means=bn.means))
                om.append(orc.Message(cnt, vkind=orc.VAL_2BIT, idx=ref.idx, codes=codes, means=means))
            else:
                b = 3
                enc = sgc.encode(layout, comp.idx, bn.counts, bn.cap, scope=0, b=b)
                oenc = orc.encode(ref.idx, cnt, seg_off, 0, b)
                gm.append(sgc.golomb_message(bn, enc))
                om.append(orc.Message(cnt, vkind=orc.VAL_2BIT, golomb=True, scope=0, b=b, codes=codes,
                                      means=means, enc=oenc))
    return gm, om


@pytest.mark.parametrize("init", [0, 1, 2])
def test_decode_accumulate_all_formats(orc, init):
    rng = np.random.default_rng(51 + init)
    layout = sgc.Layout([70000, 3, 0, 12345, 4096, 100001])
    n = layout.n
    kinds = ["raw_f32", "golomb_f32", "golomb_sbc", "raw_2bit", "golomb_2bit", "golomb_f32_seg",
             "raw_f32", "golomb_sbc", "golomb_f32", "raw_2bit"]
    gm, om = make_messages(orc, layout, rng, kinds)
    start = rng.normal(0, 1e-3, n).astype(np.float32)
    start[::101] = -0.0
    base = rng.normal(0, 1e-3, n).astype(np.float32)
    out = dev(start)
    announce(f"decode_accumulate W={len(gm)} init={init}")
    st = sgc.decode_accumulate(layout, gm, out, init=init, base=dev(base))
    torch.cuda.synchronize()
    ref = np.zeros(n, np.float32) if init == 0 else base.copy() if init == 1 else start.copy()
    ost = orc.decode_accumulate(om, np.array(layout.seg_off, np.int64), ref)
    assert ost == 0 and int(host(st)[0]) == 0
    assert_bitwise(host(out), ref, f"decode_accumulate init={init}")


def test_decode_accumulate_many_workers(orc):
    # more messages than one decode batch and one merge batch hold
    rng = np.random.default_rng(61)
    layout = sgc.Layout([50000])
    kinds = ["golomb_f32", "raw_f32"] * 18
    gm, om = make_messages(orc, layout, rng, kinds, ppm=50000)
    out = torch.zeros(layout.n, dtype=torch.float32, device="cuda")
    sgc.decode_accumulate(layout, gm, out)
    ref = np.zeros(layout.n, np.float32)
    orc.decode_accumulate(om, np.array(layout.seg_off, np.int64), ref)
    torch.cuda.synchronize()
    assert_bitwise(host(out), ref, "36 workers")


def test_corrupt_message_is_skipped(orc):
    rng = np.random.default_rng(71)
    layout = sgc.Layout([60000])
    gm, om = make_messages(orc, layout, rng, ["golomb_f32", "golomb_f32", "raw_f32"])
    # truncate the second message's stream by two bits
    bad = gm[1]
    nb = bad.enc.nbits.clone()
    nb[0] -= 2
    bad.enc = sgc.Encoded(bad.enc.words, bad.enc.word_off, nb, bad.enc.chunk_off, bad.enc.status, bad.enc.scope,
                          bad.enc.b, bad.enc.cap)
    out = torch.zeros(layout.n, dtype=torch.float32, device="cuda")
    st = sgc.decode_accumulate(layout, gm, out)
    ref = np.zeros(layout.n, np.float32)
    ost = orc.decode_accumulate([om[0], om[2]], np.array(layout.seg_off, np.int64), ref)
    torch.cuda.synchronize()
    assert int(host(st)[0]) & sgc.STATUS_CORRUPT
    assert_bitwise(host(out), ref, "corrupt message skipped")
    # a non-ascending raw message is skipped too
    raw = gm[2]
    idx = raw.idx.clone()
    if int(raw.counts[-1]) > 2:
        idx[1], idx[2] = idx[2].item(), idx[1].item()
    gm2 = [gm[0], sgc.Message(sgc.MSG_RAW_F32, raw.counts, raw.cap, idx=idx, val=raw.val)]
    out2 = torch.zeros(layout.n, dtype=torch.float32, device="cuda")
    st2 = sgc.decode_accumulate(layout, gm2, out2)
    ref2 = np.zeros(layout.n, np.float32)
    orc.decode_accumulate([om[0]], np.array(layout.seg_off, np.int64), ref2)
    torch.cuda.synchronize()
    assert int(host(st2)[0]) & sgc.STATUS_CORRUPT
    assert_bitwise(host(out2), ref2, "non-ascending raw skipped")


def test_zero_messages_initialises(orc):
    layout = sgc.Layout([10000, 7])
    base = np.random.default_rng(2).normal(0, 1, layout.n).astype(np.float32)
    out = torch.full((layout.n,), 3.0, device="cuda")
    sgc.decode_accumulate(layout, [], out, init=sgc.INIT_BASE, base=dev(base))
    torch.cuda.synchronize()
    assert_bitwise(host(out), base, "W=0 base")
    sgc.decode_accumulate(layout, [], out, init=sgc.INIT_ZERO)
    torch.cuda.synchronize()
    assert_bitwise(host(out), np.zeros(layout.n, np.float32), "W=0 zero")
