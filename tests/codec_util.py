"""Shared steps of the codec parity tests: run a stage on both sides and
compare (compress, binarize), and build matching GPU / oracle messages."""
import numpy as np
import torch

import compressed_sgd_amd as sgc
from gpu_util import announce, assert_bitwise, dev, host

REL = 1e-6  # binarization means: the GPU sums in a different, fixed order


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
