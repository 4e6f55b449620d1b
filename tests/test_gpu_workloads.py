"""The whole hot path on each workload's shapes, in the launch configuration
the benchmark uses.

Where the CPU oracle finishes in seconds, every stage is compared with it bit
for bit (binarize means within 1e-6 relative, see codec_util).  At the full
sizes (97.8M and 2^30 elements) the exact top-k selection is checked through
the properties that define it -- k entries, every unsent key at most the
smallest sent key, ties sent lowest index first, sent values and residuals
equal to the accumulated gradient bit for bit -- evaluated with plain torch
ops on the same device; Rice streams are compared with the oracle's encoding
of the same indices, and the dense accumulation with a plain in-order
scatter of the messages' values.
"""
import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
import workloads as W
from codec_util import check_binarize, check_encode
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu


def oracle_sparse(orc, comp):
    """The GPU compress output as an oracle Sparse (host copies)."""
    counts = host(comp.counts)
    total = int(counts[-1])
    return orc.Sparse(host(comp.idx)[:total].copy(), host(comp.val)[:total].copy(), counts, 0)


def check_topk(acc, comp, r_after, k_expected, what, seg_off=None):
    """Exact top-k by magnitude (lower index first among equal keys), per
    segment if seg_off is given, from the defining properties."""
    announce(f"top-k properties {what}")
    counts = comp.counts.long()
    total = int(counts[-1])
    assert total == k_expected, f"{what}: kept {total}, want {k_expected}"
    idx = comp.idx[:total].long()
    val = comp.val[:total]
    if total > 1:
        assert bool((idx[1:] > idx[:-1]).all()), f"{what}: indices not ascending"
    keys = acc.view(torch.int32) & 0x7FFFFFFF
    assert torch.equal(val.view(torch.int32), acc[idx].view(torch.int32)), f"{what}: sent values"
    kept = torch.zeros(acc.numel(), dtype=torch.bool, device=acc.device)
    kept[idx] = True
    want_r = torch.where(kept, torch.zeros_like(acc), acc)
    assert torch.equal(r_after.view(torch.int32), want_r.view(torch.int32)), f"{what}: residual"
    bounds = [(0, acc.numel(), 0, total)] if seg_off is None else \
        [(int(seg_off[t]), int(seg_off[t + 1]), int(counts[:t].sum()), int(counts[:t + 1].sum()))
         for t in range(len(seg_off) - 1)]
    for lo, hi, e0, e1 in bounds:
        if e1 == e0:
            continue
        kseg = keys[lo:hi]
        mseg = kept[lo:hi]
        T = int(keys[idx[e0:e1]].min())
        if bool((~mseg).any()):
            assert int(kseg[~mseg].max()) <= T, f"{what}: an unsent key is larger than a sent one"
        tied_unsent = torch.nonzero((~mseg) & (kseg == T)).flatten()
        if tied_unsent.numel():
            tied_sent = torch.nonzero(mseg & (kseg == T)).flatten()
            assert int(tied_sent.max()) < int(tied_unsent.min()), f"{what}: ties not lowest index first"


def test_mlp_mnist_two_bit_four_workers(orc):
    # global top-1% + 2-bit quantization, 4 workers, all 10 steps of the
    # workload with carried residuals: raw 2-bit messages in even steps,
    # Rice-coded positions (b = 6) in odd ones
    w = W.MLP_MNIST
    layout = sgc.Layout(w.seg_numel)
    seg_off = np.array(layout.seg_off, np.int64)
    b = sgc.rice_param(w.keep_ppm / 1e6)
    res = [torch.zeros(w.numel, dtype=torch.float32, device="cuda") for _ in range(w.workers)]
    for step in range(w.steps):
        gm, om = [], []
        for wk in range(w.workers):
            g = W.gradient(w, wk, step, device="cuda")
            rd = res[wk]
            acc = rd + g
            comp = sgc.compress(layout, g, rd, keep_ppm=w.keep_ppm)
            torch.cuda.synchronize()
            check_topk(acc, comp, rd, layout.keep_total(sgc.GLOBAL, w.keep_ppm), f"mlp s{step} w{wk}")
            ref = oracle_sparse(orc, comp)
            r_host = host(rd).copy()
            bn, ob = check_binarize(orc, layout, comp, ref, rd, r_host, sgc.BIN_2BIT, f"mlp s{step} w{wk}")
            codes, means = host(bn.codes).view(np.uint32), host(bn.means)
            if step % 2 == 0:
                gm.append(sgc.Message(sgc.MSG_RAW_2BIT, bn.counts, bn.cap, idx=comp.idx, codes=bn.codes,
                                      means=bn.means))
                om.append(orc.Message(host(bn.counts), vkind=orc.VAL_2BIT, idx=ref.idx, codes=codes, means=means))
            else:
                enc, oenc = check_encode(orc, layout, ref.idx, host(bn.counts), 0, b, f"mlp s{step} w{wk}")
                gm.append(sgc.golomb_message(bn, enc))
                om.append(orc.Message(host(bn.counts), vkind=orc.VAL_2BIT, golomb=True, scope=0, b=b, codes=codes,
                                      means=means, enc=oenc))
        out = torch.empty(w.numel, dtype=torch.float32, device="cuda")
        announce(f"mlp decode_accumulate step {step}")
        st = sgc.decode_accumulate(layout, gm, out)
        ref_out = np.zeros(w.numel, np.float32)
        assert orc.decode_accumulate(om, seg_off, ref_out) == 0
        torch.cuda.synchronize()
        assert int(host(st)[0]) == 0
        assert_bitwise(host(out), ref_out, f"mlp step {step} sum of 4 workers")


def test_nmt_rnn_global_plus_local(orc):
    # global top-1% of 97.8M elements; node 0 adds the 4 workers' raw messages
    # (its own among them) to its fresh local gradient.  The streams are also
    # Rice coded (b = 6) and compared with the oracle: zero runs of ~10^6
    # elements make this the long-run encoder case.
    w = W.NMT_RNN
    layout = sgc.Layout(w.seg_numel)
    b = sgc.rice_param(w.keep_ppm / 1e6)
    k = layout.keep_total(sgc.GLOBAL, w.keep_ppm)
    msgs, sent = [], []
    local = None
    for wk in range(w.workers):
        g = W.gradient(w, wk, 0, device="cuda")
        if wk == 0:
            local = g.clone()
        rd = torch.zeros(w.numel, dtype=torch.float32, device="cuda")
        acc = rd + g
        comp = sgc.compress(layout, g, rd, keep_ppm=w.keep_ppm)
        torch.cuda.synchronize()
        check_topk(acc, comp, rd, k, f"nmt w{wk}")
        total = int(host(comp.counts)[-1])
        idx = host(comp.idx)[:total]
        check_encode(orc, layout, idx, host(comp.counts), 0, b, f"nmt w{wk}")
        msgs.append(sgc.raw_message(comp))
        sent.append((idx.astype(np.int64), host(comp.val)[:total].copy()))
        del g, acc, rd
    out = torch.empty(w.numel, dtype=torch.float32, device="cuda")
    announce("nmt decode_accumulate on the local gradient")
    st = sgc.decode_accumulate(layout, msgs, out, init=sgc.INIT_BASE, base=local)
    ref = host(local).copy()
    for idx, val in sent:  # one addition per element and message, in message order
        ref[idx] = ref[idx] + val
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    assert_bitwise(host(out), ref, "nmt local + 4 workers")


def test_resnet50_sbc_eight_workers(orc):
    # per-tensor top-0.1% + SBC + per-tensor Rice streams (b = 9), 8 workers,
    # 2 rounds of 7 delayed accumulations and one exchange each
    w = W.RESNET50
    layout = sgc.Layout(w.seg_numel)
    seg_off = np.array(layout.seg_off, np.int64)
    b = sgc.rice_param(w.keep_ppm / 1e6)
    k = layout.keep_total(sgc.PER_SEGMENT, w.keep_ppm)
    res = [torch.zeros(w.numel, dtype=torch.float32, device="cuda") for _ in range(w.workers)]
    for rnd in range(2):
        gm, om = [], []
        for wk in range(w.workers):
            rd = res[wk]
            for s_ in range(w.delay - 1):  # communication delay: accumulate only
                sgc.compress(layout, W.gradient(w, wk, rnd * w.delay + s_, device="cuda"), rd,
                             mode=sgc.ACCUMULATE_ONLY)
            g = W.gradient(w, wk, rnd * w.delay + w.delay - 1, device="cuda")
            acc = rd + g
            comp = sgc.compress(layout, g, rd, keep_ppm=w.keep_ppm, scope=sgc.PER_SEGMENT)
            torch.cuda.synchronize()
            check_topk(acc, comp, rd, k, f"resnet r{rnd} w{wk}", seg_off=seg_off)
            ref = oracle_sparse(orc, comp)
            r_host = host(rd).copy()
            bn, ob = check_binarize(orc, layout, comp, ref, rd, r_host, sgc.BIN_SBC, f"resnet r{rnd} w{wk}")
            cnt = host(bn.counts)
            sidx = host(bn.idx)[:int(cnt[-1])]
            enc, oenc = check_encode(orc, layout, sidx, cnt, 1, b, f"resnet r{rnd} w{wk}")
            gm.append(sgc.golomb_message(bn, enc))
            om.append(orc.Message(cnt, vkind=orc.VAL_SBC, golomb=True, scope=1, b=b, means=host(bn.means),
                                  enc=oenc))
        out = torch.empty(w.numel, dtype=torch.float32, device="cuda")
        announce(f"resnet decode_accumulate round {rnd}")
        st = sgc.decode_accumulate(layout, gm, out)
        ref_out = np.zeros(w.numel, np.float32)
        assert orc.decode_accumulate(om, seg_off, ref_out) == 0
        torch.cuda.synchronize()
        assert int(host(st)[0]) == 0
        assert_bitwise(host(out), ref_out, f"resnet round {rnd} sum of 8 workers")


def test_flat_1g_compress_encode_full_size(orc):
    # the benchmark's step: exact global top-1% of 2^30 + Rice (b = 6)
    w = W.FLAT_1G
    layout = sgc.Layout(w.seg_numel)
    ppm = 10000
    b = sgc.rice_param(ppm / 1e6)
    k = layout.keep_total(sgc.GLOBAL, ppm)
    rd = torch.zeros(w.numel, dtype=torch.float32, device="cuda")
    for step in range(2):
        g = W.gradient(w, 0, step, device="cuda")
        acc = rd + g
        comp = sgc.compress(layout, g, rd, keep_ppm=ppm)
        torch.cuda.synchronize()
        del g
        check_topk(acc, comp, rd, k, f"flat-1G step {step}")
        del acc
        enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=b)
        torch.cuda.synchronize()
        idx = host(comp.idx)[:k]
        ref = orc.encode(idx, host(comp.counts), np.array(layout.seg_off, np.int64), 0, b)
        nw = int(ref.word_off[-1])
        assert_bitwise(host(enc.words[:nw]).view(np.uint32), ref.words, f"flat-1G step {step} words")
        assert_bitwise(host(enc.nbits).view(np.uint64), ref.nbits, f"flat-1G step {step} nbits")
        assert_bitwise(host(enc.chunk_off[:ref.chunk_off.size]).view(np.uint64), ref.chunk_off,
                       f"flat-1G step {step} chunk table")


@pytest.mark.parametrize("ppm", [260000, 300000])
def test_high_density_split_chunk_scan(ppm):
    # 2^28 elements at 26% and 30% kept: more than 16,384 chunks of kept entries, so the
    # compaction's chunk-count scan is split over workgroups; exact top-k through its
    # defining properties (the oracle's full sort is too slow at this size)
    w = W.FLAT_1G
    n = 1 << 28
    layout = sgc.Layout([n])
    g = W.gradient(w, 0, 0, device="cuda", numel=n)
    rd = torch.zeros(n, dtype=torch.float32, device="cuda")
    acc = rd + g
    k = layout.keep_total(sgc.GLOBAL, ppm)
    assert (k + 4095) // 4096 > 16384
    comp = sgc.compress(layout, g, rd, keep_ppm=ppm)
    torch.cuda.synchronize()
    check_topk(acc, comp, rd, k, f"2^28 at {ppm / 1e4:g}%")


def test_flat_1g_sampled_full_size(orc):
    # sampled-threshold top-0.1%, then top-1% on the residual it leaves, over
    # all 2^30 elements: indices, values, counts, status and the whole
    # residual bit for bit against the oracle (its own sample of the same acc)
    w = W.FLAT_1G
    layout = sgc.Layout(w.seg_numel)
    seg_off = np.array(layout.seg_off, np.int64)
    rd = torch.zeros(w.numel, dtype=torch.float32, device="cuda")
    r = np.zeros(w.numel, np.float32)
    for step, ppm in enumerate((1000, 10000)):
        announce(f"flat-1G sampled step {step} ppm={ppm}")
        g = W.gradient(w, 0, step, device="cuda")
        comp = sgc.compress(layout, g, rd, mode=sgc.SAMPLED, keep_ppm=ppm)
        torch.cuda.synchronize()
        gh = host(g)
        del g
        ref = orc.compress_sampled(gh, r, seg_off, sgc.GLOBAL, ppm, comp.cap)
        del gh
        counts = host(comp.counts)
        total = int(counts[-1])
        assert_bitwise(counts, ref.counts, f"flat-1G sampled step {step} counts")
        assert_bitwise(host(comp.idx)[:total], ref.idx, f"flat-1G sampled step {step} idx")
        assert_bitwise(host(comp.val)[:total], ref.val, f"flat-1G sampled step {step} val")
        assert (int(host(comp.status)[0]) & sgc.STATUS_TRUNCATED) == (ref.status & 1)
        assert_bitwise(host(rd), r, f"flat-1G sampled step {step} residual")


def test_flat_1g_decode_accumulate_sixteen_workers(orc):
    # 16 workers' top-0.1% Rice messages (b = 9) summed into 2^30 elements;
    # each worker's exact selection is checked through its defining
    # properties, each stream against the oracle's encoding of its indices,
    # and the 16-worker sum against the oracle's decode-accumulate of the
    # oracle's own streams
    w = W.FLAT_1G
    layout = sgc.Layout(w.seg_numel)
    seg_off = np.array(layout.seg_off, np.int64)
    ppm = 1000
    b = sgc.rice_param(ppm / 1e6)
    k = layout.keep_total(sgc.GLOBAL, ppm)
    msgs, omsgs = [], []
    rd = torch.zeros(w.numel, dtype=torch.float32, device="cuda")
    for wk in range(w.workers):
        g = W.gradient(w, wk, 0, device="cuda")
        rd.zero_()
        acc = rd + g
        comp = sgc.compress(layout, g, rd, keep_ppm=ppm)
        enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, b=b)
        torch.cuda.synchronize()
        del g
        check_topk(acc, comp, rd, k, f"flat-1G worker {wk} top-0.1%")
        del acc
        msgs.append(sgc.golomb_message(comp, enc))
        total = int(host(comp.counts)[-1])
        counts = host(comp.counts)
        ref = orc.encode(host(comp.idx)[:total], counts, seg_off, 0, b)
        nw = int(ref.word_off[-1])
        assert_bitwise(host(enc.words[:nw]).view(np.uint32), ref.words, f"worker {wk} words")
        assert_bitwise(host(enc.chunk_off[:ref.chunk_off.size]).view(np.uint64), ref.chunk_off,
                       f"worker {wk} chunk table")
        omsgs.append(orc.Message(counts, golomb=True, scope=orc.GLOBAL, b=b, val=host(comp.val)[:total], enc=ref))
    del rd
    out = torch.empty(w.numel, dtype=torch.float32, device="cuda")
    announce("flat-1G decode_accumulate 16 x 0.1%")
    st = sgc.decode_accumulate(layout, msgs, out)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    want = np.zeros(w.numel, np.float32)
    assert orc.decode_accumulate(omsgs, seg_off, want) == 0
    assert_bitwise(host(out).view(np.uint32), want.view(np.uint32), "flat-1G 16-worker sum")


@pytest.mark.parametrize("scope", [sgc.GLOBAL, sgc.PER_SEGMENT])
def test_maximum_size(orc, scope):
    # n = 2^31 - 1, the largest layout the int32 indices allow: top-0.1% with
    # the last elements large, Rice coded, then accumulated onto zeros
    sizes = [1 << 30, (1 << 30) - 1]
    layout = sgc.Layout(sizes)
    n = layout.n
    assert n == (1 << 31) - 1
    ppm = 1000
    b = sgc.rice_param(ppm / 1e6)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77 + scope)
    g = torch.randn(n, dtype=torch.float32, device="cuda", generator=gen).mul_(1e-4)
    g[-5:] = torch.tensor([1.0, -2.0, 3.0, -4.0, 5.0], device="cuda")  # the very last indices are kept
    rd = torch.zeros(n, dtype=torch.float32, device="cuda")
    acc = rd + g
    comp = sgc.compress(layout, g, rd, keep_ppm=ppm, scope=scope)
    torch.cuda.synchronize()
    del g
    k = layout.keep_total(scope, ppm)
    check_topk(acc, comp, rd, k, f"2^31-1 scope {scope}",
               seg_off=None if scope == sgc.GLOBAL else np.array(layout.seg_off, np.int64))
    del acc
    total = int(host(comp.counts)[-1])
    idx = host(comp.idx)[:total]
    assert idx[-1] == n - 1
    enc, _ = check_encode(orc, layout, idx, host(comp.counts), scope, b, f"2^31-1 scope {scope}")
    msgs = [sgc.raw_message(comp), sgc.golomb_message(comp, enc)]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    announce(f"decode_accumulate 2^31-1 scope {scope}")
    st = sgc.decode_accumulate(layout, msgs, out)
    ref = torch.zeros(n, dtype=torch.float32, device="cuda")
    sel = comp.idx[:total].long()
    for _ in range(2):
        ref[sel] = ref[sel] + comp.val[:total]
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), "2^31-1 sum"
