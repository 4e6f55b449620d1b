"""GPU parity of sgc_binarize, sgc_encode and sgc_decode_accumulate.

Bitstreams, chunk tables, indices, 2-bit codes and dense accumulations must
match the oracle bit for bit.  Binarization means must match within 1e-6
relative (the GPU sums in a different, fixed order); the GPU residual must
then equal fp32(v - mean_gpu) exactly, and the sent index set must match
the oracle's except on a segment whose two means are a near-tie.
"""
import dataclasses

import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
import workloads as W
from codec_util import check_binarize, check_encode, compress_both, make_messages
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu


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


@pytest.mark.parametrize("scope", [0, 1])
def test_encode_split_offset_scan(orc, scope):
    # About 36M codes: more than 16,384 encode blocks of 2048, so the block-offset scan is
    # split over workgroups (part totals, then a prefix per part); two streams per message
    # in per-segment scope.  Words, offsets, bit counts and the chunk table bitwise.
    rng = np.random.default_rng(77 + scope)
    n = 1 << 28
    layout = sgc.Layout([n // 2, n // 2])
    idx = np.flatnonzero(rng.random(n, dtype=np.float32) < 0.134).astype(np.int32)
    half = int(np.searchsorted(idx, n // 2))
    counts = np.array([half, idx.size - half, idx.size], np.int64)
    assert idx.size > 16384 * 2048
    check_encode(orc, layout, idx, counts, scope, 3, f"split scan scope{scope}")


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


@pytest.mark.parametrize("init", [sgc.INIT_BASE, sgc.INIT_INPLACE])
def test_decode_accumulate_many_kinds_batches(orc, init):
    # 35 messages of all six kinds on a ragged layout: three merge batches
    # (the later ones add in place) onto a base or onto out itself; message
    # 19 (second merge batch, third decode batch) is two bits short and must
    # be the only one left out
    rng = np.random.default_rng(67 + init)
    layout = sgc.Layout([40000, 0, 13, 70000, 4096])
    n = layout.n
    kinds = ["raw_f32", "golomb_f32", "golomb_f32_seg", "golomb_sbc", "raw_2bit", "golomb_2bit"] * 6
    kinds = kinds[:35]
    gm, om = make_messages(orc, layout, rng, kinds, ppm=30000)
    assert kinds[19] == "golomb_f32"
    e = gm[19].enc
    nb = e.nbits.clone()
    nb[0] -= 2
    gm[19] = dataclasses.replace(gm[19], enc=sgc.Encoded(e.words, e.word_off, nb, e.chunk_off, e.status, e.scope,
                                                         e.b, e.cap))
    start = rng.normal(0, 1e-3, n).astype(np.float32)
    base = rng.normal(0, 1e-3, n).astype(np.float32)
    out = dev(start)
    announce(f"35 messages, six kinds, init={init}, message 19 corrupt")
    st = sgc.decode_accumulate(layout, gm, out, init=init, base=dev(base))
    ref = (base if init == sgc.INIT_BASE else start).copy()
    ost = orc.decode_accumulate(om[:19] + om[20:], np.array(layout.seg_off, np.int64), ref)
    torch.cuda.synchronize()
    assert ost == 0
    assert int(host(st)[0]) & sgc.STATUS_CORRUPT
    assert_bitwise(host(out), ref, f"35 messages init={init}")


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


def test_positions_past_stream_size_in_whole_group_are_corrupt(orc):
    # A Rice stream written for a 50,100-element tensor, decoded as a
    # 50,000-element one: 600 codes, only the last four (codes 596..599, the
    # last whole group of four in the last 256-code chunk) lie past the
    # stream's size.  No later chunk-table entry and no partial group follows
    # them, and the bit count is consistent, so only the decoder's check on a
    # whole group's positions can reject the message.  It must be skipped,
    # with the corrupt status, and the other message summed exactly.
    rng = np.random.default_rng(79)
    n = 50000
    layout = sgc.Layout([n])
    gm, om = make_messages(orc, layout, rng, ["golomb_f32"])
    head = np.sort(rng.choice(n - 100, size=596, replace=False)).astype(np.int32)
    tail = np.array([n + 3, n + 17, n + 40, n + 71], np.int32)
    idx = np.concatenate([head, tail])
    total = idx.size
    counts = np.array([total, total], np.int64)
    b = 6
    oenc = orc.encode(idx, counts, np.array([0, n + 100], np.int64), orc.GLOBAL, b)
    nw = int(oenc.word_off[-1])
    bound = int(sgc.lib().sgc_encode_word_bound(layout.handle, sgc.GLOBAL, b, total))
    assert nw <= bound  # the set-up's word check passes
    enc = sgc.Encoded(dev(oenc.words.view(np.int32)), dev(oenc.word_off.view(np.int64)),
                      dev(oenc.nbits.view(np.int64)), dev(oenc.chunk_off.view(np.int64)),
                      torch.zeros(1, dtype=torch.int32, device="cuda"), sgc.GLOBAL, b, total)
    val = dev(rng.normal(0, 1e-3, total).astype(np.float32))
    bad = sgc.Message(sgc.MSG_GOLOMB_F32, dev(counts), total, scope=sgc.GLOBAL, b=b, val=val, enc=enc)
    out = torch.zeros(n, dtype=torch.float32, device="cuda")
    announce("positions past the stream size in the last whole group")
    st = sgc.decode_accumulate(layout, [gm[0], bad], out)
    ref = np.zeros(n, np.float32)
    assert orc.decode_accumulate([om[0]], np.array(layout.seg_off, np.int64), ref) == 0
    torch.cuda.synchronize()
    assert int(host(st)[0]) & sgc.STATUS_CORRUPT
    assert_bitwise(host(out), ref, "message with positions past its stream skipped")


def test_corrupt_per_segment_stream_is_skipped(orc):
    # per-tensor Rice streams over 1500 tensors, one message corrupted at a
    # tensor past the first 1024 (the set-up's later rounds); each corruption
    # keeps every read inside the message's buffers (same chunk counts and
    # total), so only the checks decide: a shifted stream offset (set-up), a
    # stream two bits short, and one code moved from an earlier tensor's count
    # to this one's (decoder: one stream ends early, the other has bits left).  The message is skipped and the others summed exactly.
    rng = np.random.default_rng(73)
    sizes = [int(x) for x in rng.integers(0, 2500, 1500)]
    for t in range(0, len(sizes), 5):
        sizes[t] = 0
    layout = sgc.Layout(sizes)
    gm, om = make_messages(orc, layout, rng, ["golomb_f32_seg", "golomb_f32_seg", "golomb_sbc"])
    ref = np.zeros(layout.n, np.float32)
    orc.decode_accumulate([om[0], om[2]], np.array(layout.seg_off, np.int64), ref)
    good = gm[1]
    cnt = host(good.counts).astype(np.int64)
    s = max(t for t in range(1025, layout.nseg) if cnt[t] >= 2 and cnt[t] % sgc.CHUNK_CODES != 0)
    s2 = min(t for t in range(layout.nseg) if cnt[t] >= 2 and cnt[t] % sgc.CHUNK_CODES != 1)
    e = good.enc

    def variant(what, words=None, word_off=None, nbits=None, counts=None):
        enc = sgc.Encoded(e.words if words is None else words, e.word_off if word_off is None else word_off,
                          e.nbits if nbits is None else nbits, e.chunk_off, e.status, e.scope, e.b, e.cap)
        bad = dataclasses.replace(good, counts=good.counts if counts is None else counts, enc=enc)
        out = torch.zeros(layout.n, dtype=torch.float32, device="cuda")
        announce(f"corrupt per-tensor stream: {what} at tensor {s}")
        st = sgc.decode_accumulate(layout, [gm[0], bad, gm[2]], out)
        torch.cuda.synchronize()
        assert int(host(st)[0]) & sgc.STATUS_CORRUPT, what
        assert_bitwise(host(out), ref, f"{what}: corrupt message skipped")

    wo = e.word_off.clone()
    wo[s] += 1
    variant("stream offset shifted", word_off=wo)
    nb = e.nbits.clone()
    nb[s] -= 2
    variant("stream two bits short", nbits=nb)
    c2 = good.counts.clone()
    c2[s] += 1
    c2[s2] -= 1
    variant(f"one code moved from tensor {s2}", counts=c2)
    # and the untouched message decodes
    out = torch.zeros(layout.n, dtype=torch.float32, device="cuda")
    st = sgc.decode_accumulate(layout, gm, out)
    full = np.zeros(layout.n, np.float32)
    orc.decode_accumulate(om, np.array(layout.seg_off, np.int64), full)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 0
    assert_bitwise(host(out), full, "uncorrupted")


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


def test_sparse_messages_long_gaps(orc):
    # entries far apart, clustered at either end, or absent: the output-tile
    # table is then mostly filled by search rather than by the entries
    layout = sgc.Layout([1 << 23, 5000])
    n = layout.n
    seg_off = np.array(layout.seg_off, np.int64)
    rng = np.random.default_rng(81)
    sets = [np.array([5, 6, 7, 100000, 8000000], np.int64),
            np.arange(n - 300, n - 1, 7, dtype=np.int64),
            np.array([0], np.int64),
            np.array([n - 1], np.int64),
            np.zeros(0, np.int64)]
    gm, om = [], []
    for s_i, idx in enumerate(sets):
        counts = np.array([(idx < seg_off[1]).sum(), (idx >= seg_off[1]).sum(), idx.size], np.int64)
        val = rng.normal(0, 1, idx.size).astype(np.float32)
        cap = max(idx.size, 1)
        idx_d = dev(np.concatenate([idx, np.zeros(cap - idx.size, np.int64)]).astype(np.int32))
        val_d = dev(np.concatenate([val, np.zeros(cap - idx.size, np.float32)]))
        cnt_d = dev(counts)
        if s_i % 2 == 0:
            gm.append(sgc.Message(sgc.MSG_RAW_F32, cnt_d, cap, idx=idx_d, val=val_d))
            om.append(orc.Message(counts, idx=idx.astype(np.int32), val=val))
        else:
            b = 2
            enc = sgc.encode(layout, idx_d, cnt_d, cap, scope=1, b=b)
            oenc = orc.encode(idx.astype(np.int32), counts, seg_off, 1, b)
            gm.append(sgc.golomb_message(sgc.Compressed(idx_d, val_d, cnt_d, None, cap), enc))
            om.append(orc.Message(counts, golomb=True, scope=1, b=b, val=val, enc=oenc))
    ref = np.zeros(n, np.float32)
    assert orc.decode_accumulate(om, seg_off, ref) == 0
    # a workspace full of stale bytes: every table entry the call reads must be its own
    arr = (sgc.MessageDesc * len(gm))(*[m.desc() for m in gm])
    nbytes = sgc.lib().sgc_decode_accumulate_workspace(layout.handle, arr, len(gm))
    for fill in (0x00, 0x7F, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        announce(f"decode_accumulate sparse long gaps W={len(gm)} workspace bytes {fill:#x}")
        st = sgc.decode_accumulate(layout, gm, out, ws=ws)
        torch.cuda.synchronize()
        assert int(host(st)[0]) == 0
        assert_bitwise(host(out), ref, f"sparse long gaps, workspace bytes {fill:#x}")
