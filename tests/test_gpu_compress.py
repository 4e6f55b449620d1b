"""GPU parity of sgc_compress against the CPU oracle (bit-exact).

Indices, kept values, residuals and per-segment counts must match the
oracle bit for bit, for exact and sampled selection, global and per-segment
scope, across ragged segment tables, ties, zeros, clustered inputs that
overflow the per-tile candidate regions, and inputs that defeat the probe
sample (the full-pass path).  Each case runs through both compress pipelines
(the `path` fixture: gather and window), whatever the kept fraction.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
import workloads as W
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(params=[sgc.PATH_GATHER, sgc.PATH_WINDOW], ids=["gather", "window"])
def path(request):
    return request.param


def check_step(orc, layout, g, r, *, mode, scope, ppm, cap=None, sample_div=1000, sample_min=65536, what="",
               path=sgc.PATH_AUTO):
    """Run one compress step on both sides; r (host) is advanced like the GPU residual."""
    announce(f"compress {what} n={layout.n} nseg={layout.nseg} mode={mode} scope={scope} ppm={ppm} path={path}")
    gd, rd = dev(g), dev(r)
    out = sgc.compress(layout, gd, rd, mode=mode, scope=scope, keep_ppm=ppm, cap=cap,
                       sample_div=sample_div, sample_min=sample_min, path=path)
    torch.cuda.synchronize()
    seg_off = np.array(layout.seg_off, np.int64)
    if mode == sgc.EXACT:
        ref = orc.compress_exact(g, r, seg_off, scope, ppm, cap=out.cap)
    else:
        ref = orc.compress_sampled(g, r, seg_off, scope, ppm, out.cap, sample_div, sample_min)
    counts = host(out.counts)
    total = int(counts[-1])
    assert_bitwise(counts, ref.counts, f"{what} counts")
    assert_bitwise(host(out.idx)[:total], ref.idx, f"{what} idx")
    assert_bitwise(host(out.val)[:total], ref.val, f"{what} val")
    assert_bitwise(host(rd), r, f"{what} residual")
    st = int(host(out.status)[0])
    if mode == sgc.SAMPLED:
        assert (st & sgc.STATUS_TRUNCATED) == (ref.status & 1), f"{what} truncation flag"
    return out, st


@pytest.mark.parametrize("steps", [3])
def test_flat_1m_exact_three_steps(orc, path, steps):
    w = W.FLAT_1M
    layout = sgc.Layout(w.seg_numel)
    r = np.zeros(w.numel, np.float32)
    for s in range(steps):
        g = W.gradient(w, 0, s).numpy()
        check_step(orc, layout, g, r, mode=sgc.EXACT, scope=w.scope, ppm=w.keep_ppm, path=path,
                   what=f"flat-1M step {s}")


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("scope", [0, 1])
@pytest.mark.parametrize("ppm", [0, 1000, 10000, 250000, 1000000])
def test_ragged_segments(orc, path, seed, scope, ppm):
    rng = np.random.default_rng(100 + seed)
    sizes = [0, 1, 3, 5, 10, 17, 4095, 4097, 8191, 8193, 12345, 0, 64, 70001]
    rng.shuffle(sizes)
    layout = sgc.Layout(sizes)
    n = layout.n
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    r = np.zeros(n, np.float32)
    for s in range(2):
        check_step(orc, layout, g, r, mode=sgc.EXACT, scope=scope, ppm=ppm, path=path, what=f"ragged seed{seed} s{s}")
        g = rng.laplace(0, 1e-3, n).astype(np.float32)


@pytest.mark.parametrize("scope", [0, 1])
def test_ties_and_zeros(orc, path, scope):
    rng = np.random.default_rng(7)
    layout = sgc.Layout([30000, 50000, 7, 20000])
    n = layout.n
    # coarse quantized values: massive ties at every magnitude, signed zeros
    g = (rng.integers(-6, 7, n) * 0.125).astype(np.float32)
    g[rng.random(n) < 0.3] = -0.0
    r = np.zeros(n, np.float32)
    check_step(orc, layout, g, r, mode=sgc.EXACT, scope=scope, ppm=10000, path=path, what="quantized ties")
    # all zeros: the threshold is 0 and the lowest indices win
    z = np.zeros(n, np.float32)
    z[::3] = -0.0
    r2 = np.zeros(n, np.float32)
    check_step(orc, layout, z, r2, mode=sgc.EXACT, scope=scope, ppm=10000, path=path, what="all zeros")


def test_probe_defeated_takes_full_pass_path(orc, path):
    # Large values sit exactly where the exact mode's probe reads (at n = 2^20: runs of 16
    # elements starting at 2048 + 4096 j), so the probe overestimates the threshold, fewer than
    # k candidates pass, and the selection falls back to full passes over the residual.
    n = 1 << 20
    g = np.random.default_rng(1).normal(0, 1e-4, n).astype(np.float32)
    runs = (2048 + 4096 * np.arange(n // 4096))[:, None] + np.arange(16)[None, :]
    g[runs.ravel()] = 1.0 + np.arange(runs.size, dtype=np.float32) * 1e-3
    layout = sgc.Layout([n])
    r = np.zeros(n, np.float32)
    out, st = check_step(orc, layout, g, r, mode=sgc.EXACT, scope=0, ppm=10000, path=path, what="probe defeated")
    assert st & sgc.STATUS_DENSE_PATH


def test_all_tied_candidates(orc, path):
    # Segments of equal magnitudes make every element a candidate (the candidate bound is that
    # magnitude).  Gather: at 1% its candidate array holds 4K + 2^18 = 280,144 entries; per
    # tensor the first segment's 100,000 fit, the second's 300,000 do not (full passes over the
    # residual), and the small normal segment after them is also taken by full passes; globally
    # 400,000 candidates, full passes.  Window: every sampled key is the same, so there is no
    # sure bound; the whole tie run is the window, the tiles' window lists overflow and the
    # selection reads the regions.  Ties go to the lowest indices either way.
    rng = np.random.default_rng(12)
    sizes = [100000, 300000, 50000]
    n = sum(sizes)
    g = np.empty(n, np.float32)
    g[:100000] = 1.0
    g[100000:400000] = -1.0  # the same magnitude: one run of 400,000 tied candidates in global scope
    g[400000:] = rng.normal(0, 1e-3, 50000).astype(np.float32)
    layout = sgc.Layout(sizes)
    for scope in (1, 0):
        r = np.zeros(n, np.float32)
        out, st = check_step(orc, layout, g, r, mode=sgc.EXACT, scope=scope, ppm=10000, path=path,
                             what=f"all tied scope{scope}")
        if path == sgc.PATH_GATHER:
            assert st & sgc.STATUS_DENSE_PATH


def _probe_positions(n):
    # where the exact mode's probe reads at these sizes: runs of 16 elements from 2048 + 4096 j
    return ((2048 + 4096 * np.arange(n // 4096))[:, None] + np.arange(16)[None, :]).ravel()


def test_sure_bound_exceeded_takes_all_candidates(orc):
    # Window pipeline.  |values| are 10% smaller where the probe reads, so the sampled threshold
    # is low: more than k entries lie above the sure bound, and the selection takes every
    # candidate as its window (no region overflows at 10%: about 16% of each tile are
    # candidates, regions hold 25%).
    n = 1 << 21
    rng = np.random.default_rng(31)
    g = rng.normal(0, 1.0, n).astype(np.float32)
    g[_probe_positions(n)] *= np.float32(0.9)
    layout = sgc.Layout([n])
    r = np.zeros(n, np.float32)
    out, st = check_step(orc, layout, g, r, mode=sgc.EXACT, scope=0, ppm=100000, path=sgc.PATH_WINDOW,
                         what="sure bound exceeded")
    assert st & sgc.STATUS_DENSE_PATH


def test_dense_and_wide_with_candidate_masks(orc):
    # Window pipeline at 25% kept, where regions keep candidate masks in place of offsets.
    # Large values where the probe reads: fewer than k candidates, the group is selected
    # from the residual, and selection pass 0 first restores acc from the masked regions.
    # Values 10% smaller there: more than k sure entries, every candidate is searched.
    n = 1 << 20
    rng = np.random.default_rng(33)
    layout = sgc.Layout([n])
    g = rng.normal(0, 1e-4, n).astype(np.float32)
    pp = _probe_positions(n)
    g[pp] = 1.0 + np.arange(pp.size, dtype=np.float32) * 1e-3
    out, st = check_step(orc, layout, g, np.zeros(n, np.float32), mode=sgc.EXACT, scope=0, ppm=250000,
                         path=sgc.PATH_WINDOW, what="probe defeated, masks")
    assert st & sgc.STATUS_DENSE_PATH
    g = rng.normal(0, 1.0, 1 << 21).astype(np.float32)
    g[_probe_positions(1 << 21)] *= np.float32(0.9)
    for scope, sizes in ((0, [1 << 21]), (1, [1 << 20, 1 << 20])):
        out, st = check_step(orc, sgc.Layout(sizes), g, np.zeros(1 << 21, np.float32), mode=sgc.EXACT, scope=scope,
                             ppm=250000, path=sgc.PATH_WINDOW, what=f"sure bound exceeded, masks, scope{scope}")
        if scope == 0:  # per tensor, each group's own probe keeps a window here: parity only
            assert st & sgc.STATUS_DENSE_PATH


def test_sure_bound_exceeded_in_overflowed_tiles(orc):
    # Window pipeline.  Tiny values where the probe reads, ordinary ones everywhere else: every element is a
    # candidate and sure, every region overflows, and the tiles are worked from the residual.
    # (At 10% of 2^20 or more elements the probe takes enough samples to set a sure bound.)
    n = 1 << 21
    rng = np.random.default_rng(32)
    g = rng.normal(0, 1.0, n).astype(np.float32)
    g[_probe_positions(n)] = rng.normal(0, 1e-6, _probe_positions(n).size).astype(np.float32)
    layout = sgc.Layout([n // 2, n // 2])
    for scope in (0, 1):
        r = np.zeros(n, np.float32)
        out, st = check_step(orc, layout, g, r, mode=sgc.EXACT, scope=scope, ppm=100000,
                             path=sgc.PATH_WINDOW, what=f"sure bound exceeded, overflowed, scope{scope}")
        assert st & sgc.STATUS_DENSE_PATH


def test_clustered_overflowing_tiles(orc, path):
    # All large values in a few contiguous runs: some tiles hold far more candidates than
    # their region, and those tiles are redone from the residual.
    n = 1 << 21
    rng = np.random.default_rng(5)
    g = rng.normal(0, 1e-5, n).astype(np.float32)
    for start in (5000, 300000, 1500007):
        g[start:start + 9000] = rng.laplace(0, 1.0, 9000).astype(np.float32)
    layout = sgc.Layout([n // 2, n // 2])
    for scope in (0, 1):
        r = np.zeros(n, np.float32)
        check_step(orc, layout, g, r, mode=sgc.EXACT, scope=scope, ppm=10000, path=path, what=f"clustered scope{scope}")
        r = np.zeros(n, np.float32)
        check_step(orc, layout, g, r, mode=sgc.SAMPLED, scope=scope, ppm=10000, cap=n, path=path,
                   what=f"clustered sampled{scope}")


@pytest.mark.parametrize("ppm", [60000, 150000, 400000])
def test_clustered_overflow_at_larger_regions(orc, path, ppm):
    # At these kept fractions the regions hold 512, 1024 and 4096 slots (a power of two near 1.5x
    # the expected candidates of a tile); runs of huge values still overflow the smaller ones.
    n = 1 << 21
    rng = np.random.default_rng(6)
    g = rng.normal(0, 1e-5, n).astype(np.float32)
    for start in (7000, 400001):
        g[start:start + 20000] = rng.laplace(0, 1.0, 20000).astype(np.float32)
    layout = sgc.Layout([n // 3, n - n // 3])
    for scope in (0, 1):
        r = np.zeros(n, np.float32)
        check_step(orc, layout, g, r, mode=sgc.EXACT, scope=scope, ppm=ppm, path=path,
                   what=f"clustered {ppm} scope{scope}")
        check_step(orc, layout, g * np.float32(0.25), r, mode=sgc.EXACT, scope=scope, ppm=ppm,
                   path=path, what=f"clustered {ppm} scope{scope} step 2")


@pytest.mark.parametrize("scope", [0, 1])
@pytest.mark.parametrize("ppm", [1000, 10000])
def test_sampled_matches_oracle(orc, path, scope, ppm):
    rng = np.random.default_rng(11)
    layout = sgc.Layout([1 << 20, 300000, 4096, 1, 99999])
    n = layout.n
    r = np.zeros(n, np.float32)
    for s in range(2):
        g = rng.laplace(0, 1e-3, n).astype(np.float32)
        check_step(orc, layout, g, r, mode=sgc.SAMPLED, scope=scope, ppm=ppm, path=path, what=f"sampled s{s}")


def test_sampled_truncation(orc, path):
    rng = np.random.default_rng(12)
    n = 500000
    layout = sgc.Layout([n])
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    r = np.zeros(n, np.float32)
    out, st = check_step(orc, layout, g, r, mode=sgc.SAMPLED, scope=0, ppm=10000, cap=3000, path=path, what="truncated")
    assert st & sgc.STATUS_TRUNCATED


def test_accumulate_only(orc):
    rng = np.random.default_rng(13)
    for n in (1, 3, 4, 1023, 1 << 20, (1 << 20) + 7):
        layout = sgc.Layout([n])
        g = rng.laplace(0, 1e-3, n).astype(np.float32)
        r = rng.laplace(0, 1e-3, n).astype(np.float32)
        rd = dev(r)
        sgc.compress(layout, dev(g), rd, mode=sgc.ACCUMULATE_ONLY)
        orc.accumulate(g, r)
        assert_bitwise(host(rd), r, f"accumulate n={n}")


def test_mlp_mnist_global_two_steps(orc, path):
    w = W.MLP_MNIST
    layout = sgc.Layout(w.seg_numel)
    r = np.zeros(w.numel, np.float32)
    for s in range(2):
        g = W.gradient(w, 0, s).numpy()
        check_step(orc, layout, g, r, mode=sgc.EXACT, scope=w.scope, ppm=w.keep_ppm, path=path, what=f"mlp step {s}")


def test_resnet50_delay_per_tensor(orc, path):
    w = W.RESNET50
    layout = sgc.Layout(w.seg_numel)
    r = np.zeros(w.numel, np.float32)
    rd = dev(r)
    for s in range(w.delay - 1):
        g = W.gradient(w, 0, s).numpy()
        sgc.compress(layout, dev(g), rd, mode=sgc.ACCUMULATE_ONLY)
        orc.accumulate(g, r)
    assert_bitwise(host(rd), r, "resnet delay accumulate")
    g = W.gradient(w, 0, w.delay - 1).numpy()
    check_step(orc, layout, g, r, mode=sgc.EXACT, scope=w.scope, ppm=w.keep_ppm, path=path, what="resnet exchange")


def test_empty_layout(orc, path):
    layout = sgc.Layout([0, 0])
    g = torch.zeros(0, dtype=torch.float32, device="cuda")
    r = torch.zeros(0, dtype=torch.float32, device="cuda")
    out = sgc.compress(layout, g, r, keep_ppm=10000, path=path)
    torch.cuda.synchronize()
    assert host(out.counts).tolist() == [0, 0, 0]


@pytest.mark.parametrize("fill", [0x00, 0x7F, 0xFF])
def test_stale_workspace(orc, path, fill):
    # every workspace byte a call reads is written by that call first
    rng = np.random.default_rng(17)
    layout = sgc.Layout([300000, 4097, 1 << 20])
    n = layout.n
    seg_off = np.array(layout.seg_off, np.int64)
    for scope in (0, 1):
        g = rng.laplace(0, 1e-3, n).astype(np.float32)
        r = np.zeros(n, np.float32)
        opts = sgc.CompressOpts(sgc.EXACT, scope, 10000, 1000, 65536, path)
        cap = layout.keep_total(scope, 10000)
        nbytes = sgc.lib().sgc_compress_workspace(layout.handle, C.byref(opts), cap)
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        announce(f"compress stale workspace {fill:#x} scope={scope}")
        rd = dev(r)
        out = sgc.compress(layout, dev(g), rd, scope=scope, keep_ppm=10000, ws=ws, path=path)
        ref = orc.compress_exact(g, r, seg_off, scope, 10000, cap=out.cap)
        torch.cuda.synchronize()
        total = int(ref.counts[-1])
        assert_bitwise(host(out.counts), ref.counts, "counts")
        assert_bitwise(host(out.idx)[:total], ref.idx, "idx")
        assert_bitwise(host(rd), r, "residual")
        b = 5
        enb = sgc.lib().sgc_encode_workspace(layout.handle, scope, out.cap)
        ews = torch.full((enb,), fill, dtype=torch.uint8, device="cuda")
        enc = sgc.encode(layout, out.idx, out.counts, out.cap, scope=scope, b=b, ws=ews)
        oenc = orc.encode(ref.idx, ref.counts, seg_off, scope, b)
        torch.cuda.synchronize()
        nw = int(oenc.word_off[-1])
        assert_bitwise(host(enc.words).view(np.uint32)[:nw], oenc.words, "words")
        assert_bitwise(host(enc.chunk_off).view(np.uint64)[:oenc.chunk_off.size], oenc.chunk_off, "chunk table")


@pytest.mark.parametrize("mode", [sgc.EXACT, sgc.SAMPLED])
@pytest.mark.parametrize("bmode", [sgc.BIN_SBC, sgc.BIN_2BIT])
@pytest.mark.parametrize("scope", [0, 1])
def test_hold_then_held_binarize(orc, path, mode, bmode, scope):
    # compress with the hold flag leaves acc at the kept entries; binarize with the held flag then
    # gives exactly what compress + binarize without the flags give, writing half as much
    rng = np.random.default_rng(41)
    layout = sgc.Layout([1 << 20, 300001, 4096, 77])
    n = layout.n
    seg_off = np.array(layout.seg_off, np.int64)
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    r0 = rng.laplace(0, 1e-3, n).astype(np.float32)
    cap = None if mode == sgc.EXACT else 40000
    announce(f"hold/held mode={mode} bmode={bmode} scope={scope}")
    outs = []
    for hold in (False, True):
        rd = dev(r0)
        comp = sgc.compress(layout, dev(g), rd, mode=mode, scope=scope, keep_ppm=10000, cap=cap, hold=hold,
                            path=path)
        torch.cuda.synchronize()
        if hold:  # the residual after compress: acc at the sent entries
            r_ref = r0.copy()
            ref = (orc.compress_exact(g, r_ref, seg_off, scope, 10000, cap=comp.cap) if mode == sgc.EXACT else
                   orc.compress_sampled(g, r_ref, seg_off, scope, 10000, comp.cap))
            orc.hold_kept(ref, r_ref)
            assert_bitwise(host(rd), r_ref, "held residual after compress")
        bn = sgc.binarize(layout, comp, rd, bmode, held=hold)
        torch.cuda.synchronize()
        outs.append((host(rd), host(bn.counts), host(bn.means),
                     host(bn.idx)[:int(host(bn.counts)[-1])] if bn.idx is not None else None,
                     host(bn.codes) if bn.codes is not None else None))
    (r1, c1, m1, i1, k1), (r2, c2, m2, i2, k2) = outs
    assert_bitwise(r2, r1, "residual after binarize")
    assert_bitwise(c2, c1, "counts")
    assert_bitwise(m2, m1, "means")
    if i1 is not None:
        assert_bitwise(i2, i1, "sent indices")
    if k1 is not None:
        assert_bitwise(k2, k1, "2-bit codes")
