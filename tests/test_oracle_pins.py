"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something it does not compute itself:
values printed on the pages (tests/golden), closed forms, brute force on
tiny inputs, hand-worked examples, invariants the method guarantees, and
special cases that reduce to a plain library routine.

Citations:
  [AH17]  "Sparse Communication for Distributed Gradient Descent" (Aji & Heafield)
  [AHB19] "Combining Global Sparse Gradients with Local Gradients in Distributed
          Neural Network Training" (Aji, Heafield & Bogoychev)
  [SBC]   "Sparse Binary Compression: Towards Distributed Deep Learning with
          minimal Communication" (Sattler et al.)
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    return vals


# ---------------------------------------------------------------- keep count
def test_keep_count_flat_1m_workload(orc):
    # The flat 2^20-element workload is specified at drop ratio 99% with k = 10486.
    assert orc.keep_count(1 << 20, 10000) == 10486


@pytest.mark.parametrize("n", [1, 7, 10, 64, 100, 999, 1000, 1001, 4096, 2359296, (1 << 31) - 1])
@pytest.mark.parametrize("ppm", [0, 1, 1000, 10000, 250000, 999999, 1000000])
def test_keep_count_is_smallest_k_reaching_fraction(orc, n, ppm):
    # [AH17] Abstract / [SBC] Sparse Binarization: keep (at least) the fraction p.
    # k is the least integer with k/n >= ppm/1e6, never more than n.
    k = orc.keep_count(n, ppm)
    assert 0 <= k <= n
    assert Fraction(k, n) >= Fraction(ppm, 10**6)
    if k > 0:
        assert Fraction(k - 1, n) < Fraction(ppm, 10**6)


def test_keep_count_small_tensors_keep_one(orc):
    # A 64-element BN vector at top-0.1% still sends its largest entry.
    assert orc.keep_count(64, 1000) == 1
    # 1 - 0.99 is not exactly 0.01 in binary floating point; integers avoid k = 2 at n = 100.
    assert orc.keep_count(100, 10000) == 1


# ------------------------------------------------------------- Rice lengths
def test_rice_mean_bits_matches_page(orc):
    # [SBC] §II Optimal Position Encoding prints 8.38 bits and x1.9 vs 16 bits at p = 0.01.
    gold = read_golden("rice_bits_p001.txt")
    e7 = orc.rice_expected_bits(7, gold["p"])
    assert round(e7, 2) == gold["mean_bits"]
    assert round(16.0 / e7, 1) == gold["ratio_vs_16bit"]


@pytest.mark.parametrize("b,p", [(0, 0.5), (3, 0.1), (6, 0.01), (7, 0.01), (9, 0.001), (2, 0.9)])
def test_rice_expected_bits_equals_series(orc, b, p):
    # Direct sum over the geometric gap law P(z) = (1-p)^z p of the code length b + 1 + floor(z/2^b).
    total, z, mass = 0.0, 0, 0.0
    while mass < 1 - 1e-15 and z < 10_000_000:
        pz = (1 - p) ** z * p
        total += pz * (b + 1 + (z >> b))
        mass += pz
        z += 1
    assert orc.rice_expected_bits(b, p) == pytest.approx(total, rel=1e-9)


def test_rice_param_argmin(orc):
    assert orc.rice_param(0.01) == 6
    assert orc.rice_param(0.001) == 9
    # [SBC] §I: dense updates need no position bits; with every element present all gaps are 0.
    assert orc.rice_param(1.0) == 0
    assert orc.rice_expected_bits(0, 1.0) == 1.0


def test_rice_measured_bits_page_value(orc):
    # Encode Bernoulli(0.01) positions with b = 7 and compare the mean code length with the page's 8.38.
    rng = np.random.default_rng(7)
    n = 4_000_000
    pos = np.flatnonzero(rng.random(n) < 0.01).astype(np.int32)
    counts = np.array([pos.size, pos.size], np.int64)
    enc = orc.encode(pos, counts, [0, n], orc.GLOBAL, 7)
    mean_bits = int(enc.nbits[0]) / pos.size
    # std of one code length ~ sqrt(q)/(1-q) (geometric unary part); 4 sigma band
    q = (1 - 0.01) ** 128
    sigma = math.sqrt(q) / (1 - q) / math.sqrt(pos.size)
    assert abs(mean_bits - 8.38) < 4 * sigma + 0.005


# ------------------------------------------------------- exact selection
vec = st.lists(st.sampled_from([0.0, -0.0, 0.5, -0.5, 0.25, -0.25, 1.0, -1.0, 3.0, -2.0, 1e-40, -1e-40]),
               min_size=0, max_size=14)


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(g=vec, rv=vec, ppm=st.sampled_from([0, 1, 100000, 250000, 500000, 999999, 1000000]),
       cuts=st.lists(st.integers(0, 14), max_size=3), scope=st.sampled_from([0, 1]))
def test_exact_select_matches_rank_count(orc, g, rv, ppm, cuts, scope):
    n = min(len(g), len(rv))
    g = np.array(g[:n], np.float32)
    r = np.array(rv[:n], np.float32)
    bounds = sorted({0, n} | {c for c in cuts if c <= n})
    seg_off = np.array(bounds if len(bounds) > 1 else [0, n], np.int64)
    acc = (r + g).astype(np.float32)          # numpy fp32 add is IEEE round-to-nearest-even
    groups = [(0, n)] if scope == 0 else [(int(seg_off[t]), int(seg_off[t + 1])) for t in range(len(seg_off) - 1)]
    want = []
    for lo, hi in groups:
        k = bf.ceil_frac((hi - lo) * ppm, 10**6)
        want += bf.kept_by_rank(acc, lo, hi, k)
    want = sorted(want)
    r2 = r.copy()
    sp = orc.compress_exact(g, r2, seg_off, scope, ppm)
    assert sp.idx.tolist() == want
    assert sp.val.view(np.uint32).tolist() == acc[want].view(np.uint32).tolist()
    expect_r = acc.copy()
    expect_r[want] = 0.0
    assert r2.view(np.uint32).tolist() == expect_r.view(np.uint32).tolist()
    for t in range(len(seg_off) - 1):
        assert sp.counts[t] == sum(1 for i in want if seg_off[t] <= i < seg_off[t + 1])
    assert sp.counts[-1] == len(want)


def test_worked_example_topk(orc):
    # acc = [0.5, -0.5, 0.25, -1.0, 0.5, 0.0], k = 3: -1.0 first, then the 0.5-magnitude tie
    # is won by indices 0 and 1 over 4 (lower index wins).
    acc = np.array([0.5, -0.5, 0.25, -1.0, 0.5, 0.0], np.float32)
    r = np.zeros(6, np.float32)
    sp = orc.compress_exact(acc, r, [0, 6], orc.GLOBAL, 500000)   # 50% of 6 = 3
    assert sp.idx.tolist() == [0, 1, 3]
    assert sp.val.tolist() == [0.5, -0.5, -1.0]
    assert r.tolist() == [0.0, 0.0, 0.25, 0.0, 0.5, 0.0]


def test_exact_invariants_flat_1m(orc):
    import workloads as W
    w = W.FLAT_1M
    r = np.zeros(w.numel, np.float32)
    k = orc.keep_count(w.numel, w.keep_ppm)
    for step in range(w.steps):
        g = W.gradient(w, 0, step).numpy()
        acc = (r + g).astype(np.float32)
        sp = orc.compress_exact(g, r, w.seg_off, w.scope, w.keep_ppm)
        assert sp.idx.size == k == sp.counts[-1]
        assert np.all(np.diff(sp.idx) > 0)
        kept = np.zeros(w.numel, bool)
        kept[sp.idx] = True
        mk = np.abs(acc[kept]).min()
        md = np.abs(acc[~kept]).max()
        assert mk >= md
        if mk == md:   # ties at the threshold go to the lower indices
            assert np.flatnonzero(kept & (np.abs(acc) == mk)).max() < np.flatnonzero(~kept & (np.abs(acc) == md)).min()
        # residual + sent == acc, bitwise
        rebuilt = r.copy()
        rebuilt[sp.idx] = rebuilt[sp.idx] + sp.val
        assert np.array_equal(rebuilt.view(np.uint32), acc.view(np.uint32))
        assert np.all(r[sp.idx].view(np.uint32) == 0)


def test_resume_equals_straight_run(orc, tmp_path):
    # The only state carried between steps is the residual: save/restore it mid-run.
    import workloads as W
    w = W.FLAT_1M
    gs = [W.gradient(w, 0, s, numel=65536).numpy() for s in range(3)]
    r1 = np.zeros(65536, np.float32)
    outs1 = [orc.compress_exact(g, r1, [0, 65536], 0, 10000) for g in gs]
    r2 = np.zeros(65536, np.float32)
    outs2 = [orc.compress_exact(g, r2, [0, 65536], 0, 10000) for g in gs[:2]]
    np.save(tmp_path / "res.npy", r2)
    r3 = np.load(tmp_path / "res.npy")
    outs2.append(orc.compress_exact(gs[2], r3, [0, 65536], 0, 10000))
    assert np.array_equal(r1.view(np.uint32), r3.view(np.uint32))
    for a, b in zip(outs1, outs2):
        assert np.array_equal(a.idx, b.idx) and np.array_equal(a.val.view(np.uint32), b.val.view(np.uint32))


def test_delay_one_is_plain_step_and_delay_two_sums(orc):
    # [SBC] §II Communication Delay: n = 1 is regular DSGD; with n = 2 the first draw is
    # only accumulated, so the exchange sees fp32(g1 + g2).
    rng = np.random.default_rng(3)
    g1 = rng.laplace(0, 1e-3, 5000).astype(np.float32)
    g2 = rng.laplace(0, 1e-3, 5000).astype(np.float32)
    r = np.zeros(5000, np.float32)
    orc.accumulate(g1, r)
    assert np.array_equal(r, g1)
    sp = orc.compress_exact(g2, r, [0, 5000], 0, 10000)
    r_ref = np.zeros(5000, np.float32)
    sp_ref = orc.compress_exact((g1 + g2).astype(np.float32), r_ref, [0, 5000], 0, 10000)
    assert np.array_equal(sp.idx, sp_ref.idx) and np.array_equal(sp.val, sp_ref.val)
    assert np.array_equal(r, r_ref)


# ------------------------------------------------------ momentum correction
# [SBC] appendix A (Momentum Correction, Warm-up Training and Momentum Masking):
# the momentum-corrected gradient goes into the residual; the momentum of the
# sent entries is set to zero.  Reading: u <- fp32(fp32(beta*u) + g) first.
fvals = st.sampled_from([0.0, 0.5, -0.5, 0.25, -0.25, 1.0, -1.0, 3.0, -2.0, 1.5e-3, -7e-5, 1e-40, 6.5e4])


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(u=st.lists(fvals, min_size=0, max_size=12), g=st.lists(fvals, min_size=0, max_size=12),
       beta=st.sampled_from([0.0, 0.5, 0.9, 0.99, 1.0, -0.25]))
def test_momentum_correct_matches_numpy(orc, u, g, beta):
    n = min(len(u), len(g))
    u = np.array(u[:n], np.float32)
    g = np.array(g[:n], np.float32)
    want = (np.float32(beta) * u).astype(np.float32) + g      # two IEEE fp32 roundings, no fused multiply-add
    got = u.copy()
    orc.momentum_correct(beta, g, got)
    assert got.view(np.uint32).tolist() == want.astype(np.float32).view(np.uint32).tolist()


@settings(max_examples=200, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(u=st.lists(fvals, min_size=0, max_size=12), g=vec, rv=vec, beta=st.sampled_from([0.5, 0.9]),
       ppm=st.sampled_from([0, 100000, 250000, 500000, 1000000]), scope=st.sampled_from([0, 1]))
def test_momentum_step_matches_rank_count(orc, u, g, rv, beta, ppm, scope):
    n = min(len(u), len(g), len(rv))
    u = np.array(u[:n], np.float32)
    g = np.array(g[:n], np.float32)
    r = np.array(rv[:n], np.float32)
    seg_off = np.array([0, n // 2, n], np.int64)
    u1 = ((np.float32(beta) * u).astype(np.float32) + g).astype(np.float32)
    acc = (r + u1).astype(np.float32)
    groups = [(0, n)] if scope == 0 else [(int(seg_off[t]), int(seg_off[t + 1])) for t in range(2)]
    want = []
    for lo, hi in groups:
        want += bf.kept_by_rank(acc, lo, hi, bf.ceil_frac((hi - lo) * ppm, 10**6))
    want = sorted(want)
    u2, r2 = u.copy(), r.copy()
    sp = orc.compress_momentum(g, u2, r2, beta, seg_off, scope, ppm)
    assert sp.idx.tolist() == want
    assert sp.val.view(np.uint32).tolist() == acc[want].view(np.uint32).tolist()
    er, eu = acc.copy(), u1.copy()
    er[want] = 0.0
    eu[want] = 0.0
    assert r2.view(np.uint32).tolist() == er.view(np.uint32).tolist()
    assert u2.view(np.uint32).tolist() == eu.view(np.uint32).tolist()


def test_worked_example_momentum(orc):
    # beta = 0.5: u' = 0.5*[2, -2, 0, 4] + [1, 1, 1, -3] = [2, 0, 1, -1]; acc = r + u' with
    # r = [0, 0.5, 0, 0] gives [2, 0.5, 1, -1]; keep 2 of 4: 2, then the |1| tie goes to index 2.
    u = np.array([2, -2, 0, 4], np.float32)
    g = np.array([1, 1, 1, -3], np.float32)
    r = np.array([0, 0.5, 0, 0], np.float32)
    sp = orc.compress_momentum(g, u, r, 0.5, [0, 4], orc.GLOBAL, 500000)
    assert sp.idx.tolist() == [0, 2] and sp.val.tolist() == [2.0, 1.0]
    assert r.tolist() == [0.0, 0.5, 0.0, -1.0]
    assert u.tolist() == [0.0, 0.0, 0.0, -1.0]


def test_momentum_zero_beta_is_plain_step(orc):
    # beta = 0: u' = g (no negative zeros here), so the step is the plain one and u holds g masked
    rng = np.random.default_rng(5)
    n = 20000
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    u = rng.normal(0, 1, n).astype(np.float32)
    r = rng.laplace(0, 1e-3, n).astype(np.float32)
    r_ref = r.copy()
    sp = orc.compress_momentum(g, u, r, 0.0, [0, n], orc.GLOBAL, 10000)
    sp_ref = orc.compress_exact(g, r_ref, [0, n], orc.GLOBAL, 10000)
    assert np.array_equal(sp.idx, sp_ref.idx) and np.array_equal(sp.val.view(np.uint32), sp_ref.val.view(np.uint32))
    assert np.array_equal(r.view(np.uint32), r_ref.view(np.uint32))
    want_u = g.copy()
    want_u[sp.idx] = 0.0
    assert np.array_equal(u.view(np.uint32), want_u.view(np.uint32))


def test_momentum_invariants_over_steps(orc):
    # every step: residual + sent == fp32(residual + u'), bitwise; u == u' outside the sent set
    rng = np.random.default_rng(6)
    n = 30000
    u = np.zeros(n, np.float32)
    r = np.zeros(n, np.float32)
    for step in range(4):
        g = rng.laplace(0, 1e-3, n).astype(np.float32)
        u1 = ((np.float32(0.9) * u).astype(np.float32) + g).astype(np.float32)
        acc = (r + u1).astype(np.float32)
        sp = orc.compress_momentum(g, u, r, 0.9, [0, n], orc.GLOBAL, 10000)
        assert sp.idx.size == orc.keep_count(n, 10000)
        rebuilt = r.copy()
        rebuilt[sp.idx] = rebuilt[sp.idx] + sp.val
        assert np.array_equal(rebuilt.view(np.uint32), acc.view(np.uint32))
        keep = np.zeros(n, bool)
        keep[sp.idx] = True
        assert np.array_equal(u[~keep].view(np.uint32), u1[~keep].view(np.uint32))
        assert np.all(u[keep].view(np.uint32) == 0)


def test_hold_kept_then_held_binarize_equals_plain_pair(orc):
    # the hold flag only defers the residual write of the sent entries: with acc held there, the
    # held binarize must give the residual the plain pair gives, and the held residual itself is
    # acc at the sent entries and the plain residual elsewhere
    rng = np.random.default_rng(8)
    n = 40000
    seg_off = np.array([0, 15000, 15001, n], np.int64)
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    r0 = rng.laplace(0, 1e-3, n).astype(np.float32)
    acc = (r0 + g).astype(np.float32)
    for mode in (orc.BIN_SBC, orc.BIN_2BIT):
        ra, rb = r0.copy(), r0.copy()
        spa = orc.compress_exact(g, ra, seg_off, orc.PER_SEGMENT, 10000)
        spb = orc.compress_exact(g, rb, seg_off, orc.PER_SEGMENT, 10000)
        orc.hold_kept(spb, rb)
        assert np.array_equal(rb.view(np.uint32), acc.view(np.uint32))
        ba = orc.binarize(spa, 3, mode, ra)
        bb = orc.binarize_held(spb, 3, mode, rb)
        assert np.array_equal(ra.view(np.uint32), rb.view(np.uint32))
        assert np.array_equal(ba.means.view(np.uint32), bb.means.view(np.uint32))


# ------------------------------------------------------------ sampled mode
def test_sampled_full_sample_is_superlevel_set(orc):
    rng = np.random.default_rng(11)
    n = 20000
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    g[100:140] = 0.003          # ties, some of which straddle the threshold
    r0 = np.zeros(n, np.float32)
    k = orc.keep_count(n, 10000)
    # sample_min >= n -> every element is sampled: T is the k-th largest |acc|
    r = r0.copy()
    sp = orc.compress_sampled(g, r, [0, n], 0, 10000, cap=n, sample_div=1, sample_min=n)
    T = np.sort(np.abs(g))[::-1][k - 1]
    assert sp.idx.tolist() == np.flatnonzero(np.abs(g) >= T).tolist()
    re = r0.copy()
    ex = orc.compress_exact(g, re, [0, n], 0, 10000)
    assert set(ex.idx.tolist()) <= set(sp.idx.tolist())


def test_sampled_count_within_binomial_band(orc):
    rng = np.random.default_rng(5)
    n = 1 << 21
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    r = np.zeros(n, np.float32)
    sp = orc.compress_sampled(g, r, [0, n], 0, 10000, cap=n)
    kept = np.zeros(n, bool)
    kept[sp.idx] = True
    assert np.abs(g[kept]).min() > np.abs(g[~kept]).max()    # superlevel set
    s = orc.sample_count(n)
    p = 0.01
    rel_sigma = math.sqrt((1 - p) / (s * p))
    assert abs(sp.idx.size / (n * p) - 1) < 5 * rel_sigma + 2.0 / (s * p)


# The sampled-threshold mode of "Sparse Communication for Distributed Gradient
# Descent" (Abstract: a threshold found from a sample of the update) is defined
# in a method section the page no longer holds.  The reading fixed for it:
#   s  = min(m, max(sample_min, ceil(m / sample_div)))   samples per group,
#   i_j = floor((2j+1) m / (2s)), j = 0..s-1            systematic positions,
#   ks = ceil(s * ppm / 1e6); T = ks-th largest sampled |acc|; keep |acc| >= T.
# The literal values below are worked out by hand from that reading.
@pytest.mark.parametrize("m,div,smin,want", [
    (0, 1000, 65536, 0),                 # empty group
    (10, 1000, 65536, 10),               # m below sample_min: every element
    (65535, 1000, 65536, 65535),
    (65536, 1000, 65536, 65536),
    (65537, 1000, 65536, 65536),         # ceil(65537/1000) = 66 < sample_min
    (65536000, 1000, 65536, 65536),      # m/div = sample_min exactly
    (65536001, 1000, 65536, 65537),      # ceil(65536.001) = 65537
    (1 << 30, 1000, 65536, 1073742),     # ceil(1073741.824)
    (7, 3, 2, 3),                        # ceil(7/3) = 3 > 2
    (6, 3, 2, 2),                        # 6/3 = 2 exactly
    (999, 1000, 0, 1),                   # m < div: one sample
    (5, 10, 1, 1),
    (3000, 1000, 0, 3),
    (3001, 1000, 0, 4),
])
def test_sample_count_literal(orc, m, div, smin, want):
    assert orc.sample_count(m, div, smin) == want


def test_sampled_positions_literal_m10(orc):
    # m = 10, sample_div = 1000, sample_min = 4 -> s = min(10, max(4, 1)) = 4.
    # Positions floor((2j+1)*10/8): 10/8, 30/8, 50/8, 70/8 -> 1, 3, 6, 8.
    # Sampled |acc| = |-2|, |6|, |-4|, |5| = 2, 6, 4, 5; ppm 500000 -> ks =
    # ceil(4/2) = 2, so T = 5 (the 2nd largest) and every |acc| >= 5 is kept:
    # indices 0 (9), 2 (8), 3 (6), 4 (-7), 8 (5), 9 (-10).
    acc = np.array([9, -2, 8, 6, -7, 1, -4, 3, 5, -10], np.float32)
    r = np.zeros(10, np.float32)
    sp = orc.compress_sampled(acc, r, [0, 10], orc.GLOBAL, 500000, cap=10, sample_div=1000, sample_min=4)
    assert sp.idx.tolist() == [0, 2, 3, 4, 8, 9]
    assert sp.val.tolist() == [9, 8, 6, -7, 5, -10]
    assert sp.counts.tolist() == [6, 6]
    assert r.tolist() == [0, -2, 0, 0, 0, 1, -4, 3, 0, 0]
    assert sp.status == 0


def test_sampled_positions_literal_two_segments(orc):
    # Two tensors of 10 and 20 elements, sample_div = 1000, sample_min = 4.
    # Per tensor: tensor 0 as in the m = 10 case (positions 1, 3, 6, 8);
    # tensor 1 has s = 4 and positions floor((2j+1)*20/8) = 2, 7, 12, 17,
    # i.e. global 12, 17, 22, 27.  Over the whole vector (m = 30, s = 4):
    # floor((2j+1)*30/8) = 3, 11, 18, 26.
    a0 = [9, -2, 8, 6, -7, 1, -4, 3, 5, -10]
    a1 = [0.5, 7, -3, 0.25, 11, 2, 1, -6, 0.75, 4, 13, -1, 8, 9, -0.5, 1.5, 3.5, 2.5, 5, -12]
    acc = np.array(a0 + a1, np.float32)
    # Per tensor, ppm 500000 -> ks = 2.  Tensor 0: T = 5 -> local 0, 2, 3, 4, 8, 9.
    # Tensor 1 samples local 2, 7, 12, 17: |-3|, |-6|, |8|, |2.5| -> T = 6 ->
    # local |acc| >= 6: 1 (7), 4 (11), 7 (-6), 10 (13), 12 (8), 13 (9), 19 (-12)
    # -> global 11, 14, 17, 20, 22, 23, 29.
    r = np.zeros(30, np.float32)
    sp = orc.compress_sampled(acc, r, [0, 10, 30], orc.PER_SEGMENT, 500000, cap=30, sample_div=1000,
                              sample_min=4)
    assert sp.idx.tolist() == [0, 2, 3, 4, 8, 9, 11, 14, 17, 20, 22, 23, 29]
    assert sp.counts.tolist() == [6, 7, 13]
    # Globally: samples at 3, 11, 18, 26 -> |6|, |7|, |0.75|, |3.5|; ks = 2 -> T = 6 ->
    # every |acc| >= 6: 0, 2, 3, 4, 9 (tensor 0) and 11, 14, 17, 20, 22, 23, 29.
    r = np.zeros(30, np.float32)
    sp = orc.compress_sampled(acc, r, [0, 10, 30], orc.GLOBAL, 500000, cap=30, sample_div=1000, sample_min=4)
    assert sp.idx.tolist() == [0, 2, 3, 4, 9, 11, 14, 17, 20, 22, 23, 29]
    assert sp.counts.tolist() == [5, 7, 12]


def test_sampled_positions_literal_default_sizes(orc):
    # m = 100000 with the default sample_div = 1000, sample_min = 65536:
    # s = 65536, positions floor((2j+1)*100000/131072): j = 0 -> 0, j = 1 ->
    # floor(300000/131072) = 2, j = 65535 -> floor(99999.23...) = 99999.
    # Element 1 is not sampled (positions 0 and 2 bracket it).  With ppm = 1,
    # ks = ceil(65536/1e6) = 1, so T = the largest sampled |acc|.
    m = 100000
    acc = np.zeros(m, np.float32)
    acc[1] = 2.0        # not sampled: cannot raise T
    acc[2] = 1.0        # sampled (j = 1): T = 1.0
    acc[50000] = 0.5    # below T
    r = np.zeros(m, np.float32)
    sp = orc.compress_sampled(acc, r, [0, m], orc.GLOBAL, 1, cap=m)
    assert sp.idx.tolist() == [1, 2]
    # Only the last element sampled (j = 65535 -> 99999): T = |acc[99999]|.
    acc = np.zeros(m, np.float32)
    acc[99998] = 4.0    # floor((2*65534+1)*100000/131072) = 99997: not sampled
    acc[99999] = 3.0
    acc[7] = 3.5
    r = np.zeros(m, np.float32)
    sp = orc.compress_sampled(acc, r, [0, m], orc.GLOBAL, 1, cap=m)
    assert sp.idx.tolist() == [7, 99998, 99999]


def test_sampled_truncation_keeps_residual(orc):
    rng = np.random.default_rng(9)
    n = 10000
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    r = np.zeros(n, np.float32)
    full = orc.compress_sampled(g, r.copy(), [0, n], 0, 100000, cap=n, sample_min=n)
    cap = full.idx.size // 2
    r2 = np.zeros(n, np.float32)
    sp = orc.compress_sampled(g, r2, [0, n], 0, 100000, cap=cap, sample_min=n)
    assert sp.status & orc.STATUS_TRUNCATED
    assert sp.idx.tolist() == full.idx[:cap].tolist()
    rest = full.idx[cap:]
    assert np.array_equal(r2[rest], g[rest])
    assert np.all(r2[sp.idx] == 0)


# -------------------------------------------------------------- binarize
def _w1_sparse(orc):
    acc = np.array([0.5, -0.5, 0.25, -1.0, 0.5, 0.0], np.float32)
    r = np.zeros(6, np.float32)
    sp = orc.compress_exact(acc, r, [0, 6], orc.GLOBAL, 500000)
    return sp, r


def test_worked_example_sbc(orc):
    # Kept values 0.5 | -0.5, -1.0: mean+ = 0.5, mean- = 0.75 -> the negative side is sent
    # as one mean -0.75 ([SBC] §II Sparse Binarization), the rest returns to the residual.
    sp, r = _w1_sparse(orc)
    out = orc.binarize(sp, 1, orc.BIN_SBC, r)
    assert out.idx.tolist() == [1, 3]
    assert out.means.tolist() == [-0.75]
    assert out.counts.tolist() == [2, 2]
    assert r.tolist() == [0.5, 0.25, 0.25, -0.25, 0.5, 0.0]


def test_worked_example_2bit(orc):
    sp, r = _w1_sparse(orc)
    out = orc.binarize(sp, 1, orc.BIN_2BIT, r)
    codes = [(int(out.codes[0]) >> (2 * j)) & 3 for j in range(3)]
    assert codes == [1, 2, 2]
    assert out.means.tolist() == [0.5, -0.75]
    assert r.tolist() == [0.0, 0.25, 0.25, -0.25, 0.5, 0.0]


@settings(max_examples=150, deadline=None)
@given(vals=st.lists(st.floats(-4, 4, allow_nan=False, width=32), min_size=1, max_size=40),
       cut=st.integers(0, 40))
def test_sbc_means_are_exact_projections(orc, vals, cut):
    # The sent mean is the least-squares single value of its side ([SBC] appendix C projection):
    # compare with the exact rational mean rounded to fp32; the chosen side has the larger |mean|.
    v = np.array(vals, np.float32)
    n = v.size
    cut = min(cut, n)
    seg_off = np.array([0, cut, n], np.int64)
    sp = type("S", (), {})()
    sp.idx = np.arange(n, dtype=np.int32)
    sp.val = v
    sp.counts = np.array([cut, n - cut, n], np.int64)
    r = np.zeros(n, np.float32)
    out = orc.binarize(sp, 2, orc.BIN_SBC, r)
    e0 = 0
    for t in range(2):
        seg = v[seg_off[t]:seg_off[t + 1]]
        pos, neg = seg[seg > 0], seg[seg < 0]
        mp = float(np.float32(float(bf.exact_mean(pos)))) if pos.size else 0.0
        mn = float(np.float32(float(bf.exact_mean(-neg)))) if neg.size else 0.0
        sent = out.idx[e0:e0 + out.counts[t]]
        e0 += out.counts[t]
        if pos.size == 0 and neg.size == 0:
            assert sent.size == 0 and out.means[t] == 0
            continue
        m = float(out.means[t])
        side_pos = m > 0 or (m == 0 and pos.size > 0)
        exp = mp if side_pos else mn
        assert abs(abs(m) - exp) <= bf.ulp32(exp)
        other = mn if side_pos else mp
        assert abs(m) >= other - 2 * bf.ulp32(max(other, 1e-30))
        want_idx = seg_off[t] + np.flatnonzero(seg > 0 if side_pos else seg < 0)
        assert sent.tolist() == want_idx.tolist()
        # residuals: sent entries keep v - mean, the others get v back
        for i in range(seg_off[t], seg_off[t + 1]):
            want = np.float32(v[i] - np.float32(m)) if i in set(want_idx.tolist()) else v[i]
            assert r[i].view(np.uint32) == np.float32(want).view(np.uint32)
        # projection: the residual of the sent side sums to ~0
        if want_idx.size:
            res = sum(Fraction(float(v[i])) for i in want_idx) - want_idx.size * Fraction(m)
            assert abs(float(res)) <= want_idx.size * bf.ulp32(abs(m)) + 1e-30


# ------------------------------------------------------------------- Rice
def test_worked_example_rice_b2(orc):
    # positions [0, 5, 6, 20] -> gaps [0, 4, 0, 13]; b = 2 codes 000|1000|000|111010
    enc = orc.encode(np.array([0, 5, 6, 20], np.int32), np.array([4, 4], np.int64), [0, 32], orc.GLOBAL, 2)
    assert int(enc.nbits[0]) == 16
    assert enc.words.tolist() == [0x00005C08]
    assert enc.chunk_off.tolist() == [0, 0]


def test_worked_example_rice_b3(orc):
    # positions [3, 40] -> gaps [3, 36]; b = 3 codes 0110|11110001
    enc = orc.encode(np.array([3, 40], np.int32), np.array([2, 2], np.int64), [0, 64], orc.GLOBAL, 3)
    assert int(enc.nbits[0]) == 12
    assert enc.words.tolist() == [0x000008F6]


@settings(max_examples=200, deadline=None)
@given(data=st.data(), b=st.integers(0, 9), nseg=st.integers(1, 4), scope=st.sampled_from([0, 1]))
def test_rice_matches_bit_strings(orc, data, b, nseg, scope):
    sizes = [data.draw(st.integers(0, 700)) for _ in range(nseg)]
    seg_off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    n = int(seg_off[-1])
    sel = sorted(data.draw(st.sets(st.integers(0, max(n - 1, 0)), max_size=min(n, 300)))) if n else []
    idx = np.array(sel, np.int32)
    counts = np.array([sum(1 for i in sel if seg_off[t] <= i < seg_off[t + 1]) for t in range(nseg)] + [len(sel)],
                      np.int64)
    enc = orc.encode(idx, counts, seg_off, scope, b)
    streams = [(0, n, sel)] if scope == 0 else \
        [(int(seg_off[t]), int(seg_off[t + 1]), [i for i in sel if seg_off[t] <= i < seg_off[t + 1]])
         for t in range(nseg)]
    words = []
    chunks = []
    for s, (lo, hi, items) in enumerate(streams):
        local = [i - lo for i in items]
        bits = bf.rice_bits_string(local, b)
        assert int(enc.nbits[s]) == len(bits)
        assert int(enc.word_off[s]) == len(words)
        words += bf.pack_bits(bits)
        # chunk table: (bit offset, position reached) of every 256th code
        for c in range(0, len(local), orc.CHUNK_CODES):
            chunks.append(len(bf.rice_bits_string(local[:c], b)))
            chunks.append(local[c - 1] + 1 if c else 0)
        back, used = bf.parse_rice(bits, len(local), b)
        assert back == local and used == len(bits)
        # oracle decoder agrees
        w0, w1 = int(enc.word_off[s]), int(enc.word_off[s + 1])
        pos, stt = orc.decode_stream(enc.words[w0:w1], int(enc.nbits[s]), len(local), b, hi - lo)
        assert stt == 0 and pos.tolist() == local
    assert enc.words.tolist() == words
    assert enc.chunk_off.tolist() == chunks


def test_rice_size_bound(orc):
    # bits <= k (b+1) + floor((n-k)/2^b): the sum of floor(z/2^b) is at most floor(sum z / 2^b).
    rng = np.random.default_rng(1)
    for b in (0, 3, 6, 9):
        n = 50000
        pos = np.flatnonzero(rng.random(n) < 0.02).astype(np.int32)
        enc = orc.encode(pos, np.array([pos.size, pos.size], np.int64), [0, n], 0, b)
        assert int(enc.nbits[0]) <= pos.size * (b + 1) + ((n - pos.size) >> b)


def test_decode_detects_corruption(orc):
    pos = np.array([2, 9, 40, 41, 300], np.int32)
    enc = orc.encode(pos, np.array([5, 5], np.int64), [0, 512], 0, 3)
    nb = int(enc.nbits[0])
    _, st = orc.decode_stream(enc.words, nb, 5, 3, 512)
    assert st == 0
    _, st = orc.decode_stream(enc.words, nb - 2, 5, 3, 512)        # truncated stream
    assert st & orc.STATUS_CORRUPT
    _, st = orc.decode_stream(enc.words, nb, 5, 3, 200)             # position beyond the shape
    assert st & orc.STATUS_CORRUPT
    _, st = orc.decode_stream(enc.words, nb, 4, 3, 512)             # bits left over
    assert st & orc.STATUS_CORRUPT
    _, st = orc.decode_stream(enc.words, nb, 5, 3, 512, chunk_off=np.array([1, 0], np.uint64))
    assert st & orc.STATUS_CORRUPT
    _, st = orc.decode_stream(enc.words, nb, 5, 3, 512, chunk_off=np.array([0, 1], np.uint64))
    assert st & orc.STATUS_CORRUPT
    _, st = orc.decode_stream(enc.words, nb, 5, 3, 512, chunk_off=np.array([0, 0], np.uint64))
    assert st == 0


# ------------------------------------------------------ decode + accumulate
def _random_message(orc, rng, n, seg_off, ppm, g_scale=1e-3):
    g = rng.laplace(0, g_scale, n).astype(np.float32)
    r = np.zeros(n, np.float32)
    return orc.compress_exact(g, r, seg_off, 0, ppm), g


def test_single_raw_message_densifies(orc):
    rng = np.random.default_rng(2)
    n = 3000
    sp, _ = _random_message(orc, rng, n, [0, n], 50000)
    out = np.zeros(n, np.float32)
    st = orc.decode_accumulate([orc.Message(sp.counts, idx=sp.idx, val=sp.val)], [0, n], out)
    want = np.zeros(n, np.float32)
    want[sp.idx] = sp.val
    assert st == 0 and np.array_equal(out.view(np.uint32), want.view(np.uint32))


def test_ordered_sum_equals_dense_numpy(orc):
    # [SBC] §I (server / all-reduce sum) with [AHB19] Abstract (local dense gradient as base):
    # out = base + densify(m0) + ... added in worker order, present entries only.
    rng = np.random.default_rng(4)
    seg = [0, 700, 701, 4000]
    n = seg[-1]
    base = rng.normal(0, 1e-3, n).astype(np.float32)
    base[::97] = -0.0
    msgs, dense = [], []
    for w in range(5):
        sp, _ = _random_message(orc, rng, n, seg, 30000)
        if w % 2:
            enc = orc.encode(sp.idx, sp.counts, seg, 1, 4)
            msgs.append(orc.Message(sp.counts, golomb=True, scope=1, b=4, val=sp.val, enc=enc))
        else:
            msgs.append(orc.Message(sp.counts, idx=sp.idx, val=sp.val))
        dense.append(sp)
    out = base.copy()
    st = orc.decode_accumulate(msgs, seg, out)
    want = base.copy()
    for sp in dense:
        m = np.zeros(n, bool)
        m[sp.idx] = True
        d = np.zeros(n, np.float32)
        d[sp.idx] = sp.val
        want[m] = want[m] + d[m]
    assert st == 0 and np.array_equal(out.view(np.uint32), want.view(np.uint32))
    # absent entries keep the base bits (including -0.0)
    untouched = np.ones(n, bool)
    for sp in dense:
        untouched[sp.idx] = False
    assert np.array_equal(out[untouched].view(np.uint32), base[untouched].view(np.uint32))


def test_sbc_and_2bit_messages_round_trip(orc):
    rng = np.random.default_rng(8)
    seg = np.array([0, 1000, 1064, 5000], np.int64)
    n = int(seg[-1])
    g = rng.laplace(0, 1e-3, n).astype(np.float32)
    r = np.zeros(n, np.float32)
    sp = orc.compress_exact(g, r, seg, 1, 20000)
    r_sbc = r.copy()
    sbc = orc.binarize(sp, 3, orc.BIN_SBC, r_sbc)
    enc = orc.encode(sbc.idx, sbc.counts, seg, 1, 5)
    out = np.zeros(n, np.float32)
    st = orc.decode_accumulate([orc.Message(sbc.counts, vkind=orc.VAL_SBC, golomb=True, scope=1, b=5,
                                            means=sbc.means, enc=enc)], seg, out)
    assert st == 0
    e0 = 0
    for t in range(3):
        ids = sbc.idx[e0:e0 + sbc.counts[t]]
        e0 += sbc.counts[t]
        assert np.all(out[ids] == sbc.means[t])
    assert np.count_nonzero(out) == sbc.idx.size
    # sent + residual == acc within one rounding per entry
    acc = g
    rec = (r_sbc + out).astype(np.float32)
    assert np.all(np.abs(rec - acc) <= np.spacing(np.abs(acc)) + 1e-45)
    # 2-bit
    r2 = r.copy()
    q = orc.binarize(sp, 3, orc.BIN_2BIT, r2)
    out2 = np.zeros(n, np.float32)
    st = orc.decode_accumulate([orc.Message(q.counts, vkind=orc.VAL_2BIT, idx=q.idx, codes=q.codes,
                                            means=q.means)], seg, out2)
    assert st == 0
    assert set(np.unique(out2[sp.idx]).tolist()) <= set(q.means.tolist())
    assert np.all(np.sign(out2[sp.idx]) == np.sign(sp.val))


def test_sbc_equal_means_send_positive_side(orc):
    # Reading of [SBC] §II Sparse Binarization when both means are equal: the positive side is sent.
    sp = type("S", (), {})()
    sp.idx = np.array([0, 1, 2, 3], np.int32)
    sp.val = np.array([0.5, -0.25, -0.75, 0.5], np.float32)
    sp.counts = np.array([4, 4], np.int64)
    r = np.zeros(4, np.float32)
    out = orc.binarize(sp, 1, orc.BIN_SBC, r)
    assert out.means.tolist() == [0.5] and out.idx.tolist() == [0, 3]
    assert r.tolist() == [0.0, -0.25, -0.75, 0.0]


# ------------------------------------------------------------- warm-up
# [SBC] appendix A (Warm-up Training): the kept fraction falls exponentially
# from 25% to 0.1% over the first epochs.  Reading: geometric interpolation
# in kept parts per million over the warm-up steps, rounded to the nearest
# integer.  Literal values from 250000 * 0.004^(t/(T-1)) evaluated in 60-digit
# decimal arithmetic (none lies near a rounding boundary):
WARMUP_6 = [250000, 82861, 27464, 9103, 3017, 1000]            # 82861.35, 27464.01, 9102.82, 3017.09
WARMUP_20 = [250000, 186953, 139806, 104549, 78183, 58466, 43722, 32696, 24450, 18284,
             13673, 10225, 7646, 5718, 4276, 3198, 2391, 1788, 1337, 1000]


def test_warmup_schedule_literal(orc):
    assert [orc.warmup_ppm(t, 6) for t in range(6)] == WARMUP_6
    assert [orc.warmup_ppm(t, 20) for t in range(20)] == WARMUP_20
    # after the warm-up the kept fraction stays at its end value
    assert orc.warmup_ppm(6, 6) == orc.warmup_ppm(1000, 6) == 1000
    assert orc.warmup_ppm(0, 1) == 1000
    assert orc.warmup_ppm(3, 7, 1000, 1000) == 1000
    assert orc.warmup_ppm(-1, 6) == -1 and orc.warmup_ppm(0, 0) == -1 and orc.warmup_ppm(0, 6, 0, 1000) == -1


def test_warmup_schedule_is_geometric(orc):
    # consecutive ratios are constant up to the rounding of each term
    for T in (6, 20, 50):
        ps = [orc.warmup_ppm(t, T) for t in range(T)]
        r = (1000 / 250000) ** (1 / (T - 1))
        for a, b in zip(ps, ps[1:]):
            assert abs(b - a * r) <= 0.5 + 0.5 * r + 1e-9
        assert all(b < a for a, b in zip(ps, ps[1:]))
