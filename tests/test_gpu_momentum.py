"""GPU parity of compress with momentum correction and masking against the oracle.

[SBC] appendix A (Momentum Correction, Warm-up Training and Momentum Masking):
u <- beta*u + g goes into the residual, and the momentum of sent entries is
zeroed.  Each case runs several steps carrying both the residual and the
momentum, and compares indices, values, counts, residual and momentum
bitwise: exact and sampled modes, both scopes, ragged segments, tiles whose
candidate regions overflow (the redo path), inputs that defeat the probe (the
full-pass path), accumulate-only, a stale workspace, and beta = 0.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu


def run_steps(orc, layout, grads, beta, *, mode=sgc.EXACT, scope=0, ppm=10000, cap=None, u0=None, r0=None,
              what="", ws_fill=None, path=sgc.PATH_AUTO):
    """Step both sides through `grads`; returns the last status word."""
    n = layout.n
    u = np.zeros(n, np.float32) if u0 is None else u0.copy()
    r = np.zeros(n, np.float32) if r0 is None else r0.copy()
    ud, rd = dev(u), dev(r)
    seg_off = np.array(layout.seg_off, np.int64)
    st = 0
    for s, g in enumerate(grads):
        announce(f"momentum {what} step {s} n={n} nseg={layout.nseg} mode={mode} scope={scope} ppm={ppm} beta={beta} "
                 f"path={path}")
        ws = None
        if ws_fill is not None:
            opts = sgc.CompressOpts(mode, scope, ppm, 1000, 65536, path)
            c = cap if cap is not None else layout.keep_total(scope, ppm)
            nbytes = sgc.lib().sgc_compress_momentum_workspace(layout.handle, C.byref(opts), c)
            ws = torch.full((nbytes,), ws_fill, dtype=torch.uint8, device="cuda")
        out = sgc.compress_momentum(layout, dev(g), ud, rd, beta, mode=mode, scope=scope, keep_ppm=ppm, cap=cap,
                                    ws=ws, path=path)
        torch.cuda.synchronize()
        ref = orc.compress_momentum(g, u, r, beta, seg_off, scope, ppm, sampled=(mode == sgc.SAMPLED), cap=out.cap)
        counts = host(out.counts)
        total = int(counts[-1])
        assert_bitwise(counts, ref.counts, f"{what} s{s} counts")
        assert_bitwise(host(out.idx)[:total], ref.idx, f"{what} s{s} idx")
        assert_bitwise(host(out.val)[:total], ref.val, f"{what} s{s} val")
        assert_bitwise(host(rd), r, f"{what} s{s} residual")
        assert_bitwise(host(ud), u, f"{what} s{s} momentum")
        st = int(host(out.status)[0])
    return st


@pytest.mark.parametrize("path", [sgc.PATH_GATHER, sgc.PATH_WINDOW], ids=["gather", "window"])
@pytest.mark.parametrize("scope", [0, 1])
@pytest.mark.parametrize("ppm", [1000, 10000, 250000])
def test_exact_ragged_steps(orc, scope, ppm, path):
    rng = np.random.default_rng(21)
    layout = sgc.Layout([1 << 20, 300001, 4096, 1, 0, 99999])
    grads = [rng.laplace(0, 1e-3, layout.n).astype(np.float32) for _ in range(3)]
    run_steps(orc, layout, grads, 0.9, scope=scope, ppm=ppm, path=path, what=f"exact ppm{ppm}")


@pytest.mark.parametrize("path", [sgc.PATH_GATHER, sgc.PATH_WINDOW], ids=["gather", "window"])
@pytest.mark.parametrize("scope", [0, 1])
def test_sampled_steps(orc, scope, path):
    rng = np.random.default_rng(22)
    layout = sgc.Layout([1 << 20, 300000, 4096, 1, 99999])
    grads = [rng.laplace(0, 1e-3, layout.n).astype(np.float32) for _ in range(3)]
    run_steps(orc, layout, grads, 0.9, mode=sgc.SAMPLED, scope=scope, ppm=10000, path=path, what="sampled")


@pytest.mark.parametrize("mode", [sgc.EXACT, sgc.SAMPLED])
def test_many_segments_per_tensor(orc, mode):
    # 2100 tensors (every seventh empty), per-tensor selection: the per-segment bookkeeping
    # runs in several rounds of its workgroup; three steps carry residual and momentum
    rng = np.random.default_rng(23)
    sizes = [int(x) for x in rng.integers(0, 3000, 2100)]
    for t in range(0, len(sizes), 7):
        sizes[t] = 0
    layout = sgc.Layout(sizes)
    grads = [rng.laplace(0, 1e-3, layout.n).astype(np.float32) for _ in range(3)]
    run_steps(orc, layout, grads, 0.9, mode=mode, scope=1, ppm=20000, what="2100 tensors")


def test_sampled_truncation_keeps_momentum(orc):
    rng = np.random.default_rng(23)
    n = 500000
    layout = sgc.Layout([n])
    grads = [rng.laplace(0, 1e-3, n).astype(np.float32) for _ in range(2)]
    st = run_steps(orc, layout, grads, 0.5, mode=sgc.SAMPLED, ppm=10000, cap=3000, what="truncated")
    assert st & sgc.STATUS_TRUNCATED


def test_clustered_overflowing_tiles(orc):
    # contiguous runs of large values: some tiles hold more candidates than their region and are
    # redone from r and u (which pass 1 leaves as acc and u' there)
    n = 1 << 21
    rng = np.random.default_rng(24)
    g = rng.normal(0, 1e-5, n).astype(np.float32)
    for start in (5000, 300000, 1500007):
        g[start:start + 9000] = rng.laplace(0, 1.0, 9000).astype(np.float32)
    layout = sgc.Layout([n // 2, n // 2])
    u0 = rng.normal(0, 1e-3, n).astype(np.float32)
    for scope in (0, 1):
        run_steps(orc, layout, [g, g * np.float32(0.5)], 0.9, scope=scope, u0=u0, what=f"clustered scope{scope}")
        run_steps(orc, layout, [g], 0.9, mode=sgc.SAMPLED, scope=scope, cap=n, u0=u0, what=f"clustered sampled{scope}")


def test_probe_defeated_takes_full_pass_path(orc):
    # large values exactly where the probe reads: fewer than k candidates, full passes over r
    n = 1 << 20
    g = np.random.default_rng(25).normal(0, 1e-4, n).astype(np.float32)
    runs = (2048 + 4096 * np.arange(n // 4096))[:, None] + np.arange(16)[None, :]
    g[runs.ravel()] = 1.0 + np.arange(runs.size, dtype=np.float32) * 1e-3
    layout = sgc.Layout([n])
    st = run_steps(orc, layout, [g], 0.9, what="probe defeated")
    assert st & sgc.STATUS_DENSE_PATH


def test_beta_zero_and_negative(orc):
    rng = np.random.default_rng(26)
    layout = sgc.Layout([200000, 77777])
    grads = [rng.laplace(0, 1e-3, layout.n).astype(np.float32) for _ in range(2)]
    u0 = rng.normal(0, 1e-3, layout.n).astype(np.float32)
    run_steps(orc, layout, grads, 0.0, u0=u0, what="beta 0")
    run_steps(orc, layout, grads, -0.25, u0=u0, what="beta -0.25")


def test_accumulate_only(orc):
    rng = np.random.default_rng(27)
    for n in (1, 3, 4, 1023, 1 << 20, (1 << 20) + 7):
        layout = sgc.Layout([n])
        g = rng.laplace(0, 1e-3, n).astype(np.float32)
        u = rng.normal(0, 1e-3, n).astype(np.float32)
        r = rng.laplace(0, 1e-3, n).astype(np.float32)
        ud, rd = dev(u), dev(r)
        announce(f"momentum accumulate-only n={n}")
        sgc.compress_momentum(layout, dev(g), ud, rd, 0.9, mode=sgc.ACCUMULATE_ONLY)
        orc.momentum_correct(0.9, g, u)
        orc.accumulate(u, r)
        torch.cuda.synchronize()
        assert_bitwise(host(ud), u, f"accumulate n={n} momentum")
        assert_bitwise(host(rd), r, f"accumulate n={n} residual")


@pytest.mark.parametrize("fill", [0x00, 0xFF])
def test_stale_workspace(orc, fill):
    rng = np.random.default_rng(28)
    layout = sgc.Layout([300000, 4097, 1 << 20])
    grads = [rng.laplace(0, 1e-3, layout.n).astype(np.float32) for _ in range(2)]
    for scope in (0, 1):
        run_steps(orc, layout, grads, 0.9, scope=scope, ws_fill=fill, what=f"stale {fill:#x}")


def test_argument_errors():
    layout = sgc.Layout([1000])
    g = torch.zeros(1000, device="cuda")
    u = torch.zeros(1000, device="cuda")
    r = torch.zeros(1000, device="cuda")
    opts = sgc.CompressOpts(sgc.EXACT, 0, 10000, 1000, 65536)
    lib = sgc.lib()
    nbytes = lib.sgc_compress_momentum_workspace(layout.handle, C.byref(opts), 10)
    assert nbytes > lib.sgc_compress_workspace(layout.handle, C.byref(opts), 10)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    idx = torch.empty(10, dtype=torch.int32, device="cuda")
    val = torch.empty(10, device="cuda")
    cnt = torch.empty(2, dtype=torch.int64, device="cuda")
    p = lambda t: C.c_void_p(t.data_ptr())
    call = lambda beta, uu: lib.sgc_compress_momentum(layout.handle, C.byref(opts), beta, p(g), uu, p(r), p(idx),
                                                      p(val), 10, p(cnt), None, p(ws), nbytes, None)
    assert call(float("nan"), p(u)) == sgc.EINVAL
    assert call(float("inf"), p(u)) == sgc.EINVAL
    assert call(0.9, None) == sgc.EINVAL
    assert call(0.9, C.c_void_p(u.data_ptr() + 4)) == sgc.EINVAL
