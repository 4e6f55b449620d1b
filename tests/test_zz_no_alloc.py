"""sgc_compress_noalloc -- the compress step with the library's own scratch
buffer, for callers that cannot allocate -- against sgc_compress on the same
state: two calls in a row, the second on a smaller input (the scratch
buffer keeps the first call's contents), bitwise in every output.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
import workloads as W
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu


def _both(layout, g, r0, **kw):
    """The same step through sgc_compress and sgc_compress_noalloc, from the same residual."""
    ra, rb = dev(r0), dev(r0)
    gd = dev(g)
    a = sgc.compress(layout, gd, ra, **kw)
    b = sgc.compress_noalloc(layout, gd, rb, **kw)
    torch.cuda.synchronize()
    return a, ra, b, rb


def _same(a, ra, b, rb, what):
    total = int(host(a.counts)[-1])
    assert_bitwise(host(b.counts), host(a.counts), f"{what}: counts")
    assert_bitwise(host(b.idx)[:total], host(a.idx)[:total], f"{what}: idx")
    assert_bitwise(host(b.val)[:total], host(a.val)[:total], f"{what}: val")
    assert_bitwise(host(rb), host(ra), f"{what}: residual")
    assert_bitwise(host(b.status), host(a.status), f"{what}: status")
    return total


def test_noalloc_equals_compress_two_calls():
    rng = np.random.default_rng(2024)
    # call 1: the MNIST MLP layout (20.0M elements, 6 tensors), global exact top-1%,
    # from a nonzero residual
    w = W.MLP_MNIST
    big = sgc.Layout(w.seg_numel)
    g = W.gradient(w, 0, 0).numpy()
    r0 = (rng.normal(0, 5e-3, big.n) * (rng.random(big.n) < 0.3)).astype(np.float32)
    announce("no-alloc call 1: mlp-mnist 20.0M, exact global top-1%")
    a, ra, b, rb = _both(big, g, r0, keep_ppm=w.keep_ppm)
    assert _same(a, ra, b, rb, "call 1") == big.keep_total(sgc.GLOBAL, w.keep_ppm)
    # call 2: a smaller, ragged layout, sampled per-tensor top-2% (the scratch
    # buffer still holds call 1's candidates, histograms and counters)
    small = sgc.Layout([300001, 17, 0, 700003, 4096])
    g2 = rng.laplace(0, 1e-3, small.n).astype(np.float32)
    r2 = (rng.normal(0, 1e-3, small.n) * (rng.random(small.n) < 0.5)).astype(np.float32)
    announce("no-alloc call 2: 1.0M ragged, sampled per-tensor top-2%")
    a, ra, b, rb = _both(small, g2, r2, mode=sgc.SAMPLED, scope=sgc.PER_SEGMENT, keep_ppm=20000)
    assert _same(a, ra, b, rb, "call 2") > 0
    # call 3: smaller again, exact per tensor, the hold flag
    tiny = sgc.Layout([5000, 3, 2000])
    g3 = rng.laplace(0, 1e-3, tiny.n).astype(np.float32)
    announce("no-alloc call 3: 7003 elements, exact per-tensor top-10%, hold")
    a, ra, b, rb = _both(tiny, g3, np.zeros(tiny.n, np.float32), scope=sgc.PER_SEGMENT, keep_ppm=100000,
                         hold=True)
    _same(a, ra, b, rb, "call 3")


def test_noalloc_refuses_beyond_scratch_and_accumulates():
    lib = sgc.lib()
    # 2^27 elements at top-10% needs far more workspace than the scratch buffer:
    # refused before any GPU work (the stand-in pointers are never touched)
    lay = sgc.Layout([1 << 27])
    o = sgc.CompressOpts(sgc.EXACT, sgc.GLOBAL, 100000, 1000, 65536)
    k = lay.keep_total(sgc.GLOBAL, 100000)
    assert lib.sgc_compress_workspace(lay.handle, C.byref(o), k) > sgc.NOALLOC_SCRATCH_BYTES
    A = C.c_void_p(4096)
    assert lib.sgc_compress_noalloc(lay.handle, C.byref(o), A, A, A, A, k, A, None, None) == sgc.ENOSPC
    assert lib.sgc_compress_noalloc(None, C.byref(o), A, A, A, A, k, A, None, None) == sgc.EINVAL
    # accumulate-only mode needs no workspace at all
    small = sgc.Layout([1000, 23])
    g = torch.randn(small.n, device="cuda")
    r = torch.randn(small.n, device="cuda")
    want = (r + g).cpu()
    sgc.compress_noalloc(small, g, r, mode=sgc.ACCUMULATE_ONLY)
    torch.cuda.synchronize()
    assert_bitwise(host(r), want.numpy(), "accumulate-only")
