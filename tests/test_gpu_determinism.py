"""Results do not depend on what the caller's workspace held.

Every call is made on the same inputs with its workspace zeroed, filled
with 0x5a bytes (large positive integers, huge floats) and filled with 0xff
bytes (-1 integers, NaNs).  The outputs (their valid parts), the residual
and the status words must be identical bytes.  A kernel that
read workspace memory no earlier kernel of the call had written would show
up here as a difference (or as a mismatch against the oracle elsewhere only
by luck of the allocator's contents).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import compressed_sgd_amd as sgc
from codec_util import make_messages
from gpu_util import announce, assert_bitwise, dev, host

pytestmark = pytest.mark.gpu

SIZES = [300000, 5, 0, 1 << 20, 77777, 4096]
FILLS = (0x00, 0x5A, 0xFF)


def _ws(nbytes: int, fill: int) -> torch.Tensor:
    return torch.full((max(nbytes, 256),), fill, dtype=torch.uint8, device="cuda")


def _chunk_entries(layout, counts: np.ndarray, scope: int) -> int:
    per = [int(counts[-1])] if scope == sgc.GLOBAL else np.diff(counts[:layout.nseg + 1]).tolist()
    return 2 * sum((c + sgc.CHUNK_CODES - 1) // sgc.CHUNK_CODES for c in per)


def _compress_encode(layout, g, r0, fill, mode, scope, ppm, path, b):
    r = r0.clone()
    copts = dict(mode=mode, scope=scope, keep_ppm=ppm, path=path)
    outs = []
    for step in range(2):  # a carried residual: the second step starts from the first's
        nb = sgc.compress_workspace_bytes(layout, **copts)
        comp = sgc.compress(layout, g[step], r, ws=_ws(nb, fill), **copts)
        enc = sgc.encode(layout, comp.idx, comp.counts, comp.cap, scope=scope, b=b,
                         ws=_ws(sgc.encode_workspace_bytes(layout, scope, comp.cap), fill))
        torch.cuda.synchronize()
        counts = host(comp.counts)
        total = int(counts[-1])
        word_off = host(enc.word_off).view(np.uint64)
        outs.append({
            "counts": counts, "idx": host(comp.idx[:total]), "val": host(comp.val[:total]),
            "status": host(comp.status), "word_off": word_off, "nbits": host(enc.nbits),
            "words": host(enc.words[:int(word_off[-1])]),
            "chunk_off": host(enc.chunk_off[:_chunk_entries(layout, counts, scope)]),
            "enc_status": host(enc.status), "residual": host(r),
        })
    return outs


@pytest.mark.parametrize("path", [sgc.PATH_GATHER, sgc.PATH_WINDOW], ids=["gather", "window"])
@pytest.mark.parametrize("mode,scope,ppm", [(sgc.EXACT, sgc.GLOBAL, 10000), (sgc.EXACT, sgc.PER_SEGMENT, 10000),
                                            (sgc.EXACT, sgc.GLOBAL, 250000), (sgc.SAMPLED, sgc.GLOBAL, 1000)],
                         ids=["exact-global-1pct", "exact-pertensor-1pct", "exact-global-25pct",
                              "sampled-global-0.1pct"])
def test_compress_encode_independent_of_workspace(path, mode, scope, ppm):
    layout = sgc.Layout(SIZES)
    n = layout.n
    rng = np.random.default_rng(71)
    g = [dev(rng.laplace(0, 1e-3, n).astype(np.float32)) for _ in range(2)]
    r0 = dev(rng.normal(0, 1e-4, n).astype(np.float32))
    b = sgc.rice_param(ppm / 1e6)
    announce(f"workspace independence: compress+encode path={path} mode={mode} scope={scope} ppm={ppm}")
    runs = [_compress_encode(layout, g, r0, fill, mode, scope, ppm, path, b) for fill in FILLS]
    for fill, a in zip(FILLS[1:], runs[1:]):
        for step in range(2):
            for key in a[step]:
                assert_bitwise(a[step][key], runs[0][step][key], f"fill {fill:#x} step {step} {key}")
    for step in range(2):
        assert int(runs[0][step]["status"][0]) & ~int(sgc.STATUS_DENSE_PATH) == 0


def test_binarize_independent_of_workspace():
    layout = sgc.Layout(SIZES)
    n = layout.n
    rng = np.random.default_rng(72)
    g = dev(rng.laplace(0, 1e-3, n).astype(np.float32))
    for mode in (sgc.BIN_SBC, sgc.BIN_2BIT):
        res = []
        for fill in FILLS:
            announce(f"workspace independence: binarize mode={mode} fill={fill:#x}")
            r = torch.zeros(n, dtype=torch.float32, device="cuda")
            comp = sgc.compress(layout, g, r, scope=sgc.PER_SEGMENT, keep_ppm=10000)
            bn = sgc.binarize(layout, comp, r, mode, ws=_ws(sgc.binarize_workspace_bytes(layout, comp.cap), fill))
            torch.cuda.synchronize()
            counts = host(bn.counts)
            total = int(counts[-1])
            out = {"counts": counts, "means": host(bn.means), "residual": host(r)}
            if mode == sgc.BIN_SBC:
                out["idx"] = host(bn.idx[:total])
            else:
                out["codes"] = host(bn.codes[:(total + 15) // 16])
            res.append(out)
        for fill, r in zip(FILLS[1:], res[1:]):
            for key in res[0]:
                assert_bitwise(r[key], res[0][key], f"binarize mode={mode} fill {fill:#x} {key}")


@pytest.mark.parametrize("init", [sgc.INIT_ZERO, sgc.INIT_BASE])
def test_decode_accumulate_independent_of_workspace(orc, init):
    # per-tensor streams that end and start inside one output tile, empty
    # tensors, raw and coded messages in one batch
    layout = sgc.Layout(SIZES + [3, 0, 9000, 1, 200000])
    n = layout.n
    rng = np.random.default_rng(73)
    kinds = ["golomb_f32_seg", "raw_f32", "golomb_sbc", "golomb_f32", "raw_2bit", "golomb_2bit", "golomb_f32_seg"]
    gm, _ = make_messages(orc, layout, rng, kinds)
    base = dev(rng.normal(0, 1e-3, n).astype(np.float32))
    nb = sgc.decode_accumulate_workspace_bytes(layout, gm)
    outs = []
    for fill in FILLS:
        announce(f"workspace independence: decode_accumulate W={len(gm)} init={init} fill={fill:#x}")
        out = torch.zeros(n, dtype=torch.float32, device="cuda")
        st = sgc.decode_accumulate(layout, gm, out, init=init, base=base, ws=_ws(nb, fill))
        torch.cuda.synchronize()
        outs.append((host(out), host(st)))
    for fill, (o, st) in zip(FILLS, outs):
        assert int(st[0]) == 0, f"fill {fill:#x}: status {int(st[0])}"
        assert_bitwise(o, outs[0][0], f"decode_accumulate init={init} fill {fill:#x}")
