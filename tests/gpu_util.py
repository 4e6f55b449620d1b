"""Helpers of the GPU parity tests: host <-> device copies and bitwise compares."""
from __future__ import annotations

import sys

import numpy as np
import torch


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bits(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a


def assert_bitwise(got, want, what: str):
    got, want = bits(got), bits(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    if not np.array_equal(got, want):
        bad = np.flatnonzero(got != want)
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} mismatches, first at {i}: got {got[i]!r} want {want[i]!r}")


def announce(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()
