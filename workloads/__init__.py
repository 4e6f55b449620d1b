"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds NO arithmetic of the compression method: it only describes
the parameter-tensor shapes of the workloads the pages train on and draws
seeded synthetic gradients of the stated distributions.  Both the HIP path
and the CPU oracle consume the exact bytes drawn here.

Workloads (the models stand in for the pages' datasets and trained weights,
which are not needed: only tensor shapes and gradient statistics matter):

* ``flat-1M``     one flat fp32 tensor of 2^20 elements ~ Laplace(0, 1e-3),
                  drop ratio 99%, 3 steps.
* ``mlp-mnist``   the 3-layer MNIST MLP of "Sparse Communication for
                  Distributed Gradient Descent" (Introduction): 784x4096,
                  4096x4096, 4096x10 weights plus biases, ~ Normal(0, 1e-2);
                  global top-1%, 2-bit quantization, 4 workers, 10 steps.
* ``nmt-rnn``     an NMT RNN of the same page (Introduction: three large
                  embedding matrices dominate, only rows of words seen in the
                  batch are nonzero): three 50000x512 embeddings with ~2000
                  Zipf(1.1) rows ~ Laplace(0, 1e-3), 20 recurrent 1024x1024
                  ~ Normal(0, 1e-4); global top-1%, 4 workers + local.
* ``resnet50``    the 161 parameter tensors of ResNet-50 (the "Sparse Binary
                  Compression" testbed, Networks and Datasets), registration
                  order, ~ Laplace(0, 1e-3) / sqrt(fan_in) (1-D unscaled);
                  delay 8, per-tensor top-0.1%, SBC, Rice, 8 workers.
* ``flat-1G``     one flat tensor of 2^30 elements: 99% ~ Normal(0, 1e-4),
                  1% ~ Laplace(0, 1e-2); top-0.1% and top-1%, 16 workers.

Laplace(0, beta) uses beta as the scale (std = sqrt(2) beta), drawn as
beta * (E1 - E2) with E1, E2 ~ Exp(1); Normal(0, sigma) uses sigma as the std.
Seed rule: seed = 1_000_000 * workload_id + 1_000 * worker + step.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import torch

GLOBAL = 0
PER_SEGMENT = 1


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    tensors: Tuple[Tuple[str, Tuple[int, ...]], ...]
    keep_ppm: int
    scope: int
    workers: int
    steps: int
    delay: int = 1
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def seg_numel(self) -> List[int]:
        return [math.prod(s) for _, s in self.tensors]

    @property
    def numel(self) -> int:
        return sum(self.seg_numel)

    @property
    def seg_off(self) -> List[int]:
        off = [0]
        for m in self.seg_numel:
            off.append(off[-1] + m)
        return off


def resnet50_tensors() -> List[Tuple[str, Tuple[int, ...]]]:
    """Parameter tensors of torchvision's resnet50 in registration order."""
    t: List[Tuple[str, Tuple[int, ...]]] = [
        ("conv1.weight", (64, 3, 7, 7)), ("bn1.weight", (64,)), ("bn1.bias", (64,))]
    inplanes = 64
    for li, (planes, blocks) in enumerate([(64, 3), (128, 4), (256, 6), (512, 3)], 1):
        for bi in range(blocks):
            p = f"layer{li}.{bi}."
            t += [(p + "conv1.weight", (planes, inplanes, 1, 1)),
                  (p + "bn1.weight", (planes,)), (p + "bn1.bias", (planes,)),
                  (p + "conv2.weight", (planes, planes, 3, 3)),
                  (p + "bn2.weight", (planes,)), (p + "bn2.bias", (planes,)),
                  (p + "conv3.weight", (planes * 4, planes, 1, 1)),
                  (p + "bn3.weight", (planes * 4,)), (p + "bn3.bias", (planes * 4,))]
            if bi == 0:
                t += [(p + "downsample.0.weight", (planes * 4, inplanes, 1, 1)),
                      (p + "downsample.1.weight", (planes * 4,)),
                      (p + "downsample.1.bias", (planes * 4,))]
            inplanes = planes * 4
    t += [("fc.weight", (1000, 2048)), ("fc.bias", (1000,))]
    return t


FLAT_1M = Workload("flat-1M", 0, (("flat", (1 << 20,)),), 10000, GLOBAL, 1, 3)
MLP_MNIST = Workload(
    "mlp-mnist", 1,
    (("W1", (784, 4096)), ("b1", (4096,)), ("W2", (4096, 4096)), ("b2", (4096,)),
     ("W3", (4096, 10)), ("b3", (10,))),
    10000, GLOBAL, 4, 10)
NMT_RNN = Workload(
    "nmt-rnn", 2,
    tuple([("E_src", (50000, 512)), ("E_tgt_in", (50000, 512)), ("E_tgt_out", (50000, 512))]
          + [(f"R{i}", (1024, 1024)) for i in range(1, 21)]),
    10000, GLOBAL, 4, 3, extra={"rows": 2000, "zipf": 1.1})
RESNET50 = Workload("resnet50", 3, tuple(resnet50_tensors()), 1000, PER_SEGMENT, 8, 2, delay=8)
FLAT_1G = Workload("flat-1G", 4, (("flat", (1 << 30,)),), 1000, GLOBAL, 16, 3)

WORKLOADS = {w.name: w for w in (FLAT_1M, MLP_MNIST, NMT_RNN, RESNET50, FLAT_1G)}


def seed_of(w: Workload, worker: int, step: int) -> int:
    return 1_000_000 * w.wid + 1_000 * worker + step


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def laplace(n: int, beta: float, gen: torch.Generator, device) -> torch.Tensor:
    e1 = torch.empty(n, dtype=torch.float32, device=device).exponential_(generator=gen)
    e2 = torch.empty(n, dtype=torch.float32, device=device).exponential_(generator=gen)
    return (e1 - e2).mul_(beta)


def normal(n: int, sigma: float, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(n, dtype=torch.float32, device=device, generator=gen).mul_(sigma)


def zipf_rows(vocab: int, rows: int, s: float, gen: torch.Generator) -> torch.Tensor:
    """Distinct row ids drawn with P(rank r) ~ r^-s until `rows` are distinct."""
    w = torch.arange(1, vocab + 1, dtype=torch.float64).pow(-s)
    seen: List[int] = []
    have = set()
    while len(seen) < rows:
        draw = torch.multinomial(w, 4 * rows, replacement=True, generator=gen)
        for r in draw.tolist():
            if r not in have:
                have.add(r)
                seen.append(r)
                if len(seen) == rows:
                    break
    return torch.tensor(sorted(seen), dtype=torch.int64)


def fan_in(shape: Sequence[int]) -> int:
    return math.prod(shape[1:]) if len(shape) >= 2 else 1


def gradient(w: Workload, worker: int, step: int, device="cpu", numel: int | None = None) -> torch.Tensor:
    """One worker's fresh fp32 gradient for one step, flattened in tensor order.

    ``numel`` truncates flat workloads (a prefix of the same draw recipe with
    the same seed), used for reduced-size checks.
    """
    device = torch.device(device)
    gen = _gen(seed_of(w, worker, step), device)
    if w.name == "flat-1M":
        return laplace(numel or w.numel, 1e-3, gen, device)
    if w.name == "flat-1G":
        n = numel or w.numel
        out = normal(n, 1e-4, gen, device)
        heavy = torch.rand(n, device=device, generator=gen) < 0.01
        lap = laplace(n, 1e-2, gen, device)
        out = torch.where(heavy, lap, out)
        del heavy, lap
        return out
    if w.name == "mlp-mnist":
        return normal(w.numel, 1e-2, gen, device)
    if w.name == "resnet50":
        parts = []
        for _, shape in w.tensors:
            m = math.prod(shape)
            x = laplace(m, 1e-3, gen, device)
            if len(shape) >= 2:
                x.div_(math.sqrt(fan_in(shape)))
            parts.append(x)
        return torch.cat(parts)
    if w.name == "nmt-rnn":
        cpu_gen = _gen(seed_of(w, worker, step), "cpu")
        parts = []
        for name, shape in w.tensors:
            m = math.prod(shape)
            if name.startswith("E_"):
                emb = torch.zeros(shape, dtype=torch.float32, device=device)
                ids = zipf_rows(shape[0], w.extra["rows"], w.extra["zipf"], cpu_gen).to(device)
                emb[ids] = laplace(ids.numel() * shape[1], 1e-3, gen, device).view(-1, shape[1])
                parts.append(emb.view(-1))
            else:
                parts.append(normal(m, 1e-4, gen, device))
        return torch.cat(parts)
    raise KeyError(w.name)


def small_segments(rng: torch.Generator, nseg: int, max_len: int) -> List[int]:
    """Random segment sizes in [0, max_len] for ragged/edge-case tests."""
    return torch.randint(0, max_len + 1, (nseg,), generator=rng).tolist()
