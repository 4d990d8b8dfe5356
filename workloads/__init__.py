"""Seeded synthetic workloads for the AdaComp compressor.

This module is shared by the tests, the benchmark and the smoke entry point.
It builds layer (segment) tables and draws seeded gradients ``dW``; it holds
none of the compressor's arithmetic.  Both the GPU path and the CPU oracle are
fed from it: gradients are drawn with torch on the device that will use them
and copied to the host for the oracle, so both sides see the same bits.

The training workloads the pages measure on (MNIST/CIFAR10/ImageNet CNNs,
BN50-DNN, a Shakespeare LSTM: "AdaComp" AIMech page, Application claim,
Table 2) need datasets and trained models that are not available.  These
synthetic gradients stand in for them with the layer shapes, bin lengths
(L_T = 50 for conv, 500 for FC/LSTM) and magnitude structure of those layers.

A segment is ``(offset, numel, bin_len)``: ``numel`` elements of the flat
float32 buffers starting at element ``offset``, compressed with bins of
``bin_len`` elements.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, List, Optional, Sequence, Tuple

import torch

Segment = Tuple[int, int, int]

CONV_BIN = 50
FC_BIN = 500


@dataclass
class Layer:
    name: str
    shape: Tuple[int, ...]
    bin_len: int
    # Kind of gradient drawn for this layer, see ``fill_dw``.
    dist: str
    scale: float                 # std (normal) or b (laplace)
    active_p: float = 1.0        # per-bin activity probability
    active_gain: float = 1.0     # multiplier of active bins
    idle_gain: float = 1.0       # multiplier of inactive bins

    @property
    def numel(self) -> int:
        return math.prod(self.shape)


@dataclass
class Workload:
    name: str
    index: int                   # used in the seed formula
    layers: List[Layer]
    steps: int
    decode_messages: int = 0
    segments: List[Segment] = field(default_factory=list)

    def __post_init__(self):
        off = 0
        self.segments = []
        for ly in self.layers:
            self.segments.append((off, ly.numel, ly.bin_len))
            off += (ly.numel + 3) // 4 * 4     # keep every offset 16-byte aligned

    @property
    def span(self) -> int:
        return max(o + n for o, n, _ in self.segments)

    @property
    def numel(self) -> int:
        return sum(n for _, n, _ in self.segments)

    @property
    def bins(self) -> int:
        return sum((n + b - 1) // b for _, n, b in self.segments)


def seed_of(workload_index: int, learner: int, step: int) -> int:
    return 1_000_000 * workload_index + 1000 * learner + step


def _fc_single() -> Workload:
    return Workload("fc_100x1000", 1,
                    [Layer("fc", (100, 1000), FC_BIN, "normal", 1e-3)], steps=10)


def _conv_stack() -> Workload:
    layers = []
    for c in (64, 128, 256, 512):
        fan_in = c * 3 * 3
        layers.append(Layer(f"conv{c}", (c, c, 3, 3), CONV_BIN, "laplace",
                            1e-2 / math.sqrt(fan_in)))
    return Workload("conv_stack_4", 2, layers, steps=50)


def _fc_lstm() -> Workload:
    # Sparse input activity: each bin is active with probability 0.3; inactive
    # bins carry 1e-3 of the gradient scale.
    kw = dict(active_p=0.3, active_gain=1.0, idle_gain=1e-3)
    return Workload("fc_lstm_25m", 3, [
        Layer("lstm_gates", (4 * 1024, 2048), FC_BIN, "normal", 1e-3, **kw),
        Layer("fc", (4096, 4096), FC_BIN, "normal", 1e-3, **kw),
    ], steps=50)


def resnet50_shapes() -> List[Tuple[str, Tuple[int, ...]]]:
    """The 161 weight and bias tensors of the standard ResNet-50, in the usual
    parameter order: stem conv 7x7 + BN, four bottleneck stages of 3, 4, 6
    and 3 blocks (widths 64, 128, 256, 512, expansion 4, a 1x1 projection in
    each stage's first block), each conv followed by BN gamma and beta, and
    the final 2048 -> 1000 classifier."""
    out: List[Tuple[str, Tuple[int, ...]]] = []

    def conv(name, cout, cin, k):
        out.append((name + ".weight", (cout, cin, k, k)))

    def bn(name, c):
        out.append((name + ".weight", (c,)))
        out.append((name + ".bias", (c,)))

    conv("conv1", 64, 3, 7)
    bn("bn1", 64)
    inplanes = 64
    for stage, (width, blocks) in enumerate(zip((64, 128, 256, 512), (3, 4, 6, 3)), 1):
        for i in range(blocks):
            p = f"layer{stage}.{i}"
            conv(p + ".conv1", width, inplanes, 1)
            bn(p + ".bn1", width)
            conv(p + ".conv2", width, width, 3)
            bn(p + ".bn2", width)
            conv(p + ".conv3", width * 4, width, 1)
            bn(p + ".bn3", width * 4)
            if i == 0:
                conv(p + ".downsample.0", width * 4, inplanes, 1)
                bn(p + ".downsample.1", width * 4)
            inplanes = width * 4
    out.append(("fc.weight", (1000, 2048)))
    out.append(("fc.bias", (1000,)))
    return out


def _resnet50() -> Workload:
    layers = []
    for name, shape in resnet50_shapes():
        if len(shape) == 4:
            fan_in = shape[1] * shape[2] * shape[3]
        elif len(shape) == 2:
            fan_in = shape[1]
        else:
            fan_in = shape[0]          # 1-D tensors: fan_in = numel
        lt = FC_BIN if name.startswith("fc.") else CONV_BIN
        layers.append(Layer(name, shape, lt, "normal", 1e-2 / math.sqrt(fan_in)))
    return Workload("resnet50_161", 4, layers, steps=20)


def _large() -> Workload:
    # Bursty: each bin is scaled by 100 with probability 0.05.
    layers = [Layer(f"w{i}", (4096, 4096), FC_BIN, "normal", 1e-3,
                    active_p=0.05, active_gain=100.0, idle_gain=1.0)
              for i in range(64)]
    return Workload("large_64x4096x4096", 5, layers, steps=10, decode_messages=16)


WORKLOADS = {
    "fc": _fc_single,
    "conv": _conv_stack,
    "fc_lstm": _fc_lstm,
    "resnet50": _resnet50,
    "large": _large,
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]()


def custom(segments: Sequence[Segment], dist: str = "normal", scale: float = 1e-3,
           name: str = "custom", index: int = 9) -> Workload:
    """A workload over an explicit segment table (used for edge cases)."""
    wl = Workload(name, index, [], steps=1)
    wl.segments = [tuple(int(x) for x in s) for s in segments]
    wl.layers = [Layer(f"s{i}", (n,), b, dist, scale) for i, (_, n, b) in enumerate(wl.segments)]
    return wl


def _fill_layer(view: torch.Tensor, ly: Layer, gen: torch.Generator) -> None:
    n = view.numel()
    if ly.dist == "normal":
        view.normal_(0.0, ly.scale, generator=gen)
    elif ly.dist == "laplace":
        # Inverse-CDF sampling from u in the open interval (0, 1).
        u = torch.empty(n, dtype=torch.float64, device=view.device).uniform_(generator=gen)
        u = u * (1.0 - 2.0 ** -40) + 2.0 ** -41
        x = torch.where(u < 0.5, torch.log(2.0 * u), -torch.log(2.0 - 2.0 * u))
        view.copy_((x * ly.scale).to(torch.float32))
    elif ly.dist == "zero":
        view.zero_()
    else:
        raise ValueError(ly.dist)
    if ly.active_p < 1.0:
        nb = (n + ly.bin_len - 1) // ly.bin_len
        act = torch.rand(nb, generator=gen, device=view.device) < ly.active_p
        gain = torch.where(act, torch.tensor(ly.active_gain, device=view.device),
                           torch.tensor(ly.idle_gain, device=view.device)).to(torch.float32)
        view.mul_(gain.repeat_interleave(ly.bin_len)[:n])


def fill_dw(buf: torch.Tensor, wl: Workload, learner: int, step: int) -> torch.Tensor:
    """Draw the gradient of (learner, step) into the flat float32 ``buf``
    (length >= ``wl.span``); elements outside every segment are set to 0."""
    if buf.dtype != torch.float32 or buf.dim() != 1 or buf.numel() < wl.span:
        raise ValueError("buf must be a 1-D float32 tensor of at least span elements")
    gen = torch.Generator(device=buf.device)
    gen.manual_seed(seed_of(wl.index, learner, step))
    buf.zero_()
    for (off, n, _), ly in zip(wl.segments, wl.layers):
        _fill_layer(buf[off:off + n], ly, gen)
    return buf


def make_dw(wl: Workload, learner: int, step: int, device="cpu") -> torch.Tensor:
    buf = torch.empty(alloc_len(wl), dtype=torch.float32, device=device)
    return fill_dw(buf, wl, learner, step)


def alloc_len(wl: Workload) -> int:
    """Length to allocate for the flat buffers: the span rounded up to 4."""
    return (wl.span + 3) // 4 * 4
