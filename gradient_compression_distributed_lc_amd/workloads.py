"""Seeded synthetic gradient sets with the shapes of the pages' workloads.

This module holds no codec arithmetic: it only lists tensor shapes and draws
seeded random values.  Both the GPU tests/benchmark and the CPU oracle read the
arrays it returns, so they see identical inputs.

The 3LC page ("3LC: Lightweight and Effective Traffic Compression for
Distributed Machine Learning", abstract and main findings) trains ResNet-110
on CIFAR-10; the DeepReduce page ("DeepReduce: A Sparse-tensor Communication
Framework for Distributed Deep Learning", main findings) uses ResNet-50 and
BERT.  No dataset or trained weight is used: only the models' parameter
shapes, with gradient-like random values:

* ``single_1m``     one tensor, n = 1,048,576, N(0, 1e-3), seed 1, s = 1.0
* ``single_16m``    one tensor, n = 16,777,216, per element Bernoulli(0.1)
                    chooses Laplace(0, scale 1e-2), else N(0, 1e-5);
                    step t uses seed 200 + t; s = 1.5, 10 steps
* ``resnet110``     329 tensors, 1,727,962 values, N(0, 1e-3/sqrt(fan_in)),
                    seed 3, s = 1.9
* ``resnet50``      161 tensors, 25,557,032 values, Bernoulli(0.5) exact
                    zeros, else N(0, 1e-4), seed 4, s in {1.0, 1.5, 1.9}
* ``bert_large``    391 tensors (all BERT-large parameters), 335,141,888
                    values, Bernoulli(0.3) exact zeros, else N(0, 1e-4);
                    worker w uses seed 500 + w; s = 1.75
* ``bert_large_core`` the 145 weight matrices of BERT-large only
                    (333,244,416 values), same distribution.

Conventions: N(0, a) has standard deviation a; Laplace(0, b) has scale b;
numpy ``default_rng(seed)`` (PCG64); a flat float32 array is drawn in tensor
order: first the normals (or the mixture's parts), then the uniforms of the
zero mask.  Exact zeros are +0.0.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Workload:
    name: str
    sizes: list[int]
    s_values: list[float]
    description: str
    names: list[str] = field(default_factory=list)
    fan_in: list[int] = field(default_factory=list)

    @property
    def total(self) -> int:
        return int(sum(self.sizes))

    @property
    def count(self) -> int:
        return len(self.sizes)


# ----------------------------------------------------------------------------
# parameter shapes


def resnet110_shapes():
    """CIFAR ResNet-110: 3 stages x 18 basic blocks at 16/32/64 channels,
    option-A shortcuts (no parameters), BN scale and shift per conv, FC 64->10.
    Returns (names, sizes, fan_in)."""
    names, sizes, fans = [], [], []

    def add(name, size, fan):
        names.append(name)
        sizes.append(int(size))
        fans.append(int(fan))

    add("conv1.weight", 16 * 3 * 3 * 3, 27)
    add("bn1.weight", 16, 1)
    add("bn1.bias", 16, 1)
    cin = 16
    for stage, ch in enumerate((16, 32, 64), start=1):
        for blk in range(18):
            p = f"layer{stage}.{blk}"
            add(f"{p}.conv1.weight", ch * cin * 9, cin * 9)
            add(f"{p}.bn1.weight", ch, 1)
            add(f"{p}.bn1.bias", ch, 1)
            add(f"{p}.conv2.weight", ch * ch * 9, ch * 9)
            add(f"{p}.bn2.weight", ch, 1)
            add(f"{p}.bn2.bias", ch, 1)
            cin = ch
    add("fc.weight", 10 * 64, 64)
    add("fc.bias", 10, 64)
    return names, sizes, fans


def resnet50_shapes():
    """ImageNet ResNet-50 (bottleneck blocks [3, 4, 6, 3], projection
    shortcuts, BN scale/shift, FC 2048->1000).  Returns (names, sizes)."""
    names, sizes = [], []

    def add(name, size):
        names.append(name)
        sizes.append(int(size))

    add("conv1.weight", 64 * 3 * 7 * 7)
    add("bn1.weight", 64)
    add("bn1.bias", 64)
    cin = 64
    for li, (blocks, width) in enumerate(((3, 64), (4, 128), (6, 256), (3, 512)), start=1):
        cout = width * 4
        for b in range(blocks):
            p = f"layer{li}.{b}"
            add(f"{p}.conv1.weight", width * cin)
            add(f"{p}.bn1.weight", width)
            add(f"{p}.bn1.bias", width)
            add(f"{p}.conv2.weight", width * width * 9)
            add(f"{p}.bn2.weight", width)
            add(f"{p}.bn2.bias", width)
            add(f"{p}.conv3.weight", cout * width)
            add(f"{p}.bn3.weight", cout)
            add(f"{p}.bn3.bias", cout)
            if b == 0:
                add(f"{p}.downsample.0.weight", cout * cin)
                add(f"{p}.downsample.1.weight", cout)
                add(f"{p}.downsample.1.bias", cout)
            cin = cout
    add("fc.weight", 1000 * 2048)
    add("fc.bias", 1000)
    return names, sizes


def bert_large_shapes(core_only: bool = False):
    """BERT-large (24 layers, hidden 1024, FFN 4096, vocab 30522, 512
    positions, 2 token types).  ``core_only`` keeps the word embedding and the
    six weight matrices per layer (145 tensors).  Returns (names, sizes)."""
    H, F, V, P, T, NL = 1024, 4096, 30522, 512, 2, 24
    names, sizes = [], []

    def add(name, size):
        names.append(name)
        sizes.append(int(size))

    add("embeddings.word_embeddings.weight", V * H)
    if not core_only:
        add("embeddings.position_embeddings.weight", P * H)
        add("embeddings.token_type_embeddings.weight", T * H)
        add("embeddings.LayerNorm.weight", H)
        add("embeddings.LayerNorm.bias", H)
    for layer in range(NL):
        p = f"encoder.layer.{layer}"
        for m in ("attention.self.query", "attention.self.key", "attention.self.value",
                  "attention.output.dense"):
            add(f"{p}.{m}.weight", H * H)
            if not core_only:
                add(f"{p}.{m}.bias", H)
        if not core_only:
            add(f"{p}.attention.output.LayerNorm.weight", H)
            add(f"{p}.attention.output.LayerNorm.bias", H)
        add(f"{p}.intermediate.dense.weight", F * H)
        if not core_only:
            add(f"{p}.intermediate.dense.bias", F)
        add(f"{p}.output.dense.weight", H * F)
        if not core_only:
            add(f"{p}.output.dense.bias", H)
            add(f"{p}.output.LayerNorm.weight", H)
            add(f"{p}.output.LayerNorm.bias", H)
    if not core_only:
        add("pooler.dense.weight", H * H)
        add("pooler.dense.bias", H)
    return names, sizes


# ----------------------------------------------------------------------------
# workloads


def get(name: str) -> Workload:
    if name == "single_1m":
        return Workload(name, [1_048_576], [1.0], "one fp32 tensor, n=1,048,576, N(0,1e-3), seed 1")
    if name == "single_16m":
        return Workload(name, [16_777_216], [1.5],
                        "one fp32 tensor, n=16,777,216, 0.9 N(0,1e-5) + 0.1 Laplace(0,1e-2), "
                        "seed 200+t for step t, 10 steps with carried error")
    if name == "resnet110":
        names, sizes, fans = resnet110_shapes()
        return Workload(name, sizes, [1.9], "ResNet-110 (CIFAR) gradient set, N(0,1e-3/sqrt(fan_in))",
                        names, fans)
    if name == "resnet50":
        names, sizes = resnet50_shapes()
        return Workload(name, sizes, [1.0, 1.5, 1.9],
                        "ResNet-50 gradient set, 50% exact zeros, rest N(0,1e-4)", names)
    if name in ("bert_large", "bert_large_core"):
        core = name == "bert_large_core"
        names, sizes = bert_large_shapes(core_only=core)
        return Workload(name, sizes, [1.75],
                        "BERT-large gradient set%s, 30%% exact zeros, rest N(0,1e-4)"
                        % (" (weight matrices only)" if core else ""), names)
    raise KeyError(name)


WORKLOADS = ("single_1m", "single_16m", "resnet110", "resnet50", "bert_large", "bert_large_core")


def seed_for(name: str, step: int = 0, worker: int = 0) -> int:
    return {"single_1m": 1, "single_16m": 200 + step, "resnet110": 3, "resnet50": 4,
            "bert_large": 500 + worker, "bert_large_core": 500 + worker}[name]


def _zero_mask(rng, x, p_zero):
    mask = rng.random(x.size, dtype=np.float32) < np.float32(p_zero)
    x[mask] = np.float32(0.0)


def generate(name: str, step: int = 0, worker: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """Flat float32 gradient array of the workload (tensors back to back)."""
    w = get(name)
    rng = np.random.default_rng(seed_for(name, step, worker))
    N = w.total
    x = out if out is not None else np.empty(N, dtype=np.float32)
    if name == "single_1m":
        rng.standard_normal(N, dtype=np.float32, out=x)
        x *= np.float32(1e-3)
    elif name == "single_16m":
        rng.standard_normal(N, dtype=np.float32, out=x)
        x *= np.float32(1e-5)
        lap = rng.laplace(0.0, 1e-2, N).astype(np.float32)
        pick = rng.random(N, dtype=np.float32) < np.float32(0.1)
        x[pick] = lap[pick]
    elif name == "resnet110":
        rng.standard_normal(N, dtype=np.float32, out=x)
        off = 0
        for size, fan in zip(w.sizes, w.fan_in):
            x[off:off + size] *= np.float32(1e-3 / np.sqrt(fan))
            off += size
    elif name == "resnet50":
        rng.standard_normal(N, dtype=np.float32, out=x)
        x *= np.float32(1e-4)
        _zero_mask(rng, x, 0.5)
    elif name in ("bert_large", "bert_large_core"):
        rng.standard_normal(N, dtype=np.float32, out=x)
        x *= np.float32(1e-4)
        _zero_mask(rng, x, 0.3)
    else:
        raise KeyError(name)
    return x


def offsets(sizes) -> np.ndarray:
    """Element offset of each tensor in the flat array, plus the total."""
    o = np.zeros(len(sizes) + 1, dtype=np.int64)
    np.cumsum(np.asarray(sizes, dtype=np.int64), out=o[1:])
    return o


def random_sizes(rng, count: int, max_size: int) -> list[int]:
    """Ragged tensor sizes for stress tests: a log-uniform mix from 1 to max_size."""
    logs = rng.uniform(0.0, np.log(max_size), count)
    return [max(1, int(np.exp(v))) for v in logs]
