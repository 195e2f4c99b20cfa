"""The five synthetic workloads of the DP-SGD clip/sum/noise step, plus helpers
to derive smaller parity-test variants of them.

Each workload is a list of linear layers (d_in -> d_out); a LoRA adapter counts
as two linear layers (the down-projection d -> r, then the up-projection
r -> d), so an adapter of rank r on a d x d matrix has r*(d + d) trainables.
Inputs per layer are activations A[B, T, d_in] and output gradients
G[B, T, d_out], drawn by the seeded generator in this package.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

F32 = 0
BF16 = 1
DTYPE_NAMES = {F32: "f32", BF16: "bf16"}
ELEM_BYTES = {F32: 4, BF16: 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: Tuple[Tuple[int, int], ...]          # (d_in, d_out) per linear layer, plan order
    layer_names: Tuple[str, ...]
    dtype: int
    B: int                                       # records per physical batch (one library call)
    logical_B: int                               # records per logical step (noise drawn once)
    T: int                                       # tokens per record
    C: float
    sigma: float
    data_seed: int
    a_std: float = 1.0
    g_std: float = 1.0
    heavy_every: int = 0                         # records i with i % heavy_every == 0 are Student-t
    g_norm_targets: Optional[Tuple[float, ...]] = None  # per-record target gradient norms (workload 1)
    noise_seed: int = 0
    description: str = ""

    @property
    def n_layers(self) -> int:
        return len(self.layers)

    @property
    def n_params(self) -> int:
        return sum(a * b for a, b in self.layers)

    @property
    def n_phys(self) -> int:
        return self.logical_B // self.B

    def input_bytes_per_batch(self) -> int:
        e = ELEM_BYTES[self.dtype]
        return sum(self.B * self.T * (a + b) * e for a, b in self.layers)

    def record_scale(self, layer: int, tensor: int, record: int) -> float:
        """Standard deviation multiplier of record `record` in (layer, tensor)."""
        if tensor == 0:
            return self.a_std
        if self.g_norm_targets is not None:
            d_in, d_out = self.layers[layer]
            # E||A_i^T G_i||_F^2 = T * d_in * d_out for unit-variance entries
            return self.g_norm_targets[record % len(self.g_norm_targets)] / math.sqrt(
                self.T * d_in * d_out)
        return self.g_std

    def record_heavy(self, record: int) -> int:
        return 1 if (self.heavy_every and record % self.heavy_every == 0) else 0

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _lora(n_blocks: int, projs: List[str], d: int, r: int) -> Tuple[tuple, tuple]:
    layers, names = [], []
    for k in range(n_blocks):
        for p in projs:
            layers += [(d, r), (r, d)]
            names += [f"{k}.{p}.lora_A", f"{k}.{p}.lora_B"]
    return tuple(layers), tuple(names)


def workload(idx: int) -> Workload:
    """Workloads 1..5 at full size."""
    if idx == 1:
        return Workload(
            name="dense64x32_fp32_B8_T4", layers=((64, 32),), layer_names=("linear",), dtype=F32,
            B=8, logical_B=8, T=4, C=1.0, sigma=1.0, data_seed=0x5EED0001,
            g_norm_targets=tuple(10.0 ** (-1.0 + 2.0 * i / 7.0) for i in range(8)),
            description="one fp32 linear 64->32, 8 records x 4 tokens, record norms 0.1..10")
    if idx == 2:
        layers, names = _lora(12, ["q", "v"], 768, 8)
        return Workload(
            name="opt125m_lora_r8_qv_fp32_B16_T128", layers=layers, layer_names=names, dtype=F32,
            B=16, logical_B=16, T=128, C=1.0, sigma=1.0, data_seed=0x5EED0002,
            description="OPT-125M-shaped rank-8 LoRA on q,v of 12 blocks (hidden 768), fp32")
    if idx == 3:
        layers, names = _lora(32, ["q", "k", "v", "o"], 4096, 16)
        return Workload(
            name="7b_lora_r16_qkvo_bf16_B256_T512", layers=layers, layer_names=names, dtype=BF16,
            B=256, logical_B=256, T=512, C=0.5, sigma=0.8, data_seed=0x5EED0003,
            a_std=0.02, g_std=0.02, heavy_every=100,
            description="7B-shaped rank-16 LoRA on q,k,v,o of 32 blocks (hidden 4096), bf16, "
                        "records 0,100,200 Student-t(3)")
    if idx == 4:
        return Workload(
            name="dense4096_bf16_B64_T256", layers=((4096, 4096),) * 4,
            layer_names=tuple(f"linear{k}" for k in range(4)), dtype=BF16,
            B=64, logical_B=64, T=256, C=1.0, sigma=1.1, data_seed=0x5EED0004,
            a_std=1.0, g_std=1e-3,
            description="four dense 4096x4096 bf16 layers, 64 records x 256 tokens")
    if idx == 5:
        layers, names = _lora(24, ["x"], 1024, 8)
        names = tuple(n.replace(".x.", ".") for n in names)
        return Workload(
            name="lora_r8_h1024_bf16_B4096_virtual256_T256", layers=layers, layer_names=names,
            dtype=BF16, B=256, logical_B=4096, T=256, C=1.0, sigma=0.6, data_seed=0x5EED0005,
            description="rank-8 LoRA on 24 layers of hidden 1024, bf16, logical batch 4096 "
                        "in 16 physical batches of 256, noise once")
    raise ValueError(idx)


def reduced(idx: int) -> Workload:
    """Small variants of each workload that the CPU oracle finishes in seconds, with the same
    layer structure kinds, dtype and value distributions, but fewer/smaller layers and records.
    Sizes are chosen to span several kernel tiles and to leave ragged tails."""
    w = workload(idx)
    if idx == 1:
        return w
    if idx == 2:
        layers, names = _lora(2, ["q", "v"], 768, 8)
        return w.with_(name="opt125m_lora_r8_fp32_reduced", layers=layers, layer_names=names,
                       B=5, logical_B=5, T=40)
    if idx == 3:
        layers, names = _lora(1, ["q", "k"], 4096, 16)
        return w.with_(name="7b_lora_r16_bf16_reduced", layers=layers, layer_names=names,
                       B=5, logical_B=5, T=72, heavy_every=3)
    if idx == 4:
        return w.with_(name="dense_bf16_reduced", layers=((320, 272), (272, 320)),
                       layer_names=("linear0", "linear1"), B=3, logical_B=3, T=48)
    if idx == 5:
        layers, names = _lora(2, ["x"], 1024, 8)
        return w.with_(name="lora_r8_h1024_bf16_virtual_reduced", layers=layers,
                       layer_names=names, B=3, logical_B=9, T=40)
    raise ValueError(idx)
