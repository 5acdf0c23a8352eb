"""The synthetic layer shapes the operator is tested and measured on.

Each workload is a set of linear layers (W is N x K, quantized with block
length d and lifted dimension D, so D/d bits per weight) plus the batch sizes
and activation dtype it runs at. The shapes are those of Llama-3-8B/70B MLP
and attention projections, Qwen-2.5-32B MLP projections and an 8192-wide
prefill GEMM; the bit-widths are the paper's worked rates (2.4 = LQ-24/10,
2.5 = 5/2 and 2.67 = 8/3 from the codeword-generation figure of the LiftQuant
paper). No model weights or datasets are involved: every tensor is drawn from
the seeded distributions in ``workloads.gen``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple


@dataclass(frozen=True)
class LayerSpec:
    name: str
    K: int          # input features
    N: int          # output features
    d: int          # block length in the original weight space
    D: int          # lifted dimension (sign bits per block)
    hb: int         # Hadamard block size of the whitening transform
    seed: int

    @property
    def Kb(self) -> int:
        return -(-self.K // self.d)

    @property
    def Kpad(self) -> int:
        return self.Kb * self.d

    @property
    def L(self) -> int:
        return self.Kb * self.D


@dataclass(frozen=True)
class Workload:
    name: str
    layers: Tuple[LayerSpec, ...]
    batches: Tuple[int, ...]
    xdtype: str                 # "f32" or "bf16"
    outlier_frac: float = 0.0   # fraction of input channels scaled up
    outlier_gain: float = 1.0
    note: str = ""


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny",
        (LayerSpec("tiny", K=512, N=512, d=2, D=5, hb=512, seed=101),),
        batches=(1,), xdtype="f32",
        note="K=N=512, 2.5 bit, fp32 activations"),
    "llama3_8b_mlp": Workload(
        "llama3_8b_mlp",
        (LayerSpec("gate_up", K=4096, N=14336, d=10, D=24, hb=1024, seed=201),
         LayerSpec("down", K=14336, N=4096, d=10, D=24, hb=1024, seed=202)),
        batches=(1,), xdtype="bf16",
        note="Llama-3-8B MLP at 2.4 bit, batch-1 decode"),
    "llama3_70b": Workload(
        "llama3_70b",
        (LayerSpec("gate_up", K=8192, N=28672, d=10, D=24, hb=1024, seed=301),
         LayerSpec("down", K=28672, N=8192, d=10, D=24, hb=1024, seed=302),
         LayerSpec("qkv", K=8192, N=10240, d=10, D=24, hb=1024, seed=303)),
        batches=(1, 4, 16), xdtype="bf16",
        note="Llama-3-70B MLP and QKV at 2.4 bit"),
    "qwen25_32b": Workload(
        "qwen25_32b",
        (LayerSpec("up", K=5120, N=27648, d=2, D=5, hb=1024, seed=401),
         LayerSpec("down", K=27648, N=5120, d=2, D=5, hb=1024, seed=402)),
        batches=(16, 64), xdtype="bf16", outlier_frac=0.01, outlier_gain=20.0,
        note="Qwen-2.5-32B MLP at 2.5 bit, 1% outlier channels x20"),
    "prefill": Workload(
        "prefill",
        (LayerSpec("sq", K=8192, N=8192, d=3, D=8, hb=1024, seed=501),
         LayerSpec("wide", K=8192, N=28672, d=3, D=8, hb=1024, seed=502)),
        batches=(2048,), xdtype="bf16",
        note="2048-token prefill GEMM at 2.67 bit"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def all_layers() -> List[Tuple[Workload, LayerSpec]]:
    return [(w, l) for w in WORKLOADS.values() for l in w.layers]
