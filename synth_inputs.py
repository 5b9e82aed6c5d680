"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws random numbers and
rounds them to the storage dtype, so that the HIP path and the FP64 oracle
see bit-identical input values.

Recipe (per workload):
  * a fresh generator per workload, seeded with the workload's seed, draws
    Q, then K, then V;
  * small workloads use numpy's PCG64 ``default_rng(seed).standard_normal``
    in float32 on the host (the generator family of the lecture's demo 1);
  * the large workloads (hundreds of MB to GB) use torch's Philox generator
    on the GPU (``torch.Generator(device).manual_seed(seed)``) so that no
    multi-GB host draw or copy is needed; samples for the oracle are copied
    back from those same device tensors;
  * values are ``std * N(0, 1)`` and are rounded to the storage dtype with
    round-to-nearest-even; the oracle widens the rounded values to float64.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Shape:
    B: int
    H: int
    N: int
    Nk: int
    d: int
    dv: int


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shapes: tuple          # tuple of Shape
    dtype: str             # "f32" | "bf16" | "f16"
    causal: tuple          # causal settings exercised
    std: float = 1.0
    seed: int = 0
    num_splits: int = 0    # > 0: split-KV decode workload
    description: str = ""


WORKLOADS = {
    "single_head_f32": Workload(
        "single_head_f32", (Shape(1, 1, 256, 256, 64, 64),), "f32", (False,), 1.0, 0,
        description="one head, N=Nk=256, d=64, fp32, non-causal, seed 0"),
    "ragged_f32": Workload(
        "ragged_f32", (Shape(1, 1, 300, 300, 64, 64), Shape(1, 1, 77, 513, 32, 32),
                       Shape(1, 1, 1, 1000, 64, 64)), "f32", (False, True), 1.0, 0,
        description="one head, fp32, tile-ragged shapes, causal and non-causal, seed 0"),
    "prefill_b64_h16_n1024_d64": Workload(
        "prefill_b64_h16_n1024_d64", (Shape(64, 16, 1024, 1024, 64, 64),), "bf16", (True,),
        0.5, 3, description="GPT-2-medium-shaped prefill: B=64, H=16, N=Nk=1024, d=64, "
                            "bf16, causal, inputs 0.5*N(0,1)"),
    "prefill_b2_h32_n8192_d128": Workload(
        "prefill_b2_h32_n8192_d128", (Shape(2, 32, 8192, 8192, 128, 128),), "bf16", (True,),
        1.0, 4, description="long prefill: B=2, H=32, N=Nk=8192, d=128, bf16, causal"),
    "decode_b8_h32_nk32768_d128": Workload(
        "decode_b8_h32_nk32768_d128", (Shape(8, 32, 1, 32768, 128, 128),), "bf16", (False,),
        1.0, 5, num_splits=64,
        description="split-KV decode: B=8, H=32, N=1, Nk=32768, d=128, bf16, 64 splits"),
}


def host_qkv(shape: Shape, seed: int, std: float = 1.0):
    """Q, K, V as float32 numpy arrays [B,H,N,d], [B,H,Nk,d], [B,H,Nk,dv]."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((shape.B, shape.H, shape.N, shape.d), dtype=np.float32)
    k = rng.standard_normal((shape.B, shape.H, shape.Nk, shape.d), dtype=np.float32)
    v = rng.standard_normal((shape.B, shape.H, shape.Nk, shape.dv), dtype=np.float32)
    if std != 1.0:
        q, k, v = (x * np.float32(std) for x in (q, k, v))
    return q, k, v


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]


def to_storage(x_f32, dtype: str, device="cpu"):
    """numpy float32 -> torch tensor in the storage dtype (round-to-nearest-even)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x_f32)).to(device=device,
                                                            dtype=torch_dtype(dtype))


def device_qkv(shape: Shape, seed: int, dtype: str, device, std: float = 1.0):
    """Q, K, V drawn on ``device`` with a seeded torch generator, in the storage dtype."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    td = torch_dtype(dtype)
    out = []
    for n, dd in ((shape.N, shape.d), (shape.Nk, shape.d), (shape.Nk, shape.dv)):
        x = torch.randn((shape.B, shape.H, n, dd), generator=g, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out.append(x.to(td))
        del x
    return tuple(out)


def as_f64(t) -> np.ndarray:
    """A storage-dtype torch tensor (any device) widened exactly to float64 numpy."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()
