"""Seeded synthetic inputs and workload sizes, shared by the tests, the oracle's
callers and the benchmark.

This module holds random-number generation, dtype rounding and the sizes of the
workloads, and nothing of the attention or cache arithmetic. Neither the oracle
nor the HIP library imports it; callers generate arrays here and hand the same
values to both sides.

Streams: every tensor is drawn from its own stream keyed by
(workload, tensor, batch element, chunk, rewrite), so one batch element's
values never depend on how many other batch elements exist -- a B=2 run
contains two B=1 runs exactly (LingBot-World PR #53, section Verification,
checks B=2 against B=1 bit for bit).

* ``normal_f32`` -- numpy PCG64 seeded through SeedSequence(key); host side.
* ``device_normal`` -- torch's generator on a device seeded from the same key
  (a different stream than the host one; used where the host would be too slow
  to draw the values, e.g. 774M-element query tensors).
* ``round_to`` -- fp32 -> bf16/fp16/fp32 with round-to-nearest-even (torch CPU).
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

try:
    import torch
except ImportError:  # the oracle tests need numpy only
    torch = None

WORKLOAD_IDS = {"tiny": 1, "decode": 2, "ring": 3, "multiuser": 4, "ragged": 5, "misc": 9}
TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "index": 4, "extra": 5}


def seed_key(workload: str, tensor: str, b: int = 0, chunk: int = 0, rewrite: int = 0,
             base_seed: int = 0) -> list[int]:
    return [int(base_seed), WORKLOAD_IDS[workload], TENSOR_IDS[tensor], int(b), int(chunk),
            int(rewrite)]


def normal_f32(shape, key, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) fp32 values from PCG64(SeedSequence(key))."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[name]


def round_to(x: np.ndarray, dtype: str):
    """fp32 array -> CPU torch tensor of dtype ('f32', 'bf16', 'f16'), RNE rounding."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(_torch_dtype(dtype))


def as_f64(t) -> np.ndarray:
    """Exact fp64 copy of a tensor's values (bf16/fp16/fp32 upcasts are exact)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def per_batch_normal(B: int, row_shape, workload: str, tensor: str, chunk: int = 0,
                     rewrite: int = 0, std: float = 1.0, dtype: str = "f32"):
    """[B, *row_shape] tensor whose slice b comes from its own stream."""
    parts = [normal_f32(row_shape, seed_key(workload, tensor, b, chunk, rewrite), std)
             for b in range(B)]
    return round_to(np.stack(parts), dtype)


def _device_seed(key) -> int:
    h = hashlib.sha256(",".join(str(int(k)) for k in key).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def device_normal(shape, key, dtype: str, device, std: float = 1.0):
    """N(0, std^2) drawn with torch's generator on `device`, then rounded to dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(_device_seed(key))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(_torch_dtype(dtype))


def per_batch_device_normal(B: int, row_shape, workload: str, tensor: str, device, dtype: str,
                            chunk: int = 0, rewrite: int = 0, std: float = 1.0):
    out = torch.empty((B,) + tuple(row_shape), dtype=_torch_dtype(dtype), device=device)
    for b in range(B):
        out[b] = device_normal(row_shape, seed_key(workload, tensor, b, chunk, rewrite), dtype,
                               device, std)
    return out


# ----------------------------------------------------------------------------------------
# Workload sizes (the shapes of the pages' workloads; values are synthetic N(0,1))
# ----------------------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Tiny:
    """fp32, H=2, D=64, capacity 64, seven 8-token chunks written at [8c, 8c+8)."""
    B: int = 2
    H: int = 2
    D: int = 64
    cap: int = 64
    chunk: int = 8
    n_chunks: int = 7
    dtype: str = "f32"


@dataclasses.dataclass(frozen=True)
class Decode:
    """fp16/bf16, B=1, 32 query heads on 8 KV heads, D=128, capacity 32768, prompt of
    234 tokens (causal prefill) then 1024 single-token steps; values N(0,1)/sqrt(128)."""
    B: int = 1
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    cap: int = 32768
    prompt: int = 234
    steps: int = 1024
    std: float = 1.0 / np.sqrt(128.0)


@dataclasses.dataclass(frozen=True)
class Ring:
    """bf16, B=2 (cond/uncond), 12 heads, D=128, 3-frame chunks of 4680 tokens, 7 slots
    (21 frames = 32760 tokens) with the first chunk pinned, 4 rewrites per chunk,
    12 chunks then a reset."""
    B: int = 2
    H: int = 12
    D: int = 128
    C: int = 4680
    n_slots: int = 7
    sink: int = 1
    rewrites: int = 4
    n_chunks: int = 12


@dataclasses.dataclass(frozen=True)
class MultiUser:
    """bf16, B=8, 40 heads, D=128, capacity 16384, 16 chunks of 1024 written at one shared
    index; block-causal inside the current chunk (block 1 = causal)."""
    B: int = 8
    H: int = 40
    D: int = 128
    cap: int = 16384
    chunk: int = 1024
    n_chunks: int = 16
    block: int = 1


@dataclasses.dataclass(frozen=True)
class Ragged:
    """bf16, 2 CFG branches, 40 heads, D=128, padded Q of 75600 tokens per branch, K/V
    packed by cu_seqlens_kv, max_seqlen_kv 512."""
    B: int = 2
    H: int = 40
    D: int = 128
    Tq: int = 75600
    max_kv: int = 512
    skews: tuple = ((512, 448), (512, 256), (512, 51))
