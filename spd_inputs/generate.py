"""Seeded synthetic inputs: random-init weights and uniform random prompts.

Both the CPU oracle and the GPU path load their inputs from here, so they see
identical bits. Nothing here is part of the method: it draws numbers, and
stores them in the workload's weight format.

Recipe:
  * every matrix ~ N(0, weight_std^2), drawn in float32 and stored as bfloat16
    (round to nearest even) for bf16 workloads, as float32 otherwise;
  * RMSNorm gains are 1.0, stored as float32;
  * proj_init == "select_deepest": W_proj = [0 | ... | 0 | I] + N(0, proj_noise_std^2);
  * prompt ids are i.i.d. uniform in [0, vocab).
Each tensor is drawn in chunks of 2^22 values, chunk c of tensor `name` from
PCG64(SeedSequence([weight_seed, crc32(name), c])), so tensors can be drawn
independently and in parallel, and the result does not depend on thread count.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterable, Optional

import numpy as np

from .configs import ModelConfig, tensor_names, tensor_shape

CHUNK = 1 << 22


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _draw(name: str, seed: int, numel: int, std: float, bf16: bool) -> np.ndarray:
    key = zlib.crc32(name.encode())
    out = np.empty(numel, dtype=np.uint16 if bf16 else np.float32)
    for c0 in range(0, numel, CHUNK):
        c1 = min(numel, c0 + CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key, c0 // CHUNK])))
        x = g.standard_normal(c1 - c0, dtype=np.float32)
        x *= np.float32(std)
        out[c0:c1] = _f32_to_bf16_bits(x) if bf16 else x
    return out


def make_tensor(cfg: ModelConfig, name: str) -> np.ndarray:
    """One weight tensor. bf16 tensors come back as uint16 bit patterns."""
    shape = tensor_shape(cfg, name)
    if name.endswith("norm"):
        return np.ones(shape, dtype=np.float32)
    bf16 = cfg.dtype == "bf16"
    numel = int(np.prod(shape))
    if name == "pdm.proj" and cfg.proj_init == "select_deepest":
        d = cfg.d_model
        noise = _draw(name, cfg.weight_seed, numel, cfg.proj_noise_std, False).reshape(shape)
        noise[:, shape[1] - d:] += np.eye(d, dtype=np.float32)
        return _f32_to_bf16_bits(noise).reshape(shape) if bf16 else noise
    return _draw(name, cfg.weight_seed, numel, cfg.weight_std, bf16).reshape(shape)


def make_weights(cfg: ModelConfig, names: Optional[Iterable[str]] = None,
                 threads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All (or the named) weight tensors of a workload, drawn in parallel."""
    names = list(names) if names is not None else tensor_names(cfg)
    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as ex:
        arrays = list(ex.map(lambda nm: make_tensor(cfg, nm), names))
    return dict(zip(names, arrays))


def make_prompt(cfg: ModelConfig, length: Optional[int] = None, seed: Optional[int] = None) -> np.ndarray:
    length = cfg.prompt_len if length is None else length
    seed = cfg.prompt_seed if seed is None else seed
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x50524F4D])))
    return g.integers(0, cfg.vocab, size=length, dtype=np.int64).astype(np.int32)


def weight_bytes(cfg: ModelConfig) -> int:
    per = 2 if cfg.dtype == "bf16" else 4
    tot = 0
    for nm in tensor_names(cfg):
        n = int(np.prod(tensor_shape(cfg, nm)))
        tot += n * (4 if nm.endswith("norm") else per)
    return tot
