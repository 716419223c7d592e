"""Seeded synthetic inputs shared by the oracle-side and the HIP-side tests.

This module only draws random numbers and stores them in the storage types the
kernels read (IEEE f32, bf16 bit patterns, int32, u8).  It holds none of the
method's arithmetic: no op, no gradient, no reduction.

Two generators:

* ``host_*``: numpy ``default_rng([seed, stream])``, one stream per named
  tensor, f64 draws rounded to the storage type.  Used for every case the
  oracle checks in full.
* ``device_*``: torch's seeded philox generator on the GPU, for the full-size
  workloads (several GB per tensor) that would take minutes to draw on the
  host.  The oracle then reads sampled rows of the same *input* tensor back to
  the host; nothing it compares against is produced by the library.

bf16 values are carried as ``uint16`` bit patterns (the upper half of the f32
pattern, round-to-nearest-even), which is the layout the library reads.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "host_normal", "host_uniform_int", "host_zipf_int", "host_bf16_bits", "bf16_bits_to_f32",
    "device_normal", "device_uniform_int", "STREAMS",
]

# Stable stream ids for named tensors, so every test and the bench draw the
# same values for "x", "gamma", ... of a workload.
STREAMS = {
    "x": 1, "gamma": 2, "beta": 3, "bias": 4, "targets": 5, "dout": 6,
    "g": 7, "u": 8, "a": 9, "b": 10, "w": 11, "logits": 12, "q": 13, "k": 14,
    "v": 15, "resid": 16, "d2": 17, "d3": 18, "wq": 20, "wk": 21, "wv": 22,
    "wo": 23, "wg": 24, "wu": 25, "wd": 26, "wout": 27, "w1": 28, "w2": 29, "ids": 30, "emb": 31,
}


def _stream(name_or_id) -> int:
    if isinstance(name_or_id, str):
        return STREAMS[name_or_id]
    return int(name_or_id)


def host_bf16_bits(x) -> np.ndarray:
    """Round f32 values to bf16 (nearest, ties to even) and return the uint16
    bit patterns.  NaN is kept quiet."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(f)
    r = np.where(nan, (u >> 16).astype(np.uint32) | 0x40, r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to f32 (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def host_normal(shape, seed: int, stream, mean: float = 0.0, std: float = 1.0,
                dtype: str = "f32") -> np.ndarray:
    """N(mean, std^2) draws in f64 from stream ``(seed, stream)``, stored as
    ``dtype`` ("f32" -> float32 array, "bf16" -> uint16 bit patterns,
    "f64" -> float64)."""
    g = np.random.default_rng([int(seed), _stream(stream)])
    x = g.standard_normal(size=shape) * std + mean
    if dtype == "f64":
        return x
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return host_bf16_bits(x.astype(np.float32))
    raise ValueError(dtype)


def host_uniform_int(shape, low: int, high: int, seed: int, stream) -> np.ndarray:
    """Uniform int32 in [low, high) from stream ``(seed, stream)``."""
    g = np.random.default_rng([int(seed), _stream(stream)])
    return g.integers(low, high, size=shape, dtype=np.int64).astype(np.int32)


def host_zipf_int(shape, vocab: int, a: float, seed: int, stream) -> np.ndarray:
    """Token ids with a Zipf(a) rank distribution folded into [0, vocab)
    (rank k -> id (k - 1) mod vocab), int32, from stream ``(seed, stream)``:
    a few ids repeat very often, most rarely, as in text."""
    g = np.random.default_rng([int(seed), _stream(stream)])
    return ((g.zipf(a, size=shape) - 1) % vocab).astype(np.int32)


def _torch_gen(seed: int, stream, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1000003 + _stream(stream)) & 0x7FFFFFFFFFFFFFFF)
    return g


def device_normal(shape, seed: int, stream, mean: float = 0.0, std: float = 1.0,
                  dtype: str = "f32", device="cuda", chunk_rows: int = 4096):
    """N(mean, std^2) drawn on the GPU by torch's seeded generator, stored as
    f32 or bf16 (a torch tensor).  Drawn in row chunks so no f32 temporary
    larger than ``chunk_rows`` rows exists next to a bf16 result."""
    import torch
    g = _torch_gen(seed, stream, device)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    out = torch.empty(shape, dtype=tdt, device=device)
    flat = out.view(-1, shape[-1]) if len(shape) > 1 else out.view(1, -1)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        t = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        if mean != 0.0:
            t.add_(mean)
        flat[r0:r1].copy_(t)
    return out


def device_uniform_int(shape, low: int, high: int, seed: int, stream, device="cuda"):
    """Uniform int32 in [low, high) drawn on the GPU by torch's generator."""
    import torch
    g = _torch_gen(seed, stream, device)
    return torch.randint(low, high, shape, generator=g, device=device,
                         dtype=torch.int64).to(torch.int32)
