"""Seeded, counter-based synthetic inputs shared by the oracle and the HIP path.

This module generates numbers only. It holds none of the method's arithmetic
(no attention, no allocation): both sides of every parity check draw their
K/V/Q values and their random workload choices from here, so that the two
implementations start from bit-identical inputs and share nothing else.

Definition (the device generator in ``gen.hip`` implements the same one):

* ``mix(z)`` is the SplitMix64 output finaliser published by Steele, Lea and
  Flood, "Fast splittable pseudorandom number generators" (OOPSLA 2014), with
  the multiplier pair used by the widely published ``splitmix64`` reference
  code.  All arithmetic is modulo 2**64.
* The i-th output of a SplitMix64 generator whose state starts at ``s`` is
  ``mix(s + (i + 1) * GAMMA)``.
* A stream is keyed ``key(seed, stream) = mix(seed + (stream + 1) * GAMMA)``.
* Element ``i`` of a stream is ``TABLE[mix(key + (i + 1) * GAMMA) >> 48]``.
* ``TABLE[j]`` is the standard normal quantile at ``(j + 0.5) / 65536``
  (``statistics.NormalDist().inv_cdf``), rounded once to float32 and, for
  bf16 inputs, once more from float32 to bf16 with round-to-nearest-even.
  So values are a 65 536-level quantised N(0, 1), truncated at about +-4.32.
* Uniform integers in ``[0, n)`` are ``(mix(...) >> 32) % n``.

Streams are ``(kind << 40) | index`` with the kinds below, so that every
append call, query call and random choice of a workload owns its own stream.
"""

from __future__ import annotations

import statistics

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MUL1 = 0xBF58476D1CE4E5B9
MUL2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

KIND_K = 1
KIND_V = 2
KIND_Q = 3
KIND_SHAPE = 4
KIND_ACCEPT = 5


def stream_id(kind: int, index: int) -> int:
    if not (0 <= index < (1 << 40)):
        raise ValueError("stream index out of range")
    return (kind << 40) | index


def mix_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (mod 2**64)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MUL1) & MASK64
    z = ((z ^ (z >> 27)) * MUL2) & MASK64
    return z ^ (z >> 31)


def _mix_np(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(MUL1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(MUL2)
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, stream: int) -> int:
    return mix_int(seed + (stream + 1) * GAMMA)


def raw_u64(seed: int, stream: int, index: np.ndarray) -> np.ndarray:
    """64-bit outputs ``mix(key + (index + 1) * GAMMA)`` for an index array."""
    key = np.uint64(stream_key(seed, stream))
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + (idx + np.uint64(1)) * np.uint64(GAMMA)
        return _mix_np(z)


def _bf16_rne_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returned as float32."""
    u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    bias = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    r = ((u + bias) >> np.uint64(16)) << np.uint64(16)
    return r.astype(np.uint32).view(np.float32)


_TABLE_F32 = None


def normal_table(dtype: str) -> np.ndarray:
    """The 65 536-entry quantised-normal table for ``dtype`` ('f32' or 'bf16'), as float32."""
    global _TABLE_F32
    if _TABLE_F32 is None:
        nd = statistics.NormalDist()
        t = np.array([nd.inv_cdf((j + 0.5) / 65536.0) for j in range(65536)], dtype=np.float64)
        _TABLE_F32 = t.astype(np.float32)
    if dtype == "f32":
        return _TABLE_F32.copy()
    if dtype == "bf16":
        return _bf16_rne_from_f32(_TABLE_F32)
    raise ValueError(dtype)


def normal_table_bits(dtype: str) -> np.ndarray:
    """Table as raw bits: uint16 for bf16, uint32 for f32 (what the device kernel reads)."""
    t = normal_table(dtype)
    if dtype == "bf16":
        return (t.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return t.view(np.uint32).copy()


def values(seed: int, stream: int, index, dtype: str) -> np.ndarray:
    """Elements ``index`` of a stream, as float32 (exactly representable in ``dtype``)."""
    t = normal_table(dtype)
    z = raw_u64(seed, stream, index)
    return t[(z >> np.uint64(48)).astype(np.int64)]


def values_range(seed: int, stream: int, start: int, count: int, dtype: str) -> np.ndarray:
    return values(seed, stream, np.arange(start, start + count, dtype=np.uint64), dtype)


def uniform_int(seed: int, stream: int, index: int, n: int) -> int:
    """Element ``index`` of a stream as a uniform integer in [0, n)."""
    key = stream_key(seed, stream)
    z = mix_int(key + (index + 1) * GAMMA)
    return (z >> 32) % n
