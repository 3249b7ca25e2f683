"""Seeded synthetic inputs for the 4-bit codebook GEMV workloads.

This module only draws numbers: it holds none of the method's arithmetic
(no codebook, no scale, no packing, no product).  Both the oracle side and
the HIP side of every test and of the benchmark take their inputs from here.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style: output i of stream
`seed` is the SplitMix64 finaliser applied to seed + (i + 1) * golden_gamma.
Two outputs make one Box-Muller pair of standard normals (cosine branch for
the even element, sine branch for the odd one), computed in fp64.

The value distributions follow the deep-fold "Decode V2" page's shapes of a
3B-class decoder (section 6 bench table: down 2048x11008, gate/up, lm_head
151936x2048) with synthetic values standing in for checkpoint tensors:
W ~ N(0, 0.02^2) in fp32; x in bf16 (round to nearest even from fp64), either
N(0,1), unit-RMS N(0,1) (an RMSNorm output with gain 1), or SwiGLU-like
silu(a) * b with a, b ~ N(0,1) (the input of a down projection).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 17  # pairs per chunk: keeps temporaries below glibc's mmap threshold

# The five workloads: name -> (M, K, weight seed, x recipe, N).
CONFIGS = {
    "tiny": dict(M=256, K=512, seed=0, x="normal", N=1),
    "down": dict(M=2048, K=11008, seed=1, x="swiglu", N=1),
    "gateup": dict(M=22016, K=2048, seed=2, x="unit_rms", N=1),
    "lm_head": dict(M=151936, K=2048, seed=3, x="unit_rms", N=1),
    "smalln": dict(M=11008, K=2048, seed=4, x="unit_rms", N=32),
}


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of the counter-based SplitMix64 stream."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def normal(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Standard normals start .. start+n-1 of stream `seed` (fp64)."""
    if n == 0:
        return np.zeros(0)
    p0, p1 = start // 2, (start + n + 1) // 2
    out = np.empty(2 * (p1 - p0))
    for c0 in range(p0, p1, _CHUNK):
        c1 = min(p1, c0 + _CHUNK)
        z = splitmix64(seed, 2 * c0, 2 * (c1 - c0))
        u = (z >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)
        u1 = 1.0 - u[0::2]  # in (0, 1]
        u2 = u[1::2]
        r = np.sqrt(-2.0 * np.log(u1))
        t = 2.0 * np.pi * u2
        blk = out[2 * (c0 - p0): 2 * (c1 - p0)]
        blk[0::2] = r * np.cos(t)
        blk[1::2] = r * np.sin(t)
    off = start - 2 * p0
    return out[off: off + n]


def bf16_rne_bits(v) -> np.ndarray:
    """fp64 values -> bf16 bit patterns, one rounding to nearest even.

    Done on the fp64 bit pattern (no detour through fp32, which would round
    twice).  Inputs must be finite and within the normal bf16 range; the
    generated activations always are.
    """
    v = np.ascontiguousarray(v, np.float64)
    a = np.abs(v)
    nz = a[a != 0]
    if not np.all(np.isfinite(v)) or (nz.size and (nz.min() < 2.0 ** -126 or nz.max() >= 2.0 ** 127)):
        raise ValueError("bf16_rne_bits: value outside the normal bf16 range")
    b = v.view(np.uint64)
    shift = np.uint64(45)  # fp64 keeps 52 fraction bits, bf16 keeps 7
    with np.errstate(over="ignore"):
        lsb = (b >> shift) & np.uint64(1)
        b = b + (np.uint64((1 << 44) - 1) + lsb)
    b = b & ~np.uint64((1 << 45) - 1)
    r = b.view(np.float64).astype(np.float32)  # exact: 8 significant bits
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def weights(M: int, K: int, seed: int, std: float = 0.02, threads: int | None = None) -> np.ndarray:
    """W fp32 [M, K] ~ N(0, std^2).  Chunks are independent (counter-based
    stream), so they are drawn on several threads; the result does not depend
    on the thread count."""
    W = np.empty((M, K), np.float32)
    flat = W.reshape(-1)
    n = M * K
    step = 1 << 20

    def fill(s):
        e = min(n, s + step)
        flat[s:e] = (std * normal(seed, e - s, start=s)).astype(np.float32)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    starts = range(0, n, step)
    if threads <= 1 or n <= step:
        for s in starts:
            fill(s)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, starts))
    return W


def activation(K: int, seed: int, recipe: str, row: int = 0) -> np.ndarray:
    """x bf16 bits [K] for one token.  Stream seed*1000003+17 (+ row) keeps x
    independent of W's stream."""
    s = (seed * 1000003 + 17 + 7919 * row) & 0xFFFFFFFFFFFFFFFF
    if recipe == "normal":
        v = normal(s, K)
    elif recipe == "unit_rms":
        z = normal(s, K)
        v = z / np.sqrt(np.mean(z * z))
    elif recipe == "swiglu":
        a = normal(s, K)
        b = normal(s ^ 0x5DEECE66D, K)
        v = a / (1.0 + np.exp(-a)) * b
    else:
        raise ValueError(recipe)
    return bf16_rne_bits(v)


def activations(N: int, K: int, seed: int, recipe: str) -> np.ndarray:
    """X bf16 bits [N, K]: N independent tokens."""
    return np.stack([activation(K, seed, recipe, row=n) for n in range(N)]) if N else np.zeros((0, K), np.uint16)


def config_inputs(name: str, n_tokens: int | None = None):
    """(W fp32 [M,K], x or X bf16 bits) for a named workload."""
    c = CONFIGS[name]
    W = weights(c["M"], c["K"], c["seed"])
    N = c["N"] if n_tokens is None else n_tokens
    if N == 1 and n_tokens is None:
        return W, activation(c["K"], c["seed"], c["x"])
    return W, activations(N, c["K"], c["seed"], c["x"])
