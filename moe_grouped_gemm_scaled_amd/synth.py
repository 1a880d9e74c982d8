"""Seeded synthetic inputs shared by the tests and the benchmark.

This module holds no arithmetic of the method (no quantisation, no GEMM):
only a counter-based generator, the workload shapes and the MoE row layouts.
The same arrays are handed to the HIP path and to the CPU oracle.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014) in counter form,
    x_i = mix64(s0 + (i + 1) * 0x9E3779B97F4A7C15),
    s0  = (seed * 0x9E3779B97F4A7C15) xor stream,
uniform u_i = (x_i >> 11) * 2^-53, standard normal by the Box-Muller transform
in fp64 from (1 - u_{2j}, u_{2j+1}), rounded to fp32.  Integers in [lo, hi]
are lo + floor(u * (hi - lo + 1)).

Streams: 0 = A, 1 = B, 2 = C, 3 = counts (token counts, masked_m).
"""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

STREAM_A, STREAM_B, STREAM_C, STREAM_COUNTS = 0, 1, 2, 3

_CHUNK = 1 << 22


def _mix64(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _base(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        return np.uint64((int(seed) * 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF) ^ np.uint64(stream)


def raw_u64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """x_i for i in [start, start + count)."""
    s0 = _base(seed, stream)
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix64(s0 + i * GOLDEN)


def uniform(seed: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    """n fp64 uniforms in [0, 1)."""
    return (raw_u64(seed, stream, start, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_f32(seed: int, stream: int, shape) -> np.ndarray:
    """fp32 N(0, 1) array of the given shape (C order), in chunks of 2^22
    values; chunks are independent (counter-based), so large arrays are
    filled by a few threads at once (numpy releases the GIL in these loops)
    with the same result."""
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.float32)

    def fill(lo):
        cnt = min(_CHUNK, n - lo)
        u = uniform(seed, stream, 2 * cnt, start=2 * lo)
        u1 = 1.0 - u[0::2]
        u2 = u[1::2]
        out[lo:lo + cnt] = (np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)).astype(np.float32)

    starts = range(0, n, _CHUNK)
    if n <= 2 * _CHUNK:
        for lo in starts:
            fill(lo)
    else:
        with concurrent.futures.ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, starts))
    return out.reshape(shape)


def randint(seed: int, stream: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform in [lo, hi] (inclusive), int64."""
    u = uniform(seed, stream, n)
    return (lo + np.floor(u * (hi - lo + 1))).astype(np.int64)


def random_codes(seed: int, stream: int, shape, allow_nan: bool = False) -> np.ndarray:
    """Uniformly random E4M3 bit patterns (uint8); NaN codes 0x7F/0xFF replaced by +-448 unless allowed."""
    n = int(np.prod(shape, dtype=np.int64))
    q = (raw_u64(seed, stream, 0, n) >> np.uint64(56)).astype(np.uint8)
    if not allow_nan:
        q[q == 0x7F] = 0x7E
        q[q == 0xFF] = 0xFE
    return q.reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bit patterns.

    Used only to prepare the bf16 C operand from fp32 draws; inputs are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return (u >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16_bits(seed: int, stream: int, shape) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(seed, stream, shape))


# --------------------------------------------------------------------------
# MoE row layouts
# --------------------------------------------------------------------------

def contiguous_m_indices(counts, align: int = 128) -> np.ndarray:
    """Concatenate per-expert segments, each padded up to a multiple of `align`
    rows; valid rows carry the expert id, padding rows carry -1."""
    parts = []
    for g, c in enumerate(counts):
        c = int(c)
        padded = (c + align - 1) // align * align
        seg = np.full(padded, -1, dtype=np.int32)
        seg[:c] = g
        parts.append(seg)
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int32)


# --------------------------------------------------------------------------
# Workloads (sizes of the measured configurations)
# --------------------------------------------------------------------------

SEED_BASE = 1000

DENSE_SMALL = dict(name="dense_128x256x512", M=128, N=256, K=512, with_c=False, seed=SEED_BASE + 0)

DECODE_NK = [(2112, 7168), (24576, 1536), (7168, 16384)]
DECODE_M = [64, 128]
DECODE = [dict(name=f"decode_m{m}_n{n}_k{k}", M=m, N=n, K=k, with_c=False, seed=SEED_BASE + 1)
          for m in DECODE_M for (n, k) in DECODE_NK]

PREFILL_NK = [(4096, 7168), (7168, 2048), (24576, 1536)]
PREFILL = [dict(name=f"prefill_m4096_n{n}_k{k}", M=4096, N=n, K=k, with_c=True, seed=SEED_BASE + 2)
           for (n, k) in PREFILL_NK]

CONTIGUOUS = dict(name="contiguous_g8_n4096_k7168", G=8, N=4096, K=7168, count_lo=1, count_hi=4096,
                  align=128, seed=SEED_BASE + 3)

MASKED = dict(name="masked_g16_cap256_n7168_k2048", G=16, M_cap=256, N=7168, K=2048, mm_lo=0, mm_hi=256,
              seed=SEED_BASE + 4)


def contiguous_counts(cfg=CONTIGUOUS) -> np.ndarray:
    return randint(cfg["seed"], STREAM_COUNTS, cfg["G"], cfg["count_lo"], cfg["count_hi"])


def masked_counts(cfg=MASKED) -> np.ndarray:
    return randint(cfg["seed"], STREAM_COUNTS, cfg["G"], cfg["mm_lo"], cfg["mm_hi"]).astype(np.int32)


# --------------------------------------------------------------------------
# MQA logits inputs (the v3.2 indexer's scoring: q [S, H, 128] and kv
# [S_kv, 128] E4M3, kv_scale [S_kv], weights [S, H], key ranges [S])
# --------------------------------------------------------------------------

STREAM_Q, STREAM_KV, STREAM_KV_SCALE, STREAM_WEIGHTS = 10, 11, 12, 13

# One prefill chunk of 4096 query tokens at the end of an 8192-token context,
# causal: query i sees keys [0, S_kv - S + i + 1).  64 heads of dim 128 (the
# indexer's head layout).
MQA = dict(name="mqa_s4096_skv8192_h64", S=4096, S_kv=8192, H=64, D=128, seed=SEED_BASE + 5)


def mqa_tensors(seed: int, S: int, H: int, S_kv: int, D: int = 128):
    """q, kv (uniformly random E4M3 codes, no NaN), kv_scale (positive,
    2^-9 (1 + u)), weights (N(0, 1) / sqrt(H))."""
    q = random_codes(seed, STREAM_Q, (S, H, D))
    kv = random_codes(seed, STREAM_KV, (S_kv, D))
    kv_scale = ((1.0 + uniform(seed, STREAM_KV_SCALE, S_kv)) * 2.0 ** -9).astype(np.float32)
    weights = (normal_f32(seed, STREAM_WEIGHTS, (S, H)) / np.float32(np.sqrt(H))).astype(np.float32)
    return q, kv, kv_scale, weights


def causal_ranges(S: int, S_kv: int):
    """Queries are the last S of S_kv tokens: query i sees keys [0, S_kv - S + i + 1)."""
    ks = np.zeros(S, dtype=np.int32)
    ke = (S_kv - S + 1 + np.arange(S)).astype(np.int32)
    return ks, ke


def packed_ranges(lengths):
    """Sequences packed back to back (S = S_kv = sum of lengths), causal within
    each: query i of a sequence starting at b sees keys [b, i + 1)."""
    ks, ke, b = [], [], 0
    for L in lengths:
        L = int(L)
        ks.append(np.full(L, b, dtype=np.int32))
        ke.append((b + 1 + np.arange(L)).astype(np.int32))
        b += L
    return np.concatenate(ks), np.concatenate(ke)


# K-grouped TN contiguous (MoE weight gradient): the expert down-projection's
# weight gradient dW[g] = dY_g^T X_g, with M = 7168 (hidden), N = 2048 (expert
# intermediate) and the 8 experts' token counts of the contiguous workload,
# each padded to 128 rows, as the K groups; no C (a fresh gradient).
KGROUPED = dict(name="kgrouped_g8_m7168_n2048", G=8, M=7168, N=2048, with_c=False, seed=SEED_BASE + 6)


def kgrouped_sizes(cfg=KGROUPED) -> np.ndarray:
    counts = contiguous_counts()
    return ((counts + 127) // 128 * 128).astype(np.int32)
