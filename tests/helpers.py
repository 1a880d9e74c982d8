"""Shared helpers of the GPU parity tests.

Inputs come from the seeded generator and are quantised by the oracle; the
HIP path only ever receives copies of them.  Expected values come only from
the oracle.

Tolerance (the stated acceptance bar for the GEMM):
    |D - D_ref| <= ulp_bf16(D_ref) + 1e-4 * max|D_ref|
where D_ref is the oracle's unrounded fp64 result, ulp_bf16(x) = 2^(floor(log2|x|) - 7)
(2^-133 below the normal range), and the max runs over the computed elements
being compared.  The fp32 accumulation on the GPU adds at most one rounding
per 128-wide K block plus the final bf16 rounding (half an ulp), far inside it.
"""
import numpy as np
import torch

import oracle
from moe_grouped_gemm_scaled_amd import synth

SENTINEL = 0x7FA5          # a bf16 NaN payload that rounding a finite fp32 never produces
GUARD = 64                 # guard elements before and after every output buffer


def ulp_bf16(x):
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.where(ax >= 2.0 ** -126, np.ldexp(1.0, (e - 7).astype(np.int64)), 2.0 ** -133)


def check_close(got_bits, ref, where=""):
    """got_bits: uint16 bf16 patterns; ref: fp64 oracle values (same shape)."""
    got = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(ref)), where
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    tol = ulp_bf16(ref) + 1e-4 * scale
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    if np.any(bad):
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{where}: {int(bad.sum())} of {bad.size} outside tolerance; first {i.tolist()}: "
                             f"got {got[bad][:5]}, ref {ref[bad][:5]}, tol {tol[bad][:5]}")
    return float(np.max(err / np.maximum(tol, 1e-300))) if err.size else 0.0


# ------------------------------------------------------------ device transfer

def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Guarded:
    """A bf16 output tensor filled with SENTINEL, with guard bands around it."""

    def __init__(self, shape):
        self.shape = tuple(shape)
        n = int(np.prod(self.shape))
        self.flat = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.int16, device="cuda")
        self.t = self.flat[GUARD:GUARD + n].view(torch.bfloat16).view(self.shape)

    def bits(self) -> np.ndarray:
        return host_bits(self.t)

    def guards_intact(self) -> bool:
        f = self.flat.cpu().numpy().view(np.uint16)
        return bool(np.all(f[:GUARD] == SENTINEL) and np.all(f[-GUARD:] == SENTINEL))


# ------------------------------------------------------------ problems

def dense_problem(M, N, K, seed, with_c, ue8m0=False):
    xa = synth.normal_f32(seed, synth.STREAM_A, (M, K))
    xb = synth.normal_f32(seed, synth.STREAM_B, (N, K))
    a, sfa = oracle.quantize_1x128(xa, ue8m0=ue8m0)
    b, sfb = oracle.quantize_128x128(xb, ue8m0=ue8m0)
    c = synth.normal_bf16_bits(seed, synth.STREAM_C, (M, N)) if with_c else None
    return dict(a=a, sfa=sfa, b=b, sfb=sfb, c=c, M=M, N=N, K=K)


def contiguous_problem(counts, N, K, seed, with_c=False, ue8m0=False):
    m_idx = synth.contiguous_m_indices(counts)
    M_total = m_idx.size
    G = len(counts)
    xa = synth.normal_f32(seed, synth.STREAM_A, (M_total, K))
    xb = synth.normal_f32(seed, synth.STREAM_B, (G, N, K))
    a, sfa = oracle.quantize_1x128(xa, ue8m0=ue8m0)
    b, sfb = oracle.quantize_128x128(xb, ue8m0=ue8m0)
    c = synth.normal_bf16_bits(seed, synth.STREAM_C, (M_total, N)) if with_c else None
    return dict(a=a, sfa=sfa, b=b, sfb=sfb, c=c, m_indices=m_idx, M_total=M_total, N=N, K=K, G=G)


def masked_problem(G, M_cap, N, K, masked_m, seed, with_c=False, ue8m0=False):
    xa = synth.normal_f32(seed, synth.STREAM_A, (G, M_cap, K))
    xb = synth.normal_f32(seed, synth.STREAM_B, (G, N, K))
    a, sfa = oracle.quantize_1x128(xa, ue8m0=ue8m0)
    b, sfb = oracle.quantize_128x128(xb, ue8m0=ue8m0)
    c = synth.normal_bf16_bits(seed, synth.STREAM_C, (G, M_cap, N)) if with_c else None
    return dict(a=a, sfa=sfa, b=b, sfb=sfb, c=c, masked_m=np.asarray(masked_m, dtype=np.int32),
                G=G, M_cap=M_cap, N=N, K=K)


def sample_indices(n, count, seed, stream=9):
    """Sorted unique indices in [0, n) including both ends."""
    if n <= count:
        return np.arange(n, dtype=np.int32)
    pick = synth.randint(seed, stream, count, 0, n - 1)
    return np.unique(np.concatenate([pick, [0, n - 1]])).astype(np.int32)


def stratified_indices(n, seed, stream=20, within=None):
    """One index in every aligned block of 16 of [0, n) (the last block may be
    partial), its position in the block cycling over all 16 values from a
    seeded start, plus n - 1.  A mesh of such rows and columns compares every
    output tile of any width that is a multiple of 16, and every
    (row mod 16, column mod 16) position, i.e. every lane and register of the
    16x16 matrix-instruction layout.  `within`: only indices in this sorted
    array (blocks without any are skipped)."""
    start = int(synth.randint(seed, stream, 1, 0, 15)[0])
    out = []
    for b in range((n + 15) // 16):
        lo, hi = 16 * b, min(16 * b + 16, n)
        cand = np.arange(lo, hi) if within is None else within[(within >= lo) & (within < hi)]
        if cand.size == 0:
            continue
        want = lo + (start + 7 * b) % 16
        out.append(int(cand[np.argmin(np.abs(cand - want))]))
    last = n - 1 if within is None else (int(within[-1]) if within.size else None)
    if last is not None:
        out.append(last)
    return np.unique(np.array(out, dtype=np.int32))
