"""GPU parity of the K-grouped TN contiguous GEMM
(dg_k_grouped_fp8_gemm_tn_contiguous) against the oracle.

Both operands are stored with K as the slow index and reach the matrix
instructions through transposing LDS reads; B carries one scale per column
and 128 K rows, so the promotion multiplies by a per-column scale.  Cases:
both tile configurations, empty groups (D = C exactly), C aliasing D, M and N
tails within the 16-column granularity, and the weight-gradient workload at
full size, sampled.  Tolerance: the GEMMs' bar without the bf16 rounding,
    |D - D_ref| <= 2^-20 |D_ref| + 1e-4 max|D_ref|  (max over the group's compared elements).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import binding as dg
from moe_grouped_gemm_scaled_amd import synth

pytestmark = pytest.mark.gpu

UNTOUCHED = np.float32(np.nan)


def announce(msg):
    print(f"\n[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.lib()
    yield
    torch.cuda.synchronize()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def problem(seed, ks, M, N, with_c):
    """Activations quantised 1x128 along K by the oracle: the [K, M] operand is
    the transpose of a [M, K] array quantised per row and 128-column block."""
    K = int(np.sum(ks))
    xa = synth.normal_f32(seed, synth.STREAM_A, (M, K))
    xb = synth.normal_f32(seed, synth.STREAM_B, (N, K))
    qa, sa = oracle.quantize_1x128(xa, ld_sf=M)
    qb, sb = oracle.quantize_1x128(xb, ld_sf=N)
    a = np.ascontiguousarray(qa.T)                 # [K, M]
    b = np.ascontiguousarray(qb.T)                 # [K, N]
    c = synth.normal_f32(seed, synth.STREAM_C, (len(ks), M, N)) if with_c else None
    return a, sa[:, :M].copy(), b, sb[:, :N].copy(), np.asarray(ks, np.int32), c


def run(a, sfa, b, sfb, ks, c, alias=False):
    G, M, N = len(ks), a.shape[1], b.shape[1]
    guard = 64
    flat = torch.full((G * M * N + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    d = flat[guard:guard + G * M * N].view(G, M, N)
    ct = None
    if c is not None:
        if alias:
            d.copy_(dev(c))
            ct = d
        else:
            ct = dev(c)
    dg.k_grouped_fp8_gemm_tn_contiguous(dev(a), dev(sfa), dev(b), dev(sfb), dev(ks), d, c=ct)
    torch.cuda.synchronize()
    host = flat.cpu().numpy()
    assert np.all(np.isnan(host[:guard])) and np.all(np.isnan(host[-guard:])), "write outside D"
    return host[guard:guard + G * M * N].reshape(G, M, N)


def check(got, ref, where):
    got = got.astype(np.float64)
    assert got.shape == ref.shape and np.all(np.isfinite(ref))
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    tol = 2.0 ** -20 * np.abs(ref) + 1e-4 * scale
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    if np.any(bad):
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{where}: {int(bad.sum())} of {bad.size} outside tolerance; first {i.tolist()}: "
                             f"got {got[bad][:5]}, ref {ref[bad][:5]}, tol {tol[bad][:5]}")


CASES = [([256, 0, 128, 384], 128, 144, True, False),       # 128x128 tiles, an empty group, N tail
         ([512, 128, 0, 640], 272, 400, False, False),       # 256x256 tiles, M and N tails
         ([1024], 256, 256, True, True),                    # C aliasing D
         ([128, 128, 128], 64, 48, True, False)]             # tiny M and N


@pytest.mark.parametrize("ks,M,N,with_c,alias", CASES)
def test_k_grouped(ks, M, N, with_c, alias):
    announce(f"k-grouped ks={ks} M={M} N={N} C={with_c} alias={alias}")
    a, sfa, b, sfb, ksa, c = problem(80 + M + N, ks, M, N, with_c)
    got = run(a, sfa, b, sfb, ksa, c, alias)
    ref = oracle.k_grouped_tn(a, sfa, b, sfb, ksa, c)
    for g in range(len(ks)):
        if ks[g] == 0:
            want = c[g] if c is not None else np.zeros((M, N), np.float32)
            assert np.array_equal(got[g], want), f"empty group {g}: D must equal C"
        else:
            check(got[g], ref[g], f"group {g} ({dg.last_config()})")


def test_k_grouped_all_groups_empty():
    announce("k-grouped all groups empty")
    M, N = 128, 128
    a, sfa, b, sfb, _, c = problem(84, [128], M, N, True)
    ks = np.zeros(3, np.int32)
    c3 = synth.normal_f32(84, 7, (3, M, N))
    got = run(a, sfa, b, sfb, ks, c3)
    assert np.array_equal(got, c3)
    got0 = run(a, sfa, b, sfb, ks, None)
    assert np.all(got0 == 0)


def test_k_grouped_full_size_sampled():
    """The weight-gradient workload in the launch configuration the benchmark
    times, on sampled elements of every group."""
    cfg = synth.KGROUPED
    ks = synth.kgrouped_sizes(cfg)
    M, N = cfg["M"], cfg["N"]
    announce(f"k-grouped full size {cfg['name']} ks={ks.tolist()}")
    a, sfa, b, sfb, ksa, c = problem(cfg["seed"], ks, M, N, cfg["with_c"])
    got = run(a, sfa, b, sfb, ksa, c)
    for g in range(len(ks)):
        ms = np.unique(np.concatenate([synth.randint(cfg["seed"], 20 + g, 40, 0, M - 1), [0, M - 1]]))
        ns = np.unique(np.concatenate([synth.randint(cfg["seed"], 40 + g, 40, 0, N - 1), [0, N - 1]]))
        mm, nn = np.meshgrid(ms, ns, indexing="ij")
        gs = np.full(mm.size, g, np.int32)
        ref = oracle.k_grouped_tn_at(a, sfa, b, sfb, ksa, c, gs, mm.reshape(-1), nn.reshape(-1))
        check(got[g][mm, nn].reshape(-1), ref, f"{cfg['name']} group {g} ({dg.last_config()})")


def test_k_grouped_many_groups_with_empties():
    """40 groups of 0 to 512 rows (a third empty): the per-tile scan over the
    group sizes and the group-major tile numbering."""
    sizes = synth.randint(86, 3, 40, 0, 4) * 128
    sizes[::3] = 0
    ks = sizes.astype(np.int32)
    M, N = 128, 160
    announce(f"k-grouped 40 groups, K={int(ks.sum())}")
    a, sfa, b, sfb, ksa, c = problem(86, ks, M, N, True)
    got = run(a, sfa, b, sfb, ksa, c)
    ref = oracle.k_grouped_tn(a, sfa, b, sfb, ksa, c)
    for g in range(len(ks)):
        if ks[g] == 0:
            assert np.array_equal(got[g], c[g]), g
        else:
            check(got[g], ref[g], f"group {g}")
