"""GPU parity of the NN, TN and TT layouts (dg_fp8_gemm_nn / _tn / _tt)
against the oracle's definition on the logical operands.

An operand stored MN-major ([K][M] or [K][N]) reaches the matrix
instructions through transposing LDS reads; these tests cover both tile
configurations (128x128 and 256x256), M and N tails within the 16-column
granularity, every layout with and without C, a bit-exact permutation case
that pins the transposed read (which K row lands in which byte of which
lane), and the prefill workloads at full size, sampled.  Tolerance as for the
NT GEMM: |D - D_ref| <= ulp_bf16(D_ref) + 1e-4 max|D_ref|.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_scaled_amd import binding as dg
from moe_grouped_gemm_scaled_amd import synth

from helpers import Guarded, check_close, dense_problem, dev, dev_bf16, sample_indices

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dg.lib()
    yield
    torch.cuda.synchronize()


def stored(layout, a, b):
    """Logical a[M,K], b[N,K] -> the arrays the layout stores."""
    a_st = np.ascontiguousarray(a.T) if layout[0] == "t" else a
    b_st = np.ascontiguousarray(b.T) if layout[1] == "n" else b
    return a_st, b_st


def run(layout, a_st, sfa, b_st, sfb, c, M, N):
    out = Guarded((M, N))
    dg.fp8_gemm(layout, dev(a_st), dev(sfa), dev(b_st), dev(sfb), out.t, c=dev_bf16(c) if c is not None else None)
    torch.cuda.synchronize()
    assert out.guards_intact()
    return out.bits()


# (M, N, K, with_c): 128x128 tiles with tails, a small M, and 256x256 tiles
# (long K); M (N) stays a multiple of 16 where A (B) is stored MN-major
SHAPES = [(256, 384, 512, True), (304, 528, 768, False), (64, 256, 1024, True), (512, 512, 2304, True),
          (272, 400, 2432, False)]


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("M,N,K,with_c", SHAPES)
def test_layout_dense(layout, M, N, K, with_c):
    announce(f"layout {layout} M={M} N={N} K={K} C={with_c}")
    p = dense_problem(M, N, K, seed=M + 7 * N + K, with_c=with_c)
    a_st, b_st = stored(layout, p["a"], p["b"])
    got = run(layout, a_st, p["sfa"], b_st, p["sfb"], p["c"], M, N)
    assert f"layout={layout}" in dg.last_config(), dg.last_config()
    ref = oracle.gemm_layout(layout, a_st, p["sfa"], b_st, p["sfb"], p["c"])
    check_close(got, ref, f"{layout} {M}x{N}x{K} ({dg.last_config()})")


@pytest.mark.parametrize("layout", ["nn", "tt"])
def test_layout_k_major_operand_any_size(layout):
    """The K-major operand of NN (A) and TT (B) takes any size."""
    M, N = (300, 256) if layout == "nn" else (256, 300)
    K = 640
    announce(f"layout {layout} ragged K-major side M={M} N={N}")
    p = dense_problem(M, N, K, seed=91, with_c=True)
    a_st, b_st = stored(layout, p["a"], p["b"])
    got = run(layout, a_st, p["sfa"], b_st, p["sfb"], p["c"], M, N)
    ref = oracle.gemm_layout(layout, a_st, p["sfa"], b_st, p["sfb"], p["c"])
    check_close(got, ref, f"{layout} ragged ({dg.last_config()})")


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("M,K", [(256, 512), (512, 2304)])
def test_layout_permutation_bitexact(layout, M, K):
    """B(n, k) = 1 exactly when k = perm(n), power-of-two scales: D[m, n] is
    the single product A(m, perm(n)) * sfa * sfb, so any mix-up of K rows,
    lanes or bytes in the transposing reads changes bits."""
    N = K
    announce(f"layout {layout} permutation M={M} K={K}")
    a = synth.random_codes(92, 0, (M, K))
    perm = np.argsort(synth.uniform(92, 1, N))
    b = np.zeros((N, K), dtype=np.uint8)
    b[np.arange(N), perm] = 0x38
    ea = synth.randint(92, 4, (K // 128) * M, -6, 6).reshape(K // 128, M)
    eb = synth.randint(92, 5, (N // 128) * (K // 128), -6, 6).reshape(N // 128, K // 128)
    sfa = np.ldexp(np.float32(1.0), ea).astype(np.float32)
    sfb = np.ldexp(np.float32(1.0), eb).astype(np.float32)
    a_st, b_st = stored(layout, a, b)
    got = run(layout, a_st, sfa, b_st, sfb, None, M, N)
    ref = oracle.gemm_layout(layout, a_st, sfa, b_st, sfb, None)
    assert np.all(ref.astype(np.float32).astype(np.float64) == ref)
    ref_bits = synth.f32_to_bf16_bits(ref.astype(np.float32))
    eq = (got == ref_bits) | ((ref == 0) & ((got & 0x7FFF) == 0))
    assert np.all(eq), np.argwhere(~eq)[:5]


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("cfg", synth.PREFILL, ids=lambda c: c["name"])
def test_layout_prefill_full_size_sampled(layout, cfg):
    """The prefill workloads in each layout, in the launch configuration the
    benchmark times, on sampled elements (N tail included)."""
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    announce(f"layout {layout} full size {cfg['name']}")
    p = dense_problem(M, N, K, cfg["seed"], cfg["with_c"])
    a_st, b_st = stored(layout, p["a"], p["b"])
    got = run(layout, a_st, p["sfa"], b_st, p["sfb"], p["c"], M, N)
    ms = sample_indices(M, 96, cfg["seed"], stream=10)
    ns = sample_indices(N, 96, cfg["seed"], stream=11)
    ns = np.unique(np.concatenate([ns, np.arange(max(0, N - 40), N)])).astype(np.int32)
    mm, nn = np.meshgrid(ms, ns, indexing="ij")
    ref = oracle.gemm_layout_at(layout, a_st, p["sfa"], b_st, p["sfb"], p["c"], mm.reshape(-1), nn.reshape(-1))
    check_close(got[mm, nn].reshape(-1), ref, f"{cfg['name']} {layout}")
